// Internal interfaces between the C ABI layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace onetrans {

typedef __attribute__((address_space(3))) void lds_void;

// GELU(x) = x Phi(x), Phi the standard normal CDF, with erfc from Abramowitz & Stegun,
// Handbook of Mathematical Functions, formula 7.1.26 (|error of erf| <= 1.5e-7 for all x):
// erfc(z) = (a1 t + ... + a5 t^5) exp(-z^2), t = 1 / (1 + p z), z >= 0. Written as
//   GELU(x) = max(x, 0) - |x| Phi(-|x|),  Phi(-|x|) = erfc(|x| / sqrt 2) / 2,
// which holds for both signs, with 1/2 folded into the coefficients and 1/sqrt 2 into p:
// 12 VALU operations plus one reciprocal and one exp2. The approximation error is three
// orders of magnitude below the fp16 rounding applied to the result.
__device__ __forceinline__ float gelu_as(float x) {
  constexpr float kP = 0.3275911f * 0.70710678118654752f;
  constexpr float kA1 = 0.5f * 0.254829592f, kA2 = 0.5f * -0.284496736f, kA3 = 0.5f * 1.421413741f,
                  kA4 = 0.5f * -1.453152027f, kA5 = 0.5f * 1.061405429f;
  constexpr float kE = -0.5f * 1.4426950408889634f;  // exp(-x^2 / 2) = exp2(kE x^2)
  const float a = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(kP, a, 1.0f));
  float q = fmaf(kA5, t, kA4);
  q = fmaf(q, t, kA3);
  q = fmaf(q, t, kA2);
  q = fmaf(q, t, kA1);
  const float e = __builtin_amdgcn_exp2f((x * x) * kE);
  return fmaf(-(a * (q * t)), e, fmaxf(x, 0.0f));
}

// v_permlane32_swap of v with a copy of itself: lo holds the low half's values in both
// halves, hi the high half's. (The elements are copied out before the bit casts: a
// __builtin_bit_cast of a vector element reads element 0 with this compiler.)
__device__ __forceinline__ void swap_halves(float v, float& lo, float& hi) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t a = r[0], b = r[1];
  lo = __builtin_bit_cast(float, a);
  hi = __builtin_bit_cast(float, b);
}

// The value that lane l ^ 32 holds (no LDS traffic). Both lanes of a pair must be active.
__device__ __forceinline__ float other_half(float v) {
  float lo, hi;
  swap_halves(v, lo, hi);
  return (threadIdx.x & 32) ? lo : hi;
}

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4):
// lane i's bytes land at lds + 16 * i. The 16-byte form exists only on gfx950, so the
// host compilation pass, which never runs device code, does not see the builtin.
__device__ __forceinline__ void dma16(const void* g, lds_void* l) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
#endif
}

// The same 16-byte DMA through a buffer resource: the address is the resource's base +
// soff (wave-uniform, an SGPR) + voff (per lane), so no 64-bit address arithmetic per
// lane; reads at or past the resource's byte count return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, lds_void* l) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, voff, soff, 0, 0);
#endif
}

// Maxima as plain v_max instructions. The builtin fmaxf of values the compiler cannot
// prove quiet (matrix-core results) first canonicalises each input with an extra
// instruction; scores are never signalling NaNs.
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// the max of 16 values (v[0] .. v[15]): seven v_max3 and one v_max in one block
template <class V>
__device__ __forceinline__ float vmax16(const V& v) {
  float m;
  asm("v_max3_f32 %0, %1, %2, %3\n\t"
      "v_max3_f32 %0, %0, %4, %5\n\t"
      "v_max3_f32 %0, %0, %6, %7\n\t"
      "v_max3_f32 %0, %0, %8, %9\n\t"
      "v_max3_f32 %0, %0, %10, %11\n\t"
      "v_max3_f32 %0, %0, %12, %13\n\t"
      "v_max3_f32 %0, %0, %14, %15\n\t"
      "v_max_f32 %0, %0, %16"
      : "=&v"(m)
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]), "v"(v[8]),
        "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15]));
  return m;
}
// max(v, value of lane l ^ 32) in every lane
__device__ __forceinline__ float max_halves(float v) {
  float lo, hi;
  swap_halves(v, lo, hi);
  return vmax(lo, hi);
}

// Row addressing shared by the GEMM prologue/epilogue.
//
// A GEMM covers `groups` groups of M rows each. Row r of group g
// decodes to seg = r / rows_per_seg, t = r % rows_per_seg, and touches:
//   residual row : res + seg*res_seg_stride + (res_row_base + t)*res_row_stride + g*res_group_stride
//   hidden row   : hid + ((seg*rows_per_seg + t)*row_mult + g) * ld_hid
//   token index  : t*row_mult + g   (used by the Q/K/V scatter)
// The S side uses one group with seg = user, t = row within the user's block;
// the NS side uses one group per NS position with seg = 0, t = candidate.
struct RowMap {
  int rows_per_seg;
  int row_mult;
  long res_seg_stride, res_row_base, res_row_stride, res_group_stride;
};

// Deferred RMSNorm. RMSNorm(x) W = r (x * g) W with r = 1 / sqrt(mean(x^2) + eps), one
// number per row, so the norm needs no pass of its own: whichever kernel writes residual
// rows (input conversion, attention, FFN down) also writes the operand of the next linear
// map, fp16 x * g (g: the gain of the norm that comes next), and partial sums of x^2 over
// the columns it owns; the GEMM that reads the operand sums the row's partials and scales
// its output row by r. Partials sit in rows of `ss_stride` floats (hidden-row addressing
// like the operand): FFN down writes slot c / 32 for columns c .. c + 31, attention slot h
// for head h, input conversion slot 0 for the whole row.
// Fixed slots keep the sums deterministic: every output is a function of its own row.
struct NormOut {
  _Float16* xg;              // operand rows [hidden row][d]; NULL: no norm follows
  const float* gain;         // gain row of group g at gain + g * gain_group_stride
  long gain_group_stride;
  float* ss;                 // partials [hidden row][ss_stride]
  int ss_stride;
};
__host__ __device__ constexpr int ss_stride_for(int d) { return ((d / 32 + 3) / 4) * 4; }

struct GemmParams {
  int M, N, K, groups;
  RowMap rm;
  // A operand: fp16 rows at a_in + hidden_row * K (x * g rows or FFN hidden rows)
  const _Float16* a_in;
  // QKV / FFN up: deferred RMSNorm of the A rows, r from ss_in[hidden row][0 .. ss_parts)
  // (ss_parts <= 32, rows of ss_stride floats); NULL: no row scale
  const float* ss_in; int ss_parts, ss_stride; float eps;
  // B operand: weights [N][K] (fp16 or E4M3FN codes), per-group stride in elements
  const void* w;
  long w_group_stride;
  const float* wscale;       // E4M3 only: scale[group*5 + scale_idx0 + col/scale_col_div]
  int scale_idx0, scale_col_div;
  // epilogue: Q/K/V scatter
  int d, dh;
  __bf16* q; long q_seg_stride, q_head_stride; int q_from;
  // K rows [.][H][slots][dh]; V either transposed (vt: [.][H][dh][kv_cap], the S cache)
  // or, when vt is NULL, row-major like K (v: the per-candidate NS values)
  __bf16* k; __bf16* vt; __bf16* v; long kv_seg_stride, kv_head_stride; int kv_cap, kv_slot_base;
  // epilogue: GELU into hidden rows (ld = N)
  _Float16* hid_out;
  // epilogue: residual add (residual addressing), then the next norm's operand (FFN down)
  float* res_out;
  NormOut nout;
};

enum GemmKind { GEMM_QKV = 0, GEMM_FFN_UP = 1, GEMM_FFN_DOWN = 2 };

// ns selects the private-weight (NS) instance; fp8_weights only applies to it.
hipError_t launch_gemm(GemmKind kind, bool fp8_weights, bool ns, const GemmParams& p, hipStream_t s);

// Attention of `nq` queries per (seg, head) against a K/V block (cache layout:
// K [.][H][cap][dh], V transposed [.][H][dh][cap]) plus, for NS queries, the
// candidate's own NS keys. Output is added to the residual rows.
struct AttnParams {
  int nq, H, d;
  const __bf16* q; long q_seg_stride, q_head_stride;         // q[seg][h][i][dh]
  float* res; long res_seg_stride, res_row_base, res_row_stride;  // row of query i
  const __bf16* k; const __bf16* vt; long kv_seg_stride, kv_head_stride; int kv_cap;
  int n_keys;        // filled key slots
  int key_pos0;      // global position of key slot 0
  int q_pos0;        // global position of query 0 (S queries: causal limit)
  const int* valid_from;   // [seg] first valid global position
  // NS only: own keys and values of the rows, row-major kn, vn [seg][H][nq][dh] (strides
  // kn_seg_stride, kn_head_stride); P NS tokens per group of rows
  const __bf16* kn; const __bf16* vn; long kn_seg_stride, kn_head_stride; int P;
  // NS only, one segment: n_x keys every query sees in full (the user's cached NS rows),
  // row-major xk, xv [H][n_x][dh]; n_x = 0: none
  const __bf16* xk; const __bf16* xv; long x_head_stride; int n_x;
  float scale_log2;  // log2(e) / sqrt(dh)
  // the FFN norm's operand: hidden row seg * nq + i, gain group i % P, partial slot h
  NormOut nout;
};

hipError_t launch_attention(bool ns, int dh, const AttnParams& p, int n_seg, hipStream_t s);

// The kernel instance launch_attention picks for nq queries per (segment, head).
enum AttnRoute {
  ATTN_NS2_64_2, ATTN_NS2_64_1, ATTN_NS2_32_2, ATTN_NS2_32_1,
  ATTN_NSSPLIT_64_GROUPED, ATTN_NSSPLIT_32_GROUPED, ATTN_NSSPLIT_64, ATTN_NSSPLIT_32,
  ATTN_SPLIT_64_GROUPED, ATTN_SPLIT_32_GROUPED, ATTN_SPLIT_64, ATTN_SPLIT_32,
  ATTN_TILE_64_4, ATTN_TILE_32_4, ATTN_TILE_64_2, ATTN_TILE_32_2,
  ATTN_ROUTE_COUNT
};
AttnRoute attention_route(bool ns, int dh, int nq, int H, int n_seg);
const char* attention_route_name(AttnRoute r);

// Zeroes cache slots [from[l], cap[l]) of `blocks` (user, head) blocks of every layer l in
// one launch: K [blocks][cap][dh] and V^T [blocks][dh][cap]. Key tiles that reach past
// the filled length then read zeros.
constexpr int ONETRANS_CLEAR_MAX_LAYERS = 16;
struct ClearTailParams {
  __bf16* k[ONETRANS_CLEAR_MAX_LAYERS];
  __bf16* vt[ONETRANS_CLEAR_MAX_LAYERS];
  int cap[ONETRANS_CLEAR_MAX_LAYERS], from[ONETRANS_CLEAR_MAX_LAYERS];
  int n_layers, blocks, dh;
};
hipError_t launch_cache_clear_tail(const ClearTailParams& p, hipStream_t s);

// Input rows (bf16) -> fp32 residual rows plus the first norm's operand and one partial
// per row. Row i of user i / rows_per_seg; with s_lens (S prefill) the first
// rows_per_seg - len_u rows of user u are padding and become zero, and valid_from[u]
// records the first valid one. Gain group of row i: i % P.
struct InputParams {
  const uint16_t* tok;
  const int* s_lens; int* valid_from;
  int n_rows, rows_per_seg, d, P;
  float* x;
  NormOut nout;
};
hipError_t launch_input_rows(const InputParams& p, hipStream_t s);

// Elementwise helpers.
hipError_t launch_bf16_to_f16(const uint16_t* src, _Float16* dst, long n, hipStream_t s);
// G weight matrices [N][K] (bf16 -> fp16, or E4M3 codes) into the GEMMs' panel layout
// [G][N/32][K/64][32][64]; N % 32 == 0 and K % 64 == 0.
hipError_t launch_pack_panels(const void* src, void* dst, bool fp8, long G, int N, int K, hipStream_t s);
hipError_t launch_copy_rows_f32(const float* src, long src_seg_stride, float* dst, long dst_seg_stride,
                                long row_elems, int n_seg, hipStream_t s);
hipError_t launch_cache_read(const __bf16* k, const __bf16* vt, int H, int dh, int cap, int rows,
                             __bf16* k_out, __bf16* v_out, hipStream_t s);

}  // namespace onetrans
