// Internal interfaces between the C ABI layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace onetrans {

// Row addressing shared by the GEMM prologue/epilogue.
//
// A GEMM covers `groups` groups (blockIdx.z) of M rows each. Row r of group g
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

struct GemmParams {
  int M, N, K, groups;
  RowMap rm;
  // A operand: fp32 residual rows normalised by RMSNorm (norm mode), or fp16 hidden rows
  const float* res_in;       // norm mode source (residual addressing)
  const float* gain;         // [K] per group, stride gain_group_stride
  long gain_group_stride;
  float eps;
  const _Float16* hid_in;    // plain mode source (hidden addressing, ld = K)
  // B operand: weights [N][K] (fp16 or E4M3FN codes), per-group stride in elements
  const void* w;
  long w_group_stride;
  const float* wscale;       // E4M3 only: scale[group*5 + scale_idx0 + col/scale_col_div]
  int scale_idx0, scale_col_div;
  // epilogue: Q/K/V scatter
  int d, dh;
  __bf16* q; long q_seg_stride, q_head_stride; int q_from;
  __bf16* k; __bf16* vt; long kv_seg_stride, kv_head_stride; int kv_cap, kv_slot_base;
  // epilogue: GELU into hidden rows (ld = N)
  _Float16* hid_out;
  // epilogue: residual add (residual addressing)
  float* res_out;
};

enum GemmKind { GEMM_QKV = 0, GEMM_FFN_UP = 1, GEMM_FFN_DOWN = 2 };

hipError_t launch_gemm(GemmKind kind, bool fp8_weights, const GemmParams& p, hipStream_t s);

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
  const int* valid_from;   // [seg] first valid global position (NS: one value)
  // NS only: own keys of the candidates, kn [H][nq][dh], vtn [H][dh][nq]; P NS tokens each
  const __bf16* kn; const __bf16* vtn; long kn_head_stride; int P;
  float scale_log2;  // log2(e) / sqrt(dh)
};

hipError_t launch_attention(bool ns, int dh, const AttnParams& p, int n_seg, hipStream_t s);

// Elementwise helpers.
hipError_t launch_bf16_to_f16(const uint16_t* src, _Float16* dst, long n, hipStream_t s);
hipError_t launch_s_input(const uint16_t* tok, const int* s_lens, float* x, int* valid_from,
                          int B, int s_len, int d, hipStream_t s);
hipError_t launch_bf16_to_f32(const uint16_t* src, float* dst, long n, hipStream_t s);
hipError_t launch_copy_rows_f32(const float* src, long src_seg_stride, float* dst, long dst_seg_stride,
                                long row_elems, int n_seg, hipStream_t s);
hipError_t launch_cache_read(const __bf16* k, const __bf16* vt, int H, int dh, int cap, int rows,
                             __bf16* k_out, __bf16* v_out, hipStream_t s);

}  // namespace onetrans
