// Flash-style attention of the OneTrans block on gfx950 (bf16 MFMA, fp32 softmax).
//
// Visibility (agihunt.info OneTrans summary, "method"): an S query sees the
// valid S keys up to its own position; an NS query sees every valid S key of
// the layer plus its candidate's NS keys up to itself. Queries of a pyramid
// layer are the tail of the layer input while the keys cover all of it, so the
// causal limit is aligned bottom-right through global positions.
//
// Layout trick: the kernel computes S^T = K Q^T and O^T = V^T P^T with
// v_mfma_f32_32x32x16_bf16, so every lane owns one query (lane & 31) in all
// three of S^T, P^T and O^T. The online-softmax max and sum stay inside a lane
// pair (lane, lane ^ 32) and need one cross-lane exchange per key block; P never
// leaves registers. The cached V is stored transposed ([dh][key]) so the V^T
// operand is a plain row read.
//
// Data movement: each wave owns 32 queries; K and V^T tiles of 64 keys travel global ->
// LDS with buffer_load_dwordx4 ... lds (base in a buffer resource, so no per-lane 64-bit
// address arithmetic). Three kernels: the tile kernel (the waves of a workgroup share a
// ring of three tiles), the NS kernel (two waves per query block, each scoring one 32-key
// half of every tile of a shared ring) and the key-split kernel (waves of one query block
// take every KS-th tile through private rings, merged at the end). Tile rows are
// XOR-swizzled in 16-byte chunks so the fragment reads are bank-conflict free. The result
// is added to the fp32 residual rows (z = x + o) without rounding.
#include <math.h>

#include <type_traits>
#include "internal.h"

namespace onetrans {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int KT = 64;      // keys per tile
constexpr int STAGES = 3;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Barrier without the release fence of __syncthreads (see gemm.hip). It first waits for
// this wave's LDS reads to return (lgkmcnt 0): a ring slot is refilled by DMA right after
// the barrier, and the compiler may defer a read's wait to its MFMA, past the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int DH>
struct Softmax {
  float m = -INFINITY, l = 0.f;  // running max (raw score units) and sum of this lane's query
  f32x16 o[DH / 32];
};

// Online-softmax update with NB 32-key blocks of raw scores (masked entries -inf), the
// running max as reference. The scale 1/sqrt(dh) * log2(e) is applied inside exp2 as one
// fma. The O accumulators are rescaled only when some lane's max moved: otherwise the
// factor is exactly 1 and the multiply is skipped. Returns the bf16 probabilities packed
// as the B operands of the P.V product.
template <int DH, int NB>
__device__ __forceinline__ void softmax_update(Softmax<DH>& st, const f32x16 (&sc)[NB], bf16x8 (&pb)[NB][2],
                                               float scale) {
  float mt = vmax16(sc[0]);
#pragma unroll
  for (int b = 1; b < NB; ++b) mt = vmax(mt, vmax16(sc[b]));
  mt = max_halves(mt);
  const float m_new = fmaxf(st.m, mt);
  if (__builtin_amdgcn_ballot_w64(m_new > st.m) != 0) {
    const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((st.m - m_new) * scale);
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) st.o[db][j] *= alpha;
    st.m = m_new;
  }
  const float msub = st.m == -INFINITY ? 0.f : -st.m * scale;
  float ps = 0.f;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(sc[b][8 * c + i], scale, msub));
        ps += pv;
        pb[b][c][i] = (__bf16)pv;
      }
  st.l += ps;
}

// 32 row-major keys [t0, t0 + 32) of a K / V block (rows past n_rows - 1 are read as that
// row and masked) into the online-softmax state st of this lane's query, for the keys
// where vis(key) holds: the NS rows' own keys and the user's cached NS rows. The mask is a
// select per score. The V operand rows load after the exponentials: loaded with the K rows
// they would be held across the softmax, which raises the register count of the callers.
// Register j of the scores holds key t0 + 8*(j/4) + 4*(lane/32) + j%4 (rows in order), so
// the 8 probabilities of P.V operand c are keys t0 + 16c + 4*(lane/32) + {0..3, 8..11}.
template <int DH, class Vis>
__device__ __forceinline__ void own_key_block(Softmax<DH>& st, const bf16x8 (&qf)[DH / 16], const __bf16* knb,
                                              const __bf16* vnb, int n_rows, int t0, bool q_ok, float scale_log2,
                                              Vis vis) {
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const int krow = min(t0 + l32, n_rows - 1);
  f32x16 sk[1];
#pragma unroll
  for (int j = 0; j < 16; ++j) sk[0][j] = 0.f;
#pragma unroll
  for (int s = 0; s < DH / 16; ++s) {
    const bf16x8 a = *(const bf16x8*)(knb + (long)krow * DH + s * 16 + half * 8);
    sk[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sk[0], 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int key = t0 + 8 * (j >> 2) + half * 4 + (j & 3);
    sk[0][j] = (q_ok & vis(key)) ? sk[0][j] : -INFINITY;
  }
  bf16x8 pk[1][2];
  softmax_update<DH, 1>(st, sk, pk, scale_log2);
  bf16x8 va[2][DH / 32];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int key = min(t0 + 16 * c + half * 4 + (i & 3) + 8 * (i >> 2), n_rows - 1);
        va[c][db][i] = vnb[(long)key * DH + db * 32 + l32];
      }
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
      st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[c][db], pk[0][c], st.o[db], 0, 0, 0);
}

// Pieces of one 64-key tile against a wave's 32 queries. sb holds the tile: K rows
// (XOR-swizzled 16-byte chunks) followed by V^T rows of 64 keys (128 bytes each).
//
// Key order. The MFMA output puts S^T row 8*(j/4) + 4*(lane/32) + j%4 in register j. The
// K operand's rows are taken with bits 2 and 3 of the row index swapped (within each
// 16-key group, rows 4-7 and 8-11 trade places), so register j of block kb holds key
//   kb*32 + 16*(j/8) + 8*(lane/32) + j%8,
// and the 8 probabilities a lane packs for one P.V operand are 8 consecutive keys: the
// matching V^T operand is a single 16-byte LDS read.
__device__ __forceinline__ int key_perm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// S^T = K Q^T (raw scores)
template <int DH>
__device__ __forceinline__ void qk_tile(const char* sb, const bf16x8 (&qf)[DH / 16], f32x16 (&sc)[2]) {
  constexpr int KROW = DH * 2, KCH = KROW / 16;
  const int lane = threadIdx.x & 63, half = lane >> 5;
  const int pl = key_perm(lane & 31);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int j = 0; j < 16; ++j) sc[kb][j] = 0.f;
    const int r = kb * 32 + pl;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
      const int c = 2 * s + half;
      const int cs = KCH == 8 ? (c ^ ((r >> 1) & 7)) : (c ^ ((r >> 2) & 3));
      const bf16x8 a = *(const bf16x8*)(sb + r * KROW + cs * 16);
      sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sc[kb], 0, 0, 0);
    }
  }
}

// keys of slots outside [key_lo, my_lim) get -inf (tile starting at slot t0)
__device__ __forceinline__ void mask_tile(f32x16 (&sc)[2], int t0, int key_lo, int my_lim) {
  const int half = (threadIdx.x >> 5) & 1;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int slot = t0 + kb * 32 + 16 * (j >> 3) + 8 * half + (j & 7);
      if (slot < key_lo || slot >= my_lim) sc[kb][j] = -INFINITY;
    }
}

// One whole tile: scores, masking when a bound falls inside it, then the two 32-key halves
// in turn: the half's max against the lazy reference (moved, with a rescale of l and O,
// only when it passes the reference by more than 8 in log2 units), its exponentials and
// its P.V. Going half by half lets the second half's score MFMAs run under the first
// half's softmax and the first half's P.V under the second half's exponentials; a wave
// that has its SIMD to itself (the key-split kernel) otherwise waits for each in turn.
template <int DH>
__device__ __forceinline__ void attn_tile(const char* sb, int t0, int key_lo, int my_lim, bool edge,
                                          const bf16x8 (&qf)[DH / 16], Softmax<DH>& st, float scale) {
  constexpr int KROW = DH * 2, K_BYTES = KT * KROW;
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  f32x16 sc[2];
  qk_tile<DH>(sb, qf, sc);
  if (edge) mask_tile(sc, t0, key_lo, my_lim);
  const float tau = 8.f / scale;
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const float mt = max_halves(vmax16(sc[kb]));
    if (__builtin_amdgcn_ballot_w64(mt > st.m + tau) != 0) {
      const bool up = mt > st.m + tau;
      const float alpha = up ? __builtin_amdgcn_exp2f((st.m - mt) * scale) : 1.f;
      if (up) st.m = mt;
      st.l *= alpha;
#pragma unroll
      for (int db = 0; db < DH / 32; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) st.o[db][j] *= alpha;
    }
    const float msub = st.m == -INFINITY ? 0.f : -st.m * scale;
    bf16x8 pb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[c][i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[kb][8 * c + i], scale, msub));
    // O^T += V^T P^T over this half's keys kb*32 + 16c + 8*half + 0..7
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int db = 0; db < DH / 32; ++db) {
        const int r = db * 32 + l32;
        const int ch = 4 * kb + 2 * c + half;
        const bf16x8 a = *(const bf16x8*)(sb + K_BYTES + r * 128 + ((ch ^ ((r >> 1) & 7)) << 4));
        st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c], st.o[db], 0, 0, 0);
      }
    // the half's probability sum on the matrix core: an all-ones A operand turns every
    // output row of 1 P^T into the column sums (the same bf16 P that multiplies V). Both
    // half-waves get the full sum while l is kept as per-half partial sums that are added
    // at the end, so each half adds half of it (exact in fp32).
    f32x16 ls = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pb[0], f32x16{}, 0, 0, 0);
    ls = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pb[1], ls, 0, 0, 0);
    st.l += 0.5f * ls[0];
  }
}

// Output of query row qi, in two parts. out_row_load fetches this lane's half of head h's
// residual columns (4 consecutive columns per register group) and, with EARLY_G, the FFN
// norm's gains for them; kernels call it before streaming any key tile, so the loads
// overlap the whole key loop (and, being older than every tile load, keep the tile waits
// exact). Without EARLY_G (32 fewer registers held through the loop, for kernels whose
// occupancy they would cut) the gains load in out_row_store, before any store.
// out_row_store adds the normalised attention output, writes the residual back, then the
// norm's operand x * g and the head's partial sum of squares (deferred RMSNorm, slot h).
// Both lanes of the row's pair take part.
template <int DH>
struct OutRow {
  float4 x[DH / 32][4];
  float4 g[DH / 32][4];
};

template <int DH, bool EARLY_G>
__device__ __forceinline__ void load_gains(const AttnParams& p, int h, int qi, OutRow<DH>& r) {
  const NormOut& no = p.nout;
  if (!no.xg) return;
  const int half = (threadIdx.x >> 5) & 1;
  const float* grow = no.gain + (long)(qi % p.P) * no.gain_group_stride + h * DH + half * 4;
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) r.g[db][gi] = *(const float4*)(grow + db * 32 + 8 * gi);
}

template <int DH, bool EARLY_G>
__device__ __forceinline__ void out_row_load(const AttnParams& p, int seg, int h, int qi, OutRow<DH>& r) {
  const int half = (threadIdx.x >> 5) & 1;
  const float* rrow = p.res + seg * p.res_seg_stride + (p.res_row_base + qi) * p.res_row_stride + h * DH + half * 4;
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) r.x[db][gi] = *(const float4*)(rrow + db * 32 + 8 * gi);
  if (EARLY_G) load_gains<DH, true>(p, h, qi, r);
}

template <int DH, bool EARLY_G>
__device__ __forceinline__ void out_row_store(const AttnParams& p, int seg, int h, int qi, OutRow<DH>& r,
                                              const f32x16 (&o)[DH / 32], float inv) {
  const int half = (threadIdx.x >> 5) & 1;
  if (!EARLY_G) load_gains<DH, false>(p, h, qi, r);
  float* rrow = p.res + seg * p.res_seg_stride + (p.res_row_base + qi) * p.res_row_stride + h * DH + half * 4;
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      float4& v = r.x[db][gi];
      v.x += o[db][4 * gi + 0] * inv;
      v.y += o[db][4 * gi + 1] * inv;
      v.z += o[db][4 * gi + 2] * inv;
      v.w += o[db][4 * gi + 3] * inv;
      *(float4*)(rrow + db * 32 + 8 * gi) = v;
    }
  const NormOut& no = p.nout;
  if (!no.xg) return;
  const long hr = (long)seg * p.nq + qi;
  _Float16* xrow = no.xg + hr * p.d + h * DH + half * 4;
  float part = 0.f;
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const float4 v = r.x[db][gi], g4 = r.g[db][gi];
      part += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      const f16x4 hv = {(_Float16)(v.x * g4.x), (_Float16)(v.y * g4.y), (_Float16)(v.z * g4.z), (_Float16)(v.w * g4.w)};
      *(f16x4*)(xrow + db * 32 + 8 * gi) = hv;
    }
  part += other_half(part);
  if (half == 0) no.ss[hr * no.ss_stride + h] = part;
}

template <int DH, int NW>
__global__ __launch_bounds__(NW * 64) void attn_kernel(AttnParams p) {
  constexpr int KROW = DH * 2;                // bytes per K row (64 or 128)
  constexpr int K_BYTES = KT * KROW;
  constexpr int V_BYTES = DH * KT * 2;        // DH rows of 64 keys (128 B)
  constexpr int STAGE = K_BYTES + V_BYTES;
  constexpr int K_INSTR = K_BYTES / 1024 / NW;  // DMA instructions per wave and tile
  constexpr int V_INSTR = V_BYTES / 1024 / NW;
  static_assert(K_INSTR >= 1 && V_INSTR >= 1 && K_BYTES % (1024 * NW) == 0 && V_BYTES % (1024 * NW) == 0, "tile split");
  constexpr int PER_TILE = K_INSTR + V_INSTR;
  constexpr int KCH = KROW / 16;              // 16-byte chunks per K row
  constexpr int KRPI = 64 / KCH;              // K rows per wave instruction
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];

  // the wave index is uniform: kept in a scalar register, so per-wave LDS addresses are too
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int h = blockIdx.y, seg = blockIdx.z;
  const int wq0 = blockIdx.x * (NW * 32) + wave * 32;
  const int qi = wq0 + l32;
  const bool q_ok = qi < p.nq;
  const bool wave_live = wq0 < p.nq;

  // Q^T operand: lane holds Q[qi][s*16 + half*8 + 0..7]
  bf16x8 qf[DH / 16];
  {
    const __bf16* qrow = p.q + seg * p.q_seg_stride + h * p.q_head_stride + (long)(q_ok ? qi : 0) * DH;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
      bf16x8 v = *(const bf16x8*)(qrow + s * 16 + half * 8);
      if (!q_ok) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (__bf16)0.f;
      }
      qf[s] = v;
    }
  }

  const int vf = p.valid_from[seg];
  const int key_lo = max(0, vf - p.key_pos0);
  int key_hi = p.n_keys;   // exclusive slot bound of the tiles this workgroup loads
  int my_lim = p.n_keys;   // exclusive slot bound of this lane's query
  int wave_lim = p.n_keys; // exclusive slot bound of this wave's queries
  int wave_lim_lo = p.n_keys;  // smallest bound among them: tiles below it need no upper mask
  {
    const int qlast_blk = min((int)blockIdx.x * (NW * 32) + NW * 32 - 1, p.nq - 1);
    const int qlast_wave = min(wq0 + 31, p.nq - 1);
    key_hi = min(key_hi, p.q_pos0 + qlast_blk - p.key_pos0 + 1);
    wave_lim = min(wave_lim, p.q_pos0 + qlast_wave - p.key_pos0 + 1);
    wave_lim_lo = min(wave_lim_lo, p.q_pos0 + wq0 - p.key_pos0 + 1);
    my_lim = min(my_lim, p.q_pos0 + qi - p.key_pos0 + 1);
  }
  if (!q_ok) my_lim = 0;
  if (wq0 + 31 >= p.nq) wave_lim_lo = 0;  // a partial wave: some lanes see no keys

  Softmax<DH> st;
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) st.o[db][j] = 0.f;

  // ---- per-lane sources of the tile DMA (slots beyond the filled length hold zeros) ----
  // K [cap][dh] and V^T [dh][cap] of this (segment, head) as buffer resources
  const __amdgpu_buffer_rsrc_t krs =
      buffer_rsrc(p.k + seg * p.kv_seg_stride + h * p.kv_head_stride, (uint32_t)p.kv_cap * KROW);
  const __amdgpu_buffer_rsrc_t vrs =
      buffer_rsrc(p.vt + seg * p.kv_seg_stride + h * p.kv_head_stride, (uint32_t)p.kv_cap * DH * 2);
  uint32_t k_off[K_INSTR], v_off[V_INSTR];  // per-lane byte offsets from the uniform tile base
#pragma unroll
  for (int i = 0; i < K_INSTR; ++i) {
    const int r = (wave * K_INSTR + i) * KRPI + lane / KCH;
    const int c = lane % KCH;
    const int cs = KCH == 8 ? (c ^ ((r >> 1) & 7)) : (c ^ ((r >> 2) & 3));
    k_off[i] = (uint32_t)(r * KROW + cs * 16);
  }
#pragma unroll
  for (int i = 0; i < V_INSTR; ++i) {
    const int r = (wave * V_INSTR + i) * 8 + (lane >> 3);   // dh row
    v_off[i] = (uint32_t)r * (uint32_t)p.kv_cap * 2u + ((((lane & 7) ^ ((r >> 1) & 7))) << 4);
  }
  auto issue = [&](int t0, int stage) {
    char* sb = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < K_INSTR; ++i)
      dma16_buf(krs, k_off[i], (uint32_t)t0 * KROW, (lds_void*)(sb + (wave * K_INSTR + i) * 1024));
#pragma unroll
    for (int i = 0; i < V_INSTR; ++i)
      dma16_buf(vrs, v_off[i], (uint32_t)t0 * 2, (lds_void*)(sb + K_BYTES + (wave * V_INSTR + i) * 1024));
  };

  constexpr bool EARLY_G = NW <= 2;
  OutRow<DH> orow;
  if (q_ok) out_row_load<DH, EARLY_G>(p, seg, h, qi, orow);

  const int t_first = (key_lo / KT) * KT;
  const int ntiles = key_hi > t_first ? (key_hi - t_first + KT - 1) / KT : 0;
  // The first STAGES - 1 tiles issue whatever ntiles is (past the cached keys they read
  // zeros into slots the loop never reads): with a fixed count the compiler waits for the
  // query loads above without waiting for this burst. The waits below count them, and the
  // one after the loop keeps a wave from ending while a DMA still writes this LDS.
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) issue(t_first + s * KT, s);

#pragma unroll 1
  for (int it = 0; it < ntiles; ++it) {
    if (it + 1 < ntiles) wait_vmcnt<PER_TILE>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (it + STAGES - 1 < ntiles) issue(t_first + (it + STAGES - 1) * KT, (it + STAGES - 1) % STAGES);
    const int t0 = t_first + it * KT;
    if (wave_live && t0 < wave_lim) {
      attn_tile<DH>(smem + (it % STAGES) * STAGE, t0, key_lo, my_lim, t0 < key_lo || t0 + KT > wave_lim_lo, qf, st,
                    p.scale_log2);
    }
  }
  wait_vmcnt<0>();

  const float l_tot = st.l + __shfl_xor(st.l, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_ok) out_row_store<DH, EARLY_G>(p, seg, h, qi, orow, st.o, inv);
}

// NS queries with every 64-key tile split between two waves: wave pair (2b, 2b + 1) holds
// query block b, and wave 2b + kh scores keys kh*32 .. kh*32 + 31 of each tile. Every NS
// lane sees the same cached-key range [key_lo, n_keys), so all waves walk the same tiles
// of one shared stream; splitting the keys doubles the waves per SIMD, which hides the
// latencies of the per-tile chain (LDS read, MFMA, max exchange, exponentials, P.V).
// After the last tile the halves' (max, sum, O) merge through LDS; the key-half-0 wave
// adds the candidate's own NS keys first and writes the result. Each tile's scores are
// issued to the matrix core one iteration ahead, so the exponentials of a tile run while
// the next tile's S^T is being computed.
template <int DH, int NB>
__global__ __launch_bounds__(NB * 128) void attn_ns2_kernel(AttnParams p) {
  constexpr int NW = 2 * NB;                  // waves per workgroup
  constexpr int KROW = DH * 2;
  constexpr int K_BYTES = KT * KROW;
  constexpr int V_BYTES = DH * KT * 2;
  constexpr int STAGE = K_BYTES + V_BYTES;
  constexpr int K_INSTR = K_BYTES / 1024 / NW;  // DMA instructions per wave and tile
  constexpr int V_INSTR = V_BYTES / 1024 / NW;
  static_assert(K_INSTR >= 1 && V_INSTR >= 1 && K_BYTES % (1024 * NW) == 0 && V_BYTES % (1024 * NW) == 0, "tile split");
  constexpr int PER_TILE = K_INSTR + V_INSTR;
  constexpr int KCH = KROW / 16;
  constexpr int KRPI = 64 / KCH;
  constexpr int MERGE = 64 * (2 + 16 * (DH / 32)) * 4;  // one wave's m, l and O for 64 lanes
  static_assert(NB * MERGE <= STAGES * STAGE, "merge area");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int qb = wave >> 1, kh = wave & 1;
  const int h = blockIdx.y, seg = blockIdx.z;
  const int wq0 = blockIdx.x * (NB * 32) + qb * 32;
  const int qi = wq0 + l32;
  const bool q_ok = qi < p.nq;
  const bool wave_live = wq0 < p.nq;

  bf16x8 qf[DH / 16];
  {
    const __bf16* qrow = p.q + seg * p.q_seg_stride + h * p.q_head_stride + (long)(q_ok ? qi : 0) * DH;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
      bf16x8 v = *(const bf16x8*)(qrow + s * 16 + half * 8);
      if (!q_ok) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (__bf16)0.f;
      }
      qf[s] = v;
    }
  }
  const int key_lo = max(0, p.valid_from[seg] - p.key_pos0);
  const int n_keys = p.n_keys;
  const int my_lim = q_ok ? n_keys : 0;
  const int full_lim = wq0 + 31 < p.nq ? n_keys : 0;  // tiles ending at or below it need no mask

  Softmax<DH> st;
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) st.o[db][j] = 0.f;

  // ---- per-lane sources of the tile DMA (slots beyond the filled length hold zeros) ----
  // K [cap][dh] and V^T [dh][cap] of this (segment, head) as buffer resources
  const __amdgpu_buffer_rsrc_t krs =
      buffer_rsrc(p.k + seg * p.kv_seg_stride + h * p.kv_head_stride, (uint32_t)p.kv_cap * KROW);
  const __amdgpu_buffer_rsrc_t vrs =
      buffer_rsrc(p.vt + seg * p.kv_seg_stride + h * p.kv_head_stride, (uint32_t)p.kv_cap * DH * 2);
  uint32_t k_off[K_INSTR], v_off[V_INSTR];
#pragma unroll
  for (int i = 0; i < K_INSTR; ++i) {
    const int r = (wave * K_INSTR + i) * KRPI + lane / KCH;
    const int c = lane % KCH;
    const int cs = KCH == 8 ? (c ^ ((r >> 1) & 7)) : (c ^ ((r >> 2) & 3));
    k_off[i] = (uint32_t)(r * KROW + cs * 16);
  }
#pragma unroll
  for (int i = 0; i < V_INSTR; ++i) {
    const int r = (wave * V_INSTR + i) * 8 + (lane >> 3);   // dh row
    v_off[i] = (uint32_t)r * (uint32_t)p.kv_cap * 2u + ((((lane & 7) ^ ((r >> 1) & 7))) << 4);
  }
  const int t_first = (key_lo / KT) * KT;
  const int ntiles = n_keys > t_first ? (n_keys - t_first + KT - 1) / KT : 0;

  // K and V^T of a tile travel in rings of their own: iteration it reads K of tile it + 1
  // (whose scores go to the matrix core first, so that tile it's softmax runs under them)
  // and V^T of tile it. Issue order: K(0); K(1), V(0); K(2), V(1); then iteration it
  // issues K(it + 3) and V(it + 2) into the slots that iteration it - 1 finished reading.
  // Tile j lives in slot j % 3 of both rings; the loop is unrolled three times so that
  // every slot offset is a compile-time constant.
  static_assert(STAGES == 3, "ring of three slots");
  char* const kring = smem;
  char* const vring = smem + STAGES * K_BYTES;
  auto issue_k = [&](int j, int slot) {
    char* sb = kring + slot * K_BYTES;
#pragma unroll
    for (int i = 0; i < K_INSTR; ++i)
      dma16_buf(krs, k_off[i], (uint32_t)(t_first + j * KT) * KROW, (lds_void*)(sb + (wave * K_INSTR + i) * 1024));
  };
  auto issue_v = [&](int j, int slot) {
    char* sb = vring + slot * V_BYTES;
#pragma unroll
    for (int i = 0; i < V_INSTR; ++i)
      dma16_buf(vrs, v_off[i], (uint32_t)(t_first + j * KT) * 2, (lds_void*)(sb + (wave * V_INSTR + i) * 1024));
  };
  // per-lane parts of the fragment addresses (the slot adds a constant)
  const int pl = key_perm(l32);  // score row order: see qk_tile
  uint32_t k_frag[DH / 16], v_frag[2][DH / 32];
  {
    const int r = kh * 32 + pl;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
      const int c = 2 * s + half;
      const int cs = KCH == 8 ? (c ^ ((r >> 1) & 7)) : (c ^ ((r >> 2) & 3));
      k_frag[s] = (uint32_t)(r * KROW + cs * 16);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int db = 0; db < DH / 32; ++db) {
        const int rv = db * 32 + l32;
        const int ch = 4 * kh + 2 * c + half;
        v_frag[c][db] = (uint32_t)(rv * 128 + ((ch ^ ((rv >> 1) & 7)) << 4));
      }
  }
  // raw scores S^T of this wave's 32 keys of the tile in K slot `slot`
  auto scores = [&](int slot, f32x16& sc) {
    const char* sb = kring + slot * K_BYTES;
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = 0.f;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s)
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(sb + k_frag[s]), qf[s], sc, 0, 0, 0);
  };
  // The first five issue whatever ntiles is: a tile past the cached keys reads zeros
  // (buffer bounds) into ring slots the key loop never reads, and a fixed count lets the
  // compiler wait for the query loads above without waiting for this burst (behind a
  // conditional issue it cannot count the loads in flight and waits for all of them).
  // Every wait below counts these five, so a shorter walk only waits for more of them.
  issue_k(0, 0);
  issue_k(1, 1);
  issue_v(0, 0);
  issue_k(2, 2);
  issue_v(1, 1);

  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};
  // Lazy rescaling: the reference max st.m only moves when a tile's max exceeds it by more
  // than 8 in log2 units (probabilities then stay below 2^8, far inside fp32 and bf16 range;
  // any reference gives the same normalised result), which on typical scores leaves the
  // rescale of O to the first tile.
  const float scale = p.scale_log2;
  const float tau = 8.f / scale;
  // per-lane loop state derived from st.m, recomputed only when it moves: the exponent
  // offset -m * scale (0 while no key was seen) and the threshold m + tau
  float msub = 0.f, thr = -INFINITY;
  auto tile_max = [&](const f32x16& v) { return max_halves(vmax16(v)); };
  // move the reference of the lanes whose tile max passed the threshold (call under a
  // wave-uniform branch) and rescale their running sum and O
  auto raise_ref = [&](float mt) {
    const bool up = mt > thr;
    const float alpha = up ? __builtin_amdgcn_exp2f((st.m - mt) * scale) : 1.f;
    if (up) {
      st.m = mt;
      msub = -mt * scale;
      thr = mt + tau;
    }
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) st.o[db][j] *= alpha;
  };
  f32x16 sc;
  if (ntiles > 0) {
    // only K(0) is needed here: leave K(1), V(0), K(2), V(1) in flight
    wait_vmcnt<2 * PER_TILE>();
    lds_barrier();
    scores(0, sc);
  }
  // iteration it with tile it in slot S0 (= it % 3)
  auto step = [&](auto S0C, int it) __attribute__((always_inline)) {
    constexpr int S0 = decltype(S0C)::value, S1 = (S0 + 1) % 3, S2 = (S0 + 2) % 3;
    if (it + 2 < ntiles) wait_vmcnt<PER_TILE>();  // K(it + 1) and V(it) are in
    else if (it + 1 < ntiles) wait_vmcnt<V_INSTR>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (it + 3 < ntiles) issue_k(it + 3, S0);
    if (it + 2 < ntiles) issue_v(it + 2, S2);
    // next tile's scores first (after the last tile this reads a slot nobody writes any
    // more; the result is unused)
    f32x16 sn;
    scores(S1, sn);
    __builtin_amdgcn_sched_barrier(0);
    const int t0 = t_first + it * KT;
    if (t0 < key_lo || t0 + KT > full_lim) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int slot = t0 + kh * 32 + 16 * (j >> 3) + 8 * half + (j & 7);
        if (slot < key_lo || slot >= my_lim) sc[j] = -INFINITY;
      }
    }
    const float mt = tile_max(sc);
    if (__builtin_amdgcn_ballot_w64(mt > thr) != 0) raise_ref(mt);
    bf16x8 pb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[c][i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[8 * c + i], scale, msub));
    const char* vb = vring + S0 * V_BYTES;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int db = 0; db < DH / 32; ++db)
        st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vb + v_frag[c][db]), pb[c], st.o[db], 0, 0, 0);
    // this half's sum of the same bf16 probabilities that multiply V
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x2 pr = {pb[c][2 * i], pb[c][2 * i + 1]};
        st.l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, st.l, false);
      }
    sc = sn;
  };
  // Steady-state iteration: both DMAs issue, no key of the tile is masked. In-order issue
  // would stall on each of the four dependent score MFMAs of the next tile, so they are
  // interleaved with this tile's exponentials, and every fragment read of the iteration
  // is issued up front. The exponentials use the current reference max; the rare tile
  // that moves it recomputes them after the rescale.
  auto step_fast = [&](auto S0C, int it) __attribute__((always_inline)) {
    constexpr int S0 = decltype(S0C)::value, S1 = (S0 + 1) % 3, S2 = (S0 + 2) % 3;
    wait_vmcnt<PER_TILE>();  // K(it + 1) and V(it) are in
    lds_barrier();
    issue_k(it + 3, S0);
    issue_v(it + 2, S2);
    const char* kb = kring + S1 * K_BYTES;
    const char* vb = vring + S0 * V_BYTES;
    bf16x8 kf[DH / 16], vf[2 * (DH / 32)];
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) kf[s] = *(const bf16x8*)(kb + k_frag[s]);
    const float mt = tile_max(sc);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 sn;
#pragma unroll
    for (int i = 0; i < 16; ++i) sn[i] = 0.f;
    bf16x8 pb[2];
    constexpr int EPM = 16 / (DH / 16);  // exponentials per score MFMA
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
      sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], sn, 0, 0, 0);
#pragma unroll
      for (int e = s * EPM; e < (s + 1) * EPM; ++e) pb[e / 8][e % 8] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[e], scale, msub));
      // the V^T fragments of this tile, one per score MFMA (the K fragment just consumed
      // frees its registers)
      if (s < 2 * (DH / 32)) vf[s] = *(const bf16x8*)(vb + v_frag[s / (DH / 32)][s % (DH / 32)]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // keep the exponentials here, under the score MFMAs (the compiler would otherwise sink
    // them past the branch below)
    asm volatile("" : "+v"(pb[0]), "+v"(pb[1]));
    if (__builtin_amdgcn_ballot_w64(mt > thr) != 0) {
      raise_ref(mt);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[c][i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[8 * c + i], scale, msub));
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int db = 0; db < DH / 32; ++db)
        st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[c * (DH / 32) + db], pb[c], st.o[db], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x2 pr = {pb[c][2 * i], pb[c][2 * i + 1]};
        st.l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, st.l, false);
      }
    sc = sn;
  };
  // a group of three iterations from `it` (a multiple of 3) may take the steady-state form
  // when every query of the wave is valid, the first tile needs no padding mask and the
  // group ends at least three tiles before the last (so every DMA issues and the last,
  // possibly partial, tile is not in it)
  const bool all_q = full_lim == n_keys;
  const int it_fast = key_lo > t_first ? 1 : 0;
  // (separate loops: one loop holding both forms needs about 35 more registers)
  auto group = [&](int it) __attribute__((always_inline)) {
    step(std::integral_constant<int, 0>{}, it);
    step(std::integral_constant<int, 1>{}, it + 1);
    step(std::integral_constant<int, 2>{}, it + 2);
  };
  int it = 0;
#pragma unroll 1
  for (; it + 3 <= ntiles && !(all_q && it >= it_fast && it + 5 < ntiles); it += 3) group(it);
#pragma unroll 1
  for (; all_q && it + 5 < ntiles; it += 3) {
    step_fast(std::integral_constant<int, 0>{}, it);
    step_fast(std::integral_constant<int, 1>{}, it + 1);
    step_fast(std::integral_constant<int, 2>{}, it + 2);
  }
#pragma unroll 1
  for (; it + 3 <= ntiles; it += 3) group(it);
  if (it < ntiles) step(std::integral_constant<int, 0>{}, it);
  if (it + 1 < ntiles) step(std::integral_constant<int, 1>{}, it + 1);

  // the output row's residual and gains, loaded under the own-key phase and the merge
  OutRow<DH> orow;
  if (kh == 0 && q_ok) out_row_load<DH, false>(p, seg, h, qi, orow);
  if (kh == 0 && wave_live) {
    auto key_block = [&](const __bf16* knb, const __bf16* vnb, int n_rows, int t0, auto vis) {
      own_key_block<DH>(st, qf, knb, vnb, n_rows, t0, q_ok, p.scale_log2, vis);
    };
    // the user's cached NS rows: earlier NS positions, seen in full by every query
    if (p.n_x > 0) {
      const __bf16* xkb = p.xk + h * p.x_head_stride;
      const __bf16* xvb = p.xv + h * p.x_head_stride;
      const int n_x = p.n_x;
#pragma unroll 1
      for (int t0 = 0; t0 < n_x; t0 += 32) key_block(xkb, xvb, n_x, t0, [&](int key) { return key < n_x; });
    }
    // the candidate's own NS keys: query g = c*P + k sees g' in [c*P, g];
    // NS K and V are row-major [H][nq][dh]
    const int P = p.P;
    const int g_lo = (wq0 / P) * P;
    const int g_hi = min(wq0 + 31, p.nq - 1);
    const int my_first = (qi / P) * P;
#pragma unroll 1
    for (int t0 = g_lo; t0 <= g_hi; t0 += 32)
      key_block(p.kn + seg * p.kn_seg_stride + h * p.kn_head_stride, p.vn + seg * p.kn_seg_stride + h * p.kn_head_stride,
                p.nq, t0, [&](int key) { return (key <= qi) & (key >= my_first); });
  }

  // ---- merge the two key halves of each query block (LDS of the tile ring is free) ----
  const float l_half = st.l + __shfl_xor(st.l, 32);
  // no DMA of this wave is still writing the ring (with no cached key to walk, the first
  // five were never waited for) and every wave is past its last tile read
  wait_vmcnt<0>();
  __syncthreads();
  float* mw = (float*)(smem + qb * MERGE);
  if (kh == 1) {
    mw[lane] = st.m;
    mw[64 + lane] = l_half;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) mw[128 + (db * 16 + j) * 64 + lane] = st.o[db][j];
  }
  __syncthreads();
  if (kh == 1 || !q_ok) return;
  const float m1 = mw[lane], l1 = mw[64 + lane];
  const float m = fmaxf(st.m, m1);
  const float f0 = st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((st.m - m) * p.scale_log2);
  const float f1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m1 - m) * p.scale_log2);
  const float l_tot = l_half * f0 + l1 * f1;
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) st.o[db][j] = st.o[db][j] * f0 + mw[128 + (db * 16 + j) * 64 + lane] * f1;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  out_row_store<DH, false>(p, seg, h, qi, orow, st.o, inv);
}

// Attention with the keys of one 32-query block split over KS waves: wave w takes key
// tiles w, w + KS, ... through a private 2-stage LDS ring (no barriers while streaming),
// and the partial (max, sum, O) of the waves merge through LDS at the end. Used when there
// are few query blocks and long key ranges, where a plain kernel's critical path is one
// wave walking every key tile: S queries of one user's prefill or of appends (causal
// limits), and with NS the few NS queries of the user-side pass (every cached key
// [key_lo, n_keys) visible; after the merge, wave 0 adds the user's cached NS rows and
// the block's own NS keys as attn_ns2_kernel does).
template <int DH, int KS, bool GROUPED, bool NS>
__global__ __launch_bounds__(KS * 64) void attn_split_kernel(AttnParams p) {
  constexpr int KROW = DH * 2;
  constexpr int K_BYTES = KT * KROW;
  constexpr int V_BYTES = DH * KT * 2;
  constexpr int STAGE = K_BYTES + V_BYTES;
  constexpr int K_INSTR = K_BYTES / 1024, V_INSTR = V_BYTES / 1024;  // per tile, one wave
  constexpr int PER_TILE = K_INSTR + V_INSTR;
  constexpr int KCH = KROW / 16, KRPI = 64 / KCH;
  constexpr int MERGE = 64 * (2 + 16 * (DH / 32)) * 4;  // per wave: m, l and O of 64 lanes
  constexpr int SMEM = KS * 2 * STAGE > KS * MERGE ? KS * 2 * STAGE : KS * MERGE;
  static_assert(K_BYTES % 1024 == 0 && V_BYTES % 1024 == 0, "tile split");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  // the wave index as a wave-uniform value: the tile offsets and ring addresses derived
  // from it go to the buffer DMA's scalar operands (a per-lane value there makes the
  // compiler loop over its distinct values around every DMA instruction)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  // (query block, head, segment). GROUPED: a 1-D grid numbered so that each XCD holds a
  // contiguous range of them (the hardware deals workgroup L to XCD L % 8): the query
  // blocks of one (segment, head) are neighbours, run on one XCD at the same time and share
  // its L2 copy of that head's K/V stream instead of fetching it once per block.
  int bx, h, seg;
  if constexpr (GROUPED) {
    const int n_blk = (p.nq + 31) / 32;
    const int total = gridDim.x, L = blockIdx.x;
    const int x = L % 8, pos = x * (total / 8) + min(x, total % 8) + L / 8;
    bx = pos % n_blk;
    h = (pos / n_blk) % p.H;
    seg = pos / (n_blk * p.H);
  } else {
    bx = blockIdx.x;
    h = blockIdx.y;
    seg = blockIdx.z;
  }
  const int wq0 = bx * 32;
  const int qi = wq0 + l32;
  const bool q_ok = qi < p.nq;

  const int vf = p.valid_from[seg];
  const int key_lo = max(0, vf - p.key_pos0);
  const int qlast = min(wq0 + 31, p.nq - 1);
  // exclusive end of this block's keys, the end below which a tile needs no mask, this
  // lane's end: causal for S queries, every cached key for NS queries
  const int key_hi = NS ? p.n_keys : min(p.n_keys, p.q_pos0 + qlast - p.key_pos0 + 1);
  const int lim_lo = wq0 + 31 < p.nq ? (NS ? p.n_keys : min(p.n_keys, p.q_pos0 + wq0 - p.key_pos0 + 1)) : 0;
  const int my_lim = q_ok ? (NS ? p.n_keys : min(p.n_keys, p.q_pos0 + qi - p.key_pos0 + 1)) : 0;

  Softmax<DH> st;
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) st.o[db][j] = 0.f;

  const int t_first = (key_lo / KT) * KT;
  const int ntiles = key_hi > t_first ? (key_hi - t_first + KT - 1) / KT : 0;
  const int n_my = wave < ntiles ? (ntiles - wave + KS - 1) / KS : 0;
  const __amdgpu_buffer_rsrc_t krs =
      buffer_rsrc(p.k + seg * p.kv_seg_stride + h * p.kv_head_stride, (uint32_t)p.kv_cap * KROW);
  const __amdgpu_buffer_rsrc_t vrs =
      buffer_rsrc(p.vt + seg * p.kv_seg_stride + h * p.kv_head_stride, (uint32_t)p.kv_cap * DH * 2);
  char* ring = smem + wave * 2 * STAGE;
  auto issue = [&](int j) {
    const int t0 = t_first + (wave + j * KS) * KT;
    char* sb = ring + (j & 1) * STAGE;
#pragma unroll
    for (int i = 0; i < K_INSTR; ++i) {
      const int r = i * KRPI + lane / KCH, c = lane % KCH;
      const int cs = KCH == 8 ? (c ^ ((r >> 1) & 7)) : (c ^ ((r >> 2) & 3));
      dma16_buf(krs, (uint32_t)(r * KROW + cs * 16), (uint32_t)t0 * KROW, (lds_void*)(sb + i * 1024));
    }
#pragma unroll
    for (int i = 0; i < V_INSTR; ++i) {
      const int r = i * 8 + (lane >> 3);  // dh row
      dma16_buf(vrs, (uint32_t)r * (uint32_t)p.kv_cap * 2u + ((((lane & 7) ^ ((r >> 1) & 7))) << 4),
                (uint32_t)t0 * 2, (lds_void*)(sb + K_BYTES + i * 1024));
    }
  };
  // The first tile issues before the query and output-row loads, and whatever n_my is (a
  // wave with no tile reads zeros or unused keys into its own ring, waited for before the
  // merge reuses the LDS): behind loads still in flight, or a conditional issue, the
  // compiler made it wait for all of them first.
  issue(0);
  bf16x8 qf[DH / 16];
  {
    const __bf16* qrow = p.q + seg * p.q_seg_stride + h * p.q_head_stride + (long)(q_ok ? qi : 0) * DH;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
      bf16x8 v = *(const bf16x8*)(qrow + s * 16 + half * 8);
      if (!q_ok) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (__bf16)0.f;
      }
      qf[s] = v;
    }
  }
  OutRow<DH> orow;  // wave 0 writes the merged rows
  if (wave == 0 && q_ok) out_row_load<DH, true>(p, seg, h, qi, orow);
#pragma unroll 1
  for (int j = 0; j < n_my; ++j) {
    if (j + 1 < n_my) {
      issue(j + 1);
      wait_vmcnt<PER_TILE>();
    } else {
      wait_vmcnt<0>();
    }
    const int t0 = t_first + (wave + j * KS) * KT;
    attn_tile<DH>(ring + (j & 1) * STAGE, t0, key_lo, my_lim, t0 < key_lo || t0 + KT > lim_lo, qf, st,
                  p.scale_log2);
  }

  // ---- merge: every wave's lane l holds the same query and O layout ----
  wait_vmcnt<0>();  // a wave without tiles has not waited for its first DMA yet
  __syncthreads();  // all rings are done; reuse the LDS for the partial results
  float* mw = (float*)(smem + wave * MERGE);
  mw[lane] = st.m;
  mw[64 + lane] = st.l + __shfl_xor(st.l, 32);
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) mw[128 + (db * 16 + j) * 64 + lane] = st.o[db][j];
  __syncthreads();
  if (wave != 0) return;
  float m_all = -INFINITY;
#pragma unroll
  for (int w = 0; w < KS; ++w) m_all = fmaxf(m_all, ((const float*)(smem + w * MERGE))[lane]);
  float l_all = 0.f;
  f32x16 o[DH / 32];
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[db][j] = 0.f;
#pragma unroll
  for (int w = 0; w < KS; ++w) {
    const float* src = (const float*)(smem + w * MERGE);
    const float mwv = src[lane];
    const float f = mwv == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mwv - m_all) * p.scale_log2);
    l_all += src[64 + lane] * f;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[db][j] += src[128 + (db * 16 + j) * 64 + lane] * f;
  }
  if constexpr (NS) {
    // the merged state continues (l kept as per-half partial sums again: each half-wave
    // holds half of the full sum, exact in fp32) through the user's cached NS rows and the
    // block's own NS keys, 32 row-major keys [t0, t0 + 32) at a time (rows past n_rows - 1
    // are read as that row and masked), visible to this lane when vis(key) holds
    Softmax<DH> st2;
    st2.m = m_all;
    st2.l = 0.5f * l_all;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db) st2.o[db] = o[db];
    auto key_block = [&](const __bf16* knb, const __bf16* vnb, int n_rows, int t0, auto vis) {
      own_key_block<DH>(st2, qf, knb, vnb, n_rows, t0, q_ok, p.scale_log2, vis);
    };
    if (p.n_x > 0) {
      const __bf16* xkb = p.xk + h * p.x_head_stride;
      const __bf16* xvb = p.xv + h * p.x_head_stride;
      const int n_x = p.n_x;
#pragma unroll 1
      for (int t0 = 0; t0 < n_x; t0 += 32) key_block(xkb, xvb, n_x, t0, [&](int key) { return key < n_x; });
    }
    // query g = c*P + k sees own keys g' in [c*P, g]; NS K and V are row-major [H][nq][dh]
    const int P = p.P;
    const int g_lo = (wq0 / P) * P;
    const int g_hi = min(wq0 + 31, p.nq - 1);
    const int my_first = (qi / P) * P;
#pragma unroll 1
    for (int t0 = g_lo; t0 <= g_hi; t0 += 32)
      key_block(p.kn + seg * p.kn_seg_stride + h * p.kn_head_stride, p.vn + seg * p.kn_seg_stride + h * p.kn_head_stride,
                p.nq, t0, [&](int key) { return (key <= qi) & (key >= my_first); });
    l_all = st2.l + __shfl_xor(st2.l, 32);
#pragma unroll
    for (int db = 0; db < DH / 32; ++db) o[db] = st2.o[db];
  }
  if (!q_ok) return;
  const float inv = l_all > 0.f ? 1.f / l_all : 0.f;
  out_row_store<DH, true>(p, seg, h, qi, orow, o, inv);
}

// Zero the K rows and V^T columns [from, cap) of every (user, head) block of every layer
// (blockIdx.z), so that key tiles reaching past the filled length read finite values.
__global__ void cache_clear_tail_kernel(ClearTailParams p) {
  const int l = blockIdx.z, b = blockIdx.y;
  const int cap = p.cap[l], from = p.from[l], dh = p.dh;
  const int n = cap - from;
  __bf16* kb = p.k[l] + (long)b * cap * dh;
  __bf16* vb = p.vt[l] + (long)b * dh * cap;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n * dh; i += gridDim.x * blockDim.x) {
    kb[(long)from * dh + i] = (__bf16)0.f;
    const int r = i / n, c = i - r * n;
    vb[(long)r * cap + from + c] = (__bf16)0.f;
  }
}

}  // namespace

template <int DH, int NB>
void launch_attn_ns2(const AttnParams& p, int n_seg, hipStream_t s) {
  dim3 grid((p.nq + NB * 32 - 1) / (NB * 32), p.H, n_seg);
  hipLaunchKernelGGL((attn_ns2_kernel<DH, NB>), grid, dim3(NB * 128), 0, s, p);
}

template <int DH, int NW>
void launch_attn_nw(const AttnParams& p, int n_seg, hipStream_t s) {
  dim3 grid((p.nq + NW * 32 - 1) / (NW * 32), p.H, n_seg);
  hipLaunchKernelGGL((attn_kernel<DH, NW>), grid, dim3(NW * 64), 0, s, p);
}

// Which kernel instance runs a launch: 32 queries per wave, a workgroup's waves share the
// K/V tiles. NS: each tile's keys split over two waves per query block, 2 query blocks (4
// waves) per workgroup when there are blocks for 512 such workgroups, else 1; with at most
// 256 blocks (the user-side pass, a handful of candidates) the key tiles split over five
// waves per block as for S queries, so that one block's walk is not the launch. S: with few
// query blocks (one user's prefill, appends) each block's keys are split over five waves
// (head dim 64: their double-buffered tile rings fill the 160 KB of LDS; four for head dim
// 32), the blocks of one (user, head) grouped on one XCD when there are several users, except
// for several users with 2-4 blocks each (appends), whose key-split workgroups would hold a
// CU each with five waves: there two blocks share a tile-kernel workgroup (three per CU).
// With many (a batch of users' prefill) 4 or 2 query blocks share a workgroup's key stream.
// The K/V of a layer is L2-resident, so streaming it to more workgroups is cheap.
AttnRoute attention_route(bool ns, int dh, int nq, int H, int n_seg) {
  const long blocks32 = (long)((nq + 31) / 32) * H * n_seg;
  const bool d64 = dh == 64;
  if (ns) {
    // few NS query blocks (the user-side pass, a handful of candidates): keys split over waves
    if (blocks32 <= 256) {
      if (n_seg > 1) return d64 ? ATTN_NSSPLIT_64_GROUPED : ATTN_NSSPLIT_32_GROUPED;
      return d64 ? ATTN_NSSPLIT_64 : ATTN_NSSPLIT_32;
    }
    if (blocks32 >= 2L * 512) return d64 ? ATTN_NS2_64_2 : ATTN_NS2_32_2;
    return d64 ? ATTN_NS2_64_1 : ATTN_NS2_32_1;
  }
  if (blocks32 < 2L * 512) {
    // several users with 2-4 query blocks each (appends): two blocks share a workgroup's
    // key stream, three such workgroups per CU
    if (n_seg > 1 && nq > 32 && nq <= 128) return d64 ? ATTN_TILE_64_2 : ATTN_TILE_32_2;
    if (n_seg > 1) return d64 ? ATTN_SPLIT_64_GROUPED : ATTN_SPLIT_32_GROUPED;
    return d64 ? ATTN_SPLIT_64 : ATTN_SPLIT_32;
  }
  if (blocks32 >= 4L * 512) return d64 ? ATTN_TILE_64_4 : ATTN_TILE_32_4;
  return d64 ? ATTN_TILE_64_2 : ATTN_TILE_32_2;  // 1024 <= blocks32 < 2048
}

const char* attention_route_name(AttnRoute r) {
  switch (r) {
    case ATTN_NS2_64_2: return "attn_ns2_kernel<64,2>";
    case ATTN_NS2_64_1: return "attn_ns2_kernel<64,1>";
    case ATTN_NS2_32_2: return "attn_ns2_kernel<32,2>";
    case ATTN_NS2_32_1: return "attn_ns2_kernel<32,1>";
    case ATTN_NSSPLIT_64_GROUPED: return "attn_split_kernel<64,5,true,ns>";
    case ATTN_NSSPLIT_32_GROUPED: return "attn_split_kernel<32,4,true,ns>";
    case ATTN_NSSPLIT_64: return "attn_split_kernel<64,5,false,ns>";
    case ATTN_NSSPLIT_32: return "attn_split_kernel<32,4,false,ns>";
    case ATTN_SPLIT_64_GROUPED: return "attn_split_kernel<64,5,true>";
    case ATTN_SPLIT_32_GROUPED: return "attn_split_kernel<32,4,true>";
    case ATTN_SPLIT_64: return "attn_split_kernel<64,5,false>";
    case ATTN_SPLIT_32: return "attn_split_kernel<32,4,false>";
    case ATTN_TILE_64_4: return "attn_kernel<64,4>";
    case ATTN_TILE_32_4: return "attn_kernel<32,4>";
    case ATTN_TILE_64_2: return "attn_kernel<64,2>";
    case ATTN_TILE_32_2: return "attn_kernel<32,2>";
    default: return "none";
  }
}

hipError_t launch_attention(bool ns, int dh, const AttnParams& p, int n_seg, hipStream_t s) {
  if (p.nq <= 0 || n_seg <= 0) return hipSuccess;
  if (p.kv_cap % KT != 0 || (dh != 32 && dh != 64)) return hipErrorInvalidValue;
  // NS segments (their own cached keys each) come with no shared extra keys
  if (ns && n_seg != 1 && p.n_x > 0) return hipErrorInvalidValue;
  const dim3 grouped_grid((p.nq + 31) / 32 * p.H * n_seg), split_grid((p.nq + 31) / 32, p.H, n_seg);
  switch (attention_route(ns, dh, p.nq, p.H, n_seg)) {
    case ATTN_NS2_64_2: launch_attn_ns2<64, 2>(p, n_seg, s); break;
    case ATTN_NS2_64_1: launch_attn_ns2<64, 1>(p, n_seg, s); break;
    case ATTN_NS2_32_2: launch_attn_ns2<32, 2>(p, n_seg, s); break;
    case ATTN_NS2_32_1: launch_attn_ns2<32, 1>(p, n_seg, s); break;
    case ATTN_NSSPLIT_64_GROUPED:
      hipLaunchKernelGGL((attn_split_kernel<64, 5, true, true>), grouped_grid, dim3(320), 0, s, p);
      break;
    case ATTN_NSSPLIT_32_GROUPED:
      hipLaunchKernelGGL((attn_split_kernel<32, 4, true, true>), grouped_grid, dim3(256), 0, s, p);
      break;
    case ATTN_NSSPLIT_64:
      hipLaunchKernelGGL((attn_split_kernel<64, 5, false, true>), split_grid, dim3(320), 0, s, p);
      break;
    case ATTN_NSSPLIT_32:
      hipLaunchKernelGGL((attn_split_kernel<32, 4, false, true>), split_grid, dim3(256), 0, s, p);
      break;
    case ATTN_SPLIT_64_GROUPED:
      hipLaunchKernelGGL((attn_split_kernel<64, 5, true, false>), grouped_grid, dim3(320), 0, s, p);
      break;
    case ATTN_SPLIT_32_GROUPED:
      hipLaunchKernelGGL((attn_split_kernel<32, 4, true, false>), grouped_grid, dim3(256), 0, s, p);
      break;
    case ATTN_SPLIT_64:
      hipLaunchKernelGGL((attn_split_kernel<64, 5, false, false>), split_grid, dim3(320), 0, s, p);
      break;
    case ATTN_SPLIT_32:
      hipLaunchKernelGGL((attn_split_kernel<32, 4, false, false>), split_grid, dim3(256), 0, s, p);
      break;
    case ATTN_TILE_64_4: launch_attn_nw<64, 4>(p, n_seg, s); break;
    case ATTN_TILE_32_4: launch_attn_nw<32, 4>(p, n_seg, s); break;
    case ATTN_TILE_64_2: launch_attn_nw<64, 2>(p, n_seg, s); break;
    case ATTN_TILE_32_2: launch_attn_nw<32, 2>(p, n_seg, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_cache_clear_tail(const ClearTailParams& p, hipStream_t s) {
  if (p.n_layers <= 0 || p.blocks <= 0) return hipSuccess;
  if (p.n_layers > ONETRANS_CLEAR_MAX_LAYERS) return hipErrorInvalidValue;
  int widest = 0;
  for (int l = 0; l < p.n_layers; ++l)
    if (p.cap[l] - p.from[l] > widest) widest = p.cap[l] - p.from[l];
  if (widest <= 0) return hipSuccess;
  int gx = (widest * p.dh + 255) / 256;
  if (gx > 64) gx = 64;
  hipLaunchKernelGGL(cache_clear_tail_kernel, dim3(gx, p.blocks, p.n_layers), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace onetrans
