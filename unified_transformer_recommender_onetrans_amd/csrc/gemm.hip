// Grouped GEMMs of the OneTrans block on gfx950 MFMA (fp16 operands, fp32 accumulate).
//
// One kernel template covers the linear maps of a layer (agihunt.info OneTrans
// summary, "method": shared S-token QKV/FFN, private per-NS-position QKV/FFN):
//   GEMM_QKV      : A = RMSNorm'd rows (fp16), B = W_QKV [3d][d];
//                   epilogue writes bf16 Q / K / V (V transposed for the S cache)
//   GEMM_FFN_UP   : A = RMSNorm'd rows (fp16), B = W1 [F][d];
//                   epilogue GELU -> fp16 hidden rows
//   GEMM_FFN_DOWN : A = fp16 hidden rows, B = W2 [d][F];
//                   epilogue adds into the fp32 residual rows in place
// A group is one NS position (private weights) or the shared S weights.
//
// Persistent schedule. The work list (BM x BN output tiles of every group) is
// split into 8 contiguous ranges, one per XCD (the hardware dispatches block L to
// XCD L % 8), and each XCD's workgroups take its items round-robin, so the
// workgroups of one XCD work on neighbouring tiles that share weight rows and
// activation rows in that XCD's L2. Each workgroup keeps STAGES-1 k-tiles in
// flight across item boundaries: the next item's first tiles stream in while
// the current item finishes, and its epilogue writes straight from the
// accumulators, so the operand ring never drains.
//
// Two workgroups share a CU (LDS <= 80 KB and <= 256 registers per lane each), so
// one workgroup's epilogue (GELU, format conversion, stores) overlaps the other's
// MFMA loop.
//
// Data movement: k-tiles go global -> LDS with global_load_lds_dwordx4 (16 bytes
// per lane, 1 KB per wave instruction). LDS rows are 64 or 128 bytes with their
// 16-byte chunks XOR-swizzled by row, which keeps the MFMA fragment reads free of
// bank conflicts on the 64-bank LDS.
//
// MFMA: v_mfma_f32_32x32x16_f16, 4 waves in a 2 x 2 grid, each owning a
// (BM/2) x (BN/2) block of 32x32 accumulators. A lane ends up holding one output
// column and groups of four consecutive rows, so each epilogue store instruction
// writes 32 consecutive columns (64 or 128 contiguous bytes) of two rows.
#include "internal.h"

namespace onetrans {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int N_XCD = 8;

__device__ __forceinline__ long res_row_off(const RowMap& rm, int seg, int t, int g) {
  return (long)seg * rm.res_seg_stride + (rm.res_row_base + t) * rm.res_row_stride + (long)g * rm.res_group_stride;
}
__device__ __forceinline__ long hid_row(const RowMap& rm, int seg, int t, int g) {
  return ((long)seg * rm.rows_per_seg + t) * rm.row_mult + g;
}
// row -> (seg, t) without an integer division: float estimate, then one correction
__device__ __forceinline__ void split_row(int row, int rps, float inv_rps, int& seg, int& t) {
  seg = (int)((float)row * inv_rps);
  t = row - seg * rps;
  if (t < 0) { --seg; t += rps; }
  else if (t >= rps) { ++seg; t -= rps; }
}

// Exact OCP E4M3FN -> fp16 for the two codes held in bits 0-7 and 16-23 of x.
// Normal codes: the fp16 exponent is the E4M3 exponent field + 8 (bias 15 vs 7),
// mantissa bits move up by 7. Zero / subnormal codes (exponent field 0) are
// m * 2^-9, taken through an exact float conversion.
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t x) {
  uint32_t r = (((x & 0x007F007Fu) << 7) + 0x20002000u) | ((x & 0x00800080u) << 8);
  if (__builtin_expect(((x & 0x00000078u) == 0) || ((x & 0x00780000u) == 0), 0)) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      uint32_t c = (x >> (16 * hh)) & 0xFFu;
      if ((c & 0x78u) == 0) {
        _Float16 v = (_Float16)((float)(c & 7u) * 0.001953125f);
        uint32_t bits = (uint32_t)__builtin_bit_cast(uint16_t, v) | ((c & 0x80u) << 8);
        r = (r & ~(0xFFFFu << (16 * hh))) | (bits << (16 * hh));
      }
    }
  }
  return r;
}

// 8 E4M3 codes (two dwords) -> 8 halfs in order.
__device__ __forceinline__ f16x8 e4m3x8_to_f16(uint2 c) {
  const uint32_t in[2] = {c.x, c.y};
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t a = e4m3x2_to_f16x2(in[i] & 0x00FF00FFu);         // codes 0, 2
    const uint32_t b = e4m3x2_to_f16x2((in[i] >> 8) & 0x00FF00FFu);  // codes 1, 3
    out[2 * i] = (a & 0xFFFFu) | (b << 16);
    out[2 * i + 1] = (a >> 16) | (b & 0xFFFF0000u);
  }
  return __builtin_bit_cast(f16x8, make_uint4(out[0], out[1], out[2], out[3]));
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// Wait until at most `later` k-tiles of PT loads each are still in flight. Only loads
// are counted: loads retire in order, so a pending store can delay this wait but never
// satisfy it early.
template <int PT, int MAXL>
__device__ __forceinline__ void wait_tiles(int later) {
  if constexpr (MAXL == 0) {
    wait_vmcnt<0>();
  } else {
    if (later >= MAXL) wait_vmcnt<PT * MAXL>();
    else wait_tiles<PT, MAXL - 1>(later);
  }
}

// Workgroup barrier without the release fence __syncthreads() carries (which
// would wait for every load in flight, draining the pipeline). The explicit
// vmcnt waits before it make the DMA'd tile visible; the empty asm statements
// keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// physical 16-byte chunk of logical chunk c in LDS row r (rows of ROWB bytes)
template <int ROWB>
__device__ __forceinline__ int swz(int c, int r) {
  static_assert(ROWB == 64 || ROWB == 128, "row size");
  return ROWB == 128 ? (c ^ ((r >> 1) & 7)) : (c ^ ((r >> 2) & 3));
}

// SIDE (0 = shared S weights, 1 = private NS weights) only names the instance.
template <int KIND, bool FP8, int SIDE, int BM, int BN, int BK, int STAGES, int WPC>
__global__ __launch_bounds__(256, WPC) void gemm_kernel(GemmParams p, int n_tiles_m, int n_tiles_n, int n_items) {
  constexpr int MI = BM / 64, NI = BN / 64;  // 32x32 blocks per wave
  constexpr int AROW = BK * 2;               // bytes per LDS row: fp16 activations
  constexpr int BROW = FP8 ? BK : BK * 2;    // E4M3 codes or fp16 weights
  constexpr int A_BYTES = BM * AROW, B_BYTES = BN * BROW, STAGE = A_BYTES + B_BYTES;
  constexpr int A_INSTR = A_BYTES / 4096, B_INSTR = B_BYTES / 4096;  // per wave and k-tile
  constexpr int PT = A_INSTR + B_INSTR;
  constexpr int A_RPI = 1024 / AROW, B_RPI = 1024 / BROW;  // rows per DMA instruction
  constexpr int A_CPR = AROW / 16, B_CPR = BROW / 16;      // 16-byte chunks per row
  static_assert(A_INSTR >= 1 && B_INSTR >= 1 && A_BYTES % 4096 == 0 && B_BYTES % 4096 == 0, "tile shape");
  static_assert(STAGES * STAGE <= 160 * 1024 / WPC, "LDS of WPC workgroups per CU");
  static_assert(!FP8 || BROW == 64, "E4M3 tiles use 64-byte rows");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const RowMap rm = p.rm;
  const int M = p.M, N = p.N, K = p.K;
  const float inv_rps = 1.0f / (float)rm.rows_per_seg;
  const int nk = K / BK;

  // ---- this workgroup's items ----
  const int G = gridDim.x, L = blockIdx.x;
  const int xcd = L % N_XCD, jx = L / N_XCD;
  const int nx = G / N_XCD + (xcd < G % N_XCD ? 1 : 0);
  const int per = n_items / N_XCD, rem = n_items % N_XCD;
  const int ib = xcd * per + min(xcd, rem) + jx;
  const int cnt = per + (xcd < rem ? 1 : 0);
  const int my_items = jx < cnt ? (cnt - jx + nx - 1) / nx : 0;
  const int total_steps = my_items * nk;

  // ---- issue side: per-lane sources of the direct-to-LDS loads for the item being fetched ----
  const char* a_src[A_INSTR];
  const char* b_src[B_INSTR];
  int iss_t = 0, iss_kt = 0;  // item and k-tile of the next step to issue
  auto set_sources = [&](int t) {
    const int w = ib + t * nx;
    const int mt = w % n_tiles_m, nt = (w / n_tiles_m) % n_tiles_n, g = w / (n_tiles_m * n_tiles_n);
    const int m0 = mt * BM, n0 = nt * BN;
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) {
      const int r = (wave * A_INSTR + i) * A_RPI + lane / A_CPR;
      const int row = min(m0 + r, M - 1);
      int seg, tt;
      split_row(row, rm.rows_per_seg, inv_rps, seg, tt);
      a_src[i] = (const char*)(p.a_in + hid_row(rm, seg, tt, g) * (long)K) + (swz<AROW>(lane % A_CPR, r) << 4);
    }
    const char* wbase = (const char*)p.w + (long)g * p.w_group_stride * (FP8 ? 1 : 2);
#pragma unroll
    for (int i = 0; i < B_INSTR; ++i) {
      const int r = (wave * B_INSTR + i) * B_RPI + lane / B_CPR;
      const int n = min(n0 + r, N - 1);
      b_src[i] = wbase + (long)n * K * (FP8 ? 1 : 2) + (swz<BROW>(lane % B_CPR, r) << 4);
    }
  };
  auto issue = [&](int s) {
    if (iss_kt == 0) set_sources(iss_t);
    char* st = smem + (s % STAGES) * STAGE;
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i)
      dma16(a_src[i] + iss_kt * AROW, (lds_void*)(st + (wave * A_INSTR + i) * 1024));
#pragma unroll
    for (int i = 0; i < B_INSTR; ++i)
      dma16(b_src[i] + iss_kt * BROW, (lds_void*)(st + A_BYTES + (wave * B_INSTR + i) * 1024));
    if (++iss_kt == nk) { iss_kt = 0; ++iss_t; }
  };

  int s_issue = 0;
  for (; s_issue < STAGES - 1 && s_issue < total_steps; ++s_issue) issue(s_issue);
  int landed = 0;  // steps below this are known to be in LDS

#pragma unroll 1
  for (int t = 0; t < my_items; ++t) {
    f32x16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.f;

#pragma unroll 1
    for (int kt = 0; kt < nk; ++kt) {
      const int s = t * nk + kt;
      if (s >= landed) wait_tiles<PT, STAGES - 2>(s_issue - 1 - s);
      lds_barrier();  // all waves' parts of step s are in; step s-1's stage is free
      if (s_issue < total_steps) { issue(s_issue); ++s_issue; }
      const char* st = smem + (s % STAGES) * STAGE;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        f16x8 a[MI], b[NI];
        const int c = 2 * ks + (lane >> 5);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          const int r = wm * (BM / 2) + mi * 32 + (lane & 31);
          a[mi] = *(const f16x8*)(st + r * AROW + (swz<AROW>(c, r) << 4));
        }
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int r = wn * (BN / 2) + ni * 32 + (lane & 31);
          if (FP8)
            b[ni] = e4m3x8_to_f16(*(const uint2*)(st + A_BYTES + r * 64 + (swz<64>(ks, r) << 4) + (lane >> 5) * 8));
          else
            b[ni] = *(const f16x8*)(st + A_BYTES + r * BROW + (swz<BROW>(c, r) << 4));
        }
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
      }
    }

    // ---- epilogue. Lane holds column (lane % 32) of each 32x32 block and, in
    // registers 4q..4q+3, rows 8q + 4*(lane/32) + 0..3: a store instruction covers
    // 32 consecutive columns of two rows ----
    const int w = ib + t * nx;
    const int mt = w % n_tiles_m, nt = (w / n_tiles_m) % n_tiles_n, g = w / (n_tiles_m * n_tiles_n);
    const int m0 = mt * BM, n0 = nt * BN;
    const float scale = FP8 ? p.wscale[g * 5 + p.scale_idx0 + n0 / p.scale_col_div] : 1.f;
    const int col0 = n0 + wn * (BN / 2) + (lane & 31);     // + ni*32
    const int row_w = m0 + wm * (BM / 2) + 4 * (lane >> 5);  // + mi*32 + 8q + e
    const int rps = rm.rows_per_seg;
    // row r = row_w + mi*32 + 8q + e  ->  (seg, t) of its first row, then step within the group
    auto group_start = [&](int r0, int& seg, int& tt) { split_row(r0, rps, inv_rps, seg, tt); };
    auto step = [&](int& seg, int& tt) {
      if (++tt >= rps) { tt = 0; ++seg; }
    };
    if (KIND == GEMM_FFN_DOWN) {
      float old[MI][4][4][NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int seg, tt;
          group_start(min(row_w + mi * 32 + 8 * q, M - 1), seg, tt);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float* src = p.res_out + res_row_off(rm, seg, tt, g) + col0;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) old[mi][q][e][ni] = src[ni * 32];
            if (row_w + mi * 32 + 8 * q + e + 1 < M) step(seg, tt);
          }
        }
      wait_vmcnt<0>();
      landed = s_issue;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r0 = row_w + mi * 32 + 8 * q;
          if (r0 >= M) continue;
          int seg, tt;
          group_start(r0, seg, tt);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (r0 + e >= M) break;
            float* dst = p.res_out + res_row_off(rm, seg, tt, g) + col0;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) dst[ni * 32] = old[mi][q][e][ni] + acc[mi][ni][4 * q + e] * scale;
            step(seg, tt);
          }
        }
    } else if (KIND == GEMM_FFN_UP) {
      wait_vmcnt<0>();
      landed = s_issue;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r0 = row_w + mi * 32 + 8 * q;
          if (r0 >= M) continue;
          int seg, tt;
          group_start(r0, seg, tt);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (r0 + e >= M) break;
            _Float16* dst = p.hid_out + hid_row(rm, seg, tt, g) * N + col0;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) dst[ni * 32] = (_Float16)gelu_as(acc[mi][ni][4 * q + e] * scale);
            step(seg, tt);
          }
        }
    } else {
      wait_vmcnt<0>();
      landed = s_issue;
      // BN divides d, so the whole tile lies in one of Q, K, V
      const int typ = n0 / p.d;
      const int dsh = p.dh == 64 ? 6 : 5;
      long cofs[NI];  // per lane: head and in-head offset of its column in each block
      int cjj[NI], chead[NI];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int c = col0 + ni * 32 - typ * p.d;
        chead[ni] = c >> dsh;
        cjj[ni] = c & (p.dh - 1);
        cofs[ni] = (long)chead[ni] * (typ == 0 ? p.q_head_stride : p.kv_head_stride) + cjj[ni];
      }
      const bool vt_mode = typ == 2 && p.vt != nullptr;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r0 = row_w + mi * 32 + 8 * q;
          if (r0 >= M) continue;
          int seg, tt;
          group_start(r0, seg, tt);
          if (vt_mode) {
            // transposed V: the four rows of the group are four key slots of one column
            const long ki = p.kv_slot_base + (long)tt * rm.row_mult + g;
            if (rm.row_mult == 1 && r0 + 3 < M && tt + 3 < rps && (ki & 3) == 0) {
#pragma unroll
              for (int ni = 0; ni < NI; ++ni) {
                const bf16x4 o = {(__bf16)(acc[mi][ni][4 * q] * scale), (__bf16)(acc[mi][ni][4 * q + 1] * scale),
                                  (__bf16)(acc[mi][ni][4 * q + 2] * scale), (__bf16)(acc[mi][ni][4 * q + 3] * scale)};
                *(bf16x4*)(p.vt + seg * p.kv_seg_stride + chead[ni] * p.kv_head_stride + (long)cjj[ni] * p.kv_cap + ki) = o;
              }
              continue;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (r0 + e >= M) break;
              const long k1 = p.kv_slot_base + (long)tt * rm.row_mult + g;
#pragma unroll
              for (int ni = 0; ni < NI; ++ni)
                p.vt[seg * p.kv_seg_stride + chead[ni] * p.kv_head_stride + (long)cjj[ni] * p.kv_cap + k1] =
                    (__bf16)(acc[mi][ni][4 * q + e] * scale);
              step(seg, tt);
            }
            continue;
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (r0 + e >= M) break;
            const int ti = tt * rm.row_mult + g;
            __bf16* base;
            if (typ == 0) {
              const int qi = ti - p.q_from;
              base = qi < 0 ? nullptr : p.q + seg * p.q_seg_stride + (long)qi * p.dh;
            } else {
              base = (typ == 1 ? p.k : p.v) + seg * p.kv_seg_stride + (p.kv_slot_base + ti) * (long)p.dh;
            }
            if (base != nullptr) {
#pragma unroll
              for (int ni = 0; ni < NI; ++ni) base[cofs[ni]] = (__bf16)(acc[mi][ni][4 * q + e] * scale);
            }
            step(seg, tt);
          }
        }
    }
  }
}

struct TileCfg {
  int bm, bn;
};

template <int KD, bool FP8, int SIDE, int BM, int BN, int BK, int ST, int WPC>
void launch_one(const GemmParams& p, hipStream_t s) {
  const int tm = (p.M + BM - 1) / BM, tn = p.N / BN;
  const long items = (long)tm * tn * p.groups;
  const int grid = (int)(items < WPC * 256 ? items : WPC * 256);
  hipLaunchKernelGGL((gemm_kernel<KD, FP8, SIDE, BM, BN, BK, ST, WPC>), dim3(grid), dim3(256), 0, s, p, tm, tn,
                     (int)items);
}

template <int KD, int SIDE, int BM, int BN>
void launch_cfg(bool fp8, const GemmParams& p, hipStream_t s) {
  if constexpr (SIDE == 1) {
    if (fp8) {
      launch_one<KD, true, SIDE, BM, BN, 64, 3, 2>(p, s);
      return;
    }
  }
  if constexpr (BM * BN >= 128 * 128) launch_one<KD, false, SIDE, BM, BN, 32, 4, 2>(p, s);
  else launch_one<KD, false, SIDE, BM, BN, 64, 3, 2>(p, s);
}

// Cost model for the tile choice: the busiest CU's share of output tiles times the
// tile's work, with a penalty for small tiles, whose operand traffic per flop is higher.
double tile_cost(const GemmParams& p, int bm, int bn) {
  const long items = (long)((p.M + bm - 1) / bm) * (p.N / bn) * p.groups;
  const double per_cu = (double)((items + 255) / 256);
  const double work = (double)bm * bn;
  const double pen = bm * bn >= 128 * 128 ? 1.0 : (bm * bn >= 128 * 64 ? 1.2 : 1.6);
  return per_cu * work * pen;
}

template <int KD, int SIDE>
void launch_kind(bool fp8, const GemmParams& p, hipStream_t s) {
  // BN = 128 needs N % 128 == 0 and, for Q / K / V, d % 128 == 0 (a tile never straddles two of them)
  const bool n128 = p.N % 128 == 0 && (KD != GEMM_QKV || p.d % 128 == 0);
  const TileCfg cands[3] = {{128, 128}, {128, 64}, {64, 64}};
  int best = -1;
  double best_cost = 0;
  for (int i = 0; i < 3; ++i) {
    if (cands[i].bn == 128 && !n128) continue;
    const double c = tile_cost(p, cands[i].bm, cands[i].bn);
    if (best < 0 || c < best_cost) { best = i; best_cost = c; }
  }
  if (best == 0) launch_cfg<KD, SIDE, 128, 128>(fp8, p, s);
  else if (best == 1) launch_cfg<KD, SIDE, 128, 64>(fp8, p, s);
  else launch_cfg<KD, SIDE, 64, 64>(fp8, p, s);
}

}  // namespace

hipError_t launch_gemm(GemmKind kind, bool fp8, bool ns, const GemmParams& p, hipStream_t s) {
  if (p.M <= 0 || p.groups <= 0) return hipSuccess;
  if (p.K % 64 != 0 || p.N % 64 != 0 || (kind == GEMM_QKV && (p.d % 64 != 0 || (p.dh != 32 && p.dh != 64))))
    return hipErrorInvalidValue;
  if (fp8 && !ns) return hipErrorInvalidValue;  // E4M3 weights are private NS weights only
  if (kind == GEMM_QKV) {
    if (ns) launch_kind<GEMM_QKV, 1>(fp8, p, s); else launch_kind<GEMM_QKV, 0>(false, p, s);
  } else if (kind == GEMM_FFN_UP) {
    if (ns) launch_kind<GEMM_FFN_UP, 1>(fp8, p, s); else launch_kind<GEMM_FFN_UP, 0>(false, p, s);
  } else {
    if (ns) launch_kind<GEMM_FFN_DOWN, 1>(fp8, p, s); else launch_kind<GEMM_FFN_DOWN, 0>(false, p, s);
  }
  return hipGetLastError();
}

}  // namespace onetrans
