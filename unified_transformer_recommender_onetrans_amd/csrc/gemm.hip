// Grouped GEMMs of the OneTrans block on gfx950 MFMA (fp16 operands, fp32 accumulate).
//
// One kernel template covers the linear maps of a layer (agihunt.info OneTrans
// summary, "method": shared S-token QKV/FFN, private per-NS-position QKV/FFN):
//   GEMM_QKV      : A = x * g rows (fp16), B = W_QKV [3d][d]; epilogue scales the row by
//                   its RMSNorm factor r and writes bf16 Q / K / V (V transposed for
//                   the S cache)
//   GEMM_FFN_UP   : A = x * g rows (fp16), B = W1 [F][d]; epilogue GELU(r * acc) ->
//                   fp16 hidden rows
//   GEMM_FFN_DOWN : A = fp16 hidden rows, B = W2 [d][F]; epilogue adds into the fp32
//                   residual rows in place and writes the next norm's x * g rows and
//                   partial sums of squares (the deferred RMSNorm described with NormOut)
// A group is one NS position (private weights) or the shared S weights.
//
// Persistent schedule, one workgroup of 8 or 12 waves per CU. The work list (BM x BN
// output tiles of every group) is split into 8 contiguous ranges, one per XCD
// (the hardware dispatches block L to XCD L % 8), and each XCD's workgroups take
// its items round-robin, so neighbouring tiles that share weight rows and
// activation rows run together in that XCD's L2.
//
// Warp specialisation. Loads and stores share one vmcnt counter on gfx9, so a
// wave that both streams operands and writes results must wait for its own
// stores whenever it waits for a k-tile. Here the last four waves only stream: they
// issue the k-tiles (global -> LDS with global_load_lds_dwordx4, 16 bytes per lane),
// wait for them and meet the compute waves at one barrier per k-tile. The first 4
// (or 8, for 256x192 tiles of E4M3 weights: two per SIMD) only compute: MFMA from LDS, then the
// epilogue's stores, which drain in the background while the loaders keep up to
// STAGES-1 k-tiles of the next item in flight. The ring holds 2-8 stages (about
// 112-144 KB of LDS).
//
// LDS rows are 128 bytes (64 halfs of k) or 64 bytes (64 E4M3 codes) with their
// 16-byte chunks XOR-swizzled by row, so the MFMA fragment reads are free of bank
// conflicts on the 64-bank LDS.
//
// MFMA: v_mfma_f32_32x32x16_f16 with the weight fragment as the first operand; the
// compute waves form a WM x (4/WM) grid, each owning a block of 32x32 accumulators. A
// lane ends up holding one output row and groups of four consecutive columns, so the
// epilogue writes 16 contiguous bytes per lane and instruction. E4M3 weights are
// decoded to fp16 exactly in registers after the LDS read.
#include "gemm_common.h"

namespace onetrans {
namespace {

// SIDE (0 = shared S weights, 1 = private NS weights) only names the instance.
// Waves 0 .. CW-1 compute (a WM x (CW/WM) grid over the tile), the next four load.
template <int KIND, bool FP8, int SIDE, int BM, int BN, int STAGES, int WM, int CW>
__global__ __launch_bounds__((CW + 4) * 64, 1) void gemm_kernel(GemmParams p, int n_tiles_m, int n_tiles_n,
                                                               int n_items, int n_fast) {
  constexpr int BK = 64;
  constexpr int WN = CW / WM;
  constexpr int TM = BM / WM, TN = BN / WN;  // one compute wave's part of the tile
  constexpr int MI = TM / 32, NI = TN / 32;  // 32x32 blocks per compute wave
  constexpr int AROW = BK * 2;               // bytes per LDS row: fp16 activations
  constexpr int BROW = FP8 ? BK : BK * 2;    // E4M3 codes or fp16 weights
  constexpr int A_BYTES = BM * AROW, B_BYTES = BN * BROW, STAGE = A_BYTES + B_BYTES;
  constexpr int A_INSTR = A_BYTES / 4096, B_INSTR = B_BYTES / 4096;  // per loader wave and k-tile
  constexpr int PT = A_INSTR + B_INSTR;
  constexpr int A_RPI = 1024 / AROW, B_RPI = 1024 / BROW;  // rows per DMA instruction
  constexpr int A_CPR = AROW / 16, B_CPR = BROW / 16;      // 16-byte chunks per row
  static_assert((CW == 4 || CW == 8) && WM * WN == CW && TM % 32 == 0 && TN % 32 == 0, "wave grid");
  static_assert(A_INSTR >= 1 && B_INSTR >= 1 && A_BYTES % 4096 == 0 && B_BYTES % 4096 == 0, "tile shape");
  static_assert(STAGES >= 2 && STAGES * STAGE <= 159 * 1024, "LDS");
  static_assert(PT * (STAGES - 2) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  // item w -> (M tile, N tile, group). Consecutive items share the tile of the slower index,
  // which they then read from their XCD's L2: the N index runs fastest (n_fast) when a
  // group's activation rows outweigh its weight rows, else the M index.
  auto tile_of = [&](int w, int& mt, int& nt, int& g) {
    const int r = w % (n_tiles_m * n_tiles_n);
    g = w / (n_tiles_m * n_tiles_n);
    if (n_fast) { nt = r % n_tiles_n; mt = r / n_tiles_n; }
    else { mt = r % n_tiles_m; nt = r / n_tiles_m; }
  };

  if (wave >= CW) {
    // ================= loader waves: the only waves that touch vmcnt for operands =================
    const int lw = wave - CW;
    const char* a_src[A_INSTR];
    const char* b_src[B_INSTR];
    int iss_t = 0, iss_kt = 0;  // item and k-tile of the next step to issue
    auto issue = [&](int s) {
      if (iss_kt == 0) {
        const int w = ib + iss_t * nx;
        int mt, nt, g;
        tile_of(w, mt, nt, g);
        const int m0 = mt * BM, n0 = nt * BN;
#pragma unroll
        for (int i = 0; i < A_INSTR; ++i) {
          const int r = (lw * A_INSTR + i) * A_RPI + lane / A_CPR;
          const int row = min(m0 + r, M - 1);
          int seg, tt;
          split_row(row, rm.rows_per_seg, inv_rps, seg, tt);
          a_src[i] = (const char*)(p.a_in + hid_row(rm, seg, tt, g) * (long)K) + (swz<AROW>(lane % A_CPR, r) << 4);
        }
        const char* wbase = (const char*)p.w + (long)g * p.w_group_stride * (FP8 ? 1 : 2);
#pragma unroll
        for (int i = 0; i < B_INSTR; ++i) {
          const int r = (lw * B_INSTR + i) * B_RPI + lane / B_CPR;
          const int n = n0 + r;  // N % BN == 0
          b_src[i] = wbase + ((long)(n >> 5) * (K >> 6) * 2048 + (n & 31) * 64) * (FP8 ? 1 : 2) +
                     (swz<BROW>(lane % B_CPR, r) << 4);
        }
      }
      char* st = smem + (s % STAGES) * STAGE;
#pragma unroll
      for (int i = 0; i < A_INSTR; ++i)
        dma16(a_src[i] + iss_kt * AROW, (lds_void*)(st + (lw * A_INSTR + i) * 1024));
#pragma unroll
      for (int i = 0; i < B_INSTR; ++i)
        dma16(b_src[i] + iss_kt * (2048 * (FP8 ? 1 : 2)), (lds_void*)(st + A_BYTES + (lw * B_INSTR + i) * 1024));
      if (++iss_kt == nk) { iss_kt = 0; ++iss_t; }
    };
    int s_issue = 0;
    for (; s_issue < STAGES - 1 && s_issue < total_steps; ++s_issue) issue(s_issue);
#pragma unroll 1
    for (int s = 0; s < total_steps; ++s) {
      wait_tiles<PT, STAGES - 2>(s_issue - 1 - s);  // this wave's part of step s is in LDS
      lds_barrier();                                // everyone's part is in; step s-1's stage is free
      if (s_issue < total_steps) { issue(s_issue); ++s_issue; }
    }
    return;
  }

  // ================= compute waves: MFMA and epilogue stores, never wait for operand loads =================
  const int wm = wave / WN, wn = wave % WN;
  constexpr int KS = BK / 16;  // 16-wide k-steps per k-tile (even: the fragment buffers alternate)
  static_assert(KS % 2 == 0, "k-steps per tile");
  // Fragments of one k-step, double-buffered with four compute waves: the reads of step
  // ks + 1 are issued before the MFMAs of step ks, so LDS latency hides under them. With
  // eight (two per SIMD) the other wave's MFMAs cover it and one buffer keeps registers
  // for the accumulators. E4M3 weights stay as codes until the MFMA that takes them.
  constexpr int NBUF = CW == 8 ? 1 : 2;
  f16x8 af[NBUF][MI];
  f16x8 bf[NBUF][FP8 ? 1 : NI];
  uint2 b8[NBUF][FP8 ? NI : 1];
  auto read_frags = [&](int s, int ks, int b) {
    const char* st = smem + (s % STAGES) * STAGE;
    const int c = 2 * ks + (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int r = wm * TM + mi * 32 + (lane & 31);
      af[b][mi] = *(const f16x8*)(st + r * AROW + (swz<AROW>(c, r) << 4));
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int r = wn * TN + ni * 32 + (lane & 31);
      if constexpr (FP8)
        b8[b][ni] = *(const uint2*)(st + A_BYTES + r * 64 + (swz<64>(ks, r) << 4) + (lane >> 5) * 8);
      else
        bf[b][ni] = *(const f16x8*)(st + A_BYTES + r * BROW + (swz<BROW>(c, r) << 4));
    }
  };
  // the first step's tile is in LDS (one barrier per step, as the loaders)
  if (my_items > 0) {
    lds_barrier();
    if constexpr (NBUF == 2) read_frags(0, 0, 0);
  }
#pragma unroll 1
  for (int t = 0; t < my_items; ++t) {
    f32x16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.f;

    int mt_, nt_, g_;
    tile_of(ib + t * nx, mt_, nt_, g_);
    TilePre<KIND, MI, NI> pre;
    tile_prefetch<KIND, MI, NI, TM, TN>(p, mt_ * BM, nt_ * BN, g_, wm, wn, pre);

#pragma unroll 1
    for (int kt = 0; kt < nk; ++kt) {
      const int s = t * nk + kt;
      if constexpr (NBUF == 1) {
        if (s > 0) lds_barrier();  // certifies step s and hands step s - 1's stage back
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          read_frags(s, ks, 0);
          __builtin_amdgcn_s_waitcnt(0xC07F);
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            f16x8 wf;
            if constexpr (FP8) wf = e4m3x8_to_f16(b8[0][ni]);
            else wf = bf[0][ni];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf, af[0][mi], acc[mi][ni], 0, 0, 0);
          }
        }
        continue;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int b = ks & 1;
        // this step's fragments, read one step ago, have arrived; waiting before the next
        // reads are issued keeps the compiler from waiting for those as well
        __builtin_amdgcn_s_waitcnt(0xC07F);
        if (ks + 1 < KS) {
          read_frags(s, ks + 1, (b ^ 1) % NBUF);
        } else if (s + 1 < total_steps) {
          // every wave has read its last fragments of step s: the barrier hands that stage
          // back to the loaders and certifies step s + 1, whose first fragments are read now
          lds_barrier();
          read_frags(s + 1, 0, (b ^ 1) % NBUF);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          f16x8 wf;
          if constexpr (FP8) wf = e4m3x8_to_f16(b8[b % NBUF][ni]);
          else wf = bf[b % NBUF][ni];
#pragma unroll
          for (int mi = 0; mi < MI; ++mi)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf, af[b % NBUF][mi], acc[mi][ni], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    tile_epilogue<KIND, FP8, MI, NI, TM, TN>(p, acc, mt_ * BM, nt_ * BN, g_, wm, wn, pre);
  }
}

// One 256x192 output tile per workgroup (no persistence; with more tiles than CUs the
// hardware starts each workgroup as a CU frees up), for fp16 weights: fewer operand bytes
// per CU than smaller tiles (each weight row is fetched once per 256 rows, each activation
// row once per 192 columns), and a workgroup that starts late (its CU held by concurrent
// work) delays one tile only. With one tile per workgroup no epilogue store ever precedes
// a k-tile wait, so all 8
// waves both stream operands and compute (a 4 x 2 grid of 64x96 parts, 96 accumulators
// per lane at two waves per SIMD). k-tiles are 64 wide, so every row of a k-tile is one
// whole 128-byte line (a weight k-tile is six contiguous 4 KB panel blocks); the 56 KB
// stages leave room for a ring of two (the next k-tile streams while this one is
// multiplied). Each k-tile is 56 DMA instructions of 1 KB, 4 of A and 3 of B per wave.
template <int KIND, int SIDE>
__global__ __launch_bounds__(512, 1) void gemm_tile256_kernel(GemmParams p, int n_tiles_n, int n_tiles_m) {
  constexpr int BM = 256, BN = 192, BK = 64, STAGES = 2;
  constexpr int WN = 2, TM = 64, TN = 96, MI = TM / 32, NI = TN / 32;
  constexpr int ROW = BK * 2;  // bytes per LDS row (fp16)
  constexpr int A_BYTES = BM * ROW, STAGE = (BM + BN) * ROW;
  constexpr int RPI = 1024 / ROW, CPR = ROW / 16;  // rows per DMA instruction, chunks per row
  static_assert(STAGES * STAGE <= 159 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const RowMap rm = p.rm;
  const int M = p.M, N = p.N, K = p.K;
  const float inv_rps = 1.0f / (float)rm.rows_per_seg;
  const int nk = K / BK;
  // tile of this workgroup: each XCD (workgroup L runs on XCD L % 8) takes a contiguous range
  // of tiles, the N index fastest, so the tiles of one activation block share that XCD's L2
  // (then M, then the group)
  const int total = gridDim.x, L = blockIdx.x;
  const int x = L % N_XCD, w = x * (total / N_XCD) + min(x, total % N_XCD) + L / N_XCD;
  const int nt = w % n_tiles_n, mt = (w / n_tiles_n) % n_tiles_m, g = w / (n_tiles_n * n_tiles_m);
  const int n0 = nt * BN, m0 = mt * BM;

  // per-lane DMA sources: A instructions 4w .. 4w+3, B instructions 3w .. 3w+2
  const char* a_src[4];
  const char* b_src[3];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (4 * wave + i) * RPI + lane / CPR;
    const int row = min(m0 + r, M - 1);
    int seg, tt;
    split_row(row, rm.rows_per_seg, inv_rps, seg, tt);
    a_src[i] = (const char*)(p.a_in + hid_row(rm, seg, tt, g) * (long)K) + (swz<ROW>(lane % CPR, r) << 4);
  }
  const char* wbase = (const char*)p.w + (long)g * p.w_group_stride * 2;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int bi = 3 * wave + i;
    const int r = bi * RPI + lane / CPR;
    const int n = n0 + r;
    b_src[i] = wbase + ((long)(n >> 5) * (K >> 6) * 2048 + (n & 31) * 64) * 2 + (swz<ROW>(lane % CPR, r) << 4);
  }
  auto issue = [&](int kt) {
    char* st = smem + (kt % STAGES) * STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(a_src[i] + kt * ROW, (lds_void*)(st + (4 * wave + i) * 1024));
#pragma unroll
    for (int i = 0; i < 3; ++i) dma16(b_src[i] + (long)kt * 4096, (lds_void*)(st + A_BYTES + (3 * wave + i) * 1024));
  };
  // this wave's part of k-tile kt is in LDS
  auto wait_kt = [&](int later) { wait_tiles<7, STAGES - 2>(later); };

  const int wm = wave / WN, wn = wave % WN;
  f32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.f;
  TilePre<KIND, MI, NI> pre;
  tile_prefetch<KIND, MI, NI, TM, TN>(p, m0, n0, g, wm, wn, pre);

  for (int kt = 0; kt < STAGES - 1 && kt < nk; ++kt) issue(kt);
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    wait_kt(min(STAGES - 2, nk - 1 - kt));
    lds_barrier();  // k-tile kt is in for everyone; everyone is done with kt - 1, whose slot refills now
    if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);
    const char* st = smem + (kt % STAGES) * STAGE;
    f16x8 af[4][MI], bf[4][NI];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = 2 * ks + (lane >> 5);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int r = wm * TM + mi * 32 + (lane & 31);
        af[ks][mi] = *(const f16x8*)(st + r * ROW + (swz<ROW>(c, r) << 4));
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int r = wn * TN + ni * 32 + (lane & 31);
        bf[ks][ni] = *(const f16x8*)(st + A_BYTES + r * ROW + (swz<ROW>(c, r) << 4));
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[ks][ni], af[ks][mi], acc[mi][ni], 0, 0, 0);
  }
  tile_epilogue<KIND, false, MI, NI, TM, TN>(p, acc, m0, n0, g, wm, wn, pre);
}

// Tile shapes: (BM, BN, compute waves along M). 96-wide tiles are fp16-only (a 96-row E4M3
// tile is not a whole number of 4 KB DMA rounds). The operand ring takes up to 159 KB of
// LDS, at most 8 stages.
template <int KD, int BM, int BN, int WM, bool FP8>
constexpr int stages_for() {
  constexpr int stage = BM * 128 + BN * (FP8 ? 64 : 128);
  constexpr int n = (159 * 1024) / stage;
  return n > 8 ? 8 : n;
}

template <int KD, bool FP8, int SIDE, int BM, int BN, int WM, int CW>
void launch_one(const GemmParams& p, hipStream_t s) {
  const int tm = (p.M + BM - 1) / BM, tn = p.N / BN;
  const long items = (long)tm * tn * p.groups;
  const int grid = (int)(items < 256 ? items : 256);  // one workgroup per CU
  const int n_fast = (long)p.M > (long)p.N ? 1 : 0;  // a group's rows: activations M x K, weights N x K
  hipLaunchKernelGGL((gemm_kernel<KD, FP8, SIDE, BM, BN, stages_for<KD, BM, BN, WM, FP8>(), WM, CW>), dim3(grid),
                     dim3((CW + 4) * 64), 0, s, p, tm, tn, (int)items, n_fast);
}

template <int KD, int SIDE, int BM, int BN, int WM, int CW = 4>
void launch_cfg(bool fp8, const GemmParams& p, hipStream_t s) {
  if constexpr (SIDE == 1 && BN != 96) {
    if (fp8) {
      launch_one<KD, true, SIDE, BM, BN, WM, CW>(p, s);
      return;
    }
  }
  launch_one<KD, false, SIDE, BM, BN, WM, CW>(p, s);
}

struct TileCfg {
  int bm, bn;
};

// The GEMMs here are bound by the L2 -> LDS operand feed, so the cost of a tile shape is
// the busiest CU's item count times the operand bytes per item and k.
double tile_cost(const GemmParams& p, bool fp8, int bm, int bn) {
  const long items = (long)((p.M + bm - 1) / bm) * (p.N / bn) * p.groups;
  return (double)((items + 255) / 256) * (bm + bn * (fp8 ? 0.5 : 1.0));
}

template <int KD, int SIDE>
void launch_kind(bool fp8, const GemmParams& p, hipStream_t s) {
  // a Q / K / V tile must not straddle two of them: BN divides d
  auto fits = [&](int bn) {
    return p.N % bn == 0 && (KD != GEMM_QKV || p.d % bn == 0) && !(fp8 && bn == 96) &&
           !(KD == GEMM_FFN_DOWN && bn == 192);
  };
  // ties go to the earlier entry: the smaller tile, which leaves fewer CUs idle in the last round
  const TileCfg cands[7] = {{128, 96}, {128, 128}, {256, 96}, {256, 128}, {128, 64}, {64, 64}, {256, 192}};
  int best = -1;
  double best_cost = 0;
  for (int i = 0; i < 7; ++i) {
    if (!fits(cands[i].bn)) continue;
    const double c = tile_cost(p, fp8, cands[i].bm, cands[i].bn);
    if (best < 0 || c < best_cost) { best = i; best_cost = c; }
  }
  // 256x192: one tile per workgroup with fp16 weights, persistent with eight compute waves
  // with E4M3 weights
  if (best == 6) {
    if constexpr (KD != GEMM_FFN_DOWN) {  // (never picked for FFN down: see fits)
      if (!fp8) {
        const int tn = p.N / 192, tm = (p.M + 255) / 256;
        hipLaunchKernelGGL((gemm_tile256_kernel<KD, SIDE>), dim3(tm * tn * p.groups), dim3(512), 0, s, p, tn, tm);
        return;
      }
      if constexpr (SIDE == 1) launch_one<KD, true, SIDE, 256, 192, 4, 8>(p, s);  // E4M3: NS weights only
    }
    return;
  }
  switch (best) {
    case 0: launch_cfg<KD, SIDE, 128, 96, 4>(fp8, p, s); break;
    case 1: launch_cfg<KD, SIDE, 128, 128, 2>(fp8, p, s); break;
    case 2: launch_cfg<KD, SIDE, 256, 96, 4>(fp8, p, s); break;
    case 3: launch_cfg<KD, SIDE, 256, 128, 2>(fp8, p, s); break;
    case 4: launch_cfg<KD, SIDE, 128, 64, 2>(fp8, p, s); break;
    default: launch_cfg<KD, SIDE, 64, 64, 2>(fp8, p, s); break;
  }
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
