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
// Persistent schedule, one workgroup of 8 waves per CU. The work list (BM x BN
// output tiles of every group) is split into 8 contiguous ranges, one per XCD
// (the hardware dispatches block L to XCD L % 8), and each XCD's workgroups take
// its items round-robin, so neighbouring tiles that share weight rows and
// activation rows run together in that XCD's L2.
//
// Warp specialisation. Loads and stores share one vmcnt counter on gfx9, so a
// wave that both streams operands and writes results must wait for its own
// stores whenever it waits for a k-tile. Here waves 4-7 only stream: they issue
// the k-tiles (global -> LDS with global_load_lds_dwordx4, 16 bytes per lane),
// wait for them and meet the compute waves at one barrier per k-tile. Waves 0-3
// only compute: MFMA from LDS, then the epilogue's stores, which drain in the
// background while the loaders keep up to STAGES-1 k-tiles of the next item in
// flight. The ring holds 3-8 stages (about 128-144 KB of LDS).
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

// 8 OCP E4M3FN codes (two dwords, code i in byte i) -> 8 halfs in order, with the gfx950
// conversion instruction at scale 1, which is exact: every E4M3FN value, subnormals
// included, is an fp16 value.
__device__ __forceinline__ f16x8 e4m3x8_to_f16(uint2 c) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.x, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.x, 1.0f, true);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.y, 1.0f, false);
  const f16x2 e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.y, 1.0f, true);
  const f16x8 r = {a[0], a[1], b[0], b[1], d[0], d[1], e[0], e[1]};
  return r;
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
  // this wave's LDS reads have returned (lgkmcnt 0; vmcnt and expcnt unconstrained): the
  // loaders refill the stage read last right after the barrier, and the compiler may defer
  // a fragment read's wait to its MFMA, past the barrier
  __builtin_amdgcn_s_waitcnt(0xC07F);
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
// Waves 0-3 compute (a WM x (4/WM) grid over the tile), waves 4-7 load.
template <int KIND, bool FP8, int SIDE, int BM, int BN, int STAGES, int WM>
__global__ __launch_bounds__(512, 1) void gemm_kernel(GemmParams p, int n_tiles_m, int n_tiles_n, int n_items,
                                                      int n_fast) {
  constexpr int BK = 64;
  constexpr int WN = 4 / WM;
  constexpr int TM = BM / WM, TN = BN / WN;  // one compute wave's part of the tile
  constexpr int MI = TM / 32, NI = TN / 32;  // 32x32 blocks per compute wave
  constexpr int AROW = BK * 2;               // bytes per LDS row: fp16 activations
  constexpr int BROW = FP8 ? BK : BK * 2;    // E4M3 codes or fp16 weights
  constexpr int A_BYTES = BM * AROW, B_BYTES = BN * BROW, STAGE = A_BYTES + B_BYTES;
  constexpr int A_INSTR = A_BYTES / 4096, B_INSTR = B_BYTES / 4096;  // per loader wave and k-tile
  constexpr int PT = A_INSTR + B_INSTR;
  constexpr int A_RPI = 1024 / AROW, B_RPI = 1024 / BROW;  // rows per DMA instruction
  constexpr int A_CPR = AROW / 16, B_CPR = BROW / 16;      // 16-byte chunks per row
  static_assert(WM * WN == 4 && TM % 32 == 0 && TN % 32 == 0, "wave grid");
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

  if (wave >= 4) {
    // ================= loader waves: the only waves that touch vmcnt for operands =================
    const int lw = wave - 4;
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
          const int n = min(n0 + r, N - 1);
          b_src[i] = wbase + (long)n * K * (FP8 ? 1 : 2) + (swz<BROW>(lane % B_CPR, r) << 4);
        }
      }
      char* st = smem + (s % STAGES) * STAGE;
#pragma unroll
      for (int i = 0; i < A_INSTR; ++i)
        dma16(a_src[i] + iss_kt * AROW, (lds_void*)(st + (lw * A_INSTR + i) * 1024));
#pragma unroll
      for (int i = 0; i < B_INSTR; ++i)
        dma16(b_src[i] + iss_kt * BROW, (lds_void*)(st + A_BYTES + (lw * B_INSTR + i) * 1024));
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
#pragma unroll 1
  for (int t = 0; t < my_items; ++t) {
    f32x16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.f;

    // deferred RMSNorm (QKV, FFN up): load this item's row partials now, so that they have
    // arrived by the epilogue. Chunks of four partials alternate between the half-waves;
    // chunks 0-3 (16 partials) are held through the k-loop, any beyond load in the epilogue.
    const float* ss_rows[MI];
    float4 ss_raw[MI][2];
    if (KIND != GEMM_FFN_DOWN && p.ss_in) {
      const int w = ib + t * nx;
      int mt, nt, g;
      tile_of(w, mt, nt, g);
      const int last_chunk = p.ss_stride / 4 - 1;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int row = min(mt * BM + wm * TM + mi * 32 + (lane & 31), M - 1);
        int seg, tt;
        split_row(row, rm.rows_per_seg, inv_rps, seg, tt);
        ss_rows[mi] = p.ss_in + hid_row(rm, seg, tt, g) * p.ss_stride;
#pragma unroll
        for (int j = 0; j < 2; ++j) ss_raw[mi][j] = *(const float4*)(ss_rows[mi] + 4 * min(2 * j + (lane >> 5), last_chunk));
      }
    }
    // FFN down with few accumulator blocks per wave: load the residual rows of this item now
    // as well (each element belongs to one item, so nothing writes them in between)
    constexpr bool X_EARLY = KIND == GEMM_FFN_DOWN && MI * NI <= 3;
    float4 x_pre[X_EARLY ? MI : 1][X_EARLY ? NI : 1][4];
    if constexpr (X_EARLY) {
      const int w = ib + t * nx;
      int mt, nt, g;
      tile_of(w, mt, nt, g);
      const int col = nt * BN + wn * TN + 4 * (lane >> 5);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int row = min(mt * BM + wm * TM + mi * 32 + (lane & 31), M - 1);
        int seg, tt;
        split_row(row, rm.rows_per_seg, inv_rps, seg, tt);
        const float* rrow = p.res_out + res_row_off(rm, seg, tt, g) + col;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int q = 0; q < 4; ++q) x_pre[mi][ni][q] = *(const float4*)(rrow + ni * 32 + 8 * q);
      }
    }
    // the partials of chunk c4 that exist (the rest of a row's slots may hold stale data)
    auto chunk_sum = [&](float4 v, int c4) {
      const int b = 4 * c4, n = p.ss_parts;
      return (b < n ? v.x : 0.f) + (b + 1 < n ? v.y : 0.f) + (b + 2 < n ? v.z : 0.f) + (b + 3 < n ? v.w : 0.f);
    };

#pragma unroll 1
    for (int kt = 0; kt < nk; ++kt) {
      const int s = t * nk + kt;
      lds_barrier();  // step s is in LDS
      const char* st = smem + (s % STAGES) * STAGE;
      // Fragments of a group of 16-wide k-steps are all read before its MFMAs: with one
      // register set per k-step the reads of step ks + 1 could only start after step ks's
      // MFMAs had consumed the registers, exposing the LDS latency at every k-step.
      constexpr int KS = BK / 16;
      constexpr int FG = MI + NI <= 4 ? KS : KS / 2;  // k-steps per group (register budget)
#pragma unroll
      for (int g0 = 0; g0 < KS; g0 += FG) {
        f16x8 a[FG][MI];
        f16x8 b[FG][NI];
        uint2 b8[FG][NI];
#pragma unroll
        for (int kk = 0; kk < FG; ++kk) {
          const int ks = g0 + kk;
          const int c = 2 * ks + (lane >> 5);
#pragma unroll
          for (int mi = 0; mi < MI; ++mi) {
            const int r = wm * TM + mi * 32 + (lane & 31);
            a[kk][mi] = *(const f16x8*)(st + r * AROW + (swz<AROW>(c, r) << 4));
          }
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            const int r = wn * TN + ni * 32 + (lane & 31);
            if (FP8)
              b8[kk][ni] = *(const uint2*)(st + A_BYTES + r * 64 + (swz<64>(ks, r) << 4) + (lane >> 5) * 8);
            else
              b[kk][ni] = *(const f16x8*)(st + A_BYTES + r * BROW + (swz<BROW>(c, r) << 4));
          }
        }
        __builtin_amdgcn_sched_barrier(0);  // keep every read of the group ahead of its MFMAs
#pragma unroll
        for (int kk = 0; kk < FG; ++kk) {
          if (FP8) {
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) b[kk][ni] = e4m3x8_to_f16(b8[kk][ni]);
          }
#pragma unroll
          for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b[kk][ni], a[kk][mi], acc[mi][ni], 0, 0, 0);
        }
      }
    }

    // ---- epilogue. With the weight fragment first in the MFMA, lane holds output row
    // (lane % 32) of each 32x32 block and, in registers 4q..4q+3, columns
    // 8q + 4*(lane/32) + 0..3. ----
    const int w = ib + t * nx;
    int mt, nt, g;
    tile_of(w, mt, nt, g);
    const int m0 = mt * BM, n0 = nt * BN;
    const float scale = FP8 ? p.wscale[g * 5 + p.scale_idx0 + n0 / p.scale_col_div] : 1.f;
    const int half = lane >> 5;
    const int col_l = n0 + wn * TN;                // + ni*32 + 8q + 4*half
    const int row_l = m0 + wm * TM + (lane & 31);  // + mi*32
    if (KIND == GEMM_FFN_DOWN) {
      // fp32 residual rows: read-modify-write 16 bytes per (block, register group); then
      // the next norm's operand x * g and one partial sum of squares per 32 columns
      const NormOut& no = p.nout;
      // the gains (the same columns for every row) before any store: a wait for a load
      // issued after a store also waits for that store
      float4 gv[NI][4];
      if (no.xg) {
        const float* grow = no.gain + (long)g * no.gain_group_stride + col_l + 4 * half;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int q = 0; q < 4; ++q) gv[ni][q] = *(const float4*)(grow + ni * 32 + 8 * q);
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int row = row_l + mi * 32;
        if (row >= M) continue;  // both half-waves hold the same row
        int seg, tt;
        split_row(row, rm.rows_per_seg, inv_rps, seg, tt);
        float* rrow = p.res_out + res_row_off(rm, seg, tt, g) + col_l + 4 * half;
        float4 x[NI][4];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if constexpr (X_EARLY) x[ni][q] = x_pre[mi][ni][q];
            else x[ni][q] = *(const float4*)(rrow + ni * 32 + 8 * q);
          }
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x16& a = acc[mi][ni];
            float4& v = x[ni][q];
            v.x += a[4 * q + 0] * scale;
            v.y += a[4 * q + 1] * scale;
            v.z += a[4 * q + 2] * scale;
            v.w += a[4 * q + 3] * scale;
            *(float4*)(rrow + ni * 32 + 8 * q) = v;
          }
        if (no.xg) {
          const long hr = hid_row(rm, seg, tt, g);
          _Float16* xrow = no.xg + hr * N + col_l + 4 * half;
          float* srow = no.ss + hr * no.ss_stride + (col_l >> 5);
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            float part = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 v = x[ni][q], gg = gv[ni][q];
              part += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
              const f16x4 o = {(_Float16)(v.x * gg.x), (_Float16)(v.y * gg.y), (_Float16)(v.z * gg.z),
                               (_Float16)(v.w * gg.w)};
              *(f16x4*)(xrow + ni * 32 + 8 * q) = o;
            }
            part += other_half(part);
            if (half == 0) srow[ni] = part;
          }
        }
      }
    } else {
      // ---- 16-bit outputs (Q / K / V, GELU hidden rows), straight from registers. Packed
      // to 16-bit pairs, groups q and q+1 trade halves across the two half-waves
      // (v_permlane32_swap), after which a lane holds 8 consecutive columns of one group:
      // one 16-byte store each. Rows are scaled by the deferred RMSNorm factor. ----
      auto pack2 = [&](float x, float y) -> uint32_t {
        if (KIND == GEMM_FFN_UP) {
          const _Float16 hx = (_Float16)x, hy = (_Float16)y;
          return (uint32_t)__builtin_bit_cast(uint16_t, hx) | ((uint32_t)__builtin_bit_cast(uint16_t, hy) << 16);
        }
        const __bf16 bx = (__bf16)x, by = (__bf16)y;
        return (uint32_t)__builtin_bit_cast(uint16_t, bx) | ((uint32_t)__builtin_bit_cast(uint16_t, by) << 16);
      };
      const int typ = KIND == GEMM_QKV ? n0 / p.d : 0;
      const bool vt_mode = KIND == GEMM_QKV && typ == 2 && p.vt != nullptr;
      const int dsh = p.dh == 64 ? 6 : 5;
      // every row factor before the first store: on gfx9 a wait for a load issued
      // after a store also waits for that store
      float srow[MI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        srow[mi] = scale;
        if (p.ss_in) {
          float sum = chunk_sum(ss_raw[mi][0], half) + chunk_sum(ss_raw[mi][1], 2 + half);
          for (int c4 = 4 + half; 4 * c4 < p.ss_parts; c4 += 2) sum += chunk_sum(*(const float4*)(ss_rows[mi] + 4 * c4), c4);
          sum += other_half(sum);
          srow[mi] *= 1.0f / sqrtf(sum / (float)K + p.eps);
        }
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int row = row_l + mi * 32;
        if (row >= M) continue;
        int seg, tt;
        split_row(row, rm.rows_per_seg, inv_rps, seg, tt);
        const float sr = srow[mi];
        auto val = [&](float x) { return KIND == GEMM_FFN_UP ? gelu_as(x * sr) : x * sr; };
        if (vt_mode) {
          // transposed V: lanes hold 32 consecutive key slots of each column
          __bf16* base = p.vt + seg * p.kv_seg_stride + p.kv_slot_base + (long)tt * rm.row_mult + g;
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int cc = col_l - typ * p.d + ni * 32 + 8 * q + 4 * half + e;
                base[(cc >> dsh) * p.kv_head_stride + (long)(cc & (p.dh - 1)) * p.kv_cap] =
                    (__bf16)val(acc[mi][ni][4 * q + e]);
              }
          continue;
        }
        long rbase;  // element offset of this row's first column (16-bit outputs)
        long head_stride = 0;
        __bf16* out = nullptr;
        if (KIND == GEMM_FFN_UP) {
          rbase = hid_row(rm, seg, tt, g) * N;
        } else {
          const long ti = (long)tt * rm.row_mult + g;
          if (typ == 0) {
            if (ti < p.q_from) continue;
            rbase = seg * p.q_seg_stride + (ti - p.q_from) * p.dh;
            head_stride = p.q_head_stride;
            out = p.q;
          } else {
            rbase = seg * p.kv_seg_stride + (p.kv_slot_base + ti) * p.dh;
            head_stride = p.kv_head_stride;
            out = typ == 1 ? p.k : p.v;
          }
        }
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int qq = 0; qq < 4; qq += 2) {
            const f32x16& v = acc[mi][ni];
            const int j0 = 4 * qq, j1 = 4 * qq + 4;
            const auto lo = __builtin_amdgcn_permlane32_swap(pack2(val(v[j0]), val(v[j0 + 1])),
                                                             pack2(val(v[j1]), val(v[j1 + 1])), false, false);
            const auto hi = __builtin_amdgcn_permlane32_swap(pack2(val(v[j0 + 2]), val(v[j0 + 3])),
                                                             pack2(val(v[j1 + 2]), val(v[j1 + 3])), false, false);
            const uint4 chunk = make_uint4(lo[0], hi[0], lo[1], hi[1]);
            const int c = col_l + ni * 32 + 8 * (qq + half);
            if (KIND == GEMM_FFN_UP) {
              *(uint4*)(p.hid_out + rbase + c) = chunk;
            } else {
              const int cc = c - typ * p.d;
              *(uint4*)(out + rbase + (cc >> dsh) * head_stride + (cc & (p.dh - 1))) = chunk;
            }
          }
      }
    }
  }
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

template <int KD, bool FP8, int SIDE, int BM, int BN, int WM>
void launch_one(const GemmParams& p, hipStream_t s) {
  const int tm = (p.M + BM - 1) / BM, tn = p.N / BN;
  const long items = (long)tm * tn * p.groups;
  const int grid = (int)(items < 256 ? items : 256);  // one workgroup per CU
  const int n_fast = (long)p.M > (long)p.N ? 1 : 0;  // a group's rows: activations M x K, weights N x K
  hipLaunchKernelGGL((gemm_kernel<KD, FP8, SIDE, BM, BN, stages_for<KD, BM, BN, WM, FP8>(), WM>), dim3(grid), dim3(512), 0, s,
                     p, tm, tn, (int)items, n_fast);
}

template <int KD, int SIDE, int BM, int BN, int WM>
void launch_cfg(bool fp8, const GemmParams& p, hipStream_t s) {
  if constexpr (SIDE == 1 && BN != 96) {
    if (fp8) {
      launch_one<KD, true, SIDE, BM, BN, WM>(p, s);
      return;
    }
  }
  launch_one<KD, false, SIDE, BM, BN, WM>(p, s);
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
  auto fits = [&](int bn) { return p.N % bn == 0 && (KD != GEMM_QKV || p.d % bn == 0) && !(fp8 && bn == 96); };
  // ties go to the earlier entry: the smaller tile, which leaves fewer CUs idle in the last round
  const TileCfg cands[6] = {{128, 96}, {128, 128}, {256, 96}, {256, 128}, {128, 64}, {64, 64}};
  int best = -1;
  double best_cost = 0;
  for (int i = 0; i < 6; ++i) {
    if (!fits(cands[i].bn)) continue;
    const double c = tile_cost(p, fp8, cands[i].bm, cands[i].bn);
    if (best < 0 || c < best_cost) { best = i; best_cost = c; }
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
