// Pieces of the grouped GEMM (gemm.hip) kept apart from its main loop: row addressing, the
// k-tile wait and barrier helpers, the LDS swizzle, E4M3 decoding, and the per-tile work
// around the k-loop (row-factor prefetch, fused epilogues).
//
// Output layout of the k-loop. With the weight fragment as the first MFMA operand
// (v_mfma_f32_32x32x16_f16), lane l of a wave holds output row (l % 32) of each 32x32 block
// and, in registers 4q..4q+3, columns 8q + 4*(l/32) + 0..3. A wave owns MI x NI such blocks
// of a TM x TN part of the BM x BN tile.
#pragma once
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

// Global loads a tile's epilogue needs, issued before its k-loop so they arrive under it:
// the deferred RMSNorm partials of the tile's rows (QKV, FFN up) and, for FFN down with few
// accumulator blocks per wave, the residual rows it updates (each element belongs to one
// tile, so nothing writes them in between).
template <int KIND, int MI, int NI>
struct TilePre {
  static constexpr bool X_EARLY = KIND == GEMM_FFN_DOWN && MI * NI <= 3;
  const float* ss_rows[MI];
  float4 ss_raw[MI][2];
  float4 x_pre[X_EARLY ? MI : 1][X_EARLY ? NI : 1][4];
};

template <int KIND, int MI, int NI, int TM, int TN>
__device__ __forceinline__ void tile_prefetch(const GemmParams& p, int m0, int n0, int g, int wm, int wn,
                                              TilePre<KIND, MI, NI>& pre) {
  const int lane = threadIdx.x & 63;
  const RowMap& rm = p.rm;
  const float inv_rps = 1.0f / (float)rm.rows_per_seg;
  // row partials: chunks of four alternate between the half-waves; chunks 0-3 (16 partials)
  // are held through the k-loop, any beyond load in the epilogue
  if (KIND != GEMM_FFN_DOWN && p.ss_in) {
    const int last_chunk = p.ss_stride / 4 - 1;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int row = min(m0 + wm * TM + mi * 32 + (lane & 31), p.M - 1);
      int seg, tt;
      split_row(row, rm.rows_per_seg, inv_rps, seg, tt);
      pre.ss_rows[mi] = p.ss_in + hid_row(rm, seg, tt, g) * p.ss_stride;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        pre.ss_raw[mi][j] = *(const float4*)(pre.ss_rows[mi] + 4 * min(2 * j + (lane >> 5), last_chunk));
    }
  }
  if constexpr (TilePre<KIND, MI, NI>::X_EARLY) {
    const int col = n0 + wn * TN + 4 * (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int row = min(m0 + wm * TM + mi * 32 + (lane & 31), p.M - 1);
      int seg, tt;
      split_row(row, rm.rows_per_seg, inv_rps, seg, tt);
      const float* rrow = p.res_out + res_row_off(rm, seg, tt, g) + col;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int q = 0; q < 4; ++q) pre.x_pre[mi][ni][q] = *(const float4*)(rrow + ni * 32 + 8 * q);
    }
  }
}

// The fused epilogue of one tile (the accumulators of this wave's blocks):
//   QKV: row factor r of the deferred RMSNorm, bf16 Q / K / V scattered to their head
//        layouts (V transposed for the S cache);
//   FFN up: GELU(r * acc) as fp16 hidden rows;
//   FFN down: fp32 residual rows updated in place, then the next norm's operand x * g and
//        one partial sum of squares per 32 columns.
template <int KIND, bool FP8, int MI, int NI, int TM, int TN>
__device__ __forceinline__ void tile_epilogue(const GemmParams& p, const f32x16 (&acc)[MI][NI], int m0, int n0, int g,
                                              int wm, int wn, TilePre<KIND, MI, NI>& pre) {
  const int lane = threadIdx.x & 63;
  const RowMap& rm = p.rm;
  const int M = p.M, N = p.N, K = p.K;
  const float inv_rps = 1.0f / (float)rm.rows_per_seg;
  const float scale = FP8 ? p.wscale[g * 5 + p.scale_idx0 + n0 / p.scale_col_div] : 1.f;
  const int half = lane >> 5;
  const int col_l = n0 + wn * TN;                // + ni*32 + 8q + 4*half
  const int row_l = m0 + wm * TM + (lane & 31);  // + mi*32
  // the partials of chunk c4 that exist (the rest of a row's slots may hold stale data)
  auto chunk_sum = [&](float4 v, int c4) {
    const int b = 4 * c4, n = p.ss_parts;
    return (b < n ? v.x : 0.f) + (b + 1 < n ? v.y : 0.f) + (b + 2 < n ? v.z : 0.f) + (b + 3 < n ? v.w : 0.f);
  };
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
          if constexpr (TilePre<KIND, MI, NI>::X_EARLY) x[ni][q] = pre.x_pre[mi][ni][q];
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
        float sum = chunk_sum(pre.ss_raw[mi][0], half) + chunk_sum(pre.ss_raw[mi][1], 2 + half);
        for (int c4 = 4 + half; 4 * c4 < p.ss_parts; c4 += 2)
          sum += chunk_sum(*(const float4*)(pre.ss_rows[mi] + 4 * c4), c4);
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

}  // namespace
}  // namespace onetrans
