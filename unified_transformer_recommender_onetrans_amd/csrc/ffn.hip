// Fused pre-norm FFN of the NS tokens on gfx950 (fp16 / E4M3 weights, fp32 accumulate).
//
// For NS position k (private weights; agihunt.info OneTrans summary, "method")
// and a block of BM = 64 candidates, one workgroup of 8 waves computes
//   y = z + W2_k GELU(W1_k RMSNorm(z; g_ffn,k))
// without writing the hidden activations anywhere:
//   prologue  z rows -> RMSNorm -> fp16 MFMA A-fragments held in registers for the
//             whole kernel (the lane pair (l, l ^ 32) covers one full row)
//   per chunk of FC = 128 hidden units:
//     W1 phase: h = Xs W1_k[chunk]^T      (64 x 128: one 32x32 block per wave)
//     Hs = fp16 GELU(h)                    (LDS)
//     W2 phase: acc += Hs W2_k[:, chunk]^T (64 x D accumulated in registers)
//   epilogue  y = z + acc written back in place; when the next layer's gain is
//             given, its attention pre-norm RMSNorm(y; g_attn,k) is written as
//             fp16 rows for the next QKV projection (the rows are complete here).
// Weight tiles stream global -> LDS with global_load_lds_dwordx4, STAGES - 1 = 4
// tiles (~96 KB) in flight, which is what a CU needs to pull cache-resident data
// at full rate; their rows are XOR-swizzled in 16-byte chunks and read with the
// asm helpers of internal.h. Hs rows are padded by 16 bytes, which makes the
// 16-lane fragment reads bank-conflict free. The tile loops inside a chunk are
// unrolled so every LDS offset except the stage base is a compile-time immediate.
#include <math.h>

#include <type_traits>

#include "internal.h"

namespace onetrans {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 64, FC = 128, WAVES = 8, STAGES = 5;

template <int I, int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  if constexpr (I < N) {
    fn(std::integral_constant<int, I>());
    static_for<I + 1, N>(fn);
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ long res_row_off(const RowMap& rm, int seg, int t, int g) {
  return (long)seg * rm.res_seg_stride + (rm.res_row_base + t) * rm.res_row_stride + (long)g * rm.res_group_stride;
}
__device__ __forceinline__ void split_row(int row, int rps, float inv_rps, int& seg, int& t) {
  seg = (int)((float)row * inv_rps);
  t = row - seg * rps;
  if (t < 0) { --seg; t += rps; }
  else if (t >= rps) { ++seg; t -= rps; }
}

// Exact E4M3FN -> fp16 (see gemm.hip for the derivation).
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
__device__ __forceinline__ f16x8 e4m3x8_to_f16(u32x2 c) {
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t a = e4m3x2_to_f16x2(c[i] & 0x00FF00FFu);
    const uint32_t b = e4m3x2_to_f16x2((c[i] >> 8) & 0x00FF00FFu);
    out[2 * i] = (a & 0xFFFFu) | (b << 16);
    out[2 * i + 1] = (a >> 16) | (b & 0xFFFF0000u);
  }
  return __builtin_bit_cast(f16x8, make_uint4(out[0], out[1], out[2], out[3]));
}

template <int D, bool FP8>
__global__ __launch_bounds__(512) void ffn_fused_kernel(FfnParams p, int n_mt) {
  constexpr int EB = FP8 ? 1 : 2;                 // weight bytes per element
  constexpr int NB = D / 128;                     // 32-column output blocks per wave
  constexpr int W1_TILE = FC * 128;               // 128 hidden rows x 128 B of k
  constexpr int W2_TILE = D * 64;                 // D output rows x 64 B of k
  constexpr int STAGE = W1_TILE > W2_TILE ? W1_TILE : W2_TILE;
  constexpr int W1_INSTR = W1_TILE / 1024 / WAVES;
  constexpr int W2_INSTR = W2_TILE / 1024 / WAVES;
  constexpr int N_W1 = D * EB / 128;              // W1 tiles per chunk
  constexpr int N_W2 = FC * EB / 64;              // W2 tiles per chunk
  constexpr int TPC = N_W1 + N_W2;
  constexpr int K1 = 128 / EB, K2 = 64 / EB;      // k per tile
  constexpr int S1 = K1 / 16, S2 = K2 / 16;       // MFMA k-steps per tile
  constexpr int HROW = FC * 2 + 16;                // padded row bytes
  constexpr int KS = D / 16;                      // k-steps over the model width
  static_assert(W1_INSTR >= 1 && W2_INSTR >= 1 && S1 % 4 == 0 && NB <= 3, "tile split");
  __shared__ __attribute__((aligned(1024))) char ring[STAGES * STAGE];
  __shared__ __attribute__((aligned(16))) char Hs[BM * HROW];
  __shared__ float red[4][BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  // XCD-aware order: the row blocks of one NS position are consecutive work items
  const int total = gridDim.x, L = blockIdx.x;
  const int xcd = L % 8, local = L / 8, per = total / 8, rem = total % 8;
  const int w = xcd * per + min(xcd, rem) + local;
  const int mt = w % n_mt, g = w / n_mt;
  const int m0 = mt * BM;
  const RowMap rm = p.rm;
  const float inv_rps = 1.0f / (float)rm.rows_per_seg;
  const int n_chunks = p.F / FC;
  const int T = n_chunks * TPC;

  // ---- DMA sources (per lane) ----
  const char* w1 = (const char*)p.w1 + (long)g * p.w1_group_stride * EB;
  const char* w2 = (const char*)p.w2 + (long)g * p.w2_group_stride * EB;
  long w1_off[W1_INSTR], w2_off[W2_INSTR];
#pragma unroll
  for (int i = 0; i < W1_INSTR; ++i) {
    const int r = (wave * W1_INSTR + i) * 8 + (lane >> 3);
    w1_off[i] = (long)r * D * EB + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
  }
#pragma unroll
  for (int i = 0; i < W2_INSTR; ++i) {
    const int r = (wave * W2_INSTR + i) * 16 + (lane >> 2);
    w2_off[i] = (long)r * p.F * EB + (((lane & 3) ^ ((r >> 2) & 3)) << 4);
  }
  // tile tc (wave-uniform): chunk tc / TPC, tile u = tc % TPC; W1 tiles first, then W2
  auto issue = [&](int tc) {
    if (tc >= T) return;
    const int f = tc / TPC, u = tc - f * TPC;
    char* sb = ring + (tc % STAGES) * STAGE;
    if (u < N_W1) {
      const char* src = w1 + (long)f * FC * D * EB + u * 128;
#pragma unroll
      for (int i = 0; i < W1_INSTR; ++i) dma16(src + w1_off[i], (lds_void*)(sb + (wave * W1_INSTR + i) * 1024));
    } else {
      const char* src = w2 + (long)f * FC * EB + (u - N_W1) * 64;
#pragma unroll
      for (int i = 0; i < W2_INSTR; ++i) dma16(src + w2_off[i], (lds_void*)(sb + (wave * W2_INSTR + i) * 1024));
    }
  };
#pragma unroll
  for (int t = 0; t < STAGES - 1; ++t) issue(t);

  const int rb = wave & 1, cb = wave >> 1;       // h block of this wave (rows 32rb, hidden cols 32cb)
  const int wr = wave & 1, wc = wave >> 1;       // output rows 32wr, columns wc*D/4 .. +D/4

  // ---- prologue: A fragments xf[ks] = fp16 RMSNorm(z)[row 32rb + l32][16 ks + 8 half .. +8] ----
  f16x8 xf[KS];
  {
    const int row = min(m0 + rb * 32 + l32, p.M - 1);
    int seg, t;
    split_row(row, rm.rows_per_seg, inv_rps, seg, t);
    const float* src = p.res + res_row_off(rm, seg, t, g) + half * 8;
    const float* gain = p.gain + (long)g * p.gain_group_stride + half * 8;
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float4 a = *(const float4*)(src + ks * 16), b = *(const float4*)(src + ks * 16 + 4);
      ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w + b.x * b.x + b.y * b.y + b.z * b.z + b.w * b.w;
    }
    ss += __shfl_xor(ss, 32);  // the partner lane holds the other half of the row
    const float ri = 1.0f / sqrtf(ss / (float)D + p.eps);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float4 a = *(const float4*)(src + ks * 16), b = *(const float4*)(src + ks * 16 + 4);
      const float4 ga = *(const float4*)(gain + ks * 16), gb = *(const float4*)(gain + ks * 16 + 4);
      xf[ks] = f16x8{(_Float16)(a.x * ri * ga.x), (_Float16)(a.y * ri * ga.y), (_Float16)(a.z * ri * ga.z),
                     (_Float16)(a.w * ri * ga.w), (_Float16)(b.x * ri * gb.x), (_Float16)(b.y * ri * gb.y),
                     (_Float16)(b.z * ri * gb.z), (_Float16)(b.w * ri * gb.w)};
    }
  }

  // ---- per-lane LDS read offsets ----
  const char* ha = Hs + (wr * 32 + l32) * HROW + half * 16;
  uint32_t b1[S1];
  {
    const int br = cb * 32 + l32;
#pragma unroll
    for (int s = 0; s < S1; ++s)
      b1[s] = br * 128 + (FP8 ? (((s ^ ((br >> 1) & 7)) << 4) + half * 8) : (((2 * s + half) ^ ((br >> 1) & 7)) << 4));
  }
  uint32_t b2[3][S2];
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    const int br = wc * (D / 4) + (b < NB ? b : 0) * 32 + l32;
#pragma unroll
    for (int s = 0; s < S2; ++s)
      b2[b][s] = br * 64 + (FP8 ? (((s ^ ((br >> 2) & 3)) << 4) + half * 8) : (((2 * s + half) ^ ((br >> 2) & 3)) << 4));
  }
  const uint32_t ring_lds = lds_addr(ring);
  const float s1 = FP8 ? p.wscale[g * 5 + 3] : 1.f;
  const float s2 = FP8 ? p.wscale[g * 5 + 4] : 1.f;

  f32x16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[b][j] = 0.f;

  // DMA ops per wave of the tile at chunk position u, and of the STAGES - 2 tiles after it
  constexpr auto instr_at = [](int u) constexpr { return (u % TPC) < N_W1 ? W1_INSTR : W2_INSTR; };
  // wait until tile tc (chunk position U) has landed while the later tiles stay in
  // flight, sync, then send tile tc + STAGES - 1
  auto begin_tile = [&](int tc, auto U) -> uint32_t {
    constexpr int u = decltype(U)::value;
    constexpr int ahead = [&]() constexpr {
      int a = 0;
      for (int i = 1; i <= STAGES - 2; ++i) a += instr_at(u + i);
      return a;
    }();
    if (tc + STAGES - 2 < T) wait_vmcnt<ahead>();
    else wait_vmcnt<0>();
    lds_barrier();
    issue(tc + STAGES - 1);
    return ring_lds + (tc % STAGES) * STAGE;
  };

#pragma unroll 1
  for (int f = 0; f < n_chunks; ++f) {
    const int tc0 = f * TPC;
    // ---- W1 phase ----
    f32x16 hacc;
#pragma unroll
    for (int j = 0; j < 16; ++j) hacc[j] = 0.f;
    static_for<0, N_W1>([&](auto U) {
      constexpr int u = decltype(U)::value;
      const uint32_t sb = begin_tile(tc0 + u, U);
      f16x8 bv[S1];
      if (FP8) {
        u32x2 raw[S1];
#pragma unroll
        for (int s = 0; s < S1; s += 4)
          lds_read_b64x4(raw[s], raw[s + 1], raw[s + 2], raw[s + 3], sb + b1[s], sb + b1[s + 1], sb + b1[s + 2],
                         sb + b1[s + 3]);
#pragma unroll
        for (int s = 0; s < S1; ++s) bv[s] = e4m3x8_to_f16(raw[s]);
      } else {
        u32x4 raw[S1];
#pragma unroll
        for (int s = 0; s < S1; s += 4)
          lds_read_b128x4(raw[s], raw[s + 1], raw[s + 2], raw[s + 3], sb + b1[s], sb + b1[s + 1], sb + b1[s + 2],
                          sb + b1[s + 3]);
#pragma unroll
        for (int s = 0; s < S1; ++s) bv[s] = __builtin_bit_cast(f16x8, raw[s]);
      }
#pragma unroll
      for (int s = 0; s < S1; ++s) hacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(xf[u * S1 + s], bv[s], hacc, 0, 0, 0);
    });
    // GELU -> Hs (lane holds hidden col 32cb + l32, rows 32rb + 8(j/4) + 4half + j%4)
    {
      char* hw = Hs + (rb * 32 + half * 4) * HROW + (cb * 32 + l32) * 2;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        *(_Float16*)(hw + (8 * (j >> 2) + (j & 3)) * HROW) = (_Float16)gelu_as(hacc[j] * s1);
    }
    // ---- W2 phase ----
    static_for<0, N_W2>([&](auto J) {
      constexpr int j2 = decltype(J)::value;
      const uint32_t sb = begin_tile(tc0 + N_W1 + j2, std::integral_constant<int, N_W1 + j2>());
#pragma unroll
      for (int s = 0; s < S2; ++s) {
        const f16x8 a = *(const f16x8*)(ha + (j2 * K2 + s * 16) * 2);
        f16x8 bv[3];
        if (FP8) {
          u32x2 raw[4];
          lds_read_b64x4(raw[0], raw[1], raw[2], raw[3], sb + b2[0][s], sb + b2[1][s], sb + b2[2][s], sb + b2[0][s]);
#pragma unroll
          for (int b = 0; b < NB; ++b) bv[b] = e4m3x8_to_f16(raw[b]);
        } else {
          u32x4 raw[3];
          if (NB == 3) lds_read_b128x3(raw[0], raw[1], raw[2], sb + b2[0][s], sb + b2[1][s], sb + b2[2][s]);
          else if (NB == 2) lds_read_b128x2(raw[0], raw[1], sb + b2[0][s], sb + b2[1][s]);
          else lds_read_b128x1(raw[0], sb + b2[0][s]);
#pragma unroll
          for (int b = 0; b < NB; ++b) bv[b] = __builtin_bit_cast(f16x8, raw[b]);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bv[b], acc[b], 0, 0, 0);
      }
    });
  }

  // ---- epilogue: y = z + s2 * acc in place, then (optionally) the next pre-norm ----
  float ss[16];
  float y[NB][16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = wr * 32 + 8 * (j >> 2) + half * 4 + (j & 3);
    const int row = m0 + r;
    const bool ok = row < p.M;
    int seg, t;
    split_row(ok ? row : 0, rm.rows_per_seg, inv_rps, seg, t);
    float* dst = p.res + res_row_off(rm, seg, t, g) + wc * (D / 4) + l32;
    ss[j] = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float v = 0.f;
      if (ok) {
        v = dst[b * 32] + s2 * acc[b][j];
        dst[b * 32] = v;
      }
      y[b][j] = v;
      ss[j] += v * v;
    }
  }
  if (p.next_xn != nullptr) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) ss[j] += __shfl_xor(ss[j], off);
    }
    if (l32 == 0) {
#pragma unroll
      for (int j = 0; j < 16; ++j) red[wc][wr * 32 + 8 * (j >> 2) + half * 4 + (j & 3)] = ss[j];
    }
    __syncthreads();
    const float* gn = p.next_gain + (long)g * p.gain_group_stride + wc * (D / 4) + l32;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = wr * 32 + 8 * (j >> 2) + half * 4 + (j & 3);
      const int row = m0 + r;
      if (row >= p.M) continue;
      const float tot = red[0][r] + red[1][r] + red[2][r] + red[3][r];
      const float ri = 1.0f / sqrtf(tot / (float)D + p.eps);
      int seg, t;
      split_row(row, rm.rows_per_seg, inv_rps, seg, t);
      _Float16* dst = p.next_xn + (((long)seg * rm.rows_per_seg + t) * rm.row_mult + g) * D + wc * (D / 4) + l32;
#pragma unroll
      for (int b = 0; b < NB; ++b) dst[b * 32] = (_Float16)(y[b][j] * ri * gn[b * 32]);
    }
  }
}

template <int D>
void launch_d(bool fp8, const FfnParams& p, hipStream_t s) {
  const int n_mt = (p.M + BM - 1) / BM;
  dim3 grid(n_mt * p.groups), block(512);
  if (fp8) hipLaunchKernelGGL((ffn_fused_kernel<D, true>), grid, block, 0, s, p, n_mt);
  else hipLaunchKernelGGL((ffn_fused_kernel<D, false>), grid, block, 0, s, p, n_mt);
}

}  // namespace

bool ffn_fused_supported(int d, int F) { return (d == 128 || d == 256 || d == 384) && F % FC == 0; }

hipError_t launch_ffn_fused(bool fp8, const FfnParams& p, hipStream_t s) {
  if (p.M <= 0 || p.groups <= 0) return hipSuccess;
  if (!ffn_fused_supported(p.d, p.F)) return hipErrorInvalidValue;
  if (p.d == 384) launch_d<384>(fp8, p, s);
  else if (p.d == 256) launch_d<256>(fp8, p, s);
  else launch_d<128>(fp8, p, s);
  return hipGetLastError();
}

}  // namespace onetrans
