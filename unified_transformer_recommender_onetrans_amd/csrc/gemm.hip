// Grouped GEMMs of the OneTrans block on gfx950 MFMA (fp16 operands, fp32 accumulate).
//
// One kernel template covers the five linear maps of a layer (agihunt.info
// OneTrans summary, "method": shared S-token QKV/FFN, private per-NS-position
// QKV/FFN, RMSNorm pre-norm):
//   GEMM_QKV      : A = RMSNorm(residual rows) -> fp16, B = W_QKV [3d][d];
//                   epilogue scatters bf16 Q / K / V^T into the attention layouts
//   GEMM_FFN_UP   : A = RMSNorm(residual rows) -> fp16, B = W1 [F][d];
//                   epilogue GELU(erf) -> fp16 hidden rows
//   GEMM_FFN_DOWN : A = fp16 hidden rows, B = W2 [d][F];
//                   epilogue adds into the fp32 residual rows in place
// blockIdx.z selects the group (the NS position for private weights; 0 for the
// shared S weights). Tiles: 128x128 per workgroup of 4 waves, each wave 64x64 as
// 2x2 blocks of v_mfma_f32_32x32x16_f16, K staged through LDS 64 at a time with
// the next tile's global loads in flight during the MFMAs.
#include "internal.h"

namespace onetrans {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_LD = BK + 8;  // halfs per LDS row (padding breaks bank conflicts)

__device__ __forceinline__ long res_row_off(const RowMap& rm, int seg, int t, int g) {
  return (long)seg * rm.res_seg_stride + (rm.res_row_base + t) * rm.res_row_stride + (long)g * rm.res_group_stride;
}
__device__ __forceinline__ long hid_row(const RowMap& rm, int seg, int t, int g) {
  return ((long)seg * rm.rows_per_seg + t) * rm.row_mult + g;
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

// 16 E4M3 codes (one uint4) -> 16 halfs (two uint4), in order.
__device__ __forceinline__ void e4m3x16_to_f16(uint4 c, uint4& lo, uint4& hi) {
  uint32_t in[4] = {c.x, c.y, c.z, c.w};
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t a = e4m3x2_to_f16x2(in[i] & 0x00FF00FFu);         // codes 0, 2
    uint32_t b = e4m3x2_to_f16x2((in[i] >> 8) & 0x00FF00FFu);  // codes 1, 3
    out[2 * i] = (a & 0xFFFFu) | (b << 16);
    out[2 * i + 1] = (a >> 16) | (b & 0xFFFF0000u);
  }
  lo = make_uint4(out[0], out[1], out[2], out[3]);
  hi = make_uint4(out[4], out[5], out[6], out[7]);
}

__device__ __forceinline__ float gelu_erf(float v) { return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f)); }

template <int KIND, bool FP8>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p) {
  constexpr bool NORM = (KIND != GEMM_FFN_DOWN);
  __shared__ __attribute__((aligned(16))) _Float16 As[BM * LDS_LD];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[BN * LDS_LD];
  __shared__ float rinv_s[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM, g = blockIdx.z;
  const RowMap rm = p.rm;
  const int M = p.M, N = p.N, K = p.K;

  // ---- A row offsets owned by this thread ----
  // norm mode: 8 rows (tid>>4) + 16i, float4 column chunk tid&15
  // plain mode: 4 rows (tid>>3) + 32i, 8-half chunk tid&7
  constexpr int A_ROWS = NORM ? 8 : 4;
  long a_off[A_ROWS];
  bool a_ok[A_ROWS];
#pragma unroll
  for (int i = 0; i < A_ROWS; ++i) {
    int r = NORM ? ((tid >> 4) + 16 * i) : ((tid >> 3) + 32 * i);
    int row = m0 + r;
    a_ok[i] = row < M;
    int rr = a_ok[i] ? row : 0;
    int seg = rr / rm.rows_per_seg, t = rr - seg * rm.rows_per_seg;
    a_off[i] = NORM ? res_row_off(rm, seg, t, g) : hid_row(rm, seg, t, g) * (long)K;
  }
  const float* gain = NORM ? (p.gain + (long)g * p.gain_group_stride) : nullptr;

  // ---- RMSNorm prologue: 1/rms of the workgroup's rows (16 lanes per row) ----
  if (NORM) {
    const int sub = tid & 15;
#pragma unroll 1
    for (int pass = 0; pass < BM / 16; ++pass) {
      int r = (tid >> 4) + 16 * pass;
      int row = m0 + r;
      float ss = 0.f;
      if (row < M) {
        int seg = row / rm.rows_per_seg, t = row - seg * rm.rows_per_seg;
        const float* src = p.res_in + res_row_off(rm, seg, t, g);
        for (int c = sub * 4; c < K; c += 64) {
          float4 v = *(const float4*)(src + c);
          ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        }
      }
      ss += __shfl_xor(ss, 8);
      ss += __shfl_xor(ss, 4);
      ss += __shfl_xor(ss, 2);
      ss += __shfl_xor(ss, 1);
      if (sub == 0) rinv_s[r] = (row < M) ? 1.0f / sqrtf(ss / (float)K + p.eps) : 0.f;
    }
    __syncthreads();
  }

  // ---- B row offsets: fp16 4 rows (tid>>3)+32i chunk tid&7; fp8 2 rows (tid>>2)+64i chunk tid&3 ----
  constexpr int B_ROWS = FP8 ? 2 : 4;
  const char* wbase = (const char*)p.w + (long)g * p.w_group_stride * (FP8 ? 1 : 2);
  long b_off[B_ROWS];
  bool b_ok[B_ROWS];
#pragma unroll
  for (int i = 0; i < B_ROWS; ++i) {
    int n = FP8 ? ((tid >> 2) + 64 * i) : ((tid >> 3) + 32 * i);
    b_ok[i] = (n0 + n) < N;
    b_off[i] = (long)(b_ok[i] ? (n0 + n) : 0) * K;
  }

  float4 areg_f[NORM ? 8 : 1];
  uint4 areg_h[NORM ? 1 : 4];
  uint4 breg[B_ROWS];

  auto load_global = [&](int k0) {
    if (NORM) {
      const int c = k0 + (tid & 15) * 4;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        areg_f[i] = a_ok[i] ? *(const float4*)(p.res_in + a_off[i] + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      const int c = k0 + (tid & 7) * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        areg_h[i] = a_ok[i] ? *(const uint4*)(p.hid_in + a_off[i] + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_ROWS; ++i) {
      if (FP8) {
        const int c = k0 + (tid & 3) * 16;
        breg[i] = b_ok[i] ? *(const uint4*)(wbase + b_off[i] + c) : make_uint4(0, 0, 0, 0);
      } else {
        const int c = k0 + (tid & 7) * 8;
        breg[i] = b_ok[i] ? *(const uint4*)(wbase + (b_off[i] + c) * 2) : make_uint4(0, 0, 0, 0);
      }
    }
  };

  auto store_lds = [&](int k0) {
    if (NORM) {
      const int cc = (tid & 15) * 4;
      const float4 gv = *(const float4*)(gain + k0 + cc);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = (tid >> 4) + 16 * i;
        const float s = rinv_s[r];
        f16x4 hv;
        hv[0] = (_Float16)(areg_f[i].x * s * gv.x);
        hv[1] = (_Float16)(areg_f[i].y * s * gv.y);
        hv[2] = (_Float16)(areg_f[i].z * s * gv.z);
        hv[3] = (_Float16)(areg_f[i].w * s * gv.w);
        *(f16x4*)&As[r * LDS_LD + cc] = hv;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 3) + 32 * i;
        *(uint4*)&As[r * LDS_LD + (tid & 7) * 8] = areg_h[i];
      }
    }
#pragma unroll
    for (int i = 0; i < B_ROWS; ++i) {
      if (FP8) {
        const int r = (tid >> 2) + 64 * i;
        uint4 lo, hi;
        e4m3x16_to_f16(breg[i], lo, hi);
        *(uint4*)&Bs[r * LDS_LD + (tid & 3) * 16] = lo;
        *(uint4*)&Bs[r * LDS_LD + (tid & 3) * 16 + 8] = hi;
      } else {
        const int r = (tid >> 3) + 32 * i;
        *(uint4*)&Bs[r * LDS_LD + (tid & 7) * 8] = breg[i];
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.f;

  load_global(0);
#pragma unroll 1
  for (int k0 = 0; k0 < K; k0 += BK) {
    store_lds(k0);
    __syncthreads();
    if (k0 + BK < K) load_global(k0 + BK);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      f16x8 a[2], b[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        a[mi] = *(const f16x8*)&As[(wm * 64 + mi * 32 + (lane & 31)) * LDS_LD + s * 16 + (lane >> 5) * 8];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        b[ni] = *(const f16x8*)&Bs[(wn * 64 + ni * 32 + (lane & 31)) * LDS_LD + s * 16 + (lane >> 5) * 8];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- epilogue ----
  // lane holds, per 32x32 block, column lane&31 and rows 8*(j/4) + (lane/32)*4 + j%4
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    const int col = n0 + wn * 64 + ni * 32 + (lane & 31);
    if (col >= N) continue;
    float scale = 1.f;
    if (FP8) scale = p.wscale[g * 5 + p.scale_idx0 + col / p.scale_col_div];
    int typ = 0, head = 0, jj = 0;
    if (KIND == GEMM_QKV) {
      typ = col / p.d;
      const int within = col - typ * p.d;
      head = within / p.dh;
      jj = within - head * p.dh;
    }
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int row = m0 + wm * 64 + mi * 32 + 8 * (j >> 2) + (lane >> 5) * 4 + (j & 3);
        if (row >= M) continue;
        const float v = acc[mi][ni][j] * scale;
        const int seg = row / rm.rows_per_seg, t = row - seg * rm.rows_per_seg;
        if (KIND == GEMM_QKV) {
          const int ti = t * rm.row_mult + g;
          if (typ == 0) {
            const int qi = ti - p.q_from;
            if (qi >= 0) p.q[seg * p.q_seg_stride + head * p.q_head_stride + (long)qi * p.dh + jj] = (__bf16)v;
          } else {
            const long base = seg * p.kv_seg_stride + head * p.kv_head_stride;
            const long ki = p.kv_slot_base + ti;
            if (typ == 1) p.k[base + ki * p.dh + jj] = (__bf16)v;
            else p.vt[base + (long)jj * p.kv_cap + ki] = (__bf16)v;
          }
        } else if (KIND == GEMM_FFN_UP) {
          p.hid_out[hid_row(rm, seg, t, g) * N + col] = (_Float16)gelu_erf(v);
        } else {
          float* dst = p.res_out + res_row_off(rm, seg, t, g) + col;
          *dst = *dst + v;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(GemmKind kind, bool fp8, const GemmParams& p, hipStream_t s) {
  if (p.M <= 0 || p.groups <= 0) return hipSuccess;
  dim3 grid((p.N + BN - 1) / BN, (p.M + BM - 1) / BM, p.groups);
  dim3 block(256);
#define OT_LAUNCH(KD, F8) hipLaunchKernelGGL((gemm_kernel<KD, F8>), grid, block, 0, s, p)
  if (kind == GEMM_QKV) { if (fp8) OT_LAUNCH(GEMM_QKV, true); else OT_LAUNCH(GEMM_QKV, false); }
  else if (kind == GEMM_FFN_UP) { if (fp8) OT_LAUNCH(GEMM_FFN_UP, true); else OT_LAUNCH(GEMM_FFN_UP, false); }
  else { if (fp8) OT_LAUNCH(GEMM_FFN_DOWN, true); else OT_LAUNCH(GEMM_FFN_DOWN, false); }
#undef OT_LAUNCH
  return hipGetLastError();
}

}  // namespace onetrans
