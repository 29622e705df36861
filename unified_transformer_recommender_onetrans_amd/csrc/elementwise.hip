// Small bandwidth-bound helpers: weight packing, input conversion, output copies.
#include "internal.h"

namespace onetrans {
namespace {

// bf16 -> fp16, 8 elements per thread (exact for |w| >= 2^-17; below that the
// fp16 subnormal grid rounds to nearest even).
__global__ void bf16_to_f16_kernel(const uint16_t* __restrict__ src, _Float16* __restrict__ dst, long n) {
  const long i0 = ((long)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i0 + 8 <= n) {
    const uint4 v = *(const uint4*)(src + i0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    _Float16 o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = (_Float16)__builtin_bit_cast(float, w[i] << 16);
      o[2 * i + 1] = (_Float16)__builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    }
    *(uint4*)(dst + i0) = *(const uint4*)o;
  } else {
    for (long i = i0; i < n; ++i) dst[i] = (_Float16)__builtin_bit_cast(float, (uint32_t)src[i] << 16);
  }
}

// Weight matrices [G][N][K] (row n = output column of the linear map) into panels
// [G][N/32][K/64][32][64]: every 32-row, 64-wide block is one contiguous 4 KB (fp16) or
// 2 KB (E4M3) run, so a GEMM k-tile of a weight tile reads whole contiguous blocks instead
// of 64- or 128-byte pieces of rows K elements apart. bf16 becomes fp16 as in
// bf16_to_f16_kernel; E4M3 codes are copied. One thread per 16 output bytes.
template <bool FP8>
__global__ void pack_panels_kernel(const void* __restrict__ src, void* __restrict__ dst, long n_chunks, int N, int K) {
  constexpr int E = FP8 ? 16 : 8;  // elements per 16-byte chunk
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_chunks) return;
  const long per_row = K / E, per_mat = (long)N * per_row;
  const long g = i / per_mat, r = i - g * per_mat;
  const int n = (int)(r / per_row), k = (int)(r - (long)n * per_row) * E;
  const long si = g * (long)N * K + (long)n * K + k;
  const long di = g * (long)N * K + ((long)(n >> 5) * (K >> 6) + (k >> 6)) * 2048 + (n & 31) * 64 + (k & 63);
  if constexpr (FP8) {
    *(uint4*)((uint8_t*)dst + di) = *(const uint4*)((const uint8_t*)src + si);
  } else {
    const uint4 v = *(const uint4*)((const uint16_t*)src + si);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    _Float16 o[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[2 * j] = (_Float16)__builtin_bit_cast(float, w[j] << 16);
      o[2 * j + 1] = (_Float16)__builtin_bit_cast(float, w[j] & 0xFFFF0000u);
    }
    *(uint4*)((_Float16*)dst + di) = *(const uint4*)o;
  }
}

// One wave per input row: bf16 -> fp32 residual, the first norm's operand x * g (fp16) and
// the row's sum of squares (slot 0). 8 elements per lane and chunk, d <= 1024.
__global__ __launch_bounds__(256) void input_rows_kernel(InputParams p) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.n_rows) return;
  const int u = row / p.rows_per_seg, t = row - u * p.rows_per_seg;
  bool valid = true;
  if (p.s_lens) {
    int len = p.s_lens[u];
    len = len < 0 ? 0 : (len > p.rows_per_seg ? p.rows_per_seg : len);
    const int vf = p.rows_per_seg - len;
    if (t == 0 && lane == 0) p.valid_from[u] = vf;
    valid = t >= vf;
  }
  const long base = (long)row * p.d;
  const NormOut& no = p.nout;
  const float* gain = no.gain + (long)(row % p.P) * no.gain_group_stride;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = (lane + 64 * i) * 8;
    if (c >= p.d) break;
    float4 g0 = make_float4(0.f, 0.f, 0.f, 0.f), g1 = g0;
    if (no.xg) {  // before the stores: a later wait for them would also wait for the stores
      g0 = *(const float4*)(gain + c);
      g1 = *(const float4*)(gain + c + 4);
    }
    float v[8];
    if (valid) {
      const uint4 w = *(const uint4*)(p.tok + base + c);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = __builtin_bit_cast(float, ws[j] << 16);
        v[2 * j + 1] = __builtin_bit_cast(float, ws[j] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.f;
    }
    *(float4*)(p.x + base + c) = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(p.x + base + c + 4) = make_float4(v[4], v[5], v[6], v[7]);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += v[j] * v[j];
    if (no.xg) {
      typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
      const f16x8 o = {(_Float16)(v[0] * g0.x), (_Float16)(v[1] * g0.y), (_Float16)(v[2] * g0.z),
                       (_Float16)(v[3] * g0.w), (_Float16)(v[4] * g1.x), (_Float16)(v[5] * g1.y),
                       (_Float16)(v[6] * g1.z), (_Float16)(v[7] * g1.w)};
      *(f16x8*)(no.xg + base + c) = o;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if (no.xg && lane == 0) no.ss[(long)row * no.ss_stride] = ss;
}

__global__ void copy_rows_kernel(const float* __restrict__ src, long src_seg_stride, float* __restrict__ dst,
                                 long dst_seg_stride, long row_elems) {
  const int sgi = blockIdx.y;
  for (long i = ((long)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < row_elems; i += (long)gridDim.x * blockDim.x * 4)
    *(float4*)(dst + sgi * dst_seg_stride + i) = *(const float4*)(src + sgi * src_seg_stride + i);
}

// Cache K [H][cap][dh] and V^T [H][dh][cap] of one user -> K, V [rows][H*dh].
__global__ void cache_read_kernel(const __bf16* __restrict__ k, const __bf16* __restrict__ vt, int H, int dh, int cap,
                                  int rows, __bf16* __restrict__ k_out, __bf16* __restrict__ v_out) {
  const int r = blockIdx.x;
  for (int c = threadIdx.x; c < H * dh; c += blockDim.x) {
    const int h = c / dh, j = c - h * dh;
    k_out[(long)r * H * dh + c] = k[((long)h * cap + r) * dh + j];
    v_out[(long)r * H * dh + c] = vt[((long)h * dh + j) * cap + r];
  }
}

}  // namespace

hipError_t launch_bf16_to_f16(const uint16_t* src, _Float16* dst, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long threads = (n + 7) / 8;
  hipLaunchKernelGGL(bf16_to_f16_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_pack_panels(const void* src, void* dst, bool fp8, long G, int N, int K, hipStream_t s) {
  if (G <= 0 || N <= 0 || K <= 0) return hipSuccess;
  if (N % 32 != 0 || K % 64 != 0) return hipErrorInvalidValue;
  const long chunks = G * (long)N * K / (fp8 ? 16 : 8);
  const dim3 grid((unsigned)((chunks + 255) / 256));
  if (fp8) hipLaunchKernelGGL(pack_panels_kernel<true>, grid, dim3(256), 0, s, src, dst, chunks, N, K);
  else hipLaunchKernelGGL(pack_panels_kernel<false>, grid, dim3(256), 0, s, src, dst, chunks, N, K);
  return hipGetLastError();
}

hipError_t launch_input_rows(const InputParams& p, hipStream_t s) {
  if (p.n_rows <= 0) return hipSuccess;
  if (p.d % 8 != 0 || p.d > 1024 || p.P < 1 || p.rows_per_seg < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(input_rows_kernel, dim3((unsigned)((p.n_rows + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_copy_rows_f32(const float* src, long src_seg_stride, float* dst, long dst_seg_stride, long row_elems,
                                int n_seg, hipStream_t s) {
  if (n_seg <= 0 || row_elems <= 0) return hipSuccess;
  long blocks = (row_elems / 4 + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(copy_rows_kernel, dim3((unsigned)blocks, n_seg), dim3(256), 0, s, src, src_seg_stride, dst,
                     dst_seg_stride, row_elems);
  return hipGetLastError();
}

hipError_t launch_cache_read(const __bf16* k, const __bf16* vt, int H, int dh, int cap, int rows, __bf16* k_out,
                             __bf16* v_out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(cache_read_kernel, dim3(rows), dim3(256), 0, s, k, vt, H, dh, cap, rows, k_out, v_out);
  return hipGetLastError();
}

}  // namespace onetrans
