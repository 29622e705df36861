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

__global__ void bf16_to_f32_kernel(const uint16_t* __restrict__ src, float* __restrict__ dst, long n) {
  const long i0 = ((long)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i0 + 8 <= n) {
    const uint4 v = *(const uint4*)(src + i0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float4 a, b;
    a.x = __builtin_bit_cast(float, w[0] << 16); a.y = __builtin_bit_cast(float, w[0] & 0xFFFF0000u);
    a.z = __builtin_bit_cast(float, w[1] << 16); a.w = __builtin_bit_cast(float, w[1] & 0xFFFF0000u);
    b.x = __builtin_bit_cast(float, w[2] << 16); b.y = __builtin_bit_cast(float, w[2] & 0xFFFF0000u);
    b.z = __builtin_bit_cast(float, w[3] << 16); b.w = __builtin_bit_cast(float, w[3] & 0xFFFF0000u);
    *(float4*)(dst + i0) = a;
    *(float4*)(dst + i0 + 4) = b;
  } else {
    for (long i = i0; i < n; ++i) dst[i] = __builtin_bit_cast(float, (uint32_t)src[i] << 16);
  }
}

// S-token input rows -> fp32 residual; padding slots (before s_len - len_u) become 0.
// One thread per 8 elements of a row; also records the user's first valid slot.
__global__ void s_input_kernel(const uint16_t* __restrict__ tok, const int* __restrict__ s_lens,
                               float* __restrict__ x, int* __restrict__ valid_from, int s_len, int d) {
  const int u = blockIdx.y;
  const long row = (long)blockIdx.x;  // slot
  int len = s_lens[u];
  len = len < 0 ? 0 : (len > s_len ? s_len : len);
  const int vf = s_len - len;
  if (row == 0 && threadIdx.x == 0) valid_from[u] = vf;
  const long base = ((long)u * s_len + row) * d;
  for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (row >= vf) {
      const uint4 v = *(const uint4*)(tok + base + c);
      a.x = __builtin_bit_cast(float, v.x << 16); a.y = __builtin_bit_cast(float, v.x & 0xFFFF0000u);
      a.z = __builtin_bit_cast(float, v.y << 16); a.w = __builtin_bit_cast(float, v.y & 0xFFFF0000u);
      b.x = __builtin_bit_cast(float, v.z << 16); b.y = __builtin_bit_cast(float, v.z & 0xFFFF0000u);
      b.z = __builtin_bit_cast(float, v.w << 16); b.w = __builtin_bit_cast(float, v.w & 0xFFFF0000u);
    }
    *(float4*)(x + base + c) = a;
    *(float4*)(x + base + c + 4) = b;
  }
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

// One wave per row: sum of squares over d (lane-strided, coalesced), wave
// reduction, then the scaled row written as fp16.
__global__ __launch_bounds__(256) void rmsnorm_f16_kernel(NormParams p) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int g = blockIdx.y;
  if (row >= p.M) return;
  const RowMap& rm = p.rm;
  const int seg = row / rm.rows_per_seg, t = row - seg * rm.rows_per_seg;
  const float* src = p.res + (long)seg * rm.res_seg_stride + (rm.res_row_base + t) * rm.res_row_stride +
                     (long)g * rm.res_group_stride;
  const float* gain = p.gain + (long)g * p.gain_group_stride;
  _Float16* dst = p.out + (((long)seg * rm.rows_per_seg + t) * rm.row_mult + g) * p.d;
  constexpr int MAXE = 16;  // d <= 1024
  float v[MAXE];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXE; ++i) {
    const int c = lane + 64 * i;
    v[i] = c < p.d ? src[c] : 0.f;
    ss += v[i] * v[i];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float r = 1.0f / sqrtf(ss / (float)p.d + p.eps);
#pragma unroll
  for (int i = 0; i < MAXE; ++i) {
    const int c = lane + 64 * i;
    if (c < p.d) dst[c] = (_Float16)(v[i] * r * gain[c]);
  }
}

// Two rows per wave (32 lanes each), NV float4 per lane (d = 128 * NV): 16-byte loads,
// a 32-lane reduction and 8-byte fp16 stores. Flattened row f = row * groups + group,
// so consecutive waves walk memory in order for candidate-major NS rows.
template <int NV>
__global__ __launch_bounds__(256) void rmsnorm_f16_v4_kernel(NormParams p) {
  const int lane = threadIdx.x & 63, l32 = lane & 31;
  const long f = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * 2 + (lane >> 5);
  if (f >= (long)p.M * p.groups) return;  // the two halves never exchange data
  const int row = (int)(f / p.groups), g = (int)(f - (long)row * p.groups);
  const RowMap& rm = p.rm;
  const int seg = row / rm.rows_per_seg, t = row - seg * rm.rows_per_seg;
  const float4* src = (const float4*)(p.res + (long)seg * rm.res_seg_stride + (rm.res_row_base + t) * rm.res_row_stride +
                                      (long)g * rm.res_group_stride);
  const float4* gain = (const float4*)(p.gain + (long)g * p.gain_group_stride);
  _Float16* dst = p.out + (((long)seg * rm.rows_per_seg + t) * rm.row_mult + g) * p.d;
  float4 v[NV];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    v[i] = src[l32 + 32 * i];
    ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
  }
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float r = 1.0f / sqrtf(ss / (float)p.d + p.eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const float4 gv = gain[l32 + 32 * i];
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    const f16x4 o = {(_Float16)(v[i].x * r * gv.x), (_Float16)(v[i].y * r * gv.y), (_Float16)(v[i].z * r * gv.z),
                     (_Float16)(v[i].w * r * gv.w)};
    *(f16x4*)(dst + 4 * (l32 + 32 * i)) = o;
  }
}

}  // namespace

hipError_t launch_rmsnorm(const NormParams& p, hipStream_t s) {
  if (p.M <= 0 || p.groups <= 0) return hipSuccess;
  const long rows = (long)p.M * p.groups;
  const dim3 grid((unsigned)((rows + 7) / 8));
  switch (p.d % 128 == 0 ? p.d / 128 : 0) {
    case 1: hipLaunchKernelGGL(rmsnorm_f16_v4_kernel<1>, grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL(rmsnorm_f16_v4_kernel<2>, grid, dim3(256), 0, s, p); break;
    case 3: hipLaunchKernelGGL(rmsnorm_f16_v4_kernel<3>, grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL(rmsnorm_f16_v4_kernel<4>, grid, dim3(256), 0, s, p); break;
    case 5: hipLaunchKernelGGL(rmsnorm_f16_v4_kernel<5>, grid, dim3(256), 0, s, p); break;
    case 6: hipLaunchKernelGGL(rmsnorm_f16_v4_kernel<6>, grid, dim3(256), 0, s, p); break;
    case 7: hipLaunchKernelGGL(rmsnorm_f16_v4_kernel<7>, grid, dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL(rmsnorm_f16_v4_kernel<8>, grid, dim3(256), 0, s, p); break;
    default:  // d not a multiple of 128: one row per wave
      hipLaunchKernelGGL(rmsnorm_f16_kernel, dim3((p.M + 3) / 4, p.groups), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_bf16_to_f16(const uint16_t* src, _Float16* dst, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long threads = (n + 7) / 8;
  hipLaunchKernelGGL(bf16_to_f16_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_bf16_to_f32(const uint16_t* src, float* dst, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long threads = (n + 7) / 8;
  hipLaunchKernelGGL(bf16_to_f32_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_s_input(const uint16_t* tok, const int* s_lens, float* x, int* valid_from, int B, int s_len, int d,
                          hipStream_t s) {
  if (B <= 0) return hipSuccess;
  const int threads = d / 8 < 64 ? 64 : (d / 8 > 128 ? 128 : d / 8);
  hipLaunchKernelGGL(s_input_kernel, dim3(s_len, B), dim3(threads), 0, s, tok, s_lens, x, valid_from, s_len, d);
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
