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
// pair (lane, lane ^ 32) and need one cross-lane exchange per key tile; P never
// leaves registers. V is stored transposed ([dh][key]) so the V^T operand is a
// plain row read. Each wave owns 32 queries; a workgroup of 4 waves shares the
// K / V^T tiles (64 keys) staged through LDS. The result is added to the fp32
// residual rows (z = x + o) without rounding.
#include <math.h>
#include "internal.h"

namespace onetrans {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int KT = 64;  // keys per LDS tile

template <int DH>
struct Softmax {
  float m = -INFINITY, l = 0.f;
  f32x16 o[DH / 32];
};

// Online-softmax update with one 32-key block of scores already masked and
// scaled into log2 units; returns the bf16 probabilities packed as the two
// B operands (keys 0-15 and 16-31 of the block in the lane's slot order).
template <int DH, int NB>
__device__ __forceinline__ void softmax_update(Softmax<DH>& st, f32x16 (&sc)[NB], bf16x8 (&pb)[NB][2]) {
  float mt = -INFINITY;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < 16; ++j) mt = fmaxf(mt, sc[b][j]);
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  const float m_new = fmaxf(st.m, mt);
  const bool none = (m_new == -INFINITY);
  const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(st.m - m_new);
  const float msub = none ? 0.f : m_new;
  float ps = 0.f;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pv = __builtin_amdgcn_exp2f(sc[b][8 * c + i] - msub);
        ps += pv;
        pb[b][c][i] = (__bf16)pv;
      }
  st.l = st.l * alpha + ps;
  st.m = m_new;
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) st.o[db][j] *= alpha;
}

template <int DH, bool NS>
__global__ __launch_bounds__(256) void attn_kernel(AttnParams p) {
  constexpr int KLD = DH + 8;  // K tile row stride (bf16)
  constexpr int VLD = KT + 8;  // V^T tile row stride (bf16)
  __shared__ __attribute__((aligned(16))) __bf16 Ks[KT * KLD];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[DH * VLD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int h = blockIdx.y, seg = blockIdx.z;
  const int wq0 = blockIdx.x * 128 + wave * 32;
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
  if (!NS) {
    const int qlast_blk = min((int)blockIdx.x * 128 + 127, p.nq - 1);
    const int qlast_wave = min(wq0 + 31, p.nq - 1);
    key_hi = min(key_hi, p.q_pos0 + qlast_blk - p.key_pos0 + 1);
    wave_lim = min(wave_lim, p.q_pos0 + qlast_wave - p.key_pos0 + 1);
    my_lim = min(my_lim, p.q_pos0 + qi - p.key_pos0 + 1);
  }
  if (!q_ok) my_lim = 0;

  Softmax<DH> st;
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) st.o[db][j] = 0.f;

  const __bf16* kbase = p.k + seg * p.kv_seg_stride + h * p.kv_head_stride;
  const __bf16* vbase = p.vt + seg * p.kv_seg_stride + h * p.kv_head_stride;

#pragma unroll 1
  for (int t0 = (key_lo / KT) * KT; t0 < key_hi; t0 += KT) {
    // stage K rows [t0, t0+KT) and V^T columns [t0, t0+KT); slots outside [key_lo, key_hi) read as 0
    for (int c = tid; c < KT * DH / 8; c += 256) {
      const int r = c / (DH / 8), cc = c - r * (DH / 8);
      const int slot = t0 + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (slot >= key_lo && slot < key_hi) v = *(const uint4*)(kbase + (long)slot * DH + cc * 8);
      *(uint4*)&Ks[r * KLD + cc * 8] = v;
    }
    for (int c = tid; c < DH * KT / 8; c += 256) {
      const int r = c / (KT / 8), cc = c - r * (KT / 8);
      const int s0 = t0 + cc * 8;
      const __bf16* src = vbase + (long)r * p.kv_cap + s0;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (s0 >= key_lo && s0 + 8 <= key_hi) {
        v = *(const uint4*)src;
      } else if (s0 + 8 > key_lo && s0 < key_hi) {
        bf16x8 e;
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = (s0 + i >= key_lo && s0 + i < key_hi) ? src[i] : (__bf16)0.f;
        v = __builtin_bit_cast(uint4, e);
      }
      *(uint4*)&Vs[r * VLD + cc * 8] = v;
    }
    __syncthreads();
    if (wave_live && t0 < wave_lim) {
      f32x16 sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) sc[kb][j] = 0.f;
#pragma unroll
        for (int s = 0; s < DH / 16; ++s) {
          const bf16x8 a = *(const bf16x8*)&Ks[(kb * 32 + l32) * KLD + s * 16 + half * 8];
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sc[kb], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int slot = t0 + kb * 32 + 8 * (j >> 2) + half * 4 + (j & 3);
          const bool vis = slot >= key_lo && slot < my_lim;
          sc[kb][j] = vis ? sc[kb][j] * p.scale_log2 : -INFINITY;
        }
      }
      bf16x8 pb[2][2];
      softmax_update<DH, 2>(st, sc, pb);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int db = 0; db < DH / 32; ++db) {
            const __bf16* vr = &Vs[(db * 32 + l32) * VLD + kb * 32 + 16 * c + half * 4];
            const bf16x4 lo = *(const bf16x4*)vr;
            const bf16x4 hi = *(const bf16x4*)(vr + 8);
            const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][c], st.o[db], 0, 0, 0);
          }
    }
    __syncthreads();
  }

  if (NS && wave_live) {
    // the candidate's own NS keys: query g = c*P + k sees g' in [c*P, g]
    const int P = p.P;
    const int g_lo = (wq0 / P) * P;
    const int g_hi = min(wq0 + 31, p.nq - 1);
    const int my_first = (qi / P) * P;
    const __bf16* knb = p.kn + h * p.kn_head_stride;
    const __bf16* vnb = p.vtn + h * p.kn_head_stride;
#pragma unroll 1
    for (int t0 = g_lo; t0 <= g_hi; t0 += 32) {
      f32x16 sc[1];
#pragma unroll
      for (int j = 0; j < 16; ++j) sc[0][j] = 0.f;
      const int krow = t0 + l32;
#pragma unroll
      for (int s = 0; s < DH / 16; ++s) {
        bf16x8 a;
        if (krow < p.nq) a = *(const bf16x8*)(knb + (long)krow * DH + s * 16 + half * 8);
        else {
#pragma unroll
          for (int i = 0; i < 8; ++i) a[i] = (__bf16)0.f;
        }
        sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sc[0], 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = t0 + 8 * (j >> 2) + half * 4 + (j & 3);
        const bool vis = q_ok && key <= qi && key >= my_first;
        sc[0][j] = vis ? sc[0][j] * p.scale_log2 : -INFINITY;
      }
      bf16x8 pb[1][2];
      softmax_update<DH, 1>(st, sc, pb);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int db = 0; db < DH / 32; ++db) {
          const __bf16* vr = vnb + (long)(db * 32 + l32) * p.nq;
          bf16x8 a;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int key = t0 + 16 * c + half * 4 + (i & 3) + 8 * (i >> 2);
            a[i] = key < p.nq ? vr[key] : (__bf16)0.f;
          }
          st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[0][c], st.o[db], 0, 0, 0);
        }
    }
  }

  const float l_tot = st.l + __shfl_xor(st.l, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_ok) {
    float* rrow = p.res + seg * p.res_seg_stride + (p.res_row_base + qi) * p.res_row_stride + h * DH;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        float4* dst = (float4*)(rrow + db * 32 + 8 * gi + half * 4);
        float4 r = *dst;
        r.x += st.o[db][4 * gi + 0] * inv;
        r.y += st.o[db][4 * gi + 1] * inv;
        r.z += st.o[db][4 * gi + 2] * inv;
        r.w += st.o[db][4 * gi + 3] * inv;
        *dst = r;
      }
  }
}

}  // namespace

hipError_t launch_attention(bool ns, int dh, const AttnParams& p, int n_seg, hipStream_t s) {
  if (p.nq <= 0 || n_seg <= 0) return hipSuccess;
  dim3 grid((p.nq + 127) / 128, p.H, n_seg);
  dim3 block(256);
  if (dh == 64) {
    if (ns) hipLaunchKernelGGL((attn_kernel<64, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_kernel<64, false>), grid, block, 0, s, p);
  } else if (dh == 32) {
    if (ns) hipLaunchKernelGGL((attn_kernel<32, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_kernel<32, false>), grid, block, 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace onetrans
