// Grouped GEMMs of the OneTrans block on gfx950 MFMA (fp16 operands, fp32 accumulate).
//
// One kernel template covers the linear maps of a layer (agihunt.info OneTrans
// summary, "method": shared S-token QKV/FFN, private per-NS-position QKV/FFN):
//   GEMM_QKV      : A = RMSNorm'd rows (fp16), B = W_QKV [3d][d];
//                   epilogue scatters bf16 Q / K / V (V^T for the S cache)
//   GEMM_FFN_UP   : A = RMSNorm'd rows (fp16), B = W1 [F][d];
//                   epilogue GELU(erf) -> fp16 hidden rows
//   GEMM_FFN_DOWN : A = fp16 hidden rows, B = W2 [d][F];
//                   epilogue adds into the fp32 residual rows in place
// A group is one NS position (private weights) or the shared S weights.
//
// Data movement: A and B tiles (BK = 64) go straight from global memory into
// LDS with global_load_lds_dwordx4, STAGES tiles in flight, so the waves never
// stage operands through registers and several memory round trips overlap.
// LDS rows are 128 B (fp16) or 64 B (E4M3 codes); the 16-byte chunks of a row
// are XOR-swizzled by row so that the MFMA fragment reads (16 lanes, 16 rows,
// one chunk column) hit 16 distinct bank groups.
//
// Tiles: BM x BN per workgroup of 4 waves (2 x 2), each wave a grid of 32x32
// blocks of v_mfma_f32_32x32x16_f16.
//
// Work order: the 1-D grid is dispatched round-robin over the 8 XCDs, so block
// L runs on XCD L % 8. Each XCD is handed a contiguous range of the work list,
// which is ordered M-tile fastest, then N-tile, then group: workgroups that
// share a weight tile (same N-tile and group) or an activation block (same
// group) run on the same XCD and meet in its L2.
#include "internal.h"

namespace onetrans {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;
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

__device__ __forceinline__ float gelu_erf(float v) { return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f)); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
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

// SIDE (0 = shared S weights, 1 = private NS weights) only names the instance.
template <int KIND, bool FP8, int SIDE, int BM, int BN, int STAGES>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p, int n_tiles_m, int n_tiles_n) {
  constexpr int MI = BM / 64, NI = BN / 64;      // 32x32 blocks per wave
  constexpr int A_BYTES = BM * 128;              // BM rows x 64 halfs
  constexpr int B_ROW = FP8 ? 64 : 128;          // bytes per B row of the tile
  constexpr int B_BYTES = BN * B_ROW;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_INSTR = A_BYTES / 1024 / 4;    // 1 KB per wave instruction, 4 waves
  constexpr int B_INSTR = B_BYTES / 1024 / 4;
  constexpr int PER_TILE = A_INSTR + B_INSTR;    // vector-memory ops per wave per tile
  static_assert(A_INSTR >= 1 && B_INSTR >= 1, "tile too small");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];

  // ---- XCD-aware work assignment ----
  const int total = gridDim.x, L = blockIdx.x;
  const int xcd = L % N_XCD, local = L / N_XCD;
  const int per = total / N_XCD, rem = total % N_XCD;
  const int w = xcd * per + min(xcd, rem) + local;
  const int mt = w % n_tiles_m;
  const int nt = (w / n_tiles_m) % n_tiles_n;
  const int g = w / (n_tiles_m * n_tiles_n);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = nt * BN, m0 = mt * BM;
  const RowMap rm = p.rm;
  const int M = p.M, N = p.N, K = p.K;
  const float inv_rps = 1.0f / (float)rm.rows_per_seg;

  // ---- per-lane global sources of the direct-to-LDS loads ----
  // A: instruction i of wave w fills rows (w*A_INSTR + i)*8 + lane/8, LDS chunk lane%8,
  //    which holds global chunk (lane%8) ^ ((row>>1)&7)
  const char* a_src[A_INSTR];
#pragma unroll
  for (int i = 0; i < A_INSTR; ++i) {
    const int r = (wave * A_INSTR + i) * 8 + (lane >> 3);
    const int row = min(m0 + r, M - 1);
    int seg, t;
    split_row(row, rm.rows_per_seg, inv_rps, seg, t);
    a_src[i] = (const char*)(p.a_in + hid_row(rm, seg, t, g) * (long)K) + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
  }
  const char* wbase = (const char*)p.w + (long)g * p.w_group_stride * (FP8 ? 1 : 2);
  const char* b_src[B_INSTR];
#pragma unroll
  for (int i = 0; i < B_INSTR; ++i) {
    if (FP8) {  // 16 rows of 64 B per instruction, chunk lane%4 holds global chunk (lane%4) ^ ((row>>2)&3)
      const int r = (wave * B_INSTR + i) * 16 + (lane >> 2);
      const int n = min(n0 + r, N - 1);
      b_src[i] = wbase + (long)n * K + (((lane & 3) ^ ((r >> 2) & 3)) << 4);
    } else {
      const int r = (wave * B_INSTR + i) * 8 + (lane >> 3);
      const int n = min(n0 + r, N - 1);
      b_src[i] = wbase + (long)n * K * 2 + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
    }
  }

  auto issue = [&](int kt, int stage) {
    char* st = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i)
      dma16(a_src[i] + kt * (BK * 2), (lds_void*)(st + (wave * A_INSTR + i) * 1024));
#pragma unroll
    for (int i = 0; i < B_INSTR; ++i)
      dma16(b_src[i] + kt * (FP8 ? BK : BK * 2),
                                       (lds_void*)(st + A_BYTES + (wave * B_INSTR + i) * 1024));
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.f;

  const int nk = K / BK;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue(s, s);

#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    // tile kt has landed once at most (STAGES-2) later tiles are still in flight
    if (kt + STAGES - 2 < nk) wait_vmcnt<PER_TILE * (STAGES - 2)>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
    const char* st = smem + (kt % STAGES) * STAGE;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      f16x8 a[MI], b[NI];
      const int c = 2 * s + (lane >> 5);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int r = wm * (BM / 2) + mi * 32 + (lane & 31);
        a[mi] = *(const f16x8*)(st + r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int r = wn * (BN / 2) + ni * 32 + (lane & 31);
        if (FP8) b[ni] = e4m3x8_to_f16(*(const uint2*)(st + A_BYTES + r * 64 + ((s ^ ((r >> 2) & 3)) << 4) +
                                                        (lane >> 5) * 8));
        else b[ni] = *(const f16x8*)(st + A_BYTES + r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
  }

  // ---- epilogue: per 32x32 block, lane holds column lane & 31 and rows
  // 8*(j/4) + (lane/32)*4 + j%4 (four consecutive rows per j/4) ----
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    const int col = n0 + wn * (BN / 2) + ni * 32 + (lane & 31);
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
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int row0 = m0 + wm * (BM / 2) + mi * 32 + 8 * jg + (lane >> 5) * 4;
        if (row0 >= M) continue;
        int seg, t0;
        split_row(row0, rm.rows_per_seg, inv_rps, seg, t0);
        const bool whole = (row0 + 3 < M) && (t0 + 3 < rm.rows_per_seg);  // four rows, one segment
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[mi][ni][4 * jg + r] * scale;
        if (KIND == GEMM_QKV && typ == 2 && p.vt != nullptr && rm.row_mult == 1 && whole) {
          // V^T rows: the four rows are four consecutive key slots
          const long ki = p.kv_slot_base + t0;
          __bf16* dst = p.vt + seg * p.kv_seg_stride + head * p.kv_head_stride + (long)jj * p.kv_cap + ki;
          if ((ki & 3) == 0) {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            bf16x4 pk = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
            *(bf16x4*)dst = pk;
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[r] = (__bf16)v[r];
          }
          continue;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int sg = seg, t = t0 + r;
          if (row0 + r >= M) break;
          if (t >= rm.rows_per_seg) { t -= rm.rows_per_seg; ++sg; }
          if (KIND == GEMM_QKV) {
            const int ti = t * rm.row_mult + g;
            if (typ == 0) {
              const int qi = ti - p.q_from;
              if (qi >= 0) p.q[sg * p.q_seg_stride + head * p.q_head_stride + (long)qi * p.dh + jj] = (__bf16)v[r];
            } else {
              const long base = sg * p.kv_seg_stride + head * p.kv_head_stride;
              const long ki = p.kv_slot_base + ti;
              if (typ == 1) p.k[base + ki * p.dh + jj] = (__bf16)v[r];
              else if (p.vt != nullptr) p.vt[base + (long)jj * p.kv_cap + ki] = (__bf16)v[r];
              else p.v[base + ki * p.dh + jj] = (__bf16)v[r];
            }
          } else if (KIND == GEMM_FFN_UP) {
            p.hid_out[hid_row(rm, sg, t, g) * N + col] = (_Float16)gelu_erf(v[r]);
          } else {
            float* dst = p.res_out + res_row_off(rm, sg, t, g) + col;
            *dst = *dst + v[r];
          }
        }
      }
    }
  }
}

template <int KD, int BM, int BN>
void launch_tiles(bool fp8, bool ns, const GemmParams& p, hipStream_t s) {
  const int tm = (p.M + BM - 1) / BM, tn = (p.N + BN - 1) / BN;
  dim3 grid(tm * tn * p.groups), block(256);
  if (!ns) hipLaunchKernelGGL((gemm_kernel<KD, false, 0, BM, BN, 3>), grid, block, 0, s, p, tm, tn);
  else if (fp8) hipLaunchKernelGGL((gemm_kernel<KD, true, 1, BM, BN, 3>), grid, block, 0, s, p, tm, tn);
  else hipLaunchKernelGGL((gemm_kernel<KD, false, 1, BM, BN, 3>), grid, block, 0, s, p, tm, tn);
}

template <int KD>
void launch_kind(bool fp8, bool ns, const GemmParams& p, hipStream_t s) {
  // 128x128 tiles when they give at least two workgroups per CU, else 64x64
  const long big = (long)((p.M + 127) / 128) * ((p.N + 127) / 128) * p.groups;
  if (big >= 512) launch_tiles<KD, 128, 128>(fp8, ns, p, s);
  else launch_tiles<KD, 64, 64>(fp8, ns, p, s);
}

}  // namespace

hipError_t launch_gemm(GemmKind kind, bool fp8, bool ns, const GemmParams& p, hipStream_t s) {
  if (p.M <= 0 || p.groups <= 0) return hipSuccess;
  if (p.K % BK != 0) return hipErrorInvalidValue;
  if (kind == GEMM_QKV) launch_kind<GEMM_QKV>(fp8, ns, p, s);
  else if (kind == GEMM_FFN_UP) launch_kind<GEMM_FFN_UP>(fp8, ns, p, s);
  else launch_kind<GEMM_FFN_DOWN>(fp8, ns, p, s);
  return hipGetLastError();
}

}  // namespace onetrans
