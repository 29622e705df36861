// C ABI of the OneTrans block forward: validation, memory layouts and the
// per-layer launch sequence. Every step of the computation runs in the HIP
// kernels of gemm.hip, attention.hip and elementwise.hip.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "onetrans.h"
#include "internal.h"

using namespace onetrans;

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

struct Shape {
  int L, d, H, dh, F, P, s_len, append_cap;
  int Pu, Pc;  // user-side NS positions 0..Pu-1; a candidate's rows Pu..P-1 (Pc of them)
  int q[ONETRANS_MAX_LAYERS], n[ONETRANS_MAX_LAYERS], cap[ONETRANS_MAX_LAYERS];
  bool fp8;
  float eps;
};

int make_shape(const onetrans_config* c, Shape& s) {
  if (!c) return fail(ONETRANS_ERR_INVALID_ARG, "config is NULL");
  if (c->n_layers < 1 || c->n_layers > ONETRANS_MAX_LAYERS)
    return fail(ONETRANS_ERR_UNSUPPORTED, "n_layers must be in [1, 16]");
  if (c->d_model < 64 || c->d_model > 1024 || c->d_model % 64)
    return fail(ONETRANS_ERR_UNSUPPORTED, "d_model must be a multiple of 64 in [64, 1024]");
  if (c->n_heads < 1 || c->d_model % c->n_heads)
    return fail(ONETRANS_ERR_UNSUPPORTED, "n_heads must divide d_model");
  const int dh = c->d_model / c->n_heads;
  if (dh != 32 && dh != 64) return fail(ONETRANS_ERR_UNSUPPORTED, "head_dim must be 32 or 64");
  if (c->ffn_hidden < 64 || c->ffn_hidden % 64) return fail(ONETRANS_ERR_UNSUPPORTED, "ffn_hidden must be a positive multiple of 64");
  if (c->n_ns < 1 || c->n_ns > 256) return fail(ONETRANS_ERR_UNSUPPORTED, "n_ns must be in [1, 256]");
  if (c->s_len < 1 || c->s_len > (1 << 20)) return fail(ONETRANS_ERR_UNSUPPORTED, "s_len must be in [1, 2^20]");
  if (c->append_cap < 0 || c->append_cap > (1 << 20)) return fail(ONETRANS_ERR_UNSUPPORTED, "append_cap must be in [0, 2^20]");
  if (!(c->rms_eps > 0.f) || !isfinite(c->rms_eps)) return fail(ONETRANS_ERR_INVALID_ARG, "rms_eps must be positive and finite");
  if (c->ns_wdtype != ONETRANS_W_BF16 && c->ns_wdtype != ONETRANS_W_FP8_E4M3)
    return fail(ONETRANS_ERR_UNSUPPORTED, "ns_wdtype must be ONETRANS_W_BF16 or ONETRANS_W_FP8_E4M3");
  if (c->n_ns_user < 0 || c->n_ns_user > c->n_ns) return fail(ONETRANS_ERR_UNSUPPORTED, "n_ns_user must be in [0, n_ns]");
  s.L = c->n_layers; s.d = c->d_model; s.H = c->n_heads; s.dh = dh; s.F = c->ffn_hidden; s.P = c->n_ns;
  s.Pu = c->n_ns_user; s.Pc = c->n_ns - c->n_ns_user;
  s.s_len = c->s_len; s.append_cap = c->append_cap; s.fp8 = c->ns_wdtype == ONETRANS_W_FP8_E4M3; s.eps = c->rms_eps;
  int prev = c->s_len;
  for (int l = 0; l < s.L; ++l) {
    const int q = c->q_sched[l];
    if (q < 1 || q > prev)
      return fail(ONETRANS_ERR_UNSUPPORTED, "q_sched must satisfy 1 <= q_sched[l] <= q_sched[l-1] (q_sched[0] <= s_len)");
    s.n[l] = prev;
    s.q[l] = q;
    s.cap[l] = (prev + s.append_cap + 63) / 64 * 64;  // tiles of 64 keys never read past the layer's block
    prev = q;
  }
  return ONETRANS_OK;
}

// Key of the user-side shape a cache is laid out for: a 64-bit FNV-1a hash of every
// config field the cache layout (and the cached values' meaning) depends on.
uint64_t layout_key(const onetrans_config* c) {
  uint64_t h = 1469598103934665603ull;
  auto mix = [&](uint32_t v) {
    for (int i = 0; i < 4; ++i) {
      h ^= (v >> (8 * i)) & 0xff;
      h *= 1099511628211ull;
    }
  };
  mix(c->n_layers); mix(c->d_model); mix(c->n_heads); mix(c->s_len); mix(c->append_cap); mix(c->n_ns_user);
  uint32_t e;
  memcpy(&e, &c->rms_eps, 4);
  mix(e);
  for (int l = 0; l < c->n_layers; ++l) mix(c->q_sched[l]);
  return h;
}

int check_cache_key(const onetrans_config* c, const onetrans_kv_cache* cache) {
  if (cache->layout_key != layout_key(c))
    return fail(ONETRANS_ERR_INVALID_ARG, "cache was laid out for another user-side shape");
  return ONETRANS_OK;
}

struct LayerOffsets {
  size_t s_wqkv, s_w1, s_w2, s_ga, s_gf, ns_wqkv, ns_w1, ns_w2, ns_scale, ns_ga, ns_gf;
};

// Packed buffer: per layer, fp16 S weights, fp32 S gains, fp16 (or E4M3 codes) NS
// weights, fp32 NS scales and gains; every array starts on a 256-byte boundary.
size_t packed_layout(const Shape& s, LayerOffsets* lo) {
  size_t off = 0;
  const size_t d = s.d, F = s.F, P = s.P, nsb = s.fp8 ? 1 : 2;
  for (int l = 0; l < s.L; ++l) {
    LayerOffsets o;
    o.s_wqkv = off; off = align_up(off + 3 * d * d * 2);
    o.s_w1 = off; off = align_up(off + F * d * 2);
    o.s_w2 = off; off = align_up(off + d * F * 2);
    o.s_ga = off; off = align_up(off + d * 4);
    o.s_gf = off; off = align_up(off + d * 4);
    o.ns_wqkv = off; off = align_up(off + P * 3 * d * d * nsb);
    o.ns_w1 = off; off = align_up(off + P * F * d * nsb);
    o.ns_w2 = off; off = align_up(off + P * d * F * nsb);
    o.ns_scale = off; off = align_up(off + P * 5 * 4);
    o.ns_ga = off; off = align_up(off + P * d * 4);
    o.ns_gf = off; off = align_up(off + P * d * 4);
    if (lo) lo[l] = o;
  }
  return off;
}

// Cache buffer: valid_from int32 [B], then per layer K bf16 [B][H][cap_l][dh]
// and V^T bf16 [B][H][dh][cap_l]; with user-side NS rows, per layer their K and V
// bf16 [B][H][Pu][dh] (row-major, as the NS attention reads own keys), then their
// inputs bf16 [B][Pu][d].
struct UserNsOff {
  size_t k[ONETRANS_MAX_LAYERS], v[ONETRANS_MAX_LAYERS], tok;
};
size_t cache_layout(const Shape& s, int B, size_t* k_off, size_t* v_off, UserNsOff* un = nullptr) {
  size_t off = align_up((size_t)B * 4);
  for (int l = 0; l < s.L; ++l) {
    const size_t blk = (size_t)B * s.H * s.cap[l] * s.dh * 2;
    if (k_off) k_off[l] = off;
    off = align_up(off + blk);
    if (v_off) v_off[l] = off;
    off = align_up(off + blk);
  }
  if (s.Pu > 0) {
    const size_t blk = (size_t)B * s.H * s.Pu * s.dh * 2;
    for (int l = 0; l < s.L; ++l) {
      if (un) un->k[l] = off;
      off = align_up(off + blk);
      if (un) un->v[l] = off;
      off = align_up(off + blk);
    }
    if (un) un->tok = off;
    off = align_up(off + (size_t)B * s.Pu * s.d * 2);
  }
  return off;
}

// Every path keeps, per activation row, the fp16 operand of the next linear map (xn: x * g
// or the norm-free FFN hidden row) and the row's partial sums of squares (ss, deferred
// RMSNorm: ss_stride_for(d) floats per row).
struct PrefillWs { size_t x, q, xn, ss, hid, total; };
PrefillWs prefill_ws(const Shape& s, int B) {
  PrefillWs w;
  size_t off = 0;
  const size_t rows = (size_t)B * s.s_len;
  w.x = off; off = align_up(off + rows * s.d * 4);
  w.q = off; off = align_up(off + (size_t)B * s.H * s.q[0] * s.dh * 2);
  w.xn = off; off = align_up(off + rows * s.d * 2);
  w.ss = off; off = align_up(off + rows * ss_stride_for(s.d) * 4);
  w.hid = off; off = align_up(off + (size_t)B * s.q[0] * s.F * 2);
  w.total = off;
  return w;
}

struct AppendWs { size_t q, xn, ss, hid, total; };
AppendWs append_ws(const Shape& s, int B, int m) {
  AppendWs w;
  size_t off = 0;
  const size_t rows = (size_t)B * m;
  w.q = off; off = align_up(off + (size_t)B * s.H * m * s.dh * 2);
  w.xn = off; off = align_up(off + rows * s.d * 2);
  w.ss = off; off = align_up(off + rows * ss_stride_for(s.d) * 4);
  w.hid = off; off = align_up(off + rows * s.F * 2);
  w.total = off;
  return w;
}

struct ScoreWs { size_t qn, kn, vn, xn, ss, hid, total; };
// C groups of Pn NS rows
ScoreWs score_ws(const Shape& s, int C, int Pn) {
  ScoreWs w;
  size_t off = 0;
  const size_t rows = (size_t)C * Pn;
  w.qn = off; off = align_up(off + rows * s.d * 2);
  w.kn = off; off = align_up(off + rows * s.d * 2);
  w.vn = off; off = align_up(off + rows * s.d * 2);
  w.xn = off; off = align_up(off + rows * s.d * 2);
  w.ss = off; off = align_up(off + rows * ss_stride_for(s.d) * 4);
  w.hid = off; off = align_up(off + rows * s.F * 2);
  w.total = off;
  return w;
}

// The user-side NS pass of B users (B groups of Pu rows) plus their fp32 output rows when
// the caller asked for none, run in a workspace after the S side has finished with it.
size_t user_pass_ws(const Shape& s, int B) {
  if (s.Pu == 0) return 0;
  return score_ws(s, B, s.Pu).total + align_up((size_t)B * s.Pu * s.d * 4);
}

size_t prefill_need(const Shape& s, int B) { return std::max(prefill_ws(s, B).total, user_pass_ws(s, B)); }
size_t append_need(const Shape& s, int B, int m) { return std::max(append_ws(s, B, m).total, user_pass_ws(s, B)); }

GemmParams base_gemm(const Shape& s) {
  GemmParams g;
  memset(&g, 0, sizeof(g));
  g.d = s.d;
  g.dh = s.dh;

  g.scale_col_div = 1 << 30;
  g.groups = 1;
  g.ss_stride = ss_stride_for(s.d);
  g.eps = s.eps;
  return g;
}

int hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ONETRANS_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return ONETRANS_OK;
}

#define OT_HIP(call, what)                      \
  do {                                          \
    int rc_ = hip_check((call), (what));        \
    if (rc_ != ONETRANS_OK) return rc_;         \
  } while (0)

// ---- kernel timing diagnostics: HIP events around launches of selected families ----
struct TimingRec {
  int fam;
  hipEvent_t a, b;
};
uint32_t g_timing_mask = 0;
std::vector<TimingRec> g_timing;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pooled_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

struct FamilyTimer {
  int fam;
  hipStream_t st;
  hipEvent_t a = nullptr;
  FamilyTimer(int f, hipStream_t s) : fam(f), st(s) {
    if (g_timing_mask & (1u << f)) {
      a = pooled_event();
      if (a && hipEventRecord(a, st) != hipSuccess) a = nullptr;
    }
  }
  ~FamilyTimer() {
    if (!a) return;
    hipEvent_t b = pooled_event();
    if (b && hipEventRecord(b, st) == hipSuccess) g_timing.push_back({fam, a, b});
    else g_event_pool.push_back(a);
  }
};

float scale_log2(const Shape& s) { return (float)(1.4426950408889634 / sqrt((double)s.dh)); }

// ---- one S-side layer over `rows` rows per user (prefill: the layer input;
// append: the new events), queries are the last `q` of them ----
struct SLayerArgs {
  int B, rows, q;
  float* x; long x_seg_stride, x_row_base;  // residual rows of user u: x + u*x_seg_stride + (x_row_base + t)*d
  __bf16* k; __bf16* vt; int cap, slot_base, n_keys, key_pos0;
  const int* valid_from;
  __bf16* qbuf; _Float16* xn; _Float16* hid;
  float* ss; int ss_parts;   // the layer input's partial sums (deferred RMSNorm) and their count
  const float* next_ga;      // attention-norm gain of the next layer; NULL after the last
  hipEvent_t kv_done;        // recorded once the layer's K/V rows are written; may be NULL
};

NormOut norm_out(const Shape& s, _Float16* xg, const float* gain, long gain_group_stride, float* ss) {
  NormOut n;
  n.xg = gain ? xg : nullptr;
  n.gain = gain;
  n.gain_group_stride = gain_group_stride;
  n.ss = ss;
  n.ss_stride = ss_stride_for(s.d);
  return n;
}

int run_s_layer(const Shape& s, const char* pk, const LayerOffsets& lo, const SLayerArgs& a, hipStream_t st) {
  const long d = s.d;
  RowMap all{a.rows, 1, a.x_seg_stride, a.x_row_base, d, 0};
  RowMap tail{a.q, 1, a.x_seg_stride, a.x_row_base + (a.rows - a.q), d, 0};

  GemmParams g = base_gemm(s);
  g.M = a.B * a.rows; g.N = 3 * s.d; g.K = s.d;
  g.rm = all;
  g.a_in = a.xn;
  g.ss_in = a.ss; g.ss_parts = a.ss_parts;
  g.w = pk + lo.s_wqkv;
  g.q = a.qbuf; g.q_seg_stride = (long)s.H * a.q * s.dh; g.q_head_stride = (long)a.q * s.dh; g.q_from = a.rows - a.q;
  g.k = a.k; g.vt = a.vt; g.kv_seg_stride = (long)s.H * a.cap * s.dh; g.kv_head_stride = (long)a.cap * s.dh;
  g.kv_cap = a.cap; g.kv_slot_base = a.slot_base;
  {
    FamilyTimer t(ONETRANS_K_S_QKV, st);
    OT_HIP(launch_gemm(GEMM_QKV, false, false, g, st), "S QKV GEMM launch");
  }
  if (a.kv_done) OT_HIP(hipEventRecord(a.kv_done, st), "layer event record");

  AttnParams at;
  memset(&at, 0, sizeof(at));
  at.nq = a.q; at.H = s.H; at.d = s.d;
  at.q = a.qbuf; at.q_seg_stride = g.q_seg_stride; at.q_head_stride = g.q_head_stride;
  at.res = a.x; at.res_seg_stride = a.x_seg_stride; at.res_row_base = tail.res_row_base; at.res_row_stride = d;
  at.k = a.k; at.vt = a.vt; at.kv_seg_stride = g.kv_seg_stride; at.kv_head_stride = g.kv_head_stride; at.kv_cap = a.cap;
  at.n_keys = a.n_keys; at.key_pos0 = a.key_pos0;
  at.q_pos0 = a.key_pos0 + a.slot_base + (a.rows - a.q);
  at.valid_from = a.valid_from;
  at.P = 1;
  at.scale_log2 = scale_log2(s);
  at.nout = norm_out(s, a.xn, (const float*)(pk + lo.s_gf), 0, a.ss);
  {
    FamilyTimer t(ONETRANS_K_S_ATTN, st);
    OT_HIP(launch_attention(false, s.dh, at, a.B, st), "S attention launch");
  }

  GemmParams u = base_gemm(s);
  u.M = a.B * a.q; u.N = s.F; u.K = s.d;
  u.rm = tail;
  u.a_in = a.xn;
  u.ss_in = a.ss; u.ss_parts = s.H;
  u.w = pk + lo.s_w1;
  u.hid_out = a.hid;
  {
    FamilyTimer t(ONETRANS_K_S_FFN_UP, st);
    OT_HIP(launch_gemm(GEMM_FFN_UP, false, false, u, st), "S FFN up launch");
  }

  GemmParams dn = base_gemm(s);
  dn.M = a.B * a.q; dn.N = s.d; dn.K = s.F;
  dn.rm = tail;
  dn.a_in = a.hid;
  dn.w = pk + lo.s_w2;
  dn.res_out = a.x;
  dn.nout = norm_out(s, a.xn, a.next_ga, 0, a.ss);
  {
    FamilyTimer t(ONETRANS_K_S_FFN_DOWN, st);
    OT_HIP(launch_gemm(GEMM_FFN_DOWN, false, false, dn, st), "S FFN down launch");
  }
  return ONETRANS_OK;
}

// One pass of NS rows through every layer: C groups of Pn rows, the NS positions
// p0..p0+Pn-1 of the sequence (private parameters of those positions).
//   - candidate pass (p0 = Pu): the rows also see the user's cached NS rows, uk / uv
//     (per layer, [H][Pu][dh] of this user);
//   - user pass (p0 = 0, Pn = Pu, C = the number of users, user = 0): group c is user c's
//     NS rows, which see that user's cached S rows (one attention segment per user); the
//     rows' K/V of each layer go to uk / uv ([B][H][Pu][dh], users 0..C-1).
struct NsPass {
  int p0 = 0, Pn = 0;
  bool user_pass = false;
  __bf16* uk[ONETRANS_MAX_LAYERS] = {};
  __bf16* uv[ONETRANS_MAX_LAYERS] = {};
};

// kv_ready (may be NULL): per layer, an event after which that layer's cache K/V is
// complete; the NS attention of the layer waits for it.
int score_impl(const Shape& s, const char* pk, const LayerOffsets* lo, const char* cache_buf, const size_t* k_off,
               const size_t* v_off, int n_appended, int user, const NsPass& ps, const uint16_t* ns_tokens, int C,
               float* ns_out, char* ws, hipStream_t st, const hipEvent_t* kv_ready = nullptr) {
  if (C == 0 || ps.Pn == 0) return ONETRANS_OK;
  const int Pn = ps.Pn, p0 = ps.p0;
  const ScoreWs w = score_ws(s, C, Pn);
  __bf16* qn = (__bf16*)(ws + w.qn);
  _Float16* xn = (_Float16*)(ws + w.xn);
  float* ss = (float*)(ws + w.ss);
  _Float16* hid = (_Float16*)(ws + w.hid);
  const long d = s.d, rows = (long)C * Pn;
  const size_t nsb = s.fp8 ? 1 : 2;  // bytes per packed NS weight
  const int* vf = (const int*)cache_buf;
  {
    InputParams ip;
    memset(&ip, 0, sizeof(ip));
    ip.tok = ns_tokens; ip.n_rows = (int)rows; ip.rows_per_seg = (int)rows; ip.d = s.d; ip.P = Pn;
    ip.x = ns_out;
    ip.nout = norm_out(s, xn, (const float*)(pk + lo[0].ns_ga) + p0 * d, d, ss);
    FamilyTimer t(ONETRANS_K_ELEMENTWISE, st);
    OT_HIP(launch_input_rows(ip, st), "NS input conversion launch");
  }
  // candidates: one segment of C groups; user pass: one segment per user (row c * Pn + j
  // either way; the segment index only places K/V and picks the user's cached keys)
  const RowMap rm = ps.user_pass ? RowMap{1, Pn, Pn * d, 0, Pn * d, d} : RowMap{C, Pn, 0, 0, Pn * d, d};
  const int n_seg = ps.user_pass ? C : 1;
  for (int l = 0; l < s.L; ++l) {
    const long cap = s.cap[l];
    const int len = s.n[l] + n_appended;
    // this pass's own K / V rows: the workspace, or the user's cache rows in the user pass
    __bf16* kn = ps.user_pass ? ps.uk[l] : (__bf16*)(ws + w.kn);
    __bf16* vn = ps.user_pass ? ps.uv[l] : (__bf16*)(ws + w.vn);
    const float* scales = (const float*)(pk + lo[l].ns_scale) + p0 * 5;
    GemmParams g = base_gemm(s);
    g.M = C; g.N = 3 * s.d; g.K = s.d; g.groups = Pn;
    g.rm = rm;
    g.a_in = xn;
    g.ss_in = ss; g.ss_parts = l == 0 ? 1 : s.d / 32;
    g.w = pk + lo[l].ns_wqkv + p0 * 3 * d * d * nsb; g.w_group_stride = 3 * d * d;
    g.wscale = scales; g.scale_idx0 = 0; g.scale_col_div = s.d;
    g.q = qn; g.q_seg_stride = ps.user_pass ? Pn * s.dh : 0; g.q_head_stride = rows * s.dh; g.q_from = 0;
    g.k = kn; g.vt = nullptr; g.v = vn; g.kv_slot_base = 0;
    if (ps.user_pass) {  // the cache's [user][H][Pu][dh] blocks
      g.kv_seg_stride = (long)s.H * Pn * s.dh; g.kv_head_stride = (long)Pn * s.dh; g.kv_cap = Pn;
    } else {
      g.kv_seg_stride = 0; g.kv_head_stride = rows * s.dh; g.kv_cap = (int)rows;
    }
    {
      FamilyTimer t(ONETRANS_K_NS_QKV, st);
      OT_HIP(launch_gemm(GEMM_QKV, s.fp8, true, g, st), "NS QKV GEMM launch");
    }

    AttnParams at;
    memset(&at, 0, sizeof(at));
    at.nq = (int)(rows / n_seg); at.H = s.H; at.d = s.d;
    at.q = qn; at.q_seg_stride = g.q_seg_stride; at.q_head_stride = rows * s.dh;
    at.res = ns_out; at.res_seg_stride = ps.user_pass ? Pn * d : 0; at.res_row_base = 0; at.res_row_stride = d;
    const long user_off = (long)user * s.H * cap * s.dh;
    at.k = (const __bf16*)(cache_buf + k_off[l]) + user_off;
    at.vt = (const __bf16*)(cache_buf + v_off[l]) + user_off;
    at.kv_seg_stride = ps.user_pass ? (long)s.H * cap * s.dh : 0; at.kv_head_stride = cap * s.dh; at.kv_cap = (int)cap;
    at.n_keys = len; at.key_pos0 = s.s_len - s.n[l]; at.q_pos0 = 0;
    at.valid_from = vf + user;
    at.kn = kn; at.vn = vn; at.kn_seg_stride = g.kv_seg_stride; at.kn_head_stride = g.kv_head_stride; at.P = Pn;
    if (!ps.user_pass && p0 > 0) {
      at.xk = ps.uk[l]; at.xv = ps.uv[l]; at.x_head_stride = (long)p0 * s.dh; at.n_x = p0;
    }
    at.scale_log2 = scale_log2(s);
    at.nout = norm_out(s, xn, (const float*)(pk + lo[l].ns_gf) + p0 * d, d, ss);
    if (kv_ready) OT_HIP(hipStreamWaitEvent(st, kv_ready[l], 0), "layer event wait");
    {
      FamilyTimer t(ONETRANS_K_NS_ATTN, st);
      OT_HIP(launch_attention(true, s.dh, at, n_seg, st), "NS attention launch");
    }

    GemmParams u = base_gemm(s);
    u.M = C; u.N = s.F; u.K = s.d; u.groups = Pn;
    u.rm = rm;
    u.a_in = xn;
    u.ss_in = ss; u.ss_parts = s.H;
    u.w = pk + lo[l].ns_w1 + p0 * (size_t)s.F * d * nsb; u.w_group_stride = (long)s.F * d;
    u.wscale = scales; u.scale_idx0 = 3;
    u.hid_out = hid;
    {
      FamilyTimer t(ONETRANS_K_NS_FFN_UP, st);
      OT_HIP(launch_gemm(GEMM_FFN_UP, s.fp8, true, u, st), "NS FFN up launch");
    }

    GemmParams dn = base_gemm(s);
    dn.M = C; dn.N = s.d; dn.K = s.F; dn.groups = Pn;
    dn.rm = rm;
    dn.a_in = hid;
    dn.w = pk + lo[l].ns_w2 + p0 * (size_t)d * s.F * nsb; dn.w_group_stride = d * s.F;
    dn.wscale = scales; dn.scale_idx0 = 4;
    dn.res_out = ns_out;
    dn.nout = norm_out(s, xn, l + 1 < s.L ? (const float*)(pk + lo[l + 1].ns_ga) + p0 * d : nullptr, d, ss);
    {
      FamilyTimer t(ONETRANS_K_NS_FFN_DOWN, st);
      OT_HIP(launch_gemm(GEMM_FFN_DOWN, s.fp8, true, dn, st), "NS FFN down launch");
    }
  }
  return ONETRANS_OK;
}

// The user-side NS rows of users [0, B) through every layer against their current
// cache (n_appended events after the prefill): inputs from the cache's copy, K/V of
// each layer into the cache, outputs to ns_user_out [B][Pu][d] when non-NULL.
int user_ns_impl(const Shape& s, const char* pk, const LayerOffsets* lo, char* cache_buf, const size_t* k_off,
                 const size_t* v_off, const UserNsOff& un, int B, int n_appended, float* ns_user_out, char* ws,
                 hipStream_t st) {
  if (s.Pu == 0 || B == 0) return ONETRANS_OK;
  NsPass ps;
  ps.p0 = 0; ps.Pn = s.Pu; ps.user_pass = true;
  for (int l = 0; l < s.L; ++l) {
    ps.uk[l] = (__bf16*)(cache_buf + un.k[l]);
    ps.uv[l] = (__bf16*)(cache_buf + un.v[l]);
  }
  float* out = ns_user_out ? ns_user_out : (float*)(ws + score_ws(s, B, s.Pu).total);
  return score_impl(s, pk, lo, cache_buf, k_off, v_off, n_appended, 0, ps, (const uint16_t*)(cache_buf + un.tok), B,
                    out, ws, st);
}

// The candidate pass of one user's C candidates.
NsPass candidate_pass(const Shape& s, char* cache_buf, const UserNsOff& un, int user) {
  NsPass ps;
  ps.p0 = s.Pu; ps.Pn = s.Pc;
  if (s.Pu > 0) {
    const long ublk = (long)s.H * s.Pu * s.dh;
    for (int l = 0; l < s.L; ++l) {
      ps.uk[l] = (__bf16*)(cache_buf + un.k[l]) + user * ublk;
      ps.uv[l] = (__bf16*)(cache_buf + un.v[l]) + user * ublk;
    }
  }
  return ps;
}

// kv_done (may be NULL): per layer, an event recorded once that layer's cache K/V is written
// (only without user-side NS rows). With them, the user NS inputs are copied into the
// cache and the user pass runs after the S side.
int prefill_impl(const Shape& s, const char* pk, const LayerOffsets* lo, const uint16_t* s_tokens,
                 const int32_t* s_lens, int B, char* cache_buf, const size_t* k_off, const size_t* v_off,
                 const UserNsOff& un, const uint16_t* ns_user_tokens, float* s_out, float* ns_user_out, char* ws,
                 hipStream_t st, const hipEvent_t* kv_done = nullptr) {
  const PrefillWs w = prefill_ws(s, B);
  float* x = (float*)(ws + w.x);
  float* ss = (float*)(ws + w.ss);
  _Float16* xn = (_Float16*)(ws + w.xn);
  int* vf = (int*)cache_buf;
  {
    InputParams ip;
    memset(&ip, 0, sizeof(ip));
    ip.tok = s_tokens; ip.s_lens = s_lens; ip.valid_from = vf;
    ip.n_rows = B * s.s_len; ip.rows_per_seg = s.s_len; ip.d = s.d; ip.P = 1;
    ip.x = x;
    ip.nout = norm_out(s, xn, (const float*)(pk + lo[0].s_ga), 0, ss);
    FamilyTimer t(ONETRANS_K_ELEMENTWISE, st);
    OT_HIP(launch_input_rows(ip, st), "S input conversion launch");
  }
  {
    ClearTailParams ct;
    memset(&ct, 0, sizeof(ct));
    ct.n_layers = s.L; ct.blocks = B * s.H; ct.dh = s.dh;
    for (int l = 0; l < s.L; ++l) {
      ct.k[l] = (__bf16*)(cache_buf + k_off[l]);
      ct.vt[l] = (__bf16*)(cache_buf + v_off[l]);
      ct.cap[l] = s.cap[l];
      ct.from[l] = s.n[l];
    }
    FamilyTimer t(ONETRANS_K_ELEMENTWISE, st);
    OT_HIP(launch_cache_clear_tail(ct, st), "cache tail clear launch");
  }
  for (int l = 0; l < s.L; ++l) {
    SLayerArgs a;
    a.B = B; a.rows = s.n[l]; a.q = s.q[l];
    a.x = x; a.x_seg_stride = (long)s.s_len * s.d; a.x_row_base = s.s_len - s.n[l];
    a.k = (__bf16*)(cache_buf + k_off[l]); a.vt = (__bf16*)(cache_buf + v_off[l]);
    a.cap = s.cap[l]; a.slot_base = 0; a.n_keys = s.n[l]; a.key_pos0 = s.s_len - s.n[l];
    a.valid_from = vf;
    a.qbuf = (__bf16*)(ws + w.q); a.xn = xn; a.hid = (_Float16*)(ws + w.hid);
    a.ss = ss; a.ss_parts = l == 0 ? 1 : s.d / 32;
    a.next_ga = l + 1 < s.L ? (const float*)(pk + lo[l + 1].s_ga) : nullptr;
    a.kv_done = kv_done ? kv_done[l] : nullptr;
    int rc = run_s_layer(s, pk, lo[l], a, st);
    if (rc) return rc;
  }
  const int qL = s.q[s.L - 1];
  {
    FamilyTimer t(ONETRANS_K_ELEMENTWISE, st);
    OT_HIP(launch_copy_rows_f32(x + (long)(s.s_len - qL) * s.d, (long)s.s_len * s.d, s_out, (long)qL * s.d,
                              (long)qL * s.d, B, st),
         "S output copy launch");
  }
  if (s.Pu > 0) {
    OT_HIP(hipMemcpyAsync(cache_buf + un.tok, ns_user_tokens, (size_t)B * s.Pu * s.d * 2, hipMemcpyDeviceToDevice, st),
           "user NS input copy");
    int rc = user_ns_impl(s, pk, lo, cache_buf, k_off, v_off, un, B, 0, ns_user_out, ws, st);
    if (rc) return rc;
  }
  return ONETRANS_OK;
}

// A second stream per thread and device for block_forward, with its fork / join and
// per-layer events; created on first use (default priority) and kept until the process
// ends. Thread-local, so calls from different threads stay independent.
struct SideStream {
  hipStream_t st = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  hipEvent_t layer[ONETRANS_MAX_LAYERS] = {};
};
constexpr int kMaxDevices = 64;
thread_local SideStream g_side[kMaxDevices];

int side_stream(SideStream** out) {
  int dev = 0;
  OT_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(ONETRANS_ERR_UNSUPPORTED, "device index out of range");
  SideStream& ss = g_side[dev];
  if (!ss.st) {
    OT_HIP(hipStreamCreateWithFlags(&ss.st, hipStreamNonBlocking), "side stream create");
    OT_HIP(hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming), "event create");
    OT_HIP(hipEventCreateWithFlags(&ss.join, hipEventDisableTiming), "event create");
    for (int l = 0; l < ONETRANS_MAX_LAYERS; ++l)
      OT_HIP(hipEventCreateWithFlags(&ss.layer[l], hipEventDisableTiming), "event create");
  }
  *out = &ss;
  return ONETRANS_OK;
}

}  // namespace

extern "C" {

const char* onetrans_status_str(int status) {
  switch (status) {
    case ONETRANS_OK: return "ok";
    case ONETRANS_ERR_INVALID_ARG: return "invalid argument";
    case ONETRANS_ERR_UNSUPPORTED: return "unsupported shape";
    case ONETRANS_ERR_WORKSPACE: return "buffer too small";
    case ONETRANS_ERR_CAPACITY: return "cache append capacity exceeded";
    case ONETRANS_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* onetrans_last_error(void) { return g_last_error.c_str(); }

int onetrans_check_config(const onetrans_config* cfg) {
  Shape s;
  return make_shape(cfg, s);
}

size_t onetrans_packed_weight_bytes(const onetrans_config* cfg) {
  Shape s;
  if (make_shape(cfg, s)) return 0;
  return packed_layout(s, nullptr);
}

int onetrans_pack_weights(const onetrans_config* cfg, const onetrans_layer_weights* layers, void* packed,
                          size_t packed_bytes, hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, s);
  if (rc) return rc;
  if (!layers || !packed) return fail(ONETRANS_ERR_INVALID_ARG, "layers and packed must be non-NULL");
  if (!aligned16(packed)) return fail(ONETRANS_ERR_INVALID_ARG, "packed must be 16-byte aligned");
  LayerOffsets lo[ONETRANS_MAX_LAYERS];
  const size_t need = packed_layout(s, lo);
  if (packed_bytes < need) return fail(ONETRANS_ERR_WORKSPACE, "packed buffer too small");
  for (int l = 0; l < s.L; ++l) {
    const onetrans_layer_weights& w = layers[l];
    if (!w.s_wqkv || !w.s_w1 || !w.s_w2 || !w.s_g_attn || !w.s_g_ffn || !w.ns_wqkv || !w.ns_w1 || !w.ns_w2 ||
        !w.ns_g_attn || !w.ns_g_ffn)
      return fail(ONETRANS_ERR_INVALID_ARG, "layer " + std::to_string(l) + ": a weight pointer is NULL");
    if (s.fp8 && !w.ns_scale) return fail(ONETRANS_ERR_INVALID_ARG, "E4M3 NS weights need ns_scale");
    const void* ptrs[] = {w.s_wqkv, w.s_w1, w.s_w2, w.s_g_attn, w.s_g_ffn, w.ns_wqkv, w.ns_w1, w.ns_w2, w.ns_g_attn, w.ns_g_ffn};
    for (const void* p : ptrs)
      if (!aligned16(p)) return fail(ONETRANS_ERR_INVALID_ARG, "layer " + std::to_string(l) + ": weight pointers must be 16-byte aligned");
  }
  char* pk = (char*)packed;
  const long d = s.d, F = s.F, P = s.P;
  for (int l = 0; l < s.L; ++l) {
    const onetrans_layer_weights& w = layers[l];
    const LayerOffsets& o = lo[l];
    OT_HIP(launch_pack_panels(w.s_wqkv, pk + o.s_wqkv, false, 1, 3 * d, d, stream), "pack");
    OT_HIP(launch_pack_panels(w.s_w1, pk + o.s_w1, false, 1, F, d, stream), "pack");
    OT_HIP(launch_pack_panels(w.s_w2, pk + o.s_w2, false, 1, d, F, stream), "pack");
    OT_HIP(hipMemcpyAsync(pk + o.s_ga, w.s_g_attn, d * 4, hipMemcpyDeviceToDevice, stream), "pack copy");
    OT_HIP(hipMemcpyAsync(pk + o.s_gf, w.s_g_ffn, d * 4, hipMemcpyDeviceToDevice, stream), "pack copy");
    if (s.fp8) {
      OT_HIP(launch_pack_panels(w.ns_wqkv, pk + o.ns_wqkv, true, P, 3 * d, d, stream), "pack");
      OT_HIP(launch_pack_panels(w.ns_w1, pk + o.ns_w1, true, P, F, d, stream), "pack");
      OT_HIP(launch_pack_panels(w.ns_w2, pk + o.ns_w2, true, P, d, F, stream), "pack");
      OT_HIP(hipMemcpyAsync(pk + o.ns_scale, w.ns_scale, P * 5 * 4, hipMemcpyDeviceToDevice, stream), "pack copy");
    } else {
      OT_HIP(launch_pack_panels(w.ns_wqkv, pk + o.ns_wqkv, false, P, 3 * d, d, stream), "pack");
      OT_HIP(launch_pack_panels(w.ns_w1, pk + o.ns_w1, false, P, F, d, stream), "pack");
      OT_HIP(launch_pack_panels(w.ns_w2, pk + o.ns_w2, false, P, d, F, stream), "pack");
    }
    OT_HIP(hipMemcpyAsync(pk + o.ns_ga, w.ns_g_attn, P * d * 4, hipMemcpyDeviceToDevice, stream), "pack copy");
    OT_HIP(hipMemcpyAsync(pk + o.ns_gf, w.ns_g_ffn, P * d * 4, hipMemcpyDeviceToDevice, stream), "pack copy");
  }
  return ONETRANS_OK;
}

size_t onetrans_kv_cache_bytes(const onetrans_config* cfg, int32_t n_users) {
  Shape s;
  if (make_shape(cfg, s) || n_users < 1) return 0;
  return cache_layout(s, n_users, nullptr, nullptr);
}

int onetrans_kv_cache_init(const onetrans_config* cfg, int32_t n_users, void* buf, size_t bytes,
                           onetrans_kv_cache* out) {
  Shape s;
  int rc = make_shape(cfg, s);
  if (rc) return rc;
  if (!buf || !out) return fail(ONETRANS_ERR_INVALID_ARG, "buf and out must be non-NULL");
  if (!aligned16(buf)) return fail(ONETRANS_ERR_INVALID_ARG, "cache buffer must be 16-byte aligned");
  if (n_users < 1) return fail(ONETRANS_ERR_INVALID_ARG, "n_users must be >= 1");
  if (bytes < cache_layout(s, n_users, nullptr, nullptr)) return fail(ONETRANS_ERR_WORKSPACE, "cache buffer too small");
  out->buf = buf;
  out->bytes = bytes;
  out->n_users = n_users;
  out->n_appended = 0;
  out->prefilled = 0;
  out->layout_key = layout_key(cfg);
  return ONETRANS_OK;
}

size_t onetrans_workspace_bytes(const onetrans_config* cfg, int32_t max_users, int32_t max_candidates,
                                int32_t max_append) {
  Shape s;
  if (make_shape(cfg, s) || max_users < 0 || max_candidates < 0 || max_append < 0) return 0;
  return std::max({prefill_need(s, max_users), append_need(s, max_users, max_append), score_ws(s, max_candidates, s.Pc).total});
}

size_t onetrans_block_forward_workspace_bytes(const onetrans_config* cfg, int32_t B, int32_t C) {
  Shape s;
  if (make_shape(cfg, s) || B < 1 || C < 0) return 0;
  // the cache, then the prefill's and the scoring's workspaces side by side (they run
  // concurrently)
  return cache_layout(s, B, nullptr, nullptr) + prefill_need(s, B) + score_ws(s, C, s.Pc).total;
}

int onetrans_user_prefill(const onetrans_config* cfg, const void* packed, const uint16_t* s_tokens,
                          const int32_t* s_lens, int32_t B, const uint16_t* ns_user_tokens, onetrans_kv_cache* cache,
                          float* s_out, float* ns_user_out, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, s);
  if (rc) return rc;
  if (!packed || !s_tokens || !s_lens || !cache || !cache->buf || !s_out || !workspace)
    return fail(ONETRANS_ERR_INVALID_ARG, "a pointer argument is NULL");
  if ((s.Pu > 0) != (ns_user_tokens != nullptr))
    return fail(ONETRANS_ERR_INVALID_ARG, "ns_user_tokens must be given exactly when n_ns_user > 0");
  if (!aligned16(packed) || !aligned16(s_tokens) || !aligned16(s_out) || !aligned16(workspace) ||
      !aligned16(ns_user_tokens) || !aligned16(ns_user_out))
    return fail(ONETRANS_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  if (B < 1 || B > cache->n_users) return fail(ONETRANS_ERR_INVALID_ARG, "B must be in [1, cache->n_users]");
  if ((rc = check_cache_key(cfg, cache))) return rc;
  if (cache->bytes < cache_layout(s, cache->n_users, nullptr, nullptr))
    return fail(ONETRANS_ERR_WORKSPACE, "cache buffer smaller than its n_users needs");
  if (workspace_bytes < prefill_need(s, B)) return fail(ONETRANS_ERR_WORKSPACE, "workspace too small for prefill");
  LayerOffsets lo[ONETRANS_MAX_LAYERS];
  packed_layout(s, lo);
  size_t k_off[ONETRANS_MAX_LAYERS], v_off[ONETRANS_MAX_LAYERS];
  UserNsOff un;
  cache_layout(s, cache->n_users, k_off, v_off, &un);
  rc = prefill_impl(s, (const char*)packed, lo, s_tokens, s_lens, B, (char*)cache->buf, k_off, v_off, un,
                    ns_user_tokens, s_out, ns_user_out, (char*)workspace, stream);
  if (rc) return rc;
  cache->n_appended = 0;
  cache->prefilled = B;
  return ONETRANS_OK;
}

int onetrans_kv_append(const onetrans_config* cfg, const void* packed, const uint16_t* new_tokens, int32_t m,
                       onetrans_kv_cache* cache, float* new_out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, s);
  if (rc) return rc;
  if (!packed || !cache || !cache->buf) return fail(ONETRANS_ERR_INVALID_ARG, "a pointer argument is NULL");
  if ((rc = check_cache_key(cfg, cache))) return rc;
  if (cache->prefilled < 1 || cache->prefilled > cache->n_users)
    return fail(ONETRANS_ERR_INVALID_ARG, "cache has not been prefilled");
  if (m < 0) return fail(ONETRANS_ERR_INVALID_ARG, "m must be >= 0");
  if (cache->n_appended + (long)m > s.append_cap) return fail(ONETRANS_ERR_CAPACITY, "append exceeds append_cap");
  if (m == 0) return ONETRANS_OK;
  if (!new_tokens || !new_out || !workspace) return fail(ONETRANS_ERR_INVALID_ARG, "a pointer argument is NULL");
  if (!aligned16(packed) || !aligned16(new_tokens) || !aligned16(new_out) || !aligned16(workspace))
    return fail(ONETRANS_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  const int B = cache->prefilled;  // users [0, B) hold a prefill; the layout is that of n_users
  if (cache->bytes < cache_layout(s, cache->n_users, nullptr, nullptr))
    return fail(ONETRANS_ERR_WORKSPACE, "cache buffer smaller than its n_users needs");
  const AppendWs w = append_ws(s, B, m);
  if (workspace_bytes < append_need(s, B, m)) return fail(ONETRANS_ERR_WORKSPACE, "workspace too small for append");
  LayerOffsets lo[ONETRANS_MAX_LAYERS];
  packed_layout(s, lo);
  size_t k_off[ONETRANS_MAX_LAYERS], v_off[ONETRANS_MAX_LAYERS];
  UserNsOff un;
  cache_layout(s, cache->n_users, k_off, v_off, &un);
  char* cb = (char*)cache->buf;
  char* ws = (char*)workspace;
  _Float16* xn = (_Float16*)(ws + w.xn);
  float* ss = (float*)(ws + w.ss);
  {
    InputParams ip;
    memset(&ip, 0, sizeof(ip));
    ip.tok = new_tokens; ip.n_rows = B * m; ip.rows_per_seg = m; ip.d = s.d; ip.P = 1;
    ip.x = new_out;
    ip.nout = norm_out(s, xn, (const float*)((const char*)packed + lo[0].s_ga), 0, ss);
    FamilyTimer t(ONETRANS_K_ELEMENTWISE, stream);
    OT_HIP(launch_input_rows(ip, stream), "append input conversion launch");
  }
  for (int l = 0; l < s.L; ++l) {
    const int len = s.n[l] + cache->n_appended;
    SLayerArgs a;
    a.B = B; a.rows = m; a.q = m;
    a.x = new_out; a.x_seg_stride = (long)m * s.d; a.x_row_base = 0;
    a.k = (__bf16*)(cb + k_off[l]); a.vt = (__bf16*)(cb + v_off[l]);
    a.cap = s.cap[l]; a.slot_base = len; a.n_keys = len + m; a.key_pos0 = s.s_len - s.n[l];
    a.valid_from = (const int*)cb;
    a.qbuf = (__bf16*)(ws + w.q); a.xn = xn; a.hid = (_Float16*)(ws + w.hid);
    a.ss = ss; a.ss_parts = l == 0 ? 1 : s.d / 32;
    a.next_ga = l + 1 < s.L ? (const float*)((const char*)packed + lo[l + 1].s_ga) : nullptr;
    a.kv_done = nullptr;
    rc = run_s_layer(s, (const char*)packed, lo[l], a, stream);
    if (rc) return rc;
  }
  cache->n_appended += m;
  // the user-side NS rows see the grown history: recompute them from the kept inputs
  return user_ns_impl(s, (const char*)packed, lo, cb, k_off, v_off, un, B, cache->n_appended, nullptr, ws, stream);
}

}  // extern "C"

namespace {

// Host checks of a scoring call (no device work). *done is set when there is nothing to
// launch (C == 0).
int score_check(const onetrans_config* cfg, Shape& s, const void* packed, const onetrans_kv_cache* cache, int32_t user,
                const uint16_t* ns_tokens, int32_t C, float* ns_out, bool* done) {
  *done = false;
  int rc = make_shape(cfg, s);
  if (rc) return rc;
  if (!packed || !cache || !cache->buf) return fail(ONETRANS_ERR_INVALID_ARG, "a pointer argument is NULL");
  if ((rc = check_cache_key(cfg, cache))) return rc;
  if (cache->prefilled < 1 || cache->prefilled > cache->n_users)
    return fail(ONETRANS_ERR_INVALID_ARG, "cache has not been prefilled");
  if (user < 0 || user >= cache->prefilled) return fail(ONETRANS_ERR_INVALID_ARG, "user out of range (not prefilled)");
  if (C < 0) return fail(ONETRANS_ERR_INVALID_ARG, "C must be >= 0");
  if (C == 0) {
    *done = true;
    return ONETRANS_OK;
  }
  if (!ns_tokens || !ns_out) return fail(ONETRANS_ERR_INVALID_ARG, "a pointer argument is NULL");
  if (!aligned16(packed) || !aligned16(ns_tokens) || !aligned16(ns_out))
    return fail(ONETRANS_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  if ((long)C * s.Pc > (1L << 26)) return fail(ONETRANS_ERR_UNSUPPORTED, "C * (n_ns - n_ns_user) must be <= 2^26");
  if (cache->bytes < cache_layout(s, cache->n_users, nullptr, nullptr))
    return fail(ONETRANS_ERR_WORKSPACE, "cache buffer smaller than its n_users needs");
  return ONETRANS_OK;
}

int score_run(const Shape& s, const void* packed, const onetrans_kv_cache* cache, int32_t user,
              const uint16_t* ns_tokens, int32_t C, float* ns_out, char* ws, hipStream_t stream) {
  LayerOffsets lo[ONETRANS_MAX_LAYERS];
  packed_layout(s, lo);
  size_t k_off[ONETRANS_MAX_LAYERS], v_off[ONETRANS_MAX_LAYERS];
  UserNsOff un;
  cache_layout(s, cache->n_users, k_off, v_off, &un);
  char* cb = (char*)cache->buf;
  return score_impl(s, (const char*)packed, lo, cb, k_off, v_off, cache->n_appended, user,
                    candidate_pass(s, cb, un, user), ns_tokens, C, ns_out, ws, stream);
}

// ---- scratch of the allocation-free scoring call ----
// One array per GPU the library runs on, held until the process ends. Host code never uses
// the name `scratch` as an address (on the host it only stands in for the symbol): the
// device address comes from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) char scratch[ONETRANS_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(char** out) {
  int dev = 0;
  OT_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(ONETRANS_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    OT_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "scratch symbol address");
    if (!p) return fail(ONETRANS_ERR_HIP, "scratch symbol address is NULL");
    g_scratch_ptr[dev] = (char*)p;
  }
  *out = g_scratch_ptr[dev];
  return ONETRANS_OK;
}

}  // namespace

extern "C" {

int onetrans_score_candidates(const onetrans_config* cfg, const void* packed, const onetrans_kv_cache* cache,
                              int32_t user, const uint16_t* ns_tokens, int32_t C, float* ns_out, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  Shape s;
  bool done = false;
  int rc = score_check(cfg, s, packed, cache, user, ns_tokens, C, ns_out, &done);
  if (rc || done) return rc;
  if (!workspace) return fail(ONETRANS_ERR_INVALID_ARG, "a pointer argument is NULL");
  if (!aligned16(workspace)) return fail(ONETRANS_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  if (workspace_bytes < score_ws(s, C, s.Pc).total) return fail(ONETRANS_ERR_WORKSPACE, "workspace too small for scoring");
  return score_run(s, packed, cache, user, ns_tokens, C, ns_out, (char*)workspace, stream);
}

int onetrans_score_candidates_noalloc(const onetrans_config* cfg, const void* packed, const onetrans_kv_cache* cache,
                                      int32_t user, const uint16_t* ns_tokens, int32_t C, float* ns_out,
                                      hipStream_t stream) {
  Shape s;
  bool done = false;
  int rc = score_check(cfg, s, packed, cache, user, ns_tokens, C, ns_out, &done);
  if (rc || done) return rc;
  const size_t need = score_ws(s, C, s.Pc).total;
  if (need > (size_t)ONETRANS_NOALLOC_SCRATCH_BYTES)
    return fail(ONETRANS_ERR_WORKSPACE, "scoring " + std::to_string(C) + " candidates needs " + std::to_string(need) +
                                            " bytes of scratch; the allocation-free call holds " +
                                            std::to_string((size_t)ONETRANS_NOALLOC_SCRATCH_BYTES) +
                                            " (score fewer candidates per call, or use onetrans_score_candidates)");
  char* ws = nullptr;
  if ((rc = scratch_of_current_device(&ws))) return rc;
  return score_run(s, packed, cache, user, ns_tokens, C, ns_out, ws, stream);
}

int onetrans_block_forward(const onetrans_config* cfg, const void* packed, const uint16_t* s_tokens,
                           const int32_t* s_lens, int32_t B, const uint16_t* ns_user_tokens, const uint16_t* ns_tokens,
                           int32_t C, float* s_out, float* ns_out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, s);
  if (rc) return rc;
  const bool cand = C > 0 && s.Pc > 0;  // candidate rows to score
  if (!packed || !s_tokens || !s_lens || !s_out || !workspace || (cand && (!ns_tokens || !ns_out)))
    return fail(ONETRANS_ERR_INVALID_ARG, "a pointer argument is NULL");
  if ((s.Pu > 0) != (ns_user_tokens != nullptr))
    return fail(ONETRANS_ERR_INVALID_ARG, "ns_user_tokens must be given exactly when n_ns_user > 0");
  if (!aligned16(packed) || !aligned16(s_tokens) || !aligned16(s_out) || !aligned16(workspace) ||
      !aligned16(ns_user_tokens) || (cand && (!aligned16(ns_tokens) || !aligned16(ns_out))))
    return fail(ONETRANS_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  if (B < 1 || C < 0) return fail(ONETRANS_ERR_INVALID_ARG, "B must be >= 1 and C >= 0");
  if ((long)C * s.Pc > (1L << 26)) return fail(ONETRANS_ERR_UNSUPPORTED, "C * (n_ns - n_ns_user) must be <= 2^26");
  if (workspace_bytes < onetrans_block_forward_workspace_bytes(cfg, B, C))
    return fail(ONETRANS_ERR_WORKSPACE, "workspace too small for block_forward");
  LayerOffsets lo[ONETRANS_MAX_LAYERS];
  packed_layout(s, lo);
  size_t k_off[ONETRANS_MAX_LAYERS], v_off[ONETRANS_MAX_LAYERS];
  UserNsOff un;
  const size_t cache_bytes = cache_layout(s, B, k_off, v_off, &un);
  char* cb = (char*)workspace;
  char* pws = cb + cache_bytes;
  char* sws = pws + prefill_need(s, B);
  const long per_user = (long)C * s.Pc * s.d;
  if (!cand || s.Pu > 0) {
    // everything on `stream`: the whole user side, then each user's candidates
    rc = prefill_impl(s, (const char*)packed, lo, s_tokens, s_lens, B, cb, k_off, v_off, un, ns_user_tokens, s_out,
                      nullptr, pws, stream);
    if (rc || !cand) return rc;
    for (int u = 0; u < B; ++u) {
      rc = score_impl(s, (const char*)packed, lo, cb, k_off, v_off, 0, u, candidate_pass(s, cb, un, u),
                      ns_tokens + u * per_user, C, ns_out + u * per_user, sws, stream);
      if (rc) return rc;
    }
    return ONETRANS_OK;
  }
  // The S side runs on `stream`; the NS side on this thread's second stream, which starts
  // after everything queued on `stream` so far and whose layer l waits only for the
  // event after the S side's layer-l QKV (the cache rows it reads). The NS side's small
  // dependence on the S side lets the latency-bound S layers fill idle CUs.
  SideStream* side = nullptr;
  rc = side_stream(&side);
  if (rc) return rc;
  OT_HIP(hipEventRecord(side->fork, stream), "fork event record");
  OT_HIP(hipStreamWaitEvent(side->st, side->fork, 0), "fork event wait");
  rc = prefill_impl(s, (const char*)packed, lo, s_tokens, s_lens, B, cb, k_off, v_off, un, nullptr, s_out, nullptr,
                    pws, stream, side->layer);
  if (rc) return rc;
  for (int u = 0; u < B; ++u) {
    rc = score_impl(s, (const char*)packed, lo, cb, k_off, v_off, 0, u, candidate_pass(s, cb, un, u),
                    ns_tokens + u * per_user, C, ns_out + u * per_user, sws, side->st, side->layer);
    if (rc) return rc;
  }
  OT_HIP(hipEventRecord(side->join, side->st), "join event record");
  OT_HIP(hipStreamWaitEvent(stream, side->join, 0), "join event wait");
  return ONETRANS_OK;
}

int onetrans_kv_cache_read(const onetrans_config* cfg, const onetrans_kv_cache* cache, int32_t layer, int32_t user,
                           int32_t rows, uint16_t* k_out, uint16_t* v_out, hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, s);
  if (rc) return rc;
  if (!cache || !cache->buf || !k_out || !v_out) return fail(ONETRANS_ERR_INVALID_ARG, "a pointer argument is NULL");
  if ((rc = check_cache_key(cfg, cache))) return rc;
  if (layer < 0 || layer >= s.L) return fail(ONETRANS_ERR_INVALID_ARG, "layer out of range");
  if (user < 0 || user >= cache->prefilled || cache->prefilled > cache->n_users)
    return fail(ONETRANS_ERR_INVALID_ARG, "user out of range (not prefilled)");
  if (rows < 0 || rows > s.n[layer] + cache->n_appended) return fail(ONETRANS_ERR_INVALID_ARG, "rows beyond the filled length");
  size_t k_off[ONETRANS_MAX_LAYERS], v_off[ONETRANS_MAX_LAYERS];
  cache_layout(s, cache->n_users, k_off, v_off);
  const long uo = (long)user * s.H * s.cap[layer] * s.dh;
  const char* cb = (const char*)cache->buf;
  OT_HIP(launch_cache_read((const __bf16*)(cb + k_off[layer]) + uo, (const __bf16*)(cb + v_off[layer]) + uo, s.H, s.dh,
                           s.cap[layer], rows, (__bf16*)k_out, (__bf16*)v_out, stream),
         "cache read launch");
  return ONETRANS_OK;
}

const char* onetrans_attention_route(int32_t ns, int32_t head_dim, int32_t n_queries, int32_t n_heads,
                                     int32_t n_seg) {
  if ((head_dim != 32 && head_dim != 64) || n_queries < 1 || n_heads < 1 || n_seg < 1) return "none";
  return attention_route_name(attention_route(ns != 0, head_dim, n_queries, n_heads, n_seg));
}

int onetrans_kernel_timing_enable(uint32_t mask) {
  for (const TimingRec& r : g_timing) {
    (void)hipEventSynchronize(r.b);
    g_event_pool.push_back(r.a);
    g_event_pool.push_back(r.b);
  }
  g_timing.clear();
  g_timing_mask = mask & ((1u << ONETRANS_K_COUNT) - 1);
  return ONETRANS_OK;
}

int onetrans_kernel_timing_read(int family, double* total_ms, int64_t* launches) {
  if (family < 0 || family >= ONETRANS_K_COUNT || !total_ms || !launches)
    return fail(ONETRANS_ERR_INVALID_ARG, "bad kernel family or NULL output");
  double sum = 0.0;
  int64_t n = 0;
  for (const TimingRec& r : g_timing) {
    if (r.fam != family) continue;
    OT_HIP(hipEventSynchronize(r.b), "event synchronize");
    float ms = 0.f;
    OT_HIP(hipEventElapsedTime(&ms, r.a, r.b), "event elapsed time");
    sum += ms;
    ++n;
  }
  *total_ms = sum;
  *launches = n;
  return ONETRANS_OK;
}

}  // extern "C"
