/*
 * onetrans.h - C ABI of the OneTrans block-stack forward pass on MI355X (gfx950).
 *
 * The method (agihunt.info summary of OneTrans, arXiv 2510.26104, "method"
 * paragraphs; asterzephyr.xyz blog, designs two to four):
 *   - one token sequence per (user, candidate): S-tokens (behaviour history)
 *     first, then n_ns NS-tokens (user / item / context fields);
 *   - every block is a pre-norm (RMSNorm) causal Transformer layer with mixed
 *     parameters: all S-tokens share one QKV projection and one FFN, NS position
 *     k has its own private QKV projection and FFN;
 *   - an S-token sees earlier events and itself; an NS-token sees every present
 *     S-token and the NS-tokens up to itself;
 *   - pyramid: layer l keeps only the last q_l S rows as queries, while its keys
 *     and values cover all S rows that enter the layer;
 *   - the S side never sees NS tokens, so its per-layer K/V is computed once per
 *     user, cached, extended by newly arrived events, and shared by every
 *     candidate; only the NS side runs per candidate. The user side also covers
 *     profile fields (asterzephyr.xyz, design four): the first n_ns_user NS
 *     positions may hold user fields, which depend on the user only, so they
 *     are computed once in the prefill and their K/V is cached beside the S
 *     side's; a candidate's rows (positions n_ns_user..n_ns-1) see them as
 *     earlier NS rows.
 * Readings where the pages are silent: no biases; no output projection (heads
 * are concatenated into the residual); score scale 1/sqrt(head_dim); RMSNorm
 * x / sqrt(mean(x^2) + eps) * g; FFN = W2 GELU_erf(W1 x) with a residual; no
 * positional term inside the block; an appended event is a query at every layer.
 *
 * Conventions for every call:
 *   - Device memory is owned by the caller (for instance torch tensors). The
 *     library allocates no device memory and keeps no pointer after a call
 *     returns. "dev" marks device pointers, "host" host pointers.
 *   - Compute calls are asynchronous on `stream` (NULL = the default stream).
 *     They validate every argument on the host first and return a status with
 *     no side effect when something is wrong. A launch failure returns
 *     ONETRANS_ERR_HIP; faults inside kernels surface at the caller's next
 *     synchronisation.
 *   - Matrices use the torch Linear layout [out][in]; all arrays are dense,
 *     row-major and 16-byte aligned.
 *   - Numerics: RMSNorm, softmax and the residual stream in fp32; the five
 *     linear maps take fp16 operands (bf16 weights converted at pack time, exact
 *     inside the range stated at onetrans_pack_weights; E4M3FN weights decoded
 *     exactly) with fp32 accumulation; attention
 *     takes bf16 Q, K, V and probabilities with fp32 accumulation. A norm
 *     feeding a linear map is applied as r * ((x * g) W): the operand is
 *     x * g rounded to fp16 and the row factor r = 1/sqrt(mean(x^2) + eps)
 *     (fp32) scales the accumulator, so every |x_j g_j| of the residual
 *     stream must stay below 65504 (fp16 range); entries below 2^-14 (6.1e-5)
 *     fall on the fp16 subnormal grid (step 2^-24), so rows whose rms is far
 *     below 1e-3 lose relative precision in their linear maps.
 *   - Not thread-safe for concurrent calls that share a workspace or a cache;
 *     calls on distinct workspaces and caches are independent.
 *   - onetrans_last_error() returns a thread-local description of the last
 *     failure of the calling thread.
 */
#ifndef ONETRANS_H
#define ONETRANS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ONETRANS_MAX_LAYERS 16

typedef enum {
  ONETRANS_OK = 0,
  ONETRANS_ERR_INVALID_ARG = 1,   /* NULL pointer, bad size, misaligned pointer */
  ONETRANS_ERR_UNSUPPORTED = 2,   /* shape outside the supported set (see onetrans_config) */
  ONETRANS_ERR_WORKSPACE = 3,     /* workspace or buffer smaller than the sizing call asks */
  ONETRANS_ERR_CAPACITY = 4,      /* append beyond the cache's append capacity */
  ONETRANS_ERR_HIP = 5            /* a HIP runtime call or kernel launch failed */
} onetrans_status;

typedef enum { ONETRANS_W_BF16 = 0, ONETRANS_W_FP8_E4M3 = 1 } onetrans_wdtype;

/* Model shape. Supported: 1 <= n_layers <= 16; d_model % 64 == 0 and
 * d_model <= 1024; head_dim = d_model / n_heads in {32, 64}; ffn_hidden % 64 == 0;
 * 1 <= n_ns <= 256; s_len >= 1; q_sched[0] <= s_len and
 * q_sched[l] <= q_sched[l-1], every q_sched[l] >= 1 (pyramid: layer l keeps
 * the last q_sched[l] S rows; layer l's input has n_l = s_len (l = 0) or
 * q_sched[l-1] rows); append_cap >= 0 (events a cache can take after its
 * prefill); rms_eps > 0; ns_wdtype one of onetrans_wdtype (S weights are always
 * bf16); 0 <= n_ns_user <= n_ns (user-side NS positions, computed in the
 * prefill; 0: every NS position belongs to the candidate). */
typedef struct onetrans_config {
  int32_t n_layers, d_model, n_heads, ffn_hidden, n_ns, s_len;
  int32_t q_sched[ONETRANS_MAX_LAYERS];
  int32_t append_cap;
  float rms_eps;
  int32_t ns_wdtype;
  int32_t n_ns_user;
} onetrans_config;

/* One layer's parameters as the caller holds them (dev pointers, read only).
 *   s_wqkv  bf16 [3d][d]   rows 0..d-1 = W_Q, d..2d-1 = W_K, 2d..3d-1 = W_V
 *   s_w1    bf16 [F][d]    s_w2 bf16 [d][F]
 *   s_g_attn, s_g_ffn  fp32 [d]       RMSNorm gains of the S rows
 *   ns_wqkv bf16|e4m3 [n_ns][3d][d]   ns_w1 [n_ns][F][d]   ns_w2 [n_ns][d][F]
 *   ns_scale fp32 [n_ns][5]  per-matrix scale (W_Q, W_K, W_V, W1, W2) when the
 *            NS weights are E4M3FN codes (effective weight = scale * code); NULL for bf16
 *   ns_g_attn, ns_g_ffn fp32 [n_ns][d]  RMSNorm gains of NS position k */
typedef struct onetrans_layer_weights {
  const void *s_wqkv, *s_w1, *s_w2;
  const float *s_g_attn, *s_g_ffn;
  const void *ns_wqkv, *ns_w1, *ns_w2;
  const float *ns_scale;
  const float *ns_g_attn, *ns_g_ffn;
} onetrans_layer_weights;

/* A per-user, per-layer user-side K/V cache living in one caller-owned device
 * buffer (layout private to the library; it is plain device memory, so it can
 * be copied, saved and restored byte for byte together with this struct).
 * Layer l holds n_l + append_cap S rows per user; rows [0, n_l + n_appended) are
 * filled. With n_ns_user > 0 it also holds, per layer and user, the K/V of the
 * user-side NS rows and the user-side NS inputs (for the recompute after an
 * append). Fields are set by onetrans_kv_cache_init and updated by the calls. */
typedef struct onetrans_kv_cache {
  void* buf;            /* dev, onetrans_kv_cache_bytes(cfg, n_users) bytes */
  size_t bytes;
  int32_t n_users;
  int32_t n_appended;   /* events appended since the prefill (same for all users) */
  int32_t prefilled;    /* users [0, prefilled) hold a prefill (set by onetrans_user_prefill; 0 before) */
  uint64_t layout_key;  /* the user-side shape the cache was laid out for (set by init) */
} onetrans_kv_cache;

/* Multi-stage scoring on one cache (the successor system, OneTrans-V2: retrieval,
 * pre-rank and fine-rank become tasks of one model that encodes the user's behaviour
 * once per request while each stage keeps its own candidate features; rss.com
 * OneTrans-V2 podcast page, "Key takeaways", first item, and the welcome.ai OneTrans-V2
 * summary, "Academic Abstract"): the cache depends only on the
 * user-side shape (n_layers, d_model, n_heads, s_len, q_sched, append_cap,
 * n_ns_user, rms_eps) and on the S weights. Any config that shares that shape, with
 * its own n_ns, ns_wdtype and packed NS weights, may score against a cache another
 * such config prefilled; every call checks layout_key and rejects a cache laid out
 * for another user-side shape with ONETRANS_ERR_INVALID_ARG (no launch). The
 * user-side NS rows (n_ns_user > 0) are those of the model that ran the prefill. */

/* ---- sizing, packing, cache set-up (host calls) -------------------------- */

/* Validates a config: ONETRANS_OK or the reason it is not supported. */
int onetrans_check_config(const onetrans_config* cfg);

/* Bytes of the packed weight buffer the compute calls read. 0 on a bad config. */
size_t onetrans_packed_weight_bytes(const onetrans_config* cfg);

/* Converts the caller's per-layer weights (layers[cfg->n_layers]) into the
 * packed device buffer `packed` (bf16 weights become fp16, E4M3FN codes are
 * copied, both rearranged into the GEMMs' blocked layout; fp32 gains/scales are
 * copied). Asynchronous on `stream`. The packed buffer
 * must stay alive and unchanged while compute calls use it.
 * Range: the bf16 -> fp16 conversion (round to nearest even) is exact for weights
 * with 2^-17 <= |w| < 65536 (the largest such bf16 value is 65280) and for zero; smaller magnitudes are rounded to the
 * fp16 subnormal grid (step 2^-24) and larger ones become infinite. The call does
 * not inspect the values; keep weights inside that range. */
int onetrans_pack_weights(const onetrans_config* cfg, const onetrans_layer_weights* layers,
                          void* packed, size_t packed_bytes, hipStream_t stream);

/* Bytes of a K/V cache for n_users users. 0 on a bad config or n_users < 1. */
size_t onetrans_kv_cache_bytes(const onetrans_config* cfg, int32_t n_users);

/* Fills *out for a cache of n_users users in `buf` (no device work). */
int onetrans_kv_cache_init(const onetrans_config* cfg, int32_t n_users, void* buf, size_t bytes,
                           onetrans_kv_cache* out);

/* Workspace bytes that cover every compute call with at most max_users users,
 * max_candidates candidates per call and max_append appended events per call. */
size_t onetrans_workspace_bytes(const onetrans_config* cfg, int32_t max_users,
                                int32_t max_candidates, int32_t max_append);

/* ---- compute calls (asynchronous on stream) ------------------------------ */

/* User prefill (agihunt.info OneTrans summary, pyramid / KV paragraph: the S side
 * runs once per user; asterzephyr.xyz blog, design four: the user side, profile
 * fields included, is computed ahead and cached).
 * Runs the S side of B users through every layer, writes each
 * layer's K/V (all n_l input rows) into `cache` and returns the last layer's
 * S outputs; then, with n_ns_user > 0, runs each user's user-side NS rows
 * (NS positions 0..n_ns_user-1, after every S row) and caches their K/V too.
 *   s_tokens  dev bf16 [B][s_len][d]; user u's history is right-aligned: its
 *             s_lens[u] events sit in slots [s_len - s_lens[u], s_len); the
 *             padding slots' contents are ignored (treated as zero)
 *   s_lens    dev int32 [B]; values are clamped to [0, s_len]
 *   ns_user_tokens dev bf16 [B][n_ns_user][d]; must be NULL iff n_ns_user == 0
 *   s_out     dev fp32 [B][q_sched[L-1]][d]; rows of padding slots are 0
 *   ns_user_out dev fp32 [B][n_ns_user][d]: the user NS rows after the last
 *             layer, or NULL (not returned)
 * The cache must have been initialised for at least B users; it is reset
 * (n_appended = 0, prefilled = B): scoring, appends and reads then accept users
 * [0, B) only, until the next prefill. */
int onetrans_user_prefill(const onetrans_config* cfg, const void* packed,
                          const uint16_t* s_tokens, const int32_t* s_lens, int32_t B,
                          const uint16_t* ns_user_tokens, onetrans_kv_cache* cache, float* s_out,
                          float* ns_user_out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* KV append (agihunt.info OneTrans summary, pyramid / KV paragraph: sequence K/V
 * can be appended across requests).
 * m newly arrived events per user (for the B = cache->prefilled users)
 * enter every layer as queries at the next global positions; each sees the
 * user's valid cached rows and the new events up to itself. Their K/V rows are
 * appended in place and cache->n_appended grows by m (host-side, at enqueue).
 *   new_tokens dev bf16 [B][m][d], B = cache->prefilled
 *   new_out    dev fp32 [B][m][d]: the new events' outputs after the last layer
 * With n_ns_user > 0 the user-side NS rows see the grown history, so their
 * cached K/V is recomputed from the inputs the prefill kept.
 * Returns ONETRANS_ERR_CAPACITY if n_appended + m > cfg->append_cap. */
int onetrans_kv_append(const onetrans_config* cfg, const void* packed,
                       const uint16_t* new_tokens, int32_t m, onetrans_kv_cache* cache,
                       float* new_out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Candidate scoring (agihunt.info OneTrans summary, pyramid / KV paragraph: the NS
 * side runs per candidate against the shared S side; block paragraph: each NS token
 * sees the full history and the NS tokens before it).
 * The NS side of C candidates of user `user` against that
 * user's cached user-side K/V (cross-request KV sharing). A candidate has
 * Pc = n_ns - n_ns_user rows, NS positions n_ns_user..n_ns-1.
 *   ns_tokens dev bf16 [C][Pc][d]
 *   ns_out    dev fp32 [C][Pc][d]: the candidate rows after the last layer
 * user must be below cache->prefilled. C may be 0 (no work); so may Pc. */
int onetrans_score_candidates(const onetrans_config* cfg, const void* packed,
                              const onetrans_kv_cache* cache, int32_t user,
                              const uint16_t* ns_tokens, int32_t C, float* ns_out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Allocation-free scoring, for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Same computation and arguments as onetrans_score_candidates without the
 * workspace: its scratch is one static device array of ONETRANS_NOALLOC_SCRATCH_BYTES per
 * GPU, which the library holds from the first call on that GPU until the process ends.
 * The call allocates nothing (no hipMalloc, no library allocation). Returns
 * ONETRANS_ERR_WORKSPACE with no launch when the call needs more scratch than that
 * (the need is onetrans_workspace_bytes(cfg, 0, C, 0); at the OneTrans-L shape, 256
 * candidates of 32 NS rows need about 51 MB). Calls that overlap on one GPU (concurrent
 * streams, threads) share the array and race; serialise them. Nothing in the array
 * needs to start at zero, so its contents from an earlier call are harmless. */
#define ONETRANS_NOALLOC_SCRATCH_BYTES (64u << 20)
int onetrans_score_candidates_noalloc(const onetrans_config* cfg, const void* packed,
                                      const onetrans_kv_cache* cache, int32_t user,
                                      const uint16_t* ns_tokens, int32_t C, float* ns_out,
                                      hipStream_t stream);

/* Block forward (agihunt.info OneTrans summary, block and pyramid / KV paragraphs).
 * Full pass without a persistent cache: prefill of B users into a cache held
 * in the workspace, then scoring of each user's C candidates.
 *   s_tokens, s_lens, ns_user_tokens, s_out as in onetrans_user_prefill
 *   ns_tokens dev bf16 [B][C][Pc][d], ns_out dev fp32 [B][C][Pc][d]
 *   (Pc = n_ns - n_ns_user)
 * Size the workspace with onetrans_block_forward_workspace_bytes (the cache plus
 * separate prefill and scoring areas). Without user-side NS rows the S side
 * runs on `stream` and the NS side concurrently on a second stream that the
 * library creates on first use for the calling thread and device (default
 * priority, kept until the process ends); NS layer l waits only for the S
 * side's layer-l cache rows. With user-side NS rows both run on `stream`, the
 * candidates after the whole user side. Work queued on `stream` after the call
 * waits for everything. */
size_t onetrans_block_forward_workspace_bytes(const onetrans_config* cfg, int32_t B, int32_t C);
int onetrans_block_forward(const onetrans_config* cfg, const void* packed,
                           const uint16_t* s_tokens, const int32_t* s_lens, int32_t B,
                           const uint16_t* ns_user_tokens, const uint16_t* ns_tokens, int32_t C,
                           float* s_out, float* ns_out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* ---- diagnostics --------------------------------------------------------- */

const char* onetrans_status_str(int status);
const char* onetrans_last_error(void);

/* Copies layer `layer`'s cached K and V rows [0, rows) of user `user` (below
 * cache->prefilled) into k_out and v_out (dev bf16 [rows][d] each, heads
 * concatenated along d), for inspection and tests. rows must not exceed the
 * layer's filled length. */
int onetrans_kv_cache_read(const onetrans_config* cfg, const onetrans_kv_cache* cache, int32_t layer,
                           int32_t user, int32_t rows, uint16_t* k_out, uint16_t* v_out,
                           hipStream_t stream);

/* The attention kernel instance a launch of n_queries queries per (segment, head)
 * runs on (ns: 1 for NS queries against a cache, 0 for S queries; n_seg: users in
 * one launch), as a static string such as "attn_kernel<64,4>", or "none" for
 * arguments no launch takes. Pure host logic, for tests that check which
 * instances a workload reaches. */
const char* onetrans_attention_route(int32_t ns, int32_t head_dim, int32_t n_queries, int32_t n_heads,
                                     int32_t n_seg);

/* Kernel timing (diagnostics). While a family's bit is set in `mask`
 * (bit k = 1 << onetrans_kernel_family k), each launch of that family is
 * bracketed by two HIP events recorded on the launch's stream. Enabling resets
 * all totals; onetrans_kernel_timing_read waits for the recorded events of one
 * family and returns the summed device milliseconds and the launch count since
 * the reset. mask = 0 turns timing off. Process-wide, not thread-safe. */
typedef enum {
  ONETRANS_K_S_QKV = 0, ONETRANS_K_S_ATTN = 1, ONETRANS_K_S_FFN_UP = 2, ONETRANS_K_S_FFN_DOWN = 3,
  ONETRANS_K_NS_QKV = 4, ONETRANS_K_NS_ATTN = 5, ONETRANS_K_NS_FFN_UP = 6, ONETRANS_K_NS_FFN_DOWN = 7,
  ONETRANS_K_ELEMENTWISE = 8,
  ONETRANS_K_COUNT = 9
} onetrans_kernel_family;
int onetrans_kernel_timing_enable(uint32_t mask);
int onetrans_kernel_timing_read(int family, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* ONETRANS_H */
