"""Plain fp64 CPU oracle of the OneTrans block-stack forward pass.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, links or runs
this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
do. It shares no code with the HIP path.

What it computes (agihunt.info summary of OneTrans, arXiv 2510.26104, "method"
paragraphs; the asterzephyr.xyz blog, designs two to four, corroborates):

* One token sequence per (user, candidate): S-tokens (behaviour history) first,
  then NS-tokens (user/item/context fields).
* Each block is a pre-norm causal Transformer layer with mixed parameters: every
  S-token uses one shared QKV projection and FFN; NS position k uses its own
  private QKV projection and FFN. RMSNorm is the pre-norm.
* Causal mask: an S-token sees earlier events (and itself); an NS-token sees the
  whole present history plus the NS-tokens before it (and itself).
* Pyramid: layer l keeps only the last q_l S-rows as queries (and as its S
  output); keys and values cover every S-row that is input to the layer.
* Cross-request KV sharing: because S precedes NS, the S-side K/V of every layer
  is computed once per user and reused for every candidate; appended events
  extend it. The user side also covers the profile fields (asterzephyr.xyz,
  design four): when the first P_u NS positions hold user fields, they depend
  on the user only, so they are computed once per user as well, their K/V is
  cached beside the S-side K/V, and the candidate rows (positions P_u..P-1) see
  them like any earlier NS row.

Readings where the pages are silent (each is listed in the design notes):
  no biases, no output projection (heads are concatenated and added to the
  residual), 1/sqrt(head_dim) score scale, head h owns columns
  [h*dh, (h+1)*dh), RMSNorm x / sqrt(mean(x^2) + eps) * g with eps inside the
  root, GELU in its exact erf form, FFN hidden = W1 then GELU then W2, no
  positional term inside the block, outputs are the residual stream after the
  last layer (no final norm), the pyramid keeps the tail, padding slots of a
  right-aligned history are never keys and their rows are zero, an appended
  event is a query at every layer (exact extension of the sequence).

Everything is float64. Inputs are the exact values the GPU consumes (bf16 values,
or E4M3FN codes times their fp32 scale, and fp32 gains).

Parity status of each function: every function here is pinned by the tests in
tests/test_oracle.py (closed forms, a torch special case, brute-force causality,
invariants, the E4M3FN code table, math.erf).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np
from scipy.special import erf as _erf


# ---------------------------------------------------------------------------
# Elementary pieces
# ---------------------------------------------------------------------------

def e4m3fn_to_float(codes) -> np.ndarray:
    """Decode OCP FP8 E4M3FN bit patterns: 1 sign, 4 exponent (bias 7), 3 mantissa bits.

    Exponent field 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; there is
    no infinity (the largest finite magnitude is 1.75 * 2^8 = 448).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, mag)
    return sign * mag


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2 over the last axis) + eps) * g."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU: x * Phi(x) = x/2 * (1 + erf(x / sqrt 2))."""
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def ffn(z: np.ndarray, g: np.ndarray, w1: np.ndarray, w2: np.ndarray, eps: float) -> np.ndarray:
    """Pre-norm FFN sub-layer with its residual: z + W2 GELU(W1 RMSNorm(z))."""
    return z + gelu(rmsnorm(z, g, eps) @ w1.T) @ w2.T


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, visible: np.ndarray, n_heads: int) -> np.ndarray:
    """Multi-head softmax attention under a boolean visibility mask.

    q [..., R, d], k and v [..., J, d] (broadcast over leading axes), visible
    [..., R, J]. Head h uses columns [h*dh, (h+1)*dh); scores are scaled by
    1/sqrt(dh); heads are concatenated. A row with no visible key yields 0.
    """
    d = q.shape[-1]
    dh = d // n_heads
    out = np.zeros(np.broadcast_shapes(q.shape[:-2], k.shape[:-2]) + (q.shape[-2], d))
    any_vis = visible.any(axis=-1, keepdims=True)
    for h in range(n_heads):
        sl = slice(h * dh, (h + 1) * dh)
        s = q[..., sl] @ np.swapaxes(k[..., sl], -1, -2) / math.sqrt(dh)
        s = np.where(visible, s, -np.inf)
        mx = np.where(any_vis, s.max(axis=-1, keepdims=True), 0.0)
        p = np.where(visible, np.exp(s - mx), 0.0)
        den = p.sum(axis=-1, keepdims=True)
        p = p / np.where(den > 0, den, 1.0)
        out[..., sl] = p @ v[..., sl]
    return out


# ---------------------------------------------------------------------------
# Weights
# ---------------------------------------------------------------------------

@dataclass
class Layer:
    """One OneTrans block's parameters in float64, torch Linear layout [out][in]."""
    s_wq: np.ndarray
    s_wk: np.ndarray
    s_wv: np.ndarray
    s_w1: np.ndarray
    s_w2: np.ndarray
    s_ga: np.ndarray
    s_gf: np.ndarray
    ns_wq: np.ndarray   # [P, d, d]
    ns_wk: np.ndarray
    ns_wv: np.ndarray
    ns_w1: np.ndarray   # [P, F, d]
    ns_w2: np.ndarray   # [P, d, F]
    ns_ga: np.ndarray   # [P, d]
    ns_gf: np.ndarray   # [P, d]


def layers_from_arrays(raw: Sequence[dict]) -> List[Layer]:
    """Convert per-layer weight dicts to float64 (E4M3FN codes are decoded and scaled).

    Keys: s_wqkv [3d,d], s_w1, s_w2, s_g_attn, s_g_ffn, ns_wqkv [P,3d,d], ns_w1,
    ns_w2, ns_g_attn [P,d], ns_g_ffn [P,d], ns_scale ([P,5] per (q,k,v,w1,w2)
    matrix when the NS weights are E4M3FN codes, else None).
    """
    out = []
    for r in raw:
        d = r["s_wqkv"].shape[1]
        sq = np.asarray(r["s_wqkv"], np.float64)
        nq, n1, n2 = r["ns_wqkv"], r["ns_w1"], r["ns_w2"]
        if r.get("ns_scale") is not None:
            sc = np.asarray(r["ns_scale"], np.float64)
            nq = e4m3fn_to_float(nq)
            for j in range(3):
                nq[:, j * d:(j + 1) * d] *= sc[:, j, None, None]
            n1 = e4m3fn_to_float(n1) * sc[:, 3, None, None]
            n2 = e4m3fn_to_float(n2) * sc[:, 4, None, None]
        else:
            nq, n1, n2 = (np.asarray(a, np.float64) for a in (nq, n1, n2))
        out.append(Layer(
            s_wq=sq[:d], s_wk=sq[d:2 * d], s_wv=sq[2 * d:],
            s_w1=np.asarray(r["s_w1"], np.float64), s_w2=np.asarray(r["s_w2"], np.float64),
            s_ga=np.asarray(r["s_g_attn"], np.float64), s_gf=np.asarray(r["s_g_ffn"], np.float64),
            ns_wq=nq[:, :d], ns_wk=nq[:, d:2 * d], ns_wv=nq[:, 2 * d:],
            ns_w1=n1, ns_w2=n2,
            ns_ga=np.asarray(r["ns_g_attn"], np.float64), ns_gf=np.asarray(r["ns_g_ffn"], np.float64)))
    return out


# ---------------------------------------------------------------------------
# The literal definition: full recompute of one (user, candidate) sequence
# ---------------------------------------------------------------------------

def forward_dense(layers: Sequence[Layer], q_sched: Sequence[int], n_heads: int, eps: float,
                  s_tokens: np.ndarray, s_valid: int, ns_tokens: np.ndarray):
    """Run the whole block stack over [S ; NS] for one user and one candidate.

    s_tokens [L_S, d] (right-aligned; the first L_S - s_valid slots are padding,
    their contents ignored), ns_tokens [P, d]. Every present row is computed as
    a query (all S rows, not only the tail), then the pyramid keeps the last
    q_l S rows.

    Returns (s_tail [q_{L-1}, d], ns_out [P, d], kv) where kv[l] = (K, V) of the
    S rows present at layer l ([n_l, d] each).
    """
    L_S = s_tokens.shape[0]
    P = ns_tokens.shape[0]
    valid_from = L_S - s_valid
    pos = np.arange(L_S)
    xs = np.array(s_tokens, np.float64)
    xs[pos < valid_from] = 0.0
    xn = np.array(ns_tokens, np.float64)
    kv = []
    for l, W in enumerate(layers):
        n = xs.shape[0]
        X = np.concatenate([xs, xn], axis=0)
        R = n + P
        s_ok = pos >= valid_from                     # S rows that are real events
        # per-row pre-norm and projections (shared for S rows, private per NS position)
        A = np.empty_like(X)
        A[:n] = rmsnorm(X[:n], W.s_ga, eps)
        for k in range(P):
            A[n + k] = rmsnorm(X[n + k], W.ns_ga[k], eps)
        Q = np.empty_like(X); K = np.empty_like(X); V = np.empty_like(X)
        Q[:n], K[:n], V[:n] = A[:n] @ W.s_wq.T, A[:n] @ W.s_wk.T, A[:n] @ W.s_wv.T
        for k in range(P):
            Q[n + k], K[n + k], V[n + k] = W.ns_wq[k] @ A[n + k], W.ns_wk[k] @ A[n + k], W.ns_wv[k] @ A[n + k]
        kv.append((K[:n].copy(), V[:n].copy()))
        # visibility
        vis = np.zeros((R, R), bool)
        for i in range(n):
            if s_ok[i]:
                vis[i, :i + 1] = s_ok[:i + 1]
        for k in range(P):
            vis[n + k, :n] = s_ok
            vis[n + k, n:n + k + 1] = True
        Z = X + attend(Q, K, V, vis, n_heads)
        Y = np.empty_like(Z)
        Y[:n] = ffn(Z[:n], W.s_gf, W.s_w1, W.s_w2, eps)
        for k in range(P):
            Y[n + k] = ffn(Z[n + k], W.ns_gf[k], W.ns_w1[k], W.ns_w2[k], eps)
        Y[:n][~s_ok] = 0.0                            # padding rows stay zero
        q = q_sched[l]
        xs, pos, xn = Y[n - q:n], pos[n - q:], Y[n:]
    return xs, xn, kv


# ---------------------------------------------------------------------------
# The fast form: S side once per user, NS side per candidate
# ---------------------------------------------------------------------------

@dataclass
class UserCache:
    """User-side K/V of one user, per layer.

    Row r of layer l holds global position base[l] + r; rows at global
    positions < valid_from are padding and are never keys. With user-side NS
    fields, ns_tokens holds their inputs [P_u, d], nk / nv their K/V per layer
    [P_u, d] and ns_out their outputs after the last layer.
    """
    base: List[int]
    valid_from: int
    k: List[np.ndarray] = field(default_factory=list)
    v: List[np.ndarray] = field(default_factory=list)
    ns_tokens: Optional[np.ndarray] = None
    nk: List[np.ndarray] = field(default_factory=list)
    nv: List[np.ndarray] = field(default_factory=list)
    ns_out: Optional[np.ndarray] = None

    def length(self, l: int) -> int:
        return self.k[l].shape[0]

    @property
    def n_user_ns(self) -> int:
        return 0 if self.ns_tokens is None else self.ns_tokens.shape[0]


def prefill(layers: Sequence[Layer], q_sched: Sequence[int], n_heads: int, eps: float,
            s_tokens: np.ndarray, s_valid: int,
            ns_user_tokens: Optional[np.ndarray] = None) -> Tuple[UserCache, np.ndarray]:
    """User side of one user: per-layer K/V for every present S row, queries only
    for the tail; then, given ns_user_tokens [P_u, d], the user-side NS rows
    (NS positions 0..P_u-1) and their per-layer K/V.

    Returns (cache, s_tail [q_{L-1}, d]).
    """
    L_S = s_tokens.shape[0]
    valid_from = L_S - s_valid
    pos = np.arange(L_S)
    x = np.array(s_tokens, np.float64)
    x[pos < valid_from] = 0.0
    cache = UserCache(base=[], valid_from=valid_from)
    for l, W in enumerate(layers):
        n = x.shape[0]
        q = q_sched[l]
        a = rmsnorm(x, W.s_ga, eps)
        cache.base.append(int(pos[0]))
        cache.k.append(a @ W.s_wk.T)
        cache.v.append(a @ W.s_wv.T)
        qrows = a[n - q:] @ W.s_wq.T
        qpos = pos[n - q:]
        vis = (pos[None, :] <= qpos[:, None]) & (pos[None, :] >= valid_from) & (qpos[:, None] >= valid_from)
        z = x[n - q:] + attend(qrows, cache.k[l], cache.v[l], vis, n_heads)
        y = ffn(z, W.s_gf, W.s_w1, W.s_w2, eps)
        y[qpos < valid_from] = 0.0
        x, pos = y, qpos
    if ns_user_tokens is not None and ns_user_tokens.shape[0] > 0:
        _user_ns(layers, n_heads, eps, cache, np.array(ns_user_tokens, np.float64))
    return cache, x


def _user_ns(layers: Sequence[Layer], n_heads: int, eps: float, cache: UserCache, tokens: np.ndarray) -> None:
    """(Re)compute the user-side NS rows of a cache from their inputs [P_u, d]:
    they are NS positions 0..P_u-1 of every candidate's sequence, so they see the
    valid cached S rows of each layer and the user NS rows up to themselves."""
    cache.ns_tokens = tokens
    nk, nv = [], []
    out = _ns_rows(layers, n_heads, eps, cache, tokens[None], 0, capture=(nk, nv))
    cache.nk, cache.nv, cache.ns_out = nk, nv, out[0]


def append(layers: Sequence[Layer], n_heads: int, eps: float, cache: UserCache,
           new_tokens: np.ndarray) -> Tuple[UserCache, np.ndarray]:
    """Extend a user's cache by m new events (queries at every layer).

    The new rows take the next global positions after the cached ones. Each new
    row sees every valid cached row of its layer and the new rows up to itself.
    Returns (extended cache, new rows' outputs after the last layer [m, d]).
    """
    x = np.array(new_tokens, np.float64)
    m = x.shape[0]
    out = UserCache(base=list(cache.base), valid_from=cache.valid_from)
    for l, W in enumerate(layers):
        n_old = cache.length(l)
        kpos = cache.base[l] + np.arange(n_old + m)
        qpos = kpos[n_old:]
        a = rmsnorm(x, W.s_ga, eps)
        k = np.concatenate([cache.k[l], a @ W.s_wk.T])
        v = np.concatenate([cache.v[l], a @ W.s_wv.T])
        out.k.append(k)
        out.v.append(v)
        vis = (kpos[None, :] <= qpos[:, None]) & (kpos[None, :] >= cache.valid_from)
        z = x + attend(a @ W.s_wq.T, k, v, vis, n_heads)
        x = ffn(z, W.s_gf, W.s_w1, W.s_w2, eps)
    if cache.n_user_ns:  # the user NS rows see the grown history: recompute them
        _user_ns(layers, n_heads, eps, out, cache.ns_tokens)
    return out, x


def _ns_rows(layers: Sequence[Layer], n_heads: int, eps: float, cache: UserCache, tokens: np.ndarray,
             p0: int, capture=None) -> np.ndarray:
    """NS rows of C independent groups against one user's cache: tokens [C, Pn, d]
    are NS positions p0..p0+Pn-1 (private parameters of those positions). Row j
    of a group sees every valid cached S row of the layer, every cached user NS
    row when p0 > 0 (those are positions 0..p0-1), and its group's rows 0..j.
    With capture = (nk, nv), the rows' K and V of each layer are appended to the
    two lists (C must be 1). Returns the rows after the last layer [C, Pn, d]."""
    C, Pn, d = tokens.shape
    y = np.array(tokens, np.float64)
    causal = np.tril(np.ones((Pn, Pn), bool))
    ks = slice(p0, p0 + Pn)
    for l, W in enumerate(layers):
        n = cache.length(l)
        s_ok = (cache.base[l] + np.arange(n)) >= cache.valid_from
        a = np.stack([rmsnorm(y[:, j], W.ns_ga[p0 + j], eps) for j in range(Pn)], axis=1)
        qn = np.einsum("cpi,poi->cpo", a, W.ns_wq[ks])
        kn = np.einsum("cpi,poi->cpo", a, W.ns_wk[ks])
        vn = np.einsum("cpi,poi->cpo", a, W.ns_wv[ks])
        if capture is not None:
            capture[0].append(kn[0].copy())
            capture[1].append(vn[0].copy())
        k_parts, v_parts, vis_parts = [cache.k[l]], [cache.v[l]], [np.broadcast_to(s_ok, (Pn, n))]
        if p0 > 0:
            k_parts.append(cache.nk[l]); v_parts.append(cache.nv[l]); vis_parts.append(np.ones((Pn, p0), bool))
        keys = np.concatenate([np.broadcast_to(kp, (C,) + kp.shape) for kp in k_parts] + [kn], axis=1)
        vals = np.concatenate([np.broadcast_to(vp, (C,) + vp.shape) for vp in v_parts] + [vn], axis=1)
        vis = np.concatenate(vis_parts + [causal], axis=1)
        z = y + attend(qn, keys, vals, vis, n_heads)
        y = np.stack([ffn(z[:, j], W.ns_gf[p0 + j], W.ns_w1[p0 + j], W.ns_w2[p0 + j], eps) for j in range(Pn)], axis=1)
    return y


def score(layers: Sequence[Layer], n_heads: int, eps: float, cache: UserCache,
          ns_tokens: np.ndarray, chunk: int = 64) -> np.ndarray:
    """NS side of C candidates against one user's cache: ns_tokens [C, Pc, d] -> [C, Pc, d].

    The candidate rows are NS positions P_u..P_u+Pc-1 (P_u = the cache's user NS
    rows, 0 without them). Row k of a candidate sees every valid cached S row of
    the layer, every user NS row, and that candidate's rows up to itself.
    Candidates are independent; they are processed ``chunk`` at a time only to
    bound memory.
    """
    C, P, d = ns_tokens.shape
    out = np.empty((C, P, d))
    for c0 in range(0, C, chunk):
        out[c0:c0 + chunk] = _ns_rows(layers, n_heads, eps, cache, ns_tokens[c0:c0 + chunk], cache.n_user_ns)
    return out


def block_forward(layers: Sequence[Layer], q_sched: Sequence[int], n_heads: int, eps: float,
                  s_tokens: np.ndarray, s_lens: np.ndarray, ns_tokens: np.ndarray,
                  ns_user_tokens: Optional[np.ndarray] = None):
    """Full pass for B users: s_tokens [B, L_S, d], s_lens [B], ns_tokens [B, C, Pc, d]
    (candidate rows) and optionally ns_user_tokens [B, P_u, d] (user NS rows).

    Returns (s_tail [B, q_{L-1}, d], ns_out [B, C, Pc, d]).
    """
    tails, outs = [], []
    for u in range(s_tokens.shape[0]):
        cache, tail = prefill(layers, q_sched, n_heads, eps, s_tokens[u], int(s_lens[u]),
                              None if ns_user_tokens is None else ns_user_tokens[u])
        tails.append(tail)
        outs.append(score(layers, n_heads, eps, cache, ns_tokens[u]))
    return np.stack(tails), np.stack(outs)
