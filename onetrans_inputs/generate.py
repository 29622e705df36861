"""Seeded synthetic inputs for the OneTrans block forward.

This module draws numbers and rounds them to the storage formats both sides
consume (bf16, OCP E4M3FN with a per-matrix fp32 scale). It holds none of the
method's arithmetic: no norm, projection, attention or FFN is computed here.
Both the fp64 oracle (via the tests) and the HIP path (via the binding) take
the arrays it returns.

Distributions follow the workload definitions: token embeddings N(0, 1),
weights N(0, 1/d) with d the model width (also for W2, whose fan-in is the FFN
hidden size), RMSNorm gains 1 + N(0, 0.1) where the second argument is a
variance. Seeds: ``SeedSequence(seed).spawn(5)`` gives independent streams for
[weights+gains, S tokens, NS tokens, lengths, appended tokens], so changing the
candidate or user count never changes the weights.

Draw order inside the weight stream, layer by layer:
  S:  Wq[d,d], Wk[d,d], Wv[d,d], W1[F,d], W2[d,F], g_attn[d], g_ffn[d]
  NS: Wq[n_ns,d,d], Wk, Wv, W1[n_ns,F,d], W2[n_ns,d,F]
      (+ g_attn[n_ns,d], g_ffn[n_ns,d] when ``ns_private_gains``)
Without private NS gains, every NS position uses the layer's S gains (one gain
per sublayer per layer).

Matrices use the torch Linear layout [out][in]: y = W @ x.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

from .workloads import Workload

E4M3_MAX = 448.0


def bf16_round(x) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even); returned as float32."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32)
    # finite inputs only: the largest finite pattern plus the bias stays below 2^32
    u = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return u.view(np.float32).reshape(f.shape)


def e4m3_quantize(w: np.ndarray):
    """Per-matrix scale s = amax / 448 and E4M3FN codes of w / s (RNE, saturating).

    The cast itself is torch's float8_e4m3fn conversion; the codes are returned
    as uint8 bit patterns.
    """
    import torch

    amax = float(np.max(np.abs(w)))
    scale = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
    x = np.clip((w / np.float64(scale)).astype(np.float32), -E4M3_MAX, E4M3_MAX)
    codes = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def _streams(seed: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(5)]


def make_weights(wl: Workload, seed: int = 0, ns_private_gains: bool = False) -> List[Dict[str, np.ndarray]]:
    """Per-layer weight dicts (float32 arrays holding bf16 values, or uint8 E4M3 codes)."""
    gen = _streams(seed)[0]
    d, F, P = wl.d_model, wl.ffn_hidden, wl.n_ns
    sd = np.float32(np.sqrt(1.0 / d))
    gsd = np.float32(np.sqrt(0.1))

    def normal(shape):  # fp32 draws; weights are rounded to bf16 / E4M3 afterwards
        return gen.standard_normal(shape, dtype=np.float32)

    layers = []
    for _ in range(wl.n_layers):
        s_wq = normal((d, d)) * sd
        s_wk = normal((d, d)) * sd
        s_wv = normal((d, d)) * sd
        s_w1 = normal((F, d)) * sd
        s_w2 = normal((d, F)) * sd
        g_a = (1.0 + normal(d) * gsd).astype(np.float32)
        g_f = (1.0 + normal(d) * gsd).astype(np.float32)
        ns_wq = normal((P, d, d)) * sd
        ns_wk = normal((P, d, d)) * sd
        ns_wv = normal((P, d, d)) * sd
        ns_w1 = normal((P, F, d)) * sd
        ns_w2 = normal((P, d, F)) * sd
        if ns_private_gains:
            ns_ga = (1.0 + normal((P, d)) * gsd).astype(np.float32)
            ns_gf = (1.0 + normal((P, d)) * gsd).astype(np.float32)
        else:
            ns_ga = np.broadcast_to(g_a, (P, d)).copy()
            ns_gf = np.broadcast_to(g_f, (P, d)).copy()
        lw = {
            "s_wqkv": bf16_round(np.concatenate([s_wq, s_wk, s_wv], axis=0)),
            "s_w1": bf16_round(s_w1),
            "s_w2": bf16_round(s_w2),
            "s_g_attn": g_a,
            "s_g_ffn": g_f,
            "ns_g_attn": ns_ga,
            "ns_g_ffn": ns_gf,
        }
        if wl.ns_wdtype == "bf16":
            lw["ns_wqkv"] = bf16_round(np.concatenate([ns_wq, ns_wk, ns_wv], axis=1))
            lw["ns_w1"] = bf16_round(ns_w1)
            lw["ns_w2"] = bf16_round(ns_w2)
            lw["ns_scale"] = None
        elif wl.ns_wdtype == "e4m3":
            qkv = np.empty((P, 3 * d, d), np.uint8)
            w1 = np.empty((P, F, d), np.uint8)
            w2 = np.empty((P, d, F), np.uint8)
            scale = np.empty((P, 5), np.float32)
            for k in range(P):
                for j, w in enumerate((ns_wq[k], ns_wk[k], ns_wv[k])):
                    qkv[k, j * d:(j + 1) * d], scale[k, j] = e4m3_quantize(w)
                w1[k], scale[k, 3] = e4m3_quantize(ns_w1[k])
                w2[k], scale[k, 4] = e4m3_quantize(ns_w2[k])
            lw["ns_wqkv"], lw["ns_w1"], lw["ns_w2"], lw["ns_scale"] = qkv, w1, w2, scale
        else:
            raise ValueError(f"unknown ns_wdtype {wl.ns_wdtype!r}")
        layers.append(lw)
    return layers


def make_s_tokens(wl: Workload, seed: int = 0, n_users: Optional[int] = None):
    """S-token embeddings [B, s_len, d] (bf16 values) and valid lengths [B] (int32).

    Histories are right-aligned: user u's valid tokens sit in slots
    [s_len - len_u, s_len); the padding slots before them hold zeros.
    """
    B = wl.n_users if n_users is None else n_users
    st = _streams(seed)
    x = bf16_round(st[1].standard_normal((B, wl.s_len, wl.d_model)))
    if wl.len_range is None:
        lens = np.full(B, wl.s_len, np.int32)
    else:
        lo, hi = wl.len_range
        lens = st[3].integers(lo, hi + 1, size=B).astype(np.int32)
    for u in range(B):
        x[u, : wl.s_len - lens[u]] = 0.0
    return x, lens


def make_ns_tokens(wl: Workload, seed: int = 0, n_users: Optional[int] = None,
                   n_candidates: Optional[int] = None) -> np.ndarray:
    """NS-token embeddings [B, C, n_ns, d] (bf16 values)."""
    B = wl.n_users if n_users is None else n_users
    C = wl.n_candidates if n_candidates is None else n_candidates
    rng = _streams(seed)[2]
    return bf16_round(rng.standard_normal((B, C, wl.n_ns, wl.d_model)))


def make_append_tokens(wl: Workload, seed: int = 0, n_users: Optional[int] = None,
                       m: Optional[int] = None) -> np.ndarray:
    """Newly arrived S-token embeddings [B, m, d] (bf16 values)."""
    B = wl.n_users if n_users is None else n_users
    m = wl.append_m if m is None else m
    rng = _streams(seed)[4]
    return bf16_round(rng.standard_normal((B, m, wl.d_model)))
