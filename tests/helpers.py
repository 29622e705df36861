"""Shared helpers of the GPU tests: seeded inputs -> device tensors, oracle runs, error metrics."""
from __future__ import annotations

import functools

import numpy as np

import oracle as O
from onetrans_inputs import Workload, make_weights

EPS = 1e-6
# max-abs / relative-L2 bars on fp32 outputs (bf16 weights; E4M3 NS weights)
TOL = {"bf16": (3e-2, 1e-2), "e4m3": (5e-2, 2e-2)}


@functools.lru_cache(maxsize=4)
def weights(wl: Workload, seed: int = 0, private_gains: bool = False):
    raw = make_weights(wl, seed=seed, ns_private_gains=private_gains)
    return raw, O.layers_from_arrays(raw)


def config(wl: Workload, append_cap: int = 0, n_ns_user: int = 0):
    from unified_transformer_recommender_onetrans_amd import make_config
    return make_config(wl.n_layers, wl.d_model, wl.n_heads, wl.ffn_hidden, wl.n_ns, wl.s_len, wl.q_sched,
                       append_cap=append_cap, rms_eps=wl.rms_eps, ns_wdtype=wl.ns_wdtype, n_ns_user=n_ns_user)


def bf16_dev(a: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device).to(torch.bfloat16)


def device_weights(raw, device="cuda"):
    import torch
    out = []
    for lw in raw:
        d = {}
        for k, v in lw.items():
            if v is None:
                d[k] = None
            elif v.dtype == np.uint8:
                d[k] = torch.from_numpy(np.ascontiguousarray(v)).to(device)
            elif k.startswith(("s_g", "ns_g", "ns_scale")):
                d[k] = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(device)
            else:
                d[k] = bf16_dev(v, device)
        out.append(d)
    return out


def model(wl: Workload, seed: int = 0, append_cap: int = 0, private_gains: bool = False, device="cuda",
          n_ns_user: int = 0):
    from unified_transformer_recommender_onetrans_amd import OneTrans
    raw, lay = weights(wl, seed, private_gains)
    return OneTrans(config(wl, append_cap, n_ns_user), device_weights(raw, device), device=device), lay


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / den) if den > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_close(got, ref, wdtype: str = "bf16", what: str = "", n_layers: int = 8):
    """The stated bars hold for models of up to 8 layers (every workload's depth). The
    precision plan's rounding accumulates over the sublayers, so a deeper model gets the
    max-abs bar times n_layers / 8, the relative-L2 bar unchanged (the growth with depth is
    pinned on the CPU in test_precision_study.py)."""
    ma, rl = errors(got, ref)
    bar_ma, bar_rl = TOL[wdtype]
    bar_ma *= max(1.0, n_layers / 8)
    print(f"    {what}: max-abs {ma:.3e} (bar {bar_ma}) rel-L2 {rl:.3e} (bar {bar_rl})", flush=True)
    assert ma <= bar_ma and rl <= bar_rl, f"{what}: max-abs {ma:.3e} rel-L2 {rl:.3e}"
