"""CPU study: how far the NS side moves from the fp64 oracle when the operands of its
linear maps are rounded to a narrower format.

Collected as a slow CPU test (``-m slow``, about 15 s at C = 4); it also runs as a
script from the repository root: ``python tests/test_precision_study.py [C] [--fp8-weights]``.

The oracle's NS side calls ``rmsnorm`` and ``gelu`` for exactly the two values that
feed the linear maps of a row: the normalised input of Q/K/V and FFN up, and the
GELU output that feeds FFN down. The study wraps those two functions so that their
results are rounded (round to nearest even, saturating) before use, scores C
candidates of the OneTrans-L shape against one prefilled user, and reports max-abs
and relative-L2 distances to the unrounded oracle over the final NS rows:

- fp16: the operand format the GPU path uses for its linear maps;
- bf16: 16-bit with the fp32 exponent range;
- e4m3 per row: OCP E4M3FN with one fp32 scale per row (amax / 448), the
  usual activation quantisation of a W8A8 scheme;
- e4m3 unscaled: E4M3FN of the raw values (all of them lie far inside its range).

The S side is left at fp64, so every number is the cost of the NS operand format
alone. Test infrastructure: it calls the oracle and nothing of the GPU path.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle as O  # noqa: E402
import oracle.onetrans_oracle as OO  # noqa: E402
from onetrans_inputs import CANDIDATE_HEAVY_FP8, ONETRANS_L, make_ns_tokens, make_s_tokens, make_weights  # noqa: E402


def round_grid(x: np.ndarray, mant_bits: int, min_exp: int, max_val: float) -> np.ndarray:
    """Round to the nearest value of a binary float format with `mant_bits` stored mantissa
    bits, smallest normal exponent `min_exp` (subnormals below it) and largest finite value
    `max_val` (saturating); ties to even."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    step = np.exp2(np.maximum(e, min_exp) - mant_bits)
    return np.sign(x) * np.minimum(np.round(ax / step) * step, max_val)


FORMATS = {
    "fp16": lambda x: round_grid(x, 10, -14, 65504.0),
    "bf16": lambda x: round_grid(x, 7, -126, 3.3895313892515355e38),
    "e4m3 per row": lambda x: _scaled_e4m3(x),
    "e4m3 unscaled": lambda x: round_grid(x, 3, -6, 448.0),
}


def _scaled_e4m3(x: np.ndarray) -> np.ndarray:
    amax = np.max(np.abs(x), axis=-1, keepdims=True)
    s = np.where(amax > 0, amax / 448.0, 1.0)
    return round_grid(x / s, 3, -6, 448.0) * s


def study(C: int, fp8_weights: bool = False) -> dict:
    """{format: (max-abs, rel-L2)} of the final NS rows of C OneTrans-L candidates."""
    wl = CANDIDATE_HEAVY_FP8 if fp8_weights else ONETRANS_L
    lay = O.layers_from_arrays(make_weights(wl))
    s, lens = make_s_tokens(wl)
    ns = make_ns_tokens(wl, n_candidates=C)[0]
    cache, _ = O.prefill(lay, wl.q_sched, wl.n_heads, wl.rms_eps, s[0], int(lens[0]))
    ref = O.score(lay, wl.n_heads, wl.rms_eps, cache, ns)
    print(f"{wl.name}, C = {C}, final NS rows rms {np.sqrt(np.mean(ref ** 2)):.2f}, max |.| {np.abs(ref).max():.1f}")
    rms, gel = OO.rmsnorm, OO.gelu
    out = {}
    for name, rnd in FORMATS.items():
        OO.rmsnorm = lambda x, g, eps, rnd=rnd: rnd(rms(x, g, eps))
        OO.gelu = lambda x, rnd=rnd: rnd(gel(x))
        try:
            got = O.score(lay, wl.n_heads, wl.rms_eps, cache, ns)
        finally:
            OO.rmsnorm, OO.gelu = rms, gel
        d = got - ref
        out[name] = (float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(ref)))
        print(f"  {name:14s} max-abs {out[name][0]:.3e}  rel-L2 {out[name][1]:.3e}")
    return out


@pytest.mark.slow
def test_operand_formats_against_the_parity_bars():
    # the operand formats of the NS linear maps, against the bars the GPU path must meet
    # (3e-2 / 1e-2 for bf16 weights, 5e-2 / 2e-2 for E4M3 weights): fp16 (what the path
    # uses) sits well inside them; bf16 operands already exceed the max-abs bar; E4M3
    # activations (a W8A8 scheme) miss both bars by an order of magnitude, whatever
    # the scale granularity
    r = study(4)
    assert r["fp16"][0] < 1.5e-2 and r["fp16"][1] < 2e-3
    assert r["bf16"][0] > 3e-2
    assert r["e4m3 per row"][0] > 0.5 and r["e4m3 per row"][1] > 2e-2
    assert r["e4m3 unscaled"][0] > 0.5 and r["e4m3 unscaled"][1] > 2e-2


def main() -> None:
    args = [a for a in sys.argv[1:] if not a.startswith("--")]
    study(int(args[0]) if args else 8, "--fp8-weights" in sys.argv)


if __name__ == "__main__":
    main()


def test_rounding_grows_with_depth():
    """Why deeper models get a wider max-abs bar: the oracle with the GPU plan's roundings
    (fp16 operands of the linear maps, bf16 Q / K / V) moves a 64-wide model's final rows by
    less than the stated 3e-2 at 8 layers but by more at 16, and by less than 3e-2 * 16 / 8."""
    from onetrans_inputs import Workload
    wl = Workload(name="depth", n_layers=16, d_model=64, n_heads=1, ffn_hidden=64, s_len=40,
                  q_sched=tuple(range(40, 8, -2)), n_ns=2, n_users=2, n_candidates=3)
    lens = np.array([40, 7], np.int32)
    f16, b16 = FORMATS["fp16"], FORMATS["bf16"]
    rms, gelu, att = OO.rmsnorm, OO.gelu, OO.attend

    def final_rows(L, emulate):
        w = wl.with_(n_layers=L, q_sched=wl.q_sched[:L])
        s, _ = make_s_tokens(w)
        for u in range(s.shape[0]):
            s[u, : w.s_len - lens[u]] = 0.0
        try:
            if emulate:
                OO.rmsnorm = lambda x, g, eps: f16(rms(x, g, eps))
                OO.gelu = lambda x: f16(gelu(x))
                OO.attend = lambda q, k, v, vis, h: att(b16(q), b16(k), b16(v), vis, h)
            t, n = O.block_forward(O.layers_from_arrays(make_weights(w)), w.q_sched, w.n_heads, 1e-6, s, lens,
                                   make_ns_tokens(w))
        finally:
            OO.rmsnorm, OO.gelu, OO.attend = rms, gelu, att
        return np.concatenate([t.ravel(), n.ravel()])

    dev = {L: float(np.abs(final_rows(L, True) - final_rows(L, False)).max()) for L in (8, 16)}
    print("max-abs moved by the emulated roundings:", dev)
    assert dev[8] < 3e-2 < dev[16] < 3e-2 * 16 / 8

