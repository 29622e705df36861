"""CPU study: how far the NS side moves from the fp64 oracle when the operands of its
linear maps are rounded to a narrower format.

Run from the repository root: ``python tests/precision_study.py [C] [--fp8-weights]``.
(Not a pytest module; it takes about a minute at C = 8.)

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


def main() -> None:
    args = [a for a in sys.argv[1:] if not a.startswith("--")]
    C = int(args[0]) if args else 8
    wl = CANDIDATE_HEAVY_FP8 if "--fp8-weights" in sys.argv else ONETRANS_L
    lay = O.layers_from_arrays(make_weights(wl))
    s, lens = make_s_tokens(wl)
    ns = make_ns_tokens(wl, n_candidates=C)[0]
    cache, _ = O.prefill(lay, wl.q_sched, wl.n_heads, wl.rms_eps, s[0], int(lens[0]))
    ref = O.score(lay, wl.n_heads, wl.rms_eps, cache, ns)
    print(f"{wl.name}, C = {C}, final NS rows rms {np.sqrt(np.mean(ref ** 2)):.2f}, max |.| {np.abs(ref).max():.1f}")
    rms, gel = OO.rmsnorm, OO.gelu
    for name, rnd in FORMATS.items():
        OO.rmsnorm = lambda x, g, eps, rnd=rnd: rnd(rms(x, g, eps))
        OO.gelu = lambda x, rnd=rnd: rnd(gel(x))
        try:
            got = O.score(lay, wl.n_heads, wl.rms_eps, cache, ns)
        finally:
            OO.rmsnorm, OO.gelu = rms, gel
        d = got - ref
        print(f"  {name:14s} max-abs {np.abs(d).max():.3e}  rel-L2 {np.linalg.norm(d) / np.linalg.norm(ref):.3e}")


if __name__ == "__main__":
    main()
