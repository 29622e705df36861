"""Workload shapes for the OneTrans block forward.

Shapes only: no arithmetic of the method lives here. Sources (the pages):

* agihunt.info summary of OneTrans (arXiv 2510.26104), "model sizes" paragraph:
  OneTransS has 6 layers, width 256, 4 heads and sequential queries 1190 -> 12;
  OneTransL has 8 layers, width 384 and sequential queries 1500 -> 16.
* Same page, "limitations" paragraph: pyramid lengths are a heuristic rounded to
  multiples of 32.

The NS-token count (32), FFN ratio (4d), head count of the L shape (6, head
dim 64), batch sizes and candidate counts are not on the pages; they are the
fixed workload definitions this repository measures.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


def pyramid_schedule(s_len: int, q_last: int, n_layers: int, multiple: int = 32) -> Tuple[int, ...]:
    """Per-layer S-query counts q_0..q_{L-1}.

    Endpoints are exact (q_0 = s_len, q_{L-1} = q_last). Interior layers take the
    linear interpolation between them rounded half-up to the nearest multiple of
    ``multiple`` (the pages say the lengths are rounded to multiples of 32 but do
    not print the interior values).
    """
    if n_layers == 1:
        return (s_len,)
    out = []
    for l in range(n_layers):
        if l == 0:
            out.append(s_len)
        elif l == n_layers - 1:
            out.append(q_last)
        else:
            t = s_len + (q_last - s_len) * l / (n_layers - 1)
            out.append(int((t / multiple) + 0.5) * multiple)
    return tuple(out)


@dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    ffn_hidden: int
    s_len: int
    q_sched: Tuple[int, ...]
    n_ns: int
    n_users: int
    n_candidates: int
    ns_wdtype: str = "bf16"          # "bf16" or "e4m3"
    len_range: Optional[Tuple[int, int]] = None   # inclusive; None = every user full length
    append_m: int = 0
    rms_eps: float = 1e-6

    @property
    def head_dim(self) -> int:
        return self.d_model // self.n_heads

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY = Workload(
    name="tiny", n_layers=1, d_model=64, n_heads=2, ffn_hidden=256, s_len=64,
    q_sched=(64,), n_ns=8, n_users=1, n_candidates=4)

ONETRANS_S = Workload(
    name="onetrans_s", n_layers=6, d_model=256, n_heads=4, ffn_hidden=1024, s_len=1190,
    q_sched=pyramid_schedule(1190, 12, 6), n_ns=32, n_users=1, n_candidates=128)

ONETRANS_L = Workload(
    name="onetrans_l", n_layers=8, d_model=384, n_heads=6, ffn_hidden=1536, s_len=1500,
    q_sched=pyramid_schedule(1500, 16, 8), n_ns=32, n_users=1, n_candidates=256)

PREFILL_BATCH = ONETRANS_L.with_(
    name="prefill_batch", n_users=64, n_candidates=0, len_range=(1000, 1500), append_m=64)

CANDIDATE_HEAVY_FP8 = ONETRANS_L.with_(
    name="candidate_heavy_fp8", n_candidates=4096, ns_wdtype="e4m3")

ALL = {w.name: w for w in (TINY, ONETRANS_S, ONETRANS_L, PREFILL_BATCH, CANDIDATE_HEAVY_FP8)}
