"""The benchmark's algorithmic FLOP model against brute-force enumeration of the
rows and visible (query, key) pairs, including padding and the pyramid."""
import numpy as np
import pytest

import bench
from onetrans_inputs import ONETRANS_L, Workload


def brute_prefill(wl, lens):
    d, F = wl.d_model, wl.ffn_hidden
    tot = 0
    for ln in lens:
        vf = wl.s_len - ln
        present = list(range(wl.s_len))
        for q in wl.q_sched:
            keys = [p for p in present if p >= vf]
            queries = [p for p in present[len(present) - q:] if p >= vf]
            pairs = sum(1 for qp in queries for kp in keys if kp <= qp)
            tot += 2 * d * d * 2 * len(keys) + 2 * d * d * len(queries) + 4 * d * pairs + 4 * d * F * len(queries)
            present = present[len(present) - q:]
    return tot


def brute_score(wl, ln, m_appended=0):
    d, F, P = wl.d_model, wl.ffn_hidden, wl.n_ns
    vf = wl.s_len - ln
    present = list(range(wl.s_len))
    tot = 0
    for q in wl.q_sched:
        nk = sum(1 for p in present if p >= vf) + m_appended
        pairs = sum(nk + k + 1 for k in range(P))
        tot += 2 * d * 3 * d * P + 4 * d * pairs + 4 * d * F * P
        present = present[len(present) - q:]
    return tot


def brute_append(wl, ln, m):
    d, F = wl.d_model, wl.ffn_hidden
    vf = wl.s_len - ln
    present = list(range(wl.s_len))
    tot = 0
    for q in wl.q_sched:
        nk = sum(1 for p in present if p >= vf)
        pairs = sum(nk + t + 1 for t in range(m))
        tot += 2 * d * 3 * d * m + 4 * d * pairs + 4 * d * F * m
        present = present[len(present) - q:]
    return tot


WL = Workload(name="m", n_layers=3, d_model=64, n_heads=2, ffn_hidden=128, s_len=50, q_sched=(40, 21, 3),
              n_ns=5, n_users=3, n_candidates=2)


@pytest.mark.parametrize("lens", [[50], [50, 7, 1, 30], [0, 3]])
def test_prefill_flops(lens):
    assert bench.prefill_flops(WL, lens) == brute_prefill(WL, lens)


@pytest.mark.parametrize("ln", [50, 22, 2, 0])
def test_score_and_append_flops(ln):
    assert bench.score_flops_per_candidate(WL, bench.cache_valid_rows(WL, ln)) == brute_score(WL, ln)
    assert bench.append_flops(WL, [ln], 6) == brute_append(WL, ln, 6)


def brute_score_user_ns(wl, ln, Pu):
    # a candidate's rows Pu..P-1: valid S keys + all Pu user rows + own rows up to itself
    d, F, P = wl.d_model, wl.ffn_hidden, wl.n_ns
    vf = wl.s_len - ln
    present = list(range(wl.s_len))
    tot = 0
    for q in wl.q_sched:
        nk = sum(1 for p in present if p >= vf)
        rows = list(range(Pu, P))
        pairs = sum(nk + Pu + (k - Pu) + 1 for k in rows)
        tot += 2 * d * 3 * d * len(rows) + 4 * d * pairs + 4 * d * F * len(rows)
        present = present[len(present) - q:]
    return tot


@pytest.mark.parametrize("ln,Pu", [(1500, 8), (1200, 1), (1500, 0)])
def test_user_ns_score_flops(ln, Pu):
    nk = bench.cache_valid_rows(ONETRANS_L, ln)
    assert bench.score_flops_user_ns(ONETRANS_L, nk, Pu) == pytest.approx(brute_score_user_ns(ONETRANS_L, ln, Pu), rel=1e-12)
    if Pu == 0:
        assert bench.score_flops_user_ns(ONETRANS_L, nk, 0) == pytest.approx(bench.score_flops_per_candidate(ONETRANS_L, nk))


def test_kernel_work_sums_to_step_flops():
    wl = ONETRANS_L
    nk = bench.cache_valid_rows(wl, 1500)
    w = bench.kernel_work(wl, 256, nk, lens=[1500])
    total = sum(f for f, _ in w.values())
    want = bench.prefill_flops(wl, [1500]) + 256 * bench.score_flops_per_candidate(wl, nk)
    assert abs(total - want) / want < 1e-12
    # 27.0 GFLOP per full-length prefill and 1.208 GFLOP per candidate, counted by hand from
    # the OneTrans-L shape (2 per MAC over the needed rows, 4 d per visible pair)
    assert abs(bench.prefill_flops(wl, [1500]) / 1e9 - 27.0) < 0.01
    assert abs(bench.score_flops_per_candidate(wl, nk) / 1e9 - 1.208) < 1e-3


def test_gpus_above_one_exits_with_message():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True,
                       cwd=bench.ROOT, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stdout
