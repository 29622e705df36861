"""Benchmark of the OneTrans block forward on one MI355X.

One step = onetrans_block_forward on the OneTransL-shape workload: the S side of
one user (1500 events, pyramid 1500 -> 16 over 8 layers) is prefilled into the
K/V cache, then C = 256 candidates (32 NS tokens each) are scored against it.
`value` is candidates scored per second over the timed steps; TFLOP/s counts
the algorithmic work of the step (prefill + scoring). The same JSON line also
carries:
  roofline      the dominant kernel family, timed live with HIP events on the
                stream it runs on, against MI355X peaks. A timing event costs
                about 6 us of pipeline drain per record, so the events run in a
                second pass of the same number of identical steps right after
                the timed steps, which carry no per-launch events
  step_ms_p10_p50_p90  the spread of single steps, from events around each step of
                a further pass (every record drains the pipeline)
  scoring_only  candidate scoring against an already-filled cache (the serving
                steady state the cross-request K/V sharing targets), with a roofline
                entry for the same dominant kernel family timed there: the kernel on
                its own, without the CUs that the block forward's concurrent S side
                holds inside its event intervals
  user_ns       the same user with its first 8 NS positions as user-side fields:
                they run once in the prefill and are cached; each candidate then
                runs its 24 item / context rows against S keys + user NS keys
  multi_stage   three scoring stages with their own NS weights and token counts
                against the same cache (retrieval 4096 x 8 NS tokens, pre-rank
                1024 x 16, fine-rank 256 x 32), the shared-user-context path of
                the successor system
  prefill_batch 64 users, lengths U{1000..1500}, prefill throughput; also the time
                of the same prefill with 8 user-side NS fields per user
  append        64 new events for each of those 64 users, appended to the cache
  onetrans_s, candidate_heavy_fp8
                the OneTrans-S block forward (C = 128) and the candidate-heavy one
                (OneTrans-L shape, C = 4096, E4M3 NS weights), each with its own
                roofline entry for its dominant kernel family and its own oracle
                baseline (every 8th candidate for C = 4096)
  check         the last timed step's outputs are finite and equal, bit for bit,
                to scoring the same candidates against a separately prefilled cache
  cpu_baseline  the fp64 oracle on the host cores on a bounded sample (also inside
                prefill_batch / append: every 8th user, prefills/s and appends/s)
Inputs are seeded synthetic data with the workloads' shapes and distributions.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from onetrans_inputs import (CANDIDATE_HEAVY_FP8, ONETRANS_L, ONETRANS_S, PREFILL_BATCH,  # noqa: E402
                             make_append_tokens, make_ns_tokens, make_s_tokens, make_weights)

METRIC = "candidates scored/s + TFLOP/s (% bf16 MFMA peak), OneTransL-shape block fwd"
PEAK_TFLOPS_16BIT = 2500.0     # MI355X dense fp16 / bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
RIDGE = PEAK_TFLOPS_16BIT * 1e12 / (PEAK_HBM_GBS * 1e9)


# ---------------------------------------------------------------------------
# Algorithmic work model: 2 flops per MAC of the projections / FFN over the rows
# actually needed (valid events; queries only for Q and the FFN), 4*d flops per
# visible (query, key) pair; padding, masked and pruned work excluded. Bytes:
# each operand a kernel must read or write, once.
# ---------------------------------------------------------------------------

def layer_rows(wl):
    n, prev = [], wl.s_len
    for q in wl.q_sched:
        n.append(prev)
        prev = q
    return n, list(wl.q_sched)


def _valid(lo: int, hi: int, vf: int) -> int:
    return max(0, hi - max(lo, vf))


def prefill_flops(wl, lens) -> float:
    d, F = wl.d_model, wl.ffn_hidden
    n, q = layer_rows(wl)
    tot = 0.0
    for ln in lens:
        vf = wl.s_len - int(ln)
        for l in range(wl.n_layers):
            base, qbase = wl.s_len - n[l], wl.s_len - q[l]
            nv, qv = _valid(base, wl.s_len, vf), _valid(qbase, wl.s_len, vf)
            kstart = max(base, vf)
            first_q = wl.s_len - qv
            lead = first_q - kstart          # keys before the first valid query
            pairs = qv * (lead + 1) + qv * (qv - 1) / 2
            tot += 2 * d * d * (2 * nv + qv) + 4 * d * pairs + 4 * d * F * qv
    return tot


def cache_valid_rows(wl, ln: int, n_appended: int = 0):
    n, _ = layer_rows(wl)
    vf = wl.s_len - int(ln)
    return [_valid(wl.s_len - n[l], wl.s_len, vf) + n_appended for l in range(wl.n_layers)]


def append_flops(wl, lens, m: int) -> float:
    d, F = wl.d_model, wl.ffn_hidden
    tot = 0.0
    for ln in lens:
        for nk in cache_valid_rows(wl, ln):
            tot += 2 * d * 3 * d * m + 4 * d * (m * nk + m * (m + 1) / 2) + 4 * d * F * m
    return tot


def score_flops_per_candidate(wl, nk) -> float:
    d, F, P = wl.d_model, wl.ffn_hidden, wl.n_ns
    return sum(2 * d * 3 * d * P + 4 * d * (P * k + P * (P + 1) / 2) + 4 * d * F * P for k in nk)


def score_flops_user_ns(wl, nk, Pu: int) -> float:
    """Per candidate with Pu user-side NS rows cached: its Pc = P - Pu rows see the nk
    cached S rows, the Pu user rows and its own rows up to themselves."""
    d, F, Pc = wl.d_model, wl.ffn_hidden, wl.n_ns - Pu
    return sum(2 * d * 3 * d * Pc + 4 * d * (Pc * (k + Pu) + Pc * (Pc + 1) / 2) + 4 * d * F * Pc for k in nk)


def kernel_work(wl, C: int, nk, lens=None, m: int = 0):
    """Per-family algorithmic (flops, bytes) summed over one call's launches.

    NS families: one scoring call of C candidates with valid cached rows nk[l].
    S families: one prefill (lens given, m = 0) or one append of m events.
    """
    d, F, P, L = wl.d_model, wl.ffn_hidden, wl.n_ns, wl.n_layers
    wb = 1 if wl.ns_wdtype == "e4m3" else 2
    R = C * P
    w = {}
    if C:
        w["ns_qkv"] = (L * 2 * R * d * 3 * d, L * (P * 3 * d * d * wb + R * d * 4 + R * 3 * d * 2 + P * d * 4))
        w["ns_attn"] = (sum(4 * d * C * (P * k + P * (P + 1) / 2) for k in nk),
                        sum(2 * k * d * 2 + R * 3 * d * 2 + R * d * 8 for k in nk))
        w["ns_ffn_up"] = (L * 2 * R * d * F, L * (P * F * d * wb + R * d * 4 + R * F * 2 + P * d * 4))
        w["ns_ffn_down"] = (L * 2 * R * F * d, L * (P * d * F * wb + R * F * 2 + R * d * 8))
    if lens is not None:
        n, q = layer_rows(wl)
        fl = {"s_qkv": 0.0, "s_attn": 0.0, "s_ffn_up": 0.0, "s_ffn_down": 0.0}
        by = dict(fl)
        for ln in lens:
            vf = wl.s_len - int(ln)
            for l in range(L):
                if m == 0:
                    base, qbase = wl.s_len - n[l], wl.s_len - q[l]
                    nv, qv = _valid(base, wl.s_len, vf), _valid(qbase, wl.s_len, vf)
                    lead = (wl.s_len - qv) - max(base, vf)
                    pairs = qv * (lead + 1) + qv * (qv - 1) / 2
                    kv_read = nv
                else:
                    nv = qv = m
                    nk_l = cache_valid_rows(wl, ln)[l]
                    pairs = m * nk_l + m * (m + 1) / 2
                    kv_read = nk_l + m
                fl["s_qkv"] += 2 * d * d * (2 * nv + qv)
                by["s_qkv"] += nv * d * 4 + (2 * nv + qv) * d * 2
                fl["s_attn"] += 4 * d * pairs
                by["s_attn"] += kv_read * d * 2 * 2 + qv * d * 2 + qv * d * 8
                fl["s_ffn_up"] += 2 * d * F * qv
                by["s_ffn_up"] += qv * d * 4 + qv * F * 2
                fl["s_ffn_down"] += 2 * d * F * qv
                by["s_ffn_down"] += qv * F * 2 + qv * d * 8
        for l in range(L):  # shared S weights, once per launch
            by["s_qkv"] += 3 * d * d * 2
            by["s_ffn_up"] += F * d * 2
            by["s_ffn_down"] += d * F * 2
        for k in fl:
            w[k] = (fl[k], by[k])
    return w


# ---------------------------------------------------------------------------

def device_weights(raw, dev):
    import torch
    out = []
    for lw in raw:
        dd = {}
        for k, v in lw.items():
            if v is None:
                dd[k] = None
            elif v.dtype == np.uint8 or k.startswith(("s_g", "ns_g", "ns_scale")):
                dd[k] = torch.from_numpy(np.ascontiguousarray(v)).to(dev)
            else:
                dd[k] = torch.from_numpy(np.ascontiguousarray(v)).to(dev).to(torch.bfloat16)
        out.append(dd)
    return out


def bf16(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)


def timed(fn, steps, warmup, sync):
    for _ in range(warmup):
        fn()
    sync()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    sync()
    return time.perf_counter() - t0


# Source files whose text decides each kernel family's memory traffic.
FAMILY_SOURCES = {
    "s_qkv": "gemm.hip", "s_ffn_up": "gemm.hip", "s_ffn_down": "gemm.hip", "ns_qkv": "gemm.hip",
    "ns_ffn_up": "gemm.hip", "ns_ffn_down": "gemm.hip", "s_attn": "attention.hip", "ns_attn": "attention.hip",
    "elementwise": "elementwise.hip",
}
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "unified_transformer_recommender_onetrans_amd", "csrc")


def source_digest(family: str) -> str:
    """sha256 over the family's kernel source and the shared device header."""
    import hashlib
    h = hashlib.sha256()
    for f in (FAMILY_SOURCES[family], "internal.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(family: str, workload: str):
    """HBM bytes per launch from the committed counter summary (rocprofv3 FETCH_SIZE and WRITE_SIZE,
    scaled by a copy kernel's calibration), or None when there is none or the kernel source changed
    since it was taken."""
    path = os.path.join(PROFILES, f"traffic_{workload}_{family}.md")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                kv[k.strip()] = v.strip().strip("`")
    if kv.get("source_sha256") != source_digest(family):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def roofline_entry(family, flops, nbytes, ms, launches, traffic=None):
    """The dominant kernel family against the MI355X peaks. The path's step is bound by the
    matrix cores at its arithmetic intensity (the algorithmic flop / byte ratio of the whole
    step lies above the ridge), so the entry is priced against the dense 16-bit MFMA peak;
    the family's own algorithmic bytes give its HBM fraction beside it."""
    sec = ms / 1e3
    ach = flops / sec / 1e12
    gbs = nbytes / sec / 1e9
    return {"kernel": family, "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_TFLOPS_16BIT,
            "unit": "TFLOP/s", "frac": round(ach / PEAK_TFLOPS_16BIT, 4), "traffic": traffic,
            "launches": launches, "avg_launch_us": round(ms / launches * 1e3, 2),
            "algorithmic_flops_per_launch": flops / launches, "algorithmic_bytes_per_launch": nbytes / launches,
            "algorithmic_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "flop_per_byte": round(flops / nbytes, 1) if nbytes else None}


def copy_calibration(mib: int, reps: int) -> None:
    """A plain device-to-device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib * 1024 * 1024
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "reps": reps}))


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the affinity size
        return len(os.sched_getaffinity(0))


def cpu_baseline(wl, raw, s, lens, ns, budget_s: float, stride: int = 1):
    """The fp64 oracle (as it stands) on the host: one user's prefill, then candidates
    0, stride, 2*stride, ... scored in chunks of 16 until about `budget_s` seconds of CPU
    work have been spent (or the sample is done). The rate scales the scoring time to C."""
    import oracle as O
    lay = O.layers_from_arrays(raw)
    C = ns.shape[1]
    sample = np.arange(0, C, stride)
    t0 = time.perf_counter()
    cache, _ = O.prefill(lay, wl.q_sched, wl.n_heads, wl.rms_eps, s[0], int(lens[0]))
    t1 = time.perf_counter()
    done = 0
    while done < len(sample) and (done == 0 or time.perf_counter() - t1 < budget_s):
        idx = sample[done:done + 16]
        O.score(lay, wl.n_heads, wl.rms_eps, cache, ns[0][idx])
        done += len(idx)
    t2 = time.perf_counter()
    step = (t1 - t0) + (t2 - t1) * C / done
    which = "candidates" if stride == 1 else f"every {stride}th candidate"
    return {"value": round(C / step, 2), "unit": "candidates/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"one user's prefill ({t1 - t0:.1f} s) + {done} candidates ({which}) of {C} scored "
                      f"({t2 - t1:.1f} s); the step time scales the scoring time linearly to C={C}",
            "seconds": round(t2 - t0, 2)}


def cpu_baseline_prefill_append(wl, raw, s, lens, new, budget_s: float, stride: int = 8):
    """The oracle's prefill and append of users 0, stride, 2*stride, ... of the batch
    until about `budget_s` seconds have been spent; rates in prefills/s and appends/s."""
    import oracle as O
    lay = O.layers_from_arrays(raw)
    users = list(range(0, s.shape[0], stride))
    t_pre = t_app = 0.0
    done = 0
    t0 = time.perf_counter()
    for u in users:
        a = time.perf_counter()
        cache, _ = O.prefill(lay, wl.q_sched, wl.n_heads, wl.rms_eps, s[u], int(lens[u]))
        b = time.perf_counter()
        O.append(lay, wl.n_heads, wl.rms_eps, cache, new[u])
        c = time.perf_counter()
        t_pre += b - a
        t_app += c - b
        done += 1
        if c - t0 > budget_s:
            break
    smp = f"users {users[0]}, {users[1] if done > 1 else ''}... every {stride}th, {done} of {s.shape[0]}"
    return ({"value": round(done / t_pre, 3), "unit": "prefills/s", "cores": _blas_threads(), "kind": "oracle",
             "sample": f"{smp}: prefill {t_pre:.1f} s"},
            {"value": round(done / t_app, 3), "unit": "appends/s", "cores": _blas_threads(), "kind": "oracle",
             "sample": f"{smp}: append of {new.shape[1]} events {t_app:.1f} s"})


def prefill_append_parts(raw, dev, steps, sync, log, cpu_budget=None):
    """The prefill batch (64 users, lengths U{1000..1500}) and the append of 64 new events
    per user, then the same prefill with 8 user-side NS fields per user; returns the
    "prefill_batch" and "append" entries of the JSON line."""
    import torch
    from unified_transformer_recommender_onetrans_amd import OneTrans, make_config
    res = {}
    pw = PREFILL_BATCH
    log("[bench] prefill batch / append")
    ps, plens = make_s_tokens(pw)
    pnew = make_append_tokens(pw)
    cfg2 = make_config(pw.n_layers, pw.d_model, pw.n_heads, pw.ffn_hidden, pw.n_ns, pw.s_len, pw.q_sched,
                       append_cap=pw.append_m, rms_eps=pw.rms_eps)
    m2 = OneTrans(cfg2, device_weights(raw, dev), device=dev)
    ps_d, pl_d, pn_d = bf16(ps, dev), torch.from_numpy(plens).to(dev), bf16(pnew, dev)
    pcache = m2.new_cache(pw.n_users)
    psteps = max(3, steps // 4)
    el_p = timed(lambda: m2.user_prefill(ps_d, pl_d, pcache), psteps, 1, sync)
    pfl = prefill_flops(pw, plens)
    pt = pfl / (el_p / psteps) / 1e12

    def app():
        pcache.c.n_appended = 0  # rewrite the same rows each time: identical work per call
        m2.kv_append(pn_d, pcache)
    el_a = timed(app, psteps, 1, sync)
    afl = append_flops(pw, plens, pw.append_m)
    aw = kernel_work(pw, 0, None, lens=plens, m=pw.append_m)
    abytes = sum(b for _, b in aw.values())
    t_a = el_a / psteps
    res["prefill_batch"] = {"users": pw.n_users, "prefills_per_s": round(pw.n_users / (el_p / psteps), 1),
                            "ms_per_call": round(el_p / psteps * 1e3, 3), "tflops": round(pt, 2),
                            "pct_bf16_mfma_peak": round(100 * pt / PEAK_TFLOPS_16BIT, 2)}
    res["append"] = {"users": pw.n_users, "events_per_user": pw.append_m,
                     "appends_per_s": round(pw.n_users / t_a, 1),
                     "events_per_s": round(pw.n_users * pw.append_m / t_a, 1),
                     "ms_per_call": round(t_a * 1e3, 4), "tflops": round(afl / t_a / 1e12, 2),
                     "algorithmic_gbs": round(abytes / t_a / 1e9, 1),
                     "pct_hbm_peak": round(100 * abytes / t_a / 1e9 / PEAK_HBM_GBS, 2)}
    del m2, pcache
    # the same 64 users with 8 user-side NS fields each: their pass runs once for the batch
    cfg4 = make_config(pw.n_layers, pw.d_model, pw.n_heads, pw.ffn_hidden, pw.n_ns, pw.s_len, pw.q_sched,
                       rms_eps=pw.rms_eps, n_ns_user=8)
    m4 = OneTrans(cfg4, device_weights(raw, dev), device=dev)
    pu_d = bf16(np.ascontiguousarray(make_ns_tokens(pw, n_users=pw.n_users, n_candidates=1)[:, 0, :8]), dev)
    c4 = m4.new_cache(pw.n_users)
    el_pu = timed(lambda: m4.user_prefill(ps_d, pl_d, c4, ns_user_tokens=pu_d), psteps, 1, sync)
    res["prefill_batch"]["ms_per_call_with_8_user_ns_fields"] = round(el_pu / psteps * 1e3, 3)
    del m4, c4
    if cpu_budget:
        log("[bench] oracle CPU baseline: prefill batch / append")
        res["prefill_batch"]["cpu_baseline"], res["append"]["cpu_baseline"] = cpu_baseline_prefill_append(
            pw, raw, ps, plens, pnew, cpu_budget)
    return res


def block_forward_part(wl, raw, dev, steps, warmup, sync, log, check=False):
    """Timed block_forward steps of one workload (1 user prefill + C candidates scored):
    throughput, the single-step spread and the roofline entry of the dominant kernel
    family. Returns (entry, model, device inputs, step callable)."""
    import torch
    from unified_transformer_recommender_onetrans_amd import OneTrans, make_config
    from unified_transformer_recommender_onetrans_amd._capi import (KERNEL_FAMILIES, kernel_timing_enable,
                                                                     kernel_timing_read)
    C = wl.n_candidates
    s, lens = make_s_tokens(wl)
    ns = make_ns_tokens(wl)
    cfg = make_config(wl.n_layers, wl.d_model, wl.n_heads, wl.ffn_hidden, wl.n_ns, wl.s_len, wl.q_sched,
                      rms_eps=wl.rms_eps, ns_wdtype=wl.ns_wdtype)
    model = OneTrans(cfg, device_weights(raw, dev), device=dev)
    s_d, l_d, ns_d = bf16(s, dev), torch.from_numpy(lens).to(dev), bf16(ns, dev)
    step = lambda: model.block_forward(s_d, l_d, ns_d)
    nk = cache_valid_rows(wl, int(lens[0]))
    step_flops = prefill_flops(wl, lens) + C * score_flops_per_candidate(wl, nk)
    work = kernel_work(wl, C, nk, lens=lens)

    # warmup: one cold step untimed, then the rest with every family timed to find the dominant one
    step()
    sync()
    kernel_timing_enable(KERNEL_FAMILIES)
    nw = max(1, warmup)
    for _ in range(nw):
        step()
    sync()
    per_family = {f: kernel_timing_read(f) for f in KERNEL_FAMILIES}
    events_us = {f: round(ms / nw * 1e3, 1) for f, (ms, n) in per_family.items() if n}
    dominant = max((f for f in per_family if f in work), key=lambda f: per_family[f][0])

    # timed steps (no per-launch events: each one drains the pipeline), then the same
    # number of identical steps with the dominant family event-timed on its stream
    log(f"[bench] {wl.name}: timing {steps} steps (dominant kernel family: {dominant})")
    kernel_timing_enable([])
    sync()
    t0 = time.perf_counter()
    for _ in range(steps):
        s_out, ns_out = step()
    sync()
    el = time.perf_counter() - t0
    kernel_timing_enable([dominant])
    for _ in range(steps):
        step()
    sync()
    ms_dom, n_dom = kernel_timing_read(dominant)
    kernel_timing_enable([])
    # the spread of single steps: the same number of steps again, each between two events
    # on the caller's stream (a record drains the pipeline, so these are not the timed steps)
    cur = torch.cuda.current_stream(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        e0.record(cur)
        step()
        e1.record(cur)
    sync()
    per_step = np.sort([e0.elapsed_time(e1) for e0, e1 in evs])
    pct = lambda q: round(float(np.percentile(per_step, q)), 4)
    fl, by = work[dominant]
    roof = roofline_entry(dominant, fl * steps, by * steps, ms_dom, n_dom, measured_traffic(dominant, wl.name))
    tflops = step_flops / (el / steps) / 1e12
    entry = {
        "candidates_per_s": round(C * steps / el, 1), "ms_per_step": round(el / steps * 1e3, 4),
        "tflops": round(tflops, 2), "pct_bf16_mfma_peak": round(100 * tflops / PEAK_TFLOPS_16BIT, 2),
        "step_gflop": round(step_flops / 1e9, 2), "steps": steps,
        "workload": (f"{wl.name} block_forward: 1 user x {wl.s_len} S events (pyramid {wl.q_sched[0]}->"
                     f"{wl.q_sched[-1]}, {wl.n_layers} layers, d={wl.d_model}, {wl.n_heads} heads), C={C} "
                     f"candidates x {wl.n_ns} NS tokens" + (", E4M3 NS weights" if wl.ns_wdtype == "e4m3" else "")),
        "roofline": roof,
        # HIP events around every launch of each family during the warm-up steps: each record
        # drains its stream (about 6 us) and the two streams overlap, so these per-family sums
        # do not add up to the step time
        "kernel_event_us_per_step_nonadditive": events_us,
        "step_ms_p10_p50_p90": [pct(10), pct(50), pct(90)],
    }
    if check:
        # the last timed step's outputs: finite, and equal bit for bit to scoring the same
        # candidates against a separately prefilled cache
        cache = model.new_cache(1)
        tail = model.user_prefill(s_d, l_d, cache)
        ref = model.score_candidates(cache, 0, ns_d[0])
        sync()
        entry["check"] = {"finite": bool(torch.isfinite(ns_out).all().item() and torch.isfinite(s_out).all().item()),
                          "block_forward_equals_scoring": bool(torch.equal(ns_out[0], ref) and torch.equal(s_out, tail))}
        del cache
    return entry, model, (s, lens, ns, s_d, l_d, ns_d), nk


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sub", action="store_true",
                    help="only the headline workload (no scoring-only, user-side, multi-stage, prefill batch, "
                         "append, OneTrans-S or candidate-heavy parts)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU work budget of each oracle baseline")
    ap.add_argument("--workload", default="onetrans_l", choices=["onetrans_l", "onetrans_s", "candidate_heavy_fp8"])
    ap.add_argument("--prefill-append-only", action="store_true",
                    help="only the prefill-batch / append measurements (one JSON line of their own)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a device copy of this many MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.copy_calibration_mib > 0:
        copy_calibration(args.copy_calibration_mib, 5)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 (the multi-GPU design is "
                                   "documented, not built)", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import __graft_entry__
    from unified_transformer_recommender_onetrans_amd import LIB_PATH, OneTrans, make_config
    from unified_transformer_recommender_onetrans_amd._capi import kernel_timing_enable, kernel_timing_read
    if not os.path.exists(LIB_PATH):
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    sync = lambda: torch.cuda.synchronize(dev)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    cpu_budget = None if args.no_cpu_baseline else args.cpu_seconds
    if args.prefill_append_only:
        print(json.dumps(prefill_append_parts(make_weights(PREFILL_BATCH), dev, args.steps, sync, log, cpu_budget)),
              flush=True)
        return

    wl = {"onetrans_l": ONETRANS_L, "onetrans_s": ONETRANS_S, "candidate_heavy_fp8": CANDIDATE_HEAVY_FP8}[
        args.workload]
    C = wl.n_candidates
    log(f"[bench] generating {wl.name} inputs")
    raw = make_weights(wl)
    head, model, (s, lens, ns, s_d, l_d, ns_d), nk = block_forward_part(wl, raw, dev, args.steps, args.warmup,
                                                                         sync, log, check=True)
    out = {
        "metric": METRIC, "value": head["candidates_per_s"], "unit": "candidates/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp16/bf16",
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": head["workload"], "global_batch": C, "seq_len": wl.s_len + wl.n_ns},
        "tflops": head["tflops"], "pct_bf16_mfma_peak": head["pct_bf16_mfma_peak"],
        "step_gflop": head["step_gflop"],
        "roofline": head["roofline"],
        "kernel_event_us_per_step_nonadditive": head["kernel_event_us_per_step_nonadditive"],
        "step_ms_p10_p50_p90": head["step_ms_p10_p50_p90"],
        "check": head["check"],
    }

    if not args.no_sub:
        # scoring only, cache filled once (untimed)
        cache = model.new_cache(1)
        model.user_prefill(s_d, l_d, cache)
        sc_out = torch.empty(C, wl.n_ns, wl.d_model, dtype=torch.float32, device=dev)
        sc = lambda: model.score_candidates(cache, 0, ns_d[0], out=sc_out)
        el_s = timed(sc, args.steps, args.warmup, sync)
        sflops = C * score_flops_per_candidate(wl, nk)
        out["scoring_only"] = {"candidates_per_s": round(C * args.steps / el_s, 1),
                               "ms_per_call": round(el_s / args.steps * 1e3, 4),
                               "tflops": round(sflops / (el_s / args.steps) / 1e12, 2),
                               "pct_bf16_mfma_peak": round(100 * sflops / (el_s / args.steps) / 1e12 /
                                                           PEAK_TFLOPS_16BIT, 2)}
        # the headline's dominant kernel family timed on its own: the same launches during
        # scoring calls against the resident cache, where no concurrent S-side kernel holds
        # CUs (in the block forward its event interval also holds those waits)
        dom = head["roofline"]["kernel"]
        sc_work = kernel_work(wl, C, nk)
        if dom in sc_work:
            kernel_timing_enable([dom])
            for _ in range(args.steps):
                sc()
            sync()
            ms_d, n_d = kernel_timing_read(dom)
            kernel_timing_enable([])
            fl_d, by_d = sc_work[dom]
            out["scoring_only"]["roofline"] = roofline_entry(dom, fl_d * args.steps, by_d * args.steps, ms_d, n_d,
                                                             measured_traffic(dom, wl.name))
        del cache
        # user-side NS fields: the first 8 NS positions belong to the user (one candidate's
        # rows stand in for the user's fields), prefilled once; candidates bring 24 rows
        Pu = 8
        cfg3 = make_config(wl.n_layers, wl.d_model, wl.n_heads, wl.ffn_hidden, wl.n_ns, wl.s_len, wl.q_sched,
                           rms_eps=wl.rms_eps, ns_wdtype=wl.ns_wdtype, n_ns_user=Pu)
        m3 = OneTrans(cfg3, device_weights(raw, dev), device=dev)
        un_d = ns_d[0, 0, :Pu].unsqueeze(0).contiguous()
        cn_d = ns_d[0, :, Pu:].contiguous()
        cache3 = m3.new_cache(1)
        usteps = max(3, args.steps // 4)
        el_up = timed(lambda: m3.user_prefill(s_d, l_d, cache3, ns_user_tokens=un_d), usteps, 1, sync)
        out3 = torch.empty(C, wl.n_ns - Pu, wl.d_model, dtype=torch.float32, device=dev)
        el_us = timed(lambda: m3.score_candidates(cache3, 0, cn_d, out=out3), args.steps, args.warmup, sync)
        ufl = C * score_flops_user_ns(wl, nk, Pu)
        out["user_ns"] = {"n_ns_user": Pu, "candidate_rows": wl.n_ns - Pu,
                          "candidates_per_s": round(C * args.steps / el_us, 1),
                          "ms_per_call": round(el_us / args.steps * 1e3, 4),
                          "tflops": round(ufl / (el_us / args.steps) / 1e12, 2),
                          "pct_bf16_mfma_peak": round(100 * ufl / (el_us / args.steps) / 1e12 / PEAK_TFLOPS_16BIT, 2),
                          "prefill_ms_with_user_ns": round(el_up / usteps * 1e3, 4)}
        del m3, cache3
        # multi-stage scoring on one cache: each stage packs its own NS weights (seeded per
        # stage) next to the shared S weights and scores against the cache prefilled above
        log("[bench] multi-stage scoring")
        cache = model.new_cache(1)
        model.user_prefill(s_d, l_d, cache)
        stages = []
        for sname, n_ns_st, c_st, seed in (("retrieval", 8, 4096, 11), ("pre_rank", 16, 1024, 12), ("fine_rank", 32, 256, 0)):
            wl_st = wl.with_(n_ns=n_ns_st, n_candidates=c_st)
            raw_st = [dict(lw) for lw in make_weights(wl_st, seed=seed)]
            for lw, la in zip(raw_st, raw):
                for k in ("s_wqkv", "s_w1", "s_w2", "s_g_attn", "s_g_ffn"):
                    lw[k] = la[k]
            cfg_st = make_config(wl.n_layers, wl.d_model, wl.n_heads, wl.ffn_hidden, n_ns_st, wl.s_len, wl.q_sched,
                                 rms_eps=wl.rms_eps, ns_wdtype=wl.ns_wdtype)
            m_st = OneTrans(cfg_st, device_weights(raw_st, dev), device=dev)
            t_st = bf16(make_ns_tokens(wl_st, seed=seed)[0], dev)
            o_st = torch.empty(c_st, n_ns_st, wl.d_model, dtype=torch.float32, device=dev)
            stages.append((sname, m_st, t_st, o_st, c_st, n_ns_st, score_flops_per_candidate(wl_st, nk)))
        msteps = max(3, args.steps // 2)
        run_all = lambda: [st[1].score_candidates(cache, 0, st[2], out=st[3]) for st in stages]
        el_ms = timed(run_all, msteps, 2, sync)
        per = {}
        for sname, m_st, t_st, o_st, c_st, n_ns_st, fl_st in stages:
            t1 = timed(lambda: m_st.score_candidates(cache, 0, t_st, out=o_st), msteps, 2, sync) / msteps
            per[sname] = {"candidates": c_st, "ns_tokens": n_ns_st, "ms": round(t1 * 1e3, 4),
                          "candidates_per_s": round(c_st / t1, 1), "tflops": round(fl_st * c_st / t1 / 1e12, 2)}
        out["multi_stage"] = {"ms_all_stages": round(el_ms / msteps * 1e3, 4), "stages": per}
        del stages, cache, model
        out.update(prefill_append_parts(raw, dev, args.steps, sync, log, cpu_budget))
        # the other block-forward workloads: OneTrans-S (C = 128) and the candidate-heavy
        # E4M3 case (C = 4096), each with its own roofline entry
        for other in (ONETRANS_S, CANDIDATE_HEAVY_FP8):
            if other.name == wl.name:
                continue
            log(f"[bench] generating {other.name} inputs")
            raw_o = make_weights(other)
            ent, m_o, (so, lo, nso, *_), _ = block_forward_part(other, raw_o, dev, args.steps, args.warmup, sync,
                                                                log, check=True)
            del m_o
            torch.cuda.empty_cache()
            if cpu_budget:
                log(f"[bench] oracle CPU baseline: {other.name}")
                big = other.n_candidates >= 1024  # every 8th candidate, with twice the budget
                ent["cpu_baseline"] = cpu_baseline(other, raw_o, so, lo, nso, cpu_budget * (2 if big else 1),
                                                   stride=8 if big else 1)
            out[other.name] = ent

    if cpu_budget:
        log("[bench] oracle CPU baseline")
        out["cpu_baseline"] = cpu_baseline(wl, raw, s, lens, ns, cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
