"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small cases compare every output element; the full-size workloads run in the
benchmark's launch configuration and compare sampled users / candidates that
the oracle computes one by one. Bars: max-abs 3e-2 and relative L2 1e-2 on
the fp32 outputs (5e-2 / 2e-2 with E4M3 NS weights).
"""
import numpy as np
import pytest

import oracle as O
from onetrans_inputs import (CANDIDATE_HEAVY_FP8, ONETRANS_L, ONETRANS_S, PREFILL_BATCH, TINY, Workload,
                             bf16_round, make_append_tokens, make_ns_tokens, make_s_tokens, make_weights)
from helpers import EPS, assert_close, bf16_dev, config, device_weights, model, weights

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# small cases: ragged tiles, general NS counts, padding (including an empty
# history), head_dim 32 and 64, pyramid drops to a single-digit tail
SMALL = {
    "a_dh32_P5": (Workload(name="a", n_layers=2, d_model=64, n_heads=2, ffn_hidden=128, s_len=300,
                           q_sched=(250, 97), n_ns=5, n_users=3, n_candidates=7), [300, 41, 0]),
    "b_dh64_P32": (Workload(name="b", n_layers=3, d_model=128, n_heads=2, ffn_hidden=256, s_len=200,
                            q_sched=(200, 130, 3), n_ns=32, n_users=2, n_candidates=5), [200, 1]),
    "c_fp8": (Workload(name="c", n_layers=3, d_model=128, n_heads=2, ffn_hidden=256, s_len=200,
                       q_sched=(200, 130, 3), n_ns=32, n_users=2, n_candidates=5, ns_wdtype="e4m3"), [150, 200]),
    "d_single": (Workload(name="d", n_layers=1, d_model=64, n_heads=1, ffn_hidden=64, s_len=1, q_sched=(1,),
                          n_ns=1, n_users=1, n_candidates=1), [1]),
    "e_P40": (Workload(name="e", n_layers=2, d_model=192, n_heads=3, ffn_hidden=192, s_len=70,
                       q_sched=(64, 33), n_ns=40, n_users=1, n_candidates=3), [70]),
    "tiny": (TINY, [64]),
    # key ranges of 10 tiles with every query block full: the NS attention's steady-state
    # iterations (one and two query blocks per workgroup, dh 32 and 64; 260-1024 query
    # blocks, above the key-split instances' range) against the oracle
    "f_dh32_long": (Workload(name="f", n_layers=2, d_model=64, n_heads=2, ffn_hidden=128, s_len=600,
                             q_sched=(600, 300), n_ns=16, n_users=1, n_candidates=264), [600]),
    "g_dh32_nb2": (Workload(name="g", n_layers=2, d_model=128, n_heads=4, ffn_hidden=256, s_len=520,
                            q_sched=(520, 260), n_ns=32, n_users=1, n_candidates=256), [470]),
    "h_dh64_long": (Workload(name="h", n_layers=2, d_model=128, n_heads=2, ffn_hidden=256, s_len=640,
                             q_sched=(640, 320), n_ns=8, n_users=2, n_candidates=520), [640, 590]),
    # wide models: 16 heads, and more than 16 norm-partial slots per row at d = 1024 (the GEMM
    # epilogue loads those beyond the first 16 after its k-loop); F not a multiple of 128
    "n_d1024_dh64": (Workload(name="n", n_layers=2, d_model=1024, n_heads=16, ffn_hidden=1088, s_len=96,
                              q_sched=(96, 40), n_ns=3, n_users=2, n_candidates=4), [96, 50]),
    "o_d512_dh32": (Workload(name="o", n_layers=3, d_model=512, n_heads=16, ffn_hidden=640, s_len=130,
                             q_sched=(130, 70, 9), n_ns=6, n_users=1, n_candidates=9), [117]),
    # the largest layer count (16) and the largest NS token count (256: 256 private weight
    # groups per GEMM, own-key ranges of 8 key blocks per candidate)
    "p_16layers": (Workload(name="p", n_layers=16, d_model=64, n_heads=1, ffn_hidden=64, s_len=40,
                            q_sched=tuple(range(40, 8, -2)), n_ns=2, n_users=2, n_candidates=3), [40, 7]),
    "q_P256": (Workload(name="q", n_layers=2, d_model=64, n_heads=2, ffn_hidden=64, s_len=50,
                        q_sched=(50, 20), n_ns=256, n_users=1, n_candidates=20), [43]),
    # a history of 10000 events (the pages speak of behaviour sequences beyond 10000 steps)
    # in 10240 slots: 160 key tiles per query block in the first layer
    "r_long10k": (Workload(name="r", n_layers=2, d_model=64, n_heads=2, ffn_hidden=128, s_len=10240,
                           q_sched=(10240, 100), n_ns=4, n_users=1, n_candidates=6), [10000]),
}


# many users' prefill in one launch: the S attention's tile instances with four and two
# query blocks per workgroup (dh 32: 2048 and 1024 query blocks; dh 64: 1536), ragged
# right-aligned histories from a single event to the full length
MANY_USERS = {
    "i_dh32_16users": Workload(name="i", n_layers=2, d_model=64, n_heads=2, ffn_hidden=128, s_len=2048,
                               q_sched=(2048, 1024), n_ns=4, n_users=16, n_candidates=3),
    "j_dh64_12users": Workload(name="j", n_layers=2, d_model=128, n_heads=2, ffn_hidden=256, s_len=2048,
                               q_sched=(2048, 1000), n_ns=4, n_users=12, n_candidates=3),
    # d = 192, F = 768: the S QKV and FFN up GEMMs of 24k and 12k rows take 256x192 tiles,
    # one per workgroup, many per group
    "m_d192_12users": Workload(name="m", n_layers=2, d_model=192, n_heads=3, ffn_hidden=768, s_len=2048,
                               q_sched=(2048, 1000), n_ns=4, n_users=12, n_candidates=3),
}


def _many_lens(wl):
    base = [wl.s_len, 1, 1500, wl.s_len - 1, 33, 1024, 2000, 64, 65, 1999, 700, 1, 1200, 1800, 5, 2048]
    return [min(x, wl.s_len) for x in base[:wl.n_users]]


def _inputs(wl, lens):
    s, _ = make_s_tokens(wl)
    lens = np.asarray(lens, np.int32)
    for u in range(s.shape[0]):
        s[u, : wl.s_len - lens[u]] = 0.0
    return s, lens, make_ns_tokens(wl)


def _dev(s, lens, ns):
    return bf16_dev(s), torch.from_numpy(lens).cuda(), bf16_dev(ns)


@pytest.mark.parametrize("name", list(SMALL))
def test_block_forward_matches_oracle(name):
    wl, lens = SMALL[name]
    print(f"case {name}", flush=True)
    m, lay = model(wl, private_gains=(name == "c_fp8"))
    s, lens, ns = _inputs(wl, lens)
    s_out, ns_out = m.block_forward(*_dev(s, lens, ns))
    torch.cuda.synchronize()
    ref_t, ref_n = O.block_forward(lay, wl.q_sched, wl.n_heads, EPS, s, lens, ns)
    assert_close(s_out.cpu().numpy(), ref_t, wl.ns_wdtype, "S tail", wl.n_layers)
    assert_close(ns_out.cpu().numpy(), ref_n, wl.ns_wdtype, "NS out", wl.n_layers)
    # padding rows of the S tail are exactly zero
    qL = wl.q_sched[-1]
    for u, ln in enumerate(lens):
        npad = min(qL, max(0, qL - int(ln)))
        assert np.all(s_out[u, :npad].cpu().numpy() == 0.0)


@pytest.mark.parametrize("name", ["a_dh32_P5", "b_dh64_P32", "c_fp8", "tiny", "n_d1024_dh64"])
def test_prefill_append_score_match_oracle(name):
    wl, lens = SMALL[name]
    print(f"case {name}", flush=True)
    m1, m2 = 13, 6
    mdl, lay = model(wl, append_cap=m1 + m2 + 1, private_gains=(name == "c_fp8"))
    s, lens, ns = _inputs(wl, lens)
    sd, ld, nd = _dev(s, lens, ns)
    B = s.shape[0]
    cache = mdl.new_cache(B)
    s_out = mdl.user_prefill(sd, ld, cache)
    new1 = make_append_tokens(wl, m=m1)
    new2 = make_append_tokens(wl, seed=1, m=m2)
    out1 = mdl.kv_append(bf16_dev(new1), cache)
    out2 = mdl.kv_append(bf16_dev(new2), cache)
    assert cache.n_appended == m1 + m2
    scores = [mdl.score_candidates(cache, u, nd[u]) for u in range(B)]
    torch.cuda.synchronize()
    for u in range(B):
        oc, ot = O.prefill(lay, wl.q_sched, wl.n_heads, EPS, s[u], int(lens[u]))
        assert_close(s_out[u].cpu().numpy(), ot, wl.ns_wdtype, f"user {u} S tail")
        oc, o1 = O.append(lay, wl.n_heads, EPS, oc, new1[u])
        oc, o2 = O.append(lay, wl.n_heads, EPS, oc, new2[u])
        assert_close(out1[u].cpu().numpy(), o1, wl.ns_wdtype, f"user {u} append 1")
        assert_close(out2[u].cpu().numpy(), o2, wl.ns_wdtype, f"user {u} append 2")
        assert_close(scores[u].cpu().numpy(), O.score(lay, wl.n_heads, EPS, oc, ns[u]), wl.ns_wdtype,
                     f"user {u} score after appends")
        for l in (0, wl.n_layers - 1):
            rows = oc.length(l)
            k, v = cache.read_layer(l, u, rows)
            ok = (oc.base[l] + np.arange(rows)) >= oc.valid_from
            assert_close(k.float().cpu().numpy()[ok], oc.k[l][ok], "bf16", f"user {u} layer {l} cached K")
            assert_close(v.float().cpu().numpy()[ok], oc.v[l][ok], "bf16", f"user {u} layer {l} cached V")


@pytest.mark.parametrize("name", list(MANY_USERS))
def test_many_user_prefill_tile_kernels(name):
    wl = MANY_USERS[name]
    print(f"case {name}: B={wl.n_users}", flush=True)
    m = 7
    mdl, lay = model(wl, append_cap=m)
    s, lens, ns = _inputs(wl, _many_lens(wl))
    sd, ld, nd = _dev(s, lens, ns)
    B = s.shape[0]
    cache = mdl.new_cache(B)
    s_out = mdl.user_prefill(sd, ld, cache)
    new = make_append_tokens(wl, m=m)
    app = mdl.kv_append(bf16_dev(new), cache)
    scored = {u: mdl.score_candidates(cache, u, nd[u]) for u in (0, 1, B - 1)}
    torch.cuda.synchronize()
    s_out, app = s_out.cpu().numpy(), app.cpu().numpy()
    for u in range(B):
        oc, ot = O.prefill(lay, wl.q_sched, wl.n_heads, EPS, s[u], int(lens[u]))
        assert_close(s_out[u], ot, wl.ns_wdtype, f"user {u} (len {lens[u]}) S tail")
        oc, oa = O.append(lay, wl.n_heads, EPS, oc, new[u])
        assert_close(app[u], oa, wl.ns_wdtype, f"user {u} appended rows")
        if u in scored:
            assert_close(scored[u].cpu().numpy(), O.score(lay, wl.n_heads, EPS, oc, ns[u]), wl.ns_wdtype,
                         f"user {u} scores after the append")


def test_one_tile_per_workgroup_gemms():
    """160 candidates x 48 NS positions at d = 192, F = 768: the NS QKV (N = 576) and FFN up
    (N = 768) GEMMs take one 256x192 tile per workgroup (the smaller tiles would need three
    rounds of the chip), with 96 padding rows in every tile; every output is compared."""
    wl = Workload(name="t256", n_layers=2, d_model=192, n_heads=3, ffn_hidden=768, s_len=200,
                  q_sched=(200, 64), n_ns=48, n_users=1, n_candidates=160)
    m, lay = model(wl)
    s, lens, ns = _inputs(wl, [170])
    s_out, ns_out = m.block_forward(*_dev(s, lens, ns))
    torch.cuda.synchronize()
    ref_t, ref_n = O.block_forward(lay, wl.q_sched, wl.n_heads, EPS, s, lens, ns)
    assert_close(s_out.cpu().numpy(), ref_t, wl.ns_wdtype, "S tail")
    assert_close(ns_out.cpu().numpy(), ref_n, wl.ns_wdtype, "NS out")


@pytest.mark.parametrize("wdtype", ["bf16", "e4m3"])
def test_256x192_gemms_with_more_tiles_than_cus(wdtype):
    """2048 candidates x 16 NS positions at d = 192, F = 384: the NS QKV (N = 576) and FFN up
    (N = 384) GEMMs take 256x192 tiles, 384 and 256 of them over 8 row tiles (bf16: one tile
    per workgroup; E4M3: the persistent kernel with eight compute waves, several tiles per
    workgroup); every output is compared."""
    wl = Workload(name="p8", n_layers=2, d_model=192, n_heads=3, ffn_hidden=384, s_len=160,
                  q_sched=(160, 40), n_ns=16, n_users=1, n_candidates=2048, ns_wdtype=wdtype)
    m, lay = model(wl)
    s, lens, ns = _inputs(wl, [150])
    sd, ld, nd = _dev(s, lens, ns)
    cache = m.new_cache(1)
    m.user_prefill(sd, ld, cache)
    got = m.score_candidates(cache, 0, nd[0])
    torch.cuda.synchronize()
    oc, _ = O.prefill(lay, wl.q_sched, wl.n_heads, EPS, s[0], int(lens[0]))
    assert_close(got.cpu().numpy(), O.score(lay, wl.n_heads, EPS, oc, ns[0]), wdtype, "NS rows")


# appends to many users with several query blocks per (user, head) in the S attention (two
# blocks per workgroup of the tile kernel); 80 new events leave a ragged block
MANY_APPENDS = {
    "k_dh32_64users_m80": (Workload(name="k", n_layers=2, d_model=64, n_heads=2, ffn_hidden=128, s_len=300,
                                    q_sched=(300, 150), n_ns=4, n_users=64, n_candidates=2), 80),
    "l_dh64_64users_m96": (Workload(name="l", n_layers=2, d_model=128, n_heads=2, ffn_hidden=256, s_len=300,
                                    q_sched=(300, 97), n_ns=4, n_users=64, n_candidates=2), 96),
}


@pytest.mark.parametrize("name", list(MANY_APPENDS))
def test_many_user_append_several_query_blocks(name):
    from unified_transformer_recommender_onetrans_amd._capi import lib
    wl, m = MANY_APPENDS[name]
    B = wl.n_users
    assert lib().onetrans_attention_route(0, wl.head_dim, m, wl.n_heads, B).decode() == f"attn_kernel<{wl.head_dim},2>"
    print(f"case {name}: B={B} m={m}", flush=True)
    mdl, lay = model(wl, append_cap=m)
    base = [300, 0, 1, 33, 64, 65, 127, 128, 129, 200, 255, 256, 257, 299]
    lens = [base[u % len(base)] for u in range(B)]
    s, lens, ns = _inputs(wl, lens)
    sd, ld, nd = _dev(s, lens, ns)
    cache = mdl.new_cache(B)
    mdl.user_prefill(sd, ld, cache)
    new = make_append_tokens(wl, m=m)
    app = mdl.kv_append(bf16_dev(new), cache)
    scored = {u: mdl.score_candidates(cache, u, nd[u]) for u in (0, 1, B - 1)}
    torch.cuda.synchronize()
    app = app.cpu().numpy()
    for u in range(B):
        oc, _ = O.prefill(lay, wl.q_sched, wl.n_heads, EPS, s[u], int(lens[u]))
        oc, oa = O.append(lay, wl.n_heads, EPS, oc, new[u])
        assert_close(app[u], oa, wl.ns_wdtype, f"user {u} (len {lens[u]}) appended rows")
        if u in scored:
            assert_close(scored[u].cpu().numpy(), O.score(lay, wl.n_heads, EPS, oc, ns[u]), wl.ns_wdtype,
                         f"user {u} scores after the append")


def test_peaked_attention_moves_softmax_reference():
    """Cached keys far above the first key tile's scores: the NS kernel's online softmax
    has to move its reference maximum in the middle of the key stream (its rescale
    path) and must still match the oracle."""
    from unified_transformer_recommender_onetrans_amd import OneTrans
    wl = Workload(name="peak", n_layers=2, d_model=128, n_heads=2, ffn_hidden=256, s_len=300,
                  q_sched=(300, 64), n_ns=32, n_users=1, n_candidates=3)
    raw, _ = weights(wl)
    raw = [dict(lw) for lw in raw]
    d = wl.d_model
    eye = np.eye(d, dtype=np.float32)
    for lw in raw:  # W_Q = 1.5 I (NS) / I (S) and W_K = I, so scores are scaled dot products
        sq = lw["s_wqkv"].copy()
        sq[:d], sq[d:2 * d] = eye, eye
        nq = lw["ns_wqkv"].copy()
        nq[:, :d], nq[:, d:2 * d] = 1.5 * eye, eye
        lw["s_wqkv"], lw["ns_wqkv"] = sq, nq
    lay = O.layers_from_arrays(raw)
    s, lens, ns = _inputs(wl, [300])
    s[0, 128:] = ns[0, 0, 0]  # later events repeat candidate 0's first NS token
    # the premise, from the oracle's layer-0 quantities: for NS query (candidate 0, row 0)
    # the best cached key beats the best key of the first 64-key tile by more than 8 in
    # log2 units in every head
    W = lay[0]
    q0 = O.rmsnorm(np.asarray(ns[0, 0, 0], np.float64), W.ns_ga[0], EPS) @ W.ns_wq[0].T
    kS = O.rmsnorm(np.asarray(s[0], np.float64), W.s_ga, EPS) @ W.s_wk.T
    dh = d // wl.n_heads
    for h in range(wl.n_heads):
        sl = slice(h * dh, (h + 1) * dh)
        logits = kS[:, sl] @ q0[sl] / np.sqrt(dh)
        assert (logits.max() - logits[:64].max()) * np.log2(np.e) > 8.5
    m = OneTrans(config(wl), device_weights(raw))
    s_out, ns_out = m.block_forward(*_dev(s, lens, ns))
    torch.cuda.synchronize()
    ref_t, ref_n = O.block_forward(lay, wl.q_sched, wl.n_heads, EPS, s, lens, ns)
    assert_close(s_out.cpu().numpy(), ref_t, wl.ns_wdtype, "S tail")
    assert_close(ns_out.cpu().numpy(), ref_n, wl.ns_wdtype, "NS out")
    assert_close(ns_out[0, 0, 0].cpu().numpy(), ref_n[0, 0, 0], wl.ns_wdtype, "NS row of the peaked query")


def test_peaked_many_user_prefill_moves_softmax_reference():
    """The many-user prefill's tile kernel (attn_kernel<64, 4>) with keys far above the first
    key tile's scores: with W_Q = W_K = I on the S side and every user's later events
    repeating one token, the lazy softmax reference of the S queries has to move in the
    middle of the key stream, and the S tails must still match the oracle."""
    from unified_transformer_recommender_onetrans_amd import OneTrans
    from unified_transformer_recommender_onetrans_amd._capi import lib
    wl = Workload(name="peak_many", n_layers=2, d_model=128, n_heads=2, ffn_hidden=256, s_len=2048,
                  q_sched=(2048, 1000), n_ns=4, n_users=16, n_candidates=2)
    assert lib().onetrans_attention_route(0, 64, 2048, 2, 16).decode() == "attn_kernel<64,4>"
    raw, _ = weights(wl)
    raw = [dict(lw) for lw in raw]
    d = wl.d_model
    eye = np.eye(d, dtype=np.float32)
    for lw in raw:
        sq = lw["s_wqkv"].copy()
        sq[:d], sq[d:2 * d] = eye, eye
        lw["s_wqkv"] = sq
    lay = O.layers_from_arrays(raw)
    lens = _many_lens(wl)
    s, lens, ns = _inputs(wl, lens)
    for u in range(wl.n_users):
        first = wl.s_len - int(lens[u])
        if lens[u] > 128:
            s[u, first + 128:] = s[u, first + 128]  # events from the 129th on repeat that one
    # the premise, from the oracle's layer-0 quantities: for user 0's last S query the best
    # key beats the best key of the first 64-key tile by more than 8 in log2 units
    W = lay[0]
    x0 = O.rmsnorm(np.asarray(s[0], np.float64), W.s_ga, EPS)
    qS, kS = x0 @ W.s_wq.T, x0 @ W.s_wk.T
    dh = d // wl.n_heads
    for h in range(wl.n_heads):
        sl = slice(h * dh, (h + 1) * dh)
        logits = kS[:, sl] @ qS[-1, sl] / np.sqrt(dh)
        assert (logits.max() - logits[:64].max()) * np.log2(np.e) > 8.5
    m = OneTrans(config(wl), device_weights(raw))
    cache = m.new_cache(wl.n_users)
    s_out = m.user_prefill(bf16_dev(s), torch.from_numpy(lens).cuda(), cache)
    torch.cuda.synchronize()
    s_out = s_out.cpu().numpy()
    for u in range(wl.n_users):
        _, ot = O.prefill(lay, wl.q_sched, wl.n_heads, EPS, s[u], int(lens[u]))
        assert_close(s_out[u], ot, wl.ns_wdtype, f"user {u} (len {lens[u]}) S tail")


# user-side NS rows: (workload, histories, n_ns_user)
USER_NS = {
    "b_dh64_P32_u8": (SMALL["b_dh64_P32"][0], [200, 1], 8),
    "a_dh32_P5_u2": (SMALL["a_dh32_P5"][0], [300, 41, 0], 2),
    "c_fp8_u4": (SMALL["c_fp8"][0], [150, 200], 4),
}


def _user_inputs(wl, lens, Pu):
    s, lens, ns = _inputs(wl, lens)
    rng = np.random.default_rng(21)
    un = rng.standard_normal((s.shape[0], Pu, wl.d_model)).astype(np.float32)
    un = torch.from_numpy(un).to(torch.bfloat16).float().numpy()  # bf16 values, as both sides consume
    return s, lens, np.ascontiguousarray(ns[:, :, Pu:]), un


@pytest.mark.parametrize("name", list(USER_NS))
def test_user_ns_block_forward_matches_oracle(name):
    wl, lens, Pu = USER_NS[name]
    print(f"case {name}", flush=True)
    m, lay = model(wl, private_gains=(name == "c_fp8_u4"), n_ns_user=Pu)
    s, lens, cn, un = _user_inputs(wl, lens, Pu)
    s_out, ns_out = m.block_forward(*_dev(s, lens, cn), ns_user_tokens=bf16_dev(un))
    torch.cuda.synchronize()
    ref_t, ref_n = O.block_forward(lay, wl.q_sched, wl.n_heads, EPS, s, lens, cn, un)
    assert ns_out.shape == (s.shape[0], cn.shape[1], wl.n_ns - Pu, wl.d_model)
    assert_close(s_out.cpu().numpy(), ref_t, wl.ns_wdtype, "S tail")
    assert_close(ns_out.cpu().numpy(), ref_n, wl.ns_wdtype, "candidate NS out")


@pytest.mark.parametrize("name", ["b_dh64_P32_u8", "a_dh32_P5_u2"])
def test_user_ns_prefill_append_score_match_oracle(name):
    wl, lens, Pu = USER_NS[name]
    print(f"case {name}", flush=True)
    m1 = 9
    mdl, lay = model(wl, append_cap=m1, n_ns_user=Pu)
    s, lens, cn, un = _user_inputs(wl, lens, Pu)
    sd, ld, nd = _dev(s, lens, cn)
    B = s.shape[0]
    cache = mdl.new_cache(B)
    _, un_out = mdl.user_prefill(sd, ld, cache, ns_user_tokens=bf16_dev(un), return_user_ns=True)
    before = [mdl.score_candidates(cache, u, nd[u]) for u in range(B)]
    new1 = make_append_tokens(wl, m=m1)
    mdl.kv_append(bf16_dev(new1), cache)
    after = [mdl.score_candidates(cache, u, nd[u]) for u in range(B)]
    torch.cuda.synchronize()
    for u in range(B):
        oc, _ = O.prefill(lay, wl.q_sched, wl.n_heads, EPS, s[u], int(lens[u]), un[u])
        assert_close(un_out[u].cpu().numpy(), oc.ns_out, wl.ns_wdtype, f"user {u} user NS rows")
        assert_close(before[u].cpu().numpy(), O.score(lay, wl.n_heads, EPS, oc, cn[u]), wl.ns_wdtype,
                     f"user {u} score")
        oc2, _ = O.append(lay, wl.n_heads, EPS, oc, new1[u])
        assert_close(after[u].cpu().numpy(), O.score(lay, wl.n_heads, EPS, oc2, cn[u]), wl.ns_wdtype,
                     f"user {u} score after append")


def test_user_ns_batched_pass_equals_single_user_passes():
    # the user pass of several users runs as one launch per kernel, one attention segment per
    # user; each user's rows must come out exactly as from a prefill of that user alone
    wl, lens, Pu = USER_NS["a_dh32_P5_u2"]
    mdl, _ = model(wl, n_ns_user=Pu)
    s, lens, cn, un = _user_inputs(wl, lens, Pu)
    sd, ld, nd = _dev(s, lens, cn)
    B = s.shape[0]
    cache = mdl.new_cache(B)
    _, un_all = mdl.user_prefill(sd, ld, cache, ns_user_tokens=bf16_dev(un), return_user_ns=True)
    for u in range(B):
        c1 = mdl.new_cache(1)
        _, un_one = mdl.user_prefill(sd[u:u + 1].contiguous(), ld[u:u + 1].contiguous(), c1,
                                     ns_user_tokens=bf16_dev(un[u:u + 1]), return_user_ns=True)
        assert torch.equal(un_one[0], un_all[u]), f"user {u}"
        assert torch.equal(mdl.score_candidates(c1, 0, nd[u]), mdl.score_candidates(cache, u, nd[u])), f"user {u}"


def test_user_ns_score_equals_block_forward():
    # the same kernels on the same inputs: scoring against a prefilled cache reproduces
    # block_forward bit for bit, also with user-side NS rows
    wl, lens, Pu = USER_NS["b_dh64_P32_u8"]
    mdl, _ = model(wl, n_ns_user=Pu)
    s, lens, cn, un = _user_inputs(wl, lens, Pu)
    sd, ld, nd = _dev(s, lens, cn)
    _, ns_bf = mdl.block_forward(sd, ld, nd, ns_user_tokens=bf16_dev(un))
    cache = mdl.new_cache(s.shape[0])
    mdl.user_prefill(sd, ld, cache, ns_user_tokens=bf16_dev(un))
    for u in range(s.shape[0]):
        assert torch.equal(mdl.score_candidates(cache, u, nd[u]), ns_bf[u])


def test_multi_stage_scoring_on_one_cache():
    # stages with their own NS weights, NS token counts and weight types score against
    # one prefilled cache (the successor system's retrieval / pre-rank / fine-rank
    # stages share the user context); each matches the oracle with its own NS layers
    from unified_transformer_recommender_onetrans_amd import OneTrans
    wl_a, lens = SMALL["b_dh64_P32"]
    raw_a, lay_a = weights(wl_a)
    s_keys = ("s_wqkv", "s_w1", "s_w2", "s_g_attn", "s_g_ffn")
    s, lens, ns_a = _inputs(wl_a, lens)
    sd, ld = bf16_dev(s), torch.from_numpy(lens).cuda()
    ma = OneTrans(config(wl_a), device_weights(raw_a))
    cache = ma.new_cache(s.shape[0])
    ma.user_prefill(sd, ld, cache)
    for name, n_ns, wdtype, n_cand, seed in (("retrieval", 8, "bf16", 9, 1), ("pre-rank", 16, "e4m3", 4, 2),
                                             ("fine-rank", 32, "bf16", 5, 0)):
        wl = wl_a.with_(n_ns=n_ns, ns_wdtype=wdtype, n_candidates=n_cand)
        raw = [dict(lw) for lw in make_weights(wl, seed=seed)]
        for lw, la in zip(raw, raw_a):
            for k in s_keys:
                lw[k] = la[k]
        lay = O.layers_from_arrays(raw)
        m = OneTrans(config(wl), device_weights(raw))
        toks = make_ns_tokens(wl, seed=seed)
        got = [m.score_candidates(cache, u, bf16_dev(toks[u])) for u in range(s.shape[0])]
        torch.cuda.synchronize()
        for u in range(s.shape[0]):
            oc, _ = O.prefill(lay_a, wl_a.q_sched, wl_a.n_heads, EPS, s[u], int(lens[u]))
            assert_close(got[u].cpu().numpy(), O.score(lay, wl.n_heads, EPS, oc, toks[u]), wdtype,
                         f"{name} stage, user {u}")


def test_zero_candidates_and_capacity_errors():
    from unified_transformer_recommender_onetrans_amd import OneTransError
    wl, lens = SMALL["b_dh64_P32"]
    mdl, _ = model(wl, append_cap=4)
    s, lens, ns = _inputs(wl, lens)
    sd, ld, nd = _dev(s, lens, ns)
    cache = mdl.new_cache(2)
    mdl.user_prefill(sd, ld, cache)
    out = mdl.score_candidates(cache, 0, nd[0][:0])
    assert out.shape == (0, wl.n_ns, wl.d_model)
    with pytest.raises(OneTransError):
        mdl.kv_append(bf16_dev(make_append_tokens(wl, n_users=2, m=5)), cache)
    assert cache.n_appended == 0
    with pytest.raises(OneTransError):
        mdl.score_candidates(cache, 2, nd[0])


def test_append_fills_cache_to_capacity():
    # append_cap = 56 with 200 input rows at layers 0 and 1: their caches hold exactly 256
    # keys (four 64-key tiles, no rounding slack), and two appends (40 + 16 events) fill them
    # to the last slot; outputs and scoring against the full cache match the oracle, and
    # one event more is refused without touching the cache
    from unified_transformer_recommender_onetrans_amd import OneTransError
    wl, lens = SMALL["b_dh64_P32"]
    print("case b_dh64_P32, append_cap 56", flush=True)
    mdl, lay = model(wl, append_cap=56)
    s, lens, ns = _inputs(wl, lens)
    sd, ld, nd = _dev(s, lens, ns)
    B = s.shape[0]
    cache = mdl.new_cache(B)
    mdl.user_prefill(sd, ld, cache)
    new1 = make_append_tokens(wl, m=40)
    new2 = make_append_tokens(wl, seed=1, m=16)
    out1 = mdl.kv_append(bf16_dev(new1), cache)
    out2 = mdl.kv_append(bf16_dev(new2), cache)
    assert cache.n_appended == 56
    with pytest.raises(OneTransError):
        mdl.kv_append(bf16_dev(make_append_tokens(wl, seed=2, m=1)), cache)
    assert cache.n_appended == 56
    scores = [mdl.score_candidates(cache, u, nd[u]) for u in range(B)]
    torch.cuda.synchronize()
    for u in range(B):
        oc, _ = O.prefill(lay, wl.q_sched, wl.n_heads, EPS, s[u], int(lens[u]))
        oc, o1 = O.append(lay, wl.n_heads, EPS, oc, new1[u])
        oc, o2 = O.append(lay, wl.n_heads, EPS, oc, new2[u])
        assert_close(out1[u].cpu().numpy(), o1, wl.ns_wdtype, f"user {u} append 1")
        assert_close(out2[u].cpu().numpy(), o2, wl.ns_wdtype, f"user {u} append 2")
        assert_close(scores[u].cpu().numpy(), O.score(lay, wl.n_heads, EPS, oc, ns[u]), wl.ns_wdtype,
                     f"user {u} score against the full cache")


# ---------------------------------------------------------------------------
# invariants on the GPU
# ---------------------------------------------------------------------------

def test_causality_bit_exact():
    wl, lens = SMALL["b_dh64_P32"]
    mdl, _ = model(wl)
    s, lens, ns = _inputs(wl, [200, 200])
    base_t, base_n = mdl.block_forward(*_dev(s, lens, ns))
    j = wl.s_len - 2            # perturb the second-to-last event of user 0
    s2 = s.copy()
    s2[0, j] += 1.0
    t2, n2 = mdl.block_forward(*_dev(s2, lens, ns))
    torch.cuda.synchronize()
    tail_pos = np.arange(wl.s_len - wl.q_sched[-1], wl.s_len)
    before = tail_pos < j
    assert torch.equal(t2[0][before], base_t[0][before])
    assert (t2[0][~before] - base_t[0][~before]).abs().amax(dim=1).min() > 0
    assert (n2[0] - base_n[0]).abs().amax(dim=-1).min() > 0
    assert torch.equal(t2[1], base_t[1]) and torch.equal(n2[1], base_n[1])


def test_score_equals_block_forward_and_subsets():
    wl, lens = SMALL["b_dh64_P32"]
    mdl, _ = model(wl)
    s, lens, ns = _inputs(wl, lens)
    sd, ld, nd = _dev(s, lens, ns)
    _, ns_bf = mdl.block_forward(sd, ld, nd)
    cache = mdl.new_cache(2)
    mdl.user_prefill(sd, ld, cache)
    for u in range(2):
        full = mdl.score_candidates(cache, u, nd[u])
        assert torch.equal(full, ns_bf[u])
        sub = mdl.score_candidates(cache, u, nd[u][1:4].contiguous())
        assert torch.equal(sub, full[1:4])
        perm = torch.tensor([3, 0, 4, 1, 2], device="cuda")
        assert torch.equal(mdl.score_candidates(cache, u, nd[u][perm].contiguous()), full[perm])


def test_append_equals_reprefill_on_gpu():
    wl, lens = SMALL["b_dh64_P32"]
    m = 9
    mdl, _ = model(wl, append_cap=m)
    s, lens, ns = _inputs(wl, lens)
    cache = mdl.new_cache(2)
    mdl.user_prefill(bf16_dev(s), torch.from_numpy(lens).cuda(), cache)
    new = make_append_tokens(wl, n_users=2, m=m)
    got = mdl.kv_append(bf16_dev(new), cache)
    wl2 = wl.with_(s_len=wl.s_len + m, q_sched=tuple(q + m for q in wl.q_sched))
    mdl2, _ = model(wl2)
    cache2 = mdl2.new_cache(2)
    tail2 = mdl2.user_prefill(bf16_dev(np.concatenate([s, new], axis=1)), torch.from_numpy(lens + m).cuda(), cache2)
    sc1 = mdl.score_candidates(cache, 1, bf16_dev(ns[1]))
    sc2 = mdl2.score_candidates(cache2, 1, bf16_dev(ns[1]))
    torch.cuda.synchronize()
    np.testing.assert_allclose(got.cpu().numpy(), tail2[:, -m:].cpu().numpy(), rtol=0, atol=1e-5)
    np.testing.assert_allclose(sc1.cpu().numpy(), sc2.cpu().numpy(), rtol=0, atol=1e-5)


# ---------------------------------------------------------------------------
# full-size workloads (benchmark launch configuration), sampled outputs
# ---------------------------------------------------------------------------

def _score_sampled(wl, sample):
    print(f"workload {wl.name}: C={wl.n_candidates}", flush=True)
    mdl, lay = model(wl)
    s, lens = make_s_tokens(wl)
    ns = make_ns_tokens(wl)
    cache = mdl.new_cache(1)
    tail = mdl.user_prefill(bf16_dev(s), torch.from_numpy(lens).cuda(), cache)
    out = mdl.score_candidates(cache, 0, bf16_dev(ns[0]))
    torch.cuda.synchronize()
    oc, ot = O.prefill(lay, wl.q_sched, wl.n_heads, EPS, s[0], int(lens[0]))
    assert_close(tail[0].cpu().numpy(), ot, "bf16", "S tail")
    got = out[sample].cpu().numpy()
    ref = np.empty_like(got, dtype=np.float64)
    for i in range(0, len(sample), 64):  # the oracle in chunks, with progress lines
        ref[i:i + 64] = O.score(lay, wl.n_heads, EPS, oc, ns[0][sample[i:i + 64]])
        print(f"    oracle: {min(i + 64, len(sample))} of {len(sample)} sampled candidates", flush=True)
    assert_close(got, ref, wl.ns_wdtype, f"{len(sample)} sampled candidates")
    return out, cache, mdl, lay, s, lens, ns


def test_onetrans_s_full_size_sampled():
    _score_sampled(ONETRANS_S, np.array([0, 37, 90, 127]))


def test_onetrans_l_full_size_sampled():
    _score_sampled(ONETRANS_L, np.array([0, 1, 100, 201, 255]))


def test_onetrans_l_block_forward_full_size():
    # the bench's step (block_forward at the OneTrans-L shape, C = 256; S side on the caller's
    # stream, NS side on the second stream gated by per-layer events) must reproduce scoring
    # against a separately prefilled cache bit for bit for all 256 candidates, and the oracle
    # on a sample
    wl = ONETRANS_L
    print(f"workload {wl.name}: block_forward C={wl.n_candidates}", flush=True)
    mdl, lay = model(wl)
    s, lens = make_s_tokens(wl)
    ns = make_ns_tokens(wl)
    sd, ld, nd = bf16_dev(s), torch.from_numpy(lens).cuda(), bf16_dev(ns)
    for rep in range(3):  # repeated steps, as the bench runs them
        t_bf, n_bf = mdl.block_forward(sd, ld, nd)
    cache = mdl.new_cache(1)
    tail = mdl.user_prefill(sd, ld, cache)
    n_sc = mdl.score_candidates(cache, 0, nd[0])
    torch.cuda.synchronize()
    assert torch.equal(t_bf, tail)
    assert torch.equal(n_bf[0], n_sc), "block_forward differs from scoring on a prefilled cache"
    oc, ot = O.prefill(lay, wl.q_sched, wl.n_heads, EPS, s[0], int(lens[0]))
    assert_close(t_bf[0].cpu().numpy(), ot, "bf16", "S tail")
    sample = np.array([0, 77, 128, 255])
    assert_close(n_bf[0][sample].cpu().numpy(), O.score(lay, wl.n_heads, EPS, oc, ns[0][sample]), "bf16",
                 f"candidates {list(sample)}")


@pytest.mark.parametrize("scale", [1e-4, 1e2])
def test_scaled_inputs_match_oracle(scale):
    # S and NS inputs scaled far from N(0, 1): the deferred RMSNorm keeps x * g in fp16, so
    # small rows sit near the fp16 subnormal range and large rows near its top
    wl, lens = SMALL["b_dh64_P32"]
    print(f"case b_dh64_P32 scaled by {scale}", flush=True)
    mdl, lay = model(wl)
    s, lens, ns = _inputs(wl, lens)
    s = bf16_round(s * scale)
    ns = bf16_round(ns * scale)
    s_out, ns_out = mdl.block_forward(*_dev(s, lens, ns))
    torch.cuda.synchronize()
    ref_t, ref_n = O.block_forward(lay, wl.q_sched, wl.n_heads, EPS, s, lens, ns)
    assert_close(s_out.cpu().numpy(), ref_t, wl.ns_wdtype, "S tail")
    assert_close(ns_out.cpu().numpy(), ref_n, wl.ns_wdtype, "NS out")


@pytest.mark.timeout(600)
def test_candidate_heavy_fp8_full_size_sampled():
    # every 8th candidate (512 of 4096), each compared element by element with the oracle
    _score_sampled(CANDIDATE_HEAVY_FP8, np.arange(0, CANDIDATE_HEAVY_FP8.n_candidates, 8))


def test_onetrans_l_user_ns_full_size_sampled():
    # the bench's user-side NS configuration: 8 of the 32 NS positions cached with the
    # user (the first candidate's rows stand in for the user fields), 256 candidates of 24
    # rows scored in the launch configuration the bench times
    wl, Pu = ONETRANS_L, 8
    print(f"workload {wl.name}: C={wl.n_candidates}, n_ns_user={Pu}", flush=True)
    mdl, lay = model(wl, n_ns_user=Pu)
    s, lens = make_s_tokens(wl)
    ns = make_ns_tokens(wl)
    un, cn = ns[:, 0, :Pu], np.ascontiguousarray(ns[0, :, Pu:])
    cache = mdl.new_cache(1)
    _, un_out = mdl.user_prefill(bf16_dev(s), torch.from_numpy(lens).cuda(), cache, ns_user_tokens=bf16_dev(un),
                                 return_user_ns=True)
    out = mdl.score_candidates(cache, 0, bf16_dev(cn))
    torch.cuda.synchronize()
    oc, _ = O.prefill(lay, wl.q_sched, wl.n_heads, EPS, s[0], int(lens[0]), un[0])
    assert_close(un_out[0].cpu().numpy(), oc.ns_out, "bf16", "user NS rows")
    sample = np.array([0, 3, 128, 254, 255])
    assert_close(out[sample].cpu().numpy(), O.score(lay, wl.n_heads, EPS, oc, cn[sample]), "bf16",
                 f"candidates {list(sample)}")


def test_prefill_batch_and_append_full_size_sampled():
    wl = PREFILL_BATCH
    print(f"workload {wl.name}: B={wl.n_users} m={wl.append_m}", flush=True)
    mdl, lay = model(wl, append_cap=wl.append_m)
    s, lens = make_s_tokens(wl)
    new = make_append_tokens(wl)
    cache = mdl.new_cache(wl.n_users)
    tail = mdl.user_prefill(bf16_dev(s), torch.from_numpy(lens).cuda(), cache)
    got = mdl.kv_append(bf16_dev(new), cache)
    torch.cuda.synchronize()
    for u in (0, int(np.argmin(lens)), 63):
        oc, ot = O.prefill(lay, wl.q_sched, wl.n_heads, EPS, s[u], int(lens[u]))
        assert_close(tail[u].cpu().numpy(), ot, "bf16", f"user {u} (len {lens[u]}) S tail")
        oc, on = O.append(lay, wl.n_heads, EPS, oc, new[u])
        assert_close(got[u].cpu().numpy(), on, "bf16", f"user {u} appended rows")
        l = wl.n_layers - 1
        k, v = cache.read_layer(l, u, oc.length(l))
        ok = (oc.base[l] + np.arange(oc.length(l))) >= oc.valid_from
        assert_close(k.float().cpu().numpy()[ok], oc.k[l][ok], "bf16", f"user {u} last-layer cached K")
        assert_close(v.float().cpu().numpy()[ok], oc.v[l][ok], "bf16", f"user {u} last-layer cached V")


def test_prefill_batch_user_ns_full_size_sampled():
    # the bench's 64-user prefill with 8 user-side NS fields per user (one attention segment
    # per user), then an append that recomputes them; sampled users against the oracle: their
    # user NS rows after the prefill, then two candidates scored against the grown cache
    wl, Pu = PREFILL_BATCH, 8
    print(f"workload {wl.name}: B={wl.n_users} n_ns_user={Pu} m={wl.append_m}", flush=True)
    mdl, lay = model(wl, append_cap=wl.append_m, n_ns_user=Pu)
    s, lens = make_s_tokens(wl)
    ns = make_ns_tokens(wl, n_users=wl.n_users, n_candidates=2)
    un = np.ascontiguousarray(ns[:, 0, :Pu])
    cn = np.ascontiguousarray(ns[:, :, Pu:])
    new = make_append_tokens(wl)
    cache = mdl.new_cache(wl.n_users)
    _, un_out = mdl.user_prefill(bf16_dev(s), torch.from_numpy(lens).cuda(), cache, ns_user_tokens=bf16_dev(un),
                                 return_user_ns=True)
    un_out = un_out.cpu().numpy()
    mdl.kv_append(bf16_dev(new), cache)
    sample = (0, int(np.argmin(lens)), 63)
    scored = {u: mdl.score_candidates(cache, u, bf16_dev(cn[u])).cpu().numpy() for u in sample}
    for u in sample:
        oc, _ = O.prefill(lay, wl.q_sched, wl.n_heads, EPS, s[u], int(lens[u]), un[u])
        assert_close(un_out[u], oc.ns_out, "bf16", f"user {u} (len {lens[u]}) user NS rows")
        oc, _ = O.append(lay, wl.n_heads, EPS, oc, new[u])
        assert_close(scored[u], O.score(lay, wl.n_heads, EPS, oc, cn[u]), "bf16", f"user {u} candidates after append")


def test_hip_graph_replays_match_eager():
    # scoring and the block forward captured in a HIP graph (through torch's capture of the
    # current stream; the block forward also forks its second stream inside the capture):
    # every replay, with eager work and synchronisations between replays, must reproduce
    # the eager outputs bit for bit
    wl, lens = SMALL["b_dh64_P32"]
    mdl, _ = model(wl)
    s, lens, ns = _inputs(wl, lens)
    sd, ld, nd = _dev(s, lens, ns)
    cache = mdl.new_cache(s.shape[0])
    mdl.user_prefill(sd, ld, cache)
    eager_sc = mdl.score_candidates(cache, 0, nd[0]).clone()
    eager_t, eager_n = (x.clone() for x in mdl.block_forward(sd, ld, nd))
    torch.cuda.synchronize()
    out_sc = torch.empty_like(eager_sc)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream, as torch's capture expects
        mdl.score_candidates(cache, 0, nd[0], out=out_sc)
        mdl.block_forward(sd, ld, nd)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g_sc, g_bf = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_sc):
        mdl.score_candidates(cache, 0, nd[0], out=out_sc)
    with torch.cuda.graph(g_bf):
        bf_t, bf_n = mdl.block_forward(sd, ld, nd)
    for i in range(4):
        out_sc.fill_(float("nan"))
        bf_n.fill_(float("nan"))
        torch.cuda.synchronize()
        g_sc.replay()
        g_bf.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_sc, eager_sc), f"scoring replay {i}"
        assert torch.equal(bf_t, eager_t) and torch.equal(bf_n, eager_n), f"block forward replay {i}"
