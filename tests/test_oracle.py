"""Pins of the fp64 oracle against facts other than itself.

The pages print no worked example, so the oracle is pinned by closed forms, a
special case that reduces to a plain causal Transformer computed with torch's
own RMSNorm / scaled-dot-product attention / GELU, brute-force causality and
parameter-locality perturbations, the E4M3FN code table, math.erf, and the
invariants the method promises (KV sharing, pyramid tail, append, padding,
candidate independence). Each is chosen so that a plausible slip (a dropped
term, a wrong mask edge, a transposed weight, a wrong NS index, a wrong scale)
fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from onetrans_inputs import TINY, Workload, make_ns_tokens, make_s_tokens, make_weights

EPS = 1e-6


def rand_layers(rng, L, d, Fh, P, tie=False, wscale=None):
    """Random fp64 layers; ``tie`` copies the S weights and gains into every NS position."""
    sd = (1.0 / d) ** 0.5 if wscale is None else wscale
    out = []
    for _ in range(L):
        s = dict(s_wq=rng.normal(0, sd, (d, d)), s_wk=rng.normal(0, sd, (d, d)),
                 s_wv=rng.normal(0, sd, (d, d)), s_w1=rng.normal(0, sd, (Fh, d)),
                 s_w2=rng.normal(0, sd, (d, Fh)), s_ga=1 + rng.normal(0, 0.3, d),
                 s_gf=1 + rng.normal(0, 0.3, d))
        if tie:
            ns = {("ns_" + k[2:]): np.broadcast_to(v, (P,) + v.shape).copy() for k, v in s.items()}
        else:
            ns = dict(ns_wq=rng.normal(0, sd, (P, d, d)), ns_wk=rng.normal(0, sd, (P, d, d)),
                      ns_wv=rng.normal(0, sd, (P, d, d)), ns_w1=rng.normal(0, sd, (P, Fh, d)),
                      ns_w2=rng.normal(0, sd, (P, d, Fh)), ns_ga=1 + rng.normal(0, 0.3, (P, d)),
                      ns_gf=1 + rng.normal(0, 0.3, (P, d)))
        out.append(O.Layer(**s, **ns))
    return out


# ---------------------------------------------------------------------------
# Elementary pieces
# ---------------------------------------------------------------------------

def test_rmsnorm_closed_form():
    # a constant row a*1 normalises to g * a / sqrt(a^2 + eps)
    d = 16
    g = np.linspace(0.5, 1.5, d)
    for a in (3.0, -0.25, 1e-4):
        got = O.rmsnorm(np.full(d, a), g, EPS)
        np.testing.assert_allclose(got, g * a / math.sqrt(a * a + EPS), rtol=1e-14)
    # scale invariance (up to eps): RMSNorm(c x) == RMSNorm(x) for c > 0
    x = np.random.default_rng(0).normal(size=(4, d))
    np.testing.assert_allclose(O.rmsnorm(7 * x, g, 0.0), O.rmsnorm(x, g, 0.0), rtol=1e-13)


def test_gelu_against_math_erf():
    xs = np.linspace(-8, 8, 2001)
    ref = np.array([0.5 * x * (1 + math.erf(x / math.sqrt(2))) for x in xs])
    np.testing.assert_allclose(O.gelu(xs), ref, rtol=1e-14, atol=1e-15)
    assert O.gelu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(O.gelu(np.array([12.0, -12.0])), [12.0, 0.0], atol=1e-20)
    # the torch CPU implementation of the exact form agrees too
    np.testing.assert_allclose(O.gelu(xs), F.gelu(torch.tensor(xs)).numpy(), rtol=1e-12, atol=1e-15)


def test_e4m3fn_code_table_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3fn_to_float(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9


def test_generator_weights_dequantise_consistently():
    # bf16 storage and E4M3 codes x scale approximate the same fp64 draws: a wrong
    # scale index (q/k/v/w1/w2) or a transposed matrix would break the bound.
    wl = TINY.with_(n_ns=3)
    a = O.layers_from_arrays(make_weights(wl, seed=5))[0]
    b = O.layers_from_arrays(make_weights(wl.with_(ns_wdtype="e4m3"), seed=5))[0]
    for name in ("ns_wq", "ns_wk", "ns_wv", "ns_w1", "ns_w2"):
        wa, wb = getattr(a, name), getattr(b, name)
        for k in range(3):
            amax = np.abs(wa[k]).max()
            bound = (2.0 ** -4 + 2.0 ** -8) * np.abs(wa[k]) + amax / 448 * 2.0 ** -9 * 1.01
            assert np.all(np.abs(wa[k] - wb[k]) <= bound), name
    assert np.array_equal(a.s_wq, b.s_wq)


# ---------------------------------------------------------------------------
# Closed forms of the whole block
# ---------------------------------------------------------------------------

def test_single_token_closed_form():
    # one S token, no NS: attention over one key returns v, so
    # out = x + v + W2 GELU(W1 RMSNorm(x + v)), with v = W_V RMSNorm(x)
    rng = np.random.default_rng(1)
    d, Fh = 8, 24
    lay = rand_layers(rng, 1, d, Fh, 0)
    W = lay[0]
    x = rng.normal(size=(1, d))
    r = np.sqrt(np.sum(x[0] ** 2) / d + EPS)
    v = W.s_wv @ (x[0] / r * W.s_ga)
    z = x[0] + v
    rz = np.sqrt(np.sum(z ** 2) / d + EPS)
    h = W.s_w1 @ (z / rz * W.s_gf)
    h = np.array([0.5 * t * (1 + math.erf(t / math.sqrt(2))) for t in h])
    want = z + W.s_w2 @ h
    tail, ns, _ = O.forward_dense(lay, [1], 2, EPS, x, 1, np.zeros((0, d)))
    np.testing.assert_allclose(tail[0], want, rtol=1e-12)
    _, tail2 = O.prefill(lay, [1], 2, EPS, x, 1)
    np.testing.assert_allclose(tail2[0], want, rtol=1e-12)


@pytest.mark.parametrize("L_S,s_valid,q0", [(6, 6, 6), (6, 4, 3), (7, 7, 2), (5, 2, 5)])
def test_uniform_attention_closed_form(L_S, s_valid, q0):
    # W_Q = 0 makes every visible score 0, so each row averages the V rows it may
    # see. With W_V = I, gains 1, eps ~ 0 and one-hot inputs c*e_j, V rows are
    # sign(c) sqrt(d) e_j; W_2 = 0 removes the FFN. So out_r = x_r + mean of those.
    # Pins: self-inclusive causal mask, bottom-right tail alignment, padding
    # exclusion, NS sees all valid S plus NS up to itself.
    rng = np.random.default_rng(2)
    d, P, H = 16, 3, 2
    eps = 1e-30
    lay = rand_layers(rng, 1, d, 8, P)
    W = lay[0]
    W.s_wq[:] = 0; W.ns_wq[:] = 0
    W.s_wv[:] = np.eye(d); W.ns_wv[:] = np.eye(d)
    W.s_ga[:] = 1; W.ns_ga[:] = 1
    W.s_w2[:] = 0; W.ns_w2[:] = 0
    cs = rng.choice([-2.0, -0.5, 0.7, 3.0], size=L_S)
    cn = rng.choice([-1.5, 0.4, 2.5], size=P)
    xs = np.zeros((L_S, d)); xn = np.zeros((P, d))
    vs = np.zeros((L_S, d)); vn = np.zeros((P, d))
    for j in range(L_S):
        xs[j, j % d] = cs[j]; vs[j, j % d] = np.sign(cs[j]) * math.sqrt(d)
    for k in range(P):
        xn[k, (L_S + k) % d] = cn[k]; vn[k, (L_S + k) % d] = np.sign(cn[k]) * math.sqrt(d)
    vf = L_S - s_valid
    want_s = []
    for i in range(L_S - q0, L_S):
        if i < vf:
            want_s.append(np.zeros(d))
        else:
            want_s.append(xs[i] + np.mean([vs[j] for j in range(vf, i + 1)], axis=0))
    want_n = [xn[k] + np.mean([vs[j] for j in range(vf, L_S)] + [vn[t] for t in range(k + 1)], axis=0)
              for k in range(P)]
    tail, ns, _ = O.forward_dense(lay, [q0], H, eps, xs, s_valid, xn)
    np.testing.assert_allclose(tail, np.array(want_s), atol=1e-12)
    np.testing.assert_allclose(ns, np.array(want_n), atol=1e-12)
    cache, tail2 = O.prefill(lay, [q0], H, eps, xs, s_valid)
    np.testing.assert_allclose(tail2, np.array(want_s), atol=1e-12)
    np.testing.assert_allclose(O.score(lay, H, eps, cache, xn[None])[0], np.array(want_n), atol=1e-12)


def torch_plain_causal_transformer(x, layers, n_heads, eps):
    """A homogeneous pre-norm causal Transformer written with torch's own primitives."""
    X = torch.tensor(x, dtype=torch.float64)[None]
    T, d = X.shape[1], X.shape[2]
    dh = d // n_heads
    mask = torch.ones(T, T, dtype=torch.bool).tril()
    t = lambda a: torch.tensor(a, dtype=torch.float64)
    for W in layers:
        a = F.rms_norm(X, (d,), weight=t(W.s_ga), eps=eps)
        q, k, v = (F.linear(a, t(w)).view(1, T, n_heads, dh).transpose(1, 2) for w in (W.s_wq, W.s_wk, W.s_wv))
        o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask)
        X = X + o.transpose(1, 2).reshape(1, T, d)
        X = X + F.linear(F.gelu(F.linear(F.rms_norm(X, (d,), weight=t(W.s_gf), eps=eps), t(W.s_w1))), t(W.s_w2))
    return X[0].numpy()


@pytest.mark.parametrize("P", [0, 5])
def test_tied_weights_reduce_to_plain_causal_transformer(P):
    # With every NS weight and gain tied to the S ones and no pyramid (q_l = n_l),
    # OneTrans is an ordinary pre-norm causal Transformer over [S ; NS].
    rng = np.random.default_rng(3)
    L, d, Fh, H, L_S = 3, 24, 40, 3, 9
    lay = rand_layers(rng, L, d, Fh, P, tie=True)
    xs = rng.normal(size=(L_S, d)); xn = rng.normal(size=(P, d))
    ref = torch_plain_causal_transformer(np.concatenate([xs, xn]), lay, H, EPS)
    tail, ns, _ = O.forward_dense(lay, [L_S] * L, H, EPS, xs, L_S, xn)
    np.testing.assert_allclose(tail, ref[:L_S], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ns, ref[L_S:], rtol=1e-10, atol=1e-12)
    cache, tail2 = O.prefill(lay, [L_S] * L, H, EPS, xs, L_S)
    np.testing.assert_allclose(tail2, ref[:L_S], rtol=1e-10, atol=1e-12)
    if P:
        np.testing.assert_allclose(O.score(lay, H, EPS, cache, xn[None])[0], ref[L_S:], rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# Brute-force causality and parameter locality
# ---------------------------------------------------------------------------

def _toy(seed=4, L=2, d=16, Fh=32, P=4, L_S=10):
    rng = np.random.default_rng(seed)
    return rng, rand_layers(rng, L, d, Fh, P), rng.normal(size=(L_S, d)), rng.normal(size=(P, d))


def test_causality_perturb_s_token():
    rng, lay, xs, xn = _toy()
    H, L_S = 2, xs.shape[0]
    q = [L_S, L_S]
    t0, n0, _ = O.forward_dense(lay, q, H, EPS, xs, L_S, xn)
    for j in (0, 4, L_S - 1):
        xs2 = xs.copy(); xs2[j] += rng.normal(size=xs.shape[1])
        t1, n1, _ = O.forward_dense(lay, q, H, EPS, xs2, L_S, xn)
        np.testing.assert_array_equal(t1[:j], t0[:j])          # earlier events unchanged
        assert np.all(np.abs(t1[j:] - t0[j:]).max(axis=1) > 1e-9)   # later ones change
        assert np.all(np.abs(n1 - n0).max(axis=1) > 1e-9)          # every NS token sees it


def test_causality_perturb_ns_token():
    rng, lay, xs, xn = _toy()
    H, L_S, P = 2, xs.shape[0], xn.shape[0]
    q = [L_S, 6]
    t0, n0, _ = O.forward_dense(lay, q, H, EPS, xs, L_S, xn)
    for k in range(P):
        xn2 = xn.copy(); xn2[k] += rng.normal(size=xn.shape[1])
        t1, n1, _ = O.forward_dense(lay, q, H, EPS, xs, L_S, xn2)
        np.testing.assert_array_equal(t1, t0)                  # S side never sees NS
        np.testing.assert_array_equal(n1[:k], n0[:k])
        assert np.all(np.abs(n1[k:] - n0[k:]).max(axis=1) > 1e-9)


@pytest.mark.parametrize("name,first_changed,only_self", [
    ("ns_wq", 0, True), ("ns_w1", 0, True), ("ns_w2", 0, True), ("ns_gf", 0, True),
    ("ns_wk", 0, False), ("ns_wv", 0, False), ("ns_ga", 0, False)])
def test_private_parameters_act_on_their_position(name, first_changed, only_self):
    # Changing NS position k's private weights changes row k (and, through its
    # K/V, later NS rows); earlier NS rows and the S side never move.
    rng, lay, xs, xn = _toy(L=1)
    H, L_S, P = 2, xs.shape[0], xn.shape[0]
    t0, n0, _ = O.forward_dense(lay, [L_S], H, EPS, xs, L_S, xn)
    for k in range(P):
        lay2 = [O.Layer(**{f: getattr(lay[0], f).copy() for f in lay[0].__dataclass_fields__})]
        arr = getattr(lay2[0], name)
        arr[k] += rng.normal(0, 0.3, arr[k].shape)
        t1, n1, _ = O.forward_dense(lay2, [L_S], H, EPS, xs, L_S, xn)
        np.testing.assert_array_equal(t1, t0)
        np.testing.assert_array_equal(n1[:k], n0[:k])
        assert np.abs(n1[k] - n0[k]).max() > 1e-9
        if only_self:
            np.testing.assert_array_equal(n1[k + 1:], n0[k + 1:])
        else:
            assert all(np.abs(n1[t] - n0[t]).max() > 1e-9 for t in range(k + 1, P))


# ---------------------------------------------------------------------------
# Invariants of the fast form
# ---------------------------------------------------------------------------

def _gen_case(wl, seed=0, private_gains=False):
    lay = O.layers_from_arrays(make_weights(wl, seed=seed, ns_private_gains=private_gains))
    s, lens = make_s_tokens(wl, seed=seed)
    ns = make_ns_tokens(wl, seed=seed)
    return lay, s, lens, ns


@pytest.mark.parametrize("private_gains", [False, True])
@pytest.mark.parametrize("wl", [
    TINY,
    Workload(name="toy_pyr", n_layers=3, d_model=32, n_heads=2, ffn_hidden=64, s_len=40,
             q_sched=(33, 17, 5), n_ns=6, n_users=2, n_candidates=3, len_range=(12, 40)),
    Workload(name="toy_pad", n_layers=2, d_model=32, n_heads=4, ffn_hidden=96, s_len=24,
             q_sched=(24, 20), n_ns=4, n_users=3, n_candidates=2, len_range=(3, 12)),
])
def test_fast_equals_dense(wl, private_gains):
    # S side once per user + NS per candidate == full recompute per candidate
    lay, s, lens, ns = _gen_case(wl, private_gains=private_gains)
    H = wl.n_heads
    tails, outs = O.block_forward(lay, wl.q_sched, H, EPS, s, lens, ns)
    for u in range(s.shape[0]):
        cache, _ = O.prefill(lay, wl.q_sched, H, EPS, s[u], int(lens[u]))
        for c in range(ns.shape[1]):
            t, n, kv = O.forward_dense(lay, wl.q_sched, H, EPS, s[u], int(lens[u]), ns[u, c])
            np.testing.assert_allclose(tails[u], t, rtol=1e-11, atol=1e-11)
            np.testing.assert_allclose(outs[u, c], n, rtol=1e-11, atol=1e-11)
        ok = lambda l: (cache.base[l] + np.arange(cache.length(l))) >= cache.valid_from
        for l in range(wl.n_layers):
            np.testing.assert_allclose(cache.k[l][ok(l)], kv[l][0][ok(l)], rtol=1e-11, atol=1e-11)
            np.testing.assert_allclose(cache.v[l][ok(l)], kv[l][1][ok(l)], rtol=1e-11, atol=1e-11)


def test_pyramid_layer_is_tail_of_unpruned_layer():
    rng, lay, xs, xn = _toy(L=1)
    H, L_S = 2, xs.shape[0]
    full, nf, _ = O.forward_dense(lay, [L_S], H, EPS, xs, L_S, xn)
    for q in (1, 3, L_S - 1):
        tail, nq, _ = O.forward_dense(lay, [q], H, EPS, xs, L_S, xn)
        np.testing.assert_array_equal(tail, full[L_S - q:])
        np.testing.assert_array_equal(nq, nf)
        _, t2 = O.prefill(lay, [q], H, EPS, xs, L_S)
        np.testing.assert_allclose(t2, full[L_S - q:], rtol=1e-12, atol=1e-13)


def test_padding_equals_shorter_history():
    # a right-aligned history of v valid events behaves like the unpadded history
    rng, lay, xs, xn = _toy(L=2)
    H, L_S = 2, xs.shape[0]
    v = 6
    q = [5, 3]
    padded = xs.copy(); padded[:L_S - v] = rng.normal(size=(L_S - v, xs.shape[1]))  # junk is ignored
    t_pad, n_pad, _ = O.forward_dense(lay, q, H, EPS, padded, v, xn)
    t_short, n_short, _ = O.forward_dense(lay, q, H, EPS, xs[L_S - v:], v, xn)
    np.testing.assert_allclose(t_pad, t_short, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(n_pad, n_short, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("s_valid,m", [(40, 5), (23, 8), (13, 1)])
def test_append_equals_reprefill(s_valid, m):
    # prefill(n) + append(m) == prefill(n + m) with every q_l raised by m
    wl = Workload(name="toy_app", n_layers=3, d_model=32, n_heads=2, ffn_hidden=64, s_len=40,
                  q_sched=(36, 20, 4), n_ns=4, n_users=1, n_candidates=3)
    lay = O.layers_from_arrays(make_weights(wl, seed=7))
    rng = np.random.default_rng(7)
    xs = rng.normal(size=(wl.s_len, wl.d_model))
    new = rng.normal(size=(m, wl.d_model))
    ns = rng.normal(size=(3, wl.n_ns, wl.d_model))
    H = wl.n_heads
    cache, tail = O.prefill(lay, wl.q_sched, H, EPS, xs, s_valid)
    cache2, new_out = O.append(lay, H, EPS, cache, new)
    q2 = [q + m for q in wl.q_sched]
    ref_cache, ref_tail = O.prefill(lay, q2, H, EPS, np.concatenate([xs, new]), s_valid + m)
    np.testing.assert_allclose(new_out, ref_tail[-m:], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(tail, ref_tail[:-m], rtol=1e-11, atol=1e-12)
    assert cache2.base == ref_cache.base and cache2.valid_from == ref_cache.valid_from
    for l in range(wl.n_layers):
        np.testing.assert_allclose(cache2.k[l], ref_cache.k[l], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(cache2.v[l], ref_cache.v[l], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(O.score(lay, H, EPS, cache2, ns), O.score(lay, H, EPS, ref_cache, ns),
                               rtol=1e-11, atol=1e-12)
    # two appends in a row == one append of both
    c_a, o_a = O.append(lay, H, EPS, cache, new[:1])
    c_b, o_b = O.append(lay, H, EPS, c_a, new[1:])
    if m > 1:
        np.testing.assert_allclose(np.concatenate([o_a, o_b]), new_out, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# User-side NS fields, computed once per user and cached
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("Pu,s_valid", [(2, 7), (1, 10), (4, 3)])
def test_user_ns_cached_equals_literal(Pu, s_valid):
    # NS positions 0..Pu-1 computed once in the user's prefill and cached; each
    # candidate's rows Pu..P-1 scored against that cache == the literal definition
    # over [S ; user NS ; candidate NS], candidate by candidate
    rng = np.random.default_rng(11)
    L, d, Fh, H, L_S, P, C = 3, 16, 32, 2, 10, 5, 3
    lay = rand_layers(rng, L, d, Fh, P)
    q = [8, 5, 2]
    xs = rng.normal(size=(L_S, d))
    un = rng.normal(size=(Pu, d))
    cn = rng.normal(size=(C, P - Pu, d))
    cache, tail = O.prefill(lay, q, H, EPS, xs, s_valid, un)
    assert cache.n_user_ns == Pu and len(cache.nk) == L and cache.nk[0].shape == (Pu, d)
    got = O.score(lay, H, EPS, cache, cn)
    for c in range(C):
        t_ref, n_ref, _ = O.forward_dense(lay, q, H, EPS, xs, s_valid, np.concatenate([un, cn[c]]))
        np.testing.assert_allclose(tail, t_ref, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(cache.ns_out, n_ref[:Pu], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(got[c], n_ref[Pu:], rtol=1e-11, atol=1e-12)


def test_user_ns_rows_see_candidates_nowhere():
    # a user NS row's output does not depend on any candidate row (they come later),
    # while every candidate row does depend on the user NS rows
    rng = np.random.default_rng(13)
    L, d, Fh, H, L_S, P, Pu = 2, 16, 32, 2, 8, 4, 2
    lay = rand_layers(rng, L, d, Fh, P)
    xs = rng.normal(size=(L_S, d))
    un = rng.normal(size=(Pu, d))
    cn = rng.normal(size=(P - Pu, d))
    _, n1, _ = O.forward_dense(lay, [L_S] * L, H, EPS, xs, L_S, np.concatenate([un, cn]))
    _, n2, _ = O.forward_dense(lay, [L_S] * L, H, EPS, xs, L_S, np.concatenate([un, cn + 1.0]))
    np.testing.assert_array_equal(n1[:Pu], n2[:Pu])
    un2 = un.copy(); un2[0] += 1.0
    _, n3, _ = O.forward_dense(lay, [L_S] * L, H, EPS, xs, L_S, np.concatenate([un2, cn]))
    assert np.all(np.abs(n3[Pu:] - n1[Pu:]).max(axis=1) > 1e-6)


@pytest.mark.parametrize("m", [1, 4])
def test_user_ns_append_equals_reprefill(m):
    # appended events change what the user NS rows see: append recomputes them, and
    # the result equals a prefill of the longer history with the same user fields
    rng = np.random.default_rng(12)
    L, d, Fh, H, L_S, P, Pu = 2, 16, 32, 2, 12, 4, 2
    lay = rand_layers(rng, L, d, Fh, P)
    q, s_valid = [10, 4], 9
    xs = rng.normal(size=(L_S, d))
    un = rng.normal(size=(Pu, d))
    new = rng.normal(size=(m, d))
    cn = rng.normal(size=(3, P - Pu, d))
    cache, _ = O.prefill(lay, q, H, EPS, xs, s_valid, un)
    cache2, _ = O.append(lay, H, EPS, cache, new)
    ref, _ = O.prefill(lay, [x + m for x in q], H, EPS, np.concatenate([xs, new]), s_valid + m, un)
    np.testing.assert_allclose(cache2.ns_out, ref.ns_out, rtol=1e-11, atol=1e-12)
    for l in range(L):
        np.testing.assert_allclose(cache2.nk[l], ref.nk[l], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(cache2.nv[l], ref.nv[l], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(O.score(lay, H, EPS, cache2, cn), O.score(lay, H, EPS, ref, cn), rtol=1e-11, atol=1e-12)
    # and the appended history did change the user NS rows
    assert np.abs(cache2.ns_out - cache.ns_out).max() > 1e-6


def test_candidates_are_independent_and_permutation_equivariant():
    wl = TINY.with_(n_candidates=6)
    lay, s, lens, ns = _gen_case(wl, seed=11)
    cache, _ = O.prefill(lay, wl.q_sched, wl.n_heads, EPS, s[0], int(lens[0]))
    full = O.score(lay, wl.n_heads, EPS, cache, ns[0])
    perm = np.array([4, 1, 5, 0, 3, 2])
    # equal up to the rounding order of batched BLAS calls
    close = lambda a, b: np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    close(O.score(lay, wl.n_heads, EPS, cache, ns[0][perm]), full[perm])
    close(O.score(lay, wl.n_heads, EPS, cache, ns[0][2:4]), full[2:4])
    close(O.score(lay, wl.n_heads, EPS, cache, ns[0], chunk=4), full)
