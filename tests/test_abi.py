"""Host-side tests of the C ABI (no GPU): exports, config validation, sizing,
argument validation of the compute calls (each call here fails validation
before anything reaches the device)."""
import ctypes
import os
import re

import pytest

from unified_transformer_recommender_onetrans_amd import _capi as C
from unified_transformer_recommender_onetrans_amd.api import make_config

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "onetrans.h")
OK, INVALID, UNSUPPORTED, WORKSPACE, CAPACITY = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(C.LIB_PATH):
        from unified_transformer_recommender_onetrans_amd.build import build
        build()
    return C.lib()


def l_cfg(**kw):
    base = dict(n_layers=8, d_model=384, n_heads=6, ffn_hidden=1536, n_ns=32, s_len=1500,
                q_sched=(1500, 1280, 1088, 864, 640, 448, 224, 16), append_cap=64)
    base.update(kw)
    return make_config(**base)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\*]+\s+\**(onetrans_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(C.EXPORTS), "ctypes declarations out of sync with the header"


def test_valid_configs(lib):
    assert lib.onetrans_check_config(ctypes.byref(l_cfg())) == OK
    tiny = make_config(1, 64, 2, 256, 8, 64, (64,))
    assert lib.onetrans_check_config(ctypes.byref(tiny)) == OK
    assert lib.onetrans_check_config(ctypes.byref(l_cfg(ns_wdtype="e4m3"))) == OK
    assert lib.onetrans_check_config(ctypes.byref(l_cfg(n_heads=12))) == OK          # head_dim 32
    assert lib.onetrans_check_config(ctypes.byref(l_cfg(d_model=320, n_heads=5))) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(d_model=352, n_heads=11), UNSUPPORTED),                # head_dim 32 but d % 64 != 0
    (dict(n_heads=4), UNSUPPORTED),                              # head_dim 96
    (dict(d_model=1088, n_heads=17), UNSUPPORTED),               # d > 1024
    (dict(ffn_hidden=1000), UNSUPPORTED),
    (dict(n_ns=0), UNSUPPORTED),
    (dict(n_ns=257), UNSUPPORTED),
    (dict(q_sched=(1500, 1280, 1300, 864, 640, 448, 224, 16)), UNSUPPORTED),   # increasing
    (dict(q_sched=(1501, 1280, 1088, 864, 640, 448, 224, 16)), UNSUPPORTED),   # q_0 > s_len
    (dict(q_sched=(1500, 1280, 1088, 864, 640, 448, 224, 0)), UNSUPPORTED),    # q = 0
    (dict(append_cap=-1), UNSUPPORTED),
    (dict(rms_eps=0.0), INVALID),
])
def test_invalid_configs(lib, kw, code):
    cfg = l_cfg(**kw)
    assert lib.onetrans_check_config(ctypes.byref(cfg)) == code
    assert lib.onetrans_last_error().decode()
    assert lib.onetrans_packed_weight_bytes(ctypes.byref(cfg)) == 0
    assert lib.onetrans_kv_cache_bytes(ctypes.byref(cfg), 1) == 0


def test_bad_layer_count_and_wdtype(lib):
    cfg = l_cfg()
    cfg.n_layers = 17
    assert lib.onetrans_check_config(ctypes.byref(cfg)) == UNSUPPORTED
    cfg = l_cfg()
    cfg.ns_wdtype = 7
    assert lib.onetrans_check_config(ctypes.byref(cfg)) == UNSUPPORTED
    assert lib.onetrans_check_config(None) == INVALID


def test_sizes(lib):
    cfg = l_cfg()
    d, F, P, L = 384, 1536, 32, 8
    pk = lib.onetrans_packed_weight_bytes(ctypes.byref(cfg))
    weights = L * 2 * (3 * d * d + 2 * F * d) * (1 + P)
    assert weights <= pk <= weights + L * (P * (2 * d * 4 + 20) + 2 * d * 4 + 11 * 256)
    pk8 = lib.onetrans_packed_weight_bytes(ctypes.byref(l_cfg(ns_wdtype="e4m3")))
    assert pk8 < pk
    c1 = lib.onetrans_kv_cache_bytes(ctypes.byref(cfg), 1)
    c64 = lib.onetrans_kv_cache_bytes(ctypes.byref(cfg), 64)
    rows = sum([1500, 1500, 1280, 1088, 864, 640, 448, 224]) + 8 * 64
    assert c1 >= rows * d * 2 * 2 and 60 * c1 < c64 <= 64 * c1 + 256
    assert lib.onetrans_kv_cache_bytes(ctypes.byref(cfg), 0) == 0
    ws = lib.onetrans_workspace_bytes(ctypes.byref(cfg), 64, 4096, 64)
    assert ws >= 4096 * P * (3 * d + F) * 2
    assert ws >= 64 * 1500 * d * 4
    bf = lib.onetrans_block_forward_workspace_bytes(ctypes.byref(cfg), 2, 256)
    assert bf > lib.onetrans_kv_cache_bytes(ctypes.byref(cfg), 2)


def test_cache_init_validation(lib):
    cfg = l_cfg()
    need = lib.onetrans_kv_cache_bytes(ctypes.byref(cfg), 2)
    c = C.KVCache()
    fake = 1 << 40  # never dereferenced: kv_cache_init does no device work
    assert lib.onetrans_kv_cache_init(ctypes.byref(cfg), 2, fake, need - 1, ctypes.byref(c)) == WORKSPACE
    assert lib.onetrans_kv_cache_init(ctypes.byref(cfg), 2, fake + 8, need, ctypes.byref(c)) == INVALID
    assert lib.onetrans_kv_cache_init(ctypes.byref(cfg), 0, fake, need, ctypes.byref(c)) == INVALID
    assert lib.onetrans_kv_cache_init(ctypes.byref(cfg), 2, fake, need, ctypes.byref(c)) == OK
    assert c.n_users == 2 and c.n_appended == 0 and c.prefilled == 0 and c.bytes == need


def _cache(lib, cfg, n_users=2, prefilled=1, n_appended=0):
    c = C.KVCache()
    need = lib.onetrans_kv_cache_bytes(ctypes.byref(cfg), n_users)
    assert lib.onetrans_kv_cache_init(ctypes.byref(cfg), n_users, 1 << 40, need, ctypes.byref(c)) == OK
    c.prefilled, c.n_appended = prefilled, n_appended
    return c


def test_compute_calls_reject_bad_arguments(lib):
    # every call below fails host validation and returns before any device work
    cfg = l_cfg()
    F = 1 << 41  # fake 16-byte-aligned "device" addresses, never dereferenced
    c = _cache(lib, cfg)
    big = 1 << 40
    # prefill
    assert lib.onetrans_user_prefill(ctypes.byref(cfg), None, F, F, 1, None, ctypes.byref(c), F, None, F, big, None) == INVALID
    assert lib.onetrans_user_prefill(ctypes.byref(cfg), F, F, F, 3, None, ctypes.byref(c), F, None, F, big, None) == INVALID
    assert lib.onetrans_user_prefill(ctypes.byref(cfg), F, F, F, 1, None, ctypes.byref(c), F + 4, None, F, big, None) == INVALID
    assert lib.onetrans_user_prefill(ctypes.byref(cfg), F, F, F, 2, None, ctypes.byref(c), F, None, F, 1024, None) == WORKSPACE
    # append
    assert lib.onetrans_kv_append(ctypes.byref(cfg), F, F, 65, ctypes.byref(c), F, F, big, None) == CAPACITY
    c2 = _cache(lib, cfg, n_appended=60)
    assert lib.onetrans_kv_append(ctypes.byref(cfg), F, F, 5, ctypes.byref(c2), F, F, big, None) == CAPACITY
    assert lib.onetrans_kv_append(ctypes.byref(cfg), F, F, 4, ctypes.byref(c2), F, F, 16, None) == WORKSPACE
    assert lib.onetrans_kv_append(ctypes.byref(cfg), F, F, -1, ctypes.byref(c), F, F, big, None) == INVALID
    assert lib.onetrans_kv_append(ctypes.byref(cfg), F, F, 0, ctypes.byref(c), F, F, big, None) == OK  # no-op
    cu = _cache(lib, cfg, prefilled=0)
    assert lib.onetrans_kv_append(ctypes.byref(cfg), F, F, 1, ctypes.byref(cu), F, F, big, None) == INVALID
    # score: only prefilled users (c holds 2 users, 1 prefilled)
    assert lib.onetrans_score_candidates(ctypes.byref(cfg), F, ctypes.byref(c), 2, F, 8, F, F, big, None) == INVALID
    assert lib.onetrans_score_candidates(ctypes.byref(cfg), F, ctypes.byref(c), 1, F, 8, F, F, big, None) == INVALID
    assert "not prefilled" in lib.onetrans_last_error().decode()
    assert lib.onetrans_kv_cache_read(ctypes.byref(cfg), ctypes.byref(c), 0, 1, 1, F, F, None) == INVALID
    cbad = _cache(lib, cfg, prefilled=3)  # a struct that claims more prefilled users than it holds
    assert lib.onetrans_score_candidates(ctypes.byref(cfg), F, ctypes.byref(cbad), 0, F, 8, F, F, big, None) == INVALID
    assert lib.onetrans_kv_append(ctypes.byref(cfg), F, F, 1, ctypes.byref(cbad), F, F, big, None) == INVALID
    assert lib.onetrans_score_candidates(ctypes.byref(cfg), F, ctypes.byref(c), -1, F, 8, F, F, big, None) == INVALID
    assert lib.onetrans_score_candidates(ctypes.byref(cfg), F, ctypes.byref(cu), 0, F, 8, F, F, big, None) == INVALID
    assert lib.onetrans_score_candidates(ctypes.byref(cfg), F, ctypes.byref(c), 0, F, 8, F, F, 100, None) == WORKSPACE
    assert lib.onetrans_score_candidates(ctypes.byref(cfg), F, ctypes.byref(c), 0, F, -1, F, F, big, None) == INVALID
    assert lib.onetrans_score_candidates(ctypes.byref(cfg), F, ctypes.byref(c), 0, F, 0, F, F, big, None) == OK
    assert lib.onetrans_score_candidates(ctypes.byref(cfg), F, ctypes.byref(c), 0, F + 2, 8, F, F, big, None) == INVALID
    # block_forward
    assert lib.onetrans_block_forward(ctypes.byref(cfg), F, F, F, 0, None, F, 4, F, F, F, big, None) == INVALID
    assert lib.onetrans_block_forward(ctypes.byref(cfg), F, F, F, 1, None, F, 4, F, F, F, 10, None) == WORKSPACE
    assert lib.onetrans_block_forward(ctypes.byref(cfg), F, F, F, 1, None, None, 4, F, None, F, big, None) == INVALID
    # cache read
    assert lib.onetrans_kv_cache_read(ctypes.byref(cfg), ctypes.byref(c), 8, 0, 1, F, F, None) == INVALID
    assert lib.onetrans_kv_cache_read(ctypes.byref(cfg), ctypes.byref(c), 0, 0, 1501, F, F, None) == INVALID
    # pack
    assert lib.onetrans_pack_weights(ctypes.byref(cfg), None, F, big, None) == INVALID
    lw = (C.LayerWeights * 8)()
    need = lib.onetrans_packed_weight_bytes(ctypes.byref(cfg))
    assert lib.onetrans_pack_weights(ctypes.byref(cfg), lw, F, need - 1, None) == WORKSPACE
    assert lib.onetrans_pack_weights(ctypes.byref(cfg), lw, F, need, None) == INVALID  # NULL weight pointers


def test_user_ns_rows_validation(lib):
    # n_ns_user: range check, a larger cache, and the user tokens given exactly when > 0
    cfg = l_cfg()
    base = lib.onetrans_kv_cache_bytes(ctypes.byref(cfg), 2)
    cfg.n_ns_user = cfg.n_ns + 1
    assert lib.onetrans_check_config(ctypes.byref(cfg)) == UNSUPPORTED
    cfg.n_ns_user = -1
    assert lib.onetrans_check_config(ctypes.byref(cfg)) == UNSUPPORTED
    cfg.n_ns_user = 8
    assert lib.onetrans_check_config(ctypes.byref(cfg)) == OK
    d = cfg.d_model
    grown = lib.onetrans_kv_cache_bytes(ctypes.byref(cfg), 2)
    assert grown >= base + 2 * 8 * d * 2 * (2 * cfg.n_layers + 1)
    F = 1 << 41
    big = 1 << 40
    c = _cache(lib, cfg)
    assert lib.onetrans_user_prefill(ctypes.byref(cfg), F, F, F, 1, None, ctypes.byref(c), F, None, F, big, None) == INVALID
    assert lib.onetrans_user_prefill(ctypes.byref(cfg), F, F, F, 1, F + 8, ctypes.byref(c), F, None, F, big, None) == INVALID
    assert lib.onetrans_block_forward(ctypes.byref(cfg), F, F, F, 1, None, F, 4, F, F, F, big, None) == INVALID
    cfg0 = l_cfg()
    c0 = _cache(lib, cfg0)
    assert lib.onetrans_user_prefill(ctypes.byref(cfg0), F, F, F, 1, F, ctypes.byref(c0), F, None, F, big, None) == INVALID
    # all NS positions user-side: a candidate has no rows, scoring does nothing
    cfg.n_ns_user = cfg.n_ns
    c1 = _cache(lib, cfg)
    assert lib.onetrans_score_candidates(ctypes.byref(cfg), F, ctypes.byref(c1), 0, F, 8, F, F, big, None) == OK


def test_cache_layout_key_gates_other_user_side_shapes(lib):
    # a stage config that differs only in its NS side (n_ns, weight type) may use the
    # cache; one that differs in the user-side shape is rejected before any device work
    F = 1 << 41
    big = 1 << 40
    cfg = l_cfg()
    c = _cache(lib, cfg)
    stage = l_cfg()
    stage.n_ns = 8
    stage.ns_wdtype = C.W_FP8_E4M3
    assert lib.onetrans_score_candidates(ctypes.byref(stage), F, ctypes.byref(c), 0, F, 0, F, F, big, None) == OK
    for field, value in (("s_len", 1499), ("append_cap", 63), ("n_ns_user", 1), ("n_heads", 12)):
        other = l_cfg()
        setattr(other, field, value)
        if field == "s_len":
            other.q_sched[0] = 1499
        assert lib.onetrans_check_config(ctypes.byref(other)) == OK
        assert lib.onetrans_score_candidates(ctypes.byref(other), F, ctypes.byref(c), 0, F, 0, F, F, big, None) == INVALID
        assert lib.onetrans_kv_append(ctypes.byref(other), F, F, 1, ctypes.byref(c), F, F, big, None) == INVALID
        assert lib.onetrans_user_prefill(ctypes.byref(other), F, F, F, 1, F if other.n_ns_user else None,
                                         ctypes.byref(c), F, None, F, big, None) == INVALID
    other = l_cfg()
    other.q_sched[3] -= 1
    assert lib.onetrans_kv_cache_read(ctypes.byref(other), ctypes.byref(c), 0, 0, 1, F, F, None) == INVALID


def test_status_strings(lib):
    for code in range(6):
        assert lib.onetrans_status_str(code).decode()
    assert lib.onetrans_status_str(99).decode() == "unknown status"


def test_noalloc_scoring_rejects_before_any_device_work(lib):
    # the allocation-free scoring call: the same checks as scoring, and a clear error when
    # the call needs more than the static scratch holds (no launch, no device query)
    cfg = l_cfg()
    F = 1 << 41
    c = _cache(lib, cfg)
    f = lib.onetrans_score_candidates_noalloc
    assert f(ctypes.byref(cfg), F, ctypes.byref(c), 0, F, 0, F, None) == OK          # nothing to do
    assert f(ctypes.byref(cfg), F, ctypes.byref(c), 1, F, 8, F, None) == INVALID     # user not prefilled
    assert f(ctypes.byref(cfg), F, ctypes.byref(c), 0, F + 2, 8, F, None) == INVALID
    assert f(ctypes.byref(cfg), None, ctypes.byref(c), 0, F, 8, F, None) == INVALID
    need = lib.onetrans_workspace_bytes(ctypes.byref(cfg), 0, 4096, 0)
    assert need > 64 << 20
    assert f(ctypes.byref(cfg), F, ctypes.byref(c), 0, F, 4096, F, None) == WORKSPACE
    msg = lib.onetrans_last_error().decode()
    assert "scratch" in msg and str(64 << 20) in msg
    assert lib.onetrans_workspace_bytes(ctypes.byref(cfg), 0, 256, 0) <= 64 << 20  # the L shape's C = 256 fits
