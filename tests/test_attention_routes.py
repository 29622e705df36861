"""Which attention kernel instance each launch takes (host dispatch logic, no GPU).

The library compiles sixteen attention instances; the dispatch picks one from the
query count per (segment, head), the head count and the number of segments. These
tests pin that the GPU parity workloads together reach every compiled instance, so
no instance is left unexercised by the element-wise comparisons against the oracle.
"""
import os

import pytest

from unified_transformer_recommender_onetrans_amd import _capi as C

ALL_ROUTES = {
    "attn_ns2_kernel<64,2>", "attn_ns2_kernel<64,1>", "attn_ns2_kernel<32,2>", "attn_ns2_kernel<32,1>",
    "attn_split_kernel<64,5,true,ns>", "attn_split_kernel<32,4,true,ns>", "attn_split_kernel<64,5,false,ns>",
    "attn_split_kernel<32,4,false,ns>",
    "attn_split_kernel<64,5,true>", "attn_split_kernel<32,4,true>", "attn_split_kernel<64,5,false>",
    "attn_split_kernel<32,4,false>", "attn_kernel<64,4>", "attn_kernel<32,4>", "attn_kernel<64,2>",
    "attn_kernel<32,2>",
}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(C.LIB_PATH):
        from unified_transformer_recommender_onetrans_amd.build import build
        build()
    return C.lib()


def route(lib, ns, dh, nq, H, n_seg):
    return lib.onetrans_attention_route(int(ns), dh, nq, H, n_seg).decode()


def prefill_routes(lib, wl, B):
    return [route(lib, False, wl.head_dim, q, wl.n_heads, B) for q in wl.q_sched]


def test_dispatch_thresholds(lib):
    # 32 queries per block; S: < 1024 blocks split the keys, >= 2048 four blocks share a
    # workgroup, in between two; NS: >= 1024 blocks two query blocks per workgroup
    assert route(lib, False, 64, 32 * 511, 2, 1) == "attn_split_kernel<64,5,false>"
    assert route(lib, False, 64, 32 * 256, 2, 2) == "attn_kernel<64,2>"
    assert route(lib, False, 64, 32 * 1023, 2, 1) == "attn_kernel<64,2>"
    assert route(lib, False, 64, 32 * 1024, 2, 1) == "attn_kernel<64,4>"
    assert route(lib, False, 32, 32 * 100, 2, 3) == "attn_split_kernel<32,4,true>"
    # several users with 2-4 query blocks each (appends): the tile kernel, two blocks a workgroup
    assert route(lib, False, 64, 64, 6, 64) == "attn_kernel<64,2>"
    assert route(lib, False, 64, 128, 6, 8) == "attn_kernel<64,2>"
    assert route(lib, False, 64, 129, 6, 8) == "attn_split_kernel<64,5,true>"
    assert route(lib, False, 32, 32, 6, 64) == "attn_split_kernel<32,4,true>"
    assert route(lib, True, 64, 32 * 511, 2, 1) == "attn_ns2_kernel<64,1>"
    # NS with at most 256 query blocks: keys split over five (four) waves per block
    assert route(lib, True, 64, 32 * 128, 2, 1) == "attn_split_kernel<64,5,false,ns>"
    assert route(lib, True, 64, 32 * 129, 2, 1) == "attn_ns2_kernel<64,1>"
    assert route(lib, True, 64, 8, 6, 42) == "attn_split_kernel<64,5,true,ns>"
    assert route(lib, True, 32, 5, 2, 3) == "attn_split_kernel<32,4,true,ns>"
    assert route(lib, True, 32, 32 * 512, 2, 1) == "attn_ns2_kernel<32,2>"
    assert route(lib, False, 48, 32, 2, 1) == "none"
    assert route(lib, False, 64, 0, 2, 1) == "none"


def test_gpu_parity_workloads_reach_every_instance(lib):
    import test_gpu_parity as G
    from onetrans_inputs import CANDIDATE_HEAVY_FP8, ONETRANS_L, ONETRANS_S, PREFILL_BATCH
    reached = set()
    # small cases: block_forward / prefill of all users, scoring of one user's candidates,
    # appends of 13 and 6 events (test_prefill_append_score_match_oracle)
    for wl, lens in G.SMALL.values():
        B = len(lens)
        reached.update(prefill_routes(lib, wl, B))
        reached.add(route(lib, True, wl.head_dim, wl.n_candidates * wl.n_ns, wl.n_heads, 1))
        for m in (13, 6):
            reached.add(route(lib, False, wl.head_dim, m, wl.n_heads, B))
    # user-side NS passes (one segment per user) and their candidates
    for wl, lens, Pu in G.USER_NS.values():
        reached.add(route(lib, True, wl.head_dim, Pu, wl.n_heads, len(lens)))
        reached.add(route(lib, True, wl.head_dim, wl.n_candidates * (wl.n_ns - Pu), wl.n_heads, 1))
    # many-user prefills (test_many_user_prefill_tile_kernels)
    for wl in G.MANY_USERS.values():
        reached.update(prefill_routes(lib, wl, wl.n_users))
    # full-size workloads
    for wl in (ONETRANS_S, ONETRANS_L, CANDIDATE_HEAVY_FP8):
        reached.update(prefill_routes(lib, wl, 1))
        reached.add(route(lib, True, wl.head_dim, wl.n_candidates * wl.n_ns, wl.n_heads, 1))
    reached.update(prefill_routes(lib, PREFILL_BATCH, PREFILL_BATCH.n_users))
    assert reached >= ALL_ROUTES, sorted(ALL_ROUTES - reached)


def test_many_user_workloads_reach_the_tile_instances(lib):
    import test_gpu_parity as G
    got = {name: prefill_routes(lib, wl, wl.n_users) for name, wl in G.MANY_USERS.items()}
    assert got["i_dh32_16users"] == ["attn_kernel<32,4>", "attn_kernel<32,2>"]
    assert got["j_dh64_12users"][0] == "attn_kernel<64,2>"
