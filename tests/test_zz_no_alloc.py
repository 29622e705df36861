"""The allocation-free scoring entry point (static per-GPU scratch) against the workspace
entry point, through the C ABI: two calls in a row, the second with fewer candidates, each
equal bit for bit to onetrans_score_candidates on the same inputs (the same kernels run on
the same data, so the outputs must not differ at all)."""
import numpy as np
import pytest

from onetrans_inputs import ONETRANS_L, make_ns_tokens, make_s_tokens
from helpers import bf16_dev, model

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def test_noalloc_scoring_equals_workspace_scoring():
    wl = ONETRANS_L
    print(f"workload {wl.name}: noalloc scoring C=256 then C=37", flush=True)
    mdl, _ = model(wl)
    s, lens = make_s_tokens(wl)
    ns = make_ns_tokens(wl)
    cache = mdl.new_cache(1)
    mdl.user_prefill(bf16_dev(s), torch.from_numpy(lens).cuda(), cache)
    nd = bf16_dev(ns[0])
    for C in (256, 37):
        tok = nd[:C].contiguous()
        ref = mdl.score_candidates(cache, 0, tok)
        out = torch.full_like(ref, float("nan"))
        got = mdl.score_candidates_noalloc(cache, 0, tok, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.isfinite(got).all()
        assert torch.equal(got, ref), f"C={C}: max diff {(got - ref).abs().max().item():.3e}"
    # a request beyond the static scratch fails on the host with a clear error
    from unified_transformer_recommender_onetrans_amd import OneTransError
    big = bf16_dev(make_ns_tokens(wl, n_candidates=4096)[0])
    with pytest.raises(OneTransError, match="scratch"):
        mdl.score_candidates_noalloc(cache, 0, big)
