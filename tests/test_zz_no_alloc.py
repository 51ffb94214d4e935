"""The allocation-free token selection (hisa_token_select_noalloc) against the
workspace form (hisa_token_select) on the same inputs: token ids and scores
equal bit for bit, on two calls in a row, the second with a smaller input
(the shared scratch keeps the first call's contents)."""
import pytest
import torch

import long_context_indexer_block_amd as H
from parity import log
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(name, **kw):
    base = dict(kind="prefill", batch=1, L=2048, B=64, m=8, k=128, d_idx=64, Hq=1, Hkv=1, Dk=64,
                Dv=64)
    base.update(kw)
    return Workload(name, **base)


# the first call takes the bucketed path (many pairs), the second, smaller,
# scores its pairs in place (one query per sequence)
CASES = [
    _case("bucketed", L=8192, B=128, m=8, k=256, d_idx=128),
    _case("decode", kind="decode", batch=4, L=3000, B=64, m=6, k=100, d_idx=64),
]


def _blocks(w, inp):
    _, split = H.hisa_block_summary(inp["kidx"], w.B)
    return H.hisa_select_blocks(H.hisa_block_score(inp["qidx"], inp["q_pos"], split, w.B),
                                inp["q_pos"], w.B, w.m)


def test_noalloc_matches_workspace_form():
    for i, w in enumerate(CASES):
        log(f"case noalloc call {i}: {w}")
        inp = make_inputs(w, DEV, seed=20 + i)
        bidx = _blocks(w, inp)
        need = H.hisa_token_select_workspace_bytes(w.batch, w.queries, w.L, w.B, w.m, w.k)
        assert 0 < need <= H.NOALLOC_SCRATCH_BYTES
        ref_idx, ref_sc = H.hisa_token_select(inp["qidx"], inp["kidx"], inp["q_pos"], bidx, w.B,
                                              w.k)
        idx = torch.full_like(ref_idx, 7)
        sc = torch.full_like(ref_sc, 3.0)
        H.hisa_token_select_noalloc(inp["qidx"], inp["kidx"], inp["q_pos"], bidx, w.B, w.k, idx,
                                    sc)
        # ids only (no scores requested) as well
        idx2 = torch.full_like(ref_idx, 9)
        H.hisa_token_select_noalloc(inp["qidx"], inp["kidx"], inp["q_pos"], bidx, w.B, w.k, idx2)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), f"call {i}: token ids differ"
        assert torch.equal(sc.view(torch.int32), ref_sc.view(torch.int32)), f"call {i}: scores"
        assert torch.equal(idx2, ref_idx), f"call {i}: token ids (no scores) differ"


def test_noalloc_rejects_large_shapes():
    w = _case("large", L=16384, B=128, m=32, k=2048, d_idx=128)
    inp = make_inputs(w, DEV, seed=30)
    bidx = torch.zeros(1, w.queries, w.m, dtype=torch.int32, device=DEV)
    idx = torch.empty(1, w.queries, w.k, dtype=torch.int32, device=DEV)
    with pytest.raises(H.HisaError) as e:
        H.hisa_token_select_noalloc(inp["qidx"], inp["kidx"], inp["q_pos"], bidx, w.B, w.k, idx)
    assert e.value.status == 3 and "scratch" in str(e.value)
