"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Index sets and indexer scores must match bit for bit (integer-valued indexer
data makes every score exact in fp32); attention outputs must be within
max-abs 2e-2 and mean-abs 2e-3 of the oracle (plus a 1e-2 relative-norm
check). Small shapes are checked on every query; the full-size workloads on
sampled queries that include the edge positions."""
import math
import os

import numpy as np
import pytest
import torch

import long_context_indexer_block_amd as H
import oracle.hisa_oracle as O
from long_context_indexer_block_amd.pipeline import (AutoPipeline, DecodeSession, FlatPipeline,
                                                     HierPipeline, HilsDecode, HilsPrefill)
from parity import (SeqOracle, check_attention, check_index_rows, check_score_rows, f64, log)
from workloads import WORKLOADS, Workload, make_inputs, sample_positions

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _mk(name, **kw):
    base = dict(kind="prefill", batch=1, L=2048, B=64, m=8, k=128, d_idx=64, Hq=1, Hkv=1, Dk=128,
                Dv=128)
    base.update(kw)
    return Workload(name, **base)


SMALL = [
    WORKLOADS["prefill_2k_tiny"],
    _mk("ragged_mqa", batch=2, L=1000, B=128, m=4, k=100, d_idx=128, Hq=16, Hkv=1),
    _mk("m2_padded", L=700, B=64, m=2, k=600, d_idx=64, Hq=4, Hkv=4, Dk=64, Dv=64),
    _mk("b256_gqa", L=1536, B=256, m=3, k=300, d_idx=64, Hq=8, Hkv=2, Dk=64, Dv=64),
    _mk("suffix_nq", L=1024, nq=200, B=64, m=5, k=96, d_idx=128, Hq=2, Hkv=1),
    _mk("mla_small", L=1024, B=128, m=4, k=256, d_idx=128, Hq=64, Hkv=1, Dk=576, Dv=512, mla=True,
        sigma=1.0 / 24.0),
    _mk("mla_unit", L=640, B=64, m=3, k=160, d_idx=64, Hq=64, Hkv=1, Dk=576, Dv=512, mla=True,
        sigma=1.0),
    # two sequences and 13 queries each (not a multiple of the 8 XCDs the
    # latent kernel deals its queries to)
    _mk("mla_batch2", batch=2, L=900, nq=13, B=64, m=4, k=200, d_idx=64, Hq=64, Hkv=1, Dk=576,
        Dv=512, mla=True, sigma=1.0 / 24.0),
    _mk("k1_decode", kind="decode", batch=3, L=3000, B=128, m=6, k=1, d_idx=128, Hq=16, Hkv=1),
    # an odd k (ids written one by one), and more than 8192 candidates per
    # query (the block-parallel select instead of the row-parallel one)
    _mk("odd_k", L=1500, B=128, m=5, k=77, d_idx=64, Hq=2, Hkv=1),
    _mk("wide_10240", L=12288, nq=48, B=256, m=40, k=500, d_idx=64, Hq=1, Hkv=1),
    # 3 x 4687 blocks: the bucket-count scan runs over four chunks of keys,
    # the last one ragged
    _mk("many_blocks_decode", kind="decode", batch=3, L=299963, B=64, m=8, k=256, d_idx=64, Hq=4,
        Hkv=1),
]


def _rows(w, n_sample=None):
    nq = w.queries
    if n_sample is None or n_sample >= nq:
        return list(range(nq))
    pos0 = w.L - nq
    ps = [p for p in sample_positions(w, n_sample) if p >= pos0]
    return sorted({p - pos0 for p in ps})


def _run_hier(w, inp):
    p = HierPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.B,
                     w.m, w.k, w.scale, want_scores=True, want_lse=True)
    p.run()
    torch.cuda.synchronize()
    return p


def _check_hier(w, inp, p, rows, attn_rows=None, what=""):
    attn_rows = rows if attn_rows is None else attn_rows
    bs = p.block_scores.cpu().numpy()
    bi = p.block_idx.cpu().numpy()
    ti = p.token_idx.cpu().numpy()
    ts = p.token_scores.cpu().numpy()
    out = p.out
    for b in range(w.batch):
        so = SeqOracle(inp, b, w.B)
        rb, rs, rt, rv = [], [], [], []
        for r in rows:
            bidx, bsc, tidx, tval = so.hier(r, w.m, w.k)
            rb.append(bidx), rs.append(bsc), rt.append(tidx), rv.append(tval)
        check_score_rows(bs[b, rows], np.stack(rs), f"{what} block scores b={b}")
        check_index_rows(bi[b, rows], np.stack(rb), f"{what} block_idx b={b}")
        check_index_rows(ti[b, rows], np.stack(rt), f"{what} token_idx b={b}")
        check_score_rows(ts[b, rows], np.stack(rv), f"{what} token scores b={b}")
        if attn_rows:
            go = out[b, attn_rows].float().cpu().numpy()
            ro = np.stack([so.attend(r, rt[rows.index(r)], w.scale)[0] for r in attn_rows])
            mx, mean, rel = check_attention(go, ro, f"{what} attention b={b}")
            log(f"  {what} b={b}: attention max-abs {mx:.2e} mean-abs {mean:.2e} rel {rel:.2e}")


# ------------------------------------------------------------------ pieces
@pytest.mark.parametrize("L,B,d,proj", [(2048, 64, 64, False), (1000, 128, 128, False),
                                        (777, 256, 64, True)])
def test_block_summary_exact(L, B, d, proj):
    log(f"case block_summary L={L} B={B} d={d} proj={proj}")
    g = torch.Generator(device=DEV).manual_seed(1)
    kidx = torch.randint(-8, 9, (2, L, d), generator=g, device=DEV).to(torch.bfloat16)
    W = torch.randint(-1, 2, (d, d), generator=g, device=DEV).to(torch.bfloat16) if proj else None
    summ, split = H.hisa_block_summary(kidx, B, proj=W)
    torch.cuda.synchronize()
    for b in range(2):
        ref = O.block_summary(f64(kidx[b]), B, None if W is None else f64(W))
        full = L // B
        # complete blocks: the mean of integers over a power-of-two count is exact
        check_score_rows(summ[b, :full].cpu().numpy(), ref[:full], "summary")
        if full < ref.shape[0]:   # partial last block: one division by its row count
            np.testing.assert_allclose(summ[b, full:].cpu().numpy(), ref[full:], rtol=2e-7, atol=1e-5)
        tot = f64(split[b]).sum(axis=1)       # hi + mid + lo, exact in fp64
        cnt = np.array([min(L, (c + 1) * B) - c * B for c in range(ref.shape[0])])
        # integer-valued keys (and projection): every row sum is an integer
        np.testing.assert_array_equal(tot, np.rint(ref * cnt[:, None]))


@pytest.mark.parametrize("nq", [24, 512], ids=["few_queries", "many_queries"])
@pytest.mark.parametrize("n_rows,m", [(40, 8), (130, 12), (1026, 64), (5000, 40), (16384, 32),
                                      (3000, 70)])
def test_select_blocks_ties(n_rows, m, nq):
    # integer scores from a narrow range (many ties at the threshold, +0.0 and
    # -0.0 among them). Few queries take the workgroup histogram select (16
    # waves with the lane-maximum bound beyond 4098 blocks when at most 32 are
    # free: the (16384, 32) case); from 1024 queries on, one wave per query up
    # to 1024 candidates, 16 waves and a union of their kept candidates beyond
    # (the histogram select when the union would not fit). Exact sets against
    # the oracle.
    B = 64
    log(f"case select_blocks n_rows={n_rows} m={m} nq={nq}")
    g = torch.Generator(device="cpu").manual_seed(n_rows * 131 + m)
    sc = torch.randint(-5, 6, (2, nq, n_rows), generator=g).float()
    neg0 = (sc == 0) & (torch.rand(sc.shape, generator=g) < 0.5)
    sc = torch.where(neg0, torch.tensor(-0.0), sc)
    pos = torch.randint(0, n_rows * B, (2, nq), generator=g, dtype=torch.int32)
    pos[:, 0] = n_rows * B - 1          # the most candidates
    pos[:, 1] = 0                       # block 0 only
    pos[:, 2] = B * (m - 1)             # exactly enough blocks for all of them
    pos[:, 3] = B * m                   # one candidate too many
    out = H.hisa_select_blocks(sc.to(DEV), pos.to(DEV), B, m).cpu().numpy()
    rows = list(range(nq)) if nq <= 64 else list(range(8)) + list(range(8, nq, 13))
    for b in range(2):
        ref = np.stack([O.select_blocks_for_query(sc[b, i].double().numpy(), int(pos[b, i]), B, m)
                        for i in rows])
        check_index_rows(out[b, rows], ref, f"select_blocks b={b}")


@pytest.mark.parametrize("n_rows,m", [(4099, 20), (6000, 34), (16384, 32), (16384, 35)])
def test_select_blocks_few_spread(n_rows, m):
    # few queries, spread scores: beyond 4098 blocks with at most 32 free
    # slots each of 16 waves keeps its best through the lane-maximum bound
    # (survivors compacted in LDS), wave 0 the best of their union; m = 35
    # is the first to take the histogram select again. Exact sets.
    B = 64
    log(f"case select_blocks_few_spread n_rows={n_rows} m={m}")
    g = torch.Generator(device="cpu").manual_seed(n_rows * 7 + m)
    nq = 6
    sc = torch.randn(3, nq, n_rows, generator=g)
    pos = torch.randint(0, n_rows * B, (3, nq), generator=g, dtype=torch.int32)
    pos[:, 0] = n_rows * B - 1
    pos[:, 1] = B * (m - 1)
    pos[:, 2] = B * m
    pos[:, 3] = B * (n_rows // 2) + 5
    out = H.hisa_select_blocks(sc.to(DEV), pos.to(DEV), B, m).cpu().numpy()
    for b in range(3):
        ref = np.stack([O.select_blocks_for_query(sc[b, i].double().numpy(), int(pos[b, i]), B, m)
                        for i in range(nq)])
        check_index_rows(out[b], ref, f"select_blocks_few_spread b={b}")


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_hier_pipeline_small(w):
    log(f"case hier {w}")
    inp = make_inputs(w, DEV, seed=3)
    p = _run_hier(w, inp)
    _check_hier(w, inp, p, _rows(w), what=w.name)


@pytest.mark.parametrize("w", SMALL[:5], ids=[w.name for w in SMALL[:5]])
def test_flat_small(w):
    log(f"case flat {w}")
    inp = make_inputs(w, DEV, seed=4)
    f = FlatPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.k,
                     w.scale, want_scores=True)
    f.run()
    torch.cuda.synchronize()
    ti, ts = f.token_idx.cpu().numpy(), f.token_scores.cpu().numpy()
    rows = _rows(w)
    for b in range(w.batch):
        so = SeqOracle(inp, b, w.B, with_attention=False)
        ref = [so.flat(r, w.k) for r in rows]
        check_index_rows(ti[b, rows], np.stack([x[0] for x in ref]), f"{w.name} flat idx")
        check_score_rows(ts[b, rows], np.stack([x[1] for x in ref]), f"{w.name} flat scores")


def test_coverage_hier_equals_flat_gpu():
    # every query with t < m*B keeps all its blocks, so both indexers agree
    w = _mk("coverage", L=4096, B=128, m=32, k=256, d_idx=128)
    log(f"case coverage {w}")
    inp = make_inputs(w, DEV, seed=5)
    p = _run_hier(w, inp)
    f = FlatPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.k,
                     w.scale)
    f.run()
    torch.cuda.synchronize()
    assert torch.equal(p.token_idx, f.token_idx)
    assert torch.equal(p.out, f.out)


def test_token_select_bucketed_many_keys():
    # enough pairs that they are bucketed by key block (over 256 MB of direct
    # reads) and more than 4096 key blocks, so the bucket-count scan runs over
    # several chunks of keys with a ragged last one: 2 x 2100 blocks of 64
    w = _mk("bucketed_4200_keys", batch=2, L=2100 * 64 - 5, nq=512, B=64, m=40, k=300, d_idx=64,
            Hq=1, Hkv=1)
    assert w.batch * w.queries * w.m * w.B * w.d_idx * 2 > 256 << 20
    assert w.batch * w.n_blocks > 4096
    log(f"case {w}")
    inp = make_inputs(w, DEV, seed=13)
    p = _run_hier(w, inp)
    rows = list(range(0, 512, 61)) + [510, 511]
    _check_hier(w, inp, p, rows, attn_rows=rows[-2:], what=w.name)


@pytest.mark.parametrize("B,m", [(128, 128), (64, 256)])
def test_token_select_16k_candidates(B, m):
    # m*B = 16384 candidates per query (up to 256 slots) and enough queries
    # for the 8-wave row select; sampled rows against the oracle
    w = _mk(f"cand16k_B{B}_m{m}", L=20480, nq=1024, B=B, m=m, k=3000, d_idx=64, Hq=1, Hkv=1)
    log(f"case {w}")
    inp = make_inputs(w, DEV, seed=9)
    p = _run_hier(w, inp)
    rows = list(range(0, 1024, 97)) + [1022, 1023]
    _check_hier(w, inp, p, rows, attn_rows=rows[-3:], what=w.name)


@pytest.mark.parametrize("cluster", ["spread", "three_values", "near_k", "spread_few", "near_n"])
def test_token_select_wide_range_scores(cluster):
    # token scores crafted to defeat the value-range histogram: the query is
    # the unit vector e0, so a token's score is its key's first element. Six
    # tokens hold +-2^100, +-2^66, +-2^33 and all others lie in [-1, 1], so
    # each of the three histogram levels finds the K-th largest value in one
    # bin holding nearly every candidate and the exact bisection on order
    # keys decides; every block is kept (m*B covers the prefix), 1024 queries
    # take the 32-row, 4-wave select over 8192 candidates
    # (near_k: no outliers, the queries at positions 1536..2559, so around t =
    # k the K-th largest value is among the smallest, in the histogram's
    # lowest bins, where the masked tokens of the query's own block and the
    # empty slots are counted too)
    # (spread_few: 64 queries, the 16-wave form of the select; near_n: k just
    # below the candidate count, so the K-th largest value lies in the
    # lowest bin together with the masked tokens of the query's own block,
    # and the bin's copy finds fewer candidates than the histogram counted)
    L = 2560 if cluster == "near_k" else 8192
    nq = 64 if cluster == "spread_few" else 1024
    k = 8162 if cluster == "near_n" else 2048
    w = _mk(f"wide_range_{cluster}", L=L, nq=nq, B=128, m=64, k=k, d_idx=64, Hq=1, Hkv=1)
    log(f"case {w}")
    inp = make_inputs(w, DEV, seed=21)
    g = torch.Generator().manual_seed(22)
    # values on a grid of 1/64; block 0 holds the outliers, whose fp32 block
    # mean depends on the summation order, so block scores are not compared
    # here (every block is kept either way); token ids and scores are exact
    if cluster == "three_values":
        vals = torch.tensor([-0.5, 0.25, 0.75])[torch.randint(0, 3, (w.L,), generator=g)]
    else:
        vals = torch.randint(-64, 65, (w.L,), generator=g).float() / 64.0
    if cluster not in ("near_k", "near_n"):
        for j, x in zip((5, 6, 7, 8, 9, 10), (2.0 ** 100, -(2.0 ** 100), 2.0 ** 66, -(2.0 ** 66),
                                              2.0 ** 33, -(2.0 ** 33))):
            vals[j] = x
    kidx = torch.zeros(w.batch, w.L, w.d_idx)
    kidx[:, :, 0] = vals
    qidx = torch.zeros(w.batch, w.queries, w.d_idx)
    qidx[:, :, 0] = 1.0
    inp["kidx"].copy_(kidx.to(torch.bfloat16))
    inp["qidx"].copy_(qidx.to(torch.bfloat16))
    p = _run_hier(w, inp)
    if cluster == "near_k":
        rows = [t - (L - 1024) for t in (1600, 2046, 2047, 2048, 2049, 2050, 2100, 2175, 2176,
                                         2559)]
    elif cluster == "near_n":
        rows = [t - (L - 1024) for t in (8000, 8160, 8161, 8162, 8163, 8170, 8191)]
    else:
        rows = sorted(set(range(0, nq, nq // 8 - 1)) | {nq - 1})
    so = SeqOracle(inp, 0, w.B, with_attention=False)
    ref = [so.hier(r, w.m, w.k) for r in rows]
    check_index_rows(p.block_idx[0, rows].cpu().numpy(), np.stack([x[0] for x in ref]),
                     f"{w.name} block_idx")
    check_index_rows(p.token_idx[0, rows].cpu().numpy(), np.stack([x[2] for x in ref]),
                     f"{w.name} token_idx")
    check_score_rows(p.token_scores[0, rows].cpu().numpy(), np.stack([x[3] for x in ref]),
                     f"{w.name} token scores")


@pytest.mark.parametrize("L,hier", [(4096, False), (12288, True)])
def test_auto_pipeline(L, hier):
    # the runtime policy: the flat indexer below 8192 keys, else the
    # hierarchical one with m = max(64, L // 2000) = 64 here
    w = _mk("auto", L=L, nq=96, B=128, m=64, k=256, d_idx=64, Hq=2, Hkv=1)
    log(f"case auto {w}")
    inp = make_inputs(w, DEV, seed=8)
    a = AutoPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.B,
                     w.k, w.scale, want_scores=True)
    assert a.hierarchical == hier and a.m == 64
    a.run()
    if hier:
        r = HierPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.B,
                         64, w.k, w.scale)
    else:
        r = FlatPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.k,
                         w.scale)
    r.run()
    torch.cuda.synchronize()
    assert torch.equal(a.token_idx, r.token_idx) and torch.equal(a.out, r.out)
    so = SeqOracle(inp, 0, w.B, with_attention=False)
    rows = [0, 47, 95]
    ti = a.token_idx.cpu().numpy()
    ref = [so.hier(x, 64, w.k)[2] if hier else so.flat(x, w.k)[0] for x in rows]
    check_index_rows(ti[0, rows], np.stack(ref), "auto token_idx")


def test_decode_session_grows_like_a_rebuild():
    # caches with room to grow: each grow() recomputes only the summary rows
    # of the blocks the new tokens fall in; every step must equal a pipeline
    # built from scratch at that length (same kernels: bit-exact)
    w = _mk("grow", kind="decode", batch=3, L=1000, B=64, m=4, k=100, d_idx=64, Hq=4, Hkv=1)
    log(f"case decode session {w}")
    inp = make_inputs(w, DEV, seed=10)
    kidx, k, v, q, qidx = inp["kidx"], inp["k"], inp["v"], inp["q"], inp["qidx"]
    s = DecodeSession(kidx, k, v, 700, w.Hq, w.B, w.m, w.k, w.scale)
    for L in (700, 701, 703, 704, 705, 735, 768, 769, 1000):
        if L != s.L:
            s.grow(L)
        s.step(q, qidx)
        pos = torch.full((w.batch, 1), L - 1, dtype=torch.int32, device=DEV)
        r = HierPipeline(kidx[:, :L], qidx, pos, q, k[:, :L], v[:, :L], w.B, w.m, w.k, w.scale)
        r.run()
        torch.cuda.synchronize()
        n = -(-L // w.B)
        assert torch.equal(s.split[:, :n], r.split), L
        assert torch.equal(s.block_idx, r.block_idx) and torch.equal(s.token_idx, r.token_idx), L
        assert torch.equal(s.out, r.out), L
        # and against the oracle on the cache cut to L tokens
        for b in range(w.batch):
            kb = f64(kidx[b, :L])
            bidx, _, tidx, _ = O.hier_query(f64(qidx[b, 0]), kb, O.block_summary(kb, w.B), L - 1,
                                            w.B, w.m, w.k)
            check_index_rows(s.block_idx[b].cpu().numpy(), bidx[None], f"session block_idx L={L}")
            check_index_rows(s.token_idx[b].cpu().numpy(), tidx[None], f"session token_idx L={L}")
            ro, _ = O.sparse_attention_for_query(f64(q[b, 0]), f64(k[b, :L]), f64(v[b, :L]), tidx,
                                                 w.scale)
            check_attention(s.out[b, 0].float().cpu().numpy(), ro, f"session attention L={L} b={b}")
    # the incrementally built rows against the oracle (integer keys: exact)
    for b in range(w.batch):
        ref = O.block_summary(f64(kidx[b]), w.B)
        cnt = np.array([min(1000, (c + 1) * w.B) - c * w.B for c in range(ref.shape[0])])
        np.testing.assert_array_equal(f64(s.split[b]).sum(axis=1), np.rint(ref * cnt[:, None]))


def test_decode_graph_replays_match_eager():
    # the decode step as a HIP graph; each replay (with eager work and a
    # synchronisation in between) must equal the eager step on the same queries
    w = _mk("graph", kind="decode", batch=4, L=6000, B=128, m=8, k=512, d_idx=128, Hq=16, Hkv=1)
    log(f"case decode graph {w}")
    inp = make_inputs(w, DEV, seed=11)
    s = DecodeSession(inp["kidx"], inp["k"], inp["v"], w.L, w.Hq, w.B, w.m, w.k, w.scale)
    q, qidx = inp["q"].clone(), inp["qidx"].clone()
    g = s.capture(q, qidx)
    gen = torch.Generator(device=DEV).manual_seed(12)
    for rep in range(4):
        q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(torch.bfloat16))
        qidx.copy_(torch.randint(-8, 9, qidx.shape, generator=gen, device=DEV).to(torch.bfloat16))
        g.replay()
        torch.cuda.synchronize()
        got_idx, got_out = s.token_idx.clone(), s.out.clone()
        s.step(q, qidx)  # eager, on the same queries
        torch.cuda.synchronize()
        assert torch.equal(got_idx, s.token_idx), rep
        assert torch.equal(got_out, s.out), rep


@pytest.mark.parametrize("shape", ["direct", "bucketed"])
def test_prefill_step_graph_replays_match_eager(shape):
    # the prefill step as one HIP graph (the calls the benchmark captures):
    # each replay, on fresh queries, with eager work and a synchronisation in
    # between, must equal the eager step on the same queries. "direct" scores
    # pairs straight from block_idx, "bucketed" buckets them by key block
    # (its tables cleared by fill kernels inside the graph).
    if shape == "direct":
        w = _mk("pgraph_direct", L=2048, B=64, m=8, k=128, d_idx=64, Hq=2, Hkv=1)
    else:
        w = _mk("pgraph_bucketed", L=8192, nq=1024, B=128, m=64, k=512, d_idx=64, Hq=2, Hkv=1)
    log(f"case prefill graph {w}")
    inp = make_inputs(w, DEV, seed=13)
    p = HierPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.B,
                     w.m, w.k, w.scale)
    calls = [
        p.summarize,
        lambda: H.hisa_block_score(p.qidx, p.q_pos, p.split, p.B, out=p.block_scores),
        lambda: H.hisa_select_blocks(p.block_scores, p.q_pos, p.B, p.m, out=p.block_idx),
        lambda: H.hisa_token_select(p.qidx, p.kidx, p.q_pos, p.block_idx, p.B, p.k_top,
                                    token_idx=p.token_idx, want_scores=False, workspace=p.ws),
        p.attend,
    ]
    for c in calls:  # warm-up outside the capture
        c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    gen = torch.Generator(device=DEV).manual_seed(14)
    for rep in range(3):
        p.qidx.copy_(torch.randint(-8, 9, p.qidx.shape, generator=gen, device=DEV)
                     .to(torch.bfloat16))
        p.q.copy_(torch.randn(p.q.shape, generator=gen, device=DEV).to(torch.bfloat16))
        g.replay()
        torch.cuda.synchronize()
        got = (p.block_idx.clone(), p.token_idx.clone(), p.out.clone())
        for c in calls:  # eager, on the same queries
            c()
        torch.cuda.synchronize()
        assert torch.equal(got[0], p.block_idx), rep
        assert torch.equal(got[1], p.token_idx), rep
        assert torch.equal(got[2], p.out), rep


def test_hils_decode_graph_replays_match_eager():
    # routing and two-level attention of the two-level decode as one HIP
    # graph, as the benchmark times it; every replay equals the eager step
    w = WORKLOADS["hils_decode_1m"].with_(name="hgraph", batch=2, L=9000, m=16, Hq=4, Hkv=4)
    log(f"case hils decode graph {w}")
    inp = make_inputs(w, DEV, seed=15)
    sc = 1.0 / math.sqrt(w.Dk)
    hd = HilsDecode(inp["q"], inp["k"], inp["v"], inp["w_proj"], w.B, w.m, sc, sc)
    hd.run(build=True)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        hd.route()
        hd.attend()
    gen = torch.Generator(device=DEV).manual_seed(16)
    for rep in range(3):
        hd.q.copy_(torch.randn(hd.q.shape, generator=gen, device=DEV).to(torch.bfloat16))
        g.replay()
        torch.cuda.synchronize()
        got_idx, got_out = hd.chunk_idx.clone(), hd.out.clone()
        hd.route()
        hd.attend()
        torch.cuda.synchronize()
        assert torch.equal(got_idx, hd.chunk_idx), rep
        assert torch.equal(got_out, hd.out), rep


def test_determinism_and_decode_matches_prefill_row():
    w = _mk("det", L=3072, B=128, m=6, k=200, d_idx=128, Hq=16, Hkv=1)
    log(f"case determinism {w}")
    inp = make_inputs(w, DEV, seed=6)
    p1 = _run_hier(w, inp)
    t1, o1 = p1.token_idx.clone(), p1.out.clone()
    p1.run()
    torch.cuda.synchronize()
    assert torch.equal(t1, p1.token_idx) and torch.equal(o1, p1.out)
    # decode at t = L-1 on the same cache equals prefill row L-1
    d = HierPipeline(inp["kidx"], inp["qidx"][:, -1:].contiguous(), inp["q_pos"][:, -1:].contiguous(),
                     inp["q"][:, -1:].contiguous(), inp["k"], inp["v"], w.B, w.m, w.k, w.scale)
    d.run()
    torch.cuda.synchronize()
    assert torch.equal(d.token_idx[:, 0], t1[:, -1])
    # one query splits its token list over several waves (another fp32
    # summation order); without the workspace it runs like a prefill row
    assert d.attn_ws is not None
    check_attention(d.out[:, 0].float().cpu().numpy(), o1[:, -1].float().cpu().numpy(),
                    "decode split vs prefill row")
    d.attn_ws = None
    d.attend()
    torch.cuda.synchronize()
    assert torch.equal(d.out[:, 0], o1[:, -1])


# ------------------------------------------------------------------ workloads
def test_workload_prefill_16k_mqa():
    w = WORKLOADS["prefill_16k_mqa"]
    log(f"case {w.name}")
    inp = make_inputs(w, DEV, seed=0)
    p = _run_hier(w, inp)
    rows = _rows(w, 40)
    _check_hier(w, inp, p, rows, what=w.name)
    # the step as the benchmark times it at this size: 4 query slabs, the
    # selection on one stream, the slabs' attention alternating on two; the
    # same block and token ids, and the same output bits (this attention's
    # summation order does not depend on the schedule)
    o = HierPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.B,
                     w.m, w.k, w.scale, overlap_slabs=4)
    assert len(o.slabs) == 4
    o.run_overlapped()
    o.run_overlapped()
    torch.cuda.synchronize()
    assert torch.equal(o.block_idx, p.block_idx) and torch.equal(o.token_idx, p.token_idx)
    assert torch.equal(o.out, p.out)


def _rows_64k(w, slabs, n_total=4096, seed=0):
    """Rows of the 64K check: every slab boundary (last row of a slab, first
    of the next), the edge positions, the first and last two rows, and
    seeded random rows up to n_total."""
    nq = w.queries
    sl = -(-nq // slabs)
    rows = set()
    for s0 in range(sl, nq, sl):
        rows.update((s0 - 1, s0))
    rows.update(p for p in sample_positions(w, 0) if p < nq)
    rows.update((0, 1, nq - 2, nq - 1))
    g = np.random.default_rng(seed)
    while len(rows) < n_total:
        rows.add(int(g.integers(0, nq)))
    return sorted(rows)


def _attn_rows_64k(w, slabs):
    """Attention rows: slab boundaries, edges and seeded rows, 64 or more."""
    nq = w.queries
    sl = -(-nq // slabs)
    rows = {0, 1, 127, 128, 2047, 2048, 8191, 8192, nq - 1}
    rows.update(s0 for s0 in range(sl, nq, sl))
    rows.update(s0 - 1 for s0 in range(sl, nq, sl))
    g = np.random.default_rng(1)
    while len(rows) < 72:
        rows.add(int(g.integers(0, nq)))
    return sorted(rows)


@pytest.fixture(scope="module")
def inputs_64k():
    w = WORKLOADS["prefill_64k_mla"]
    inp = make_inputs(w, DEV, seed=0)
    torch.cuda.synchronize()
    yield w, inp
    del inp
    torch.cuda.empty_cache()


def test_workload_prefill_64k_mla_timed_step(inputs_64k):
    # the step exactly as the benchmark times it: 16 query slabs, the block
    # scores, block and token selection of slab i+1 on one stream while slab
    # i attends on another (HierPipeline.run_overlapped, no scores, no LSE);
    # block scores, block ids and token ids against the oracle bit for bit on
    # 4096 rows (every slab boundary, the edges), attention on 72 rows
    import oracle_pool as OP
    w, inp = inputs_64k
    slabs = 16
    log(f"case {w.name} timed step, {slabs} overlapped slabs")
    p = HierPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.B,
                     w.m, w.k, w.scale, overlap_slabs=slabs)
    assert len(p.slabs) == slabs
    p.run_overlapped()
    p.run_overlapped()
    torch.cuda.synchronize()
    rows = _rows_64k(w, slabs)
    arows = _attn_rows_64k(w, slabs)
    ridx = torch.tensor(rows, device=DEV)
    bs = p.block_scores[0, ridx].cpu().numpy()
    bi = p.block_idx[0, ridx].cpu().numpy()
    ti_all = p.token_idx.clone()
    out_all = p.out.clone()
    ti = ti_all[0, ridx].cpu().numpy()
    aidx = torch.tensor(arows, device=DEV)
    go = out_all[0, aidx].float().cpu().numpy()
    # the one-stream step on the same buffers gives the same ids; the outputs
    # agree up to the fp32 summation order (the latent kernel sums a query's
    # tiles starting from a clock-chosen tile), and bit for bit in list order
    p.run()
    torch.cuda.synchronize()
    assert torch.equal(p.token_idx, ti_all)
    check_attention(p.out[0, aidx].float().cpu().numpy(), go, "64k one-stream vs overlapped")
    os.environ["HISA_MLA_ROT_TICKS"] = "0"
    try:
        p.run_overlapped()
        torch.cuda.synchronize()
        o_list = p.out.clone()
        p.run()
        torch.cuda.synchronize()
        assert torch.equal(p.out, o_list)
        check_attention(o_list[0, aidx].float().cpu().numpy(), go, "64k list order vs rotated")
    finally:
        del os.environ["HISA_MLA_ROT_TICKS"]
    kidx = inp["kidx"][0].float().cpu().numpy()
    qidx = inp["qidx"][0].float().cpu().numpy()
    pos = inp["q_pos"][0].cpu().numpy()
    log(f"  oracle on {len(rows)} rows, {OP.workers()} workers")
    ref = OP.hier_rows(kidx, qidx, pos, w.B, w.m, w.k, rows)
    check_score_rows(bs, np.stack([ref[r][1] for r in rows]), "64k timed block scores")
    check_index_rows(bi, np.stack([ref[r][0] for r in rows]), "64k timed block_idx")
    check_index_rows(ti, np.stack([ref[r][2] for r in rows]), "64k timed token_idx")
    # attention rows on the oracle's own token lists
    K = inp["k"][0].float().cpu().numpy()
    V = inp["v"][0].float().cpu().numpy()
    qa = inp["q"][0, aidx].float().cpu().numpy()
    jobs = [(r, qa[i], ref[r][2] if r in ref else None) for i, r in enumerate(arows)]
    missing = [r for r in arows if r not in ref]
    if missing:
        extra = OP.hier_rows(kidx, qidx, pos, w.B, w.m, w.k, missing)
        jobs = [(r, q, t if t is not None else extra[r][2]) for r, q, t in jobs]
    log(f"  oracle attention on {len(arows)} rows")
    att = OP.attend_rows(K, V, w.scale, jobs)
    mx, mean, rel = check_attention(go, np.stack([att[r][0] for r in arows]), "64k timed attention")
    log(f"  64k timed step: attention max-abs {mx:.2e} mean-abs {mean:.2e} rel {rel:.2e}")


def test_workload_prefill_64k_mla_scores(inputs_64k):
    # the same overlapped step asked for its token scores: scores bit for bit
    # on the same 4096 rows
    import oracle_pool as OP
    w, inp = inputs_64k
    log(f"case {w.name} overlapped step with token scores")
    p = HierPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.B,
                     w.m, w.k, w.scale, want_scores=True, overlap_slabs=16)
    p.run_overlapped()
    torch.cuda.synchronize()
    rows = _rows_64k(w, 16)
    ridx = torch.tensor(rows, device=DEV)
    ti = p.token_idx[0, ridx].cpu().numpy()
    ts = p.token_scores[0, ridx].cpu().numpy()
    del p
    torch.cuda.empty_cache()
    ref = OP.hier_rows(inp["kidx"][0].float().cpu().numpy(), inp["qidx"][0].float().cpu().numpy(),
                       inp["q_pos"][0].cpu().numpy(), w.B, w.m, w.k, rows)
    check_index_rows(ti, np.stack([ref[r][2] for r in rows]), "64k token_idx (scores run)")
    check_score_rows(ts, np.stack([ref[r][3] for r in rows]), "64k token scores")


def test_workload_prefill_64k_flat(inputs_64k):
    # the flat comparison path as the benchmark runs it (16 overlapped
    # slabs), ids and scores on the same 4096 rows
    import oracle_pool as OP
    w, inp = inputs_64k
    log(f"case {w.name} flat path, overlapped slabs")
    f = FlatPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.k,
                     w.scale, want_scores=True, overlap_slabs=16)
    f.run_overlapped()
    torch.cuda.synchronize()
    rows = _rows_64k(w, 16)
    ridx = torch.tensor(rows, device=DEV)
    ti = f.token_idx[0, ridx].cpu().numpy()
    ts = f.token_scores[0, ridx].cpu().numpy()
    del f
    torch.cuda.empty_cache()
    log(f"  flat oracle on {len(rows)} rows, {OP.workers()} workers")
    ref = OP.flat_rows(inp["kidx"][0].float().cpu().numpy(), inp["qidx"][0].float().cpu().numpy(),
                       inp["q_pos"][0].cpu().numpy(), w.k, rows)
    check_index_rows(ti, np.stack([ref[r][0] for r in rows]), "flat 64k token_idx")
    check_score_rows(ts, np.stack([ref[r][1] for r in rows]), "flat 64k scores")


def test_workload_decode_128k_b64():
    w = WORKLOADS["decode_128k_b64"]
    log(f"case {w.name}")
    inp = make_inputs(w, DEV, seed=0)
    p = _run_hier(w, inp)
    bi, ti, ts = (p.block_idx.cpu().numpy(), p.token_idx.cpu().numpy(),
                  p.token_scores.cpu().numpy())
    for b in range(w.batch):
        so = SeqOracle(inp, b, w.B)
        bidx, _, tidx, tval = so.hier(0, w.m, w.k)
        check_index_rows(bi[b, :1], bidx[None], f"decode block_idx b={b}")
        check_index_rows(ti[b, :1], tidx[None], f"decode token_idx b={b}")
        check_score_rows(ts[b, :1], tval[None], f"decode token scores b={b}")
        ro, _ = so.attend(0, tidx, w.scale)
        check_attention(p.out[b, 0].float().cpu().numpy(), ro, f"decode attention b={b}")


def _hils_check(w, exact, split=True, scales=None):
    inp = make_inputs(w, DEV, seed=0)
    C, m = w.B, w.m
    sc = 1.0 / math.sqrt(w.Dk)
    s_chunk, s_token = (sc, sc) if scales is None else scales
    hd = HilsDecode(inp["q"], inp["k"], inp["v"], inp["w_proj"], C, m, s_chunk, s_token)
    # few (sequence, head) pairs: the chunks are spread over workgroups and
    # merged, unless the workspace is withheld
    assert hd.ws is not None
    if not split:
        hd.ws = None
    hd.run(build=True)
    torch.cuda.synchronize()
    t = w.L - 1
    Wp = f64(inp["w_proj"])
    got_idx = hd.chunk_idx.view(w.batch, w.Hq, m).cpu().numpy()
    outs = hd.out.float().cpu().numpy()
    excluded = 0
    for b in range(w.batch):
        for h in range(w.Hq):
            K = f64(inp["k"][b, :, h])
            V = f64(inp["v"][b, :, h])
            q = f64(inp["q"][b, h])
            khat = O.block_summary(K, C, proj=Wp)
            ref_out, ref_idx = O.hils_decode_head(q, K, V, khat, t, C, m, s_chunk, s_token)
            if exact:
                check_index_rows(got_idx[b, h:h + 1], ref_idx[None],
                                 f"hils int chunk_idx b={b} h={h}")
                # complete chunks: a mean over a power-of-two count, exact; a
                # partial last chunk: one division by its token count
                full = w.L // C
                gk = hd.khat[b * w.Hq + h].cpu().numpy()
                check_score_rows(gk[:full], khat[:full], f"hils int khat b={b} h={h}")
                if full < khat.shape[0]:
                    np.testing.assert_allclose(gk[full:], khat[full:], rtol=2e-7, atol=1e-5)
            elif not np.array_equal(got_idx[b, h], ref_idx):
                # N(0,1) chunk scores are not exact in fp32: accept a different
                # set only when the oracle's last kept and first dropped free
                # scores are closer than an fp32 error bound of the two dot
                # products.
                raw = khat @ q
                bt = t // C
                cand = np.arange(1, bt)
                order = cand[np.lexsort((cand, -raw[cand]))]
                gap = raw[order[m - 3]] - raw[order[m - 2]]
                bound = 4 * 2.0 ** -24 * w.Dk * 2 * np.abs(khat[order[m - 3:m - 1]] * q).sum()
                assert gap <= bound, f"hils b={b} h={h}: chunk sets differ with gap {gap} > {bound}"
                excluded += 1
                # the output is still checked: the oracle's two-level combine
                # over the chunk set the GPU chose
                gi = got_idx[b, h]
                logits = [s_chunk * float(khat[c] @ q) if c >= 0 else 0.0 for c in gi]
                ref_out = O.hils_combine(q, K, V, gi, logits, t, C, s_token)
            check_attention(outs[b, h:h + 1], ref_out[None], f"hils out b={b} h={h}")
    log(f"  hils exact={exact}: heads excluded as near-ties: {excluded}")
    return excluded


# small two-level decodes in the integer twin (exact routing): head width 128,
# chunks of 128 and 256 tokens (several 64-token groups each), a partial local
# chunk, m = 64 (four chunks per wave), two sequences
HILS_SMALL = [
    WORKLOADS["hils_decode_1m"].with_(name="hils_d128_c128", batch=2, L=5000, B=128, m=8, Hq=4,
                                      Hkv=4, Dk=128, Dv=128, d_idx=128, int_mode=True),
    WORKLOADS["hils_decode_1m"].with_(name="hils_c256", batch=1, L=3000, B=256, m=6, Hq=3, Hkv=3,
                                      int_mode=True),
    WORKLOADS["hils_decode_1m"].with_(name="hils_c64_m64", batch=2, L=4100, B=64, m=64, Hq=2,
                                      Hkv=2, int_mode=True),
]


@pytest.mark.parametrize("split", [True, False], ids=["split", "one_workgroup_per_pair"])
@pytest.mark.parametrize("w", HILS_SMALL, ids=[w.name for w in HILS_SMALL])
def test_hils_small(w, split):
    log(f"case hils small {w} split={split}")
    assert _hils_check(w, exact=True, split=split) == 0


@pytest.mark.parametrize("split", [True, False], ids=["split", "one_workgroup_per_pair"])
def test_hils_unequal_scales(split):
    # chunk-logit and token-logit scales that differ (0.5 and 0.125): a kernel
    # that dropped or swapped either would leave the tolerance
    w = HILS_SMALL[0]
    log(f"case hils unequal scales {w} split={split}")
    assert _hils_check(w, exact=True, split=split, scales=(0.5, 0.125)) == 0


def test_workload_hils_decode_int_twin():
    w = WORKLOADS["hils_decode_1m"].with_(int_mode=True)
    log(f"case hils int twin {w}")
    assert _hils_check(w, exact=True) == 0


def test_workload_hils_decode_1m():
    w = WORKLOADS["hils_decode_1m"]
    log(f"case hils N(0,1) {w}")
    assert _hils_check(w, exact=False) <= 2


# ---------------------------------------------------------------- two-level prefill
def _hils_prefill_check(w, exact, positions=None, heads=None, bucketed=True, subset=False,
                        slab=65536, scales=None):
    """Run the causal two-level prefill of workload w on the GPU and check the
    queries at `positions` (default: all) of `heads` (default: all) against
    the oracle's decode of the tokens up to each query. bucketed=False runs
    the per-query kernel (no workspace); subset=True runs the GPU on the
    queries at `positions` only (the full cache, a sample of its queries)."""
    inp = make_inputs(w, DEV, seed=0)
    C, m, nq = w.B, w.m, w.queries
    sc = 1.0 / math.sqrt(w.Dk)
    s_chunk, s_token = (sc, sc) if scales is None else scales
    first = w.L - nq
    rows = list(range(nq)) if positions is None else [t - first for t in positions]
    ridx = torch.tensor(rows, dtype=torch.long, device=DEV)
    q_in, pos_in = inp["q"], inp["q_pos"]
    if subset:
        q_in, pos_in = q_in[:, ridx].contiguous(), pos_in[:, ridx].contiguous()
    hp = HilsPrefill(q_in, inp["k"], inp["v"], inp["w_proj"], pos_in, C, m, s_chunk, s_token,
                     slab=slab)
    assert hp.ws is not None
    if not bucketed:
        hp.ws = None
    hp.run()
    torch.cuda.synchronize()
    Wp = f64(inp["w_proj"])
    qpos = inp["q_pos"].cpu().numpy()
    gidx = ridx if not subset else torch.arange(len(rows), device=DEV)
    got_idx = hp.chunk_ids().view(w.batch, w.Hq, q_in.shape[1], m)[:, :, gidx].cpu().numpy()
    outs = hp.out[:, gidx].float().cpu().numpy()      # [b, rows, H, D]
    qs = inp["q"][:, ridx].cpu()
    excluded = 0
    for b in range(w.batch):
        for h in (range(w.Hq) if heads is None else heads):
            K = f64(inp["k"][b, :, h])
            V = f64(inp["v"][b, :, h])
            khat = O.block_summary(K, C, proj=Wp)
            keep, refs = [], []
            for r, i in enumerate(rows):
                t = int(qpos[b, i])
                q = f64(qs[b, r, h])
                ref_out, ref_idx = O.hils_prefill_query(q, K, V, Wp, khat, t, C, m, s_chunk,
                                                        s_token)
                if not np.array_equal(got_idx[b, h, r], ref_idx):
                    assert not exact, (f"hils prefill chunk_idx b={b} h={h} t={t}: gpu "
                                       f"{got_idx[b, h, r].tolist()} ref {ref_idx.tolist()}")
                    # N(0,1) chunk scores: a different set is accepted only at a
                    # near tie of the last kept and first dropped free chunk
                    raw = khat @ q
                    bt = t // C
                    cand = np.arange(1, bt)
                    order = cand[np.lexsort((cand, -raw[cand]))]
                    gap = raw[order[m - 3]] - raw[order[m - 2]]
                    bound = 4 * 2.0 ** -24 * w.Dk * 2 * np.abs(khat[order[m - 3:m - 1]] * q).sum()
                    assert gap <= bound, f"b={b} h={h} t={t}: chunk sets differ, gap {gap}"
                    excluded += 1
                    # the output is still checked: the oracle's two-level
                    # combine over the chunk set the GPU chose (the local
                    # chunk keyed by its tokens up to t)
                    kl = Wp @ K[bt * C: t + 1].mean(axis=0)
                    gi = got_idx[b, h, r]
                    logits = [0.0 if c < 0 else
                              s_chunk * float((kl if c == bt else khat[c]) @ q) for c in gi]
                    ref_out = O.hils_combine(q, K, V, gi, logits, t, C, s_token)
                keep.append(r)
                refs.append(ref_out)
            if keep:
                check_attention(outs[b, keep, h], np.stack(refs), f"hils prefill out b={b} h={h}")
    log(f"  hils prefill exact={exact}: queries excluded as near-ties: {excluded}")
    return excluded


# every position of small causal prefills in the integer twin (exact
# routing): queries inside the first chunk (only chunk 0), across chunk
# boundaries, a partial last chunk, head width 128, chunks of 128 and 256
# tokens (several 64-token groups per chunk), m = 64, two sequences
HILS_PREFILL_SMALL = [
    WORKLOADS["hils_prefill_64k"].with_(name="hilsp_c64", batch=2, L=700, m=8, Hq=3, Hkv=3,
                                        int_mode=True),
    WORKLOADS["hils_prefill_64k"].with_(name="hilsp_d128_c128", batch=1, L=1500, B=128, m=6,
                                        Hq=2, Hkv=2, Dk=128, Dv=128, d_idx=128, nq=700,
                                        int_mode=True),
    WORKLOADS["hils_prefill_64k"].with_(name="hilsp_c256", batch=2, L=2100, B=256, m=4, Hq=2,
                                        Hkv=2, nq=900, int_mode=True),
    WORKLOADS["hils_prefill_64k"].with_(name="hilsp_c64_m64", batch=1, L=4480, m=64, Hq=1,
                                        Hkv=1, nq=400, int_mode=True),
    WORKLOADS["hils_prefill_64k"].with_(name="hilsp_d128_c256", batch=1, L=3000, B=256, m=5,
                                        Hq=2, Hkv=2, Dk=128, Dv=128, d_idx=128, nq=600,
                                        int_mode=True),
]


@pytest.mark.parametrize("bucketed", [True, False], ids=["bucketed", "per_query"])
@pytest.mark.parametrize("w", HILS_PREFILL_SMALL, ids=[w.name for w in HILS_PREFILL_SMALL])
def test_hils_prefill_small(w, bucketed):
    log(f"case hils prefill small {w} bucketed={bucketed}")
    assert _hils_prefill_check(w, exact=True, bucketed=bucketed) == 0


@pytest.mark.parametrize("bucketed", [True, False], ids=["bucketed", "per_query"])
def test_hils_prefill_unequal_scales(bucketed):
    # chunk-logit scale 0.5, token-logit scale 0.125 on every position
    w = HILS_PREFILL_SMALL[0]
    log(f"case hils prefill unequal scales {w} bucketed={bucketed}")
    assert _hils_prefill_check(w, exact=True, bucketed=bucketed, scales=(0.5, 0.125)) == 0


def test_hils_prefill_slabs():
    # queries in ragged slabs of 256 (700 = 256 + 256 + 188)
    w = HILS_PREFILL_SMALL[0]
    log(f"case hils prefill in slabs {w}")
    assert _hils_prefill_check(w, exact=True, slab=256) == 0


def test_hils_prefill_streamed_routing():
    # more chunks than the fused routing keeps on chip (1094 > 1026): the
    # streamed selection; a sample of the queries runs
    w = WORKLOADS["hils_prefill_64k"].with_(name="hilsp_1094", L=70000, Hq=2, Hkv=2,
                                            int_mode=True)
    log(f"case hils prefill, streamed routing {w}")
    assert _hils_prefill_check(w, exact=True, positions=sample_positions(w, 40), subset=True) == 0


def test_hils_prefill_streamed_routing_d128():
    # head width 128 through the streamed routing (1172 chunks of 64)
    w = WORKLOADS["hils_prefill_64k"].with_(name="hilsp_d128_1172", L=75000, Hq=2, Hkv=2,
                                            Dk=128, Dv=128, d_idx=128, m=16, int_mode=True)
    log(f"case hils prefill, streamed routing, width 128 {w}")
    assert _hils_prefill_check(w, exact=True, positions=sample_positions(w, 32), subset=True) == 0


def test_hils_prefill_overlapped_equals_sequential():
    # routing of the next slab on another stream: the same chunk ids and outputs
    w = HILS_PREFILL_SMALL[0]
    inp = make_inputs(w, DEV, seed=2)
    sc = 1.0 / math.sqrt(w.Dk)
    a = HilsPrefill(inp["q"], inp["k"], inp["v"], inp["w_proj"], inp["q_pos"], w.B, w.m, sc, sc,
                    slab=256)
    a.run()
    ref_idx, ref_out = a.chunk_ids().clone(), a.out.clone()
    for _ in range(2):
        a.run_overlapped()
    torch.cuda.synchronize()
    assert torch.equal(a.chunk_ids(), ref_idx)
    assert torch.equal(a.out, ref_out)


def test_hils_prefill_no_projection():
    # plain-mean chunk keys (proj None) on both paths
    w = HILS_PREFILL_SMALL[0]
    inp = make_inputs(w, DEV, seed=1)
    sc = 1.0 / math.sqrt(w.Dk)
    hp = HilsPrefill(inp["q"], inp["k"], inp["v"], None, inp["q_pos"], w.B, w.m, sc, sc)
    out_b = hp.run().clone()
    hp.ws = None
    out_q = hp.run()
    torch.cuda.synchronize()
    I = np.eye(w.Dk)
    for b in range(w.batch):
        for h in range(w.Hq):
            K = f64(inp["k"][b, :, h])
            V = f64(inp["v"][b, :, h])
            khat = O.block_summary(K, w.B)
            refs = np.stack([O.hils_prefill_query(f64(inp["q"][b, i, h]), K, V, I, khat, i, w.B,
                                                  w.m, sc, sc)[0] for i in range(w.L)])
            for o, nm in ((out_b, "bucketed"), (out_q, "per query")):
                check_attention(o[b, :, h].float().cpu().numpy(), refs,
                                f"no-proj {nm} b={b} h={h}")


def test_hils_prefill_matches_decode_at_last_position():
    # the last query of a prefill is the decode at L-1 over the same cache
    w = HILS_PREFILL_SMALL[0]
    inp = make_inputs(w, DEV, seed=0)
    sc = 1.0 / math.sqrt(w.Dk)
    hp = HilsPrefill(inp["q"], inp["k"], inp["v"], inp["w_proj"], inp["q_pos"], w.B, w.m, sc, sc)
    hp.run()
    q_last = inp["q"][:, -1].contiguous()
    hd = HilsDecode(q_last, inp["k"], inp["v"], inp["w_proj"], w.B, w.m, sc, sc)
    hd.ws = None
    hd.run(build=True)
    torch.cuda.synchronize()
    assert torch.equal(hp.chunk_ids()[:, -1], hd.chunk_idx.view(-1, w.m))
    check_attention(hp.out[:, -1].float().cpu().numpy(), hd.out.float().cpu().numpy(),
                    "prefill last query vs decode")


def test_workload_hils_prefill_64k_int_twin_sampled():
    w = WORKLOADS["hils_prefill_64k"].with_(int_mode=True)
    log(f"case hils prefill 64K int twin, sampled {w}")
    assert _hils_prefill_check(w, exact=True, positions=sample_positions(w, 24),
                               heads=[0, 7, 15]) == 0


def test_workload_hils_prefill_512k_sampled():
    # the 512K cache (8192 chunks) with a sample of its queries
    w = WORKLOADS["hils_prefill_512k"]
    log(f"case hils prefill 512K N(0,1), sampled {w}")
    assert _hils_prefill_check(w, exact=False, positions=sample_positions(w, 24),
                               heads=[0, 9, 15], subset=True) <= 3


def test_workload_hils_prefill_64k_sampled():
    w = WORKLOADS["hils_prefill_64k"]
    log(f"case hils prefill 64K N(0,1), sampled {w}")
    assert _hils_prefill_check(w, exact=False, positions=sample_positions(w, 24),
                               heads=[0, 5, 10, 15]) <= 4


# ---------------------------------------------------------------- fused routing
# (batch, nq, L, B, d, m, positions, value range): one case per item count of
# the selection (n_rows up to 66, 130, 258, 514, 1026), queries not a multiple
# of the 16-query tile, queries in the first block, m above the candidate
# count, and small integer values so that many scores tie
ROUTE_CASES = [
    (2, 100, 3000, 64, 64, 8, "random", 8),
    (1, 333, 9000, 64, 128, 16, "random", 2),
    (3, 50, 20000, 64, 64, 32, "random", 1),
    (1, 200, 32768, 64, 64, 40, "last", 8),
    (1, 1000, 65536, 64, 64, 32, "prefill", 1),
    (1, 77, 65600, 64, 64, 64, "random", 8),
    (2, 40, 4096, 256, 64, 4, "random", 1),
    # streamed selection (more than 1026 blocks): ragged tiles, first-block
    # queries, heavy ties through the buffer cuts, K at its limit of 128
    (1, 300, 70000, 64, 64, 32, "random", 1),
    (2, 100, 262144, 64, 128, 64, "random", 8),
    (1, 64, 524288, 64, 64, 130, "random", 1),
    (1, 50, 300000, 128, 64, 8, "last", 8),
    (1, 2000, 140000, 64, 64, 16, "prefill", 8),
    # the two buffer sizes of the streamed selection at their boundary (more
    # than 3072 blocks: K = 64 takes 32 queries and 128 entries, K = 65 16
    # queries and 256)
    (1, 200, 200000, 64, 64, 66, "random", 1),
    (1, 200, 200000, 64, 64, 67, "random", 1),
    (1, 100, 196700, 64, 64, 32, "random", 8),
    # scores held on chip (m above the streamed selection's limit of 130)
    (1, 300, 65600, 64, 64, 200, "random", 1),
    (2, 100, 40000, 128, 128, 140, "prefill", 8),
    # one query per sequence (decode): with the workspace the blocks of each
    # query are split over workgroups in parts of 256 and merged; a 1M-token
    # cache in 64-token chunks (16384 blocks, 64 parts, 1920 survivors), mass
    # ties, one free slot, queries with fewer candidates than slots
    (16, 1, 131072, 128, 128, 64, "last", 8),
    (4, 1, 1048576, 64, 64, 32, "last", 8),
    (8, 1, 65536, 64, 64, 64, "random", 1),
    (8, 1, 65536, 64, 64, 3, "random", 1),
    (32, 1, 16384, 128, 64, 40, "random", 8),
]


@pytest.mark.parametrize("split", [True, False], ids=["workspace", "no_workspace"])
@pytest.mark.parametrize("case", ROUTE_CASES, ids=[f"n{c[2] // c[3]}_q{c[1]}" for c in ROUTE_CASES])
def test_route_blocks_equals_score_then_select(case, split):
    b, nq, L, B, d, m, kind, vr = case
    log(f"case fused route {case} workspace={split}")
    g = torch.Generator(device=DEV).manual_seed(7)
    kidx = torch.randint(-vr, vr + 1, (b, L, d), generator=g, device=DEV).to(torch.bfloat16)
    qidx = torch.randint(-vr, vr + 1, (b, nq, d), generator=g, device=DEV).to(torch.bfloat16)
    if kind == "random":
        q_pos = torch.randint(0, L, (b, nq), generator=g, device=DEV, dtype=torch.int32)
    elif kind == "last":
        q_pos = torch.full((b, nq), L - 1, dtype=torch.int32, device=DEV)
    else:
        q_pos = torch.arange(L - nq, L, dtype=torch.int32, device=DEV).expand(b, nq).contiguous()
    edges = torch.tensor([0, B - 1, B], dtype=torch.int32, device=DEV)
    if nq >= 3:
        q_pos[:, :3] = edges
    elif b >= 8:
        q_pos[:3, 0] = edges  # the first block's queries, one per sequence
    _, split_t = H.hisa_block_summary(kidx, B)
    ref = H.hisa_select_blocks(H.hisa_block_score(qidx, q_pos, split_t, B), q_pos, B, m)
    got = H.hisa_route_blocks(qidx, q_pos, split_t, B, m, workspace="auto" if split else None)
    torch.cuda.synchronize()
    check_index_rows(got.view(-1, m).cpu().numpy(), ref.view(-1, m).cpu().numpy(), "fused route")


def test_flat_overlapped_equals_sequential():
    # slabs of 683 queries: enough (query, head) items that the attention
    # never splits its lists, so the results match bit for bit
    w = WORKLOADS["prefill_2k_tiny"]
    inp = make_inputs(w, DEV, seed=4)
    a = FlatPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.k,
                     w.scale, want_lse=True)
    b = FlatPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.k,
                     w.scale, want_lse=True, overlap_slabs=3)
    a.run()
    for _ in range(2):
        b.run_overlapped()
    torch.cuda.synchronize()
    assert torch.equal(a.token_idx, b.token_idx)
    assert torch.equal(a.out, b.out)
    assert torch.equal(a.lse, b.lse)


def test_overlapped_step_equals_sequential():
    # query slabs (ragged: 2048 = 683 + 683 + 682) with the block scores,
    # block and token selection of the next slab on another stream: the same
    # block ids, ids, scores, outputs, LSE
    w = WORKLOADS["prefill_2k_tiny"]
    inp = make_inputs(w, DEV, seed=3)
    kw = dict(want_scores=True, want_lse=True)
    a = HierPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.B,
                     w.m, w.k, w.scale, **kw)
    b = HierPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.B,
                     w.m, w.k, w.scale, overlap_slabs=3, **kw)
    assert len(b.slabs) == 3
    a.run()
    for _ in range(2):
        b.run_overlapped()
    torch.cuda.synchronize()
    assert torch.equal(a.block_scores.view(torch.int32), b.block_scores.view(torch.int32))
    assert torch.equal(a.block_idx, b.block_idx)
    assert torch.equal(a.token_idx, b.token_idx)
    # bit patterns: the padding is NaN
    assert torch.equal(a.token_scores.view(torch.int32), b.token_scores.view(torch.int32))
    assert torch.equal(a.out, b.out)
    assert torch.equal(a.lse, b.lse)
