"""Pins for the CPU oracle: each test checks it against something other than
itself — hand-worked values, brute-force enumeration, closed forms, the
textbook attention routine, or invariants the pages state."""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.hisa_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _none_to_inf(xs):
    return np.array([-np.inf if x is None else x for x in xs], dtype=np.float64)


# --------------------------------------------------------------- hand-worked
def test_golden_indexer():
    g = json.load(open(GOLD))["indexer"]
    kidx = np.array(g["kidx"], dtype=np.float64)
    B, m, k = g["B"], g["m"], g["k"]
    summ = O.block_summary(kidx, B)
    np.testing.assert_array_equal(summ, np.array(g["summary"], dtype=np.float64))
    for qq in g["queries"]:
        t, q = qq["t"], np.array(qq["q"], dtype=np.float64)
        bidx, bs, tidx, tval = O.hier_query(q, kidx, summ, t, B, m, k)
        np.testing.assert_array_equal(bs, _none_to_inf(qq["block_scores"]))
        assert bidx.tolist() == qq["block_idx"]
        assert tidx.tolist() == qq["token_idx"]
        exp_val = np.array([np.nan if v is None else v for v in qq["token_scores"]])
        np.testing.assert_array_equal(tval, exp_val)
        fidx, _ = O.flat_select_for_query(q, kidx, t, k)
        assert fidx.tolist() == qq["flat_token_idx"]


def test_golden_attention():
    g = json.load(open(GOLD))["attention"]
    out, lse = O.sparse_attention_for_query(np.array(g["q"]), np.array(g["K"]),
                                            np.array(g["V"]), g["idx"], g["scale"])
    np.testing.assert_allclose(out, np.array(g["out"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(g["lse"]), rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", ["hils", "hils_scaled"])
def test_golden_hils(case):
    # "hils_scaled" has unequal chunk and token scales (0.5 and 2), so the
    # chunk logit scale and the token logit scale are each pinned
    g = json.load(open(GOLD))[case]
    K = np.array(g["K"])
    khat = O.block_summary(K, g["C"], proj=np.array(g["W"]))
    out, chosen = O.hils_decode_head(np.array(g["q"]), K, np.array(g["V"]), khat, g["t"],
                                     g["C"], g["m"], g["scale_chunk"], g["scale_token"])
    assert chosen.tolist() == g["chosen"]
    np.testing.assert_allclose(out, np.array(g["out"]), rtol=0, atol=1e-12)


# --------------------------------------------------------------- summaries
def test_summary_closed_forms():
    L, B, d = 23, 4, 3
    kidx = np.zeros((L, d))
    kidx[:, 0] = np.arange(L)          # column 0 = token id
    kidx[:, 1] = 5.0                   # constant column
    kidx[:, 2] = np.arange(L) % B      # position inside the block
    s = O.block_summary(kidx, B)
    assert s.shape == (6, d)
    for c in range(6):
        lo, hi = c * B, min(L, (c + 1) * B)
        assert s[c, 0] == (lo + hi - 1) / 2.0
        assert s[c, 1] == 5.0
        assert s[c, 2] == (hi - lo - 1) / 2.0


def test_summary_projection_orientation():
    # W shifts coordinates: khat[i] = mean[i+1]; its transpose would shift the
    # other way, so this catches a transposed projection.
    d, B = 4, 2
    kidx = np.array([[1, 2, 3, 4], [3, 6, 9, 12]], dtype=np.float64)
    W = np.zeros((d, d))
    for i in range(d - 1):
        W[i, i + 1] = 1.0
    khat = O.block_summary(kidx, B, proj=W)
    np.testing.assert_array_equal(khat[0], [4.0, 6.0, 8.0, 0.0])


def test_block_scores_exact_rationals():
    rng = np.random.default_rng(1)
    L, B, d = 40, 8, 5
    kidx = rng.integers(-8, 9, (L, d))
    q = rng.integers(-8, 9, d)
    s = O.block_summary(kidx.astype(np.float64), B)
    for t in [0, 7, 8, 17, 39]:
        sc = O.block_scores_for_query(q.astype(np.float64), s, t, B)
        b = t // B
        for c in range(s.shape[0]):
            if c >= b:
                assert sc[c] == -np.inf
            else:
                exact = sum(Fraction(int(q[i]) * int(kidx[j, i]), B)
                            for j in range(c * B, (c + 1) * B) for i in range(d))
                assert Fraction(sc[c]) == exact


# --------------------------------------------------------------- brute force
def _brute_topk(values, ids, k):
    """The kept set is the subset whose keys (value, -id), sorted descending,
    are lexicographically largest; enumerate every subset of size min(k, n)."""
    n = len(ids)
    kk = min(k, n)
    best, best_key = None, None
    for sub in itertools.combinations(range(n), kk):
        key = sorted(((values[i] + 0.0, -ids[i]) for i in sub), reverse=True)
        if best_key is None or key > best_key:
            best, best_key = sub, key
    return sorted(ids[i] for i in best)


@pytest.mark.parametrize("seed", range(12))
def test_block_select_brute_force(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.choice([4, 8]))
    L = int(rng.integers(8, 97))
    m = int(rng.choice([2, 3, 4]))
    d = int(rng.choice([2, 4]))
    kidx = rng.integers(-2, 3, (L, d)).astype(np.float64)   # small range: many ties
    s = O.block_summary(kidx, B)
    for t in range(L):
        q = rng.integers(-2, 3, d).astype(np.float64)
        sc = O.block_scores_for_query(q, s, t, B)
        got = O.select_blocks_for_query(sc, t, B, m)
        b = t // B
        forced = [0] if b == 0 else [0, b]
        cand = list(range(1, b))
        free = m - len(forced)
        if len(cand) <= free:
            exp = list(range(b + 1))
        else:
            exp = sorted(forced + _brute_topk([sc[c] for c in cand], cand, free))
        assert [c for c in got.tolist() if c >= 0] == exp
        assert got.tolist()[len(exp):] == [-1] * (m - len(exp))
        assert 0 in got and b in got                     # forced blocks present


@pytest.mark.parametrize("seed", range(12))
def test_token_select_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.choice([2, 4]))
    L = int(rng.integers(4, 25))
    d = int(rng.choice([2, 4]))
    k = int(rng.integers(1, 7))
    kidx = rng.integers(-2, 3, (L, d)).astype(np.float64)
    for t in range(L):
        q = rng.integers(-2, 3, d).astype(np.float64)
        nb = t // B + 1
        kept = sorted(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False).tolist())
        bidx = np.array(kept + [-1], dtype=np.int64)
        got, val = O.token_select_for_query(q, kidx, bidx, t, B, k)
        cand = [j for c in kept for j in range(c * B, min((c + 1) * B, t + 1))]
        u = [float(kidx[j] @ q) for j in cand]
        exp = _brute_topk(u, cand, k)
        assert [j for j in got.tolist() if j >= 0] == exp
        for j, v in zip(got, val):
            if j >= 0:
                assert v == float(kidx[j] @ q)


# --------------------------------------------------------------- invariants
@pytest.mark.parametrize("seed", range(4))
def test_coverage_hier_equals_flat(seed):
    # When m*B covers the causal prefix every block is kept, and hierarchical
    # selection is the flat top-k (the method falls back to the original
    # indexer on short inputs).
    rng = np.random.default_rng(200 + seed)
    L, B, m, k, d = 96, 8, 5, 9, 4
    kidx = rng.integers(-8, 9, (L, d)).astype(np.float64)
    s = O.block_summary(kidx, B)
    for t in range(L):
        q = rng.integers(-8, 9, d).astype(np.float64)
        _, _, hidx, _ = O.hier_query(q, kidx, s, t, B, m, k)
        fidx, _ = O.flat_select_for_query(q, kidx, t, k)
        if t < m * B:
            assert hidx.tolist() == fidx.tolist()
    # m >= number of blocks: equal everywhere
    for t in range(L):
        q = rng.integers(-8, 9, d).astype(np.float64)
        _, _, hidx, _ = O.hier_query(q, kidx, s, t, B, L // B, k)
        fidx, _ = O.flat_select_for_query(q, kidx, t, k)
        assert hidx.tolist() == fidx.tolist()


def test_negative_zero_is_a_tie():
    vals = np.array([0.0, -0.0, 0.0])
    ids = np.array([5, 2, 9])
    idx, _ = O.topk_lowest_index(vals, ids, 2)
    assert idx.tolist() == [2, 5]


# --------------------------------------------------------------- attention
def _sdpa(q, K, V, idx, scale):
    """torch scaled-dot-product attention in float64 with a boolean mask."""
    Hq, Dk = q.shape
    L, Hkv, _ = K.shape
    g = Hq // Hkv
    Kx = torch.from_numpy(K).repeat_interleave(g, dim=1).permute(1, 0, 2)   # [Hq, L, Dk]
    Vx = torch.from_numpy(V).repeat_interleave(g, dim=1).permute(1, 0, 2)
    mask = torch.zeros(Hq, 1, L, dtype=torch.bool)
    for j in idx:
        if j >= 0:
            mask[:, :, j] = True
    qq = torch.from_numpy(q).unsqueeze(1)                                   # [Hq, 1, Dk]
    o = torch.nn.functional.scaled_dot_product_attention(qq, Kx, Vx, attn_mask=mask, scale=scale)
    return o[:, 0].numpy()


@pytest.mark.parametrize("Hq,Hkv,Dk,Dv", [(1, 1, 8, 8), (4, 2, 6, 5), (8, 1, 12, 10), (3, 3, 4, 4)])
def test_attention_vs_sdpa(Hq, Hkv, Dk, Dv):
    rng = np.random.default_rng(Hq * 100 + Dk)
    L = 37
    q = rng.standard_normal((Hq, Dk))
    K = rng.standard_normal((L, Hkv, Dk))
    V = rng.standard_normal((L, Hkv, Dv))
    idx = np.array(sorted(rng.choice(L, 11, replace=False).tolist()) + [-1, -1])
    out, lse = O.sparse_attention_for_query(q, K, V, idx, 0.3)
    np.testing.assert_allclose(out, _sdpa(q, K, V, idx, 0.3), rtol=1e-12, atol=1e-12)
    # log-sum-exp closed form for one head
    g = Hq // Hkv
    sel = idx[idx >= 0]
    s = 0.3 * (K[sel, 0 // g] @ q[0])
    assert abs(lse[0] - math.log(np.exp(s).sum())) < 1e-12


def test_attention_mla_alias():
    rng = np.random.default_rng(7)
    L, H, Dk, Dv = 20, 4, 9, 6
    kv = rng.standard_normal((L, 1, Dk))
    q = rng.standard_normal((H, Dk))
    idx = np.array([0, 3, 4, 19])
    out, _ = O.sparse_attention_for_query(q, kv, kv[..., :Dv], idx, 0.25)
    np.testing.assert_allclose(out, _sdpa(q, kv, np.ascontiguousarray(kv[..., :Dv]), idx, 0.25),
                               rtol=1e-12, atol=1e-12)


def test_dense_causal_reduction():
    # With k >= t+1 and every block kept, hierarchical sparse attention is
    # ordinary causal attention.
    rng = np.random.default_rng(11)
    L, B, d, H, D = 24, 4, 3, 2, 5
    kidx = rng.integers(-8, 9, (L, d)).astype(np.float64)
    qidx = rng.integers(-8, 9, (L, d)).astype(np.float64)
    q = rng.standard_normal((L, H, D))
    K = rng.standard_normal((L, 1, D))
    V = rng.standard_normal((L, 1, D))
    res = O.hier_pipeline(kidx, qidx, q, K, V, list(range(L)), list(range(L)), B, L // B, L, 0.5)
    qq = torch.from_numpy(q).permute(1, 0, 2)
    kk = torch.from_numpy(K).expand(L, H, D).permute(1, 0, 2)
    vv = torch.from_numpy(V).expand(L, H, D).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True, scale=0.5)
    np.testing.assert_allclose(res["out"], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_constant_values():
    rng = np.random.default_rng(3)
    L, H, D = 30, 4, 8
    K = rng.standard_normal((L, 1, D))
    V = np.tile(rng.standard_normal(D), (L, 1, 1)).reshape(L, 1, D)
    out, _ = O.sparse_attention_for_query(rng.standard_normal((H, D)), K, V,
                                          [1, 5, 9, 29, -1], 1.0)
    np.testing.assert_allclose(out, np.tile(V[0, 0], (H, 1)), rtol=0, atol=1e-12)


def test_empty_index_set():
    out, lse = O.sparse_attention_for_query(np.ones((2, 3)), np.ones((4, 1, 3)),
                                            np.ones((4, 1, 3)), [-1, -1], 1.0)
    assert (out == 0).all() and (lse == -np.inf).all()


# --------------------------------------------------------------- two-level
def test_hils_exact_chunk_mass():
    # With each chunk's logit set to the log of its exact attention mass
    # (log-sum-exp of its token scores), the two-level output is flat sparse
    # attention over the union of the chosen chunks.
    rng = np.random.default_rng(5)
    L, C, D = 64, 8, 6
    t = 61
    q = rng.standard_normal(D)
    K = rng.standard_normal((L, D))
    V = rng.standard_normal((L, D))
    chunks = [0, 2, 5, 7]
    sc = 0.4
    lse = []
    for c in chunks:
        j = np.arange(c * C, min((c + 1) * C, t + 1))
        s = sc * (K[j] @ q)
        lse.append(np.log(np.exp(s).sum()))
    two = O.hils_combine(q, K, V, chunks, lse, t, C, sc)
    union = [j for c in chunks for j in range(c * C, min((c + 1) * C, t + 1))]
    flat, _ = O.sparse_attention_for_query(q[None], K[:, None], V[:, None], union, sc)
    np.testing.assert_allclose(two, flat[0], rtol=1e-12, atol=1e-12)
    one = O.hils_combine(q, K, V, [2], [123.0], t, C, sc)
    intra, _ = O.sparse_attention_for_query(q[None], K[:, None], V[:, None],
                                            list(range(16, 24)), sc)
    np.testing.assert_allclose(one, intra[0], rtol=1e-12, atol=1e-12)


def test_hils_routing_forced_and_count():
    rng = np.random.default_rng(9)
    L, C, D, m = 200, 8, 4, 5
    K = rng.standard_normal((L, D))
    V = rng.standard_normal((L, D))
    W = rng.standard_normal((D, D))
    khat = O.block_summary(K, C, proj=W)
    for t in [0, 7, 8, 40, 199]:
        q = rng.standard_normal(D)
        _, chosen = O.hils_decode_head(q, K, V, khat, t, C, m, 0.5, 0.5)
        b = t // C
        kept = [c for c in chosen if c >= 0]
        assert 0 in kept and b in kept
        assert len(kept) == min(m, b + 1)
        # the free picks beat every dropped candidate
        free = [c for c in kept if c not in (0, b)]
        dropped = [c for c in range(1, b) if c not in kept]
        if free and dropped:
            assert min(khat[c] @ q for c in free) >= max(khat[c] @ q for c in dropped)


def test_hils_prefill_is_decode_of_the_prefix():
    # a prefill query at t equals the decode of the cache cut after t: its
    # chunk keys rebuilt from the first t+1 tokens, so the local chunk's key
    # covers only the tokens up to the query; tokens after t change nothing
    rng = np.random.default_rng(21)
    L, C, D, m = 300, 16, 8, 6
    K = rng.standard_normal((L, D))
    V = rng.standard_normal((L, D))
    W = rng.standard_normal((D, D)) / 3
    khat = O.block_summary(K, C, proj=W)
    for t in [0, 5, 15, 16, 17, 100, 159, 160, 299]:
        q = rng.standard_normal(D)
        out, chosen = O.hils_prefill_query(q, K, V, W, khat, t, C, m, 0.3, 0.4)
        kp = O.block_summary(K[: t + 1], C, proj=W)
        ref, ref_chosen = O.hils_decode_head(q, K[: t + 1], V[: t + 1], kp, t, C, m, 0.3, 0.4)
        np.testing.assert_array_equal(chosen, ref_chosen)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
        K2, V2 = K.copy(), V.copy()
        K2[t + 1:] = rng.standard_normal(K2[t + 1:].shape)
        V2[t + 1:] = rng.standard_normal(V2[t + 1:].shape)
        out2, chosen2 = O.hils_prefill_query(q, K2, V2, W, O.block_summary(K2, C, proj=W), t, C,
                                             m, 0.3, 0.4)
        np.testing.assert_array_equal(chosen, chosen2)
        np.testing.assert_allclose(out, out2, rtol=1e-12, atol=1e-12)
    # at the last position it is the decode itself
    q = rng.standard_normal(D)
    a, ca = O.hils_prefill_query(q, K, V, W, khat, L - 1, C, m, 0.3, 0.4)
    b_, cb = O.hils_decode_head(q, K, V, khat, L - 1, C, m, 0.3, 0.4)
    np.testing.assert_array_equal(ca, cb)
    np.testing.assert_allclose(a, b_, rtol=1e-12, atol=1e-12)
