"""CPU oracle: hierarchical (block-then-token) sparse retrieval, flat top-k
retrieval, sparse attention over the retrieved tokens, and the two-level
(chunk x token) softmax decode.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check of the entry
module and the cpu_baseline leg of the benchmark may import this module.
The GPU library never calls it and shares no code, table or constant with
it. Everything here is plain numpy in float64 on bf16-valued inputs upcast
to float64, one query at a time, in the order the pages describe the method.

Sources, cited by page title and section:
  [HISA-news]  QbitAI news article "HISA: hierarchical indexed sparse
               attention" (m.digipub.cc), parts "block-level coarse filter",
               "fine token selection inside the kept blocks", "complexity"
               and "seamless replacement".
  [HISA-expl]  "PKU HISA sparse attention mechanism: 3x long-text efficiency"
               (intelliparadigm.com), sections 1.1, 1.2.1, 1.2.2 and 1.3.
  [HiLS]       "Tencent Hunyuan HiLS-Attention: learnable hierarchical sparse
               attention for infinite context" (ai-engineering pages, Ch01.911),
               sections "learnable chunk-mass proxy" and "hierarchical softmax
               decomposition".
  [HiLS-7B]    "HiLS-Attention-7B hierarchical sparse mechanism explained"
               (mlqm.cn), section "what is HiLS-Attention".

Readings taken where the pages are silent or ambiguous (each is listed in
the design notes of the repository):
  * the forced "last" block is the query's own (local) block, and the two
    forced blocks count toward m;
  * only complete blocks strictly before the local block compete; block 0
    is forced anyway;
  * the block feature is the mean of the indexer keys of the block; the
    scoring function at both levels is the raw dot product;
  * token selection is one global top-k over the union of the kept blocks;
  * ties go to the lowest index, at both levels; -0.0 equals +0.0;
  * attention is causal and inclusive (a query sees its own token); an
    empty index set gives a zero output and log-sum-exp -inf;
  * index outputs are ascending with -1 padding.

Pinning status: every function below is pinned by CPU tests against brute
force, closed forms, textbook reductions (torch scaled-dot-product attention
in float64) and invariants the pages state. Nothing here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _f64(x):
    """bf16/float torch tensor or array -> float64 numpy array."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Step 1: block summaries.  [HISA-expl] 1.2.1 (fixed-size blocks, mean pooling
# as the block feature); [HISA-news] "block-level coarse filter" (one overall
# feature vector per block).  [HiLS] "learnable chunk-mass proxy" replaces the
# mean by a compressed chunk key; the two-level decode stands in a fixed
# linear projection W of the mean (khat = W @ mean).
# ---------------------------------------------------------------------------
def block_summary(kidx, B, proj=None):
    """kidx [L, d] -> summary [ceil(L/B), d].

    Row c is the mean of rows c*B .. min(L, (c+1)*B) - 1.  A final partial
    block is averaged over the rows it has.  With `proj` ([d_out, d]) each
    row is mapped to proj @ mean.
    """
    kidx = _f64(kidx)
    L, d = kidx.shape
    n_rows = -(-L // B)
    out = np.zeros((n_rows, d if proj is None else _f64(proj).shape[0]))
    for c in range(n_rows):
        rows = kidx[c * B: min(L, (c + 1) * B)]
        mean = rows.sum(axis=0) / rows.shape[0]
        out[c] = mean if proj is None else _f64(proj) @ mean
    return out


# ---------------------------------------------------------------------------
# Step 2: block scores.  [HISA-expl] 1.2.1 item 2 and [HISA-news] "block-level
# coarse filter": the indexer's own score (a dot product) against the block
# features only.
# ---------------------------------------------------------------------------
def block_scores_for_query(q, summary, t, B):
    """Scores of query q (position t) against every block.

    Entry c is q . summary[c] for complete blocks c < t // B and -inf for
    the local block and every later one.
    """
    q = _f64(q)
    summary = _f64(summary)
    b = t // B
    s = np.full(summary.shape[0], NEG_INF)
    if b > 0:
        s[:b] = summary[:b] @ q
    return s


def _rank_desc_lowest_index(values, ids):
    """Positions of `values` ordered by (value descending, id ascending)."""
    v = np.asarray(values, dtype=np.float64) + 0.0   # -0.0 -> +0.0
    return np.lexsort((np.asarray(ids), -v))


# ---------------------------------------------------------------------------
# Step 3: top-m blocks with the first and the local block forced.
# [HISA-expl] 1.2.1 item 3 (keep the m best blocks, always keep the first and
# the last); [HISA-news] "block-level coarse filter" (keep m, drop the rest)
# and the note that the first and the last block are always chosen.
# ---------------------------------------------------------------------------
def select_blocks_for_query(scores, t, B, m):
    """Return int64 [m]: the kept block ids in ascending order, -1 padded."""
    assert m >= 2
    b = t // B
    forced = [0] if b == 0 else [0, b]
    cand = np.arange(1, b)
    free = m - len(forced)
    if cand.size <= free:
        kept = list(range(0, b + 1))
    else:
        order = _rank_desc_lowest_index(np.asarray(scores)[cand], cand)
        kept = forced + [int(c) for c in cand[order[:free]]]
    out = np.full(m, -1, dtype=np.int64)
    kept = sorted(kept)
    out[: len(kept)] = kept
    return out


# ---------------------------------------------------------------------------
# Step 4: token-level top-k inside the kept blocks.  [HISA-expl] 1.2.2 and
# [HISA-news] "fine token selection": score every token of the kept blocks
# with the original indexer and keep the k best; the result has the flat
# indexer's format ([HISA-news] "seamless replacement").
# ---------------------------------------------------------------------------
def token_candidates(block_idx, t, B):
    """Causal token ids (j <= t) of the kept blocks, ascending."""
    ids = []
    for c in sorted(int(c) for c in block_idx if c >= 0):
        ids.extend(range(c * B, min((c + 1) * B, t + 1)))
    return np.asarray(ids, dtype=np.int64)


def topk_lowest_index(values, ids, k):
    """Keep min(k, n) entries by (value desc, id asc).

    Returns (kept ids ascending, -1 padded to k; their values, nan padded).
    """
    ids = np.asarray(ids, dtype=np.int64)
    values = np.asarray(values, dtype=np.float64)
    order = _rank_desc_lowest_index(values, ids)[:k]
    keep = np.sort(ids[order])
    out = np.full(k, -1, dtype=np.int64)
    out[: keep.size] = keep
    val = np.full(k, np.nan)
    pos = {int(j): i for i, j in enumerate(ids)}
    for i, j in enumerate(keep):
        val[i] = values[pos[int(j)]] + 0.0
    return out, val


def token_select_for_query(q, kidx, block_idx, t, B, k):
    q = _f64(q)
    kidx = _f64(kidx)
    cand = token_candidates(block_idx, t, B)
    u = kidx[cand] @ q if cand.size else np.zeros(0)
    return topk_lowest_index(u, cand, k)


# ---------------------------------------------------------------------------
# Flat comparison indexer.  [HISA-expl] 1.1 item 1 and [HISA-news] (the
# original token-level indexer scores every earlier token, then keeps the
# best ones: quadratic in L).
# ---------------------------------------------------------------------------
def flat_select_for_query(q, kidx, t, k):
    q = _f64(q)
    kidx = _f64(kidx)
    cand = np.arange(t + 1, dtype=np.int64)
    return topk_lowest_index(kidx[: t + 1] @ q, cand, k)


# ---------------------------------------------------------------------------
# Step 5: softmax attention over the selected tokens only.  [HISA-expl] 1.1
# (attention computed only between the query and the selected key tokens);
# [HISA-news] "seamless replacement" (the downstream sparse attention is left
# as it is).  Head h reads kv head h // (Hq / Hkv).
# ---------------------------------------------------------------------------
def sparse_attention_for_query(q, K, V, idx, scale):
    """q [Hq, Dk], K [L, Hkv, Dk], V [L, Hkv, Dv], idx with -1 padding.

    Returns (out [Hq, Dv], lse [Hq]) in float64, lse = log sum exp(scale*q.k).
    """
    q = _f64(q)
    K = _f64(K)
    V = _f64(V)
    Hq = q.shape[0]
    Hkv, Dv = K.shape[1], V.shape[2]
    group = Hq // Hkv
    sel = np.asarray([int(j) for j in idx if j >= 0], dtype=np.int64)
    out = np.zeros((Hq, Dv))
    lse = np.full(Hq, NEG_INF)
    if sel.size == 0:
        return out, lse
    for h in range(Hq):
        g = h // group
        s = scale * (K[sel, g, :] @ q[h])
        mx = s.max()
        p = np.exp(s - mx)
        z = p.sum()
        out[h] = (p / z) @ V[sel, g, :]
        lse[h] = mx + np.log(z)
    return out, lse


# ---------------------------------------------------------------------------
# Whole paths over a list of query positions of one sequence.
# ---------------------------------------------------------------------------
def hier_query(qidx_t, kidx, summary, t, B, m, k):
    """Steps 2-4 for one query. Returns (block_idx, block_scores, token_idx, token_scores)."""
    bs = block_scores_for_query(qidx_t, summary, t, B)
    bidx = select_blocks_for_query(bs, t, B, m)
    tidx, tval = token_select_for_query(qidx_t, kidx, bidx, t, B, k)
    return bidx, bs, tidx, tval


def hier_pipeline(kidx, qidx, q, K, V, positions, rows, B, m, k, scale):
    """Steps 1-5 for the queries at `rows` (rows of qidx/q) with positions
    `positions` (absolute token positions).  Returns a dict of arrays."""
    kidx, qidx, q, K, V = _f64(kidx), _f64(qidx), _f64(q), _f64(K), _f64(V)
    summary = block_summary(kidx, B)
    out = {"block_idx": [], "token_idx": [], "token_scores": [], "out": [], "lse": []}
    for r, t in zip(rows, positions):
        bidx, _, tidx, tval = hier_query(qidx[r], kidx, summary, int(t), B, m, k)
        o, lse = sparse_attention_for_query(q[r], K, V, tidx, scale)
        out["block_idx"].append(bidx)
        out["token_idx"].append(tidx)
        out["token_scores"].append(tval)
        out["out"].append(o)
        out["lse"].append(lse)
    return {key: np.stack(v) for key, v in out.items()}


def flat_pipeline(kidx, qidx, q, K, V, positions, rows, k, scale):
    kidx, qidx, q, K, V = _f64(kidx), _f64(qidx), _f64(q), _f64(K), _f64(V)
    out = {"token_idx": [], "token_scores": [], "out": [], "lse": []}
    for r, t in zip(rows, positions):
        tidx, tval = flat_select_for_query(qidx[r], kidx, int(t), k)
        o, lse = sparse_attention_for_query(q[r], K, V, tidx, scale)
        out["token_idx"].append(tidx)
        out["token_scores"].append(tval)
        out["out"].append(o)
        out["lse"].append(lse)
    return {key: np.stack(v) for key, v in out.items()}


# ---------------------------------------------------------------------------
# Two-level softmax decode.  [HiLS] "hierarchical softmax decomposition":
# attention weight = inter-chunk share x intra-chunk share; [HiLS-7B] "what
# is HiLS-Attention": chunks are routed by scores against compressed chunk
# keys, then fine attention runs inside the chosen chunks.
# ---------------------------------------------------------------------------
def hils_combine(q, K, V, chunks, logits, t, C, scale_token):
    """q [D], K/V [L, D] (one head), chunks: chosen chunk ids (-1 ignored),
    logits: the chunk logit of each entry of `chunks`.

    Output = sum_c softmax_c(logits) * a_c with a_c the softmax attention of
    q over the tokens j <= t of chunk c.
    """
    q = _f64(q)
    K = _f64(K)
    V = _f64(V)
    cs = [int(c) for c in chunks if c >= 0]
    lg = np.asarray([float(logits[i]) for i, c in enumerate(chunks) if c >= 0])
    w = np.exp(lg - lg.max())
    w = w / w.sum()
    out = np.zeros(V.shape[1])
    for wc, c in zip(w, cs):
        j = np.arange(c * C, min((c + 1) * C, t + 1))
        s = scale_token * (K[j] @ q)
        p = np.exp(s - s.max())
        out += wc * ((p / p.sum()) @ V[j])
    return out


def hils_decode_head(q, K, V, khat, t, C, m, scale_chunk, scale_token):
    """One head of the two-level decode at position t.

    khat [n_chunks, D]: chunk keys.  Routing keeps chunk 0 and the local
    chunk t // C, plus the best of chunks 1 .. t//C - 1 by q . khat (ties to
    the lowest id), m in total.  The chunk logit is scale_chunk * q . khat_c.
    Returns (out [D], chosen chunk ids [m] ascending -1 padded).
    """
    q = _f64(q)
    khat = _f64(khat)
    C = int(C)
    raw = block_scores_for_query(q, khat, t, C)
    chosen = select_blocks_for_query(raw, t, C, m)
    logits = [scale_chunk * float(khat[c] @ q) if c >= 0 else 0.0 for c in chosen]
    return hils_combine(q, K, V, chosen, logits, t, C, scale_token), chosen


def hils_prefill_query(q, K, V, W, khat, t, C, m, scale_chunk, scale_token):
    """One head, the query at position t of a causal two-level prefill: the
    decode of the first t+1 tokens.  Complete chunks keep their keys (rows of
    khat, the projected means of all their tokens); the local chunk t // C
    takes the projected mean of its tokens <= t only, as the decode's local
    chunk does at t = L-1.  Returns (out [D], chosen chunk ids [m])."""
    b = t // C
    rows = _f64(K)[b * C: t + 1]
    kh = _f64(khat)[: b + 1].copy()
    kh[b] = _f64(W) @ (rows.sum(axis=0) / rows.shape[0])
    return hils_decode_head(q, K, V, kh, t, C, m, scale_chunk, scale_token)
