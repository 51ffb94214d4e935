"""Whole paths over preallocated device buffers (every step is a libhisa call).

HierPipeline: block summary -> block score -> top-m blocks -> token top-k
              -> sparse attention (HISA explainer 1.2-1.3; HISA news article).
FlatPipeline: flat indexer top-k -> sparse attention (the comparison path).
AutoPipeline: one of the two by the runtime policy of hisa_auto_plan (flat
              below 8192 keys, m = max(64, L // 2000)).
DecodeSession: batched decode over caches that grow in place; appending
              tokens recomputes only the summary rows of the blocks they touch.
HilsDecode:   chunk keys (once per cache) -> chunk scores -> top-m chunks
              -> two-level softmax attention (HiLS chapter).
"""
from __future__ import annotations

import torch

from . import (flat_indexer_topk, flat_indexer_topk_workspace_bytes, hils_two_level_attn_fwd,
               hils_prefill_workspace, hils_two_level_prefill_fwd, hils_workspace,
               hisa_auto_plan, route_supported, hisa_block_score, hisa_block_summary,
               hisa_block_summary_update, hisa_route_blocks, hisa_select_blocks, route_workspace,
               hisa_token_select, hisa_token_select_workspace_bytes, sparse_attn_fwd,
               sparse_attn_workspace)


def _attend_slabs(pipe, streams, workspaces):
    """The query slabs' attention, each slab after its selection's event, the
    slabs taken in turn by the attention streams (each with its own
    workspace), so that the next slab fills the compute units the last
    workgroups of a slab leave idle."""
    lse = pipe.lse
    for i, ((s0, s1), done) in enumerate(zip(pipe.slabs, pipe.slab_done)):
        st, ws = streams[i % len(streams)], workspaces[i % len(streams)]
        with torch.cuda.stream(st):
            st.wait_event(done)
            sparse_attn_fwd(pipe.q[:, s0:s1], pipe.k, pipe.v, pipe.token_idx[:, s0:s1],
                            pipe.scale, out=pipe.out[:, s0:s1],
                            lse=None if lse is None else lse[:, s0:s1],
                            want_lse=lse is not None, workspace=ws)


class HierPipeline:
    """The hierarchical step a1-a5. overlap_slabs > 1 (one sequence only) sets
    up run_overlapped(): the block scores, block and token selection of query
    slab i+1 on one stream while slab i attends on another (two attention
    streams, taking the slabs in turn)."""

    def __init__(self, kidx, qidx, q_pos, q, k, v, B, m, k_top, scale, want_scores=False,
                 want_lse=False, overlap_slabs=0):
        self.kidx, self.qidx, self.q_pos, self.q, self.k, self.v = kidx, qidx, q_pos, q, k, v
        self.B, self.m, self.k_top, self.scale = B, m, k_top, scale
        b, L, d = kidx.shape
        nq = qidx.shape[1]
        dev = kidx.device
        n = -(-L // B)
        self.summary = torch.empty(b, n, d, dtype=torch.float32, device=dev)
        self.split = torch.empty(b, n, 3, d, dtype=torch.bfloat16, device=dev)
        self.block_scores = torch.empty(b, nq, n, dtype=torch.float32, device=dev)
        self.block_idx = torch.empty(b, nq, m, dtype=torch.int32, device=dev)
        self.token_idx = torch.empty(b, nq, k_top, dtype=torch.int32, device=dev)
        self.token_scores = (torch.empty(b, nq, k_top, dtype=torch.float32, device=dev)
                             if want_scores else None)
        nbytes = hisa_token_select_workspace_bytes(b, nq, L, B, m, k_top)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        Hq, Dv = q.shape[2], v.shape[-1]
        self.out = torch.empty(b, nq, Hq, Dv, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(b, nq, Hq, dtype=torch.float32, device=dev) if want_lse else None
        self.attn_ws = sparse_attn_workspace(q, k, v, self.token_idx)
        self.slabs = []
        if overlap_slabs > 1 and b == 1 and nq >= overlap_slabs:
            sl = -(-nq // overlap_slabs)
            self.slabs = [(s0, min(nq, s0 + sl)) for s0 in range(0, nq, sl)]
            self.slab_pos = [q_pos[:, s0:s1].contiguous() for s0, s1 in self.slabs]
            self.slab_done = [torch.cuda.Event() for _ in self.slabs]
            nbytes = hisa_token_select_workspace_bytes(1, sl, L, B, m, k_top)
            self.slab_ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
            self.slab_attn_ws = sparse_attn_workspace(q[:, :sl], k, v, self.token_idx[:, :sl])
            # one stream selects, two alternate the slabs' attention (so that
            # the next slab fills the compute units the last workgroups of a
            # slab leave idle: 64K 19.30-19.38 -> 19.04-19.19 ms and 19.57 ->
            # 19.48 ms on two hosts; a third attention stream gained nothing),
            # each with its own attention workspace
            self.streams = tuple(torch.cuda.Stream(device=dev) for _ in range(3))
            self.slab_attn_wss = [self.slab_attn_ws, sparse_attn_workspace(
                q[:, :sl], k, v, self.token_idx[:, :sl])]

    def summarize(self):
        hisa_block_summary(self.kidx, self.B, summary=self.summary, split=self.split)

    def index(self, summarize=True):
        if summarize:
            self.summarize()
        hisa_block_score(self.qidx, self.q_pos, self.split, self.B, out=self.block_scores)
        hisa_select_blocks(self.block_scores, self.q_pos, self.B, self.m, out=self.block_idx)
        hisa_token_select(self.qidx, self.kidx, self.q_pos, self.block_idx, self.B, self.k_top,
                          token_idx=self.token_idx, token_scores=self.token_scores,
                          want_scores=self.token_scores is not None, workspace=self.ws)

    def attend(self):
        sparse_attn_fwd(self.q, self.k, self.v, self.token_idx, self.scale, out=self.out,
                        lse=self.lse, want_lse=self.lse is not None, workspace=self.attn_ws)

    def run(self, summarize=True):
        self.index(summarize)
        self.attend()
        return self.out

    def run_overlapped(self, summarize=True):
        """The same step, the query slabs' block scores, block and token
        selection (one stream) ahead of their attention (two streams taking
        the slabs in turn); same results as run()."""
        if not self.slabs:
            return self.run(summarize)
        sa = self.streams[0]
        cur = torch.cuda.current_stream()
        for st in self.streams:
            st.wait_stream(cur)
        ts = self.token_scores
        with torch.cuda.stream(sa):
            if summarize:
                self.summarize()
            for (s0, s1), pos, done in zip(self.slabs, self.slab_pos, self.slab_done):
                hisa_block_score(self.qidx[:, s0:s1], pos, self.split, self.B,
                                 out=self.block_scores[:, s0:s1])
                hisa_select_blocks(self.block_scores[:, s0:s1], pos, self.B, self.m,
                                   out=self.block_idx[:, s0:s1])
                hisa_token_select(self.qidx[:, s0:s1], self.kidx, pos, self.block_idx[:, s0:s1],
                                  self.B, self.k_top, token_idx=self.token_idx[:, s0:s1],
                                  token_scores=None if ts is None else ts[:, s0:s1],
                                  want_scores=ts is not None, workspace=self.slab_ws)
                done.record(sa)
        _attend_slabs(self, self.streams[1:], self.slab_attn_wss)
        for st in self.streams:
            cur.wait_stream(st)
        return self.out


class FlatPipeline:
    """The flat step (score every causal token, top k, attention);
    overlap_slabs > 1 (one sequence only) sets up run_overlapped() as for
    HierPipeline."""

    def __init__(self, kidx, qidx, q_pos, q, k, v, k_top, scale, want_scores=False,
                 want_lse=False, overlap_slabs=0):
        self.kidx, self.qidx, self.q_pos, self.q, self.k, self.v = kidx, qidx, q_pos, q, k, v
        self.k_top, self.scale = k_top, scale
        b, L, d = kidx.shape
        nq = qidx.shape[1]
        dev = kidx.device
        self.token_idx = torch.empty(b, nq, k_top, dtype=torch.int32, device=dev)
        self.token_scores = (torch.empty(b, nq, k_top, dtype=torch.float32, device=dev)
                             if want_scores else None)
        nbytes = flat_indexer_topk_workspace_bytes(b, nq, L, k_top)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        Hq, Dv = q.shape[2], v.shape[-1]
        self.out = torch.empty(b, nq, Hq, Dv, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(b, nq, Hq, dtype=torch.float32, device=dev) if want_lse else None
        self.attn_ws = sparse_attn_workspace(q, k, v, self.token_idx)
        self.slabs = []
        if overlap_slabs > 1 and b == 1 and nq >= overlap_slabs:
            sl = -(-nq // overlap_slabs)
            self.slabs = [(s0, min(nq, s0 + sl)) for s0 in range(0, nq, sl)]
            self.slab_pos = [q_pos[:, s0:s1].contiguous() for s0, s1 in self.slabs]
            self.slab_done = [torch.cuda.Event() for _ in self.slabs]
            nbytes = flat_indexer_topk_workspace_bytes(1, sl, L, k_top)
            self.slab_ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
            # one stream selects, two take the slabs' attention in turn, as in
            # the hierarchical step
            self.slab_attn_wss = [sparse_attn_workspace(q[:, :sl], k, v, self.token_idx[:, :sl])
                                  for _ in range(2)]
            self.streams = tuple(torch.cuda.Stream(device=dev) for _ in range(3))

    def index(self):
        flat_indexer_topk(self.qidx, self.kidx, self.q_pos, self.k_top, token_idx=self.token_idx,
                          token_scores=self.token_scores,
                          want_scores=self.token_scores is not None, workspace=self.ws)

    def attend(self):
        sparse_attn_fwd(self.q, self.k, self.v, self.token_idx, self.scale, out=self.out,
                        lse=self.lse, want_lse=self.lse is not None, workspace=self.attn_ws)

    def run(self):
        self.index()
        self.attend()
        return self.out

    def run_overlapped(self):
        """The flat selection of query slab i+1 (one stream) while slab i
        attends (two streams taking the slabs in turn); same results as
        run()."""
        if not self.slabs:
            return self.run()
        sa = self.streams[0]
        cur = torch.cuda.current_stream()
        for st in self.streams:
            st.wait_stream(cur)
        ts = self.token_scores
        with torch.cuda.stream(sa):
            for (s0, s1), pos, done in zip(self.slabs, self.slab_pos, self.slab_done):
                flat_indexer_topk(self.qidx[:, s0:s1], self.kidx, pos, self.k_top,
                                  token_idx=self.token_idx[:, s0:s1],
                                  token_scores=None if ts is None else ts[:, s0:s1],
                                  want_scores=ts is not None, workspace=self.slab_ws)
                done.record(sa)
        _attend_slabs(self, self.streams[1:], self.slab_attn_wss)
        for st in self.streams:
            cur.wait_stream(st)
        return self.out


class AutoPipeline:
    """The hierarchical or the flat path, chosen from L and B by
    hisa_auto_plan (HISA explainer 1.3 item 3 and 3.2 item 2)."""

    def __init__(self, kidx, qidx, q_pos, q, k, v, B, k_top, scale, want_scores=False,
                 want_lse=False):
        L = kidx.shape[1]
        self.hierarchical, self.m = hisa_auto_plan(L, B)
        if self.hierarchical:
            self.path = HierPipeline(kidx, qidx, q_pos, q, k, v, B, self.m, k_top, scale,
                                     want_scores=want_scores, want_lse=want_lse)
        else:
            self.path = FlatPipeline(kidx, qidx, q_pos, q, k, v, k_top, scale,
                                     want_scores=want_scores, want_lse=want_lse)

    def __getattr__(self, name):  # token_idx, token_scores, out, lse, ...
        return getattr(self.__dict__["path"], name)

    def run(self):
        return self.path.run()


class DecodeSession:
    """One new query per sequence per step over caches with room to grow.

    kidx [b, Lmax, d], k [b, Lmax, Hkv, Dk], v [b, Lmax, Hkv, Dv] are the
    caller's caches; the first L tokens are valid. The summary table keeps a
    row for every block the caches can reach. After the caller writes new
    tokens behind the valid ones, grow(L_new) recomputes only the rows of the
    blocks those tokens fall in; step(q, qidx) runs block scores, top-m blocks,
    token top-k and attention for the queries at position L-1."""

    def __init__(self, kidx, k, v, L, Hq, B, m, k_top, scale):
        from . import lib, sparse_attn_workspace  # noqa: F401
        self.kidx, self.kc, self.vc = kidx, k, v
        self.B, self.m, self.k_top, self.scale = B, m, k_top, scale
        b, Lmax, d = kidx.shape
        dev = kidx.device
        cap = -(-Lmax // B)
        self.split = torch.empty(b, cap, 3, d, dtype=torch.bfloat16, device=dev)
        self.q_pos = torch.empty(b, 1, dtype=torch.int32, device=dev)
        self.block_scores = torch.empty(b, 1, cap, dtype=torch.float32, device=dev)
        self.block_idx = torch.empty(b, 1, m, dtype=torch.int32, device=dev)
        self.token_idx = torch.empty(b, 1, k_top, dtype=torch.int32, device=dev)
        nbytes = hisa_token_select_workspace_bytes(b, 1, Lmax, B, m, k_top)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        Hkv, Dk, Dv = k.shape[2], k.shape[3], v.shape[3]
        n = lib().sparse_attn_fwd_workspace_bytes(b, 1, Hq, Hkv, Dk, Dv, k_top)
        self.attn_ws = torch.empty(n, dtype=torch.uint8, device=dev) if n else None
        self.out = torch.empty(b, 1, Hq, Dv, dtype=torch.bfloat16, device=dev)
        # one query per sequence: blocks scored and selected in parts over
        # several workgroups when the shape allows it (same block_idx)
        self.route_ws = route_workspace(b, 1, cap, m, dev)
        self.L = 0
        self.grow(L)

    def grow(self, L_new):
        """The caches now hold L_new tokens: refresh the rows of the blocks
        from the one holding the first new token on."""
        assert self.L < L_new <= self.kidx.shape[1]
        hisa_block_summary_update(self.kidx, L_new, self.B, None, self.split,
                                  first_row=self.L // self.B)
        self.L = L_new
        self.q_pos.fill_(L_new - 1)

    def step(self, q, qidx):
        """q [b, 1, Hq, Dk], qidx [b, 1, d]: the queries at position L-1."""
        L = self.L
        if self.route_ws is not None:
            hisa_route_blocks(qidx, self.q_pos, self.split, self.B, self.m, out=self.block_idx,
                              workspace=self.route_ws)
        else:
            hisa_block_score(qidx, self.q_pos, self.split, self.B, out=self.block_scores)
            hisa_select_blocks(self.block_scores, self.q_pos, self.B, self.m, out=self.block_idx)
        hisa_token_select(qidx, self.kidx[:, :L], self.q_pos, self.block_idx, self.B, self.k_top,
                          token_idx=self.token_idx, want_scores=False, workspace=self.ws)
        sparse_attn_fwd(q, self.kc[:, :L], self.vc[:, :L], self.token_idx, self.scale,
                        out=self.out, workspace=self.attn_ws)
        return self.out

    def capture(self, q, qidx):
        """step(q, qidx) at the current length as a HIP graph: copy the next
        queries into q and qidx, then replay() (the step enqueues kernel
        launches only, no allocation and no memset). Valid until grow()."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(q, qidx)
        return g


class HilsDecode:
    """Two-level decode at position L-1 for every (sequence, head)."""

    def __init__(self, q, k, v, w_proj, C, m, scale_chunk, scale_token):
        self.q, self.k, self.v, self.w_proj = q, k, v, w_proj
        self.C, self.m, self.scale_chunk, self.scale_token = C, m, scale_chunk, scale_token
        b, L, H, D = k.shape
        dev = k.device
        n = -(-L // C)
        self.n = n
        self.khat = torch.empty(b * H, n, D, dtype=torch.float32, device=dev)
        self.split = torch.empty(b * H, n, 3, D, dtype=torch.bfloat16, device=dev)
        self.q_pos = torch.full((b * H, 1), L - 1, dtype=torch.int32, device=dev)
        self.scores = torch.empty(b * H, 1, n, dtype=torch.float32, device=dev)
        self.chunk_idx = torch.empty(b * H, 1, m, dtype=torch.int32, device=dev)
        self.out = torch.empty(b, H, D, dtype=torch.bfloat16, device=dev)
        self.ws = hils_workspace(b, H, D, m, dev)
        # few (sequence, head) pairs over many chunks: routed in parts over
        # several workgroups (same chunk_idx as score then select)
        self.route_ws = route_workspace(b * H, 1, n, m, dev)

    def build_keys(self):
        # every (sequence, head) pair is one routed sequence: x[bi] viewed as
        # [H, L, D] (no copy) gives rows bi*H .. bi*H + H - 1 of the key table
        b, L, H, D = self.k.shape
        for bi in range(b):
            kv = self.k[bi].permute(1, 0, 2)
            hisa_block_summary(kv, self.C, proj=self.w_proj, summary=self.khat[bi * H:(bi + 1) * H],
                               split=self.split[bi * H:(bi + 1) * H])

    def route(self):
        b, H, D = self.q.shape
        qv = self.q.reshape(b * H, 1, D)
        if self.route_ws is not None:
            hisa_route_blocks(qv, self.q_pos, self.split, self.C, self.m, out=self.chunk_idx,
                              workspace=self.route_ws)
        else:
            hisa_block_score(qv, self.q_pos, self.split, self.C, out=self.scores)
            hisa_select_blocks(self.scores, self.q_pos, self.C, self.m, out=self.chunk_idx)

    def attend(self):
        hils_two_level_attn_fwd(self.q, self.k, self.v, self.khat, self.chunk_idx.view(-1, self.m),
                                self.C, self.scale_chunk, self.scale_token, out=self.out,
                                workspace=self.ws)

    def run(self, build=False):
        if build:
            self.build_keys()
        self.route()
        self.attend()
        return self.out


class HilsPrefill:
    """Causal two-level prefill: the query at position q_pos[b, i] of every
    head routes over the chunk keys before it (chunk 0 and its own chunk
    forced) and attends within its chosen chunks, as the decode of the tokens
    up to it would.

    q [b, nq, H, D], k/v [b, L, H, D] bf16, w_proj [D, D] bf16 (or None for
    plain-mean chunk keys), q_pos [b, nq] int32. Queries run in slabs of at
    most `slab` positions, which bounds the attention's scratch memory (its
    per-entry partial results)."""

    def __init__(self, q, k, v, w_proj, q_pos, C, m, scale_chunk, scale_token, slab=65536):
        self.q, self.k, self.v, self.w_proj, self.q_pos = q, k, v, w_proj, q_pos
        self.C, self.m, self.scale_chunk, self.scale_token = C, m, scale_chunk, scale_token
        b, nq, H, D = q.shape
        L = k.shape[1]
        dev = k.device
        n = -(-L // C)
        self.n = n
        self.khat = torch.empty(b * H, n, D, dtype=torch.float32, device=dev)
        self.split = torch.empty(b * H, n, 3, D, dtype=torch.bfloat16, device=dev)
        self.slabs = [(s0, min(nq, s0 + slab)) for s0 in range(0, nq, slab)]
        S = self.slabs[0][1] - self.slabs[0][0]
        self.slab_pos = [q_pos[:, s0:s1].contiguous() for s0, s1 in self.slabs]
        # routed sequence b*H + h reads the positions of sequence b
        self.slab_pos_h = [p.repeat_interleave(H, dim=0).contiguous() for p in self.slab_pos]
        self.slab_idx = [torch.empty(b * H, s1 - s0, m, dtype=torch.int32, device=dev)
                         for s0, s1 in self.slabs]
        # routing never writes chunk scores to memory (m <= 64 is always supported)
        assert route_supported(n, m)
        self.out = torch.empty(b, nq, H, D, dtype=torch.bfloat16, device=dev)
        # bucketed attention (None: one workgroup per query and head)
        self.ws = hils_prefill_workspace(b, S, L, H, D, C, m, dev)
        self.slab_done = [torch.cuda.Event() for _ in self.slabs]
        self.streams = (torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev))

    def chunk_ids(self):
        """The chosen chunks of every query, [b*H, nq, m]."""
        return self.slab_idx[0] if len(self.slabs) == 1 else torch.cat(self.slab_idx, dim=1)

    def build_keys(self):
        b, L, H, D = self.k.shape
        for bi in range(b):
            kv = self.k[bi].permute(1, 0, 2)
            hisa_block_summary(kv, self.C, proj=self.w_proj, summary=self.khat[bi * H:(bi + 1) * H],
                               split=self.split[bi * H:(bi + 1) * H])

    def route_slab(self, i):
        # q[bi] viewed as [H, nq, D] (no copy): head h is routed sequence bi*H + h
        b, nq, H, D = self.q.shape
        s0, s1 = self.slabs[i]
        for bi in range(b):
            rows = slice(bi * H, (bi + 1) * H)
            hisa_route_blocks(self.q[bi, s0:s1].permute(1, 0, 2), self.slab_pos_h[i][rows],
                              self.split[rows], self.C, self.m, out=self.slab_idx[i][rows])

    def attend_slab(self, i):
        s0, s1 = self.slabs[i]
        hils_two_level_prefill_fwd(self.q[:, s0:s1], self.k, self.v, self.khat,
                                   self.slab_idx[i], self.slab_pos[i], self.C, self.scale_chunk,
                                   self.scale_token, proj=self.w_proj, out=self.out[:, s0:s1],
                                   workspace=self.ws)

    def route(self):
        for i in range(len(self.slabs)):
            self.route_slab(i)

    def attend(self):
        for i in range(len(self.slabs)):
            self.attend_slab(i)

    def run_overlapped(self, build=True):
        """The same prefill with the routing of slab i+1 (stream A) running
        while slab i attends (stream B)."""
        sa, sb = self.streams
        cur = torch.cuda.current_stream()
        sa.wait_stream(cur)
        sb.wait_stream(cur)
        with torch.cuda.stream(sa):
            if build:
                self.build_keys()
            for i, done in enumerate(self.slab_done):
                self.route_slab(i)
                done.record(sa)
        with torch.cuda.stream(sb):
            for i, done in enumerate(self.slab_done):
                sb.wait_event(done)
                self.attend_slab(i)
        cur.wait_stream(sa)
        cur.wait_stream(sb)
        return self.out

    def run(self, build=True):
        if build:
            self.build_keys()
        self.route()
        self.attend()
        return self.out
