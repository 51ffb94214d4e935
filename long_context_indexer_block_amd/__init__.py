"""Python binding of libhisa (hierarchical sparse retrieval + sparse attention
on MI355X). Argument marshalling only: every step runs in the HIP kernels of
libhisa.so; there is no CPU or PyTorch fallback. Calling any entry point
without the built library raises.

Each function takes torch tensors on the current HIP device, passes their
data pointers, strides and the current stream to the C ABI, and raises
HisaError on a non-OK status.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# HISA_LIBRARY may name another build of the same library (the host-sanitized
# test copy); by default the in-tree libhisa.so is loaded
LIB_PATH = os.environ.get("HISA_LIBRARY") or os.path.join(_PKG, "libhisa.so")
_lib = None


class HisaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"hisa status {status}: {msg}")
        self.status = status


class Strides(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("token", ctypes.c_int64), ("head", ctypes.c_int64)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_S = ctypes.c_size_t
_SIGS = {
    "hisa_last_error": (ctypes.c_char_p, []),
    "hisa_abi_version": (_I, []),
    "hisa_block_summary": (_I, [_P, Strides, _I, _I, _I, _I, _P, _P, _P, _P]),
    "hisa_block_summary_update": (_I, [_P, Strides, _I, _I, _I, _I, _P, _P, _P, _I, _I, _P]),
    "hisa_block_score": (_I, [_P, Strides, _P, _I, _I, _P, _I, _I, _I, _P, _P]),
    "hisa_select_blocks": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "hisa_route_blocks": (_I, [_P, Strides, _P, _I, _I, _P, _I, _I, _I, _I, _P, _P, _S, _P]),
    "hisa_route_blocks_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "hisa_token_select": (_I, [_P, Strides, _P, Strides, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                               _P, _P, _P, _S, _P]),
    "hisa_token_select_workspace_bytes": (_S, [_I, _I, _I, _I, _I, _I]),
    "hisa_token_select_noalloc": (_I, [_P, Strides, _P, Strides, _P, _P, _I, _I, _I, _I, _I, _I,
                                       _I, _P, _P, _P]),
    "flat_indexer_topk": (_I, [_P, Strides, _P, Strides, _P, _I, _I, _I, _I, _I, _P, _P, _P, _S,
                               _P]),
    "flat_indexer_topk_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "hisa_auto_plan": (_I, [_I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "sparse_attn_fwd": (_I, [_P, Strides, _P, Strides, _P, Strides, _I, _I, _I, _I, _I, _I, _I,
                             _P, _I, _F, _P, Strides, _P, _P, _S, _P]),
    "sparse_attn_fwd_workspace_bytes": (_S, [_I, _I, _I, _I, _I, _I, _I]),
    "hils_two_level_attn_fwd": (_I, [_P, Strides, _P, Strides, _P, Strides, _P, _P, _I, _I, _I,
                                     _I, _I, _I, _I, _F, _F, _P, Strides, _P, _S, _P]),
    "hils_two_level_attn_fwd_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "hils_two_level_prefill_fwd": (_I, [_P, Strides, _P, Strides, _P, Strides, _P, _P, _P, _P,
                                        _I, _I, _I, _I, _I, _I, _I, _I, _F, _F, _P, Strides, _P,
                                        _S, _P]),
    "hils_two_level_prefill_fwd_workspace_bytes": (_S, [_I, _I, _I, _I, _I, _I, _I]),
    "hisa_gather_probe": (_I, [_P, ctypes.c_int64, _I, _I, _P, _I, _I, _I, _I, _I, _P]),
}
EXPORTS = [n for n in _SIGS]


def lib():
    """Load libhisa.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise HisaError(-1, f"{LIB_PATH} not built; run `python -m "
                                "long_context_indexer_block_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(st):
    if st != 0:
        raise HisaError(st, lib().hisa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _str3(t, dims):
    """Strides (batch, token, head) of tensor t; `dims` names its leading dims."""
    s = dict(zip(dims, t.stride()))
    return Strides(s.get("b", 0), s.get("t", 0), s.get("h", 0))


def _need(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.stride(-1) != 1:
        raise ValueError(f"{name} needs a contiguous last dimension")


# ----------------------------------------------------------------- indexer
def hisa_block_summary(kidx, B, proj=None, summary=None, split=None, want_split=True):
    """kidx [b, L, d] bf16 -> (summary fp32 [b, ceil(L/B), d], split bf16 [b, n, 3, d])."""
    _need(kidx, torch.bfloat16, "kidx")
    b, L, d = kidx.shape
    n = -(-L // B)
    if summary is None:
        summary = torch.empty(b, n, d, dtype=torch.float32, device=kidx.device)
    if split is None and want_split:
        split = torch.empty(b, n, 3, d, dtype=torch.bfloat16, device=kidx.device)
    _check(lib().hisa_block_summary(_ptr(kidx), _str3(kidx, "bt"), b, L, d, B, _ptr(proj),
                                    _ptr(summary), _ptr(split), _stream()))
    return summary, split


def hisa_block_summary_update(kidx, L, B, summary, split, first_row=None, proj=None):
    """Recompute rows first_row .. ceil(L/B)-1 (default: the row of token L-1)
    of summary [b, cap, d] / split [b, cap, 3, d] from the first L rows of
    kidx [b, >=L, d] (a cache with room to grow)."""
    _need(kidx, torch.bfloat16, "kidx")
    b, _, d = kidx.shape
    tab = summary if summary is not None else split
    cap = tab.shape[1]
    if first_row is None:
        first_row = (L - 1) // B
    _check(lib().hisa_block_summary_update(_ptr(kidx), _str3(kidx, "bt"), b, int(L), d, B,
                                           _ptr(proj), _ptr(summary), _ptr(split), cap,
                                           int(first_row), _stream()))
    return summary, split


def hisa_block_score(qidx, q_pos, split, B, out=None):
    """qidx [b, nq, d] bf16, q_pos [b, nq] int32, split [b, n, 3, d] -> scores [b, nq, n] fp32."""
    _need(qidx, torch.bfloat16, "qidx")
    b, nq, d = qidx.shape
    n = split.shape[1]
    if out is None:
        out = torch.empty(b, nq, n, dtype=torch.float32, device=qidx.device)
    _check(lib().hisa_block_score(_ptr(qidx), _str3(qidx, "bt"), _ptr(q_pos), b, nq, _ptr(split),
                                  n, d, B, _ptr(out), _stream()))
    return out


def hisa_select_blocks(block_scores, q_pos, B, m, out=None):
    b, nq, n = block_scores.shape
    if out is None:
        out = torch.empty(b, nq, m, dtype=torch.int32, device=block_scores.device)
    _check(lib().hisa_select_blocks(_ptr(block_scores), _ptr(q_pos), b, nq, n, B, m, _ptr(out),
                                    _stream()))
    return out


ROUTE_MAX_ROWS = 64 * 16 + 2      # scores kept on chip up to this many blocks
ROUTE_STREAM_MAX_M = 130          # streamed selection for m up to this
ROUTE_STREAM_MAX_ROWS = 65537     # and up to this many blocks


def route_supported(n_rows, m):
    return n_rows <= ROUTE_MAX_ROWS or (m <= ROUTE_STREAM_MAX_M and n_rows <= ROUTE_STREAM_MAX_ROWS)


def route_workspace(batch, nq, n_rows, m, device):
    """Workspace for hisa_route_blocks on this shape (None when it needs none)."""
    n = int(lib().hisa_route_blocks_workspace_bytes(batch, nq, n_rows, m))
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def hisa_route_blocks(qidx, q_pos, split, B, m, out=None, workspace="auto"):
    """Steps 2 and 3 fused: qidx [b, nq, d] bf16, q_pos [b, nq] int32, split
    [b, n, 3, d] (route_supported(n, m)) -> block_idx [b, nq, m] int32.
    workspace: "auto" allocates what the shape asks for (few queries split
    their blocks over several workgroups), None runs without, or a uint8
    tensor from route_workspace()."""
    _need(qidx, torch.bfloat16, "qidx")
    b, nq, d = qidx.shape
    n = split.shape[1]
    if out is None:
        out = torch.empty(b, nq, m, dtype=torch.int32, device=qidx.device)
    if isinstance(workspace, str):
        workspace = route_workspace(b, nq, n, m, qidx.device)
    wsb = 0 if workspace is None else workspace.numel()
    _check(lib().hisa_route_blocks(_ptr(qidx), _str3(qidx, "bt"), _ptr(q_pos), b, nq, _ptr(split),
                                   n, d, B, m, _ptr(out), _ptr(workspace), wsb, _stream()))
    return out


def hisa_token_select_workspace_bytes(batch, nq, L, B, m, k):
    return int(lib().hisa_token_select_workspace_bytes(batch, nq, L, B, m, k))


def flat_indexer_topk_workspace_bytes(batch, nq, L, k):
    return int(lib().flat_indexer_topk_workspace_bytes(batch, nq, L, k))


def _workspace(nbytes, device, ws):
    if ws is not None and ws.numel() >= nbytes:
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def hisa_token_select(qidx, kidx, q_pos, block_idx, B, k, token_idx=None, token_scores=None,
                      want_scores=True, workspace=None):
    _need(qidx, torch.bfloat16, "qidx")
    _need(kidx, torch.bfloat16, "kidx")
    b, nq, d = qidx.shape
    L = kidx.shape[1]
    m = block_idx.shape[-1]
    dev = qidx.device
    if token_idx is None:
        token_idx = torch.empty(b, nq, k, dtype=torch.int32, device=dev)
    if token_scores is None and want_scores:
        token_scores = torch.empty(b, nq, k, dtype=torch.float32, device=dev)
    nbytes = hisa_token_select_workspace_bytes(b, nq, L, B, m, k)
    ws = _workspace(nbytes, dev, workspace)
    _check(lib().hisa_token_select(_ptr(qidx), _str3(qidx, "bt"), _ptr(kidx), _str3(kidx, "bt"),
                                   _ptr(q_pos), _ptr(block_idx), b, nq, L, d, B, m, k,
                                   _ptr(token_idx), _ptr(token_scores), _ptr(ws), ws.numel(),
                                   _stream()))
    return token_idx, token_scores


NOALLOC_SCRATCH_BYTES = 64 << 20


def hisa_token_select_noalloc(qidx, kidx, q_pos, block_idx, B, k, token_idx, token_scores=None):
    """hisa_token_select with the library's fixed scratch instead of a
    workspace: nothing is allocated (token_idx, and token_scores if wanted,
    are caller-provided)."""
    _need(qidx, torch.bfloat16, "qidx")
    _need(kidx, torch.bfloat16, "kidx")
    b, nq, d = qidx.shape
    L = kidx.shape[1]
    m = block_idx.shape[-1]
    _check(lib().hisa_token_select_noalloc(_ptr(qidx), _str3(qidx, "bt"), _ptr(kidx),
                                           _str3(kidx, "bt"), _ptr(q_pos), _ptr(block_idx), b, nq,
                                           L, d, B, m, k, _ptr(token_idx), _ptr(token_scores),
                                           _stream()))
    return token_idx, token_scores


def flat_indexer_topk(qidx, kidx, q_pos, k, token_idx=None, token_scores=None, want_scores=True,
                      workspace=None):
    _need(qidx, torch.bfloat16, "qidx")
    _need(kidx, torch.bfloat16, "kidx")
    b, nq, d = qidx.shape
    L = kidx.shape[1]
    dev = qidx.device
    if token_idx is None:
        token_idx = torch.empty(b, nq, k, dtype=torch.int32, device=dev)
    if token_scores is None and want_scores:
        token_scores = torch.empty(b, nq, k, dtype=torch.float32, device=dev)
    nbytes = flat_indexer_topk_workspace_bytes(b, nq, L, k)
    ws = _workspace(nbytes, dev, workspace)
    _check(lib().flat_indexer_topk(_ptr(qidx), _str3(qidx, "bt"), _ptr(kidx), _str3(kidx, "bt"),
                                   _ptr(q_pos), b, nq, L, d, k, _ptr(token_idx),
                                   _ptr(token_scores), _ptr(ws), ws.numel(), _stream()))
    return token_idx, token_scores


def hisa_auto_plan(L, B):
    """(hierarchical, m) for L keys and block size B: the flat indexer below
    8192 keys, m = max(64, L // 2000) clamped to 16384 // B."""
    h, m = _I(0), _I(0)
    _check(lib().hisa_auto_plan(int(L), int(B), ctypes.byref(h), ctypes.byref(m)))
    return bool(h.value), m.value


# ----------------------------------------------------------------- attention
def sparse_attn_workspace(q, k, v, token_idx):
    """Workspace for sparse_attn_fwd on these shapes (None when it needs none)."""
    b, nq, Hq, Dk = q.shape
    n = lib().sparse_attn_fwd_workspace_bytes(b, nq, Hq, k.shape[2], Dk, v.shape[-1],
                                              token_idx.shape[-1])
    return torch.empty(n, dtype=torch.uint8, device=q.device) if n else None


def sparse_attn_fwd(q, k, v, token_idx, scale, out=None, lse=None, want_lse=False,
                    workspace="auto"):
    """q [b, nq, Hq, Dk], k [b, L, Hkv, Dk], v [b, L, Hkv, Dv] (may be a view of k),
    token_idx [b, nq, topk] int32 -> out [b, nq, Hq, Dv] bf16 (, lse [b, nq, Hq]).
    workspace: "auto" allocates what the shape asks for, None runs unsplit, or a
    uint8 tensor from sparse_attn_workspace()."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, nm)
    b, nq, Hq, Dk = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    Dv = v.shape[-1]
    topk = token_idx.shape[-1]
    if out is None:
        out = torch.empty(b, nq, Hq, Dv, dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(b, nq, Hq, dtype=torch.float32, device=q.device)
    if isinstance(workspace, str):
        workspace = sparse_attn_workspace(q, k, v, token_idx)
    wsb = 0 if workspace is None else workspace.numel()
    _check(lib().sparse_attn_fwd(_ptr(q), _str3(q, "bth"), _ptr(k), _str3(k, "bth"), _ptr(v),
                                 _str3(v, "bth"), b, nq, L, Hq, Hkv, Dk, Dv, _ptr(token_idx), topk,
                                 float(scale), _ptr(out), _str3(out, "bth"), _ptr(lse),
                                 _ptr(workspace), wsb, _stream()))
    return (out, lse) if want_lse else out


def hils_workspace(b, H, D, m, device):
    """Workspace for hils_two_level_attn_fwd on these shapes (None when it needs none)."""
    n = lib().hils_two_level_attn_fwd_workspace_bytes(b, H, D, m)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def hils_two_level_attn_fwd(q, k, v, khat, chunk_idx, C, scale_chunk, scale_token, out=None,
                            workspace="auto"):
    """q [b, H, D], k/v [b, L, H, D], khat [b*H, n, D] fp32, chunk_idx [b*H, m] -> out [b, H, D].
    workspace: "auto" allocates what the shape asks for, None runs one workgroup per
    (sequence, head), or a uint8 tensor from hils_workspace()."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, nm)
    b, H, D = q.shape
    L = k.shape[1]
    n = khat.shape[1]
    m = chunk_idx.shape[-1]
    if out is None:
        out = torch.empty(b, H, D, dtype=torch.bfloat16, device=q.device)
    if isinstance(workspace, str):
        workspace = hils_workspace(b, H, D, m, q.device)
    wsb = 0 if workspace is None else workspace.numel()
    _check(lib().hils_two_level_attn_fwd(_ptr(q), _str3(q, "bh"), _ptr(k), _str3(k, "bth"),
                                         _ptr(v), _str3(v, "bth"), _ptr(khat), _ptr(chunk_idx), b,
                                         L, H, D, C, n, m, float(scale_chunk), float(scale_token),
                                         _ptr(out), _str3(out, "bh"), _ptr(workspace), wsb,
                                         _stream()))
    return out


def hils_prefill_workspace(b, nq, L, H, D, C, m, device):
    """Workspace for the bucketed hils_two_level_prefill_fwd on these shapes."""
    n = lib().hils_two_level_prefill_fwd_workspace_bytes(b, nq, L, H, D, C, m)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def hils_two_level_prefill_fwd(q, k, v, khat, chunk_idx, q_pos, C, scale_chunk, scale_token,
                               proj=None, out=None, workspace="auto"):
    """q [b, nq, H, D], k/v [b, L, H, D], khat [b*H, n, D] fp32, chunk_idx [b*H, nq, m],
    q_pos [b, nq] int32, proj [D, D] bf16 or None -> out [b, nq, H, D].
    workspace: "auto" allocates the bucketed path's scratch, None runs one
    workgroup per (query, head), or a uint8 tensor from hils_prefill_workspace()."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, nm)
    for t, nm in ((khat, "khat"), (chunk_idx, "chunk_idx"), (q_pos, "q_pos")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    b, nq, H, D = q.shape
    L = k.shape[1]
    n = khat.shape[1]
    m = chunk_idx.shape[-1]
    if out is None:
        out = torch.empty(b, nq, H, D, dtype=torch.bfloat16, device=q.device)
    if isinstance(workspace, str):
        workspace = hils_prefill_workspace(b, nq, L, H, D, C, m, q.device)
    wsb = 0 if workspace is None else workspace.numel()
    _check(lib().hils_two_level_prefill_fwd(_ptr(q), _str3(q, "bth"), _ptr(k), _str3(k, "bth"),
                                            _ptr(v), _str3(v, "bth"), _ptr(khat),
                                            _ptr(chunk_idx), _ptr(proj), _ptr(q_pos), b, nq, L, H,
                                            D, C, n, m, float(scale_chunk), float(scale_token),
                                            _ptr(out), _str3(out, "bth"), _ptr(workspace), wsb,
                                            _stream()))
    return out


# ----------------------------------------------------------------- measurement
def hisa_gather_probe(table, ids, row_bytes, waves=4, depth=2, rot_ticks=0):
    """Stream the rows ids [nq, topk] name from table [n_rows, row_stride] (any
    dtype, rows contiguous) into on-chip memory the way the attention kernels
    gather them, and discard them (a gather-rate ceiling). Enqueued on the
    current stream; returns nothing."""
    if not table.is_cuda or not ids.is_cuda:
        raise TypeError("table and ids must be device tensors")
    if ids.dtype != torch.int32 or not ids.is_contiguous() or ids.dim() != 2:
        raise ValueError("ids must be a contiguous int32 [nq, topk] tensor")
    n_rows = table.shape[0]
    stride = table.stride(0) * table.element_size()
    nq, topk = ids.shape
    _check(lib().hisa_gather_probe(_ptr(table), stride, int(row_bytes), n_rows, _ptr(ids), nq,
                                   topk, int(waves), int(depth), int(rot_ticks), _stream()))


# ----------------------------------------------------------------- pipelines
from .pipeline import HierPipeline, FlatPipeline, HilsDecode, HilsPrefill  # noqa: E402,F401
