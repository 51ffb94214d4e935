"""Named workloads and seeded synthetic inputs.

This module holds shapes and random draws only: it contains none of the
method's arithmetic (no pooling, scoring, selection or attention). Both the
GPU path (through tests and bench.py) and the CPU oracle receive the tensors
drawn here.

The pages measure on model activations and public long-context suites that
are not available; these draws stand in for them with the same sizes:

* indexer queries/keys are integer-valued, uniform on [-8, 8], stored as
  bf16, so every indexer score is exact in fp32 and selections compare
  bit for bit;
* attention Q/K/V are bf16 draws of N(0, sigma^2).

Draw order per workload: Kidx, Qidx, Q, K (or the MLA latent KV), V, W.
Large tensors are drawn in slabs of rows on the target device, so the draw
is deterministic for a given device type and seed.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

SLAB_ROWS = 65536


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill", "decode", "hils" or "hils_prefill"
    batch: int           # independent sequences
    L: int               # cached tokens per sequence
    B: int               # block (chunk) size
    m: int               # blocks kept per query, forced ones included
    k: int               # tokens kept per query (prefill/decode); 0 for hils
    d_idx: int           # indexer head dim
    Hq: int              # attention query heads
    Hkv: int             # attention kv heads
    Dk: int              # q/k head dim
    Dv: int              # v head dim
    mla: bool = False    # V is the first Dv columns of the latent K row
    sigma: float = 1.0   # std of attention inputs
    int_mode: bool = False  # hils only: integer-valued q/k/W twin
    nq: Optional[int] = None  # queries per sequence; default L (prefill) or 1

    @property
    def queries(self) -> int:
        if self.nq is not None:
            return self.nq
        return self.L if self.kind in ("prefill", "hils_prefill") else 1

    @property
    def n_blocks(self) -> int:
        return -(-self.L // self.B)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.Dk)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: tiny prefill, MQA prefill at 16K, MLA prefill at 64K
# (the headline, also run through the flat indexer), batched decode at 128K
# and two-level-softmax decode at 1M.
WORKLOADS = {
    "prefill_2k_tiny": Workload("prefill_2k_tiny", "prefill", 1, 2048, 64, 8, 128, 64,
                                1, 1, 128, 128),
    "prefill_16k_mqa": Workload("prefill_16k_mqa", "prefill", 1, 16384, 128, 32, 2048, 128,
                                16, 1, 128, 128),
    "prefill_64k_mla": Workload("prefill_64k_mla", "prefill", 1, 65536, 128, 64, 2048, 128,
                                64, 1, 576, 512, mla=True, sigma=1.0 / math.sqrt(576.0)),
    "decode_128k_b64": Workload("decode_128k_b64", "decode", 64, 131072, 128, 64, 2048, 128,
                                16, 1, 128, 128),
    "hils_decode_1m": Workload("hils_decode_1m", "hils", 1, 1048576, 64, 32, 0, 64,
                               16, 16, 64, 64),
    "hils_prefill_64k": Workload("hils_prefill_64k", "hils_prefill", 1, 65536, 64, 32, 0, 64,
                                 16, 16, 64, 64),
    "hils_prefill_512k": Workload("hils_prefill_512k", "hils_prefill", 1, 524288, 64, 32, 0, 64,
                                  16, 16, 64, 64),
}
HEADLINE = "prefill_64k_mla"


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randint_bf16(shape, g, device):
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1, shape[-1]) if len(shape) > 1 else out.view(1, -1)
    for r0 in range(0, flat.shape[0], SLAB_ROWS):
        r1 = min(flat.shape[0], r0 + SLAB_ROWS)
        flat[r0:r1] = torch.randint(-8, 9, (r1 - r0, flat.shape[1]), generator=g,
                                    device=device, dtype=torch.int32).to(torch.bfloat16)
    return out


def _randn_bf16(shape, g, device, sigma):
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1, shape[-1]) if len(shape) > 1 else out.view(1, -1)
    rows_per_slab = max(1, (SLAB_ROWS * 128) // flat.shape[1])
    for r0 in range(0, flat.shape[0], rows_per_slab):
        r1 = min(flat.shape[0], r0 + rows_per_slab)
        x = torch.randn((r1 - r0, flat.shape[1]), generator=g, device=device,
                        dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        flat[r0:r1] = x.to(torch.bfloat16)
    return out


def make_inputs(w: Workload, device="cpu", seed: int = 0) -> dict:
    """Draw every input of workload `w` on `device` with a seeded generator.

    Returns a dict of tensors:
      prefill/decode: kidx [b, L, d], qidx [b, nq, d], q [b, nq, Hq, Dk],
        k [b, L, Hkv, Dk], v [b, L, Hkv, Dv] (a strided view of k when mla),
        q_pos [b, nq] int32.
      hils: k, v [b, L, H, D], q [b, H, D], w_proj [D, D], q_pos [b] (= L-1).
      hils_prefill: as hils with q [b, nq, H, D] and q_pos [b, nq] (the
        last nq positions).
    """
    g = _gen(device, seed)
    nq = w.queries
    out = {}
    if w.kind in ("hils", "hils_prefill"):
        H, D = w.Hq, w.Dk
        qshape = (w.batch, H, D) if w.kind == "hils" else (w.batch, nq, H, D)
        if w.int_mode:
            out["k"] = _randint_bf16((w.batch, w.L, H, D), g, device)
            out["v"] = _randn_bf16((w.batch, w.L, H, D), g, device, 1.0)
            out["q"] = _randint_bf16(qshape, g, device)
            wp = torch.randint(-1, 2, (D, D), generator=g, device=device, dtype=torch.int32)
            out["w_proj"] = wp.to(torch.bfloat16)
        else:
            out["k"] = _randn_bf16((w.batch, w.L, H, D), g, device, w.sigma)
            out["v"] = _randn_bf16((w.batch, w.L, H, D), g, device, w.sigma)
            out["q"] = _randn_bf16(qshape, g, device, w.sigma)
            wp = torch.randn((D, D), generator=g, device=device, dtype=torch.float32)
            out["w_proj"] = (wp / math.sqrt(D)).to(torch.bfloat16)
        if w.kind == "hils":
            out["q_pos"] = torch.full((w.batch,), w.L - 1, dtype=torch.int32, device=device)
        else:
            pos = torch.arange(w.L - nq, w.L, dtype=torch.int32, device=device)
            out["q_pos"] = pos.unsqueeze(0).expand(w.batch, nq).contiguous()
        return out

    out["kidx"] = _randint_bf16((w.batch, w.L, w.d_idx), g, device)
    out["qidx"] = _randint_bf16((w.batch, nq, w.d_idx), g, device)
    out["q"] = _randn_bf16((w.batch, nq, w.Hq, w.Dk), g, device, w.sigma)
    if w.mla:
        assert w.Hkv == 1 and w.Dv <= w.Dk
        kv = _randn_bf16((w.batch, w.L, 1, w.Dk), g, device, w.sigma)
        out["k"] = kv
        out["v"] = kv[..., : w.Dv]
    else:
        out["k"] = _randn_bf16((w.batch, w.L, w.Hkv, w.Dk), g, device, w.sigma)
        out["v"] = _randn_bf16((w.batch, w.L, w.Hkv, w.Dv), g, device, w.sigma)
    if w.kind == "prefill":
        pos = torch.arange(w.L - nq, w.L, dtype=torch.int32, device=device)
        out["q_pos"] = pos.unsqueeze(0).expand(w.batch, nq).contiguous()
    else:
        out["q_pos"] = torch.full((w.batch, nq), w.L - 1, dtype=torch.int32, device=device)
    return out


def sample_positions(w: Workload, n: int, seed: int = 0) -> list:
    """Query positions for sampled checks: fixed edge positions plus seeded picks."""
    L, B, m, k = w.L, w.B, w.m, max(w.k, 1)
    edges = [0, 1, B - 1, B, B + 1, k - 1, k, m * B - 1, m * B, L - 2, L - 1]
    edges = sorted({p for p in edges if 0 <= p < L})
    g = torch.Generator().manual_seed(seed)
    extra = torch.randint(0, L, (max(0, n - len(edges)),), generator=g).tolist()
    return sorted(set(edges) | set(extra))
