"""Helpers for the GPU parity tests: run the oracle on selected query rows
and compare with what the HIP path produced (no test functions here)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle.hisa_oracle as O

# attention tolerances (fp64 oracle cast to fp32 vs bf16 GPU output upcast)
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
REL_NORM = 1e-2   # also relative: the 64K MLA outputs are ~1e-3 in size


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def check_attention(gpu, ref, what=""):
    g = np.asarray(gpu, dtype=np.float32).astype(np.float64)
    r = np.asarray(ref, dtype=np.float64).astype(np.float32).astype(np.float64)
    err = np.abs(g - r)
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    mx, mean = float(err.max()), float(err.mean())
    rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
    assert mx <= MAX_ABS, f"{what}: max-abs {mx:.3e}"
    assert mean <= MEAN_ABS, f"{what}: mean-abs {mean:.3e}"
    assert rel <= REL_NORM, f"{what}: relative error {rel:.3e}"
    return mx, mean, rel


def check_index_rows(gpu_rows, ref_rows, what=""):
    g = np.asarray(gpu_rows, dtype=np.int64)
    r = np.asarray(ref_rows, dtype=np.int64)
    if not np.array_equal(g, r):
        bad = np.argwhere((g != r).any(axis=-1))[:5]
        raise AssertionError(f"{what}: index mismatch at rows {bad.ravel().tolist()}:\n"
                             f"gpu {g[bad[0][0]].tolist()[:16]}\nref {r[bad[0][0]].tolist()[:16]}")


def check_score_rows(gpu_rows, ref_rows, what=""):
    g = np.asarray(gpu_rows, dtype=np.float32)
    r = np.asarray(ref_rows, dtype=np.float64).astype(np.float32)
    same = (g == r) | (np.isnan(g) & np.isnan(r))
    if not same.all():
        i = np.argwhere(~same)[0]
        raise AssertionError(f"{what}: score mismatch at {i.tolist()}: {g[tuple(i)]} vs {r[tuple(i)]}")


class SeqOracle:
    """Oracle state for one sequence b of a prefill/decode input dict."""

    def __init__(self, inp, b, B, with_attention=True):
        self.kidx = f64(inp["kidx"][b])
        self.qidx = f64(inp["qidx"][b])
        self.pos = inp["q_pos"][b].cpu().numpy()
        self.B = B
        self.summary = O.block_summary(self.kidx, B)
        if with_attention:
            self.q = inp["q"][b]
            self.K = f64(inp["k"][b])
            self.V = f64(inp["v"][b])

    def hier(self, r, m, k):
        return O.hier_query(self.qidx[r], self.kidx, self.summary, int(self.pos[r]), self.B, m, k)

    def flat(self, r, k):
        return O.flat_select_for_query(self.qidx[r], self.kidx, int(self.pos[r]), k)

    def attend(self, r, idx, scale):
        return O.sparse_attention_for_query(f64(self.q[r]), self.K, self.V, idx, scale)
