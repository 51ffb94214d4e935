"""The CPU oracle over many query rows at once, for the GPU parity tests.

The same oracle functions, called row by row as the single-process tests do,
only spread over worker processes. Workers are spawned (not forked from the
test process, which holds GPU state) and import numpy and the oracle only:
they never touch the GPU. Inputs reach each worker once, at start-up, as
float32 arrays (bf16 values are exact in float32) and are widened to float64
there. No test functions here.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

import oracle.hisa_oracle as O

_S: dict = {}


def _init(state):
    for key, val in state.items():
        _S[key] = val.astype(np.float64) if isinstance(val, np.ndarray) and \
            val.dtype == np.float32 else val
    if "kidx" in _S:
        _S["summary"] = O.block_summary(_S["kidx"], _S["B"])


def _hier(r):
    return r, O.hier_query(_S["qidx"][r], _S["kidx"], _S["summary"], int(_S["pos"][r]), _S["B"],
                           _S["m"], _S["k"])


def _flat(r):
    return r, O.flat_select_for_query(_S["qidx"][r], _S["kidx"], int(_S["pos"][r]), _S["k"])


def _attend(job):
    r, q, idx = job
    return r, O.sparse_attention_for_query(np.asarray(q, dtype=np.float64), _S["K"], _S["V"], idx,
                                           _S["scale"])


def workers():
    """Worker count: the host's CPUs, at most 16 (the share of one GPU machine)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _pool(state):
    return ProcessPoolExecutor(max_workers=workers(), mp_context=mp.get_context("spawn"),
                               initializer=_init, initargs=(state,))


_ONE_THREAD = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def _run(state, fn, jobs):
    # one BLAS thread per worker (the pool supplies the parallelism); the
    # workers read these at start-up, so they are set while the pool runs
    saved = {v: os.environ.get(v) for v in _ONE_THREAD}
    os.environ.update({v: "1" for v in _ONE_THREAD})
    try:
        with _pool(state) as ex:
            return dict(ex.map(fn, jobs, chunksize=max(1, len(jobs) // (8 * workers()))))
    finally:
        for v, old in saved.items():
            if old is None:
                os.environ.pop(v, None)
            else:
                os.environ[v] = old


def hier_rows(kidx, qidx, pos, B, m, k, rows):
    """{row: oracle hier_query result} of one sequence (kidx [L, d], qidx
    [nq, d] float32, pos [nq])."""
    st = dict(kidx=np.asarray(kidx, np.float32), qidx=np.asarray(qidx, np.float32),
              pos=np.asarray(pos), B=B, m=m, k=k)
    return _run(st, _hier, list(rows))


def flat_rows(kidx, qidx, pos, k, rows):
    """{row: oracle flat_select_for_query result} of one sequence."""
    st = dict(kidx=np.asarray(kidx, np.float32), qidx=np.asarray(qidx, np.float32),
              pos=np.asarray(pos), k=k, B=1)
    return _run(st, _flat, list(rows))


def attend_rows(K, V, scale, jobs):
    """{row: oracle sparse_attention_for_query result} for jobs of (row, q
    [Hq, Dk] float32, token ids) over K [L, Hkv, Dk], V [L, Hkv, Dv]."""
    st = dict(K=np.asarray(K, np.float32), V=np.asarray(V, np.float32), scale=scale)
    return _run(st, _attend, list(jobs))
