"""Benchmark: one step = the whole hierarchical path (block summary, block
scores, top-m blocks, token top-k, sparse attention) over the 64K-token MLA
prefill (65536 queries, B=128, m=64, k=2048, 64 query heads over one
576/512 latent kv head), inputs resident in HBM.

Prints one JSON line: queries/s, per-stage milliseconds (HIP events on the
launch stream), the dominant kernel's roofline, the flat-indexer comparison
and the CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-flat] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak
METRIC = "indexer+sparse-attn queries/s at 64K"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_64k_mla")
    ap.add_argument("--no-flat", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    return ap.parse_args()


def indexer_flop(w):
    """Algorithmic indexer work of one prefill step: 2*d flop per scored
    (query, candidate block) pair and per scored (query, candidate token)
    pair, with the candidate counts the method defines (blocks 1..b-1; the
    causal tokens of the kept blocks: all of them while b+1 <= m, else m-1
    full blocks plus the local block's prefix)."""
    import numpy as np
    t = np.arange(w.L - w.queries, w.L, dtype=np.int64)
    b = t // w.B
    blocks = np.maximum(b - 1, 0)
    tokens = np.where(b + 1 <= w.m, t + 1, (w.m - 1) * w.B + (t - b * w.B + 1))
    return float(2 * w.d_idx * (blocks.sum() + tokens.sum()) * w.batch)


def cpu_baseline(w, inp, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    per-query steps 2-5 for seeded query positions until the time budget is
    spent (the one-off block summary is timed separately)."""
    import numpy as np
    import torch

    import oracle.hisa_oracle as O
    from workloads import sample_positions

    kidx = inp["kidx"][0].to("cpu", torch.float64).numpy()
    qidx = inp["qidx"][0].to("cpu", torch.float64).numpy()
    K = inp["k"][0].to("cpu", torch.float64).numpy()
    V = inp["v"][0].to("cpu", torch.float64).numpy()
    t0 = time.perf_counter()
    summ = O.block_summary(kidx, w.B)
    t_summary = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    pos = sample_positions(w, 64)
    rng.shuffle(pos)
    done = 0
    t0 = time.perf_counter()
    for t in pos:
        _, _, tidx, _ = O.hier_query(qidx[t], kidx, summ, int(t), w.B, w.m, w.k)
        O.sparse_attention_for_query(inp["q"][0, t].to("cpu", torch.float64).numpy(), K, V, tidx,
                                     w.scale)
        done += 1
        if time.perf_counter() - t0 > budget_s and done >= 4:
            break
    el = time.perf_counter() - t0
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        aff = os.cpu_count()
    threads = int(os.environ.get("OMP_NUM_THREADS", aff))
    return {"value": done / el, "unit": "queries/s", "cores": min(threads, aff), "kind": "oracle",
            "sample": f"{done} seeded query positions of the 64K MLA prefill (edges included), "
                      f"steps 2-5 per query (block scores, top-m, token top-k, 64-head MLA "
                      f"attention) in numpy float64; one-off block summary {t_summary:.2f} s "
                      f"not included; host cpu_count={os.cpu_count()}, affinity={aff}"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the path has no "
              "multi-GPU form in this build", file=sys.stderr)
        sys.exit(2)
    import torch

    import long_context_indexer_block_amd as H  # noqa: F401  (raises without libhisa.so)
    from long_context_indexer_block_amd.pipeline import FlatPipeline, HierPipeline
    from workloads import WORKLOADS, make_inputs

    w = WORKLOADS[a.workload]
    assert w.kind == "prefill", "the timed step is the prefill path"
    torch.cuda.set_device(0)
    log(f"generating {w.name} inputs on the GPU")
    inp = make_inputs(w, "cuda", seed=0)
    torch.cuda.synchronize()
    nq = w.batch * w.queries
    p = HierPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.B,
                     w.m, w.k, w.scale)

    stages = ["summary", "block_score", "select_blocks", "token_select", "attention"]
    calls = [
        p.summarize,
        lambda: H.hisa_block_score(p.qidx, p.q_pos, p.split, p.B, out=p.block_scores),
        lambda: H.hisa_select_blocks(p.block_scores, p.q_pos, p.B, p.m, out=p.block_idx),
        lambda: H.hisa_token_select(p.qidx, p.kidx, p.q_pos, p.block_idx, p.B, p.k_top,
                                    token_idx=p.token_idx, want_scores=False, workspace=p.ws),
        p.attend,
    ]

    def step(evs=None):
        for i, c in enumerate(calls):
            if evs is not None:
                evs[i].record()
            c()
        if evs is not None:
            evs[-1].record()

    log(f"warmup {a.warmup}")
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    # algorithmic work of the attention launch: 2*(Dk+Dv) flop per (query, head, kept token)
    n_sel = int((p.token_idx >= 0).sum().item())
    attn_flop = 2.0 * n_sel * w.Hq * (w.Dk + w.Dv)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
          for _ in range(a.steps)]
    log(f"timing {a.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(a.steps):
        step(ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = {n: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(a.steps)) / a.steps
                for i, n in enumerate(stages)}
    ms_step = wall * 1e3 / a.steps
    qps = nq * a.steps / wall
    attn_ms = stage_ms["attention"]
    achieved = attn_flop / (attn_ms * 1e-3) / 1e12
    indexer_ms = sum(stage_ms[s] for s in stages[:4])

    res = {
        "metric": METRIC, "value": qps, "unit": "queries/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "queries": nq, "L": w.L, "B": w.B,
                   "m": w.m, "k": w.k, "indexer_d": w.d_idx, "Hq": w.Hq, "Hkv": w.Hkv,
                   "Dk": w.Dk, "Dv": w.Dv, "kv": "MLA latent, V = first 512 columns of K"},
        "stage_ms": stage_ms,
        "roofline": {"kernel": "sparse_attn (MLA 576/512, 64 heads)", "bound": "mfma",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "alg_flop_per_launch": attn_flop, "kept_tokens": n_sel},
    }
    idx_flop = indexer_flop(w)
    t_roof = (attn_flop + idx_flop) / (PEAK_BF16_TFLOPS * 1e12)
    res["path_roofline"] = {"bound": "mfma", "alg_flop": attn_flop + idx_flop,
                            "t_roof_ms": t_roof * 1e3, "frac": t_roof / (ms_step * 1e-3)}
    del ev
    if not a.no_flat:
        log("flat comparison")
        del p
        torch.cuda.empty_cache()
        f = FlatPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.k,
                         w.scale)
        for _ in range(max(1, a.warmup - 1)):
            f.run()
        fs = max(2, a.steps // 2)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3 * fs)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(fs):
            e[3 * s].record()
            f.index()
            e[3 * s + 1].record()
            f.attend()
            e[3 * s + 2].record()
        torch.cuda.synchronize()
        fwall = (time.perf_counter() - t0) * 1e3 / fs
        f_idx = sum(e[3 * s].elapsed_time(e[3 * s + 1]) for s in range(fs)) / fs
        res["flat"] = {"ms_per_step": fwall, "indexer_ms": f_idx,
                       "speedup_vs_flat": fwall / ms_step,
                       "indexer_speedup_vs_flat": f_idx / indexer_ms}
        del f
    if not a.no_cpu:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(w, inp, a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
