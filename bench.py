"""Benchmark: one step = the whole hierarchical path (block summary, block
scores, top-m blocks, token top-k, sparse attention) over the 64K-token MLA
prefill (65536 queries, B=128, m=64, k=2048, 64 query heads over one
576/512 latent kv head), inputs resident in HBM.

Prints one JSON line: queries/s of the step with the token selection of
each query slab overlapping the attention of the slab before it (two
streams), per-stage milliseconds from a run of the stages one after another
(HIP events on the launch stream), the dominant kernel's roofline, the
flat-indexer comparison and the CPU oracle timed on a bounded sample of the
same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-flat] [--no-cpu]
       python bench.py --sweep [--workload NAME]   (block size / kept-block sweep)
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak
METRIC = "indexer+sparse-attn queries/s at 64K; % HBM/MFMA roofline; speedup vs flat"


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
    ap.add_argument("--overlap-slabs", type=int, default=-1,
                    help="prefill: query slabs whose token selection overlaps the attention of "
                         "the slab before (0: stages one after another; default: 16 from 32768 "
                         "queries on, 4 from 8192)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--bw-probe", type=int, default=0,
                    help="time a plain fill of this many bytes and a copy of half of them "
                         "(the HBM rates the selection kernels are compared with)")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="only run a plain device copy of this many bytes (counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="only time the indexer (steps 1-4) for block sizes 64/128/256 and "
                         "several m on this workload, one JSON line each, with the share of "
                         "the flat indexer's tokens each keeps")
    ap.add_argument("--attn-only", action="store_true",
                    help="prefill: select the tokens once, then time only the sparse attention "
                         "launch over all queries (for counter passes and kernel A/B runs)")
    ap.add_argument("--attn-ids", default="selected", choices=["selected", "hot"],
                    help="--attn-only: the selected ids, or every query reading the same "
                         "rows 0..k-1 (all served from L2: the kernel's own ceiling)")
    ap.add_argument("--attn-kept", default="",
                    help="--attn-only: comma-separated kept-token counts k' (each <= k); time "
                         "the attention over the first k' ids of every list (or rows 0..k'-1 "
                         "with --attn-ids hot) and fit time = fixed + per-token * k'")
    ap.add_argument("--gather-probe", action="store_true",
                    help="prefill: time the gather-rate probe (the attention's row gathers "
                         "alone) on the selected ids, on the same lists shifted to one hot "
                         "set of rows, and on contiguous rows; one JSON line")
    ap.add_argument("--write-counters", default="",
                    help="only summarise rocprofv3 --pmc csv folders found under this folder "
                         "(one per pass) into a markdown table (--counters-out)")
    ap.add_argument("--counters-out", default="")
    ap.add_argument("--counters-kernel", default="attn")
    ap.add_argument("--counters-title", default="")
    ap.add_argument("--counters-note", default="",
                    help="a paragraph placed under the title of a written summary")
    ap.add_argument("--counters-command", default="")
    ap.add_argument("--write-trace-md", default="",
                    help="only summarise a rocprofv3 --kernel-trace csv folder into a markdown "
                         "table of the library's kernels, split by grid size (--counters-out, "
                         "--counters-title, --counters-command)")
    ap.add_argument("--write-bytes-md", default="",
                    help="only summarise the FETCH_SIZE / WRITE_SIZE passes of a traffic "
                         "folder (fetch/, write/, cfetch/, cwrite/) per kernel and grid size "
                         "into markdown (--counters-out, --counters-title, --counters-command)")
    ap.add_argument("--write-traffic", default="",
                    help="only summarise rocprofv3 byte counters found under this folder "
                         "(fetch/, write/, cfetch/, cwrite/) into the traffic record")
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
    pos = sample_positions(w, 400)
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


def kernel_source_hash():
    import hashlib
    path = os.path.join(ROOT, "long_context_indexer_block_amd", "csrc", "attention_mla.hip")
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def measured_traffic():
    """HBM bytes per attention launch from the committed counter summary
    (rocprofv3 FETCH_SIZE and WRITE_SIZE, scaled by the factor a plain copy
    of known size gives), or None when the kernel changed since then."""
    path = os.path.join(ROOT, "profiles", "attention_mla_64k_traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_mla_64k_traffic.json")
TRAFFIC_PASSES = {
    "fetch": "FETCH_SIZE", "write": "WRITE_SIZE", "cfetch": "FETCH_SIZE", "cwrite": "WRITE_SIZE"}


def counter_rows(folder, counter):
    """(kernel name, value, grid size) of every dispatch in a rocprofv3 counter csv."""
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter csv under {folder}")
    rows = []
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"]),
                             int(r.get("Grid_Size") or 0)))
    return rows


def write_traffic(folder, copy_bytes=1 << 30):
    """Traffic record of the MLA attention kernel from four counter passes:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of one bench step, and the
    same counters over a plain copy of `copy_bytes`, whose known size gives
    the factor from counter units to bytes. The step launches the attention
    over all queries (the launch the roofline times) and per query slab: only
    the all-query launches (the largest grid) are taken."""
    def one(sub, pick):
        rows = [(v, gsz) for name, v, gsz in
                counter_rows(os.path.join(folder, sub), TRAFFIC_PASSES[sub]) if pick(name)]
        if not rows:
            raise SystemExit(f"no matching dispatch in {sub}")
        top = max(gsz for _, gsz in rows)
        return [v for v, gsz in rows if gsz == top]
    attn = lambda n: "mla_attn_kernel" in n
    copy = lambda n: "copyBuffer" in n or ("copy" in n.lower() and "Fill" not in n)
    f_kib = one("fetch", attn)
    w_kib = one("write", attn)
    cf = max(one("cfetch", copy))
    cw = max(one("cwrite", copy))
    fs, ws = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    fk, wk = sum(f_kib) / len(f_kib), sum(w_kib) / len(w_kib)
    rec = {
        "kernel": "hisa::mla::mla_attn_kernel", "workload": "prefill_64k_mla",
        "source_file": "long_context_indexer_block_amd/csrc/attention_mla.hip",
        "source_sha256": kernel_source_hash(),
        "fetch_size_kib": fk, "write_size_kib": wk, "copy_probe_bytes": copy_bytes,
        "copy_fetch_size_kib": cf, "copy_write_size_kib": cw,
        "fetch_scale": fs, "write_scale": ws,
        "hbm_bytes_per_launch": int(round(fk * 1024 * fs + wk * 1024 * ws)),
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/fetch -o run -- "
            "python3 bench.py --no-cpu --no-flat --steps 1 --warmup 0",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/write -o run -- "
            "python3 bench.py --no-cpu --no-flat --steps 1 --warmup 0",
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/cfetch -o run -- "
            f"python3 bench.py --copy-probe {copy_bytes}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/cwrite -o run -- "
            f"python3 bench.py --copy-probe {copy_bytes}",
            "python3 bench.py --write-traffic <dir>"],
    }
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def copy_probe(nbytes):
    """A plain device copy of `nbytes` (for calibrating the byte counters)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes}))


def bw_probe(nbytes, reps=20):
    """HIP-event times of a plain fill of `nbytes` and of a copy of nbytes/2
    (read and write): the rates of simple streaming kernels on this chip."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty(nbytes // 8, dtype=torch.float32, device="cuda")
    c = torch.empty_like(b)
    def ms(f):
        for _ in range(3):
            f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    fill = ms(lambda: a.fill_(1.0))
    copy = ms(lambda: c.copy_(b))
    print(json.dumps({"bw_probe_bytes": nbytes, "fill_ms": fill, "fill_TBps": nbytes / fill / 1e9,
                      "copy_bytes": nbytes // 2, "copy_ms": copy,
                      "copy_TBps_read_plus_write": nbytes / copy / 1e9}))


def timed(calls, steps, warmup):
    """Run `calls` (a list of thunks) as one step; HIP events around each."""
    import torch
    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        for i, c in enumerate(calls):
            ev[s][i].record()
            c()
        ev[s][-1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage = [sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)) / steps
             for i in range(len(calls))]
    return wall, stage


def graph_ms(call_groups, steps):
    """Capture each list of calls as one HIP graph (the calls enqueue kernel
    launches only) and time `steps` replays, round-robin over the graphs,
    with the host clock between synchronisations. Returns ms per replay."""
    import torch
    graphs = []
    for calls in call_groups:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in calls:
                c()
        graphs.append(g)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        graphs[s % len(graphs)].replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def base_record(w, a, nq, wall, dtype="bf16"):
    ms_step = wall * 1e3 / a.steps
    return {
        "metric": METRIC, "value": nq * a.steps / wall, "unit": "queries/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": w.name, "kind": w.kind, "batch": w.batch, "queries": nq, "L": w.L,
                   "B": w.B, "m": w.m, "k": w.k, "indexer_d": w.d_idx, "Hq": w.Hq,
                   "Hkv": w.Hkv, "Dk": w.Dk, "Dv": w.Dv},
    }


def bench_prefill(w, a, inp):
    import torch

    import long_context_indexer_block_amd as H
    from long_context_indexer_block_amd.pipeline import FlatPipeline, HierPipeline

    nq = w.batch * w.queries
    # query slabs whose token selection overlaps the attention of the slab before
    slabs = a.overlap_slabs if a.overlap_slabs >= 0 else (
        16 if nq >= 32768 else 4 if nq >= 8192 else 0)
    p = HierPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.B,
                     w.m, w.k, w.scale, overlap_slabs=slabs)
    stages = ["summary", "block_score", "select_blocks", "token_select", "attention"]
    calls = [
        p.summarize,
        lambda: H.hisa_block_score(p.qidx, p.q_pos, p.split, p.B, out=p.block_scores),
        lambda: H.hisa_select_blocks(p.block_scores, p.q_pos, p.B, p.m, out=p.block_idx),
        lambda: H.hisa_token_select(p.qidx, p.kidx, p.q_pos, p.block_idx, p.B, p.k_top,
                                    token_idx=p.token_idx, want_scores=False, workspace=p.ws),
        p.attend,
    ]
    log(f"timing {a.steps} steps (warmup {a.warmup}), stages one after another")
    wall_seq, stage = timed(calls, a.steps, a.warmup)
    stage_ms = dict(zip(stages, stage))
    log(f"timing {a.steps} steps (warmup {a.warmup}), slabs overlapped")
    wall, _ = timed([p.run_overlapped], a.steps, a.warmup)
    # algorithmic work of the attention launch: 2*(Dk+Dv) flop per (query, head, kept token)
    n_sel = int((p.token_idx >= 0).sum().item())
    attn_flop = 2.0 * n_sel * w.Hq * (w.Dk + w.Dv)
    achieved = attn_flop / (stage_ms["attention"] * 1e-3) / 1e12
    res = base_record(w, a, nq, wall)
    ms_step = res["ms_per_step"]
    res["config"]["kv"] = ("MLA latent, V = first 512 columns of K" if w.mla else
                           f"{w.Hkv} kv head(s)")
    res["stage_ms"] = stage_ms
    res["sequential"] = {"ms_per_step": wall_seq * 1e3 / a.steps,
                         "note": "stages one after another; stage_ms are from this run",
                         "overlap_slabs": len(p.slabs)}
    # the same step replayed as one HIP graph (no per-launch host cost)
    g_ms = graph_ms([calls], a.steps)
    res["graph"] = {"ms_per_step": g_ms, "queries_per_s": nq / (g_ms * 1e-3)}
    traffic = measured_traffic() if (w.mla and w.name == "prefill_64k_mla") else None
    res["roofline"] = {"kernel": f"sparse_attn ({w.Hq} heads, Dk {w.Dk}, Dv {w.Dv})",
                       "scope": "the dominant kernel, one launch over all queries; the whole "
                                "step against its roofline is path_roofline",
                       "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                       "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                       "traffic": traffic, "alg_flop_per_launch": attn_flop,
                       "kept_tokens": n_sel}
    # the measured memory-side ceiling: the same rows gathered and discarded
    g_ms, g_w, g_d = gather_ceiling(w, inp, p.token_idx[0].contiguous(), max(3, a.steps // 3))
    res["gather_ceiling"] = {
        "probe_ms": g_ms, "attention_ms": stage_ms["attention"],
        "frac": g_ms / stage_ms["attention"], "probe_waves": g_w, "probe_depth": g_d,
        "note": "hisa_gather_probe on the attention's own id lists (list order): the time the "
                "row gathers alone take; frac = that / the attention launch"}
    idx_flop = indexer_flop(w)
    t_roof = (attn_flop + idx_flop) / (PEAK_BF16_TFLOPS * 1e12)
    res["path_roofline"] = {"bound": "mfma", "alg_flop": attn_flop + idx_flop,
                            "t_roof_ms": t_roof * 1e3, "frac": t_roof / (ms_step * 1e-3)}
    if not a.no_flat:
        log("flat comparison")
        ws_needed = H.flat_indexer_topk_workspace_bytes(w.batch, w.queries, w.L, w.k)
        del p
        torch.cuda.empty_cache()
        # the flat step runs with the same slabs and overlap as the hierarchical one
        f = FlatPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"],
                         w.k, w.scale, overlap_slabs=slabs)
        fs = max(2, a.steps // 2)
        fwall_seq, fstage = timed([f.index, f.attend], fs, max(1, a.warmup - 1))
        fwall, _ = timed([f.run_overlapped], fs, max(1, a.warmup - 1))
        f_ms = fwall * 1e3 / fs
        idx_ms = sum(stage_ms[s] for s in stages[:4])
        res["flat"] = {"ms_per_step": f_ms, "sequential_ms_per_step": fwall_seq * 1e3 / fs,
                       "indexer_ms": fstage[0], "attention_ms": fstage[1],
                       "workspace_bytes": ws_needed, "speedup_vs_flat": f_ms / ms_step,
                       "indexer_speedup_vs_flat": fstage[0] / idx_ms}
        del f
    return res


def attn_table(w, inp):
    """The K table the attention gathers from as [L, row] (batch 1), and its
    row width in bytes: the 576-wide latent row, or one kv head's K row."""
    k = inp["k"][0, :, 0, :]
    return k, k.shape[-1] * k.element_size()


def time_launch(fn, steps, warmup=1):
    """Mean milliseconds of fn() over `steps` calls, HIP events on the current
    stream (the one every binding call enqueues on)."""
    import torch
    for _ in range(warmup):
        fn()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def gather_ceiling(w, inp, ids, steps, configs=((4, 2), (8, 1), (8, 2), (4, 3))):
    """Best time of the gather-rate probe over `configs` (waves, depth) on the
    id lists the attention reads, in list order: the time that gathering those
    rows alone takes (twice the K-row time when K and V are separate rows).
    Returns (ms, waves, depth)."""
    import long_context_indexer_block_amd as H
    table, row_bytes = attn_table(w, inp)
    rows_per_token = 1 if w.mla else 2
    best = None
    for wv, dp in configs:
        ms = rows_per_token * time_launch(
            lambda: H.hisa_gather_probe(table, ids, row_bytes, wv, dp, 0), steps)
        if best is None or ms < best[0]:
            best = (ms, wv, dp)
    return best


def bench_attn_only(w, a, inp):
    """Select the tokens once, then time the attention launch over all queries
    alone (HIP events on its stream)."""
    from long_context_indexer_block_amd.pipeline import HierPipeline
    p = HierPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.B,
                     w.m, w.k, w.scale)
    p.index()
    if a.attn_ids == "hot":
        import torch
        nq, k = p.token_idx.shape[1], p.token_idx.shape[2]
        p.token_idx.copy_(torch.arange(k, dtype=torch.int32, device=p.token_idx.device)
                          .expand_as(p.token_idx))
    ms = time_launch(p.attend, a.steps, a.warmup)
    n_sel = int((p.token_idx >= 0).sum().item())
    flop = 2.0 * n_sel * w.Hq * (w.Dk + w.Dv)
    tf = flop / (ms * 1e-3) / 1e12
    return {"attn_only": w.name, "ids": a.attn_ids, "ms": ms, "tflops": tf,
            "frac_mfma": tf / PEAK_BF16_TFLOPS,
            "kept_tokens": n_sel, "steps": a.steps, "warmup": a.warmup}


def bench_attn_kept(w, a, inp):
    """The attention launch over all queries on the first k' ids of each
    selected list (contiguous copies), for several k': the least-squares line
    time = fixed + per_token * k' separates the cost that scales with the
    kept tokens from the part that does not (the Q rows read and the output
    rows written once per query)."""
    import numpy as np
    import torch
    import long_context_indexer_block_amd as H
    from long_context_indexer_block_amd.pipeline import HierPipeline
    p = HierPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.B,
                     w.m, w.k, w.scale)
    p.index()
    nq = p.token_idx.shape[1]
    ks = sorted(int(x) for x in a.attn_kept.split(","))
    if ks[0] < 1 or ks[-1] > w.k:
        raise SystemExit(f"--attn-kept values must lie in 1..{w.k}")
    ms = []
    for kk in ks:
        if a.attn_ids == "hot":
            ids = torch.arange(kk, dtype=torch.int32, device="cuda").expand(1, nq, kk).contiguous()
        else:
            ids = p.token_idx[:, :, :kk].contiguous()
        ms.append(time_launch(lambda: H.sparse_attn_fwd(p.q, p.k, p.v, ids, w.scale, out=p.out,
                                                        workspace=p.attn_ws), a.steps, a.warmup))
        log(f"k'={kk}: {ms[-1]:.3f} ms")
    slope, fixed = np.polyfit(np.array(ks, dtype=np.float64), np.array(ms), 1)
    return {"attn_kept": w.name, "ids": a.attn_ids, "queries": nq, "kept": ks, "ms": ms,
            "fixed_ms": fixed, "ms_per_1024_tokens": slope * 1024,
            "fixed_us_per_query_per_cu": fixed * 1e3 / (nq / 256),
            "steps": a.steps, "warmup": a.warmup}


def bench_gather_probe(w, a, inp):
    """The gather-rate probe on id sets of the workload's shape: the ids the
    hierarchical selection keeps (also read in a clock-rotated order, see
    hisa_gather_probe), the same count of rows shared by every query (served
    from L2), contiguous rows per query, uniformly random rows of the table
    (no sharing between neighbouring queries), and uniformly random rows of a
    4 GB table (beyond the last-level cache); the attention launch on the kept
    ids timed beside them."""
    import torch

    import long_context_indexer_block_amd as H
    from long_context_indexer_block_amd.pipeline import HierPipeline
    p = HierPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.B,
                     w.m, w.k, w.scale)
    p.index()
    ids = p.token_idx[0].contiguous()
    nq, topk = ids.shape
    dev = ids.device
    table, row_bytes = attn_table(w, inp)
    g = torch.Generator(device=dev).manual_seed(5)
    hot = torch.arange(topk, dtype=torch.int32, device=dev).expand(nq, topk).contiguous()
    seq = ((torch.arange(nq, dtype=torch.int64, device=dev)[:, None] * 97 +
            torch.arange(topk, dtype=torch.int64, device=dev)[None]) % w.L).to(torch.int32)
    uni = torch.randint(0, w.L, (nq, topk), generator=g, device=dev, dtype=torch.int32)
    big_rows = (4 << 30) // row_bytes
    big = torch.empty(big_rows, row_bytes // 2, dtype=torch.bfloat16, device=dev)
    uni_big = torch.randint(0, big_rows, (nq, topk), generator=g, device=dev, dtype=torch.int32)
    rows_read = nq * (-(-topk // 32) * 32)
    out = {"gather_probe": w.name, "row_bytes": row_bytes, "rows_per_launch": rows_read,
           "bytes_per_launch": rows_read * row_bytes, "results": []}
    grid = ((4, 1), (4, 2), (4, 3), (8, 1), (8, 2), (8, 3))
    runs = [("selected", ids, table, wv, dp, 0) for wv, dp in grid]
    runs += [("selected_rotated", ids, table, wv, dp, r) for wv, dp in ((4, 2), (8, 1))
             for r in (32, 64, 128, 256)]
    runs += [("hot_rows", hot, table, wv, dp, 0) for wv, dp in ((4, 2), (8, 1))]
    runs += [("contiguous", seq, table, wv, dp, 0) for wv, dp in ((4, 2), (8, 1))]
    runs += [("uniform", uni, table, wv, dp, 0) for wv, dp in ((4, 2), (8, 1), (8, 2))]
    runs += [("uniform_4GB_table", uni_big, big, wv, dp, 0) for wv, dp in ((4, 2), (8, 1), (8, 2))]
    for name, idset, tab, wv, dp, rot in runs:
        ms = time_launch(lambda: H.hisa_gather_probe(tab, idset, row_bytes, wv, dp, rot), a.steps)
        out["results"].append({"ids": name, "waves": wv, "depth": dp, "rot_ticks": rot, "ms": ms,
                               "GBps": rows_read * row_bytes / (ms * 1e-3) / 1e9})
    ams = time_launch(p.attend, a.steps)
    out["attention_ms"] = ams
    # the attention kernels gather each kept token's K row and, unless V is
    # the latent row itself, its V row as well
    per_token = row_bytes if w.mla else row_bytes * 2
    out["attention_gather_GBps"] = rows_read * per_token / (ams * 1e-3) / 1e9
    return out


def _short(name):
    return name.split("(")[0].replace("void ", "")


def write_trace_md(folder, out_path, title, command, note=""):
    """Per (kernel, grid size) of the library's kernels (namespace hisa) in a
    rocprofv3 kernel trace: calls, mean / median / min / max duration in us
    and share of the GPU time of all dispatches in the trace. The median
    leaves out the first, cold call of a short run (the bench's timed region
    excludes its warm-up calls)."""
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel trace under {folder}")
    per, total = {}, 0.0
    for f in files:
        for r in csv.DictReader(open(f)):
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            total += d
            if "hisa::" not in r["Kernel_Name"]:
                continue
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            per.setdefault((_short(r["Kernel_Name"]), grid), []).append(d)
    rows = sorted(per.items(), key=lambda kv: -sum(kv[1]))
    lines = [f"# {title}", ""] + ([note.strip(), ""] if note else []) + [
             "Command (repository root, on the GPU host):", "", "```",
             command.strip(), "```", "",
             "Durations in microseconds (rocprofv3 kernel trace); rows split by grid size "
             "(threads); the share is of all GPU time in the trace (input generation included).",
             "", "| kernel | grid (threads) | calls | avg us | median us | min us | max us | "
             "% of GPU time |",
             "|---|---|---|---|---|---|---|---|"]
    for (name, grid), ds in rows:
        sd = sorted(ds)
        med = sd[len(sd) // 2] if len(sd) % 2 else 0.5 * (sd[len(sd) // 2 - 1] + sd[len(sd) // 2])
        lines.append(f"| `{name}` | {grid:,} | {len(ds)} | {sum(ds) / len(ds):.1f} | {med:.1f} | "
                     f"{min(ds):.1f} | {max(ds):.1f} | {100 * sum(ds) / total:.2f} |")
    text = "\n".join(lines) + "\n"
    if out_path:
        with open(out_path, "w") as fh:
            fh.write(text)
    print(text)


def write_bytes_md(folder, out_path, title, command, note="", copy_bytes=1 << 30):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the library's kernels
    per (kernel, grid size), scaled to bytes by the factors a plain copy of
    `copy_bytes` gives (its fetch and write counts against its size)."""
    def rows(sub, counter):
        out = {}
        for name, v, grid in counter_rows(os.path.join(folder, sub), counter):
            out.setdefault((_short(name), grid), []).append(v)
        return out
    copy = lambda n: "copyBuffer" in n or ("copy" in n.lower() and "Fill" not in n)
    cf = max(v for (n, _), vs in rows("cfetch", "FETCH_SIZE").items() if copy(n) for v in vs)
    cw = max(v for (n, _), vs in rows("cwrite", "WRITE_SIZE").items() if copy(n) for v in vs)
    fs, ws = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    fe, wr = rows("fetch", "FETCH_SIZE"), rows("write", "WRITE_SIZE")
    lines = [f"# {title}", ""] + ([note.strip(), ""] if note else []) + [
             "Commands (repository root, each a run of its own):", "", "```",
             command.strip(), "```", "",
             f"Calibration: a plain {copy_bytes:,}-byte device copy reads FETCH_SIZE = "
             f"{cf:,.2f} KiB and WRITE_SIZE = {cw:,.2f} KiB, so fetch counts are scaled by "
             f"{fs:.5f} and write counts by {ws:.5f}. The counters sit between L2 and the "
             "memory fabric: reads the Infinity Cache serves count as well.", "",
             "| kernel | grid (threads) | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB (scaled) | "
             "written GB (scaled) |", "|---|---|---|---|---|---|"]
    for key in fe:
        if "hisa::" not in key[0] or key not in wr:
            continue
        f_kib = sum(fe[key]) / len(fe[key])
        w_kib = sum(wr[key]) / len(wr[key])
        lines.append(f"| `{key[0]}` | {key[1]:,} | {f_kib:,.1f} | {w_kib:,.1f} | "
                     f"{f_kib * 1024 * fs / 1e9:.3f} | {w_kib * 1024 * ws / 1e9:.3f} |")
    text = "\n".join(lines) + "\n"
    if out_path:
        with open(out_path, "w") as fh:
            fh.write(text)
    print(text)


N_XCD, N_CU, N_SIMD, CLOCK_GHZ = 8, 256, 1024, 2.4   # MI355X


def write_counters(folder, out_path, kernel_sub, title="", command="", note=""):
    """Summarise rocprofv3 --pmc csv folders (one per pass, any names) for the
    dispatches of kernels whose name holds `kernel_sub`, largest grid only:
    the mean of every counter per dispatch and the figures derived from them.
    GRBM_GUI_ACTIVE comes summed over the eight XCDs, so the kernel's cycles
    are that / 8; MFMA busy is SQ_VALU_MFMA_BUSY_CYCLES per SIMD over those
    cycles, and over the cycles of the datasheet clock (2.4 GHz) in the
    dispatch's measured duration; LDS bank-conflict cycles are set against
    the cycles the LDS was busy with indexed operations; L2 hit rate is
    TCC_HIT / (TCC_HIT + TCC_MISS)."""
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(folder, "**", "*counter_collection.csv"),
                             recursive=True))
    if not files:
        raise SystemExit(f"no counter csv under {folder}")
    per = {}
    dur = {}
    for f in files:
        rows = [r for r in csv.DictReader(open(f)) if kernel_sub in r["Kernel_Name"]]
        if not rows:
            continue
        top = max(int(r.get("Grid_Size") or 0) for r in rows)
        for r in rows:
            if int(r.get("Grid_Size") or 0) != top:
                continue
            key = (r["Kernel_Name"].split("(")[0], top)
            d = per.setdefault(key, {})
            d.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            dur.setdefault(key, {})[(f, r["Dispatch_Id"])] = (
                int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines = [f"# {title}", ""] if title else []
    if note:
        lines += [note.strip(), ""]
    if command:
        lines += ["Commands (repository root, each pass a run of its own):", "", "```",
                  command.strip(), "```", ""]
    for (name, grid), d in per.items():
        avg = {c: sum(v) / len(v) for c, v in d.items()}
        ds = list(dur[(name, grid)].values())
        ns = sum(ds) / len(ds)
        lines.append(f"## `{name}` (grid {grid:,} threads)\n")
        lines.append(f"Mean dispatch duration under the counter runs: {ns / 1e6:.3f} ms "
                     f"({len(ds)} dispatches).\n")
        lines.append("| counter | mean per dispatch | dispatches |")
        lines.append("|---|---|---|")
        for c in sorted(avg):
            lines.append(f"| {c} | {avg[c]:,.0f} | {len(d[c])} |")
        der = []
        gui = avg.get("GRBM_GUI_ACTIVE")
        cyc = gui / N_XCD if gui else None
        if cyc:
            der.append(("kernel cycles (GRBM_GUI_ACTIVE / 8 XCDs)", f"{cyc:,.0f}"))
            der.append(("clock implied (cycles / duration)", f"{cyc / ns:.3f} GHz"))
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD
            der.append(("MFMA busy cycles per SIMD", f"{busy:,.0f}"))
            if cyc:
                der.append(("MFMA busy / kernel cycles", f"{busy / cyc:.3f}"))
            der.append(("MFMA busy / (duration x 2.4 GHz): fraction of the datasheet peak",
                        f"{busy / (ns * CLOCK_GHZ):.3f}"))
        if "SQ_LDS_BANK_CONFLICT" in avg and avg.get("SQ_LDS_IDX_ACTIVE"):
            der.append(("LDS bank-conflict cycles / LDS indexed-active cycles",
                        f"{avg['SQ_LDS_BANK_CONFLICT'] / avg['SQ_LDS_IDX_ACTIVE']:.3f}"))
        if "SQ_LDS_BANK_CONFLICT" in avg and avg.get("SQ_ACTIVE_INST_LDS"):
            der.append(("LDS bank-conflict cycles / SQ_ACTIVE_INST_LDS",
                        f"{avg['SQ_LDS_BANK_CONFLICT'] / avg['SQ_ACTIVE_INST_LDS']:.3f}"))
        if cyc and "SQ_LDS_IDX_ACTIVE" in avg:
            der.append(("LDS indexed-active cycles per CU / kernel cycles",
                        f"{avg['SQ_LDS_IDX_ACTIVE'] / N_CU / cyc:.3f}"))
        if "TCC_HIT_sum" in avg and "TCC_MISS_sum" in avg:
            tot = avg["TCC_HIT_sum"] + avg["TCC_MISS_sum"]
            if tot:
                der.append(("L2 hit rate (TCC_HIT / (TCC_HIT + TCC_MISS))",
                            f"{avg['TCC_HIT_sum'] / tot:.3f}"))
        waves = grid / 64.0
        for c in ("SQ_INSTS_LDS", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_SALU"):
            if c in avg:
                der.append((f"{c} per wave", f"{avg[c] / waves:,.1f}"))
        if "SQ_WAIT_INST_LDS" in avg and "SQ_WAVE_CYCLES" in avg and avg["SQ_WAVE_CYCLES"]:
            der.append(("SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES (share of wave time waiting to "
                        "issue LDS)", f"{avg['SQ_WAIT_INST_LDS'] / avg['SQ_WAVE_CYCLES']:.3f}"))
        if der:
            lines.append("")
            lines.append("| derived | value |")
            lines.append("|---|---|")
            for k, v in der:
                lines.append(f"| {k} | {v} |")
        lines.append("")
    text = "\n".join(lines)
    if out_path:
        with open(out_path, "w") as fh:
            fh.write(text + "\n")
    print(text)


def bench_decode(w, a, inp):
    import torch

    import long_context_indexer_block_amd as H
    from long_context_indexer_block_amd.pipeline import HierPipeline

    nq = w.batch * w.queries
    p = HierPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.B,
                     w.m, w.k, w.scale)
    # the block summaries belong to the cache: built once, timed apart
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    p.summarize()
    e1.record()
    torch.cuda.synchronize()
    summary_ms = e0.elapsed_time(e1)
    # Per-step HBM bytes exceed a single step's cache reuse only if the cache
    # is cold: rotate through 4 query sets so the 235 MB working set of one
    # step is not served from the 256 MB last-level cache every time.
    qsets = [inp["qidx"]] + [torch.roll(inp["qidx"], shifts=i, dims=0) for i in (1, 2, 3)]
    qs = [inp["q"]] + [torch.roll(inp["q"], shifts=i, dims=0) for i in (1, 2, 3)]
    state = {"i": 0}

    def pick():
        i = state["i"] = (state["i"] + 1) % 4
        p.qidx, p.q = qsets[i], qs[i]

    # one query per sequence: block scores and top-m blocks in one call, the
    # blocks of each query split over several workgroups (same block_idx)
    n_rows = p.split.shape[1]
    route_ws = H.route_workspace(w.batch, w.queries, n_rows, w.m, p.split.device)
    if route_ws is not None:
        stages = ["rotate_query_set", "route", "token_select", "attention"]
        route = [lambda: H.hisa_route_blocks(p.qidx, p.q_pos, p.split, p.B, p.m, out=p.block_idx,
                                             workspace=route_ws)]
    else:
        stages = ["rotate_query_set", "block_score", "select_blocks", "token_select", "attention"]
        route = [lambda: H.hisa_block_score(p.qidx, p.q_pos, p.split, p.B, out=p.block_scores),
                 lambda: H.hisa_select_blocks(p.block_scores, p.q_pos, p.B, p.m,
                                              out=p.block_idx)]
    calls = [pick] + route + [
        lambda: H.hisa_token_select(p.qidx, p.kidx, p.q_pos, p.block_idx, p.B, p.k_top,
                                    token_idx=p.token_idx, want_scores=False, workspace=p.ws),
        p.attend,
    ]
    # the step as one call (as the prefill steps are timed); the per-stage
    # times come from a second run with an event between the stages, which
    # is instrumentation, not part of the step
    wall_staged, stage = timed(calls, a.steps, a.warmup)
    wall, _ = timed([lambda: [c() for c in calls]], a.steps, a.warmup)
    res = base_record(w, a, nq, wall)
    res["stage_ms"] = dict(zip(stages, stage))
    res["staged"] = {"ms_per_step": wall_staged * 1e3 / a.steps,
                     "note": "the same step with an event between stages; stage_ms are from "
                             "this run"}
    res["summary_build_ms"] = summary_ms
    # the same step captured as HIP graphs, one per query set, and replayed:
    # the per-launch host cost goes away
    def use(i):
        p.qidx, p.q = qsets[i], qs[i]
    g_ms = graph_ms([[lambda i=i: use(i)] + calls[1:] for i in range(4)], a.steps)
    res["graph"] = {"ms_per_step": g_ms, "queries_per_s": nq / (g_ms * 1e-3)}
    # per-step compulsory HBM bytes: summaries (hi/mid/lo), the kept blocks'
    # keys, the kept tokens' K and V rows
    n_sel = int((p.token_idx >= 0).sum().item())
    nblk_kept = int((p.block_idx >= 0).sum().item())
    # (fp32 block summaries of the candidate blocks, as the method defines them;
    # the kernel reads their exact bf16 hi/mid/lo form, 1.5x these bytes)
    bytes_step = (w.batch * w.n_blocks * w.d_idx * 4 + nblk_kept * w.B * w.d_idx * 2 +
                  n_sel * (w.Dk + w.Dv) * 2 * w.Hkv)
    ms = res["ms_per_step"]
    res["roofline"] = {"kernel": "whole decode step", "bound": "hbm",
                       "achieved": bytes_step / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                       "unit": "GB/s", "frac": bytes_step / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                       "traffic": None, "alg_bytes_per_step": bytes_step}
    return res


def bench_hils(w, a, inp):
    import torch

    from long_context_indexer_block_amd.pipeline import HilsDecode

    sc = 1.0 / math.sqrt(w.Dk)
    hd = HilsDecode(inp["q"], inp["k"], inp["v"], inp["w_proj"], w.B, w.m, sc, sc)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    hd.build_keys()
    e1.record()
    torch.cuda.synchronize()
    # the step as one call; per-stage times from a run with an event between
    # the stages (instrumentation, not part of the step)
    wall_staged, stage = timed([hd.route, hd.attend], a.steps, a.warmup)
    wall, _ = timed([lambda: (hd.route(), hd.attend())], a.steps, a.warmup)
    res = base_record(w, a, w.batch * w.Hq, wall)
    res["config"]["queries"] = w.batch
    res["value"] = w.batch * a.steps / wall
    res["stage_ms"] = {"route": stage[0], "two_level_attention": stage[1]}
    res["staged"] = {"ms_per_step": wall_staged * 1e3 / a.steps,
                     "note": "the same step with an event between stages; stage_ms are from "
                             "this run"}
    g_ms = graph_ms([[hd.route, hd.attend]], a.steps)
    res["graph"] = {"ms_per_step": g_ms, "queries_per_s": w.batch / (g_ms * 1e-3)}
    res["chunk_key_build_ms"] = e0.elapsed_time(e1)
    n = hd.n
    # fp32 chunk keys of every chunk, then the chosen chunks' K and V rows
    bytes_step = (w.batch * w.Hq * n * w.Dk * 4 +
                  w.batch * w.Hq * w.m * w.B * w.Dk * 2 * 2)
    ms = res["ms_per_step"]
    res["roofline"] = {"kernel": "whole two-level decode step", "bound": "hbm",
                       "achieved": bytes_step / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                       "unit": "GB/s", "frac": bytes_step / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                       "traffic": None, "alg_bytes_per_step": bytes_step}
    return res


PEAK_FP32_VEC_TFLOPS = 157.3   # MI355X fp32 vector peak (256 CUs x 2.4 GHz x 256 flop/clk)


def hils_prefill_flop(w):
    """Algorithmic vector work of one causal two-level prefill: per (query,
    head), 4*D flop per attended token (its score and its share of the value
    sum), 2*D per chosen chunk (the chunk logit) and 2*D*D for the local
    chunk's projected key. A query at t keeps min(t//C + 1, m) chunks: the
    complete ones hold C tokens, the local one t - (t//C)*C + 1."""
    import numpy as np
    t = np.arange(w.L - w.queries, w.L, dtype=np.int64)
    bt = t // w.B
    chunks = np.minimum(bt + 1, w.m)
    tokens = (chunks - 1) * w.B + (t - bt * w.B + 1)
    D = w.Dk
    per_head = 4 * D * tokens.sum() + 2 * D * chunks.sum() + 2 * D * D * t.size
    return float(per_head * w.Hq * w.batch)


def hils_prefill_bytes(w):
    """Algorithmic HBM bytes of one bucketed two-level attention call (the
    entries are the (query, head, chosen chunk) triples, min(t//C + 1, m) per
    query and head):
      bucketing   chunk ids read twice, entry ids written: 12 B per id slot;
      local keys  K read once (2D B per token and head), the fp32 key table
                  written (4D B);
      tiles       per entry the query row (2D B) read and the fp16 partial
                  row (2D B), its exponent and logit (5 B) written; each
                  chunk's K and V rows (4CD B) read once per head;
      combine     per entry the partial row, exponent, logit and chunk id
                  (2D + 9 B) read; per query and head the output row (2D B)
                  written."""
    import numpy as np
    t = np.arange(w.L - w.queries, w.L, dtype=np.int64)
    entries = float(np.minimum(t // w.B + 1, w.m).sum()) * w.Hq * w.batch
    slots = float(w.queries * w.m * w.Hq * w.batch)
    D, C = w.Dk, w.B
    heads = w.Hq * w.batch
    n_chunks = -(-w.L // C)
    return (12 * slots + 6 * D * w.L * heads + entries * (4 * D + 5) + 4 * C * D * n_chunks * heads
            + entries * (2 * D + 9) + 2 * D * w.queries * heads)


def bench_hils_prefill(w, a, inp):
    from long_context_indexer_block_amd.pipeline import HilsPrefill

    sc = 1.0 / math.sqrt(w.Dk)
    hp = HilsPrefill(inp["q"], inp["k"], inp["v"], inp["w_proj"], inp["q_pos"], w.B, w.m, sc, sc)
    wall, stage = timed([hp.build_keys, hp.route, hp.attend], a.steps, a.warmup)
    res = base_record(w, a, w.batch * w.queries, wall)
    res["stage_ms"] = {"chunk_keys": stage[0], "route": stage[1], "two_level_attention": stage[2]}
    nbytes = hils_prefill_bytes(w)
    ach = nbytes / (stage[2] * 1e-3) / 1e9
    res["roofline"] = {"kernel": "two-level attention call (bucketing, local keys, tiles, "
                                 "combine)", "bound": "hbm", "achieved": ach,
                       "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                       "traffic": None, "alg_bytes_per_launch": nbytes,
                       "vector_flop_per_launch": hils_prefill_flop(w)}
    return res


def cpu_baseline_hils_prefill(w, inp, budget_s):
    """The CPU oracle on a bounded sample of the two-level prefill: seeded
    (position, head) queries until the time budget is spent; the chunk keys
    of the sampled heads are built once beforehand and not timed."""
    import numpy as np
    import torch

    import oracle.hisa_oracle as O
    from workloads import sample_positions

    Wp = inp["w_proj"].to("cpu", torch.float64).numpy()
    heads = [0, w.Hq // 2, w.Hq - 1]
    kv = {}
    for h in heads:
        K = inp["k"][0, :, h].to("cpu", torch.float64).numpy()
        V = inp["v"][0, :, h].to("cpu", torch.float64).numpy()
        kv[h] = (K, V, O.block_summary(K, w.B, proj=Wp))
    pos = sample_positions(w, 20000)
    rng = np.random.default_rng(0)
    rng.shuffle(pos)
    first = w.L - w.queries
    sc = 1.0 / math.sqrt(w.Dk)
    done = 0
    t0 = time.perf_counter()
    for i, t in enumerate(pos):
        h = heads[i % len(heads)]
        K, V, khat = kv[h]
        q = inp["q"][0, t - first, h].to("cpu", torch.float64).numpy()
        O.hils_prefill_query(q, K, V, Wp, khat, int(t), w.B, w.m, sc, sc)
        done += 1
        if time.perf_counter() - t0 > budget_s and done >= 4:
            break
    el = time.perf_counter() - t0
    aff = len(os.sched_getaffinity(0))
    threads = int(os.environ.get("OMP_NUM_THREADS", aff))
    # one query position covers all Hq heads
    return {"value": done / el / w.Hq, "unit": "queries/s", "cores": min(threads, aff),
            "kind": "oracle",
            "sample": f"{done} seeded (position, head) queries of the {w.name} prefill in numpy "
                      f"float64 (routing and two-level softmax), scaled to positions of all "
                      f"{w.Hq} heads; chunk keys built beforehand, not timed"}


def recall_vs_flat(hier_idx, flat_idx, chunk=4096):
    """Mean over queries of |hier ∩ flat| / |flat| for ascending, -1 padded
    token lists [b, nq, k] (the flat indexer's exact top-k as the reference)."""
    import torch
    hit = tot = 0
    h2 = hier_idx.reshape(-1, hier_idx.shape[-1])
    f2 = flat_idx.reshape(-1, flat_idx.shape[-1])
    for i in range(0, h2.shape[0], chunk):
        h, f = h2[i:i + chunk], f2[i:i + chunk].contiguous()
        # the -1 padding sits after the ids: map it past them to keep rows sorted
        h = torch.where(h < 0, torch.iinfo(torch.int32).max, h).contiguous()
        pos = torch.searchsorted(h, f).clamp_(max=h.shape[1] - 1)
        found = (h.gather(1, pos) == f) & (f >= 0)
        n = (f >= 0).sum(1).clamp_(min=1)
        hit += (found.sum(1).double() / n.double()).sum().item()
        tot += h.shape[0]
    return hit / tot


def bench_sweep(w, a, inp):
    """Block size and kept-block sweep of the hierarchical indexer (steps 1-4,
    the cost the two knobs move; the attention over k tokens is the same for
    every setting), against the flat indexer on the same inputs."""
    import torch

    import long_context_indexer_block_amd as H
    from long_context_indexer_block_amd.pipeline import FlatPipeline, HierPipeline

    steps, warmup = max(2, a.steps // 2), max(1, a.warmup)
    f = FlatPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"], w.k,
                     w.scale)
    fwall, _ = timed([f.index], steps, warmup)
    flat_idx = f.token_idx.clone()
    flat_ms = fwall * 1e3 / steps
    del f
    torch.cuda.empty_cache()
    print(json.dumps({"sweep": w.name, "path": "flat", "index_ms": flat_ms}), flush=True)
    auto_h, auto_m = H.hisa_auto_plan(w.L, w.B)
    for B in (64, 128, 256):
        for m in (32, 64, 128):
            if m * B > 16384:
                continue
            p = HierPipeline(inp["kidx"], inp["qidx"], inp["q_pos"], inp["q"], inp["k"], inp["v"],
                             B, m, w.k, w.scale)
            calls = [
                p.summarize,
                lambda: H.hisa_block_score(p.qidx, p.q_pos, p.split, p.B, out=p.block_scores),
                lambda: H.hisa_select_blocks(p.block_scores, p.q_pos, p.B, p.m, out=p.block_idx),
                lambda: H.hisa_token_select(p.qidx, p.kidx, p.q_pos, p.block_idx, p.B, p.k_top,
                                            token_idx=p.token_idx, want_scores=False,
                                            workspace=p.ws),
            ]
            wall, stage = timed(calls, steps, warmup)
            ms = wall * 1e3 / steps
            rec = {"sweep": w.name, "path": "hierarchical", "B": B, "m": m,
                   "auto_plan": bool(auto_h and B == w.B and m == auto_m), "index_ms": ms,
                   "stage_ms": dict(zip(["summary", "block_score", "select_blocks",
                                         "token_select"], stage)),
                   "speedup_vs_flat": flat_ms / ms,
                   "recall_vs_flat": recall_vs_flat(p.token_idx, flat_idx)}
            print(json.dumps(rec), flush=True)
            del p
            torch.cuda.empty_cache()


def main():
    a = parse()
    if a.write_traffic:
        write_traffic(a.write_traffic)
        return
    if a.write_counters:
        write_counters(a.write_counters, a.counters_out, a.counters_kernel,
                       a.counters_title, a.counters_command, a.counters_note)
        return
    if a.write_trace_md:
        write_trace_md(a.write_trace_md, a.counters_out, a.counters_title, a.counters_command,
                       a.counters_note)
        return
    if a.write_bytes_md:
        write_bytes_md(a.write_bytes_md, a.counters_out, a.counters_title, a.counters_command,
                       a.counters_note)
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the path has no "
              "multi-GPU form", file=sys.stderr)
        sys.exit(2)
    import torch

    import long_context_indexer_block_amd as H  # noqa: F401  (raises without libhisa.so)
    from workloads import WORKLOADS, make_inputs

    if a.copy_probe:
        copy_probe(a.copy_probe)
        return
    if a.bw_probe:
        bw_probe(a.bw_probe)
        return
    w = WORKLOADS[a.workload]
    torch.cuda.set_device(0)
    log(f"generating {w.name} inputs on the GPU")
    inp = make_inputs(w, "cuda", seed=0)
    torch.cuda.synchronize()
    if a.sweep:
        bench_sweep(w, a, inp)
        return
    if a.attn_only:
        res = bench_attn_kept(w, a, inp) if a.attn_kept else bench_attn_only(w, a, inp)
        print(json.dumps(res), flush=True)
        return
    if a.gather_probe:
        print(json.dumps(bench_gather_probe(w, a, inp)), flush=True)
        return
    if w.kind == "prefill":
        res = bench_prefill(w, a, inp)
    elif w.kind == "decode":
        res = bench_decode(w, a, inp)
    elif w.kind == "hils_prefill":
        res = bench_hils_prefill(w, a, inp)
    else:
        res = bench_hils(w, a, inp)
    if not a.no_cpu and w.kind == "prefill":
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(w, inp, a.cpu_seconds)
    elif not a.no_cpu and w.kind == "hils_prefill":
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline_hils_prefill(w, inp, a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
