"""Benchmark of the weight-absorbed MLA decode path on one MI355X.

One step = one full decode of the workload through the C ABI: a single
mla_decode (mla_sparse_decode) call, which enqueues the split-KV scheduling
pass, the main pass and the split merge, over inputs already resident in
HBM.  Steps rotate over several copies of the latent cache so consecutive
steps do not find it in the 256 MB last-level cache.  Steps are timed as
replays of one HIP graph per cache copy holding that call, the way a serving
loop runs a graph-capturable decode: Python argument checks per call take
longer than the smaller workloads' GPU time, so plain stream launches from
Python (also reported) can leave the GPU waiting.  Each replay runs one step
per cache copy back to back, as a serving loop's graph holds many layers'
calls; one step per replay is reported too.  Events sit only around the
timed loop.  The main kernel is timed from back-to-back single-kernel
graph replays with an event between consecutive ones.  Before any timed
loop, steps run for --settle-s seconds: the GPU's clocks settle only under
sustained work.

Prints one JSON line.  `value` is algorithmic TFLOP/s of the whole step;
`roofline` describes the main kernel (mla_attend) timed with HIP events on
the stream it runs on (mean, as rocprofv3 reports it; also p10/median/p90
and the median per cache copy); `roofline_step` is the same algorithmic
bytes over the whole step; `cpu_baseline` is the CPU oracle timed on a
bounded sample of the same workload on this host's cores available to the
job.

Algorithmic work (per query row and visible token): 2*576 FLOP for the
score and 2*512 for the output, 2176 in all; bytes: every visible cached
token once (1152 B bf16, 576 B + 4 B scale fp8), plus q (1152 B per row),
out (1024 B per row) and lse (4 B per row), plus sparse indices.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import mla_synth as S  # noqa: E402

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
FLOP_PER_ROW_TOKEN = 2 * 576 + 2 * 512


def visible_counts(inp) -> np.ndarray:
    """Visible tokens per (b, s) row group: [B, Sq]."""
    B, Sq = inp["B"], inp["Sq"]
    L = inp["cache_seqlens"].numpy().astype(np.int64)
    if inp["indices"] is not None:
        ix = inp["indices"].numpy()
        return ((ix >= 0) & (ix < L[:, None, None])).sum(axis=2)
    if inp["causal"]:
        s = np.arange(Sq)[None, :]
        return np.clip(L[:, None] - Sq + s + 1, 0, None)
    return np.repeat(L[:, None], Sq, axis=1)


def algorithmic(inp):
    """(FLOP, bytes) of one decode of `inp`."""
    H = inp["H"]
    vis = visible_counts(inp)
    flop = float(vis.sum()) * H * FLOP_PER_ROW_TOKEN
    tok_bytes = 576 + 4 if inp["kv_dtype"] == "fp8" else 1152
    if inp["indices"] is not None:
        tokens = float(vis.sum())          # each (b, s) reads its own list
    else:
        tokens = float(inp["cache_seqlens"].clamp(min=0).sum())
    rows = inp["B"] * inp["Sq"] * H
    nbytes = tokens * tok_bytes + rows * (1152 + 1024 + 4)
    if inp["indices"] is not None:
        nbytes += inp["indices"].numel() * 4
    return flop, nbytes


def kernel_source_sha(inp=None) -> str:
    """First 16 hex of the SHA-256 of the source file holding the main
    kernel for `inp` (the head-group sparse kernel has a file of its own)."""
    name = "mla_kernels.hip"
    if inp is not None and "_hg" in main_kernel_name(inp):
        name = "mla_sparse.hip"
    p = os.path.join(ROOT, "mla_latent_kv_12_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def measured_traffic(workload: str, inp=None):
    """HBM bytes per main-kernel launch from the committed counter summary,
    or None when there is none or the kernel source changed since."""
    p = os.path.join(ROOT, "profiles", f"traffic_attend_{workload}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_sha") != kernel_source_sha(inp):
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, target_s: float):
    import oracle
    # every core this job may use: OMP_NUM_THREADS when the host sets it (the
    # CPU share a job gets), else the process's affinity set
    cores = oracle.default_threads()
    H, Sq = inp["H"], inp["Sq"]
    vis = visible_counts(inp)                     # [B, Sq]
    per_row_flop = np.repeat(vis.reshape(-1), H) * FLOP_PER_ROW_TOKEN
    # calibrate on a few rows, then time a sample sized to about target_s
    t0 = time.perf_counter()
    oracle.decode(inp, rows=range(min(cores, per_row_flop.size)), nthreads=cores)
    dt = time.perf_counter() - t0
    rate = per_row_flop[:cores].sum() / max(dt, 1e-6)
    want = rate * target_s
    n = int(np.searchsorted(np.cumsum(per_row_flop), want)) + 1
    n = max(cores, min(n, per_row_flop.size))
    t0 = time.perf_counter()
    oracle.decode(inp, rows=range(n), nthreads=cores)
    dt = time.perf_counter() - t0
    flop = float(per_row_flop[:n].sum())
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"first {n} of {per_row_flop.size} query rows (all their visible tokens), fp64",
            "nproc": os.cpu_count(), "affinity_cpus": affinity,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"), "cpu_model": cpu_model()}


def settle(fn, seconds: float):
    """Runs fn(k) until `seconds` of wall time have passed (untimed)."""
    t0 = time.perf_counter()
    k = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn(k)
            k += 1
        torch.cuda.synchronize()


def main_kernel_name(inp) -> str:
    """Name of the main-pass kernel the library launches for this input."""
    if inp["indices"] is not None and inp["kv_dtype"] != "fp8":
        # head-group kernel, then the merge of split index ranges: the
        # attend stage (and the whole sparse step)
        return "decode_bf16_sparse_hg + combine_hg"
    rows = inp["H"] if inp["indices"] is not None else inp["Sq"] * inp["H"]
    rows = min(rows, 128)
    shape = "r4" if rows > 64 else "r2" if rows > 32 else "r1w"
    kind = "sparse" if inp["indices"] is not None else "dense"
    return f"decode_{'fp8' if inp['kv_dtype'] == 'fp8' else 'bf16'}_{kind}_{shape}"


def bench_append(args):
    """Times mla_kv_append of the workload's B*Sq new rows into its cache.

    Algorithmic bytes per row: the new bf16 row read (1152 B), the block-table
    entry and length read (8 B), the row written (1152 B bf16, or 576 B codes
    + 4 B scale fp8)."""
    import mla_latent_kv_12_amd as mla
    dev = torch.device("cuda:0")
    inp = S.make_inputs(S.config(args.workload), poison=False)
    B, Sq = inp["B"], inp["Sq"]
    fp8 = inp["kv_dtype"] == "fp8"
    kv = inp["kv_pages"].to(dev)
    sc = inp["kv_scales"].to(dev) if fp8 else None
    bt, L = inp["block_table"].to(dev), inp["cache_seqlens"].to(dev)
    new = S._randn_bf16((B, Sq, 576), torch.Generator().manual_seed(99)).to(dev)
    settle(lambda _: mla.kv_append(new, kv, bt, L, kv_scales=sc), args.settle_s)
    for _ in range(args.warmup):
        mla.kv_append(new, kv, bt, L, kv_scales=sc)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        mla.kv_append(new, kv, bt, L, kv_scales=sc)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    rows = B * Sq
    nbytes = rows * (1152 + 8 + (580 if fp8 else 1152))
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "KV-cache append GB/s", "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8" if fp8 else "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "op": "kv_append", "rows": rows,
                   "kv": inp["kv_dtype"]},
        "alg_bytes": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 6), "traffic": None,
                     "kernel": "append_kernel", "kernel_ms": round(ms, 5),
                     "note": "a few hundred KB per launch: launch latency, not bandwidth, bounds it"},
    }), flush=True)


def bench_select(args):
    """Times mla_dsa_select on the sparse workload's shape: one score per
    64-token block of every query's context, 16 blocks selected (1 initial,
    2 local).  Algorithmic bytes: the score rows read (4 B per block) and the
    token lists written (4 B per listed token)."""
    import mla_latent_kv_12_amd as mla
    dev = torch.device("cuda:0")
    cfg = S.config(args.workload if S.CONFIGS[args.workload]["topk"] > 0 else "dsa_sparse")
    inp = S.make_inputs(dict(cfg, B=cfg["B"]), poison=False, unselected="nan")
    B, Sq, topk = inp["B"], inp["Sq"], inp["topk"]
    L = inp["cache_seqlens"].to(dev)
    nbk = int(inp["block_table"].shape[1])
    scores = torch.randn((B, Sq, nbk), generator=torch.Generator().manual_seed(98)).to(dev)
    n_sel = topk // 64
    idx = torch.empty((B, Sq, topk), dtype=torch.int32, device=dev)
    settle(lambda _: mla.dsa_select(scores, L, n_select=n_sel, indices=idx), args.settle_s)
    for _ in range(args.warmup):
        mla.dsa_select(scores, L, n_select=n_sel, indices=idx)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        mla.dsa_select(scores, L, n_select=n_sel, indices=idx)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    nbytes = B * Sq * (nbk * 4 + topk * 4) + B * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "DSA block top-k selection GB/s", "value": round(gbs, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "op": "dsa_select", "queries": B * Sq, "blocks": nbk,
                   "n_select": n_sel},
        "alg_bytes": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 6), "traffic": None,
                     "kernel": "select_kernel", "kernel_ms": round(ms, 5),
                     "note": "one workgroup per query, a few hundred KB in all: latency-bound"},
    }), flush=True)


def bench_proj(args):
    """Times mla_absorb_query or mla_project_out for the workload's B*Sq query
    rows and H heads (d_h = 128, d_c = 512), random N(0, 1/512) bf16 weights.
    Algorithmic bytes: the weights (H*128*512*2) read once, the input rows
    read and the output rows written; FLOP 2*M*H*128*512."""
    import mla_latent_kv_12_amd as mla
    dev = torch.device("cuda:0")
    cfg = S.config(args.workload)
    M, H = cfg["B"] * cfg["Sq"], cfg["H"]
    gen = torch.Generator().manual_seed(97)
    absorb = args.op == "absorb"
    kin, kout = (128, 512) if absorb else (512, 128)
    x = torch.randn((M, H, kin), generator=gen).to(torch.bfloat16).to(dev)
    w = (torch.randn((H, kout, kin), generator=gen) * 512 ** -0.5).to(torch.bfloat16).to(dev)
    out = torch.empty((M, H, kout), dtype=torch.bfloat16, device=dev)
    f = mla.absorb_query if absorb else mla.project_out
    settle(lambda _: f(x, w, out=out), args.settle_s)
    for _ in range(args.warmup):
        f(x, w, out=out)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        f(x, w, out=out)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    nbytes = H * 128 * 512 * 2 + M * H * (kin + kout) * 2
    flop = 2.0 * M * H * 128 * 512
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": f"MLA {'query absorption' if absorb else 'output projection'} GB/s", "value": round(gbs, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "op": args.op, "M": M, "H": H},
        "alg_bytes": nbytes, "alg_flop": flop, "tflops": round(flop / (ms * 1e-3) / 1e12, 3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 5), "traffic": None, "kernel": "head_gemm_kernel",
                     "kernel_ms": round(ms, 5)},
    }), flush=True)


def bench_layer(args):
    """Times the whole absorbed decode layer on a dense workload as
    mla_decode_layer (absorption with the schedule in the same launch, main
    pass, merge, projection: four launches) against the same computation as
    separate calls (mla_absorb_query,
    mla_decode -- schedule, main pass, merge -- and mla_project_out), both as
    graph replays of one layer per cache copy, random N(0, 1/512) weights.
    Algorithmic bytes: every cached token once, q_c, q_rope, o and lse per
    row, and both weight tensors once; FLOP: the decode's plus 2*128*512 per
    row and head for each projection."""
    import mla_latent_kv_12_amd as mla
    dev = torch.device("cuda:0")
    inp = S.make_inputs(S.config(args.workload), poison=False)
    if inp["indices"] is not None:
        raise SystemExit("--op layer runs dense workloads")
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    B, Sq, H = inp["B"], inp["Sq"], inp["H"]
    M = B * Sq
    gen = torch.Generator().manual_seed(98)
    q_c = torch.randn((B, Sq, H, 128), generator=gen).to(torch.bfloat16).to(dev)
    w_uk_t = (torch.randn((H, 512, 128), generator=gen) * 512 ** -0.5).to(torch.bfloat16).to(dev)
    w_uv = (torch.randn((H, 128, 512), generator=gen) * 512 ** -0.5).to(torch.bfloat16).to(dev)
    kvs = [g["kv_pages"]] + [g["kv_pages"].clone() for _ in range(args.copies - 1)]
    scs = [g["kv_scales"]] * args.copies if g["kv_scales"] is None else \
        [g["kv_scales"]] + [g["kv_scales"].clone() for _ in range(args.copies - 1)]
    ws_layer = torch.empty(mla.layer_workspace_size(B, Sq, H), dtype=torch.uint8, device=dev)
    ws = mla.alloc_workspace(B, Sq, H)
    o = torch.empty((B, Sq, H, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Sq, H), dtype=torch.float32, device=dev)
    q_nope = torch.empty((B, Sq, H, 512), dtype=torch.bfloat16, device=dev)
    out = torch.empty((B, Sq, H, 512), dtype=torch.bfloat16, device=dev)

    def fused(i):
        mla.decode_layer(q_c, w_uk_t, g["q_rope"], w_uv, kvs[i], g["block_table"], g["cache_seqlens"],
                         g["softmax_scale"], kv_scales=scs[i], causal=g["causal"], o=o, lse=lse,
                         workspace=ws_layer)

    def separate(i):
        mla.absorb_query(q_c, w_uk_t, out=q_nope)
        mla.decode(q_nope, g["q_rope"], kvs[i], g["block_table"], g["cache_seqlens"], g["softmax_scale"],
                   kv_scales=scs[i], causal=g["causal"], out=out, lse=lse, workspace=ws)
        mla.project_out(out, w_uv, out=o)

    def graph_of(fn):
        for i in range(args.copies):
            fn(i)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(args.copies):
                fn(i)
        torch.cuda.synchronize()
        return gr

    g_fused, g_sep = graph_of(fused), graph_of(separate)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < args.settle_s:
        g_fused.replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_rep = max(1, args.steps // args.copies)

    def timed(gr):
        for _ in range(max(1, args.warmup // args.copies)):
            gr.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n_rep):
            gr.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (n_rep * args.copies)

    ms_sep = timed(g_sep)
    ms = timed(g_fused)
    ms_sep = min(ms_sep, timed(g_sep))   # order effects: each timed after the other once
    dflop, _ = algorithmic(inp)
    flop = dflop + 2 * 2.0 * M * H * 128 * 512
    tokens = float(inp["cache_seqlens"].clamp(min=0).sum())
    tok_bytes = 576 + 4 if inp["kv_dtype"] == "fp8" else 1152
    nbytes = tokens * tok_bytes + M * H * (128 * 2 + 64 * 2 + 128 * 2 + 4) + 2 * H * 128 * 512 * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "MLA absorbed decode layer (W_UK, decode, W_UV) TFLOP/s", "value": round(flop / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": n_rep * args.copies, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "op": "layer", "B": B, "Sq": Sq, "H": H,
                   "cache_copies": args.copies, "launch": "hip_graph"},
        "ms_per_step_separate_calls": round(ms_sep, 5), "speedup_vs_separate": round(ms_sep / ms, 4),
        # the layer: absorption (with the schedule beside it), main pass,
        # merge, projection; the separate calls: absorption, main pass
        # (scheduling itself), merge, projection
        "launches_fused": 4, "launches_separate": 4,
        "alg_bytes": nbytes, "alg_flop": flop,
        "roofline_step": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(gbs / HBM_PEAK_GBS, 4)},
    }), flush=True)


def bench_prefill(args):
    """Times mla_prefill: causal MHA over decompressed per-head K/V, B=1,
    T=--prefill-len, H=128, d_qk 192, d_v 128, bf16 N(0,1).  FLOP: each of
    the T(T+1)/2 visible (query, key) pairs per head costs 2*192 (score) +
    2*128 (output); MFMA-bound, against the dense bf16 peak."""
    import mla_latent_kv_12_amd as mla
    dev = torch.device("cuda:0")
    B, T, H = 1, args.prefill_len, 128
    gen = torch.Generator().manual_seed(96)
    q = torch.randn((B, T, H, 192), generator=gen).to(torch.bfloat16).to(dev)
    k = torch.randn((B, T, H, 192), generator=gen).to(torch.bfloat16).to(dev)
    v = torch.randn((B, T, H, 128), generator=gen).to(torch.bfloat16).to(dev)
    out = torch.empty((B, T, H, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    scale = 1.0 / np.sqrt(192.0)
    settle(lambda _: mla.prefill(q, k, v, scale, out=out, lse=lse), args.settle_s)
    for _ in range(args.warmup):
        mla.prefill(q, k, v, scale, out=out, lse=lse)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        mla.prefill(q, k, v, scale, out=out, lse=lse)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    flop = B * H * (T * (T + 1) / 2) * 2 * (192 + 128)
    tfs = flop / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "MLA non-absorbed prefill TFLOP/s", "value": round(tfs, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": {"workload": "prefill", "op": "prefill", "B": B, "T": T, "H": H,
                                        "causal": True},
        "alg_flop": flop,
        "roofline": {"bound": "mfma", "achieved": round(tfs, 2), "peak": MFMA_BF16_PEAK_TFS,
                     "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4), "traffic": None,
                     "kernel": "prefill_kernel", "kernel_ms": round(ms, 5)},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsv3_decode", choices=list(S.CONFIGS))
    ap.add_argument("--copies", type=int, default=3, help="cache copies rotated over steps")
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="seconds of untimed steps before the warmup steps (clock settling)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run plain 1 GiB device copies (calibrates HBM byte counters)")
    ap.add_argument("--op", default="decode",
                    choices=["decode", "layer", "append", "select", "absorb", "project", "prefill"],
                    help="decode: the decode step (default); append: the cache append alone; "
                         "select: the DSA block top-k selection alone (sparse workloads); "
                         "layer: W_UK absorption, decode and W_UV projection, fused against "
                         "separate calls (dense workloads); "
                         "absorb / project: the W_UK query absorption / W_UV output projection; "
                         "prefill: non-absorbed causal MHA, B=1, T=--prefill-len, H=128")
    ap.add_argument("--prefill-len", type=int, default=4096)
    args = ap.parse_args()
    if args.copy_probe:
        # Known traffic: each copy reads and writes exactly 1 GiB.
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": src.numel() * 4, "copies": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(each GPU would run this path on its own share of the batch)", file=sys.stderr)
        sys.exit(2)

    if args.op == "append":
        bench_append(args)
        return
    if args.op == "select":
        bench_select(args)
        return
    if args.op in ("absorb", "project"):
        bench_proj(args)
        return
    if args.op == "prefill":
        bench_prefill(args)
        return
    if args.op == "layer":
        bench_layer(args)
        return

    import mla_latent_kv_12_amd as mla
    dev = torch.device("cuda:0")
    cfg = S.config(args.workload)
    inp = S.make_inputs(cfg, poison=False)
    flop, nbytes = algorithmic(inp)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    kvs = [g["kv_pages"]] + [g["kv_pages"].clone() for _ in range(args.copies - 1)]
    scs = [g["kv_scales"]] * args.copies if g["kv_scales"] is None else \
        [g["kv_scales"]] + [g["kv_scales"].clone() for _ in range(args.copies - 1)]
    B, Sq, H = inp["B"], inp["Sq"], inp["H"]
    topk = inp["topk"]
    ws = mla.alloc_workspace(B, Sq, H, topk)
    out = torch.empty((B, Sq, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Sq, H), dtype=torch.float32, device=dev)

    def step(k):
        """One decode step: a single C-ABI call that enqueues the scheduling
        pass, the main pass and the combine."""
        i = k % args.copies
        if topk:
            mla.sparse_decode(g["q_nope"], g["q_rope"], kvs[i], g["block_table"],
                              g["cache_seqlens"], g["indices"], g["softmax_scale"],
                              kv_scales=scs[i], out=out, lse=lse, workspace=ws)
        else:
            mla.decode(g["q_nope"], g["q_rope"], kvs[i], g["block_table"], g["cache_seqlens"],
                       g["softmax_scale"], kv_scales=scs[i], causal=g["causal"], out=out,
                       lse=lse, workspace=ws)

    def attend(k):
        i = k % args.copies
        mla.attend(g["q_nope"], g["q_rope"], kvs[i], g["block_table"], g["cache_seqlens"],
                   g["softmax_scale"], ws, kv_scales=scs[i], indices=g["indices"],
                   causal=g["causal"], out=out, lse=lse)

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)

    def timed(fn):
        """Mean ms per call of fn(k) over args.steps calls, events only
        around the whole loop."""
        torch.cuda.synchronize()
        t_start.record()
        for k in range(args.steps):
            fn(k)
        t_end.record()
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_end) / args.steps

    def capture(fn):
        """One HIP graph per cache copy holding fn(copy); the library's calls
        never allocate or synchronise, so they capture as they are."""
        graphs = []
        for i in range(args.copies):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                fn(i)
            graphs.append(gr)
        torch.cuda.synchronize()
        return lambda k: graphs[k % args.copies].replay()

    # Graphs: a whole step (plan + main + combine), the main pass alone (on a
    # plan computed before capture) and main + combine (plan reused).
    for k in range(args.copies):
        step(k)
    torch.cuda.synchronize()
    g_step = capture(step)
    # a serving loop holds many layers' decode calls in one graph: each
    # replay of g_steps runs `copies` consecutive steps (one per cache
    # copy), which share the replay's launch the same way
    g_steps = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_steps):
        for i in range(args.copies):
            step(i)
    torch.cuda.synchronize()
    mla.plan(g["cache_seqlens"], B, Sq, H, ws, topk=topk)
    torch.cuda.synchronize()
    g_attend = capture(attend)

    def planned(k):
        attend(k)
        mla.combine(g["cache_seqlens"], B, Sq, H, out, lse, ws, topk=topk)

    g_planned = capture(planned)

    # The GPU's clocks settle only after some sustained work: the first loop
    # a process times ran ~15% slower than the same loop repeated.  Steps for
    # at least --settle-s seconds go first, then the --warmup steps.
    settle(g_step, args.settle_s)
    for k in range(args.warmup):
        g_step(k)
    n_rep = max(1, args.steps // args.copies)
    torch.cuda.synchronize()
    t_start.record()
    for k in range(n_rep):
        g_steps.replay()
    t_end.record()
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / (n_rep * args.copies)
    settle(g_step, args.settle_s / 2)
    ms_one_per_graph = timed(g_step)
    assert torch.isfinite(lse).all(), "non-finite lse"
    # the same step as plain stream launches from Python (one mla_decode call
    # per step); host-side argument checks can leave the GPU waiting here
    for k in range(args.warmup):
        step(k)
    ms_eager = timed(step)
    # every graph timed below first runs on its own until the clocks settle:
    # the host-side work in between leaves the GPU idle long enough to drop
    # them again (a main kernel timed right after it ran ~15% slower)
    settle(g_planned, args.settle_s / 2)
    ms_planned = timed(g_planned)

    # The main kernel on its own: one graph holding 4 * copies back-to-back
    # launches (the cache copies in rotation), events only around its
    # replays; the mean per launch is what a kernel trace averages.  Event
    # pairs around single launches measured ~20 us longer per launch than the
    # trace, so they only give the spread (p10/median/p90, per cache copy).
    per = 4 * args.copies
    many = torch.cuda.CUDAGraph()
    with torch.cuda.graph(many):
        for j in range(per):
            attend(j)
    reps = max(3, args.steps // per)
    settle(lambda k: many.replay(), args.settle_s)
    torch.cuda.synchronize()
    t_start.record()
    for k in range(reps):
        many.replay()
    t_end.record()
    torch.cuda.synchronize()
    attend_ms = t_start.elapsed_time(t_end) / (reps * per)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    settle(g_attend, args.settle_s / 2)
    for k in range(args.steps):
        evs[k][0].record()
        g_attend(k)
        evs[k][1].record()
    torch.cuda.synchronize()
    attend_all = np.array([a.elapsed_time(b) for a, b in evs])

    tflops = flop / (ms * 1e-3) / 1e12
    achieved_gbs = nbytes / (attend_ms * 1e-3) / 1e9
    ai = flop / nbytes
    bound = "hbm" if ai < MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4)}
    else:
        a_tf = flop / (attend_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(a_tf, 2), "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(a_tf / MFMA_BF16_PEAK_TFS, 4)}
    roof["traffic"] = measured_traffic(args.workload, inp)
    roof["kernel"] = main_kernel_name(inp)
    roof["kernel_ms"] = round(attend_ms, 5)
    # spread of single launches (event pairs: each ~20 us above the trace)
    roof["single_launch_ms_p10_median_p90"] = [round(float(np.percentile(attend_all, q)), 5) for q in (10, 50, 90)]
    # median single-launch time per cache copy (steps k, k + copies, ...)
    roof["single_launch_ms_median_per_cache_copy"] = [
        round(float(np.median(attend_all[i::args.copies])), 5) for i in range(args.copies)]
    roof["mfma_frac"] = round(flop / (attend_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4)
    # the same algorithmic bytes over the whole step (plan + main pass +
    # combine, as launched), the figure `value` is quoted on
    step_gbs = nbytes / (ms * 1e-3) / 1e9
    roof_step = {"bound": roof["bound"], "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS,
                 "unit": "GB/s", "frac": round(step_gbs / HBM_PEAK_GBS, 4)}

    res = {
        "metric": "MLA absorbed decode TFLOPS + HBM GB/s (% roofline), B=64 H=128 L~8K",
        "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "Sq": Sq, "H": H,
                   "tokens": int(inp["cache_seqlens"].sum()), "kv": inp["kv_dtype"],
                   "topk": topk, "seed": inp["seed"], "cache_copies": args.copies,
                   "launch": "hip_graph"},
        "ms_per_step_stream_launch": round(ms_eager, 5),
        "ms_per_step_one_step_per_graph": round(ms_one_per_graph, 5),
        "ms_per_step_plan_reused": round(ms_planned, 5),
        "gbps_step": round(nbytes / (ms * 1e-3) / 1e9, 1),
        "alg_bytes": nbytes, "alg_flop": flop,
        "roofline": roof,
        "roofline_step": roof_step,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
