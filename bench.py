"""Benchmark of the weight-absorbed MLA decode path on one MI355X.

One step = one full decode of the workload through the C ABI: the split-KV
scheduling pass (mla_plan), the main pass (mla_attend) and the split merge
(mla_combine), over inputs already resident in HBM.  Steps rotate over
several copies of the latent cache so consecutive steps do not find it in
the 256 MB last-level cache.  `--graph` times replays of the three calls
captured as one HIP graph per cache copy instead of plain stream launches
(the calls never allocate or synchronise, so they capture as they are; on
MI355X this measured the same step time).

Prints one JSON line.  `value` is algorithmic TFLOP/s of the whole step;
`roofline` describes the main kernel (mla_attend) timed with HIP events on
the stream it runs on; `cpu_baseline` is the CPU oracle timed on a bounded
sample of the same workload on this host.

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


def kernel_source_sha() -> str:
    p = os.path.join(ROOT, "mla_latent_kv_12_amd", "csrc", "mla_kernels.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per main-kernel launch from the committed counter summary,
    or None when there is none or the kernel source changed since."""
    p = os.path.join(ROOT, "profiles", f"traffic_attend_{workload}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_sha") != kernel_source_sha():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(inp, target_s: float):
    import oracle
    cores = min(os.cpu_count() or 1, int(os.environ.get("OMP_NUM_THREADS", "16") or 16), 16)
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
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"first {n} of {per_row_flop.size} query rows (all their visible tokens), fp64"}


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
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="time HIP graph replays of the step")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run plain 1 GiB device copies (calibrates HBM byte counters)")
    ap.add_argument("--op", default="decode", choices=["decode", "append", "select", "absorb", "project", "prefill"],
                    help="decode: the decode step (default); append: the cache append alone; "
                         "select: the DSA block top-k selection alone (sparse workloads); "
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

    def step(k, ev=None):
        i = k % args.copies
        mla.plan(g["cache_seqlens"], B, Sq, H, ws, topk=topk)
        if ev is not None:
            ev[0].record()
        mla.attend(g["q_nope"], g["q_rope"], kvs[i], g["block_table"], g["cache_seqlens"],
                   g["softmax_scale"], ws, kv_scales=scs[i], indices=g["indices"],
                   causal=g["causal"], out=out, lse=lse)
        if ev is not None:
            ev[1].record()
        mla.combine(g["cache_seqlens"], B, Sq, H, out, lse, ws, topk=topk)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for k in range(args.steps):
        step(k, evs[k])
    t_end.record()
    torch.cuda.synchronize()
    ms_eager = t_start.elapsed_time(t_end) / args.steps
    attend_all = np.array([a.elapsed_time(b) for a, b in evs])
    attend_ms = float(attend_all.mean())
    assert torch.isfinite(lse).all(), "non-finite lse"
    ms = ms_eager

    # The same steps with the scheduling pass run once and reused (a decode
    # step runs mla_plan once for all its layers): main pass + combine.
    mla.plan(g["cache_seqlens"], B, Sq, H, ws, topk=topk)
    torch.cuda.synchronize()
    t_start.record()
    for k in range(args.steps):
        i = k % args.copies
        mla.attend(g["q_nope"], g["q_rope"], kvs[i], g["block_table"], g["cache_seqlens"],
                   g["softmax_scale"], ws, kv_scales=scs[i], indices=g["indices"],
                   causal=g["causal"], out=out, lse=lse)
        mla.combine(g["cache_seqlens"], B, Sq, H, out, lse, ws, topk=topk)
    t_end.record()
    torch.cuda.synchronize()
    ms_planned = t_start.elapsed_time(t_end) / args.steps
    if args.graph:
        # One graph per cache copy; replayed in the same rotation.
        graphs = []
        for i in range(args.copies):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                step(i)
            graphs.append(gr)
        for k in range(args.warmup):
            graphs[k % args.copies].replay()
        torch.cuda.synchronize()
        t_start.record()
        for k in range(args.steps):
            graphs[k % args.copies].replay()
        t_end.record()
        torch.cuda.synchronize()
        ms = t_start.elapsed_time(t_end) / args.steps
        assert torch.isfinite(lse).all(), "non-finite lse"

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
    roof["traffic"] = measured_traffic(args.workload)
    roof["kernel"] = "mla_attend (decode_*_r4 / r2 / r1w)"
    roof["kernel_ms"] = round(attend_ms, 5)
    roof["kernel_ms_p10_median_p90"] = [round(float(np.percentile(attend_all, q)), 5) for q in (10, 50, 90)]
    roof["mfma_frac"] = round(flop / (attend_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4)

    res = {
        "metric": "MLA absorbed decode TFLOPS + HBM GB/s (% roofline), B=64 H=128 L~8K",
        "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "Sq": Sq, "H": H,
                   "tokens": int(inp["cache_seqlens"].sum()), "kv": inp["kv_dtype"],
                   "topk": topk, "seed": inp["seed"], "cache_copies": args.copies,
                   "launch": "hip_graph" if args.graph else "stream"},
        "ms_per_step_stream_launch": round(ms_eager, 5),
        "ms_per_step_plan_reused": round(ms_planned, 5),
        "gbps_step": round(nbytes / (ms * 1e-3) / 1e9, 1),
        "alg_bytes": nbytes, "alg_flop": flop,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
