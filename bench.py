"""Throughput of the PISA forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wan_bf16]

One step = the whole hot path on one batch: pisa_block_stats, pisa_select and
pisa_attn_fwd (the fused pass), on seeded synthetic inputs already resident in
HBM. Prints one JSON line. ``value`` is the effective TFLOP/s of the whole step
(exact-block + zeroth-order tail + first-order FLOPs over the step time); the
per-call milliseconds, the fused kernel's roofline fraction, the same-device
dense baseline and the fp64 CPU oracle's rate on a bounded sample ride along.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "PISA attn fwd ms/call + effective TFLOP/s (%MFMA peak), Wan-shape L=75600 d=0.125"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # MI355X dense MFMA peaks
HBM_PEAK_GBS = 8000.0

# Bytes one k_pisa_fwd launch moves between L2 and memory at the Wan shape, from
# two rocprofv3 --pmc passes over this bench command (FETCH_SIZE, then
# WRITE_SIZE; KiB per dispatch, mean of the two dispatches), each scaled by what
# the same counter reads for one plain 2 GiB device copy (bench.py --calib-copy 2):
# FETCH_SIZE reads 1048612 KiB for it (scale 2.0), WRITE_SIZE 2097152 KiB (1.0).
# The figures hold only for the kernel sources they were taken on; their SHA-1
# is kept, and the figure is reported as null once the sources differ.
FUSED_TRAFFIC = {"workload": "wan_bf16",
                 "sources": ["k_fwd.hip", "pisa_dev.h", "pisa_internal.h", "pisa_abi.hip"],
                 "sha1": "8e04eef5caf51e152ec29ca28b273729e03d871c",
                 "fetch_kib": (28095046.7 + 28225541.3) / 2, "fetch_scale": 2.0,
                 "write_kib": (828397.9 + 828397.6) / 2, "write_scale": 1.0}


def fused_traffic(workload: str):
    import hashlib

    t = FUSED_TRAFFIC
    if workload != t["workload"]:
        return None
    h = hashlib.sha1()
    for f in t["sources"]:
        with open(os.path.join(ROOT, "block_sparse_attention_stats_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != t["sha1"]:
        return None
    return 1024.0 * (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"])


def flops_from_idx(idx: np.ndarray, L: int, D: int, block: int, first_order: bool,
                   per_block: bool = False) -> dict:
    """Credited FLOPs of one fused call: 4·D per exact (query, key) pair, 4·D
    per (query, unselected block) pair, 2·D² per query row of a query block
    with unselected blocks (hybrid only), or 2·D² per (query, unselected block)
    pair (per-block first-order variant: q_t H_j for every such block). Centroid
    logits of selected blocks, which the kernel computes and masks, are not
    credited."""
    B, H, n, k = idx.shape
    n_last = L - (n - 1) * block
    nq = np.full(n, block, dtype=np.float64)
    nq[-1] = n_last
    has_last = (idx == n - 1).any(axis=-1)                      # [B,H,n]
    exact_keys = k * block - (block - n_last) * has_last          # Σ_{j∈S_i} n_j
    exact = float((nq * 4.0 * D * exact_keys).sum())
    tail = float((nq * 4.0 * D * (n - k)).sum()) * B * H
    corr = float(2.0 * D * D * nq.sum() * B * H) if (first_order and k < n) else 0.0
    if per_block:
        corr = float(2.0 * D * D * nq.sum() * (n - k) * B * H)
    return dict(exact=exact, tail=tail, corr=corr, total=exact + tail + corr)


def stats_bytes(B, H, L, D, block, esz) -> dict:
    """Bytes of the statistics pass per call. ``algorithmic``: q, k, v read once;
    q̄, k̄, ΣV (fp64), the k̄ / ΣV centroid tiles and H̄ᵀ in the I/O dtype, H̄
    (fp64) and the largest key norms written. ``copies``: the operand-ordered
    copies of K and V for the fused pass (written). ``partials``: the per-run
    partial sums of H_j (written, then read once by the reduction to H̄)."""
    n = -(-L // block)
    bh = B * H
    nct = -(-n // 64)
    cb = min(1024 // block, max(1, bh * n // 512))  # blocks per statistics run
    nch = -(-n // cb)
    alg = 3.0 * L * D * esz + 3.0 * n * D * 8 + 2.0 * nct * 64 * D * esz + D * D * (8 + esz) + nch * 4
    copies = 2.0 * n * (block // 64) * 64 * D * esz
    partials = 2.0 * nch * D * D * 4
    return {"algorithmic": bh * alg, "copies": bh * copies, "partials": bh * partials}


def copy_bandwidth(dev, nbytes: int = 2 << 30) -> float:
    """GB/s of one plain device-to-device copy (read + write counted)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2.0 * nbytes * 3 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbs


def gemm_rate(dev, dtype_name: str, n: int = 8192) -> float:
    """TFLOP/s of one plain n x n x n matrix product on the device's GEMM
    library (hipBLASLt through torch.mm), contiguous operands: what the
    matrix cores reach on this machine under its power limit, next to the spec
    peak."""
    import torch
    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    a = torch.randn(n, n, device=dev, dtype=torch.float32).to(dt)
    b = torch.randn(n, n, device=dev, dtype=torch.float32).to(dt)
    c = torch.mm(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        torch.mm(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    tf = 2.0 * n ** 3 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    return tf


def cpu_baseline(w, budget_s: float = 15.0) -> dict:
    """The fp64 oracle, whole heads at a time (statistics, routing and every
    query block of the head), until the time budget is spent; at least one
    head. Credited with the same FLOPs as the GPU pass over those heads."""
    import oracle
    import synth

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    n = w.n_blocks
    topk = oracle.topk_from_density(w.density, n)
    sizes = oracle.block_sizes(w.L, w.block).astype(np.float64)
    total, t, heads = 0.0, 0.0, []
    for (b, h) in [(b, h) for b in range(w.B) for h in range(w.H)]:
        q, k, v = (synth.as_f64(x) for x in synth.head_tensors(w, b, h))
        t0 = time.perf_counter()
        st = oracle.block_stats(q, k, v, w.block)
        M = oracle.cov_norm(st["H"], st["Hbar"]) if w.cov_weight else None
        S = oracle.pooled_scores(st["qbar"], st["kbar"], w.scale, M, w.cov_weight, w.sink_idx)
        idx = oracle.select_topk(S, topk)
        for i in range(n):
            oracle.pisa_rows(q, k, v, st, idx[i], i, w.block, w.scale, w.variant == "hyd")
        t += time.perf_counter() - t0
        heads.append((b, h))
        for i in range(n):
            total += sizes[i] * (4.0 * w.D * sizes[idx[i]].sum() + 4.0 * w.D * (n - topk))
            if w.variant == "hyd" and topk < n:
                total += 2.0 * sizes[i] * w.D * w.D
        if t > budget_s:
            break
    return {"value": total / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(heads)} whole heads of {w.name} (statistics, routing and all {n} query "
                      f"blocks each) in {t:.1f}s, fp64 NumPy; input generation not timed",
            "host_cpus": len(os.sched_getaffinity(0))}


def run_sweep(dev, args):
    """Every point of the Wan-shape sweep (block x density x variant, batch 2) on
    one set of inputs: per point the statistics, routing and fused-pass times
    (HIP events, mean of 3 calls after one untimed call) and the fused pass's
    credited TFLOP/s, next to the dense baseline on the same inputs."""
    import torch

    import block_sparse_attention_stats_amd as bsa
    import synth

    base = synth.SWEEP_BASE
    t0 = time.time()
    q, k, v = synth.make_qkv(base)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    del q, k, v
    print(f"[bench] sweep inputs on device ({time.time() - t0:.1f}s)", file=sys.stderr, flush=True)

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    od = torch.empty_like(qd)
    dense_ms = timed(lambda: bsa.dense(qd, kd, vd, base.scale, out=od), reps=1)
    dflops = 4.0 * base.B * base.H * float(base.L) * base.L * base.D
    print(json.dumps({"sweep": "dense", "B": base.B, "H": base.H, "L": base.L, "D": base.D,
                      "ms": dense_ms, "tflops": dflops / (dense_ms * 1e-3) / 1e12}), flush=True)
    o = torch.empty_like(qd)
    for w in synth.sweep():
        n = w.n_blocks
        topk = bsa.topk_from_density(w.density, n)
        shape = bsa.make_shape(qd, w.block)
        st = bsa.alloc_stats(shape, dev, want_mnorm=False)
        idx = torch.empty((w.B, w.H, n, topk), dtype=torch.int32, device=dev)
        hyd = w.variant == "hyd"
        ms_stats = timed(lambda: bsa.block_stats(qd, kd, vd, w.block, out=st))
        ms_sel = timed(lambda: bsa.select(st, topk, w.scale, 0.0, None, out=idx))
        ms_fused = timed(lambda: bsa.attn_fwd(qd, st, idx, w.scale, hyd, out=o))
        f = flops_from_idx(idx.cpu().numpy(), w.L, w.D, w.block, hyd)
        ms_step = ms_stats + ms_sel + ms_fused
        print(json.dumps({"sweep": w.name, "block": w.block, "density": w.density, "variant": w.variant,
                          "topk": topk, "ms_stats": ms_stats, "ms_select": ms_sel, "ms_fused": ms_fused,
                          "fused_tflops": f["total"] / (ms_fused * 1e-3) / 1e12,
                          "exact_phase_mfma_frac": f["exact"] / (ms_fused * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"],
                          "speedup_vs_dense_fused": dense_ms / ms_fused,
                          "speedup_vs_dense_step": dense_ms / ms_step}), flush=True)
        del st, idx


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan_bf16")
    ap.add_argument("--cov-norm", choices=["fro", "spectral"], default=None,
                    help="norm of the covariance term of the workload's routing (default: its own)")
    ap.add_argument("--cov-weight", type=float, default=None,
                    help="weight of the covariance term of the workload's routing (default: its own)")
    ap.add_argument("--dense-reps", type=int, default=2)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--pb1-reps", type=int, default=2,
                    help="calls of the per-block first-order variant timed on the same selection")
    ap.add_argument("--no-pb1", action="store_true")
    ap.add_argument("--bwd-reps", type=int, default=2,
                    help="calls of the zeroth-order variant's backward pass timed on the step's selection")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--banded-reps", type=int, default=3,
                    help="calls of the fused pass timed on a local (banded) selection of the same size")
    ap.add_argument("--no-banded", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the headline step, time every block x density x variant "
                         "point of the Wan-shape sweep (batch 2) and print one JSON line per point")
    ap.add_argument("--calib-copy", type=float, default=0.0, metavar="GIB",
                    help="only run one plain device-to-device copy of GIB GiB and exit: the "
                         "known-size kernel that scales the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path shards over "
              "(batch, head) with no exchange, so N GPUs run N independent copies.", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_attention_stats_amd as bsa
    import synth

    dev = torch.device("cuda:0")
    if args.calib_copy > 0:
        nbytes = int(args.calib_copy * 2**30)
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": nbytes}), flush=True)
        return

    if args.sweep:
        run_sweep(dev, args)
        return

    w = synth.WORKLOADS[args.workload]
    if args.cov_norm:
        w = w.replace(cov_norm=args.cov_norm)
    if args.cov_weight is not None:
        if args.cov_weight < 0:
            raise SystemExit("--cov-weight must be non-negative")
        w = w.replace(cov_weight=args.cov_weight)
    t0 = time.time()
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    q, k, v = synth.make_qkv(w)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    del q, k, v
    print(f"[bench] inputs on device ({time.time() - t0:.1f}s)", file=sys.stderr, flush=True)

    n = w.n_blocks
    topk = bsa.topk_from_density(w.density, n)
    s = w.scale
    hyd = w.variant == "hyd"
    shape = bsa.make_shape(qd, w.block)
    st = bsa.alloc_stats(shape, dev, want_mnorm=w.cov_weight > 0)
    idx = torch.empty((w.B, w.H, n, topk), dtype=torch.int32, device=dev)
    o = torch.empty_like(qd)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        bsa.block_stats(qd, kd, vd, w.block, want_mnorm=w.cov_weight > 0, out=st, cov_norm=w.cov_norm)
        if ev is not None:
            ev[1].record()
        bsa.select(st, topk, s, w.cov_weight, w.sink_idx, out=idx)
        if ev is not None:
            ev[2].record()
        bsa.attn_fwd(qd, st, idx, s, hyd, out=o)
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms = {"block_stats": 0.0, "select": 0.0, "attn_fwd": 0.0}
    for e in evs:
        ms["block_stats"] += e[0].elapsed_time(e[1]) / args.steps
        ms["select"] += e[1].elapsed_time(e[2]) / args.steps
        ms["attn_fwd"] += e[2].elapsed_time(e[3]) / args.steps
    ms_step = wall * 1e3 / args.steps
    ms["total_events"] = sum(ms.values())

    f = flops_from_idx(idx.cpu().numpy(), w.L, w.D, w.block, hyd)
    fused_tflops = f["total"] / (ms["attn_fwd"] * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    esz = 2 if w.dtype == "bf16" else 4
    sbytes = stats_bytes(w.B, w.H, w.L, w.D, w.block, esz)
    copy_gbs = copy_bandwidth(dev)
    gemm_tflops = gemm_rate(dev, w.dtype)
    print(f"[bench] step {ms_step:.3f} ms: stats {ms['block_stats']:.3f} select {ms['select']:.3f} "
          f"fused {ms['attn_fwd']:.3f}; fused {fused_tflops:.1f} TFLOP/s", file=sys.stderr, flush=True)

    dense = None
    if not args.no_dense:
        od = torch.empty_like(qd)
        ws = torch.empty(bsa.load_library().dense_workspace_bytes(bsa.ctypes.byref(shape)),
                         dtype=torch.uint8, device=dev)
        bsa.dense(qd, kd, vd, s, out=od, ws=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.dense_reps):
            bsa.dense(qd, kd, vd, s, out=od, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / args.dense_reps
        dflops = 4.0 * w.B * w.H * float(w.L) * w.L * w.D
        dense = {"ms": dms, "tflops": dflops / (dms * 1e-3) / 1e12,
                 "mfma_frac": dflops / (dms * 1e-3) / 1e12 / peak,
                 "speedup_vs_pisa_step": dms / ms_step, "speedup_vs_pisa_fused": dms / ms["attn_fwd"]}
        print(f"[bench] dense {dms:.2f} ms, {dense['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        del od, ws

    pb1 = None
    if not args.no_pb1:
        op = torch.empty_like(qd)
        bsa.attn_fwd(qd, st, idx, s, "pb1", out=op)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.pb1_reps):
            bsa.attn_fwd(qd, st, idx, s, "pb1", out=op)
        e1.record()
        torch.cuda.synchronize()
        pms = e0.elapsed_time(e1) / args.pb1_reps
        fp = flops_from_idx(idx.cpu().numpy(), w.L, w.D, w.block, False, per_block=True)
        pb1 = {"kernel": "k_pisa_pb1", "ms": pms, "flops": fp["total"],
               "tflops": fp["total"] / (pms * 1e-3) / 1e12,
               "mfma_frac": fp["total"] / (pms * 1e-3) / 1e12 / peak,
               "ms_vs_hyd_fused": pms / ms["attn_fwd"],
               "speedup_vs_dense": (dense["ms"] / pms) if dense else None}
        print(f"[bench] pb1 {pms:.2f} ms, {pb1['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        del op

    bwd = None
    if not args.no_bwd:
        # backward of the zeroth-order variant on the step's statistics and
        # selection, with a seeded upstream gradient of the output's shape
        gen = torch.Generator(device=dev).manual_seed(w.seed)
        dout = torch.randn(qd.shape, generator=gen, device=dev, dtype=torch.float32).to(qd.dtype)
        # the forward hands ln D_t to the backward, as the autograd path does
        o0, lse0 = bsa.attn_fwd(qd, st, idx, s, "0th", return_lse=True)
        bws = torch.empty(bsa.load_library().pisa_bwd_workspace_bytes(bsa.ctypes.byref(shape)),
                          dtype=torch.uint8, device=dev)
        bsa.attn_bwd(qd, kd, vd, st, idx, s, o0, dout, ws=bws, lse=lse0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.bwd_reps):
            bsa.attn_bwd(qd, kd, vd, st, idx, s, o0, dout, ws=bws, lse=lse0)
        e1.record()
        torch.cuda.synchronize()
        bwd_ms = e0.elapsed_time(e1) / args.bwd_reps
        f0 = flops_from_idx(idx.cpu().numpy(), w.L, w.D, w.block, False)
        bflops = 2.5 * (f0["exact"] + f0["tail"])  # five products per (query, key or centroid) pair
        bwd = {"kernel": "pisa_attn_bwd (zeroth-order variant)", "ms": bwd_ms, "flops": bflops,
               "tflops": bflops / (bwd_ms * 1e-3) / 1e12,
               "mfma_frac": bflops / (bwd_ms * 1e-3) / 1e12 / peak,
               "ms_vs_fwd_fused": bwd_ms / ms["attn_fwd"]}
        print(f"[bench] backward (0th) {bwd_ms:.2f} ms, {bwd['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        del dout, o0, lse0, bws

    banded = None
    if not args.no_banded:
        # the same fused pass on a local selection: query block i takes the topk
        # blocks nearest to it, as real DiT selections tend to be
        start = np.clip(np.arange(n) - topk // 2, 0, n - topk)
        bidx = np.broadcast_to(start[:, None] + np.arange(topk)[None, :], (w.B, w.H, n, topk))
        bidx = torch.from_numpy(bidx.astype(np.int32).copy()).to(dev)
        ob = torch.empty_like(qd)
        bsa.attn_fwd(qd, st, bidx, s, hyd, out=ob)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.banded_reps):
            bsa.attn_fwd(qd, st, bidx, s, hyd, out=ob)
        e1.record()
        torch.cuda.synchronize()
        bms = e0.elapsed_time(e1) / args.banded_reps
        fb = flops_from_idx(bidx.cpu().numpy(), w.L, w.D, w.block, hyd)
        banded = {"selection": "banded (the topk blocks nearest each query block)", "ms": bms,
                  "tflops": fb["total"] / (bms * 1e-3) / 1e12,
                  "exact_phase_mfma_frac": fb["exact"] / (bms * 1e-3) / 1e12 / peak,
                  "ms_vs_scattered": bms / ms["attn_fwd"]}
        print(f"[bench] banded selection: fused {bms:.2f} ms", file=sys.stderr, flush=True)
        del ob, bidx

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, args.cpu_budget)

    out = {
        "metric": METRIC,
        "value": f["total"] / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded clustered-Gaussian q/k (64-token clusters), N(0,1) v",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "D": w.D, "block": w.block,
                   "density": w.density, "topk": topk, "variant": w.variant, "sink_idx": w.sink_idx,
                   "cov_weight": w.cov_weight, "cov_norm": w.cov_norm, "seed": w.seed},
        "ms": ms,
        "flops": f,
        "fused_tflops": fused_tflops,
        "exact_phase_mfma_frac": f["exact"] / (ms["attn_fwd"] * 1e-3) / 1e12 / peak,
        # the statistics pass on its algorithmic bytes; the K/V operand copies and
        # the partial sums of H_j it also writes are given apart
        "stats_gbs": sbytes["algorithmic"] / (ms["block_stats"] * 1e-3) / 1e9,
        "stats_hbm_frac": sbytes["algorithmic"] / (ms["block_stats"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "stats_bytes": sbytes,
        "stats_all_bytes_gbs": sum(sbytes.values()) / (ms["block_stats"] * 1e-3) / 1e9,
        "hbm_copy_gbs": copy_gbs,  # measured device copy, next to the 8 TB/s spec peak
        "gemm_tflops": gemm_tflops,  # measured library GEMM in the I/O dtype, next to the MFMA spec peak
        "roofline": {"kernel": "k_pisa_fwd", "bound": "mfma", "achieved": fused_tflops, "peak": peak,
                     "unit": "TFLOP/s", "frac": fused_tflops / peak,
                     "traffic": fused_traffic(w.name) if w.cov_weight == synth.WORKLOADS[w.name].cov_weight else None,
                     "traffic_unit": "bytes per launch"},
        "dense": dense,
        "pb1": pb1,
        "banded": banded,
        "bwd": bwd,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
