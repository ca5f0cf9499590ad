"""Helpers of the GPU parity tests: run the HIP path and the fp64 oracle on the
same seeded inputs and compare them to the stated bar.

Tolerances (outputs always evaluated with the oracle's own selection):
  bf16 I/O, fp32 accumulation: max-abs <= 2e-2 and mean-abs <= 2e-3;
  fp32 I/O: max-abs <= 1e-4.
Block-index sets must match exactly, except where the oracle's pooled scores
tie within 1e-6 relative at the k-th place.
"""

from __future__ import annotations

import math
import sys
import time

import numpy as np
import torch

import block_sparse_attention_stats_amd as bsa
import oracle
import synth

TOL = {"bf16": dict(max_abs=2e-2, mean_abs=2e-3), "f32": dict(max_abs=1e-4, mean_abs=1e-4)}
TIE_REL = 1e-6


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def check_idx(gpu_idx: np.ndarray, ora_idx: np.ndarray, S: np.ndarray, topk: int) -> int:
    """Returns the number of rows whose sets differ (all within the tie rule);
    raises AssertionError for any difference outside it."""
    differ = 0
    for i in range(ora_idx.shape[0]):
        g, o = set(gpu_idx[i].tolist()), set(ora_idx[i].tolist())
        assert len(g) == topk and list(gpu_idx[i]) == sorted(gpu_idx[i]), f"row {i} not a sorted set"
        if g == o:
            continue
        differ += 1
        row = np.sort(S[i])[::-1]
        kth = row[topk - 1]
        nxt = row[topk] if topk < row.size else row[topk - 1]
        band = TIE_REL * max(abs(kth), abs(nxt))
        for j in g ^ o:
            assert abs(S[i, j] - kth) <= band, f"row {i}: block {j} differs outside the tie band"
    return differ


def compare_out(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    err = np.abs(gpu.astype(np.float64) - ref)
    mx, mean = float(err.max()), float(err.mean())
    tol = TOL[dtype]
    log(f"    {what}: max-abs {mx:.3e} mean-abs {mean:.3e} (bar {tol['max_abs']:.0e}/{tol['mean_abs']:.0e})")
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    assert mx <= tol["max_abs"], f"{what}: max-abs {mx} > {tol['max_abs']}"
    assert mean <= tol["mean_abs"], f"{what}: mean-abs {mean} > {tol['mean_abs']}"
    return mx, mean


def sample_qblocks(n: int, count: int, seed: int) -> list[int]:
    if count >= n:
        return list(range(n))
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(np.arange(1, n - 1), size=count - 2, replace=False).tolist())
    return sorted(pick | {0, n - 1})


def run_gpu(w: synth.Workload, q, k, v, oracle_idx=None):
    """The whole HIP path on device tensors: stats, selection, fused pass."""
    s = w.scale
    n = w.n_blocks
    topk = bsa.topk_from_density(w.density, n)
    st = bsa.block_stats(q, k, v, w.block, want_mnorm=w.cov_weight > 0)
    idx = bsa.select(st, topk, s, w.cov_weight, w.sink_idx)
    o = bsa.attn_fwd(q, st, idx, s, w.variant)
    o_or = None
    if oracle_idx is not None:
        oi = torch.from_numpy(oracle_idx.astype(np.int32)).to(q.device)
        o_or = bsa.attn_fwd(q, st, oi, s, w.variant)
    torch.cuda.synchronize()
    return st, idx, o, o_or


def check_workload(w: synth.Workload, heads=None, qblock_sample: int | None = None,
                   check_gpu_idx_output: bool = True, seed: int = 0, qkv=None):
    """Full GPU run on all heads; oracle comparison on `heads` (default: all)
    and, per head, on `qblock_sample` query blocks (default: all). `qkv`
    replaces the generated inputs (CPU tensors of the workload's shape)."""
    t0 = time.time()
    log(f"[{w.name}] B={w.B} H={w.H} L={w.L} D={w.D} blk={w.block} d={w.density} {w.variant} "
        f"sink={w.sink_idx} cov={w.cov_weight} {w.dtype}")
    q, k, v = synth.make_qkv(w) if qkv is None else qkv
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    n = w.n_blocks
    topk = bsa.topk_from_density(w.density, n)
    assert topk == oracle.topk_from_density(w.density, n)
    heads = heads if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]
    # oracle selection of the checked heads (full), used for the output comparison
    ora = {}
    for (b, h) in heads:
        qh, kh, vh = (synth.as_f64(x[b, h]) for x in (q, k, v))
        qbs = None if qblock_sample is None else sample_qblocks(n, qblock_sample, seed + 7 * h + b)
        o_ref, idx_ref, st_ref, S = oracle.head_forward(
            qh, kh, vh, block=w.block, topk=topk, scale=w.scale, variant=w.variant,
            sink_idx=w.sink_idx, cov_weight=w.cov_weight, qblocks=qbs, want_stats=True)
        ora[(b, h)] = (o_ref, idx_ref, st_ref, S, qbs)
    idx_full = np.zeros((w.B, w.H, n, topk), dtype=np.int64)
    for (b, h), val in ora.items():
        idx_full[b, h] = val[1]
    st, idx, o, o_or = run_gpu(w, qd, kd, vd, oracle_idx=idx_full)
    res = dict(differ_rows=0, max_abs=0.0, mean_abs=0.0)
    qbar, kbar, vsum, hbar = (x.cpu().numpy() for x in (st.qbar, st.kbar, st.vsum, st.hbar))
    mnorm = st.mnorm.cpu().numpy() if st.mnorm is not None else None
    gidx = idx.cpu().numpy()
    o_g = o.float().cpu().numpy()
    o_o = o_or.float().cpu().numpy()
    for (b, h), (o_ref, idx_ref, st_ref, S, qbs) in ora.items():
        np.testing.assert_allclose(qbar[b, h], st_ref["qbar"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(kbar[b, h], st_ref["kbar"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(vsum[b, h], st_ref["vsum"], rtol=0, atol=1e-10)
        # H̄ is accumulated in fp32 (exact bf16 products): its rounding error scales with
        # the magnitude of the summed products Σ|k||v|/n, not with H̄ itself
        gscale = float((np.abs(synth.as_f64(k[b, h])).T @ np.abs(synth.as_f64(v[b, h]))).max()) / n
        np.testing.assert_allclose(hbar[b, h], st_ref["Hbar"], rtol=0, atol=2e-6 * gscale + 1e-12)
        if mnorm is not None:
            # M_j = ||H_j - H̄||_F over D² entries, each accumulated in fp32 like H̄:
            # an absolute term of the same kind (per block, times D for the norm)
            # covers values near 0, e.g. a single block, where H̄ = H_0 exactly
            kh, vh = np.abs(synth.as_f64(k[b, h])), np.abs(synth.as_f64(v[b, h]))
            bscale = max(float((kh[j * w.block:(j + 1) * w.block].T @ vh[j * w.block:(j + 1) * w.block]).max())
                         for j in range(n))
            np.testing.assert_allclose(mnorm[b, h], st_ref["M"], rtol=1e-6, atol=2e-6 * w.D * bscale)
        res["differ_rows"] += check_idx(gidx[b, h], idx_ref, S, topk)
        rows = np.arange(w.L) if qbs is None else np.concatenate(
            [np.arange(i * w.block, min(w.L, (i + 1) * w.block)) for i in qbs])
        mx, mean = compare_out(o_o[b, h, rows], o_ref[rows], w.dtype, f"head ({b},{h}) oracle idx")
        res["max_abs"] = max(res["max_abs"], mx)
        res["mean_abs"] = max(res["mean_abs"], mean)
        if check_gpu_idx_output:
            same = [i for i in (range(n) if qbs is None else qbs)
                    if np.array_equal(gidx[b, h, i], idx_ref[i])]
            if same:
                r2 = np.concatenate([np.arange(i * w.block, min(w.L, (i + 1) * w.block)) for i in same])
                np.testing.assert_array_equal(o_g[b, h, r2], o_o[b, h, r2])
    log(f"[{w.name}] ok in {time.time() - t0:.1f}s; idx rows differing within ties: {res['differ_rows']}")
    res["stats"] = st
    return res
