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


U32 = 2.0 ** -24  # unit roundoff of fp32


def gamma(m: int) -> float:
    """Recursive-summation constant: any sum of m terms in fp32 is off by at
    most gamma(m) times the sum of the terms' magnitudes."""
    return m * U32 / (1.0 - m * U32)


def stats_bounds(k: np.ndarray, v: np.ndarray, st_ref: dict, block: int, dtype: str, want_m: bool,
                 cov_norm: str = "fro"):
    """Largest errors the library's arithmetic allows in H̄ (per element) and
    in M_j (per block), for one head's fp64 k, v [L, D].

    The library forms H_j per block on MFMA: the products k_td·v_te are exact
    in fp32 for bf16 inputs (one rounding each for fp32 inputs), and a run of
    consecutive blocks (at most 1024 tokens) is summed in one fp32 accumulator
    from which k̄_j·ΣV_j (both rounded to fp32, their product rounded again) is
    subtracted as each block ends. The runs are then summed in fp64 and divided
    by n. Each run sums at most m = 1024 + 1024/block terms, so
        |ΔH̄_de| ≤ (1/n) [(γ_m + u_in) Σ_t |k_td||v_te| + (γ_m + 3u) Σ_j |k̄_jd||ΣV_je|]
    with u_in = u for fp32 inputs, else 0 (fp64 roundings are below 1e-15 of it).
    The Frobenius M_j = ||H_j − H̄||_F is formed in fp64 from the block's
    G_j = Σ_t k_tᵀv_t, accumulated in fp32 over its n_j tokens, minus
    k̄_jᵀΣV_j in fp64, minus the H̄ above, so
        |ΔM_j| ≤ ||(γ_{n_j} + u_in) |K_j|ᵀ|V_j| ||_F + ||ΔH̄ bound||_F.
    The spectral M_j = ||H_j − H̄||_2 sums G_j in fp64 (exact products, n_j
    terms: n_j·2^-53 relative) and finds the largest eigenvalue of the Gram
    matrix by a backward-stable fp64 reduction, within 1e-12 relative here;
    since | ||A||_2 − ||A'||_2 | ≤ ||A − A'||_2 ≤ ||A − A'||_F the same form of
    bound holds."""
    n = st_ref["kbar"].shape[0]
    L = k.shape[0]
    u_in = U32 if dtype == "f32" else 0.0
    m = 1024 + 1024 // block
    ka, va = np.abs(k), np.abs(v)
    kv = ka.T @ va
    kbvs = np.abs(st_ref["kbar"]).T @ np.abs(st_ref["vsum"])
    hb = ((gamma(m) + u_in) * kv + (gamma(m) + 3 * U32) * kbvs) / n + 1e-13
    if not want_m:
        return hb, None
    hb_f = float(np.sqrt((hb * hb).sum()))
    mb = np.empty(n)
    for j in range(n):
        lo, hi = j * block, min(L, (j + 1) * block)
        c = gamma(hi - lo) + u_in if cov_norm == "fro" else 1.01 * (hi - lo) * 2.0 ** -53
        g = c * (ka[lo:hi].T @ va[lo:hi])
        mb[j] = float(np.sqrt((g * g).sum())) + hb_f + 1e-12 * (1.0 + float(st_ref["M"][j]))
    return hb, mb


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
    st = bsa.block_stats(q, k, v, w.block, want_mnorm=w.cov_weight > 0, cov_norm=w.cov_norm)
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
            sink_idx=w.sink_idx, cov_weight=w.cov_weight, qblocks=qbs, want_stats=True,
            cov_ord=w.cov_norm)
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
        # H̄ and M_j: bounds derived from the library's arithmetic (stats_bounds)
        kh, vh = synth.as_f64(k[b, h]), synth.as_f64(v[b, h])
        hb_bound, m_bound = stats_bounds(kh, vh, st_ref, w.block, w.dtype, mnorm is not None, w.cov_norm)
        err_h = np.abs(hbar[b, h] - st_ref["Hbar"])
        log(f"    head ({b},{h}) H-bar: max-abs {err_h.max():.3e}, largest share of its bound "
            f"{(err_h / hb_bound).max():.2e}")
        assert (err_h <= hb_bound).all(), \
            f"H-bar off by {err_h.max():.3e}, bound {hb_bound.flat[err_h.argmax()]:.3e}"
        if mnorm is not None:
            err_m = np.abs(mnorm[b, h] - st_ref["M"])
            assert (err_m <= m_bound).all(), f"M_j off by {err_m.max():.3e}, bound {m_bound[err_m.argmax()]:.3e}"
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


# Gradients (backward of the zeroth-order variant), relative to the largest
# reference entry of each tensor: the kernels round the weights p̃ and their
# gradients dS to the I/O dtype as matrix-core operands (relative 2^-9 for
# bf16) and use the forward's rounded output for Δ_t = dO_t·o_t, so each
# gradient entry is off by a few 2^-9 of the sum of its terms' magnitudes.
# On top of that an absolute floor: dS_tx = p̃_tx (dO_t·V'_x − w_x Δ_t) takes
# the difference of two D-term fp32 dot products, each off by up to
# γ_D |dO_t|·|v|, which s·|k| (or s·|q|) carries into dq (dk); where the two
# cancel (a single key: o = v and dq = 0) that floor is all that is left.
GRAD_TOL = {"bf16": dict(max_rel=2e-2, rms_rel=1e-2), "f32": dict(max_rel=1e-4, rms_rel=1e-4)}


def compare_grad(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str, floor: float = 0.0):
    err = np.abs(gpu.astype(np.float64) - ref)
    scale = float(np.abs(ref).max())
    rms_ref = float(np.sqrt((ref ** 2).mean()))
    tol = GRAD_TOL[dtype]
    mx, rms = float(err.max()), float(np.sqrt((err ** 2).mean()))
    bar_mx, bar_rms = tol["max_rel"] * scale + floor, tol["rms_rel"] * rms_ref + floor
    log(f"    {what}: max-abs {mx:.3e} (bar {bar_mx:.3e} = {tol['max_rel']:.0e} x max|ref| + floor {floor:.1e}), "
        f"rms {rms:.3e} (bar {bar_rms:.3e})")
    assert np.isfinite(gpu).all(), f"{what}: non-finite gradient"
    assert mx <= bar_mx, f"{what}: max-abs {mx} > {bar_mx}"
    assert rms <= bar_rms, f"{what}: rms {rms} > {bar_rms}"


def grad_floor(q, k, v, do, scale: float, D: int) -> float:
    """The absolute floor above, for one head's fp64 inputs."""
    nrm = lambda x: float(np.sqrt((x * x).sum(axis=1)).max())
    return 2.0 * gamma(D) * scale * nrm(do) * nrm(v) * max(nrm(k), nrm(q)) + 1e-30


def lse_bound(q, k, v, st_ref: dict, scale: float, dtype: str, lse_ref: np.ndarray) -> np.ndarray:
    """Largest error the forward's ln D_t may carry, per row, for one head's
    fp64 inputs. The exact logits come from the inputs as read (products exact
    in fp32 for bf16) with an fp32 sum; a centroid logit uses k̄_j rounded to
    the I/O dtype, off by up to s Σ_d |q_td||k̄_jd| times its unit roundoff;
    the weights are summed in fp32, in some tiles after rounding them to the
    I/O dtype (relative 2^-9 for bf16). ln D_t moves by at most the largest
    logit error plus the relative error of the sum."""
    u_io = 2.0 ** -9 if dtype == "bf16" else U32
    qa = np.abs(q)
    cent = scale * float(u_io) * (qa @ np.abs(st_ref["kbar"]).T).max(axis=1)
    exact = scale * gamma(q.shape[1]) * (qa @ np.abs(k).T).max(axis=1)
    return np.maximum(cent, exact) + u_io + 2 * gamma(q.shape[0] + 64) + 1e-6 * (1.0 + np.abs(lse_ref))


def check_backward(w: synth.Workload, heads=None):
    """The backward pass on the GPU (all heads, the oracle's selection, the
    GPU's own forward output) against the oracle's gradients on `heads`, both
    with the forward's ln D_t handed over and with the backward recomputing
    it; and the forward's ln D_t against the oracle's."""
    t0 = time.time()
    log(f"[{w.name}] backward B={w.B} H={w.H} L={w.L} D={w.D} blk={w.block} d={w.density} "
        f"sink={w.sink_idx} {w.dtype}")
    q, k, v = synth.make_qkv(w)
    do = synth.grad_out(w)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    n = w.n_blocks
    topk = bsa.topk_from_density(w.density, n)
    heads = heads if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]
    idx = np.zeros((w.B, w.H, n, topk), dtype=np.int64)
    for (b, h) in heads:
        qh, kh, vh = (synth.as_f64(x[b, h]) for x in (q, k, v))
        _, idx[b, h] = oracle.head_forward(qh, kh, vh, block=w.block, topk=topk, scale=w.scale, variant="0th",
                                           sink_idx=w.sink_idx, cov_weight=w.cov_weight, cov_ord=w.cov_norm)
    idx_d = torch.from_numpy(idx.astype(np.int32)).to(dev)
    st = bsa.block_stats(qd, kd, vd, w.block)
    o, lse = bsa.attn_fwd(qd, st, idx_d, w.scale, "0th", return_lse=True)
    o_plain = bsa.attn_fwd(qd, st, idx_d, w.scale, "0th")
    dq, dk, dv = bsa.attn_bwd(qd, kd, vd, st, idx_d, w.scale, o, dod, lse=lse)
    dq2, dk2, dv2 = bsa.attn_bwd(qd, kd, vd, st, idx_d, w.scale, o, dod)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain), "the output does not depend on whether ln D_t is written"
    g = [x.float().cpu().numpy() for x in (dq, dk, dv)]
    g2 = [x.float().cpu().numpy() for x in (dq2, dk2, dv2)]
    lse_h = lse.cpu().numpy()
    for (b, h) in heads:
        qh, kh, vh, doh = (synth.as_f64(x[b, h]) for x in (q, k, v, do))
        lref = oracle.head_log_denominator(qh, kh, vh, block=w.block, idx=idx[b, h], scale=w.scale)
        bound = lse_bound(qh, kh, vh, oracle.block_stats(qh, kh, vh, w.block), w.scale, w.dtype, lref)
        err = np.abs(lse_h[b, h].astype(np.float64) - lref)
        log(f"    head ({b},{h}) ln D_t: max-abs {err.max():.3e}, largest fraction of its bound "
            f"{(err / bound).max():.3f}")
        assert np.isfinite(lse_h[b, h]).all() and (err <= bound).all(), "ln D_t outside its bound"
        ref = oracle.head_backward(qh, kh, vh, doh, block=w.block, idx=idx[b, h], scale=w.scale)
        fl = grad_floor(qh, kh, vh, doh, w.scale, w.D)
        for name, gg, gg2, rr in zip(("dq", "dk", "dv"), g, g2, ref):
            compare_grad(gg[b, h], rr, w.dtype, f"head ({b},{h}) {name}", fl)
            compare_grad(gg2[b, h], rr, w.dtype, f"head ({b},{h}) {name}, denominators recomputed", fl)
    log(f"[{w.name}] backward ok in {time.time() - t0:.1f}s")
    return dict(st=st, idx=idx_d, o=o, lse=lse, grads=(dq, dk, dv), inputs=(qd, kd, vd, dod))
