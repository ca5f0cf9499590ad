"""fp64 CPU oracle for PISA's piecewise sparse attention forward pass.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call anything here.
The HIP library never calls it and shares no code, header, table or helper with
it; the two meet only in the seeded input generator ``synth``.

What it computes, in the order the pages give it (sources are cited by page and
section; "gist" = the gist.science technical summary of arXiv 2602.01077,
"README" = the authors' README mirror, "skill" = the skillmd.com page):

1. partition the sequence into blocks of ``block_size`` tokens, queries and keys
   alike, the last block possibly shorter (skill, "Architecture Overview";
   README, "Attention sink for MMDiT" example with block_size=64);
2. block statistics (gist, section 2 "Core Algorithm" and "Hardware
   Implementation", pre-computation): mean-pooled query blocks q̄_i, key
   centroids k̄_j, value sums ΣV_j, the block first-order matrices
   H_j = Σ_n (k_n − k̄_j)ᵀ v_n and their mean H̄ over all blocks;
3. optional covariance norm M_j = ‖H_j − H̄‖ (gist, "Covariance-Aware Routing");
4. per-query-block scores from the pooled statistics, plus λ·M_j, with the sink
   block forced in (README, "Attention sink for MMDiT");
5. top-k per query block, indices ascending (skill, block selection snippet);
6. o_t = N_t / D_t with the exact terms of the selected blocks, the zeroth-order
   terms α_tj = exp(s q_t·k̄_j) of the unselected ones and, for the hybrid
   variant, the global first-order term (gist, "Core Algorithm", N_t equation;
   README, "Kernel variants" for the zeroth-order-only variant). The per-block
   first-order variant ("pb1") gives every unselected block its own first-order
   term α_tj·s·q_t H_j instead: the distinct per-block terms the gist's "Core
   Algorithm" replaces by the global mean H̄, and the first-order variant the
   atlas summary's results compare against.

Readings where the pages are silent or garbled (each is listed in the design doc):
  * the softmax scale s (default 1/√D) multiplies every logit and the first-order
    term, since the gist's N_t equation prints no scale;
  * D_t = Σ_S Σ_n e^{ℓ} + Σ_U n_j α_tj: the first-order part of the denominator
    vanishes identically because k̄_j is the centroid;
  * ΣV_j sums the n_j tokens actually present; H̄ is the unweighted mean over all
    n blocks, ragged block included;
  * k = clamp(floor(density·n), 1, n) in fp64, the one count rule printed (skill,
    select_critical_blocks);
  * equal scores: lower block index wins;
  * the sink takes one of the k slots (score +inf); −1 names block n−1;
  * covariance routing is additive, score = s·q̄_i·k̄_j + λ·M_j, with the Frobenius
    norm for M_j by default and the spectral norm as the option the gist's
    "‖·‖_2" names.
The last three points and the floor rule are parity unpinned by the pages: the
tests check the oracle's internal consistency for them, nothing more.
"""

from __future__ import annotations

import math

import numpy as np

SINK_NONE = None


def num_blocks(L: int, block: int) -> int:
    """Number of blocks when L tokens are cut into blocks of ``block`` tokens."""
    return -(-L // block)


def block_sizes(L: int, block: int) -> np.ndarray:
    """n_j for every block j: ``block`` except a shorter last block."""
    n = num_blocks(L, block)
    sizes = np.full(n, block, dtype=np.int64)
    sizes[-1] = L - (n - 1) * block
    return sizes


def topk_from_density(density: float, n: int) -> int:
    """k = clamp(floor(density·n), 1, n), evaluated in fp64 (skill page,
    select_critical_blocks count rule; the README passes ``density`` as a float)."""
    k = int(math.floor(float(density) * float(n)))
    return max(1, min(n, k))


def block_stats(q: np.ndarray, k: np.ndarray, v: np.ndarray, block: int) -> dict:
    """Pre-computation of the gist summary (section 2, "Hardware Implementation",
    step 1; symbols from "Core Algorithm").

    q, k, v: [L, D] float64 for one (batch, head). Returns
      qbar [n, D]  mean of the query rows of block i,
      kbar [n, D]  key centroid k̄_j,
      vsum [n, D]  ΣV_j = Σ_n v_{j,n} (a sum, not a mean),
      H    [n, D, D] H_j = Σ_n (k_{j,n} − k̄_j)ᵀ v_{j,n},
      Hbar [D, D]  mean of H_j over all n blocks,
      sizes [n]    n_j.
    """
    L, D = q.shape
    n = num_blocks(L, block)
    sizes = block_sizes(L, block)
    qbar = np.empty((n, D))
    kbar = np.empty((n, D))
    vsum = np.empty((n, D))
    H = np.empty((n, D, D))
    for j in range(n):
        lo, hi = j * block, min(L, (j + 1) * block)
        qbar[j] = q[lo:hi].sum(axis=0) / sizes[j]
        kbar[j] = k[lo:hi].sum(axis=0) / sizes[j]
        vsum[j] = v[lo:hi].sum(axis=0)
        H[j] = (k[lo:hi] - kbar[j]).T @ v[lo:hi]
    Hbar = H.sum(axis=0) / n
    return dict(qbar=qbar, kbar=kbar, vsum=vsum, H=H, Hbar=Hbar, sizes=sizes)


def cov_norm(H: np.ndarray, Hbar: np.ndarray, ord: str = "fro") -> np.ndarray:
    """M_j = ‖H_j − H̄‖ (gist, "Covariance-Aware Routing"). ``ord="fro"``: the
    Frobenius norm, sqrt of the sum of squares (the skill page's
    score_attention_blocks takes a Frobenius norm); ``ord="spectral"``: the
    2-norm the gist prints, the largest singular value (LAPACK's SVD)."""
    d = H - Hbar[None]
    if ord == "fro":
        return np.sqrt((d * d).sum(axis=(1, 2)))
    if ord == "spectral":
        return np.linalg.norm(d, ord=2, axis=(1, 2))
    raise ValueError("ord must be 'fro' or 'spectral'")


def sink_block(sink_idx, n: int):
    """Block forced into every exact set: 0 → first, −1 → last, None → none
    (README, "Attention sink for MMDiT")."""
    if sink_idx is None:
        return None
    if sink_idx == 0:
        return 0
    if sink_idx == -1:
        return n - 1
    raise ValueError("sink_idx must be None, 0 or -1")


def pooled_scores(qbar: np.ndarray, kbar: np.ndarray, scale: float, M=None,
                  cov_weight: float = 0.0, sink_idx=None) -> np.ndarray:
    """Routing scores S_ij = s·q̄_i·k̄_j + λ·M_j, the sink column set to +inf."""
    S = scale * (qbar @ kbar.T)
    if cov_weight:
        S = S + cov_weight * M[None, :]
    sb = sink_block(sink_idx, kbar.shape[0])
    if sb is not None:
        S[:, sb] = np.inf
    return S


def select_topk(S: np.ndarray, topk: int) -> np.ndarray:
    """Per row, the ``topk`` largest scores; equal scores go to the lower index;
    each row's indices are returned ascending. [n_q, topk] int64."""
    n_q, n = S.shape
    cols = np.broadcast_to(np.arange(n), S.shape)
    order = np.lexsort((cols, -S), axis=-1)  # primary key -S, then index
    return np.sort(order[:, :topk], axis=1)


def pisa_rows(q, k, v, st: dict, idx_i: np.ndarray, i: int, block: int, scale: float,
              first_order: bool, per_block: bool = False):
    """N_t, D_t and the shift m_t for every query row t of query block i.

    gist, "Core Algorithm": N_t = Σ_{S_i} Σ_n e^{ℓ_tn} v_n + Σ_{U_i} α_tj ΣV_j
    + q_t H̄ Σ_{U_i} α_tj with α_tj = exp(s q_t k̄_jᵀ); D_t holds the same exact and
    zeroth-order terms without the values, n_j α_tj for a block of n_j tokens.
    Every exponent is shifted by the row maximum m_t; the unshifted values are
    N_t·e^{m_t} and D_t·e^{m_t}.

    per_block (instead of first_order): each unselected block's own first-order
    term Σ_{U_i} α_tj s q_t H_j, the term that the global H̄ stands in for. D_t is
    the same, since the first-order part of a block's denominator is
    α_tj s q_t Σ_n (k_n − k̄_j) = 0.
    """
    L = q.shape[0]
    n = st["kbar"].shape[0]
    rows = slice(i * block, min(L, (i + 1) * block))
    Qi = q[rows]
    sel = np.asarray(idx_i)
    mask = np.ones(n, dtype=bool)
    mask[sel] = False
    uns = np.nonzero(mask)[0]
    Ksel = np.concatenate([k[j * block:min(L, (j + 1) * block)] for j in sel])
    Vsel = np.concatenate([v[j * block:min(L, (j + 1) * block)] for j in sel])
    ell = scale * (Qi @ Ksel.T)  # exact logits of the selected blocks
    m = ell.max(axis=1)
    if uns.size:
        c = scale * (Qi @ st["kbar"][uns].T)  # centroid logits of the others
        m = np.maximum(m, c.max(axis=1))
    P = np.exp(ell - m[:, None])
    Dt = P.sum(axis=1)
    Nt = P @ Vsel
    if uns.size:
        alpha = np.exp(c - m[:, None])
        Dt = Dt + alpha @ st["sizes"][uns].astype(np.float64)
        Nt = Nt + alpha @ st["vsum"][uns]
        if first_order:
            Nt = Nt + alpha.sum(axis=1)[:, None] * scale * (Qi @ st["Hbar"])
        elif per_block:
            for u, j in enumerate(uns):
                Nt = Nt + alpha[:, u:u + 1] * scale * (Qi @ st["H"][j])
    return Nt, Dt, m


def dense_rows(q, k, v, rows: slice, scale: float) -> np.ndarray:
    """Plain softmax(s·QKᵀ)·V for the given query rows (skill page,
    compute_exact_attention, used only as the definition of dense attention)."""
    ell = scale * (q[rows] @ k.T)
    ell = ell - ell.max(axis=1, keepdims=True)
    P = np.exp(ell)
    return (P @ v) / P.sum(axis=1, keepdims=True)


def head_forward(q, k, v, *, block: int, topk: int, scale: float, variant: str = "hyd",
                 sink_idx=None, cov_weight: float = 0.0, idx=None, qblocks=None,
                 want_stats: bool = False, cov_ord: str = "fro"):
    """Whole forward pass for one (batch, head).

    q, k, v [L, D] float64. ``idx`` overrides the selection; ``qblocks`` limits
    the output to those query blocks (other rows are NaN). Returns (o, idx) or
    (o, idx, stats, scores).
    """
    if variant not in ("hyd", "0th", "pb1"):
        raise ValueError("variant must be 'hyd', '0th' or 'pb1'")
    L, D = q.shape
    st = block_stats(q, k, v, block)
    n = st["kbar"].shape[0]
    M = cov_norm(st["H"], st["Hbar"], cov_ord) if cov_weight else None
    st["M"] = M
    S = pooled_scores(st["qbar"], st["kbar"], scale, M, cov_weight, sink_idx)
    if idx is None:
        idx = select_topk(S, topk)
    o = np.full((L, D), np.nan)
    for i in (range(n) if qblocks is None else qblocks):
        Nt, Dt, _ = pisa_rows(q, k, v, st, idx[i], i, block, scale, variant == "hyd",
                              variant == "pb1")
        o[i * block:min(L, (i + 1) * block)] = Nt / Dt[:, None]
    if want_stats:
        return o, idx, st, S
    return o, idx


def head_log_denominator(q, k, v, *, block: int, idx: np.ndarray, scale: float) -> np.ndarray:
    """ln D_t for every row of one (batch, head) under the selection idx: the
    natural log of the denominator of the gist's "Core Algorithm" N_t / D_t,
    taken over unshifted exponentials (m_t plus the log of the shifted sum).
    It is the same for all three variants, whose first-order terms add nothing
    to D_t. q, k, v: [L, D] float64; returns [L]."""
    L = q.shape[0]
    st = block_stats(q, k, v, block)
    out = np.empty(L)
    for i in range(st["kbar"].shape[0]):
        _, Dt, m = pisa_rows(q, k, v, st, idx[i], i, block, scale, False)
        out[i * block:min(L, (i + 1) * block)] = m + np.log(Dt)
    return out


def head_backward(q, k, v, do, *, block: int, idx: np.ndarray, scale: float):
    """Gradients of the zeroth-order-only forward pass (README, "Kernel
    variants": the ``_0th`` variant is the one that supports training) with
    respect to q, k and v, for one (batch, head), the selection ``idx`` held
    fixed. q, k, v, do: [L, D] float64; returns (dq, dk, dv).

    The forward pass (gist, "Core Algorithm", N_t equation without the
    first-order term) is o_t = N_t / D_t with
      N_t = Σ_{S_i} Σ_n e^{ℓ_tn} v_n + Σ_{U_i} α_tj ΣV_j,
      D_t = Σ_{S_i} Σ_n e^{ℓ_tn}   + Σ_{U_i} n_j α_tj,
    ℓ_tn = s q_t·k_n, α_tj = e^{s q_t·k̄_j}. Writing p_tn = e^{ℓ_tn} / D_t and
    a_tj = α_tj / D_t, the chain rule gives, with Δ_t = dO_t·o_t:
      ∂L/∂ℓ_tn = p_tn (dO_t·v_n − Δ_t),
      ∂L/∂c_tj = a_tj (dO_t·ΣV_j − n_j Δ_t)        (c_tj = s q_t·k̄_j),
      dq_t    = s [Σ_{S_i} Σ_n ∂L/∂ℓ_tn k_n + Σ_{U_i} ∂L/∂c_tj k̄_j],
      dk_n   += s Σ_t ∂L/∂ℓ_tn q_t,  dv_n += Σ_t p_tn dO_t   (rows t whose block selects n's),
      dk̄_j   += s Σ_t ∂L/∂c_tj q_t,  dΣV_j += Σ_t a_tj dO_t (rows t whose block leaves j out),
    and k̄_j = (1/n_j) Σ_{n∈j} k_n, ΣV_j = Σ_{n∈j} v_n pass dk̄_j / n_j and
    dΣV_j on to every token of block j."""
    L, D = q.shape
    n = num_blocks(L, block)
    sizes = block_sizes(L, block).astype(np.float64)
    st = block_stats(q, k, v, block)
    kbar, vsum = st["kbar"], st["vsum"]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dkbar = np.zeros((n, D))
    dvsum = np.zeros((n, D))
    span = lambda j: slice(j * block, min(L, (j + 1) * block))
    for i in range(n):
        rows = span(i)
        Qi, dOi = q[rows], do[rows]
        sel = np.asarray(idx[i])
        mask = np.ones(n, dtype=bool)
        mask[sel] = False
        uns = np.nonzero(mask)[0]
        Ksel = np.concatenate([k[span(j)] for j in sel])
        Vsel = np.concatenate([v[span(j)] for j in sel])
        ell = scale * (Qi @ Ksel.T)
        c = scale * (Qi @ kbar[uns].T)
        m = ell.max(axis=1)
        if uns.size:
            m = np.maximum(m, c.max(axis=1))
        P = np.exp(ell - m[:, None])
        A = np.exp(c - m[:, None])
        Dt = P.sum(axis=1) + A @ sizes[uns]
        o = (P @ Vsel + A @ vsum[uns]) / Dt[:, None]
        p, a = P / Dt[:, None], A / Dt[:, None]
        delta = (dOi * o).sum(axis=1)
        dl = p * (dOi @ Vsel.T - delta[:, None])
        dc = a * (dOi @ vsum[uns].T - sizes[uns][None, :] * delta[:, None])
        dq[rows] = scale * (dl @ Ksel + dc @ kbar[uns])
        dK, dV = scale * (dl.T @ Qi), p.T @ dOi
        off = 0
        for j in sel:
            nj = int(sizes[j])
            dk[span(j)] += dK[off:off + nj]
            dv[span(j)] += dV[off:off + nj]
            off += nj
        dkbar[uns] += scale * (dc.T @ Qi)
        dvsum[uns] += a.T @ dOi
    for j in range(n):
        dk[span(j)] += dkbar[j] / sizes[j]
        dv[span(j)] += dvsum[j]
    return dq, dk, dv


def effective_flops(L: int, D: int, block: int, idx: np.ndarray, first_order: bool,
                    per_block: bool = False) -> float:
    """Credited FLOPs of the fused pass for one (batch, head): 4·D per exact
    (query, key) pair, 4·D per (query, unselected block) pair, and 2·D² per query
    row for the first-order term when its query block has unselected blocks
    (per_block: 2·D² per (query, unselected block) pair instead)."""
    sizes = block_sizes(L, block)
    n = sizes.size
    total = 0.0
    for i in range(idx.shape[0]):
        nq = int(sizes[i])
        exact = int(sizes[idx[i]].sum())
        nu = n - idx.shape[1]
        total += nq * (4.0 * D * exact + 4.0 * D * nu)
        if first_order and nu > 0:
            total += 2.0 * nq * D * D
        if per_block:
            total += 2.0 * nq * D * D * nu
    return total
