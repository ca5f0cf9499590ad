"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test ties one part of the oracle to something other than itself: a
hand-derived worked example, a textbook routine it must reduce to, a closed-form
asymptotic or an invariant. Pages: "gist" = gist.science technical summary of
arXiv 2602.01077, "README" = the authors' README mirror, "skill" = the
skillmd.com page.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_2block.json")


def closed_form(terms):
    return sum(float(Fraction(a, b)) * math.exp(float(Fraction(c, d))) for a, b, c, d in terms)


def sdpa(q, k, v, scale):
    """Textbook dense attention from torch (CPU, fp64), independent of the oracle."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=scale)[0, 0].numpy()


def rand_head(L, D, seed, cluster=None):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(L, D))
    k = rng.normal(size=(L, D))
    v = rng.normal(size=(L, D))
    return q, k, v


# --------------------------------------------------------------------------- P3
@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_worked_example_stats(golden):
    g = golden
    q, k, v = (np.array(g["inputs"][x], dtype=np.float64) for x in "qkv")
    st = oracle.block_stats(q, k, v, g["inputs"]["block"])
    for key in ("qbar", "kbar", "vsum", "H", "Hbar"):
        np.testing.assert_array_equal(st[key], np.array(g["stats"][key], dtype=np.float64), err_msg=key)
    M = oracle.cov_norm(st["H"], st["Hbar"])
    np.testing.assert_allclose(M, g["stats"]["M_frobenius"], rtol=0, atol=1e-15)
    S = oracle.pooled_scores(st["qbar"], st["kbar"], 1.0)
    np.testing.assert_array_equal(S, np.array(g["scores"]))
    np.testing.assert_array_equal(oracle.select_topk(S, 1), np.array(g["idx"]))


@pytest.mark.parametrize("variant", ["hyd", "0th", "pb1"])
def test_worked_example_terms(golden, variant):
    """N_t and D_t term by term against the hand-derived closed forms."""
    g = golden
    q, k, v = (np.array(g["inputs"][x], dtype=np.float64) for x in "qkv")
    st = oracle.block_stats(q, k, v, 2)
    idx = np.array(g["idx"])
    for row in g["rows"]:
        t = row["t"]
        i = t // 2
        Nt, Dt, m = oracle.pisa_rows(q, k, v, st, idx[i], i, 2, 1.0, variant == "hyd",
                                     per_block=variant == "pb1")
        r = t % 2
        N_exp = [closed_form(c) for c in row["N_" + variant]]
        D_exp = closed_form(row["D"])
        np.testing.assert_allclose(Nt[r] * math.exp(m[r]), N_exp, rtol=1e-14)
        np.testing.assert_allclose(Dt[r] * math.exp(m[r]), D_exp, rtol=1e-14)


def test_worked_example_outputs(golden):
    g = golden
    q, k, v = (np.array(g["inputs"][x], dtype=np.float64) for x in "qkv")
    for variant in ("hyd", "0th", "pb1"):
        o, idx = oracle.head_forward(q, k, v, block=2, topk=1, scale=1.0, variant=variant)
        exp = np.array([[closed_form(c) for c in row["N_" + variant]] for row in g["rows"]])
        exp /= np.array([closed_form(row["D"]) for row in g["rows"]])[:, None]
        np.testing.assert_allclose(o, exp, rtol=1e-14)
    dense = np.array([[closed_form(c) for c in row["N_dense"]] for row in g["rows"]])
    dense /= np.array([closed_form(row["D_dense"]) for row in g["rows"]])[:, None]
    np.testing.assert_allclose(oracle.dense_rows(q, k, v, slice(0, 4), 1.0), dense, rtol=1e-14)
    # with both blocks selected the method is dense attention
    o2, _ = oracle.head_forward(q, k, v, block=2, topk=2, scale=1.0)
    np.testing.assert_allclose(o2, dense, rtol=1e-14)


# --------------------------------------------------------------------------- P1
@pytest.mark.parametrize("L,D,block", [(256, 16, 64), (200, 8, 64), (300, 32, 128), (37, 4, 8)])
@pytest.mark.parametrize("variant", ["hyd", "0th", "pb1"])
def test_density_one_is_dense(L, D, block, variant):
    q, k, v = rand_head(L, D, seed=L + D)
    s = 1.0 / math.sqrt(D)
    n = oracle.num_blocks(L, block)
    k_ = oracle.topk_from_density(1.0, n)
    assert k_ == n
    o, idx = oracle.head_forward(q, k, v, block=block, topk=k_, scale=s, variant=variant)
    np.testing.assert_allclose(o, sdpa(q, k, v, s), rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.dense_rows(q, k, v, slice(0, L), s), sdpa(q, k, v, s), atol=1e-12)


# --------------------------------------------------------------------------- P2
def constant_key_head(L, D, block, seed):
    rng = np.random.default_rng(seed)
    n = oracle.num_blocks(L, block)
    c = rng.normal(size=(n, D))
    k = np.repeat(c, block, axis=0)[:L]
    q = rng.normal(size=(L, D))
    v = rng.normal(size=(L, D))
    return q, k, v


@pytest.mark.parametrize("sink", [None, 0, -1])
@pytest.mark.parametrize("variant", ["hyd", "0th", "pb1"])
@pytest.mark.parametrize("L,block,topk", [(256, 32, 2), (250, 32, 3), (77, 16, 1)])
def test_constant_key_blocks_are_exact(sink, variant, L, block, topk):
    """Constant keys in every block: H_j = 0, H̄ = 0, α_tj e^{0} exact, so the
    method equals dense attention for any selection (north star check; gist,
    "Core Algorithm")."""
    D = 8
    q, k, v = constant_key_head(L, D, block, seed=L + topk)
    s = 0.7
    o, idx, st, _ = oracle.head_forward(q, k, v, block=block, topk=topk, scale=s, variant=variant,
                                        sink_idx=sink, want_stats=True)
    assert np.abs(st["Hbar"]).max() < 1e-13
    np.testing.assert_allclose(o, sdpa(q, k, v, s), atol=1e-12)


def test_constant_unselected_blocks_only_zeroth_exact():
    """Only the unselected blocks have constant keys: the zeroth-order variant is
    exact, the hybrid is not (its H̄ averages the selected blocks' H_j too), and
    the per-block first-order variant is exact as well (its H_j are all 0)."""
    L, D, block = 192, 8, 32
    rng = np.random.default_rng(7)
    q, k, v = rand_head(L, D, seed=7)
    n = L // block
    sel = [1, 4]
    for j in range(n):
        if j not in sel:
            k[j * block:(j + 1) * block] = rng.normal(size=D)
    idx = np.tile(np.array(sel), (n, 1))
    s = 0.5
    dense = sdpa(q, k, v, s)
    o0, _ = oracle.head_forward(q, k, v, block=block, topk=2, scale=s, variant="0th", idx=idx)
    oh, _ = oracle.head_forward(q, k, v, block=block, topk=2, scale=s, variant="hyd", idx=idx)
    op, _ = oracle.head_forward(q, k, v, block=block, topk=2, scale=s, variant="pb1", idx=idx)
    np.testing.assert_allclose(o0, dense, atol=1e-12)
    np.testing.assert_allclose(op, dense, atol=1e-12)
    assert np.abs(oh - dense).max() > 1e-6


# --------------------------------------------------------------------------- P4-P7
def test_constant_values():
    L, D, block = 200, 8, 32
    q, k, _ = rand_head(L, D, 3)
    c = np.linspace(-1, 2, D)
    v = np.tile(c, (L, 1))
    for variant in ("hyd", "0th", "pb1"):
        o, _ = oracle.head_forward(q, k, v, block=block, topk=2, scale=0.4, variant=variant, sink_idx=-1)
        np.testing.assert_allclose(o, v, atol=1e-12)


def test_key_shift_invariance():
    L, D, block = 256, 8, 32
    q, k, v = rand_head(L, D, 4)
    w = np.random.default_rng(5).normal(size=D)
    o1, i1 = oracle.head_forward(q, k, v, block=block, topk=3, scale=0.6)
    o2, i2 = oracle.head_forward(q, k + w, v, block=block, topk=3, scale=0.6)
    np.testing.assert_array_equal(i1, i2)
    np.testing.assert_allclose(o1, o2, atol=1e-11)


def test_linear_in_values():
    L, D, block = 160, 8, 32
    q, k, v1 = rand_head(L, D, 6)
    v2 = np.random.default_rng(8).normal(size=(L, D))
    a, b = 0.3, -1.7
    o1, idx = oracle.head_forward(q, k, v1, block=block, topk=2, scale=0.5)
    o2, _ = oracle.head_forward(q, k, v2, block=block, topk=2, scale=0.5, idx=idx)
    o3, _ = oracle.head_forward(q, k, a * v1 + b * v2, block=block, topk=2, scale=0.5, idx=idx)
    np.testing.assert_allclose(o3, a * o1 + b * o2, atol=1e-12)


def test_permutations_inside_blocks():
    L, D, block = 200, 8, 40
    q, k, v = rand_head(L, D, 9)
    rng = np.random.default_rng(10)
    o1, i1 = oracle.head_forward(q, k, v, block=block, topk=2, scale=0.5)
    pk = np.concatenate([j * block + rng.permutation(min(block, L - j * block)) for j in range(5)])
    o2, i2 = oracle.head_forward(q, k[pk], v[pk], block=block, topk=2, scale=0.5)
    np.testing.assert_array_equal(i1, i2)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    pq = np.concatenate([j * block + rng.permutation(block) for j in range(5)])
    o3, i3 = oracle.head_forward(q[pq], k, v, block=block, topk=2, scale=0.5)
    np.testing.assert_array_equal(i1, i3)
    np.testing.assert_allclose(o3, o1[pq], atol=1e-12)


# --------------------------------------------------------------------------- P8
def test_taylor_orders():
    """k_t = c_j + ε δ_t with Σδ = 0 in every block and the same H_j in every
    block (so H̄ = H_j): the hybrid's error is second order in ε, the zeroth-order
    variant's first order (gist, "Core Algorithm": block-wise zeroth order plus
    global first-order correction). A scale s ≠ 1 makes this also pin where s
    enters the first-order term."""
    D, block, n = 4, 8, 4
    L = block * n
    rng = np.random.default_rng(11)
    delta = rng.normal(size=(block, D))
    delta -= delta.mean(axis=0)
    vb = rng.normal(size=(block, D))
    c = rng.normal(size=(n, D))
    q = rng.normal(size=(L, D))
    v = np.tile(vb, (n, 1))
    idx = np.tile(np.array([0]), (n, 1))
    errs = {}
    for eps in (2e-2, 1e-2, 5e-3):
        k = np.repeat(c, block, axis=0) + eps * np.tile(delta, (n, 1))
        dense = sdpa(q, k, v, 0.7)
        for var in ("hyd", "0th", "pb1"):
            o, _ = oracle.head_forward(q, k, v, block=block, topk=1, scale=0.7, variant=var, idx=idx)
            errs[(var, eps)] = np.abs(o - dense).max()
            if var == "pb1":  # every H_j equals H̄ here, so the two first-order terms agree
                oh, _ = oracle.head_forward(q, k, v, block=block, topk=1, scale=0.7, variant="hyd", idx=idx)
                np.testing.assert_allclose(o, oh, atol=1e-13)
    for e1, e2 in ((2e-2, 1e-2), (1e-2, 5e-3)):
        r_h = errs[("hyd", e1)] / errs[("hyd", e2)]
        r_0 = errs[("0th", e1)] / errs[("0th", e2)]
        assert 3.5 < r_h < 4.5, r_h
        assert 1.8 < r_0 < 2.2, r_0


def test_taylor_orders_distinct_blocks():
    """The same ε-scaling with a different δ pattern (hence a different H_j) in
    every block: the global H̄ no longer matches any block, so the hybrid drops to
    first order, while the per-block first-order variant stays second order
    (gist, "Core Algorithm": the distinct per-block first-order terms that H̄
    replaces)."""
    D, block, n = 4, 8, 4
    L = block * n
    rng = np.random.default_rng(21)
    delta = rng.normal(size=(n, block, D))
    delta -= delta.mean(axis=1, keepdims=True)
    v = rng.normal(size=(L, D))
    c = rng.normal(size=(n, D))
    q = rng.normal(size=(L, D))
    idx = np.tile(np.array([0]), (n, 1))
    errs = {}
    for eps in (2e-2, 1e-2, 5e-3):
        k = np.repeat(c, block, axis=0) + eps * delta.reshape(L, D)
        dense = sdpa(q, k, v, 0.7)
        for var in ("hyd", "pb1"):
            o, _ = oracle.head_forward(q, k, v, block=block, topk=1, scale=0.7, variant=var, idx=idx)
            errs[(var, eps)] = np.abs(o - dense).max()
    for e1, e2 in ((2e-2, 1e-2), (1e-2, 5e-3)):
        r_h = errs[("hyd", e1)] / errs[("hyd", e2)]
        r_p = errs[("pb1", e1)] / errs[("pb1", e2)]
        assert 1.8 < r_h < 2.3, r_h
        assert 3.5 < r_p < 4.5, r_p


# --------------------------------------------------------------------------- P9
def test_global_mean_replacement_identity_and_bound():
    """N_hyd − N_pb1 = s q_t Σ_U α_tj (H̄ − H_j) where pb1 gives every unselected
    block its own first-order term; its size is bounded through M_j (the atlas
    summary's Limitations: the error theorem covers exactly this replacement)."""
    L, D, block = 160, 6, 32
    q, k, v = rand_head(L, D, 12)
    s = 0.45
    o, idx, st, _ = oracle.head_forward(q, k, v, block=block, topk=2, scale=s, want_stats=True)
    M = oracle.cov_norm(st["H"], st["Hbar"])
    n = st["kbar"].shape[0]
    for i in range(n):
        rows = slice(i * block, min(L, (i + 1) * block))
        Nh, Dh, m = oracle.pisa_rows(q, k, v, st, idx[i], i, block, s, True)
        Npb, Dpb, mpb = oracle.pisa_rows(q, k, v, st, idx[i], i, block, s, False, per_block=True)
        np.testing.assert_array_equal(m, mpb)
        np.testing.assert_allclose(Dpb, Dh, rtol=1e-15)
        uns = [j for j in range(n) if j not in set(idx[i])]
        diff = np.zeros_like(Npb)
        bound = np.zeros(Npb.shape[0])
        for j in uns:
            a = np.exp(s * q[rows] @ st["kbar"][j] - m)
            diff += a[:, None] * s * (q[rows] @ (st["Hbar"] - st["H"][j]))
            bound += a * s * np.linalg.norm(q[rows], axis=1) * M[j]
        np.testing.assert_allclose(Nh - Npb, diff, atol=1e-12)
        assert np.all(np.linalg.norm(Nh - Npb, axis=1) <= bound + 1e-12)


@pytest.mark.parametrize("L,block,topk", [(160, 32, 2), (150, 32, 1), (100, 16, 3)])
def test_per_block_first_order_from_the_keys(L, block, topk):
    """The per-block first-order term expanded over the block's own keys:
    α_tj s q_t H_j = Σ_n α_tj (ℓ_tn − c_tj) v_n with ℓ_tn = s q_t·k_n and
    c_tj = s q_t·k̄_j, so an unselected block contributes Σ_n α_tj (1 + ℓ_tn − c_tj) v_n
    to N_t (first-order Taylor expansion of e^{ℓ_tn} about c_tj, gist "Core
    Algorithm"). Computed here from q, k, v alone, without H_j; the ragged last
    block (L not a multiple of the block) uses its actual keys."""
    D = 6
    q, k, v = rand_head(L, D, L + topk)
    s = 0.55
    o, idx, st, _ = oracle.head_forward(q, k, v, block=block, topk=topk, scale=s, variant="pb1",
                                        want_stats=True)
    n = st["kbar"].shape[0]
    for i in range(n):
        rows = slice(i * block, min(L, (i + 1) * block))
        Qi = q[rows]
        m = oracle.pisa_rows(q, k, v, st, idx[i], i, block, s, False, per_block=True)[2]
        N = np.zeros((Qi.shape[0], D))
        Dn = np.zeros(Qi.shape[0])
        for j in range(n):
            Kj, Vj = k[j * block:min(L, (j + 1) * block)], v[j * block:min(L, (j + 1) * block)]
            ell = s * Qi @ Kj.T
            if j in set(idx[i]):
                w = np.exp(ell - m[:, None])
            else:
                c = s * Qi @ Kj.mean(axis=0)
                w = np.exp(c - m)[:, None] * (1.0 + ell - c[:, None])
            N += w @ Vj
            Dn += w.sum(axis=1)
        np.testing.assert_allclose(o[rows], N / Dn[:, None], atol=1e-12)


# --------------------------------------------------------------------------- P10-P12
def test_selection_brute_force():
    rng = np.random.default_rng(13)
    for trial in range(30):
        n = int(rng.integers(1, 12))
        S = np.round(rng.normal(size=(5, n)), 1)  # rounded: many exact ties
        for kk in range(1, n + 1):
            got = oracle.select_topk(S, kk)
            for r in range(5):
                ref = sorted(sorted(range(n), key=lambda j: (-S[r, j], j))[:kk])
                assert list(got[r]) == ref
            if kk < n:
                nxt = oracle.select_topk(S, kk + 1)
                for r in range(5):
                    assert set(got[r]) <= set(nxt[r])


@pytest.mark.parametrize("sink", [0, -1])
def test_sink_always_selected(sink):
    L, D, block = 300, 8, 32
    q, k, v = rand_head(L, D, 14)
    # make the sink block unattractive
    n = oracle.num_blocks(L, block)
    sb = 0 if sink == 0 else n - 1
    k[sb * block:(sb + 1) * block] -= 50 * q.mean(axis=0)
    _, idx = oracle.head_forward(q, k, v, block=block, topk=2, scale=0.3, sink_idx=sink)
    assert np.all((idx == sb).sum(axis=1) == 1)
    _, idx1 = oracle.head_forward(q, k, v, block=block, topk=1, scale=0.3, sink_idx=sink)
    assert np.all(idx1[:, 0] == sb)


def test_pooled_score_is_mean_logit():
    """s·q̄_i·k̄_j equals the mean of the logit block s·Q_i K_jᵀ (the skill page's
    relevance = mean of QKᵀ over a block)."""
    L, D, block = 150, 8, 32
    q, k, v = rand_head(L, D, 15)
    st = oracle.block_stats(q, k, v, block)
    S = oracle.pooled_scores(st["qbar"], st["kbar"], 0.3)
    tq, tk = torch.from_numpy(q), torch.from_numpy(k)
    n = st["kbar"].shape[0]
    for i in range(n):
        for j in range(n):
            blk = 0.3 * tq[i * block:(i + 1) * block] @ tk[j * block:(j + 1) * block].T
            assert abs(S[i, j] - blk.mean().item()) < 1e-13


def test_first_order_matrix_identities():
    """H_j = Σ k_nᵀv_n − k̄_jᵀΣV_j and H̄ = (KᵀV − Σ_j k̄_jᵀΣV_j)/n."""
    L, D, block = 170, 5, 32
    q, k, v = rand_head(L, D, 16)
    st = oracle.block_stats(q, k, v, block)
    n = st["kbar"].shape[0]
    G = torch.zeros(D, D, dtype=torch.float64)
    C = np.zeros((D, D))
    for j in range(n):
        lo, hi = j * block, min(L, (j + 1) * block)
        Gj = torch.from_numpy(k[lo:hi]).T @ torch.from_numpy(v[lo:hi])
        np.testing.assert_allclose(st["H"][j], Gj.numpy() - np.outer(st["kbar"][j], st["vsum"][j]), atol=1e-12)
        C += np.outer(st["kbar"][j], st["vsum"][j])
    KV = (torch.from_numpy(k).T @ torch.from_numpy(v)).numpy()
    np.testing.assert_allclose(st["Hbar"], (KV - C) / n, atol=1e-12)
    assert st["sizes"][-1] == L - (n - 1) * block


def test_cov_norm_hand_values():
    """n = 2: H_0 − H̄ = −(H_1 − H̄), so M_0 = M_1 = ‖H_0 − H_1‖_F / 2."""
    H = np.array([[[1.0, 2.0], [3.0, 4.0]], [[-1.0, 0.0], [1.0, 2.0]]])
    Hbar = H.mean(axis=0)
    M = oracle.cov_norm(H, Hbar)
    # H_0 − H_1 = [[2,2],[2,2]] → Frobenius 4 → M = 2
    np.testing.assert_allclose(M, [2.0, 2.0], atol=1e-15)


def test_cov_weight_routing_changes_selection():
    """With a large covariance weight, routing follows M_j (plus nothing else)."""
    L, D, block = 256, 8, 32
    q, k, v = rand_head(L, D, 17)
    v[3 * block:4 * block] *= 20  # block 3 has a large first-order matrix
    _, idx, st, S = oracle.head_forward(q, k, v, block=block, topk=1, scale=0.3, cov_weight=10.0,
                                        want_stats=True)
    assert np.all(idx[:, 0] == int(np.argmax(st["M"])))


def test_density_to_k_table():
    cases = {(0.25, 16): 4, (0.15, 72): 10, (0.125, 1182): 147, (0.10, 1861): 186,
             (0.05, 1182): 59, (0.25, 1182): 295, (0.5, 1182): 591, (1.0, 1182): 1182,
             (0.05, 591): 29, (0.125, 591): 73, (0.25, 591): 147, (0.5, 591): 295, (1.0, 591): 591,
             (0.0, 10): 1, (1e-9, 10): 1, (2.0, 10): 10}
    for (d, n), k in cases.items():
        assert oracle.topk_from_density(d, n) == k, (d, n)


def test_effective_flops_counts():
    L, D, block = 130, 4, 64  # blocks of 64, 64, 2
    idx = np.array([[0], [2], [1]])
    f = oracle.effective_flops(L, D, block, idx, True)
    # rows 64,64,2; exact keys 64,2,64; 2 unselected blocks each
    exp = 64 * (4 * D * 64 + 4 * D * 2) + 64 * (4 * D * 2 + 4 * D * 2) + 2 * (4 * D * 64 + 4 * D * 2)
    exp += 2 * D * D * (64 + 64 + 2)
    assert f == exp


# ------------------------------------------------- spectral covariance norm
def test_cov_norm_spectral_worked_example(golden):
    """The two-block example with the 2-norm the gist's "Covariance-Aware
    Routing" prints: H_0 − H̄ = [[5/4, −1/4], [3/4, 1/4]] and H_1 − H̄ its
    negative. For a 2 x 2 matrix A, σ_max² = (tr AᵀA + sqrt(tr² − 4 det(A)²)) / 2;
    here tr AᵀA = 9/4 and det A = 1/2, so M_0 = M_1 = sqrt((9 + √65) / 8)."""
    g = golden
    q, k, v = (np.array(g["inputs"][x], dtype=np.float64) for x in "qkv")
    st = oracle.block_stats(q, k, v, 2)
    M = oracle.cov_norm(st["H"], st["Hbar"], "spectral")
    want = math.sqrt((9.0 + math.sqrt(65.0)) / 8.0)
    np.testing.assert_allclose(M, [want, want], rtol=1e-15, atol=0)
    assert (M < oracle.cov_norm(st["H"], st["Hbar"], "fro")).all()  # rank 2: strictly below Frobenius


def test_cov_norm_spectral_closed_forms():
    """Diagonal: the largest |entry|. Rank one u vᵀ: ‖u‖·‖v‖ (and equal to the
    Frobenius norm). A block diagonal of rotations times scales: the largest
    scale. Hbar is zero in each case, so M_j is the norm of H_j itself."""
    D = 6
    rng = np.random.default_rng(5)
    u, w = rng.normal(size=D), rng.normal(size=D)
    c, s = math.cos(0.7), math.sin(0.7)
    rot = np.eye(D)
    rot[:2, :2] = [[3 * c, -3 * s], [3 * s, 3 * c]]  # scale 3 rotation in the first plane
    rot[2, 2], rot[3, 3], rot[4, 4], rot[5, 5] = 0.5, -1.5, 2.0, 0.0
    H = np.stack([np.diag([3.0, -4.0, 1.0, 0.0, 2.5, -0.5]), np.outer(u, w), rot])
    M = oracle.cov_norm(H, np.zeros((D, D)), "spectral")
    np.testing.assert_allclose(M, [4.0, np.linalg.norm(u) * np.linalg.norm(w), 3.0], rtol=1e-14)
    np.testing.assert_allclose(M[1], oracle.cov_norm(H, np.zeros((D, D)), "fro")[1], rtol=1e-14)


def test_cov_norm_spectral_power_iteration_and_bounds():
    """On random matrices: the power iteration on AᵀA (well separated top
    singular value by construction) reaches the same value, and
    ‖A‖_2 ≤ ‖A‖_F ≤ sqrt(rank)·‖A‖_2."""
    D, n = 16, 5
    rng = np.random.default_rng(9)
    H = rng.normal(size=(n, D, D))
    H[:, 0, :] *= 8.0  # one dominant row direction: a clear gap
    Hbar = H.mean(axis=0)
    M2 = oracle.cov_norm(H, Hbar, "spectral")
    MF = oracle.cov_norm(H, Hbar, "fro")
    for j in range(n):
        A = H[j] - Hbar
        x = np.ones(D)
        for _ in range(500):
            x = A.T @ (A @ x)
            x /= np.sqrt(x @ x)
        np.testing.assert_allclose(np.sqrt(x @ (A.T @ (A @ x))), M2[j], rtol=1e-12)
    assert (M2 <= MF * (1 + 1e-15)).all() and (MF <= math.sqrt(D) * M2 * (1 + 1e-15)).all()
    with pytest.raises(ValueError):
        oracle.cov_norm(H, Hbar, "nuclear")
