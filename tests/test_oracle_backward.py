"""Pins of the oracle's backward pass of the zeroth-order-only variant (README,
"Kernel variants": the ``_0th`` form supports training), each against
something other than the backward's own formulas: central finite differences of
the oracle's forward, torch autograd of dense attention, closed forms and exact
invariants of the forward. Also the log-denominators ln D_t that a forward
pass hands to the backward."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle


def rand_inputs(L, D, seed, spread=1.0):
    rng = np.random.default_rng(seed)
    return tuple(rng.normal(scale=spread, size=(L, D)) for _ in range(4))


def rand_idx(n, topk, seed):
    rng = np.random.default_rng(seed)
    return np.stack([np.sort(rng.choice(n, size=topk, replace=False)) for _ in range(n)])


def loss(q, k, v, do, block, idx, scale):
    o, _ = oracle.head_forward(q, k, v, block=block, topk=idx.shape[1], scale=scale, variant="0th", idx=idx)
    return float((o * do).sum())


@pytest.mark.parametrize("L,D,block,topk", [(10, 3, 4, 1), (10, 3, 4, 2), (13, 2, 4, 2), (9, 4, 3, 1)])
def test_backward_matches_central_differences(L, D, block, topk):
    """Every entry of dq, dk, dv equals the central difference of
    Σ o ∘ dO (the oracle's forward, selection fixed), step 1e-5: the
    difference is exact to O(h²) ≈ 1e-10."""
    q, k, v, do = rand_inputs(L, D, seed=L * 100 + topk)
    n = oracle.num_blocks(L, block)
    idx = rand_idx(n, topk, seed=L + D)
    scale = 0.7
    dq, dk, dv = oracle.head_backward(q, k, v, do, block=block, idx=idx, scale=scale)
    h = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.empty_like(x)
        for t in range(L):
            for d in range(D):
                x0 = x[t, d]
                x[t, d] = x0 + h
                lp = loss(q, k, v, do, block, idx, scale)
                x[t, d] = x0 - h
                lm = loss(q, k, v, do, block, idx, scale)
                x[t, d] = x0
                fd[t, d] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=0, atol=1e-8, err_msg=f"d{name}")


def dense_grads(q, k, v, do, scale):
    """torch autograd of softmax(s·QKᵀ)V in fp64 on the CPU."""
    t = [torch.from_numpy(np.ascontiguousarray(x)).requires_grad_(True) for x in (q, k, v)]
    o = torch.softmax(scale * (t[0] @ t[1].T), dim=-1) @ t[2]
    (o * torch.from_numpy(do)).sum().backward()
    return tuple(x.grad.numpy() for x in t)


def test_density_one_equals_dense_autograd():
    """With every block selected there is no tail: the gradients are those of
    dense attention."""
    L, D, block = 70, 8, 16
    q, k, v, do = rand_inputs(L, D, 3)
    n = oracle.num_blocks(L, block)
    idx = np.tile(np.arange(n), (n, 1))
    g = oracle.head_backward(q, k, v, do, block=block, idx=idx, scale=0.3)
    for a, b, name in zip(g, dense_grads(q, k, v, do, 0.3), "qkv"):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12, err_msg=f"d{name}")


def test_constant_key_blocks():
    """Every key block constant (k_t = c_j): the forward equals dense attention
    for any selection, so dq and dv equal the dense gradients. A key's
    gradient from the rows of query block i is its own dense gradient where i
    selects its block, and the block mean of the dense gradients where i
    leaves the block to its centroid k̄_j (whose gradient the block's tokens
    share equally)."""
    L, D, block = 45, 5, 8
    q, _, v, do = rand_inputs(L, D, 4)
    rng = np.random.default_rng(40)
    n = oracle.num_blocks(L, block)
    c = rng.normal(size=(n, D))
    k = np.repeat(c, block, axis=0)[:L]
    span = lambda j: slice(j * block, min(L, (j + 1) * block))
    gq, _, gv = dense_grads(q, k, v, do, 0.5)
    gk_rows = []  # dense dk from the rows of each query block alone
    for i in range(n):
        do_i = np.zeros_like(do)
        do_i[span(i)] = do[span(i)]
        gk_rows.append(dense_grads(q, k, v, do_i, 0.5)[1])
    for topk in (1, 3, n - 1):
        idx = rand_idx(n, topk, seed=topk)
        dq, dk, dv = oracle.head_backward(q, k, v, do, block=block, idx=idx, scale=0.5)
        np.testing.assert_allclose(dq, gq, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv, gv, rtol=0, atol=1e-12)
        want = np.zeros_like(dk)
        for i in range(n):
            for j in range(n):
                g = gk_rows[i][span(j)]
                want[span(j)] += g if j in idx[i] else g.mean(axis=0)
        np.testing.assert_allclose(dk, want, rtol=0, atol=1e-12)


def test_invariants_of_the_forward():
    """Shifting every key by w leaves o unchanged (each logit of a row moves by
    s·q_t·w, centroids included), so Σ_n dk_n = 0; shifting every value by c
    shifts o by c, so Σ_n dv_n = Σ_t dO_t; the gradients are linear in dO."""
    L, D, block = 100, 6, 16
    q, k, v, do = rand_inputs(L, D, 5)
    _, _, _, do2 = rand_inputs(L, D, 6)
    n = oracle.num_blocks(L, block)
    idx = rand_idx(n, 2, 7)
    dq, dk, dv = oracle.head_backward(q, k, v, do, block=block, idx=idx, scale=0.4)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)
    g2 = oracle.head_backward(q, k, v, do2, block=block, idx=idx, scale=0.4)
    g12 = oracle.head_backward(q, k, v, do + 2.0 * do2, block=block, idx=idx, scale=0.4)
    for a, b, c in zip((dq, dk, dv), g2, g12):
        np.testing.assert_allclose(c, a + 2.0 * b, rtol=0, atol=1e-12)


# ------------------------------------------------------------ ln D_t
def test_log_denominator_worked_example():
    """The two-block worked example (tests/golden, D_t written by hand term
    by term, unshifted): ln D_t = ln of the sum of its terms."""
    path = os.path.join(os.path.dirname(__file__), "golden", "worked_example_2block.json")
    g = json.load(open(path))
    q, k, v = (np.array(g["inputs"][x], dtype=np.float64) for x in "qkv")
    lse = oracle.head_log_denominator(q, k, v, block=2, idx=np.array(g["idx"]), scale=1.0)
    want = [math.log(sum(a / b * math.exp(c / d) for a, b, c, d in row["D"])) for row in g["rows"]]
    np.testing.assert_allclose(lse, want, rtol=0, atol=1e-14)


def test_log_denominator_dense_and_constant_keys():
    """Every block selected: ln D_t is the log-sum-exp of the row's logits
    (torch.logsumexp in fp64). Constant key blocks: the same for any
    selection, since n_j e^{s q·k̄_j} then equals the block's exact sum. One
    token: s q·k."""
    L, D, block = 70, 6, 16
    q, k, _, _ = rand_inputs(L, D, 21)
    v = np.zeros_like(q)
    n = oracle.num_blocks(L, block)
    dense = torch.logsumexp(0.6 * (torch.from_numpy(q) @ torch.from_numpy(k).T), dim=1).numpy()
    full = np.tile(np.arange(n), (n, 1))
    np.testing.assert_allclose(oracle.head_log_denominator(q, k, v, block=block, idx=full, scale=0.6), dense,
                               rtol=0, atol=1e-12)
    kc = np.repeat(np.random.default_rng(22).normal(size=(n, D)), block, axis=0)[:L]
    dense_c = torch.logsumexp(0.6 * (torch.from_numpy(q) @ torch.from_numpy(kc).T), dim=1).numpy()
    for topk in (1, 3):
        idx = rand_idx(n, topk, seed=topk + 30)
        np.testing.assert_allclose(oracle.head_log_denominator(q, kc, v, block=block, idx=idx, scale=0.6),
                                   dense_c, rtol=0, atol=1e-12)
    one = oracle.head_log_denominator(q[:1], k[:1], v[:1], block=64, idx=np.array([[0]]), scale=0.6)
    np.testing.assert_allclose(one, [0.6 * float(q[0] @ k[0])], rtol=0, atol=1e-14)
