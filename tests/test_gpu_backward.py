"""GPU parity of the backward pass of the zeroth-order variant (through the C
ABI) with the oracle's gradients, which are pinned to finite differences of
the oracle's forward and to torch autograd of dense attention."""

import numpy as np
import pytest
import torch

import block_sparse_attention_stats_amd as bsa
import oracle
import synth
from parity import check_backward, compare_grad, grad_floor, log

pytestmark = pytest.mark.gpu

W = synth.Workload

CASES = [
    # several tiles, ragged tails, both block sizes, both dtypes, head dims, sinks
    W("bwd_bf16_ragged", 1, 2, 1000, 128, 64, 0.25, "bf16", "0th", None, 0.0, seed=401),
    W("bwd_bf16_blk128_short_last", 1, 2, 1050, 128, 128, 0.3, "bf16", "0th", -1, 0.0, seed=402),
    W("bwd_bf16_d64_sink0", 2, 1, 900, 64, 64, 0.2, "bf16", "0th", 0, 0.0, seed=403),
    W("bwd_f32_d128_sink_last", 1, 2, 700, 128, 64, 0.3, "f32", "0th", -1, 0.0, seed=404),
    W("bwd_f32_blk128_d64", 1, 1, 800, 64, 128, 0.5, "f32", "0th", None, 0.0, seed=405),
    W("bwd_bf16_many_tiles", 1, 2, 9450, 128, 64, 0.125, "bf16", "0th", None, 0.0, seed=406),
    W("bwd_bf16_cov_routing", 1, 2, 1200, 128, 64, 0.15, "bf16", "0th", 0, 0.1, seed=407),
]

EDGES = [
    W("bwd_edge_single_block", 1, 2, 40, 128, 64, 0.5, "bf16", "0th", None, 0.0, seed=411),
    W("bwd_edge_one_token_f32", 1, 1, 1, 64, 64, 1.0, "f32", "0th", -1, 0.0, seed=412),
    W("bwd_edge_one_token_bf16_blk128", 1, 2, 1, 128, 128, 1.0, "bf16", "0th", 0, 0.0, seed=413),
    W("bwd_edge_last_block_one_token", 1, 2, 65, 128, 64, 0.5, "bf16", "0th", -1, 0.0, seed=414),
    W("bwd_edge_topk_one", 1, 2, 640, 128, 64, 0.01, "bf16", "0th", None, 0.0, seed=415),
    W("bwd_edge_density_one", 1, 2, 600, 128, 64, 1.0, "bf16", "0th", None, 0.0, seed=416),
    W("bwd_edge_topk_n_minus_1", 1, 2, 500, 64, 64, 0.99, "f32", "0th", 0, 0.0, seed=417),
    W("bwd_edge_blk128_last_block_one_token", 1, 1, 129, 64, 128, 0.5, "bf16", "0th", None, 0.0, seed=418),
]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_backward_parity(w):
    check_backward(w)


@pytest.mark.parametrize("w", EDGES, ids=lambda w: w.name)
def test_backward_edges(w):
    check_backward(w)


def test_backward_flux_config():
    """The FLUX configuration (24 heads, 4608 tokens, covariance routing, sink 0)
    with the zeroth-order variant, every head against the oracle."""
    check_backward(synth.FLUX.replace(name="flux_bf16_0th_bwd", variant="0th"))


def test_backward_deterministic_and_blhd():
    """Two calls give the same bits, and [B,L,H,D] tensors give the transposed
    bits of the [B,H,L,D] call."""
    w = W("bwd_layout", 1, 3, 1500, 128, 64, 0.2, "bf16", "0th", 0, 0.0, seed=421)
    res = check_backward(w, heads=[(0, 1)])
    qd, kd, vd, dod = res["inputs"]
    st, idx, o, lse = res["st"], res["idx"], res["o"], res["lse"]
    again = bsa.attn_bwd(qd, kd, vd, st, idx, w.scale, o, dod, lse=lse)
    tr = lambda x: x.transpose(1, 2).contiguous()
    st_t = bsa.block_stats(tr(qd), tr(kd), tr(vd), w.block, layout="BLHD")
    o_t, lse_t = bsa.attn_fwd(tr(qd), st_t, idx, w.scale, "0th", return_lse=True)
    g_t = bsa.attn_bwd(tr(qd), tr(kd), tr(vd), st_t, idx, w.scale, o_t, tr(dod), lse=lse_t)
    torch.cuda.synchronize()
    assert torch.equal(lse, lse_t)  # [B,H,L] in either layout
    for a, b, c in zip(res["grads"], again, g_t):
        assert torch.equal(a, b)
        assert torch.equal(tr(a), c)


def test_autograd_through_zeroth_order_variant():
    """piecewise_sparse_attention_0th on tensors that require gradients records
    pisa_attn_bwd as its backward, fed the forward's ln D_t: loss.backward()
    gives the gradients of the direct calls bit for bit, and they match the
    oracle's."""
    w = W("bwd_autograd", 1, 2, 1000, 128, 64, 0.2, "bf16", "0th", -1, 0.0, seed=431)
    q, k, v = synth.make_qkv(w)
    do = synth.grad_out(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev).requires_grad_(True) for x in (q, k, v))
    o, idx = bsa.piecewise_sparse_attention_0th(qd, kd, vd, density=w.density, sink_idx=w.sink_idx,
                                                return_idx=True)
    (o.float() * do.to(dev).float()).sum().backward()
    torch.cuda.synchronize()
    with torch.no_grad():
        st = bsa.block_stats(qd.detach(), kd.detach(), vd.detach(), w.block)
        _, lse = bsa.attn_fwd(qd.detach(), st, idx, w.scale, "0th", return_lse=True)
        direct = bsa.attn_bwd(qd.detach(), kd.detach(), vd.detach(), st, idx, w.scale, o.detach(),
                              do.to(dev), lse=lse)
    torch.cuda.synchronize()
    for x, g in zip((qd, kd, vd), direct):
        assert torch.equal(x.grad, g)
    gidx = idx.cpu().numpy()
    for h in range(w.H):
        qh, kh, vh, doh = (synth.as_f64(x[0, h]) for x in (q, k, v, do))
        ref = oracle.head_backward(qh, kh, vh, doh, block=w.block, idx=gidx[0, h], scale=w.scale)
        fl = grad_floor(qh, kh, vh, doh, w.scale, w.D)
        for name, x, r in zip(("dq", "dk", "dv"), (qd, kd, vd), ref):
            compare_grad(x.grad[0, h].float().cpu().numpy(), r, w.dtype, f"autograd head {h} {name}", fl)
