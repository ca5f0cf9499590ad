"""pisa_attn_fwd_noalloc, the entry point that allocates nothing: through the C
ABI, its output equals that of pisa_block_stats + pisa_attn_fwd (the entry
points it stands for) bit for bit, on two calls in a row whose second input is
smaller, so the second call runs on scratch the first one left behind; a shape
that needs more than the fixed scratch is refused before anything runs."""

import pytest
import torch

import block_sparse_attention_stats_amd as bsa
import synth
from parity import log

pytestmark = pytest.mark.gpu

W = synth.Workload

CALLS = [
    # first the larger call, then a smaller one with another head dim, dtype,
    # block size and variant, so the scratch holds the first call's data
    W("noalloc_flux_like", 1, 6, 4608, 128, 64, 0.15, "bf16", "hyd", 0, 0.0, seed=301),
    W("noalloc_small", 1, 2, 1000, 64, 128, 0.3, "f32", "0th", -1, 0.0, seed=302),
]


def _reference(w, qd, kd, vd, idx):
    st = bsa.block_stats(qd, kd, vd, w.block)
    return bsa.attn_fwd(qd, st, idx, w.scale, w.variant)


def test_noalloc_matches_workspace_entry_points():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    for w in CALLS:
        log(f"[{w.name}] B={w.B} H={w.H} L={w.L} D={w.D} blk={w.block} {w.dtype} {w.variant}")
        qd, kd, vd = (x.to(dev) for x in synth.make_qkv(w))
        n = w.n_blocks
        topk = bsa.topk_from_density(w.density, n)
        st = bsa.block_stats(qd, kd, vd, w.block)
        idx = bsa.select(st, topk, w.scale, 0.0, w.sink_idx)
        o_ref = _reference(w, qd, kd, vd, idx)
        o = bsa.attn_fwd_noalloc(qd, kd, vd, idx, w.scale, w.variant, block_size=w.block)
        torch.cuda.synchronize()
        diff = (o.float() - o_ref.float()).abs().max().item()
        log(f"    max-abs difference to block_stats + attn_fwd: {diff}")
        assert torch.equal(o, o_ref), f"{w.name}: differs by up to {diff}"


def test_noalloc_refuses_shapes_beyond_its_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    # K and V copies alone take 2 * 8 * 75600 * 128 * 2 bytes = 310 MB > 256 MiB
    B, H, L, D = 1, 8, 75600, 128
    q = torch.zeros(B, H, L, D, dtype=torch.bfloat16, device=dev)
    n = bsa.num_blocks(L, 64)
    idx = torch.arange(4, dtype=torch.int32, device=dev).expand(B, H, n, 4).contiguous()
    with pytest.raises(bsa.PisaError) as err:
        bsa.attn_fwd_noalloc(q, q, q, idx, 0.1)
    assert err.value.status == bsa.PISA_ETOOBIG
    torch.cuda.synchronize()
