"""The Python binding rejects mismatched tensors before any pointer reaches the
library: shapes, dtypes and layouts of q, o, idx and the statistics are checked
against the shape the statistics were made for, then the device. CPU only; a
guard around the loaded library fails the test if any entry point other than
the workspace-size queries is called."""

import os

import pytest
import torch

import block_sparse_attention_stats_amd as bsa

pytestmark = pytest.mark.skipif(not os.path.exists(bsa.LIB_PATH), reason="libpisa.so not built")

HOST_ONLY = {"pisa_workspace_bytes", "dense_workspace_bytes", "pisa_bwd_workspace_bytes", "pisa_status_string"}


class _Guard:
    def __init__(self, lib):
        self._lib = lib

    def __getattr__(self, name):
        if name not in HOST_ONLY:
            raise AssertionError(f"{name} was called although the arguments are invalid")
        return getattr(self._lib, name)


@pytest.fixture(autouse=True)
def guard(monkeypatch):
    real = bsa.load_library()
    monkeypatch.setattr(bsa, "_lib_handle", _Guard(real))
    yield


B, H, L, D, BLK = 1, 2, 1000, 128, 64
N = bsa.num_blocks(L, BLK)


def cpu_stats(dtype=bsa.PISA_BF16, layout=0, L_=L, mnorm=True) -> bsa.Stats:
    shape = bsa.Shape(B, H, L_, D, BLK, dtype, layout)
    n = bsa.num_blocks(L_, BLK)
    f = dict(dtype=torch.float64)
    return bsa.Stats(shape, torch.zeros(B, H, n, D, **f), torch.zeros(B, H, n, D, **f),
                     torch.zeros(B, H, n, D, **f), torch.zeros(B, H, D, D, **f),
                     torch.zeros(B, H, n, **f) if mnorm else None,
                     torch.zeros(bsa.workspace_bytes(shape), dtype=torch.uint8))


def q_bf16(L_=L, layout=0):
    return torch.zeros((B, L_, H, D) if layout else (B, H, L_, D), dtype=torch.bfloat16)


def idx_ok(topk=4, n=N):
    return torch.zeros(B, H, n, topk, dtype=torch.int32)


def raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_attn_fwd_checks_every_argument():
    st = cpu_stats()
    raises("q has shape", bsa.attn_fwd, q_bf16(L_=999), st, idx_ok(), 0.1)
    raises("q has shape", bsa.attn_fwd, q_bf16(layout=1), st, idx_ok(), 0.1)  # BLHD q, BHLD stats
    raises("q has dtype", bsa.attn_fwd, torch.zeros(B, H, L, D), st, idx_ok(), 0.1)
    raises("contiguous", bsa.attn_fwd, torch.zeros(B, H, L, 2 * D, dtype=torch.bfloat16)[..., ::2], st,
           idx_ok(), 0.1)
    raises("idx has shape", bsa.attn_fwd, q_bf16(), st, idx_ok(n=N - 1), 0.1)
    raises("idx has dtype", bsa.attn_fwd, q_bf16(), st, idx_ok().long(), 0.1)
    raises("expected 1 to", bsa.attn_fwd, q_bf16(), st, idx_ok(topk=N + 1, n=N), 0.1)
    raises("idx must be", bsa.attn_fwd, q_bf16(), st, torch.zeros(N, 4, dtype=torch.int32), 0.1)
    raises("out has shape", bsa.attn_fwd, q_bf16(), st, idx_ok(), 0.1, out=q_bf16(L_=64))
    raises("out has dtype", bsa.attn_fwd, q_bf16(), st, idx_ok(), 0.1, out=torch.zeros(B, H, L, D))
    raises("unknown variant", bsa.attn_fwd, q_bf16(), st, idx_ok(), 0.1, first_order="pb2")
    # every size right: only the device is left, and it is checked last
    raises("on the GPU", bsa.attn_fwd, q_bf16(), st, idx_ok(), 0.1)
    # [B,L,H,D] statistics take [B,L,H,D] q
    raises("on the GPU", bsa.attn_fwd, q_bf16(layout=1), cpu_stats(layout=1), idx_ok(), 0.1)


def test_stats_buffers_checked():
    st = cpu_stats()
    st.qbar = torch.zeros(B, H, N + 1, D, dtype=torch.float64)
    raises("Stats.qbar", bsa.attn_fwd, q_bf16(), st, idx_ok(), 0.1)
    st = cpu_stats()
    st.hbar = torch.zeros(B, H, D, D, dtype=torch.float32)
    raises("Stats.hbar has dtype", bsa.select, st, 4, 0.1)
    st = cpu_stats()
    st.ws = st.ws[:-1]
    raises("Stats.ws holds", bsa.select, st, 4, 0.1)
    st = cpu_stats()
    st.mnorm = torch.zeros(B, H, N - 1, dtype=torch.float64)
    raises("Stats.mnorm", bsa.select, st, 4, 0.1)


def test_select_checks():
    st = cpu_stats(mnorm=False)
    raises("topk = 0", bsa.select, st, 0, 0.1)
    raises("topk = 17", bsa.select, st, N + 1, 0.1)
    raises("needs Stats.mnorm", bsa.select, st, 4, 0.1, cov_weight=0.1)
    raises("idx has shape", bsa.select, st, 4, 0.1, out=idx_ok(topk=5))
    raises("idx has dtype", bsa.select, st, 4, 0.1, out=idx_ok().long())
    raises("on the GPU", bsa.select, st, 4, 0.1, out=idx_ok())


def test_block_stats_out_checked():
    q = q_bf16()
    raises("were made for shape", bsa.block_stats, q, q, q, 64, out=cpu_stats(L_=1001))
    raises("were made for shape", bsa.block_stats, q, q, q, 128, out=cpu_stats())
    raises("needs Stats.mnorm", bsa.block_stats, q, q, q, 64, want_mnorm=True, out=cpu_stats(mnorm=False))
    raises("share shape", bsa.block_stats, q, q_bf16(L_=999), q)
    raises("on the GPU", bsa.block_stats, q, q, q, 64, out=cpu_stats())


def test_segmented_forward_checks():
    st = cpu_stats()
    q0, q1 = q_bf16(L_=600), q_bf16(L_=400)
    raises("q1 holds", bsa.attn_fwd_seg, q0, q_bf16(L_=1200), st, idx_ok(), 0.1)
    raises("q0 has shape", bsa.attn_fwd_seg, q_bf16(L_=601), q1, st, idx_ok(), 0.1)
    raises("out1 has shape", bsa.attn_fwd_seg, q0, q1, st, idx_ok(), 0.1, out1=q_bf16(L_=401))
    raises("on the GPU", bsa.attn_fwd_seg, q0, q1, st, idx_ok(), 0.1)


def test_dense_checks():
    q = q_bf16()
    raises("out has shape", bsa.dense, q, q, q, out=q_bf16(L_=10))
    raises("ws must be", bsa.dense, q, q, q, ws=torch.zeros(10, dtype=torch.int32))
    raises("on the GPU", bsa.dense, q, q, q)


def test_backward_checks():
    st = cpu_stats()
    q = q_bf16()
    lse_ok = torch.zeros(B, H, L, dtype=torch.float32)
    raises("o has shape", bsa.attn_bwd, q, q, q, st, idx_ok(), 0.1, q_bf16(L_=999), q)
    raises("dout has dtype", bsa.attn_bwd, q, q, q, st, idx_ok(), 0.1, q, torch.zeros(B, H, L, D))
    raises("idx has shape", bsa.attn_bwd, q, q, q, st, idx_ok(n=N + 1), 0.1, q, q)
    raises("lse has shape", bsa.attn_bwd, q, q, q, st, idx_ok(), 0.1, q, q, lse=torch.zeros(B, H, L + 1))
    raises("lse has dtype", bsa.attn_bwd, q, q, q, st, idx_ok(), 0.1, q, q,
           lse=torch.zeros(B, H, L, dtype=torch.float64))
    raises("on the GPU", bsa.attn_bwd, q, q, q, st, idx_ok(), 0.1, q, q, lse=lse_ok)
