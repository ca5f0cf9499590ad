"""The seeded generator is deterministic and has the workloads' shapes."""

import numpy as np
import torch

import synth


def test_deterministic_and_distinct_heads():
    a = synth.head_fp32(300, 16, 3, 0, 1)
    b = synth.head_fp32(300, 16, 3, 0, 1)
    c = synth.head_fp32(300, 16, 3, 0, 2)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    assert a[0].dtype == np.float32 and a[0].shape == (300, 16)


def test_clusters_share_means():
    q, k, v = synth.head_fp32(256, 64, 0, 0, 0)
    # within a 64-token cluster, q and k have the same mean (μ_c); across clusters not
    for c in range(4):
        sl = slice(64 * c, 64 * (c + 1))
        assert np.abs(q[sl].mean(0) - k[sl].mean(0)).mean() < 0.25
    assert abs(float(v.std()) - 1.0) < 0.05


def test_workload_shapes():
    assert synth.WAN.n_blocks == 1182 and synth.WAN.L - 1181 * 64 == 16
    assert synth.HUNYUAN.n_blocks == 1861 and synth.HUNYUAN.L - 1860 * 64 == 16
    assert synth.FLUX.n_blocks == 72 and synth.TINY.n_blocks == 16
    assert len(synth.sweep()) == 20
    q, k, v = synth.make_qkv(synth.TINY)
    assert q.shape == (1, 2, 1024, 64) and q.dtype == torch.float32
    w = synth.FLUX.replace(H=1, L=130)
    q, k, v = synth.make_qkv(w)
    assert q.dtype == torch.bfloat16 and q.shape == (1, 1, 130, 128)
