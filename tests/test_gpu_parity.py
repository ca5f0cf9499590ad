"""GPU parity of the HIP path (through the C ABI) with the fp64 oracle.

Small shapes are compared in full (every head, every query block); the
full-size DiT-shaped workloads run on all heads in the same launch
configuration as the bench and are compared on sampled heads and query blocks
that the oracle evaluates one by one.
"""

import math
import os
import subprocess

import numpy as np
import pytest
import torch

import block_sparse_attention_stats_amd as bsa
import oracle
import synth
from parity import check_workload, compare_out, log, sample_qblocks

pytestmark = pytest.mark.gpu

W = synth.Workload

SMALL = [
    # tiles spanning several sub-tiles, ragged tails, both block sizes, both dtypes
    W("small_bf16_ragged", 1, 3, 1000, 128, 64, 0.25, "bf16", "hyd", None, 0.0, seed=11),
    W("small_bf16_0th", 2, 2, 777, 128, 64, 0.2, "bf16", "0th", None, 0.0, seed=12),
    W("small_bf16_blk128", 1, 2, 1100, 128, 128, 0.3, "bf16", "hyd", None, 0.0, seed=13),
    W("small_bf16_blk128_short_last", 1, 2, 1050, 128, 128, 0.3, "bf16", "0th", -1, 0.0, seed=14),
    W("small_bf16_d64", 1, 2, 900, 64, 64, 0.25, "bf16", "hyd", 0, 0.0, seed=15),
    W("small_f32_d128", 1, 2, 700, 128, 64, 0.3, "f32", "hyd", -1, 0.0, seed=16),
    W("small_f32_blk128", 1, 1, 800, 64, 128, 0.5, "f32", "hyd", None, 0.0, seed=17),
    W("small_bf16_cov", 1, 2, 1200, 128, 64, 0.15, "bf16", "hyd", 0, 0.1, seed=18),
    W("small_bf16_cov_balanced", 1, 2, 1200, 128, 64, 0.15, "bf16", "hyd", None, 1e-3, seed=19),
    W("small_f32_cov", 1, 2, 640, 64, 64, 0.2, "f32", "0th", None, 0.05, seed=20),
]

EDGES = [
    W("edge_single_block", 1, 2, 40, 128, 64, 0.5, "bf16", "hyd", None, 0.0, seed=21),
    W("edge_one_token", 1, 1, 1, 64, 64, 1.0, "f32", "hyd", -1, 0.0, seed=22),
    W("edge_last_block_one_token", 1, 2, 65, 128, 64, 0.5, "bf16", "hyd", -1, 0.0, seed=23),
    W("edge_topk_one", 1, 2, 640, 128, 64, 0.01, "bf16", "hyd", None, 0.0, seed=24),
    W("edge_topk_one_sink_last", 1, 2, 650, 128, 64, 0.01, "bf16", "hyd", -1, 0.0, seed=25),
    W("edge_density_one", 1, 2, 600, 128, 64, 1.0, "bf16", "hyd", None, 0.0, seed=26),
    W("edge_density_one_f32", 1, 2, 333, 64, 128, 1.0, "f32", "0th", None, 0.0, seed=27),
    W("edge_topk_n_minus_1", 1, 2, 500, 128, 64, 0.99, "bf16", "hyd", 0, 0.0, seed=28),
    # one token in bf16 (a single key: the output is v), and a one-token last
    # block left to the zeroth-order term (its weight is the block-size sum
    # corrected by n_last - blk)
    W("edge_one_token_bf16_blk128_0th_sink0", 2, 1, 1, 64, 128, 0.1, "bf16", "0th", 0, 0.0, seed=5571),
    W("edge_one_token_bf16_pb1_sink_last", 1, 1, 1, 128, 64, 0.3, "bf16", "pb1", -1, 0.0, seed=5608),
    W("edge_last_block_one_token_0th_sink0", 1, 3, 65, 128, 64, 0.9, "bf16", "0th", 0, 0.0, seed=5296),
]


# per-block first-order variant: ragged tails, both block sizes and dtypes,
# a sink, covariance routing, a single block and one unselected block
PB1 = [
    W("pb1_bf16_ragged", 1, 3, 1000, 128, 64, 0.25, "bf16", "pb1", None, 0.0, seed=51),
    W("pb1_bf16_blk128_short_last", 1, 2, 1050, 128, 128, 0.3, "bf16", "pb1", -1, 0.0, seed=52),
    W("pb1_bf16_d64_sink0", 1, 2, 900, 64, 64, 0.25, "bf16", "pb1", 0, 0.0, seed=53),
    W("pb1_f32_d128", 1, 2, 700, 128, 64, 0.3, "f32", "pb1", -1, 0.0, seed=54),
    W("pb1_f32_blk128_d64", 1, 1, 800, 64, 128, 0.5, "f32", "pb1", None, 0.0, seed=55),
    W("pb1_bf16_cov", 1, 2, 1200, 128, 64, 0.15, "bf16", "pb1", 0, 0.1, seed=56),
    W("pb1_bf16_many_tiles", 1, 2, 9450, 128, 64, 0.125, "bf16", "pb1", None, 0.0, seed=57),
    W("pb1_edge_single_block", 1, 2, 40, 128, 64, 0.5, "bf16", "pb1", None, 0.0, seed=58),
    W("pb1_edge_last_block_one_token", 1, 2, 65, 128, 64, 0.5, "bf16", "pb1", -1, 0.0, seed=59),
    W("pb1_edge_topk_n_minus_1", 1, 2, 500, 128, 64, 0.99, "bf16", "pb1", 0, 0.0, seed=60),
    W("pb1_edge_density_one", 1, 2, 600, 128, 64, 1.0, "bf16", "pb1", None, 0.0, seed=61),
]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_full_parity(w):
    check_workload(w)


@pytest.mark.parametrize("w", EDGES, ids=lambda w: w.name)
def test_edge_cases(w):
    check_workload(w)


@pytest.mark.parametrize("w", PB1, ids=lambda w: w.name)
def test_per_block_first_order_parity(w):
    check_workload(w)


def test_per_block_first_order_wan_sampled():
    """The per-block first-order variant at the full Wan shape (all heads on the
    GPU), compared on sampled query blocks of two heads."""
    w = synth.WAN.replace(variant="pb1", name="wan_bf16_pb1")
    check_workload(w, heads=[(0, 3), (0, 38)], qblock_sample=6)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_per_block_first_order_careful_kernel(dtype):
    """The loose-bound input of the hybrid's careful-kernel test, per-block
    first-order variant: every query tile goes to its careful kernel, which
    shifts by the largest exponent the tile uses."""
    w = W(f"pb1_loose_bound_{dtype}", 1, 2, 700, 128, 64, 0.25, dtype, "pb1", None, 0.0, seed=42)
    q, k, v = synth.make_qkv(w)
    q[..., 0] = 0
    k[:, :, 130, :] = 0
    k[:, :, 130, 0] = 3.0e4
    res = check_workload(w, qkv=(q, k, v))
    assert redo_count(res["stats"], w) == w.B * w.H * w.n_blocks


LAYOUT_CASES = [SMALL[0], SMALL[3], SMALL[4], SMALL[5], SMALL[7], PB1[0], PB1[1],
                W("layout_spectral", 1, 2, 1100, 64, 128, 0.2, "bf16", "0th", 0, 0.05, seed=77,
                  cov_norm="spectral")]


@pytest.mark.parametrize("w", LAYOUT_CASES, ids=lambda w: w.name)
def test_blhd_layout_matches_bhld(w):
    """q, k, v given as [B,L,H,D] (layout "BLHD") and read in place: the same
    statistics, selection and output bits as the [B,H,L,D] call, whose parity
    with the oracle the other tests check; the dense baseline likewise. The
    first case is also compared with the oracle directly."""
    q, k, v = synth.make_qkv(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    qt, kt, vt = (x.transpose(1, 2).contiguous() for x in (qd, kd, vd))
    n = w.n_blocks
    topk = bsa.topk_from_density(w.density, n)
    runs = []
    for (a, b, c, lay) in ((qd, kd, vd, "BHLD"), (qt, kt, vt, "BLHD")):
        st = bsa.block_stats(a, b, c, w.block, want_mnorm=w.cov_weight > 0, layout=lay, cov_norm=w.cov_norm)
        idx = bsa.select(st, topk, w.scale, w.cov_weight, w.sink_idx)
        o = bsa.attn_fwd(a, st, idx, w.scale, w.variant)
        od = bsa.dense(a, b, c, w.scale, layout=lay)
        runs.append((st, idx, o, od))
    torch.cuda.synchronize()
    (s1, i1, o1, d1), (s2, i2, o2, d2) = runs
    for name in ("qbar", "kbar", "vsum", "hbar") + (("mnorm",) if w.cov_weight > 0 else ()):
        assert torch.equal(getattr(s1, name), getattr(s2, name)), name
    assert torch.equal(i1, i2)
    assert o2.shape == (w.B, w.L, w.H, w.D)
    assert torch.equal(o2.transpose(1, 2), o1)
    assert torch.equal(d2.transpose(1, 2), d1)
    if w is LAYOUT_CASES[0]:
        for h in range(w.H):
            qh, kh, vh = (synth.as_f64(x[0, h]) for x in (q, k, v))
            o_ref, idx_ref = oracle.head_forward(qh, kh, vh, block=w.block, topk=topk, scale=w.scale,
                                                 variant=w.variant, sink_idx=w.sink_idx,
                                                 idx=i2[0, h].cpu().numpy())
            compare_out(o2[0, :, h].float().cpu().numpy(), o_ref, w.dtype, f"BLHD head {h}")


def random_cases(count: int, seed: int, lengths=(1, 63, 64, 65, 127, 129, 500, 1000, 1777, 2600),
                 prefix: str = "rand"):
    """Seeded random small workloads over every option: length (ragged tails of
    any size, a single token), head dim, block size, density (topk 1 to n),
    variant, I/O dtype, sink and covariance weight."""
    rng = np.random.default_rng(seed)
    out = []
    for c in range(count):
        blk = int(rng.choice([64, 128]))
        L = int(rng.choice(lengths))
        out.append(W(f"{prefix}{c}", int(rng.integers(1, 3)), int(rng.integers(1, 4)), L,
                     int(rng.choice([64, 128])), blk, float(rng.choice([0.02, 0.1, 0.3, 0.6, 1.0])),
                     str(rng.choice(["bf16", "f32"])), str(rng.choice(["hyd", "0th", "pb1"])),
                     [None, 0, -1][int(rng.integers(0, 3))], float(rng.choice([0.0, 0.0, 1e-3, 0.1])),
                     seed=100 + c))
    return out


@pytest.mark.parametrize("w", random_cases(24, 2026), ids=lambda w: w.name)
def test_random_small_shapes(w):
    check_workload(w)


# longer sequences too (up to 15000 tokens, several hundred blocks)
@pytest.mark.parametrize("w", random_cases(40, 4243, lengths=(1, 17, 64, 65, 200, 777, 1500, 3000, 4100,
                                                              6000, 9001, 15000), prefix="wide"),
                         ids=lambda w: w.name)
def test_random_wider_shapes(w):
    check_workload(w)


# row lengths (blocks) for routing: the on-chip score-and-select kernel from
# one to twenty register slots per lane (full and one past full) up to its
# longest row (1280); past it the score kernel with the wavefront top-k (24, 28
# and 32 register slots, up to 2048 blocks), the workgroup top-k beyond, and
# the longest row the library takes
ROUTE_N = [1, 2, 63, 64, 256, 257, 700, 1182, 1280, 1281, 1600, 1861, 2048, 2049, 8192]


@pytest.mark.parametrize("n", ROUTE_N)
def test_routing_exact_scores_and_ties(n):
    """Selection over rows of n blocks matches the oracle's exactly: the inputs
    are small integers, so every routing score is exact in fp64 on both sides
    and neither summation order nor rounding can move a block across the k-th
    place. First every key block distinct (ties only by chance), then key
    blocks repeating with period 7, where each row holds 7 distinct scores and
    the k-th place always falls inside a run of equal scores that must go to
    the lowest indices. Several k per n, with and without a sink."""
    H = 2 if n <= 2048 else 1
    L = n * 64
    dev = torch.device("cuda:0")
    rows = np.arange(n) if n <= 2048 else np.array(sample_qblocks(n, 96, seed=n))
    ks = sorted({bsa.topk_from_density(d, n) for d in (0.01, 0.125, 0.5)} | {max(1, n - 1)})
    for period in (None, 7):
        q, k, v = synth.integer_qkv(1, H, L, 64, seed=900 + n, key_period=period)
        st = bsa.block_stats(q.to(dev), k.to(dev), v.to(dev), 64)
        ora = [oracle.block_stats(*(synth.as_f64(x[0, h]) for x in (q, k, v)), 64) for h in range(H)]
        for topk in ks:
            for sink in (None, -1):
                idx = bsa.select(st, topk, 0.125, 0.0, sink).cpu().numpy()
                for h in range(H):
                    S = oracle.pooled_scores(ora[h]["qbar"][rows], ora[h]["kbar"], 0.125, sink_idx=sink)
                    ref = oracle.select_topk(S, topk)
                    bad = np.nonzero((idx[0, h][rows] != ref).any(axis=1))[0]
                    assert bad.size == 0, (f"n={n} period={period} topk={topk} sink={sink} head {h}: "
                                           f"{bad.size} rows differ, first query block {rows[bad[0]]}")
    log(f"routing n={n}: exact over {len(rows)} query blocks x {H} heads, k in {ks}")


@pytest.mark.parametrize("n", [64, 300, 1182, 1280, 1500])
def test_routing_ties_in_the_upper_key_bits(n):
    """Scores that agree in the upper 32 bits of their order keys and differ
    only below, or not at all, right at the k-th place. q̄_i is the unit vector
    e_(i mod D) and the scale 1/8, so S_ij = k̄_j[i mod D] / 8 exactly in fp64
    on both sides. Each coordinate of k̄ holds a band of scores well above the
    cut, a cluster 1 + m·2^-52 (m < 2^31: one exponent and the same upper 20
    mantissa bits) with some values repeated, and the rest well below; k cuts
    the cluster, so the selection rests on the lower key bits and, for the
    repeated values, on the lower index. Stats are filled directly and the
    selection is compared with the oracle's exactly."""
    dev = torch.device("cuda:0")
    D, H = 64, 2
    rng = np.random.default_rng(4000 + n)
    shape = bsa.make_shape(torch.empty((1, H, n * 64, D), dtype=torch.bfloat16, device=dev), 64)
    st = bsa.alloc_stats(shape, dev, want_mnorm=False)
    qbar = np.zeros((1, H, n, D))
    for i in range(n):
        qbar[0, :, i, i % D] = 1.0
    n_above, n_cluster = n // 8, max(8, n // 4)
    kbar = np.empty((1, H, n, D))
    for h in range(H):
        for d in range(D):
            m = rng.integers(0, 1 << 31, size=n_cluster)
            m[: n_cluster // 4] = m[n_cluster // 4: 2 * (n_cluster // 4)]  # exact repeats
            col = np.concatenate([2.0 + rng.random(n_above), 1.0 + m * 2.0 ** -52,
                                  0.5 * rng.random(n - n_above - n_cluster)])
            kbar[0, h, :, d] = col[rng.permutation(n)]
    st.qbar.copy_(torch.from_numpy(qbar))
    st.kbar.copy_(torch.from_numpy(kbar))
    scale = 0.125
    for topk in (n_above + n_cluster // 2, n_above + n_cluster // 2 + 1):
        idx = bsa.select(st, topk, scale).cpu().numpy()
        for h in range(H):
            ref = oracle.select_topk(oracle.pooled_scores(qbar[0, h], kbar[0, h], scale), topk)
            bad = np.nonzero((idx[0, h] != ref).any(axis=1))[0]
            assert bad.size == 0, f"n={n} topk={topk} head {h}: {bad.size} rows differ, first {bad[0]}"
    log(f"routing n={n}: ties in the upper key bits resolved exactly, {H} heads x {n} rows")


JOINT_CASES = [
    # (workload, first-part length L0, layout): text first on a block boundary
    # (FLUX's 512 text tokens), image first with the boundary inside a block
    # (text last, Hunyuan-style), a 128-token block cut at 130, fp32, pb1
    (W("joint_flux_like", 1, 2, 4608, 128, 64, 0.15, "bf16", "hyd", 0, 0.1, seed=71), 512, "BHLD"),
    (W("joint_text_last", 1, 2, 1256, 128, 64, 0.2, "bf16", "pb1", -1, 0.0, seed=72), 1000, "BLHD"),
    (W("joint_blk128_f32", 2, 1, 700, 64, 128, 0.3, "f32", "0th", None, 0.0, seed=73), 130, "BHLD"),
    (W("joint_one_token_first", 1, 2, 900, 128, 64, 0.25, "bf16", "hyd", 0, 0.0, seed=74), 1, "BLHD"),
    (W("joint_spectral_text_last", 1, 2, 1256, 128, 64, 0.2, "bf16", "hyd", -1, 0.1, seed=76,
       cov_norm="spectral"), 1000, "BLHD"),
]


@pytest.mark.parametrize("case", JOINT_CASES, ids=lambda c: c[0].name)
def test_joint_sequence_matches_single_tensor(case):
    """A sequence passed in two tensors (tokens [0, L0) and [L0, L)) gives the
    same statistics, selection and output bits as the same sequence in one
    tensor, whose parity with the oracle the other tests check; the dense
    baseline likewise."""
    w, L0, layout = case
    q, k, v = synth.make_qkv(w)
    dev = torch.device("cuda:0")
    ax = 2 if layout == "BHLD" else 1
    full = [x.to(dev) if layout == "BHLD" else x.transpose(1, 2).contiguous().to(dev) for x in (q, k, v)]
    parts = [(x.narrow(ax, 0, L0).contiguous(), x.narrow(ax, L0, w.L - L0).contiguous()) for x in full]
    (q0, q1), (k0, k1), (v0, v1) = parts
    n = w.n_blocks
    topk = bsa.topk_from_density(w.density, n)
    st = bsa.block_stats(*full, w.block, want_mnorm=w.cov_weight > 0, layout=layout, cov_norm=w.cov_norm)
    idx = bsa.select(st, topk, w.scale, w.cov_weight, w.sink_idx)
    o = bsa.attn_fwd(full[0], st, idx, w.scale, w.variant)
    od = bsa.dense(*full, w.scale, layout=layout)
    st2 = bsa.block_stats_seg(q0, k0, v0, q1, k1, v1, w.block, want_mnorm=w.cov_weight > 0, layout=layout,
                              cov_norm=w.cov_norm)
    idx2 = bsa.select(st2, topk, w.scale, w.cov_weight, w.sink_idx)
    o0, o1 = bsa.attn_fwd_seg(q0, q1, st2, idx2, w.scale, w.variant)
    d0, d1 = bsa.dense_seg(q0, k0, v0, q1, k1, v1, w.scale, layout=layout)
    torch.cuda.synchronize()
    for name in ("qbar", "kbar", "vsum", "hbar") + (("mnorm",) if w.cov_weight > 0 else ()):
        assert torch.equal(getattr(st, name), getattr(st2, name)), name
    assert torch.equal(idx, idx2)
    assert torch.equal(torch.cat([o0, o1], ax), o)
    assert torch.equal(torch.cat([d0, d1], ax), od)


def test_mmdit_joint_attention_text_sink():
    """The adapter puts the text block in every selection (block 0 with the
    text first, block n-1 with it last) and returns the text and image outputs
    of the joint sequence, compared here with the oracle on the concatenated
    sequence."""
    H, D, Lt, Li = 2, 128, 256, 1000
    w = W("mmdit_adapter", 1, H, Lt + Li, D, 64, 0.1, "bf16", "hyd", None, 0.0, seed=75)
    q, k, v = synth.make_qkv(w)
    n = w.n_blocks
    topk = bsa.topk_from_density(w.density, n)
    dev = torch.device("cuda:0")
    for text_first in (True, False):
        if text_first:
            txt = [x[:, :, :Lt].contiguous().to(dev) for x in (q, k, v)]
            img = [x[:, :, Lt:].contiguous().to(dev) for x in (q, k, v)]
        else:
            img = [x[:, :, :Li].contiguous().to(dev) for x in (q, k, v)]
            txt = [x[:, :, Li:].contiguous().to(dev) for x in (q, k, v)]
        o_txt, o_img, idx = bsa.mmdit_joint_attention(*txt, *img, density=w.density, text_first=text_first,
                                                      return_idx=True)
        torch.cuda.synchronize()
        sink = 0 if text_first else n - 1
        assert bool((idx == sink).any(dim=-1).all())
        o = torch.cat([o_txt, o_img] if text_first else [o_img, o_txt], 2).float().cpu().numpy()
        gidx = idx.cpu().numpy()
        for h in range(H):
            qh, kh, vh = (synth.as_f64(x[0, h]) for x in (q, k, v))
            ref, ridx = oracle.head_forward(qh, kh, vh, block=64, topk=topk, scale=w.scale,
                                            sink_idx=0 if text_first else -1, idx=gidx[0, h])
            compare_out(o[0, h], ref, "bf16", f"mmdit text_first={text_first} head {h}")


C_CALLER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "pisa_c_caller")


@pytest.mark.parametrize("w", [SMALL[0], SMALL[5], PB1[1]], ids=lambda w: w.name)
def test_plain_c_caller_matches_binding(w, tmp_path):
    """tests/c_abi/pisa_c_caller.c drives the three steps through include/pisa.h
    alone (hipMalloc'd buffers, default stream, no Python or torch in that
    process): its selection and output are bit-identical to the binding's on
    the same inputs."""
    if not os.path.exists(C_CALLER):
        pytest.skip("tests/c_abi/pisa_c_caller is not built (build() compiles it with gcc)")
    q, k, v = synth.make_qkv(w)
    raw = (lambda x: x.view(torch.int16)) if w.dtype == "bf16" else (lambda x: x)
    for name, x in (("q", q), ("k", k), ("v", v)):
        raw(x).contiguous().numpy().tofile(str(tmp_path / f"{name}.bin"))
    n = w.n_blocks
    topk = bsa.topk_from_density(w.density, n)
    sink = "none" if w.sink_idx is None else str(w.sink_idx)
    dtype = bsa.PISA_BF16 if w.dtype == "bf16" else bsa.PISA_F32
    (tmp_path / "shape.txt").write_text(
        f"{w.B} {w.H} {w.L} {w.D} {w.block} {dtype} {topk} {sink} {bsa.VARIANTS[w.variant]} {w.scale!r}\n")
    log(f"[{w.name}] running the C caller")
    r = subprocess.run([C_CALLER, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    st = bsa.block_stats(qd, kd, vd, w.block)
    idx = bsa.select(st, topk, w.scale, 0.0, w.sink_idx)
    o = bsa.attn_fwd(qd, st, idx, w.scale, w.variant)
    torch.cuda.synchronize()
    c_idx = np.fromfile(str(tmp_path / "idx.bin"), dtype=np.int32).reshape(idx.shape)
    np.testing.assert_array_equal(c_idx, idx.cpu().numpy())
    c_o = np.fromfile(str(tmp_path / "o.bin"), dtype=np.int16 if w.dtype == "bf16" else np.float32)
    np.testing.assert_array_equal(c_o.reshape(o.shape), raw(o.cpu()).numpy())


# covariance routing with the spectral norm of H_j − H̄ (the gist's 2-norm)
SPECTRAL = [
    W("spec_bf16_cov", 1, 2, 1200, 128, 64, 0.15, "bf16", "hyd", 0, 0.1, seed=201, cov_norm="spectral"),
    W("spec_bf16_balanced", 1, 2, 1200, 128, 64, 0.15, "bf16", "hyd", None, 1e-3, seed=202,
      cov_norm="spectral"),
    W("spec_f32_d64_blk128_ragged", 1, 2, 1000, 64, 128, 0.2, "f32", "0th", -1, 0.05, seed=203,
      cov_norm="spectral"),
    W("spec_bf16_d64_blk64", 2, 1, 777, 64, 64, 0.3, "bf16", "pb1", None, 0.02, seed=204, cov_norm="spectral"),
    W("spec_edge_single_block", 1, 2, 40, 128, 64, 0.5, "bf16", "hyd", None, 0.1, seed=205,
      cov_norm="spectral"),
    W("spec_edge_last_block_one_token", 1, 2, 65, 128, 64, 0.5, "bf16", "hyd", -1, 0.1, seed=206,
      cov_norm="spectral"),
]


@pytest.mark.parametrize("w", SPECTRAL, ids=lambda w: w.name)
def test_spectral_covariance_routing(w):
    check_workload(w)


def test_flux_config_spectral_norm():
    """The FLUX configuration (covariance routing at weight 0.1, sink 0) with
    the spectral norm: statistics, every selection row (tie rule) and every
    output against the oracle."""
    check_workload(synth.FLUX.replace(name="flux_bf16_spectral", cov_norm="spectral"))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("rel_gap", [0.0, 2.0 ** -7])
def test_spectral_norm_repeated_top_singular_value(D, rel_gap):
    """Two blocks built so that H_0 − H̄ = 16 (e_0 u_0ᵀ + e_1 u_1ᵀ) with
    u_0 = 2 e_2 and u_1 = 2 (1 + gap) e_3, and H_1 − H̄ its negative: the two
    largest singular values are 32 and 32 (1 + gap), equal or 2^-7 apart, where
    a power iteration would stall. Every input is a small integer or a
    power-of-two fraction, exact in bf16, so the spectral norm must come out as
    32 (1 + gap) to fp64 accuracy."""
    L = 128
    k = torch.zeros(1, 1, L, D)
    v = torch.zeros(1, 1, L, D)
    for t in range(64):  # block 0: k_t = ±e_{t%2}, v_t = ±u_{t%2}, signs alternating in pairs
        s = 1.0 if (t // 2) % 2 == 0 else -1.0
        k[0, 0, t, t % 2] = s
        v[0, 0, t, 2 + t % 2] = s * 2.0 * (1.0 + (rel_gap if t % 2 else 0.0))
    k[0, 0, 64:, 5] = 3.0  # block 1: constant keys, so H_1 = 0
    v[0, 0, 64:, 7] = torch.arange(64, dtype=torch.float32) - 20.0
    q = torch.ones(1, 1, L, D)
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(torch.bfloat16).to(dev) for x in (q, k, v))
    st = bsa.block_stats(qd, kd, vd, 64, want_mnorm=True, cov_norm="spectral")
    st_f = bsa.block_stats(qd, kd, vd, 64, want_mnorm=True, cov_norm="fro")
    torch.cuda.synchronize()
    want = 32.0 * (1.0 + rel_gap)
    got = st.mnorm.cpu().numpy()[0, 0]
    np.testing.assert_allclose(got, [want, want], rtol=1e-13, atol=0)
    fro = math.sqrt(32.0 ** 2 + want ** 2)
    np.testing.assert_allclose(st_f.mnorm.cpu().numpy()[0, 0], [fro, fro], rtol=1e-6)


def test_tiny_config_full():
    check_workload(synth.TINY)


def test_flux_config_full():
    check_workload(synth.FLUX)


@pytest.mark.parametrize("variant", ["hyd", "0th", "pb1"])
def test_single_token_returns_v_exactly(variant):
    """A one-token sequence has a single key, whose softmax weight is 1, so
    o = v. In bf16 the kernels return v bit for bit: the numerator and the
    denominator take the same rounded weight, and the quotient is within an
    fp32 rounding of v, which rounds back to v."""
    dev = torch.device("cuda:0")
    for seed, (D, blk) in enumerate([(64, 64), (128, 64), (64, 128), (128, 128)] * 2):
        w = W(f"one_token_{variant}_{seed}", 2, 3, 1, D, blk, 1.0, "bf16", variant, [None, 0, -1][seed % 3],
              0.0, seed=700 + seed)
        q, k, v = (x.to(dev) for x in synth.make_qkv(w))
        st = bsa.block_stats(q, k, v, blk)
        idx = bsa.select(st, 1, w.scale, 0.0, w.sink_idx)
        o = bsa.attn_fwd(q, st, idx, w.scale, variant)
        torch.cuda.synchronize()
        assert torch.equal(o, v), f"{w.name}: max diff {(o.float() - v.float()).abs().max().item()}"


# the longest sequences the library takes: 8192 key blocks (the per-tile
# selection mask's size), with a ragged last block, both block sizes, all
# three variants
MAX_BLOCKS = [
    W("max_blocks_blk64_hyd_sink_last", 1, 1, 8192 * 64 - 13, 64, 64, 0.01, "bf16", "hyd", -1, 0.0,
      seed=81),
    W("max_blocks_blk128_0th", 1, 1, 8192 * 128 - 100, 64, 128, 0.02, "bf16", "0th", None, 0.0,
      seed=82),
    W("max_blocks_blk64_pb1_sink0", 1, 1, 8192 * 64 - 40, 64, 64, 0.01, "bf16", "pb1", 0, 0.0, seed=83),
]


@pytest.mark.parametrize("w", MAX_BLOCKS, ids=lambda w: w.name)
def test_longest_sequences_sampled(w):
    """Statistics and selection of every query block, and the output of 24
    sampled query blocks (the first and last among them), at the block count
    limit; selection rows are checked with the tie rule, outputs against the
    oracle as everywhere else."""
    assert w.n_blocks == 8192
    check_workload(w, qblock_sample=24)


def test_wan_config_sampled():
    w = synth.WAN
    check_workload(w, heads=[(0, 0), (0, 17), (0, 39)], qblock_sample=10)


def test_hunyuan_config_sampled():
    w = synth.HUNYUAN
    check_workload(w, heads=[(0, 0), (0, 23)], qblock_sample=10)


@pytest.mark.parametrize("w", synth.sweep(), ids=lambda w: w.name)
def test_sweep_points_reduced_length(w):
    """Every block x density x variant point of the sweep at L = 9450 (an
    eighth of the Wan length, same ragged tail structure), both batch rows."""
    check_workload(w.replace(L=9450, H=2), qblock_sample=None)


@pytest.fixture(scope="module")
def sweep_inputs():
    """The Wan-shape sweep's inputs (B=2, H=40, L=75600, bf16), generated once
    for all 20 full-size points."""
    t0 = __import__("time").time()
    qkv = synth.make_qkv(synth.SWEEP_BASE)
    log(f"sweep inputs generated in {__import__('time').time() - t0:.1f}s")
    return qkv


@pytest.mark.parametrize("w", synth.sweep(), ids=lambda w: w.name)
def test_sweep_full_size_sampled(w, sweep_inputs):
    """Every block x density x variant point of the sweep at its full size
    (B=2, H=40, L=75600), in the launch configuration the bench times: all 80
    heads on the GPU; for head (1, 5) every selection row against the oracle
    (tie rule) and the outputs of 6 query blocks, the first and the ragged
    last among them, against the oracle with its own selection."""
    check_workload(w, heads=[(1, 5)], qblock_sample=6, qkv=sweep_inputs)


def banded_idx(B: int, H: int, n: int, topk: int) -> np.ndarray:
    """A local selection: query block i takes the topk blocks nearest to it
    (a window of consecutive blocks, clipped at the ends), ascending."""
    start = np.clip(np.arange(n) - topk // 2, 0, n - topk)
    rows = start[:, None] + np.arange(topk)[None, :]
    return np.broadcast_to(rows, (B, H, n, topk)).astype(np.int32).copy()


@pytest.mark.parametrize("w", [
    W("banded_bf16_hyd", 1, 2, 5000, 128, 64, 0.15, "bf16", "hyd", None, 0.0, seed=91),
    W("banded_bf16_blk128_0th_ragged", 1, 2, 5050, 128, 128, 0.2, "bf16", "0th", None, 0.0, seed=92),
    W("banded_f32_d64", 1, 1, 3000, 64, 64, 0.1, "f32", "hyd", None, 0.0, seed=93),
])
def test_banded_selection_through_idx(w):
    """A local (banded) selection fed through idx, the shape real DiT
    selections take, compared in full with the oracle run on the same idx."""
    q, k, v = synth.make_qkv(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    n = w.n_blocks
    topk = bsa.topk_from_density(w.density, n)
    idx = banded_idx(w.B, w.H, n, topk)
    st = bsa.block_stats(qd, kd, vd, w.block)
    o = bsa.attn_fwd(qd, st, torch.from_numpy(idx).to(dev), w.scale, w.variant)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    for h in range(w.H):
        qh, kh, vh = (synth.as_f64(x[0, h]) for x in (q, k, v))
        ref, _ = oracle.head_forward(qh, kh, vh, block=w.block, topk=topk, scale=w.scale,
                                     variant=w.variant, idx=idx[0, h])
        compare_out(o[0, h], ref, w.dtype, f"{w.name} head {h} banded")


def redo_count(st, w) -> int:
    """Query tiles the fast kernel left to the careful (running-max) kernel in
    the last pisa_attn_fwd call: an int32 counter in the workspace, right after
    the K/V copies and the per-run key-norm maxima."""
    a256 = lambda x: (x + 255) // 256 * 256
    bh, n, spb = w.B * w.H, w.n_blocks, w.block // 64
    esz = 2 if w.dtype == "bf16" else 4
    kv = a256(bh * n * spb * 64 * w.D * esz)
    cb = min(1024 // w.block, max(1, bh * n // 512))  # blocks per statistics run
    nch = -(-n // cb)
    off = 2 * kv + a256(bh * nch * 4)
    return int(st.ws[off:off + 4].view(torch.int32).item())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_loose_logit_bound_uses_careful_kernel(dtype):
    """One huge key orthogonal to every query makes the Cauchy–Schwarz bound of
    the logits ~10^4 log2 units too high: the fast kernel must hand every query
    tile to the running-max kernel, and the result must still match."""
    w = W(f"loose_bound_{dtype}", 1, 2, 700, 128, 64, 0.25, dtype, "hyd", None, 0.0, seed=41)
    q, k, v = synth.make_qkv(w)
    q[..., 0] = 0
    k[:, :, 130, :] = 0
    k[:, :, 130, 0] = 3.0e4
    res = check_workload(w, qkv=(q, k, v))
    assert redo_count(res["stats"], w) == w.B * w.H * w.n_blocks


def test_tight_bound_uses_fast_kernel_only():
    w = synth.FLUX.replace(H=2, L=2000)
    res = check_workload(w)
    assert redo_count(res["stats"], w) == 0


def test_dense_baseline_parity():
    dev = torch.device("cuda:0")
    for w in (W("dense_bf16", 1, 2, 1000, 128, 64, 1.0, "bf16", seed=31),
              W("dense_f32", 1, 1, 777, 64, 64, 1.0, "f32", seed=32)):
        q, k, v = synth.make_qkv(w)
        o = bsa.dense(*(x.to(dev) for x in (q, k, v))).float().cpu().numpy()
        for h in range(w.H):
            ref = oracle.dense_rows(*(synth.as_f64(x[0, h]) for x in (q, k, v)), slice(0, w.L), w.scale)
            compare_out(o[0, h], ref, w.dtype, f"{w.name} head {h}")


def test_dense_baseline_wan_shape_sampled():
    w = synth.WAN.replace(H=2)
    dev = torch.device("cuda:0")
    q, k, v = synth.make_qkv(w)
    o = bsa.dense(*(x.to(dev) for x in (q, k, v))).float().cpu().numpy()
    for h in range(2):
        qh, kh, vh = (synth.as_f64(x[0, h]) for x in (q, k, v))
        for i in sample_qblocks(w.n_blocks, 4, 3):
            r = slice(i * 64, min(w.L, (i + 1) * 64))
            ref = oracle.dense_rows(qh, kh, vh, r, w.scale)
            compare_out(o[0, h, r], ref, w.dtype, f"dense wan head {h} query block {i}")


def test_density_one_equals_dense_on_gpu():
    w = W("d1", 1, 2, 1000, 128, 64, 1.0, "bf16", seed=33)
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in synth.make_qkv(w))
    o1 = bsa.piecewise_sparse_attention_hyd(q, k, v, density=1.0).float()
    o2 = bsa.dense(q, k, v).float()
    assert (o1 - o2).abs().max().item() <= 1e-2


def test_constant_values_give_constant_output():
    """Normalisation consistency at a DiT shape: v_t = c ⇒ o_t = c."""
    w = synth.FLUX.replace(H=4)
    dev = torch.device("cuda:0")
    q, k, _ = synth.make_qkv(w)
    c = torch.linspace(-2, 2, w.D, dtype=torch.float32).to(torch.bfloat16)
    v = c.expand(w.B, w.H, w.L, w.D).contiguous()
    for fn in (bsa.piecewise_sparse_attention_hyd, bsa.piecewise_sparse_attention_0th):
        o = fn(q.to(dev), k.to(dev), v.to(dev), density=w.density, sink_idx=0).float().cpu()
        assert (o - c.float()).abs().max().item() <= 2e-2


def test_deterministic_and_stream_ordered():
    w = synth.FLUX.replace(H=3)
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in synth.make_qkv(w))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o1, i1 = bsa.piecewise_sparse_attention_hyd(q, k, v, density=0.15, return_idx=True)
    s.synchronize()
    o2, i2 = bsa.piecewise_sparse_attention_hyd(q, k, v, density=0.15, return_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(o1, o2)


def test_bad_arguments_raise_before_launch():
    dev = torch.device("cuda:0")
    q = torch.zeros(1, 1, 100, 96, dtype=torch.bfloat16, device=dev)
    with pytest.raises(bsa.PisaError):
        bsa.piecewise_sparse_attention_hyd(q, q, q, density=0.5)
    q = torch.zeros(1, 1, 100, 128, dtype=torch.bfloat16, device=dev)
    st = bsa.block_stats(q, q, q)
    with pytest.raises(ValueError):
        bsa.select(st, topk=3, scale=0.1)  # n = 2: the binding refuses it before the call
    idx = torch.zeros(1, 1, 2, 3, dtype=torch.int32, device=dev)
    shape = bsa.make_shape(q, 64)
    sst = st.struct()
    # the library refuses it too, enqueueing nothing
    assert bsa.load_library().pisa_select(bsa.ctypes.byref(shape), bsa.ctypes.byref(sst), 0.1, 0.0, 3,
                                          bsa.PISA_SINK_NONE, idx.data_ptr(), None) == bsa.PISA_EINVAL
    torch.cuda.synchronize()
