"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before anything reaches a GPU (no compute calls here)."""

import ctypes
import os
import re

import pytest

import block_sparse_attention_stats_amd as bsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pisa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(bsa.LIB_PATH), reason="libpisa.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pisa_\w+|dense_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = bsa.load_library()
    names = declared_functions()
    assert set(names) == set(bsa.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def shape(B=1, H=2, L=1000, D=128, block=64, dtype=bsa.PISA_BF16, layout=0):
    return bsa.Shape(B, H, L, D, block, dtype, layout)


def test_workspace_sizes():
    lib = bsa.load_library()
    s = shape()
    total = lib.pisa_workspace_bytes(ctypes.byref(s))
    dense = lib.dense_workspace_bytes(ctypes.byref(s))
    n = 16
    kv = 2 * 2 * n * 64 * 128 * 2  # K and V copies of 2 heads
    assert dense >= kv and dense < kv + 1024
    assert total >= dense and total % 256 == 0 and dense % 256 == 0
    # rows of up to 1280 blocks are routed on chip: no score buffer; longer
    # rows pass their fp64 scores through the workspace, a chunk of heads at a time
    ws = lambda n: lib.pisa_workspace_bytes(ctypes.byref(shape(L=n * 64)))
    assert ws(1280) - ws(1279) < 1e6  # one more block of copies and statistics
    assert ws(1281) - ws(1280) >= 2 * 1281 ** 2 * 8  # the scores of both heads appear
    assert lib.pisa_workspace_bytes(ctypes.byref(shape(D=96))) == 0
    assert lib.pisa_workspace_bytes(ctypes.byref(shape(block=32))) == 0
    assert lib.pisa_workspace_bytes(ctypes.byref(shape(L=0))) == 0
    assert lib.pisa_workspace_bytes(ctypes.byref(shape(dtype=7))) == 0
    # [B,L,H,D] inputs need the same workspace; unknown layouts are rejected
    assert lib.pisa_workspace_bytes(ctypes.byref(shape(layout=1))) == total
    assert lib.dense_workspace_bytes(ctypes.byref(shape(layout=1))) == dense
    assert lib.pisa_workspace_bytes(ctypes.byref(shape(layout=2))) == 0
    assert lib.pisa_workspace_bytes(ctypes.byref(shape(layout=-1))) == 0
    assert lib.pisa_workspace_bytes(None) == 0


def test_status_strings():
    lib = bsa.load_library()
    for code in range(5):
        assert lib.pisa_status_string(code).decode()
    assert lib.pisa_last_hip_error().decode() == ""


FAKE = 0x10000  # aligned non-null host address: never dereferenced, validation fails first


def stats_struct(ws_bytes=1 << 40, mnorm=FAKE):
    return bsa.StatsStruct(FAKE, FAKE, FAKE, FAKE, mnorm, FAKE, ws_bytes)


@pytest.mark.parametrize("kw,code", [
    (dict(D=96), bsa.PISA_ENOTSUP), (dict(block=256), bsa.PISA_ENOTSUP),
    (dict(L=0), bsa.PISA_EINVAL), (dict(B=0), bsa.PISA_EINVAL), (dict(dtype=5), bsa.PISA_EINVAL),
    (dict(L=64 * 8193), bsa.PISA_ENOTSUP),
])
def test_bad_shapes_rejected(kw, code):
    lib = bsa.load_library()
    s = shape(**kw)
    st = stats_struct()
    assert lib.pisa_block_stats(ctypes.byref(s), FAKE, FAKE, FAKE, ctypes.byref(st), None) == code
    assert lib.pisa_select(ctypes.byref(s), ctypes.byref(st), 0.1, 0.0, 1, bsa.PISA_SINK_NONE, FAKE, None) == code
    assert lib.pisa_attn_fwd(ctypes.byref(s), FAKE, ctypes.byref(st), 1, FAKE, 1, 0.1, FAKE, None) == code
    assert lib.dense_attn_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, 1 << 40, None) == code


def test_bad_arguments_rejected():
    lib = bsa.load_library()
    s = shape()  # n = 16
    st = stats_struct()
    E = bsa.PISA_EINVAL
    sel = lambda st=st, scale=0.1, cw=0.0, k=2, sink=bsa.PISA_SINK_NONE, idx=FAKE: lib.pisa_select(
        ctypes.byref(s), ctypes.byref(st), scale, cw, k, sink, idx, None)
    assert sel(k=0) == E and sel(k=17) == E
    assert sel(sink=1) == E and sel(sink=-2) == E
    assert sel(cw=-1.0) == E and sel(cw=float("nan")) == E and sel(cw=float("inf")) == E
    assert sel(scale=0.0) == E and sel(scale=float("nan")) == E
    assert sel(idx=None) == E and sel(idx=FAKE + 2) == E
    assert sel(st=stats_struct(mnorm=None), cw=0.5) == E  # covariance routing needs M_j
    assert sel(st=stats_struct(ws_bytes=10)) == E  # workspace too small
    st_mis = bsa.StatsStruct(FAKE + 4, FAKE, FAKE, FAKE, None, FAKE, 1 << 40)
    assert sel(st=st_mis) == E  # misaligned fp64 buffer
    st_ws = bsa.StatsStruct(FAKE, FAKE, FAKE, FAKE, None, FAKE + 16, 1 << 40)
    assert sel(st=st_ws) == E  # workspace not 256-aligned
    for bad_ord in (1, 3, -1):  # the norm of M_j: only PISA_NORM_FRO (0) or PISA_NORM_SPECTRAL (2)
        st_ord = bsa.StatsStruct(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, bad_ord)
        assert sel(st=st_ord) == E
        assert lib.pisa_block_stats(ctypes.byref(s), FAKE, FAKE, FAKE, ctypes.byref(st_ord), None) == E
    fwd = lambda q=FAKE, o=FAKE, fo=1, idx=FAKE, k=2, scale=0.1: lib.pisa_attn_fwd(
        ctypes.byref(s), q, ctypes.byref(st), fo, idx, k, scale, o, None)
    assert fwd(q=None) == E and fwd(q=FAKE + 8) == E and fwd(o=None) == E
    assert fwd(fo=3) == E and fwd(fo=-1) == E and fwd(k=0) == E and fwd(k=17) == E and fwd(idx=None) == E
    assert fwd(scale=-1.0) == E
    fwd_lse = lambda lse=FAKE, q=FAKE, k=2: lib.pisa_attn_fwd_lse(ctypes.byref(s), q, ctypes.byref(st), 0, FAKE,
                                                                k, 0.1, FAKE, lse, None)
    assert fwd_lse(lse=None) == E and fwd_lse(lse=FAKE + 2) == E  # ln D_t output missing or misaligned
    assert fwd_lse(q=None) == E and fwd_lse(k=0) == E
    bwd = lambda lse=None, ws=FAKE, nws=1 << 40, k=2, kk=FAKE: lib.pisa_attn_bwd(
        ctypes.byref(s), FAKE, kk, FAKE, ctypes.byref(st), FAKE, k, 0.1, FAKE, lse, FAKE, FAKE, FAKE, FAKE,
        ws, nws, None)
    assert bwd(lse=FAKE + 2) == E  # misaligned ln D_t
    assert bwd(kk=None) == E and bwd(k=0) == E and bwd(ws=FAKE + 16) == E and bwd(nws=10) == E
    assert lib.pisa_block_stats(ctypes.byref(s), FAKE, None, FAKE, ctypes.byref(st), None) == E
    assert lib.pisa_block_stats(ctypes.byref(s), FAKE, FAKE, FAKE, None, None) == E
    assert lib.dense_attn_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, 10, None) == E
    assert lib.dense_attn_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, 0.1, FAKE, FAKE + 1, 1 << 40, None) == E
    assert lib.pisa_last_hip_error().decode() == ""


def test_topk_rule_matches_table():
    cases = {(0.25, 16): 4, (0.15, 72): 10, (0.125, 1182): 147, (0.10, 1861): 186,
             (0.05, 591): 29, (1.0, 591): 591, (0.0, 5): 1}
    for (d, n), k in cases.items():
        assert bsa.topk_from_density(d, n) == k


def test_segment_arguments_rejected():
    """Two-part sequences: L0 outside [1, L], or a missing or misaligned
    second-part tensor when L0 < L, fail before anything is enqueued."""
    lib = bsa.load_library()
    s = shape()  # L = 1000
    st = stats_struct()
    E = bsa.PISA_EINVAL

    def seg(L0=600, q1=FAKE, k1=FAKE, v1=FAKE, o1=FAKE):
        return ctypes.byref(bsa.Segments(L0, q1, k1, v1, o1))

    stats = lambda g: lib.pisa_block_stats_seg(ctypes.byref(s), FAKE, FAKE, FAKE, g, ctypes.byref(st), None)
    fwd = lambda g: lib.pisa_attn_fwd_seg(ctypes.byref(s), FAKE, ctypes.byref(st), 1, FAKE, 2, 0.1, FAKE,
                                          g, None)
    dense = lambda g: lib.dense_attn_fwd_seg(ctypes.byref(s), FAKE, FAKE, FAKE, g, 0.1, FAKE, FAKE,
                                             1 << 40, None)
    for call in (stats, fwd, dense):
        assert call(seg(L0=0)) == E and call(seg(L0=-5)) == E and call(seg(L0=1001)) == E
        assert call(seg(q1=None)) == E and call(seg(q1=FAKE + 8)) == E
    assert stats(seg(k1=None)) == E and stats(seg(v1=FAKE + 4)) == E
    assert fwd(seg(o1=None)) == E
    assert dense(seg(k1=None)) == E and dense(seg(o1=None)) == E



def test_noalloc_arguments_rejected_on_the_host():
    """pisa_attn_fwd_noalloc validates like pisa_attn_fwd and refuses, before
    touching the device, a shape whose intermediates exceed its fixed scratch."""
    lib = bsa.load_library()
    E = bsa.PISA_EINVAL
    s = shape()  # n = 16, fits

    def call(s=s, q=FAKE, k=FAKE, v=FAKE, fo=1, idx=FAKE, kk=2, scale=0.1, o=FAKE):
        return lib.pisa_attn_fwd_noalloc(ctypes.byref(s), q, k, v, fo, idx, kk, scale, o, None)

    assert call(k=None) == E and call(v=FAKE + 4) == E and call(q=None) == E and call(o=None) == E
    assert call(fo=3) == E and call(kk=0) == E and call(kk=17) == E and call(idx=None) == E
    assert call(scale=0.0) == E
    assert call(s=shape(D=96)) == bsa.PISA_ENOTSUP
    # K and V copies alone: 2 * 8 * 75600 * 128 * 2 bytes > 256 MiB
    assert call(s=shape(H=8, L=75600)) == bsa.PISA_ETOOBIG
    assert call(s=shape(H=40, L=75600)) == bsa.PISA_ETOOBIG
    assert lib.pisa_status_string(bsa.PISA_ETOOBIG).decode().startswith("problem larger")


def test_routing_scores_do_not_grow_with_heads():
    """At the Wan shape (1182 blocks, 11 MB of fp64 scores per head) the scores
    never reach the workspace: 80 more heads add their K/V copies and
    statistics (about 44 MB each) and nothing else. Rows beyond 1280 blocks
    run the heads in chunks over one score buffer, which does not grow with
    the head count either."""
    lib = bsa.load_library()
    ws = lambda H, L=75600: lib.pisa_workspace_bytes(ctypes.byref(shape(H=H, L=L)))
    per_head = (ws(120) - ws(40)) / 80
    n = 1182
    assert 44e6 < per_head < 45e6
    assert ws(40) < 40 * 45e6
    n = 4096
    per_head = (ws(12, n * 64) - ws(4, n * 64)) / 8
    assert per_head < 2.5 * n * 64 * 128 * 2 * 2  # copies and statistics only
