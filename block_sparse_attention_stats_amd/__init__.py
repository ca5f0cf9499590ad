"""PISA piecewise sparse attention forward pass on MI355X (gfx950).

A thin ctypes binding over ``libpisa.so`` (C ABI in ``include/pisa.h``). This
module only checks and marshals arguments and allocates outputs and workspace
with torch; every step of the computation runs in the library's HIP kernels on
torch's current stream. Importing works without a GPU; calling needs the built
library and a visible gfx950 device, otherwise it raises.

Entry points follow the authors' README (``piecewise_sparse_attention_hyd``,
``piecewise_sparse_attention_0th``, ``piecewise_sparse_attention`` alias;
keyword arguments ``density``, ``block_size``, ``sink_idx``), with
``cov_weight`` (covariance-aware routing weight, gist.science summary,
"Covariance-Aware Routing") and ``scale`` added. The three steps are also
exposed one by one: :func:`block_stats`, :func:`select`, :func:`attn_fwd`, and
the same-device dense baseline :func:`dense`.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpisa.so")

PISA_OK, PISA_EINVAL, PISA_ENOTSUP, PISA_EHIP, PISA_ETOOBIG = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_BYTES = 256 << 20  # pisa.h PISA_NOALLOC_SCRATCH_BYTES
PISA_F32, PISA_BF16 = 0, 1
PISA_SINK_NONE = -(2 ** 31)
EXPORTS = ("pisa_workspace_bytes", "pisa_block_stats", "pisa_select", "pisa_attn_fwd",
           "dense_workspace_bytes", "dense_attn_fwd", "pisa_status_string", "pisa_last_hip_error",
           "pisa_block_stats_seg", "pisa_attn_fwd_seg", "dense_attn_fwd_seg", "pisa_attn_fwd_noalloc",
           "pisa_bwd_workspace_bytes", "pisa_attn_bwd", "pisa_attn_fwd_lse")


class PisaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: {_status_text(status)}{(' (' + detail + ')') if detail else ''}")


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32),
                ("D", ctypes.c_int32), ("block", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("layout", ctypes.c_int32)]


# q, k, v, o memory layouts (pisa.h PISA_LAYOUT_*)
LAYOUTS = {"BHLD": 0, "BLHD": 1}


class Segments(ctypes.Structure):
    """A sequence held in two tensors: tokens [0, L0) in the usual q, k, v (o)
    arguments, the rest in q1, k1, v1 (o1)."""
    _fields_ = [("L0", ctypes.c_int32), ("q1", ctypes.c_void_p), ("k1", ctypes.c_void_p),
                ("v1", ctypes.c_void_p), ("o1", ctypes.c_void_p)]


class StatsStruct(ctypes.Structure):
    _fields_ = [("qbar", ctypes.c_void_p), ("kbar", ctypes.c_void_p), ("vsum", ctypes.c_void_p),
                ("hbar", ctypes.c_void_p), ("mnorm", ctypes.c_void_p), ("ws", ctypes.c_void_p),
                ("ws_bytes", ctypes.c_size_t), ("mnorm_ord", ctypes.c_int32)]


# norm of M_j = ||H_j - H-bar|| (pisa.h PISA_NORM_*)
NORMS = {"fro": 0, "spectral": 2}


def _norm_code(cov_norm: str) -> int:
    if cov_norm not in NORMS:
        raise ValueError(f"unknown cov_norm {cov_norm!r}; expected one of {sorted(NORMS)}")
    return NORMS[cov_norm]


_lib_handle = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libpisa.so (once). Raises if it has not been built."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m block_sparse_attention_stats_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, D64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double, ctypes.c_size_t
    SP, STP, SG = ctypes.POINTER(Shape), ctypes.POINTER(StatsStruct), ctypes.POINTER(Segments)
    sig = {
        "pisa_workspace_bytes": (SZ, [SP]),
        "dense_workspace_bytes": (SZ, [SP]),
        "pisa_block_stats": (I32, [SP, P, P, P, STP, P]),
        "pisa_select": (I32, [SP, STP, D64, D64, I32, I32, P, P]),
        "pisa_attn_fwd": (I32, [SP, P, STP, I32, P, I32, D64, P, P]),
        "pisa_attn_fwd_lse": (I32, [SP, P, STP, I32, P, I32, D64, P, P, P]),
        "dense_attn_fwd": (I32, [SP, P, P, P, D64, P, P, SZ, P]),
        "pisa_block_stats_seg": (I32, [SP, P, P, P, SG, STP, P]),
        "pisa_attn_fwd_seg": (I32, [SP, P, STP, I32, P, I32, D64, P, SG, P]),
        "dense_attn_fwd_seg": (I32, [SP, P, P, P, SG, D64, P, P, SZ, P]),
        "pisa_attn_fwd_noalloc": (I32, [SP, P, P, P, I32, P, I32, D64, P, P]),
        "pisa_bwd_workspace_bytes": (SZ, [SP]),
        "pisa_attn_bwd": (I32, [SP, P, P, P, STP, P, I32, D64, P, P, P, P, P, P, P, SZ, P]),
        "pisa_status_string": (ctypes.c_char_p, [I32]),
        "pisa_last_hip_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib_handle = lib
    return lib


def _status_text(status: int) -> str:
    try:
        return load_library().pisa_status_string(status).decode()
    except Exception:  # library missing: describe the code ourselves
        return {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "HIP runtime error",
                4: "problem larger than the fixed scratch"}.get(status, "?")


def _check(status: int, where: str):
    if status != PISA_OK:
        detail = load_library().pisa_last_hip_error().decode() if status == PISA_EHIP else ""
        raise PisaError(status, where, detail)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PISA_BF16
    if t.dtype == torch.float32:
        return PISA_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _check_qkv(*ts: torch.Tensor):
    ref = ts[0]
    for t in ts:
        if not isinstance(t, torch.Tensor):
            raise TypeError("q, k, v must be torch tensors")
        if t.dim() != 4:
            raise ValueError("tensors must be [batch, heads, seq, head_dim] or [batch, seq, heads, head_dim]")
        if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("q, k, v must share shape, dtype and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _on_gpu(*ts: torch.Tensor):
    """Every tensor on one GPU (checked after shapes and dtypes, so that a
    mismatch is reported as such on any device)."""
    dev = ts[0].device
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if t.device != dev:
            raise ValueError("tensors must be on the same GPU")


def _expect(t, shape, dtype, what: str):
    """t is a contiguous tensor of exactly `shape` and `dtype` (device checked later)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{what} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


_TORCH_DTYPE = {0: torch.float32, 1: torch.bfloat16}


def _io_shape(shape: "Shape", L: int | None = None) -> tuple:
    """Shape of a q, k, v or o tensor holding L tokens (default: all) of `shape`."""
    L = shape.L if L is None else L
    return (shape.B, L, shape.H, shape.D) if shape.layout == 1 else (shape.B, shape.H, L, shape.D)


def _check_io(t, shape: "Shape", what: str, L: int | None = None):
    _expect(t, _io_shape(shape, L), _TORCH_DTYPE[shape.dtype], what)


def _check_idx(idx, shape: "Shape") -> int:
    """idx is [B, H, n, topk] int32 with 1 <= topk <= n; returns topk."""
    if not isinstance(idx, torch.Tensor) or idx.dim() != 4:
        raise ValueError("idx must be a [batch, heads, blocks, topk] tensor")
    n = num_blocks(shape.L, shape.block)
    topk = int(idx.shape[-1])
    if not 1 <= topk <= n:
        raise ValueError(f"idx holds {topk} blocks per row; expected 1 to {n}")
    _expect(idx, (shape.B, shape.H, n, topk), torch.int32, "idx")
    return topk


def make_shape(q: torch.Tensor, block_size: int, layout: str = "BHLD") -> Shape:
    """Shape of q laid out as [B,H,L,D] ("BHLD") or [B,L,H,D] ("BLHD")."""
    if layout not in LAYOUTS:
        raise ValueError(f"unknown layout {layout!r}; expected one of {sorted(LAYOUTS)}")
    if layout == "BLHD":
        B, L, H, D = q.shape
    else:
        B, H, L, D = q.shape
    return Shape(B, H, L, D, block_size, _dtype_code(q), LAYOUTS[layout])


def num_blocks(L: int, block_size: int) -> int:
    return -(-L // block_size)


def topk_from_density(density: float, n: int) -> int:
    """Exact blocks per query block: clamp(floor(density * n), 1, n), in fp64."""
    k = int(math.floor(float(density) * float(n)))
    return max(1, min(n, k))


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


@dataclass
class Stats:
    """Block statistics of one call (device tensors) and the workspace they live with."""

    shape: Shape
    qbar: torch.Tensor   # [B,H,n,D] fp64
    kbar: torch.Tensor   # [B,H,n,D] fp64
    vsum: torch.Tensor   # [B,H,n,D] fp64
    hbar: torch.Tensor   # [B,H,D,D] fp64
    mnorm: torch.Tensor | None  # [B,H,n] fp64
    ws: torch.Tensor     # uint8 workspace
    mnorm_ord: str = "fro"  # norm of M_j: "fro" or "spectral"

    def check(self, shape: Shape | None = None):
        """Every buffer has the size and dtype that the shape (default: its
        own) implies; raises ValueError otherwise. The device is checked by
        the caller, with the call's other tensors (tensors())."""
        sh = self.shape
        if shape is not None and _shape_tuple(shape) != _shape_tuple(sh):
            raise ValueError(f"statistics were made for shape {_shape_tuple(sh)}, "
                             f"not {_shape_tuple(shape)}")
        n = num_blocks(sh.L, sh.block)
        f64 = torch.float64
        _expect(self.qbar, (sh.B, sh.H, n, sh.D), f64, "Stats.qbar")
        _expect(self.kbar, (sh.B, sh.H, n, sh.D), f64, "Stats.kbar")
        _expect(self.vsum, (sh.B, sh.H, n, sh.D), f64, "Stats.vsum")
        _expect(self.hbar, (sh.B, sh.H, sh.D, sh.D), f64, "Stats.hbar")
        if self.mnorm is not None:
            _expect(self.mnorm, (sh.B, sh.H, n), f64, "Stats.mnorm")
        if not isinstance(self.ws, torch.Tensor) or self.ws.dtype != torch.uint8 or self.ws.dim() != 1:
            raise ValueError("Stats.ws must be a 1-D uint8 tensor")
        if self.ws.numel() < workspace_bytes(sh):
            raise ValueError(f"Stats.ws holds {self.ws.numel()} bytes; the shape needs {workspace_bytes(sh)}")

    def tensors(self) -> list:
        return [t for t in (self.qbar, self.kbar, self.vsum, self.hbar, self.mnorm, self.ws) if t is not None]

    def struct(self) -> StatsStruct:
        return StatsStruct(self.qbar.data_ptr(), self.kbar.data_ptr(), self.vsum.data_ptr(),
                           self.hbar.data_ptr(), self.mnorm.data_ptr() if self.mnorm is not None else None,
                           self.ws.data_ptr(), self.ws.numel(), _norm_code(self.mnorm_ord))


def _shape_tuple(shape: Shape) -> tuple:
    return (shape.B, shape.H, shape.L, shape.D, shape.block, shape.dtype, shape.layout)


def workspace_bytes(shape: Shape) -> int:
    nbytes = load_library().pisa_workspace_bytes(ctypes.byref(shape))
    if nbytes == 0:
        raise PisaError(PISA_EINVAL, "pisa_workspace_bytes")
    return nbytes


def alloc_stats(shape: Shape, device, want_mnorm: bool) -> Stats:
    B, H, L, D, blk = shape.B, shape.H, shape.L, shape.D, shape.block
    n = num_blocks(L, blk)
    f64 = dict(dtype=torch.float64, device=device)
    ws = torch.empty(workspace_bytes(shape), dtype=torch.uint8, device=device)
    return Stats(shape, torch.empty((B, H, n, D), **f64), torch.empty((B, H, n, D), **f64),
                 torch.empty((B, H, n, D), **f64), torch.empty((B, H, D, D), **f64),
                 torch.empty((B, H, n), **f64) if want_mnorm else None, ws)


def block_stats(q, k, v, block_size: int = 64, want_mnorm: bool = False, out: Stats | None = None,
                layout: str = "BHLD", cov_norm: str = "fro") -> Stats:
    """Step 1: q̄, k̄, ΣV, H̄ (and M_j when ``want_mnorm``) via pisa_block_stats.
    ``layout`` is that of q, k, v (and of the output of attn_fwd with these
    statistics); the statistics themselves are [B,H,...] either way.
    ``cov_norm``: the norm of M_j, "fro" (Frobenius) or "spectral" (2-norm)."""
    _norm_code(cov_norm)
    _check_qkv(q, k, v)
    shape = make_shape(q, block_size, layout)
    if out is not None:
        out.check(shape)
        if want_mnorm and out.mnorm is None:
            raise ValueError("want_mnorm needs Stats.mnorm")
    _on_gpu(q, k, v, *(() if out is None else out.tensors()))
    st = out if out is not None else alloc_stats(shape, q.device, want_mnorm)
    st.mnorm_ord = cov_norm
    sst = st.struct()
    _check(load_library().pisa_block_stats(ctypes.byref(shape), q.data_ptr(), k.data_ptr(),
                                           v.data_ptr(), ctypes.byref(sst), _stream()),
           "pisa_block_stats")
    return st


def _sink_code(sink_idx) -> int:
    if sink_idx is None:
        return PISA_SINK_NONE
    if sink_idx in (0, -1):
        return int(sink_idx)
    raise ValueError("sink_idx must be None, 0 or -1")


def select(st: Stats, topk: int, scale: float, cov_weight: float = 0.0, sink_idx=None,
           out: torch.Tensor | None = None) -> torch.Tensor:
    """Step 2: per-query-block top-k key blocks, ascending, [B,H,n,topk] int32."""
    shape = st.shape
    st.check()
    n = num_blocks(shape.L, shape.block)
    if not 1 <= int(topk) <= n:
        raise ValueError(f"topk = {topk}; expected 1 to {n}")
    if cov_weight and st.mnorm is None:
        raise ValueError("covariance-aware routing (cov_weight > 0) needs Stats.mnorm")
    if out is not None:
        _expect(out, (shape.B, shape.H, n, int(topk)), torch.int32, "idx")
    _on_gpu(*st.tensors(), *(() if out is None else (out,)))
    idx = out if out is not None else torch.empty((shape.B, shape.H, n, topk), dtype=torch.int32,
                                                  device=st.qbar.device)
    sst = st.struct()
    _check(load_library().pisa_select(ctypes.byref(shape), ctypes.byref(sst), float(scale),
                                      float(cov_weight), int(topk), _sink_code(sink_idx),
                                      idx.data_ptr(), _stream()), "pisa_select")
    return idx


VARIANTS = {"0th": 0, "hyd": 1, "pb1": 2}


def _variant_code(first_order) -> int:
    """pisa_attn_fwd's first_order argument: True / "hyd" 1, False / "0th" 0, "pb1" 2."""
    if isinstance(first_order, str):
        if first_order not in VARIANTS:
            raise ValueError(f"unknown variant {first_order!r}; expected one of {sorted(VARIANTS)}")
        return VARIANTS[first_order]
    return 1 if first_order else 0


def attn_fwd(q, st: Stats, idx: torch.Tensor, scale: float, first_order=True,
             out: torch.Tensor | None = None, return_lse: bool = False):
    """Step 3: fused exact + zeroth-order (+ first-order) pass.

    first_order: True or "hyd" (global H̄ term), False or "0th" (none), "pb1"
    (each unselected block's own first-order term). With return_lse the call
    goes through pisa_attn_fwd_lse and returns (o, lse), lse [B,H,L] fp32 =
    ln D_t of each row, which attn_bwd can take."""
    code = _variant_code(first_order)
    shape = st.shape
    st.check()
    _check_io(q, shape, "q")
    topk = _check_idx(idx, shape)
    if out is not None:
        _check_io(out, shape, "out")
    _on_gpu(q, idx, *st.tensors(), *(() if out is None else (out,)))
    o = out if out is not None else torch.empty_like(q)
    sst = st.struct()
    lib = load_library()
    if not return_lse:
        _check(lib.pisa_attn_fwd(ctypes.byref(shape), q.data_ptr(), ctypes.byref(sst), code, idx.data_ptr(),
                                 topk, float(scale), o.data_ptr(), _stream()), "pisa_attn_fwd")
        return o
    lse = torch.empty((shape.B, shape.H, shape.L), dtype=torch.float32, device=q.device)
    _check(lib.pisa_attn_fwd_lse(ctypes.byref(shape), q.data_ptr(), ctypes.byref(sst), code, idx.data_ptr(),
                                 topk, float(scale), o.data_ptr(), lse.data_ptr(), _stream()), "pisa_attn_fwd_lse")
    return o, lse


def attn_fwd_noalloc(q, k, v, idx: torch.Tensor, scale: float, first_order=True, block_size: int = 64,
                     out: torch.Tensor | None = None, layout: str = "BHLD") -> torch.Tensor:
    """Statistics and fused pass in one call of pisa_attn_fwd_noalloc, which
    allocates no device memory and takes no workspace (its intermediates live
    in a fixed per-device array of NOALLOC_SCRATCH_BYTES). The caller passes the
    selection idx [B,H,n,topk] and may pass the output; a call whose shape
    needs more scratch raises PisaError (PISA_ETOOBIG)."""
    code = _variant_code(first_order)
    _check_qkv(q, k, v)
    shape = make_shape(q, block_size, layout)
    topk = _check_idx(idx, shape)
    if out is not None:
        _check_io(out, shape, "out")
    _on_gpu(q, k, v, idx, *(() if out is None else (out,)))
    o = out if out is not None else torch.empty_like(q)
    _check(load_library().pisa_attn_fwd_noalloc(ctypes.byref(shape), q.data_ptr(), k.data_ptr(),
                                                v.data_ptr(), code, idx.data_ptr(), topk, float(scale),
                                                o.data_ptr(), _stream()), "pisa_attn_fwd_noalloc")
    return o


def attn_bwd(q, k, v, st: Stats, idx: torch.Tensor, scale: float, o, dout, ws: torch.Tensor | None = None,
             lse: torch.Tensor | None = None):
    """Backward pass of the zeroth-order-only variant via pisa_attn_bwd: the
    gradients (dq, dk, dv) of Σ o∘dout, with the selection idx held fixed. q,
    k, v, st and idx are those of the forward call and o its output; lse, if
    given, the ln D_t that the forward returned (attn_fwd(..., return_lse=True)),
    which saves the backward a sweep."""
    _check_qkv(q, k, v)
    shape = st.shape
    st.check()
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _check_io(t, shape, name)
    topk = _check_idx(idx, shape)
    if lse is not None:
        _expect(lse, (shape.B, shape.H, shape.L), torch.float32, "lse")
    lib = load_library()
    nbytes = lib.pisa_bwd_workspace_bytes(ctypes.byref(shape))
    if nbytes == 0:
        raise PisaError(PISA_EINVAL, "pisa_bwd_workspace_bytes")
    if ws is not None and (ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous()):
        raise ValueError("ws must be a contiguous 1-D uint8 tensor")
    _on_gpu(q, k, v, o, dout, idx, *st.tensors(), *(() if ws is None else (ws,)),
            *(() if lse is None else (lse,)))
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    sst = st.struct()
    _check(lib.pisa_attn_bwd(ctypes.byref(shape), q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(sst),
                             idx.data_ptr(), topk, float(scale), o.data_ptr(),
                             None if lse is None else lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                             dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(), _stream()),
           "pisa_attn_bwd")
    return dq, dk, dv


class _Pisa0th(torch.autograd.Function):
    """The zeroth-order-only variant with a backward pass: forward through
    pisa_block_stats, pisa_select and pisa_attn_fwd, backward through
    pisa_attn_bwd (the selection held fixed)."""

    @staticmethod
    def forward(ctx, q, k, v, density, block_size, sink_idx, cov_weight, scale, layout, cov_norm):
        shape = make_shape(q, block_size, layout)
        s = 1.0 / math.sqrt(shape.D) if scale is None else float(scale)
        topk = topk_from_density(density, num_blocks(shape.L, block_size))
        st = block_stats(q, k, v, block_size, want_mnorm=cov_weight > 0, layout=layout, cov_norm=cov_norm)
        idx = select(st, topk, s, cov_weight, sink_idx)
        o, lse = attn_fwd(q, st, idx, s, False, return_lse=True)
        ctx.save_for_backward(q, k, v, o, idx, lse)
        ctx.st, ctx.scale = st, s
        ctx.mark_non_differentiable(idx)
        return o, idx

    @staticmethod
    def backward(ctx, do, _didx):
        q, k, v, o, idx, lse = ctx.saved_tensors
        dq, dk, dv = attn_bwd(q, k, v, ctx.st, idx, ctx.scale, o, do.contiguous(), lse=lse)
        return dq, dk, dv, None, None, None, None, None, None, None


def dense(q, k, v, scale: float | None = None, out: torch.Tensor | None = None,
          ws: torch.Tensor | None = None, layout: str = "BHLD") -> torch.Tensor:
    """Same-device dense attention baseline, softmax(scale·QKᵀ)V."""
    _check_qkv(q, k, v)
    shape = make_shape(q, 64, layout)
    s = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
    lib = load_library()
    nbytes = lib.dense_workspace_bytes(ctypes.byref(shape))
    if nbytes == 0:
        raise PisaError(PISA_EINVAL, "dense_workspace_bytes")
    if out is not None:
        _check_io(out, shape, "out")
    if ws is not None:
        if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
            raise ValueError("ws must be a contiguous 1-D uint8 tensor")
    _on_gpu(q, k, v, *[t for t in (out, ws) if t is not None])
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    o = out if out is not None else torch.empty_like(q)
    _check(lib.dense_attn_fwd(ctypes.byref(shape), q.data_ptr(), k.data_ptr(), v.data_ptr(), float(s),
                              o.data_ptr(), ws.data_ptr(), ws.numel(), _stream()), "dense_attn_fwd")
    return o


def piecewise_sparse_attention_hyd(q, k, v, density: float = 0.15, block_size: int = 64,
                                   sink_idx=None, cov_weight: float = 0.0, scale=None,
                                   first_order=True, return_idx: bool = False,
                                   layout: str = "BHLD", cov_norm: str = "fro"):
    """PISA forward (hybrid order: zeroth order + global first-order correction).
    q, k, v (and the output) are [B,H,L,D], or [B,L,H,D] with layout="BLHD"."""
    _check_qkv(q, k, v)
    shape = make_shape(q, block_size, layout)
    L, D = shape.L, shape.D
    s = 1.0 / math.sqrt(D) if scale is None else float(scale)
    n = num_blocks(L, block_size)
    topk = topk_from_density(density, n)
    st = block_stats(q, k, v, block_size, want_mnorm=cov_weight > 0, layout=layout, cov_norm=cov_norm)
    idx = select(st, topk, s, cov_weight, sink_idx)
    o = attn_fwd(q, st, idx, s, first_order)
    return (o, idx) if return_idx else o


def piecewise_sparse_attention_0th(q, k, v, density: float = 0.15, block_size: int = 64,
                                   sink_idx=None, cov_weight: float = 0.0, scale=None,
                                   return_idx: bool = False, layout: str = "BHLD", cov_norm: str = "fro"):
    """PISA forward, zeroth-order-only variant (no global first-order term).
    When q, k or v requires a gradient (and autograd is on), the call records
    a backward pass through pisa_attn_bwd, as the README's training example
    uses it (``out_0th.backward(...)``)."""
    if torch.is_grad_enabled() and any(t.requires_grad for t in (q, k, v)):
        _check_qkv(q, k, v)
        o, idx = _Pisa0th.apply(q, k, v, density, block_size, sink_idx, cov_weight, scale, layout, cov_norm)
        return (o, idx) if return_idx else o
    return piecewise_sparse_attention_hyd(q, k, v, density, block_size, sink_idx, cov_weight, scale,
                                          first_order=False, return_idx=return_idx, layout=layout,
                                          cov_norm=cov_norm)


def piecewise_sparse_attention_pb1(q, k, v, density: float = 0.15, block_size: int = 64,
                                   sink_idx=None, cov_weight: float = 0.0, scale=None,
                                   return_idx: bool = False, layout: str = "BHLD", cov_norm: str = "fro"):
    """PISA forward with a first-order term per unselected block (q·H_j for each
    block instead of the global H̄); costs about as much as dense attention."""
    return piecewise_sparse_attention_hyd(q, k, v, density, block_size, sink_idx, cov_weight, scale,
                                          first_order="pb1", return_idx=return_idx, layout=layout,
                                          cov_norm=cov_norm)


piecewise_sparse_attention = piecewise_sparse_attention_hyd


# --------------------------------------------------------------------------
# Joint attention over a sequence held in two tensors (MMDiT text and image
# streams), without a concatenated copy.

def _joint_shape(q0: torch.Tensor, q1: torch.Tensor, block_size: int, layout: str) -> Shape:
    shape = make_shape(q0, block_size, layout)
    s1 = make_shape(q1, block_size, layout)
    if (s1.B, s1.H, s1.D, s1.dtype) != (shape.B, shape.H, shape.D, shape.dtype):
        raise ValueError("both parts must have the same batch, heads, head_dim and dtype")
    shape.L = shape.L + s1.L
    return shape


def _segments(L0: int, q1, k1=None, v1=None, o1=None) -> Segments:
    ptr = lambda t: None if t is None else t.data_ptr()
    return Segments(L0, ptr(q1), ptr(k1), ptr(v1), ptr(o1))


def block_stats_seg(q0, k0, v0, q1, k1, v1, block_size: int = 64, want_mnorm: bool = False,
                    out: Stats | None = None, layout: str = "BHLD", cov_norm: str = "fro") -> Stats:
    """Step 1 on the sequence q0 ++ q1 (and k, v likewise), via pisa_block_stats_seg."""
    _check_qkv(q0, k0, v0)
    _check_qkv(q1, k1, v1)
    shape = _joint_shape(q0, q1, block_size, layout)
    L0 = shape.L - make_shape(q1, block_size, layout).L
    if out is not None:
        out.check(shape)
        if want_mnorm and out.mnorm is None:
            raise ValueError("want_mnorm needs Stats.mnorm")
    _norm_code(cov_norm)
    _on_gpu(q0, k0, v0, q1, k1, v1, *(() if out is None else out.tensors()))
    st = out if out is not None else alloc_stats(shape, q0.device, want_mnorm)
    st.mnorm_ord = cov_norm
    sst = st.struct()
    seg = _segments(L0, q1, k1, v1)
    _check(load_library().pisa_block_stats_seg(ctypes.byref(shape), q0.data_ptr(), k0.data_ptr(),
                                               v0.data_ptr(), ctypes.byref(seg), ctypes.byref(sst),
                                               _stream()), "pisa_block_stats_seg")
    return st


def attn_fwd_seg(q0, q1, st: Stats, idx: torch.Tensor, scale: float, first_order=True,
                 out0: torch.Tensor | None = None, out1: torch.Tensor | None = None):
    """Step 3 on the sequence q0 ++ q1; returns the output in two parts shaped
    like q0 and q1."""
    code = _variant_code(first_order)
    shape = st.shape
    st.check()
    if not isinstance(q1, torch.Tensor) or q1.dim() != 4:
        raise ValueError("q1 must be a 4-D tensor")
    L1 = int(q1.shape[1] if shape.layout == LAYOUTS["BLHD"] else q1.shape[2])
    L0 = shape.L - L1
    if not 1 <= L0 <= shape.L:
        raise ValueError(f"q1 holds {L1} tokens; the statistics' sequence has {shape.L}")
    _check_io(q0, shape, "q0", L0)
    _check_io(q1, shape, "q1", L1)
    topk = _check_idx(idx, shape)
    if out0 is not None:
        _check_io(out0, shape, "out0", L0)
    if out1 is not None:
        _check_io(out1, shape, "out1", L1)
    _on_gpu(q0, q1, idx, *st.tensors(), *[t for t in (out0, out1) if t is not None])
    o0 = out0 if out0 is not None else torch.empty_like(q0)
    o1 = out1 if out1 is not None else torch.empty_like(q1)
    sst = st.struct()
    seg = _segments(L0, q1, o1=o1)
    _check(load_library().pisa_attn_fwd_seg(ctypes.byref(shape), q0.data_ptr(), ctypes.byref(sst), code,
                                            idx.data_ptr(), topk, float(scale),
                                            o0.data_ptr(), ctypes.byref(seg), _stream()),
           "pisa_attn_fwd_seg")
    return o0, o1


def dense_seg(q0, k0, v0, q1, k1, v1, scale: float | None = None, layout: str = "BHLD"):
    """Dense baseline on the sequence q0 ++ q1; output in two parts."""
    _check_qkv(q0, k0, v0)
    _check_qkv(q1, k1, v1)
    shape = _joint_shape(q0, q1, 64, layout)
    L0 = shape.L - make_shape(q1, 64, layout).L
    _on_gpu(q0, k0, v0, q1, k1, v1)
    s = 1.0 / math.sqrt(q0.shape[-1]) if scale is None else scale
    lib = load_library()
    nbytes = lib.dense_workspace_bytes(ctypes.byref(shape))
    if nbytes == 0:
        raise PisaError(PISA_EINVAL, "dense_workspace_bytes")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q0.device)
    o0, o1 = torch.empty_like(q0), torch.empty_like(q1)
    seg = _segments(L0, q1, k1, v1, o1)
    _check(lib.dense_attn_fwd_seg(ctypes.byref(shape), q0.data_ptr(), k0.data_ptr(), v0.data_ptr(),
                                  ctypes.byref(seg), float(s), o0.data_ptr(), ws.data_ptr(), ws.numel(),
                                  _stream()), "dense_attn_fwd_seg")
    return o0, o1


def mmdit_joint_attention(txt_q, txt_k, txt_v, img_q, img_k, img_v, density: float = 0.15,
                          block_size: int = 64, text_first: bool = True, variant="hyd",
                          cov_weight: float = 0.0, scale=None, layout: str = "BHLD",
                          return_idx: bool = False, cov_norm: str = "fro"):
    """PISA over the joint text + image sequence of an MMDiT block, with the
    text block as the attention sink (README, "Attention sink for MMDiT"):
    text first (FLUX) forces block 0, text last (Hunyuan-Video) block n-1.
    Returns (o_txt, o_img), shaped like the inputs."""
    if text_first:
        parts, sink = ((txt_q, txt_k, txt_v), (img_q, img_k, img_v)), 0
    else:
        parts, sink = ((img_q, img_k, img_v), (txt_q, txt_k, txt_v)), -1
    (q0, k0, v0), (q1, k1, v1) = parts
    shape = _joint_shape(q0, q1, block_size, layout)
    s = 1.0 / math.sqrt(shape.D) if scale is None else float(scale)
    topk = topk_from_density(density, num_blocks(shape.L, block_size))
    st = block_stats_seg(q0, k0, v0, q1, k1, v1, block_size, want_mnorm=cov_weight > 0, layout=layout,
                         cov_norm=cov_norm)
    idx = select(st, topk, s, cov_weight, sink)
    o0, o1 = attn_fwd_seg(q0, q1, st, idx, s, variant)
    o_txt, o_img = (o0, o1) if text_first else (o1, o0)
    return (o_txt, o_img, idx) if return_idx else (o_txt, o_img)

