"""Seeded synthetic DiT-shaped q/k/v inputs and the named workloads.

This module only draws random numbers and names shapes. It holds none of the
attention method's arithmetic, so both the HIP path (through its tests and the
bench) and the fp64 oracle can take their inputs from it.

Recipe (the same for every workload), per (batch b, head h):
  * one generator ``numpy.random.default_rng([seed, b, h])``;
  * tokens are grouped into clusters of 64 consecutive tokens (the last cluster
    may be partial), independent of the attention block size;
  * draw order: cluster means mu_c ~ N(0, 0.5^2 I_D) (fp64), cluster spreads
    sigma_c ~ U(0.3, 1.0) (fp64), then z_q, z_k, v ~ N(0, 1) as fp32 [L, D];
  * q = mu_c + sigma_c * z_q and k = mu_c + sigma_c * z_k (computed in fp32),
    v as drawn;
  * the fp32 values are rounded to the I/O dtype (bf16 by round-to-nearest-even)
    by torch; both sides then read the *rounded* values.

The clustered keys make neighbouring keys similar, as the pages report for
non-critical blocks of pre-trained DiTs (gist.science summary, section 2 "Key
Insights", distributional stability); the real activations of Wan2.1, Hunyuan
Video and FLUX.1 are not available here and these inputs stand in for them at
the same L, H, D, block size and density.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

CLUSTER = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention workload: shape, selection settings and input seed."""

    name: str
    B: int
    H: int
    L: int
    D: int
    block: int
    density: float
    dtype: str  # "f32" or "bf16"
    variant: str = "hyd"  # "hyd" (zeroth + global first order), "0th", or "pb1" (per-block first order)
    sink_idx: int | None = None  # None, 0 or -1
    cov_weight: float = 0.0  # weight of the covariance-norm term in routing
    seed: int = 0
    cov_norm: str = "fro"  # norm of that term: "fro" (Frobenius) or "spectral" (2-norm)

    @property
    def n_blocks(self) -> int:
        return -(-self.L // self.block)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads. Text/image or frame-grid token order (FLUX: 512 text tokens
# then a 64x64 latent grid; Wan: 21 frames of 45x80; Hunyuan: 33x45x80 video
# tokens then 256 text tokens) only fixes how many tokens there are; the
# generator treats every token the same way.
TINY = Workload("tiny_f32", 1, 2, 1024, 64, 64, 0.25, "f32", "hyd", None, 0.0, seed=1)
FLUX = Workload("flux_bf16", 1, 24, 4608, 128, 64, 0.15, "bf16", "hyd", 0, 0.1, seed=2)
WAN = Workload("wan_bf16", 1, 40, 75600, 128, 64, 0.125, "bf16", "hyd", None, 0.0, seed=3)
HUNYUAN = Workload("hunyuan_bf16", 1, 24, 119056, 128, 64, 0.10, "bf16", "hyd", -1, 0.0, seed=4)
SWEEP_BASE = Workload("wan_sweep_bf16", 2, 40, 75600, 128, 64, 0.125, "bf16", "hyd", None, 0.0, seed=5)
SWEEP_DENSITIES = (0.05, 0.125, 0.25, 0.5, 1.0)
SWEEP_BLOCKS = (64, 128)
SWEEP_VARIANTS = ("0th", "hyd")


def sweep() -> list[Workload]:
    """The block x density x variant grid at the Wan shape (batch 2)."""
    out = []
    for blk in SWEEP_BLOCKS:
        for d in SWEEP_DENSITIES:
            for var in SWEEP_VARIANTS:
                out.append(SWEEP_BASE.replace(
                    name=f"wan_sweep_b{blk}_d{d}_{var}", block=blk, density=d, variant=var))
    return out


WORKLOADS = {w.name: w for w in (TINY, FLUX, WAN, HUNYUAN)}


def head_fp32(L: int, D: int, seed: int, b: int, h: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Unrounded fp32 q, k, v of shape [L, D] for one (b, h)."""
    rng = np.random.default_rng([seed, b, h])
    nc = -(-L // CLUSTER)
    mu = rng.normal(0.0, 0.5, size=(nc, D))
    sigma = rng.uniform(0.3, 1.0, size=nc)
    zq = rng.standard_normal((L, D), dtype=np.float32)
    zk = rng.standard_normal((L, D), dtype=np.float32)
    v = rng.standard_normal((L, D), dtype=np.float32)
    mu_t = np.repeat(mu.astype(np.float32), CLUSTER, axis=0)[:L]
    sg_t = np.repeat(sigma.astype(np.float32), CLUSTER)[:L, None]
    q = mu_t + sg_t * zq
    k = mu_t + sg_t * zk
    return q, k, v


def torch_dtype(name: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def head_tensors(w: Workload, b: int, h: int):
    """Rounded q, k, v of one (b, h) as CPU torch tensors [L, D] of the I/O dtype."""
    import torch
    dt = torch_dtype(w.dtype)
    return tuple(torch.from_numpy(x).to(dt) for x in head_fp32(w.L, w.D, w.seed, b, h))


def make_qkv(w: Workload, heads: list[tuple[int, int]] | None = None):
    """Rounded q, k, v as CPU torch tensors [B, H, L, D] (all heads)."""
    import torch
    dt = torch_dtype(w.dtype)
    q = torch.empty((w.B, w.H, w.L, w.D), dtype=dt)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    for b in range(w.B):
        for h in range(w.H):
            qq, kk, vv = head_tensors(w, b, h)
            q[b, h], k[b, h], v[b, h] = qq, kk, vv
    return q, k, v


def grad_out(w: Workload):
    """A seeded upstream gradient dO ~ N(0, 1), shaped [B, H, L, D] like the
    workload's q and rounded to its I/O dtype (CPU torch tensor); drawn per
    (b, h) from ``numpy.random.default_rng([seed, b, h, 1])``."""
    import torch
    dt = torch_dtype(w.dtype)
    out = torch.empty((w.B, w.H, w.L, w.D), dtype=dt)
    for b in range(w.B):
        for h in range(w.H):
            rng = np.random.default_rng([w.seed, b, h, 1])
            out[b, h] = torch.from_numpy(rng.standard_normal((w.L, w.D), dtype=np.float32)).to(dt)
    return out


def integer_qkv(B: int, H: int, L: int, D: int, seed: int, key_period: int | None = None,
                amp: int = 4):
    """q, k, v as CPU bf16 tensors [B, H, L, D] of small integers in [-amp, amp],
    drawn uniformly by ``numpy.random.default_rng([seed, b, h])`` (q, k, then v).
    With ``key_period`` p, key block j (64 tokens) repeats key block j mod p, so
    whole groups of key blocks are equal. Integers of this size are exact in
    bf16, and so are block means over 64 tokens and their dot products in fp64,
    whatever the order of summation."""
    import torch
    out = [np.empty((B, H, L, D), dtype=np.float32) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            rng = np.random.default_rng([seed, b, h])
            q, k, v = (rng.integers(-amp, amp + 1, size=(L, D)).astype(np.float32) for _ in range(3))
            if key_period:
                n = -(-L // CLUSTER)
                src = np.arange(n) % key_period
                k = np.concatenate([k[s * CLUSTER:(s + 1) * CLUSTER] for s in src])[:L]
            out[0][b, h], out[1][b, h], out[2][b, h] = q, k, v
    return tuple(torch.from_numpy(x).to(torch.bfloat16) for x in out)


def as_f64(t) -> np.ndarray:
    """The exact fp64 values of a rounded tensor (bf16 and fp32 widen exactly)."""
    return t.double().numpy()
