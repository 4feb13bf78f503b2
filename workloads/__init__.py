"""Seeded synthetic inputs for the Top-p block-sparse attention path.

This module only *makes inputs*: it holds none of the routing or attention
arithmetic, so both the fp64 CPU oracle (tests) and the GPU path can take their
inputs from here without sharing any of the method's computation.

Workloads stand in for the attention layers of video diffusion transformers
(Wan2.1/2.2-shaped, as named on the FVAttn summary page, "AI视频生成的阿喀琉斯之踵"
section and its experiments paragraph). Trained weights and real activations are
not available, so q, k and v are drawn as

    x[h, n, :] = noise[h, n, :] + alpha_h * phi(t, y, x)

where tokens are ordered (t, y, x) row-major (x fastest), noise ~ N(0, 1) and
phi is a 3-D sinusoidal position feature of dimension d (one interleaved
sin/cos block per axis).  alpha_h sets how concentrated a head's block
importance is: small alpha -> diffuse (keeps ~p of the blocks), large alpha ->
concentrated (keeps few).  Every draw is seeded:

* alpha[H] comes from ``numpy.random.default_rng(seed)``;
* the noise of tensor ``which`` (0=q, 1=k, 2=v) and head h comes from its own
  PCG64 stream ``default_rng([seed, which, h])``, so a single head can be
  regenerated alone (used to bound oracle work on the large workloads).

bf16 workloads are rounded to bfloat16 with round-to-nearest-even; both sides
receive exactly those rounded values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterable, Optional, Sequence

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "position_feature", "head_alphas",
    "make_head", "make_qkv", "bf16_round", "bf16_bits_to_f32", "f32_to_bf16_bits",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    H: int
    T: int
    Y: int
    X: int
    d: int
    block_q: int
    block_k: int
    ps: tuple            # top-p thresholds this workload runs at
    dtype: str           # "f32" or "bf16"
    alpha: tuple         # ("uniform", lo, hi) or ("loguniform", lo, hi)
    seed: int
    B: int = 1

    @property
    def N(self) -> int:
        return self.T * self.Y * self.X

    @property
    def nqb(self) -> int:
        return -(-self.N // self.block_q)

    @property
    def nkb(self) -> int:
        return -(-self.N // self.block_k)

    @property
    def rows(self) -> int:
        return self.B * self.H * self.nqb

    def describe(self) -> dict:
        return dict(name=self.name, B=self.B, H=self.H, N=self.N, T=self.T, Y=self.Y,
                    X=self.X, d=self.d, block_q=self.block_q, block_k=self.block_k,
                    p=list(self.ps), dtype=self.dtype, alpha=list(self.alpha), seed=self.seed)


# Shapes: latent frames x height x width of Wan2.1/2.2 video DiTs at 480p/720p.
WORKLOADS = {
    w.name: w for w in [
        # tiny fp32 case the oracle finishes in well under a second; also runs p=1.0
        Workload("tiny_f32_n1024", H=2, T=4, Y=16, X=16, d=64, block_q=64, block_k=64,
                 ps=(0.9, 1.0), dtype="f32", alpha=("uniform", 0.0, 3.0), seed=1001),
        # Wan2.1-1.3B-shaped layer (12 heads, 480p: 21 x 30 x 52 latent tokens)
        Workload("wan1p3b_n32760", H=12, T=21, Y=30, X=52, d=128, block_q=64, block_k=64,
                 ps=(0.9,), dtype="bf16", alpha=("uniform", 0.0, 3.0), seed=1002),
        # Wan2.1-14B-shaped layer (40 heads, 480p)
        Workload("wan14b_n32760", H=40, T=21, Y=30, X=52, d=128, block_q=64, block_k=64,
                 ps=(0.90, 0.95), dtype="bf16", alpha=("uniform", 0.0, 4.0), seed=1003),
        # 720p-shaped layer (40 heads, 21 x 45 x 80 latent tokens)
        Workload("wan14b_n75600", H=40, T=21, Y=45, X=80, d=128, block_q=64, block_k=64,
                 ps=(0.9,), dtype="bf16", alpha=("uniform", 0.0, 3.0), seed=1004),
        # the benchmark layer routed and attended with 32-token key blocks (the pages allow
        # blocks of 32 or 64 tokens)
        Workload("wan14b_n32760_bk32", H=40, T=21, Y=30, X=52, d=128, block_q=64, block_k=32,
                 ps=(0.9,), dtype="bf16", alpha=("uniform", 0.0, 4.0), seed=1003),
        # the 720p-shaped layer routed and attended with 32-token key blocks (2363 key blocks)
        Workload("wan14b_n75600_bk32", H=40, T=21, Y=45, X=80, d=128, block_q=64, block_k=32,
                 ps=(0.9,), dtype="bf16", alpha=("uniform", 0.0, 3.0), seed=1004),
        # load-skew stress: q-block 128, k-block 64, per-head alpha log-uniform
        Workload("skew_n75600_bq128", H=40, T=21, Y=45, X=80, d=128, block_q=128, block_k=64,
                 ps=(0.95,), dtype="bf16", alpha=("loguniform", 0.1, 6.0), seed=1005),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def _axis_feature(pos: np.ndarray, m: int) -> np.ndarray:
    """Interleaved [sin(pos*w_0), cos(pos*w_0), sin(pos*w_1), ...], w_i = 10000^(-2i/m)."""
    half = m // 2
    omega = 10000.0 ** (-2.0 * np.arange(half, dtype=np.float64) / m)
    ang = pos[:, None].astype(np.float64) * omega[None, :]
    out = np.empty((pos.shape[0], m), dtype=np.float64)
    out[:, 0::2] = np.sin(ang)
    out[:, 1::2] = np.cos(ang)
    return out


def position_feature(T: int, Y: int, X: int, d: int) -> np.ndarray:
    """phi[n, :] for tokens n = (t*Y + y)*X + x, shape [T*Y*X, d], float64.

    d is split into [d_t, d_y, d_x] = [d - 4*floor(d/6), 2*floor(d/6), 2*floor(d/6)]
    (44/42/42 for d=128, 24/20/20 for d=64); each part is one axis' sin/cos block.
    Unnormalised: every row has squared norm exactly d/2.
    """
    s = d // 6
    dt, dy, dx = d - 4 * s, 2 * s, 2 * s
    t = np.repeat(np.arange(T), Y * X)
    y = np.tile(np.repeat(np.arange(Y), X), T)
    x = np.tile(np.arange(X), T * Y)
    return np.concatenate([_axis_feature(t, dt), _axis_feature(y, dy), _axis_feature(x, dx)], axis=1)


def head_alphas(w: Workload) -> np.ndarray:
    """Per-head feature strength alpha[B*H] (drawn first from the workload seed)."""
    rng = np.random.default_rng(w.seed)
    kind, lo, hi = w.alpha
    n = w.B * w.H
    if kind == "uniform":
        return rng.uniform(lo, hi, size=n)
    if kind == "loguniform":
        return np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))
    raise ValueError(kind)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 -> bfloat16 with round-to-nearest-even; returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (RNE), returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


_PHI_CACHE: dict = {}


def _phi32(w: Workload) -> np.ndarray:
    key = (w.T, w.Y, w.X, w.d)
    if key not in _PHI_CACHE:
        _PHI_CACHE[key] = position_feature(w.T, w.Y, w.X, w.d).astype(np.float32)
    return _PHI_CACHE[key]


def make_head(w: Workload, which: int, h: int, alphas: Optional[np.ndarray] = None) -> np.ndarray:
    """One head of q (which=0), k (1) or v (2): float32 [N, d], already rounded to the
    workload dtype (bf16 values are exactly representable in the returned float32)."""
    if alphas is None:
        alphas = head_alphas(w)
    rng = np.random.default_rng([w.seed, which, h])
    x = rng.standard_normal((w.N, w.d), dtype=np.float32)
    x += np.float32(alphas[h]) * _phi32(w)
    if w.dtype == "bf16":
        x = bf16_round(x)
    return x


def make_qkv(w: Workload, heads: Optional[Sequence[int]] = None, which: Iterable[int] = (0, 1, 2)):
    """Tensors [B, H_sel, N, d] float32 (values already in the workload dtype) for the
    selected heads (all by default), in the order given by ``which``."""
    alphas = head_alphas(w)
    hs = list(range(w.B * w.H)) if heads is None else list(heads)
    out = []
    for wh in which:
        arr = np.empty((len(hs), w.N, w.d), dtype=np.float32)
        for i, h in enumerate(hs):
            arr[i] = make_head(w, wh, h, alphas)
        out.append(arr.reshape(1, len(hs), w.N, w.d) if heads is not None or w.B == 1
                   else arr.reshape(w.B, w.H, w.N, w.d))
    return tuple(out)


def small_case(H: int, N: int, d: int, block_q: int, block_k: int, seed: int,
               alpha: tuple = ("uniform", 0.0, 3.0), dtype: str = "bf16",
               grid: Optional[tuple] = None) -> Workload:
    """An ad-hoc workload (for parity tests at sizes the oracle finishes in seconds).
    ``grid`` = (T, Y, X) with T*Y*X == N; default is a single frame row (1, 1, N)."""
    T, Y, X = grid if grid is not None else (1, 1, N)
    assert T * Y * X == N
    return Workload(f"case_h{H}_n{N}_d{d}_bq{block_q}_bk{block_k}_s{seed}", H=H, T=T, Y=Y, X=X, d=d,
                    block_q=block_q, block_k=block_k, ps=(0.9,), dtype=dtype, alpha=alpha, seed=seed)
