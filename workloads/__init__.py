"""Seeded synthetic inputs for the SVDQuant W4A4 linear layer.

This module only *generates* tensors (activations X, weights W, bias b) and
describes the layer shapes.  It holds no step of the quantization method:
no smoothing, no SVD, no quantizer, no GEMM.  Both the CPU oracle and the
GPU library consume exactly the bytes produced here (bf16 bit patterns as
``uint16`` arrays), so a parity test compares the two on identical inputs.

The shapes and value distributions stand in for the FLUX.1 layers the pages
measure (hidden size 3072; a fused QKV projection over 4096 image + 512
text tokens; an MLP with 4x expansion), with outlier channels in the
activations and a planted low-rank component in the weights (SVDQuant
walkthrough, devpress.csdn.net, Fig. 3/Fig. 4: outliers in both X and W;
quantization handbook, section on outliers: a few channels scaled by tens).
No dataset or trained checkpoint is used.

Recipe (every tensor from its own PCG64 stream spawned from one seed):
  * X ~ N(0, 1) (or GELU(N(0,1))), then selected channels multiplied by a
    factor (fixed list or drawn without replacement, factor fixed or
    uniform in [lo, hi]).
  * W ~ N(0, w_std^2) + planted_scale * sum_i u_i v_i^T with u_i, v_i
    independent random unit vectors.
  * bias ~ N(0, bias_std^2) when bias_std > 0.
  * every tensor is rounded to bf16 (via fp32, round-to-nearest-even).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

INT4 = "int4"
FP4 = "fp4"


@dataclass(frozen=True)
class LayerConfig:
    name: str
    M: int
    K: int
    N: int
    rank: int
    fmt: str                      # INT4 or FP4
    alpha: float = 0.5
    x_kind: str = "gauss"         # "gauss" | "gelu"
    outlier_channels: Optional[Sequence[int]] = None   # fixed channel list
    n_outlier_channels: int = 0   # else: this many drawn without replacement
    outlier_lo: float = 1.0
    outlier_hi: float = 1.0       # factor ~ U[lo, hi] (lo == hi: fixed)
    w_std: float = 1.0
    planted_rank: int = 0
    planted_scale: float = 10.0
    bias_std: float = 0.0
    seed: int = 0

    def with_(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    @property
    def has_bias(self) -> bool:
        return self.bias_std > 0.0


def _c2_like(name, M, K, N, rank, fmt, bias=True):
    return LayerConfig(name=name, M=M, K=K, N=N, rank=rank, fmt=fmt,
                       n_outlier_channels=8, outlier_lo=20.0, outlier_hi=50.0,
                       w_std=1.0 / np.sqrt(K), planted_rank=8, planted_scale=10.0,
                       bias_std=0.02 if bias else 0.0)


# The layer shapes and distributions of the five measured workloads.
C1 = LayerConfig(name="c1_tiny_256x1024x1024_int4", M=256, K=1024, N=1024, rank=16,
                 fmt=INT4, outlier_channels=(0, 1, 2, 3), outlier_lo=50.0,
                 outlier_hi=50.0, w_std=1.0 / 32.0, planted_rank=4,
                 planted_scale=10.0)
C2 = _c2_like("c2_qkv_4608x3072x9216_int4", 4608, 3072, 9216, 32, INT4, bias=True)
C3 = _c2_like("c3_fc1_4608x3072x12288_fp4", 4608, 3072, 12288, 32, FP4, bias=False)
C4_INT4 = LayerConfig(name="c4_fc2_4608x12288x3072_int4", M=4608, K=12288, N=3072,
                      rank=32, fmt=INT4, x_kind="gelu", n_outlier_channels=16,
                      outlier_lo=30.0, outlier_hi=30.0, w_std=1.0 / np.sqrt(12288),
                      planted_rank=8, planted_scale=10.0)
C4_FP4 = C4_INT4.with_(name="c4_fc2_4608x12288x3072_fp4", fmt=FP4)

# the fc1 shape in the INT4 format (the same inputs as C3)
C3_INT4 = C3.with_(name="c3_fc1_4608x3072x12288_int4", fmt=INT4)

CONFIGS = {c.name: c for c in (C1, C2, C3, C3_INT4, C4_INT4, C4_FP4)}


def sweep_configs():
    """Shape sweep: tokens x (K, N) x rank, INT4, generators of the QKV workload."""
    out = []
    for M in (256, 1024, 4096, 16384):
        for K, N in ((3072, 3072), (3072, 12288), (12288, 3072)):
            for r in (16, 32, 64):
                out.append(_c2_like(f"c5_M{M}_K{K}_N{N}_r{r}", M, K, N, r, INT4,
                                    bias=True))
    return out


# --------------------------------------------------------------- bf16 bytes
def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 (numpy, RNE) -> bf16 bit pattern (RNE on the fp32 bits)."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_float(b: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns as float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------- generators
def _streams(cfg: LayerConfig):
    ss = np.random.SeedSequence(cfg.seed)
    names = ("x", "outlier", "w", "u", "v", "bias")
    return {n: np.random.Generator(np.random.PCG64(s)) for n, s in zip(names, ss.spawn(len(names)))}


def _gelu(x: np.ndarray) -> np.ndarray:
    from scipy.special import erf
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def make_x(cfg: LayerConfig, M: Optional[int] = None) -> np.ndarray:
    """Activations as bf16 bits, shape (M, K).  ``M`` overrides cfg.M (the
    first M rows of a taller draw are NOT the same tensor; a different M is a
    different workload)."""
    M = cfg.M if M is None else M
    st = _streams(cfg)
    x = st["x"].standard_normal((M, cfg.K))
    if cfg.x_kind == "gelu":
        x = _gelu(x)
    if cfg.outlier_channels is not None:
        ch = np.asarray(cfg.outlier_channels, dtype=np.int64)
        fac = np.full(len(ch), cfg.outlier_lo)
    elif cfg.n_outlier_channels > 0:
        ch = st["outlier"].choice(cfg.K, size=cfg.n_outlier_channels, replace=False)
        fac = st["outlier"].uniform(cfg.outlier_lo, cfg.outlier_hi, size=len(ch))
    else:
        ch, fac = np.zeros(0, np.int64), np.zeros(0)
    x[:, ch] *= fac[None, :]
    return to_bf16_bits(x)


def make_w(cfg: LayerConfig) -> np.ndarray:
    """Weights in the K x N orientation (Y = X W), as bf16 bits."""
    st = _streams(cfg)
    w = st["w"].standard_normal((cfg.K, cfg.N)) * cfg.w_std
    if cfg.planted_rank > 0:
        u = st["u"].standard_normal((cfg.K, cfg.planted_rank))
        v = st["v"].standard_normal((cfg.N, cfg.planted_rank))
        u /= np.linalg.norm(u, axis=0, keepdims=True)
        v /= np.linalg.norm(v, axis=0, keepdims=True)
        w += cfg.planted_scale * (u @ v.T)
    return to_bf16_bits(w)


def make_bias(cfg: LayerConfig) -> Optional[np.ndarray]:
    if not cfg.has_bias:
        return None
    st = _streams(cfg)
    return to_bf16_bits(st["bias"].standard_normal(cfg.N) * cfg.bias_std)


def make_layer(cfg: LayerConfig, M: Optional[int] = None):
    """(X bits, W bits, bias bits or None) for one workload."""
    return make_x(cfg, M), make_w(cfg), make_bias(cfg)
