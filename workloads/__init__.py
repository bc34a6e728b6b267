"""Seeded synthetic inputs for the W4A4 linear layer.

This module only draws random numbers and shapes them; it holds none of the
quantization method's arithmetic (no transform, no merge, no quantizer).  Both
the CPU oracle and the HIP path take their inputs from here, so the two sides
see bit-identical X, P1, P2 and raw W.

The shapes stand in for LLaMA-family linear layers, the workloads the
quantization pages evaluate on (FlatQuant: Flatness Matters for LLM
Quantization, "Transformer 集成" lists the transformed projections; the
FRM-PTQ page evaluates the LLaMA family).  No dataset or trained weight is
used: activations are N(0,1) with the outlier structure the FlatQuant page
describes (a few channels with large magnitude and a "pivot" first token with
massive values, section "现有方法的不足"), weights are N(0, 0.02).

Transform factors P_i are random invertible matrices Q·diag(U[0.5, 2]) with Q
from the QR factorisation of an N(0,1) matrix: invertible but not orthogonal,
matching the FlatQuant page's relaxation of orthogonality to a general
invertible affine map (section "相关工作与启发", SpinQuant item).

Draw order for every workload, from ``numpy.random.default_rng(seed)``:
activation base (for the down projection: A then B), outlier channel indices,
P1, P2, raw W.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "make_activations", "make_factors",
           "make_inputs", "random_invertible", "make_calibration_activations"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    n1: int
    n2: int
    group_size: int          # == K means one scale per output channel
    asymmetric: bool
    x_kind: str              # "normal" or "silu_product"
    outlier_channels: Optional[tuple] = None   # explicit channel list
    outlier_frac: float = 0.0                  # else: fraction of K drawn at random
    outlier_scale: float = 50.0
    pivot_token_scale: float = 0.0             # 0: no pivot token
    w_std: float = 0.02
    seed: int = 0
    description: str = ""

    @property
    def groups(self) -> int:
        return self.K // self.group_size


def _wl(**kw) -> Workload:
    return Workload(**kw)


WORKLOADS = {
    w.name: w for w in [
        _wl(name="tiny", M=16, K=256, N=256, n1=16, n2=16, group_size=256,
            asymmetric=False, x_kind="normal", outlier_channels=(7, 100),
            pivot_token_scale=100.0,
            description="tiny W4A4 linear, 16x256 -> 256, P (16,16), per-channel sym"),
        _wl(name="qkv8b", M=2048, K=4096, N=6144, n1=64, n2=64, group_size=4096,
            asymmetric=False, x_kind="normal", outlier_frac=0.005,
            pivot_token_scale=100.0,
            description="LLaMA-3-8B fused QKV prefill, 2048x4096 -> 6144, P (64,64), "
                        "per-channel sym"),
        _wl(name="gateup8b", M=2048, K=4096, N=28672, n1=64, n2=64, group_size=128,
            asymmetric=True, x_kind="normal", outlier_frac=0.005,
            pivot_token_scale=100.0,
            description="LLaMA-3-8B gate+up prefill, 2048x4096 -> 28672, P (64,64), "
                        "group-128 asym"),
        _wl(name="down8b", M=2048, K=14336, N=4096, n1=112, n2=128, group_size=128,
            asymmetric=True, x_kind="silu_product",
            description="LLaMA-3-8B down prefill, 2048x14336 -> 4096, P (112,128), "
                        "group-128 asym, X = SiLU(A)*B"),
        _wl(name="gateup70b", M=4096, K=8192, N=57344, n1=64, n2=128, group_size=8192,
            asymmetric=False, x_kind="normal", outlier_frac=0.005,
            description="LLaMA-3-70B gate+up prefill, 4096x8192 -> 57344, P (64,128), "
                        "per-channel sym"),
    ] + [
        _wl(name=f"down70b_m{m}", M=m, K=28672, N=8192, n1=224, n2=128, group_size=128,
            asymmetric=True, x_kind="normal",
            description=f"LLaMA-3-70B down decode, {m}x28672 -> 8192, P (224,128), "
                        "group-128 asym")
        for m in (1, 8, 64)
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def random_invertible(rng: np.random.Generator, n: int) -> np.ndarray:
    """Q·diag(U[0.5,2]) in float64 with Q from QR of an N(0,1) matrix."""
    g = rng.standard_normal((n, n))
    q, _ = np.linalg.qr(g)
    d = rng.uniform(0.5, 2.0, size=n)
    return q * d[None, :]


def make_activations(wl: Workload, rng: np.random.Generator, M: Optional[int] = None):
    """Activation matrix X (fp16, [M, K]) and the outlier channel indices."""
    M = wl.M if M is None else M
    K = wl.K
    if wl.x_kind == "normal":
        x = rng.standard_normal((M, K), dtype=np.float32)
    elif wl.x_kind == "silu_product":
        a = rng.standard_normal((M, K), dtype=np.float32)
        b = rng.standard_normal((M, K), dtype=np.float32)
        x = (a / (1.0 + np.exp(-a))) * b
        del a, b
    else:
        raise ValueError(wl.x_kind)
    if wl.outlier_channels is not None:
        ch = np.asarray(wl.outlier_channels, dtype=np.int64)
    elif wl.outlier_frac > 0:
        ch = np.sort(rng.choice(K, int(round(wl.outlier_frac * K)), replace=False))
    else:
        ch = np.zeros(0, dtype=np.int64)
    if ch.size:
        x[:, ch] *= np.float32(wl.outlier_scale)
    if wl.pivot_token_scale and M > 0:
        x[0, :] *= np.float32(wl.pivot_token_scale)
    return x.astype(np.float16), ch


def make_factors(wl: Workload, rng: np.random.Generator):
    """P1 [n1,n1] and P2 [n2,n2] as float32 (drawn in float64, rounded once)."""
    p1 = random_invertible(rng, wl.n1).astype(np.float32)
    p2 = random_invertible(rng, wl.n2).astype(np.float32)
    return p1, p2


def make_inputs(name_or_wl, M: Optional[int] = None, with_weights: bool = True):
    """All inputs of one workload, in the fixed draw order.

    Returns a dict with X (fp16 [M,K]), P1, P2 (fp32), c (None: the workloads
    use no channel scaling), W (fp32 [N,K] raw, un-merged weights) and the
    Workload record.  ``M`` overrides the token count (the remaining draws
    then differ from the default-M draw, which is fine for parity since both
    sides share them).
    """
    wl = name_or_wl if isinstance(name_or_wl, Workload) else get(name_or_wl)
    rng = np.random.default_rng(wl.seed)
    X, ch = make_activations(wl, rng, M)
    P1, P2 = make_factors(wl, rng)
    W = None
    if with_weights:
        W = rng.standard_normal((wl.N, wl.K), dtype=np.float32)
        W *= np.float32(wl.w_std)
    return dict(wl=wl, X=X, outlier_channels=ch, P1=P1, P2=P2, c=None, W=W)


def make_channel_scale(K: int, seed: int = 1) -> np.ndarray:
    """A positive per-channel vector c (fp32) for tests of the diag(c) option."""
    rng = np.random.default_rng(seed)
    return rng.uniform(0.25, 4.0, size=K).astype(np.float32)


def make_calibration_activations(wl: Workload, M: int, outlier_channels, seed: int) -> np.ndarray:
    """A calibration batch for static activation steps: ``M`` tokens drawn
    like the workload's activations (same kind, the given outlier channels,
    no pivot token) from ``numpy.random.default_rng(seed)``; fp16 [M, K]."""
    cal = dataclasses.replace(wl, outlier_channels=tuple(int(c) for c in outlier_channels),
                              outlier_frac=0.0, pivot_token_scale=0.0, seed=seed)
    X, _ = make_activations(cal, np.random.default_rng(seed), M)
    return X
