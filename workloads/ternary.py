"""Seeded synthetic inputs for the ternary-weight (W1.58A16) linear layer.

Like the other generators, this module only draws random numbers and shapes
them; it holds none of the method's arithmetic (no ternarization, no
product).  The oracle and the HIP path take their inputs from here.

The shapes stand in for LLaMA-3-70B decode projections (the PT2-LLM page
ternarizes LLaMA-family models and runs them weight-only with fp16
activations).  No trained weight is used.  Weights are drawn so that the
asymmetric quantizer has something to fit: each output row has its own scale
w_std * U[0.5, 2], each (row, block of 128) its own offset N(0, 0.3 * row
scale) (blocks whose values do not centre on zero, the case the page's
per-row offset mu is for), and one entry in a thousand is an outlier eight
times larger.  Activations are a decode batch: N(0,1) with a few outlier
channels x50 for the gate/up input, SiLU(A)*B for the down input.

Draw order from numpy.random.default_rng(seed): activations (A then B for the
down input), outlier channels, then per weight-row chunk of 1024 rows, from
default_rng([seed, 7, chunk]): row scales, block offsets, the N(0,1) body,
the outlier mask.  Rows are drawn chunk by chunk so that a sample of rows can
be regenerated without the whole matrix.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["TernWorkload", "TERN_WORKLOADS", "get_tern", "make_tern_activations",
           "make_tern_weights", "make_tern_inputs"]

BLOCK = 128
ROW_CHUNK = 1024


@dataclasses.dataclass(frozen=True)
class TernWorkload:
    name: str
    M: int
    K: int
    N: int
    x_kind: str                 # "normal" (with outlier channels) or "silu_product"
    outlier_frac: float = 0.005
    outlier_scale: float = 50.0
    w_std: float = 0.02
    seed: int = 0
    description: str = ""


TERN_WORKLOADS = {w.name: w for w in (
    [TernWorkload(f"tern_down70b_m{m}", M=m, K=28672, N=8192, x_kind="silu_product",
                  description=f"LLaMA-3-70B down projection decode, {m}x28672 -> 8192, "
                              "ternary weights in blocks of 128, fp16 activations")
     for m in (1, 8, 64)]
    + [TernWorkload(f"tern_gateup70b_m{m}", M=m, K=8192, N=57344, x_kind="normal",
                    description=f"LLaMA-3-70B gate+up projection decode, {m}x8192 -> 57344, "
                                "ternary weights in blocks of 128, fp16 activations")
       for m in (1, 8, 64)]
    + [TernWorkload("tern_tiny", M=5, K=512, N=100, x_kind="normal",
                    description="tiny ternary layer, 5x512 -> 100")]
)}


def get_tern(name: str) -> TernWorkload:
    return TERN_WORKLOADS[name]


def make_tern_activations(wl: TernWorkload, rng: np.random.Generator, M: Optional[int] = None):
    """X fp16 [M, K]."""
    M = wl.M if M is None else M
    if wl.x_kind == "normal":
        x = rng.standard_normal((M, wl.K), dtype=np.float32)
    elif wl.x_kind == "silu_product":
        a = rng.standard_normal((M, wl.K), dtype=np.float32)
        b = rng.standard_normal((M, wl.K), dtype=np.float32)
        x = (a / (1.0 + np.exp(-a))) * b
    else:
        raise ValueError(wl.x_kind)
    if wl.x_kind == "normal" and wl.outlier_frac > 0:
        ch = np.sort(rng.choice(wl.K, max(1, int(round(wl.outlier_frac * wl.K))), replace=False))
        x[:, ch] *= np.float32(wl.outlier_scale)
    return x.astype(np.float16)


def _weight_chunk(wl: TernWorkload, c: int) -> np.ndarray:
    r0 = c * ROW_CHUNK
    n = min(ROW_CHUNK, wl.N - r0)
    G = wl.K // BLOCK
    rng = np.random.default_rng([wl.seed, 7, c])
    scale = (wl.w_std * rng.uniform(0.5, 2.0, size=n)).astype(np.float32)
    offset = rng.standard_normal((n, G), dtype=np.float32) * np.float32(0.3)
    w = rng.standard_normal((n, G, BLOCK), dtype=np.float32)
    w += offset[..., None]
    out = rng.random((n, G, BLOCK), dtype=np.float32) < 1e-3
    w[out] *= np.float32(8.0)
    w *= scale[:, None, None]
    return w.reshape(n, wl.K)


def make_tern_weights(wl: TernWorkload, rows=None) -> np.ndarray:
    """fp32 weights [N, K] (or only the listed rows, drawn identically)."""
    if wl.K % BLOCK:
        raise ValueError("K must be a multiple of 128")
    if rows is None:
        W = np.empty((wl.N, wl.K), dtype=np.float32)
        for c in range((wl.N + ROW_CHUNK - 1) // ROW_CHUNK):
            r0 = c * ROW_CHUNK
            W[r0:r0 + ROW_CHUNK] = _weight_chunk(wl, c)
        return W
    rows = np.asarray(rows, dtype=np.int64)
    W = np.empty((rows.size, wl.K), dtype=np.float32)
    cache = {}
    for i, r in enumerate(rows.tolist()):
        c = r // ROW_CHUNK
        if c not in cache:
            cache = {c: _weight_chunk(wl, c)}
        W[i] = cache[c][r - c * ROW_CHUNK]
    return W


def make_tern_inputs(name_or_wl, M: Optional[int] = None, with_weights: bool = True):
    """dict(wl, X fp16 [M, K], Wt fp32 [N, K] or None)."""
    wl = name_or_wl if isinstance(name_or_wl, TernWorkload) else get_tern(name_or_wl)
    rng = np.random.default_rng(wl.seed)
    X = make_tern_activations(wl, rng, M)
    return dict(wl=wl, X=X, Wt=make_tern_weights(wl) if with_weights else None)
