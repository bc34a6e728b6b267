"""CPU oracle of the ternary-weight linear layer — TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the CPU-baseline leg of the benchmark
may import this module.  The product library never calls it, and it shares no
code with the HIP path.

PT2-LLM: Post-Training Ternarization for Large Language Models, section
"关键设计" item 2 (ATQ, the asymmetric ternary quantizer) and the overview:

* each row of a block of 128 columns (the quantization block size, section
  "损失函数 / 训练策略") is represented as alpha * T + mu with T in {-1, 0, 1};
* ITF alternates two closed-form steps about ten times: for fixed T the
  least-squares scale, alpha* = (m (W o T) 1 - (T 1)(W 1)) / (m (T o T) 1 - (T 1)^2),
  and for fixed (alpha, mu) the nearest grid point T* = argmin_t |Z - t| with
  Z = (W - mu) / alpha;
* mu starts at the row's mean.

The inference layer is weight-only (W1.58A16): Y = X · Ŵ^T with fp16
activations X and Ŵ[n, k] = alpha[n, g] T[n, k] + mu[n, g], g = k // 128.

Readings where the page is silent (restated with the design notes):
* mu* for fixed T is the least-squares intercept that goes with alpha*,
  mean(w) - alpha* mean(t) (the same fit the alpha* formula solves);
* the starting alpha is the mean absolute deviation of the block row from its
  mean; a block row with zero deviation is represented exactly by T = 0;
* when the alpha* denominator vanishes (T constant over the block row) alpha
  keeps its value;
* rounding is half to even; alpha and mu are stored as fp16 (one rounding from
  float64) and the final T is the nearest grid point of the stored grid;
* AGA (the activation-aware update of alpha and mu) and SSR (the column
  reordering) need calibration data and are not part of this layer; SSR's
  reordering is a column permutation, which leaves X W^T unchanged (pinned for
  the 4-bit layer).

Storage is the library's business, not the page's.  The oracle's plain form
is the codes T themselves, and, for a hand-checked encoding of the 2-bit
codes, `pack_words`: c = t + 1 in {0, 1, 2}, sixteen consecutive codes of a
row per little-endian 32-bit word, code 16 w + 2 s at bits 2 s of word w and
code 16 w + 2 s + 1 at bits 16 + 2 s (s = 0 .. 7).  The library's tiled
layout is checked through its own unpack entry point against T, alpha, mu.
"""
from __future__ import annotations

import numpy as np

from .w4a4_oracle import fp16_rne

__all__ = ["TERN_BLOCK", "itf_ternarize", "pack_words", "dequant_ternary", "ternary_linear",
           "itf_objective"]

TERN_BLOCK = 128


def _nearest_t(Z):
    return np.clip(np.rint(Z), -1, 1)


def itf_ternarize(Wt, block: int = TERN_BLOCK, iters: int = 10, store_fp16: bool = True):
    """ATQ with ITF for every (row, block).  Returns dict(T int8 [N,K],
    alpha, mu ([N,G]: fp16 if store_fp16, else float64 before storage), and
    the float64 alpha / mu of the last iteration)."""
    W = np.asarray(Wt, dtype=np.float64)
    N, K = W.shape
    if K % block:
        raise ValueError("K must be a multiple of the block size")
    G = K // block
    m = float(block)
    Wg = W.reshape(N, G, block)
    sW = Wg.sum(axis=2)
    mu = sW / m
    alpha = np.abs(Wg - mu[..., None]).mean(axis=2)
    live = alpha > 0
    safe = np.where(live, alpha, 1.0)
    T = np.where(live[..., None], _nearest_t((Wg - mu[..., None]) / safe[..., None]), 0.0)
    for _ in range(iters):
        sT = T.sum(axis=2)
        sTT = (T * T).sum(axis=2)
        sWT = (Wg * T).sum(axis=2)
        den = m * sTT - sT * sT
        ok = den > 0
        alpha = np.where(ok, (m * sWT - sT * sW) / np.where(ok, den, 1.0), alpha)
        mu = (sW - alpha * sT) / m
        live = alpha > 0
        safe = np.where(live, alpha, 1.0)
        T = np.where(live[..., None], _nearest_t((Wg - mu[..., None]) / safe[..., None]), 0.0)
    a64, m64 = alpha, mu
    if store_fp16:
        a16 = fp16_rne(alpha)
        u16 = fp16_rne(mu)
        a = a16.astype(np.float64)
        u = u16.astype(np.float64)
        live = a > 0
        safe = np.where(live, a, 1.0)
        T = np.where(live[..., None], _nearest_t((Wg - u[..., None]) / safe[..., None]), 0.0)
        alpha, mu = a16, u16
    return dict(T=T.reshape(N, K).astype(np.int8), alpha=alpha, mu=mu, alpha64=a64, mu64=m64,
                block=block)


def itf_objective(Wt, T, alpha, mu, block: int = TERN_BLOCK):
    """||W - (alpha T + mu)||_F^2 per (row, block)."""
    W = np.asarray(Wt, dtype=np.float64)
    N, K = W.shape
    G = K // block
    d = (W.reshape(N, G, block) - (np.asarray(alpha, np.float64)[..., None]
                                   * np.asarray(T, np.float64).reshape(N, G, block)
                                   + np.asarray(mu, np.float64)[..., None]))
    return (d * d).sum(axis=2)


def pack_words(T):
    """codes [..., K] in {-1, 0, 1} (K a multiple of 16) -> little-endian
    32-bit words [..., K/16], code 2s of a word's 16 at bits 2s, code 2s+1 at
    bits 16 + 2s."""
    c = np.asarray(T).astype(np.int64) + 1
    K = c.shape[-1]
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    cw = c.reshape(c.shape[:-1] + (K // 16, 16))
    word = np.zeros(cw.shape[:-1], dtype=np.int64)
    for s_ in range(8):
        word |= cw[..., 2 * s_] << (2 * s_)
        word |= cw[..., 2 * s_ + 1] << (16 + 2 * s_)
    return word.astype(np.uint32)


def dequant_ternary(tq):
    """Ŵ = alpha * T + mu, float64 [N, K]."""
    T = tq["T"].astype(np.float64)
    N, K = T.shape
    blk = tq["block"]
    a = np.repeat(np.asarray(tq["alpha"], np.float64), blk, axis=1)
    u = np.repeat(np.asarray(tq["mu"], np.float64), blk, axis=1)
    return a * T + u


def ternary_linear(X, tq, rows=None, cols=None):
    """Y64 = X · Ŵ^T written as the sum over blocks of alpha * (X_g · T_g^T)
    + mu * rowsum(X_g), float64; the same value as X @ dequant_ternary(tq).T."""
    X = np.asarray(X, dtype=np.float64)
    T = tq["T"]
    alpha = np.asarray(tq["alpha"], np.float64)
    mu = np.asarray(tq["mu"], np.float64)
    if rows is not None:
        X = X[rows]
    if cols is not None:
        T, alpha, mu = T[cols], alpha[cols], mu[cols]
    blk = tq["block"]
    G = T.shape[1] // blk
    Y = np.zeros((X.shape[0], T.shape[0]))
    for g in range(G):
        Xg = X[:, g * blk:(g + 1) * blk]
        Tg = T[:, g * blk:(g + 1) * blk].astype(np.float64)
        Y += (Xg @ Tg.T) * alpha[None, :, g] + Xg.sum(axis=1)[:, None] * mu[None, :, g]
    return Y
