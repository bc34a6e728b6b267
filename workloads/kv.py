"""Seeded synthetic inputs for the INT4 KV cache and decode attention.

Like the linear layer's generators, this module only draws random numbers
and shapes them; it holds none of the method's arithmetic.  The oracle and
the HIP path take their inputs from here.

Shapes stand in for the attention blocks of LLaMA-3 models (head size 128,
8 KV heads, 32 or 64 query heads), the model family the quantization pages
evaluate on; the FlatQuant page ("Transformer 集成") names the per-head key
and value transforms P_h and P_v.  No dataset or trained weight is used:
queries, keys and values are N(0,1), keys with a few outlier channels per head
(x8), the pattern that makes a transform worth applying before quantization;
the transforms are random invertible Q·diag(U[0.5,2]) matrices as for the
linear layer.  Context lengths are ragged, uniform in [S_max/2, S_max], with
the first sequence at exactly S_max.

Draw order from numpy.random.default_rng(seed): lengths, outlier channels,
P_h, P_v, queries; each sequence's cached history from
default_rng([seed, 1, b]) and the new decode tokens from default_rng([seed, 2]).
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import random_invertible

__all__ = ["KvWorkload", "KV_WORKLOADS", "get_kv", "make_kv_static", "make_history",
           "make_new_tokens", "make_tokens"]


@dataclasses.dataclass(frozen=True)
class KvWorkload:
    name: str
    batch: int            # sequences, one decode query each
    heads_q: int
    heads_kv: int
    head_dim: int
    max_seq: int          # cache capacity per sequence (multiple of 32)
    min_len: int          # ragged lengths uniform in [min_len, max_seq]
    outliers_per_head: int = 2
    outlier_scale: float = 8.0
    seed: int = 0
    description: str = ""

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv


KV_WORKLOADS = {w.name: w for w in [
    KvWorkload("kv_tiny", batch=3, heads_q=8, heads_kv=2, head_dim=128, max_seq=96,
               min_len=1, description="tiny decode attention, 3 sequences, GQA 4"),
    KvWorkload("attn8b", batch=64, heads_q=32, heads_kv=8, head_dim=128, max_seq=8192,
               min_len=4096,
               description="LLaMA-3-8B decode attention over an INT4 KV cache: 64 sequences, "
                           "contexts 4096..8192, 32 query / 8 KV heads of 128"),
    KvWorkload("attn70b", batch=64, heads_q=64, heads_kv=8, head_dim=128, max_seq=8192,
               min_len=4096,
               description="LLaMA-3-70B decode attention over an INT4 KV cache: 64 sequences, "
                           "contexts 4096..8192, 64 query / 8 KV heads of 128"),
]}


def get_kv(name: str) -> KvWorkload:
    return KV_WORKLOADS[name]


def make_kv_static(wl: KvWorkload):
    """lengths [B] int32, outlier channels [H_kv, n] int64, P_h and P_v
    (float32 [d, d], shared by the heads) and the decode queries
    q (fp16 [B, H_q, d])."""
    rng = np.random.default_rng(wl.seed)
    lengths = rng.integers(wl.min_len, wl.max_seq + 1, size=wl.batch).astype(np.int32)
    if wl.batch:
        lengths[0] = wl.max_seq
    och = np.stack([np.sort(rng.choice(wl.head_dim, wl.outliers_per_head, replace=False))
                    for _ in range(wl.heads_kv)])
    P_h = random_invertible(rng, wl.head_dim).astype(np.float32)
    P_v = random_invertible(rng, wl.head_dim).astype(np.float32)
    q = rng.standard_normal((wl.batch, wl.heads_q, wl.head_dim), dtype=np.float32)
    return dict(lengths=lengths, outliers=och, P_h=P_h, P_v=P_v, q=q.astype(np.float16))


def _kv_rows(wl: KvWorkload, rng, n, outliers):
    k = rng.standard_normal((n, wl.heads_kv, wl.head_dim), dtype=np.float32)
    v = rng.standard_normal((n, wl.heads_kv, wl.head_dim), dtype=np.float32)
    for h in range(wl.heads_kv):
        k[:, h, outliers[h]] *= np.float32(wl.outlier_scale)
    return k.astype(np.float16), v.astype(np.float16)


def make_history(wl: KvWorkload, b: int, length: int, outliers):
    """Post-RoPE keys and values of sequence b's first ``length`` tokens,
    fp16 [length, H_kv, d] each."""
    rng = np.random.default_rng([wl.seed, 1, b])
    return _kv_rows(wl, rng, length, outliers)


def make_new_tokens(wl: KvWorkload, outliers):
    """The decode step's new keys and values, one token per sequence,
    fp16 [B, H_kv, d] each."""
    rng = np.random.default_rng([wl.seed, 2])
    return _kv_rows(wl, rng, wl.batch, outliers)


def make_tokens(wl: KvWorkload, n: int, outliers, seed):
    """``n`` keys and values drawn like the workload's (for custom test
    layouts), fp16 [n, H_kv, d] each, from default_rng(seed)."""
    return _kv_rows(wl, np.random.default_rng(seed), n, outliers)
