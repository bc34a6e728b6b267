"""CPU oracle of the INT4 KV cache with per-head transforms — TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the CPU-baseline leg of the benchmark
may import this module.  The product library never calls it, and it shares no
code with the HIP path.

What the pages fix, and what is taken here:

* FlatQuant: Flatness Matters for LLM Quantization, "Transformer 集成": the
  self-attention block carries, besides the Kronecker-factored transforms of
  the projection inputs, a transform P_h for the key cache and a transform P_v
  for the value cache, each applied per head and not Kronecker-factored (a full
  d×d matrix, d the head size).
* FlatQuant page, "核心思想": a transform P on one operand of a product is
  undone by its inverse on the other operand.  For the attention scores
  q·kᵀ = (q·P_h⁻ᵀ)·(k·P_h)ᵀ, so the key cache holds Q(k·P_h) and the query is
  multiplied by P_h⁻ᵀ.  For the values, softmax(S)·(V·P_v) = (softmax(S)·V)·P_v,
  so the value cache holds Q(v·P_v) and P_v⁻¹ is merged offline into the
  output projection (the attention output here stays in the P_v basis).
* FPTQuant page, "核心贡献" and "实验结果": INT4 KV cache (the W4A4KV4
  setting).  The pages give no KV granularity; the reading taken is the
  activations' own quantizer (FRM-PTQ page, "初步介绍", symmetric, z = 0, with
  FlatQuant's clip α) applied to each head vector of each token:
  s = α·max_e |z_e| / 7, q = clamp(round_half_even(z / s), -8, 7).
* Attention itself (scaled dot-product with softmax, grouped query heads
  sharing a KV head) is the plain textbook definition; the pages take it as
  given.  Query head h reads KV head h // G with G = H_q / H_kv.

Cache encodings (this library's layout contract, restated in the tests):
key codes row-major per token, two codes per byte, low nibble = even channel
(the linear layer's activation packing); value codes in blocks of 8 tokens,
one 32-bit word per (block, channel) whose nibble j (bits 4j..4j+3) holds
token 8·block + j.  Scales are stored as float32 per (sequence, head, token).

Everything is float64 numpy; codes are computed with the unrounded float64
scale and dequantised with the stored float32 scale.
"""
from __future__ import annotations

import numpy as np

from .w4a4_oracle import act_scale, quantize_act, pack_nibbles, unpack_nibbles

__all__ = [
    "head_transform", "query_transform", "kv_quantize", "pack_k_cache",
    "unpack_k_cache", "pack_v_cache", "unpack_v_cache", "KvCache", "kv_append",
    "dequant_cache", "attend", "attend_loop", "attention_decode",
]


# ----------------------------------------------------------------------------
# Per-head transforms
# ----------------------------------------------------------------------------
def _per_head(P, H):
    P = np.asarray(P, dtype=np.float64)
    if P.ndim == 2:
        return np.broadcast_to(P, (H,) + P.shape)
    if P.shape[0] != H:
        raise ValueError("one matrix per head expected")
    return P


def head_transform(X, P):
    """Z[t, h] = X[t, h] · P_h for every token t and head h (float64).

    FlatQuant page, "Transformer 集成": P_h / P_v act on each head's vector.
    X is [T, H, d]; P is [d, d] (shared by all heads) or [H, d, d].
    """
    X = np.asarray(X, dtype=np.float64)
    T, H, d = X.shape
    Ph = _per_head(P, H)
    return np.einsum("thd,hde->the", X, Ph)


def query_transform(q, P_h, heads_kv: int):
    """q̃[t, h] = q[t, h] · P_{h//G}⁻ᵀ, i.e. the solution of q̃ · P_hᵀ = q.

    FlatQuant page, "核心思想": the inverse of the key-side transform goes on
    the other operand of the product, (q·P_h⁻ᵀ)·(k·P_h)ᵀ = q·kᵀ.  Solved with
    LAPACK (no explicit inverse).  q is [T, H_q, d].
    """
    q = np.asarray(q, dtype=np.float64)
    T, Hq, d = q.shape
    G = Hq // heads_kv
    Ph = _per_head(P_h, heads_kv)
    out = np.empty_like(q)
    for h in range(Hq):
        # q̃ P_hᵀ = q  <=>  P_h q̃ᵀ = qᵀ
        out[:, h, :] = np.linalg.solve(Ph[h // G], q[:, h, :].T).T
    return out


# ----------------------------------------------------------------------------
# Quantizer and cache encodings
# ----------------------------------------------------------------------------
def kv_quantize(Z, alpha: float = 1.0):
    """Per (token, head) symmetric INT4 codes of Z [T, H, d].

    The activations' quantizer (FRM-PTQ page "初步介绍"; FlatQuant page
    "额外可学习组件" for α) with one scale per head vector.  Returns
    (q int8 [T,H,d], s float64 [T,H], t float64 [T,H,d]).
    """
    Z = np.asarray(Z, dtype=np.float64)
    T, H, d = Z.shape
    rows = Z.reshape(T * H, d)
    s = act_scale(rows, alpha)
    q, t = quantize_act(rows, s)
    return q.reshape(T, H, d), s.reshape(T, H), t.reshape(T, H, d)


def pack_k_cache(codes):
    """Key codes [..., S, d] -> bytes [..., S, d/2], low nibble = even channel."""
    return pack_nibbles(codes)


def unpack_k_cache(b):
    return unpack_nibbles(b, signed=True)


def pack_v_cache(codes):
    """Value codes [..., S, d] (S a multiple of 8) -> uint32 [..., S/8, d];
    nibble j of word [blk, e] holds the code of token 8·blk + j, channel e."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    S, d = c.shape[-2], c.shape[-1]
    if S % 8:
        raise ValueError("S must be a multiple of 8")
    blk = c.reshape(c.shape[:-2] + (S // 8, 8, d))
    word = np.zeros(c.shape[:-2] + (S // 8, d), dtype=np.int64)
    for j in range(8):
        word |= blk[..., j, :] << (4 * j)
    return word.astype(np.uint32)


def unpack_v_cache(words):
    w = np.asarray(words, dtype=np.uint32).astype(np.int64)
    nb, d = w.shape[-2], w.shape[-1]
    out = np.empty(w.shape[:-2] + (nb, 8, d), dtype=np.int64)
    for j in range(8):
        out[..., j, :] = (w >> (4 * j)) & 0xF
    out = np.where(out >= 8, out - 16, out)
    return out.reshape(w.shape[:-2] + (nb * 8, d)).astype(np.int8)


class KvCache:
    """Codes and stored scales of one layer's key and value caches, unpacked.

    kq, vq: int8 [B, H, S, d]; ks, vs: float32 [B, H, S].
    """

    def __init__(self, B, H, S, d):
        self.B, self.H, self.S, self.d = B, H, S, d
        self.kq = np.zeros((B, H, S, d), dtype=np.int8)
        self.vq = np.zeros((B, H, S, d), dtype=np.int8)
        self.ks = np.zeros((B, H, S), dtype=np.float32)
        self.vs = np.zeros((B, H, S), dtype=np.float32)

    def packed(self):
        """(key bytes [B,H,S,d/2], key scales, value words [B,H,S/8,d], value scales)."""
        return pack_k_cache(self.kq), self.ks, pack_v_cache(self.vq), self.vs


def kv_append(cache: KvCache, k, v, seg_seq, seg_start, cu_tokens, P_h, P_v,
              alpha_k: float = 1.0, alpha_v: float = 1.0):
    """Write new tokens into the caches.

    Segment i holds tokens cu_tokens[i] .. cu_tokens[i+1]-1 of k / v
    ([T, H, d]); they go to sequence seg_seq[i] at positions seg_start[i],
    seg_start[i]+1, ...  Each token's head vectors are transformed
    (head_transform), quantized per head (kv_quantize) and stored with their
    float32 scales.  Returns dict(zk, zv, tk, tv, sk, sv) of the new tokens
    (float64) for near-tie checks.
    """
    zk = head_transform(k, P_h)
    zv = head_transform(v, P_v)
    qk, sk, tk = kv_quantize(zk, alpha_k)
    qv, sv, tv = kv_quantize(zv, alpha_v)
    for i in range(len(seg_seq)):
        b = int(seg_seq[i])
        p0 = int(seg_start[i])
        t0, t1 = int(cu_tokens[i]), int(cu_tokens[i + 1])
        for j, t in enumerate(range(t0, t1)):
            p = p0 + j
            cache.kq[b, :, p, :] = qk[t]
            cache.vq[b, :, p, :] = qv[t]
            cache.ks[b, :, p] = sk[t].astype(np.float32)
            cache.vs[b, :, p] = sv[t].astype(np.float32)
    return dict(zk=zk, zv=zv, tk=tk, tv=tv, sk=sk, sv=sv)


def dequant_cache(cache: KvCache, b=None):
    """k̂ = s_k · q_k and v̂ = s_v · q_v (float64), all sequences or one."""
    sl = slice(None) if b is None else slice(b, b + 1)
    kh = cache.kq[sl].astype(np.float64) * cache.ks[sl].astype(np.float64)[..., None]
    vh = cache.vq[sl].astype(np.float64) * cache.vs[sl].astype(np.float64)[..., None]
    return kh, vh


# ----------------------------------------------------------------------------
# Attention over the cache (decode: one query per sequence)
# ----------------------------------------------------------------------------
def attend(qt, Kh, Vh, lengths, sm_scale: float):
    """o[b, h] = softmax(sm_scale · qt[b,h] · K[b, h//G, :L]ᵀ) · V[b, h//G, :L].

    qt [B, H_q, d]; Kh, Vh [B, H_kv, S, d] (float values); lengths [B].  An
    empty context (L = 0) gives a zero output.  Softmax with the maximum
    subtracted (the same value in exact arithmetic).
    """
    qt = np.asarray(qt, dtype=np.float64)
    B, Hq, d = qt.shape
    Hkv = Kh.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    for b in range(B):
        L = int(lengths[b])
        if L == 0:
            continue
        for h in range(Hq):
            K = np.asarray(Kh[b, h // G, :L], dtype=np.float64)
            V = np.asarray(Vh[b, h // G, :L], dtype=np.float64)
            s = sm_scale * (K @ qt[b, h])
            p = np.exp(s - s.max())
            out[b, h] = (p @ V) / p.sum()
    return out


def attend_loop(qt, Kh, Vh, lengths, sm_scale: float):
    """attend() in Python loops with math.exp (tiny inputs only)."""
    import math
    B, Hq, d = len(qt), len(qt[0]), len(qt[0][0])
    Hkv = len(Kh[0])
    G = Hq // Hkv
    out = [[[0.0] * d for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        L = int(lengths[b])
        for h in range(Hq):
            hk = h // G
            if L == 0:
                continue
            s = []
            for t in range(L):
                acc = 0.0
                for e in range(d):
                    acc += float(qt[b][h][e]) * float(Kh[b][hk][t][e])
                s.append(sm_scale * acc)
            w = [math.exp(x) for x in s]
            tot = sum(w)
            for e in range(d):
                out[b][h][e] = sum(w[t] * float(Vh[b][hk][t][e]) for t in range(L)) / tot
    return np.array(out, dtype=np.float64)


def attention_decode(q, cache: KvCache, lengths, P_h, sm_scale: float, seqs=None):
    """Decode attention over the INT4 cache, output in the P_v basis.

    q [B, H_q, d] (post-RoPE queries, one per sequence).  q̃ = q·P_h⁻ᵀ, keys
    and values dequantised from the cache, then attend().  ``seqs`` restricts
    the work to a subset of sequences (rows of q given for those only).
    Returns float64 [len(seqs) or B, H_q, d].
    """
    qt = query_transform(q, P_h, cache.H)
    bs = range(cache.B) if seqs is None else seqs
    out = []
    for i, b in enumerate(bs):
        kh, vh = dequant_cache(cache, b)
        out.append(attend(qt[i:i + 1], kh, vh, [lengths[b]], sm_scale)[0])
    return np.array(out).reshape(len(out), q.shape[1], q.shape[2])
