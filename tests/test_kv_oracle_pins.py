"""Pins of the KV-cache oracle (oracle/kv_oracle.py) against facts that do not
come from the oracle itself: hand-derived values (tests/golden/hand_cases.json),
the exact invariance that the per-head transforms must preserve, brute force
in Python loops, closed forms of softmax attention and an independent
nearest-code search.  Wrong variants ("mutants", planted here on the CPU)
show that each pin would catch the mistake it is aimed at.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import kv_oracle as KV
import workloads as WL
from workloads import kv as WKV

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------------------
# golden hand cases
# ---------------------------------------------------------------------------
def test_golden_kv_quant_per_head():
    g = GOLD["kv_quant_per_head"]
    Z = np.array([g["Z"]])                       # [T=1, H=2, d=4]
    q, s, _ = KV.kv_quantize(Z, 1.0)
    assert s[0].tolist() == g["s"]
    assert q[0].tolist() == g["q"]
    # mutant: one scale per token across its heads
    s_tok = np.abs(Z).max() / 7.0
    q_bad = np.clip(np.rint(Z / s_tok), -8, 7)
    assert q_bad[0].tolist() != g["q"]


def test_golden_cache_layouts():
    g = GOLD["kv_cache_layout"]
    kb = KV.pack_k_cache(np.array([g["k_codes"]], dtype=np.int8))
    assert kb[0].tolist() == g["k_bytes"]
    vw = KV.pack_v_cache(np.array(g["v_codes"], dtype=np.int8).reshape(8, 1))
    assert vw.shape == (1, 1) and int(vw[0, 0]) == g["v_word"]
    assert KV.unpack_v_cache(vw).reshape(-1).tolist() == g["v_codes"]
    assert KV.unpack_k_cache(kb)[0].tolist() == g["k_codes"]


def test_golden_attend_gqa():
    g = GOLD["attend_gqa"]
    qt = np.log(3.0) * np.array([g["q_ln3_units"]], dtype=np.float64)   # [1, 4, 2]
    K = np.array([g["k"]], dtype=np.float64)                              # [1, 2, 2, 2]
    V = np.array([g["v"]], dtype=np.float64)
    out = KV.attend(qt, K, V, [2], 1.0)
    np.testing.assert_allclose(out[0], np.array(g["out"], dtype=np.float64), rtol=0, atol=1e-12)
    loop = KV.attend_loop(qt.tolist(), K.tolist(), V.tolist(), [2], 1.0)
    np.testing.assert_allclose(loop[0], np.array(g["out"], dtype=np.float64), atol=1e-12)


# ---------------------------------------------------------------------------
# invariance: the transforms cancel exactly without quantization
# ---------------------------------------------------------------------------
def _plain_attention(q, k_hist, v_hist, lengths, sm_scale, G):
    """softmax(q kᵀ) v written out once more with explicit per-head loops and
    an explicit inverse (not the oracle's code path)."""
    B, Hq, d = q.shape
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            L = lengths[b]
            if L == 0:
                continue
            K = k_hist[b][:L, h // G, :]
            V = v_hist[b][:L, h // G, :]
            s = sm_scale * (K @ q[b, h])
            w = np.exp(s - s.max())
            out[b, h] = w @ V / w.sum()
    return out


@pytest.mark.parametrize("shared", [True, False])
def test_transforms_cancel_without_quantization(shared):
    """softmax(q̃ k̃ᵀ)·ṽ·P_v⁻¹ = softmax(q kᵀ)·v with k̃ = k·P_h, ṽ = v·P_v,
    q̃ = q·P_h⁻ᵀ (FlatQuant page, 核心思想 and Transformer 集成)."""
    rng = np.random.default_rng(3)
    B, Hq, Hkv, d, S = 2, 4, 2, 16, 9
    G = Hq // Hkv
    lengths = [9, 5]
    if shared:
        Ph = WL.random_invertible(rng, d)
        Pv = WL.random_invertible(rng, d)
        Ph_h = [Ph] * Hkv
        Pv_h = [Pv] * Hkv
    else:
        Ph = np.stack([WL.random_invertible(rng, d) for _ in range(Hkv)])
        Pv = np.stack([WL.random_invertible(rng, d) for _ in range(Hkv)])
        Ph_h, Pv_h = list(Ph), list(Pv)
    q = _rand(rng, B, Hq, d)
    k_hist = [_rand(rng, S, Hkv, d) for _ in range(B)]
    v_hist = [_rand(rng, S, Hkv, d) for _ in range(B)]
    sm = 1.0 / math.sqrt(d)

    qt = KV.query_transform(q, Ph, Hkv)
    Kt = np.stack([KV.head_transform(k_hist[b], Ph).transpose(1, 0, 2) for b in range(B)])
    Vt = np.stack([KV.head_transform(v_hist[b], Pv).transpose(1, 0, 2) for b in range(B)])
    o_t = KV.attend(qt, Kt, Vt, lengths, sm)
    # undo P_v per query head's KV head with an explicit inverse
    o = np.empty_like(o_t)
    for h in range(Hq):
        o[:, h] = o_t[:, h] @ np.linalg.inv(Pv_h[h // G])
    ref = _plain_attention(q, k_hist, v_hist, lengths, sm, G)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-10)

    # mutants: q·P_h⁻¹ (transpose dropped) and P_hᵀ on the keys both break it
    q_bad = np.stack([q[:, h] @ np.linalg.inv(Ph_h[h // G]) for h in range(Hq)], axis=1)
    assert np.abs(KV.attend(q_bad, Kt, Vt, lengths, sm) - o_t).max() > 1e-3
    Kt_bad = np.stack([np.stack([k_hist[b][:, h] @ Ph_h[h].T for h in range(Hkv)])
                       for b in range(B)])
    assert np.abs(KV.attend(qt, Kt_bad, Vt, lengths, sm) - o_t).max() > 1e-3


def test_query_transform_solves_transposed_system():
    rng = np.random.default_rng(4)
    Ph = WL.random_invertible(rng, 8)
    q = _rand(rng, 3, 4, 8)
    qt = KV.query_transform(q, Ph, 2)
    np.testing.assert_allclose(qt @ Ph.T, q, atol=1e-12)
    np.testing.assert_allclose(qt, q @ np.linalg.inv(Ph).T, atol=1e-12)


def test_head_transform_is_per_head_product():
    rng = np.random.default_rng(5)
    X = _rand(rng, 4, 3, 8)
    P = np.stack([WL.random_invertible(rng, 8) for _ in range(3)])
    Z = KV.head_transform(X, P)
    for t in range(4):
        for h in range(3):
            want = [sum(X[t, h, i] * P[h, i, e] for i in range(8)) for e in range(8)]
            np.testing.assert_allclose(Z[t, h], want, atol=1e-13)


# ---------------------------------------------------------------------------
# quantizer and encodings
# ---------------------------------------------------------------------------
def test_kv_quantize_is_nearest_code():
    """Every code is the nearest point of s·{-8..7} to z (ties to even), found by
    exhaustive search over the 16 codes."""
    rng = np.random.default_rng(6)
    Z = _rand(rng, 5, 3, 16) * rng.uniform(0.1, 10, size=(5, 3, 1))
    q, s, _ = KV.kv_quantize(Z, 0.9)
    codes = np.arange(-8, 8)
    for t in range(5):
        for h in range(3):
            assert s[t, h] == 0.9 * np.abs(Z[t, h]).max() / 7.0
            for e in range(16):
                dist = np.abs(Z[t, h, e] - s[t, h] * codes)
                best = codes[dist == dist.min()]
                want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
                assert q[t, h, e] == want


def test_cache_encodings_round_trip():
    rng = np.random.default_rng(7)
    codes = rng.integers(-8, 8, size=(2, 3, 32, 16)).astype(np.int8)
    np.testing.assert_array_equal(KV.unpack_k_cache(KV.pack_k_cache(codes)), codes)
    np.testing.assert_array_equal(KV.unpack_v_cache(KV.pack_v_cache(codes)), codes)
    w = KV.pack_v_cache(codes)
    # bit arithmetic written out for one word
    b, h, blk, e = 1, 2, 3, 5
    want = 0
    for j in range(8):
        want |= (int(codes[b, h, 8 * blk + j, e]) & 0xF) << (4 * j)
    assert int(w[b, h, blk, e]) == want


def test_append_places_segments():
    """Segments land at their sequence and positions; other slots untouched."""
    rng = np.random.default_rng(8)
    B, H, S, d = 3, 2, 16, 8
    Ph = WL.random_invertible(rng, d)
    Pv = WL.random_invertible(rng, d)
    cache = KV.KvCache(B, H, S, d)
    cache.kq[:] = 5
    cache.ks[:] = 9.0
    k = _rand(rng, 5, H, d)
    v = _rand(rng, 5, H, d)
    seg_seq, seg_start, cu = [2, 0], [3, 15], [0, 4, 5]
    KV.kv_append(cache, k, v, seg_seq, seg_start, cu, Ph, Pv)
    qk, sk, _ = KV.kv_quantize(KV.head_transform(k, Ph))
    qv, sv, _ = KV.kv_quantize(KV.head_transform(v, Pv))
    for j in range(4):
        np.testing.assert_array_equal(cache.kq[2, :, 3 + j], qk[j])
        np.testing.assert_array_equal(cache.vq[2, :, 3 + j], qv[j])
        np.testing.assert_array_equal(cache.ks[2, :, 3 + j], sk[j].astype(np.float32))
    np.testing.assert_array_equal(cache.kq[0, :, 15], qk[4])
    np.testing.assert_array_equal(cache.vs[0, :, 15], sv[4].astype(np.float32))
    untouched = np.ones((B, S), dtype=bool)
    untouched[2, 3:7] = False
    untouched[0, 15] = False
    assert (cache.kq.transpose(0, 2, 1, 3)[untouched] == 5).all()
    assert (cache.ks.transpose(0, 2, 1)[untouched] == 9.0).all()


# ---------------------------------------------------------------------------
# attention: brute force and closed forms
# ---------------------------------------------------------------------------
def test_attend_matches_python_loops():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, d, S = 2, 6, 2, 5, 7
    qt = _rand(rng, B, Hq, d)
    K = _rand(rng, B, Hkv, S, d)
    V = _rand(rng, B, Hkv, S, d)
    lengths = [7, 3]
    a = KV.attend(qt, K, V, lengths, 0.37)
    b = KV.attend_loop(qt.tolist(), K.tolist(), V.tolist(), lengths, 0.37)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_attend_closed_forms():
    rng = np.random.default_rng(10)
    B, Hq, Hkv, d, S = 3, 4, 2, 6, 5
    qt = _rand(rng, B, Hq, d)
    K = _rand(rng, B, Hkv, S, d)
    V = _rand(rng, B, Hkv, S, d)
    K[2] = K[2, :, :1]            # sequence 2: all keys equal
    out = KV.attend(qt, K, V, [0, 1, 5], 0.5)
    assert (out[0] == 0).all()                                   # empty context
    for h in range(Hq):
        np.testing.assert_allclose(out[1, h], V[1, h // 2, 0], atol=1e-15)   # one token
        np.testing.assert_allclose(out[2, h], V[2, h // 2].mean(axis=0), atol=1e-14)


def test_attention_decode_end_to_end_small():
    """attention_decode on a cache filled by kv_append equals attend() on the
    dequantised cache with q̃ from the explicit inverse."""
    wl = WKV.get_kv("kv_tiny")
    st = WKV.make_kv_static(wl)
    cache = KV.KvCache(wl.batch, wl.heads_kv, wl.max_seq, wl.head_dim)
    for b in range(wl.batch):
        L = int(st["lengths"][b])
        k, v = WKV.make_history(wl, b, L, st["outliers"])
        KV.kv_append(cache, k, v, [b], [0], [0, L], st["P_h"], st["P_v"])
    sm = 1.0 / math.sqrt(wl.head_dim)
    out = KV.attention_decode(st["q"], cache, st["lengths"], st["P_h"], sm)
    qt = st["q"].astype(np.float64) @ np.linalg.inv(st["P_h"].astype(np.float64)).T
    kh, vh = KV.dequant_cache(cache)
    np.testing.assert_allclose(out, KV.attend(qt, kh, vh, st["lengths"], sm), atol=1e-10)
    # sanity: same order as the unquantized attention in the P_v basis (INT4
    # with random, untrained transforms and x8 key outliers leaves a large error)
    ref = np.zeros_like(out)
    for b in range(wl.batch):
        L = int(st["lengths"][b])
        k, v = WKV.make_history(wl, b, L, st["outliers"])
        kt = KV.head_transform(k, st["P_h"]).transpose(1, 0, 2)[None]
        vt = KV.head_transform(v, st["P_v"]).transpose(1, 0, 2)[None]
        ref[b] = KV.attend(qt[b:b + 1], kt, vt, [L], sm)[0]
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert rel < 0.5
