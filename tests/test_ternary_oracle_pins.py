"""Pins of the ternary oracle (oracle/ternary_oracle.py; PT2-LLM page, section
关键设计 item 2) against facts that do not come from the oracle itself:
a hand-worked ITF iteration in exact fractions (tests/golden/), the
least-squares optimality of the closed-form (alpha, mu) checked against
numpy's polynomial fit, the nearest-grid property by exhaustive search, the
monotone decrease of the fitting error over the alternating steps, the
dequantization bound, the layer's block-sum form against a dense matmul, and
the 2-bit word encoding.  Mutants planted here on the CPU show each pin bites.
"""
import json
import os

import numpy as np
import pytest

from oracle import ternary_oracle as TO

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def test_golden_itf_hand_case():
    g = GOLD["ternary_itf"]
    w = np.array([g["w"]], dtype=np.float32)
    r0 = TO.itf_ternarize(w, block=8, iters=0, store_fp16=False)
    assert r0["T"][0].tolist() == g["T0"]
    r1 = TO.itf_ternarize(w, block=8, iters=1, store_fp16=False)
    assert r1["alpha64"][0, 0] == pytest.approx(g["alpha1_num"] / g["alpha1_den"], rel=1e-15)
    assert r1["mu64"][0, 0] == pytest.approx(g["mu1_num"] / g["mu1_den"], rel=1e-15)
    r = TO.itf_ternarize(w, block=8)
    assert float(r["alpha"][0, 0]) == g["alpha_fp16"]
    assert float(r["mu"][0, 0]) == g["mu_fp16"]
    assert r["T"][0].tolist() == g["T"]
    words = TO.pack_words(np.array([g["packed_row16"]]))[0]
    assert list(words.astype("<u4").view(np.uint8)) == g["packed"]


def test_alpha_mu_are_least_squares_fit():
    """For fixed T the closed form is the least-squares line fit w ~ alpha t + mu:
    the (alpha, mu) of iteration k equal numpy's polynomial fit to the T that
    iteration k - 1 returned."""
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((6, 256)) * 0.02 + 0.003).astype(np.float32)
    Wg = W.astype(np.float64).reshape(6, 2, 128)
    for k in range(1, 5):
        prev = TO.itf_ternarize(W, iters=k - 1, store_fp16=False)
        cur = TO.itf_ternarize(W, iters=k, store_fp16=False)
        T = prev["T"].reshape(6, 2, 128).astype(np.float64)
        for n in range(6):
            for g in range(2):
                if np.ptp(T[n, g]) == 0:
                    continue
                slope, icpt = np.polyfit(T[n, g], Wg[n, g], 1)
                assert cur["alpha64"][n, g] == pytest.approx(slope, rel=1e-9)
                assert cur["mu64"][n, g] == pytest.approx(icpt, rel=1e-9, abs=1e-15)
    # mutant: the symmetric slope (no intercept) is a different number
    T = TO.itf_ternarize(W, iters=0, store_fp16=False)["T"].reshape(6, 2, 128)
    sym = (T[0, 0] * Wg[0, 0]).sum() / (T[0, 0] * T[0, 0]).sum()
    assert abs(sym - TO.itf_ternarize(W, iters=1, store_fp16=False)["alpha64"][0, 0]) > 1e-6


def test_t_is_nearest_grid_point():
    rng = np.random.default_rng(2)
    W = (rng.standard_normal((4, 128)) * 0.05).astype(np.float32)
    r = TO.itf_ternarize(W)
    a = r["alpha"].astype(np.float64)[:, 0]
    u = r["mu"].astype(np.float64)[:, 0]
    for n in range(4):
        for k in range(128):
            cands = np.array([-1.0, 0.0, 1.0])
            d = np.abs(W[n, k] - (a[n] * cands + u[n]))
            best = cands[d == d.min()]
            want = best[0] if len(best) == 1 else 0.0     # a tie between two codes: even (0)
            assert r["T"][n, k] == want


def test_itf_objective_never_increases():
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((8, 384)) * 0.02 + rng.uniform(-0.01, 0.01, (8, 1))).astype(np.float32)
    prev = None
    for it in range(0, 8):
        r = TO.itf_ternarize(W, iters=it, store_fp16=False)
        obj = TO.itf_objective(W, r["T"], r["alpha64"], r["mu64"])
        if prev is not None:
            assert np.all(obj <= prev * (1 + 1e-12) + 1e-18)
        prev = obj


def test_asymmetric_offset_matters():
    """A block row with a large common offset: alpha T + mu fits it far better
    than the symmetric alpha T (mutant: mu forced to 0)."""
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((1, 128)) * 0.01 + 0.05).astype(np.float32)
    r = TO.itf_ternarize(W, store_fp16=False)
    e_asym = TO.itf_objective(W, r["T"], r["alpha64"], r["mu64"])[0, 0]
    Z = W.astype(np.float64) / np.abs(W).mean()
    Ts = np.clip(np.rint(Z), -1, 1)
    a = (Ts * W).sum() / max((Ts * Ts).sum(), 1)
    e_sym = ((W - a * Ts) ** 2).sum()
    assert e_asym < 0.2 * e_sym


def test_constant_and_zero_blocks():
    W = np.zeros((2, 256), dtype=np.float32)
    W[1, :128] = 0.25
    r = TO.itf_ternarize(W)
    assert np.all(r["T"] == 0)
    assert float(r["alpha"][0, 0]) == 0.0 and float(r["mu"][0, 0]) == 0.0
    assert float(r["mu"][1, 0]) == 0.25
    np.testing.assert_array_equal(TO.dequant_ternary(r), W.astype(np.float64))


def test_dequant_bound_inside_the_grid():
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    r = TO.itf_ternarize(W)
    deq = TO.dequant_ternary(r)
    a = np.repeat(r["alpha"].astype(np.float64), 128, axis=1)
    u = np.repeat(r["mu"].astype(np.float64), 128, axis=1)
    inside = np.abs(W - u) <= 1.5 * a
    assert np.all(np.abs(W - deq)[inside] <= a[inside] / 2 * (1 + 1e-12))


def test_pack_words_bits():
    """The row-major 2-bit encoding, each word written out bit by bit: code
    16 w + 2 s of a row at bits 2 s of word w, code 16 w + 2 s + 1 at bits
    16 + 2 s, as c = t + 1."""
    rng = np.random.default_rng(6)
    N, K = 3, 64
    T = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    words = TO.pack_words(T)
    assert words.shape == (N, K // 16) and words.dtype == np.uint32
    for n in range(N):
        for w in range(K // 16):
            v = 0
            for i in range(16):
                v |= (int(T[n, 16 * w + i]) + 1) << (2 * (i // 2) + 16 * (i % 2))
            assert int(words[n, w]) == v
    # every code is recoverable from its two bits (the encoding is a bijection)
    back = np.empty_like(T)
    for i in range(16):
        back[:, i::16] = ((words >> (2 * (i // 2) + 16 * (i % 2))) & 3).astype(np.int8) - 1
    np.testing.assert_array_equal(back, T)
    with pytest.raises(ValueError):
        TO.pack_words(T[:, :8])


def test_layer_block_sum_equals_dense_matmul():
    rng = np.random.default_rng(7)
    X = rng.standard_normal((5, 384)).astype(np.float16)
    W = (rng.standard_normal((12, 384)) * 0.02).astype(np.float32)
    r = TO.itf_ternarize(W)
    Y = TO.ternary_linear(X, r)
    np.testing.assert_allclose(Y, X.astype(np.float64) @ TO.dequant_ternary(r).T,
                               rtol=1e-12, atol=1e-12)
    # mutant: the offset term dropped
    Ybad = X.astype(np.float64) @ (TO.dequant_ternary(r) - np.repeat(
        r["mu"].astype(np.float64), 128, axis=1)).T
    assert np.abs(Ybad - Y).max() > 1e-4
    # subsets
    np.testing.assert_allclose(TO.ternary_linear(X, r, rows=[1, 4], cols=[0, 7, 11]),
                               Y[[1, 4]][:, [0, 7, 11]], rtol=1e-12)
