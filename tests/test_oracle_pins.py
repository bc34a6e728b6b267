"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Brute force on tiny inputs (np.kron, explicit inverses, nearest-grid search,
exact rational rounding, Python-integer loops), hand-derived values from the
pages' formulas (tests/golden/hand_cases.json), invariants the pages state
(function preservation, column-permutation invariance) and closed forms.
Each check is also run against a deliberately wrong variant of the oracle step
("mutants", planted here on the CPU) to show that the pin would catch that
mistake.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import workloads as WL

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


# ---------------------------------------------------------------------------
# hand-derived golden values
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", ["act_quant_rne", "act_quant_clip"])
def test_golden_act_quant(case):
    g = GOLD[case]
    Z = np.array([g["Z"]])
    s = O.act_scale(Z, g["alpha"])
    assert s[0] == g["s"]
    q, _ = O.quantize_act(Z, s)
    assert q[0].tolist() == g["q"]


def test_golden_pack_bytes():
    g = GOLD["pack_bytes"]
    for pair, byte in zip(g["signed_pairs"], g["signed_bytes"]):
        assert O.pack_nibbles(np.array([pair]))[0, 0] == byte
        assert O.unpack_nibbles(np.array([[byte]], np.uint8), signed=True)[0].tolist() == pair
    for pair, byte in zip(g["unsigned_pairs"], g["unsigned_bytes"]):
        assert O.pack_nibbles(np.array([pair]))[0, 0] == byte
        assert O.unpack_nibbles(np.array([[byte]], np.uint8), signed=False)[0].tolist() == pair


def test_golden_weight_sym_row():
    g = GOLD["weight_sym_row"]
    v = np.array([g["v_fp32"]], dtype=np.float32)
    wq = O.quantize_weights(v, group_size=4, asymmetric=False)
    assert float(wq["s"][0, 0]) == g["s"]
    assert wq["codes"][0].tolist() == g["q"]
    assert float(wq["z"][0, 0]) == 0.0


def test_golden_weight_asym_group():
    g = GOLD["weight_asym_group"]
    v = np.array([g["v_fp32"]], dtype=np.float32)
    wq = O.quantize_weights(v, group_size=4, asymmetric=True)
    assert float(wq["s"][0, 0]) == g["s"]
    assert float(wq["z"][0, 0]) == g["z"]
    assert wq["codes"][0].tolist() == g["u"]


def test_golden_kron_factor_example():
    g = GOLD["kron_factor_example"]
    assert list(O.kron_factors(g["n"])) == g["factors"]
    # the factor pairs of the workloads are argmin pairs too (order as configured)
    for wl in WL.WORKLOADS.values():
        assert sorted((wl.n1, wl.n2)) == list(O.kron_factors(wl.K))


def test_golden_transform_2x2():
    g = GOLD["transform_2x2"]
    x = np.array([g["x"]])
    Z = O.kron_transform(x, np.array(g["P1"]), np.array(g["P2"]))
    assert Z[0].tolist() == g["z"]
    r = O.transform_quant(x, np.array(g["P1"]), np.array(g["P2"]))
    assert r["s_x"][0] == pytest.approx(g["s"], rel=1e-15)
    assert r["q"][0].tolist() == g["q"]
    assert r["packed"][0].tolist() == g["bytes"]


# ---------------------------------------------------------------------------
# Kronecker transform against brute force (np.kron)
# ---------------------------------------------------------------------------
def check_kron(fn, n1, n2, seed=0):
    rng = np.random.default_rng(seed)
    P1 = WL.random_invertible(rng, n1)
    P2 = WL.random_invertible(rng, n2)
    X = rng.standard_normal((5, n1 * n2))
    c = rng.uniform(0.5, 2, n1 * n2)
    want = (X * c) @ np.kron(P1, P2)
    got = fn(X, P1, P2, c)
    return np.allclose(got, want, rtol=0, atol=1e-12 * np.abs(want).max())


@pytest.mark.parametrize("n1,n2", [(2, 3), (3, 5), (4, 4), (16, 16), (7, 2)])
def test_kron_transform_bruteforce(n1, n2):
    assert check_kron(O.kron_transform, n1, n2)


def _mut_kron_p1_untransposed(X, P1, P2, c=None):
    M, K = X.shape
    Xb = (X * c).reshape(M, P1.shape[0], P2.shape[0])
    return (P1[None] @ Xb @ P2[None]).reshape(M, K)


def _mut_kron_colmajor(X, P1, P2, c=None):
    M, K = X.shape
    n1, n2 = P1.shape[0], P2.shape[0]
    Xb = (X * c).reshape(M, n2, n1).transpose(0, 2, 1)
    Z = P1.T[None] @ Xb @ P2[None]
    return Z.transpose(0, 2, 1).reshape(M, K)


def _mut_kron_no_c(X, P1, P2, c=None):
    return O.kron_transform(X, P1, P2, None)


@pytest.mark.parametrize("mut", [_mut_kron_p1_untransposed, _mut_kron_colmajor, _mut_kron_no_c])
def test_kron_pin_catches_mutants(mut):
    assert not check_kron(mut, 3, 5)


def test_merge_weights_bruteforce():
    rng = np.random.default_rng(3)
    for n1, n2 in [(2, 3), (4, 4), (8, 16)]:
        P1 = WL.random_invertible(rng, n1)
        P2 = WL.random_invertible(rng, n2)
        W = rng.standard_normal((6, n1 * n2))
        c = rng.uniform(0.5, 2, n1 * n2)
        want = (W / c) @ np.linalg.inv(np.kron(P1, P2)).T
        got = O.merge_weights(W, P1, P2, c, out_dtype=np.float64)
        assert np.allclose(got, want, rtol=0, atol=1e-12 * np.abs(want).max())


def test_function_preservation():
    """(x c P)(W̃)^T == x W^T without quantization (FlatQuant 核心思想)."""
    rng = np.random.default_rng(4)
    n1, n2 = 8, 16
    P1 = WL.random_invertible(rng, n1)
    P2 = WL.random_invertible(rng, n2)
    X = rng.standard_normal((7, n1 * n2))
    W = rng.standard_normal((9, n1 * n2))
    c = rng.uniform(0.5, 2, n1 * n2)
    Z = O.kron_transform(X, P1, P2, c)
    Wt = O.merge_weights(W, P1, P2, c, out_dtype=np.float64)
    assert np.allclose(Z @ Wt.T, X @ W.T, rtol=1e-11, atol=1e-11)


def test_orthogonal_factors_preserve_norm():
    rng = np.random.default_rng(5)
    Q1, _ = np.linalg.qr(rng.standard_normal((8, 8)))
    Q2, _ = np.linalg.qr(rng.standard_normal((4, 4)))
    X = rng.standard_normal((3, 32))
    Z = O.kron_transform(X, Q1, Q2)
    assert np.allclose(np.linalg.norm(Z, axis=1), np.linalg.norm(X, axis=1), rtol=1e-13)


def test_permutation_factors_are_reindexing():
    """P1, P2 permutation matrices: Z is x with its channels permuted, exactly."""
    rng = np.random.default_rng(6)
    n1, n2 = 4, 8
    p1 = rng.permutation(n1)
    p2 = rng.permutation(n2)
    P1 = np.eye(n1)[:, p1]
    P2 = np.eye(n2)[:, p2]
    X = rng.standard_normal((3, n1 * n2))
    Z = O.kron_transform(X, P1, P2)
    perm = (p1[:, None] * n2 + p2[None, :]).reshape(-1)
    assert np.array_equal(Z, X[:, perm])


def test_flop_and_storage_closed_forms():
    """FlatQuant Kronecker 分解: storage saved up to n/2, compute saved sqrt(n)/2."""
    for n in (256, 4096, 16384):
        r = int(np.sqrt(n))
        n1, n2 = O.kron_factors(n)
        assert (n1, n2) == (r, r)
        full_store, kron_store = n * n, n1 * n1 + n2 * n2
        assert Fraction(full_store, kron_store) == Fraction(n, 2)
        full_flops, kron_flops = 2 * n * n, 2 * n * (n1 + n2)   # per token
        assert Fraction(full_flops, kron_flops) == Fraction(r, 2)


# ---------------------------------------------------------------------------
# Quantizer against nearest-grid brute force and the RTN bound
# ---------------------------------------------------------------------------
def nearest_code_bruteforce(t, lo, hi):
    """Nearest integer of [lo, hi] to t by exhaustive search; ties -> even."""
    best = None
    for q in range(lo, hi + 1):
        d = abs(Fraction(t) - q)
        if best is None or d < best[0] or (d == best[0] and q % 2 == 0):
            best = (d, q)
    return best[1]


def test_act_quant_identity_transform_bruteforce():
    rng = np.random.default_rng(7)
    X = rng.standard_normal((4, 64)) * rng.uniform(0.1, 10, (4, 1))
    X[1, 5] = 0.0
    # plant exact ties: a value at 2.5 code units
    X[2, :] = 0.0
    X[2, 0] = 7.0
    X[2, 1] = 2.5
    X[2, 2] = -3.5
    r = O.transform_quant(X, np.eye(8), np.eye(8))
    for m in range(4):
        s = Fraction(float(np.abs(X[m]).max())) / 7
        for k in range(64):
            assert r["q"][m, k] == nearest_code_bruteforce(Fraction(float(X[m, k])) / s, -8, 7)
    assert r["q"][2, :3].tolist() == [7, 2, -4]


def test_act_quant_all_zero_token():
    r = O.transform_quant(np.zeros((2, 16)), np.eye(4), np.eye(4))
    assert np.all(r["q"] == 0) and np.all(r["s_x"] == 0) and np.all(r["packed"] == 0)


def test_act_rtn_bound():
    rng = np.random.default_rng(8)
    X = rng.standard_normal((16, 256)).astype(np.float16)
    P1 = WL.random_invertible(rng, 16)
    P2 = WL.random_invertible(rng, 16)
    r = O.transform_quant(X, P1, P2)
    err = np.abs(r["Z"] - r["q"] * r["s_x"][:, None])
    assert np.all(err <= r["s_x"][:, None] / 2 * (1 + 1e-12))


def test_weight_rtn_bound_and_ranges():
    rng = np.random.default_rng(9)
    W = (rng.standard_normal((32, 512)) * 0.02).astype(np.float32)
    for g, asym in [(512, False), (128, True), (128, False), (512, True)]:
        wq = O.quantize_weights(W, g, asym)
        s = wq["s"].astype(np.float64)
        deq = O.dequant_weights(wq)
        bound = np.repeat(s, g, axis=1) / 2
        # the stored fp16 scale differs from the exact range/levels by < 2^-11
        # relative, which can push the extreme element past the half step
        assert np.all(np.abs(deq - W) <= bound * (1 + 2 ** -9) + 1e-12)
        codes = wq["codes"]
        if asym:
            assert codes.min() >= 0 and codes.max() <= 15
            z = wq["z"].astype(np.float64)
            assert np.all(z == np.rint(z)) and z.min() >= 0 and z.max() <= 15
        else:
            assert codes.min() >= -8 and codes.max() <= 7


def test_weight_codes_nearest_bruteforce():
    rng = np.random.default_rng(10)
    W = (rng.standard_normal((3, 64)) * 0.02).astype(np.float32)
    for asym in (False, True):
        wq = O.quantize_weights(W, 32, asym)
        for n in range(3):
            for k in range(64):
                g = k // 32
                s = Fraction(float(wq["s"][n, g]))
                z = int(float(wq["z"][n, g]))
                t = Fraction(float(W[n, k])) / s + z
                lo, hi = (0, 15) if asym else (-8, 7)
                assert wq["codes"][n, k] == nearest_code_bruteforce(t, lo, hi)


def test_weight_zero_group():
    W = np.zeros((2, 8), dtype=np.float32)
    W[1, :4] = 0.5
    for asym in (False, True):
        wq = O.quantize_weights(W, 4, asym)
        assert float(wq["s"][0, 0]) == 0.0 and np.all(wq["codes"][0] == 0)
        assert float(wq["s"][1, 1]) == 0.0 and np.all(wq["codes"][1, 4:] == 0)
        assert np.all(O.dequant_weights(wq)[1, :4] == pytest.approx(0.5, rel=1e-3))


def test_asym_all_positive_group_has_zero_point_zero():
    W = np.linspace(0.01, 0.3, 8, dtype=np.float32)[None, :]
    wq = O.quantize_weights(W, 8, True)
    assert float(wq["z"][0, 0]) == 0.0 and wq["codes"][0, -1] == 15
    assert wq["z"].view(np.uint16)[0, 0] == 0          # the integer 0, not -0.0


# ---------------------------------------------------------------------------
# fp16 rounding of scales against exact rational rounding on the fp16 grid
# ---------------------------------------------------------------------------
_F16 = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)


def fp16_rne_exact(x: float) -> float:
    fx = Fraction(x)
    i = int(np.searchsorted(_F16, x))
    cands = [j for j in (i - 1, i) if 0 <= j < len(_F16)]
    best = None
    for j in cands:
        d = abs(Fraction(float(_F16[j])) - fx)
        if best is None or d < best[0] or (d == best[0] and j % 2 == 0):
            best = (d, j)
    return float(_F16[best[1]])


def test_fp16_rne_against_exact_rounding():
    rng = np.random.default_rng(11)
    xs = list(rng.uniform(1e-5, 60000, 2000)) + list(rng.uniform(1e-3, 0.1, 2000))
    # values next to fp16 midpoints, closer than a float32 ulp: a conversion
    # through float32 would round these twice and get some wrong
    for j in range(1, 2000, 7):
        mid = (_F16[j] + _F16[j + 1]) / 2
        for d in (-1, 1):
            xs.append(float(np.nextafter(mid, mid + d)))
            xs.append(mid * (1 + d * 2 ** -30))
        xs.append(mid)
    for x in xs:
        assert float(O.fp16_rne(x)) == fp16_rne_exact(x), x


# ---------------------------------------------------------------------------
# exact integer GEMM and epilogue
# ---------------------------------------------------------------------------
def _tiny_codes(seed=12, M=3, N=4, K=16, g=8, asym=True):
    rng = np.random.default_rng(seed)
    qx = rng.integers(-8, 8, (M, K)).astype(np.int8)
    if asym:
        wc = rng.integers(0, 16, (N, K)).astype(np.int8)
        z = rng.integers(0, 16, (N, K // g)).astype(np.float16)
    else:
        wc = rng.integers(-8, 8, (N, K)).astype(np.int8)
        z = np.zeros((N, K // g), np.float16)
    return qx, wc, z


@pytest.mark.parametrize("asym", [False, True])
def test_int_gemm_paths_agree(asym):
    qx, wc, z = _tiny_codes(asym=asym)
    D_loop = O.int_gemm_loop(qx, wc, z, 8)
    assert np.array_equal(O.int_gemm(qx, wc, z, 8, exact_fp64=True), D_loop)
    assert np.array_equal(O.int_gemm(qx, wc, z, 8, exact_fp64=False), D_loop)


def test_int_gemm_extreme_magnitude_exact():
    K = 28672
    qx = np.full((1, K), -8, np.int8)
    wc = np.full((1, K), 0, np.int8)
    z = np.full((1, K // 128), 15, np.float16)
    D = O.int_gemm(qx, wc, z, 128)
    assert np.all(D == 128 * 8 * 15)
    Dk = O.int_gemm(qx, wc, np.full((1, 1), 15, np.float16), K)
    assert Dk[0, 0, 0] == K * 8 * 15 == 3440640


def test_int_gemm_column_permutation_invariance():
    """PT2-LLM 关键设计 1: joint column permutation keeps X' W'^T = X W^T."""
    rng = np.random.default_rng(13)
    qx = rng.integers(-8, 8, (5, 64)).astype(np.int8)
    wc = rng.integers(-8, 8, (6, 64)).astype(np.int8)
    z = np.zeros((6, 1), np.float16)
    perm = rng.permutation(64)
    assert np.array_equal(O.int_gemm(qx, wc, z, 64), O.int_gemm(qx[:, perm], wc[:, perm], z, 64))


def test_zero_point_identity():
    qx, wc, z = _tiny_codes(seed=14)
    D = O.int_gemm(qx, wc, z, 8)
    raw = O.int_gemm(qx, wc, np.zeros_like(z), 8)
    qsum = qx.astype(np.int64).reshape(3, 2, 8).sum(axis=2)            # [M, G]
    corr = qsum[:, None, :] * z.astype(np.int64)[None, :, :]
    assert np.array_equal(D, raw - corr)


def _mut_gemm_drop_z(qx, wc, z, g):
    return O.int_gemm(qx, wc, np.zeros_like(z), g)


def test_gemm_pin_catches_dropped_zero_point():
    qx, wc, z = _tiny_codes(seed=15)
    assert not np.array_equal(_mut_gemm_drop_z(qx, wc, z, 8), O.int_gemm_loop(qx, wc, z, 8))


@pytest.mark.parametrize("g,asym", [(64, False), (16, True), (64, True)])
def test_epilogue_equals_dequantized_matmul(g, asym):
    """s_x·Σ_g s_w·D == (s_x q_x)(s_w (u - z))^T: integer-then-scale equals
    the dequantize-then-multiply simulation the pages evaluate with."""
    rng = np.random.default_rng(16)
    X = rng.standard_normal((6, 64)).astype(np.float16)
    P1 = WL.random_invertible(rng, 8)
    P2 = WL.random_invertible(rng, 8)
    W = (rng.standard_normal((5, 64)) * 0.02).astype(np.float32)
    wq = O.quantize_weights(O.merge_weights(W, P1, P2), g, asym)
    out = O.linear(X, P1, P2, wq)
    sim = O.dequant_act(out["act"]["q"], out["act"]["s_x"]) @ O.dequant_weights(wq).T
    assert np.allclose(out["Y64"], sim, rtol=1e-12, atol=1e-12 * np.abs(sim).max())
    # and the quantized layer approximates the float layer X W^T
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.linalg.norm(out["Y64"] - ref) < 0.6 * np.linalg.norm(ref)


@pytest.mark.parametrize("g,asym", [(8, True), (16, False), (32, True)])
def test_epilogue_by_group_matches_brute_force(g, asym):
    """The group-by-group form (chunked over channels, a subset of channels)
    gives the dequantize-then-multiply product and, for the magnitude of the
    summed terms, s_x·Σ_g s_w·|D| with D from the pure-Python triple loop."""
    rng = np.random.default_rng(17 + g)
    M, N, K = 5, 7, 32
    qx = rng.integers(-8, 8, (M, K)).astype(np.int8)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    wq = O.quantize_weights(W, g, asym)
    sx = rng.uniform(0.1, 2, M).astype(np.float32)
    cols = np.array([6, 0, 3, 4])
    Y, A = O.epilogue_by_group(qx, wq, sx, cols=cols, chunk=3)
    sim = O.dequant_act(qx, sx) @ O.dequant_weights(wq)[cols].T
    assert np.allclose(Y, sim, rtol=1e-13, atol=1e-13 * np.abs(sim).max())
    D = O.int_gemm_loop(qx, wq["codes"][cols], wq["z"][cols], g)
    absum = np.zeros((M, len(cols)))
    for m in range(M):
        for j in range(len(cols)):
            absum[m, j] = float(sx[m]) * sum(float(wq["s"][cols[j], h]) * abs(int(D[m, j, h]))
                                              for h in range(K // g))
    assert np.allclose(A, absum, rtol=1e-13, atol=0)
    if asym:
        # mutant: a dropped zero point changes the product
        wq0 = dict(wq, z=np.zeros_like(wq["z"]))
        Y0, _ = O.epilogue_by_group(qx, wq0, sx, cols=cols)
        assert not np.allclose(Y0, sim, rtol=1e-6)


def test_linear_rows_cols_subset_consistent():
    inp = WL.make_inputs("tiny")
    Wt = O.merge_weights(inp["W"], inp["P1"], inp["P2"])
    wq = O.quantize_weights(Wt, 256, False)
    full = O.linear(inp["X"], inp["P1"], inp["P2"], wq)
    rows, cols = np.array([0, 3, 15]), np.array([1, 100, 255])
    sub = O.linear(inp["X"], inp["P1"], inp["P2"], wq, rows=rows, cols=cols)
    assert np.array_equal(sub["Y64"], full["Y64"][np.ix_(rows, cols)])


# ---------------------------------------------------------------------------
# static activation quantization (steps fixed offline) and step migration
# ---------------------------------------------------------------------------
def test_golden_act_static_tensor():
    g = GOLD["act_static_tensor"]
    q, _, s_x = O.quantize_act_static(np.array([g["Z"]]), [g["step"]], per_channel=False)
    assert q[0].tolist() == g["q"] and s_x[0] == g["s_x"]


def test_golden_act_static_channel():
    g = GOLD["act_static_channel"]
    q, _, s_x = O.quantize_act_static(np.array([g["Z"]]), g["steps"], per_channel=True)
    assert q[0].tolist() == g["q"] and s_x[0] == g["s_x"]


def test_golden_qsm_migration():
    g = GOLD["qsm_migration"]
    Wm = O.migrate_steps(np.array([g["W"]], dtype=np.float32), g["steps"])
    assert Wm[0].tolist() == g["W_migrated"]
    q = np.array(g["q"])
    # integer codes against the migrated row, as a Python-integer/rational sum
    y = sum(Fraction(int(a)) * Fraction(float(b)) for a, b in zip(q, Wm[0]))
    assert y == Fraction(g["y"])


def test_static_tensor_step_equal_to_dynamic_scale_matches_dynamic():
    """A per-tensor step equal to the token's own dynamic scale reproduces the
    dynamic codes: static quantization differs only in where the step comes from."""
    rng = np.random.default_rng(40)
    Z = rng.standard_normal((7, 96)) * rng.uniform(0.1, 30, (7, 1))
    for alpha in (1.0, 0.8):
        s = O.act_scale(Z, alpha)
        qd, _ = O.quantize_act(Z, s)
        for m in range(Z.shape[0]):
            qs, _, sx = O.quantize_act_static(Z[m:m + 1], [s[m]], per_channel=False)
            assert np.array_equal(qs[0], qd[m]) and sx[0] == s[m]


def _static_nearest_bruteforce(Z, steps):
    """Nearest point of the clipped grid {step·q : q in [-8, 7]}, ties to the
    even code, found by scanning all 16 codes with exact rationals."""
    out = np.zeros(Z.shape, dtype=np.int64)
    for idx, z in np.ndenumerate(Z):
        st = Fraction(float(steps[idx[1]]))
        zf = Fraction(float(z))
        best = min(range(-8, 8), key=lambda c: (abs(zf - st * c), c % 2))
        out[idx] = best
    return out


def _mut_static_divide_by_alpha_scale(Z, steps, per_channel):
    # plausible slip: re-deriving the scale from the data instead of the fixed step
    q, _ = O.quantize_act(Z, O.act_scale(Z, 1.0))
    return q, None, np.ones(Z.shape[0])


def _mut_static_channel_steps_transposed(Z, steps, per_channel):
    st = np.asarray(steps)[::-1]
    return O.quantize_act_static(Z, st, per_channel)


@pytest.mark.parametrize("mut", [None, _mut_static_divide_by_alpha_scale,
                                 _mut_static_channel_steps_transposed])
def test_static_channel_codes_bruteforce(mut):
    rng = np.random.default_rng(41)
    Z = rng.standard_normal((5, 12)) * 6
    Z[0, :4] = [0.5, 1.5, -2.5, 3.5]           # ties on a unit step
    steps = np.concatenate([[1.0, 1.0, 1.0, 1.0], rng.uniform(0.2, 3.0, 8)])
    want = _static_nearest_bruteforce(Z, steps)
    fn = O.quantize_act_static if mut is None else mut
    q = fn(Z, steps, True)[0]
    assert np.array_equal(q, want) == (mut is None)


def test_static_rtn_bound():
    """Inside the clip range the static code is within half a step of z."""
    rng = np.random.default_rng(42)
    Z = rng.standard_normal((9, 64))
    steps = rng.uniform(0.3, 1.0, 64)
    q, t, _ = O.quantize_act_static(Z, steps, True)
    inside = np.abs(t) <= 7
    err = np.abs(Z - q * steps[None, :])
    assert np.all(err[inside] <= steps[None, :].repeat(9, 0)[inside] / 2 + 1e-15)
    assert np.all(q[~inside] == np.where(t[~inside] > 0, 7, -8))


def test_qsm_layer_equals_step_dequantized_matmul():
    """With per-channel steps migrated into the weights and weight codes that
    are exact (power-of-two channel scales), the static layer equals
    (q·step) W^T exactly and stays within sum_k |W[n,k]|·step_k/2 of Z W^T."""
    rng = np.random.default_rng(43)
    n1, n2, N = 4, 8, 6
    K = n1 * n2
    steps = 2.0 ** rng.integers(-3, 2, K)
    ints = rng.integers(-7, 8, (N, K))
    ints[:, 0] = 7                               # each row reaches |code| 7
    cn = 2.0 ** rng.integers(-6, -2, N)
    W = (cn[:, None] * ints / steps[None, :]).astype(np.float32)   # exact in fp32
    Wm = O.migrate_steps(W, steps)
    assert np.array_equal(Wm.astype(np.float64), cn[:, None] * ints)
    wq = O.quantize_weights(Wm, K, False)
    assert np.array_equal(wq["codes"], ints)
    P1, P2 = np.eye(n1), np.eye(n2)
    X = (rng.uniform(-7.0, 7.0, (5, K)) * steps[None, :]).astype(np.float16)
    X[0, :3] = [100, -100, 0]                    # clipped entries in row 0
    out = O.linear_static(X, P1, P2, wq, steps, per_channel=True)
    deq = out["act"]["q"] * steps[None, :]
    assert np.array_equal(out["Y64"], deq @ W.astype(np.float64).T)
    Zx = X.astype(np.float64)
    bound = (np.abs(W.astype(np.float64)) @ steps) / 2
    t = Zx / steps[None, :]
    rows_inside = np.all((t <= 7.5) & (t >= -8.5), axis=1)
    err = np.abs(out["Y64"] - Zx @ W.astype(np.float64).T)
    assert rows_inside.sum() == 4 and not rows_inside[0]
    assert np.all(err[rows_inside] <= bound[None, :] + 1e-12)


def _mut_migrate_divides(Wt, steps, out_dtype=np.float32):
    return (np.asarray(Wt, np.float64) / np.asarray(steps).reshape(1, -1)).astype(out_dtype)


def test_qsm_pin_catches_dividing_migration():
    g = GOLD["qsm_migration"]
    Wm = _mut_migrate_divides(np.array([g["W"]], dtype=np.float32), g["steps"])
    assert Wm[0].tolist() != g["W_migrated"]


def test_static_tensor_layer_transform_and_epilogue():
    """Per-tensor static layer: s_x is the step on every token, and the layer
    equals the dequantize-then-multiply simulation (step·q)(s_w·codes)^T."""
    rng = np.random.default_rng(44)
    X = rng.standard_normal((6, 64)).astype(np.float16)
    P1 = WL.random_invertible(rng, 8)
    P2 = WL.random_invertible(rng, 8)
    W = (rng.standard_normal((5, 64)) * 0.02).astype(np.float32)
    wq = O.quantize_weights(O.merge_weights(W, P1, P2), 64, False)
    step = 0.37
    out = O.linear_static(X, P1, P2, wq, [step], per_channel=False)
    assert np.all(out["act"]["s_x"] == step)
    sim = O.dequant_act(out["act"]["q"], out["act"]["s_x"]) @ O.dequant_weights(wq).T
    assert np.allclose(out["Y64"], sim, rtol=1e-12, atol=1e-12 * np.abs(sim).max())


def test_static_rejects_wrong_step_count():
    with pytest.raises(ValueError):
        O.quantize_act_static(np.zeros((2, 4)), [1.0, 2.0], per_channel=True)
    with pytest.raises(ValueError):
        O.quantize_act_static(np.zeros((2, 4)), [1.0, 2.0], per_channel=False)


def test_calibrate_steps_hand_case():
    """Zc = [[1, -14, 0], [-7, 3.5, 0]]: range 14 -> step 2 for the tensor;
    per channel 7/7 = 1, 14/7 = 2 and 1 for the all-zero channel."""
    Zc = np.array([[1.0, -14.0, 0.0], [-7.0, 3.5, 0.0]])
    assert O.calibrate_steps(Zc, False).tolist() == [2.0]
    assert O.calibrate_steps(Zc, True).tolist() == [1.0, 2.0, 1.0]
    assert O.calibrate_steps(Zc, False, ratio=0.5).tolist() == [1.0]


def test_calibrated_steps_cover_their_own_batch():
    """Steps calibrated (ratio 1) on a batch quantize that batch without
    clipping: every |t| <= 7, so no code reaches -8, and every channel's (or
    the tensor's) largest magnitude maps to code +-7."""
    rng = np.random.default_rng(45)
    Z = rng.standard_normal((20, 48)) * rng.uniform(0.1, 10, 48)[None, :]
    for pc in (False, True):
        st = O.calibrate_steps(Z, pc)
        q, t, _ = O.quantize_act_static(Z, st.astype(np.float64), pc)
        assert np.all(np.abs(t) <= 7 * (1 + 1e-6)) and not (q == -8).any()
        if pc:
            assert np.all(np.abs(q).max(axis=0) == 7)
        else:
            assert np.abs(q).max() == 7


# ---------------------------------------------------------------------------
# 3-bit codes (W3A3, FRM-PTQ page)
# ---------------------------------------------------------------------------
def test_golden_act_quant_3bit():
    g = GOLD["act_quant_3bit"]
    Z = np.array([g["Z"]])
    s = O.act_scale(Z, 1.0, bits=3)
    assert s[0] == g["s_alpha1"]
    assert O.quantize_act(Z, s, bits=3)[0][0].tolist() == g["q_alpha1"]
    s = O.act_scale(Z, 0.5, bits=3)
    assert s[0] == g["s_alpha05"]
    assert O.quantize_act(Z, s, bits=3)[0][0].tolist() == g["q_alpha05"]
    # mutant: the 4-bit scale on 3-bit codes
    q_bad, _ = O.quantize_act(Z, O.act_scale(Z, 1.0, bits=4), bits=3)
    assert q_bad[0].tolist() != g["q_alpha1"]


def test_golden_weight_3bit():
    g = GOLD["weight_3bit"]
    wq = O.quantize_weights(np.array([g["sym_v"]], dtype=np.float32), 4, False, bits=3)
    assert float(wq["s"][0, 0]) == g["sym_s"] and wq["codes"][0].tolist() == g["sym_q"]
    wq = O.quantize_weights(np.array([g["asym_v"]], dtype=np.float32), 4, True, bits=3)
    assert float(wq["s"][0, 0]) == g["asym_s"] and float(wq["z"][0, 0]) == g["asym_z"]
    assert wq["codes"][0].tolist() == g["asym_u"]


def test_3bit_codes_nearest_bruteforce():
    rng = np.random.default_rng(31)
    X = rng.standard_normal((3, 32)) * rng.uniform(0.1, 10, (3, 1))
    r = O.transform_quant(X, np.eye(4), np.eye(8), bits=3)
    for m in range(3):
        s = Fraction(float(np.abs(X[m]).max())) / 3
        for k in range(32):
            assert r["q"][m, k] == nearest_code_bruteforce(Fraction(float(X[m, k])) / s, -4, 3)
    W = (rng.standard_normal((2, 64)) * 0.02).astype(np.float32)
    for asym in (False, True):
        wq = O.quantize_weights(W, 32, asym, bits=3)
        for n in range(2):
            for k in range(64):
                gidx = k // 32
                s = Fraction(float(wq["s"][n, gidx]))
                z = int(float(wq["z"][n, gidx]))
                t = Fraction(float(W[n, k])) / s + z
                lo, hi = (0, 7) if asym else (-4, 3)
                assert wq["codes"][n, k] == nearest_code_bruteforce(t, lo, hi)


def test_3bit_rtn_bounds():
    rng = np.random.default_rng(32)
    X = rng.standard_normal((8, 256)).astype(np.float16)
    P1 = WL.random_invertible(rng, 16)
    P2 = WL.random_invertible(rng, 16)
    r = O.transform_quant(X, P1, P2, bits=3)
    assert r["q"].min() >= -4 and r["q"].max() <= 3
    err = np.abs(r["Z"] - r["q"] * r["s_x"][:, None])
    assert np.all(err <= r["s_x"][:, None] / 2 * (1 + 1e-12))
    W = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    wq = O.quantize_weights(W, 128, True, bits=3)
    assert wq["codes"].min() >= 0 and wq["codes"].max() <= 7
    deq = O.dequant_weights(wq)
    bound = np.repeat(wq["s"].astype(np.float64), 128, axis=1) / 2
    assert np.all(np.abs(deq - W) <= bound * (1 + 2 ** -9) + 1e-12)
