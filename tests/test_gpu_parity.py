"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Levels (for every step of the layer):
  1. packed activation codes bit-exact except within 1e-4 of a rounding tie;
     weight codes, scales and zero points bit-exact;
  2. given the oracle's codes, the int32 accumulators bit-exact;
  3. fp16 output within half an fp16 ulp plus fp32 epilogue rounding per
     element and relative L2 <= 1e-3, against the oracle's product and
     epilogue on the same codes: the oracle's codes for the GEMM entry
     points, the library's own codes and token scales for the whole layer.
Shapes span several tiles with ragged tails, the edge cases (empty, one
token, all-zero token, all-zero weight row, clipping, diag(c), every group
mode) and every (n1, n2) pair of the LLaMA-shaped workloads.
"""
import numpy as np
import pytest

import oracle as O
import workloads as WL
from gpu_common import (assert_codes_match, assert_layer_close, assert_y_close, custom_workload,
                        kernel_override, log, prepared, rel_l2, to_dev, torch_dev)

pytestmark = pytest.mark.gpu


def W():
    import w4a4_post_quantized_amd as lib
    return lib


def gpu_act(inp, X=None, c=None, alpha=1.0):
    torch, dev = torch_dev()
    X = inp["X"] if X is None else X
    Xq, sx = W().transform_quant(to_dev(X), to_dev(inp["P1"]), to_dev(inp["P2"]),
                                 None if c is None else to_dev(c), alpha)
    torch.cuda.synchronize()
    return Xq.cpu().numpy(), sx.cpu().numpy()


# ---------------------------------------------------------------------------
# activation path
# ---------------------------------------------------------------------------
def test_transform_permutation_is_exact():
    """P1, P2 permutations: the transform is a pure reindexing, exact in fp32."""
    log("transform permutation (16,32) M=37")
    rng = np.random.default_rng(1)
    n1, n2, M = 16, 32, 37
    p1, p2 = rng.permutation(n1), rng.permutation(n2)
    P1 = np.eye(n1, dtype=np.float32)[:, p1]
    P2 = np.eye(n2, dtype=np.float32)[:, p2]
    X = rng.standard_normal((M, n1 * n2)).astype(np.float16)
    Z = W().transform(to_dev(X), to_dev(P1), to_dev(P2)).cpu().numpy()
    perm = (p1[:, None] * n2 + p2[None, :]).reshape(-1)
    assert np.array_equal(Z, X[:, perm].astype(np.float32))
    r = O.transform_quant(X, P1, P2)
    Xq, sx = gpu_act(dict(X=X, P1=P1, P2=P2))
    assert_codes_match(O.unpack_nibbles(Xq, True), r["q"], r["t"])


FACTORS = [(16, 16), (32, 32), (64, 64), (64, 128), (112, 128), (224, 128), (8, 2), (128, 256),
           (160, 128), (256, 128)]


@pytest.mark.parametrize("n1,n2,with_c", [(a, b, False) for a, b in FACTORS] +
                         [(16, 16, True), (32, 64, True), (64, 64, True), (64, 128, True)])
def test_transform_accuracy(n1, n2, with_c):
    """fp32 Z against the fp64 oracle, in code units of the token's scale."""
    log(f"transform accuracy ({n1},{n2}) c={with_c}")
    wl = custom_workload(M=19, n1=n1, n2=n2, N=16, outliers=(3, n1 * n2 - 5), pivot=100.0, seed=n1)
    inp = WL.make_inputs(wl, with_weights=False)
    c = WL.make_channel_scale(wl.K, seed=n1 + n2) if with_c else None
    Zg = W().transform(to_dev(inp["X"]), to_dev(inp["P1"]), to_dev(inp["P2"]),
                       None if c is None else to_dev(c)).cpu().numpy()
    Zo = O.kron_transform(inp["X"], inp["P1"], inp["P2"], c)
    s = O.act_scale(Zo)
    err = np.abs(Zg - Zo) / s[:, None]
    log(f"  max error {err.max():.3e} code units")
    assert err.max() < 2e-5


@pytest.mark.parametrize("n1,n2,M", [(16, 16, 16), (64, 64, 130), (112, 128, 9), (224, 128, 3),
                                     (64, 128, 65), (128, 256, 2), (224, 128, 1), (224, 128, 37),
                                     (192, 128, 5)])
def test_transform_quant_parity(n1, n2, M):
    log(f"transform_quant ({n1},{n2}) M={M}")
    wl = custom_workload(M=M, n1=n1, n2=n2, N=16, outliers=(7, 100), pivot=100.0, seed=M)
    inp = WL.make_inputs(wl, with_weights=False)
    r = O.transform_quant(inp["X"], inp["P1"], inp["P2"])
    Xq, sx = gpu_act(inp)
    n = assert_codes_match(O.unpack_nibbles(Xq, True), r["q"], r["t"])
    log(f"  excused tie cells: {n}")
    np.testing.assert_allclose(sx, r["s_x"], rtol=2e-6, atol=0)


# diag(c) on every activation path: the wave-per-token kernel (n1, n2 <= 64;
# M = 3000 gives the (64, 64) waves several tokens each, and the scaled c
# vectors move the kernel's power-of-two prescale of c far from 1), and the
# split kernels (n2 = 128, n1 > 128)
@pytest.mark.parametrize("n1,n2,M,cmul", [(16, 16, 37, 1.0), (32, 32, 300, 1.0), (16, 64, 9, 1.0),
                                          (32, 64, 40, 1.0), (64, 64, 130, 1.0),
                                          (64, 64, 3000, 1.0), (64, 64, 50, 300.0),
                                          (32, 32, 20, 1.0 / 512), (64, 128, 33, 1.0),
                                          (224, 128, 5, 1.0)])
def test_transform_quant_channel_scale_and_clip(n1, n2, M, cmul):
    log(f"transform_quant with diag(c) x {cmul} and alpha_a = 0.6, ({n1},{n2}) M={M}")
    wl = custom_workload(M=M, n1=n1, n2=n2, N=16, outliers=(5,), pivot=30.0, seed=5 + n1 + M)
    inp = WL.make_inputs(wl, with_weights=False)
    c = (WL.make_channel_scale(wl.K, seed=3 + n2) * np.float32(cmul)).astype(np.float32)
    r = O.transform_quant(inp["X"], inp["P1"], inp["P2"], c=c, alpha_a=0.6)
    assert (r["q"] == -8).any() or (r["q"] == 7).any()
    Xq, sx = gpu_act(inp, c=c, alpha=0.6)
    assert_codes_match(O.unpack_nibbles(Xq, True), r["q"], r["t"])
    np.testing.assert_allclose(sx, r["s_x"], rtol=2e-6)


def test_transform_quant_edge_cases():
    torch, dev = torch_dev()
    log("transform_quant edge cases: M=0, M=1, all-zero token")
    wl = custom_workload(M=5, n1=16, n2=16, N=16, seed=9)
    inp = WL.make_inputs(wl, with_weights=False)
    X = inp["X"].copy()
    X[2] = 0
    r = O.transform_quant(X, inp["P1"], inp["P2"])
    Xq, sx = gpu_act(inp, X=X)
    assert sx[2] == 0 and np.all(Xq[2] == 0)
    assert_codes_match(O.unpack_nibbles(Xq, True), r["q"], r["t"])
    # one token
    Xq1, sx1 = gpu_act(inp, X=X[3:4])
    assert np.array_equal(Xq1[0], Xq[3]) and sx1[0] == sx[3]
    # empty
    Xq0, sx0 = W().transform_quant(torch.empty((0, 256), dtype=torch.float16, device=dev),
                                   to_dev(inp["P1"]), to_dev(inp["P2"]))
    assert Xq0.shape == (0, 128)


# ---------------------------------------------------------------------------
# weights
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,K,g,asym,alpha", [(96, 256, 256, False, 1.0), (96, 256, 128, True, 1.0),
                                              (50, 1024, 128, False, 0.9),
                                              (33, 1024, 1024, True, 1.0),
                                              (40, 2048, 256, True, 0.75)])
def test_pack_weights_bit_exact(N, K, g, asym, alpha):
    log(f"pack_weights N={N} K={K} g={g} asym={asym} alpha={alpha}")
    rng = np.random.default_rng(K + N)
    Wt = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wt[3] = 0.0                       # all-zero row
    Wt[4, :g] = np.abs(Wt[4, :g])     # all-positive group (z = 0 for asym)
    wq = O.quantize_weights(Wt, g, asym, alpha)
    desc, Wq, sw, zw = W().pack_weights(to_dev(Wt), g, asym, alpha)
    assert np.array_equal(Wq.cpu().numpy(), wq["packed"])
    assert np.array_equal(sw.cpu().numpy().view(np.uint16), wq["s"].view(np.uint16))
    if asym:
        assert np.array_equal(zw.cpu().numpy().view(np.uint16), wq["z"].view(np.uint16))


def test_pack_weights_scale_rounding_near_fp16_ties():
    """Rows whose max/7 lies within a float32 ulp of an fp16 rounding tie: a
    conversion through float32 would round twice and miss some of these."""
    log("pack_weights fp16 tie rows")
    f16 = np.arange(0x1800, 0x2800, 37, dtype=np.uint16).view(np.float16).astype(np.float64)
    rows = []
    for h in f16:
        nxt = np.nextafter(np.float16(h), np.float16(1)).astype(np.float64)
        mid = (h + nxt) / 2
        for a in (np.float32(mid * 7), np.nextafter(np.float32(mid * 7), np.float32(1)),
                  np.nextafter(np.float32(mid * 7), np.float32(0))):
            r = np.zeros(128, np.float32)
            r[0] = a
            r[1:] = np.linspace(-a, a, 127, dtype=np.float32) * np.float32(0.9)
            rows.append(r)
    Wt = np.stack(rows)
    for asym in (False, True):
        wq = O.quantize_weights(Wt, 128, asym)
        desc, Wq, sw, zw = W().pack_weights(to_dev(Wt), 128, asym)
        assert np.array_equal(sw.cpu().numpy().view(np.uint16), wq["s"].view(np.uint16))
        assert np.array_equal(Wq.cpu().numpy(), wq["packed"])


@pytest.mark.parametrize("n1,n2,N,with_c", [(16, 16, 40, False), (8, 32, 17, True),
                                            (64, 64, 8, False), (224, 128, 3, True)])
def test_merge_weights(n1, n2, N, with_c):
    log(f"merge_weights ({n1},{n2}) N={N} c={with_c}")
    rng = np.random.default_rng(n1 * n2 + N)
    P1 = WL.random_invertible(rng, n1).astype(np.float32)
    P2 = WL.random_invertible(rng, n2).astype(np.float32)
    Wr = (rng.standard_normal((N, n1 * n2)) * 0.02).astype(np.float32)
    c = WL.make_channel_scale(n1 * n2) if with_c else None
    want = O.merge_weights(Wr, P1, P2, c, out_dtype=np.float64)
    got = W().merge_weights(to_dev(Wr), to_dev(P1), to_dev(P2),
                            None if c is None else to_dev(c)).cpu().numpy()
    err = np.abs(got - want) / np.abs(want).max(axis=1, keepdims=True)
    log(f"  max rel error {err.max():.2e}")
    assert err.max() < 1e-6


def test_merge_weights_rejects_singular():
    torch, dev = torch_dev()
    P1 = np.eye(16, dtype=np.float32)
    P1[5] = P1[4]
    with pytest.raises(W().W4A4Error):
        W().merge_weights(to_dev(np.zeros((4, 256), np.float32)), to_dev(P1),
                          to_dev(np.eye(16, dtype=np.float32)))


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------
GEMM_CASES = [
    # M, N, K, group, asym
    (16, 256, 256, 256, False),
    (300, 520, 1024, 1024, False),
    (300, 520, 1024, 128, True),
    (77, 200, 2048, 256, True),
    (257, 384, 512, 512, True),
    (64, 192, 4096, 128, False),
    (1, 136, 1024, 128, True),
    (130, 130, 384, 128, False),
]


def _codes(M, N, K, g, asym, seed):
    rng = np.random.default_rng(seed)
    qx = rng.integers(-8, 8, (M, K)).astype(np.int8)
    if asym:
        wc = rng.integers(0, 16, (N, K)).astype(np.int8)
        z = rng.integers(0, 16, (N, K // g)).astype(np.float16)
    else:
        wc = rng.integers(-8, 8, (N, K)).astype(np.int8)
        z = np.zeros((N, K // g), np.float16)
    # extremes: a row and a column at the magnitude limits
    qx[0, :] = -8
    if asym:
        wc[0, :] = 0
        z[0, :] = 15
    else:
        wc[0, :] = -8
    return qx, wc, z


@pytest.mark.parametrize("M,N,K,g,asym", GEMM_CASES)
def test_gemm_i32_bit_exact(M, N, K, g, asym):
    log(f"gemm_i32 M={M} N={N} K={K} g={g} asym={asym}")
    qx, wc, z = _codes(M, N, K, g, asym, seed=M + N + K)
    D_or = O.int_gemm(qx, wc, z, g)
    desc = W().WeightDesc(N, K, g, int(asym))
    D = W().gemm_i32(to_dev(O.pack_nibbles(qx)), desc, to_dev(O.pack_nibbles(wc)),
                     to_dev(z) if asym else None).cpu().numpy()
    assert np.array_equal(D, D_or)


@pytest.mark.parametrize("M,N,K,g,asym", GEMM_CASES)
def test_gemm_fp16_given_codes(M, N, K, g, asym):
    log(f"gemm fp16 M={M} N={N} K={K} g={g} asym={asym}")
    qx, wc, z = _codes(M, N, K, g, asym, seed=M * 7 + N + K)
    rng = np.random.default_rng(M + 3)
    sx = (rng.uniform(0.5, 3, M) * 0.05).astype(np.float32)
    sw = (rng.uniform(0.5, 2, (N, K // g)) * 0.003).astype(np.float16)
    D_or = O.int_gemm(qx, wc, z, g)
    Y64 = O.epilogue(D_or, sx, sw)
    A = O.epilogue(np.abs(D_or), sx, sw)
    desc = W().WeightDesc(N, K, g, int(asym))
    Y = W().gemm(to_dev(O.pack_nibbles(qx)), to_dev(sx), desc, to_dev(O.pack_nibbles(wc)),
                 to_dev(sw), to_dev(z) if asym else None).cpu().numpy()
    assert_y_close(Y, Y64, A)


# ---------------------------------------------------------------------------
# whole layer on small shapes
# ---------------------------------------------------------------------------
def _layer_parity(inp, c=None, alpha=1.0):
    wl = inp["wl"]
    torch, dev = torch_dev()
    wq = O.quantize_weights(inp["Wt"], wl.group_size, wl.asymmetric)
    ref = O.linear(inp["X"], inp["P1"], inp["P2"], wq, c=c, alpha_a=alpha)
    desc, Wq, sw, zw = W().pack_weights(to_dev(inp["Wt"]), wl.group_size, wl.asymmetric)
    assert np.array_equal(Wq.cpu().numpy(), wq["packed"])
    cd = None if c is None else to_dev(c)
    Y = W().linear(to_dev(inp["X"]), to_dev(inp["P1"]), to_dev(inp["P2"]), desc, Wq, sw, zw,
                   c=cd, alpha_a=alpha).cpu().numpy()
    Xq, sx = W().transform_quant(to_dev(inp["X"]), to_dev(inp["P1"]), to_dev(inp["P2"]), cd, alpha)
    gq = O.unpack_nibbles(Xq.cpu().numpy(), True)
    n = assert_codes_match(gq, ref["act"]["q"], ref["act"]["t"])
    rel = assert_layer_close(Y, gq, sx.cpu().numpy(), wq)
    log(f"  linear relative L2 {rel:.2e} on the library's codes ({n} tie cells), "
        f"{rel_l2(Y, ref['Y64']):.2e} against the oracle's own codes")
    return Y, ref


def test_linear_tiny_config():
    log("linear: tiny config (16x256 -> 256, P (16,16))")
    _layer_parity(prepared("tiny"))


@pytest.mark.parametrize("wl", [
    custom_workload(M=300, n1=32, n2=32, N=520, outliers=(1, 900), pivot=100.0, seed=11),
    custom_workload(M=77, n1=64, n2=32, N=264, group_size=128, asym=True, seed=12),
    custom_workload(M=5, n1=112, n2=128, N=72, group_size=128, asym=True,
                    x_kind="silu_product", seed=13),
], ids=lambda w: w.name)
def test_linear_small_shapes(wl):
    log(f"linear: {wl.name}")
    _layer_parity(prepared(wl))


@pytest.mark.parametrize("n1,n2,M,N,static", [(64, 64, 130, 200, False), (112, 128, 97, 136, False),
                                               (64, 128, 70, 264, False), (32, 64, 129, 72, False),
                                               (64, 64, 131, 136, True), (16, 64, 150, 72, False)])
def test_linear_group_sums_from_transform(n1, n2, M, N, static):
    """Asymmetric groups of 128 above the decode sizes: the transform kernel
    of w4a4_linear also writes the per-token group sums of its codes for the
    GEMM's zero-point correction (no pre-pass).  The layer must equal
    w4a4_transform_quant followed by w4a4_gemm (which sums the codes in its
    own pre-pass) bit for bit, and the oracle's layer on those codes."""
    log(f"linear, group sums from the transform: ({n1},{n2}) M={M} N={N} static={static}")
    torch, dev = torch_dev()
    wl = custom_workload(M=M, n1=n1, n2=n2, N=N, group_size=128, asym=True, seed=31 + n1 + M)
    inp = prepared(wl)
    X, P1, P2 = to_dev(inp["X"]), to_dev(inp["P1"]), to_dev(inp["P2"])
    desc, Wq, sw, zw = W().pack_weights(to_dev(inp["Wt"]), 128, True)
    if static:
        steps = to_dev(np.array([0.37], np.float32))
        Y = W().linear_static(X, P1, P2, steps, False, desc, Wq, sw, zw).cpu().numpy()
        Xq, sx = W().transform_quant_static(X, P1, P2, steps, False)
    else:
        Y = W().linear(X, P1, P2, desc, Wq, sw, zw).cpu().numpy()
        Xq, sx = W().transform_quant(X, P1, P2)
    Y2 = W().gemm(Xq, sx, desc, Wq, sw, zw).cpu().numpy()
    assert np.array_equal(Y.view(np.uint16), Y2.view(np.uint16))
    wq = O.quantize_weights(inp["Wt"], 128, True)
    gq = O.unpack_nibbles(Xq.cpu().numpy(), True)
    rel = assert_layer_close(Y, gq, sx.cpu().numpy(), wq)
    log(f"  relative L2 {rel:.2e} on the library's codes")


@pytest.mark.parametrize("n1,n2,M,N", [(16, 32, 70, 136), (64, 64, 200, 264)])
def test_linear_with_channel_scale_and_clip(n1, n2, M, N):
    log(f"linear with diag(c), alpha_a 0.8, ({n1},{n2}) M={M} N={N}")
    wl = custom_workload(M=M, n1=n1, n2=n2, N=N, group_size=256, asym=True, seed=21)
    inp = WL.make_inputs(wl)
    c = WL.make_channel_scale(wl.K, seed=4)
    inp["Wt"] = O.merge_weights(inp["W"], inp["P1"], inp["P2"], c)
    _layer_parity(inp, c=c, alpha=0.8)


NUM_TILE_CONFIGS = 13
NUM_DECODE_VARIANTS = 5


def test_kernel_config_counts():
    L = W()
    assert L.kernel_config_count(L.OVERRIDE_PREFILL_TILE) == NUM_TILE_CONFIGS
    assert L.kernel_config_count(L.OVERRIDE_DECODE) == NUM_DECODE_VARIANTS


@pytest.mark.parametrize("tile", range(NUM_TILE_CONFIGS))
@pytest.mark.parametrize("M,N,K,g,asym", [(300, 520, 1024, 1024, False), (300, 520, 1024, 128, True),
                                          (300, 520, 1024, 128, False), (513, 392, 512, 512, True),
                                          (200, 264, 2048, 256, True),
                                          (300, 519, 1152, 128, True)])
def test_gemm_every_tile_config(tile, M, N, K, g, asym):
    """Every tile configuration the dispatcher can pick (forced through
    w4a4_set_kernel_override; configs without a per-group variant fall back
    to the default one) against the oracle, with ragged M and N."""
    log(f"gemm tile {tile}: M={M} N={N} K={K} g={g} asym={asym}")
    qx, wc, z = _codes(M, N, K, g, asym, seed=tile + 100)
    rng = np.random.default_rng(tile)
    sx = (rng.uniform(0.5, 3, M) * 0.05).astype(np.float32)
    sw = (rng.uniform(0.5, 2, (N, K // g)) * 0.003).astype(np.float16)
    D_or = O.int_gemm(qx, wc, z, g)
    desc = W().WeightDesc(N, K, g, int(asym))
    with kernel_override(W().OVERRIDE_PREFILL_TILE, tile):
        log(f"  kernel {W().gemm_kernel_name(M, desc)}")
        Y = W().gemm(to_dev(O.pack_nibbles(qx)), to_dev(sx), desc, to_dev(O.pack_nibbles(wc)),
                     to_dev(sw), to_dev(z) if asym else None).cpu().numpy()
    assert_y_close(Y, O.epilogue(D_or, sx, sw), O.epilogue(np.abs(D_or), sx, sw))


@pytest.mark.parametrize("variant", range(NUM_DECODE_VARIANTS))
@pytest.mark.parametrize("M,N,K,g,asym", [
    (1, 520, 2944, 128, True),        # K tiles not a multiple of the waves
    (13, 392, 1024, 1024, False),     # fewer K tiles than waves
    (17, 264, 2560, 256, True),       # wave ranges that split a weight group
    (33, 200, 2048, 2048, True),      # asymmetric per-channel
    (64, 520, 1536, 128, False),      # symmetric per-group
    (50, 136, 4096, 512, True),
    (16, 264, 16384, 128, True),      # activations too large to stage in LDS
    (8, 72, 28672, 128, True),        # the 70B down projection's K, staged
])
def test_gemm_decode_variants(variant, M, N, K, g, asym):
    """Every decode configuration (M <= 64: one, two or four 16-row fragments,
    forced through w4a4_set_kernel_override) against the oracle, ragged N."""
    log(f"gemm decode variant {variant}: M={M} N={N} K={K} g={g} asym={asym}")
    desc = W().WeightDesc(N, K, g, int(asym))
    qx, wc, z = _codes(M, N, K, g, asym, seed=variant + 7 * M)
    rng = np.random.default_rng(variant + M)
    sx = (rng.uniform(0.5, 3, M) * 0.05).astype(np.float32)
    sw = (rng.uniform(0.5, 2, (N, K // g)) * 0.003).astype(np.float16)
    D_or = O.int_gemm(qx, wc, z, g)
    with kernel_override(W().OVERRIDE_DECODE, variant):
        assert W().gemm_kernel_name(M, desc).startswith("k_gemm_dec")
        Y = W().gemm(to_dev(O.pack_nibbles(qx)), to_dev(sx), desc, to_dev(O.pack_nibbles(wc)),
                     to_dev(sw), to_dev(z) if asym else None).cpu().numpy()
    assert_y_close(Y, O.epilogue(D_or, sx, sw), O.epilogue(np.abs(D_or), sx, sw))
