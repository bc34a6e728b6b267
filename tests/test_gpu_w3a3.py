"""GPU parity of the 3-bit variant of the layer (W3A3; FRM-PTQ page,
introduction and contributions, with the quantizer of its section 初步介绍 at
b = 3), through the C ABI entry points w4a4_transform_quant_bits,
w4a4_pack_weights_bits and w4a4_linear_bits.

Checks: activation codes in [-4, 3] bit-exact against the oracle except within
the 1e-4 tie window, on every transform kernel family (wave, fused, column
block, split); token scales to fp32 rounding; packed 3-bit weight codes, scales
and zero points bit-exact; the whole layer within the same bound as the 4-bit
layer; and bits = 4 through the _bits entry points equal to the plain ones.
"""
import numpy as np
import pytest

import oracle as O
import workloads as WL
from gpu_common import assert_codes_match, assert_layer_close, custom_workload, log, rel_l2, \
    to_dev, torch_dev

pytestmark = pytest.mark.gpu


def W():
    import w4a4_post_quantized_amd as lib
    return lib


@pytest.mark.parametrize("n1,n2,M", [(16, 16, 16), (64, 64, 130), (64, 128, 65), (112, 128, 9),
                                     (224, 128, 37), (128, 256, 2), (8, 32, 19)])
def test_transform_quant_3bit(n1, n2, M):
    log(f"transform_quant_bits 3 ({n1},{n2}) M={M}")
    wl = custom_workload(M=M, n1=n1, n2=n2, N=16, outliers=(7, 100), pivot=100.0, seed=M + 3)
    inp = WL.make_inputs(wl, with_weights=False)
    r = O.transform_quant(inp["X"], inp["P1"], inp["P2"], bits=3)
    Xq, sx = W().transform_quant_bits(to_dev(inp["X"]), to_dev(inp["P1"]), to_dev(inp["P2"]), 3)
    q = O.unpack_nibbles(Xq.cpu().numpy(), True)
    assert q.min() >= -4 and q.max() <= 3
    n = assert_codes_match(q, r["q"], r["t"])
    log(f"  excused tie cells: {n}")
    np.testing.assert_allclose(sx.cpu().numpy(), r["s_x"], rtol=2e-6, atol=0)


def test_transform_quant_3bit_clip_reaches_minus4():
    wl = custom_workload(M=24, n1=32, n2=64, N=16, outliers=(5,), pivot=30.0, seed=8)
    inp = WL.make_inputs(wl, with_weights=False)
    r = O.transform_quant(inp["X"], inp["P1"], inp["P2"], alpha_a=0.6, bits=3)
    assert (r["q"] == -4).any() and (r["q"] == 3).any()
    Xq, sx = W().transform_quant_bits(to_dev(inp["X"]), to_dev(inp["P1"]), to_dev(inp["P2"]), 3,
                                      alpha_a=0.6)
    assert_codes_match(O.unpack_nibbles(Xq.cpu().numpy(), True), r["q"], r["t"])
    np.testing.assert_allclose(sx.cpu().numpy(), r["s_x"], rtol=2e-6)


@pytest.mark.parametrize("N,K,g,asym,alpha", [(96, 256, 256, False, 1.0), (96, 256, 128, True, 1.0),
                                              (40, 2048, 256, True, 0.75), (33, 1024, 1024, False, 0.9)])
def test_pack_weights_3bit_bit_exact(N, K, g, asym, alpha):
    log(f"pack_weights_bits 3 N={N} K={K} g={g} asym={asym}")
    rng = np.random.default_rng(K + N + 3)
    Wt = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wt[3] = 0.0
    Wt[4, :g] = np.abs(Wt[4, :g])
    wq = O.quantize_weights(Wt, g, asym, alpha, bits=3)
    desc, Wq, sw, zw = W().pack_weights_bits(to_dev(Wt), g, asym, 3, alpha)
    assert np.array_equal(Wq.cpu().numpy(), wq["packed"])
    assert np.array_equal(sw.cpu().numpy().view(np.uint16), wq["s"].view(np.uint16))
    if asym:
        assert np.array_equal(zw.cpu().numpy().view(np.uint16), wq["z"].view(np.uint16))


@pytest.mark.parametrize("wl", [
    custom_workload(M=300, n1=32, n2=32, N=520, outliers=(1, 900), pivot=100.0, seed=41),
    custom_workload(M=77, n1=64, n2=32, N=264, group_size=128, asym=True, seed=42),
    custom_workload(M=5, n1=112, n2=128, N=72, group_size=128, asym=True,
                    x_kind="silu_product", seed=43),
], ids=lambda w: w.name)
def test_linear_3bit(wl):
    log(f"linear_bits 3: {wl.name}")
    inp = WL.make_inputs(wl)
    Wt = O.merge_weights(inp["W"], inp["P1"], inp["P2"])
    wq = O.quantize_weights(Wt, wl.group_size, wl.asymmetric, bits=3)
    ref = O.linear(inp["X"], inp["P1"], inp["P2"], wq, bits=3)
    desc, Wq, sw, zw = W().pack_weights_bits(to_dev(Wt), wl.group_size, wl.asymmetric, 3)
    assert np.array_equal(Wq.cpu().numpy(), wq["packed"])
    X, P1, P2 = to_dev(inp["X"]), to_dev(inp["P1"]), to_dev(inp["P2"])
    Y = W().linear_bits(X, P1, P2, 3, desc, Wq, sw, zw).cpu().numpy()
    Xq, sx = W().transform_quant_bits(X, P1, P2, 3)
    gq = O.unpack_nibbles(Xq.cpu().numpy(), True)
    n = assert_codes_match(gq, ref["act"]["q"], ref["act"]["t"])
    rel = assert_layer_close(Y, gq, sx.cpu().numpy(), wq)
    log(f"  relative L2 {rel:.2e} on the library's codes ({n} tie cells), "
        f"{rel_l2(Y, ref['Y64']):.2e} against the oracle's own codes")


def test_bits4_entry_points_equal_plain():
    wl = custom_workload(M=33, n1=32, n2=32, N=136, group_size=128, asym=True, seed=44)
    inp = WL.make_inputs(wl)
    Wt = to_dev(O.merge_weights(inp["W"], inp["P1"], inp["P2"]))
    X, P1, P2 = to_dev(inp["X"]), to_dev(inp["P1"]), to_dev(inp["P2"])
    d4, Wq4, sw4, zw4 = W().pack_weights(Wt, 128, True)
    db, Wqb, swb, zwb = W().pack_weights_bits(Wt, 128, True, 4)
    assert np.array_equal(Wq4.cpu().numpy(), Wqb.cpu().numpy())
    assert np.array_equal(sw4.cpu().numpy(), swb.cpu().numpy())
    Y4 = W().linear(X, P1, P2, d4, Wq4, sw4, zw4).cpu().numpy()
    Yb = W().linear_bits(X, P1, P2, 4, db, Wqb, swb, zwb).cpu().numpy()
    assert np.array_equal(Y4.view(np.uint16), Yb.view(np.uint16))
