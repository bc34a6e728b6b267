"""GPU parity of static activation quantization (steps fixed offline) and
of the step migration, through the C ABI, against the CPU oracle.

FPTQuant page, section 核心贡献: one step for the whole tensor; MergeQuant
page, sections 核心思路 and 关键设计 items 1-2: one step per channel, folded
into the weights.  Steps are calibrated by the oracle on a separate seeded
calibration batch (an oracle result used as a shared input) with a clipping
ratio below 1, so that the tested batch has clipped codes at both ends.
Codes must match bit for bit except within the 1e-4 tie window; the token
scale must be the step (per tensor) or exactly 1 (per channel); migrated
weights must match bit for bit; the whole layer must meet the same bound as
the dynamic layer.
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


def static_inputs(wl, per_channel, ratio=0.8, c=None, M_cal=48):
    inp = WL.make_inputs(wl, with_weights=wl.N > 0)
    Xc = WL.make_calibration_activations(wl, M_cal, inp["outlier_channels"], seed=wl.seed + 7919)
    Zc = O.kron_transform(Xc, inp["P1"], inp["P2"], c)
    inp["steps"] = O.calibrate_steps(Zc, per_channel, ratio)
    return inp


# every activation path: wave (n1, n2 <= 64, with or without diag(c)),
# fused (n2 = 128), column-block (n1 > 128), split (other shapes, and diag(c)
# with n2 = 128 or n1 > 128)
SHAPES = [(16, 16, 37), (64, 64, 130), (32, 64, 9), (64, 128, 65), (112, 128, 9),
          (224, 128, 3), (224, 128, 37), (128, 256, 2), (8, 2, 5)]


@pytest.mark.parametrize("per_channel", [False, True], ids=["tensor", "channel"])
@pytest.mark.parametrize("n1,n2,M", SHAPES)
def test_transform_quant_static_parity(n1, n2, M, per_channel):
    log(f"transform_quant_static ({n1},{n2}) M={M} per_channel={per_channel}")
    wl = custom_workload(M=M, n1=n1, n2=n2, N=0, outliers=(7, n1 * n2 - 3), pivot=30.0, seed=M + n1)
    inp = static_inputs(wl, per_channel)
    st = inp["steps"]
    r = O.transform_quant_static(inp["X"], inp["P1"], inp["P2"], st.astype(np.float64), per_channel)
    Xq, sx = W().transform_quant_static(to_dev(inp["X"]), to_dev(inp["P1"]), to_dev(inp["P2"]),
                                        to_dev(st), per_channel)
    torch, _ = torch_dev()
    torch.cuda.synchronize()
    q = O.unpack_nibbles(Xq.cpu().numpy(), True)
    n = assert_codes_match(q, r["q"], r["t"])
    assert (r["q"] == 7).any() and (r["q"] == -8).any()     # the clip range is exercised
    want_sx = np.ones(M) if per_channel else np.full(M, st[0], dtype=np.float64)
    assert np.array_equal(sx.cpu().numpy().astype(np.float64), want_sx)
    log(f"  excused tie cells: {n}")


@pytest.mark.parametrize("per_channel", [False, True], ids=["tensor", "channel"])
@pytest.mark.parametrize("n1,n2,M", [(32, 64, 40), (64, 64, 2100), (16, 16, 11), (64, 128, 20)])
def test_transform_quant_static_with_channel_scale(n1, n2, M, per_channel):
    log(f"transform_quant_static with diag(c), ({n1},{n2}) M={M} per_channel={per_channel}")
    wl = custom_workload(M=M, n1=n1, n2=n2, N=0, outliers=(5,), pivot=30.0, seed=5)
    c = WL.make_channel_scale(wl.K, seed=3)
    inp = static_inputs(wl, per_channel, c=c)
    st = inp["steps"]
    r = O.transform_quant_static(inp["X"], inp["P1"], inp["P2"], st.astype(np.float64),
                                 per_channel, c=c)
    Xq, sx = W().transform_quant_static(to_dev(inp["X"]), to_dev(inp["P1"]), to_dev(inp["P2"]),
                                        to_dev(st), per_channel, c=to_dev(c))
    assert_codes_match(O.unpack_nibbles(Xq.cpu().numpy(), True), r["q"], r["t"])


def test_transform_quant_static_edge_cases():
    """Empty batch; an all-zero token (codes 0, scale still the step); a
    per-tensor step equal to each token's dynamic scale reproduces the
    dynamic codes on the GPU as well."""
    torch, dev = torch_dev()
    log("transform_quant_static edge cases")
    wl = custom_workload(M=6, n1=64, n2=64, N=0, seed=31)
    inp = static_inputs(wl, False)
    X = inp["X"].copy()
    X[2] = 0
    st = inp["steps"]
    Xq, sx = W().transform_quant_static(to_dev(X), to_dev(inp["P1"]), to_dev(inp["P2"]),
                                        to_dev(st), False)
    assert np.all(Xq.cpu().numpy()[2] == 0) and sx.cpu().numpy()[2] == st[0]
    Xq0, _ = W().transform_quant_static(torch.empty((0, wl.K), dtype=torch.float16, device=dev),
                                        to_dev(inp["P1"]), to_dev(inp["P2"]), to_dev(st), False)
    assert Xq0.shape == (0, wl.K // 2)
    # one token, its own dynamic scale as the static step
    Xd, sd = W().transform_quant(to_dev(X[3:4]), to_dev(inp["P1"]), to_dev(inp["P2"]))
    Xs, ss = W().transform_quant_static(to_dev(X[3:4]), to_dev(inp["P1"]), to_dev(inp["P2"]),
                                        sd.clone(), False)
    assert np.array_equal(Xs.cpu().numpy(), Xd.cpu().numpy())
    assert ss.cpu().numpy()[0] == sd.cpu().numpy()[0]


@pytest.mark.parametrize("N,K", [(96, 256), (33, 4096), (7, 14336)])
def test_migrate_steps_bit_exact(N, K):
    log(f"migrate_steps N={N} K={K}")
    rng = np.random.default_rng(N + K)
    Wt = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    st = rng.uniform(1e-3, 5.0, K).astype(np.float32)
    want = O.migrate_steps(Wt, st)
    got = W().migrate_steps(to_dev(Wt), to_dev(st)).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # in place
    d = to_dev(Wt)
    W().migrate_steps(d, to_dev(st), out=d)
    assert np.array_equal(d.cpu().numpy().view(np.uint32), want.view(np.uint32))


LAYERS = [
    custom_workload(M=130, n1=64, n2=64, N=520, outliers=(1, 900), pivot=30.0, seed=41),
    custom_workload(M=9, n1=112, n2=128, N=136, group_size=128, asym=True,
                    x_kind="silu_product", seed=42),
    custom_workload(M=5, n1=224, n2=128, N=72, seed=43),
    custom_workload(M=300, n1=32, n2=32, N=264, group_size=256, asym=True, seed=44),
]


@pytest.mark.parametrize("per_channel", [False, True], ids=["tensor", "channel"])
@pytest.mark.parametrize("wl", LAYERS, ids=lambda w: w.name)
def test_linear_static_parity(wl, per_channel):
    """Whole layer.  Per channel: the oracle migrates the steps into the
    merged weights and quantizes them; the GPU migrates on the device
    (bit-exact to the oracle's) and packs; the layer then needs no
    activation scale (s_x = 1)."""
    log(f"linear_static {wl.name} per_channel={per_channel}")
    inp = static_inputs(wl, per_channel)
    st = inp["steps"]
    Wt = O.merge_weights(inp["W"], inp["P1"], inp["P2"])
    Wt_dev = to_dev(Wt)
    if per_channel:
        Wt = O.migrate_steps(Wt, st)
        Wt_dev = W().migrate_steps(Wt_dev, to_dev(st))
        assert np.array_equal(Wt_dev.cpu().numpy().view(np.uint32), Wt.view(np.uint32))
    wq = O.quantize_weights(Wt, wl.group_size, wl.asymmetric)
    ref = O.linear_static(inp["X"], inp["P1"], inp["P2"], wq, st.astype(np.float64), per_channel)
    desc, Wq, sw, zw = W().pack_weights(Wt_dev, wl.group_size, wl.asymmetric)
    assert np.array_equal(Wq.cpu().numpy(), wq["packed"])
    Xd, P1d, P2d, std = to_dev(inp["X"]), to_dev(inp["P1"]), to_dev(inp["P2"]), to_dev(st)
    Y = W().linear_static(Xd, P1d, P2d, std, per_channel, desc, Wq, sw, zw).cpu().numpy()
    Xq, sx = W().transform_quant_static(Xd, P1d, P2d, std, per_channel)
    gq = O.unpack_nibbles(Xq.cpu().numpy(), True)
    n = assert_codes_match(gq, ref["act"]["q"], ref["act"]["t"])
    rel = assert_layer_close(Y, gq, sx.cpu().numpy(), wq)
    log(f"  relative L2 {rel:.2e} on the library's codes ({n} tie cells), "
        f"{rel_l2(Y, ref['Y64']):.2e} against the oracle's own codes")
