"""GPU parity of the INT4 x INT4 product on the fp6 matrix pipe
(w4a4_pack_weights_f6, w4a4_gemm_f6, w4a4_linear_f6).

The layer is the same as w4a4_gemm's (FlatQuant page, section 核心思想; FRM-PTQ
page, section 初步介绍); every code v is held as the fp6 E2M3 number v / 2 and
the products are summed exactly, so the checks are those of the int8 path:
  * the fp6 weights, decoded here on the CPU from the documented layout,
    hold exactly (u - z) / 2 or q / 2 of the oracle's codes, zero in padding;
  * the fp16 GEMM output on the oracle's codes within half an fp16 ulp plus
    4e-6 of the summed magnitude, for every tile configuration, ragged M, N;
  * the whole layer against the oracle (codes may flip only at rounding ties).
"""
import numpy as np
import pytest

import oracle as O
import workloads as WL
from gpu_common import (assert_codes_match, assert_layer_close, assert_y_close, custom_workload,
                        kernel_override, log, prepared,
                        rel_l2, sample_rows, to_dev, torch_dev)

pytestmark = pytest.mark.gpu

NUM_F6_TILES = 6


def W():
    import w4a4_post_quantized_amd as lib
    return lib


def e2m3_value(code):
    """fp6 E2M3 (1 sign, 2 exponent with bias 1, 3 mantissa bits) -> float."""
    code = np.asarray(code, dtype=np.int64)
    s = np.where(code & 32, -1.0, 1.0)
    e = (code >> 3) & 3
    m = code & 7
    mag = np.where(e == 0, m / 8.0, (1.0 + m / 8.0) * np.exp2(e - 1.0))
    return s * mag


def decode_f6(buf, R, K):
    """The fp6 layout -> values [Rp, K]: fragment (rt, kt) of 32 rows x 64
    codes at ((kt // 2) * Rp / 32 + rt) * 3072 + (kt % 2) * 1536; lane l (row
    l % 32, codes 32 (l // 32) + i) owns dwords 2p, 2p + 1 of plane p at
    512 p + 8 l, code i at bits 6 i of its 192 bits."""
    Rp = (R + 31) // 32 * 32
    b = np.asarray(buf, dtype=np.uint8)
    out = np.zeros((Rp, K))
    for kt in range(K // 64):
        for rt in range(Rp // 32):
            base = ((kt // 2) * (Rp // 32) + rt) * 3072 + (kt % 2) * 1536
            planes = [b[base + 512 * p: base + 512 * (p + 1)].view("<u4").reshape(64, 2)
                      for p in range(3)]
            words = np.concatenate(planes, axis=1).astype(np.uint64)     # [lane, 6 dwords]
            bits = np.zeros((64,), dtype=object)
            for d in range(5, -1, -1):
                bits = (bits << 32) | words[:, d].astype(object)
            for l in range(64):
                v = int(bits[l])
                codes = [(v >> (6 * i)) & 63 for i in range(32)]
                r = rt * 32 + l % 32
                k0 = kt * 64 + 32 * (l // 32)
                out[r, k0:k0 + 32] = e2m3_value(codes)
    return out


@pytest.mark.parametrize("N,K,g,asym", [(40, 256, 256, False), (72, 384, 128, True),
                                         (33, 1024, 512, True)])
def test_weights_f6_hold_the_codes(N, K, g, asym):
    log(f"pack_weights_f6 N={N} K={K} g={g} asym={asym}")
    rng = np.random.default_rng(N + K)
    Wt = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    wq = O.quantize_weights(Wt, g, asym)
    desc = W().WeightDesc(N, K, g, int(asym))
    z = to_dev(wq["z"]) if asym else None
    W6 = W().pack_weights_f6(desc, to_dev(wq["packed"]), z).cpu().numpy()
    assert W6.size == (N + 31) // 32 * 32 * K * 3 // 4
    vals = decode_f6(W6, N, K)
    codes = wq["codes"].astype(np.float64)
    if asym:
        codes = codes - np.repeat(wq["z"].astype(np.float64), g, axis=1)
    np.testing.assert_array_equal(vals[:N], codes / 2)
    assert not vals[N:].any()


def _codes(M, N, K, g, asym, seed):
    rng = np.random.default_rng(seed)
    qx = rng.integers(-8, 8, size=(M, K)).astype(np.int8)
    if asym:
        wc = rng.integers(0, 16, size=(N, K)).astype(np.int8)
        z = rng.integers(0, 16, size=(N, K // g)).astype(np.float16)
    else:
        wc = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
        z = np.zeros((N, K // g), np.float16)
    return qx, wc, z


@pytest.mark.parametrize("tile", range(NUM_F6_TILES))
@pytest.mark.parametrize("M,N,K,g,asym", [(300, 520, 1024, 1024, False), (300, 520, 1024, 128, True),
                                          (513, 392, 512, 512, True), (70, 96, 128, 128, False),
                                          (260, 264, 2048, 256, False), (1, 33, 128, 128, True),
                                          (31, 1, 256, 256, False), (130, 200, 5120, 128, True),
                                          (64, 96, 1536, 128, False), (129, 136, 12288, 128, True)])
def test_gemm_f6_every_tile(tile, M, N, K, g, asym):
    """Every fp6 tile configuration (forced through w4a4_set_kernel_override; the
    per-channel-only ones fall back to the default for per-group weights)
    against the oracle's exact integer product, extreme codes included."""
    log(f"gemm_f6 tile {tile}: M={M} N={N} K={K} g={g} asym={asym}")
    qx, wc, z = _codes(M, N, K, g, asym, seed=tile + 200)
    qx[0, :] = -8                                   # the extreme products
    wc[0, :] = 0 if asym else -8
    if asym:
        z[0, :] = 15
    rng = np.random.default_rng(tile)
    sx = (rng.uniform(0.5, 3, M) * 0.05).astype(np.float32)
    sw = (rng.uniform(0.5, 2, (N, K // g)) * 0.003).astype(np.float16)
    D_or = O.int_gemm(qx, wc, z, g)
    desc = W().WeightDesc(N, K, g, int(asym))
    W6 = W().pack_weights_f6(desc, to_dev(O.pack_nibbles(wc)), to_dev(z) if asym else None)
    with kernel_override(W().OVERRIDE_F6_TILE, tile):
        Y = W().gemm_f6(to_dev(O.pack_nibbles(qx)), to_dev(sx), desc, W6, to_dev(sw)).cpu().numpy()
    assert_y_close(Y, O.epilogue(D_or, sx, sw), O.epilogue(np.abs(D_or), sx, sw))


def test_f6_config_count():
    assert W().kernel_config_count(W().OVERRIDE_F6_TILE) == NUM_F6_TILES


def test_gemm_f6_group_scale_table_offsets():
    """Groups of 128 codes stage their scales in LDS with 16-byte copies of
    the scale table: tables at 16-byte aligned offsets inside a larger buffer
    give the oracle's result, and a table that is not 16-byte aligned is
    refused by the entry point."""
    torch, dev = torch_dev()
    M, N, K, g = 200, 136, 4096, 128
    qx, wc, z = _codes(M, N, K, g, True, seed=77)
    rng = np.random.default_rng(78)
    sx = (rng.uniform(0.5, 3, M) * 0.05).astype(np.float32)
    sw = (rng.uniform(0.5, 2, (N, K // g)) * 0.003).astype(np.float16)
    ref = O.epilogue(O.int_gemm(qx, wc, z, g), sx, sw)
    A = O.epilogue(np.abs(O.int_gemm(qx, wc, z, g)), sx, sw)
    desc = W().WeightDesc(N, K, g, 1)
    W6 = W().pack_weights_f6(desc, to_dev(O.pack_nibbles(wc)), to_dev(z))
    Xq, sx_d = to_dev(O.pack_nibbles(qx)), to_dev(sx)
    for off in (0, 8, 1):
        log(f"gemm_f6 scale table at element offset {off}")
        big = torch.zeros(N * (K // g) + off, dtype=torch.float16, device=dev)
        big[off:] = to_dev(sw).reshape(-1)
        sw_d = big[off:].view(N, K // g)
        if off % 8:
            with pytest.raises(W().W4A4Error, match="aligned"):
                W().gemm_f6(Xq, sx_d, desc, W6, sw_d)
            continue
        Y = W().gemm_f6(Xq, sx_d, desc, W6, sw_d).cpu().numpy()
        assert_y_close(Y, ref, A)


def _layer_parity_f6(inp, c=None, alpha=1.0):
    wl = inp["wl"]
    wq = O.quantize_weights(inp["Wt"], wl.group_size, wl.asymmetric)
    ref = O.linear(inp["X"], inp["P1"], inp["P2"], wq, c=c, alpha_a=alpha)
    desc, Wq, sw, zw = W().pack_weights(to_dev(inp["Wt"]), wl.group_size, wl.asymmetric)
    assert np.array_equal(Wq.cpu().numpy(), wq["packed"])
    W6 = W().pack_weights_f6(desc, Wq, zw)
    cd = None if c is None else to_dev(c)
    Y = W().linear_f6(to_dev(inp["X"]), to_dev(inp["P1"]), to_dev(inp["P2"]), desc, W6, sw,
                      c=cd, alpha_a=alpha).cpu().numpy()
    Xq, sx = W().transform_quant(to_dev(inp["X"]), to_dev(inp["P1"]), to_dev(inp["P2"]), cd, alpha)
    gq = O.unpack_nibbles(Xq.cpu().numpy(), True)
    assert_codes_match(gq, ref["act"]["q"], ref["act"]["t"])
    rel = assert_layer_close(Y, gq, sx.cpu().numpy(), wq, what="linear_f6")
    log(f"  linear_f6 relative L2 {rel:.2e} on the library's codes, "
        f"{rel_l2(Y, ref['Y64']):.2e} against the oracle's own codes")


@pytest.mark.parametrize("wl", [
    custom_workload(M=300, n1=32, n2=32, N=520, outliers=(1, 900), pivot=100.0, seed=11),
    custom_workload(M=77, n1=64, n2=32, N=264, group_size=128, asym=True, seed=12),
    custom_workload(M=130, n1=112, n2=128, N=72, group_size=128, asym=True,
                    x_kind="silu_product", seed=13),
], ids=lambda w: w.name)
def test_linear_f6_small_shapes(wl):
    log(f"linear_f6: {wl.name}")
    _layer_parity_f6(prepared(wl))


def test_linear_f6_with_channel_scale_and_clip():
    wl = custom_workload(M=70, n1=16, n2=32, N=136, group_size=256, asym=True, seed=21)
    inp = WL.make_inputs(wl)
    c = WL.make_channel_scale(wl.K, seed=4)
    inp["Wt"] = O.merge_weights(inp["W"], inp["P1"], inp["P2"], c)
    _layer_parity_f6(inp, c=c, alpha=0.8)


@pytest.mark.parametrize("name", ["qkv8b", "down8b"])
def test_full_size_f6(name):
    """The full prefill shape in the configuration the benchmark times
    (w4a4_linear_f6), on sampled tokens x channels against the oracle; raw
    weights serve as W̃ as in the int8 full-size tests."""
    torch, dev = torch_dev()
    wl = WL.get(name)
    log(f"[{name}] f6 full size M={wl.M} K={wl.K} N={wl.N}")
    inp = WL.make_inputs(name)
    rows = sample_rows(wl.M)
    rng = np.random.default_rng(7)
    cols = np.unique(np.concatenate([[0, wl.N - 1], rng.choice(wl.N, 256, replace=False)]))
    desc, Wq, sw, zw = W().pack_weights(to_dev(inp["W"]), wl.group_size, wl.asymmetric)
    W6 = W().pack_weights_f6(desc, Wq, zw)
    X_d, P1_d, P2_d = to_dev(inp["X"]), to_dev(inp["P1"]), to_dev(inp["P2"])
    Y = W().linear_f6(X_d, P1_d, P2_d, desc, W6, sw)
    Xq, sx = W().transform_quant(X_d, P1_d, P2_d)
    torch.cuda.synchronize()
    act = O.transform_quant(inp["X"], inp["P1"], inp["P2"])
    gq_all = O.unpack_nibbles(Xq.cpu().numpy(), True)
    n = assert_codes_match(gq_all, act["q"], act["t"], what=f"{name} activation codes")
    wq_s = O.quantize_weights(inp["W"][cols], wl.group_size, wl.asymmetric)
    Ys = Y.index_select(0, torch.as_tensor(rows, device=dev)).index_select(
        1, torch.as_tensor(cols, device=dev)).cpu().numpy()
    rel = assert_layer_close(Ys, gq_all[rows], sx.cpu().numpy()[rows], wq_s,
                             what=f"{name} linear_f6")
    log(f"[{name}] linear_f6 relative L2 on samples {rel:.2e} on the library's codes "
        f"({n} tie cells over all tokens)")
