"""Level 2 of the parity contract on every kernel the layer's timed paths run:
given identical codes, the integer sums are exact.

The product is D[m,n,g] = Σ_{k in g} q_x[m,k]·(u[n,k] - z[n,g]) (FlatQuant
page, section 核心思想: the layer is the product of the two quantized
matrices; FRM-PTQ page, section 初步介绍: codes with a zero point per group).
The timed kernels return fp16 Y = s_x·Σ_g s_w·D, not D.  Here every token
scale and weight scale is a power of two (0.5, 1 or 2) and the codes are
mostly in {-1, 0, 1} with a sprinkle of the extreme codes, so that every
output Y is a number fp16 holds exactly (checked on the host before the GPU
runs).  Each kernel's own arithmetic (int32 MFMA sums, power-of-two unshifts,
fp32 folds of exactly representable integers) is then exact too, and the GPU
result must equal the oracle's bit for bit: an accumulator off by one would
show as a wrong output.

Covered: every prefill tile configuration (per channel, one-tile groups,
longer groups, symmetric and asymmetric weights), every decode variant, the
fp6-pipe tiles, and the single-kernel decode layer (identity transform and a
static step of 1, so its codes equal the input).
"""
import numpy as np
import pytest

import oracle as O
from gpu_common import kernel_override, log, to_dev, torch_dev

pytestmark = pytest.mark.gpu

NUM_TILE_CONFIGS = 13
NUM_DECODE_VARIANTS = 5
NUM_F6_TILES = 6


def W():
    import w4a4_post_quantized_amd as lib
    return lib


def _draw(rng, shape, lo, hi):
    """Codes in {-1, 0, 1}, 1 % of them at the extremes lo / hi."""
    c = rng.choice(np.array([-1, 0, 1], np.int64), size=shape, p=[0.3, 0.4, 0.3])
    ext = rng.random(shape) < 0.01
    c[ext] = rng.choice(np.array([lo, hi], np.int64), size=int(ext.sum()))
    return c


def exact_case(M, N, K, g, asym, seed, token_scales=(0.5, 1.0, 2.0)):
    """Codes and power-of-two scales whose layer output fp16 holds exactly.

    Returns (qx int8 [M,K], wc int8 [N,K], z fp16 [N,G], sx fp32 [M],
    sw fp16 [N,G], Y64 float64 [M,N]).  Activation codes are thinned (a
    deterministic half of the nonzero ones set to 0) until every output is
    an fp16 number of magnitude <= 1024."""
    rng = np.random.default_rng(seed)
    G = K // g
    qx = _draw(rng, (M, K), -8, 7)
    if asym:
        z = rng.integers(1, 15, (N, G))
        wc = np.clip(np.repeat(z, g, axis=1) + _draw(rng, (N, K), -15, 15), 0, 15)
        z16 = z.astype(np.float16)
    else:
        wc = _draw(rng, (N, K), -8, 7)
        z16 = np.zeros((N, G), np.float16)
    sx = rng.choice(np.array(token_scales, np.float32), M)
    sw = rng.choice(np.array([0.5, 1.0, 2.0], np.float16), (N, G))
    wc8 = wc.astype(np.int8)
    for _ in range(12):
        qx8 = qx.astype(np.int8)
        D = O.int_gemm(qx8, wc8, z16, g)
        Y64 = O.epilogue(D, sx, sw)
        if np.abs(Y64).max() <= 1024 and np.array_equal(Y64.astype(np.float16).astype(np.float64), Y64):
            return qx8, wc8, z16, sx, sw, Y64
        nz = np.argwhere(qx != 0)
        drop = nz[rng.random(len(nz)) < 0.5]
        qx[drop[:, 0], drop[:, 1]] = 0
    raise AssertionError("could not draw an exactly representable case")


def run_gemm(qx, wc, z, sx, sw, g, asym):
    desc = W().WeightDesc(wc.shape[0], wc.shape[1], g, int(asym))
    Y = W().gemm(to_dev(O.pack_nibbles(qx)), to_dev(sx), desc, to_dev(O.pack_nibbles(wc)),
                 to_dev(sw), to_dev(z) if asym else None)
    return desc, Y.cpu().numpy()


def assert_exact(Y, Y64, what):
    Yd = Y.astype(np.float64)
    bad = Yd != Y64
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} outputs differ from the exact sums, "
                             f"first {i}: gpu {Yd[i]} exact {Y64[i]}")


PREFILL_CASES = [
    # M, N, K, group, asym
    (300, 520, 1024, 1024, False),
    (300, 520, 1024, 1024, True),
    (300, 520, 1024, 128, True),
    (300, 520, 1024, 128, False),
    (200, 264, 2048, 256, True),
    (257, 136, 4096, 128, True),
    (130, 519, 1152, 128, True),      # N x G odd: the last scale word is half used
]


def test_exact_cases_are_representable():
    """The construction itself: outputs large enough to exercise the sums
    (some beyond what the 16 low bits of a wrong accumulator would show)."""
    for (M, N, K, g, asym) in PREFILL_CASES:
        *_, Y64 = exact_case(M, N, K, g, asym, seed=M + K)
        assert np.abs(Y64).max() >= 64


@pytest.mark.parametrize("tile", range(NUM_TILE_CONFIGS))
@pytest.mark.parametrize("M,N,K,g,asym", PREFILL_CASES)
def test_prefill_tile_exact(tile, M, N, K, g, asym):
    log(f"exact prefill tile {tile}: M={M} N={N} K={K} g={g} asym={asym}")
    qx, wc, z, sx, sw, Y64 = exact_case(M, N, K, g, asym, seed=M + K + tile)
    with kernel_override(W().OVERRIDE_PREFILL_TILE, tile):
        desc, Y = run_gemm(qx, wc, z, sx, sw, g, asym)
        name = W().gemm_kernel_name(M, desc)
    log(f"  {name}")
    assert_exact(Y, Y64, name)


DECODE_CASES = [
    (1, 520, 2944, 128, True),
    (13, 392, 1024, 1024, False),
    (17, 264, 2560, 256, True),
    (33, 200, 2048, 2048, True),
    (64, 520, 1536, 128, False),
    (16, 264, 16384, 128, True),
    (8, 72, 28672, 128, True),
]


@pytest.mark.parametrize("variant", range(NUM_DECODE_VARIANTS))
@pytest.mark.parametrize("M,N,K,g,asym", DECODE_CASES)
def test_decode_variant_exact(variant, M, N, K, g, asym):
    log(f"exact decode variant {variant}: M={M} N={N} K={K} g={g} asym={asym}")
    qx, wc, z, sx, sw, Y64 = exact_case(M, N, K, g, asym, seed=3 * M + K + variant)
    with kernel_override(W().OVERRIDE_DECODE, variant):
        desc, Y = run_gemm(qx, wc, z, sx, sw, g, asym)
        name = W().gemm_kernel_name(M, desc)
    assert name.startswith("k_gemm_dec")
    assert_exact(Y, Y64, name)


@pytest.mark.parametrize("tile", range(NUM_F6_TILES))
@pytest.mark.parametrize("M,N,K,g,asym", [(300, 520, 1024, 1024, False), (300, 520, 1024, 128, True),
                                          (130, 200, 5120, 128, True), (260, 264, 2048, 256, False),
                                          (31, 40, 256, 256, False)])
def test_f6_tile_exact(tile, M, N, K, g, asym):
    log(f"exact fp6 tile {tile}: M={M} N={N} K={K} g={g} asym={asym}")
    qx, wc, z, sx, sw, Y64 = exact_case(M, N, K, g, asym, seed=5 * M + K + tile)
    desc = W().WeightDesc(N, K, g, int(asym))
    W6 = W().pack_weights_f6(desc, to_dev(O.pack_nibbles(wc)), to_dev(z) if asym else None)
    with kernel_override(W().OVERRIDE_F6_TILE, tile):
        Y = W().gemm_f6(to_dev(O.pack_nibbles(qx)), to_dev(sx), desc, W6, to_dev(sw)).cpu().numpy()
        name = W().gemm_f6_kernel_name(M, desc)
    assert_exact(Y, Y64, name)


@pytest.mark.parametrize("M,n1,N,g,asym", [(1, 224, 264, 128, True), (5, 224, 136, None, False),
                                            (16, 64, 200, 128, True), (3, 64, 72, 512, False)])
def test_linear_decode_exact(M, n1, N, g, asym):
    """The single-kernel decode layer with P1 = P2 = I and one static step of
    1: its codes are the integer inputs, its token scale 1, so its output is
    the exact integer product scaled by the power-of-two weight scales."""
    torch, dev = torch_dev()
    n2 = 128
    K = n1 * n2
    g = g or K
    log(f"exact linear_decode M={M} P=({n1},{n2}) N={N} g={g} asym={asym}")
    qx, wc, z, _, sw, Y64 = exact_case(M, N, K, g, asym, seed=11 * M + n1, token_scales=(1.0,))
    desc = W().WeightDesc(N, K, g, int(asym))
    sync = W().decode_sync_buffer(dev)
    Y = W().linear_decode(to_dev(qx.astype(np.float16)), to_dev(np.eye(n1, dtype=np.float32)),
                          to_dev(np.eye(n2, dtype=np.float32)), desc, to_dev(O.pack_nibbles(wc)),
                          to_dev(sw), to_dev(z) if asym else None, sync=sync,
                          steps=to_dev(np.ones(1, np.float32)), per_channel=False).cpu().numpy()
    assert int(sync.cpu().numpy()[W().DECODE_SYNC_ERROR_WORD]) == 0
    assert_exact(Y, Y64, "k_linear_dec")
