"""Host-side model of the copy addresses of the symmetric int8 prefill GEMM
(k_gemm_dl in gemm.hip, per-channel symmetric weights).

Those copies are issued as global_load_lds_dwordx4 with a wave-uniform 64-bit
base in scalar registers and a 32-bit per-lane byte offset
(dma16_async_sv and uniform_base in common.hpp).  The base is read with readfirstlane, which
returns a signed 32-bit value per half; the 64-bit base must be assembled from
the two halves each ZERO-extended.  This test models, in exact Python
integers, (a) the per-lane pointer the compiler-built copies use
(row pointer + chunk + K tile, the asymmetric path) and (b) the scalar-base
form (tile base + K tile, plus the lane offset), for every prefill tile shape
with symmetric weights, ragged M and N, every workgroup, wave, lane, copy and
K tile, and with operand buffers whose low address word is >= 2^31.  It
checks that the zero-extended assembly reproduces every pointer, and that a
sign-extended low half (the form that once faulted the GPU) would not.  A
second model covers the 4-byte copies of the weight scales and zero points
that the one-tile-group kernels stage per K tile.  Nothing here runs on a GPU.
"""
import numpy as np
import pytest

MASK64 = (1 << 64) - 1
BK_BYTES = 64                     # packed bytes of a 128-code K tile row

# (BM, BN, WAVES_M, WAVES_N) of every k_gemm_dl configuration that runs
# symmetric per-channel weights through the scalar-base copies
TILES = [(256, 256, 2, 4), (128, 128, 2, 2), (256, 128, 4, 2), (128, 256, 2, 4),
         (256, 256, 4, 4), (128, 384, 2, 4), (128, 384, 4, 4)]


def assemble(base, sign_extend_low=False):
    """The 64-bit scalar base built from readfirstlane of the two halves."""
    lo = base & 0xFFFFFFFF
    hi = (base >> 32) & 0xFFFFFFFF
    if sign_extend_low and lo >= 1 << 31:
        lo_w = (lo - (1 << 32)) & MASK64          # int32 widened with its sign
    else:
        lo_w = lo                                 # uint32 widened with zeros
    return ((hi << 32) | lo_w) & MASK64


def lane_layout(BM, BN, NW, M, N, K, m0, n0):
    """[copies, waves, lanes] arrays: which operand (A?), clamped source row,
    16-byte chunk, and the 32-bit lane offset from the tile's first row."""
    KB = K // 2
    LPW = (BM + BN) * 4 // (64 * NW)
    i = np.arange(LPW)[:, None, None]
    w = np.arange(NW)[None, :, None]
    lane = np.arange(64)[None, None, :]
    j = (i * NW + w) * 64 + lane
    isA = ((i * NW + w) * 64 < BM * 4) & np.ones_like(lane, dtype=bool)
    jj = np.where(isA, j, j - BM * 4)
    row = jj >> 2
    c = (jj & 3) ^ ((row >> 2) & 3)
    r = np.where(isA, np.minimum(m0 + row, M - 1), np.minimum(n0 + row, N - 1))
    off = (r - np.where(isA, m0, n0)) * KB + c * 16
    return isA, r, c, off


@pytest.mark.parametrize("BM,BN,WM,WN", TILES)
@pytest.mark.parametrize("M,N,K", [(300, 520, 1024), (2048, 6144, 4096), (257, 136, 384),
                                   (65, 1, 128), (4096, 1000, 8192)])
def test_scalar_base_copies_reach_every_lane_pointer(BM, BN, WM, WN, M, N, K):
    NW = WM * WN
    KB = K // 2
    KT = K // 128
    # operand buffers whose low address words are >= 2^31 (tile bases move
    # from there across the K tiles and rows)
    Xq = 0x00007F3A_9C40_0000
    Wq = 0x00007F3B_FFF0_0100
    assert (Xq & 0xFFFFFFFF) >= 1 << 31 and (Wq & 0xFFFFFFFF) >= 1 << 31
    kts = sorted({0, 1, KT - 1, KT // 2, KT, KT + 2})          # issue clamps kt to KT - 1
    sign_differs = 0
    for m0 in range(0, M, BM):
        for n0 in range(0, N, BN):
            isA, r, c, off = lane_layout(BM, BN, NW, M, N, K, m0, n0)
            assert off.min() >= 0 and off.max() < 1 << 32          # a 32-bit unsigned offset
            for kt in kts:
                kc = min(kt, KT - 1)
                # per-lane pointers of the compiler-built copies
                want = np.where(isA, Xq, Wq) + r * KB + c * 16 + kc * BK_BYTES
                for src_base, sel in ((Xq, isA), (Wq, ~isA)):
                    tile_base = src_base + (m0 if src_base == Xq else n0) * KB + kc * BK_BYTES
                    good = assemble(tile_base)
                    bad = assemble(tile_base, sign_extend_low=True)
                    got = good + off[sel]
                    assert np.array_equal(got, want[sel])
                    if bad != good:
                        sign_differs += 1
                        # the wrapped 64-bit sums of the sign-extended base
                        wrapped = np.uint64(bad) + off[sel].astype(np.uint64)
                        assert not np.array_equal(wrapped, want[sel].astype(np.uint64))
    assert sign_differs > 0          # the buffers above do exercise the sign bit


def test_assembly_on_edge_bases():
    for base in (0x0000_7FFF_FFFF_FFF0, 0x0000_7F00_8000_0000, 0x0000_7F00_7FFF_FFF0, 0x10):
        assert assemble(base) == base
        lo = base & 0xFFFFFFFF
        if lo >= 1 << 31:
            assert assemble(base, sign_extend_low=True) == base | 0xFFFFFFFF_00000000
        else:
            assert assemble(base, sign_extend_low=True) == base


# (BM, BN, WAVES_M, WAVES_N) of the k_gemm_dl configurations that run groups
# of one K tile (128 codes)
GROUP_TILES = [(128, 128, 2, 2), (256, 128, 4, 2), (128, 256, 2, 4)]
SZSLOT = 256


@pytest.mark.parametrize("BM,BN,WM,WN", GROUP_TILES)
@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("N,K", [(520, 1024), (136, 384), (1, 128), (28672, 4096), (77, 14336)])
def test_scale_copies_address_every_group_scale(BM, BN, WM, WN, asym, N, K):
    """One-tile-group scale copies: wave w copies, per tile kt, the aligned
    4-byte word holding element row * G + kt of the scale (or zero-point)
    array for the 64 rows of its item into its LDS slot; the reading lane
    takes the half that the element's parity selects.  Every copied word
    lies inside the array rounded up to whole words, the offset fits 32 bits,
    the slots of the waves do not overlap, and every (row, group) a B
    fragment reads is the element it needs."""
    NW = WM * WN
    G = K // 128
    KT = G
    kinds = 2 if asym else 1
    SZI = kinds * BN // 64
    assert SZI <= NW
    for n0 in range(0, N, BN):
        for kt in sorted({0, 1, KT - 1, KT // 2, KT + 1}):
            kc = min(kt, KT - 1)
            lds = {}
            for w in range(NW):
                it = w % SZI
                kind = 1 if it >= BN // 64 else 0
                lane = np.arange(64)
                row = np.minimum(n0 + (it % (BN // 64)) * 64 + lane, N - 1)
                e0 = row * G
                off = 2 * ((e0 + kc) & ~1)
                assert off.max() < 1 << 32
                assert off.min() >= 0 and (off + 4).max() <= 2 * (N * G + (N * G) % 2)
                assert (off % 4 == 0).all()
                slot = w * SZSLOT + 4 * lane
                assert slot.max() + 4 <= (w + 1) * SZSLOT
                for l in range(64):
                    word_elems = (off[l] // 2, off[l] // 2 + 1)
                    lds[slot[l]] = (kind, word_elems)
            # readers: every B row the tile's waves hold
            for rr in range(BN):
                rowg = min(n0 + rr, N - 1)
                want = rowg * G + kc
                base = (rr >> 6) * SZSLOT + 4 * (rr & 63)
                for kind in range(kinds):
                    k_, elems = lds[kind * (BN // 64) * SZSLOT + base]
                    assert k_ == kind
                    half = (rowg * G + kc) & 1
                    assert elems[half] == want
