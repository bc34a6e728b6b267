"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects invalid calls before touching the GPU (no compute
call is made here; pointers are fake, non-null, and never dereferenced because
validation fails first)."""
import ctypes
import os
import re

import pytest

import w4a4_post_quantized_amd as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000          # 16-byte aligned, never dereferenced
MISALIGNED = 0x10008


def header_functions():
    src = open(os.path.join(ROOT, "include", "w4a4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a4_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert names == sorted(W.EXPORTED_SYMBOLS)
    L = ctypes.CDLL(W.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    assert W.version() == 0x000200
    L = W.lib()
    assert L.w4a4_status_str(0) == b"W4A4_OK"
    assert L.w4a4_status_str(-3) == b"W4A4_ERR_ALIGNMENT"
    assert L.w4a4_status_str(42) == b"W4A4_ERR_UNKNOWN"


def desc(N=256, K=256, g=256, asym=0):
    return ctypes.byref(W.WeightDesc(N, K, g, asym))


def last():
    return W.lib().w4a4_last_error().decode()


def test_gemm_validation():
    L = W.lib()
    args = lambda **kw: dict(dict(Xq=FAKE, sx=FAKE, M=16, d=desc(), Wq=FAKE, sw=FAKE, zw=None,
                                  Y=FAKE, ws=None, wsb=0), **kw)

    def call(**kw):
        a = args(**kw)
        return L.w4a4_gemm(a["Xq"], a["sx"], a["M"], a["d"], a["Wq"], a["sw"], a["zw"], a["Y"],
                           a["ws"], a["wsb"], None)

    assert call(Xq=None) == -1 and "Xq" in last()
    assert call(Y=None) == -1
    assert call(M=-1) == -1
    assert call(Xq=MISALIGNED) == -3
    assert call(d=desc(K=200, g=200)) == -2          # K % 128
    assert call(d=desc(K=512, g=64)) == -2           # group not multiple of 128
    assert call(d=desc(K=512, g=384)) == -2          # group does not divide K
    assert call(d=desc(N=0)) == -1
    assert call(d=desc(asym=1)) == -1 and "z_w" in last()   # asym needs z_w
    assert call(d=desc(asym=2)) == -1
    assert call(d=None) == -1
    assert call(d=desc(K=131072, g=131072)) == -2
    assert call(M=0) == 0                             # empty: nothing to do, no launch


def test_gemm_i32_validation():
    L = W.lib()
    assert L.w4a4_gemm_i32(FAKE, 4, desc(), FAKE, None, None, None) == -1
    assert L.w4a4_gemm_i32(FAKE, 4, desc(), FAKE, None, MISALIGNED, None) == -3


def test_transform_quant_validation():
    L = W.lib()

    def call(X=FAKE, M=4, n1=16, n2=16, P1=FAKE, P2=FAKE, c=None, a=1.0, Xq=FAKE, sx=FAKE,
             ws=FAKE, wsb=1 << 30):
        return L.w4a4_transform_quant(X, M, n1, n2, P1, P2, c, a, Xq, sx, ws, wsb, None)

    assert call(X=None) == -1
    assert call(P1=None) == -1
    assert call(n1=0) == -1
    assert call(n1=300) == -2
    assert call(n1=3, n2=5) == -2                     # K % 16
    assert call(a=0.0) == -1 and call(a=1.5) == -1
    assert call(c=MISALIGNED) == -3
    # with c, (64, 128) runs the split path and needs a workspace
    need = L.w4a4_transform_quant_workspace_bytes(4, 64, 128, 1)
    assert need > 0
    assert call(n1=64, n2=128, c=FAKE, wsb=need - 1) == -4
    assert call(n1=64, n2=128, c=FAKE, ws=None) == -4
    assert L.w4a4_transform_quant_workspace_bytes(4, 64, 128, 0) == 0
    # (16, 16) runs the wave kernel, with or without c, and needs no workspace
    assert L.w4a4_transform_quant_workspace_bytes(4, 16, 16, 0) == 0
    assert L.w4a4_transform_quant_workspace_bytes(4, 16, 16, 1) == 0
    assert call(M=0, X=None) == 0


def test_pack_and_merge_validation():
    L = W.lib()
    assert L.w4a4_pack_weights(desc(), None, 1.0, FAKE, FAKE, None, None) == -1
    assert L.w4a4_pack_weights(desc(asym=1), FAKE, 1.0, FAKE, FAKE, None, None) == -1
    assert L.w4a4_pack_weights(desc(), FAKE, 0.0, FAKE, FAKE, None, None) == -1
    assert L.w4a4_pack_weights(desc(K=256, g=3), FAKE, 1.0, FAKE, FAKE, None, None) == -2
    nb = L.w4a4_merge_workspace_bytes(16, 16, 256)
    assert nb > 0 and L.w4a4_merge_workspace_bytes(16, 16, 255) == 0
    assert L.w4a4_merge_weights(FAKE, 8, 256, 16, 16, FAKE, FAKE, None, FAKE, FAKE, nb - 1, None) == -4
    assert L.w4a4_merge_weights(FAKE, 8, 250, 16, 16, FAKE, FAKE, None, FAKE, FAKE, nb, None) == -1
    assert L.w4a4_merge_weights(FAKE, 8, 256, 16, 16, FAKE, None, None, FAKE, FAKE, nb, None) == -1


def test_linear_validation():
    L = W.lib()
    d = desc(N=256, K=256, g=256)
    nb = L.w4a4_linear_workspace_bytes(16, 16, 16, 0, d)
    assert nb >= 16 * 128 + 16 * 4

    def call(n1=16, n2=16, ws=FAKE, wsb=nb, d=d, zw=None):
        return L.w4a4_linear(FAKE, 16, n1, n2, FAKE, FAKE, None, 1.0, d, FAKE, FAKE, zw, FAKE,
                             ws, wsb, None)

    assert call(n1=8, n2=16) == -1                    # desc K != n1*n2
    assert call(wsb=nb - 1) == -4
    assert call(ws=None) == -1
    assert call(d=desc(N=256, K=256, g=128, asym=1)) == -1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import importlib
    monkeypatch.setattr(W, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(W, "_lib", None)
    with pytest.raises(ImportError):
        W.lib()


def test_gemm_kernel_name_query():
    """The configuration name is a host-side query: decode kernels for at most
    64 tokens, the prefill kernels above; invalid descriptors give NULL."""
    assert W.gemm_kernel_name(1, W.WeightDesc(8192, 28672, 128, 1)).startswith("k_gemm_dec<FM 1")
    assert W.gemm_kernel_name(64, W.WeightDesc(8192, 28672, 128, 1)).startswith("k_gemm_dec_split<FM 4")
    assert W.gemm_kernel_name(32, W.WeightDesc(8192, 28672, 128, 1)).startswith("k_gemm_dec_split<FM 2")
    # 8 tokens stage their activations in LDS: the register-streamed kernel;
    # 16 tokens of 28672 codes do not fit: the split kernel
    assert W.gemm_kernel_name(8, W.WeightDesc(8192, 28672, 128, 1)).startswith("k_gemm_dec<FM 1")
    assert W.gemm_kernel_name(16, W.WeightDesc(8192, 28672, 128, 1)).startswith("k_gemm_dec_split<FM 1")
    assert W.gemm_kernel_name(16, W.WeightDesc(8192, 4096, 128, 1)).startswith("k_gemm_dec<FM 1")
    # other group sizes keep the register-streamed kernel
    assert W.gemm_kernel_name(64, W.WeightDesc(8192, 28672, 512, 1)).startswith("k_gemm_dec<FM 4")
    assert W.gemm_kernel_name(2048, W.WeightDesc(6144, 4096, 4096, 0)).startswith("k_gemm_dl<")
    assert W.gemm_kernel_name(2048, W.WeightDesc(28672, 4096, 128, 1)).startswith("k_gemm")
    # groups of 128: 128x128 tiles up to K = 8192, 256x128 tiles above
    assert W.gemm_kernel_name(2048, W.WeightDesc(28672, 4096, 128, 1)) == \
        "k_gemm_dl<128x128, waves 2x2, 4 stages>"
    assert W.gemm_kernel_name(2048, W.WeightDesc(4096, 14336, 128, 1)) == \
        "k_gemm_dl<256x128, waves 4x2, 4 stages>"
    with pytest.raises(W.W4A4Error):
        W.gemm_kernel_name(16, W.WeightDesc(256, 200, 200, 0))


def test_decode_split_workspace():
    """The split-K decode kernel's partial sums: S ranges x M x N int32, S the
    smallest split giving 256 workgroups of 256 columns whose activations
    and scale tables fit the LDS (28672 -> 8192: 32 column blocks, 8 ranges of
    28 tiles; 28 tiles of 64 rows take 115.7 KiB and two tables 30 KiB)."""
    L = W.lib()
    d = W.WeightDesc(8192, 28672, 128, 1)
    assert L.w4a4_gemm_workspace_bytes(64, ctypes.byref(d)) == 8 * 64 * 8192 * 4
    assert L.w4a4_gemm_workspace_bytes(8, ctypes.byref(d)) == 8 * 8 * 8192 * 4
    # 57344 columns: 224 blocks, two ranges of 32 tiles (K 8192)
    d = W.WeightDesc(57344, 8192, 128, 1)
    assert L.w4a4_gemm_workspace_bytes(40, ctypes.byref(d)) == 2 * 40 * 57344 * 4
    # the LDS bound: 256 column blocks fill the CUs with one range, but 64
    # staged rows of 64 tiles take 257 KiB: two ranges of 32 tiles
    d = W.WeightDesc(65536, 8192, 8192, 0)
    assert L.w4a4_gemm_workspace_bytes(64, ctypes.byref(d)) == 2 * 64 * 65536 * 4
    # group sizes other than one tile or the whole row take no workspace
    assert L.w4a4_gemm_workspace_bytes(64, ctypes.byref(W.WeightDesc(8192, 28672, 512, 1))) == 0


def test_kernel_override_is_a_host_setting():
    """The selection override changes which configuration a query reports,
    restores the automatic choice with -1, and rejects unknown kinds."""
    d = W.WeightDesc(28672, 4096, 128, 1)
    auto = W.gemm_kernel_name(2048, d)
    n = W.kernel_config_count(W.OVERRIDE_PREFILL_TILE)
    names = set()
    for t in range(n):
        assert W.set_kernel_override(W.OVERRIDE_PREFILL_TILE, t) == (t - 1 if t else -1)
        names.add(W.gemm_kernel_name(2048, W.WeightDesc(6144, 4096, 4096, 0)))
    assert len(names) == n                      # every per-channel config is distinct
    assert W.set_kernel_override(W.OVERRIDE_PREFILL_TILE, -1) == n - 1
    assert W.gemm_kernel_name(2048, d) == auto
    assert W.set_kernel_override(W.OVERRIDE_DECODE, 2) == -1
    v2 = W.gemm_kernel_name(8, d)
    W.set_kernel_override(W.OVERRIDE_DECODE, 3)
    assert W.gemm_kernel_name(8, d) != v2
    W.set_kernel_override(W.OVERRIDE_DECODE, -1)
    assert W.kernel_config_count(W.OVERRIDE_DECODE) == 5
    W.set_kernel_override(W.OVERRIDE_DECODE, 4)           # the split-K kernel, any M
    assert W.gemm_kernel_name(8, d).startswith("k_gemm_dec_split<FM 1")
    W.set_kernel_override(W.OVERRIDE_DECODE, -1)
    assert W.kernel_config_count(W.OVERRIDE_F6_TILE) >= 1
    L = W.lib()
    assert L.w4a4_set_kernel_override(4, 0) == -1 and "kind" in last()
    assert W.set_kernel_override(W.OVERRIDE_TILE_GROUP, 4) == -1
    assert W.set_kernel_override(W.OVERRIDE_TILE_GROUP, -1) == 4
    assert L.w4a4_set_kernel_override(0, -2) == -1
    assert L.w4a4_kernel_config_count(-1) == -1


def test_static_entry_points_validation():
    L = W.lib()

    def tq(X=FAKE, M=4, n1=16, n2=16, st=FAKE, pc=0, Xq=FAKE, sx=FAKE, c=None):
        return L.w4a4_transform_quant_static(X, M, n1, n2, FAKE, FAKE, c, st, pc, Xq, sx, FAKE,
                                             1 << 30, None)

    assert tq(st=None) == -1 and "steps" in last()
    assert tq(pc=2) == -1 and "per_channel" in last()
    assert tq(st=MISALIGNED) == -3
    assert tq(X=None) == -1
    assert tq(n1=3, n2=5) == -2
    assert tq(M=0, X=None) == 0                       # empty: nothing to do

    assert L.w4a4_migrate_steps(FAKE, 8, 256, None, FAKE, None) == -1
    assert L.w4a4_migrate_steps(FAKE, 8, 258, FAKE, FAKE, None) == -2   # K % 4
    assert L.w4a4_migrate_steps(FAKE, -1, 256, FAKE, FAKE, None) == -1
    assert L.w4a4_migrate_steps(MISALIGNED, 8, 256, FAKE, FAKE, None) == -3
    assert L.w4a4_migrate_steps(None, 0, 256, FAKE, FAKE, None) == 0     # empty

    d = desc(N=256, K=256, g=256)
    nb = L.w4a4_linear_workspace_bytes(16, 16, 16, 0, d)

    def lin(st=FAKE, pc=1, n1=16, wsb=nb):
        return L.w4a4_linear_static(FAKE, 16, n1, 16, FAKE, FAKE, None, st, pc, d, FAKE, FAKE,
                                    None, FAKE, FAKE, wsb, None)

    assert lin(st=None) == -1
    assert lin(pc=-1) == -1
    assert lin(n1=8) == -1                            # desc K != n1*n2
    assert lin(wsb=nb - 1) == -4
    assert lin(st=MISALIGNED) == -3


def test_linear_decode_validation():
    L = W.lib()
    d = desc(N=256, K=28672, g=128, asym=1)
    nb = L.w4a4_linear_decode_workspace_bytes(1, 224, 128)
    assert nb >= 28672 // 2 + 4
    assert L.w4a4_linear_decode_workspace_bytes(0, 224, 128) == 0
    assert L.w4a4_linear_decode_workspace_bytes(17, 224, 128) == 0

    def call(M=1, n1=224, sync=FAKE, pc=0, zw=FAKE, d=d, alpha=1.0):
        return L.w4a4_linear_decode(FAKE, M, n1, 128, FAKE, FAKE, alpha, None, pc, d, FAKE, FAKE,
                                    zw, FAKE, FAKE, nb, sync, None)

    assert call(sync=None) == -1 and "sync" in last()
    assert call(pc=3) == -1
    assert call(alpha=0.0) == -1
    assert call(n1=112) == -1                          # desc K != n1*n2
    assert call(zw=None) == -1                         # asymmetric weights need z_w
    assert call(M=17) == -2 and "16 tokens" in last()
    assert call(sync=MISALIGNED) == -3
    assert call(M=0) == 0                              # empty: nothing to do
    hdr = open(os.path.join(ROOT, "include", "w4a4.h")).read()
    assert f"#define W4A4_DECODE_SYNC_BYTES {W.DECODE_SYNC_BYTES}" in hdr
    assert f"#define W4A4_DECODE_SYNC_ERROR_WORD {W.DECODE_SYNC_ERROR_WORD}" in hdr


def test_kv_cache_bytes_and_workspaces():
    L = W.lib()
    assert W.kv_cache_bytes(2, 8, 64) == (2 * 8 * 64 * 64, 2 * 8 * 64 * 64, 2 * 8 * 64 * 4)
    k = ctypes.c_size_t()
    assert L.w4a4_kv_cache_bytes(2, 8, 64, 48, ctypes.byref(k), None, None) == -2   # max_seq % 32
    assert L.w4a4_kv_cache_bytes(2, 8, 96, 64, ctypes.byref(k), None, None) == -2   # head size
    assert L.w4a4_kv_cache_bytes(-1, 8, 128, 64, None, None, None) == -1
    assert L.w4a4_kv_cache_bytes(2, 0, 128, 64, None, None, None) == -1
    assert L.w4a4_kv_query_factor_workspace_bytes(128, 1) >= 2 * 128 * 128 * 8
    assert L.w4a4_kv_query_factor_workspace_bytes(64, 1) == 0
    assert L.w4a4_attn_decode_workspace_bytes(4, 32, 8, 128, 1024) >= 4 * 32 * 128 * 4
    assert L.w4a4_attn_decode_workspace_bytes(4, 30, 8, 128, 1024) == 0    # heads_q % heads_kv
    assert L.w4a4_attn_decode_workspace_bytes(4, 136, 8, 128, 1024) == 0   # G = 17
    hdr = open(os.path.join(ROOT, "include", "w4a4.h")).read()
    assert f"#define W4A4_KV_HEAD_DIM {W.KV_HEAD_DIM}" in hdr


def test_kv_append_validation():
    L = W.lib()

    def call(T=4, S=2, H=8, d=128, ph=0, ak=1.0, av=1.0, B=2, ms=64, k=FAKE, kc=FAKE, vs=FAKE):
        return L.w4a4_kv_append(k, FAKE, T, FAKE, FAKE, FAKE, S, H, d, FAKE, FAKE, ph, ak, av,
                                kc, FAKE, FAKE, vs, B, ms, None)

    assert call(d=64) == -2 and "head_dim" in last()
    assert call(ms=40) == -2
    assert call(H=0) == -1
    assert call(T=-1) == -1
    assert call(S=-1) == -1
    assert call(ph=2) == -1
    assert call(ak=0.0) == -1 and "alpha" in last()
    assert call(av=1.5) == -1
    assert call(k=None) == -1 and "k is NULL" in last()
    assert call(kc=MISALIGNED) == -3
    assert call(vs=None) == -1
    assert call(T=0) == 0 and call(S=0) == 0 and call(B=0) == 0    # nothing to write


def test_attn_decode_validation():
    L = W.lib()
    nb = L.w4a4_attn_decode_workspace_bytes(2, 8, 2, 128, 64)

    def call(B=2, Hq=8, Hkv=2, d=128, ph=0, ms=64, sm=0.08, ws=FAKE, wsb=nb, out=FAKE, ln=FAKE):
        return L.w4a4_attn_decode(FAKE, B, Hq, Hkv, d, FAKE, ph, FAKE, FAKE, FAKE, FAKE, ln, ms, sm,
                                  out, ws, wsb, None)

    assert call(Hq=9) == -1 and "multiple" in last()
    assert call(Hq=34) == -2                                   # G = 17
    assert call(d=256) == -2
    assert call(ms=0) == -2
    assert call(sm=0.0) == -1 and "sm_scale" in last()
    assert call(sm=float("inf")) == -1
    assert call(sm=float("nan")) == -1
    assert call(ph=5) == -1
    assert call(ln=None) == -1 and "lengths" in last()
    assert call(out=MISALIGNED) == -3
    assert call(wsb=nb - 1) == -4
    assert call(ws=None) == -1
    assert call(B=0) == 0


def test_kv_query_factor_validation():
    L = W.lib()
    nb = L.w4a4_kv_query_factor_workspace_bytes(128, 2)
    assert L.w4a4_kv_query_factor(FAKE, 128, 2, FAKE, FAKE, nb - 1, None) == -4
    assert L.w4a4_kv_query_factor(FAKE, 64, 2, FAKE, FAKE, nb, None) == -2
    assert L.w4a4_kv_query_factor(FAKE, 128, 0, FAKE, FAKE, nb, None) == -1
    assert L.w4a4_kv_query_factor(None, 128, 2, FAKE, FAKE, nb, None) == -1
    assert L.w4a4_kv_query_factor(MISALIGNED, 128, 2, FAKE, FAKE, nb, None) == -3


def test_bits_entry_points_validation():
    L = W.lib()
    d = desc(N=256, K=256, g=128, asym=1)
    assert L.w4a4_pack_weights_bits(d, FAKE, 1.0, 5, FAKE, FAKE, FAKE, None) == -2
    assert "bits" in last()
    assert L.w4a4_pack_weights_bits(d, FAKE, 1.0, 2, FAKE, FAKE, FAKE, None) == -2
    assert L.w4a4_pack_weights_bits(d, FAKE, 1.0, 3, FAKE, FAKE, None, None) == -1   # z_w
    assert L.w4a4_transform_quant_bits(FAKE, 4, 16, 16, FAKE, FAKE, None, 1.0, 8, FAKE, FAKE,
                                       FAKE, 1 << 20, None) == -2
    assert L.w4a4_transform_quant_bits(FAKE, 0, 16, 16, FAKE, FAKE, None, 1.0, 3, FAKE, FAKE,
                                       FAKE, 1 << 20, None) == 0
    assert L.w4a4_linear_bits(FAKE, 4, 16, 16, FAKE, FAKE, None, 1.0, 1, d, FAKE, FAKE, FAKE,
                              FAKE, FAKE, 1 << 20, None) == -2


def test_ternary_entry_points_validation():
    L = W.lib()
    # K not a multiple of the block, M above the decode limit, bad iteration count
    assert L.w4a4_pack_ternary(FAKE, 8, 200, 10, FAKE, FAKE, None) == -2
    assert L.w4a4_pack_ternary(FAKE, 8, 256, -1, FAKE, FAKE, None) == -1
    assert L.w4a4_pack_ternary(FAKE, 0, 256, 10, FAKE, FAKE, None) == -1
    assert L.w4a4_pack_ternary(FAKE, 8, 256, 10, None, FAKE, None) == -1
    assert L.w4a4_pack_ternary(MISALIGNED, 8, 256, 10, FAKE, FAKE, None) == -3
    assert L.w4a4_ternary_gemm(FAKE, 65, 64, 256, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -2
    assert "decode" in last()
    assert L.w4a4_ternary_gemm(FAKE, 4, 64, 256, FAKE, MISALIGNED, FAKE, FAKE, 1 << 20, None) == -3
    assert L.w4a4_ternary_gemm(FAKE, 0, 64, 256, FAKE, FAKE, FAKE, FAKE, 0, None) == 0
    tq, am = W.ternary_weight_bytes(20, 384)
    assert (tq, am) == (32 * 96, 32 * 3 * 4)
    nb = ctypes.c_size_t(0)
    assert L.w4a4_ternary_weight_bytes(20, 300, ctypes.byref(nb), ctypes.byref(nb)) == -2
    assert L.w4a4_ternary_weight_bytes(20, 384, None, ctypes.byref(nb)) == -1
    # workspace: none when the tiles fill the GPU, else fp32 partials of a K split
    assert W.ternary_gemm_workspace_bytes(65, 64, 256) == 0
    assert W.ternary_gemm_workspace_bytes(0, 64, 256) == 0
    assert W.ternary_gemm_workspace_bytes(1, 8192, 28672) == 0
    nb = W.ternary_gemm_workspace_bytes(1, 64, 65536)
    assert nb > 0 and nb % (1 * 64 * 4) == 0
    assert L.w4a4_ternary_gemm(FAKE, 1, 64, 65536, FAKE, FAKE, FAKE, None, 0, None) == -4


def test_f6_entry_points_validation():
    L = W.lib()
    d = desc(N=100, K=256, g=128, asym=1)
    assert W.weights_f6_bytes(W.WeightDesc(100, 256, 128, 1)) == 128 * 256 * 3 // 4
    assert L.w4a4_pack_weights_f6(d, FAKE, None, FAKE, None) == -1        # z_w for asymmetric
    assert L.w4a4_pack_weights_f6(d, MISALIGNED, FAKE, FAKE, None) == -3
    assert W.gemm_f6_workspace_bytes(40, W.WeightDesc(100, 256, 128, 1)) >= 64 * 256 * 3 // 4
    assert L.w4a4_gemm_f6(FAKE, FAKE, 40, d, FAKE, FAKE, FAKE, FAKE, 16, None) == -4
    assert L.w4a4_gemm_f6(FAKE, FAKE, 0, d, FAKE, FAKE, FAKE, None, 0, None) == 0
    assert L.w4a4_gemm_f6(FAKE, FAKE, -1, d, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    assert "k_gemm_f6" in W.gemm_f6_kernel_name(2048, W.WeightDesc(6144, 4096, 4096, 0))
    assert L.w4a4_linear_f6(FAKE, 4, 16, 16, FAKE, FAKE, None, 1.5, desc(N=64, K=256, g=256),
                            FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -1   # alpha_a


def test_read_probe_validation():
    L = W.lib()
    assert L.w4a4_read_probe(None, 0, None, None) == 0          # nothing to read
    assert L.w4a4_read_probe(None, 16, FAKE, None) == -1
    assert L.w4a4_read_probe(FAKE, 16, None, None) == -1
    assert L.w4a4_read_probe(FAKE, 24, FAKE, None) == -1         # not a multiple of 16
    assert L.w4a4_read_probe(MISALIGNED, 16, FAKE, None) == -3
    assert L.w4a4_read_probe(FAKE, 16, MISALIGNED, None) == -3
