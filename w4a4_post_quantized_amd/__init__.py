"""Python binding of libw4a4 — the W4A4 quantized linear layer on MI355X.

Argument marshalling only: every function forwards torch tensors' device
pointers, sizes and the current HIP stream to the C entry point of the same
name (include/w4a4.h) and raises W4A4Error on a non-zero status.  PyTorch is
used for device memory and streams; all arithmetic runs in the HIP kernels of
libw4a4.so.  There is no fallback: importing the package fails loudly when the
library has not been built (``python -m w4a4_post_quantized_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "W4A4Error", "WeightDesc", "lib", "LIB_PATH", "EXPORTED_SYMBOLS", "read_probe",
    "OVERRIDE_PREFILL_TILE", "OVERRIDE_DECODE", "OVERRIDE_F6_TILE", "OVERRIDE_TILE_GROUP",
    "set_kernel_override",
    "kernel_config_count",
    "merge_weights", "pack_weights", "transform_quant", "transform", "gemm",
    "gemm_i32", "gemm_kernel_name", "linear", "linear_noalloc", "NOALLOC_SCRATCH_BYTES",
    "merge_workspace_bytes", "transform_quant_workspace_bytes",
    "gemm_workspace_bytes", "linear_workspace_bytes", "version",
    "migrate_steps", "transform_quant_static", "linear_static",
    "linear_decode", "linear_decode_workspace_bytes", "decode_sync_buffer",
    "DECODE_SYNC_BYTES", "DECODE_SYNC_ERROR_WORD",
    "KV_HEAD_DIM", "KvCache", "kv_cache_bytes", "kv_query_factor", "kv_append",
    "attn_decode_workspace_bytes", "attn_decode",
    "pack_weights_bits", "transform_quant_bits", "linear_bits",
    "TERNARY_BLOCK", "TERNARY_MAX_M", "ternary_weight_bytes", "pack_ternary", "unpack_ternary",
    "ternary_gemm_workspace_bytes",
    "ternary_gemm",
    "weights_f6_bytes", "pack_weights_f6", "gemm_f6_workspace_bytes", "gemm_f6",
    "gemm_f6_kernel_name", "linear_f6_workspace_bytes", "linear_f6",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4a4.so")

# every function include/w4a4.h declares
EXPORTED_SYMBOLS = [
    "w4a4_version", "w4a4_status_str", "w4a4_last_error", "w4a4_set_kernel_override",
    "w4a4_kernel_config_count",
    "w4a4_merge_workspace_bytes", "w4a4_merge_weights", "w4a4_pack_weights",
    "w4a4_migrate_steps",
    "w4a4_transform_quant_workspace_bytes", "w4a4_transform_quant", "w4a4_transform_quant_static",
    "w4a4_transform",
    "w4a4_gemm_workspace_bytes", "w4a4_gemm", "w4a4_gemm_i32", "w4a4_gemm_kernel_name",
    "w4a4_linear_workspace_bytes", "w4a4_linear", "w4a4_linear_noalloc", "w4a4_linear_static",
    "w4a4_linear_decode_workspace_bytes", "w4a4_linear_decode",
    "w4a4_kv_cache_bytes", "w4a4_kv_query_factor_workspace_bytes", "w4a4_kv_query_factor",
    "w4a4_kv_append", "w4a4_attn_decode_workspace_bytes", "w4a4_attn_decode",
    "w4a4_pack_weights_bits", "w4a4_transform_quant_bits", "w4a4_linear_bits",
    "w4a4_ternary_weight_bytes", "w4a4_pack_ternary", "w4a4_unpack_ternary",
    "w4a4_ternary_gemm_workspace_bytes",
    "w4a4_ternary_gemm",
    "w4a4_weights_f6_bytes", "w4a4_pack_weights_f6", "w4a4_gemm_f6_workspace_bytes",
    "w4a4_gemm_f6", "w4a4_gemm_f6_kernel_name", "w4a4_linear_f6_workspace_bytes",
    "w4a4_linear_f6",
    "w4a4_read_probe",
]

DECODE_SYNC_BYTES = 1024          # W4A4_DECODE_SYNC_BYTES
DECODE_SYNC_ERROR_WORD = 128      # W4A4_DECODE_SYNC_ERROR_WORD
KV_HEAD_DIM = 128                 # W4A4_KV_HEAD_DIM
TERNARY_BLOCK = 128               # W4A4_TERNARY_BLOCK
TERNARY_MAX_M = 64                # W4A4_TERNARY_MAX_M


class W4A4Error(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func} failed with {status}: {msg}")
        self.status = status


class WeightDesc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("asymmetric", ctypes.c_int32)]

    def __repr__(self):
        return (f"WeightDesc(N={self.N}, K={self.K}, group_size={self.group_size}, "
                f"asymmetric={self.asymmetric})")

    @property
    def groups(self) -> int:
        return self.K // self.group_size


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libw4a4.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m w4a4_post_quantized_amd.build`")
        # PyTorch's HIP runtime must be the process's one: loading torch first
        # makes the library's libamdhip64.so.7 resolve to it (loaded the other
        # way round, torch would bring a second runtime and the library's
        # calls would see no device)
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        dp = ctypes.POINTER(WeightDesc)
        szp = ctypes.POINTER(ctypes.c_size_t)
        sig = {
            "w4a4_version": (ctypes.c_int, []),
            "w4a4_status_str": (ctypes.c_char_p, [ctypes.c_int]),
            "w4a4_last_error": (ctypes.c_char_p, []),
            "w4a4_set_kernel_override": (ctypes.c_int, [i32, i32]),
            "w4a4_kernel_config_count": (ctypes.c_int, [i32]),
            "w4a4_merge_workspace_bytes": (sz, [i32, i32, i32]),
            "w4a4_merge_weights": (ctypes.c_int, [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
            "w4a4_pack_weights": (ctypes.c_int, [dp, vp, f32, vp, vp, vp, vp]),
            "w4a4_transform_quant_workspace_bytes": (sz, [i32, i32, i32, i32]),
            "w4a4_transform_quant": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp, f32, vp, vp, vp, sz, vp]),
            "w4a4_transform": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
            "w4a4_gemm_workspace_bytes": (sz, [i32, dp]),
            "w4a4_gemm": (ctypes.c_int, [vp, vp, i32, dp, vp, vp, vp, vp, vp, sz, vp]),
            "w4a4_gemm_i32": (ctypes.c_int, [vp, i32, dp, vp, vp, vp, vp]),
            "w4a4_gemm_kernel_name": (ctypes.c_char_p, [i32, dp]),
            "w4a4_weights_f6_bytes": (sz, [dp]),
            "w4a4_pack_weights_f6": (ctypes.c_int, [dp, vp, vp, vp, vp]),
            "w4a4_gemm_f6_workspace_bytes": (sz, [i32, dp]),
            "w4a4_gemm_f6": (ctypes.c_int, [vp, vp, i32, dp, vp, vp, vp, vp, sz, vp]),
            "w4a4_gemm_f6_kernel_name": (ctypes.c_char_p, [i32, dp]),
            "w4a4_linear_f6_workspace_bytes": (sz, [i32, i32, i32, i32, dp]),
            "w4a4_linear_f6": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp, ctypes.c_float, dp,
                                              vp, vp, vp, vp, sz, vp]),
            "w4a4_linear_workspace_bytes": (sz, [i32, i32, i32, i32, dp]),
            "w4a4_linear": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp, f32, dp, vp, vp, vp, vp, vp, sz, vp]),
            "w4a4_linear_noalloc": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp, f32, dp, vp, vp,
                                                   vp, vp, vp]),
            "w4a4_migrate_steps": (ctypes.c_int, [vp, i32, i32, vp, vp, vp]),
            "w4a4_transform_quant_static": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp, vp, i32, vp, vp,
                                                           vp, sz, vp]),
            "w4a4_linear_static": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp, vp, i32, dp, vp, vp, vp,
                                                  vp, vp, sz, vp]),
            "w4a4_linear_decode_workspace_bytes": (sz, [i32, i32, i32]),
            "w4a4_linear_decode": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, f32, vp, i32, dp, vp, vp,
                                                  vp, vp, vp, sz, vp, vp]),
            "w4a4_pack_weights_bits": (ctypes.c_int, [dp, vp, f32, i32, vp, vp, vp, vp]),
            "w4a4_transform_quant_bits": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp, f32, i32,
                                                         vp, vp, vp, sz, vp]),
            "w4a4_linear_bits": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp, f32, i32, dp, vp,
                                                vp, vp, vp, vp, sz, vp]),
            "w4a4_ternary_weight_bytes": (ctypes.c_int, [i32, i32, szp, szp]),
            "w4a4_pack_ternary": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp]),
            "w4a4_unpack_ternary": (ctypes.c_int, [vp, vp, i32, i32, vp, vp, vp, vp]),
            "w4a4_ternary_gemm_workspace_bytes": (sz, [i32, i32, i32]),
            "w4a4_read_probe": (ctypes.c_int, [vp, sz, vp, vp]),
            "w4a4_ternary_gemm": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]),
            "w4a4_kv_cache_bytes": (ctypes.c_int, [i32, i32, i32, i32, szp, szp, szp]),
            "w4a4_kv_query_factor_workspace_bytes": (sz, [i32, i32]),
            "w4a4_kv_query_factor": (ctypes.c_int, [vp, i32, i32, vp, vp, sz, vp]),
            "w4a4_kv_append": (ctypes.c_int, [vp, vp, i32, vp, vp, vp, i32, i32, i32, vp, vp, i32,
                                              f32, f32, vp, vp, vp, vp, i32, i32, vp]),
            "w4a4_attn_decode_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
            "w4a4_attn_decode": (ctypes.c_int, [vp, i32, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp,
                                                i32, f32, vp, vp, sz, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def version() -> int:
    return lib().w4a4_version()


OVERRIDE_PREFILL_TILE = 0         # W4A4_OVERRIDE_PREFILL_TILE
OVERRIDE_DECODE = 1               # W4A4_OVERRIDE_DECODE
OVERRIDE_F6_TILE = 2              # W4A4_OVERRIDE_F6_TILE
OVERRIDE_TILE_GROUP = 3           # W4A4_OVERRIDE_TILE_GROUP


def set_kernel_override(which: int, index: int) -> int:
    """Force a kernel configuration (tests and sweeps); -1 = automatic.
    Returns the previous index."""
    r = lib().w4a4_set_kernel_override(which, index)
    if r < -1:
        _check(r, "w4a4_set_kernel_override")
    return r


def kernel_config_count(which: int) -> int:
    r = lib().w4a4_kernel_config_count(which)
    if r < 0:
        _check(r, "w4a4_kernel_config_count")
    return r


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _p(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return getattr(stream, "cuda_stream", stream)
    return _torch().cuda.current_stream().cuda_stream


def _check(status: int, func: str):
    if status != 0:
        msg = lib().w4a4_last_error().decode(errors="replace")
        raise W4A4Error(status, func, msg)


def _need(t, dtype, shape, name):
    torch = _torch()
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous() or t.device.type != "cuda":
        raise ValueError(f"{name} must be a contiguous CUDA (HIP) tensor")
    return torch


def _ws(nbytes: int, device, ws=None):
    torch = _torch()
    if nbytes == 0:
        return None
    if ws is not None:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _desc(N, K, group_size, asymmetric) -> WeightDesc:
    return WeightDesc(int(N), int(K), int(group_size), int(bool(asymmetric)))


# ---------------------------------------------------------------------------
# workspace sizes
# ---------------------------------------------------------------------------
def merge_workspace_bytes(n1: int, n2: int) -> int:
    return lib().w4a4_merge_workspace_bytes(n1, n2, n1 * n2)


def transform_quant_workspace_bytes(M: int, n1: int, n2: int, has_c: bool = False) -> int:
    return lib().w4a4_transform_quant_workspace_bytes(M, n1, n2, int(bool(has_c)))


def gemm_workspace_bytes(M: int, desc: WeightDesc) -> int:
    return lib().w4a4_gemm_workspace_bytes(M, ctypes.byref(desc))


def linear_workspace_bytes(M: int, n1: int, n2: int, desc: WeightDesc, has_c: bool = False) -> int:
    return lib().w4a4_linear_workspace_bytes(M, n1, n2, int(bool(has_c)), ctypes.byref(desc))


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def merge_weights(W, P1, P2, c=None, out=None, stream=None):
    """W̃ = W · diag(1/c) · (P1 ⊗ P2)^-T on the device (fp32 [N, K])."""
    torch = _torch()
    N, K = W.shape
    n1, n2 = P1.shape[0], P2.shape[0]
    _need(W, torch.float32, (N, K), "W")
    _need(P1, torch.float32, (n1, n1), "P1")
    _need(P2, torch.float32, (n2, n2), "P2")
    if c is not None:
        _need(c, torch.float32, (K,), "c")
    Wt = out if out is not None else torch.empty_like(W)
    nb = merge_workspace_bytes(n1, n2)
    ws = _ws(nb, W.device)
    _check(lib().w4a4_merge_weights(_p(W), N, K, n1, n2, _p(P1), _p(P2), _p(c), _p(Wt),
                                    _p(ws), nb, _stream(stream)), "w4a4_merge_weights")
    return Wt


def pack_weights(Wt, group_size: int, asymmetric: bool, alpha_w: float = 1.0, stream=None):
    """Quantize merged weights: returns (desc, Wq uint8 [N,K/2], s_w fp16 [N,G],
    z_w fp16 [N,G] or None)."""
    torch = _torch()
    N, K = Wt.shape
    _need(Wt, torch.float32, (N, K), "Wt")
    desc = _desc(N, K, group_size, asymmetric)
    G = K // group_size if group_size > 0 else 0
    Wq = torch.empty((N, K // 2), dtype=torch.uint8, device=Wt.device)
    s_w = torch.empty((N, max(G, 1)), dtype=torch.float16, device=Wt.device)
    z_w = torch.empty((N, max(G, 1)), dtype=torch.float16, device=Wt.device) if asymmetric else None
    _check(lib().w4a4_pack_weights(ctypes.byref(desc), _p(Wt), float(alpha_w), _p(Wq), _p(s_w),
                                   _p(z_w), _stream(stream)), "w4a4_pack_weights")
    return desc, Wq, s_w, z_w


def transform_quant(X, P1, P2, c=None, alpha_a: float = 1.0, out=None, ws=None, stream=None):
    """Fused transform + per-token INT4 quantization: returns (Xq [M,K/2], s_x [M])."""
    torch = _torch()
    M, K = X.shape
    n1, n2 = P1.shape[0], P2.shape[0]
    _need(X, torch.float16, (M, K), "X")
    _need(P1, torch.float32, (n1, n1), "P1")
    _need(P2, torch.float32, (n2, n2), "P2")
    if c is not None:
        _need(c, torch.float32, (K,), "c")
    if out is None:
        Xq = torch.empty((M, K // 2), dtype=torch.uint8, device=X.device)
        s_x = torch.empty((M,), dtype=torch.float32, device=X.device)
    else:
        Xq, s_x = out
    nb = transform_quant_workspace_bytes(M, n1, n2, c is not None)
    ws = _ws(nb, X.device, ws)
    _check(lib().w4a4_transform_quant(_p(X), M, n1, n2, _p(P1), _p(P2), _p(c), float(alpha_a),
                                      _p(Xq), _p(s_x), _p(ws), nb if ws is None else ws.numel(),
                                      _stream(stream)), "w4a4_transform_quant")
    return Xq, s_x


def transform_quant_static(X, P1, P2, steps, per_channel: bool, c=None, out=None, ws=None,
                           stream=None):
    """Transform + INT4 quantization with offline steps (steps [1] per tensor,
    [K] per channel): returns (Xq [M,K/2], s_x [M])."""
    torch = _torch()
    M, K = X.shape
    n1, n2 = P1.shape[0], P2.shape[0]
    _need(X, torch.float16, (M, K), "X")
    _need(P1, torch.float32, (n1, n1), "P1")
    _need(P2, torch.float32, (n2, n2), "P2")
    _need(steps, torch.float32, (K if per_channel else 1,), "steps")
    if c is not None:
        _need(c, torch.float32, (K,), "c")
    if out is None:
        Xq = torch.empty((M, K // 2), dtype=torch.uint8, device=X.device)
        s_x = torch.empty((M,), dtype=torch.float32, device=X.device)
    else:
        Xq, s_x = out
    nb = transform_quant_workspace_bytes(M, n1, n2, c is not None)
    ws = _ws(nb, X.device, ws)
    _check(lib().w4a4_transform_quant_static(_p(X), M, n1, n2, _p(P1), _p(P2), _p(c), _p(steps),
                                             int(bool(per_channel)), _p(Xq), _p(s_x), _p(ws),
                                             nb if ws is None else ws.numel(), _stream(stream)),
           "w4a4_transform_quant_static")
    return Xq, s_x


def migrate_steps(Wt, steps, out=None, stream=None):
    """Wm [N, K] fp32 = Wt · diag(steps): per-channel activation steps folded
    into the weights (pass out=Wt for in place)."""
    torch = _torch()
    N, K = Wt.shape
    _need(Wt, torch.float32, (N, K), "Wt")
    _need(steps, torch.float32, (K,), "steps")
    Wm = out if out is not None else torch.empty_like(Wt)
    _check(lib().w4a4_migrate_steps(_p(Wt), N, K, _p(steps), _p(Wm), _stream(stream)),
           "w4a4_migrate_steps")
    return Wm


def transform(X, P1, P2, c=None, stream=None):
    """Debug form: the fp32 transformed activations Z [M, K]."""
    torch = _torch()
    M, K = X.shape
    n1, n2 = P1.shape[0], P2.shape[0]
    _need(X, torch.float16, (M, K), "X")
    Z = torch.empty((M, K), dtype=torch.float32, device=X.device)
    nb = transform_quant_workspace_bytes(M, n1, n2, c is not None)
    ws = _ws(nb, X.device)
    _check(lib().w4a4_transform(_p(X), M, n1, n2, _p(P1), _p(P2), _p(c), _p(Z), _p(ws), nb,
                                _stream(stream)), "w4a4_transform")
    return Z


def gemm(Xq, s_x, desc: WeightDesc, Wq, s_w, z_w=None, out=None, ws=None, stream=None):
    """Y [M, N] fp16 = dequant(Xq · Wq^T)."""
    torch = _torch()
    M = Xq.shape[0]
    Y = out if out is not None else torch.empty((M, desc.N), dtype=torch.float16, device=Xq.device)
    nb = gemm_workspace_bytes(M, desc)
    ws = _ws(nb, Xq.device, ws)
    _check(lib().w4a4_gemm(_p(Xq), _p(s_x), M, ctypes.byref(desc), _p(Wq), _p(s_w), _p(z_w), _p(Y),
                           _p(ws), nb if ws is None else ws.numel(), _stream(stream)), "w4a4_gemm")
    return Y


def gemm_i32(Xq, desc: WeightDesc, Wq, z_w=None, stream=None):
    """Exact int32 accumulators D [M, N, G]."""
    torch = _torch()
    M = Xq.shape[0]
    D = torch.empty((M, desc.N, desc.groups), dtype=torch.int32, device=Xq.device)
    _check(lib().w4a4_gemm_i32(_p(Xq), M, ctypes.byref(desc), _p(Wq), _p(z_w), _p(D),
                               _stream(stream)), "w4a4_gemm_i32")
    return D


def gemm_kernel_name(M: int, desc: WeightDesc) -> str:
    """Name of the kernel configuration w4a4_gemm uses for M tokens."""
    name = lib().w4a4_gemm_kernel_name(M, ctypes.byref(desc))
    if name is None:
        _check(-1, "w4a4_gemm_kernel_name")
    return name.decode()


def linear(X, P1, P2, desc: WeightDesc, Wq, s_w, z_w=None, c=None, alpha_a: float = 1.0,
           out=None, ws=None, stream=None):
    """Whole W4A4 layer: Y [M, N] fp16."""
    torch = _torch()
    M, K = X.shape
    n1, n2 = P1.shape[0], P2.shape[0]
    Y = out if out is not None else torch.empty((M, desc.N), dtype=torch.float16, device=X.device)
    nb = linear_workspace_bytes(M, n1, n2, desc, c is not None)
    ws = _ws(nb, X.device, ws)
    _check(lib().w4a4_linear(_p(X), M, n1, n2, _p(P1), _p(P2), _p(c), float(alpha_a),
                             ctypes.byref(desc), _p(Wq), _p(s_w), _p(z_w), _p(Y), _p(ws),
                             nb if ws is None else ws.numel(), _stream(stream)), "w4a4_linear")
    return Y


NOALLOC_SCRATCH_BYTES = 32 << 20   # W4A4_NOALLOC_SCRATCH_BYTES


def linear_noalloc(X, P1, P2, desc: WeightDesc, Wq, s_w, z_w=None, c=None, alpha_a: float = 1.0,
                   out=None, stream=None):
    """w4a4_linear with the library's own device scratch instead of a
    workspace (the library allocates nothing).  `out` should be given by
    callers that cannot allocate; otherwise the output is allocated here."""
    torch = _torch()
    M, K = X.shape
    n1, n2 = P1.shape[0], P2.shape[0]
    Y = out if out is not None else torch.empty((M, desc.N), dtype=torch.float16, device=X.device)
    _check(lib().w4a4_linear_noalloc(_p(X), M, n1, n2, _p(P1), _p(P2), _p(c), float(alpha_a),
                                     ctypes.byref(desc), _p(Wq), _p(s_w), _p(z_w), _p(Y),
                                     _stream(stream)), "w4a4_linear_noalloc")
    return Y


def linear_static(X, P1, P2, steps, per_channel: bool, desc: WeightDesc, Wq, s_w, z_w=None,
                  c=None, out=None, ws=None, stream=None):
    """Whole W4A4 layer with static activation steps: Y [M, N] fp16."""
    torch = _torch()
    M, K = X.shape
    n1, n2 = P1.shape[0], P2.shape[0]
    _need(steps, torch.float32, (K if per_channel else 1,), "steps")
    Y = out if out is not None else torch.empty((M, desc.N), dtype=torch.float16, device=X.device)
    nb = linear_workspace_bytes(M, n1, n2, desc, c is not None)
    ws = _ws(nb, X.device, ws)
    _check(lib().w4a4_linear_static(_p(X), M, n1, n2, _p(P1), _p(P2), _p(c), _p(steps),
                                    int(bool(per_channel)), ctypes.byref(desc), _p(Wq), _p(s_w),
                                    _p(z_w), _p(Y), _p(ws), nb if ws is None else ws.numel(),
                                    _stream(stream)), "w4a4_linear_static")
    return Y


def linear_decode_workspace_bytes(M: int, n1: int, n2: int) -> int:
    return lib().w4a4_linear_decode_workspace_bytes(M, n1, n2)


def decode_sync_buffer(device):
    """A zero-filled sync buffer for linear_decode (reuse it across calls)."""
    torch = _torch()
    return torch.zeros(DECODE_SYNC_BYTES // 4, dtype=torch.int32, device=device)


def linear_decode(X, P1, P2, desc: WeightDesc, Wq, s_w, z_w=None, sync=None, alpha_a: float = 1.0,
                  steps=None, per_channel: bool = False, out=None, ws=None, stream=None):
    """The whole layer for M <= 16 tokens in one kernel launch: Y [M, N] fp16."""
    torch = _torch()
    M, K = X.shape
    n1, n2 = P1.shape[0], P2.shape[0]
    _need(X, torch.float16, (M, K), "X")
    if steps is not None:
        _need(steps, torch.float32, (K if per_channel else 1,), "steps")
    if sync is None:
        raise ValueError("linear_decode needs a sync buffer (decode_sync_buffer)")
    Y = out if out is not None else torch.empty((M, desc.N), dtype=torch.float16, device=X.device)
    nb = linear_decode_workspace_bytes(M, n1, n2)
    ws = _ws(nb, X.device, ws)
    _check(lib().w4a4_linear_decode(_p(X), M, n1, n2, _p(P1), _p(P2), float(alpha_a), _p(steps),
                                    int(bool(per_channel)), ctypes.byref(desc), _p(Wq), _p(s_w),
                                    _p(z_w), _p(Y), _p(ws), nb if ws is None else ws.numel(),
                                    _p(sync), _stream(stream)), "w4a4_linear_decode")
    return Y


# ---------------------------------------------------------------------------
# INT4 KV cache with per-head transforms, decode attention
# ---------------------------------------------------------------------------
def kv_cache_bytes(batch: int, heads_kv: int, max_seq: int, head_dim: int = KV_HEAD_DIM):
    """(key bytes, value bytes, scale bytes) of one layer's cache buffers."""
    k, v, sc = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().w4a4_kv_cache_bytes(batch, heads_kv, head_dim, max_seq, ctypes.byref(k),
                                     ctypes.byref(v), ctypes.byref(sc)), "w4a4_kv_cache_bytes")
    return k.value, v.value, sc.value


class KvCache:
    """One layer's INT4 KV cache buffers in the layout of include/w4a4.h:
    k_cache uint8 [B, H, S, 64], v_cache int32 [B, H, S/8, 128] (the bits of
    the uint32 words), k_scale / v_scale float32 [B, H, S]."""

    def __init__(self, batch: int, heads_kv: int, max_seq: int, device, zero: bool = True):
        torch = _torch()
        kv_cache_bytes(batch, heads_kv, max_seq)          # validates the shape
        make = torch.zeros if zero else torch.empty
        self.batch, self.heads_kv, self.max_seq = batch, heads_kv, max_seq
        d = KV_HEAD_DIM
        self.k_cache = make((batch, heads_kv, max_seq, d // 2), dtype=torch.uint8, device=device)
        self.v_cache = make((batch, heads_kv, max_seq // 8, d), dtype=torch.int32, device=device)
        self.k_scale = make((batch, heads_kv, max_seq), dtype=torch.float32, device=device)
        self.v_scale = make((batch, heads_kv, max_seq), dtype=torch.float32, device=device)

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size()
                   for t in (self.k_cache, self.v_cache, self.k_scale, self.v_scale))


def kv_query_factor(P_h, out=None, stream=None):
    """P_h^-T (float32) of a [d, d] or [H, d, d] stack of per-head key transforms."""
    torch = _torch()
    d = P_h.shape[-1]
    count = 1 if P_h.dim() == 2 else P_h.shape[0]
    _need(P_h, torch.float32, tuple(P_h.shape), "P_h")
    out = out if out is not None else torch.empty_like(P_h)
    nb = lib().w4a4_kv_query_factor_workspace_bytes(d, count)
    ws = _ws(nb, P_h.device)
    _check(lib().w4a4_kv_query_factor(_p(P_h), d, count, _p(out), _p(ws), nb, _stream(stream)),
           "w4a4_kv_query_factor")
    return out


def kv_append(k, v, seg_seq, seg_start, cu_tokens, P_h, P_v, cache: KvCache,
              alpha_k: float = 1.0, alpha_v: float = 1.0, stream=None):
    """Transform, quantize and write tokens into ``cache`` (see w4a4_kv_append).
    k, v: fp16 [T, H, 128]; seg_seq, seg_start: int32 [S]; cu_tokens: int32 [S+1]."""
    torch = _torch()
    T, H, d = k.shape
    _need(k, torch.float16, (T, H, d), "k")
    _need(v, torch.float16, (T, H, d), "v")
    S = seg_seq.shape[0]
    _need(seg_seq, torch.int32, (S,), "seg_seq")
    _need(seg_start, torch.int32, (S,), "seg_start")
    _need(cu_tokens, torch.int32, (S + 1,), "cu_tokens")
    per_head = P_h.dim() == 3
    _need(P_h, torch.float32, tuple(P_h.shape), "P_h")
    _need(P_v, torch.float32, tuple(P_h.shape), "P_v")
    _check(lib().w4a4_kv_append(_p(k), _p(v), T, _p(seg_seq), _p(seg_start), _p(cu_tokens), S, H, d,
                                _p(P_h), _p(P_v), int(per_head), float(alpha_k), float(alpha_v),
                                _p(cache.k_cache), _p(cache.k_scale), _p(cache.v_cache),
                                _p(cache.v_scale), cache.batch, cache.max_seq, _stream(stream)),
           "w4a4_kv_append")


def attn_decode_workspace_bytes(batch: int, heads_q: int, heads_kv: int, max_seq: int) -> int:
    return lib().w4a4_attn_decode_workspace_bytes(batch, heads_q, heads_kv, KV_HEAD_DIM, max_seq)


def attn_decode(q, P_h_inv_t, cache: KvCache, lengths, sm_scale: float, out=None, ws=None,
                stream=None):
    """Decode attention over the INT4 cache: out [B, H_q, 128] fp16 in the P_v basis."""
    torch = _torch()
    B, Hq, d = q.shape
    _need(q, torch.float16, (B, Hq, d), "q")
    _need(lengths, torch.int32, (B,), "lengths")
    per_head = P_h_inv_t.dim() == 3
    _need(P_h_inv_t, torch.float32, tuple(P_h_inv_t.shape), "P_h_inv_t")
    out = out if out is not None else torch.empty((B, Hq, d), dtype=torch.float16, device=q.device)
    nb = attn_decode_workspace_bytes(B, Hq, cache.heads_kv, cache.max_seq)
    ws = _ws(nb, q.device, ws)
    _check(lib().w4a4_attn_decode(_p(q), B, Hq, cache.heads_kv, d, _p(P_h_inv_t), int(per_head),
                                  _p(cache.k_cache), _p(cache.k_scale), _p(cache.v_cache),
                                  _p(cache.v_scale), _p(lengths), cache.max_seq, float(sm_scale),
                                  _p(out), _p(ws), nb if ws is None else ws.numel(),
                                  _stream(stream)), "w4a4_attn_decode")
    return out


# ---------------------------------------------------------------------------
# 3-bit codes (W3A3): the same layer with codes in [-4, 3] / [0, 7]
# ---------------------------------------------------------------------------
def pack_weights_bits(Wt, group_size: int, asymmetric: bool, bits: int, alpha_w: float = 1.0,
                      stream=None):
    """pack_weights with b-bit codes (b = 3 or 4), one code per nibble."""
    torch = _torch()
    N, K = Wt.shape
    _need(Wt, torch.float32, (N, K), "Wt")
    desc = _desc(N, K, group_size, asymmetric)
    G = K // group_size if group_size > 0 else 0
    Wq = torch.empty((N, K // 2), dtype=torch.uint8, device=Wt.device)
    s_w = torch.empty((N, max(G, 1)), dtype=torch.float16, device=Wt.device)
    z_w = torch.empty((N, max(G, 1)), dtype=torch.float16, device=Wt.device) if asymmetric else None
    _check(lib().w4a4_pack_weights_bits(ctypes.byref(desc), _p(Wt), float(alpha_w), int(bits),
                                        _p(Wq), _p(s_w), _p(z_w), _stream(stream)),
           "w4a4_pack_weights_bits")
    return desc, Wq, s_w, z_w


def transform_quant_bits(X, P1, P2, bits: int, c=None, alpha_a: float = 1.0, out=None, ws=None,
                         stream=None):
    """transform_quant with b-bit activation codes: returns (Xq [M,K/2], s_x [M])."""
    torch = _torch()
    M, K = X.shape
    n1, n2 = P1.shape[0], P2.shape[0]
    _need(X, torch.float16, (M, K), "X")
    _need(P1, torch.float32, (n1, n1), "P1")
    _need(P2, torch.float32, (n2, n2), "P2")
    if c is not None:
        _need(c, torch.float32, (K,), "c")
    if out is None:
        Xq = torch.empty((M, K // 2), dtype=torch.uint8, device=X.device)
        s_x = torch.empty((M,), dtype=torch.float32, device=X.device)
    else:
        Xq, s_x = out
    nb = transform_quant_workspace_bytes(M, n1, n2, c is not None)
    ws = _ws(nb, X.device, ws)
    _check(lib().w4a4_transform_quant_bits(_p(X), M, n1, n2, _p(P1), _p(P2), _p(c),
                                           float(alpha_a), int(bits), _p(Xq), _p(s_x), _p(ws),
                                           nb if ws is None else ws.numel(), _stream(stream)),
           "w4a4_transform_quant_bits")
    return Xq, s_x


def linear_bits(X, P1, P2, bits: int, desc: WeightDesc, Wq, s_w, z_w=None, c=None,
                alpha_a: float = 1.0, out=None, ws=None, stream=None):
    """The whole layer with b-bit codes (weights packed by pack_weights_bits)."""
    torch = _torch()
    M, K = X.shape
    n1, n2 = P1.shape[0], P2.shape[0]
    Y = out if out is not None else torch.empty((M, desc.N), dtype=torch.float16, device=X.device)
    nb = linear_workspace_bytes(M, n1, n2, desc, c is not None)
    ws = _ws(nb, X.device, ws)
    _check(lib().w4a4_linear_bits(_p(X), M, n1, n2, _p(P1), _p(P2), _p(c), float(alpha_a),
                                  int(bits), ctypes.byref(desc), _p(Wq), _p(s_w), _p(z_w), _p(Y),
                                  _p(ws), nb if ws is None else ws.numel(), _stream(stream)),
           "w4a4_linear_bits")
    return Y


# ---------------------------------------------------------------------------
# Ternary weights (W1.58A16)
# ---------------------------------------------------------------------------
def ternary_weight_bytes(N: int, K: int):
    """(bytes of Tq, bytes of am) for N rows of K weights (rows tiled by 16)."""
    tq, am = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib().w4a4_ternary_weight_bytes(N, K, ctypes.byref(tq), ctypes.byref(am)),
           "w4a4_ternary_weight_bytes")
    return tq.value, am.value


def pack_ternary(Wt, iters: int = 10, stream=None):
    """Ternarize fp32 weights [N, K]: returns (Tq uint8 [bytes], am int32 [words])
    in the tiled layout (am holds the bits of the uint32 parameter words)."""
    torch = _torch()
    N, K = Wt.shape
    _need(Wt, torch.float32, (N, K), "Wt")
    tqb, amb = ternary_weight_bytes(N, K)
    Tq = torch.empty((tqb,), dtype=torch.uint8, device=Wt.device)
    am = torch.empty((amb // 4,), dtype=torch.int32, device=Wt.device)
    _check(lib().w4a4_pack_ternary(_p(Wt), N, K, int(iters), _p(Tq), _p(am), _stream(stream)),
           "w4a4_pack_ternary")
    return Tq, am


def unpack_ternary(Tq, am, N: int, K: int, stream=None):
    """The tiled layout back to (T int8 [N, K], alpha fp16 [N, K/128],
    mu fp16 [N, K/128])."""
    torch = _torch()
    T = torch.empty((N, K), dtype=torch.int8, device=Tq.device)
    alpha = torch.empty((N, K // TERNARY_BLOCK), dtype=torch.float16, device=Tq.device)
    mu = torch.empty_like(alpha)
    _check(lib().w4a4_unpack_ternary(_p(Tq), _p(am), N, K, _p(T), _p(alpha), _p(mu),
                                     _stream(stream)), "w4a4_unpack_ternary")
    return T, alpha, mu


def ternary_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return lib().w4a4_ternary_gemm_workspace_bytes(M, N, K)


def ternary_gemm(X, Tq, am, N: int, out=None, ws=None, stream=None):
    """Y [M, N] fp16 = X [M, K] fp16 times the ternary weights of N rows
    (M <= TERNARY_MAX_M)."""
    torch = _torch()
    M, K = X.shape
    _need(X, torch.float16, (M, K), "X")
    tqb, amb = ternary_weight_bytes(N, K)
    _need(Tq, torch.uint8, (tqb,), "Tq")
    _need(am, torch.int32, (amb // 4,), "am")
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=X.device)
    nb = ternary_gemm_workspace_bytes(M, N, K)
    ws = _ws(nb, X.device, ws)
    _check(lib().w4a4_ternary_gemm(_p(X), M, N, K, _p(Tq), _p(am), _p(Y), _p(ws),
                                   nb if ws is None else ws.numel(), _stream(stream)),
           "w4a4_ternary_gemm")
    return Y


def read_probe(buf, out, stream=None):
    """Measurement aid: a plain streaming read of the whole of `buf` (a
    contiguous device tensor of a multiple of 16 bytes); the XOR of its 32-bit
    words is XORed into `out` (an int32 device tensor of one element)."""
    torch = _torch()
    if not (buf.is_cuda and buf.is_contiguous()):
        raise ValueError("buf must be a contiguous CUDA (HIP) tensor")
    _need(out, torch.int32, (1,), "out")
    _check(lib().w4a4_read_probe(_p(buf), buf.numel() * buf.element_size(), _p(out),
                                 _stream(stream)), "w4a4_read_probe")


# ---------------------------------------------------------------------------
# INT4 GEMM on the fp6 matrix pipe (prefill)
# ---------------------------------------------------------------------------
def weights_f6_bytes(desc: WeightDesc) -> int:
    return lib().w4a4_weights_f6_bytes(ctypes.byref(desc))


def pack_weights_f6(desc: WeightDesc, Wq, z_w=None, stream=None):
    """Packed INT4 weights (and zero points) -> uint8 [weights_f6_bytes] in the fp6 layout."""
    torch = _torch()
    W6 = torch.empty((weights_f6_bytes(desc),), dtype=torch.uint8, device=Wq.device)
    _check(lib().w4a4_pack_weights_f6(ctypes.byref(desc), _p(Wq), _p(z_w), _p(W6), _stream(stream)),
           "w4a4_pack_weights_f6")
    return W6


def gemm_f6_workspace_bytes(M: int, desc: WeightDesc) -> int:
    return lib().w4a4_gemm_f6_workspace_bytes(M, ctypes.byref(desc))


def gemm_f6(Xq, s_x, desc: WeightDesc, W6, s_w, out=None, ws=None, stream=None):
    """Y [M, N] fp16 = dequant(Xq · W^T) with the product on the fp6 pipe."""
    torch = _torch()
    M = Xq.shape[0]
    Y = out if out is not None else torch.empty((M, desc.N), dtype=torch.float16, device=Xq.device)
    nb = gemm_f6_workspace_bytes(M, desc)
    ws = _ws(nb, Xq.device, ws)
    _check(lib().w4a4_gemm_f6(_p(Xq), _p(s_x), M, ctypes.byref(desc), _p(W6), _p(s_w), _p(Y),
                              _p(ws), nb if ws is None else ws.numel(), _stream(stream)),
           "w4a4_gemm_f6")
    return Y


def gemm_f6_kernel_name(M: int, desc: WeightDesc) -> str:
    name = lib().w4a4_gemm_f6_kernel_name(M, ctypes.byref(desc))
    if name is None:
        raise W4A4Error(-1, "w4a4_gemm_f6_kernel_name", lib().w4a4_last_error().decode())
    return name.decode()


def linear_f6_workspace_bytes(M: int, n1: int, n2: int, desc: WeightDesc, has_c: bool = False) -> int:
    return lib().w4a4_linear_f6_workspace_bytes(M, n1, n2, int(bool(has_c)), ctypes.byref(desc))


def linear_f6(X, P1, P2, desc: WeightDesc, W6, s_w, c=None, alpha_a: float = 1.0, out=None,
              ws=None, stream=None):
    """Whole W4A4 layer with the product on the fp6 pipe: Y [M, N] fp16."""
    torch = _torch()
    M, K = X.shape
    n1, n2 = P1.shape[0], P2.shape[0]
    Y = out if out is not None else torch.empty((M, desc.N), dtype=torch.float16, device=X.device)
    nb = linear_f6_workspace_bytes(M, n1, n2, desc, c is not None)
    ws = _ws(nb, X.device, ws)
    _check(lib().w4a4_linear_f6(_p(X), M, n1, n2, _p(P1), _p(P2), _p(c), float(alpha_a),
                                ctypes.byref(desc), _p(W6), _p(s_w), _p(Y), _p(ws),
                                nb if ws is None else ws.numel(), _stream(stream)),
           "w4a4_linear_f6")
    return Y
