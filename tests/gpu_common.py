"""Shared helpers of the GPU parity tests (inputs, comparisons, tolerances).

Inputs come from the seeded generators in workloads/ and, for the merged
weights, from the oracle (an oracle result used as a shared input, never the
other way round).  Nothing here reads a HIP result back into the oracle.
"""
import contextlib
import functools
import sys

import numpy as np

import oracle as O
import workloads as WL

WINDOW = 1e-4          # tie window for activation codes, in code units
REL_L2 = 1e-3          # end-to-end fp16 output bound (relative L2)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@contextlib.contextmanager
def kernel_override(which, index):
    """Force one kernel configuration (w4a4_set_kernel_override) for the
    duration of a block, then restore the previous choice."""
    import w4a4_post_quantized_amd as L
    prev = L.set_kernel_override(which, index)
    try:
        yield
    finally:
        L.set_kernel_override(which, prev)


def torch_dev():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device")
    return torch, torch.device("cuda:0")


def to_dev(a, dtype=None):
    torch, dev = torch_dev()
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev)


def custom_workload(M, n1, n2, N, group_size=None, asym=False, x_kind="normal",
                    outliers=(), pivot=0.0, seed=0):
    K = n1 * n2
    return WL.Workload(name=f"custom_{M}_{n1}x{n2}_{N}", M=M, K=K, N=N, n1=n1, n2=n2,
                       group_size=group_size or K, asymmetric=asym, x_kind=x_kind,
                       outlier_channels=tuple(outliers) if outliers else None,
                       pivot_token_scale=pivot, seed=seed)


@functools.lru_cache(maxsize=4)
def prepared(name_or_wl, M=None):
    """Inputs and the oracle's merged fp32 weights for a workload (cached)."""
    inp = WL.make_inputs(name_or_wl, M=M)
    inp["Wt"] = O.merge_weights(inp["W"], inp["P1"], inp["P2"], inp["c"])
    return inp


def assert_codes_match(gpu_codes, or_codes, t, window=WINDOW, what="codes"):
    """Bit-exact except where the oracle's t is within `window` of a tie
    between the two (adjacent) codes.  Returns the number of excused cells."""
    g = np.asarray(gpu_codes).astype(np.int16)
    o = np.asarray(or_codes).astype(np.int16)
    diff = g != o
    if not diff.any():
        return 0
    lo = np.minimum(g, o)
    excused = (np.abs(g - o) == 1) & (np.abs(t - (lo + 0.5)) < window)
    bad = diff & ~excused
    if bad.any():
        idx = np.argwhere(bad)[:5]
        det = [(tuple(i), int(g[tuple(i)]), int(o[tuple(i)]), float(t[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} mismatches outside the tie window, "
                             f"first (index, gpu, oracle, t): {det}")
    return int(diff.sum())


def ulp16(y):
    a = np.abs(np.asarray(y, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def _element_bound(Yg, Y64, A, rel_term):
    """Elements outside |Y - Y64| <= ulp16(Y64)/2 + rel_term*A: (count, first
    index) -- half an fp16 ulp for the output rounding plus fp32 rounding of
    the summed terms, whose magnitude A bounds."""
    err = np.abs(Yg - Y64)
    tol = 0.5 * ulp16(Y64) * (1 + 1e-9) + rel_term * A
    bad = err > tol
    if not bad.any():
        return 0, None, None
    i = tuple(np.argwhere(bad)[0])
    return int(bad.sum()), i, tol[i]


def assert_y_close(Y_gpu, Y64, A=None, rel_term=4e-6, what="Y"):
    """Per element: |Y - Y64| <= ulp16(Y64)/2 + rel_term*A (A = magnitude of
    the summed terms, defaults to |Y64|); and relative L2 <= REL_L2."""
    Yg = np.asarray(Y_gpu, dtype=np.float64)
    A = np.abs(Y64) if A is None else A
    nbad, i, t = _element_bound(Yg, Y64, A, rel_term)
    if nbad:
        raise AssertionError(f"{what}: {nbad} elements out of bound, first {i}: "
                             f"gpu {Yg[i]} oracle {Y64[i]} tol {t}")
    rel = np.linalg.norm(Yg - Y64) / max(np.linalg.norm(Y64), 1e-300)
    assert rel <= REL_L2, f"{what}: relative L2 {rel}"
    return rel


def assert_layer_close(Y_gpu, gq, gsx, wq, cols=None, what="linear", chunk=1024,
                       rel_term=4e-6):
    """Level 3 of the parity contract, given the library's own codes.

    The reference is the oracle's exact integer product and float64 epilogue
    applied to the activation codes `gq` [R, K] and fp32 token scales `gsx`
    [R] that the library itself produced (those codes are checked against
    the oracle's separately, bit-exact outside the tie window), and to the
    oracle's weight codes and scales (`wq`, bit-exact with the library's).
    Every compared element meets the per-element bound of assert_y_close,
    and the relative L2 error over all of them is <= REL_L2.  `cols` selects
    output channels (all by default); the product is taken `chunk` channels
    at a time to bound host memory at full size."""
    Yg_all = np.asarray(Y_gpu, dtype=np.float64)
    ncol = wq["codes"].shape[0] if cols is None else len(cols)
    assert Yg_all.shape == (len(gq), ncol), (Yg_all.shape, len(gq), ncol)
    col_idx = np.arange(ncol) if cols is None else np.asarray(cols)
    gsx = np.asarray(gsx, dtype=np.float64)
    num = den = 0.0
    for c0 in range(0, ncol, chunk):
        cc = col_idx[c0:c0 + chunk]
        Y64, A = O.epilogue_by_group(gq, wq, gsx, cols=cc)
        Yg = Yg_all[:, c0:c0 + chunk]
        nbad, i, t = _element_bound(Yg, Y64, A, rel_term)
        if nbad:
            raise AssertionError(f"{what}: {nbad} elements out of bound in channels "
                                 f"{c0}..{c0 + len(cc) - 1}, first {i}: gpu {Yg[i]} "
                                 f"oracle on the library's codes {Y64[i]} tol {t}")
        num += float(np.sum((Yg - Y64) ** 2))
        den += float(np.sum(Y64 ** 2))
    rel = np.sqrt(num) / max(np.sqrt(den), 1e-300)
    assert rel <= REL_L2, f"{what}: relative L2 {rel}"
    return rel


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def sample_rows(M, k=13, seed=0):
    rng = np.random.default_rng(seed + 1000)
    base = {0, 1, M - 1} if M > 2 else set(range(M))
    extra = set(rng.choice(M, min(k, M), replace=False).tolist()) if M > 0 else set()
    return np.array(sorted(base | extra), dtype=np.int64)
