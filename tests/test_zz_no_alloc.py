"""w4a4_linear_noalloc through the C ABI: the layer for callers that cannot
allocate, with its workspace in the library's own device scratch.

Checks: two calls in a row (the second with fewer tokens, so it reads a
scratch the first one left larger) give fp16 outputs equal, bit for bit, to
w4a4_linear's on the same inputs (same kernels, same arithmetic), and meet
the oracle's bound on the library's own codes; a call whose workspace would
not fit the scratch is refused before anything runs.
"""
import ctypes

import numpy as np
import pytest

import oracle as O
from gpu_common import assert_layer_close, custom_workload, log, prepared, to_dev, torch_dev

pytestmark = pytest.mark.gpu


def W():
    import w4a4_post_quantized_amd as lib
    return lib


def noalloc_call(X, P1, P2, desc, Wq, sw, zw, Y):
    """The C entry point itself (pointers and sizes; no workspace argument)."""
    torch, dev = torch_dev()
    L = W()
    M, K = X.shape
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    return L.lib().w4a4_linear_noalloc(p(X), M, P1.shape[0], P2.shape[0], p(P1), p(P2), None,
                                       ctypes.c_float(1.0), ctypes.byref(desc), p(Wq), p(sw), p(zw),
                                       p(Y), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("wl", [
    custom_workload(M=300, n1=32, n2=32, N=520, outliers=(1, 900), pivot=100.0, seed=61),
    custom_workload(M=9, n1=224, n2=128, N=264, group_size=128, asym=True, seed=62),
], ids=lambda w: w.name)
def test_noalloc_matches_linear(wl):
    torch, dev = torch_dev()
    L = W()
    inp = prepared(wl)
    wq = O.quantize_weights(inp["Wt"], wl.group_size, wl.asymmetric)
    desc, Wq, sw, zw = L.pack_weights(to_dev(inp["Wt"]), wl.group_size, wl.asymmetric)
    P1, P2 = to_dev(inp["P1"]), to_dev(inp["P2"])
    for M in (wl.M, max(1, wl.M // 4)):            # the second call is smaller
        log(f"noalloc {wl.name}: M={M}")
        X = to_dev(inp["X"][:M])
        Y = torch.full((M, wl.N), float("nan"), dtype=torch.float16, device=dev)
        assert noalloc_call(X, P1, P2, desc, Wq, sw, zw, Y) == 0, L.lib().w4a4_last_error()
        Y_ref = L.linear(X, P1, P2, desc, Wq, sw, zw)
        torch.cuda.synchronize()
        Yn, Yr = Y.cpu().numpy(), Y_ref.cpu().numpy()
        assert np.array_equal(Yn.view(np.uint16), Yr.view(np.uint16))
        Xq, sx = L.transform_quant(X, P1, P2)
        rel = assert_layer_close(Yn, O.unpack_nibbles(Xq.cpu().numpy(), True), sx.cpu().numpy(), wq)
        log(f"  equal to w4a4_linear; relative L2 {rel:.2e} on the library's codes")


def test_noalloc_refuses_what_does_not_fit():
    torch, dev = torch_dev()
    L = W()
    M, n, N = 20000, 64, 64                      # packed activations alone: 41 MB > 32 MiB
    K = n * n
    X = torch.zeros((M, K), dtype=torch.float16, device=dev)
    P = torch.eye(n, dtype=torch.float32, device=dev)
    desc, Wq, sw, zw = L.pack_weights(torch.zeros((N, K), dtype=torch.float32, device=dev), K, False)
    Y = torch.zeros((M, N), dtype=torch.float16, device=dev)
    assert L.linear_workspace_bytes(M, n, n, desc) > L.NOALLOC_SCRATCH_BYTES
    assert noalloc_call(X, P, P, desc, Wq, sw, None, Y) == -2
    assert "scratch" in L.lib().w4a4_last_error().decode()
    torch.cuda.synchronize()
    assert not Y.any()
