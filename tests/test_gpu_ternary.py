"""GPU parity of the ternary-weight layer (W1.58A16; PT2-LLM page, section
关键设计 item 2: ATQ fitted by ITF), through the C ABI entry points
w4a4_pack_ternary, w4a4_unpack_ternary and w4a4_ternary_gemm.

Checks:
* pack: the library's tiled storage, read back through its own unpack entry
  point (the documented bijection), gives codes T and fp16 alpha, mu equal
  to the oracle's bit for bit (both sides run ITF in float64 and round alpha
  and mu to fp16 once), including all-zero and constant block rows, and a
  full-size weight matrix on sampled rows;
* unpack is an inverse: padding rows stay zero and unpacking touches only
  the N real rows;
* product: Y (fp16) from the library's own packed weights against the
  oracle's float64 layer on the oracle's (equal) T, alpha, mu, per element
  within half an fp16 ulp of the result plus 4e-6 times the magnitude of the
  summed terms, over decode batches that span the row tiles (M = 1 .. 64,
  ragged), ragged N, K splits, and the full LLaMA-3-70B decode shapes on
  sampled output columns.
"""
import numpy as np
import pytest

from oracle import ternary_oracle as TO
from workloads import ternary as WT
from gpu_common import log, rel_l2, to_dev, torch_dev, ulp16

pytestmark = pytest.mark.gpu

REL_TERM = 4e-6


def W():
    import w4a4_post_quantized_amd as lib
    return lib


def gpu_pack(Wt_np, iters=10):
    Tq, am = W().pack_ternary(to_dev(Wt_np), iters=iters)
    return Tq, am


def assert_pack_equal(Tq, am, r, N, K, rows=None, what="pack"):
    """The library's packed weights, unpacked by the library, against the
    oracle's ternarization `r` (of the rows `rows` of the matrix)."""
    torch, dev = torch_dev()
    T, a, u = W().unpack_ternary(Tq, am, N, K)
    if rows is not None:
        idx = torch.as_tensor(rows, device=T.device)
        T, a, u = T.index_select(0, idx), a.index_select(0, idx), u.index_select(0, idx)
    T, a, u = T.cpu().numpy(), a.cpu().numpy(), u.cpu().numpy()
    bad_a = np.argwhere(a.view(np.uint16) != r["alpha"].view(np.uint16))
    bad_u = np.argwhere(u.view(np.uint16) != r["mu"].view(np.uint16))
    bad_t = np.argwhere(T != r["T"])
    assert bad_a.size == 0, f"{what}: {len(bad_a)} alpha differ, first {bad_a[:3].tolist()}"
    assert bad_u.size == 0, f"{what}: {len(bad_u)} mu differ, first {bad_u[:3].tolist()}"
    assert bad_t.size == 0, f"{what}: {len(bad_t)} codes differ, first {bad_t[:3].tolist()}"


def magnitude(X, r, cols=None):
    """Sum over blocks of (3|alpha| + |mu|) * sum |x| over the block: a bound on
    the magnitude of every term the kernel adds (alpha 2^24 acc, (mu - alpha) S)."""
    X = np.abs(np.asarray(X, np.float64))
    a = np.abs(r["alpha"].astype(np.float64))
    u = np.abs(r["mu"].astype(np.float64))
    if cols is not None:
        a, u = a[cols], u[cols]
    G = a.shape[1]
    Xs = X.reshape(X.shape[0], G, -1).sum(axis=2)          # [M, G]
    return Xs @ (3 * a + u).T


def assert_tern_close(Yg, Y64, A, what):
    Yg = np.asarray(Yg, np.float64)
    err = np.abs(Yg - Y64)
    tol = 0.5 * ulp16(Y64) * (1 + 1e-9) + REL_TERM * A
    bad = err > tol
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of bound, first {i}: "
                             f"gpu {Yg[i]} oracle {Y64[i]} tol {tol[i]}")
    return rel_l2(Yg, Y64)


@pytest.mark.parametrize("N,K", [(7, 128), (64, 512), (301, 1152), (1000, 4096)])
def test_pack_bit_exact(N, K):
    log(f"pack_ternary N={N} K={K}")
    wl = WT.TernWorkload("t", M=1, K=K, N=N, x_kind="normal", seed=N + K)
    Wt = WT.make_tern_weights(wl)
    Wt[0] = 0.0                                  # zero row
    if N > 2:
        Wt[2, :128] = 0.25                       # constant block row (exact mean)
        Wt[2, 5] = -0.25                         # ... but one entry: T fits it with alpha
    r = TO.itf_ternarize(Wt)
    Tq, am = gpu_pack(Wt)
    assert_pack_equal(Tq, am, r, N, K, what=f"pack N={N} K={K}")
    # padding rows (N up to a multiple of 16) hold zero bytes and zero words
    tqb, amb = W().ternary_weight_bytes(N, K)
    assert Tq.numel() == tqb and am.numel() * 4 == amb
    if N % 16:
        Np = (N + 15) // 16 * 16
        Tp, ap, up = W().unpack_ternary(Tq, am, Np, K)      # the padding rows as well
        assert (Tp.cpu().numpy()[N:] == -1).all()            # zero bytes: every c = 0
        assert not ap.cpu().numpy()[N:].view(np.uint16).any()
        assert not up.cpu().numpy()[N:].view(np.uint16).any()


@pytest.mark.parametrize("iters", [0, 1, 3])
def test_pack_iteration_counts(iters):
    log(f"pack_ternary iters={iters}")
    wl = WT.TernWorkload("t", M=1, K=768, N=96, x_kind="normal", seed=11 + iters)
    Wt = WT.make_tern_weights(wl)
    r = TO.itf_ternarize(Wt, iters=iters)
    Tq, am = gpu_pack(Wt, iters)
    assert_pack_equal(Tq, am, r, 96, 768, what=f"pack iters={iters}")


@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (5, 100, 512), (16, 64, 4096), (17, 130, 1024),
                                   (33, 257, 2048), (64, 192, 1280), (64, 1000, 8192),
                                   (2, 3000, 384), (40, 77, 640), (8, 4096, 896), (3, 50, 128),
                                   (4, 300, 1280), (2, 96, 16384), (20, 64, 8192), (12, 200, 8192),
                                   (9, 64, 12288), (1, 32, 65536), (12, 48, 32768), (3, 50, 8192),
                                   (7, 33, 4096), (64, 16, 128), (17, 1, 256), (64, 40, 384)])
def test_gemm_parity(M, N, K):
    log(f"ternary_gemm M={M} N={N} K={K}")
    wl = WT.TernWorkload("t", M=M, K=K, N=N, x_kind="silu_product" if M % 2 else "normal",
                         seed=M * 7 + N)
    inp = WT.make_tern_inputs(wl)
    r = TO.itf_ternarize(inp["Wt"])
    Tq, am = gpu_pack(inp["Wt"])
    assert_pack_equal(Tq, am, r, N, K, what=f"pack N={N} K={K}")
    Y64 = TO.ternary_linear(inp["X"], r)
    Y = W().ternary_gemm(to_dev(inp["X"]), Tq, am, N)
    rel = assert_tern_close(Y.cpu().numpy(), Y64, magnitude(inp["X"], r), f"M={M} N={N} K={K}")
    log(f"  rel L2 {rel:.2e}")


def test_gemm_zero_rows_and_m0():
    torch, dev = torch_dev()
    wl = WT.TernWorkload("t", M=9, K=256, N=64, x_kind="normal", seed=3)
    inp = WT.make_tern_inputs(wl)
    X = inp["X"].copy()
    X[4] = 0
    r = TO.itf_ternarize(inp["Wt"])
    Tq, am = gpu_pack(inp["Wt"])
    assert_pack_equal(Tq, am, r, 64, 256)
    Y = W().ternary_gemm(to_dev(X), Tq, am, 64).cpu().numpy()
    assert np.all(Y[4] == 0)
    assert_tern_close(Y, TO.ternary_linear(X, r), magnitude(X, r), "zero row")
    Y0 = W().ternary_gemm(torch.empty((0, 256), dtype=torch.float16, device=dev), Tq, am, 64)
    assert tuple(Y0.shape) == (0, 64)


@pytest.mark.parametrize("name", ["tern_down70b_m8", "tern_gateup70b_m64", "tern_down70b_m1"])
def test_full_size_sampled(name):
    """The full decode shape in the launch configuration the benchmark times:
    the GPU packs the whole matrix; sampled weight rows are packed by the
    oracle and must match bit for bit; the matching output columns are
    compared with the oracle's layer on those rows.  The library's codes and
    parameters come back through its own unpack entry point."""
    log(f"full size {name}")
    torch, dev = torch_dev()
    wl = WT.get_tern(name)
    inp = WT.make_tern_inputs(wl)
    Tq, am = gpu_pack(inp["Wt"])
    Y = W().ternary_gemm(to_dev(inp["X"]), Tq, am, wl.N).cpu().numpy()
    rng = np.random.default_rng(5)
    cols = np.unique(np.concatenate([[0, 1, wl.N - 1], rng.choice(wl.N, 21, replace=False)]))
    Ws = WT.make_tern_weights(wl, rows=cols)
    np.testing.assert_array_equal(Ws, inp["Wt"][cols])
    r = TO.itf_ternarize(Ws)
    assert_pack_equal(Tq, am, r, wl.N, wl.K, rows=cols, what=f"{name} sampled rows")
    Y64 = TO.ternary_linear(inp["X"], r)
    rel = assert_tern_close(Y[:, cols], Y64, magnitude(inp["X"], r), name)
    log(f"  rel L2 {rel:.2e}")
    del Tq, am
    torch.cuda.empty_cache()
