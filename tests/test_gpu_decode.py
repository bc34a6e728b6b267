"""GPU parity of the single-kernel decode layer (w4a4_linear_decode) through
the C ABI.

The kernel computes what w4a4_linear / w4a4_linear_static compute, in one
launch (FlatQuant page, section 高效 Kernel 设计; MergeQuant page, section
问题定义).  Checks, per case:
  * the packed activation codes the kernel leaves in its workspace equal the
    oracle's up to the 1e-4 tie window, and its token scales match;
  * the fp16 output meets the per-element bound and relative L2 <= 1e-3
    against the oracle's product and epilogue on the kernel's own codes and
    token scales;
  * for n1 = 224 in per-channel weight mode the output equals the two-launch
    path's bit for bit (same column-block transform arithmetic, exact int32
    sums); elsewhere the two differ only by fp32 summation order and ties;
  * the sync buffer's error word stays zero, across consecutive calls with
    different token counts on one sync buffer.
Shapes: n2 = 128 with n1 = 224 (the 70B down projection's factors) and
n1 = 64, ragged N, every weight mode, dynamic and static activation scales.
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


def ws_codes(ws, M, n1, n2):
    """Packed codes and token scales the kernel left in its workspace
    (layout: Xq [M,K/2], then s_x [M] 256-byte aligned)."""
    K = n1 * n2
    a256 = lambda b: (b + 255) // 256 * 256
    off = 0
    h = ws.cpu().numpy()
    Xq = h[off:off + M * K // 2].reshape(M, K // 2)
    off2 = off + a256(M * K // 2)
    sx = h[off2:off2 + 4 * M].view(np.float32)
    return Xq, sx


def run_case(wl, mode, sync, alpha=1.0, seed_cal=7919):
    """mode: 'dynamic', 'tensor' or 'channel'."""
    torch, dev = torch_dev()
    L = W()
    inp = WL.make_inputs(wl)
    M, K = wl.M, wl.K
    per_channel = mode == "channel"
    steps = None
    Wt = O.merge_weights(inp["W"], inp["P1"], inp["P2"])
    if mode != "dynamic":
        Xc = WL.make_calibration_activations(wl, 48, inp["outlier_channels"], seed=wl.seed + seed_cal)
        steps = O.calibrate_steps(O.kron_transform(Xc, inp["P1"], inp["P2"]), per_channel, 0.8)
        if per_channel:
            Wt = O.migrate_steps(Wt, steps)
    wq = O.quantize_weights(Wt, wl.group_size, wl.asymmetric)
    if mode == "dynamic":
        ref = O.linear(inp["X"], inp["P1"], inp["P2"], wq, alpha_a=alpha)
    else:
        ref = O.linear_static(inp["X"], inp["P1"], inp["P2"], wq, steps.astype(np.float64), per_channel)
    desc, Wq, sw, zw = L.pack_weights(to_dev(Wt), wl.group_size, wl.asymmetric)
    Xd, P1d, P2d = to_dev(inp["X"]), to_dev(inp["P1"]), to_dev(inp["P2"])
    std = None if steps is None else to_dev(steps)
    ws = torch.empty(L.linear_decode_workspace_bytes(M, wl.n1, wl.n2), dtype=torch.uint8, device=dev)
    Y = L.linear_decode(Xd, P1d, P2d, desc, Wq, sw, zw, sync=sync, alpha_a=alpha, steps=std,
                        per_channel=per_channel, ws=ws)
    torch.cuda.synchronize()
    err = int(sync.cpu().numpy()[L.DECODE_SYNC_ERROR_WORD])
    assert err == 0, "the decode kernel timed out waiting for its activations"
    Xq, sx = ws_codes(ws, M, wl.n1, wl.n2)
    q = O.unpack_nibbles(Xq, True)
    n = assert_codes_match(q, ref["act"]["q"], ref["act"]["t"])
    np.testing.assert_allclose(sx.astype(np.float64), ref["act"]["s_x"], rtol=2e-6)
    Yh = Y.cpu().numpy()
    assert_layer_close(Yh, q, sx, wq)
    # the two-launch path on the same inputs
    if mode == "dynamic":
        Y2 = L.linear(Xd, P1d, P2d, desc, Wq, sw, zw, alpha_a=alpha).cpu().numpy()
    else:
        Y2 = L.linear_static(Xd, P1d, P2d, std, per_channel, desc, Wq, sw, zw).cpu().numpy()
    d = rel_l2(Yh, Y2)
    log(f"  excused tie cells {n}; rel L2 vs oracle {rel_l2(Yh, ref['Y64']):.2e}, vs two-launch {d:.2e}")
    return Yh, Y2


CASES = [
    # (M, n1, N, group_size or None, asym)
    (1, 224, 264, 128, True),
    (3, 224, 520, 128, False),
    (8, 224, 136, None, False),
    (10, 224, 200, 256, True),
    (1, 64, 1040, None, True),
    (5, 64, 264, 128, True),
    (16, 64, 72, 512, False),
]


@pytest.mark.parametrize("mode", ["dynamic", "tensor", "channel"])
@pytest.mark.parametrize("M,n1,N,g,asym", CASES)
def test_linear_decode_parity(M, n1, N, g, asym, mode):
    torch, dev = torch_dev()
    log(f"linear_decode M={M} P=({n1},128) N={N} g={g} asym={asym} {mode}")
    wl = custom_workload(M=M, n1=n1, n2=128, N=N, group_size=g, asym=asym, outliers=(5, 999),
                         pivot=20.0 if M > 1 else 0.0, seed=100 + M + n1)
    sync = W().decode_sync_buffer(dev)
    Y, Y2 = run_case(wl, mode, sync)
    if g is None and n1 == 224:
        # same transform arithmetic (column blocks) and exact int32 sums
        assert np.array_equal(Y.view(np.uint16), Y2.view(np.uint16))


def test_linear_decode_clip_alpha():
    torch, dev = torch_dev()
    log("linear_decode with alpha_a = 0.7")
    wl = custom_workload(M=4, n1=224, n2=128, N=96, group_size=128, asym=True, seed=77)
    run_case(wl, "dynamic", W().decode_sync_buffer(dev), alpha=0.7)


def test_linear_decode_consecutive_calls_share_sync():
    """One sync buffer across calls with different token counts and modes:
    the per-call tag keeps every call's counters separate."""
    torch, dev = torch_dev()
    sync = W().decode_sync_buffer(dev)
    for i, (M, mode) in enumerate([(1, "dynamic"), (8, "dynamic"), (1, "tensor"), (9, "channel"),
                                   (2, "dynamic")]):
        log(f"consecutive call {i}: M={M} {mode}")
        wl = custom_workload(M=M, n1=224, n2=128, N=152, group_size=128, asym=True, seed=300 + i)
        run_case(wl, mode, sync)


def test_linear_decode_unsupported():
    torch, dev = torch_dev()
    L = W()
    wl = custom_workload(M=2, n1=112, n2=128, N=64, seed=5)
    inp = WL.make_inputs(wl)
    desc, Wq, sw, zw = L.pack_weights(to_dev(inp["W"]), wl.K, False)
    sync = L.decode_sync_buffer(dev)
    with pytest.raises(L.W4A4Error) as e:
        L.linear_decode(to_dev(inp["X"]), to_dev(inp["P1"]), to_dev(inp["P2"]), desc, Wq, sw,
                        sync=sync)
    assert e.value.status == -2
    wl = custom_workload(M=17, n1=64, n2=128, N=64, seed=6)
    inp = WL.make_inputs(wl)
    desc, Wq, sw, zw = L.pack_weights(to_dev(inp["W"]), wl.K, False)
    with pytest.raises(L.W4A4Error) as e:
        L.linear_decode(to_dev(inp["X"]), to_dev(inp["P1"]), to_dev(inp["P2"]), desc, Wq, sw,
                        sync=sync, ws=torch.empty(1 << 20, dtype=torch.uint8, device=dev))
    assert e.value.status in (-1, -2)
    # 16 tokens of K = 28672 do not fit one CU's LDS next to the scale table
    wl = custom_workload(M=16, n1=224, n2=128, N=64, seed=7)
    inp = WL.make_inputs(wl)
    desc, Wq, sw, zw = L.pack_weights(to_dev(inp["W"]), 128, False)
    with pytest.raises(L.W4A4Error) as e:
        L.linear_decode(to_dev(inp["X"]), to_dev(inp["P1"]), to_dev(inp["P2"]), desc, Wq, sw,
                        sync=sync)
    assert e.value.status == -2 and "LDS" in str(e.value)
