"""The seeded generators: shapes, determinism and the stated input structure."""
import numpy as np
import pytest

import workloads as WL


def test_tiny_structure():
    inp = WL.make_inputs("tiny")
    X = inp["X"]
    assert X.shape == (16, 256) and X.dtype == np.float16
    assert inp["P1"].shape == (16, 16) and inp["P1"].dtype == np.float32
    assert inp["W"].shape == (256, 256) and inp["W"].dtype == np.float32
    assert list(inp["outlier_channels"]) == [7, 100]
    # token 0 (x100) and outlier channels (x50) dominate
    a = np.abs(X.astype(np.float64))
    assert a[0].mean() > 30 * a[1:].mean()
    assert a[1:, [7, 100]].mean() > 20 * np.delete(a[1:], [7, 100], axis=1).mean()


def test_deterministic():
    a = WL.make_inputs("tiny")
    b = WL.make_inputs("tiny")
    for k in ("X", "P1", "P2", "W"):
        assert np.array_equal(a[k], b[k])


def test_factors_invertible_not_orthogonal():
    inp = WL.make_inputs("tiny", with_weights=False)
    P1 = inp["P1"].astype(np.float64)
    sv = np.linalg.svd(P1, compute_uv=False)
    assert 0.45 < sv.min() and sv.max() < 2.05
    assert not np.allclose(P1.T @ P1, np.eye(16), atol=1e-2)


@pytest.mark.parametrize("name", ["qkv8b", "down8b"])
def test_activation_shapes_medium(name):
    wl = WL.get(name)
    rng = np.random.default_rng(wl.seed)
    X, ch = WL.make_activations(wl, rng, M=8)
    assert X.shape == (8, wl.K) and np.isfinite(X.astype(np.float32)).all()
    if name == "qkv8b":
        assert ch.size == round(0.005 * wl.K) == 20
    else:
        assert ch.size == 0


def test_all_workloads_consistent():
    for wl in WL.WORKLOADS.values():
        assert wl.n1 * wl.n2 == wl.K and wl.K % wl.group_size == 0


def test_kv_workloads_deterministic_and_shaped():
    from workloads import kv as WKV
    wl = WKV.get_kv("kv_tiny")
    a = WKV.make_kv_static(wl)
    b = WKV.make_kv_static(wl)
    for key in ("lengths", "outliers", "P_h", "P_v", "q"):
        np.testing.assert_array_equal(a[key], b[key])
    assert a["lengths"][0] == wl.max_seq
    assert ((a["lengths"] >= wl.min_len) & (a["lengths"] <= wl.max_seq)).all()
    assert a["q"].shape == (wl.batch, wl.heads_q, wl.head_dim) and a["q"].dtype == np.float16
    k, v = WKV.make_history(wl, 1, 17, a["outliers"])
    k2, _ = WKV.make_history(wl, 1, 17, a["outliers"])
    np.testing.assert_array_equal(k, k2)
    assert k.shape == (17, wl.heads_kv, wl.head_dim) and v.dtype == np.float16
    for w in WKV.KV_WORKLOADS.values():
        assert w.max_seq % 32 == 0 and w.heads_q % w.heads_kv == 0


def test_ternary_workloads_deterministic_and_row_sampling():
    from workloads import ternary as WT
    wl = WT.TernWorkload("t", M=3, K=256, N=2100, x_kind="silu_product", seed=4)
    a = WT.make_tern_inputs(wl)
    b = WT.make_tern_inputs(wl)
    assert a["X"].dtype == np.float16 and a["X"].shape == (3, 256)
    assert a["Wt"].dtype == np.float32 and a["Wt"].shape == (2100, 256)
    np.testing.assert_array_equal(a["X"], b["X"])
    np.testing.assert_array_equal(a["Wt"], b["Wt"])
    rows = [0, 1023, 1024, 2099, 5]
    np.testing.assert_array_equal(WT.make_tern_weights(wl, rows=rows), a["Wt"][rows])
    # blocks carry their own offsets: block means spread well beyond sampling noise
    means = a["Wt"].reshape(2100, 2, 128).mean(axis=2) / np.abs(a["Wt"]).mean()
    assert means.std() > 0.15
    for name, w in WT.TERN_WORKLOADS.items():
        assert w.K % 128 == 0 and w.M <= 64, name
