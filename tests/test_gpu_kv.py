"""GPU parity of the INT4 KV cache (w4a4_kv_append, w4a4_kv_query_factor) and
of the decode attention over it (w4a4_attn_decode), through the C ABI.

FlatQuant page, section Transformer 集成 (per-head transforms P_h, P_v of the
key and value caches); FPTQuant page, section 核心贡献 (INT4 KV cache).

Checks:
  * appended codes equal the oracle's bit for bit except within the 1e-4 tie
    window, scales match to float32 rounding, and every cache cell the call
    does not own (other positions, other sequences, the other tokens of a
    shared value word) keeps its previous contents exactly; segments that
    fall outside the cache are skipped;
  * the attention output on an oracle-built cache is within one fp16 ulp
    (plus 1e-5 of the row's largest magnitude) of the oracle's float64 value,
    relative L2 <= 1e-3 overall, for empty, single-token, tile-edge and full
    contexts, GQA groups of 1, 4, 8 and 16, shared and per-head transforms,
    one chunk and many, and value scales spread over six decades;
  * GPU append followed by GPU attention against the oracle's append and
    attention;
  * the LLaMA-3-8B and -70B decode workloads at full size (64 sequences, up
    to 8192 cached tokens) in the benchmark's launch configuration, on
    sampled sequences.
"""
import math

import numpy as np
import pytest

from oracle import kv_oracle as KV
import workloads as WL
from workloads import kv as WKV
from gpu_common import assert_codes_match, log, rel_l2, to_dev, torch_dev, ulp16

pytestmark = pytest.mark.gpu


def W():
    import w4a4_post_quantized_amd as lib
    return lib


def tiny_wl(**kw):
    base = dict(name="custom", batch=1, heads_q=8, heads_kv=2, head_dim=128, max_seq=64,
                min_len=1)
    base.update(kw)
    return WKV.KvWorkload(**base)


def random_cache_contents(rng, B, H, S):
    """Arbitrary prior contents: key bytes, value words, positive scales."""
    kb = rng.integers(0, 256, size=(B, H, S, 64), dtype=np.uint8)
    vw = rng.integers(0, 2 ** 32, size=(B, H, S // 8, 128), dtype=np.uint64).astype(np.uint32)
    ks = rng.uniform(0.01, 1.0, size=(B, H, S)).astype(np.float32)
    vs = rng.uniform(0.01, 1.0, size=(B, H, S)).astype(np.float32)
    return kb, vw, ks, vs


def upload_cache(kb, vw, ks, vs):
    torch, dev = torch_dev()
    B, H, S, _ = kb.shape
    c = W().KvCache(B, H, S, dev, zero=False)
    c.k_cache.copy_(torch.from_numpy(kb))
    c.v_cache.copy_(torch.from_numpy(vw.view(np.int32)))
    c.k_scale.copy_(torch.from_numpy(ks))
    c.v_scale.copy_(torch.from_numpy(vs))
    return c


def download_cache(c):
    return (c.k_cache.cpu().numpy(), c.v_cache.cpu().numpy().view(np.uint32),
            c.k_scale.cpu().numpy(), c.v_scale.cpu().numpy())


def oracle_cache_from(kb, vw, ks, vs):
    B, H, S, _ = kb.shape
    oc = KV.KvCache(B, H, S, 128)
    oc.kq[:] = KV.unpack_k_cache(kb)
    oc.vq[:] = KV.unpack_v_cache(vw)
    oc.ks[:] = ks
    oc.vs[:] = vs
    return oc


# ---------------------------------------------------------------------------
# w4a4_kv_query_factor
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("count", [1, 3])
def test_query_factor_is_inverse_transpose(count):
    torch, dev = torch_dev()
    rng = np.random.default_rng(20 + count)
    P = np.stack([WL.random_invertible(rng, 128).astype(np.float32) for _ in range(count)])
    if count == 1:
        P = P[0]
    log(f"kv_query_factor count={count}")
    got = W().kv_query_factor(to_dev(P)).cpu().numpy().astype(np.float64)
    Pm = P.reshape(-1, 128, 128).astype(np.float64)
    want = np.stack([np.linalg.inv(p).T for p in Pm]).reshape(got.shape)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-6 * np.abs(want).max())


def test_query_factor_rejects_singular():
    torch, dev = torch_dev()
    P = np.eye(128, dtype=np.float32)
    P[5] = P[7]
    with pytest.raises(W().W4A4Error, match="singular"):
        W().kv_query_factor(to_dev(P))


# ---------------------------------------------------------------------------
# w4a4_kv_append
# ---------------------------------------------------------------------------
def run_append_case(name, B, H, S, segs, per_head=False, alpha_k=1.0, alpha_v=1.0, seed=0,
                    invalid=()):
    """segs: list of (seq, start, n) written; invalid: (seq, start, n) segments
    the call must skip (their tokens are still present in k and v)."""
    torch, dev = torch_dev()
    rng = np.random.default_rng(seed)
    wl = tiny_wl(heads_kv=H, max_seq=S, batch=B)
    all_segs = list(segs) + list(invalid)
    T = sum(n for _, _, n in all_segs)
    och = np.stack([np.sort(rng.choice(128, 2, replace=False)) for _ in range(H)])
    k, v = WKV.make_tokens(wl, T, och, seed + 1)
    if per_head:
        P_h = np.stack([WL.random_invertible(rng, 128) for _ in range(H)]).astype(np.float32)
        P_v = np.stack([WL.random_invertible(rng, 128) for _ in range(H)]).astype(np.float32)
    else:
        P_h = WL.random_invertible(rng, 128).astype(np.float32)
        P_v = WL.random_invertible(rng, 128).astype(np.float32)
    init = random_cache_contents(rng, B, H, S)
    # order the segments as given, invalid ones interleaved at the end
    seg_seq = np.array([s for s, _, _ in all_segs], dtype=np.int32)
    seg_start = np.array([p for _, p, _ in all_segs], dtype=np.int32)
    cu = np.concatenate([[0], np.cumsum([n for _, _, n in all_segs])]).astype(np.int32)

    log(f"kv_append case={name} B={B} H={H} S={S} T={T} segments={len(all_segs)}")
    cache = upload_cache(*init)
    W().kv_append(to_dev(k), to_dev(v), to_dev(seg_seq), to_dev(seg_start), to_dev(cu),
                  to_dev(P_h), to_dev(P_v), cache, alpha_k, alpha_v)
    torch.cuda.synchronize()
    gk, gv, gks, gvs = download_cache(cache)

    # oracle: the valid segments only (positions past S dropped)
    oc = oracle_cache_from(*init)
    ntok = len(segs)
    vseq, vstart, vcu = [], [], [0]
    t_off = 0
    for s, p, n in segs:
        vseq.append(s)
        vstart.append(p)
        vcu.append(vcu[-1] + n)
    res = KV.kv_append(oc, k[:cu[ntok]], v[:cu[ntok]], vseq, vstart, vcu, P_h, P_v,
                       alpha_k, alpha_v)
    # tie-window map: t of the written cells, NaN elsewhere (no excuse)
    tk = np.full(oc.kq.shape, np.nan)
    tv = np.full(oc.vq.shape, np.nan)
    for i, (s, p, n) in enumerate(segs):
        for j in range(n):
            t = vcu[i] + j
            tk[s, :, p + j] = res["tk"][t]
            tv[s, :, p + j] = res["tv"][t]
    ek = assert_codes_match(KV.unpack_k_cache(gk), oc.kq, tk, what="key codes")
    ev = assert_codes_match(KV.unpack_v_cache(gv), oc.vq, tv, what="value codes")
    written = ~np.isnan(tk[..., 0])
    np.testing.assert_allclose(gks[written], oc.ks[written], rtol=2e-6, atol=0)
    np.testing.assert_allclose(gvs[written], oc.vs[written], rtol=2e-6, atol=0)
    np.testing.assert_array_equal(gks[~written], init[2][~written])
    np.testing.assert_array_equal(gvs[~written], init[3][~written])
    # bytes of untouched positions are exactly the prior contents
    np.testing.assert_array_equal(gk[~written], init[0][~written])
    log(f"  ok: {int(written.sum())} head vectors written, tie flips key {ek} value {ev}")


def test_append_decode_positions():
    # one token per sequence, at the tile and word edges
    segs = [(0, 0, 1), (3, 63, 1), (1, 31, 1), (2, 32, 1), (5, 17, 1), (4, 8, 1)]
    run_append_case("decode", B=6, H=8, S=64, segs=segs, seed=1)


def test_append_prefill_ragged():
    segs = [(2, 13, 100), (0, 0, 64), (1, 29, 7), (1, 200, 1), (0, 255, 1)]
    run_append_case("prefill", B=3, H=8, S=256, segs=segs, seed=2)


def test_append_per_head_and_clip():
    segs = [(1, 5, 40), (0, 62, 3)]
    run_append_case("per_head_clip", B=2, H=4, S=96, segs=segs, per_head=True,
                    alpha_k=0.9, alpha_v=0.8, seed=3)


def test_append_skips_out_of_cache_segments():
    # valid: (0, 3, 5); clipped: (1, 61, 10) writes positions 61..63 only
    segs = [(0, 3, 5), (1, 61, 3)]
    invalid = [(-1, 0, 4), (2, 0, 4), (0, -5, 3), (0, 64, 2)]
    torch, dev = torch_dev()
    # the clipped segment: pass 10 tokens, the oracle sees the first 3
    rng = np.random.default_rng(4)
    B, H, S = 2, 2, 64
    wl = tiny_wl(heads_kv=H, max_seq=S, batch=B)
    och = np.stack([np.sort(rng.choice(128, 2, replace=False)) for _ in range(H)])
    P_h = WL.random_invertible(rng, 128).astype(np.float32)
    P_v = WL.random_invertible(rng, 128).astype(np.float32)
    all_segs = [(0, 3, 5), (1, 61, 10)] + invalid
    T = sum(n for _, _, n in all_segs)
    k, v = WKV.make_tokens(wl, T, och, 5)
    init = random_cache_contents(rng, B, H, S)
    seg_seq = np.array([s for s, _, _ in all_segs], dtype=np.int32)
    seg_start = np.array([p for _, p, _ in all_segs], dtype=np.int32)
    cu = np.concatenate([[0], np.cumsum([n for _, _, n in all_segs])]).astype(np.int32)
    log("kv_append case=skips")
    cache = upload_cache(*init)
    W().kv_append(to_dev(k), to_dev(v), to_dev(seg_seq), to_dev(seg_start), to_dev(cu),
                  to_dev(P_h), to_dev(P_v), cache)
    torch.cuda.synchronize()
    gk, gv, gks, gvs = download_cache(cache)
    oc = oracle_cache_from(*init)
    ksel = np.concatenate([k[0:5], k[5:8]])
    vsel = np.concatenate([v[0:5], v[5:8]])
    res = KV.kv_append(oc, ksel, vsel, [0, 1], [3, 61], [0, 5, 8], P_h, P_v)
    tk = np.full(oc.kq.shape, np.nan)
    tv = np.full(oc.vq.shape, np.nan)
    for i, (s, p, n) in enumerate(segs):
        for j in range(n):
            tk[s, :, p + j] = res["tk"][[0, 5][i] + j]
            tv[s, :, p + j] = res["tv"][[0, 5][i] + j]
    assert_codes_match(KV.unpack_k_cache(gk), oc.kq, tk, what="key codes")
    assert_codes_match(KV.unpack_v_cache(gv), oc.vq, tv, what="value codes")
    written = ~np.isnan(tk[..., 0])
    assert int(written.sum()) == (5 + 3) * H
    np.testing.assert_array_equal(gks[~written], init[2][~written])
    np.testing.assert_array_equal(gk[~written], init[0][~written])


# ---------------------------------------------------------------------------
# w4a4_attn_decode
# ---------------------------------------------------------------------------
def assert_attn_close(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    rowmax = np.abs(ref).max(axis=-1, keepdims=True)
    bound = ulp16(ref) + 1e-5 * rowmax
    err = np.abs(got - ref)
    bad = err > bound
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of bound, first {i}: "
                             f"gpu {got[i]} oracle {ref[i]} bound {bound[i]}")
    if np.abs(ref).max() > 0:
        assert rel_l2(got, ref) <= 1e-3, what


def build_oracle_cache(wl, lengths, P_h, P_v, outliers, value_spread=0.0, seed=0):
    """Cache filled by the oracle's append of each sequence's history."""
    oc = KV.KvCache(wl.batch, wl.heads_kv, wl.max_seq, 128)
    rng = np.random.default_rng(seed)
    for b in range(wl.batch):
        L = int(lengths[b])
        if L == 0:
            continue
        k, v = WKV.make_history(wl, b, L, outliers)
        if value_spread:
            f = 10.0 ** rng.uniform(-value_spread, value_spread, size=(L, 1, 1))
            v = (v.astype(np.float64) * f).astype(np.float16)
        KV.kv_append(oc, k, v, [b], [0], [0, L], P_h, P_v)
    return oc


def run_attn_case(name, wl, lengths, per_head=False, value_spread=0.0, seed=0):
    torch, dev = torch_dev()
    rng = np.random.default_rng(seed)
    H = wl.heads_kv
    och = np.stack([np.sort(rng.choice(128, 2, replace=False)) for _ in range(H)])
    if per_head:
        P_h = np.stack([WL.random_invertible(rng, 128) for _ in range(H)]).astype(np.float32)
        P_v = np.stack([WL.random_invertible(rng, 128) for _ in range(H)]).astype(np.float32)
    else:
        P_h = WL.random_invertible(rng, 128).astype(np.float32)
        P_v = WL.random_invertible(rng, 128).astype(np.float32)
    q = rng.standard_normal((wl.batch, wl.heads_q, 128)).astype(np.float16)
    lengths = np.asarray(lengths, dtype=np.int32)
    oc = build_oracle_cache(wl, lengths, P_h, P_v, och, value_spread, seed)
    sm = 1.0 / math.sqrt(128)
    ref = KV.attention_decode(q, oc, lengths, P_h, sm)
    kb, ks, vw, vs = oc.packed()
    log(f"attn_decode case={name} B={wl.batch} Hq={wl.heads_q} Hkv={H} S={wl.max_seq} "
        f"lengths={lengths.tolist()[:8]} per_head={per_head}")
    cache = upload_cache(kb, vw, ks, vs)
    Pinv = W().kv_query_factor(to_dev(P_h))
    out = W().attn_decode(to_dev(q), Pinv, cache, to_dev(lengths), sm)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert_attn_close(got, ref, name)
    assert (got[lengths == 0] == 0).all()
    log(f"  ok: rel L2 {rel_l2(got, ref):.2e}")


def test_attn_context_edges():
    lengths = [96, 0, 1, 31, 32, 33, 95]
    wl = tiny_wl(batch=len(lengths), heads_q=8, heads_kv=2, max_seq=96)
    run_attn_case("edges_g4", wl, lengths, seed=10)


@pytest.mark.parametrize("hq,hkv", [(2, 2), (16, 2), (16, 1)])
def test_attn_group_sizes(hq, hkv):
    lengths = [64, 17, 40]
    wl = tiny_wl(batch=3, heads_q=hq, heads_kv=hkv, max_seq=64)
    run_attn_case(f"g{hq // hkv}", wl, lengths, seed=11)


def test_attn_per_head_transforms():
    wl = tiny_wl(batch=3, heads_q=8, heads_kv=4, max_seq=128)
    run_attn_case("per_head", wl, [128, 70, 5], per_head=True, seed=12)


def test_attn_many_chunks():
    # small grids shrink the chunk to 128 positions: 16 chunks per sequence
    wl = tiny_wl(batch=2, heads_q=8, heads_kv=2, max_seq=2048)
    run_attn_case("chunks", wl, [2048, 1500], seed=13)


def test_attn_value_scales_spread():
    wl = tiny_wl(batch=2, heads_q=8, heads_kv=2, max_seq=512)
    run_attn_case("value_spread", wl, [512, 300], value_spread=3.0, seed=14)


def test_append_then_attend_end_to_end():
    """GPU append of every history (one prefill call, four segments), then GPU
    attention; the oracle appends and attends on its own."""
    torch, dev = torch_dev()
    wl = tiny_wl(batch=4, heads_q=16, heads_kv=4, max_seq=512)
    st_rng = np.random.default_rng(15)
    och = np.stack([np.sort(st_rng.choice(128, 2, replace=False)) for _ in range(4)])
    P_h = WL.random_invertible(st_rng, 128).astype(np.float32)
    P_v = WL.random_invertible(st_rng, 128).astype(np.float32)
    lengths = np.array([512, 333, 1, 64], dtype=np.int32)
    q = st_rng.standard_normal((4, 16, 128)).astype(np.float16)
    hist = [WKV.make_history(wl, b, int(lengths[b]), och) for b in range(4)]
    k = np.concatenate([h[0] for h in hist])
    v = np.concatenate([h[1] for h in hist])
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    log("append+attend end to end")
    cache = W().KvCache(4, 4, 512, dev)
    W().kv_append(to_dev(k), to_dev(v), to_dev(np.arange(4, dtype=np.int32)),
                  to_dev(np.zeros(4, dtype=np.int32)), to_dev(cu), to_dev(P_h), to_dev(P_v),
                  cache)
    Pinv = W().kv_query_factor(to_dev(P_h))
    sm = 1.0 / math.sqrt(128)
    out = W().attn_decode(to_dev(q), Pinv, cache, to_dev(lengths), sm)
    torch.cuda.synchronize()
    oc = KV.KvCache(4, 4, 512, 128)
    res = KV.kv_append(oc, k, v, list(range(4)), [0] * 4, cu, P_h, P_v)
    gk, gv, _, _ = download_cache(cache)
    tk = np.full(oc.kq.shape, np.nan)
    for b in range(4):
        tk[b, :, :lengths[b]] = res["tk"][cu[b]:cu[b + 1]].transpose(1, 0, 2)
    flips = assert_codes_match(KV.unpack_k_cache(gk)[~np.isnan(tk)],
                               oc.kq[~np.isnan(tk)], tk[~np.isnan(tk)], what="key codes")
    ref = KV.attention_decode(q, oc, lengths, P_h, sm)
    got = out.cpu().numpy().astype(np.float64)
    if flips == 0:
        assert_attn_close(got, ref, "end_to_end")
    else:
        assert rel_l2(got, ref) <= 1e-3
    log(f"  ok: rel L2 {rel_l2(got, ref):.2e}, key tie flips {flips}")


# ---------------------------------------------------------------------------
# full-size decode workloads, sampled sequences
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["attn8b", "attn70b"])
def test_attn_full_size_sampled(name):
    torch, dev = torch_dev()
    wl = WKV.get_kv(name)
    st = WKV.make_kv_static(wl)
    lengths = st["lengths"]
    sampled = [0, 17, wl.batch - 1]
    log(f"full size {name}: B={wl.batch} S={wl.max_seq} sampled={sampled}")
    # every sequence gets arbitrary contents; the sampled ones are appended
    # from their generated histories with the library
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    cache = W().KvCache(wl.batch, wl.heads_kv, wl.max_seq, dev, zero=False)
    cache.k_cache.copy_(torch.randint(0, 256, cache.k_cache.shape, generator=g, device=dev,
                                      dtype=torch.int32).to(torch.uint8))
    cache.v_cache.copy_(torch.randint(-2 ** 31, 2 ** 31 - 1, cache.v_cache.shape, generator=g,
                                      device=dev, dtype=torch.int32))
    cache.k_scale.uniform_(0.05, 1.0, generator=g)
    cache.v_scale.uniform_(0.05, 1.0, generator=g)
    hist = [WKV.make_history(wl, b, int(lengths[b]), st["outliers"]) for b in sampled]
    k = np.concatenate([h[0] for h in hist])
    v = np.concatenate([h[1] for h in hist])
    cu = np.concatenate([[0], np.cumsum([lengths[b] for b in sampled])]).astype(np.int32)
    W().kv_append(to_dev(k), to_dev(v), to_dev(np.array(sampled, dtype=np.int32)),
                  to_dev(np.zeros(len(sampled), dtype=np.int32)), to_dev(cu),
                  to_dev(st["P_h"]), to_dev(st["P_v"]), cache)
    Pinv = W().kv_query_factor(to_dev(st["P_h"]))
    sm = 1.0 / math.sqrt(128)
    out = W().attn_decode(to_dev(st["q"]), Pinv, cache, to_dev(lengths), sm)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    for i, b in enumerate(sampled):
        L = int(lengths[b])
        oc = KV.KvCache(1, wl.heads_kv, wl.max_seq, 128)
        res = KV.kv_append(oc, hist[i][0], hist[i][1], [0], [0], [0, L], st["P_h"], st["P_v"])
        gk = cache.k_cache[b, :, :L].cpu().numpy()
        gv = cache.v_cache[b, :, :(L + 7) // 8].cpu().numpy().view(np.uint32)
        tk = res["tk"].transpose(1, 0, 2)
        flips = assert_codes_match(KV.unpack_k_cache(gk), oc.kq[0, :, :L], tk,
                                   what=f"{name} seq {b} key codes")
        vcodes = KV.unpack_v_cache(gv)[:, :L]
        flips += assert_codes_match(vcodes, oc.vq[0, :, :L], res["tv"].transpose(1, 0, 2),
                                    what=f"{name} seq {b} value codes")
        qb = st["q"][b:b + 1]
        ref = KV.attention_decode(qb, oc, np.array([L]), st["P_h"], sm)[0]
        if flips == 0:
            assert_attn_close(got[b], ref, f"{name} seq {b}")
        else:
            assert rel_l2(got[b], ref) <= 1e-3
        log(f"  seq {b} (L={L}): rel L2 {rel_l2(got[b], ref):.2e}, tie flips {flips}")
