"""CPU oracle of the W4A4 quantized linear layer — TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the CPU-baseline leg of the benchmark
may import this module.  The product library never calls it, and it shares no
code with the HIP path.

Every step is plain numpy in float64, written from the pages:

* FlatQuant: Flatness Matters for LLM Quantization (paper notes)
  - "核心思想": the layer computes Q(X P) · Q(P^-1 W^T), an invertible affine
    transform P on the activations and its inverse merged into the weights.
  - "Kronecker 分解": P = P1 ⊗ P2 and the vec trick: the activation side is
    P1^T ×1 X̃ ×2 P2, the weight side P1^-1 ×1 W̃ ×2 (P2^-1)^T.  Also the
    argmin n1+n2 choice of the factor sizes (n = 8192 -> (64, 128)).
  - "额外可学习组件": per-channel scaling diag(c) before the transform, and
    clipping thresholds α_w, α_a in (0, 1].
  - "高效 Kernel 设计": transform and quantization fused per token tile, the
    intermediate kept on chip (here: float64, never rounded before Q()).
  - "亮点与洞察" item 3: round-to-nearest (RTN) quantizer.
* FRM-PTQ: Feature Relationship Matching Enhanced Low-Bit Post-Training
  Quantization for Large Language Models, "初步介绍": the uniform quantizer
  Q(W) = clamp(round(W/s) + z, 0, 2^b - 1); and the introduction's
  multi-granularity (group-wise) weight quantization.
* FPTQuant: Function-Preserving Transforms for LLM Quantization, section
  "3. 伪动态残差缩放": a per-token scale commutes with a bias-free linear map,
  so the activation scale can be applied after the integer product.
* PT2-LLM: Post-Training Ternarization for Large Language Models, "关键设计"
  item 1: a joint column permutation leaves X W^T unchanged.
* Static activation quantization (steps fixed offline, no runtime absmax):
  FPTQuant page, "核心贡献" item on static INT4 quantization (one step per
  tensor); MergeQuant page, "核心思路" and "关键设计" item 2 (per-channel
  steps migrated into the weights of the linear layer, "QSM").

W3A3 (FRM-PTQ page, introduction and its contributions: weights and
activations at 3 bits) is the same layer with b = 3; the codes are stored one
per nibble like the 4-bit ones.

Readings where the pages are silent or garbled:
round half to even; symmetric activations s = α·max|z|/7 with codes clamped to
[-8, 7]; asymmetric weights with zero-inclusive range, s = (hi-lo)/15 and
z = clamp(round(-lo/s), 0, 15); weight scales stored in fp16 (direct RNE from
float64) and the codes computed with the stored scale; a zero scale gives zero
codes; row-major vec order k = i*n2 + j.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "kron_factors", "kron_transform", "act_scale", "quantize_act",
    "transform_quant", "pack_nibbles", "unpack_nibbles", "merge_weights",
    "fp16_rne", "quantize_weights", "int_gemm", "int_gemm_loop",
    "epilogue", "epilogue_by_group", "linear", "dequant_act", "dequant_weights",
    "quantize_act_static", "transform_quant_static", "migrate_steps", "linear_static",
    "calibrate_steps", "code_range",
]

QMIN, QMAX = -8, 7          # signed 4-bit code range (b = 4)
UMAX = 15                   # unsigned 4-bit code range, 2^b - 1


def code_range(bits: int):
    """(qmin, qmax, umax) of b-bit codes: signed [-2^(b-1), 2^(b-1) - 1],
    unsigned [0, 2^b - 1] (FRM-PTQ page, "初步介绍": the unsigned range of the
    uniform quantizer is 0 .. 2^b - 1; its introduction evaluates b = 4 and
    b = 3, W4A4 and W3A3)."""
    if bits not in (3, 4):
        raise ValueError("bits must be 3 or 4")
    return -(1 << (bits - 1)), (1 << (bits - 1)) - 1, (1 << bits) - 1


# ----------------------------------------------------------------------------
# Factor sizes (FlatQuant page, "Kronecker 分解": pick n1, n2 minimising n1+n2)
# ----------------------------------------------------------------------------
def kron_factors(n: int):
    """(n1, n2) with n1*n2 == n, n1 <= n2, minimising n1 + n2."""
    best = None
    for a in range(1, int(np.sqrt(n)) + 1):
        if n % a == 0:
            b = n // a
            if best is None or a + b < best[0] + best[1]:
                best = (a, b)
    return best


# ----------------------------------------------------------------------------
# Activation side
# ----------------------------------------------------------------------------
def kron_transform(X, P1, P2, c=None):
    """Z_m = P1^T · reshape(x_m ⊙ c, n1, n2) · P2, float64.

    FlatQuant page, "Kronecker 分解": the left factor of the vec-trick
    expression, P1^T ×1 X̃ ×2 P2; "额外可学习组件": diag(c) precedes the
    transform.  The token row is reshaped row-major (k = i*n2 + j), for which
    this equals x_m · (P1 ⊗ P2).
    """
    X64 = np.asarray(X, dtype=np.float64)
    M, K = X64.shape
    P1 = np.asarray(P1, dtype=np.float64)
    P2 = np.asarray(P2, dtype=np.float64)
    n1, n2 = P1.shape[0], P2.shape[0]
    if n1 * n2 != K:
        raise ValueError("K must equal n1*n2")
    if c is not None:
        X64 = X64 * np.asarray(c, dtype=np.float64)[None, :]
    Xb = X64.reshape(M, n1, n2)
    Z = np.matmul(np.matmul(P1.T[None, :, :], Xb), P2[None, :, :])
    return Z.reshape(M, K)


def act_scale(Z, alpha_a: float = 1.0, bits: int = 4):
    """Per-token symmetric scale s_x[m] = α_a · max_k |Z[m,k]| / qmax (float64),
    qmax = 2^(bits-1) - 1 (7 for INT4, 3 for INT3).

    FRM-PTQ page, "初步介绍" (uniform quantizer, here with z = 0 and the
    signed range of b = 4 bits); FlatQuant page, "额外可学习组件" (α_a clips
    the range).
    """
    a = np.max(np.abs(Z), axis=1) if Z.shape[1] else np.zeros(Z.shape[0])
    return np.float64(alpha_a) * a / code_range(bits)[1]


def quantize_act(Z, s, bits: int = 4):
    """q = clamp(round_half_even(Z / s), qmin, qmax) ([-8, 7] for INT4, [-4, 3]
    for INT3); s == 0 gives q = 0.

    Returns (q int8 [M,K], t float64 [M,K]) where t = Z/s is kept so parity
    checks can find values within a small window of a rounding tie.
    FRM-PTQ page "初步介绍"; FlatQuant page "亮点与洞察" item 3 (RTN).
    """
    s = np.asarray(s, dtype=np.float64)
    safe = np.where(s > 0, s, 1.0)
    t = np.asarray(Z, dtype=np.float64) / safe[:, None]
    t = np.where((s > 0)[:, None], t, 0.0)
    qmin, qmax, _ = code_range(bits)
    q = np.clip(np.rint(t), qmin, qmax).astype(np.int8)   # np.rint: half to even
    return q, t


def transform_quant(X, P1, P2, c=None, alpha_a: float = 1.0, bits: int = 4):
    """Online activation path: transform, per-token scale, quantize, pack.

    FlatQuant page "高效 Kernel 设计": transform and quantization of one
    token tile in one step.  Returns dict(Z, s_x, q, t, packed).
    """
    Z = kron_transform(X, P1, P2, c)
    s_x = act_scale(Z, alpha_a, bits)
    q, t = quantize_act(Z, s_x, bits)
    return dict(Z=Z, s_x=s_x, q=q, t=t, packed=pack_nibbles(q))


def pack_nibbles(q):
    """byte[..., j] = (q[2j] & 0xF) | (q[2j+1] & 0xF) << 4 (low nibble = even k).

    Two 4-bit codes per byte; signed codes are stored as two's-complement
    nibbles, unsigned codes as themselves.
    """
    q = np.asarray(q)
    if q.shape[-1] % 2:
        raise ValueError("last dimension must be even")
    v = q.astype(np.int64) & 0xF
    return (v[..., 0::2] | (v[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b, signed: bool):
    """Inverse of pack_nibbles."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    lo = b & 0xF
    hi = b >> 4
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    if signed:
        out = np.where(out >= 8, out - 16, out)
    return out.astype(np.int8)


# ----------------------------------------------------------------------------
# Weight side (offline)
# ----------------------------------------------------------------------------
def merge_weights(W, P1, P2, c=None, out_dtype=np.float32):
    """W̃ = W · diag(1/c) · (P1 ⊗ P2)^-T, row by row P1^-1 · W̄_n · P2^-T.

    FlatQuant page, "Kronecker 分解": the weight-side factor
    P1^-1 ×1 W̃ ×2 (P2^-1)^T of the vec-trick expression; "额外可学习组件":
    diag(c) on the activations is undone on the weights.  Computed in float64
    and rounded once to ``out_dtype``.
    """
    W64 = np.asarray(W, dtype=np.float64)
    N, K = W64.shape
    P1 = np.asarray(P1, dtype=np.float64)
    P2 = np.asarray(P2, dtype=np.float64)
    n1, n2 = P1.shape[0], P2.shape[0]
    if n1 * n2 != K:
        raise ValueError("K must equal n1*n2")
    if c is not None:
        W64 = W64 / np.asarray(c, dtype=np.float64)[None, :]
    P1i = np.linalg.inv(P1)
    P2iT = np.linalg.inv(P2).T
    out = np.empty((N, K), dtype=out_dtype)
    chunk = max(1, (1 << 22) // K)
    for r0 in range(0, N, chunk):
        r1 = min(N, r0 + chunk)
        Wb = W64[r0:r1].reshape(r1 - r0, n1, n2)
        R = np.matmul(np.matmul(P1i[None, :, :], Wb), P2iT[None, :, :])
        out[r0:r1] = R.reshape(r1 - r0, K).astype(out_dtype)
    return out


def fp16_rne(x):
    """float64 -> nearest float16, ties to even, as a direct conversion.

    numpy converts float64 to float16 in one rounding step (no intermediate
    float32), which is what the stored weight scales need.
    """
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def quantize_weights(Wt, group_size: int, asymmetric: bool, alpha_w: float = 1.0,
                     bits: int = 4):
    """Round-to-nearest INT4 weights, per output channel or per group.

    FRM-PTQ page, "初步介绍": Q(W) = clamp(round(W/s) + z, 0, 2^b - 1); the
    introduction's multi-granularity group quantization gives group_size.
    FlatQuant page, "额外可学习组件": α_w clips the range.

    Symmetric: s = fp16(α·max|v| / qmax), q = clamp(round(v/s), qmin, qmax),
    z = 0.  Asymmetric: lo = α·min(min v, 0), hi = α·max(max v, 0),
    s = fp16((hi - lo)/umax), z = clamp(round(-lo/s), 0, umax),
    u = clamp(round(v/s) + z, 0, umax).  (qmin, qmax, umax) = (-8, 7, 15) for
    b = 4 and (-4, 3, 7) for b = 3.  Codes use the stored fp16 scale.
    A stored scale of 0 gives codes 0 and z = 0.

    Returns dict(codes int8 [N,K] (signed q, or unsigned u), s fp16 [N,G],
    z fp16 [N,G] (zeros when symmetric), packed uint8 [N,K/2]).
    """
    V = np.asarray(Wt, dtype=np.float64)
    N, K = V.shape
    if K % group_size:
        raise ValueError("K must be a multiple of group_size")
    G = K // group_size
    Vg = V.reshape(N, G, group_size)
    a = np.float64(alpha_w)
    qmin, qmax, umax = code_range(bits)
    if not asymmetric:
        s16 = fp16_rne(a * np.max(np.abs(Vg), axis=2) / qmax)
        s = s16.astype(np.float64)
        safe = np.where(s > 0, s, 1.0)
        q = np.clip(np.rint(Vg / safe[:, :, None]), qmin, qmax)
        q = np.where((s > 0)[:, :, None], q, 0)
        z16 = np.zeros((N, G), dtype=np.float16)
    else:
        lo = a * np.minimum(np.min(Vg, axis=2), 0.0)
        hi = a * np.maximum(np.max(Vg, axis=2), 0.0)
        s16 = fp16_rne((hi - lo) / umax)
        s = s16.astype(np.float64)
        safe = np.where(s > 0, s, 1.0)
        # z is an integer in [0, umax]; adding +0.0 turns the -0.0 that
        # rint(-0/s) gives for an all-positive group into the integer 0
        z = np.clip(np.rint(-lo / safe), 0, umax) + 0.0
        z = np.where(s > 0, z, 0.0)
        q = np.clip(np.rint(Vg / safe[:, :, None]) + z[:, :, None], 0, umax)
        q = np.where((s > 0)[:, :, None], q, 0)
        z16 = z.astype(np.float16)
    codes = q.reshape(N, K).astype(np.int8)
    return dict(codes=codes, s=s16, z=z16, packed=pack_nibbles(codes),
                group_size=group_size, asymmetric=asymmetric, bits=bits)


# ----------------------------------------------------------------------------
# Integer product and epilogue
# ----------------------------------------------------------------------------
def _centered(wcodes, z, group_size):
    N, K = wcodes.shape
    G = K // group_size
    w = wcodes.astype(np.int64).reshape(N, G, group_size)
    zz = np.asarray(z, dtype=np.float64).astype(np.int64).reshape(N, G, 1)
    return w - zz


def int_gemm(qx, wcodes, z, group_size: int, exact_fp64: bool = True):
    """D[m, n, g] = Σ_{k in group g} q_x[m,k] · (u[n,k] - z[n,g]), exact.

    The integer form of the FlatQuant page's Q(XP)·Q(P^-1 W^T) product
    ("核心思想"), split by weight group.  With ``exact_fp64`` the sums run in
    float64 BLAS on integer-valued arrays; every partial sum is an integer of
    magnitude <= K·8·15 < 2^53, so the result is exact.  Otherwise int64.
    """
    qx = np.asarray(qx)
    M, K = qx.shape
    N = wcodes.shape[0]
    G = K // group_size
    wc = _centered(wcodes, z, group_size)                    # [N, G, g]
    xg = qx.astype(np.int64).reshape(M, G, group_size)       # [M, G, g]
    D = np.empty((M, N, G), dtype=np.int64)
    for g in range(G):
        if exact_fp64:
            D[:, :, g] = np.rint(xg[:, g, :].astype(np.float64)
                                 @ wc[:, g, :].astype(np.float64).T).astype(np.int64)
        else:
            D[:, :, g] = xg[:, g, :] @ wc[:, g, :].T
    return D


def int_gemm_loop(qx, wcodes, z, group_size: int):
    """Triple loop in Python integers (tiny inputs only): the same D."""
    M, K = qx.shape
    N = wcodes.shape[0]
    G = K // group_size
    D = np.zeros((M, N, G), dtype=np.int64)
    for m in range(M):
        for n in range(N):
            for k in range(K):
                g = k // group_size
                D[m, n, g] += int(qx[m, k]) * (int(wcodes[n, k]) - int(z[n, g]))
    return D


def epilogue(D, s_x, s_w):
    """Y64[m,n] = s_x[m] · Σ_g s_w[n,g] · D[m,n,g] (float64).

    FPTQuant page "3. 伪动态残差缩放": the per-token scale commutes with the
    bias-free linear, so it multiplies the integer product afterwards.
    """
    D = np.asarray(D, dtype=np.float64)
    sw = np.asarray(s_w, dtype=np.float64)
    acc = np.einsum("mng,ng->mn", D, sw)
    return np.asarray(s_x, dtype=np.float64)[:, None] * acc


def epilogue_by_group(qx, wq, s_x, cols=None, chunk: int = 1024):
    """(Y64, A) for whole-size outputs without holding D[M, N, G].

    Y64[m,n] = s_x[m] · Σ_g s_w[n,g] · D[m,n,g] -- the quantity of
    epilogue(int_gemm(...)) -- and A[m,n] = s_x[m] · Σ_g s_w[n,g] · |D[m,n,g]|,
    the magnitude of the summed terms.  D[:, :, g] is the integer product of
    group g (FlatQuant page, "核心思想"), each entry an integer of magnitude
    <= group·8·15, formed exactly by a float64 product of integer-valued
    arrays; the groups are then added in order, `chunk` output channels at a
    time (the summation order is free: the per-token scale commutes with the
    bias-free product, FPTQuant page "3. 伪动态残差缩放").  ``cols`` selects
    output channels of ``wq``.
    """
    qx = np.asarray(qx)
    M, K = qx.shape
    g = wq["group_size"]
    G = K // g
    idx = np.arange(wq["codes"].shape[0]) if cols is None else np.asarray(cols)
    x = qx.astype(np.float64).reshape(M, G, g)
    sx = np.asarray(s_x, dtype=np.float64)[:, None]
    Y = np.empty((M, len(idx)))
    A = np.empty((M, len(idx)))
    for c0 in range(0, len(idx), chunk):
        cc = idx[c0:c0 + chunk]
        w = _centered(wq["codes"][cc], wq["z"][cc], g).astype(np.float64)   # [n, G, g]
        sw = np.asarray(wq["s"][cc], dtype=np.float64)                      # [n, G]
        y = np.zeros((M, len(cc)))
        a = np.zeros((M, len(cc)))
        for j in range(G):
            Dg = x[:, j, :] @ w[:, j, :].T
            y += Dg * sw[:, j]
            a += np.abs(Dg) * sw[:, j]
        Y[:, c0:c0 + len(cc)] = sx * y
        A[:, c0:c0 + len(cc)] = sx * a
    return Y, A


def dequant_act(q, s_x):
    return np.asarray(q, dtype=np.float64) * np.asarray(s_x, dtype=np.float64)[:, None]


def dequant_weights(wq):
    """s · (u - z) per element, float64 [N, K]."""
    N, K = wq["codes"].shape
    g = wq["group_size"]
    c = _centered(wq["codes"], wq["z"], g).astype(np.float64)
    return (c * np.asarray(wq["s"], dtype=np.float64)[:, :, None]).reshape(N, K)


def linear(X, P1, P2, wq, c=None, alpha_a: float = 1.0, rows=None, cols=None, bits: int = 4):
    """Whole layer: Y64 = epilogue(int_gemm(Q(transform(X)), Q(W̃))).

    ``wq`` is the quantize_weights() result of the merged weights.  ``rows`` /
    ``cols`` restrict the computation to a subset of tokens / output channels
    (sampled checks at full size).  Returns dict(Y64, act, D).
    """
    Xs = np.asarray(X)
    if rows is not None:
        Xs = Xs[rows]
    act = transform_quant(Xs, P1, P2, c, alpha_a, bits)
    codes, s, z = wq["codes"], wq["s"], wq["z"]
    if cols is not None:
        codes, s, z = codes[cols], s[cols], z[cols]
    D = int_gemm(act["q"], codes, z, wq["group_size"])
    Y64 = epilogue(D, act["s_x"], s)
    return dict(Y64=Y64, act=act, D=D)


# ----------------------------------------------------------------------------
# Static activation quantization (steps fixed offline)
# ----------------------------------------------------------------------------
def calibrate_steps(Zc, per_channel: bool, ratio: float = 1.0):
    """Offline steps from a calibration batch of transformed activations Zc.

    The pages fix the steps offline (FPTQuant page, "核心贡献"; MergeQuant
    page, "技术框架" items 1 and 4: per-channel calibration with a clipping
    range) without giving the estimator; the plain reading taken here is the
    calibration range divided by the largest positive code:
    ratio · max|Zc| / 7 for the tensor, ratio · max_m |Zc[m, k]| / 7 per
    channel.  A channel that is zero over the whole batch gets step 1 (any
    positive step maps its zeros to code 0).  Returned as float32, the
    precision the steps are stored in.
    """
    Zc = np.abs(np.asarray(Zc, dtype=np.float64))
    if per_channel:
        st = ratio * Zc.max(axis=0) / 7.0
        st[st == 0] = 1.0
    else:
        st = np.array([ratio * Zc.max() / 7.0])
        if st[0] == 0:
            st[0] = 1.0
    return st.astype(np.float32)


def quantize_act_static(Z, steps, per_channel: bool):
    """Static INT4 activation codes with precomputed positive steps.

    FPTQuant page, "核心贡献" (static INT4): one step for the whole tensor,
    fixed offline, so no per-token absmax is taken at run time; the per-token
    scale is that step.  MergeQuant page, "核心思路" / "关键设计" item 2: one
    step per channel, migrated into the weights (see migrate_steps), so the
    activation side carries no runtime scale at all (s_x = 1).
    Codes clamp(round_half_even(Z / step), -8, 7).  Returns (q, t, s_x).
    """
    Z = np.asarray(Z, dtype=np.float64)
    st = np.asarray(steps, dtype=np.float64).reshape(-1)
    if per_channel:
        if st.shape[0] != Z.shape[1]:
            raise ValueError("one step per channel expected")
        t = Z / st[None, :]
        s_x = np.ones(Z.shape[0])
    else:
        if st.shape[0] != 1:
            raise ValueError("one step per tensor expected")
        t = Z / st[0]
        s_x = np.full(Z.shape[0], st[0])
    q = np.clip(np.rint(t), QMIN, QMAX).astype(np.int8)
    return q, t, s_x


def transform_quant_static(X, P1, P2, steps, per_channel: bool, c=None):
    """Transform, then static quantization and packing.  Returns dict(Z, s_x, q, t, packed)."""
    Z = kron_transform(X, P1, P2, c)
    q, t, s_x = quantize_act_static(Z, steps, per_channel)
    return dict(Z=Z, s_x=s_x, q=q, t=t, packed=pack_nibbles(q))


def migrate_steps(Wt, steps, out_dtype=np.float32):
    """Weight side of the step migration: W̃'[n, k] = W̃[n, k] · step_k.

    MergeQuant page, "关键设计" item 2: the per-channel activation steps are
    folded into the linear layer's weights, Σ_k (step_k q_k) W̃[n, k] =
    Σ_k q_k W̃'[n, k].  The float64 product of two float32 values is exact,
    so one rounding to float32 gives the correctly rounded product.
    """
    W64 = np.asarray(Wt, dtype=np.float64)
    st = np.asarray(steps, dtype=np.float64).reshape(1, -1)
    return (W64 * st).astype(out_dtype)


def linear_static(X, P1, P2, wq, steps, per_channel: bool, c=None, rows=None, cols=None):
    """Whole layer with static activation steps.  With per-channel steps ``wq``
    quantizes the migrated weights migrate_steps(W̃, steps).  Returns
    dict(Y64, act, D)."""
    Xs = np.asarray(X)
    if rows is not None:
        Xs = Xs[rows]
    act = transform_quant_static(Xs, P1, P2, steps, per_channel, c)
    codes, s, z = wq["codes"], wq["s"], wq["z"]
    if cols is not None:
        codes, s, z = codes[cols], s[cols], z[cols]
    D = int_gemm(act["q"], codes, z, wq["group_size"])
    Y64 = epilogue(D, act["s_x"], s)
    return dict(Y64=Y64, act=act, D=D)
