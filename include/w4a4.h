/*
 * w4a4.h — C ABI of libw4a4.so, a W4A4 quantized linear layer for AMD MI355X
 * (gfx950).
 *
 * The layer is the one the FlatQuant page ("FlatQuant: Flatness Matters for
 * LLM Quantization", section 核心思想) writes as Y ≈ Q(X P) · Q(P^-1 W^T),
 * with P = P1 ⊗ P2 (section Kronecker 分解), an optional per-channel scale
 * diag(c) and clipping thresholds (section 额外可学习组件), and the
 * activation transform fused with quantization per token tile (section
 * 高效 Kernel 设计).  The quantizer is the uniform one of the FRM-PTQ page
 * ("FRM-PTQ: Feature Relationship Matching Enhanced Low-Bit Post-Training
 * Quantization for Large Language Models", section 初步介绍), with 4-bit
 * codes; weights may use per-group scales (the same page's multi-granularity
 * group quantization).
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Buffers are caller-allocated DEVICE memory unless stated otherwise; the
 *    library keeps no pointer after the call returns and never allocates on
 *    the compute path (scratch memory comes in through `ws`).
 *  - fp16 values are passed as uint16_t bit patterns (IEEE binary16).
 *  - Layouts are row-major.  A matrix of 4-bit codes [R, K] is stored as
 *    uint8 [R, K/2]; byte j of a row holds code 2j in its low nibble and code
 *    2j+1 in its high nibble.  Signed codes (-8..7) are two's-complement
 *    nibbles; unsigned codes (0..15) are stored as is.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *    asynchronously; nothing synchronizes.  Device faults surface at the
 *    caller's next synchronization.
 *  - Return value: W4A4_OK (0) or a negative W4A4_ERR_* code.  On an error
 *    no kernel has been launched and no output has been written;
 *    w4a4_last_error() returns a message (per host thread).  Nothing aborts
 *    and no C++ exception crosses this interface.
 *  - Device pointers must be 16-byte aligned (W4A4_ERR_ALIGNMENT otherwise).
 *  - Non-finite inputs are outside the contract (codes are then undefined).
 *  - Calls are re-entrant; concurrent calls must not share output or
 *    workspace buffers.
 */
#ifndef W4A4_H_
#define W4A4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A4_OK 0
#define W4A4_ERR_INVALID_ARG (-1) /* null pointer, negative or inconsistent size */
#define W4A4_ERR_UNSUPPORTED (-2) /* valid but not supported shape (see limits) */
#define W4A4_ERR_ALIGNMENT (-3)   /* a device pointer is not 16-byte aligned */
#define W4A4_ERR_WORKSPACE (-4)   /* workspace missing or smaller than required */
#define W4A4_ERR_HIP (-5)         /* a HIP runtime call or launch failed */

/* Limits: 1 <= K <= 65536, K = n1*n2, K % 128 == 0 for the GEMM, K % 16 == 0
 * for the activation path; 1 <= n1, n2 <= 256; M >= 0; N >= 1. */
#define W4A4_MAX_K 65536
#define W4A4_MAX_FACTOR 256

/* Description of a quantized weight matrix W̃ [N, K].
 *   group_size: number of consecutive input channels sharing one scale (and
 *               zero point): K for one scale per output channel, otherwise a
 *               multiple of 128 that divides K.  G = K / group_size.
 *   asymmetric: 0 -> signed codes q in [-8, 7], zero point 0;
 *               1 -> unsigned codes u in [0, 15] with a per-group zero point
 *                    z (an integer 0..15 stored as fp16). */
typedef struct w4a4_weight_desc {
    int32_t N;
    int32_t K;
    int32_t group_size;
    int32_t asymmetric;
} w4a4_weight_desc;

/* Library version, (major << 16) | (minor << 8) | patch. */
int w4a4_version(void);

/* Static string for a status code. */
const char* w4a4_status_str(int status);

/* Message of the last failing call made by this host thread ("" if none). */
const char* w4a4_last_error(void);

/* Kernel selection override, for tests and tuning sweeps only (normal use
 * never needs it).  `which` names a dispatcher:
 *   W4A4_OVERRIDE_PREFILL_TILE  prefill GEMM configurations (M > 64);
 *   W4A4_OVERRIDE_DECODE        decode GEMM variants (M <= 64);
 *   W4A4_OVERRIDE_F6_TILE       configurations of the fp6-pipe product;
 *   W4A4_OVERRIDE_TILE_GROUP    M tiles per group in the prefill GEMM's
 *                               order of output tiles (index = the count).
 * index in [0, w4a4_kernel_config_count(which)) forces that configuration for
 * every later call in this process; -1 restores the automatic choice.  An
 * index past the table, or a configuration without the call's weight mode,
 * also leaves the choice automatic.  Process-wide and atomic, but a call
 * running on another thread may see the old or the new value.  Returns the
 * previous index (>= -1), or W4A4_ERR_INVALID_ARG for an unknown `which` or
 * an index below -1. */
#define W4A4_OVERRIDE_PREFILL_TILE 0
#define W4A4_OVERRIDE_DECODE 1
#define W4A4_OVERRIDE_F6_TILE 2
#define W4A4_OVERRIDE_TILE_GROUP 3   /* M tiles per group of the prefill tile order */
int w4a4_set_kernel_override(int32_t which, int32_t index);

/* Number of configurations behind `which` (as above), or
 * W4A4_ERR_INVALID_ARG. */
int w4a4_kernel_config_count(int32_t which);

/* ------------------------------------------------------------------------ */
/* Offline weight preparation                                               */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace w4a4_merge_weights needs for factors (n1, n2). */
size_t w4a4_merge_workspace_bytes(int32_t n1, int32_t n2, int32_t K);

/* Merge the inverse transform into the weights (offline):
 *   W̃ = W · diag(1/c) · (P1 ⊗ P2)^-T,  row n: P1^-1 · W̄_n · P2^-T,
 * FlatQuant page, section Kronecker 分解 (weight-side factor
 * P1^-1 ×1 W̃ ×2 (P2^-1)^T) and section 额外可学习组件 (diag(c) is undone
 * on the weights).  P1 and P2 are inverted on the device (Gauss-Jordan with
 * partial pivoting, float64); the merge runs in float64 and is rounded once
 * to float32.
 *   W  [N, K] fp32 (device), P1 [n1, n1] fp32, P2 [n2, n2] fp32 (device),
 *   c  [K] fp32 or NULL (no channel scaling), Wt [N, K] fp32 output.
 *   ws: device workspace of w4a4_merge_workspace_bytes(n1, n2, K) bytes.
 * Offline and not on the hot path: the call synchronizes `stream` once to
 * read back the pivots and returns W4A4_ERR_INVALID_ARG if P1 or P2 is
 * numerically singular (a pivot below 1e-300 in magnitude). */
int w4a4_merge_weights(const float* W, int32_t N, int32_t K, int32_t n1, int32_t n2,
                       const float* P1, const float* P2, const float* c, float* Wt,
                       void* ws, size_t ws_bytes, void* stream);

/* Quantize and pack merged weights W̃ [N, K] fp32 (offline).
 * FRM-PTQ page, section 初步介绍: Q(W) = clamp(round(W/s) + z, 0, 2^b - 1),
 * b = 4, round half to even; FlatQuant page, section 额外可学习组件: alpha_w
 * in (0, 1] scales the range.  Per group of desc->group_size channels:
 *   symmetric : s = fp16(alpha_w*max|v|/7), q = clamp(round(v/s), -8, 7)
 *   asymmetric: lo = alpha_w*min(min v, 0), hi = alpha_w*max(max v, 0),
 *               s = fp16((hi-lo)/15), z = clamp(round(-lo/s), 0, 15),
 *               u = clamp(round(v/s) + z, 0, 15)
 * The scale arithmetic runs in float64 and s is rounded directly to fp16;
 * codes are computed with the stored fp16 s.  A zero scale gives zero codes
 * (and z = 0).
 *   Wq  [N, K/2] uint8 packed codes,  s_w [N, G] fp16 scales,
 *   z_w [N, G] fp16 zero points (required iff asymmetric, else may be NULL). */
int w4a4_pack_weights(const w4a4_weight_desc* desc, const float* Wt, float alpha_w,
                      uint8_t* Wq, uint16_t* s_w, uint16_t* z_w, void* stream);

/* Step migration for static per-channel activation steps (offline).
 * MergeQuant page ("MergeQuant: Accurate 4-bit Static Quantization of Large
 * Language Models by Channel-wise Calibration"), sections 核心思路 and
 * 关键设计 item 2: the per-channel quantization steps of the layer's input
 * are folded into its weights, so that
 *   Σ_k (step_k · q_k) · W̃[n, k] = Σ_k q_k · Wm[n, k],  Wm[n, k] = W̃[n, k] · step_k.
 *   Wt [N, K] fp32 merged weights, steps [K] fp32 (positive), Wm [N, K] fp32
 *   output: each element is the correctly rounded fp32 product.  Wm may be
 *   Wt (in place).  K must be a multiple of 4.  Quantize Wm with
 *   w4a4_pack_weights and run the layer with w4a4_linear_static(...,
 *   per_channel = 1). */
int w4a4_migrate_steps(const float* Wt, int32_t N, int32_t K, const float* steps, float* Wm,
                       void* stream);

/* ------------------------------------------------------------------------ */
/* Online activation path                                                    */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace w4a4_transform_quant needs (0 is possible); has_c != 0
 * when the call passes a channel scale c.  Without c the common factor
 * shapes (n1 <= 128 and n2 in {16, 32, 64, 128}, both multiples of 16) run
 * one fused kernel and need no workspace. */
size_t w4a4_transform_quant_workspace_bytes(int32_t M, int32_t n1, int32_t n2, int32_t has_c);

/* Fused activation transform + per-token INT4 quantization + packing.
 * FlatQuant page, section Kronecker 分解 (activation factor P1^T ×1 X̃ ×2 P2)
 * and section 高效 Kernel 设计 (the token tile is transformed and quantized
 * on chip); section 额外可学习组件 (diag(c), alpha_a).  For each token m:
 *   Z_m  = P1^T · reshape(x_m ⊙ c, n1, n2) · P2     (row-major reshape,
 *          k = i*n2 + j; equals x_m · (P1 ⊗ P2)), computed in fp32 or better
 *   s_x[m] = alpha_a * max_k |Z_m[k]| / 7           (fp32)
 *   q    = clamp(round_half_even(Z_m / s_x[m]), -8, 7), 0 if s_x[m] == 0
 *   Xq[m, :] = packed q.
 *   X [M, K] fp16, P1 [n1, n1] fp32 (P in P = P1 ⊗ P2, NOT its transpose),
 *   P2 [n2, n2] fp32, c [K] fp32 or NULL, Xq [M, K/2] uint8, s_x [M] fp32.
 *   ws: device workspace, w4a4_transform_quant_workspace_bytes(M, n1, n2,
 *       c != NULL) bytes (may be NULL when that is 0). */
int w4a4_transform_quant(const uint16_t* X, int32_t M, int32_t n1, int32_t n2,
                         const float* P1, const float* P2, const float* c, float alpha_a,
                         uint8_t* Xq, float* s_x, void* ws, size_t ws_bytes, void* stream);

/* Static-step form of w4a4_transform_quant: the activation steps are fixed
 * offline and read from `steps`, so no per-token absmax is taken.
 *   per_channel = 0: FPTQuant page, section 核心贡献 (static INT4
 *     quantization): one step for the tensor, steps[0];
 *     q = clamp(round_half_even(Z_m / steps[0]), -8, 7), s_x[m] = steps[0].
 *   per_channel = 1: MergeQuant page, sections 核心思路 and 关键设计 items
 *     1-2 (per-channel static steps migrated into the weights): steps[K];
 *     q[k] = clamp(round_half_even(Z_m[k] / steps[k]), -8, 7), s_x[m] = 1
 *     (the steps live in the weights, see w4a4_migrate_steps).
 * Z_m, X, P1, P2, c, Xq, s_x and ws as for w4a4_transform_quant (same
 * workspace size).  steps: device fp32, 16-byte aligned, positive and finite
 * (the values stay on the device and are not checked).  The division by a
 * per-channel step uses the hardware reciprocal (within one ulp), so a code
 * may differ from the exact quotient's only where Z/step lies within a few
 * 1e-6 of a rounding tie. */
int w4a4_transform_quant_static(const uint16_t* X, int32_t M, int32_t n1, int32_t n2,
                                const float* P1, const float* P2, const float* c,
                                const float* steps, int32_t per_channel, uint8_t* Xq,
                                float* s_x, void* ws, size_t ws_bytes, void* stream);

/* Debug / parity form of the transform: writes Z [M, K] fp32 (the value that
 * w4a4_transform_quant quantizes, same kernels, same arithmetic). */
int w4a4_transform(const uint16_t* X, int32_t M, int32_t n1, int32_t n2,
                   const float* P1, const float* P2, const float* c, float* Z,
                   void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* INT4 x INT4 GEMM                                                          */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace w4a4_gemm needs for M tokens (0 is possible).  The
 * library owns its contents during a call and leaves nothing in it that a
 * later call reads:
 *  - M <= 64 with per-channel weights or groups of 128: the int32 (fp32 for
 *    groups) partial sums of the split-K decode kernel, S ranges x M x N, S
 *    chosen from the shape (e.g. 8 for K = 28672, N = 8192);
 *  - M > 64 with asymmetric groups of 128: the per-token group sums of the
 *    zero-point correction, M x (K / 128 rounded up to a multiple of 16) fp16
 *    words;
 *  - otherwise none. */
size_t w4a4_gemm_workspace_bytes(int32_t M, const w4a4_weight_desc* desc);

/* Y = dequant(Xq · Wq^T) — FlatQuant page, section 核心思想, the product
 * Q(XP) · Q(P^-1 W^T); FPTQuant page ("FPTQuant: Function-Preserving
 * Transforms for LLM Quantization", section 3. 伪动态残差缩放): a per-token
 * scale commutes with a bias-free linear, so it is applied after the integer
 * product.  With D[m,n,g] = Σ_{k in group g} q_x[m,k]·(u[n,k] - z[n,g])
 * accumulated exactly in int32:
 *   Y[m, n] = fp16( s_x[m] · Σ_g s_w[n,g] · D[m,n,g] )    (fp32 epilogue)
 *   Xq [M, K/2] uint8 (signed codes), s_x [M] fp32, Wq [N, K/2] uint8,
 *   s_w [N, G] fp16, z_w [N, G] fp16 (asymmetric only), Y [M, N] fp16.
 *   ws: device workspace, w4a4_gemm_workspace_bytes(M, desc). */
int w4a4_gemm(const uint8_t* Xq, const float* s_x, int32_t M, const w4a4_weight_desc* desc,
              const uint8_t* Wq, const uint16_t* s_w, const uint16_t* z_w, uint16_t* Y,
              void* ws, size_t ws_bytes, void* stream);

/* Debug / parity form: the exact int32 accumulators D [M, N, G] (row-major,
 * g fastest) of the same product, before any scaling. */
int w4a4_gemm_i32(const uint8_t* Xq, int32_t M, const w4a4_weight_desc* desc,
                  const uint8_t* Wq, const uint16_t* z_w, int32_t* D, void* stream);

/* Name of the kernel configuration w4a4_gemm launches for M tokens and this
 * weight layout on the current device (for traces and reports), or NULL if
 * desc is invalid (message in w4a4_last_error).  Static storage; launches
 * nothing. */
const char* w4a4_gemm_kernel_name(int32_t M, const w4a4_weight_desc* desc);

/* ------------------------------------------------------------------------ */
/* Whole layer                                                               */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace w4a4_linear needs (has_c as for transform_quant). */
size_t w4a4_linear_workspace_bytes(int32_t M, int32_t n1, int32_t n2, int32_t has_c,
                                   const w4a4_weight_desc* desc);

/* w4a4_transform_quant followed by w4a4_gemm on the same stream, with the
 * packed activations and their scales kept in `ws`:
 *   Y [M, N] fp16 = W4A4 linear of X [M, K] fp16 (K = n1*n2 = desc->K).
 * With asymmetric groups of 128 and M > 64, the token-batched transform
 * kernels also write the GEMM's per-token group sums into `ws`, so the
 * GEMM's own pre-pass is not launched; Y is that of the two calls, bit for
 * bit. */
int w4a4_linear(const uint16_t* X, int32_t M, int32_t n1, int32_t n2,
                const float* P1, const float* P2, const float* c, float alpha_a,
                const w4a4_weight_desc* desc, const uint8_t* Wq, const uint16_t* s_w,
                const uint16_t* z_w, uint16_t* Y, void* ws, size_t ws_bytes, void* stream);

/* w4a4_linear for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * kernels and results as w4a4_linear, with its workspace (packed activations,
 * their scales, the transform's intermediates) taken from a scratch array of
 * W4A4_NOALLOC_SCRATCH_BYTES that the library holds in device memory, one per
 * device it runs on, until the process ends.  The caller still passes every
 * input and the output Y.  No call allocates or frees memory; the scratch's
 * device address is looked up once per device (first call with that device
 * current).  A call whose workspace would exceed the scratch returns
 * W4A4_ERR_UNSUPPORTED and launches nothing.  Every call on a device shares
 * that device's scratch and leaves its contents behind; each call writes all
 * the scratch it reads, so nothing has to be cleared, but calls that overlap
 * on one device (several streams or threads) race on it. */
#define W4A4_NOALLOC_SCRATCH_BYTES (32u << 20)
int w4a4_linear_noalloc(const uint16_t* X, int32_t M, int32_t n1, int32_t n2, const float* P1,
                        const float* P2, const float* c, float alpha_a,
                        const w4a4_weight_desc* desc, const uint8_t* Wq, const uint16_t* s_w,
                        const uint16_t* z_w, uint16_t* Y, void* stream);

/* w4a4_linear with static activation steps (w4a4_transform_quant_static
 * followed by w4a4_gemm; same workspace as w4a4_linear).  With
 * per_channel = 1 the weights must carry the migrated steps
 * (w4a4_migrate_steps before w4a4_pack_weights): the epilogue then scales by
 * s_w alone, as the MergeQuant page's step migration (关键设计 item 2) has no
 * activation dequantization after the product. */
int w4a4_linear_static(const uint16_t* X, int32_t M, int32_t n1, int32_t n2,
                       const float* P1, const float* P2, const float* c, const float* steps,
                       int32_t per_channel, const w4a4_weight_desc* desc, const uint8_t* Wq,
                       const uint16_t* s_w, const uint16_t* z_w, uint16_t* Y, void* ws,
                       size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* 3-bit codes (W3A3)                                                        */
/* ------------------------------------------------------------------------ */
/* FRM-PTQ page, introduction and contributions (weights and activations at
 * 3 bits, W3A3) with the quantizer of its section 初步介绍 at b = 3: the same
 * layer with codes in [-4, 3] (activations and symmetric weights, scale
 * alpha * max / 3) or [0, 7] (asymmetric weights, scale (hi - lo) / 7).  The
 * codes are stored one per nibble exactly like the 4-bit ones, so
 * w4a4_gemm and every buffer layout are unchanged.  bits must be 3 or 4
 * (4 is the same as the plain entry points); anything else returns
 * W4A4_ERR_UNSUPPORTED. */
int w4a4_pack_weights_bits(const w4a4_weight_desc* desc, const float* Wt, float alpha_w,
                           int32_t bits, uint8_t* Wq, uint16_t* s_w, uint16_t* z_w,
                           void* stream);
int w4a4_transform_quant_bits(const uint16_t* X, int32_t M, int32_t n1, int32_t n2,
                              const float* P1, const float* P2, const float* c, float alpha_a,
                              int32_t bits, uint8_t* Xq, float* s_x, void* ws, size_t ws_bytes,
                              void* stream);
/* Workspace: w4a4_linear_workspace_bytes. */
int w4a4_linear_bits(const uint16_t* X, int32_t M, int32_t n1, int32_t n2, const float* P1,
                     const float* P2, const float* c, float alpha_a, int32_t bits,
                     const w4a4_weight_desc* desc, const uint8_t* Wq, const uint16_t* s_w,
                     const uint16_t* z_w, uint16_t* Y, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Ternary weights (W1.58A16)                                                */
/* ------------------------------------------------------------------------ */
/* PT2-LLM page, section 关键设计 item 2: each row of a block of 128 columns is
 * alpha * T + mu with T in {-1, 0, 1} (ATQ), fitted by ITF, which alternates
 * the closed-form least-squares (alpha, mu) for fixed T with the nearest grid
 * point T for fixed (alpha, mu), mu starting at the block row's mean and
 * alpha at its mean absolute deviation.  The layer is weight-only:
 * Y = X · Ŵ^T with fp16 activations X (no activation transform).
 *
 * Layouts (rows tiled by 16: Nt = N rounded up to a multiple of 16, padding
 * rows all zero; w4a4_ternary_weight_bytes gives the sizes):
 *   Tq  uint8 [Nt * K/4]: two-bit codes c = t + 1 in little-endian 32-bit
 *       words of 16 codes (code 2s of a word at bits 2s, code 2s + 1 at bits
 *       16 + 2s).  The 32 codes 128 g + 32 s + 8 q + j (s = 0..3, j = 0..7, in
 *       that order) of block g form lane group q's 8-byte piece (q = 0..3).
 *       Tile t = n / 16 starts at byte 4 K t; in it the pair of blocks
 *       (2p, 2p + 1) fills the 1024 bytes from 1024 p, the 16 bytes at
 *       1024 p + 16 (16 q + r) holding row r = n % 16's pieces of block 2p and
 *       then 2p + 1; an unpaired last block (odd K/128) has row r's piece q at
 *       1024 p + 8 (16 q + r);
 *   am  uint32 [Nt * K/128]: the word of (row n, block g) at
 *       ((n / 16) K/128 + g) 16 + n % 16, the block's alpha as fp16 bits in the
 *       low half and mu in the high half (both one rounding from float64). */
#define W4A4_TERNARY_BLOCK 128
#define W4A4_TERNARY_MAX_M 64

/* Bytes of Tq and of am for N rows of K weights (N >= 1, K a multiple of
 * 128); returns W4A4_OK or W4A4_ERR_INVALID_ARG / W4A4_ERR_UNSUPPORTED. */
int w4a4_ternary_weight_bytes(int32_t N, int32_t K, size_t* tq_bytes, size_t* am_bytes);

/* Offline: ternarize merged or raw fp32 weights Wt [N][K] with `iters` ITF
 * iterations (10 in the pages' setting), float64 arithmetic; the final codes
 * are the nearest points of the stored (fp16) grid.  K must be a multiple of
 * 128. */
int w4a4_pack_ternary(const float* Wt, int32_t N, int32_t K, int32_t iters, uint8_t* Tq,
                      uint32_t* am, void* stream);

/* The inverse of the tiled layout above (a bijection on the N real rows):
 * T int8 [N][K] gets the codes t in {-1, 0, 1}, row-major; alpha and mu fp16
 * [N][K/128] get the parameter halves of each block's word.  For reading
 * packed weights back (tests, inspection); one launch, no workspace.  All
 * pointers device memory, 16-byte aligned. */
int w4a4_unpack_ternary(const uint8_t* Tq, const uint32_t* am, int32_t N, int32_t K, int8_t* T,
                        uint16_t* alpha, uint16_t* mu, void* stream);

/* Bytes of workspace w4a4_ternary_gemm needs: 0 when the shape's output
 * tiles fill the GPU by themselves (ws may then be NULL), else the fp32
 * partial sums of a K split across workgroups; 0 for invalid shapes too. */
size_t w4a4_ternary_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K);

/* Y [M][N] fp16 = X [M][K] fp16 · Ŵ^T for decode-sized batches,
 * 0 <= M <= W4A4_TERNARY_MAX_M (larger M returns W4A4_ERR_UNSUPPORTED).  The
 * fp16 MFMA products are exact (codes enter as the fp16 values c * 2^-14) and
 * the sums run in fp32.  One launch; two when the workspace is non-empty (the
 * product with K split across workgroups, then the merge of the splits). */
int w4a4_ternary_gemm(const uint16_t* X, int32_t M, int32_t N, int32_t K, const uint8_t* Tq,
                      const uint32_t* am, uint16_t* Y, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* INT4 x INT4 GEMM on the fp6 matrix pipe (prefill)                         */
/* ------------------------------------------------------------------------ */
/* The same layer products as w4a4_gemm (FlatQuant page, section 核心思想;
 * FRM-PTQ page, section 初步介绍; FPTQuant page, section 3. 伪动态残差缩放):
 * D[m,n,g] = sum over the group of q_x (u - z) and
 * Y = fp16(s_x[m] sum_g s_w[n,g] D[m,n,g]).  Every code v the product takes
 * (q in [-8, 7], u - z in [-15, 15]) is held as v / 2, which an fp6 E2M3
 * number represents exactly, and the sums are exact in fp32, so D is
 * computed exactly on the fp6 matrix pipe (twice the int8 rate).  The
 * operands are kept in an fp6 fragment layout: rows padded to a multiple of
 * 32 (padding zero), 0.75 bytes per code. */

/* Bytes of the fp6 weights for desc (0 for an invalid desc). */
size_t w4a4_weights_f6_bytes(const w4a4_weight_desc* desc);

/* Offline: packed weights (w4a4_pack_weights' Wq and, if asymmetric, z_w) to
 * the fp6 layout W6 (w4a4_weights_f6_bytes bytes), exactly. */
int w4a4_pack_weights_f6(const w4a4_weight_desc* desc, const uint8_t* Wq, const uint16_t* z_w,
                         uint8_t* W6, void* stream);

/* Workspace of w4a4_gemm_f6: the activations in the fp6 layout. */
size_t w4a4_gemm_f6_workspace_bytes(int32_t M, const w4a4_weight_desc* desc);

/* Y [M][N] fp16 from packed activations Xq [M][K/2] (w4a4_transform_quant's
 * output), s_x, the fp6 weights W6 and s_w; two launches (activations to the
 * fp6 layout in ws, then the product). */
int w4a4_gemm_f6(const uint8_t* Xq, const float* s_x, int32_t M, const w4a4_weight_desc* desc,
                 const uint8_t* W6, const uint16_t* s_w, uint16_t* Y, void* ws, size_t ws_bytes,
                 void* stream);

/* Name of the kernel configuration w4a4_gemm_f6 would run (host query). */
const char* w4a4_gemm_f6_kernel_name(int32_t M, const w4a4_weight_desc* desc);

/* The whole dynamic layer (as w4a4_linear) with the product on the fp6 pipe;
 * weights from w4a4_pack_weights_f6. */
size_t w4a4_linear_f6_workspace_bytes(int32_t M, int32_t n1, int32_t n2, int32_t has_c,
                                      const w4a4_weight_desc* desc);
int w4a4_linear_f6(const uint16_t* X, int32_t M, int32_t n1, int32_t n2, const float* P1,
                   const float* P2, const float* c, float alpha_a, const w4a4_weight_desc* desc,
                   const uint8_t* W6, const uint16_t* s_w, uint16_t* Y, void* ws,
                   size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Single-kernel decode layer                                                */
/* ------------------------------------------------------------------------ */

/* Bytes of the sync buffer w4a4_linear_decode needs. */
#define W4A4_DECODE_SYNC_BYTES 1024
/* 32-bit word of the sync buffer that is non-zero once a call has timed out
 * waiting for its activations (that call's Y is then invalid). */
#define W4A4_DECODE_SYNC_ERROR_WORD 128

/* Bytes of workspace w4a4_linear_decode needs (0 for M outside [1, 16]). */
size_t w4a4_linear_decode_workspace_bytes(int32_t M, int32_t n1, int32_t n2);

/* The whole layer for a few tokens in ONE kernel launch: the same result as
 * w4a4_linear (steps == NULL) or w4a4_linear_static (steps != NULL), with
 * the weight stream starting while the activations are transformed.
 * FlatQuant page, section 高效 Kernel 设计 (transform and quantization fused
 * with the layer); MergeQuant page, section 问题定义 (the per-token quantize
 * and dequantize steps are a large share of autoregressive decoding).
 *   Arguments as for w4a4_linear / w4a4_linear_static (no diag(c)); steps
 *   NULL selects per-token dynamic scales with alpha_a, otherwise
 *   per_channel selects the static form (alpha_a is then ignored).
 *   sync: device buffer of W4A4_DECODE_SYNC_BYTES, zero-filled by the caller
 *   once before its first use; every call leaves it valid for the next (its
 *   counters carry a tag unique to each call).  Calls that share a sync
 *   buffer or a workspace must not run concurrently.
 *   ws: device workspace of w4a4_linear_decode_workspace_bytes(M, n1, n2)
 *   bytes.
 * Supported: 1 <= M <= 16, n2 = 128, n1 in {64, 224}, the activation rows
 * and the scale table of 16 weight rows within one CU's LDS, and no more
 * transform workgroups (M * n1 / 16) than the device holds at once;
 * otherwise W4A4_ERR_UNSUPPORTED and nothing runs (use w4a4_linear).  A
 * wait inside the kernel is bounded (20 ms); if it runs out, word
 * W4A4_DECODE_SYNC_ERROR_WORD of sync becomes non-zero. */
int w4a4_linear_decode(const uint16_t* X, int32_t M, int32_t n1, int32_t n2,
                       const float* P1, const float* P2, float alpha_a, const float* steps,
                       int32_t per_channel, const w4a4_weight_desc* desc, const uint8_t* Wq,
                       const uint16_t* s_w, const uint16_t* z_w, uint16_t* Y, void* ws,
                       size_t ws_bytes, uint32_t* sync, void* stream);

/* ------------------------------------------------------------------------ */
/* INT4 KV cache with per-head transforms, and decode attention over it      */
/* ------------------------------------------------------------------------ */
/* FlatQuant page, section Transformer 集成: the key cache and the value cache
 * each carry a transform applied per head, P_h and P_v (full d x d matrices,
 * not Kronecker-factored).  The caches hold Q(k·P_h) and Q(v·P_v); the query
 * takes P_h^-T so that (q·P_h^-T)·(k·P_h)^T = q·k^T (section 核心思想: the
 * inverse goes on the other operand), and P_v^-1 belongs to the output
 * projection's weights, so the attention output is in the P_v basis.
 * FPTQuant page, sections 核心贡献 and 实验结果: the KV cache in INT4
 * (W4A4KV4).  Quantizer: the activations' symmetric one per head vector of
 * each token, s = alpha * max|z| / 7 (fp32), codes clamp(rne(z / s), -8, 7).
 *
 * Cache layout of one layer (head size d = 128, the only size supported):
 *   k_cache  uint8  [batch][heads_kv][max_seq][64]: the key codes of a token
 *            and head, two per byte, low nibble = even channel;
 *   v_cache  uint32 [batch][heads_kv][max_seq / 8][128]: nibble j (bits
 *            4j..4j+3) of word [blk][ch] is the value code of token 8*blk + j,
 *            channel ch;
 *   k_scale, v_scale  float [batch][heads_kv][max_seq]: the scales.
 * Codes are two's-complement nibbles.  max_seq must be a positive multiple
 * of 32.  P matrices are float [d][d] row-major (shared by the heads) or
 * [heads_kv][d][d] (per_head = 1). */
#define W4A4_KV_HEAD_DIM 128

/* Bytes of the three cache buffers of one layer (any pointer may be NULL).
 * Returns W4A4_OK or W4A4_ERR_INVALID_ARG / W4A4_ERR_UNSUPPORTED. */
int w4a4_kv_cache_bytes(int32_t batch, int32_t heads_kv, int32_t head_dim, int32_t max_seq,
                        size_t* k_bytes, size_t* v_bytes, size_t* scale_bytes);

/* Bytes of workspace w4a4_kv_query_factor needs for count matrices. */
size_t w4a4_kv_query_factor_workspace_bytes(int32_t head_dim, int32_t count);

/* Offline: P_h_inv_t[i] = (P_h[i])^-T for count matrices of d x d (float,
 * computed in float64 by Gauss-Jordan elimination with partial pivoting and
 * rounded once).  Synchronizes the stream.  A singular matrix returns
 * W4A4_ERR_INVALID_ARG (the output is then undefined). */
int w4a4_kv_query_factor(const float* P_h, int32_t head_dim, int32_t count, float* P_h_inv_t,
                         void* ws, size_t ws_bytes, void* stream);

/* Transform, quantize and write new tokens into the caches.
 *   k, v: fp16 [tokens][heads_kv][d], post-RoPE keys and values.
 *   Segment i (0 <= i < segments) is tokens cu_tokens[i] .. cu_tokens[i+1]-1
 *   of k and v; they go to sequence seg_seq[i] at positions seg_start[i],
 *   seg_start[i]+1, ...  seg_seq, seg_start: int32 [segments] and cu_tokens:
 *   int32 [segments + 1], DEVICE arrays, cu_tokens non-decreasing.
 *   A segment whose sequence is outside [0, batch), whose start is outside
 *   [0, max_seq) or whose token range is outside [0, tokens] is skipped;
 *   positions past max_seq are dropped.  Every (sequence, position) may
 *   appear at most once per call.
 *   P_h, P_v, per_head: the per-head transforms; alpha_k, alpha_v in (0, 1]
 *   the clipping ratios.  Positions not written keep their contents (value
 *   words shared with other positions are merged).
 * Decode (one token per sequence) and prefill (long segments) use the same
 * call.  Host-checked: d = 128, heads_kv >= 1, batch >= 0, tokens >= 0,
 * segments >= 0, max_seq a positive multiple of 32, alignment. */
int w4a4_kv_append(const uint16_t* k, const uint16_t* v, int32_t tokens, const int32_t* seg_seq,
                   const int32_t* seg_start, const int32_t* cu_tokens, int32_t segments,
                   int32_t heads_kv, int32_t head_dim, const float* P_h, const float* P_v,
                   int32_t per_head, float alpha_k, float alpha_v, uint8_t* k_cache,
                   float* k_scale, uint32_t* v_cache, float* v_scale, int32_t batch,
                   int32_t max_seq, void* stream);

/* Bytes of workspace w4a4_attn_decode needs (0 for invalid shapes). */
size_t w4a4_attn_decode_workspace_bytes(int32_t batch, int32_t heads_q, int32_t heads_kv,
                                        int32_t head_dim, int32_t max_seq);

/* Decode attention over the INT4 caches, one query token per sequence:
 *   out[b][h] = softmax(sm_scale * q~[b][h] · K^[b][h/G][:L]^T) · V^[b][h/G][:L]
 * with q~ = q · P_h^-T, K^ and V^ the dequantized cache contents
 * (scale * code), L = lengths[b] clamped to [0, max_seq] and G =
 * heads_q / heads_kv.  An empty context (L = 0) gives zeros.  The output
 * stays in the P_v basis.
 *   q: fp16 [batch][heads_q][d], post-RoPE queries.
 *   P_h_inv_t: float [d][d] or [heads_kv][d][d] (per_head = 1), from
 *   w4a4_kv_query_factor.
 *   lengths: int32 [batch], DEVICE array.
 *   out: fp16 [batch][heads_q][d].
 *   ws: w4a4_attn_decode_workspace_bytes(...) bytes.
 * Host-checked: d = 128, heads_q a multiple of heads_kv with G <= 16,
 * batch >= 0, max_seq a positive multiple of 32, sm_scale finite and > 0,
 * alignment.  Three kernel launches (query transform, chunked partial
 * attention, merge). */
int w4a4_attn_decode(const uint16_t* q, int32_t batch, int32_t heads_q, int32_t heads_kv,
                     int32_t head_dim, const float* P_h_inv_t, int32_t per_head,
                     const uint8_t* k_cache, const float* k_scale, const uint32_t* v_cache,
                     const float* v_scale, const int32_t* lengths, int32_t max_seq,
                     float sm_scale, uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Measurement aid                                                           */
/* ------------------------------------------------------------------------ */

/* A plain streaming read of `bytes` bytes of device memory (16-byte loads
 * over a persistent grid), for measuring the HBM read rate one launch of
 * that size reaches: the ceiling against which the bandwidth of the decode
 * GEMM (an HBM-bound read of the packed weights) is judged.  The XOR of all
 * 32-bit words of buf is XORed into *out (device word; clear it first to
 * read the checksum).  buf and out 16-byte aligned, bytes a multiple of 16;
 * W4A4_ERR_INVALID_ARG / W4A4_ERR_ALIGNMENT otherwise.  One launch. */
int w4a4_read_probe(const void* buf, size_t bytes, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A4_H_ */
