// Internal launch interface between the C ABI layer (api.cpp) and the
// kernel translation units.  Every launcher assumes validated arguments and
// returns the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a4 {

// ---- kernel selection overrides (w4a4_set_kernel_override) -----------------
// which: 0 prefill GEMM tile, 1 decode GEMM variant, 2 fp6 tile, 3 M tiles per
// group of the prefill GEMM's tile order; -1 = automatic
constexpr int kOverrideKinds = 4;
int kernel_override(int which);
int gemm_num_tile_configs();
int gemm_num_decode_configs();
int gemm_f6_num_configs();

// ---- activation path (transform_quant.hip) --------------------------------
enum class TqPath { Fused, Cols, Split };

// Activation quantizer of one call.  Dynamic (steps == nullptr): per-token
// scale alpha * max|z| / 7.  Static: steps fixed offline, either one step for
// the whole tensor (the token scale is that step) or one step per channel
// (codes round z_k / step_k; the token scale written is 1).
// qmax: largest code, 2^(b-1) - 1 (7 for 4-bit codes, 3 for 3-bit); codes are
// clamped to [-qmax - 1, qmax] and the dynamic scale is alpha * max|z| / qmax.
struct ActQuant {
    float alpha;
    const float* steps;
    bool per_channel;
    float qmax = 7.0f;
};

TqPath tq_select_path(int M, int n1, int n2, bool has_c);
size_t tq_workspace_bytes(int M, int n1, int n2, bool has_c);

// quantize=true: Xq/s_x outputs; quantize=false: Z (fp32 [M,K]) output.
// S16 (optional, [M, Gp] fp16): the per-token group sums 16 * Σ_{k in g} q
// of the codes over groups of 128, zero for g >= K / 128, which the GEMM's
// zero-point correction takes; written only by the token-batched kernels
// (*sums_written tells), the other paths leave them to the GEMM's pre-pass.
hipError_t tq_launch(const uint16_t* X, int M, int n1, int n2, const float* P1,
                     const float* P2, const float* c, ActQuant aq, bool quantize,
                     uint8_t* Xq, float* s_x, float* Z, void* ws, size_t ws_bytes,
                     hipStream_t stream, uint16_t* S16 = nullptr, int Gp = 0,
                     bool* sums_written = nullptr);

// ---- GEMM (gemm.hip) -------------------------------------------------------
struct GemmArgs {
    const uint8_t* Xq;
    const float* s_x;
    const uint8_t* Wq;
    const uint16_t* s_w;
    const uint16_t* z_w;
    uint16_t* Y;     // fp16 output (mode fp16)
    int32_t* D;      // int32 output (mode i32)
    int M, N, K, group_size;
    bool asym;
    // per-token group sums 16 * Σ_{k in g} q_x[m,k] (fp16, [M, Gp], zero for
    // g >= G): set by gemm_launch for the prefill kernels that apply the
    // zero-point correction in the epilogue
    const uint16_t* S = nullptr;
    int Gp = 0;
    // the caller has already written S ([M, Gp] in the workspace, by the
    // transform kernel): gemm_launch skips its pre-pass
    bool sums_ready = false;
};

size_t gemm_workspace_bytes(int M, int N, int K, int group_size, bool asym);
// whether the prefill GEMM applies the zero-point correction from per-token
// group sums, and their row pitch Gp (the sums sit at the start of the GEMM
// workspace)
bool gemm_takes_group_sums(int M, int K, int group_size, bool asym, int* Gp);
// name of the configuration gemm_launch would use (launches nothing)
const char* gemm_kernel_name(const GemmArgs& a, bool i32_out);
hipError_t gemm_launch(const GemmArgs& a, bool i32_out, void* ws, size_t ws_bytes,
                       hipStream_t stream);

// ---- decode GEMM (gemm_decode.hip): batches of at most kDecodeMaxM tokens ----
constexpr int kDecodeMaxM = 64;
const char* gemm_decode_kernel_name(const GemmArgs& a);
hipError_t gemm_decode_launch(const GemmArgs& a, void* ws, size_t ws_bytes, hipStream_t stream);
// workspace of the split-K decode kernel (partial sums of M tokens x N per
// K range); 0 for shapes it does not take
size_t gemm_decode_workspace_bytes(int M, int N, int K, int group_size, bool asym);

// ---- single-kernel decode layer (linear_decode.hip) --------------------------
// ---- INT4 GEMM on the fp6 matrix pipe (gemm_f6.hip) ------------------------
struct F6Args {
    const uint8_t* X6;      // activation codes / 2, fp6 fragment layout
    const float* s_x;
    const uint8_t* W6;      // weight codes (u - z or q) / 2, fp6 fragment layout
    const uint16_t* s_w;
    uint16_t* Y;
    int M, N, K, group_size;
};
inline int f6_rows(int R) { return (R + 31) / 32 * 32; }
size_t f6_bytes(int R, int K);
hipError_t f6_convert_launch(const uint8_t* src, int R, int K, const uint16_t* z, int group_size,
                             uint8_t* dst, hipStream_t stream);
const char* gemm_f6_kernel_name(const F6Args& a);
hipError_t gemm_f6_launch(const F6Args& a, hipStream_t stream);

size_t linear_decode_workspace_bytes(int M, int n1, int n2);
// 0: supported; 1: shape not covered; 2: too much LDS; 3: the producers
// exceed the device's resident capacity
int linear_decode_check(int M, int n1, int n2, int N, int K, int group_size, bool asym,
                        int* cap);
hipError_t linear_decode_launch(const uint16_t* X, int M, int n1, int n2, const float* P1,
                                const float* P2, ActQuant aq, const GemmArgs& g, void* ws,
                                uint32_t* sync, hipStream_t stream);

// ---- INT4 KV cache (kv_cache.hip) -------------------------------------------
struct KvAppendArgs {
    const uint16_t* k;          // [tokens][heads][128] fp16
    const uint16_t* v;
    const int32_t* seg_seq;     // [segments]
    const int32_t* seg_start;   // [segments]
    const int32_t* cu_tokens;   // [segments + 1]
    const float* P_h;           // [128][128] or [heads][128][128]
    const float* P_v;
    float alpha_k, alpha_v;
    uint8_t* k_cache;
    float* k_scale;
    uint32_t* v_cache;
    float* v_scale;
    int tokens, segments, heads, batch, max_seq;
    int hpw;                    // heads per workgroup (kv_append_hpw)
};
int kv_append_hpw(int tokens, int segments, int heads);
hipError_t kv_append_launch(const KvAppendArgs& a, bool per_head, hipStream_t stream);
// out[b][h][:] = scale * q[b][h][:] · M[h / G] (fp32), G = heads_q / heads_kv
hipError_t rows_xform_launch(const uint16_t* q, int batch, int heads_q, int heads_kv,
                             const float* M, bool per_head, float scale, float* out,
                             hipStream_t stream);

// ---- decode attention over the INT4 KV cache (attention.hip) ---------------
struct AttnArgs {
    const float* qt;            // [batch][heads_q][128], scaled by sm_scale * log2(e)
    const uint8_t* k_cache;
    const float* k_scale;
    const uint32_t* v_cache;
    const float* v_scale;
    const int32_t* lengths;     // [batch]
    uint16_t* out;              // [batch][heads_q][128] fp16
    float* part;                // partial records
    int batch, heads_q, heads_kv, max_seq, chunk;
};
// positions per partial-attention workgroup for this device
int attn_chunk(int batch, int heads_kv, int max_seq);
size_t attn_partial_bytes(int batch, int heads_q, int heads_kv, int max_seq, int chunk);
hipError_t attn_decode_launch(const AttnArgs& a, hipStream_t stream);

// ---- ternary weights, W1.58A16 (ternary.hip) --------------------------------
struct TernArgs {
    const uint16_t* X;      // fp16 [M][K]
    const uint8_t* Tq;      // codes, 16-row tiles (see ternary.hip)
    const uint32_t* am;     // [N/16][K/128][16]: alpha fp16 bits low, mu high
    uint16_t* Y;            // fp16 [M][N] (no K-split)
    float* part;            // [splits][M][N] (K-split) or nullptr
    int M, N, K, gps;       // gps: groups of blocks of K per split
    int xls;                // LDS row stride of X (halfs) when X is held in LDS
};
struct TernPlan {
    int ms;       // 16-row subtiles per wave (1 or 2)
    int ns;       // 16-column subtiles per wave
    int qb;       // blocks of 128 per load stage (a group)
    bool xl;      // X (or its K slice) held in LDS
    bool nsp;     // waves split the columns instead of K
    int waves;    // waves per workgroup
    int xls;      // LDS row stride of X (halfs)
    size_t lds;   // dynamic LDS bytes
    int gps;      // groups per K-split
    int splits;   // K-splits
};
TernPlan tern_plan(int M, int N, int K, int cus);
inline int tern_rows(int N) { return (N + 15) / 16 * 16; }   // rows in storage
size_t tern_workspace_bytes(int M, int N, int K);   // for this device
hipError_t tern_pack_launch(const float* Wt, int N, int K, int iters, uint8_t* Tq, uint32_t* am,
                            hipStream_t stream);
hipError_t tern_unpack_launch(const uint8_t* Tq, const uint32_t* am, int N, int K, int8_t* T,
                              uint16_t* alpha, uint16_t* mu, hipStream_t stream);
hipError_t tern_gemm_launch(const uint16_t* X, int M, int N, int K, const uint8_t* Tq,
                            const uint32_t* am, uint16_t* Y, void* ws, hipStream_t stream);

// ---- offline weight preparation (weights.hip) ------------------------------
size_t merge_workspace_bytes(int n1, int n2, int K);
// returns hipSuccess and sets *singular when a factor has no usable pivot
hipError_t merge_launch(const float* W, int N, int K, int n1, int n2, const float* P1,
                        const float* P2, const float* c, float* Wt, void* ws,
                        hipStream_t stream, bool* singular);
// Wm[n, k] = Wt[n, k] * steps[k] (fp32, one rounding); Wm may equal Wt
hipError_t migrate_steps_launch(const float* Wt, int N, int K, const float* steps, float* Wm,
                                hipStream_t stream);
// out[i] = P[i]^-T (fp32, computed in fp64) for count n x n matrices; sets
// *singular when one has no usable pivot
size_t invert_t_workspace_bytes(int n, int count);
hipError_t invert_t_launch(const float* P, int n, int count, float* out, void* ws,
                           hipStream_t stream, bool* singular);
// bits: 4 or 3 (codes [-8, 7] / [0, 15], or [-4, 3] / [0, 7])
hipError_t pack_weights_launch(const float* Wt, int N, int K, int group_size, bool asym,
                               float alpha_w, int bits, uint8_t* Wq, uint16_t* s_w,
                               uint16_t* z_w, hipStream_t stream);

// measurement aid (measure.hip): XOR of all 32-bit words of buf into *out
hipError_t read_probe_launch(const void* buf, size_t bytes, uint32_t* out, hipStream_t stream);

}  // namespace w4a4
