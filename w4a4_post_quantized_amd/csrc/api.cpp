// C ABI of libw4a4: argument validation, status codes, workspace sizing and
// dispatch to the kernel launchers.  Validation happens entirely on the host
// before any HIP call, so an invalid call launches nothing and writes no
// output.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "internal.hpp"
#include "w4a4.h"

namespace {

thread_local char g_last_error[512] = {0};

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return W4A4_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(W4A4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, status, ...)                   \
    do {                                             \
        if (!(cond)) return fail(status, __VA_ARGS__); \
    } while (0)

#define REQUIRE_PTR(p) REQUIRE((p) != nullptr, W4A4_ERR_INVALID_ARG, "%s is NULL", #p)
#define REQUIRE_ALIGNED(p) \
    REQUIRE(aligned16(p), W4A4_ERR_ALIGNMENT, "%s is not 16-byte aligned", #p)

int check_factors(int32_t M, int32_t n1, int32_t n2) {
    REQUIRE(M >= 0, W4A4_ERR_INVALID_ARG, "M = %d is negative", M);
    REQUIRE(n1 >= 1 && n2 >= 1, W4A4_ERR_INVALID_ARG, "n1 = %d, n2 = %d must be >= 1", n1, n2);
    REQUIRE(n1 <= W4A4_MAX_FACTOR && n2 <= W4A4_MAX_FACTOR, W4A4_ERR_UNSUPPORTED,
            "n1 = %d, n2 = %d exceed %d", n1, n2, W4A4_MAX_FACTOR);
    const int64_t K = static_cast<int64_t>(n1) * n2;
    REQUIRE(K <= W4A4_MAX_K, W4A4_ERR_UNSUPPORTED, "K = n1*n2 = %lld exceeds %d",
            static_cast<long long>(K), W4A4_MAX_K);
    REQUIRE(K % 16 == 0, W4A4_ERR_UNSUPPORTED, "K = n1*n2 = %lld is not a multiple of 16",
            static_cast<long long>(K));
    return W4A4_OK;
}

int check_desc(const w4a4_weight_desc* d, bool for_gemm) {
    REQUIRE(d != nullptr, W4A4_ERR_INVALID_ARG, "desc is NULL");
    REQUIRE(d->N >= 1, W4A4_ERR_INVALID_ARG, "N = %d must be >= 1", d->N);
    REQUIRE(d->K >= 1, W4A4_ERR_INVALID_ARG, "K = %d must be >= 1", d->K);
    REQUIRE(d->K <= W4A4_MAX_K, W4A4_ERR_UNSUPPORTED, "K = %d exceeds %d", d->K, W4A4_MAX_K);
    REQUIRE(d->K % 2 == 0, W4A4_ERR_UNSUPPORTED, "K = %d is odd", d->K);
    REQUIRE(d->asymmetric == 0 || d->asymmetric == 1, W4A4_ERR_INVALID_ARG,
            "asymmetric = %d must be 0 or 1", d->asymmetric);
    REQUIRE(d->group_size >= 1 && d->K % d->group_size == 0, W4A4_ERR_UNSUPPORTED,
            "group_size = %d does not divide K = %d", d->group_size, d->K);
    if (for_gemm) {
        REQUIRE(d->K % 128 == 0, W4A4_ERR_UNSUPPORTED, "GEMM needs K %% 128 == 0 (K = %d)", d->K);
        REQUIRE(d->group_size == d->K || d->group_size % 128 == 0, W4A4_ERR_UNSUPPORTED,
                "GEMM needs group_size == K or a multiple of 128 (group_size = %d)",
                d->group_size);
    } else {
        REQUIRE(d->group_size % 2 == 0, W4A4_ERR_UNSUPPORTED, "group_size = %d is odd",
                d->group_size);
    }
    return W4A4_OK;
}

}  // namespace

namespace w4a4 {
namespace {
std::atomic<int> g_kernel_override[kOverrideKinds] = {-1, -1, -1, -1};
}  // namespace
int kernel_override(int which) { return g_kernel_override[which].load(std::memory_order_relaxed); }
}  // namespace w4a4

extern "C" {

int w4a4_version(void) { return (0 << 16) | (2 << 8) | 0; }

int w4a4_kernel_config_count(int32_t which) {
    switch (which) {
        case W4A4_OVERRIDE_PREFILL_TILE: ok(); return w4a4::gemm_num_tile_configs();
        case W4A4_OVERRIDE_DECODE: ok(); return w4a4::gemm_num_decode_configs();
        case W4A4_OVERRIDE_F6_TILE: ok(); return w4a4::gemm_f6_num_configs();
        case W4A4_OVERRIDE_TILE_GROUP: ok(); return 1 << 16;
        default: return fail(W4A4_ERR_INVALID_ARG, "unknown override kind %d", which);
    }
}

int w4a4_set_kernel_override(int32_t which, int32_t index) {
    if (which < 0 || which >= w4a4::kOverrideKinds)
        return fail(W4A4_ERR_INVALID_ARG, "unknown override kind %d", which);
    if (index < -1) return fail(W4A4_ERR_INVALID_ARG, "override index %d < -1", index);
    ok();
    return w4a4::g_kernel_override[which].exchange(index, std::memory_order_relaxed);
}

const char* w4a4_status_str(int status) {
    switch (status) {
        case W4A4_OK: return "W4A4_OK";
        case W4A4_ERR_INVALID_ARG: return "W4A4_ERR_INVALID_ARG";
        case W4A4_ERR_UNSUPPORTED: return "W4A4_ERR_UNSUPPORTED";
        case W4A4_ERR_ALIGNMENT: return "W4A4_ERR_ALIGNMENT";
        case W4A4_ERR_WORKSPACE: return "W4A4_ERR_WORKSPACE";
        case W4A4_ERR_HIP: return "W4A4_ERR_HIP";
        default: return "W4A4_ERR_UNKNOWN";
    }
}

const char* w4a4_last_error(void) { return g_last_error; }

// ---------------------------------------------------------------------------
size_t w4a4_merge_workspace_bytes(int32_t n1, int32_t n2, int32_t K) {
    if (n1 < 1 || n2 < 1 || n1 > W4A4_MAX_FACTOR || n2 > W4A4_MAX_FACTOR) return 0;
    if (K != n1 * n2) return 0;
    return w4a4::merge_workspace_bytes(n1, n2, K);
}

int w4a4_merge_weights(const float* W, int32_t N, int32_t K, int32_t n1, int32_t n2,
                       const float* P1, const float* P2, const float* c, float* Wt, void* ws,
                       size_t ws_bytes, void* stream) {
    REQUIRE(N >= 1, W4A4_ERR_INVALID_ARG, "N = %d must be >= 1", N);
    if (int s = check_factors(0, n1, n2)) return s;
    REQUIRE(K == n1 * n2, W4A4_ERR_INVALID_ARG, "K = %d != n1*n2 = %d", K, n1 * n2);
    REQUIRE_PTR(W);
    REQUIRE_PTR(P1);
    REQUIRE_PTR(P2);
    REQUIRE_PTR(Wt);
    REQUIRE_PTR(ws);
    REQUIRE_ALIGNED(W);
    REQUIRE_ALIGNED(P1);
    REQUIRE_ALIGNED(P2);
    REQUIRE_ALIGNED(Wt);
    REQUIRE_ALIGNED(ws);
    if (c) REQUIRE_ALIGNED(c);
    const size_t need = w4a4::merge_workspace_bytes(n1, n2, K);
    REQUIRE(ws_bytes >= need, W4A4_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    bool singular = false;
    hipError_t e = w4a4::merge_launch(W, N, K, n1, n2, P1, P2, c, Wt, ws,
                                      static_cast<hipStream_t>(stream), &singular);
    if (e != hipSuccess) return hip_status(e, "w4a4_merge_weights");
    REQUIRE(!singular, W4A4_ERR_INVALID_ARG, "P1 or P2 is singular");
    return ok();
}

int w4a4_pack_weights_bits(const w4a4_weight_desc* desc, const float* Wt, float alpha_w,
                           int32_t bits, uint8_t* Wq, uint16_t* s_w, uint16_t* z_w,
                           void* stream) {
    if (int s = check_desc(desc, false)) return s;
    REQUIRE(bits == 3 || bits == 4, W4A4_ERR_UNSUPPORTED, "bits = %d: only 3 and 4", bits);
    REQUIRE(alpha_w > 0.0f && alpha_w <= 1.0f, W4A4_ERR_INVALID_ARG,
            "alpha_w = %g must lie in (0, 1]", static_cast<double>(alpha_w));
    REQUIRE_PTR(Wt);
    REQUIRE_PTR(Wq);
    REQUIRE_PTR(s_w);
    if (desc->asymmetric) REQUIRE_PTR(z_w);
    REQUIRE_ALIGNED(Wt);
    REQUIRE_ALIGNED(Wq);
    REQUIRE_ALIGNED(s_w);
    if (desc->asymmetric) REQUIRE_ALIGNED(z_w);
    hipError_t e = w4a4::pack_weights_launch(Wt, desc->N, desc->K, desc->group_size,
                                             desc->asymmetric != 0, alpha_w, bits, Wq, s_w,
                                             z_w, static_cast<hipStream_t>(stream));
    return hip_status(e, "w4a4_pack_weights");
}

int w4a4_pack_weights(const w4a4_weight_desc* desc, const float* Wt, float alpha_w,
                      uint8_t* Wq, uint16_t* s_w, uint16_t* z_w, void* stream) {
    return w4a4_pack_weights_bits(desc, Wt, alpha_w, 4, Wq, s_w, z_w, stream);
}

int w4a4_migrate_steps(const float* Wt, int32_t N, int32_t K, const float* steps, float* Wm,
                       void* stream) {
    REQUIRE(N >= 0, W4A4_ERR_INVALID_ARG, "N = %d is negative", N);
    REQUIRE(K >= 1 && K <= W4A4_MAX_K, W4A4_ERR_INVALID_ARG, "K = %d outside [1, %d]", K,
            W4A4_MAX_K);
    REQUIRE(K % 4 == 0, W4A4_ERR_UNSUPPORTED, "K = %d is not a multiple of 4", K);
    if (N == 0) return ok();
    REQUIRE_PTR(Wt);
    REQUIRE_PTR(steps);
    REQUIRE_PTR(Wm);
    REQUIRE_ALIGNED(Wt);
    REQUIRE_ALIGNED(steps);
    REQUIRE_ALIGNED(Wm);
    hipError_t e = w4a4::migrate_steps_launch(Wt, N, K, steps, Wm,
                                              static_cast<hipStream_t>(stream));
    return hip_status(e, "w4a4_migrate_steps");
}

// ---------------------------------------------------------------------------
size_t w4a4_transform_quant_workspace_bytes(int32_t M, int32_t n1, int32_t n2, int32_t has_c) {
    if (M < 0 || n1 < 1 || n2 < 1 || n1 > W4A4_MAX_FACTOR || n2 > W4A4_MAX_FACTOR) return 0;
    return w4a4::tq_workspace_bytes(M, n1, n2, has_c != 0);
}

static int tq_common(const uint16_t* X, int32_t M, int32_t n1, int32_t n2, const float* P1,
                     const float* P2, const float* c, w4a4::ActQuant aq, bool quantize,
                     uint8_t* Xq, float* s_x, float* Z, void* ws, size_t ws_bytes,
                     void* stream, const char* name) {
    if (int s = check_factors(M, n1, n2)) return s;
    if (aq.steps == nullptr)
        REQUIRE(aq.alpha > 0.0f && aq.alpha <= 1.0f, W4A4_ERR_INVALID_ARG,
                "alpha_a = %g must lie in (0, 1]", static_cast<double>(aq.alpha));
    if (M == 0) return ok();
    if (aq.steps != nullptr) REQUIRE_ALIGNED(aq.steps);
    REQUIRE_PTR(X);
    REQUIRE_PTR(P1);
    REQUIRE_PTR(P2);
    REQUIRE_ALIGNED(X);
    REQUIRE_ALIGNED(P1);
    REQUIRE_ALIGNED(P2);
    if (c) REQUIRE_ALIGNED(c);
    if (quantize) {
        REQUIRE_PTR(Xq);
        REQUIRE_PTR(s_x);
        REQUIRE_ALIGNED(Xq);
        REQUIRE_ALIGNED(s_x);
    } else {
        REQUIRE_PTR(Z);
        REQUIRE_ALIGNED(Z);
    }
    const size_t need = w4a4::tq_workspace_bytes(M, n1, n2, c != nullptr);
    if (need) {
        REQUIRE(ws != nullptr && ws_bytes >= need, W4A4_ERR_WORKSPACE,
                "workspace %zu < %zu bytes", ws ? ws_bytes : 0, need);
        REQUIRE_ALIGNED(ws);
    }
    hipError_t e = w4a4::tq_launch(X, M, n1, n2, P1, P2, c, aq, quantize, Xq, s_x, Z, ws,
                                   ws_bytes, static_cast<hipStream_t>(stream));
    return hip_status(e, name);
}

int w4a4_transform_quant(const uint16_t* X, int32_t M, int32_t n1, int32_t n2,
                         const float* P1, const float* P2, const float* c, float alpha_a,
                         uint8_t* Xq, float* s_x, void* ws, size_t ws_bytes, void* stream) {
    return tq_common(X, M, n1, n2, P1, P2, c, w4a4::ActQuant{alpha_a, nullptr, false}, true, Xq,
                     s_x, nullptr, ws, ws_bytes, stream, "w4a4_transform_quant");
}

static float qmax_of(int32_t bits) { return static_cast<float>((1 << (bits - 1)) - 1); }

int w4a4_transform_quant_bits(const uint16_t* X, int32_t M, int32_t n1, int32_t n2,
                              const float* P1, const float* P2, const float* c, float alpha_a,
                              int32_t bits, uint8_t* Xq, float* s_x, void* ws, size_t ws_bytes,
                              void* stream) {
    REQUIRE(bits == 3 || bits == 4, W4A4_ERR_UNSUPPORTED, "bits = %d: only 3 and 4", bits);
    return tq_common(X, M, n1, n2, P1, P2, c,
                     w4a4::ActQuant{alpha_a, nullptr, false, qmax_of(bits)}, true, Xq, s_x,
                     nullptr, ws, ws_bytes, stream, "w4a4_transform_quant_bits");
}

int w4a4_transform_quant_static(const uint16_t* X, int32_t M, int32_t n1, int32_t n2,
                                const float* P1, const float* P2, const float* c,
                                const float* steps, int32_t per_channel, uint8_t* Xq,
                                float* s_x, void* ws, size_t ws_bytes, void* stream) {
    REQUIRE_PTR(steps);
    REQUIRE(per_channel == 0 || per_channel == 1, W4A4_ERR_INVALID_ARG,
            "per_channel = %d must be 0 or 1", per_channel);
    return tq_common(X, M, n1, n2, P1, P2, c, w4a4::ActQuant{1.0f, steps, per_channel != 0}, true,
                     Xq, s_x, nullptr, ws, ws_bytes, stream, "w4a4_transform_quant_static");
}

int w4a4_transform(const uint16_t* X, int32_t M, int32_t n1, int32_t n2, const float* P1,
                   const float* P2, const float* c, float* Z, void* ws, size_t ws_bytes,
                   void* stream) {
    return tq_common(X, M, n1, n2, P1, P2, c, w4a4::ActQuant{1.0f, nullptr, false}, false,
                     nullptr, nullptr, Z, ws, ws_bytes, stream, "w4a4_transform");
}

// ---------------------------------------------------------------------------
size_t w4a4_gemm_workspace_bytes(int32_t M, const w4a4_weight_desc* desc) {
    if (M < 0 || desc == nullptr || desc->K < 1 || desc->group_size < 1) return 0;
    return w4a4::gemm_workspace_bytes(M, desc->N, desc->K, desc->group_size,
                                      desc->asymmetric != 0);
}

static int gemm_common(const uint8_t* Xq, const float* s_x, int32_t M,
                       const w4a4_weight_desc* desc, const uint8_t* Wq, const uint16_t* s_w,
                       const uint16_t* z_w, uint16_t* Y, int32_t* D, void* ws,
                       size_t ws_bytes, void* stream, const char* name) {
    if (int s = check_desc(desc, true)) return s;
    REQUIRE(M >= 0, W4A4_ERR_INVALID_ARG, "M = %d is negative", M);
    if (M == 0) return ok();
    const bool i32 = (D != nullptr);
    REQUIRE_PTR(Xq);
    REQUIRE_PTR(Wq);
    REQUIRE_ALIGNED(Xq);
    REQUIRE_ALIGNED(Wq);
    if (desc->asymmetric) {
        REQUIRE_PTR(z_w);
        REQUIRE_ALIGNED(z_w);
    }
    if (!i32) {
        REQUIRE_PTR(s_x);
        REQUIRE_PTR(s_w);
        REQUIRE_PTR(Y);
        REQUIRE_ALIGNED(s_x);
        REQUIRE_ALIGNED(s_w);
        REQUIRE_ALIGNED(Y);
        const size_t need =
            w4a4::gemm_workspace_bytes(M, desc->N, desc->K, desc->group_size,
                                       desc->asymmetric != 0);
        if (need) {
            REQUIRE(ws != nullptr && ws_bytes >= need, W4A4_ERR_WORKSPACE,
                    "workspace %zu < %zu bytes", ws ? ws_bytes : 0, need);
            REQUIRE_ALIGNED(ws);
        }
    } else {
        REQUIRE_ALIGNED(D);
    }
    w4a4::GemmArgs a{Xq, s_x, Wq, s_w, z_w, Y, D, M, desc->N, desc->K, desc->group_size,
                     desc->asymmetric != 0};
    hipError_t e = w4a4::gemm_launch(a, i32, ws, ws_bytes, static_cast<hipStream_t>(stream));
    return hip_status(e, name);
}

int w4a4_gemm(const uint8_t* Xq, const float* s_x, int32_t M, const w4a4_weight_desc* desc,
              const uint8_t* Wq, const uint16_t* s_w, const uint16_t* z_w, uint16_t* Y,
              void* ws, size_t ws_bytes, void* stream) {
    REQUIRE_PTR(Y);
    return gemm_common(Xq, s_x, M, desc, Wq, s_w, z_w, Y, nullptr, ws, ws_bytes, stream,
                       "w4a4_gemm");
}

int w4a4_gemm_i32(const uint8_t* Xq, int32_t M, const w4a4_weight_desc* desc,
                  const uint8_t* Wq, const uint16_t* z_w, int32_t* D, void* stream) {
    REQUIRE_PTR(D);
    return gemm_common(Xq, nullptr, M, desc, Wq, nullptr, z_w, nullptr, D, nullptr, 0, stream,
                       "w4a4_gemm_i32");
}

const char* w4a4_gemm_kernel_name(int32_t M, const w4a4_weight_desc* desc) {
    if (check_desc(desc, true) != W4A4_OK) return nullptr;
    if (M < 0) {
        fail(W4A4_ERR_INVALID_ARG, "M = %d is negative", M);
        return nullptr;
    }
    ok();
    w4a4::GemmArgs a{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, M, desc->N,
                     desc->K, desc->group_size, desc->asymmetric != 0};
    return w4a4::gemm_kernel_name(a, false);
}

// ---------------------------------------------------------------------------
static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

size_t w4a4_linear_workspace_bytes(int32_t M, int32_t n1, int32_t n2, int32_t has_c,
                                   const w4a4_weight_desc* desc) {
    if (M < 0 || desc == nullptr || n1 < 1 || n2 < 1 || n1 > W4A4_MAX_FACTOR ||
        n2 > W4A4_MAX_FACTOR || desc->K < 1 || desc->group_size < 1)
        return 0;
    const size_t K = static_cast<size_t>(n1) * n2;
    const size_t tq = w4a4::tq_workspace_bytes(M, n1, n2, has_c != 0);
    const size_t gm = w4a4::gemm_workspace_bytes(M, desc->N, desc->K, desc->group_size,
                                                 desc->asymmetric != 0);
    return align256(K / 2 * M) + align256(sizeof(float) * M) + (tq > gm ? tq : gm);
}

static int linear_common(const uint16_t* X, int32_t M, int32_t n1, int32_t n2, const float* P1,
                         const float* P2, const float* c, w4a4::ActQuant aq,
                         const w4a4_weight_desc* desc, const uint8_t* Wq, const uint16_t* s_w,
                         const uint16_t* z_w, uint16_t* Y, void* ws, size_t ws_bytes,
                         void* stream, const char* name) {
    if (int s = check_desc(desc, true)) return s;
    if (int s = check_factors(M, n1, n2)) return s;
    REQUIRE(desc->K == n1 * n2, W4A4_ERR_INVALID_ARG, "desc->K = %d != n1*n2 = %d", desc->K,
            n1 * n2);
    if (aq.steps == nullptr)
        REQUIRE(aq.alpha > 0.0f && aq.alpha <= 1.0f, W4A4_ERR_INVALID_ARG,
                "alpha_a = %g must lie in (0, 1]", static_cast<double>(aq.alpha));
    if (M == 0) return ok();
    REQUIRE_PTR(X);
    REQUIRE_PTR(P1);
    REQUIRE_PTR(P2);
    REQUIRE_PTR(Wq);
    REQUIRE_PTR(s_w);
    REQUIRE_PTR(Y);
    if (desc->asymmetric) REQUIRE_PTR(z_w);
    REQUIRE_PTR(ws);
    REQUIRE_ALIGNED(X);
    REQUIRE_ALIGNED(P1);
    REQUIRE_ALIGNED(P2);
    if (c) REQUIRE_ALIGNED(c);
    if (aq.steps) REQUIRE_ALIGNED(aq.steps);
    REQUIRE_ALIGNED(Wq);
    REQUIRE_ALIGNED(s_w);
    if (desc->asymmetric) REQUIRE_ALIGNED(z_w);
    REQUIRE_ALIGNED(Y);
    REQUIRE_ALIGNED(ws);
    const size_t need = w4a4_linear_workspace_bytes(M, n1, n2, c != nullptr, desc);
    REQUIRE(ws_bytes >= need, W4A4_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);

    const size_t K = static_cast<size_t>(n1) * n2;
    char* p = static_cast<char*>(ws);
    uint8_t* Xq = reinterpret_cast<uint8_t*>(p);
    p += align256(K / 2 * M);
    float* s_x = reinterpret_cast<float*>(p);
    p += align256(sizeof(float) * M);
    void* sub = p;
    const size_t sub_bytes = ws_bytes - static_cast<size_t>(p - static_cast<char*>(ws));
    hipStream_t st = static_cast<hipStream_t>(stream);

    // asymmetric groups of 128: the transform kernel can also write the
    // per-token group sums the GEMM's zero-point correction takes, at the
    // start of the GEMM's workspace (the token-batched transforms use no
    // workspace of their own), which saves the GEMM's pre-pass launch
    int Gp = 0;
    const bool want_sums = w4a4::gemm_takes_group_sums(M, desc->K, desc->group_size,
                                                       desc->asymmetric != 0, &Gp);
    uint16_t* S16 = want_sums ? static_cast<uint16_t*>(sub) : nullptr;
    bool sums = false;
    hipError_t e = w4a4::tq_launch(X, M, n1, n2, P1, P2, c, aq, true, Xq, s_x, nullptr, sub,
                                   sub_bytes, st, S16, Gp, &sums);
    if (e != hipSuccess) return hip_status(e, name);
    w4a4::GemmArgs a{Xq, s_x, Wq, s_w, z_w, Y, nullptr, M, desc->N, desc->K, desc->group_size,
                     desc->asymmetric != 0};
    if (sums) {
        a.S = S16;
        a.Gp = Gp;
        a.sums_ready = true;
    }
    e = w4a4::gemm_launch(a, false, sub, sub_bytes, st);
    return hip_status(e, name);
}

int w4a4_linear(const uint16_t* X, int32_t M, int32_t n1, int32_t n2, const float* P1,
                const float* P2, const float* c, float alpha_a, const w4a4_weight_desc* desc,
                const uint8_t* Wq, const uint16_t* s_w, const uint16_t* z_w, uint16_t* Y,
                void* ws, size_t ws_bytes, void* stream) {
    return linear_common(X, M, n1, n2, P1, P2, c, w4a4::ActQuant{alpha_a, nullptr, false}, desc,
                         Wq, s_w, z_w, Y, ws, ws_bytes, stream, "w4a4_linear");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Scratch of w4a4_linear_noalloc: a file-scope device array (each device the
// library runs on holds its own copy until the process ends).  Host code
// never passes the array's name to a kernel: its device address is looked up
// once per device with hipGetSymbolAddress, with that device current, and
// that address is what the kernels receive.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kNoAllocScratchBytes = W4A4_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "w4a4_linear_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(W4A4_ERR_UNSUPPORTED, "w4a4_linear_noalloc: device ordinal %d >= %d", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "w4a4_linear_noalloc: hipGetSymbolAddress");
        if (p == nullptr)
            return fail(W4A4_ERR_HIP, "w4a4_linear_noalloc: no device address for the scratch");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return W4A4_OK;
}
}  // namespace

extern "C" {

int w4a4_linear_noalloc(const uint16_t* X, int32_t M, int32_t n1, int32_t n2, const float* P1,
                        const float* P2, const float* c, float alpha_a,
                        const w4a4_weight_desc* desc, const uint8_t* Wq, const uint16_t* s_w,
                        const uint16_t* z_w, uint16_t* Y, void* stream) {
    if (int s = check_desc(desc, true)) return s;
    if (int s = check_factors(M, n1, n2)) return s;
    REQUIRE(desc->K == n1 * n2, W4A4_ERR_INVALID_ARG, "desc->K = %d != n1*n2 = %d", desc->K,
            n1 * n2);
    const size_t need = w4a4_linear_workspace_bytes(M, n1, n2, c != nullptr, desc);
    REQUIRE(need <= kNoAllocScratchBytes, W4A4_ERR_UNSUPPORTED,
            "w4a4_linear_noalloc: M = %d tokens need %zu bytes of scratch, more than its %zu "
            "(W4A4_NOALLOC_SCRATCH_BYTES); use w4a4_linear with a workspace", M, need,
            kNoAllocScratchBytes);
    if (M == 0) return ok();
    void* ws = nullptr;
    if (int s = scratch_of_current_device(&ws)) return s;
    return linear_common(X, M, n1, n2, P1, P2, c, w4a4::ActQuant{alpha_a, nullptr, false}, desc,
                         Wq, s_w, z_w, Y, ws, kNoAllocScratchBytes, stream, "w4a4_linear_noalloc");
}

int w4a4_linear_bits(const uint16_t* X, int32_t M, int32_t n1, int32_t n2, const float* P1,
                     const float* P2, const float* c, float alpha_a, int32_t bits,
                     const w4a4_weight_desc* desc, const uint8_t* Wq, const uint16_t* s_w,
                     const uint16_t* z_w, uint16_t* Y, void* ws, size_t ws_bytes, void* stream) {
    REQUIRE(bits == 3 || bits == 4, W4A4_ERR_UNSUPPORTED, "bits = %d: only 3 and 4", bits);
    return linear_common(X, M, n1, n2, P1, P2, c,
                         w4a4::ActQuant{alpha_a, nullptr, false, qmax_of(bits)}, desc, Wq, s_w,
                         z_w, Y, ws, ws_bytes, stream, "w4a4_linear_bits");
}

int w4a4_linear_static(const uint16_t* X, int32_t M, int32_t n1, int32_t n2, const float* P1,
                       const float* P2, const float* c, const float* steps, int32_t per_channel,
                       const w4a4_weight_desc* desc, const uint8_t* Wq, const uint16_t* s_w,
                       const uint16_t* z_w, uint16_t* Y, void* ws, size_t ws_bytes,
                       void* stream) {
    REQUIRE_PTR(steps);
    REQUIRE(per_channel == 0 || per_channel == 1, W4A4_ERR_INVALID_ARG,
            "per_channel = %d must be 0 or 1", per_channel);
    return linear_common(X, M, n1, n2, P1, P2, c, w4a4::ActQuant{1.0f, steps, per_channel != 0},
                         desc, Wq, s_w, z_w, Y, ws, ws_bytes, stream, "w4a4_linear_static");
}

// ---------------------------------------------------------------------------
// INT4 GEMM on the fp6 matrix pipe (prefill)
// ---------------------------------------------------------------------------
size_t w4a4_weights_f6_bytes(const w4a4_weight_desc* desc) {
    if (check_desc(desc, true) != W4A4_OK) return 0;
    return w4a4::f6_bytes(desc->N, desc->K);
}

int w4a4_pack_weights_f6(const w4a4_weight_desc* desc, const uint8_t* Wq, const uint16_t* z_w,
                         uint8_t* W6, void* stream) {
    if (int s = check_desc(desc, true)) return s;
    REQUIRE_PTR(Wq);
    REQUIRE_PTR(W6);
    REQUIRE_ALIGNED(Wq);
    REQUIRE_ALIGNED(W6);
    if (desc->asymmetric) {
        REQUIRE_PTR(z_w);
        REQUIRE_ALIGNED(z_w);
    }
    hipError_t e = w4a4::f6_convert_launch(Wq, desc->N, desc->K, desc->asymmetric ? z_w : nullptr,
                                           desc->group_size, W6, static_cast<hipStream_t>(stream));
    return hip_status(e, "w4a4_pack_weights_f6");
}

size_t w4a4_gemm_f6_workspace_bytes(int32_t M, const w4a4_weight_desc* desc) {
    if (M < 0 || check_desc(desc, true) != W4A4_OK) return 0;
    ok();
    return align256(w4a4::f6_bytes(M, desc->K));
}

static int gemm_f6_common(const uint8_t* Xq, const float* s_x, int32_t M,
                          const w4a4_weight_desc* desc, const uint8_t* W6, const uint16_t* s_w,
                          uint16_t* Y, void* ws, size_t ws_bytes, hipStream_t st,
                          const char* name) {
    w4a4::F6Args a{static_cast<const uint8_t*>(ws), s_x, W6, s_w, Y, M, desc->N, desc->K,
                   desc->group_size};
    hipError_t e = w4a4::f6_convert_launch(Xq, M, desc->K, nullptr, desc->group_size,
                                           static_cast<uint8_t*>(ws), st);
    if (e == hipSuccess) e = w4a4::gemm_f6_launch(a, st);
    (void)ws_bytes;
    return hip_status(e, name);
}

int w4a4_gemm_f6(const uint8_t* Xq, const float* s_x, int32_t M, const w4a4_weight_desc* desc,
                 const uint8_t* W6, const uint16_t* s_w, uint16_t* Y, void* ws, size_t ws_bytes,
                 void* stream) {
    if (int s = check_desc(desc, true)) return s;
    REQUIRE(M >= 0, W4A4_ERR_INVALID_ARG, "M = %d is negative", M);
    if (M == 0) return ok();
    REQUIRE_PTR(Xq);
    REQUIRE_PTR(s_x);
    REQUIRE_PTR(W6);
    REQUIRE_PTR(s_w);
    REQUIRE_PTR(Y);
    REQUIRE_ALIGNED(Xq);
    REQUIRE_ALIGNED(s_x);
    REQUIRE_ALIGNED(W6);
    REQUIRE_ALIGNED(s_w);
    REQUIRE_ALIGNED(Y);
    const size_t need = w4a4_gemm_f6_workspace_bytes(M, desc);
    REQUIRE(ws != nullptr && ws_bytes >= need, W4A4_ERR_WORKSPACE, "workspace %zu < %zu bytes",
            ws ? ws_bytes : 0, need);
    REQUIRE_ALIGNED(ws);
    return gemm_f6_common(Xq, s_x, M, desc, W6, s_w, Y, ws, ws_bytes,
                          static_cast<hipStream_t>(stream), "w4a4_gemm_f6");
}

const char* w4a4_gemm_f6_kernel_name(int32_t M, const w4a4_weight_desc* desc) {
    if (check_desc(desc, true) != W4A4_OK) return nullptr;
    if (M < 0) {
        fail(W4A4_ERR_INVALID_ARG, "M = %d is negative", M);
        return nullptr;
    }
    ok();
    w4a4::F6Args a{nullptr, nullptr, nullptr, nullptr, nullptr, M, desc->N, desc->K,
                   desc->group_size};
    return w4a4::gemm_f6_kernel_name(a);
}

size_t w4a4_linear_f6_workspace_bytes(int32_t M, int32_t n1, int32_t n2, int32_t has_c,
                                      const w4a4_weight_desc* desc) {
    if (M < 0 || desc == nullptr || n1 < 1 || n2 < 1 || n1 > W4A4_MAX_FACTOR ||
        n2 > W4A4_MAX_FACTOR || desc->K < 1 || desc->group_size < 1)
        return 0;
    const size_t K = static_cast<size_t>(n1) * n2;
    const size_t tq = w4a4::tq_workspace_bytes(M, n1, n2, has_c != 0);
    const size_t x6 = align256(w4a4::f6_bytes(M, static_cast<int>(K)));
    return align256(K / 2 * M) + align256(sizeof(float) * M) + (tq > x6 ? tq : x6);
}

int w4a4_linear_f6(const uint16_t* X, int32_t M, int32_t n1, int32_t n2, const float* P1,
                   const float* P2, const float* c, float alpha_a, const w4a4_weight_desc* desc,
                   const uint8_t* W6, const uint16_t* s_w, uint16_t* Y, void* ws,
                   size_t ws_bytes, void* stream) {
    if (int s = check_desc(desc, true)) return s;
    if (int s = check_factors(M, n1, n2)) return s;
    REQUIRE(desc->K == n1 * n2, W4A4_ERR_INVALID_ARG, "desc->K = %d != n1*n2 = %d", desc->K,
            n1 * n2);
    REQUIRE(alpha_a > 0.0f && alpha_a <= 1.0f, W4A4_ERR_INVALID_ARG,
            "alpha_a = %g must lie in (0, 1]", static_cast<double>(alpha_a));
    if (M == 0) return ok();
    REQUIRE_PTR(X);
    REQUIRE_PTR(P1);
    REQUIRE_PTR(P2);
    REQUIRE_PTR(W6);
    REQUIRE_PTR(s_w);
    REQUIRE_PTR(Y);
    REQUIRE_PTR(ws);
    REQUIRE_ALIGNED(X);
    REQUIRE_ALIGNED(P1);
    REQUIRE_ALIGNED(P2);
    if (c) REQUIRE_ALIGNED(c);
    REQUIRE_ALIGNED(W6);
    REQUIRE_ALIGNED(s_w);
    REQUIRE_ALIGNED(Y);
    REQUIRE_ALIGNED(ws);
    const size_t need = w4a4_linear_f6_workspace_bytes(M, n1, n2, c != nullptr, desc);
    REQUIRE(ws_bytes >= need, W4A4_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);

    const size_t K = static_cast<size_t>(n1) * n2;
    char* p = static_cast<char*>(ws);
    uint8_t* Xq = reinterpret_cast<uint8_t*>(p);
    p += align256(K / 2 * M);
    float* s_x = reinterpret_cast<float*>(p);
    p += align256(sizeof(float) * M);
    void* sub = p;
    const size_t sub_bytes = ws_bytes - static_cast<size_t>(p - static_cast<char*>(ws));
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = w4a4::tq_launch(X, M, n1, n2, P1, P2, c, w4a4::ActQuant{alpha_a, nullptr, false},
                                   true, Xq, s_x, nullptr, sub, sub_bytes, st);
    if (e != hipSuccess) return hip_status(e, "w4a4_linear_f6");
    // the fp6 activations reuse the transform's sub-workspace once it is done
    return gemm_f6_common(Xq, s_x, M, desc, W6, s_w, Y, sub, sub_bytes, st, "w4a4_linear_f6");
}

// ---------------------------------------------------------------------------
size_t w4a4_linear_decode_workspace_bytes(int32_t M, int32_t n1, int32_t n2) {
    if (M < 1 || M > 16 || n1 < 1 || n2 < 1 || n1 > W4A4_MAX_FACTOR || n2 > W4A4_MAX_FACTOR)
        return 0;
    return w4a4::linear_decode_workspace_bytes(M, n1, n2);
}

int w4a4_linear_decode(const uint16_t* X, int32_t M, int32_t n1, int32_t n2, const float* P1,
                       const float* P2, float alpha_a, const float* steps, int32_t per_channel,
                       const w4a4_weight_desc* desc, const uint8_t* Wq, const uint16_t* s_w,
                       const uint16_t* z_w, uint16_t* Y, void* ws, size_t ws_bytes,
                       uint32_t* sync, void* stream) {
    if (int s = check_desc(desc, true)) return s;
    if (int s = check_factors(M, n1, n2)) return s;
    REQUIRE(desc->K == n1 * n2, W4A4_ERR_INVALID_ARG, "desc->K = %d != n1*n2 = %d", desc->K,
            n1 * n2);
    REQUIRE(per_channel == 0 || per_channel == 1, W4A4_ERR_INVALID_ARG,
            "per_channel = %d must be 0 or 1", per_channel);
    if (steps == nullptr)
        REQUIRE(alpha_a > 0.0f && alpha_a <= 1.0f, W4A4_ERR_INVALID_ARG,
                "alpha_a = %g must lie in (0, 1]", static_cast<double>(alpha_a));
    if (M == 0) return ok();
    REQUIRE(M <= 16, W4A4_ERR_UNSUPPORTED, "M = %d: the single-kernel decode takes at most 16 tokens", M);
    REQUIRE_PTR(X);
    REQUIRE_PTR(P1);
    REQUIRE_PTR(P2);
    REQUIRE_PTR(Wq);
    REQUIRE_PTR(s_w);
    REQUIRE_PTR(Y);
    REQUIRE_PTR(ws);
    REQUIRE_PTR(sync);
    if (desc->asymmetric) REQUIRE_PTR(z_w);
    REQUIRE_ALIGNED(X);
    REQUIRE_ALIGNED(P1);
    REQUIRE_ALIGNED(P2);
    if (steps) REQUIRE_ALIGNED(steps);
    REQUIRE_ALIGNED(Wq);
    REQUIRE_ALIGNED(s_w);
    if (desc->asymmetric) REQUIRE_ALIGNED(z_w);
    REQUIRE_ALIGNED(Y);
    REQUIRE_ALIGNED(ws);
    REQUIRE_ALIGNED(sync);
    int cap = 0;
    const int chk = w4a4::linear_decode_check(M, n1, n2, desc->N, desc->K, desc->group_size,
                                              desc->asymmetric != 0, &cap);
    REQUIRE(chk != 1, W4A4_ERR_UNSUPPORTED,
            "factors (%d, %d) have no single-kernel decode (n2 = 128, n1 in {64, 224})", n1, n2);
    REQUIRE(chk != 2, W4A4_ERR_UNSUPPORTED, "M = %d tokens of K = %d do not fit the LDS", M,
            desc->K);
    REQUIRE(chk != 3, W4A4_ERR_UNSUPPORTED,
            "the %d transform workgroups exceed the device's resident capacity (%d)",
            M * (n1 / 16), cap);
    const size_t need = w4a4::linear_decode_workspace_bytes(M, n1, n2);
    REQUIRE(ws_bytes >= need, W4A4_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    w4a4::GemmArgs g{nullptr, nullptr, Wq, s_w, z_w, Y, nullptr, M, desc->N, desc->K,
                     desc->group_size, desc->asymmetric != 0};
    hipError_t e = w4a4::linear_decode_launch(
        X, M, n1, n2, P1, P2, w4a4::ActQuant{alpha_a, steps, per_channel != 0}, g, ws, sync,
        static_cast<hipStream_t>(stream));
    return hip_status(e, "w4a4_linear_decode");
}

// ---------------------------------------------------------------------------
// INT4 KV cache and decode attention
// ---------------------------------------------------------------------------
namespace {

int check_kv_shape(int32_t batch, int32_t heads_kv, int32_t head_dim, int32_t max_seq) {
    REQUIRE(batch >= 0, W4A4_ERR_INVALID_ARG, "batch = %d is negative", batch);
    REQUIRE(heads_kv >= 1, W4A4_ERR_INVALID_ARG, "heads_kv = %d must be >= 1", heads_kv);
    REQUIRE(head_dim == W4A4_KV_HEAD_DIM, W4A4_ERR_UNSUPPORTED,
            "head_dim = %d: only %d is supported", head_dim, W4A4_KV_HEAD_DIM);
    REQUIRE(max_seq >= 32 && max_seq % 32 == 0, W4A4_ERR_UNSUPPORTED,
            "max_seq = %d must be a positive multiple of 32", max_seq);
    REQUIRE(static_cast<int64_t>(batch) * heads_kv * max_seq <= (int64_t{1} << 40),
            W4A4_ERR_UNSUPPORTED, "cache of %d x %d x %d positions is too large", batch,
            heads_kv, max_seq);
    return W4A4_OK;
}

size_t a256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

}  // namespace

int w4a4_kv_cache_bytes(int32_t batch, int32_t heads_kv, int32_t head_dim, int32_t max_seq,
                        size_t* k_bytes, size_t* v_bytes, size_t* scale_bytes) {
    if (int s = check_kv_shape(batch, heads_kv, head_dim, max_seq)) return s;
    const size_t pos = static_cast<size_t>(batch) * heads_kv * max_seq;
    if (k_bytes) *k_bytes = pos * (head_dim / 2);
    if (v_bytes) *v_bytes = pos * (head_dim / 2);
    if (scale_bytes) *scale_bytes = pos * sizeof(float);
    return ok();
}

size_t w4a4_kv_query_factor_workspace_bytes(int32_t head_dim, int32_t count) {
    if (head_dim != W4A4_KV_HEAD_DIM || count < 1 || count > 4096) return 0;
    return w4a4::invert_t_workspace_bytes(head_dim, count);
}

int w4a4_kv_query_factor(const float* P_h, int32_t head_dim, int32_t count, float* P_h_inv_t,
                         void* ws, size_t ws_bytes, void* stream) {
    REQUIRE(head_dim == W4A4_KV_HEAD_DIM, W4A4_ERR_UNSUPPORTED,
            "head_dim = %d: only %d is supported", head_dim, W4A4_KV_HEAD_DIM);
    REQUIRE(count >= 1 && count <= 4096, W4A4_ERR_INVALID_ARG,
            "count = %d must lie in [1, 4096]", count);
    REQUIRE_PTR(P_h);
    REQUIRE_PTR(P_h_inv_t);
    REQUIRE_PTR(ws);
    REQUIRE_ALIGNED(P_h);
    REQUIRE_ALIGNED(P_h_inv_t);
    REQUIRE_ALIGNED(ws);
    const size_t need = w4a4::invert_t_workspace_bytes(head_dim, count);
    REQUIRE(ws_bytes >= need, W4A4_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    bool singular = false;
    hipError_t e = w4a4::invert_t_launch(P_h, head_dim, count, P_h_inv_t, ws,
                                         static_cast<hipStream_t>(stream), &singular);
    if (e != hipSuccess) return hip_status(e, "w4a4_kv_query_factor");
    REQUIRE(!singular, W4A4_ERR_INVALID_ARG, "a P_h matrix is singular");
    return ok();
}

int w4a4_kv_append(const uint16_t* k, const uint16_t* v, int32_t tokens, const int32_t* seg_seq,
                   const int32_t* seg_start, const int32_t* cu_tokens, int32_t segments,
                   int32_t heads_kv, int32_t head_dim, const float* P_h, const float* P_v,
                   int32_t per_head, float alpha_k, float alpha_v, uint8_t* k_cache,
                   float* k_scale, uint32_t* v_cache, float* v_scale, int32_t batch,
                   int32_t max_seq, void* stream) {
    if (int s = check_kv_shape(batch, heads_kv, head_dim, max_seq)) return s;
    REQUIRE(tokens >= 0, W4A4_ERR_INVALID_ARG, "tokens = %d is negative", tokens);
    REQUIRE(segments >= 0, W4A4_ERR_INVALID_ARG, "segments = %d is negative", segments);
    REQUIRE(per_head == 0 || per_head == 1, W4A4_ERR_INVALID_ARG,
            "per_head = %d must be 0 or 1", per_head);
    REQUIRE(alpha_k > 0.0f && alpha_k <= 1.0f && alpha_v > 0.0f && alpha_v <= 1.0f,
            W4A4_ERR_INVALID_ARG, "alpha_k = %g, alpha_v = %g must lie in (0, 1]",
            static_cast<double>(alpha_k), static_cast<double>(alpha_v));
    REQUIRE(static_cast<int64_t>(tokens) * heads_kv * head_dim < (int64_t{1} << 40),
            W4A4_ERR_UNSUPPORTED, "tokens = %d is too large", tokens);
    REQUIRE(segments <= (1 << 24), W4A4_ERR_UNSUPPORTED, "segments = %d is too large",
            segments);
    if (tokens == 0 || segments == 0 || batch == 0) return ok();
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(seg_seq);
    REQUIRE_PTR(seg_start);
    REQUIRE_PTR(cu_tokens);
    REQUIRE_PTR(P_h);
    REQUIRE_PTR(P_v);
    REQUIRE_PTR(k_cache);
    REQUIRE_PTR(k_scale);
    REQUIRE_PTR(v_cache);
    REQUIRE_PTR(v_scale);
    REQUIRE_ALIGNED(k);
    REQUIRE_ALIGNED(v);
    REQUIRE_ALIGNED(P_h);
    REQUIRE_ALIGNED(P_v);
    REQUIRE_ALIGNED(k_cache);
    REQUIRE_ALIGNED(k_scale);
    REQUIRE_ALIGNED(v_cache);
    REQUIRE_ALIGNED(v_scale);
    w4a4::KvAppendArgs a{k, v, seg_seq, seg_start, cu_tokens, P_h, P_v, alpha_k, alpha_v,
                         k_cache, k_scale, v_cache, v_scale, tokens, segments, heads_kv,
                         batch, max_seq, w4a4::kv_append_hpw(tokens, segments, heads_kv)};
    hipError_t e = w4a4::kv_append_launch(a, per_head != 0, static_cast<hipStream_t>(stream));
    return hip_status(e, "w4a4_kv_append");
}

namespace {

int check_attn_shape(int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t head_dim,
                     int32_t max_seq) {
    if (int s = check_kv_shape(batch, heads_kv, head_dim, max_seq)) return s;
    REQUIRE(heads_q >= 1 && heads_q % heads_kv == 0, W4A4_ERR_INVALID_ARG,
            "heads_q = %d is not a positive multiple of heads_kv = %d", heads_q, heads_kv);
    REQUIRE(heads_q / heads_kv <= 16, W4A4_ERR_UNSUPPORTED,
            "%d query heads per KV head exceed 16", heads_q / heads_kv);
    return W4A4_OK;
}

size_t attn_ws_bytes(int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t max_seq,
                     int chunk) {
    return a256(static_cast<size_t>(batch) * heads_q * W4A4_KV_HEAD_DIM * sizeof(float)) +
           a256(w4a4::attn_partial_bytes(batch, heads_q, heads_kv, max_seq, chunk));
}

}  // namespace

size_t w4a4_attn_decode_workspace_bytes(int32_t batch, int32_t heads_q, int32_t heads_kv,
                                        int32_t head_dim, int32_t max_seq) {
    if (check_attn_shape(batch, heads_q, heads_kv, head_dim, max_seq) != W4A4_OK) return 0;
    const int chunk = w4a4::attn_chunk(batch, heads_kv, max_seq);
    return attn_ws_bytes(batch, heads_q, heads_kv, max_seq, chunk);
}

int w4a4_attn_decode(const uint16_t* q, int32_t batch, int32_t heads_q, int32_t heads_kv,
                     int32_t head_dim, const float* P_h_inv_t, int32_t per_head,
                     const uint8_t* k_cache, const float* k_scale, const uint32_t* v_cache,
                     const float* v_scale, const int32_t* lengths, int32_t max_seq,
                     float sm_scale, uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
    if (int s = check_attn_shape(batch, heads_q, heads_kv, head_dim, max_seq)) return s;
    REQUIRE(per_head == 0 || per_head == 1, W4A4_ERR_INVALID_ARG,
            "per_head = %d must be 0 or 1", per_head);
    REQUIRE(sm_scale > 0.0f && sm_scale < 3.0e38f, W4A4_ERR_INVALID_ARG,
            "sm_scale = %g must be finite and > 0", static_cast<double>(sm_scale));
    if (batch == 0) return ok();
    REQUIRE_PTR(q);
    REQUIRE_PTR(P_h_inv_t);
    REQUIRE_PTR(k_cache);
    REQUIRE_PTR(k_scale);
    REQUIRE_PTR(v_cache);
    REQUIRE_PTR(v_scale);
    REQUIRE_PTR(lengths);
    REQUIRE_PTR(out);
    REQUIRE_PTR(ws);
    REQUIRE_ALIGNED(q);
    REQUIRE_ALIGNED(P_h_inv_t);
    REQUIRE_ALIGNED(k_cache);
    REQUIRE_ALIGNED(k_scale);
    REQUIRE_ALIGNED(v_cache);
    REQUIRE_ALIGNED(v_scale);
    REQUIRE_ALIGNED(out);
    REQUIRE_ALIGNED(ws);
    const int chunk = w4a4::attn_chunk(batch, heads_kv, max_seq);
    const size_t need = attn_ws_bytes(batch, heads_q, heads_kv, max_seq, chunk);
    REQUIRE(ws_bytes >= need, W4A4_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    float* qt = static_cast<float*>(ws);
    float* part = reinterpret_cast<float*>(
        static_cast<char*>(ws) +
        a256(static_cast<size_t>(batch) * heads_q * W4A4_KV_HEAD_DIM * sizeof(float)));
    const hipStream_t st = static_cast<hipStream_t>(stream);
    // log2(e): the softmax runs in base 2
    hipError_t e = w4a4::rows_xform_launch(q, batch, heads_q, heads_kv, P_h_inv_t,
                                           per_head != 0, sm_scale * 1.4426950408889634f, qt,
                                           st);
    if (e != hipSuccess) return hip_status(e, "w4a4_attn_decode");
    w4a4::AttnArgs a{qt, k_cache, k_scale, v_cache, v_scale, lengths, out, part,
                     batch, heads_q, heads_kv, max_seq, chunk};
    e = w4a4::attn_decode_launch(a, st);
    return hip_status(e, "w4a4_attn_decode");
}

// ---------------------------------------------------------------------------
// Ternary weights (W1.58A16)
// ---------------------------------------------------------------------------
namespace {
int check_tern(int32_t M, int32_t N, int32_t K) {
    REQUIRE(M >= 0, W4A4_ERR_INVALID_ARG, "M = %d is negative", M);
    REQUIRE(N >= 1, W4A4_ERR_INVALID_ARG, "N = %d must be >= 1", N);
    REQUIRE(K >= W4A4_TERNARY_BLOCK && K % W4A4_TERNARY_BLOCK == 0 && K <= W4A4_MAX_K,
            W4A4_ERR_UNSUPPORTED, "K = %d must be a multiple of %d in [%d, %d]", K,
            W4A4_TERNARY_BLOCK, W4A4_TERNARY_BLOCK, W4A4_MAX_K);
    REQUIRE(M <= W4A4_TERNARY_MAX_M, W4A4_ERR_UNSUPPORTED,
            "M = %d: the ternary product is built for decode batches of at most %d tokens", M,
            W4A4_TERNARY_MAX_M);
    return W4A4_OK;
}
}  // namespace

int w4a4_ternary_weight_bytes(int32_t N, int32_t K, size_t* tq_bytes, size_t* am_bytes) {
    if (int s = check_tern(0, N, K)) return s;
    REQUIRE_PTR(tq_bytes);
    REQUIRE_PTR(am_bytes);
    const size_t rows = static_cast<size_t>(w4a4::tern_rows(N));
    *tq_bytes = rows * static_cast<size_t>(K) / 4;
    *am_bytes = rows * static_cast<size_t>(K / W4A4_TERNARY_BLOCK) * sizeof(uint32_t);
    return ok();
}

int w4a4_pack_ternary(const float* Wt, int32_t N, int32_t K, int32_t iters, uint8_t* Tq,
                      uint32_t* am, void* stream) {
    if (int s = check_tern(0, N, K)) return s;
    REQUIRE(iters >= 0 && iters <= 1000, W4A4_ERR_INVALID_ARG, "iters = %d outside [0, 1000]",
            iters);
    REQUIRE_PTR(Wt);
    REQUIRE_PTR(Tq);
    REQUIRE_PTR(am);
    REQUIRE_ALIGNED(Wt);
    REQUIRE_ALIGNED(Tq);
    REQUIRE_ALIGNED(am);
    hipError_t e = w4a4::tern_pack_launch(Wt, N, K, iters, Tq, am, static_cast<hipStream_t>(stream));
    return hip_status(e, "w4a4_pack_ternary");
}

int w4a4_unpack_ternary(const uint8_t* Tq, const uint32_t* am, int32_t N, int32_t K, int8_t* T,
                        uint16_t* alpha, uint16_t* mu, void* stream) {
    if (int s = check_tern(0, N, K)) return s;
    REQUIRE_PTR(Tq);
    REQUIRE_PTR(am);
    REQUIRE_PTR(T);
    REQUIRE_PTR(alpha);
    REQUIRE_PTR(mu);
    REQUIRE_ALIGNED(Tq);
    REQUIRE_ALIGNED(am);
    REQUIRE_ALIGNED(T);
    REQUIRE_ALIGNED(alpha);
    REQUIRE_ALIGNED(mu);
    hipError_t e = w4a4::tern_unpack_launch(Tq, am, N, K, T, alpha, mu, static_cast<hipStream_t>(stream));
    return hip_status(e, "w4a4_unpack_ternary");
}

size_t w4a4_ternary_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K) {
    if (check_tern(M, N, K) != W4A4_OK) return 0;
    return w4a4::tern_workspace_bytes(M, N, K);
}

int w4a4_ternary_gemm(const uint16_t* X, int32_t M, int32_t N, int32_t K, const uint8_t* Tq,
                      const uint32_t* am, uint16_t* Y, void* ws, size_t ws_bytes, void* stream) {
    if (int s = check_tern(M, N, K)) return s;
    if (M == 0) return ok();
    REQUIRE_PTR(X);
    REQUIRE_PTR(Tq);
    REQUIRE_PTR(am);
    REQUIRE_PTR(Y);
    REQUIRE_ALIGNED(X);
    REQUIRE_ALIGNED(Tq);
    REQUIRE_ALIGNED(am);
    REQUIRE_ALIGNED(Y);
    const size_t need = w4a4::tern_workspace_bytes(M, N, K);
    if (need > 0) {
        REQUIRE(ws != nullptr && ws_bytes >= need, W4A4_ERR_WORKSPACE,
                "workspace %zu < %zu bytes", ws == nullptr ? size_t{0} : ws_bytes, need);
        REQUIRE_ALIGNED(ws);
    }
    hipError_t e = w4a4::tern_gemm_launch(X, M, N, K, Tq, am, Y, ws, static_cast<hipStream_t>(stream));
    return hip_status(e, "w4a4_ternary_gemm");
}

// ---------------------------------------------------------------------------
int w4a4_read_probe(const void* buf, size_t bytes, uint32_t* out, void* stream) {
    if (bytes == 0) return ok();
    REQUIRE_PTR(buf);
    REQUIRE_PTR(out);
    REQUIRE(bytes % 16 == 0, W4A4_ERR_INVALID_ARG, "bytes = %zu is not a multiple of 16", bytes);
    REQUIRE_ALIGNED(buf);
    REQUIRE_ALIGNED(out);
    hipError_t e = w4a4::read_probe_launch(buf, bytes, out, static_cast<hipStream_t>(stream));
    return hip_status(e, "w4a4_read_probe");
}

}  // extern "C"
