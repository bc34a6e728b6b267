// Online activation path: Kronecker transform, per-token scale, INT4
// quantization and nibble packing.
//
// FlatQuant: Flatness Matters for LLM Quantization — section Kronecker 分解
// (activation factor P1^T ×1 X̃ ×2 P2, equal to x·(P1 ⊗ P2) for a row-major
// reshape), section 额外可学习组件 (diag(c) before the transform, clip α_a),
// section 高效 Kernel 设计 (transform and quantize one token tile on chip).
// FRM-PTQ page, section 初步介绍 (uniform quantizer, here symmetric 4-bit).
//
// Split path (any n1, n2): three stream-ordered kernels with fp32 FMA and a
// workspace holding T = X̄·P2 and Z = P1^T·T:
//   stage1  one block per (token m, row r of X̄): T[m, r, :]
//   stage2  one thread per element of Z, block absmax -> atomicMax per token
//   quant   8 codes per thread -> one packed 32-bit store
#include "common.hpp"
#include "internal.hpp"

namespace w4a4 {

namespace {

constexpr int kSplitThreads = 256;

__global__ __launch_bounds__(256) void k_tq_stage1(const uint16_t* __restrict__ X, int K,
                                                   int n2, const float* __restrict__ P2,
                                                   const float* __restrict__ c,
                                                   float* __restrict__ T,
                                                   uint32_t* __restrict__ amax) {
    __shared__ float xs[W4A4_MAX_FACTOR];
    const int m = blockIdx.x;
    const int r = blockIdx.y;
    const size_t base = static_cast<size_t>(m) * K + static_cast<size_t>(r) * n2;
    for (int j = threadIdx.x; j < n2; j += blockDim.x) {
        float v = h2f(X[base + j]);
        if (c) v *= c[static_cast<size_t>(r) * n2 + j];
        xs[j] = v;
    }
    if (r == 0 && threadIdx.x == 0) amax[m] = 0u;
    __syncthreads();
    for (int j = threadIdx.x; j < n2; j += blockDim.x) {
        float acc = 0.0f;
        for (int q = 0; q < n2; ++q) acc = fmaf(xs[q], P2[static_cast<size_t>(q) * n2 + j], acc);
        T[base + j] = acc;
    }
}

__global__ __launch_bounds__(256) void k_tq_stage2(const float* __restrict__ T, int K, int n1,
                                                   int n2, const float* __restrict__ P1,
                                                   float* __restrict__ Z,
                                                   uint32_t* __restrict__ amax) {
    __shared__ float red[kSplitThreads / 64];
    const int m = blockIdx.x;
    const int e = blockIdx.y * blockDim.x + threadIdx.x;
    float v = 0.0f;
    if (e < K) {
        const int i = e / n2;
        const int j = e - i * n2;
        const float* Tm = T + static_cast<size_t>(m) * K;
        float acc = 0.0f;
        for (int r = 0; r < n1; ++r)
            acc = fmaf(P1[static_cast<size_t>(r) * n1 + i], Tm[static_cast<size_t>(r) * n2 + j], acc);
        Z[static_cast<size_t>(m) * K + e] = acc;
        v = fabsf(acc);
    }
    v = wave_max(v);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = red[0];
        for (int w = 1; w < static_cast<int>(blockDim.x >> 6); ++w) b = fmaxf(b, red[w]);
        // non-negative floats order like their bit patterns
        atomicMax(&amax[m], __float_as_uint(b));
    }
}

__global__ __launch_bounds__(256) void k_tq_quant(const float* __restrict__ Z, int K, float alpha,
                                                  const uint32_t* __restrict__ amax,
                                                  uint8_t* __restrict__ Xq,
                                                  float* __restrict__ s_x) {
    const int m = blockIdx.x;
    const int idx = blockIdx.y * blockDim.x + threadIdx.x;
    const float a = __uint_as_float(amax[m]);
    const float s = alpha * a / 7.0f;
    if (idx == 0) s_x[m] = s;
    const int e0 = idx * 8;
    if (e0 >= K) return;
    const bool zero = !(s > 0.0f);
    const float* z = Z + static_cast<size_t>(m) * K + e0;
    uint32_t word = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) word |= quant_nibble(z[t], s, zero) << (4 * t);
    reinterpret_cast<uint32_t*>(Xq + static_cast<size_t>(m) * (K / 2))[idx] = word;
}

}  // namespace

TqPath tq_select_path(int M, int n1, int n2) {
    (void)M;
    (void)n1;
    (void)n2;
    return TqPath::Split;
}

static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

size_t tq_workspace_bytes(int M, int n1, int n2) {
    const size_t K = static_cast<size_t>(n1) * n2;
    if (tq_select_path(M, n1, n2) == TqPath::Split)
        return 2 * align256(sizeof(float) * K * M) + align256(sizeof(uint32_t) * M);
    return 0;
}

hipError_t tq_launch(const uint16_t* X, int M, int n1, int n2, const float* P1,
                     const float* P2, const float* c, float alpha, bool quantize,
                     uint8_t* Xq, float* s_x, float* Z, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
    (void)ws_bytes;
    if (M == 0) return hipSuccess;
    const int K = n1 * n2;
    char* p = static_cast<char*>(ws);
    float* T = reinterpret_cast<float*>(p);
    p += align256(sizeof(float) * static_cast<size_t>(K) * M);
    float* Zw = reinterpret_cast<float*>(p);
    p += align256(sizeof(float) * static_cast<size_t>(K) * M);
    uint32_t* amax = reinterpret_cast<uint32_t*>(p);
    float* Zout = quantize ? Zw : Z;

    k_tq_stage1<<<dim3(M, n1), dim3(n2 >= 256 ? 256 : ((n2 + 63) / 64) * 64), 0, stream>>>(
        X, K, n2, P2, c, T, amax);
    k_tq_stage2<<<dim3(M, ceil_div(K, kSplitThreads)), dim3(kSplitThreads), 0, stream>>>(
        T, K, n1, n2, P1, Zout, amax);
    if (quantize) {
        k_tq_quant<<<dim3(M, ceil_div(K / 8, 256)), dim3(256), 0, stream>>>(Zw, K, alpha, amax,
                                                                           Xq, s_x);
    }
    return hipGetLastError();
}

}  // namespace w4a4
