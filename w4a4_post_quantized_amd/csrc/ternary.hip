// Ternary-weight linear layer, W1.58A16: Y = X · Ŵ^T with fp16 activations and
// Ŵ[n, k] = alpha[n, g] T[n, k] + mu[n, g], T in {-1, 0, 1}, g = k / 128.
//
// PT2-LLM: Post-Training Ternarization for Large Language Models, section
// 关键设计 item 2 (ATQ: a per-row offset mu on top of the ternary grid; ITF:
// the closed-form least-squares scale for fixed T alternating with the
// nearest grid point for fixed (alpha, mu), about ten times) and the block
// size 128 of its training strategy.
//
// Storage: T as two-bit codes c = t + 1 in words of 16 codes (code 2s at bits
// 2s, code 2s + 1 at bits 16 + 2s), a row of K codes in K/4 bytes; the block
// parameters as one word per (row, block), alpha's fp16 bits low, mu's high.
//
// Kernels:
//   k_tern_pack    offline ITF in float64, one workgroup per (row, block);
//   k_tern_rowsum  S[g][m] = sum of X[m] over block g (fp32);
//   k_tern_gemm    the product for decode-sized M on fp16 MFMA: a code c
//                  is moved into the exponent field of an fp16 half, which
//                  makes it the normal number c * 2^-14 (0, 2^-14, 2^-13;
//                  one shift and one mask per two codes), so a block's MFMA
//                  sum is 2^-14 sum x c; with sum x c = sum x t + S, each
//                  block adds alpha 2^14 acc + (mu - alpha) S to the output.
//                  (Codes as fp16 subnormals c * 2^-24 cost the same but
//                  measured up to 76 fp16 ulps off on the MFMA sum.)
//   k_tern_reduce  sums the K-split partials into fp16.
#include "common.hpp"
#include "internal.hpp"

namespace w4a4 {

namespace {

constexpr int kTB = 128;          // block (group) size
constexpr int kThreads = 256;

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// offline: ITF for one (row, block), 128 threads, one weight each, float64
// ---------------------------------------------------------------------------
__device__ __forceinline__ double block_sum128(double v, double* red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const double r = red[0] + red[1];
    __syncthreads();
    return r;
}

__device__ __forceinline__ double nearest_t(double z) {
    return fmin(fmax(__builtin_rint(z), -1.0), 1.0);
}

__global__ __launch_bounds__(kTB) void k_tern_pack(const float* __restrict__ Wt, int K, int iters,
                                                   uint8_t* __restrict__ Tq,
                                                   uint32_t* __restrict__ am) {
    __shared__ double red[2];
    __shared__ uint32_t words[kTB / 16];
    const int row = blockIdx.x;
    const int g = blockIdx.y;
    const int G = K / kTB;
    const int t = threadIdx.x;
    const double w = static_cast<double>(Wt[static_cast<size_t>(row) * K + g * kTB + t]);
    const double m = static_cast<double>(kTB);
    const double sW = block_sum128(w, red);
    double mu = sW / m;
    double alpha = block_sum128(fabs(w - mu), red) / m;
    double T = alpha > 0.0 ? nearest_t((w - mu) / alpha) : 0.0;
    for (int it = 0; it < iters; ++it) {
        const double sT = block_sum128(T, red);
        const double sTT = block_sum128(T * T, red);
        const double sWT = block_sum128(w * T, red);
        const double den = m * sTT - sT * sT;
        if (den > 0.0) alpha = (m * sWT - sT * sW) / den;
        mu = (sW - alpha * sT) / m;
        T = alpha > 0.0 ? nearest_t((w - mu) / alpha) : 0.0;
    }
    // stored parameters, then the nearest point of the stored grid
    const uint16_t a16 = f64_to_f16_rne(alpha);
    const uint16_t u16 = f64_to_f16_rne(mu);
    const double a = f16_bits_to_f64(a16);
    const double u = f16_bits_to_f64(u16);
    T = a > 0.0 ? nearest_t((w - u) / a) : 0.0;
    const uint32_t c = static_cast<uint32_t>(static_cast<int>(T) + 1);
    if (t < kTB / 16) words[t] = 0;
    __syncthreads();
    atomicOr(&words[t >> 4], c << (16 * (t & 1) + 2 * ((t & 15) >> 1)));
    __syncthreads();
    if (t < kTB / 16)
        reinterpret_cast<uint32_t*>(Tq + static_cast<size_t>(row) * (K / 4) + g * (kTB / 4))[t] =
            words[t];
    if (t == 0) am[static_cast<size_t>(row) * G + g] = static_cast<uint32_t>(a16) | (static_cast<uint32_t>(u16) << 16);
}

// ---------------------------------------------------------------------------
// S[g][m] = sum_k in block g of X[m][k] (fp32, rows padded to Mpad), one wave
// per (m, g)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_tern_rowsum(const uint16_t* __restrict__ X, int M,
                                                          int K, int Mpad, float* __restrict__ S) {
    const int G = K / kTB;
    const int wid = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (wid >= M * G) return;
    const int m = wid / G;
    const int g = wid % G;
    const int lane = threadIdx.x & 63;
    const uint32_t two = *reinterpret_cast<const uint32_t*>(X + static_cast<size_t>(m) * K + g * kTB + 2 * lane);
    float v = h2f(static_cast<uint16_t>(two & 0xFFFFu)) + h2f(static_cast<uint16_t>(two >> 16));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) S[static_cast<size_t>(g) * Mpad + m] = v;
}

// Eight codes of one MFMA step as fp16 values c * 2^-14, in k order: register v
// holds codes 8h + 2v (low half) and 8h + 2v + 1 (high half), each moved from
// its bit position 8h + 2v (+ 16) to the exponent field, bits 10-11 (+ 16).
template <int H, int V>
__device__ __forceinline__ uint32_t tern_exp2(uint32_t word) {
    constexpr int sh = 10 - 8 * H - 2 * V;
    const uint32_t x = sh >= 0 ? word << (sh >= 0 ? sh : 0) : word >> (sh < 0 ? -sh : 0);
    return x & 0x0C000C00u;
}

template <int H>
__device__ __forceinline__ v8h tern8(uint32_t word) {
    const v4u r = {tern_exp2<H, 0>(word), tern_exp2<H, 1>(word), tern_exp2<H, 2>(word),
                   tern_exp2<H, 3>(word)};
    return __builtin_bit_cast(v8h, r);
}

// ---------------------------------------------------------------------------
// Product for small M.  Workgroup: 4 waves side by side along N, each 16
// output columns and MS x 16 rows; grid.z splits the blocks of K.  Lane l:
// c16 = l % 16 (A row / B column), q4 = l / 16.  MFMA step ks of block g uses
// k = 128 g + 32 q4 + 8 ks + j in slot j on both operands: the lane's A
// operand is 16 contiguous bytes of X, its B operand the codes it loaded.
// ---------------------------------------------------------------------------
template <int MS>
__global__ __launch_bounds__(kThreads) void k_tern_gemm(TernArgs a) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int c16 = lane & 15;
    const int q4 = lane >> 4;
    const int G = a.K / kTB;
    const int n = blockIdx.x * 64 + 16 * w + c16;        // this lane's output column
    const int nc = n < a.N ? n : a.N - 1;
    const int m0 = blockIdx.y * 16 * MS;
    const int gs = blockIdx.z * a.gps;
    const int ge = min(G, gs + a.gps);
    const uint8_t* trow = a.Tq + static_cast<size_t>(nc) * (a.K / 4) + 8 * q4;
    const uint32_t* amr = a.am + static_cast<size_t>(nc) * G;

    v4f facc[MS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) facc[ms] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // rows of this lane's A operand (zero past M, no load)
    const uint16_t* xrow[MS];
    bool xok[MS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
        const int m = m0 + 16 * ms + c16;
        xok[ms] = m < a.M;
        xrow[ms] = a.X + static_cast<size_t>(xok[ms] ? m : 0) * a.K + 32 * q4;
    }

    uint2 cw = gs < ge ? *reinterpret_cast<const uint2*>(trow + static_cast<size_t>(gs) * (kTB / 4))
                       : make_uint2(0, 0);
    for (int g = gs; g < ge; ++g) {
        const uint2 cur = cw;
        if (g + 1 < ge) cw = *reinterpret_cast<const uint2*>(trow + static_cast<size_t>(g + 1) * (kTB / 4));
        const uint32_t p = amr[g];
        v4f acc[MS];
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) acc[ms] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const uint32_t wd = ks < 2 ? cur.x : cur.y;
            const v8h b = (ks & 1) ? tern8<1>(wd) : tern8<0>(wd);
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) {
                v8h xa = v8h{0, 0, 0, 0, 0, 0, 0, 0};
                if (xok[ms]) xa = *reinterpret_cast<const v8h*>(xrow[ms] + g * kTB + 8 * ks);
                acc[ms] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, b, acc[ms], 0, 0, 0);
            }
        }
        // block epilogue: alpha 2^14 acc + (mu - alpha) S, rows m0 + 16 ms + 4 q4 + i
        const float al = h2f(static_cast<uint16_t>(p & 0xFFFFu));
        const float mu = h2f(static_cast<uint16_t>(p >> 16));
        const float a14 = al * 16384.0f;
        const float bm = mu - al;
        const float* Sg = a.S + static_cast<size_t>(g) * a.Mpad + m0 + 4 * q4;
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
            const float4 s = *reinterpret_cast<const float4*>(Sg + 16 * ms);
            facc[ms][0] += a14 * acc[ms][0] + bm * s.x;
            facc[ms][1] += a14 * acc[ms][1] + bm * s.y;
            facc[ms][2] += a14 * acc[ms][2] + bm * s.z;
            facc[ms][3] += a14 * acc[ms][3] + bm * s.w;
        }
    }
    if (n >= a.N) return;
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + 16 * ms + 4 * q4 + i;
            if (m >= a.M) continue;
            if (a.part)
                a.part[(static_cast<size_t>(blockIdx.z) * a.M + m) * a.N + n] = facc[ms][i];
            else
                a.Y[static_cast<size_t>(m) * a.N + n] = f2h(facc[ms][i]);
        }
}

__global__ __launch_bounds__(kThreads) void k_tern_reduce(const float* __restrict__ part, int splits,
                                                          size_t count, uint16_t* __restrict__ Y) {
    const size_t e = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (e >= count) return;
    float s = 0.0f;
    for (int z = 0; z < splits; ++z) s += part[static_cast<size_t>(z) * count + e];
    Y[e] = f2h(s);
}

}  // namespace

hipError_t tern_pack_launch(const float* Wt, int N, int K, int iters, uint8_t* Tq, uint32_t* am,
                            hipStream_t stream) {
    if (N == 0) return hipSuccess;
    k_tern_pack<<<dim3(N, K / kTB), kTB, 0, stream>>>(Wt, K, iters, Tq, am);
    return hipGetLastError();
}

TernPlan tern_plan(int M, int N, int K, int cus) {
    TernPlan p{};
    const int G = K / kTB;
    p.ms = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    p.Mpad = ((M + 63) / 64) * 64;
    const long tiles = static_cast<long>(ceil_div(N, 64)) * ceil_div(M, 16 * p.ms);
    // enough workgroups for about four per compute unit
    int splits = tiles > 0 ? static_cast<int>((4L * cus + tiles - 1) / tiles) : 1;
    if (splits < 1) splits = 1;
    if (splits > G) splits = G;
    p.gps = ceil_div(G, splits);
    p.splits = ceil_div(G, p.gps);
    return p;
}

size_t tern_workspace_bytes(int M, int N, int K) {
    const TernPlan p = tern_plan(M, N, K, device_cu_count());
    const size_t s = static_cast<size_t>(K / kTB) * p.Mpad * sizeof(float);
    const size_t part = p.splits > 1 ? static_cast<size_t>(p.splits) * M * N * sizeof(float) : 0;
    return ((s + 255) & ~static_cast<size_t>(255)) + part;
}

hipError_t tern_gemm_launch(const uint16_t* X, int M, int N, int K, const uint8_t* Tq,
                            const uint32_t* am, uint16_t* Y, void* ws, hipStream_t stream) {
    if (M == 0) return hipSuccess;
    const TernPlan p = tern_plan(M, N, K, device_cu_count());
    const int G = K / kTB;
    float* S = static_cast<float*>(ws);
    const size_t sb = static_cast<size_t>(G) * p.Mpad * sizeof(float);
    float* part = p.splits > 1
                      ? reinterpret_cast<float*>(static_cast<char*>(ws) + ((sb + 255) & ~static_cast<size_t>(255)))
                      : nullptr;
    const int waves = M * G;
    k_tern_rowsum<<<ceil_div(waves, kThreads / 64), kThreads, 0, stream>>>(X, M, K, p.Mpad, S);
    TernArgs a{X, Tq, am, S, Y, part, M, N, K, p.Mpad, p.gps};
    dim3 grid(ceil_div(N, 64), ceil_div(M, 16 * p.ms), p.splits);
    if (p.ms == 1)
        k_tern_gemm<1><<<grid, kThreads, 0, stream>>>(a);
    else if (p.ms == 2)
        k_tern_gemm<2><<<grid, kThreads, 0, stream>>>(a);
    else
        k_tern_gemm<4><<<grid, kThreads, 0, stream>>>(a);
    if (part) {
        const size_t count = static_cast<size_t>(M) * N;
        k_tern_reduce<<<static_cast<unsigned>((count + kThreads - 1) / kThreads), kThreads, 0, stream>>>(
            part, p.splits, count, Y);
    }
    return hipGetLastError();
}

}  // namespace w4a4
