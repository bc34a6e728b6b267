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
// 2s, code 2s + 1 at bits 16 + 2s), a row of K codes in K/4 bytes.  The 32
// codes that one MFMA lane group q (q = 0..3) takes from block g, codes
// 128 g + 32 q .. + 31, form an 8-byte piece; a pair of blocks (2p, 2p + 1)
// stores its 8 pieces at bytes 64 p + 16 q + 8 (g - 2p) of the row, so one
// lane reads both blocks' codes with one 16-byte load and 4 lanes read 64
// contiguous bytes; an unpaired last block stores piece q at 64 p + 8 q.  The
// block parameters are one word per (block, row), block-major [K/128][N],
// alpha's fp16 bits low, mu's high.
//
// Kernels:
//   k_tern_pack    offline ITF in float64, one workgroup per (row, block);
//   k_tern_gemm    the product for decode-sized M on fp16 MFMA: a code c
//                  is moved into the exponent field of an fp16 half, which
//                  makes it the normal number c * 2^-14 (0, 2^-14, 2^-13;
//                  one shift and one mask per two codes), so a block's MFMA
//                  sum is 2^-14 sum x c; with sum x c = sum x t + S, each
//                  block adds alpha 2^14 acc + (mu - alpha) S to the output.
//                  (Codes as fp16 subnormals c * 2^-24 cost the same but
//                  measured up to 76 fp16 ulps off on the MFMA sum.)
//   k_tern_reduce  sums the partials of a K split across workgroups (only
//                  for shapes whose tiles cannot fill the GPU) into fp16.
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
    if (t < kTB / 16) {
        // word t belongs to lane group q = t / 2 (codes 32q .. 32q + 31)
        const int q = t >> 1;
        const int pr = g >> 1;
        const int off = 2 * pr + 1 < G ? 64 * pr + 16 * q + 8 * (g & 1) : 64 * pr + 8 * q;
        reinterpret_cast<uint32_t*>(Tq + static_cast<size_t>(row) * (K / 4) + off)[t & 1] = words[t];
    }
    if (t == 0)
        am[static_cast<size_t>(g) * gridDim.x + row] =
            static_cast<uint32_t>(a16) | (static_cast<uint32_t>(u16) << 16);
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
// Product for small M.  A workgroup of kWaves waves owns NS x 16 output
// columns and MS x 16 rows; its waves split the block pairs of K between them
// (wave w takes pairs ps + w, ps + w + kWaves, ...) and add their sums in LDS
// at the end; grid.z splits K further across workgroups only when the tiles
// alone cannot fill the GPU.  Lane l: c16 = l % 16 (A row / B column), q4 =
// l / 16.  MFMA step ks of block g uses k = 128 g + 32 q4 + 8 ks + j in slot
// j on both operands: the lane's A operand is 16 contiguous bytes of X, its B
// operand codes from the 16 bytes it loaded for the pair.  One more MFMA per
// step against a B of ones gives the block row sum S of X in the output
// layout.  A stage is one pair: codes, block parameters and the A operand,
// all issued together (vector loads complete in issue order, so a load issued
// after a stage would make its use wait for the whole stage); NBUF stages
// rotate, NBUF - 1 of them loading while one is used.  The NS subtiles share
// the A operand and S.
// ---------------------------------------------------------------------------
constexpr int kWaves = 8;

template <int MS, int NS>
constexpr int tern_red_floats() { return kWaves * NS * MS * 4 * 64; }

template <int MS, int NS>
struct TernStage {
    uint4 c[NS];            // .x .y: block 2p, .z .w: block 2p + 1
    uint32_t p[2][NS];      // (alpha, mu) words
    v8h x[2][MS][4];        // A operands
};

template <int MS, int NS, int NBUF>
__global__ __launch_bounds__(kWaves * 64) void k_tern_gemm(TernArgs a) {
    __shared__ float red[tern_red_floats<MS, NS>()];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int c16 = lane & 15;
    const int q4 = lane >> 4;
    const int G = a.K / kTB;
    const int P = G / 2;                                   // full pairs
    const int ps = blockIdx.z * a.pps;
    const int pe = min(P, ps + a.pps);
    const bool last_split = blockIdx.z == gridDim.z - 1;
    const int m0 = blockIdx.y * 16 * MS;

    const uint8_t* rowp[NS];
    int ncol[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int n = blockIdx.x * (16 * NS) + 16 * s + c16;
        ncol[s] = n < a.N ? n : a.N - 1;
        rowp[s] = a.Tq + static_cast<size_t>(ncol[s]) * (a.K / 4);
    }
    // rows of this lane's A operand: output row r of an MFMA depends on A row
    // r alone, so rows past M read row M - 1 (in bounds) and their outputs are
    // dropped at the store
    const uint16_t* xrow[MS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
        const int m = min(m0 + 16 * ms + c16, a.M - 1);
        xrow[ms] = a.X + static_cast<size_t>(m) * a.K + 32 * q4;
    }

    v4f facc[NS][MS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) facc[s][ms] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    using Stage = TernStage<MS, NS>;
    auto load_x = [&](Stage& st, int j, int g) {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                st.x[j][ms][ks] = *reinterpret_cast<const v8h*>(xrow[ms] + g * kTB + 8 * ks);
    };
    auto load_pair = [&](Stage& st, int pr) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            st.c[s] = *reinterpret_cast<const uint4*>(rowp[s] + 64 * pr + 16 * q4);
            st.p[0][s] = a.am[static_cast<size_t>(2 * pr) * a.N + ncol[s]];
            st.p[1][s] = a.am[static_cast<size_t>(2 * pr + 1) * a.N + ncol[s]];
        }
        load_x(st, 0, 2 * pr);
        load_x(st, 1, 2 * pr + 1);
    };
    const v8h ones = __builtin_bit_cast(v8h, v4u{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u});
    auto compute = [&](const Stage& st, int nblk) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (j >= nblk) break;
            // block row sums of X, rows m0 + 16 ms + 4 q4 + i (every column alike)
            v4f sv[MS];
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) {
                sv[ms] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    sv[ms] = __builtin_amdgcn_mfma_f32_16x16x32_f16(st.x[j][ms][ks], ones, sv[ms], 0, 0, 0);
            }
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                v4f acc[MS];
#pragma unroll
                for (int ms = 0; ms < MS; ++ms) acc[ms] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const uint32_t wd = j == 0 ? (ks < 2 ? st.c[s].x : st.c[s].y)
                                               : (ks < 2 ? st.c[s].z : st.c[s].w);
                    const v8h bk = (ks & 1) ? tern8<1>(wd) : tern8<0>(wd);
#pragma unroll
                    for (int ms = 0; ms < MS; ++ms)
                        acc[ms] = __builtin_amdgcn_mfma_f32_16x16x32_f16(st.x[j][ms][ks], bk, acc[ms], 0, 0, 0);
                }
                // block epilogue: alpha 2^14 acc + (mu - alpha) S
                const float al = h2f(static_cast<uint16_t>(st.p[j][s] & 0xFFFFu));
                const float mu = h2f(static_cast<uint16_t>(st.p[j][s] >> 16));
                const float a14 = al * 16384.0f;
                const float bm = mu - al;
#pragma unroll
                for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        facc[s][ms][i] = __builtin_fmaf(a14, acc[ms][i], __builtin_fmaf(bm, sv[ms][i], facc[s][ms][i]));
            }
        }
    };

    // this wave's pairs: ps + w + kWaves * i, i < np; loads past the end
    // repeat the wave's last pair (in bounds, never used) so that the
    // rotation issues its loads unconditionally
    const int p1 = ps + w;
    const int np = p1 < pe ? (pe - p1 + kWaves - 1) / kWaves : 0;
    auto pair_of = [&](int i) { return p1 + kWaves * min(i, np - 1); };
    if (np > 0) {
        Stage buf[NBUF];
#pragma unroll
        for (int b = 0; b < NBUF - 1; ++b) load_pair(buf[b], pair_of(b));
        for (int i0 = 0; i0 < np; i0 += NBUF) {
#pragma unroll
            for (int b = 0; b < NBUF; ++b) {
                if (i0 + b >= np) break;
                load_pair(buf[(b + NBUF - 1) % NBUF], pair_of(i0 + b + NBUF - 1));
                compute(buf[b], 2);
            }
        }
    }
    // an unpaired last block (odd K/128), in the last split, by the last wave
    if ((G & 1) && last_split && w == kWaves - 1) {
        Stage st;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const uint2 u = *reinterpret_cast<const uint2*>(rowp[s] + 64 * P + 8 * q4);
            st.c[s] = make_uint4(u.x, u.y, 0, 0);
            st.p[0][s] = a.am[static_cast<size_t>(2 * P) * a.N + ncol[s]];
        }
        load_x(st, 0, 2 * P);
        compute(st, 1);
    }

    // sum the waves' partial results in LDS: red[w][r][lane], r = (s, ms, i)
    constexpr int R = NS * MS * 4;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[(w * R + (s * MS + ms) * 4 + i) * 64 + lane] = facc[s][ms][i];
    __syncthreads();
    for (int e = threadIdx.x; e < R * 64; e += kWaves * 64) {
        float v = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) v += red[ww * R * 64 + e];
        const int r = e / 64;
        const int l = e % 64;
        const int s = r / (MS * 4);
        const int ms = (r / 4) % MS;
        const int i = r % 4;
        const int n = blockIdx.x * (16 * NS) + 16 * s + (l & 15);
        const int m = m0 + 16 * ms + 4 * (l >> 4) + i;
        if (n >= a.N || m >= a.M) continue;
        if (a.part)
            a.part[(static_cast<size_t>(blockIdx.z) * a.M + m) * a.N + n] = v;
        else
            a.Y[static_cast<size_t>(m) * a.N + n] = f2h(v);
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
    const int P = (K / kTB) / 2;
    p.ms = M <= 16 ? 1 : 2;
    p.ns = 2;
    const long tiles = static_cast<long>(ceil_div(N, 16 * p.ns)) * ceil_div(M, 16 * p.ms);
    // at least one workgroup of kWaves waves per compute unit; split K across
    // workgroups only when the tiles fall short of that, keeping at least
    // two pairs per wave
    int splits = tiles > 0 ? static_cast<int>((static_cast<long>(cus) + tiles - 1) / tiles) : 1;
    const int cap = P / (2 * kWaves);
    if (splits > cap) splits = cap;
    if (splits < 1) splits = 1;
    p.pps = ceil_div(P, splits);
    p.splits = P > 0 ? ceil_div(P, p.pps) : 1;
    return p;
}

size_t tern_workspace_bytes(int M, int N, int K) {
    const TernPlan p = tern_plan(M, N, K, device_cu_count());
    return p.splits > 1 ? static_cast<size_t>(p.splits) * M * N * sizeof(float) : 0;
}

hipError_t tern_gemm_launch(const uint16_t* X, int M, int N, int K, const uint8_t* Tq,
                            const uint32_t* am, uint16_t* Y, void* ws, hipStream_t stream) {
    if (M == 0) return hipSuccess;
    const TernPlan p = tern_plan(M, N, K, device_cu_count());
    float* part = p.splits > 1 ? static_cast<float*>(ws) : nullptr;
    TernArgs a{X, Tq, am, Y, part, M, N, K, p.pps};
    dim3 grid(ceil_div(N, 16 * p.ns), ceil_div(M, 16 * p.ms), p.splits);
    constexpr int threads = kWaves * 64;
    if (p.ms == 1)
        k_tern_gemm<1, 2, 3><<<grid, threads, 0, stream>>>(a);
    else
        k_tern_gemm<2, 2, 2><<<grid, threads, 0, stream>>>(a);
    if (part) {
        const size_t count = static_cast<size_t>(M) * N;
        k_tern_reduce<<<static_cast<unsigned>((count + kThreads - 1) / kThreads), kThreads, 0, stream>>>(
            part, p.splits, count, Y);
    }
    return hipGetLastError();
}

}  // namespace w4a4
