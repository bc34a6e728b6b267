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
// 2s, code 2s + 1 at bits 16 + 2s).  The 32 codes that MFMA lane group q
// (q = 0..3) takes from block g, codes 128 g + 32 s + 8 q + j (step s = 0..3,
// j = 0..7) in the order (s, j), form an 8-byte piece.  Rows are tiled by 16
// (N rounded up; padding rows are zero): tile t holds 16 K / 4 bytes from
// byte 4 K t, and in it the pair of blocks (2p, 2p + 1) the 1024 bytes from
// 1024 p, lane l = 16 q + r holding row r's pieces of both blocks at 16 l; so
// one 16-byte load per lane of a wave reads a whole pair for 16 rows, 1024
// contiguous bytes.  An unpaired last block (odd K/128) holds row r's piece q
// at 1024 p + 8 (16 q + r).  The block parameters are one word per (row,
// block) at (t K/128 + g) 16 + r, alpha's fp16 bits low, mu's high.
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

__global__ __launch_bounds__(kTB) void k_tern_pack(const float* __restrict__ Wt, int N, int K, int iters,
                                                   uint8_t* __restrict__ Tq,
                                                   uint32_t* __restrict__ am) {
    __shared__ double red[2];
    __shared__ uint32_t words[kTB / 16];
    const int row = blockIdx.x;                 // 0 .. rows rounded up to 16
    const int g = blockIdx.y;
    const int G = K / kTB;
    const int t = threadIdx.x;
    const int tile = row >> 4;
    const int r = row & 15;
    uint32_t* const tq32 = reinterpret_cast<uint32_t*>(Tq + static_cast<size_t>(tile) * 4 * K);
    const int pr = g >> 1;
    // word w (0, 1) of lane group q's piece of this row and block
    auto word_at = [&](int q, int wd) -> uint32_t* {
        const int off = 2 * pr + 1 < G ? 1024 * pr + (16 * q + r) * 16 + 8 * (g & 1)
                                       : 1024 * pr + (16 * q + r) * 8;
        return tq32 + (off >> 2) + wd;
    };
    uint32_t* const amw = am + (static_cast<size_t>(tile) * G + g) * 16 + r;
    if (row >= N) {                             // padding rows: zero codes and parameters
        if (t < kTB / 16) *word_at(t >> 1, t & 1) = 0u;
        if (t == 0) *amw = 0u;
        return;
    }
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
    {
        // code t = 32 s + 8 q + j of the block goes to word 2 q + s / 2 of the
        // block, position i = 8 (s % 2) + j of that word's 16
        const int sq = t >> 5, q = (t >> 3) & 3, i = 8 * (sq & 1) + (t & 7);
        atomicOr(&words[2 * q + (sq >> 1)], c << (16 * (i & 1) + 2 * (i >> 1)));
    }
    __syncthreads();
    if (t < kTB / 16) *word_at(t >> 1, t & 1) = words[t];   // words 2q, 2q + 1: lane group q
    if (t == 0) *amw = static_cast<uint32_t>(a16) | (static_cast<uint32_t>(u16) << 16);
}

// The inverse of the storage layout k_tern_pack writes: one workgroup of 128
// threads per (row, block), thread t reading code t of the block from its
// lane group's piece (the same word and bit position the pack wrote it to),
// thread 0 the block's parameter word.  Codes go out as int8 in {-1, 0, 1}
// row-major [N][K], alpha and mu as fp16 bits [N][K/128].
__global__ __launch_bounds__(kTB) void k_tern_unpack(const uint8_t* __restrict__ Tq,
                                                     const uint32_t* __restrict__ am, int N, int K,
                                                     int8_t* __restrict__ T, uint16_t* __restrict__ alpha,
                                                     uint16_t* __restrict__ mu) {
    const int row = blockIdx.x;
    const int g = blockIdx.y;
    const int G = K / kTB;
    const int t = threadIdx.x;
    const int tile = row >> 4;
    const int r = row & 15;
    const uint32_t* const tq32 = reinterpret_cast<const uint32_t*>(Tq + static_cast<size_t>(tile) * 4 * K);
    const int pr = g >> 1;
    const int sq = t >> 5, q = (t >> 3) & 3, i = 8 * (sq & 1) + (t & 7);
    const int off = 2 * pr + 1 < G ? 1024 * pr + (16 * q + r) * 16 + 8 * (g & 1)
                                   : 1024 * pr + (16 * q + r) * 8;
    const uint32_t word = tq32[(off >> 2) + (sq >> 1)];
    const int c = static_cast<int>((word >> (16 * (i & 1) + 2 * (i >> 1))) & 3u);
    T[static_cast<size_t>(row) * K + g * kTB + t] = static_cast<int8_t>(c - 1);
    if (t == 0) {
        const uint32_t w = am[(static_cast<size_t>(tile) * G + g) * 16 + r];
        alpha[static_cast<size_t>(row) * G + g] = static_cast<uint16_t>(w & 0xFFFFu);
        mu[static_cast<size_t>(row) * G + g] = static_cast<uint16_t>(w >> 16);
    }
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
// Product for small M.  A workgroup of W waves owns NS x 16 output columns
// and MS x 16 rows; its waves split K between them in groups of QB blocks
// (wave w takes groups gs + w, gs + w + W, ...) and add their sums
// in LDS at the end; grid.z splits K further across workgroups only when the
// tiles alone cannot fill the GPU.  Lane l: c16 = l % 16 (A row / B column),
// q4 = l / 16.  MFMA step ks of block g uses k = 128 g + 32 ks + 8 q4 + j in
// slot j on both operands, so the 4 lane groups read 64 contiguous bytes of a
// row of X per step; the B operand is the lane's piece of codes.  One more
// MFMA per step against a B of ones gives the block row sum S of X in the
// output layout.  A stage is one group: codes (16 bytes per pair of blocks
// and lane, the pairs of a group in one 128-byte line when QB = 4), block
// parameters and the A operand, all issued together (vector loads complete
// in issue order, so a load issued after a stage would make its use wait for
// the whole stage); NBUF stages rotate, NBUF - 1 of them loading while one is
// used.  The NS subtiles share the A operand and S.
// ---------------------------------------------------------------------------
// LDS row stride of X (halfs) when X is held in LDS: K plus 16 bytes, so that
// rows start 4 banks apart
__host__ __device__ constexpr int tern_xl_stride(int K) { return K + 8; }
constexpr size_t kXlMax = 136 * 1024;        // X in LDS up to this size
constexpr int kLdsMax = 160 * 1024;          // LDS of one CU
size_t tern_xl_bytes(int M, int K) { return static_cast<size_t>(M) * tern_xl_stride(K) * 2; }

template <int MS, int NS, int W, bool NSP>
constexpr int tern_red_floats() { return NSP ? 1 : W * NS * MS * 4 * 64; }

template <int MS, int NS, int QB, bool XL>
struct TernStage {
    uint4 c[QB / 2][NS];    // pair h: .x .y block 2h, .z .w block 2h + 1
    uint32_t p[NS];         // (alpha, mu) word of block q4 (lane group), column c16
    v8h x[QB][MS][4];       // A operands
};
template <int MS, int NS, int QB>
struct TernStage<MS, NS, QB, true> {   // A operands read from LDS
    uint4 c[QB / 2][NS];
    uint32_t p[NS];
};


template <int MS, int NS, int QB, int NBUF, bool XL, int W, bool NSP>
__global__ __launch_bounds__(W * 64) void k_tern_gemm(TernArgs a) {
    static_assert(!NSP || XL, "column-split workgroups hold X in LDS");
    constexpr int kWaves = W;
    __shared__ float red[tern_red_floats<MS, NS, W, NSP>()];
    extern __shared__ __align__(16) _Float16 xl[];      // X [M][slice of K] when XL
    using Stage = TernStage<MS, NS, QB, XL>;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int c16 = lane & 15;
    const int q4 = lane >> 4;
    const int G = a.K / kTB;
    const int NG = G / QB;                                 // full groups
    const int gs = blockIdx.z * a.gps;
    const int ge = min(NG, gs + a.gps);
    const bool last_split = blockIdx.z == gridDim.z - 1;
    const int m0 = blockIdx.y * 16 * MS;
    // the blocks of K this workgroup reads: its groups, and in the last split
    // the blocks past the last full group
    const int kb0 = QB * gs;
    const int kb1 = last_split ? G : QB * ge;

    // 16-row tiles of the weights (clamped: tiles past the last hold no
    // output column); this lane's 16 bytes of a pair at 16 * lane
    const int ntiles = (a.N + 15) / 16;
    const uint8_t* tilep[NS];
    const uint32_t* amt[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int tile = min((NSP ? blockIdx.x * kWaves + w : blockIdx.x) * NS + s, ntiles - 1);
        tilep[s] = a.Tq + static_cast<size_t>(tile) * 4 * a.K;
        amt[s] = a.am + static_cast<size_t>(tile) * G * 16 + c16;
    }
    // rows of this lane's A operand: output row r of an MFMA depends on A row
    // r alone, so rows past M read row M - 1 (in bounds) and their outputs are
    // dropped at the store
    const uint16_t* xrow[MS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
        const int m = min(m0 + 16 * ms + c16, a.M - 1);
        xrow[ms] = a.X + static_cast<size_t>(m) * a.K + 8 * q4;
    }

    v4f facc[NS][MS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) facc[s][ms] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    auto load_x = [&](Stage& st, int j, int g) {
        if constexpr (!XL) {
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    st.x[j][ms][ks] = *reinterpret_cast<const v8h*>(xrow[ms] + g * kTB + 32 * ks);
        }
    };
    // XL (MS = 1, one row tile): this lane's row of X in LDS, blocks kb0 .. kb1
    const _Float16* xlrow = xl + static_cast<size_t>(min(c16, a.M - 1)) * a.xls + 8 * q4;
    auto a_op = [&](const Stage& st, int j, int ms, int ks, int g) -> v8h {
        if constexpr (XL)
            return *reinterpret_cast<const v8h*>(xlrow + (g - kb0) * kTB + 32 * ks);
        else
            return st.x[j][ms][ks];
    };
    // parameters of blocks g0 .. g0 + nb - 1: lane group q4 loads block
    // g0 + q4 (clamped), 64 contiguous words per wave
    auto load_p = [&](Stage& st, int g0, int nb) {
#pragma unroll
        for (int s = 0; s < NS; ++s) st.p[s] = amt[s][static_cast<size_t>(g0 + min(q4, nb - 1)) * 16];
    };
    // blocks g0 .. g0 + 2 * npair - 1 (g0 even) into the stage
    auto load_pairs = [&](Stage& st, int g0, int npair) {
#pragma unroll
        for (int h = 0; h < QB / 2; ++h) {
            if (h >= npair) break;
#pragma unroll
            for (int s = 0; s < NS; ++s)
                st.c[h][s] = *reinterpret_cast<const uint4*>(tilep[s] + 1024 * (g0 / 2 + h) + 16 * lane);
        }
        load_p(st, g0, 2 * npair);
#pragma unroll
        for (int j = 0; j < QB; ++j) {
            if (j >= 2 * npair) break;
            load_x(st, j, g0 + j);
        }
    };
    const v8h ones = __builtin_bit_cast(v8h, v4u{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u});
    auto compute = [&](const Stage& st, int g0, int nblk) {
#pragma unroll
        for (int j = 0; j < QB; ++j) {
            if (j >= nblk) break;
            v8h xa[MS][4];
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) xa[ms][ks] = a_op(st, j, ms, ks, g0 + j);
            // block row sums of X, rows m0 + 16 ms + 4 q4 + i (every column alike)
            v4f sv[MS];
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) {
                sv[ms] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    sv[ms] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[ms][ks], ones, sv[ms], 0, 0, 0);
            }
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const uint4& cp = st.c[j / 2][s];
                v4f acc[MS];
#pragma unroll
                for (int ms = 0; ms < MS; ++ms) acc[ms] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const uint32_t wd = (j & 1) == 0 ? (ks < 2 ? cp.x : cp.y) : (ks < 2 ? cp.z : cp.w);
                    const v8h bk = (ks & 1) ? tern8<1>(wd) : tern8<0>(wd);
#pragma unroll
                    for (int ms = 0; ms < MS; ++ms)
                        acc[ms] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[ms][ks], bk, acc[ms], 0, 0, 0);
                }
                // block epilogue: alpha 2^14 acc + (mu - alpha) S, with this
                // column's parameters from lane group j
                const uint32_t pj = static_cast<uint32_t>(__shfl(static_cast<int>(st.p[s]), c16 + 16 * j));
                const float al = h2f(static_cast<uint16_t>(pj & 0xFFFFu));
                const float mu = h2f(static_cast<uint16_t>(pj >> 16));
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

    // this wave's groups: all of gs .. ge - 1 when the waves split the
    // columns (NSP), else gs + w + kWaves * i; loads past the end repeat the
    // wave's last group (in bounds, never used) so that the rotation issues
    // its loads unconditionally
    const int g1 = NSP ? gs : gs + w;
    const int gstep = NSP ? 1 : kWaves;
    const int ng = g1 < ge ? (ge - g1 + gstep - 1) / gstep : 0;
    auto group_of = [&](int i) { return g1 + gstep * min(i, ng - 1); };
    Stage buf[NBUF];
    if (ng > 0) {
#pragma unroll
        for (int b = 0; b < NBUF - 1; ++b) load_pairs(buf[b], QB * group_of(b), QB / 2);
    }
    if constexpr (XL) {
        // X [M][blocks kb0 .. kb1] into LDS after the first code loads, by
        // direct-to-LDS copies retired by one wait (a loop of load-then-store
        // waited for memory once per 16-byte chunk and thread): 16-byte slot s
        // holds row s / RS, chunk s % RS (RS = xls / 8); chunks past the
        // range and rows past M are padding (copied from a valid address,
        // never read).  Lane l of copy j fills slot 64 j + l.
        const int w8 = (kb1 - kb0) * (kTB / 8);
        const int RS = a.xls / 8;
        const int nslots = a.M * RS;
        const uint16_t* xb = a.X + static_cast<size_t>(kb0) * kTB;
        uint8_t* xlb = reinterpret_cast<uint8_t*>(xl);
        for (int j = w; j * 64 < nslots; j += kWaves) {
            const int s = j * 64 + lane;
            const int m = s / RS;
            const int c = s - m * RS;
            const uint32_t off = (m < a.M && c < w8) ? static_cast<uint32_t>(m) * a.K * 2 + c * 16 : 0u;
            dma16_async_sv(xb, off, xlb + j * 1024);
        }
        wait_vmcnt<0>();
        __syncthreads();
    }
    // whole rotations of NBUF groups with no branch around a step (a branch
    // there let the compiler's waits at the join assume the fewest loads in
    // flight), a scheduling barrier keeping each step's loads ahead of its
    // arithmetic; then the last ng % NBUF groups, whose loads are in flight
    if (ng > 0) {
        int i0 = 0;
        for (; i0 + NBUF <= ng; i0 += NBUF) {
#pragma unroll
            for (int b = 0; b < NBUF; ++b) {
                load_pairs(buf[(b + NBUF - 1) % NBUF], QB * group_of(i0 + b + NBUF - 1), QB / 2);
                __builtin_amdgcn_sched_barrier(0);
                compute(buf[b], QB * group_of(i0 + b), QB);
            }
        }
#pragma unroll
        for (int b = 0; b < NBUF - 1; ++b)
            if (i0 + b < ng) compute(buf[b], QB * group_of(i0 + b), QB);
    }
    // the blocks past the last full group (G % QB of them), in the last
    // split, by every wave (NSP: each for its own columns) or the last wave:
    // whole pairs, then an unpaired last block
    const int rem = G - QB * NG;
    if (rem > 0 && last_split && (NSP || w == kWaves - 1)) {
        Stage st;
        const int g0 = QB * NG;
        const int npair = rem / 2;
        if (npair > 0) {
            load_pairs(st, g0, npair);
            compute(st, g0, 2 * npair);
        }
        if (rem & 1) {
            const int g = G - 1;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const uint2 u = *reinterpret_cast<const uint2*>(tilep[s] + 1024 * (g / 2) + 8 * lane);
                st.c[0][s] = make_uint4(u.x, u.y, 0, 0);
            }
            load_p(st, g, 1);
            load_x(st, 0, g);
            compute(st, g, 1);
        }
    }

    if constexpr (NSP) {
        // each wave owns its columns: write its sums
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int n = ((blockIdx.x * kWaves + w) * NS + s) * 16 + c16;
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = m0 + 16 * ms + 4 * q4 + i;
                    if (n >= a.N || m >= a.M) continue;
                    if (a.part)
                        a.part[(static_cast<size_t>(blockIdx.z) * a.M + m) * a.N + n] = facc[s][ms][i];
                    else
                        a.Y[static_cast<size_t>(m) * a.N + n] = f2h(facc[s][ms][i]);
                }
        }
        return;
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

// Y = fp16 of the sum over splits of part[z] (fp32 [splits][count]); each
// thread four consecutive outputs, the splits' loads issued four at a time
__global__ __launch_bounds__(kThreads) void k_tern_reduce(const float* __restrict__ part, int splits,
                                                          size_t count, uint16_t* __restrict__ Y) {
    const size_t e0 = (static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x) * 4;
    if (e0 >= count) return;
    if (e0 + 4 <= count && (count & 3) == 0) {
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        int z = 0;
        for (; z + 4 <= splits; z += 4) {
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                v[u] = *reinterpret_cast<const float4*>(part + static_cast<size_t>(z + u) * count + e0);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                acc.x += v[u].x;
                acc.y += v[u].y;
                acc.z += v[u].z;
                acc.w += v[u].w;
            }
        }
        for (; z < splits; ++z) {
            const float4 v = *reinterpret_cast<const float4*>(part + static_cast<size_t>(z) * count + e0);
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        const uint32_t lo = static_cast<uint32_t>(f2h(acc.x)) | (static_cast<uint32_t>(f2h(acc.y)) << 16);
        const uint32_t hi = static_cast<uint32_t>(f2h(acc.z)) | (static_cast<uint32_t>(f2h(acc.w)) << 16);
        *reinterpret_cast<uint2*>(Y + e0) = make_uint2(lo, hi);
        return;
    }
    for (size_t e = e0; e < e0 + 4 && e < count; ++e) {
        float acc = 0.0f;
        for (int z = 0; z < splits; ++z) acc += part[static_cast<size_t>(z) * count + e];
        Y[e] = f2h(acc);
    }
}

}  // namespace

hipError_t tern_pack_launch(const float* Wt, int N, int K, int iters, uint8_t* Tq, uint32_t* am,
                            hipStream_t stream) {
    if (N == 0) return hipSuccess;
    k_tern_pack<<<dim3(tern_rows(N), K / kTB), kTB, 0, stream>>>(Wt, N, K, iters, Tq, am);
    return hipGetLastError();
}

hipError_t tern_unpack_launch(const uint8_t* Tq, const uint32_t* am, int N, int K, int8_t* T,
                              uint16_t* alpha, uint16_t* mu, hipStream_t stream) {
    k_tern_unpack<<<dim3(N, K / kTB), kTB, 0, stream>>>(Tq, am, N, K, T, alpha, mu);
    return hipGetLastError();
}

// kernel variants: MS, NS, QB, NBUF, XL, W, NSP
struct TernVariant { int ms, ns, qb, nbuf; bool xl; int waves; bool nsp; };
// one token: waves split K, X (K halfs) in LDS
constexpr TernVariant kTernM1{1, 1, 4, 4, true, 8, false};
// 2..16 tokens: waves split the columns (8 x 32 per workgroup, so that few
// workgroups read X), workgroups split K, X's slice in LDS
constexpr TernVariant kTernM16{1, 2, 4, 4, true, 8, true};
// 17..64 tokens: tiles of 32 rows, waves split K, X from global memory
constexpr TernVariant kTernM64{2, 2, 2, 2, false, 8, false};

TernPlan tern_plan(int M, int N, int K, int cus) {
    TernPlan p{};
    const TernVariant v = M > 16 ? kTernM64 : (M > 1 || tern_xl_bytes(M, K) > kXlMax ? kTernM16 : kTernM1);
    p.ms = v.ms;
    p.ns = v.ns;
    p.qb = v.qb;
    p.xl = v.xl;
    p.nsp = v.nsp;
    p.waves = v.waves;
    const int G = K / kTB;
    const int NG = G / p.qb;
    const int cols = 16 * p.ns * (p.nsp ? p.waves : 1);
    const long tiles = static_cast<long>(ceil_div(N, cols)) * ceil_div(M, 16 * p.ms);
    // at least one workgroup per compute unit; split K across workgroups only
    // when the tiles fall short of that (or, for NSP, when X's slice must be
    // narrower to fit in LDS), keeping at least two groups per wave
    int splits = tiles > 0 ? static_cast<int>((static_cast<long>(cus) + tiles - 1) / tiles) : 1;
    const int cap = max(1, p.nsp ? NG / 2 : NG / (2 * p.waves));
    splits = max(1, min(splits, cap));
    const int rem = G - NG * p.qb;
    auto xls_of = [&](int gps) { return (p.nsp ? min(G, gps * p.qb + rem) : G) * kTB + 8; };
    auto gps_of = [&](int sp) { return NG > 0 ? ceil_div(NG, sp) : 0; };
    // NSP: X's slice (a split's groups plus the tail blocks) must fit in LDS
    while (p.nsp && splits < cap && static_cast<size_t>(M) * xls_of(gps_of(splits)) * 2 > kXlMax)
        ++splits;
    p.gps = gps_of(splits);
    p.splits = NG > 0 ? ceil_div(NG, p.gps) : 1;
    p.xls = xls_of(p.gps);
    // whole 1 KiB copies: the staging's last copy may fill past the rows
    p.lds = p.xl ? (static_cast<size_t>(M) * p.xls * 2 + 1023) / 1024 * 1024 : 0;
    return p;
}

size_t tern_workspace_bytes(int M, int N, int K) {
    const TernPlan p = tern_plan(M, N, K, device_cu_count());
    return p.splits > 1 ? static_cast<size_t>(p.splits) * M * N * sizeof(float) : 0;
}

namespace {
template <int MS, int NS, int QB, int NBUF, bool XL, int W, bool NSP>
hipError_t tern_launch(const TernArgs& a, dim3 grid, size_t lds, hipStream_t stream) {
    auto* kern = &k_tern_gemm<MS, NS, QB, NBUF, XL, W, NSP>;
    if (lds > 64 * 1024) {
        // more than the default dynamic LDS limit: raise it once per device
        static bool raised[64] = {};
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= 64 || !raised[dev]) {
            // the CU's LDS less the kernel's static reduction buffer
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    kLdsMax - static_cast<int>(sizeof(float)) * tern_red_floats<MS, NS, W, NSP>());
            if (e != hipSuccess) return e;
            if (dev >= 0 && dev < 64) raised[dev] = true;
        }
    }
    kern<<<grid, W * 64, lds, stream>>>(a);
    return hipGetLastError();
}
}  // namespace

hipError_t tern_gemm_launch(const uint16_t* X, int M, int N, int K, const uint8_t* Tq,
                            const uint32_t* am, uint16_t* Y, void* ws, hipStream_t stream) {
    if (M == 0) return hipSuccess;
    const TernPlan p = tern_plan(M, N, K, device_cu_count());
    if (p.lds + sizeof(float) * tern_red_floats<1, 2, 8, false>() > static_cast<size_t>(kLdsMax))
        return hipErrorInvalidValue;            // cannot happen for M <= 64, K <= 65536
    float* part = p.splits > 1 ? static_cast<float*>(ws) : nullptr;
    TernArgs a{X, Tq, am, Y, part, M, N, K, p.gps, p.xls};
    const int cols = 16 * p.ns * (p.nsp ? p.waves : 1);
    dim3 grid(ceil_div(N, cols), ceil_div(M, 16 * p.ms), p.splits);
    hipError_t e;
#define W4A4_TERN_LAUNCH(v)                                                                 \
    tern_launch<v.ms, v.ns, v.qb, v.nbuf, v.xl, v.waves, v.nsp>(a, grid, p.lds, stream)
    if (p.nsp)
        e = W4A4_TERN_LAUNCH(kTernM16);
    else if (p.ms == 1)
        e = W4A4_TERN_LAUNCH(kTernM1);
    else
        e = W4A4_TERN_LAUNCH(kTernM64);
#undef W4A4_TERN_LAUNCH
    if (e != hipSuccess) return e;
    if (part) {
        const size_t count = static_cast<size_t>(M) * N;
        k_tern_reduce<<<static_cast<unsigned>((count + 4 * kThreads - 1) / (4 * kThreads)), kThreads, 0,
                        stream>>>(part, p.splits, count, Y);
    }
    return hipGetLastError();
}

}  // namespace w4a4
