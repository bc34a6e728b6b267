// INT4 x INT4 GEMM on the fp6 matrix pipe (prefill).
//
// FlatQuant: Flatness Matters for LLM Quantization, section 核心思想: the
// layer is the product Q(XP) · Q(P^-1 W^T) of two quantized matrices; FRM-PTQ
// page, section 初步介绍 (codes with zero point z, per-group scales); FPTQuant
// page, section 3. 伪动态残差缩放 (the per-token scale applied afterwards).
//
//   D[m,n,g] = Σ_{k in g} q_x[m,k] · (u[n,k] - z[n,g])     exact
//   Y[m,n]   = fp16( s_x[m] · Σ_g s_w[n,g] · D[m,n,g] )
//
// Every code the layer multiplies is an integer v in [-15, 15], and v / 2 is
// exactly an fp6 E2M3 number (1 sign, 2 exponent, 3 mantissa bits: steps of
// 1/8 below 1, 1/4 below 4, 1/2 below 8).  v_mfma_scale_f32_32x32x64_f8f6f4
// multiplies 32x64 by 64x32 such operands at twice the int8 rate; the products
// (multiples of 1/4) and their sums (below 2^17 in magnitude for K <= 65536)
// are exact in its fp32 accumulator, so D = 4 · acc exactly.
//
// Operand layout in memory (X6 for activations, W6 for weights), identical
// in HBM and LDS so that tiles move with plain 16-byte direct-to-LDS copies:
//   rows padded to Rp (a multiple of 32, padding zero); a fragment is 32 rows
//   x 64 codes, 1536 bytes: lane l (row l % 32, codes 32 (l / 32) .. + 31 of
//   the fragment) owns 6 dwords, code i at bits 6 i; dwords 2p, 2p + 1 of
//   every lane form plane p (512 bytes, lane-major), so a wave reads one
//   operand with three conflict-free 8-byte LDS loads.  Fragment (rt, kt) sits
//   at ((kt / 2) Rp / 32 + rt) · 3072 + (kt % 2) · 1536: the two fragments of
//   a 128-code K tile are adjacent and a K tile of consecutive row fragments
//   is contiguous.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace w4a4 {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kFrag = 1536;         // bytes of one 32 x 64 fragment
constexpr int kTileK = 128;         // codes per K tile (two fragments)
constexpr int kFmtE2M3 = 2;         // MFMA operand format: fp6 E2M3
constexpr int kScaleOne = 127;      // E8M0 block scale 2^0

// e2m3 code of v / 2 for an integer v in [-15, 15]
__device__ __forceinline__ uint32_t e2m3_half(int v) {
    const uint32_t a = static_cast<uint32_t>(v < 0 ? -v : v);
    const uint32_t mag = a < 4 ? 4 * a : (a < 8 ? 2 * a + 8 : a + 16);
    return (v < 0 ? 32u : 0u) | mag;
}

// ---------------------------------------------------------------------------
// Conversion of packed nibbles (low nibble = even k) to the fp6 layout: one
// thread per (row < Rp, 32-code chunk).  Signed codes are sign-extended
// nibbles; asymmetric codes become u - z with the row's zero point of the
// chunk's group.  Rows past R are written as zeros.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_f6_convert(const uint8_t* __restrict__ src, int R, int K,
                                                    int Rp, const uint16_t* __restrict__ z,
                                                    int group_size, uint8_t* __restrict__ dst) {
    const int chunks = K / 32;
    const size_t t = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (t >= static_cast<size_t>(Rp) * chunks) return;
    const int r = static_cast<int>(t / chunks);
    const int c = static_cast<int>(t % chunks);
    uint32_t w[6] = {0, 0, 0, 0, 0, 0};
    if (r < R) {
        const uint4 p = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(r) * (K / 2) + 16 * c);
        const uint32_t pw[4] = {p.x, p.y, p.z, p.w};
        int zp = 0;
        if (z) zp = static_cast<int>(h2f(z[static_cast<size_t>(r) * (K / group_size) + (32 * c) / group_size]));
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int nib = static_cast<int>((pw[i >> 3] >> (4 * (i & 7))) & 0xFu);
            const int v = z ? nib - zp : ((nib ^ 8) - 8);
            const uint32_t code = e2m3_half(v);
            const int bit = 6 * i;
            w[bit >> 5] |= code << (bit & 31);
            if ((bit & 31) > 26) w[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
        }
    }
    const int rt = r >> 5;
    const int kt = c >> 1;
    const int lane = (r & 31) + 32 * (c & 1);
    uint8_t* frag = dst + (static_cast<size_t>(kt >> 1) * (Rp / 32) + rt) * (2 * kFrag) + (kt & 1) * kFrag;
#pragma unroll
    for (int p = 0; p < 3; ++p)
        *reinterpret_cast<uint2*>(frag + 512 * p + 8 * lane) = make_uint2(w[2 * p], w[2 * p + 1]);
}

// ---------------------------------------------------------------------------
// The GEMM.  A workgroup of WAVES_M x WAVES_N waves owns a BM x BN tile and
// walks K in tiles of 128 codes through STAGES LDS stages filled by direct
// copies (the same pipeline as the int8 prefill kernel: the copy of tile
// kt + STAGES - 1 is issued before tile kt is used, one barrier per tile).
// Each wave computes FM x FN 32x32 output fragments; per K tile and 64-code
// half it reads FM + FN operands (three 8-byte LDS loads each) and issues
// FM x FN MFMAs.  Rows and columns past M, N read the last fragment (in
// bounds) and are dropped at the store.
// ---------------------------------------------------------------------------
//
// Per-group weights: the sums of each group are folded into an fp32 sum with
// the group's scale at the group's end (kF6Group).  For groups of one K tile
// (128 codes) kF6G1 needs no persistent group accumulators: each fragment's
// first MFMA of a tile takes a zero register operand, and the tile's sums are
// folded at once (one FMA per element).  Its scales are staged in LDS in
// chunks of 32 groups by the same direct-to-LDS copies as the operands: a
// chunk is issued with the first K tile that uses it, and it has landed once
// that tile's wait has retired all but the newest tile's copies, so kF6G1
// runs with 3 stages.
enum F6Mode { kF6Chan = 0, kF6Group = 1, kF6G1 = 2 };
constexpr int kF6ScaleChunk = 32;   // groups per staged scale chunk (kF6G1)

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int MODE>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64) __attribute__((amdgpu_waves_per_eu(MODE == 2 ? 2 : 1))) void k_gemm_f6(
    const uint8_t* __restrict__ X6, const float* __restrict__ s_x, const uint8_t* __restrict__ W6,
    const uint16_t* __restrict__ s_w, uint16_t* __restrict__ Y, int M, int N, int K,
    int group_size) {
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M;
    constexpr int WN = BN / WAVES_N;
    constexpr int FM = WM / 32;
    constexpr int FN = WN / 32;
    static_assert(FM >= 1 && FN >= 1 && WM % 32 == 0 && WN % 32 == 0, "wave tile");
    constexpr int AF = BM / 32;                        // row fragments of A per K tile
    constexpr int STAGE_BYTES = (BM + BN) / 32 * 2 * kFrag;
    constexpr int CHUNKS = STAGE_BYTES / 16;
    static_assert(CHUNKS % (64 * NW) == 0, "whole wave loads");
    constexpr int LPW = CHUNKS / (64 * NW);
    static_assert(STAGES >= 3 && STAGES <= 4 && (STAGES - 2) * LPW < 64, "stages / vmcnt range");
    constexpr bool G1 = MODE == kF6G1;
    constexpr int CG = kF6ScaleChunk;
    constexpr int SWB = BN * CG * 2;                   // bytes of a staged scale chunk
    constexpr int SWL = SWB / 16 / (64 * NW);          // its copies per wave
    static_assert(!G1 || (STAGES == 3 && (SWB / 16) % (64 * NW) == 0), "kF6G1: 3 stages, whole wave loads");

    __shared__ __align__(16) uint8_t st0[STAGE_BYTES];
    __shared__ __align__(16) uint8_t st1[STAGE_BYTES];
    __shared__ __align__(16) uint8_t st2[STAGE_BYTES];
    __shared__ __align__(16) uint8_t st3[STAGES > 3 ? STAGE_BYTES : 16];
    // kF6G1: scales of the chunk in use, [column of the tile][32 groups] fp16
    __shared__ __align__(16) uint8_t swl[G1 ? SWB : 16];
    auto stage_ptr = [&](auto S) __attribute__((always_inline)) -> uint8_t* {
        constexpr int I = decltype(S)::value;
        if constexpr (I == 0) return st0;
        else if constexpr (I == 1) return st1;
        else if constexpr (I == 2) return st2;
        else return st3;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave / WAVES_N) * WM;
    const int wn0 = (wave % WAVES_N) * WN;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int KT = K / kTileK;
    const int TPG = group_size / kTileK;
    const int G = K / group_size;
    const int MF = (M + 31) / 32;                      // row fragments of X6
    const int NF = (N + 31) / 32;                      // row fragments of W6

    // this lane's copies: load i of a wave covers 64 consecutive 16-byte
    // slots of the stage, all in A or all in B (a fragment pair is 192
    // slots), so its base is wave-uniform (scalar registers) and only the
    // byte offset inside the K tile's slab is per lane
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t soff[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int j = (i * NW + wave_u) * 64 + lane;  // 16-byte slot in the stage
        const int f = j / (2 * kFrag / 16);            // fragment pair within the stage
        const int o = (j % (2 * kFrag / 16)) * 16;
        const int r = ((i * NW + wave_u) * 64) / (2 * kFrag / 16) < AF ? min(m0 / 32 + f, MF - 1)
                                                                       : min(n0 / 32 + f - AF, NF - 1);
        soff[i] = static_cast<uint32_t>(r) * (2 * kFrag) + o;
    }
    auto issue = [&](int kt, auto S) __attribute__((always_inline)) {
        const size_t kc = static_cast<size_t>(min(kt, KT - 1));
        const uint8_t* xb = X6 + kc * MF * (2 * kFrag);
        const uint8_t* wb = W6 + kc * NF * (2 * kFrag);
        uint8_t* stage = stage_ptr(S);
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const bool isA = ((i * NW + wave_u) * 64) / (2 * kFrag / 16) < AF;
            dma16_async_sv(isA ? xb : wb, soff[i], stage + (i * NW + wave) * 1024);
        }
    };

    // kF6G1: copies of scale chunk c (groups 32 c .. 32 c + 31 of the tile's
    // columns; 16 bytes = 8 groups of one column per lane).  Columns past N
    // read the last column and groups past G the last 8 groups (in bounds,
    // never used); the host guarantees G % 8 == 0 and 16-byte aligned s_w.
    auto issue_scales = [&](int c) __attribute__((always_inline)) {
        const int G = K / group_size;
#pragma unroll
        for (int i = 0; i < SWL; ++i) {
            const int j = (i * NW + wave) * 64 + lane;
            const int n = min(n0 + (j >> 2), N - 1);
            int g = c * CG + 8 * (j & 3);
            g = g < G ? g : G - 8;
            dma16_async(s_w + static_cast<size_t>(n) * G + g, swl + (i * NW + wave) * 1024);
        }
    };

    constexpr bool PF = MODE != kF6Chan;               // fp32 per-group sums
    v16f acc[G1 ? 1 : FM][G1 ? 1 : FN];
    float facc[PF ? FM : 1][PF ? FN : 1][16];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if constexpr (!G1) acc[a][b][r] = 0.0f;
                if constexpr (PF) facc[a][b][r] = 0.0f;
            }
    // a zero accumulator operand the compiler cannot fold into an inline
    // constant (an MFMA with an inline-zero accumulator gave wrong sums)
    v16f zc;
    if constexpr (G1) {
        float z0;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z0));
#pragma unroll
        for (int r = 0; r < 16; ++r) zc[r] = z0;
    }

    const int col = lane & 31;
    int bcol[FN];
#pragma unroll
    for (int b = 0; b < FN; ++b) bcol[b] = n0 + wn0 + 32 * b + col;

    auto read_op = [&](const uint8_t* frag) __attribute__((always_inline)) -> v8i {
        const uint2 d0 = *reinterpret_cast<const uint2*>(frag + 8 * lane);
        const uint2 d1 = *reinterpret_cast<const uint2*>(frag + 512 + 8 * lane);
        const uint2 d2 = *reinterpret_cast<const uint2*>(frag + 1024 + 8 * lane);
        return v8i{static_cast<int>(d0.x), static_cast<int>(d0.y), static_cast<int>(d1.x),
                   static_cast<int>(d1.y), static_cast<int>(d2.x), static_cast<int>(d2.y), 0, 0};
    };

    // kF6G1 tile: the two 64-code halves of every fragment from a zero
    // operand, then (after the tile's wait and barrier, when its scale chunk
    // has landed) one FMA per element with the group's scale
    auto body_g1 = [&](int kt, auto S) __attribute__((always_inline)) {
        constexpr int SI = decltype(S)::value;
        if (kt > 0 && kt % CG == 0) {
            // every wave has folded the previous chunk's last tile
            lds_barrier();
            issue_scales(kt / CG);
        }
        issue(kt + STAGES - 1, std::integral_constant<int, (SI + STAGES - 1) % STAGES>{});
        const uint8_t* stage = stage_ptr(S);
        v16f t[FM][FN];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            v8i av[FM], bv[FN];
#pragma unroll
            for (int a = 0; a < FM; ++a) av[a] = read_op(stage + (wm0 / 32 + a) * (2 * kFrag) + kk * kFrag);
#pragma unroll
            for (int b = 0; b < FN; ++b)
                bv[b] = read_op(stage + (AF + wn0 / 32 + b) * (2 * kFrag) + kk * kFrag);
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int b = 0; b < FN; ++b)
                    t[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        av[a], bv[b], kk == 0 ? zc : t[a][b], kFmtE2M3, kFmtE2M3, 0, kScaleOne, 0, kScaleOne);
        }
        wait_vmcnt<(STAGES - 2) * LPW>();
        lds_barrier();
        const int gl = kt % CG;
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            const float sw = h2f(*reinterpret_cast<const uint16_t*>(swl + (wn0 + 32 * b + col) * (2 * CG) + 2 * gl));
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int r = 0; r < 16; ++r) facc[a][b][r] = fmaf(t[a][b][r], sw, facc[a][b][r]);
        }
    };

    auto body = [&](int kt, auto S) __attribute__((always_inline)) {
        if constexpr (G1) {
            body_g1(kt, S);
            return;
        }
        constexpr int SI = decltype(S)::value;
        issue(kt + STAGES - 1, std::integral_constant<int, (SI + STAGES - 1) % STAGES>{});
        const uint8_t* stage = stage_ptr(S);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            v8i av[FM], bv[FN];
#pragma unroll
            for (int a = 0; a < FM; ++a) av[a] = read_op(stage + (wm0 / 32 + a) * (2 * kFrag) + kk * kFrag);
#pragma unroll
            for (int b = 0; b < FN; ++b)
                bv[b] = read_op(stage + (AF + wn0 / 32 + b) * (2 * kFrag) + kk * kFrag);
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int b = 0; b < FN; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        av[a], bv[b], acc[a][b], kFmtE2M3, kFmtE2M3, 0, kScaleOne, 0, kScaleOne);
        }
        if constexpr (MODE == kF6Group) {
            if (((kt + 1) % TPG) == 0) {
                const int g = kt / TPG;
                float zero;
                asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
#pragma unroll
                for (int b = 0; b < FN; ++b) {
                    const float sw = bcol[b] < N ? h2f(s_w[static_cast<size_t>(bcol[b]) * G + g]) : 0.0f;
#pragma unroll
                    for (int a = 0; a < FM; ++a)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            facc[a][b][r] = fmaf(acc[a][b][r], sw, facc[a][b][r]);
                            acc[a][b][r] = zero;
                        }
                }
            }
        }
        wait_vmcnt<(STAGES - 2) * LPW>();
        lds_barrier();
    };

    if constexpr (G1) issue_scales(0);
    static_for<0, STAGES - 1>([&](auto I) { issue(decltype(I)::value, I); });
    wait_vmcnt<(STAGES - 2) * LPW>();
    lds_barrier();

    int kt = 0;
    for (; kt + STAGES <= KT; kt += STAGES)
        static_for<0, STAGES>([&](auto I) { body(kt + decltype(I)::value, I); });
    static_for<0, STAGES - 1>([&](auto I) {
        if (kt + decltype(I)::value < KT) body(kt + decltype(I)::value, I);
    });

    // D = 4 acc; lane l holds rows 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
#pragma unroll
    for (int b = 0; b < FN; ++b) {
        const int gn = bcol[b];
        if (gn >= N) continue;
        const float sw4 = MODE == kF6Chan ? 4.0f * h2f(s_w[gn]) : 4.0f;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gm = m0 + wm0 + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (gm >= M) continue;
                float v;
                if constexpr (PF)
                    v = facc[a][b][r];
                else
                    v = acc[a][b][r];
                Y[static_cast<size_t>(gm) * N + gn] = f2h(v * sw4 * s_x[gm]);
            }
    }
}

template <int BM, int BN, int WM_, int WN_, int ST, int MODE>
hipError_t launch_f6(const F6Args& a, hipStream_t stream) {
    dim3 grid(ceil_div(a.N, BN), ceil_div(a.M, BM));
    dim3 block(WM_ * WN_ * 64);
    k_gemm_f6<BM, BN, WM_, WN_, ST, MODE><<<grid, block, 0, stream>>>(
        a.X6, a.s_x, a.W6, a.s_w, a.Y, a.M, a.N, a.K, a.group_size);
    return hipGetLastError();
}

using F6Fn = hipError_t (*)(const F6Args&, hipStream_t);
struct F6Cfg {
    const char* name;
    F6Fn chan, group;       // group: nullptr where the per-group accumulators do not fit
    F6Fn g1;                // groups of one K tile with staged scales, or nullptr
};

#define W4A4_F6(NAME, BM, BN, WM_, WN_, ST)                                                      \
    F6Cfg{NAME, &launch_f6<BM, BN, WM_, WN_, ST, kF6Chan>, &launch_f6<BM, BN, WM_, WN_, ST, kF6Group>, \
          nullptr}
#define W4A4_F6_G1(NAME, BM, BN, WM_, WN_, ST)                                                   \
    F6Cfg{NAME, &launch_f6<BM, BN, WM_, WN_, ST, kF6Chan>, &launch_f6<BM, BN, WM_, WN_, ST, kF6Group>, \
          &launch_f6<BM, BN, WM_, WN_, ST, kF6G1>}
#define W4A4_F6_CHAN(NAME, BM, BN, WM_, WN_, ST)                                                 \
    F6Cfg{NAME, &launch_f6<BM, BN, WM_, WN_, ST, kF6Chan>, nullptr, nullptr}
const F6Cfg kF6Tiles[] = {
    W4A4_F6_CHAN("k_gemm_f6<256x256, waves 2x4, 3 stages>", 256, 256, 2, 4, 3),
    W4A4_F6_CHAN("k_gemm_f6<128x384, waves 4x4, 3 stages>", 128, 384, 4, 4, 3),
    W4A4_F6("k_gemm_f6<256x128, waves 2x2, 3 stages>", 256, 128, 2, 2, 3),
    W4A4_F6("k_gemm_f6<128x128, waves 2x2, 4 stages>", 128, 128, 2, 2, 4),
    W4A4_F6_CHAN("k_gemm_f6<256x256, waves 4x4, 3 stages>", 256, 256, 4, 4, 3),
    W4A4_F6_G1("k_gemm_f6<128x128, waves 2x2, 3 stages>", 128, 128, 2, 2, 3),
};
#undef W4A4_F6
#undef W4A4_F6_G1
#undef W4A4_F6_CHAN
constexpr int kNumF6 = sizeof(kF6Tiles) / sizeof(kF6Tiles[0]);

// groups of one K tile whose scales can be staged by 16-byte copies
bool f6_g1_ok(const F6Args& a) {
    const int G = a.K / a.group_size;
    return G > 1 && a.group_size == kTileK && G % 8 == 0 &&
           (reinterpret_cast<uintptr_t>(a.s_w) & 15) == 0;
}

const F6Cfg& choose_f6(const F6Args& a) {
    const bool grouped = a.K / a.group_size > 1;
    const bool g1 = f6_g1_ok(a);
    // selection override for tests and sweeps (w4a4_set_kernel_override)
    {
        const int v = kernel_override(2);
        if (v >= 0 && v < kNumF6 &&
            (!grouped || kF6Tiles[v].group != nullptr || (g1 && kF6Tiles[v].g1 != nullptr)))
            return kF6Tiles[v];
    }
    const int cus = device_cu_count();
    const long t256 = static_cast<long>(ceil_div(a.M, 256)) * ceil_div(a.N, 256);
    const long t384 = static_cast<long>(ceil_div(a.M, 128)) * ceil_div(a.N, 384);
    const long t256x128 = static_cast<long>(ceil_div(a.M, 256)) * ceil_div(a.N, 128);
    // measured on MI355X: 256x256 tiles (8 waves) when the grid covers the
    // CUs twice, 128x384 (16 waves) for about one wave of tiles; per-group
    // weights need a second accumulator set, which fits the 4-wave tiles
    // only, and groups of one K tile take the staged-scale mode
    if (g1) return kF6Tiles[5];
    if (grouped) return t256x128 >= cus ? kF6Tiles[2] : kF6Tiles[3];
    if (t256 >= 2L * cus) return kF6Tiles[0];
    if (t384 >= cus) return kF6Tiles[1];
    if (2L * t256 >= cus) return kF6Tiles[4];
    return kF6Tiles[3];
}

}  // namespace

int gemm_f6_num_configs() { return kNumF6; }

size_t f6_bytes(int R, int K) { return static_cast<size_t>(f6_rows(R)) * K * 3 / 4; }

hipError_t f6_convert_launch(const uint8_t* src, int R, int K, const uint16_t* z, int group_size,
                             uint8_t* dst, hipStream_t stream) {
    const size_t threads = static_cast<size_t>(f6_rows(R)) * (K / 32);
    if (threads == 0) return hipSuccess;
    k_f6_convert<<<static_cast<unsigned>((threads + 255) / 256), 256, 0, stream>>>(
        src, R, K, f6_rows(R), z, group_size, dst);
    return hipGetLastError();
}

const char* gemm_f6_kernel_name(const F6Args& a) { return choose_f6(a).name; }

hipError_t gemm_f6_launch(const F6Args& a, hipStream_t stream) {
    if (a.M == 0) return hipSuccess;
    const F6Cfg& c = choose_f6(a);
    if (a.K / a.group_size == 1) return c.chan(a, stream);
    if (c.g1 != nullptr && f6_g1_ok(a)) return c.g1(a, stream);
    return c.group(a, stream);
}

}  // namespace w4a4
