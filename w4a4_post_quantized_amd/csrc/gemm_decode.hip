// Decode GEMM (M <= 64 tokens): the same INT4 x INT4 product with int32
// accumulation and dequant epilogue as the prefill kernels of gemm.hip
// (FlatQuant page, section 核心思想: the layer is Q(XP) · Q(P^-1 W^T);
// FRM-PTQ page, section 初步介绍: codes with a zero point; FPTQuant page,
// section 3. 伪动态残差缩放: the token scale commutes with the bias-free
// product), for batches small enough that streaming the packed weights from
// HBM is the whole cost.
#include "common.hpp"
#include "internal.hpp"

namespace w4a4 {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int BK = 128;          // codes per K tile

// fp16 output with one weight scale per row (G == 1), or per-group fp32
// rescale inside the K loop
enum Mode { kModeChan = 0, kModeGroup = 1 };

// ===========================================================================
// Decode kernel (M <= 64 tokens): the weight stream is the whole cost, so the
// packed weights go from HBM straight into registers, with no LDS staging.
// A workgroup owns 16*FN output columns; its NW waves split the K tiles
// evenly and each streams its range with loads D-1 tiles ahead (the tile
// index is clamped, so every step issues the same loads).  A lane loads 16
// packed bytes of one row per fragment, the row segment of its lane group
// (lane >> 4), and unpacks them into the even-code and odd-code operands of
// two 16x16x64 MFMA k-steps; A and B use the same order.  Activation rows
// past M are clamped and their sums dropped.
//
// The workgroup first copies its rows' scales and zero points (one 32-bit
// word per row and group: fp16 scale | zero point << 16) into LDS, and, when
// they fit (ALDS, one row fragment), the M activation rows; the K loop then
// reads them with LDS loads instead of one small global load per tile.  The
// waves' partial sums (exact int32 per channel, fp32 per group) are added in
// LDS in wave order and written by the whole workgroup.
// ===========================================================================
constexpr int kDecLdsMax = 160 * 1024;      // LDS of one CU
constexpr int kDecAldsMax = 152 * 1024;     // budget for staged activations + scales

template <int FM, int FN, int NW, int D, bool ASYM, int MODE, bool ALDS, bool G1>
__global__ __launch_bounds__(NW * 64) void k_gemm_dec(
    const uint8_t* __restrict__ Xq, const float* __restrict__ s_x,
    const uint8_t* __restrict__ Wq, const uint16_t* __restrict__ s_w,
    const uint16_t* __restrict__ z_w, uint16_t* __restrict__ Y, int M, int N, int K,
    int group_size) {
    static_assert(MODE == kModeChan || MODE == kModeGroup, "fp16 output modes only");
    static_assert(D >= 2 && D <= 8, "prefetch depth");
    static_assert(!ALDS || FM == 1, "staged activations: one row fragment");
    static_assert(!G1 || MODE == kModeGroup, "one-tile groups: per-group mode");
    constexpr int BN = 16 * FN;
    constexpr int NT = NW * 64;
    constexpr int SLOTS = FM * FN * 4;          // accumulator values per lane
    constexpr bool SZ = (MODE == kModeGroup) || ASYM;
    extern __shared__ __align__(16) uint8_t lds[];

    const int lane = threadIdx.x & 63;
    // wave-uniform values live in scalar registers: tile ranges, group
    // indices and the tile part of every address
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int frow = lane & 15;
    const int fks = lane >> 4;
    const int n0 = blockIdx.x * BN;
    const int KB = K / 2;
    const int KT = K / BK;
    const int TPG = group_size / BK;
    const int G = K / group_size;
    const int t0 = (KT * wave) / NW;
    const int t1 = (KT * (wave + 1)) / NW;
    const int GP = G + 1;          // scale-table row: an odd number of words
    // staged activation row: KB rounded up to 256 bytes plus 32, so that the
    // 16 rows one fragment read touches fall in distinct LDS banks
    const int AP = (KB + 255) / 256 * 256 + 32;
    uint32_t* sz = reinterpret_cast<uint32_t*>(lds);
    uint8_t* al = lds + (SZ ? BN * GP * 4 : 0);

    // per-lane byte offsets (32-bit) from the wave-uniform bases
    uint32_t aoff[FM], boff[FN], zoff[FN];
#pragma unroll
    for (int a = 0; a < FM; ++a) {
        const int r = min(a * 16 + frow, M - 1);
        aoff[a] = static_cast<uint32_t>(r) * (ALDS ? AP : KB) + fks * 16;
    }
#pragma unroll
    for (int b = 0; b < FN; ++b) {
        const int r = min(n0 + b * 16 + frow, N - 1) - n0;
        boff[b] = static_cast<uint32_t>(r) * KB + fks * 16;
        zoff[b] = static_cast<uint32_t>(b * 16 + frow) * GP;
    }
    const uint8_t* wbase = Wq + static_cast<size_t>(n0) * KB;

    v4i acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) acc[a][b] = v4i{0, 0, 0, 0};
    constexpr int GF = (MODE == kModeGroup) ? 1 : 0;
    float facc[GF ? FM : 1][GF ? FN : 1][4];
#pragma unroll
    for (int a = 0; a < (GF ? FM : 1); ++a)
#pragma unroll
        for (int b = 0; b < (GF ? FN : 1); ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) facc[a][b][r] = 0.0f;

    uint4 abuf[ALDS ? 1 : D][FM], bbuf[D][FN];
    // a zero accumulator operand the compiler cannot fold into an inline
    // constant (an MFMA with an inline-zero accumulator gave wrong sums)
    v4i zc;
    {
        int z0;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z0));
        zc = v4i{z0, z0, z0, z0};
    }
    // issue position: tile it, clamped to the last tile of the range
    int it = t0;
    auto issue = [&](auto S) {
        constexpr int SL = decltype(S)::value;
        if constexpr (!ALDS) {
            const uint8_t* xa = Xq + static_cast<size_t>(it) * 64;
#pragma unroll
            for (int a = 0; a < FM; ++a) abuf[SL][a] = *reinterpret_cast<const uint4*>(xa + aoff[a]);
        }
        const uint8_t* wb = wbase + static_cast<size_t>(it) * 64;
#pragma unroll
        for (int b = 0; b < FN; ++b) bbuf[SL][b] = *reinterpret_cast<const uint4*>(wb + boff[b]);
        it = min(it + 1, t1 - 1);
    };
    // the first D - 1 tiles' loads go out before the staging below, which
    // then overlaps them
    if (t0 < t1) static_for<0, D - 1>([&](auto U) { issue(U); });

    // ---- stage the activations and the scale table ---------------------------
    if constexpr (ALDS) {
        // activation rows by direct-to-LDS copies: 16-byte slot s of the
        // staged block holds row s / RS, chunk s % RS (RS = AP / 16); chunks
        // past the row's KB / 16 and rows past M are padding (copied from a
        // valid address, never read).  Lane l of copy j fills slot 64 j + l.
        const int RS = AP / 16;
        const int nslots = M * RS;
        for (int j = wave; j * 64 < nslots; j += NW) {
            const int s = j * 64 + lane;
            const int r = s / RS;
            const int c = s - r * RS;
            const uint32_t off = (r < M && c < KB / 16) ? static_cast<uint32_t>(r) * KB + c * 16 : 0u;
            dma16_async_sv(Xq, off, al + j * 1024);
        }
    }
    if constexpr (SZ) {
        // the wave's rows wave, wave + NW, ...: every load of a chunk of 256
        // groups is issued before the first store
        constexpr int R = (BN + NW - 1) / NW;
        for (int gb = 0; gb < G; gb += 256) {
            uint32_t v[R][4];
#pragma unroll
            for (int q = 0; q < R; ++q) {
                const int r = min(wave + q * NW, BN - 1);
                const size_t nrow = static_cast<size_t>(min(n0 + r, N - 1)) * G;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int g = min(gb + lane + 64 * j, G - 1);
                    v[q][j] = (MODE == kModeGroup) ? s_w[nrow + g] : 0u;
                    if constexpr (ASYM) v[q][j] |= static_cast<uint32_t>(h2f(z_w[nrow + g])) << 16;
                }
            }
#pragma unroll
            for (int q = 0; q < R; ++q) {
                const int r = wave + q * NW;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (r < BN && gb + lane + 64 * j < G) sz[r * GP + gb + lane + 64 * j] = v[q][j];
            }
        }
    }
    if constexpr (ALDS) wait_vmcnt<0>();            // this wave's copies have landed
    if constexpr (SZ || ALDS) __syncthreads();

    // compute position: group cg of tile t and its place cr inside the group
    int cg = t0 / TPG, cr = t0 - (t0 / TPG) * TPG;
    auto compute = [&](int t, auto S) {
        constexpr int SL = decltype(S)::value;
        v4i aev[FM], aod[FM], bev[FN], bod[FN];
#pragma unroll
        for (int a = 0; a < FM; ++a) {
            uint4 w;
            if constexpr (ALDS)
                w = *reinterpret_cast<const uint4*>(al + aoff[a] + t * 64);
            else
                w = abuf[SL][a];
            uint4 ev, od;
            unpack_signed16(w, ev, od);
            aev[a] = v4i{static_cast<int>(ev.x), static_cast<int>(ev.y), static_cast<int>(ev.z), static_cast<int>(ev.w)};
            aod[a] = v4i{static_cast<int>(od.x), static_cast<int>(od.y), static_cast<int>(od.z), static_cast<int>(od.w)};
        }
        uint32_t szv[FN];
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            if constexpr (SZ) szv[b] = sz[zoff[b] + (G1 ? t : cg)];
            uint4 ev, od;
            if constexpr (ASYM) {
                const uint32_t z = szv[b] >> 16;
                unpack_asym(bbuf[SL][b], 0x80808080u - z * 0x01010101u, ev, od);
            } else {
                unpack_signed16(bbuf[SL][b], ev, od);
            }
            bev[b] = v4i{static_cast<int>(ev.x), static_cast<int>(ev.y), static_cast<int>(ev.z), static_cast<int>(ev.w)};
            bod[b] = v4i{static_cast<int>(od.x), static_cast<int>(od.y), static_cast<int>(od.z), static_cast<int>(od.w)};
        }
        if constexpr (G1) {
            // one tile per weight group: the group's sums start from a zero
            // register operand and are folded into fp32 at once
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const float sw = h2f(static_cast<uint16_t>(szv[b] & 0xFFFFu));
#pragma unroll
                for (int a = 0; a < FM; ++a) {
                    v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(aev[a], bev[b], zc, 0, 0, 0);
                    p = __builtin_amdgcn_mfma_i32_16x16x64_i8(aod[a], bod[b], p, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        facc[a][b][r] = fmaf(static_cast<float>(p[r]), sw, facc[a][b][r]);
                }
            }
            return;
        }
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aev[a], bev[b], acc[a][b], 0, 0, 0);
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aod[a], bod[b], acc[a][b], 0, 0, 0);
        const bool group_end = (++cr == TPG);
        if constexpr (MODE == kModeGroup) {
            // end of a weight group, or of this wave's range inside one
            if (group_end || t + 1 == t1) {
#pragma unroll
                for (int b = 0; b < FN; ++b) {
                    const float sw = h2f(static_cast<uint16_t>(szv[b] & 0xFFFFu));
#pragma unroll
                    for (int a = 0; a < FM; ++a)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            facc[a][b][r] = fmaf(static_cast<float>(acc[a][b][r]), sw, facc[a][b][r]);
                            acc[a][b][r] = 0;
                        }
                }
            }
        }
        if (group_end) {
            cr = 0;
            ++cg;
        }
    };

    // Main loop over whole groups of D tiles with no branch around a step
    // (with one, the compiler's waits at the join assumed the fewest loads in
    // flight and drained the prefetch), then at most D - 1 tiles whose loads
    // are already in flight.  Tile t uses buffer slot (t - t0) % D.
    if (t0 < t1) {
        int t = t0;
        for (; t + D <= t1; t += D) {
            static_for<0, D>([&](auto U) {
                constexpr int u = decltype(U)::value;
                issue(std::integral_constant<int, (u + D - 1) % D>{});
                // keep the step's loads ahead of its arithmetic: left free,
                // the scheduler sinks them below the MFMAs and the waits for
                // the current tile then cover them too
                __builtin_amdgcn_sched_barrier(0);
                compute(t + u, std::integral_constant<int, u>{});
            });
        }
        static_for<0, D - 1>([&](auto U) {
            constexpr int u = decltype(U)::value;
            if (t + u < t1) compute(t + u, std::integral_constant<int, u>{});
        });
    }

    // ---- add the waves' partial sums in LDS, in wave order -------------------
    if constexpr (SZ || ALDS) __syncthreads();      // the staged data is dead
    float* red = reinterpret_cast<float*>(lds);     // [NW][SLOTS][64]
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = (a * FN + b) * 4 + r;
                red[(wave * SLOTS + i) * 64 + lane] = (MODE == kModeGroup) ? facc[GF ? a : 0][GF ? b : 0][r]
                                                                           : __int_as_float(acc[a][b][r]);
            }
    __syncthreads();
    constexpr float kUnshift = ASYM ? (1.0f / 16.0f) : (1.0f / 256.0f);
    for (int sl = threadIdx.x; sl < SLOTS * 64; sl += NT) {
        const int i = sl >> 6;
        const int l = sl & 63;
        const int a = i / (FN * 4);
        const int b = (i >> 2) % FN;
        const int r = i & 3;
        const int gm = a * 16 + 4 * (l >> 4) + r;
        const int gn = n0 + b * 16 + (l & 15);
        if (gm >= M || gn >= N) continue;
        float v;
        if constexpr (MODE == kModeGroup) {
            v = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) v += red[(w * SLOTS + i) * 64 + l];
        } else {
            int sum = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) sum += __float_as_int(red[(w * SLOTS + i) * 64 + l]);
            v = static_cast<float>(sum) * h2f(s_w[gn]);
        }
        Y[static_cast<size_t>(gm) * N + gn] = f2h(v * s_x[gm] * kUnshift);
    }
}

template <int FM, int FN, int NW, int D, bool ASYM, int MODE, bool ALDS, bool G1>
hipError_t launch_dec_g(const GemmArgs& a, size_t lds, hipStream_t stream) {
    auto* kern = &k_gemm_dec<FM, FN, NW, D, ASYM, MODE, ALDS, G1>;
    if (lds > 64 * 1024) {
        // more than the default dynamic LDS limit: raise it once per device
        static bool raised[64] = {};
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= 64 || !raised[dev]) {
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, kDecLdsMax);
            if (e != hipSuccess) return e;
            if (dev >= 0 && dev < 64) raised[dev] = true;
        }
    }
    kern<<<dim3(ceil_div(a.N, 16 * FN)), dim3(NW * 64), lds, stream>>>(
        a.Xq, a.s_x, a.Wq, a.s_w, a.z_w, a.Y, a.M, a.N, a.K, a.group_size);
    return hipGetLastError();
}

template <int FM, int FN, int NW, int D, bool ASYM, int MODE, bool ALDS>
hipError_t launch_dec_k(const GemmArgs& a, size_t lds, hipStream_t stream) {
    if constexpr (MODE == kModeGroup) {
        if (a.group_size == BK) return launch_dec_g<FM, FN, NW, D, ASYM, MODE, ALDS, true>(a, lds, stream);
    }
    return launch_dec_g<FM, FN, NW, D, ASYM, MODE, ALDS, false>(a, lds, stream);
}

template <int FM, int FN, int NW, int D, bool ASYM, int MODE>
hipError_t launch_dec_a(const GemmArgs& a, hipStream_t stream) {
    constexpr int BN = 16 * FN;
    const int G = a.K / a.group_size;
    const bool sz = (MODE == kModeGroup) || ASYM;
    const size_t szb = sz ? static_cast<size_t>(BN) * (G + 1) * 4 : 0;
    // staged rows at the kernel's pitch, rounded up to whole 1 KiB copies
    const size_t ap = static_cast<size_t>((a.K / 2 + 255) / 256 * 256 + 32);
    const size_t alb = (static_cast<size_t>(a.M) * ap + 1023) / 1024 * 1024;
    const size_t red = static_cast<size_t>(NW) * FM * FN * 4 * 64 * 4;
    if constexpr (FM == 1) {
        if (szb + alb <= static_cast<size_t>(kDecAldsMax))
            return launch_dec_k<FM, FN, NW, D, ASYM, MODE, true>(a, szb + alb > red ? szb + alb : red,
                                                                 stream);
    }
    return launch_dec_k<FM, FN, NW, D, ASYM, MODE, false>(a, szb > red ? szb : red, stream);
}

template <int FM, int FN, int NW, int D, int MODE>
hipError_t launch_dec(const GemmArgs& a, hipStream_t stream) {
    return a.asym ? launch_dec_a<FM, FN, NW, D, true, MODE>(a, stream)
                  : launch_dec_a<FM, FN, NW, D, false, MODE>(a, stream);
}


// ===========================================================================
// Split-K decode kernel (M <= 64 tokens): a workgroup of 8 waves owns 256
// output columns (32 per wave, two 16-column fragments) and one of S ranges
// of K tiles.  Before its K loop it copies the range's activation rows
// (packed, M rows, each padded to a bank-friendly pitch) and, for groups of one
// K tile, the range's weight scales and zero points of its columns into LDS,
// all by global_load_lds copies issued from inline assembly and retired by
// one wait.  The packed weights then stream from HBM into registers as in
// k_gemm_dec (D - 1 tiles of loads in flight per wave), and every wave
// reads its activation fragments from the staged rows.  The activations are
// thus read from L2 once per 256 columns, not once per 16 or 32 as in
// k_gemm_dec, and the weight stream has no LDS stage or barrier in its way.
// S is the smallest split that gives about one workgroup per CU, with at
// least 8 K tiles per range (the partial sums stay a small fraction of the
// weight bytes) and a staged range that fits the LDS.  Each workgroup writes its range's sums (exact
// int32 per channel, fp32 per one-tile group) for its columns;
// k_dec_split_reduce adds the ranges in a fixed order and applies the
// scales.
// ===========================================================================
constexpr int kSpCols = 256;                 // columns per workgroup
constexpr int kSpWaves = 8;
constexpr int kSpDepth = 6;                  // weight tiles in flight per wave, plus one
constexpr int kSpLds = 160 * 1024;
constexpr int kSpTargetGroups = 256;         // one workgroup per CU of MI355X
constexpr int kSpMinTiles = 8;             // K tiles per range at least (bounds the partial sums)

struct SplitPlan {
    int FM = 1;            // 16-row activation fragments
    int S = 1;             // K ranges
    int kps = 1;           // K tiles per range (the last range may be shorter)
    int ap = 0;            // bytes per staged activation row (split_row_pitch)
    int wr = 0;            // 4-byte words per scale-table row (odd)
    int a_bytes = 0;       // staged activations, a multiple of 1 KiB
    int t_bytes = 0;       // one scale (or zero-point) table, a multiple of 256 bytes
    int lds = 0;
};

int split_fm(int M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }

// bytes per staged activation row: the range's 64 kps bytes rounded up to
// 256 plus 32, so that the 16 rows one fragment read touches (4 chunks of 16
// bytes each) fall in distinct LDS banks (a pitch of 64 kps + 16 counted 2
// conflict cycles per ds_read_b128 of the workgroup, one of 32 mod 256 none)
__host__ __device__ constexpr int split_row_pitch(int kps) { return (64 * kps + 255) / 256 * 256 + 32; }

SplitPlan split_layout(int M, int kps, bool g1, bool asym) {
    SplitPlan p;
    p.FM = split_fm(M);
    p.kps = kps;
    p.ap = split_row_pitch(kps);
    p.a_bytes = ceil_div(M * p.ap, 1024) * 1024;
    p.wr = (kps / 2 + 1) | 1;
    p.t_bytes = g1 ? ceil_div(kSpCols * p.wr * 4, 256) * 256 : 0;
    p.lds = p.a_bytes + (asym ? 2 : 1) * p.t_bytes;
    return p;
}

SplitPlan split_plan(int M, int N, int K, int group_size, bool asym) {
    const int KT = K / BK;
    const bool g1 = K / group_size > 1;
    const int nbx = ceil_div(N, kSpCols);
    const int s0 = std::max(1, std::min(KT, ceil_div(kSpTargetGroups, nbx)));
    int kps = std::max(ceil_div(KT, s0), std::min(KT, kSpMinTiles));
    while (kps > 1 && split_layout(M, kps, g1, asym).lds > kSpLds) --kps;
    const int S = ceil_div(KT, kps);
    SplitPlan p = split_layout(M, ceil_div(KT, S), g1, asym);
    p.S = S;
    return p;
}

template <int FM, int D, bool ASYM, bool G1>
__global__ __launch_bounds__(kSpWaves * 64) void k_gemm_dec_split(
    const uint8_t* __restrict__ Xq, const uint8_t* __restrict__ Wq,
    const uint16_t* __restrict__ s_w, const uint16_t* __restrict__ z_w,
    int32_t* __restrict__ part, int M, int N, int K, int S, int kps, int wr, int a_bytes,
    int t_bytes) {
    static_assert(D >= 2 && D <= 8, "prefetch depth");
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int frow = lane & 15;
    const int fks = lane >> 4;
    // workgroups are dealt to the 8 XCDs in turn; when they divide evenly,
    // XCD x takes the x-th eighth of the (column block, range) list, so all
    // ranges of a column block share one L2: the rows of the scale tables
    // (one row holds every range's groups) are fetched once, not once per
    // range.  The activations are then read by every XCD (64 B per row and
    // tile, a hundredth of the weights).
    const int bid = static_cast<int>(blockIdx.x);
    const int total = static_cast<int>(gridDim.x);
    const int wid = (total & 7) == 0 ? (bid & 7) * (total >> 3) + (bid >> 3) : bid;
    const int by = wid % S;
    const int n0 = (wid / S) * kSpCols;
    const int KB = K / 2;
    const int KT = K / BK;
    const int G = G1 ? KT : 1;
    const int kt0 = by * kps;
    const int nt = min(KT, kt0 + kps) - kt0;        // >= 1: S = ceil(KT / kps)

    // ---- weight loads of the first D - 1 tiles ------------------------------
    const uint8_t* wbase = Wq + static_cast<size_t>(n0) * KB + static_cast<size_t>(kt0) * 64;
    uint32_t boff[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
        boff[b] = static_cast<uint32_t>(min(n0 + 32 * wave + 16 * b + frow, N - 1) - n0) * KB + fks * 16;
    uint4 bbuf[D][2];
    int it = 0;
    auto issue = [&](auto SL) {
        constexpr int sl = decltype(SL)::value;
        const uint8_t* wb = wbase + static_cast<size_t>(it) * 64;
#pragma unroll
        for (int b = 0; b < 2; ++b) bbuf[sl][b] = *reinterpret_cast<const uint4*>(wb + boff[b]);
        it = min(it + 1, nt - 1);
    };
    static_for<0, D - 1>([&](auto U) { issue(U); });

    // ---- stage the range's activations: slot s of 16 bytes holds row
    // s / RS, chunk s % RS (RS = split_row_pitch(kps) / 16); chunks past the
    // range's 4 nt and rows past M are padding (copied from a valid address,
    // never read).  Lane l of copy j fills slot 64 j + l.
    const int rslots = split_row_pitch(kps) / 16;
    const uint8_t* xbase = Xq + static_cast<size_t>(kt0) * 64;
    for (int j = wave; j * 64 < a_bytes / 16; j += kSpWaves) {
        const int s = j * 64 + lane;
        const int r = s / rslots;
        const int c = s - r * rslots;
        const uint32_t off = (r < M && c < 4 * nt) ? static_cast<uint32_t>(r) * KB + c * 16 : 0u;
        dma16_async_sv(xbase, off, lds + j * 1024);
    }
    // ---- stage the scale (and zero-point) table of one-tile groups: row r
    // holds the 4-byte words from the one containing element (n0 + r) G + kt0
    // on, so tile t of the range is half (p + t) % 2 of word (p + t) / 2,
    // p the parity of that first element.  Words past the array are clamped.
    if constexpr (G1) {
        const uint32_t last_word = (static_cast<uint32_t>(N) * static_cast<uint32_t>(G) - 1u) >> 1;
        for (int j = wave; j * 64 < t_bytes / 4; j += kSpWaves) {
            const int s = j * 64 + lane;
            const int r = s / wr;
            const int w = s - r * wr;
            const uint32_t e0 = static_cast<uint32_t>(min(n0 + r, N - 1)) * static_cast<uint32_t>(G) + kt0;
            const uint32_t word = min((e0 >> 1) + static_cast<uint32_t>(w), last_word);
            dma4_async_sv(s_w, 4u * word, lds + a_bytes + j * 256);
            if constexpr (ASYM) dma4_async_sv(z_w, 4u * word, lds + a_bytes + t_bytes + j * 256);
        }
    }

    // per-lane LDS offsets of the activation fragments (rows past M clamped)
    uint32_t aoff[FM];
#pragma unroll
    for (int a = 0; a < FM; ++a)
        aoff[a] = static_cast<uint32_t>(min(16 * a + frow, M - 1)) * split_row_pitch(kps) + fks * 16;
    // the lane's two columns: scale-table word base and parity, or the
    // per-channel zero point
    uint32_t tb[2], par[2], zb[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int r = 32 * wave + 16 * b + frow;
        const int ncol = min(n0 + r, N - 1);
        tb[b] = static_cast<uint32_t>(r * wr);
        par[b] = (static_cast<uint32_t>(ncol) * static_cast<uint32_t>(G) + kt0) & 1u;
        zb[b] = 0x80808080u;
        if constexpr (ASYM && !G1) zb[b] = 0x80808080u - static_cast<uint32_t>(h2f(z_w[ncol])) * 0x01010101u;
    }
    const uint32_t* stab = reinterpret_cast<const uint32_t*>(lds + a_bytes);
    const uint32_t* ztab = reinterpret_cast<const uint32_t*>(lds + a_bytes + t_bytes);

    v4i acc[FM][2];
    float facc[G1 ? FM : 1][G1 ? 2 : 1][4];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int a = 0; a < (G1 ? FM : 1); ++a)
#pragma unroll
        for (int b = 0; b < (G1 ? 2 : 1); ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) facc[a][b][r] = 0.0f;
    // a zero accumulator operand the compiler cannot fold into an inline constant
    v4i zc;
    {
        int z0;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z0));
        zc = v4i{z0, z0, z0, z0};
    }

    // every copy (and weight load) of this wave has landed; after the
    // barrier every wave's staged data is visible
    wait_vmcnt<0>();
    __syncthreads();

    auto compute = [&](int t, auto SL) {
        constexpr int sl = decltype(SL)::value;
        v4i aev[FM], aod[FM], bev[2], bod[2];
#pragma unroll
        for (int a = 0; a < FM; ++a) {
            const uint4 w = *reinterpret_cast<const uint4*>(lds + aoff[a] + t * 64);
            uint4 ev, od;
            unpack_signed16(w, ev, od);
            aev[a] = v4i{static_cast<int>(ev.x), static_cast<int>(ev.y), static_cast<int>(ev.z), static_cast<int>(ev.w)};
            aod[a] = v4i{static_cast<int>(od.x), static_cast<int>(od.y), static_cast<int>(od.z), static_cast<int>(od.w)};
        }
        float sw[2] = {0.0f, 0.0f};
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            uint32_t bias = zb[b];
            if constexpr (G1) {
                const uint32_t q = par[b] + static_cast<uint32_t>(t);
                const uint32_t wi = tb[b] + (q >> 1);
                const uint32_t sh = 16u * (q & 1u);
                sw[b] = h2f(static_cast<uint16_t>(stab[wi] >> sh));
                if constexpr (ASYM)
                    bias = 0x80808080u - static_cast<uint32_t>(h2f(static_cast<uint16_t>(ztab[wi] >> sh))) * 0x01010101u;
            }
            uint4 ev, od;
            if constexpr (ASYM)
                unpack_asym(bbuf[sl][b], bias, ev, od);
            else
                unpack_signed16(bbuf[sl][b], ev, od);
            bev[b] = v4i{static_cast<int>(ev.x), static_cast<int>(ev.y), static_cast<int>(ev.z), static_cast<int>(ev.w)};
            bod[b] = v4i{static_cast<int>(od.x), static_cast<int>(od.y), static_cast<int>(od.z), static_cast<int>(od.w)};
        }
        if constexpr (G1) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int a = 0; a < FM; ++a) {
                    v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(aev[a], bev[b], zc, 0, 0, 0);
                    p = __builtin_amdgcn_mfma_i32_16x16x64_i8(aod[a], bod[b], p, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) facc[a][b][r] = fmaf(static_cast<float>(p[r]), sw[b], facc[a][b][r]);
                }
        } else {
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aev[a], bev[b], acc[a][b], 0, 0, 0);
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aod[a], bod[b], acc[a][b], 0, 0, 0);
        }
    };

    // whole rotations of D tiles with no branch around a step, then at most
    // D - 1 tiles whose loads are in flight (as in k_gemm_dec)
    int t = 0;
    for (; t + D <= nt; t += D) {
        static_for<0, D>([&](auto U) {
            constexpr int u = decltype(U)::value;
            issue(std::integral_constant<int, (u + D - 1) % D>{});
            __builtin_amdgcn_sched_barrier(0);
            compute(t + u, std::integral_constant<int, u>{});
        });
    }
    static_for<0, D - 1>([&](auto U) {
        constexpr int u = decltype(U)::value;
        if (t + u < nt) compute(t + u, std::integral_constant<int, u>{});
    });

    // ---- this range's sums: lane (fks, frow) holds rows 16 a + 4 fks + r of
    // column n0 + 32 wave + 16 b + frow
    int32_t* pr = part + static_cast<size_t>(by) * M * N;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int gn = n0 + 32 * wave + 16 * b + frow;
        if (gn >= N) continue;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int gm = 16 * a + 4 * fks + r;
                if (gm < M)
                    pr[static_cast<size_t>(gm) * N + gn] = G1 ? __float_as_int(facc[a][b][r]) : acc[a][b][r];
            }
    }
}

// Y = fp16(s_x[m] * unshift * (sum of the ranges' sums, in range order)
//          [* s_w[n] per channel]); thread i takes outputs 4 i .. 4 i + 3 of
// the row-major [M, N] result (16-byte loads when N % 4 == 0)
template <bool ASYM, bool G1>
__global__ __launch_bounds__(256) void k_dec_split_reduce(const int32_t* __restrict__ part,
                                                          const float* __restrict__ s_x,
                                                          const uint16_t* __restrict__ s_w,
                                                          uint16_t* __restrict__ Y, int M, int N,
                                                          int splits) {
    const size_t MN = static_cast<size_t>(M) * N;
    const size_t e0 = (static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (e0 >= MN) return;
    constexpr float kUnshift = ASYM ? (1.0f / 16.0f) : (1.0f / 256.0f);
    if ((N & 3) == 0) {
        // four outputs of one row
        const int m = static_cast<int>(e0 / N);
        const int n = static_cast<int>(e0 - static_cast<size_t>(m) * N);
        float v[4];
        if constexpr (G1) {
            float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            for (int sp = 0; sp < splits; ++sp) {
                const int4 w = *reinterpret_cast<const int4*>(part + sp * MN + e0);
                acc.x += __int_as_float(w.x);
                acc.y += __int_as_float(w.y);
                acc.z += __int_as_float(w.z);
                acc.w += __int_as_float(w.w);
            }
            v[0] = acc.x; v[1] = acc.y; v[2] = acc.z; v[3] = acc.w;
        } else {
            int4 acc = make_int4(0, 0, 0, 0);
            for (int sp = 0; sp < splits; ++sp) {
                const int4 w = *reinterpret_cast<const int4*>(part + sp * MN + e0);
                acc.x += w.x;
                acc.y += w.y;
                acc.z += w.z;
                acc.w += w.w;
            }
            v[0] = static_cast<float>(acc.x) * h2f(s_w[n]);
            v[1] = static_cast<float>(acc.y) * h2f(s_w[n + 1]);
            v[2] = static_cast<float>(acc.z) * h2f(s_w[n + 2]);
            v[3] = static_cast<float>(acc.w) * h2f(s_w[n + 3]);
        }
        const float sx = s_x[m] * kUnshift;
        ushort4 o;
        o.x = f2h(v[0] * sx);
        o.y = f2h(v[1] * sx);
        o.z = f2h(v[2] * sx);
        o.w = f2h(v[3] * sx);
        *reinterpret_cast<ushort4*>(Y + e0) = o;
        return;
    }
    for (size_t e = e0; e < e0 + 4 && e < MN; ++e) {
        const int m = static_cast<int>(e / N);
        const int n = static_cast<int>(e - static_cast<size_t>(m) * N);
        float v;
        if constexpr (G1) {
            v = 0.0f;
            for (int sp = 0; sp < splits; ++sp) v += __int_as_float(part[sp * MN + e]);
        } else {
            int sum = 0;
            for (int sp = 0; sp < splits; ++sp) sum += part[sp * MN + e];
            v = static_cast<float>(sum) * h2f(s_w[n]);
        }
        Y[e] = f2h(v * s_x[m] * kUnshift);
    }
}

template <int FM, bool ASYM, bool G1>
hipError_t launch_split_k(const GemmArgs& a, const SplitPlan& p, void* ws, hipStream_t stream) {
    auto* kern = &k_gemm_dec_split<FM, kSpDepth, ASYM, G1>;
    static bool raised[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64 || !raised[dev]) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kSpLds);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) raised[dev] = true;
    }
    int32_t* part = static_cast<int32_t*>(ws);
    const unsigned groups = static_cast<unsigned>(ceil_div(a.N, kSpCols) * p.S);
    kern<<<dim3(groups), dim3(kSpWaves * 64), p.lds, stream>>>(a.Xq, a.Wq, a.s_w, a.z_w, part, a.M, a.N,
                                                                a.K, p.S, p.kps, p.wr, p.a_bytes,
                                                                p.t_bytes);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long quads = (static_cast<long>(a.M) * a.N + 3) / 4;
    k_dec_split_reduce<ASYM, G1><<<static_cast<unsigned>((quads + 255) / 256), 256, 0, stream>>>(
        part, a.s_x, a.s_w, a.Y, a.M, a.N, p.S);
    return hipGetLastError();
}

template <int FM>
hipError_t launch_split_f(const GemmArgs& a, const SplitPlan& p, void* ws, hipStream_t stream) {
    const bool g1 = (a.K / a.group_size) > 1;
    if (a.asym)
        return g1 ? launch_split_k<FM, true, true>(a, p, ws, stream)
                  : launch_split_k<FM, true, false>(a, p, ws, stream);
    return g1 ? launch_split_k<FM, false, true>(a, p, ws, stream)
              : launch_split_k<FM, false, false>(a, p, ws, stream);
}

// per channel, or groups of one K tile; at most 64 tokens
bool split_supports(const GemmArgs& a) {
    const int G = a.K / a.group_size;
    if (a.M < 1 || a.M > 64 || !(G == 1 || a.group_size == BK)) return false;
    return static_cast<size_t>(a.N) * static_cast<size_t>(G) < (size_t{1} << 31);
}

size_t split_workspace_bytes(int M, int N, int K, int group_size, bool asym) {
    const SplitPlan p = split_plan(M, N, K, group_size, asym);
    const size_t b = sizeof(int32_t) * static_cast<size_t>(p.S) * static_cast<size_t>(M) * static_cast<size_t>(N);
    return (b + 255) & ~static_cast<size_t>(255);
}

hipError_t launch_split(const GemmArgs& a, void* ws, hipStream_t stream) {
    const SplitPlan p = split_plan(a.M, a.N, a.K, a.group_size, a.asym);
    if (p.FM == 1) return launch_split_f<1>(a, p, ws, stream);
    if (p.FM == 2) return launch_split_f<2>(a, p, ws, stream);
    return launch_split_f<4>(a, p, ws, stream);
}

using LaunchFn = hipError_t (*)(const GemmArgs&, hipStream_t);

struct KernelCfg {
    const char* name;
    LaunchFn chan, group;
};

// Decode configurations (M <= 64), per row-fragment count FM = 1, 2, 4:
// 16*FN columns per workgroup, NW waves splitting K, prefetch depth D.
template <int FM, int FN, int NW, int D>
struct Dec {
    template <int MODE>
    static hipError_t run(const GemmArgs& a, hipStream_t s) { return launch_dec<FM, FN, NW, D, MODE>(a, s); }
};
#define W4A4_DEC(FM, FN, NW, D) \
    KernelCfg{"k_gemm_dec<FM " #FM ", FN " #FN ", waves " #NW ", depth " #D ">", \
              &Dec<FM, FN, NW, D>::run<kModeChan>, &Dec<FM, FN, NW, D>::run<kModeGroup>}
constexpr int kNumDec = 4;
const KernelCfg kDec[3][kNumDec] = {
    {W4A4_DEC(1, 1, 16, 4), W4A4_DEC(1, 2, 16, 4), W4A4_DEC(1, 1, 8, 6), W4A4_DEC(1, 2, 8, 6)},
    {W4A4_DEC(2, 1, 16, 4), W4A4_DEC(2, 2, 8, 4), W4A4_DEC(2, 1, 8, 4), W4A4_DEC(2, 2, 8, 3)},
    {W4A4_DEC(4, 1, 8, 3), W4A4_DEC(4, 2, 8, 4), W4A4_DEC(4, 1, 8, 6), W4A4_DEC(4, 2, 8, 6)},
};
#undef W4A4_DEC

// whether the register-streamed kernel's one-row-fragment configuration, as
// choose_dec picks it, stages the activations in LDS (launch_dec_a's test)
bool dec_staged_fits(const GemmArgs& a) {
    if (a.M > 16) return false;
    const size_t staged = static_cast<size_t>(a.M) * (a.K / 2 + 16);
    const bool wide = ceil_div(a.N, 32) >= device_cu_count() && staged > 64 * 1024;
    const int fn = wide ? 2 : 1;
    const int G = a.K / a.group_size;
    const bool sz = G > 1 || a.asym;
    const size_t szb = sz ? static_cast<size_t>(16 * fn) * (G + 1) * 4 : 0;
    const size_t ap = static_cast<size_t>((a.K / 2 + 255) / 256 * 256 + 32);
    const size_t alb = (static_cast<size_t>(a.M) * ap + 1023) / 1024 * 1024;
    return szb + alb <= static_cast<size_t>(kDecAldsMax);
}

// the split-K kernel (index kNumDec of the override), taken automatically
// from 17 tokens on, and from 9 when the register-streamed kernel cannot
// stage the activations in LDS.  Measured on MI355X (28672 -> 8192, groups
// of 128): 17 / 24 / 32 tokens 34.0 / 34.4 / 35.0 us against 34.7-37.4 /
// 37.0-39.4 / 40.7-43.6 us for the register-streamed configurations; 12 and
// 16 tokens (activations not staged) 32.0 and 32.3 us against 33.0 and
// 34.3 us; 8 tokens (staged) 34.1 against 27.7-29.5 us.
bool use_split(const GemmArgs& a) {
    if (!split_supports(a)) return false;
    const int o = kernel_override(1);
    if (o >= 0 && o <= kNumDec) return o == kNumDec;
    return a.M > 16 || (a.M > 8 && !dec_staged_fits(a));
}

const KernelCfg& choose_dec(const GemmArgs& a) {
    const int cus = device_cu_count();
    const int fi = a.M <= 16 ? 0 : (a.M <= 32 ? 1 : 2);
    const int o = kernel_override(1);
    int v = (o >= 0 && o < kNumDec) ? o : -1;
    if (v < 0) {
        // measured on MI355X (28672 -> 8192, group 128, weight copies
        // rotated): two 16-column fragments per workgroup once the staged
        // activations fill the LDS (or for two and four row fragments) and
        // the grid still covers every CU (8 tokens: 29.3 us against 32.7 us);
        // one fragment otherwise, with 8 waves and 6 tiles in flight for one
        // row fragment (1 token: 24.9 us against 26.3 us with 16 waves and 4
        // tiles) and 16 waves for more; for four row fragments 6 tiles in
        // flight (64 tokens: 56.6 against 57.3 us with 4 and 83-86 us with
        // one column fragment)
        bool wide = ceil_div(a.N, 32) >= cus;
        if (fi == 0) {
            const size_t staged = static_cast<size_t>(a.M) * (a.K / 2 + 16);
            wide = wide && staged > 64 * 1024;
        }
        if (fi == 0)
            v = wide ? 1 : 2;
        else if (fi == 2)
            v = wide ? 3 : 0;
        else
            v = wide ? 1 : 0;
    }
    return kDec[fi][v];
}

}  // namespace

int gemm_num_decode_configs() { return kNumDec + 1; }

size_t gemm_decode_workspace_bytes(int M, int N, int K, int group_size, bool asym) {
    GemmArgs a{};
    a.M = M;
    a.N = N;
    a.K = K;
    a.group_size = group_size;
    a.asym = asym;
    return split_supports(a) ? split_workspace_bytes(M, N, K, group_size, asym) : 0;
}

const char* gemm_decode_kernel_name(const GemmArgs& a) {
    if (use_split(a)) {
        const int fm = split_fm(a.M);
        return fm == 1 ? "k_gemm_dec_split<FM 1, 256 columns, waves 8, depth 6> + k_dec_split_reduce"
             : fm == 2 ? "k_gemm_dec_split<FM 2, 256 columns, waves 8, depth 6> + k_dec_split_reduce"
                       : "k_gemm_dec_split<FM 4, 256 columns, waves 8, depth 6> + k_dec_split_reduce";
    }
    return choose_dec(a).name;
}

hipError_t gemm_decode_launch(const GemmArgs& a, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (a.M == 0) return hipSuccess;
    if (use_split(a)) {
        if (ws == nullptr || ws_bytes < split_workspace_bytes(a.M, a.N, a.K, a.group_size, a.asym))
            return hipErrorInvalidValue;
        return launch_split(a, ws, stream);
    }
    const KernelCfg& k = choose_dec(a);
    return (a.K / a.group_size) > 1 ? k.group(a, stream) : k.chan(a, stream);
}

}  // namespace w4a4
