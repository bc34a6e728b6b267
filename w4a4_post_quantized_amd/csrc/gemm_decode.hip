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
    const int AP = KB + 16;        // staged activation row, padded one chunk
    uint32_t* sz = reinterpret_cast<uint32_t*>(lds);
    uint8_t* al = lds + (SZ ? BN * GP * 4 : 0);

    // ---- stage the scale table and the activations ------------------------
    if constexpr (SZ) {
        for (int r = wave; r < BN; r += NW) {
            const size_t nrow = static_cast<size_t>(min(n0 + r, N - 1)) * G;
            for (int gb = 0; gb < G; gb += 256) {
                uint32_t v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int g = min(gb + lane + 64 * j, G - 1);
                    v[j] = (MODE == kModeGroup) ? s_w[nrow + g] : 0u;
                    if constexpr (ASYM) v[j] |= static_cast<uint32_t>(h2f(z_w[nrow + g])) << 16;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (gb + lane + 64 * j < G) sz[r * GP + gb + lane + 64 * j] = v[j];
            }
        }
    }
    if constexpr (ALDS) {
        const int CH = KB / 16;
        for (int c = threadIdx.x; c < CH; c += NT)
            for (int r0 = 0; r0 < M; r0 += 4) {
                uint4 v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = *reinterpret_cast<const uint4*>(Xq + static_cast<size_t>(min(r0 + j, M - 1)) * KB + c * 16);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (r0 + j < M) *reinterpret_cast<uint4*>(al + (r0 + j) * AP + c * 16) = v[j];
            }
    }
    if constexpr (SZ || ALDS) __syncthreads();

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
        static_for<0, D - 1>([&](auto U) { issue(U); });
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
    const size_t alb = static_cast<size_t>(a.M) * (a.K / 2 + 16);
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
// Split-K decode kernel for up to 64 tokens with the copies of the prefill
// kernels.  A workgroup of 8 waves owns 128 output columns (16 per wave) and
// one of kD64Split ranges of K tiles; all its waves walk the same K tiles, so
// the activation tile (64 rows, clamped to M) is copied and unpacked once
// per workgroup.  Every K tile goes into a ring of LDS stages by
// global_load_lds copies issued from inline assembly with explicit waits
// (the compiler sees no vector load in the K loop, so none of its waits can
// drain the ring): waves 0-3 copy 16 activation rows and 16 weight rows
// each, waves 4-7 16 weight rows and one 64-row item of weight scales (and
// zero points) of the tile's group.  Per K tile the waves unpack the staged
// activation tile once into int8 even-code and odd-code halves (8 bytes of
// packed codes per lane) for the next tile, then multiply: four 16-row
// activation fragments against the wave's 16 weight rows on
// v_mfma_i32_16x16x64_i8, exactly as the register-streamed kernel above.
// Each workgroup writes its range's sums (int32 per channel, fp32 per group
// of 128) for its columns; k_dec64_reduce adds the ranges in a fixed order
// and applies the token scale.
// ===========================================================================
constexpr int kD64Rows = 64;
constexpr int kD64Cols = 128;
constexpr int kD64Waves = 8;
constexpr int kD64Stages = 6;
constexpr int kD64Split = 4;
constexpr int kD64A = kD64Rows * 64;          // packed activation tile
constexpr int kD64B = kD64Cols * 64;          // packed weight tile
constexpr int kD64SZ = 4 * 256;               // four 64-row items of 4-byte words
constexpr int kD64Stage = kD64A + kD64B + kD64SZ;
constexpr int kD64Half = kD64Rows * 4 * 16;   // one unpacked half (even or odd codes)
constexpr int kD64Lds = kD64Stages * kD64Stage + 2 * 2 * kD64Half;

template <bool ASYM, bool G1>
__global__ __launch_bounds__(kD64Waves * 64) void k_gemm_dec64(
    const uint8_t* __restrict__ Xq, const uint8_t* __restrict__ Wq,
    const uint16_t* __restrict__ s_w, const uint16_t* __restrict__ z_w,
    int32_t* __restrict__ part, int M, int N, int K, int kps) {
    constexpr int D = kD64Stages;
    constexpr int WAITN = (D - 3) * 2;          // copies per wave and tile: 2
    extern __shared__ __align__(16) uint8_t lds[];
    uint8_t* a8 = lds + D * kD64Stage;          // [buffer][even | odd] unpacked activations

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int frow = lane & 15;
    const int fks = lane >> 4;
    const int n0 = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * kD64Cols);
    const int KB = K / 2;
    const int KT = K / BK;
    const int G = G1 ? KT : 1;
    const int kt0 = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.y) * kps);
    const int nt = max(0, min(KT, kt0 + kps) - kt0);

    // ---- this wave's two copies per tile -----------------------------------
    // first: activation rows 16 w .. (waves 0-3) or weight rows 16 w .. (4-7);
    // second: weight rows 16 w .. (0-3) or scale item w - 4 (4-7).  Lane l
    // moves 16 bytes: row 16 w + l / 4, chunk l % 4 (row-major in the stage).
    const int crow = 16 * (wave & 3) + (lane >> 2);
    const int cchk = lane & 3;
    const bool first_a = wave < 4;
    const uint8_t* base1 = first_a ? Xq : Wq;
    uint32_t off1;
    if (first_a)
        off1 = static_cast<uint32_t>(min(crow, M - 1)) * KB + cchk * 16;
    else
        off1 = static_cast<uint32_t>(min(n0 + 16 * wave + (lane >> 2), N - 1) - n0) * KB + cchk * 16;
    const uint32_t off2b = static_cast<uint32_t>(min(n0 + 16 * wave + (lane >> 2), N - 1) - n0) * KB + cchk * 16;
    // scale item it = wave - 4: kind it / 2 (scale, zero point), rows 64 (it % 2) + lane
    const int it = wave & 3;
    const uint16_t* szb = (ASYM && it >= 2) ? z_w : s_w;
    const uint32_t sz_e0 = static_cast<uint32_t>(min(n0 + 64 * (it & 1) + lane, N - 1)) *
                           static_cast<uint32_t>(G);
    const int dst1 = first_a ? wave * 1024 : kD64A + wave * 1024;
    const int dst2 = first_a ? kD64A + wave * 1024 : kD64A + kD64B + it * 256;
    auto issue = [&](int i) {
        const int kc = kt0 + min(i, nt - 1);            // clamped: every step copies
        uint8_t* st = lds + (i % D) * kD64Stage;
        if (first_a) {
            dma16_async_sv(Xq + static_cast<size_t>(kc) * 64, off1, st + dst1);
            dma16_async_sv(Wq + static_cast<size_t>(n0) * KB + static_cast<size_t>(kc) * 64, off2b,
                           st + dst2);
        } else {
            dma16_async_sv(base1 + static_cast<size_t>(n0) * KB + static_cast<size_t>(kc) * 64, off1,
                           st + dst1);
            const uint32_t g = G1 ? static_cast<uint32_t>(kc) : 0u;
            dma4_async_sv(szb, 2u * ((sz_e0 + g) & ~1u), st + dst2);
        }
    };

    // ---- unpack of one staged activation tile into int8 halves -------------
    // lane j of the workgroup (512) takes 8 packed bytes: chunk j / 2 (row
    // chunk / 4, chunk % 4), half j % 2
    const int uj = wave * 64 + lane;
    const int uchunk = uj >> 1, uhalf = uj & 1;
    auto unpack_a = [&](int i, int buf) {
        const uint8_t* st = lds + (i % D) * kD64Stage;
        const uint2 w = *reinterpret_cast<const uint2*>(st + uchunk * 16 + uhalf * 8);
        const uint2 ev = make_uint2((w.x << 4) & 0xF0F0F0F0u, (w.y << 4) & 0xF0F0F0F0u);
        const uint2 od = make_uint2(w.x & 0xF0F0F0F0u, w.y & 0xF0F0F0F0u);
        uint8_t* ab = a8 + buf * 2 * kD64Half;
        *reinterpret_cast<uint2*>(ab + uchunk * 16 + uhalf * 8) = ev;
        *reinterpret_cast<uint2*>(ab + kD64Half + uchunk * 16 + uhalf * 8) = od;
    };

    // per-channel zero point of this lane's column (read before any copy)
    const int ncol = min(n0 + 16 * wave + frow, N - 1);
    uint32_t zb_chan = 0x80808080u;
    if constexpr (ASYM && !G1) zb_chan = (0x80u - static_cast<uint32_t>(h2f(z_w[ncol]))) * 0x01010101u;

    v4i acc[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) acc[a] = v4i{0, 0, 0, 0};
    float facc[G1 ? 4 : 1][4];
#pragma unroll
    for (int a = 0; a < (G1 ? 4 : 1); ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) facc[a][r] = 0.0f;
    v4i zc;
    {
        int z0;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z0));
        zc = v4i{z0, z0, z0, z0};
    }
    const int brow = 16 * wave + frow;                      // the lane's weight row in the tile
    const uint32_t spar = static_cast<uint32_t>(ncol) * static_cast<uint32_t>(G);

    if (nt > 0) {
        // prologue: tiles 0 .. D-2 in flight; tile 0 landed and unpacked
        for (int i = 0; i < D - 1; ++i) issue(i);
        wait_vmcnt<(D - 2) * 2>();
        lds_barrier();
        unpack_a(0, 0);
        for (int i = 0; i < nt; ++i) {
            // tile i + 1 has landed once at most D - 3 newer tiles' copies are
            // outstanding; after the barrier every wave's copies of it are
            // visible, every read of tile i - 1's stage is done, and the
            // unpacked tile i (written before the barrier) is visible
            wait_vmcnt<WAITN>();
            lds_barrier();
            issue(i + D - 1);
            if (i + 1 < nt) unpack_a(i + 1, (i + 1) & 1);
            const uint8_t* st = lds + (i % D) * kD64Stage;
            const uint8_t* ab = a8 + (i & 1) * 2 * kD64Half;
            const uint4 wb = *reinterpret_cast<const uint4*>(st + kD64A + brow * 64 + fks * 16);
            uint32_t zbias = zb_chan;
            float sw = 0.0f;
            if constexpr (G1) {
                const uint8_t* szs = st + kD64A + kD64B;
                const uint32_t sh = 16u * ((spar + static_cast<uint32_t>(kt0 + i)) & 1u);
                const int so = (brow >> 6) * 256 + 4 * (brow & 63);
                sw = h2f(static_cast<uint16_t>(*reinterpret_cast<const uint32_t*>(szs + so) >> sh));
                if constexpr (ASYM) {
                    const uint16_t zh = static_cast<uint16_t>(
                        *reinterpret_cast<const uint32_t*>(szs + 512 + so) >> sh);
                    zbias = (0x80u - static_cast<uint32_t>(h2f(zh))) * 0x01010101u;
                }
            }
            uint4 bev, bod;
            if constexpr (ASYM)
                unpack_asym(wb, zbias, bev, bod);
            else
                unpack_signed16(wb, bev, bod);
            const v4i be = v4i{static_cast<int>(bev.x), static_cast<int>(bev.y), static_cast<int>(bev.z), static_cast<int>(bev.w)};
            const v4i bo = v4i{static_cast<int>(bod.x), static_cast<int>(bod.y), static_cast<int>(bod.z), static_cast<int>(bod.w)};
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int ao = ((16 * a + frow) * 4 + fks) * 16;
                const v4i ae = *reinterpret_cast<const v4i*>(ab + ao);
                const v4i aod = *reinterpret_cast<const v4i*>(ab + kD64Half + ao);
                if constexpr (G1) {
                    v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(ae, be, zc, 0, 0, 0);
                    p = __builtin_amdgcn_mfma_i32_16x16x64_i8(aod, bo, p, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) facc[a][r] = fmaf(static_cast<float>(p[r]), sw, facc[a][r]);
                } else {
                    acc[a] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ae, be, acc[a], 0, 0, 0);
                    acc[a] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aod, bo, acc[a], 0, 0, 0);
                }
            }
        }
        // retire the clamped copies still in flight before the workgroup ends
        wait_vmcnt<0>();
    }

    // ---- this range's sums: lane (g, li) holds rows 16 a + 4 g + r, column li
    const int gn = n0 + 16 * wave + frow;
    if (gn < N) {
        int32_t* pr = part + static_cast<size_t>(blockIdx.y) * M * N;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int gm = 16 * a + 4 * fks + r;
                if (gm < M)
                    pr[static_cast<size_t>(gm) * N + gn] =
                        G1 ? __float_as_int(facc[a][r]) : acc[a][r];
            }
    }
}

// Y = fp16(s_x[m] * unshift * (sum of the ranges' sums, in range order)
//          [* s_w[n] per channel])
template <bool ASYM, bool G1>
__global__ __launch_bounds__(256) void k_dec64_reduce(const int32_t* __restrict__ part,
                                                      const float* __restrict__ s_x,
                                                      const uint16_t* __restrict__ s_w,
                                                      uint16_t* __restrict__ Y, int M, int N,
                                                      int splits) {
    const long e = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
    if (e >= static_cast<long>(M) * N) return;
    const int m = static_cast<int>(e / N);
    const int n = static_cast<int>(e - static_cast<long>(m) * N);
    constexpr float kUnshift = ASYM ? (1.0f / 16.0f) : (1.0f / 256.0f);
    float v;
    if constexpr (G1) {
        v = 0.0f;
        for (int sp = 0; sp < splits; ++sp) v += __int_as_float(part[static_cast<size_t>(sp) * M * N + e]);
    } else {
        int sum = 0;
        for (int sp = 0; sp < splits; ++sp) sum += part[static_cast<size_t>(sp) * M * N + e];
        v = static_cast<float>(sum) * h2f(s_w[n]);
    }
    Y[e] = f2h(v * s_x[m] * kUnshift);
}

template <bool ASYM, bool G1>
hipError_t launch_dec64_k(const GemmArgs& a, void* ws, hipStream_t stream) {
    auto* kern = &k_gemm_dec64<ASYM, G1>;
    static bool raised[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64 || !raised[dev]) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kD64Lds);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) raised[dev] = true;
    }
    const int KT = a.K / BK;
    const int kps = ceil_div(KT, kD64Split);
    int32_t* part = static_cast<int32_t*>(ws);
    kern<<<dim3(ceil_div(a.N, kD64Cols), kD64Split), dim3(kD64Waves * 64), kD64Lds, stream>>>(
        a.Xq, a.Wq, a.s_w, a.z_w, part, a.M, a.N, a.K, kps);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long total = static_cast<long>(a.M) * a.N;
    k_dec64_reduce<ASYM, G1><<<static_cast<unsigned>((total + 255) / 256), 256, 0, stream>>>(
        part, a.s_x, a.s_w, a.Y, a.M, a.N, kD64Split);
    return hipGetLastError();
}

// per channel or groups of one K tile only
bool dec64_supports(const GemmArgs& a) {
    const int G = a.K / a.group_size;
    return (G == 1 || a.group_size == BK) &&
           static_cast<size_t>(a.N) * static_cast<size_t>(G) < (size_t{1} << 31);
}

hipError_t launch_dec64(const GemmArgs& a, void* ws, hipStream_t stream) {
    const bool g1 = (a.K / a.group_size) > 1;
    if (a.asym)
        return g1 ? launch_dec64_k<true, true>(a, ws, stream) : launch_dec64_k<true, false>(a, ws, stream);
    return g1 ? launch_dec64_k<false, true>(a, ws, stream) : launch_dec64_k<false, false>(a, ws, stream);
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

// the split-K kernel (index kNumDec of the override): measured on MI355X for
// 64 tokens, 28672 -> 8192 in groups of 128 (see the K-loop comment there);
// taken automatically above 32 tokens where it applies
bool use_dec64(const GemmArgs& a) {
    if (!dec64_supports(a)) return false;
    const int o = kernel_override(1);
    if (o >= 0 && o <= kNumDec) return o == kNumDec;
    return a.M > 32;
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

size_t gemm_decode_workspace_bytes(int M, int N) {
    const size_t b = sizeof(int32_t) * kD64Split * static_cast<size_t>(M) * static_cast<size_t>(N);
    return (b + 255) & ~static_cast<size_t>(255);
}

const char* gemm_decode_kernel_name(const GemmArgs& a) {
    if (use_dec64(a)) return "k_gemm_dec64<64x128, waves 8, 6 stages, K split 4> + k_dec64_reduce";
    return choose_dec(a).name;
}

hipError_t gemm_decode_launch(const GemmArgs& a, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (a.M == 0) return hipSuccess;
    if (use_dec64(a)) {
        if (ws == nullptr || ws_bytes < gemm_decode_workspace_bytes(a.M, a.N)) return hipErrorInvalidValue;
        return launch_dec64(a, ws, stream);
    }
    const KernelCfg& k = choose_dec(a);
    return (a.K / a.group_size) > 1 ? k.group(a, stream) : k.chan(a, stream);
}

}  // namespace w4a4
