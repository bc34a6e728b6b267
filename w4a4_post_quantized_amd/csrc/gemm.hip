// INT4 x INT4 GEMM with int32 accumulation and a dequant epilogue.
//
// FlatQuant: Flatness Matters for LLM Quantization, section 核心思想: the
// layer is the product Q(XP) · Q(P^-1 W^T) of two quantized matrices.
// FRM-PTQ page, section 初步介绍 (codes with zero point z) and its
// multi-granularity group quantization (per-group weight scales).
// FPTQuant page, section 3. 伪动态残差缩放: a per-token scale commutes with a
// bias-free linear, so s_x[m] multiplies the integer product afterwards.
//
//   D[m,n,g] = Σ_{k in g} q_x[m,k] · (u[n,k] - z[n,g])     exact, int32
//   Y[m,n]   = fp16( s_x[m] · Σ_g s_w[n,g] · D[m,n,g] )     fp32 epilogue
//
// Design (gfx950):
//  * Operands are K-contiguous packed nibbles.  A workgroup of 4 waves owns a
//    BM x BN output tile and walks K in tiles of 128 codes (64 bytes a row),
//    so a K tile never straddles a weight group (group sizes are multiples
//    of 128).
//  * Global -> registers (16-byte loads) -> unpack -> int8 tiles in LDS,
//    double buffered: the loads of tile t+1 are in flight while the MFMAs of
//    tile t run, and one barrier per tile separates the buffers.
//  * Unpack keeps the nibble in the HIGH half of each byte for signed codes,
//    i.e. stores 16*q exactly (bytes (w & 0xF0) and (w << 4) & 0xF0): two
//    logic ops per 8 codes and no sign extension.  Asymmetric weights become
//    u - z in [-15, 15] (byte-wise (u + 0x80 - z) ^ 0x80).  The products are
//    then 256*q_x*q_w (sym) or 16*q_x*(u-z) (asym); the shift is undone
//    exactly (int) or folded into the fp32 scale (power of two).
//    |256 * K * 64| < 2^31 for K <= 65536 keeps int32 exact.
//  * Within a 32-code packed chunk the even codes land in one 16-byte int8
//    chunk and the odd codes in the next; A and B use the same order, so the
//    dot products are unchanged (a permutation of k inside the tile).
//  * 16-byte LDS chunks of a 128-byte row are XOR-swizzled by (row >> 1) & 7
//    so that the 16 rows one ds_read_b128 touches hit distinct banks.
//  * MFMA: v_mfma_i32_16x16x64_i8.  Lane l supplies 16 bytes of row (l & 15)
//    from k-slice (l >> 4) for A and for B; the result lane l holds rows
//    4*(l >> 4) + r, column l & 15.
#include <cstdlib>
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace w4a4 {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int BK = 128;          // codes per K tile
constexpr int ROWB = BK;         // int8 bytes per LDS row

// kModeChan: fp16 output, one weight scale per row (G == 1), scaled once at
// the end; kModeGroup: fp16 output, per-group fp32 rescale inside the K loop;
// kModeI32: exact int32 D per group.
enum Mode { kModeChan = 0, kModeGroup = 1, kModeI32 = 2 };

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// signed nibbles -> 16*q bytes; even codes in `ev`, odd codes in `od`
__device__ __forceinline__ void unpack_signed16(const uint4& w, uint4& ev, uint4& od) {
    ev.x = (w.x << 4) & 0xF0F0F0F0u;
    ev.y = (w.y << 4) & 0xF0F0F0F0u;
    ev.z = (w.z << 4) & 0xF0F0F0F0u;
    ev.w = (w.w << 4) & 0xF0F0F0F0u;
    od.x = w.x & 0xF0F0F0F0u;
    od.y = w.y & 0xF0F0F0F0u;
    od.z = w.z & 0xF0F0F0F0u;
    od.w = w.w & 0xF0F0F0F0u;
}

// unsigned nibbles u, zero point z -> bytes (u - z) as int8
__device__ __forceinline__ uint32_t usub(uint32_t u4, uint32_t bias) {
    return (u4 + bias) ^ 0x80808080u;
}
__device__ __forceinline__ void unpack_asym(const uint4& w, uint32_t bias, uint4& ev, uint4& od) {
    ev.x = usub(w.x & 0x0F0F0F0Fu, bias);
    ev.y = usub(w.y & 0x0F0F0F0Fu, bias);
    ev.z = usub(w.z & 0x0F0F0F0Fu, bias);
    ev.w = usub(w.w & 0x0F0F0F0Fu, bias);
    od.x = usub((w.x >> 4) & 0x0F0F0F0Fu, bias);
    od.y = usub((w.y >> 4) & 0x0F0F0F0Fu, bias);
    od.z = usub((w.z >> 4) & 0x0F0F0F0Fu, bias);
    od.w = usub((w.w >> 4) & 0x0F0F0F0Fu, bias);
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool ASYM, int MODE>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64) void k_gemm_w4a4(
    const uint8_t* __restrict__ Xq, const float* __restrict__ s_x,
    const uint8_t* __restrict__ Wq, const uint16_t* __restrict__ s_w,
    const uint16_t* __restrict__ z_w, uint16_t* __restrict__ Y, int32_t* __restrict__ D,
    int M, int N, int K, int group_size) {
    constexpr int kThreads = WAVES_M * WAVES_N * 64;
    constexpr int WM = BM / WAVES_M;
    constexpr int WN = BN / WAVES_N;
    constexpr int FM = WM / 16;
    constexpr int FN = WN / 16;
    constexpr int ALD = (BM * 4 + kThreads - 1) / kThreads;   // 16-byte packed chunks per thread
    constexpr int BLD = (BN * 4 + kThreads - 1) / kThreads;
    static_assert(ALD >= 1 && BLD >= 1, "tile too small for the loader");
    constexpr int TILE_BYTES = (BM + BN) * ROWB;

    __shared__ __align__(16) uint8_t smem[2 * TILE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave / WAVES_N) * WM;
    const int wn0 = (wave % WAVES_N) * WN;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int KB = K / 2;               // packed bytes per row
    const int KT = K / BK;
    const int G = K / group_size;
    const int TPG = group_size / BK;    // K tiles per group

    // ---- loader state -------------------------------------------------------
    uint4 ra[ALD], rb[BLD];
    uint32_t zb[ASYM ? BLD : 1];

    auto load_tile = [&](int kt) {
#pragma unroll
        for (int i = 0; i < ALD; ++i) {
            const int q = tid + i * kThreads;
            const int row = q >> 2, pc = q & 3;
            const int gm = m0 + row;
            if (q < BM * 4 && gm < M)
                ra[i] = *reinterpret_cast<const uint4*>(Xq + static_cast<size_t>(gm) * KB + kt * 64 + pc * 16);
            else
                ra[i] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < BLD; ++i) {
            const int q = tid + i * kThreads;
            const int row = q >> 2, pc = q & 3;
            const int gn = n0 + row;
            if (q < BN * 4 && gn < N) {
                rb[i] = *reinterpret_cast<const uint4*>(Wq + static_cast<size_t>(gn) * KB + kt * 64 + pc * 16);
                if constexpr (ASYM) {
                    const int g = (kt * BK) / group_size;
                    const uint32_t z = static_cast<uint32_t>(h2f(z_w[static_cast<size_t>(gn) * G + g]));
                    zb[i] = (0x80u - z) * 0x01010101u;
                }
            } else {
                rb[i] = make_uint4(0, 0, 0, 0);
                if constexpr (ASYM) zb[i] = 0x80808080u;
            }
        }
    };

    auto store_tile = [&](int buf) {
        uint8_t* As = smem + buf * TILE_BYTES;
        uint8_t* Bs = As + BM * ROWB;
#pragma unroll
        for (int i = 0; i < ALD; ++i) {
            const int q = tid + i * kThreads;
            if (q >= BM * 4) break;
            const int row = q >> 2, pc = q & 3;
            uint4 ev, od;
            unpack_signed16(ra[i], ev, od);
            *reinterpret_cast<uint4*>(As + row * ROWB + swz(row, 2 * pc) * 16) = ev;
            *reinterpret_cast<uint4*>(As + row * ROWB + swz(row, 2 * pc + 1) * 16) = od;
        }
#pragma unroll
        for (int i = 0; i < BLD; ++i) {
            const int q = tid + i * kThreads;
            if (q >= BN * 4) break;
            const int row = q >> 2, pc = q & 3;
            uint4 ev, od;
            if constexpr (ASYM)
                unpack_asym(rb[i], zb[i], ev, od);
            else
                unpack_signed16(rb[i], ev, od);
            *reinterpret_cast<uint4*>(Bs + row * ROWB + swz(row, 2 * pc) * 16) = ev;
            *reinterpret_cast<uint4*>(Bs + row * ROWB + swz(row, 2 * pc + 1) * 16) = od;
        }
    };

    // ---- accumulators -------------------------------------------------------
    v4i acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) acc[a][b] = v4i{0, 0, 0, 0};
    float facc[(MODE == kModeGroup) ? FM : 1][(MODE == kModeGroup) ? FN : 1][4];
    if constexpr (MODE == kModeGroup) {
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) facc[a][b][r] = 0.0f;
    }

    const int frow = lane & 15;      // fragment row supplied by this lane
    const int fks = lane >> 4;       // k-slice supplied by this lane
    const int orow = 4 * (lane >> 4);  // first output row held by this lane
    const int ocol = lane & 15;

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) load_tile(kt + 1);

        const uint8_t* As = smem + buf * TILE_BYTES;
        const uint8_t* Bs = As + BM * ROWB;
        // two MFMA k-steps of 64 codes; the fragments of step 1 are read
        // from LDS before the MFMAs of step 0 are issued
        v4i af[2][FM], bf[2][FN];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int ch = 4 * s + fks;
#pragma unroll
            for (int a = 0; a < FM; ++a) {
                const int row = wm0 + a * 16 + frow;
                af[s][a] = *reinterpret_cast<const v4i*>(As + row * ROWB + swz(row, ch) * 16);
            }
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const int row = wn0 + b * 16 + frow;
                bf[s][b] = *reinterpret_cast<const v4i*>(Bs + row * ROWB + swz(row, ch) * 16);
            }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int b = 0; b < FN; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[s][a], bf[s][b], acc[a][b],
                                                                     0, 0, 0);

        // ---- end of a weight group: fold (or emit) the exact int32 sums ----
        const bool group_end = ((kt + 1) % TPG) == 0;
        if (group_end && MODE != kModeChan) {
            const int g = kt / TPG;
            if constexpr (MODE == kModeI32) {
                constexpr int SH = ASYM ? 4 : 8;
#pragma unroll
                for (int a = 0; a < FM; ++a)
#pragma unroll
                    for (int b = 0; b < FN; ++b)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int gm = m0 + wm0 + a * 16 + orow + r;
                            const int gn = n0 + wn0 + b * 16 + ocol;
                            if (gm < M && gn < N)
                                D[(static_cast<size_t>(gm) * N + gn) * G + g] = acc[a][b][r] >> SH;
                            acc[a][b][r] = 0;
                        }
            } else if constexpr (MODE == kModeGroup) {
#pragma unroll
                for (int b = 0; b < FN; ++b) {
                    const int gn = n0 + wn0 + b * 16 + ocol;
                    const float sw = (gn < N) ? h2f(s_w[static_cast<size_t>(gn) * G + g]) : 0.0f;
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

        if (kt + 1 < KT) store_tile(buf ^ 1);
        __syncthreads();
    }

    if constexpr (MODE != kModeI32) {
        constexpr float kUnshift = ASYM ? (1.0f / 16.0f) : (1.0f / 256.0f);
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            const int gn = n0 + wn0 + b * 16 + ocol;
            if (gn >= N) continue;
            float sw1 = 1.0f;
            if constexpr (MODE == kModeChan) sw1 = h2f(s_w[gn]);
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int gm = m0 + wm0 + a * 16 + orow + r;
                    if (gm >= M) continue;
                    float v;
                    if constexpr (MODE == kModeChan)
                        v = static_cast<float>(acc[a][b][r]) * sw1;
                    else
                        v = facc[a][b][r];
                    v = v * s_x[gm] * kUnshift;
                    Y[static_cast<size_t>(gm) * N + gn] = f2h(v);
                }
        }
    }
}


// ===========================================================================
// Pipelined kernel (BM = 256, 4 or 8 waves): global loads run two K tiles
// ahead into two register staging sets; while the MFMAs of tile t run, the
// staged tile t+1 is unpacked into the other LDS buffer; both k-steps'
// fragments of tile t are read before its MFMAs; one barrier per tile.  The
// fp16 output tile is staged through LDS and written as full 16-byte row
// segments.
// ===========================================================================
template <int BN, int WAVES_N, bool ASYM, int MODE>
__global__ __launch_bounds__(2 * WAVES_N * 64) void k_gemm_pipe(
    const uint8_t* __restrict__ Xq, const float* __restrict__ s_x,
    const uint8_t* __restrict__ Wq, const uint16_t* __restrict__ s_w,
    const uint16_t* __restrict__ z_w, uint16_t* __restrict__ Y, int M, int N, int K,
    int group_size) {
    constexpr int BM = 256;
    constexpr int WAVES_M = 2;
    constexpr int NT = WAVES_M * WAVES_N * 64;
    constexpr int WM = BM / WAVES_M;
    constexpr int WN = BN / WAVES_N;
    constexpr int FM = WM / 16;
    constexpr int FN = WN / 16;
    constexpr int ALD = (BM * 4 + NT - 1) / NT;
    constexpr int BLD = (BN * 4 + NT - 1) / NT;
    constexpr int TILE_BYTES = (BM + BN) * ROWB;
    static_assert(2 * TILE_BYTES >= BM * BN * 2, "output staging must fit the tile buffers");
    static_assert(MODE != kModeI32, "fp16 output modes only");

    __shared__ __align__(16) uint8_t smem[2 * TILE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave / WAVES_N) * WM;
    const int wn0 = (wave % WAVES_N) * WN;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int KB = K / 2;
    const int KT = K / BK;
    const int G = K / group_size;
    const int TPG = group_size / BK;

    uint4 ra[2][ALD], rb[2][BLD];
    uint32_t zb[2][ASYM ? BLD : 1];

    auto load_tile = [&](int kt, auto SET) {
        constexpr int S = decltype(SET)::value;
#pragma unroll
        for (int i = 0; i < ALD; ++i) {
            const int q = tid + i * NT;
            const int row = q >> 2, pc = q & 3;
            const int gm = m0 + row;
            if (q < BM * 4 && gm < M)
                ra[S][i] = *reinterpret_cast<const uint4*>(Xq + static_cast<size_t>(gm) * KB + kt * 64 + pc * 16);
            else
                ra[S][i] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < BLD; ++i) {
            const int q = tid + i * NT;
            const int row = q >> 2, pc = q & 3;
            const int gn = n0 + row;
            if (q < BN * 4 && gn < N) {
                rb[S][i] = *reinterpret_cast<const uint4*>(Wq + static_cast<size_t>(gn) * KB + kt * 64 + pc * 16);
                if constexpr (ASYM) {
                    const int g = (kt * BK) / group_size;
                    const uint32_t z = static_cast<uint32_t>(h2f(z_w[static_cast<size_t>(gn) * G + g]));
                    zb[S][i] = (0x80u - z) * 0x01010101u;
                }
            } else {
                rb[S][i] = make_uint4(0, 0, 0, 0);
                if constexpr (ASYM) zb[S][i] = 0x80808080u;
            }
        }
    };

    auto store_tile = [&](int buf, auto SET) {
        constexpr int S = decltype(SET)::value;
        uint8_t* As = smem + buf * TILE_BYTES;
        uint8_t* Bs = As + BM * ROWB;
#pragma unroll
        for (int i = 0; i < ALD; ++i) {
            const int q = tid + i * NT;
            if (q >= BM * 4) break;
            const int row = q >> 2, pc = q & 3;
            uint4 ev, od;
            unpack_signed16(ra[S][i], ev, od);
            *reinterpret_cast<uint4*>(As + row * ROWB + swz(row, 2 * pc) * 16) = ev;
            *reinterpret_cast<uint4*>(As + row * ROWB + swz(row, 2 * pc + 1) * 16) = od;
        }
#pragma unroll
        for (int i = 0; i < BLD; ++i) {
            const int q = tid + i * NT;
            if (q >= BN * 4) break;
            const int row = q >> 2, pc = q & 3;
            uint4 ev, od;
            if constexpr (ASYM)
                unpack_asym(rb[S][i], zb[S][i], ev, od);
            else
                unpack_signed16(rb[S][i], ev, od);
            *reinterpret_cast<uint4*>(Bs + row * ROWB + swz(row, 2 * pc) * 16) = ev;
            *reinterpret_cast<uint4*>(Bs + row * ROWB + swz(row, 2 * pc + 1) * 16) = od;
        }
    };

    v4i acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) acc[a][b] = v4i{0, 0, 0, 0};
    float facc[(MODE == kModeGroup) ? FM : 1][(MODE == kModeGroup) ? FN : 1][4];
    if constexpr (MODE == kModeGroup) {
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) facc[a][b][r] = 0.0f;
    }

    const int frow = lane & 15;
    const int fks = lane >> 4;
    const int orow = 4 * (lane >> 4);
    const int ocol = lane & 15;

    auto body = [&](int kt, auto SET) {
        constexpr int S = decltype(SET)::value;        // == kt & 1
        const uint8_t* As = smem + S * TILE_BYTES;
        const uint8_t* Bs = As + BM * ROWB;
        auto read_frags = [&](int step, v4i* af, v4i* bf) {
#pragma unroll
            for (int a = 0; a < FM; ++a) {
                const int row = wm0 + a * 16 + frow;
                af[a] = *reinterpret_cast<const v4i*>(As + row * ROWB + swz(row, 4 * step + fks) * 16);
            }
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const int row = wn0 + b * 16 + frow;
                bf[b] = *reinterpret_cast<const v4i*>(Bs + row * ROWB + swz(row, 4 * step + fks) * 16);
            }
        };
        auto mfmas = [&](const v4i* af, const v4i* bf) {
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int b = 0; b < FN; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[a], bf[b], acc[a][b], 0, 0, 0);
        };
        v4i af[FM], bf[FN];
        read_frags(0, af, bf);
        // tile kt+2 -> staging set S (its previous content, tile kt, is in LDS)
        if (kt + 2 < KT) load_tile(kt + 2, std::integral_constant<int, S>{});
        // staged tile kt+1 -> the other LDS buffer (read last in iteration kt-1)
        if (kt + 1 < KT) store_tile(S ^ 1, std::integral_constant<int, S ^ 1>{});
        mfmas(af, bf);
        read_frags(1, af, bf);
        mfmas(af, bf);
        if constexpr (MODE == kModeGroup) {
            if (((kt + 1) % TPG) == 0) {
                const int g = kt / TPG;
#pragma unroll
                for (int b = 0; b < FN; ++b) {
                    const int gn = n0 + wn0 + b * 16 + ocol;
                    const float sw = (gn < N) ? h2f(s_w[static_cast<size_t>(gn) * G + g]) : 0.0f;
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
        __syncthreads();
    };

    load_tile(0, std::integral_constant<int, 0>{});
    if (KT > 1) load_tile(1, std::integral_constant<int, 1>{});
    store_tile(0, std::integral_constant<int, 0>{});
    __syncthreads();
    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {
        body(kt, std::integral_constant<int, 0>{});
        body(kt + 1, std::integral_constant<int, 1>{});
    }
    if (kt < KT) body(kt, std::integral_constant<int, 0>{});

    // ---- epilogue: fp16 tile staged in LDS, written as 16-byte row pieces ----
    constexpr float kUnshift = ASYM ? (1.0f / 16.0f) : (1.0f / 256.0f);
    uint16_t* Ys = reinterpret_cast<uint16_t*>(smem);       // [BM][BN] fp16
#pragma unroll
    for (int b = 0; b < FN; ++b) {
        const int cl = wn0 + b * 16 + ocol;
        const int gn = n0 + cl;
        float sw1 = 0.0f;
        if constexpr (MODE == kModeChan) sw1 = (gn < N) ? h2f(s_w[gn]) : 0.0f;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rl = wm0 + a * 16 + orow + r;
                const int gm = m0 + rl;
                const float sx = (gm < M) ? s_x[gm] : 0.0f;
                float v;
                if constexpr (MODE == kModeChan)
                    v = static_cast<float>(acc[a][b][r]) * sw1;
                else
                    v = facc[a][b][r];
                Ys[rl * BN + cl] = f2h(v * sx * kUnshift);
            }
    }
    __syncthreads();
    constexpr int CPR = BN / 8;            // 16-byte pieces per row
    for (int c = tid; c < BM * CPR; c += NT) {
        const int rl = c / CPR;
        const int cc = c - rl * CPR;
        const int gm = m0 + rl;
        const int gn = n0 + cc * 8;
        if (gm >= M) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(Ys + rl * BN + cc * 8);
        uint16_t* dst = Y + static_cast<size_t>(gm) * N + gn;
        if (gn + 8 <= N && (N & 7) == 0) {
            *reinterpret_cast<uint4*>(dst) = v;
        } else {
            const uint16_t* pv = reinterpret_cast<const uint16_t*>(&v);
            for (int j = 0; j < 8 && gn + j < N; ++j) dst[j] = pv[j];
        }
    }
}

template <int BN, int WAVES_N, int MODE>
hipError_t launch_pipe(const GemmArgs& a, hipStream_t stream) {
    dim3 grid(ceil_div(a.N, BN), ceil_div(a.M, 256));
    dim3 block(2 * WAVES_N * 64);
    if (a.asym)
        k_gemm_pipe<BN, WAVES_N, true, MODE><<<grid, block, 0, stream>>>(
            a.Xq, a.s_x, a.Wq, a.s_w, a.z_w, a.Y, a.M, a.N, a.K, a.group_size);
    else
        k_gemm_pipe<BN, WAVES_N, false, MODE><<<grid, block, 0, stream>>>(
            a.Xq, a.s_x, a.Wq, a.s_w, a.z_w, a.Y, a.M, a.N, a.K, a.group_size);
    return hipGetLastError();
}


// ===========================================================================
// 32x32x32 kernel: same data flow as k_gemm_w4a4 (packed tiles -> registers
// -> unpacked int8 in double-buffered LDS, one barrier per 128-code K tile),
// on v_mfma_i32_32x32x32_i8, which sustains ~96% of the int8 peak on gfx950
// where the 16x16x64 form measures ~78%.  Lane l supplies 16 bytes of row
// (l & 31) from k-slice (l >> 5); a K tile is 4 MFMA k-steps, k-step s using
// the even- and odd-code chunks of packed chunk s.  Accumulator register r of
// lane l holds row 8*(r >> 2) + 4*(l >> 5) + (r & 3), column l & 31.
// ===========================================================================
typedef int v16i __attribute__((ext_vector_type(16)));

// Interleaving pattern for the scheduler, one step per MFMA: the MFMA, then
// an even share of the remaining LDS reads, VALU instructions and LDS writes.
template <int NMF, int NRD, int NVALU, int NWR, int I = 0>
__device__ __forceinline__ void il_sched() {
    if constexpr (I < NMF) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
        constexpr int rd = (I + 1) * NRD / NMF - I * NRD / NMF;
        if constexpr (rd > 0) __builtin_amdgcn_sched_group_barrier(0x100, rd, 0);   // DS read
        constexpr int va = (I + 1) * NVALU / NMF - I * NVALU / NMF;
        if constexpr (va > 0) __builtin_amdgcn_sched_group_barrier(0x002, va, 0);   // VALU
        constexpr int wr = (I + 1) * NWR / NMF - I * NWR / NMF;
        if constexpr (wr > 0) __builtin_amdgcn_sched_group_barrier(0x200, wr, 0);   // DS write
        il_sched<NMF, NRD, NVALU, NWR, I + 1>();
    }
}


template <int BM, int BN, int WAVES_M, int WAVES_N, int PD, bool ASYM, int MODE, bool IL = false>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64) void k_gemm32(
    const uint8_t* __restrict__ Xq, const float* __restrict__ s_x,
    const uint8_t* __restrict__ Wq, const uint16_t* __restrict__ s_w,
    const uint16_t* __restrict__ z_w, uint16_t* __restrict__ Y, int M, int N, int K,
    int group_size) {
    constexpr int NT = WAVES_M * WAVES_N * 64;
    constexpr int WM = BM / WAVES_M;
    constexpr int WN = BN / WAVES_N;
    constexpr int FM = WM / 32;
    constexpr int FN = WN / 32;
    static_assert(FM >= 1 && FN >= 1 && WM % 32 == 0 && WN % 32 == 0, "wave tile");
    static_assert(PD >= 1 && PD <= 4, "prefetch depth");
    constexpr int ALD = (BM * 4 + NT - 1) / NT;
    constexpr int BLD = (BN * 4 + NT - 1) / NT;
    constexpr int TILE_BYTES = (BM + BN) * ROWB;
    static_assert(MODE != kModeI32, "fp16 output modes only");

    __shared__ __align__(16) uint8_t smem[2 * TILE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave / WAVES_N) * WM;
    const int wn0 = (wave % WAVES_N) * WN;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int KB = K / 2;
    const int KT = K / BK;
    const int G = K / group_size;
    const int TPG = group_size / BK;

    // PD register staging sets: the packed tile kt+PD is loaded while tile kt
    // is multiplied, so each load has about PD-1 iterations to arrive.  Loads
    // are branch-free (rows and tiles are clamped to valid ones; a clamped row
    // only feeds outputs that are never stored), which lets the compiler wait
    // for exactly the tile it unpacks instead of draining all loads.
    static_assert((BM * 4) % NT == 0 && (BN * 4) % NT == 0, "whole 16-byte chunks per thread");
    uint4 ra[PD][ALD], rb[PD][BLD];
    uint32_t zb[PD][ASYM ? BLD : 1];
    const uint8_t* arow[ALD];
    const uint8_t* brow[BLD];
    int bgn[BLD];
#pragma unroll
    for (int i = 0; i < ALD; ++i) {
        const int q = tid + i * NT;
        const int gm = min(m0 + (q >> 2), M - 1);
        arow[i] = Xq + static_cast<size_t>(gm) * KB + (q & 3) * 16;
    }
#pragma unroll
    for (int i = 0; i < BLD; ++i) {
        const int q = tid + i * NT;
        bgn[i] = min(n0 + (q >> 2), N - 1);
        brow[i] = Wq + static_cast<size_t>(bgn[i]) * KB + (q & 3) * 16;
    }

    auto load_tile = [&](int kt, auto SET) {
        constexpr int S = decltype(SET)::value;
        const int kc = min(kt, KT - 1);
#pragma unroll
        for (int i = 0; i < ALD; ++i) ra[S][i] = *reinterpret_cast<const uint4*>(arow[i] + kc * 64);
#pragma unroll
        for (int i = 0; i < BLD; ++i) {
            rb[S][i] = *reinterpret_cast<const uint4*>(brow[i] + kc * 64);
            if constexpr (ASYM) {
                const int g = (kc * BK) / group_size;
                const uint32_t z = static_cast<uint32_t>(h2f(z_w[static_cast<size_t>(bgn[i]) * G + g]));
                zb[S][i] = (0x80u - z) * 0x01010101u;
            }
        }
    };

    auto store_tile = [&](int buf, auto SET) {
        constexpr int S = decltype(SET)::value;
        uint8_t* As = smem + buf * TILE_BYTES;
        uint8_t* Bs = As + BM * ROWB;
#pragma unroll
        for (int i = 0; i < ALD; ++i) {
            const int q = tid + i * NT;
            const int row = q >> 2, pc = q & 3;
            uint4 ev, od;
            unpack_signed16(ra[S][i], ev, od);
            *reinterpret_cast<uint4*>(As + row * ROWB + swz(row, 2 * pc) * 16) = ev;
            *reinterpret_cast<uint4*>(As + row * ROWB + swz(row, 2 * pc + 1) * 16) = od;
        }
#pragma unroll
        for (int i = 0; i < BLD; ++i) {
            const int q = tid + i * NT;
            const int row = q >> 2, pc = q & 3;
            uint4 ev, od;
            if constexpr (ASYM)
                unpack_asym(rb[S][i], zb[S][i], ev, od);
            else
                unpack_signed16(rb[S][i], ev, od);
            *reinterpret_cast<uint4*>(Bs + row * ROWB + swz(row, 2 * pc) * 16) = ev;
            *reinterpret_cast<uint4*>(Bs + row * ROWB + swz(row, 2 * pc + 1) * 16) = od;
        }
    };

    v16i acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;
    float facc[(MODE == kModeGroup) ? FM : 1][(MODE == kModeGroup) ? FN : 1][16];
    if constexpr (MODE == kModeGroup) {
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) facc[a][b][r] = 0.0f;
    }

    const int frow = lane & 31;
    const int fks = lane >> 5;
    const int ocol = lane & 31;
    const int orow = 4 * (lane >> 5);

    // one K tile: tile kt is in LDS buffer kt & 1 and came from set kt % PD
    auto body = [&](int kt, auto SET) {
        constexpr int S = decltype(SET)::value;
        constexpr int SN = (S + 1) % PD;       // set holding tile kt + 1
        const int buf = kt & 1;
        load_tile(kt + PD, std::integral_constant<int, S>{});
        const uint8_t* As = smem + buf * TILE_BYTES;
        const uint8_t* Bs = As + BM * ROWB;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int ch = 2 * st + fks;
            v4i af[FM], bf[FN];
#pragma unroll
            for (int a = 0; a < FM; ++a) {
                const int row = wm0 + a * 32 + frow;
                af[a] = *reinterpret_cast<const v4i*>(As + row * ROWB + swz(row, ch) * 16);
            }
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const int row = wn0 + b * 32 + frow;
                bf[b] = *reinterpret_cast<const v4i*>(Bs + row * ROWB + swz(row, ch) * 16);
            }
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int b = 0; b < FN; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[a], bf[b], acc[a][b], 0, 0, 0);
        }
        if constexpr (MODE == kModeGroup) {
            if (((kt + 1) % TPG) == 0) {
                const int g = kt / TPG;
#pragma unroll
                for (int b = 0; b < FN; ++b) {
                    const int gn = n0 + wn0 + b * 32 + ocol;
                    const float sw = (gn < N) ? h2f(s_w[static_cast<size_t>(gn) * G + g]) : 0.0f;
#pragma unroll
                    for (int a = 0; a < FM; ++a)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            facc[a][b][r] = fmaf(static_cast<float>(acc[a][b][r]), sw, facc[a][b][r]);
                            acc[a][b][r] = 0;
                        }
                }
            }
        }
        // the last iteration stores a clamped duplicate that nobody reads
        store_tile(buf ^ 1, std::integral_constant<int, SN>{});
        if constexpr (IL) {
            // Instruction interleaving for the scheduler: the fragment reads of
            // k-step 0 and the global loads first, then every MFMA followed by
            // a share of the remaining LDS reads, the unpack VALU work and the
            // LDS writes of the next tile, so the MFMA pipe stays fed while
            // the wave does its other work.
            constexpr int NMF = 4 * FM * FN;              // MFMAs per tile
            constexpr int NRD = 4 * (FM + FN);            // fragment reads per tile
            constexpr int NWR = 2 * (ALD + BLD);          // LDS writes per tile
            constexpr int NVALU = 10 * (ALD + BLD);       // unpack + address VALU (approx.)
            constexpr int NVM = ALD + BLD + (ASYM ? BLD : 0);
            __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);   // DS read
            __builtin_amdgcn_sched_group_barrier(0x020, NVM, 0);       // VMEM read
            il_sched<NMF, NRD - FM - FN, NVALU, NWR>();
        }
        __syncthreads();
    };

    // prologue: tiles 0 .. PD-1 in flight, tile 0 unpacked into buffer 0
    load_tile(0, std::integral_constant<int, 0>{});
    if constexpr (PD > 1) load_tile(1, std::integral_constant<int, 1 % PD>{});
    if constexpr (PD > 2) load_tile(2, std::integral_constant<int, 2 % PD>{});
    if constexpr (PD > 3) load_tile(3, std::integral_constant<int, 3 % PD>{});
    store_tile(0, std::integral_constant<int, 0>{});
    __syncthreads();

    int kt = 0;
    for (; kt + PD <= KT; kt += PD) {
        body(kt, std::integral_constant<int, 0>{});
        if constexpr (PD > 1) body(kt + 1, std::integral_constant<int, 1 % PD>{});
        if constexpr (PD > 2) body(kt + 2, std::integral_constant<int, 2 % PD>{});
        if constexpr (PD > 3) body(kt + 3, std::integral_constant<int, 3 % PD>{});
    }
    if (kt < KT) body(kt, std::integral_constant<int, 0>{});
    if constexpr (PD > 2) if (kt + 1 < KT) body(kt + 1, std::integral_constant<int, 1 % PD>{});
    if constexpr (PD > 3) if (kt + 2 < KT) body(kt + 2, std::integral_constant<int, 2 % PD>{});

    constexpr float kUnshift = ASYM ? (1.0f / 16.0f) : (1.0f / 256.0f);
#pragma unroll
    for (int b = 0; b < FN; ++b) {
        const int gn = n0 + wn0 + b * 32 + ocol;
        if (gn >= N) continue;
        float sw1 = 1.0f;
        if constexpr (MODE == kModeChan) sw1 = h2f(s_w[gn]);
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gm = m0 + wm0 + a * 32 + 8 * (r >> 2) + orow + (r & 3);
                if (gm >= M) continue;
                float v;
                if constexpr (MODE == kModeChan)
                    v = static_cast<float>(acc[a][b][r]) * sw1;
                else
                    v = facc[a][b][r];
                Y[static_cast<size_t>(gm) * N + gn] = f2h(v * s_x[gm] * kUnshift);
            }
    }
}

template <int BM, int BN, int WM_, int WN_, int PD, int MODE, bool IL = false>
hipError_t launch32(const GemmArgs& a, hipStream_t stream) {
    dim3 grid(ceil_div(a.N, BN), ceil_div(a.M, BM));
    dim3 block(WM_ * WN_ * 64);
    if (a.asym)
        k_gemm32<BM, BN, WM_, WN_, PD, true, MODE, IL><<<grid, block, 0, stream>>>(
            a.Xq, a.s_x, a.Wq, a.s_w, a.z_w, a.Y, a.M, a.N, a.K, a.group_size);
    else
        k_gemm32<BM, BN, WM_, WN_, PD, false, MODE, IL><<<grid, block, 0, stream>>>(
            a.Xq, a.s_x, a.Wq, a.s_w, a.z_w, a.Y, a.M, a.N, a.K, a.group_size);
    return hipGetLastError();
}


// ===========================================================================
// Direct-to-LDS kernel.  Packed tiles go from HBM straight into a ring of
// STAGES LDS buffers with global_load_lds_dwordx4 (no VGPR staging, no VALU,
// no ds_write), STAGES-1 tiles in flight.  A packed row of a K tile is 64
// bytes (4 chunks of 32 codes); chunk c of row r sits at 16-byte slot
// c ^ (((r >> 1) ^ (r >> 3)) & 3), which keeps the 16 (or 8) rows one
// ds_read_b128 touches in distinct banks.  A lane reads one packed chunk and
// unpacks it into two 32x32x32 fragments: the even codes (low nibbles) for
// one k-step and the odd codes (high nibbles) for the next; A and B use the
// same order, so the products are those of the tile.  Signed codes are kept
// as 16*q (nibble in the high half of the byte); asymmetric weights become
// u - z.
// ===========================================================================
__device__ __forceinline__ int dl_slot(int row, int c) { return c ^ (((row >> 1) ^ (row >> 3)) & 3); }

// s_waitcnt with only a vmcnt condition (gfx9 encoding; expcnt and lgkmcnt
// left at their no-wait maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// 16-byte global -> LDS copy of one lane; the LDS address of lane l is
// lds_wave_base + 16 * l (the hardware adds the lane offset).
__device__ __forceinline__ void dma16(const void* src, uint8_t* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base,
                                     16, 0, 0);
}

// Workgroup barrier without a memory fence; the compiler-only fences keep
// LDS accesses from being moved across it.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, bool ASYM, int MODE>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64) void k_gemm_dl(
    const uint8_t* __restrict__ Xq, const float* __restrict__ s_x,
    const uint8_t* __restrict__ Wq, const uint16_t* __restrict__ s_w,
    const uint16_t* __restrict__ z_w, uint16_t* __restrict__ Y, int M, int N, int K,
    int group_size) {
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int NT = NW * 64;
    constexpr int WM = BM / WAVES_M;
    constexpr int WN = BN / WAVES_N;
    constexpr int FM = WM / 32;
    constexpr int FN = WN / 32;
    static_assert(FM >= 1 && FN >= 1 && WM % 32 == 0 && WN % 32 == 0, "wave tile");
    constexpr int PROW = 64;                          // packed bytes per tile row
    constexpr int STAGE_BYTES = (BM + BN) * PROW;
    constexpr int CHUNKS = (BM + BN) * 4;             // 16-byte chunks per tile
    static_assert(CHUNKS % (64 * NW) == 0 && (BM * 4) % 64 == 0, "whole wave loads");
    constexpr int LPW = CHUNKS / (64 * NW);           // load instructions per wave per tile
    static_assert(STAGES >= 3 && STAGES <= 4 && (STAGES - 2) * LPW < 64, "stages / vmcnt range");
    static_assert(MODE != kModeI32, "fp16 output modes only");

    // one LDS array per stage: distinct objects let the compiler see that
    // reads of one stage do not depend on the DMA writes into the others
    __shared__ __align__(16) uint8_t st0[STAGE_BYTES];
    __shared__ __align__(16) uint8_t st1[STAGE_BYTES];
    __shared__ __align__(16) uint8_t st2[STAGES > 2 ? STAGE_BYTES : 16];
    __shared__ __align__(16) uint8_t st3[STAGES > 3 ? STAGE_BYTES : 16];
    auto stage_ptr = [&](auto S) -> uint8_t* {
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
    const int KB = K / 2;
    const int KT = K / BK;
    const int G = K / group_size;
    const int TPG = group_size / BK;

    // this lane's source row (clamped) and chunk for each of its loads
    const uint8_t* src[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int j = (i * NW + wave) * 64 + lane;     // 16-byte slot in the stage
        const bool isA = j < BM * 4;
        const int jj = isA ? j : j - BM * 4;
        const int row = jj >> 2;
        const int c = (jj & 3) ^ (((row >> 1) ^ (row >> 3)) & 3);
        if (isA)
            src[i] = Xq + static_cast<size_t>(min(m0 + row, M - 1)) * KB + c * 16;
        else
            src[i] = Wq + static_cast<size_t>(min(n0 + row, N - 1)) * KB + c * 16;
    }
    auto issue = [&](int kt, auto S) {
        const int kc = min(kt, KT - 1);
        uint8_t* stage = stage_ptr(S);
#pragma unroll
        for (int i = 0; i < LPW; ++i)
            dma16(src[i] + kc * 64, stage + (i * NW + wave) * 1024);
    };

    v16i acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;
    float facc[(MODE == kModeGroup) ? FM : 1][(MODE == kModeGroup) ? FN : 1][16];
    if constexpr (MODE == kModeGroup) {
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) facc[a][b][r] = 0.0f;
    }

    const int frow = lane & 31;
    const int fks = lane >> 5;
    const int ocol = lane & 31;
    const int orow = 4 * (lane >> 5);
    // LDS byte offsets of this lane's fragments for chunk pair p (chunk 2p+fks)
    int aoff[2][FM], boff[2][FN];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
        for (int a = 0; a < FM; ++a) {
            const int row = wm0 + a * 32 + frow;
            aoff[p][a] = row * PROW + dl_slot(row, 2 * p + fks) * 16;
        }
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            const int row = wn0 + b * 32 + frow;
            boff[p][b] = BM * PROW + row * PROW + dl_slot(row, 2 * p + fks) * 16;
        }
    }
    int brow_g[FN];
#pragma unroll
    for (int b = 0; b < FN; ++b) brow_g[b] = min(n0 + wn0 + b * 32 + frow, N - 1);

    // one K tile: tile kt is in stage kt % STAGES; the DMA of tile
    // kt+STAGES-1 goes into the stage tile kt-1 used
    auto body = [&](int kt, auto S) {
        constexpr int SI = decltype(S)::value;
        issue(kt + STAGES - 1, std::integral_constant<int, (SI + STAGES - 1) % STAGES>{});
        const uint8_t* stage = stage_ptr(S);
        uint32_t zbias[FN];
        if constexpr (ASYM) {
            const int g = (kt * BK) / group_size;
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const uint32_t z = static_cast<uint32_t>(h2f(z_w[static_cast<size_t>(brow_g[b]) * G + g]));
                zbias[b] = (0x80u - z) * 0x01010101u;
            }
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            v4i alo[FM], ahi[FM], blo[FN], bhi[FN];
#pragma unroll
            for (int a = 0; a < FM; ++a) {
                const uint4 w = *reinterpret_cast<const uint4*>(stage + aoff[p][a]);
                uint4 ev, od;
                unpack_signed16(w, ev, od);
                alo[a] = v4i{static_cast<int>(ev.x), static_cast<int>(ev.y), static_cast<int>(ev.z), static_cast<int>(ev.w)};
                ahi[a] = v4i{static_cast<int>(od.x), static_cast<int>(od.y), static_cast<int>(od.z), static_cast<int>(od.w)};
            }
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const uint4 w = *reinterpret_cast<const uint4*>(stage + boff[p][b]);
                uint4 ev, od;
                if constexpr (ASYM)
                    unpack_asym(w, zbias[b], ev, od);
                else
                    unpack_signed16(w, ev, od);
                blo[b] = v4i{static_cast<int>(ev.x), static_cast<int>(ev.y), static_cast<int>(ev.z), static_cast<int>(ev.w)};
                bhi[b] = v4i{static_cast<int>(od.x), static_cast<int>(od.y), static_cast<int>(od.z), static_cast<int>(od.w)};
            }
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int b = 0; b < FN; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(alo[a], blo[b], acc[a][b], 0, 0, 0);
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int b = 0; b < FN; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ahi[a], bhi[b], acc[a][b], 0, 0, 0);
        }
        if constexpr (MODE == kModeGroup) {
            if (((kt + 1) % TPG) == 0) {
                const int g = kt / TPG;
#pragma unroll
                for (int b = 0; b < FN; ++b) {
                    const int gn = n0 + wn0 + b * 32 + ocol;
                    const float sw = (gn < N) ? h2f(s_w[static_cast<size_t>(gn) * G + g]) : 0.0f;
#pragma unroll
                    for (int a = 0; a < FM; ++a)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            facc[a][b][r] = fmaf(static_cast<float>(acc[a][b][r]), sw, facc[a][b][r]);
                            acc[a][b][r] = 0;
                        }
                }
            }
        }
        // tile kt+1 has landed once at most STAGES-2 tiles of this wave's
        // loads are outstanding; the barrier makes every wave's part visible
        // and retires the reads of stage kt before it is refilled.  A plain
        // s_barrier: a workgroup fence would also drain the newer DMA loads,
        // and every LDS read of this tile has already fed an MFMA.
        wait_vmcnt<(STAGES - 2) * LPW>();
        lds_barrier();
    };

    // prologue: tiles 0 .. STAGES-2 in flight; wait for tile 0
    issue(0, std::integral_constant<int, 0>{});
    issue(1, std::integral_constant<int, 1 % STAGES>{});
    if constexpr (STAGES > 3) issue(2, std::integral_constant<int, 2>{});
    wait_vmcnt<(STAGES - 2) * LPW>();
    lds_barrier();

    int kt = 0;
    for (; kt + STAGES <= KT; kt += STAGES) {
        body(kt, std::integral_constant<int, 0>{});
        body(kt + 1, std::integral_constant<int, 1>{});
        if constexpr (STAGES > 2) body(kt + 2, std::integral_constant<int, 2 % STAGES>{});
        if constexpr (STAGES > 3) body(kt + 3, std::integral_constant<int, 3 % STAGES>{});
    }
    if (kt < KT) body(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < KT) body(kt + 1, std::integral_constant<int, 1 % STAGES>{});
    if constexpr (STAGES > 3) if (kt + 2 < KT) body(kt + 2, std::integral_constant<int, 2 % STAGES>{});

    constexpr float kUnshift = ASYM ? (1.0f / 16.0f) : (1.0f / 256.0f);
#pragma unroll
    for (int b = 0; b < FN; ++b) {
        const int gn = n0 + wn0 + b * 32 + ocol;
        if (gn >= N) continue;
        float sw1 = 1.0f;
        if constexpr (MODE == kModeChan) sw1 = h2f(s_w[gn]);
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gm = m0 + wm0 + a * 32 + 8 * (r >> 2) + orow + (r & 3);
                if (gm >= M) continue;
                float v;
                if constexpr (MODE == kModeChan)
                    v = static_cast<float>(acc[a][b][r]) * sw1;
                else
                    v = facc[a][b][r];
                Y[static_cast<size_t>(gm) * N + gn] = f2h(v * s_x[gm] * kUnshift);
            }
    }
}

template <int BM, int BN, int WM_, int WN_, int ST, int MODE>
hipError_t launch_dl(const GemmArgs& a, hipStream_t stream) {
    dim3 grid(ceil_div(a.N, BN), ceil_div(a.M, BM));
    dim3 block(WM_ * WN_ * 64);
    if (a.asym)
        k_gemm_dl<BM, BN, WM_, WN_, ST, true, MODE><<<grid, block, 0, stream>>>(
            a.Xq, a.s_x, a.Wq, a.s_w, a.z_w, a.Y, a.M, a.N, a.K, a.group_size);
    else
        k_gemm_dl<BM, BN, WM_, WN_, ST, false, MODE><<<grid, block, 0, stream>>>(
            a.Xq, a.s_x, a.Wq, a.s_w, a.z_w, a.Y, a.M, a.N, a.K, a.group_size);
    return hipGetLastError();
}

template <int BM, int BN, int WM_, int WN_, int MODE>
hipError_t launch_mode(const GemmArgs& a, hipStream_t stream) {
    dim3 grid(ceil_div(a.N, BN), ceil_div(a.M, BM));
    dim3 block(WM_ * WN_ * 64);
    if (a.asym)
        k_gemm_w4a4<BM, BN, WM_, WN_, true, MODE><<<grid, block, 0, stream>>>(
            a.Xq, a.s_x, a.Wq, a.s_w, a.z_w, a.Y, a.D, a.M, a.N, a.K, a.group_size);
    else
        k_gemm_w4a4<BM, BN, WM_, WN_, false, MODE><<<grid, block, 0, stream>>>(
            a.Xq, a.s_x, a.Wq, a.s_w, a.z_w, a.Y, a.D, a.M, a.N, a.K, a.group_size);
    return hipGetLastError();
}

using LaunchFn = hipError_t (*)(const GemmArgs&, hipStream_t);

// Tile configurations (BM x BN, waves along M x N) for the fp16-output
// modes; index 0 is the default of each mode.
struct TileCfg {
    int bm, bn;
    LaunchFn chan, group;
};

#define W4A4_TILE(BM, BN, WM_, WN_)                                                     \
    TileCfg {                                                                          \
        BM, BN, &launch_mode<BM, BN, WM_, WN_, kModeChan>,                              \
            &launch_mode<BM, BN, WM_, WN_, kModeGroup>                                  \
    }
// tiles whose per-group fp32 accumulators do not fit the register file
#define W4A4_TILE_CHAN(BM, BN, WM_, WN_) \
    TileCfg { BM, BN, &launch_mode<BM, BN, WM_, WN_, kModeChan>, nullptr }

const TileCfg kTiles[] = {
    W4A4_TILE_CHAN(256, 256, 2, 4),
    W4A4_TILE_CHAN(256, 256, 2, 2),
    W4A4_TILE_CHAN(256, 192, 2, 4),
    W4A4_TILE(256, 128, 2, 4),
    W4A4_TILE(256, 128, 4, 2),
    W4A4_TILE(128, 256, 2, 4),
    W4A4_TILE(128, 128, 2, 2),
    W4A4_TILE(128, 128, 2, 4),
    TileCfg{256, 192, &launch_pipe<192, 2, kModeChan>, nullptr},
    TileCfg{256, 192, &launch_pipe<192, 4, kModeChan>, nullptr},
    TileCfg{256, 128, &launch_pipe<128, 2, kModeChan>, nullptr},
    TileCfg{256, 128, &launch_pipe<128, 4, kModeChan>, &launch_pipe<128, 4, kModeGroup>},
    // 32x32x32 kernels, prefetch depth 1..3
    TileCfg{256, 256, &launch32<256, 256, 2, 4, 1, kModeChan>, nullptr},
    TileCfg{256, 256, &launch32<256, 256, 2, 4, 2, kModeChan>, nullptr},
    TileCfg{256, 256, &launch32<256, 256, 2, 4, 3, kModeChan>, nullptr},
    TileCfg{256, 192, &launch32<256, 192, 2, 2, 1, kModeChan>, nullptr},
    TileCfg{256, 192, &launch32<256, 192, 2, 2, 2, kModeChan>, nullptr},
    TileCfg{256, 192, &launch32<256, 192, 2, 2, 3, kModeChan>, nullptr},
    TileCfg{256, 128, &launch32<256, 128, 4, 2, 1, kModeChan>, &launch32<256, 128, 4, 2, 1, kModeGroup>},
    TileCfg{256, 128, &launch32<256, 128, 4, 2, 2, kModeChan>, &launch32<256, 128, 4, 2, 2, kModeGroup>},
    TileCfg{256, 128, &launch32<256, 128, 4, 2, 3, kModeChan>, &launch32<256, 128, 4, 2, 3, kModeGroup>},
    TileCfg{128, 128, &launch32<128, 128, 2, 2, 2, kModeChan>, &launch32<128, 128, 2, 2, 2, kModeGroup>},
    TileCfg{128, 128, &launch32<128, 128, 2, 2, 3, kModeChan>, &launch32<128, 128, 2, 2, 3, kModeGroup>},
    // explicitly interleaved schedules
    TileCfg{256, 256, &launch32<256, 256, 2, 4, 3, kModeChan, true>, nullptr},
    TileCfg{256, 192, &launch32<256, 192, 2, 2, 3, kModeChan, true>, nullptr},
    TileCfg{256, 256, &launch32<256, 256, 2, 2, 2, kModeChan, true>, nullptr},
    TileCfg{256, 128, &launch32<256, 128, 4, 2, 2, kModeChan, true>, &launch32<256, 128, 4, 2, 2, kModeGroup, true>},
    TileCfg{128, 128, &launch32<128, 128, 2, 2, 3, kModeChan, true>, &launch32<128, 128, 2, 2, 3, kModeGroup, true>},
    // direct-to-LDS kernels (index 28..)
    TileCfg{256, 256, &launch_dl<256, 256, 2, 4, 3, kModeChan>, nullptr},
    TileCfg{256, 256, &launch_dl<256, 256, 2, 4, 4, kModeChan>, nullptr},
    TileCfg{256, 256, &launch_dl<256, 256, 2, 2, 4, kModeChan>, nullptr},
    TileCfg{256, 192, &launch_dl<256, 192, 2, 2, 4, kModeChan>, nullptr},
    TileCfg{256, 128, &launch_dl<256, 128, 4, 2, 4, kModeChan>, &launch_dl<256, 128, 4, 2, 4, kModeGroup>},
    TileCfg{256, 128, &launch_dl<256, 128, 2, 2, 4, kModeChan>, &launch_dl<256, 128, 2, 2, 4, kModeGroup>},
    TileCfg{128, 128, &launch_dl<128, 128, 2, 2, 4, kModeChan>, &launch_dl<128, 128, 2, 2, 4, kModeGroup>},
};
#undef W4A4_TILE
#undef W4A4_TILE_CHAN
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

// Developer override for tile sweeps and tests: W4A4_GEMM_TILE=<index into
// kTiles> (read at every call; out-of-range or unset means automatic).
int tile_override() {
    const char* e = getenv("W4A4_GEMM_TILE");
    if (e == nullptr || *e == '\0') return -1;
    const int v = atoi(e);
    return (v >= 0 && v < kNumTiles) ? v : -1;
}

}  // namespace

int gemm_num_tile_configs() { return kNumTiles; }

size_t gemm_workspace_bytes(int M, int N, int K, int group_size) {
    (void)M;
    (void)N;
    (void)K;
    (void)group_size;
    return 0;
}

hipError_t gemm_launch(const GemmArgs& a, bool i32_out, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
    (void)ws;
    (void)ws_bytes;
    if (a.M == 0) return hipSuccess;
    if (i32_out) return launch_mode<64, 64, 2, 2, kModeI32>(a, stream);
    const bool grouped = (a.K / a.group_size) > 1;
    if (a.M <= 64) {
        if (grouped) return launch_mode<64, 64, 2, 2, kModeGroup>(a, stream);
        return launch_mode<64, 64, 2, 2, kModeChan>(a, stream);
    }
    int t = tile_override();
    if (t < 0 || (grouped && kTiles[t].group == nullptr)) {
        // measured on MI355X: direct-to-LDS 256x256 tiles when the grid
        // covers the CUs several times over, direct-to-LDS 128x128 tiles for
        // about one wave of 256x256 tiles, 16x16x64 128x128 (8 waves) for the
        // per-group mode
        const int cus = device_cu_count();
        const long tiles256 = static_cast<long>(ceil_div(a.M, 256)) * ceil_div(a.N, 256);
        if (grouped)
            t = 7;
        else if (tiles256 >= 2L * cus)
            t = 29;     // direct-to-LDS 256x256, 8 waves, 4 stages
        else
            t = 34;     // direct-to-LDS 128x128, 4 waves, 4 stages
    }
    return grouped ? kTiles[t].group(a, stream) : kTiles[t].chan(a, stream);
}

}  // namespace w4a4
