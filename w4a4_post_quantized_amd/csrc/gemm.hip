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
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace w4a4 {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BK = 128;          // codes per K tile
constexpr int ROWB = BK;         // int8 bytes per LDS row

// kModeChan: fp16 output, one weight scale per row (G == 1), scaled once at
// the end; kModeGroup: fp16 output, per-group fp32 rescale inside the K loop;
// kModeI32: exact int32 D per group.
enum Mode { kModeChan = 0, kModeGroup = 1, kModeI32 = 2 };

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

template <int BM, int BN, int WAVES_M, int WAVES_N, bool ASYM, int MODE, bool G1 = false>
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

    // a zero accumulator operand the compiler cannot fold into an inline
    // constant (an MFMA with an inline-zero accumulator gave wrong sums)
    v4i zc;
    {
        int z0;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z0));
        zc = v4i{z0, z0, z0, z0};
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
        if constexpr (G1) {
            // one K tile per weight group: the group's sums start from a zero
            // register operand, so the accumulators need no clearing
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int b = 0; b < FN; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[0][a], bf[0][b], zc, 0, 0, 0);
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int b = 0; b < FN; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[1][a], bf[1][b], acc[a][b],
                                                                     0, 0, 0);
        } else {
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int a = 0; a < FM; ++a)
#pragma unroll
                    for (int b = 0; b < FN; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[s][a], bf[s][b],
                                                                         acc[a][b], 0, 0, 0);
        }

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
                            if constexpr (!G1) acc[a][b][r] = 0;
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

// XCD-aware tile order.  Workgroups are dispatched round-robin over the 8
// XCDs (workgroup L to XCD L % 8), each with its own L2.  The 1-D grid index
// is turned into a tile index t so that XCD x walks the contiguous range of
// tiles it owns, in the order its workgroups start; t runs down the M tiles
// of one column of N tiles first, so the workgroups an XCD holds at once share
// one or two weight panels (each weight panel is read into one L2 once) and
// reuse the activation panels, which stay in the L2s and the Infinity Cache.
constexpr int kXcds = 8;
__device__ __forceinline__ void xcd_tile(int L, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int T = tiles_m * tiles_n;
    const int per = T / kXcds, rem = T % kXcds;
    const int x = L % kXcds, local = L / kXcds;
    const int t = x < rem ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
    tn = t / tiles_m;
    tm = t - tn * tiles_m;
}

// s_waitcnt with only a vmcnt condition (gfx9 encoding; expcnt and lgkmcnt
// left at their no-wait maxima)
template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, bool ASYM, int MODE, bool G1 = false>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64) void k_gemm_dl(
    const uint8_t* __restrict__ Xq, const float* __restrict__ s_x,
    const uint8_t* __restrict__ Wq, const uint16_t* __restrict__ s_w,
    const uint16_t* __restrict__ z_w, uint16_t* __restrict__ Y, int M, int N, int K,
    int group_size) {
    constexpr int NW = WAVES_M * WAVES_N;
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
    // vector-memory ops a wave issues per tile besides its copies: the next
    // tile's scale (and zero point) per B fragment in one-tile-group mode
    constexpr int NSZ = G1 ? FN * (ASYM ? 2 : 1) : 0;
    constexpr int WAITN = (STAGES - 2) * LPW + (STAGES - 1) * NSZ;
    static_assert(STAGES >= 3 && STAGES <= 8 && WAITN < 64, "stages / vmcnt range");
    static_assert(MODE != kModeI32, "fp16 output modes only");
    static_assert(!G1 || MODE == kModeGroup, "one-tile groups: per-group mode");

    // one LDS array per stage: distinct objects let the compiler see that
    // reads of one stage do not depend on the DMA writes into the others
    __shared__ __align__(16) uint8_t st0[STAGE_BYTES];
    __shared__ __align__(16) uint8_t st1[STAGE_BYTES];
    __shared__ __align__(16) uint8_t st2[STAGES > 2 ? STAGE_BYTES : 16];
    __shared__ __align__(16) uint8_t st3[STAGES > 3 ? STAGE_BYTES : 16];
    __shared__ __align__(16) uint8_t st4[STAGES > 4 ? STAGE_BYTES : 16];
    __shared__ __align__(16) uint8_t st5[STAGES > 5 ? STAGE_BYTES : 16];
    __shared__ __align__(16) uint8_t st6[STAGES > 6 ? STAGE_BYTES : 16];
    __shared__ __align__(16) uint8_t st7[STAGES > 7 ? STAGE_BYTES : 16];
    auto stage_ptr = [&](auto S) -> uint8_t* {
        constexpr int I = decltype(S)::value;
        if constexpr (I == 0) return st0;
        else if constexpr (I == 1) return st1;
        else if constexpr (I == 2) return st2;
        else if constexpr (I == 3) return st3;
        else if constexpr (I == 4) return st4;
        else if constexpr (I == 5) return st5;
        else if constexpr (I == 6) return st6;
        else return st7;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave / WAVES_N) * WM;
    const int wn0 = (wave % WAVES_N) * WN;
    int tm, tn;
    xcd_tile(blockIdx.x, ceil_div(M, BM), ceil_div(N, BN), tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int KB = K / 2;
    const int KT = K / BK;
    const int G = K / group_size;
    const int TPG = group_size / BK;

    // this lane's source row (clamped) and chunk for each of its loads.
    // Symmetric weights: load i of a wave covers 64 consecutive slots, all in
    // A or all in B, so the copies take a wave-uniform base (the tile's first
    // row, scalar registers) and a 32-bit lane offset, issued from inline
    // assembly.  Asymmetric weights keep the builtin copies: their zero points
    // are loaded inside the K loop, and the compiler's waits for those loads
    // must count the copies.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    constexpr bool kBuiltinCopies = ASYM || G1;
    const uint8_t* src[kBuiltinCopies ? LPW : 1];
    uint32_t soff[kBuiltinCopies ? 1 : LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int j = (i * NW + wave_u) * 64 + lane;   // 16-byte slot in the stage
        const bool isA = (i * NW + wave_u) * 64 < BM * 4;
        const int jj = isA ? j : j - BM * 4;
        const int row = jj >> 2;
        const int c = (jj & 3) ^ (((row >> 1) ^ (row >> 3)) & 3);
        const int r = isA ? min(m0 + row, M - 1) : min(n0 + row, N - 1);
        if constexpr (kBuiltinCopies)
            src[i] = (isA ? Xq : Wq) + static_cast<size_t>(r) * KB + c * 16;
        else
            soff[i] = static_cast<uint32_t>(r - (isA ? m0 : n0)) * KB + c * 16;
    }
    auto issue = [&](int kt, auto S) {
        const int kc = min(kt, KT - 1);
        uint8_t* stage = stage_ptr(S);
        if constexpr (kBuiltinCopies) {
#pragma unroll
            for (int i = 0; i < LPW; ++i) dma16(src[i] + kc * 64, stage + (i * NW + wave) * 1024);
        } else {
            const uint8_t* xb = Xq + static_cast<size_t>(m0) * KB + kc * 64;
            const uint8_t* wb = Wq + static_cast<size_t>(n0) * KB + kc * 64;
#pragma unroll
            for (int i = 0; i < LPW; ++i)
                dma16_async_sv((i * NW + wave_u) * 64 < BM * 4 ? xb : wb, soff[i],
                               stage + (i * NW + wave) * 1024);
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

    // One-tile groups (group size 128): each K tile is one weight group.  The
    // tile's MFMA chain starts from a zero register operand and its exact
    // int32 sums are folded at once into the fp32 sums with the group's
    // scale, so no accumulator is ever cleared.  The lane's B row is its
    // output column (frow == ocol), so one scale and one zero point per B
    // fragment serve both the unpack and the fold; they are loaded one tile
    // ahead.  A zero made opaque to the compiler: an MFMA whose accumulator
    // operand was an inline-constant zero gave wrong sums.
    v16i zc16;
    const uint16_t* swp[G1 ? FN : 1];
    const uint16_t* zwp[G1 && ASYM ? FN : 1];
    uint16_t s_nx[G1 ? FN : 1], z_nx[G1 && ASYM ? FN : 1];
    if constexpr (G1) {
        int z0;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z0));
#pragma unroll
        for (int r = 0; r < 16; ++r) zc16[r] = z0;
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            swp[b] = s_w + static_cast<size_t>(brow_g[b]) * G;
            s_nx[b] = swp[b][0];
            if constexpr (ASYM) {
                zwp[b] = z_w + static_cast<size_t>(brow_g[b]) * G;
                z_nx[b] = zwp[b][0];
            }
        }
    }

    // one K tile: tile kt is in stage kt % STAGES; the DMA of tile
    // kt+STAGES-1 goes into the stage tile kt-1 used
    auto body = [&](int kt, auto S) {
        constexpr int SI = decltype(S)::value;
        issue(kt + STAGES - 1, std::integral_constant<int, (SI + STAGES - 1) % STAGES>{});
        const uint8_t* stage = stage_ptr(S);
        uint32_t zbias[FN];
        float sw_t[G1 ? FN : 1];
        if constexpr (G1) {
            // this tile's scale and zero point, then the next tile's loads
            const int kn = min(kt + 1, KT - 1);
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                sw_t[b] = h2f(s_nx[b]);
                if constexpr (ASYM) {
                    const uint32_t z = static_cast<uint32_t>(h2f(z_nx[b]));
                    zbias[b] = (0x80u - z) * 0x01010101u;
                }
                s_nx[b] = swp[b][kn];
                if constexpr (ASYM) z_nx[b] = zwp[b][kn];
            }
        } else if constexpr (ASYM) {
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
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                        alo[a], blo[b], (G1 && p == 0) ? zc16 : acc[a][b], 0, 0, 0);
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int b = 0; b < FN; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ahi[a], bhi[b], acc[a][b], 0, 0, 0);
        }
        if constexpr (G1) {
#pragma unroll
            for (int b = 0; b < FN; ++b)
#pragma unroll
                for (int a = 0; a < FM; ++a)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        facc[a][b][r] = fmaf(static_cast<float>(acc[a][b][r]), sw_t[b], facc[a][b][r]);
        } else if constexpr (MODE == kModeGroup) {
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
        // copies (and the scale loads issued after tile kt+1's copies) are
        // outstanding; the barrier makes every wave's part visible and
        // retires the reads of stage kt before it is refilled.  A plain
        // s_barrier: a workgroup fence would also drain the newer DMA loads,
        // and every LDS read of this tile has already fed an MFMA.
        wait_vmcnt<WAITN>();
        lds_barrier();
    };

    // prologue: tiles 0 .. STAGES-2 in flight; wait for tile 0
    static_for<0, STAGES - 1>([&](auto I) { issue(decltype(I)::value, I); });
    wait_vmcnt<(STAGES - 2) * LPW>();
    lds_barrier();

    int kt = 0;
    for (; kt + STAGES <= KT; kt += STAGES)
        static_for<0, STAGES>([&](auto I) { body(kt + decltype(I)::value, I); });
    static_for<0, STAGES - 1>([&](auto I) {
        if (kt + decltype(I)::value < KT) body(kt + decltype(I)::value, I);
    });

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
    // one workgroup per output tile, in a 1-D grid (tile order: xcd_tile)
    dim3 grid(ceil_div(a.N, BN) * ceil_div(a.M, BM));
    dim3 block(WM_ * WN_ * 64);
    if constexpr (MODE == kModeGroup) {
        if (a.group_size == BK) {
            if (a.asym)
                k_gemm_dl<BM, BN, WM_, WN_, ST, true, MODE, true><<<grid, block, 0, stream>>>(
                    a.Xq, a.s_x, a.Wq, a.s_w, a.z_w, a.Y, a.M, a.N, a.K, a.group_size);
            else
                k_gemm_dl<BM, BN, WM_, WN_, ST, false, MODE, true><<<grid, block, 0, stream>>>(
                    a.Xq, a.s_x, a.Wq, a.s_w, a.z_w, a.Y, a.M, a.N, a.K, a.group_size);
            return hipGetLastError();
        }
    }
    if (a.asym)
        k_gemm_dl<BM, BN, WM_, WN_, ST, true, MODE><<<grid, block, 0, stream>>>(
            a.Xq, a.s_x, a.Wq, a.s_w, a.z_w, a.Y, a.M, a.N, a.K, a.group_size);
    else
        k_gemm_dl<BM, BN, WM_, WN_, ST, false, MODE><<<grid, block, 0, stream>>>(
            a.Xq, a.s_x, a.Wq, a.s_w, a.z_w, a.Y, a.M, a.N, a.K, a.group_size);
    return hipGetLastError();
}

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
        if (it + 1 < t1) ++it;
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

    if (t0 < t1) {
        static_for<0, D - 1>([&](auto U) { issue(U); });
        for (int t = t0; t < t1; t += D) {
            static_for<0, D>([&](auto U) {
                constexpr int u = decltype(U)::value;
                issue(std::integral_constant<int, (u + D - 1) % D>{});
                if (t + u < t1) compute(t + u, std::integral_constant<int, u>{});
            });
        }
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

template <int BM, int BN, int WM_, int WN_, int MODE>
hipError_t launch_mode(const GemmArgs& a, hipStream_t stream) {
    dim3 grid(ceil_div(a.N, BN), ceil_div(a.M, BM));
    dim3 block(WM_ * WN_ * 64);
    if constexpr (MODE == kModeGroup) {
        if (a.group_size == BK) {
            if (a.asym)
                k_gemm_w4a4<BM, BN, WM_, WN_, true, MODE, true><<<grid, block, 0, stream>>>(
                    a.Xq, a.s_x, a.Wq, a.s_w, a.z_w, a.Y, a.D, a.M, a.N, a.K, a.group_size);
            else
                k_gemm_w4a4<BM, BN, WM_, WN_, false, MODE, true><<<grid, block, 0, stream>>>(
                    a.Xq, a.s_x, a.Wq, a.s_w, a.z_w, a.Y, a.D, a.M, a.N, a.K, a.group_size);
            return hipGetLastError();
        }
    }
    if (a.asym)
        k_gemm_w4a4<BM, BN, WM_, WN_, true, MODE><<<grid, block, 0, stream>>>(
            a.Xq, a.s_x, a.Wq, a.s_w, a.z_w, a.Y, a.D, a.M, a.N, a.K, a.group_size);
    else
        k_gemm_w4a4<BM, BN, WM_, WN_, false, MODE><<<grid, block, 0, stream>>>(
            a.Xq, a.s_x, a.Wq, a.s_w, a.z_w, a.Y, a.D, a.M, a.N, a.K, a.group_size);
    return hipGetLastError();
}

using LaunchFn = hipError_t (*)(const GemmArgs&, hipStream_t);

// A kernel configuration: launchers for the per-channel and per-group fp16
// modes (nullptr where the per-group fp32 accumulators would not fit the
// register file) and a name for traces.
struct KernelCfg {
    const char* name;
    LaunchFn chan, group;
};

#define W4A4_CFG(NAME, L) KernelCfg{NAME, &L<kModeChan>, &L<kModeGroup>}
#define W4A4_CFG_CHAN(NAME, L) KernelCfg{NAME, &L<kModeChan>, nullptr}

template <int MODE> hipError_t dl256x256_2x4_s4(const GemmArgs& a, hipStream_t s) { return launch_dl<256, 256, 2, 4, 4, MODE>(a, s); }
template <int MODE> hipError_t dl256x256_2x4_s3(const GemmArgs& a, hipStream_t s) { return launch_dl<256, 256, 2, 4, 3, MODE>(a, s); }
template <int MODE> hipError_t dl256x128_4x2_s4(const GemmArgs& a, hipStream_t s) { return launch_dl<256, 128, 4, 2, 4, MODE>(a, s); }
template <int MODE> hipError_t dl128x128_2x2_s4(const GemmArgs& a, hipStream_t s) { return launch_dl<128, 128, 2, 2, 4, MODE>(a, s); }
template <int MODE> hipError_t dl128x128_2x2_s3(const GemmArgs& a, hipStream_t s) { return launch_dl<128, 128, 2, 2, 3, MODE>(a, s); }
template <int MODE> hipError_t dl128x256_2x4_s3(const GemmArgs& a, hipStream_t s) { return launch_dl<128, 256, 2, 4, 3, MODE>(a, s); }
template <int MODE> hipError_t dl256x256_4x4_s3(const GemmArgs& a, hipStream_t s) { return launch_dl<256, 256, 4, 4, 3, MODE>(a, s); }
template <int MODE> hipError_t dl128x384_2x4_s4(const GemmArgs& a, hipStream_t s) { return launch_dl<128, 384, 2, 4, 4, MODE>(a, s); }
template <int MODE> hipError_t dl128x384_2x4_s3(const GemmArgs& a, hipStream_t s) { return launch_dl<128, 384, 2, 4, 3, MODE>(a, s); }
template <int MODE> hipError_t dl128x384_4x4_s3(const GemmArgs& a, hipStream_t s) { return launch_dl<128, 384, 4, 4, 3, MODE>(a, s); }
template <int MODE> hipError_t dl128x256_2x4_s4(const GemmArgs& a, hipStream_t s) { return launch_dl<128, 256, 2, 4, 4, MODE>(a, s); }


template <int MODE> hipError_t r16_256x128_2x4(const GemmArgs& a, hipStream_t s) { return launch_mode<256, 128, 2, 4, MODE>(a, s); }
template <int MODE> hipError_t r16_128x128_2x4(const GemmArgs& a, hipStream_t s) { return launch_mode<128, 128, 2, 4, MODE>(a, s); }

// Prefill configurations (M > 64).  dl: direct-to-LDS 32x32x32 kernel;
// r16: register-staged unpack-to-LDS kernel on 16x16x64.
const KernelCfg kTiles[] = {
    W4A4_CFG_CHAN("k_gemm_dl<256x256, waves 2x4, 4 stages>", dl256x256_2x4_s4),
    W4A4_CFG("k_gemm_dl<128x128, waves 2x2, 4 stages>", dl128x128_2x2_s4),
    W4A4_CFG("k_gemm_w4a4<128x128, waves 2x4>", r16_128x128_2x4),
    W4A4_CFG_CHAN("k_gemm_dl<256x256, waves 2x4, 3 stages>", dl256x256_2x4_s3),
    W4A4_CFG("k_gemm_dl<256x128, waves 4x2, 4 stages>", dl256x128_4x2_s4),
    W4A4_CFG("k_gemm_dl<128x128, waves 2x2, 3 stages>", dl128x128_2x2_s3),
    W4A4_CFG("k_gemm_w4a4<256x128, waves 2x4>", r16_256x128_2x4),
    W4A4_CFG_CHAN("k_gemm_dl<128x256, waves 2x4, 3 stages>", dl128x256_2x4_s3),
    W4A4_CFG_CHAN("k_gemm_dl<256x256, waves 4x4, 3 stages>", dl256x256_4x4_s3),
    W4A4_CFG_CHAN("k_gemm_dl<128x384, waves 2x4, 4 stages>", dl128x384_2x4_s4),
    W4A4_CFG_CHAN("k_gemm_dl<128x384, waves 2x4, 3 stages>", dl128x384_2x4_s3),
    W4A4_CFG_CHAN("k_gemm_dl<128x384, waves 4x4, 3 stages>", dl128x384_4x4_s3),
    W4A4_CFG("k_gemm_dl<128x256, waves 2x4, 4 stages>", dl128x256_2x4_s4),
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

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
    {W4A4_DEC(4, 1, 8, 3), W4A4_DEC(4, 2, 8, 3), W4A4_DEC(4, 1, 8, 2), W4A4_DEC(4, 2, 8, 2)},
};
#undef W4A4_DEC
#undef W4A4_CFG
#undef W4A4_CFG_CHAN

const KernelCfg kI32{"k_gemm_w4a4<64x64, waves 2x2, int32 out>", nullptr, nullptr};

// Selection override for tests and sweeps (w4a4_set_kernel_override): an
// index into the prefill table or the decode variants, -1 or out of range =
// automatic.
int override_index(int which, int n) {
    const int v = kernel_override(which);
    return (v >= 0 && v < n) ? v : -1;
}

const KernelCfg& choose(const GemmArgs& a) {
    const bool grouped = (a.K / a.group_size) > 1;
    const int cus = device_cu_count();
    if (a.M <= 64) {
        const int fi = a.M <= 16 ? 0 : (a.M <= 32 ? 1 : 2);
        int v = override_index(1, kNumDec);
        if (v < 0) {
            // measured on MI355X: one 16-column fragment per workgroup while
            // two workgroups fit a CU, two once the staged activations fill
            // the LDS (or for two and four row fragments) and the grid still
            // covers every CU
            bool wide = ceil_div(a.N, 32) >= cus;
            if (fi == 0) {
                const size_t staged = static_cast<size_t>(a.M) * (a.K / 2 + 16);
                wide = wide && staged > 64 * 1024;
            }
            v = wide ? 1 : 0;
        }
        return kDec[fi][v];
    }
    int t = override_index(0, kNumTiles);
    if (t < 0 || (grouped && kTiles[t].group == nullptr)) {
        // measured on MI355X: direct-to-LDS 256x256 tiles with 16 waves when
        // the grid covers the CUs at least half over (4096x8192 -> 57344 with
        // three weight copies rotated: 1486-1520 against 1545-1549 us for 8
        // waves; 2048x6144: 57 against 60 us for 128x128 tiles),
        // direct-to-LDS 128x128 tiles below that
        // (128x384 tiles with 16 waves when they give about one tile per CU:
        // 2048x6144 takes 50.6 against 53.3 us with 256x256 tiles).
        // Groups of 128: the direct-to-LDS 128x128 tile with 3 stages and
        // one-tile groups (2048x4096 -> 28672: 442 against 467 us for the
        // 16x16x64 register-staged tile); other group sizes: the 16x16x64
        // 128x128 tile (8 waves)
        const long tiles256 = static_cast<long>(ceil_div(a.M, 256)) * ceil_div(a.N, 256);
        const long tiles384 = static_cast<long>(ceil_div(a.M, 128)) * ceil_div(a.N, 384);
        if (grouped && a.group_size == BK)
            t = 5;
        else if (grouped)
            t = 2;
        else if (tiles384 >= cus && tiles384 < 2L * cus)
            t = 11;
        else if (2L * tiles256 >= cus)
            t = 8;
        else
            t = 1;
    }
    return kTiles[t];
}

}  // namespace

int gemm_num_tile_configs() { return kNumTiles; }
int gemm_num_decode_configs() { return kNumDec; }

size_t gemm_workspace_bytes(int M, int N, int K, int group_size) {
    (void)M;
    (void)N;
    (void)K;
    (void)group_size;
    return 0;
}

const char* gemm_kernel_name(const GemmArgs& a, bool i32_out) {
    if (i32_out) return kI32.name;
    return choose(a).name;
}

hipError_t gemm_launch(const GemmArgs& a, bool i32_out, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
    (void)ws;
    (void)ws_bytes;
    if (a.M == 0) return hipSuccess;
    if (i32_out) return launch_mode<64, 64, 2, 2, kModeI32>(a, stream);
    const bool grouped = (a.K / a.group_size) > 1;
    const KernelCfg& k = choose(a);
    return grouped ? k.group(a, stream) : k.chan(a, stream);
}

}  // namespace w4a4
