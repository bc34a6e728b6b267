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
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h_t __attribute__((ext_vector_type(8)));

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
// c ^ ((r >> 2) & 3).  With it the fragment reads (lane l: row l % 32,
// chunk 2p + l / 32) count no LDS bank conflict on gfx950
// (SQ_LDS_BANK_CONFLICT 0 against 4 cycles per ds_read_b128 with the
// slot c ^ (((r >> 1) ^ (r >> 3)) & 3) used before).  A lane reads one packed chunk and
// unpacks it into two 32x32x32 fragments: the even codes (low nibbles) for
// one k-step and the odd codes (high nibbles) for the next; A and B use the
// same order, so the products are those of the tile.  Signed codes are kept
// as 16*q (nibble in the high half of the byte); asymmetric weights become
// u - z.
// ===========================================================================
__device__ __forceinline__ int dl_slot(int row, int c) { return c ^ ((row >> 2) & 3); }

// XCD-aware tile order.  Workgroups are dispatched round-robin over the 8
// XCDs (workgroup L to XCD L % 8), each with its own L2.  The 1-D grid index
// is turned into a tile index t so that XCD x walks the contiguous range of
// tiles it owns, in the order its workgroups start.  t runs over groups of
// gm M tiles: down the gm M tiles of one column of N tiles, then the next
// column, then the next group of M tiles.  The workgroups an XCD holds at
// once then share gm activation panels and a few weight panels, whose K
// slices they read from that XCD's L2 at about the same time.
constexpr int kXcds = 8;
__device__ __forceinline__ void xcd_tile(int L, int tiles_m, int tiles_n, int gm, int& tm, int& tn) {
    const int T = tiles_m * tiles_n;
    const int per = T / kXcds, rem = T % kXcds;
    const int x = L % kXcds, local = L / kXcds;
    const int t = x < rem ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
    const int grp = t / (gm * tiles_n);
    const int m_base = grp * gm;
    const int gsz = min(gm, tiles_m - m_base);          // the last group may be short
    const int r = t - grp * gm * tiles_n;
    tn = r / gsz;
    tm = m_base + (r - tn * gsz);
}

// s_waitcnt with only a vmcnt condition (gfx9 encoding; expcnt and lgkmcnt
// left at their no-wait maxima)
// Per-token sums of the signed activation codes over each group of one K
// tile, times 16 (the K loop's scale of the activation operand), as fp16
// (|16 S| <= 16384, exact): S16[m, g] for g < K / 128, zero for the padding
// up to Gp.  One thread per (m, g); the 64 packed bytes of a group are
// summed as unsigned nibbles minus 16 per negative code.
__global__ __launch_bounds__(256) void k_act_group_sums(const uint8_t* __restrict__ Xq, int M,
                                                        int K, int Gp,
                                                        uint16_t* __restrict__ S16) {
    const long t = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
    if (t >= static_cast<long>(M) * Gp) return;
    const int m = static_cast<int>(t / Gp);
    const int g = static_cast<int>(t % Gp);
    int sum = 0;
    if (g < K / BK) {
        const uint4* p = reinterpret_cast<const uint4*>(Xq + static_cast<size_t>(m) * (K / 2) +
                                                        static_cast<size_t>(g) * 64);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 v = p[i];
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t w = w4[j];
                const uint32_t u = (w & 0x0F0F0F0Fu) + ((w >> 4) & 0x0F0F0F0Fu);
                sum += static_cast<int>((u * 0x01010101u) >> 24) -
                       16 * __builtin_popcount(w & 0x88888888u);
            }
        }
    }
    S16[t] = f2h(static_cast<float>(16 * sum));
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, bool ASYM, int MODE, bool G1 = false>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64) void k_gemm_dl(
    const uint8_t* __restrict__ Xq, const float* __restrict__ s_x,
    const uint8_t* __restrict__ Wq, const uint16_t* __restrict__ s_w,
    const uint16_t* __restrict__ z_w, uint16_t* __restrict__ Y, int M, int N, int K,
    int group_size, int tile_group, const uint16_t* __restrict__ Sg, int Gp) {
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M;
    constexpr int WN = BN / WAVES_N;
    constexpr int FM = WM / 32;
    constexpr int FN = WN / 32;
    static_assert(FM >= 1 && FN >= 1 && WM % 32 == 0 && WN % 32 == 0, "wave tile");
    constexpr int PROW = 64;                          // packed bytes per tile row
    constexpr int OPER_BYTES = (BM + BN) * PROW;
    // One-tile groups with asymmetric weights multiply the unsigned codes u in
    // the K loop and subtract z[n,g] * Σ_{k in g} q_x[m,k] in the epilogue
    // (Σ q (u - z) = Σ q u - z Σ q), so the loop needs no zero points.
    constexpr bool ZID = G1 && ASYM;
    // One-tile groups: a stage also holds the tile's weight scales of its BN
    // rows, copied by the same DMA as the operands: per row the aligned
    // 4-byte word that holds the 16-bit value, 64 rows
    // per copy (lane l's word lands at slot + 4 l).  Every wave issues
    // exactly one such copy per tile into its own 256-byte slot; waves past
    // the SZI items repeat item wave % SZI.
    constexpr int SZI = G1 ? BN / 64 : 1;
    static_assert(!G1 || (BN % 64 == 0 && SZI <= NW), "scale copies: at most one item per wave");
    constexpr int SZSLOT = 256;
    constexpr int STAGE_BYTES = OPER_BYTES + (G1 ? NW * SZSLOT : 0);
    constexpr int CHUNKS = (BM + BN) * 4;             // 16-byte chunks per tile
    static_assert(CHUNKS % (64 * NW) == 0 && (BM * 4) % 64 == 0, "whole wave loads");
    constexpr int LPW = CHUNKS / (64 * NW);           // load instructions per wave per tile
    constexpr int NSZ = G1 ? 1 : 0;                   // scale copies per wave per tile
    constexpr int WAITN = (STAGES - 2) * (LPW + NSZ);
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
    // LDS byte address of a stage (scalar: the copies' m0)
    auto stage_lds = [&](auto S) -> uint32_t {
        constexpr int I = decltype(S)::value;
        typedef const __attribute__((address_space(3))) uint8_t* lp;
        if constexpr (I == 0) return lds_addr((lp)st0);
        else if constexpr (I == 1) return lds_addr((lp)st1);
        else if constexpr (I == 2) return lds_addr((lp)st2);
        else if constexpr (I == 3) return lds_addr((lp)st3);
        else if constexpr (I == 4) return lds_addr((lp)st4);
        else if constexpr (I == 5) return lds_addr((lp)st5);
        else if constexpr (I == 6) return lds_addr((lp)st6);
        else return lds_addr((lp)st7);
    };
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
    xcd_tile(blockIdx.x, ceil_div(M, BM), ceil_div(N, BN), tile_group, tm, tn);
    // tile origin: workgroup-uniform, kept in scalar registers so that the
    // copies' scalar bases need no per-copy readfirstlane
    const int m0 = __builtin_amdgcn_readfirstlane(tm * BM);
    const int n0 = __builtin_amdgcn_readfirstlane(tn * BN);
    const int KB = K / 2;
    const int KT = K / BK;
    const int G = K / group_size;
    const int TPG = group_size / BK;

    // this lane's source row (clamped) and chunk for each of its loads.
    // Load i of a wave covers 64 consecutive slots, all in A or all in B, so
    // the copies take a wave-uniform base (the tile's first row, scalar
    // registers) and a 32-bit lane offset, issued from inline assembly: the
    // compiler does not see them, so it neither drains them before LDS reads
    // (as it does for the builtin copies, not knowing which bytes they write)
    // nor counts them; every wait in the K loop is explicit.  The K loop then
    // must hold no other global load (a compiler-inserted wait for it would
    // drain the copies): per-channel zero points are read once before the
    // loop, one-tile-group scales come through the stages.  Groups spanning
    // several K tiles load their scales in the loop and keep the builtin
    // copies.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    constexpr bool kBuiltinCopies = MODE == kModeGroup && !G1;
    const uint8_t* src[kBuiltinCopies ? LPW : 1];
    uint32_t soff[kBuiltinCopies ? 1 : LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int j = (i * NW + wave_u) * 64 + lane;   // 16-byte slot in the stage
        const bool isA = (i * NW + wave_u) * 64 < BM * 4;
        const int jj = isA ? j : j - BM * 4;
        const int row = jj >> 2;
        const int c = (jj & 3) ^ ((row >> 2) & 3);
        const int r = isA ? min(m0 + row, M - 1) : min(n0 + row, N - 1);
        if constexpr (kBuiltinCopies)
            src[i] = (isA ? Xq : Wq) + static_cast<size_t>(r) * KB + c * 16;
        else
            soff[i] = static_cast<uint32_t>(r - (isA ? m0 : n0)) * KB + c * 16;
    }
    // this wave's scale copy: the 64-row block of its item and the lane's
    // element index of group 0
    uint32_t sz_e0 = 0;
    if constexpr (G1)
        sz_e0 = static_cast<uint32_t>(min(n0 + (wave_u % SZI) * 64 + lane, N - 1)) *
                static_cast<uint32_t>(G);
    auto issue = [&](int kt, auto S) {
        const int kc = min(kt, KT - 1);
        uint8_t* stage = stage_ptr(S);
        const uint32_t sl = stage_lds(S);
        if constexpr (G1)
            dma4_async_sv(s_w, 2u * ((sz_e0 + static_cast<uint32_t>(kc)) & ~1u),
                          sl + static_cast<uint32_t>(OPER_BYTES + wave_u * SZSLOT));
        if constexpr (kBuiltinCopies) {
#pragma unroll
            for (int i = 0; i < LPW; ++i) dma16(src[i] + kc * 64, stage + (i * NW + wave) * 1024);
        } else {
            const uint8_t* xb = Xq + static_cast<size_t>(m0) * KB + kc * 64;
            const uint8_t* wb = Wq + static_cast<size_t>(n0) * KB + kc * 64;
#pragma unroll
            for (int i = 0; i < LPW; ++i)
                dma16_async_sv((i * NW + wave_u) * 64 < BM * 4 ? xb : wb, soff[i],
                               sl + static_cast<uint32_t>((i * NW + wave_u) * 1024));
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
    // fragment serve both the unpack and the fold; they are read from the
    // tile's stage (the half of the copied word that the element's index
    // parity selects).  A zero made opaque to the compiler: an MFMA whose
    // accumulator operand was an inline-constant zero gave wrong sums.
    v16i zc16;
    if constexpr (G1) {
        int z0;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z0));
#pragma unroll
        for (int r = 0; r < 16; ++r) zc16[r] = z0;
    }
    // per-channel zero points: read once, before any copy is in flight
    uint32_t zb_chan[(ASYM && MODE == kModeChan) ? FN : 1];
    if constexpr (ASYM && MODE == kModeChan) {
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            const uint32_t z = static_cast<uint32_t>(h2f(z_w[brow_g[b]]));
            zb_chan[b] = (0x80u - z) * 0x01010101u;
        }
    }

    // one K tile: tile kt is in stage kt % STAGES; the DMA of tile
    // kt+STAGES-1 goes into the stage tile kt-1 used.  Always inlined: a
    // body emitted out of line (the multi-tile group mode's was) keeps the
    // accumulators it captures in scratch memory.
    auto body = [&](int kt, auto S) __attribute__((always_inline)) {
        constexpr int SI = decltype(S)::value;
        issue(kt + STAGES - 1, std::integral_constant<int, (SI + STAGES - 1) % STAGES>{});
        const uint8_t* stage = stage_ptr(S);
        uint32_t zbias[FN];
        float sw_t[G1 ? FN : 1];
        if constexpr (G1) {
            // this tile's scales from its stage: item i holds rows
            // 64 i + lane
            const uint8_t* szs = stage + OPER_BYTES;
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const int rr = wn0 + b * 32 + frow;
                const int r = (rr >> 6) * SZSLOT + 4 * (rr & 63);
                const uint32_t sh = 16u * ((static_cast<uint32_t>(brow_g[b]) * static_cast<uint32_t>(G) +
                                            static_cast<uint32_t>(kt)) & 1u);
                sw_t[b] = h2f(static_cast<uint16_t>(*reinterpret_cast<const uint32_t*>(szs + r) >> sh));
            }
        } else if constexpr (ASYM && MODE == kModeChan) {
#pragma unroll
            for (int b = 0; b < FN; ++b) zbias[b] = zb_chan[b];
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
                if constexpr (ZID)
                    unpack_unsigned(w, ev, od);
                else if constexpr (ASYM)
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
    wait_vmcnt<(STAGES - 2) * (LPW + NSZ)>();
    lds_barrier();

    int kt = 0;
    for (; kt + STAGES <= KT; kt += STAGES)
        static_for<0, STAGES>([&](auto I) { body(kt + decltype(I)::value, I); });
    static_for<0, STAGES - 1>([&](auto I) {
        if (kt + decltype(I)::value < KT) body(kt + decltype(I)::value, I);
    });

    // zero-point correction (asymmetric one-tile groups): the K loop summed
    // s_w[n,g] * 16 Σ_k q_x u; subtract Σ_g (16 S[m,g]) (s_w z_w)[n,g] with
    // S[m,g] = Σ_{k in g} q_x[m,k], on the fp16 matrix pipe: 16 S is exact in
    // fp16, s z (an fp16 scale times a 4-bit integer) has at most 15
    // significant bits and is split into fp16 hi + lo, so every product is
    // exact and the accumulation is the fp32 one of the fold.  Lane (row
    // frow, half fks) supplies groups g0 + 8 fks .. + 7 of A and of B.
    if constexpr (ZID) {
        const bool vec = (G & 7) == 0;
        for (int g0 = 0; g0 < Gp; g0 += 16) {
            const int gb = g0 + 8 * fks;
            v8h_t sa[FM];
#pragma unroll
            for (int a = 0; a < FM; ++a) {
                const int row = min(m0 + wm0 + a * 32 + frow, M - 1);
                sa[a] = *reinterpret_cast<const v8h_t*>(Sg + static_cast<size_t>(row) * Gp + gb);
            }
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const size_t e0 = static_cast<size_t>(brow_g[b]) * G + gb;
                uint16_t sv[8], zv[8];
                if (vec && gb + 8 <= G) {
                    const uint4 s4 = *reinterpret_cast<const uint4*>(s_w + e0);
                    const uint4 z4 = *reinterpret_cast<const uint4*>(z_w + e0);
                    const uint32_t sw4[4] = {s4.x, s4.y, s4.z, s4.w};
                    const uint32_t zw4[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        sv[e] = static_cast<uint16_t>(sw4[e >> 1] >> (16 * (e & 1)));
                        zv[e] = static_cast<uint16_t>(zw4[e >> 1] >> (16 * (e & 1)));
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const bool in = gb + e < G;
                        sv[e] = in ? s_w[e0 + e] : uint16_t{0};
                        zv[e] = in ? z_w[e0 + e] : uint16_t{0};
                    }
                }
                v8h_t bh, bl;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const F16Pair hl = split_f16(-h2f(sv[e]) * h2f(zv[e]));
                    bh[e] = hl.hi;
                    bl[e] = hl.lo;
                }
#pragma unroll
                for (int a = 0; a < FM; ++a) {
                    v16f c;
#pragma unroll
                    for (int r = 0; r < 16; ++r) c[r] = facc[a][b][r];
                    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(sa[a], bh, c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(sa[a], bl, c, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 16; ++r) facc[a][b][r] = c[r];
                }
            }
        }
    }

    // epilogue: row by row, the wave's FN column fragments of a row one after
    // the other, so the halves of a 128-byte output line are written by
    // consecutive stores
    constexpr float kUnshift = ASYM ? (1.0f / 16.0f) : (1.0f / 256.0f);
    float sw1[FN];
#pragma unroll
    for (int b = 0; b < FN; ++b) {
        const int gn = n0 + wn0 + b * 32 + ocol;
        sw1[b] = (MODE == kModeChan && gn < N) ? h2f(s_w[gn]) : 1.0f;
    }
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int gm = m0 + wm0 + a * 32 + 8 * (r >> 2) + orow + (r & 3);
            if (gm >= M) continue;
            const float sx = s_x[gm] * kUnshift;
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const int gn = n0 + wn0 + b * 32 + ocol;
                if (gn >= N) continue;
                float v;
                if constexpr (MODE == kModeChan)
                    v = static_cast<float>(acc[a][b][r]) * sw1[b];
                else
                    v = facc[a][b][r];
                Y[static_cast<size_t>(gm) * N + gn] = f2h(v * sx);
            }
        }
}

// M tiles per group of the tile order (xcd_tile).  An XCD holds W tiles at
// once (32 CUs x the workgroups one CU holds); a group of gm M tiles then
// fetches gm activation panels (BM rows) and W / gm weight panels (BN rows)
// per K slice into the XCD's L2, least for gm = sqrt(W BN / BM); the power of
// two below it is taken.  Measured on MI355X for 4096x8192 -> 57344 in
// 256x256 tiles (W = 32, gm = 4) with three weight copies rotated: groups of 4
// took 1362-1374 us against 1384-1386 (2), 1407 (3), 1382 (6) and 1426-1478
// us for one group of all 16; for 2048x4096 -> 6144 in 128x384 tiles the
// formula gives 8 (fetch: 59 MB per launch with groups of 4).  A sweep
// override may ask for another count.
constexpr int kCusPerXcd = 32;
int tile_group_for(int tiles_m, int BM, int BN, int wgs_per_cu) {
    const int v = kernel_override(3);
    int g = 1;
    if (v >= 1) {
        g = v;
    } else {
        const double want = __builtin_sqrt(static_cast<double>(kCusPerXcd) * wgs_per_cu * BN / BM);
        while (2 * g <= want) g *= 2;
    }
    return g < tiles_m ? g : tiles_m;
}

// workgroups of kernel Kern one CU holds, cached per kernel: the kernel is a
// template argument, since every k_gemm_dl instantiation has the same
// function-pointer type (a cache keyed on that type would keep the first
// kernel's figure for all of them)
template <auto Kern>
int wgs_per_cu(int threads) {
    static int n = 0;
    if (n == 0) {
        int v = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, Kern, threads, 0) != hipSuccess || v < 1)
            v = 1;
        n = v;
    }
    return n;
}

// one launch of the instantiation Kern; the tile order's group count comes
// from that kernel's own occupancy
template <auto Kern, int BM, int BN, int NT>
hipError_t launch_dl_k(const GemmArgs& a, const uint16_t* S, int Gp, hipStream_t stream) {
    const dim3 grid(ceil_div(a.N, BN) * ceil_div(a.M, BM));
    const int tg = tile_group_for(ceil_div(a.M, BM), BM, BN, wgs_per_cu<Kern>(NT));
    Kern<<<grid, dim3(NT), 0, stream>>>(a.Xq, a.s_x, a.Wq, a.s_w, a.z_w, a.Y, a.M, a.N, a.K,
                                        a.group_size, tg, S, Gp);
    return hipGetLastError();
}

template <int BM, int BN, int WM_, int WN_, int ST, int MODE>
hipError_t launch_dl(const GemmArgs& a, hipStream_t stream) {
    // one workgroup per output tile, in a 1-D grid (tile order: xcd_tile)
    constexpr int NT = WM_ * WN_ * 64;
    if constexpr (MODE == kModeGroup) {
        if (a.group_size == BK) {
            // the scale copies address N x G 16-bit elements with 32-bit offsets
            if (static_cast<size_t>(a.N) * static_cast<size_t>(a.K / BK) >= (size_t{1} << 31))
                return hipErrorInvalidValue;
            if (a.asym && (a.S == nullptr || a.Gp < a.K / BK)) return hipErrorInvalidValue;
            if (a.asym)
                return launch_dl_k<&k_gemm_dl<BM, BN, WM_, WN_, ST, true, MODE, true>, BM, BN, NT>(
                    a, a.S, a.Gp, stream);
            return launch_dl_k<&k_gemm_dl<BM, BN, WM_, WN_, ST, false, MODE, true>, BM, BN, NT>(
                a, nullptr, 0, stream);
        }
    }
    if (a.asym)
        return launch_dl_k<&k_gemm_dl<BM, BN, WM_, WN_, ST, true, MODE>, BM, BN, NT>(a, nullptr, 0,
                                                                                  stream);
    return launch_dl_k<&k_gemm_dl<BM, BN, WM_, WN_, ST, false, MODE>, BM, BN, NT>(a, nullptr, 0,
                                                                               stream);
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

// Prefill configurations (M > 64; decode kernels: gemm_decode.hip).
// dl: direct-to-LDS 32x32x32 kernel;
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

#undef W4A4_CFG
#undef W4A4_CFG_CHAN

const KernelCfg kI32{"k_gemm_w4a4<64x64, waves 2x2, int32 out>", nullptr, nullptr};

// Selection override for tests and sweeps (w4a4_set_kernel_override): an
// index into the prefill table, -1 or out of range = automatic.
int override_index(int which, int n) {
    const int v = kernel_override(which);
    return (v >= 0 && v < n) ? v : -1;
}

const KernelCfg& choose(const GemmArgs& a) {
    const bool grouped = (a.K / a.group_size) > 1;
    const int cus = device_cu_count();
    int t = override_index(0, kNumTiles);
    if (t < 0 || (grouped && kTiles[t].group == nullptr)) {
        // measured on MI355X: direct-to-LDS 256x256 tiles with 16 waves when
        // the grid covers the CUs at least half over (4096x8192 -> 57344 with
        // three weight copies rotated: 1486-1520 against 1545-1549 us for 8
        // waves; 2048x6144: 57 against 60 us for 128x128 tiles),
        // direct-to-LDS 128x128 tiles below that
        // (128x384 tiles with 16 waves when they give about one tile per CU:
        // 2048x6144 takes 50.6 against 53.3 us with 256x256 tiles).
        // Groups of 128 (one-tile groups, direct-to-LDS): 128x128 tiles with
        // 4 waves and 4 stages up to K = 8192, 256x128 tiles with 8 waves and
        // 4 stages above (measured with scalar copy destinations, alternating
        // runs on one box: 2048x4096 -> 28672 took 333-334 us against 347-352
        // us with 256x128 tiles; 2048x14336 -> 4096 took 165-170 us with
        // 256x128 against 175 us with 128x128); other group sizes: the
        // 16x16x64 128x128 tile (8 waves)
        const long tiles256 = static_cast<long>(ceil_div(a.M, 256)) * ceil_div(a.N, 256);
        const long tiles384 = static_cast<long>(ceil_div(a.M, 128)) * ceil_div(a.N, 384);
        if (grouped && a.group_size == BK)
            t = a.K <= 8192 ? 1 : 4;
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

// prefill with asymmetric groups of one K tile: the per-token group sums
static int group_sums_pad(int K) { return (K / BK + 15) / 16 * 16; }
static bool uses_group_sums(int M, int K, int group_size, bool asym) {
    return asym && group_size == BK && M > kDecodeMaxM && K / group_size > 1;
}

bool gemm_takes_group_sums(int M, int K, int group_size, bool asym, int* Gp) {
    if (!uses_group_sums(M, K, group_size, asym)) return false;
    *Gp = group_sums_pad(K);
    return true;
}

size_t gemm_workspace_bytes(int M, int N, int K, int group_size, bool asym) {
    // decode: the split-K kernel's partial sums (per channel or groups of 128)
    if (M <= kDecodeMaxM) return gemm_decode_workspace_bytes(M, N, K, group_size, asym);
    if (!uses_group_sums(M, K, group_size, asym)) return 0;
    const size_t b = sizeof(uint16_t) * static_cast<size_t>(M) * group_sums_pad(K);
    return (b + 255) & ~static_cast<size_t>(255);
}

const char* gemm_kernel_name(const GemmArgs& a, bool i32_out) {
    if (i32_out) return kI32.name;
    if (a.M <= kDecodeMaxM) return gemm_decode_kernel_name(a);
    return choose(a).name;
}

hipError_t gemm_launch(const GemmArgs& a, bool i32_out, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
    if (a.M == 0) return hipSuccess;
    if (i32_out) return launch_mode<64, 64, 2, 2, kModeI32>(a, stream);
    if (a.M <= kDecodeMaxM) return gemm_decode_launch(a, ws, ws_bytes, stream);
    const bool grouped = (a.K / a.group_size) > 1;
    const KernelCfg& k = choose(a);
    if (!grouped) return k.chan(a, stream);
    GemmArgs g = a;
    if (uses_group_sums(a.M, a.K, a.group_size, a.asym) && a.sums_ready) {
        if (a.S == nullptr || a.Gp != group_sums_pad(a.K)) return hipErrorInvalidValue;
    } else if (uses_group_sums(a.M, a.K, a.group_size, a.asym)) {
        const size_t need = gemm_workspace_bytes(a.M, a.N, a.K, a.group_size, a.asym);
        if (ws == nullptr || ws_bytes < need) return hipErrorInvalidValue;
        g.Gp = group_sums_pad(a.K);
        uint16_t* S = static_cast<uint16_t*>(ws);
        const long total = static_cast<long>(a.M) * g.Gp;
        k_act_group_sums<<<static_cast<unsigned>((total + 255) / 256), 256, 0, stream>>>(
            a.Xq, a.M, a.K, g.Gp, S);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        g.S = S;
    }
    return k.group(g, stream);
}

}  // namespace w4a4
