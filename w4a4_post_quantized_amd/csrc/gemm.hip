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
};
#undef W4A4_TILE
#undef W4A4_TILE_CHAN
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

// Developer override for tile sweeps: W4A4_GEMM_TILE=<index into kTiles>.
int tile_override() {
    static int v = -2;
    if (v == -2) {
        const char* e = getenv("W4A4_GEMM_TILE");
        v = e ? atoi(e) : -1;
        if (v >= kNumTiles) v = -1;
    }
    return v;
}

}  // namespace

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
        // measured on MI355X: 256x256 tiles when the grid covers the CUs
        // several times over, 256x192 (8 waves) for about one wave of tiles,
        // 128x128 with 8 waves for the per-group mode
        const int cus = device_cu_count();
        const long tiles256 = static_cast<long>(ceil_div(a.M, 256)) * ceil_div(a.N, 256);
        if (grouped)
            t = 7;
        else if (tiles256 >= 2L * cus)
            t = 0;
        else
            t = (a.N % 192 == 0) ? 2 : 7;
    }
    return grouped ? kTiles[t].group(a, stream) : kTiles[t].chan(a, stream);
}

}  // namespace w4a4
