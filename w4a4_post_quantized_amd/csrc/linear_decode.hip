// Single-kernel decode layer: the activation transform, the INT4 quantization
// and the INT4 x INT4 GEMM of a few tokens (M <= 16) in one launch, so that
// the weight stream starts while the activations are still being transformed.
//
// FlatQuant: Flatness Matters for LLM Quantization, section 高效 Kernel 设计
// (the transform and the quantization of a token tile fused into the layer's
// kernels); MergeQuant page, section 问题定义 (in autoregressive decoding the
// quantize / dequantize steps around every matrix product cost a large share
// of the time).  The arithmetic is exactly that of w4a4_transform_quant (or
// its static-step form) followed by w4a4_gemm; only the schedule differs.
//
// Shapes: n2 = 128 and n1 a multiple of 32 up to 256 (K = n1 * 128), no
// diag(c).  The grid has one workgroup of 8 waves per 16 output columns.
//
//  * Producers: workgroups 0 .. U-1, U = M * n1/16, first compute one unit of
//    the transform each: token m, one 16-row block of Z and all 128 columns
//    (one wave per 16-column block), with the column-block MFMA arithmetic of
//    the transform kernels (X̄ staged in LDS, P2 split hi/lo in registers, P1
//    fragments of the block in LDS, power-of-two prescales).
//      dynamic scales: the units of a token post their absmax (a tagged
//        atomic maximum) and meet at a barrier of the token's producers;
//        each then has the token scale and quantizes its own rows;
//      static steps: the unit quantizes its rows with the steps at once.
//    The unit packs its rows, writes them to the workspace and counts itself
//    on the ready counter.
//  * Consumers: every workgroup then stages its 16 weight rows' scale table
//    in LDS, issues the loads of its first weight tiles, waits for the ready
//    counter, stages the packed activations in LDS and runs the decode GEMM
//    loop of w4a4_gemm (waves split K; partial sums added in LDS in wave
//    order, so the result does not depend on timing).
//
// Signalling.  Counters are 64-bit words holding (epoch << 32) | count with
// an epoch unique to the call; a word tagged with another epoch counts as
// zero, so nothing is reset between calls.  Writers publish with device-scope
// release fences before the atomic, readers take a device-scope acquire fence
// after it (a tagged maximum needs neither: the value is in the atomic).  A
// workgroup that waits was dispatched after every producer (the producers
// have the lowest indices and their number is checked against the device's
// resident capacity on the host), so the producers are resident or done.  Every wait is bounded by the real-time clock; a wait that runs out
// sets the error word of the sync buffer and the call's output is invalid.
#include <atomic>

#include "common.hpp"
#include "internal.hpp"

namespace w4a4 {

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kLdWaves = 8;
constexpr int kLdThreads = kLdWaves * 64;
constexpr int kLdDepth = 12;                 // weight tiles in flight per wave (+1)
constexpr int kLdN2 = 128;
constexpr int kLdLdsCU = 160 * 1024;         // LDS of one CU
constexpr int kLdLdsMax = 152 * 1024;        // dynamic LDS limit of one workgroup
constexpr int kLdBK = 128;                   // codes per K tile
constexpr uint64_t kLdWaitTicks = 2000000;  // 20 ms of the 100 MHz real-time clock

// sync buffer: 64-bit per-token counters at words 0..15, the tokens' tagged
// absmax at words 16..31, the ready counter at 64-bit word 32 (byte 256, its
// own cache line), the error word at 32-bit word 128 (byte 512)
constexpr int kSyncTokMax = 16;
constexpr int kSyncReady = 32;
constexpr int kSyncErr = 128;

enum LdMode { kLdChan = 0, kLdGroup = 1 };

constexpr int kCoherentLoad = 16;            // cache-policy bit sc1: device scope

template <int N1>
struct LdCfg {
    static_assert(N1 % 32 == 0 && N1 >= 32 && N1 <= 256, "n1: a multiple of 32 up to 256");
    static constexpr int N2 = kLdN2;
    static constexpr int K = N1 * N2;
    static constexpr int RB = N1 / 16;           // 16-row blocks of Z: units per token
    static constexpr int CB = N2 / 16;           // 16-column blocks, one per wave
    static constexpr int KS1 = N2 / 32;          // stage-1 MFMA k-steps
    static constexpr int KS2 = N1 / 32;          // stage-2 MFMA k-steps
    static constexpr int FRAG = 64 * 8;          // fp16 elements of one fragment
    static constexpr int P1BYTES = KS2 * FRAG * 2 * 2;   // hi + lo fragments of one block
    // staged X̄ row: rows of 256 bytes padded by 32 (no LDS bank conflict in
    // the stage-1 operand reads; 16 bytes gave 4 cycles per read), others 16
    static constexpr int XROW = N2 * 2 + ((N2 * 2) % 256 == 0 ? 32 : 16);
    // the staged token, rounded up to whole 64-lane copies of 16 bytes
    static constexpr int XCOPIES = (N1 * (XROW / 16) + 63) / 64;
    static constexpr int XBYTES = XCOPIES * 1024;
    static constexpr int QBYTES = 16 * N2 / 2;   // packed codes of one unit
    static constexpr int PROD_LDS = P1BYTES + XBYTES + QBYTES;
    static_assert(CB == kLdWaves, "one wave per 16-column block");
};

// One more on a tagged counter; returns the count after the increment.  The
// first contender of a call moves the word to the call's epoch with count 0
// (one compare-and-swap succeeds, the others see the new tag); every
// contender then adds 1, which never retries.
__device__ uint32_t tagged_add(uint64_t* w, uint32_t epoch) {
    uint64_t cur = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = 0; i < 64 && static_cast<uint32_t>(cur >> 32) != epoch; ++i) {
        const uint64_t fresh = static_cast<uint64_t>(epoch) << 32;
        if (__hip_atomic_compare_exchange_strong(w, &cur, fresh, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
            break;
    }
    const uint64_t old = __hip_atomic_fetch_add(w, uint64_t{1}, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    return static_cast<uint32_t>(old >> 32) == epoch ? static_cast<uint32_t>(old) + 1u : 0u;
}

struct LdArgs {
    const uint16_t* X;
    const float* P1;
    const float* P2;
    ActQuant aq;
    const uint8_t* Wq;
    const uint16_t* s_w;
    const uint16_t* z_w;
    uint16_t* Y;
    uint8_t* Xq;         // [M, K/2] packed codes
    float* s_x;          // [M]
    uint64_t* sync;
    int M, N, group_size;
    uint32_t epoch;
};

template <int N1, bool ASYM, int MODE, bool G1>
__global__ __launch_bounds__(kLdThreads) void k_linear_dec(LdArgs p) {
    using C = LdCfg<N1>;
    constexpr int K = C::K;
    constexpr int N2 = C::N2;
    constexpr int NT = kLdThreads;
    constexpr int NW = kLdWaves;
    constexpr int D = kLdDepth;
    constexpr bool SZ = (MODE == kLdGroup) || ASYM;
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ float red8[kLdWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int li = lane & 15;
    const int M = p.M;
    const bool is_static = p.aq.steps != nullptr;
    const int units = M * C::RB;

    // =====================================================================
    // Producer: unit u = (token m, 16-row block `part` of Z)
    // =====================================================================
    if (static_cast<int>(blockIdx.x) < units) {
        const int m = blockIdx.x / C::RB;
        const int part = blockIdx.x - m * C::RB;
        _Float16* p1hi = reinterpret_cast<_Float16*>(lds);
        _Float16* p1lo = p1hi + C::KS2 * C::FRAG;
        uint8_t* xs = lds + C::P1BYTES;
        uint8_t* qs = xs + C::XBYTES;
        const int cb = wave;

        // every load before the first wait: this wave's P2 columns, the
        // token's X̄ (to LDS) and the block's P1 columns (16-byte pieces)
        float p2v[C::KS1][8];
#pragma unroll
        for (int ks = 0; ks < C::KS1; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) p2v[ks][e] = p.P2[(32 * ks + 8 * g + e) * N2 + 16 * cb + li];
        // X̄ goes to LDS by direct copies: 16-byte slot s holds row s / RS,
        // chunk s % RS (RS = XROW / 16); the chunks past the row's N2 / 8 and
        // the slots past the token are padding (copied from the token's first
        // chunk, never read)
        {
            constexpr int RS = C::XROW / 16;
            const uint16_t* xb = p.X + static_cast<size_t>(m) * K;
            for (int j = wave; j < C::XCOPIES; j += NW) {
                const int s = j * 64 + lane;
                const int r = s / RS;
                const int c = s - r * RS;
                const uint32_t off = (r < N1 && c < N2 / 8) ? static_cast<uint32_t>(r * N2 * 2 + c * 16) : 0u;
                dma16_async_sv(xb, off, xs + j * 1024);
            }
        }
        constexpr int PIECES = N1 * 4;
        constexpr int MAXI = (PIECES + NT - 1) / NT;
        float4 pv[MAXI];
#pragma unroll
        for (int i = 0; i < MAXI; ++i) {
            const int idx = min(tid + i * NT, PIECES - 1);
            const int rho = idx >> 2;
            const int c4 = idx & 3;
            pv[i] = *reinterpret_cast<const float4*>(p.P1 + static_cast<size_t>(rho) * N1 + 16 * part + 4 * c4);
        }
        // all loads in flight before the first use of any
        __builtin_amdgcn_sched_barrier(0);
        float m1 = 0.0f;
#pragma unroll
        for (int i = 0; i < MAXI; ++i)
            if (tid + i * NT < PIECES)
                m1 = fmaxf(m1, fmaxf(fmaxf(fabsf(pv[i].x), fabsf(pv[i].y)),
                                     fmaxf(fabsf(pv[i].z), fabsf(pv[i].w))));
        m1 = wave_max(m1);
        if (lane == 0) red8[wave] = m1;
        // this wave's copies of X̄ have landed; after the barrier every wave's have
        wait_vmcnt<0>();
        __syncthreads();
        m1 = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) m1 = fmaxf(m1, red8[w]);
        const int e1 = m1 > 0.0f ? -ilog2f(m1) : 0;
        // fragment sk, lane (gg, ii), element e holds P1[rho][16 part + ii]
        // with rho = 32 sk + 4 gg + e (e < 4) or 32 sk + 16 + 4 gg + (e - 4)
#pragma unroll
        for (int i = 0; i < MAXI; ++i) {
            const int idx = tid + i * NT;
            if (idx < PIECES) {
                const int rho = idx >> 2;
                const int c4 = idx & 3;
                const int sk = rho >> 5;
                const int rr = rho & 31;
                const int gg = (rr & 15) >> 2;
                const int e = (rr & 3) + ((rr >> 4) << 2);
                const float vv[4] = {pv[i].x, pv[i].y, pv[i].z, pv[i].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = 4 * c4 + q;
                    const int off = (sk * 64 + gg * 16 + col) * 8 + e;
                    const float v = ldexpf(vv[q], e1);
                    {
                        const F16Pair hl = split_f16(v);
                        p1hi[off] = hl.hi;
                        p1lo[off] = hl.lo;
                    }
                }
            }
        }
        __syncthreads();

        // P2 fragments of this wave's 16 columns, prescaled per wave
        float m2 = 0.0f;
#pragma unroll
        for (int ks = 0; ks < C::KS1; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) m2 = fmaxf(m2, fabsf(p2v[ks][e]));
        m2 = wave_max(m2);
        const int e2 = m2 > 0.0f ? -ilog2f(m2) : 0;
        v8h p2hi[C::KS1], p2lo[C::KS1];
#pragma unroll
        for (int ks = 0; ks < C::KS1; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = ldexpf(p2v[ks][e], e2);
                {
                    const F16Pair hl = split_f16(v);
                    p2hi[ks][e] = hl.hi;
                    p2lo[ks][e] = hl.lo;
                }
            }

        // stage 1: T[:, cb] = X̄ · P2'[:, cb]
        v4f T[C::RB];
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) {
            v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < C::KS1; ++ks) {
                const v8h a = *reinterpret_cast<const v8h*>(xs + (16 * rb + li) * C::XROW + (32 * ks + 8 * g) * 2);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, p2hi[ks], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, p2lo[ks], acc, 0, 0, 0);
            }
            T[rb] = acc;
        }
        float tm = 0.0f;
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r) tm = fmaxf(tm, fabsf(T[rb][r]));
        tm = wave_max(tm);
        const int et = tm > 0.0f ? 14 - ilog2f(tm) : 0;
        // stage-2 B operand: accumulator rows 4g+r of row blocks 2s and 2s+1
        v8h bh[C::KS2], bl[C::KS2];
#pragma unroll
        for (int sk = 0; sk < C::KS2; ++sk)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int rb = 2 * sk + (e >> 2);
                const float v = ldexpf(T[rb][e & 3], et);
                {
                    const F16Pair hl = split_f16(v);
                    bh[sk][e] = hl.hi;
                    bl[sk][e] = hl.lo;
                }
            }
        // stage 2: rows 16 part .. 16 part + 15 of Z, columns of block cb
        v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int sk = 0; sk < C::KS2; ++sk) {
            const int off = (sk * 64 + lane) * 8;
            const v8h ah = *reinterpret_cast<const v8h*>(p1hi + off);
            const v8h al = *reinterpret_cast<const v8h*>(p1lo + off);
            z = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh[sk], z, 0, 0, 0);
            z = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl[sk], z, 0, 0, 0);
            z = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh[sk], z, 0, 0, 0);
        }
        const int unscale = -(e1 + e2 + et);
        const int row0 = 16 * part + 4 * g;          // lane holds rows row0 + r, column 16 cb + li
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = ldexpf(z[r], unscale);
        uint64_t* tok = p.sync;
        uint64_t* tokmax = p.sync + kSyncTokMax;
        uint64_t* ready = p.sync + kSyncReady;

        // the token scale: dynamic, the absmax over the token's units, which
        // meet at a barrier of the token's producers; static, the step
        float s = 1.0f;
        if (!is_static) {
            float wmax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
            wmax = wave_max(wmax);
            if (lane == 0) red8[wave] = wmax;
            __syncthreads();
            if (tid == 0) {
                float um = 0.0f;
#pragma unroll
                for (int w = 0; w < NW; ++w) um = fmaxf(um, red8[w]);
                // tagged maximum: the call's epoch in the high word dominates
                // every older value; non-negative floats order like their bits
                __hip_atomic_fetch_max(&tokmax[m], (static_cast<uint64_t>(p.epoch) << 32) | __float_as_uint(um),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                tagged_add(&tok[m], p.epoch);
                const uint64_t full = (static_cast<uint64_t>(p.epoch) << 32) | static_cast<uint32_t>(C::RB);
                const uint64_t start = __builtin_amdgcn_s_memrealtime();
                while (__hip_atomic_load(&tok[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != full) {
                    __builtin_amdgcn_s_sleep(2);
                    if (__builtin_amdgcn_s_memrealtime() - start > kLdWaitTicks) {
                        __hip_atomic_fetch_or(reinterpret_cast<uint32_t*>(p.sync) + kSyncErr, 2u,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                }
                const uint64_t tm64 = __hip_atomic_load(&tokmax[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                red8[0] = p.aq.alpha * __uint_as_float(static_cast<uint32_t>(tm64)) / p.aq.qmax;
            }
            __syncthreads();
            s = red8[0];
        } else if (!p.aq.per_channel) {
            s = p.aq.steps[0];
        }
        const bool pc = is_static && p.aq.per_channel;
        const bool zero = !(s > 0.0f);
        const float inv = zero ? 0.0f : 1.0f / s;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int k = (row0 + r) * N2 + 16 * cb + li;
            const uint32_t nib = pc ? quant_nibble_magic(v[r], __builtin_amdgcn_rcpf(p.aq.steps[k]),
                                                         p.aq.qmax)
                                    : quant_nibble(v[r], inv, zero, p.aq.qmax);
            const uint32_t odd = lane_xor1(nib);
            if ((li & 1) == 0) qs[((4 * g + r) * N2 + 16 * cb + li) >> 1] = static_cast<uint8_t>(nib | (odd << 4));
        }
        __syncthreads();
        if (tid < C::QBYTES / 16)
            reinterpret_cast<uint4*>(p.Xq + static_cast<size_t>(m) * (K / 2) + 16 * part * (N2 / 2))[tid] =
                reinterpret_cast<const uint4*>(qs)[tid];
        if (tid == 0 && part == 0) p.s_x[m] = s;
        __threadfence();                              // release this unit's codes
        __syncthreads();
        if (tid == 0) tagged_add(ready, p.epoch);
        __syncthreads();                              // producer LDS is dead
    }

    // =====================================================================
    // Consumer: 16 output columns, the decode GEMM loop
    // =====================================================================
    const int N = p.N;
    const int n0 = blockIdx.x * 16;
    if (n0 >= N) return;                              // a producer-only workgroup
    const int frow = lane & 15;
    const int fks = lane >> 4;
    constexpr int KB = K / 2;
    constexpr int KT = K / kLdBK;
    const int TPG = p.group_size / kLdBK;
    const int G = K / p.group_size;
    const int t0 = (KT * wave) / NW;
    const int t1 = (KT * (wave + 1)) / NW;
    const int GP = G + 1;                             // scale-table row: odd word count
    constexpr int AP = KB + 16;                       // staged activation row
    uint32_t* sz = reinterpret_cast<uint32_t*>(lds);
    uint8_t* al = lds + (SZ ? 16 * GP * 4 : 0);

    if constexpr (SZ) {
        for (int r = wave; r < 16; r += NW) {
            const size_t nrow = static_cast<size_t>(min(n0 + r, N - 1)) * G;
            for (int gb = 0; gb < G; gb += 256) {
                uint32_t v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int gi = min(gb + lane + 64 * j, G - 1);
                    v[j] = (MODE == kLdGroup) ? p.s_w[nrow + gi] : 0u;
                    if constexpr (ASYM) v[j] |= static_cast<uint32_t>(h2f(p.z_w[nrow + gi])) << 16;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (gb + lane + 64 * j < G) sz[r * GP + gb + lane + 64 * j] = v[j];
            }
        }
    }

    const uint32_t aoff = static_cast<uint32_t>(min(frow, M - 1)) * AP + fks * 16;
    const int rown = min(n0 + frow, N - 1) - n0;
    const uint32_t boff = static_cast<uint32_t>(rown) * KB + fks * 16;
    const uint32_t zoff = static_cast<uint32_t>(frow) * GP;
    const uint8_t* wbase = p.Wq + static_cast<size_t>(n0) * KB;

    v4i acc = v4i{0, 0, 0, 0};
    float facc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    uint4 bbuf[D];
    v4i zc;
    {
        int z0;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z0));
        zc = v4i{z0, z0, z0, z0};
    }
    int it = t0;
    auto issue = [&](auto S) {
        constexpr int SL = decltype(S)::value;
        bbuf[SL] = *reinterpret_cast<const uint4*>(wbase + static_cast<size_t>(it) * 64 + boff);
        it = min(it + 1, t1 - 1);
    };
    // the first weight tiles are in flight while the activations are made
    if (t0 < t1) static_for<0, D - 1>([&](auto U) { issue(U); });

    // ---- wait until every token is packed -----------------------------------
    if (tid == 0) {
        const uint32_t need = static_cast<uint32_t>(units);
        const uint64_t target = (static_cast<uint64_t>(p.epoch) << 32) | need;
        const uint64_t start = __builtin_amdgcn_s_memrealtime();
        int ok = 1;
        while (__hip_atomic_load(p.sync + kSyncReady, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != target) {
            // a few hundred cycles between polls keeps the polling traffic of
            // every waiting workgroup off the producers' atomics
            __builtin_amdgcn_s_sleep(10);
            if (__builtin_amdgcn_s_memrealtime() - start > kLdWaitTicks) {
                ok = 0;
                break;
            }
        }
        if (!ok)
            __hip_atomic_fetch_or(reinterpret_cast<uint32_t*>(p.sync) + kSyncErr, 1u, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();

    // ---- stage the M activation rows in LDS ---------------------------------
    {
        // 16-byte chunks, four loads in flight per thread (clamped addresses;
        // a clamped slot rewrites the last chunk with its own value)
        constexpr int CH = KB / 16;
        const int total = M * CH;
        // device-coherent loads (scope bit sc1): the codes were written back
        // by their producers before the ready counter moved, and these loads
        // read them at the device's point of coherence, with no cache
        // invalidation that would also drop the other workgroups' lines
        const __amdgpu_buffer_rsrc_t xrs =
            __builtin_amdgcn_make_buffer_rsrc(p.Xq, 0, M * KB, 0x00020000);
        auto ld = [&](int i) {
            return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrs, i * 16, 0, kCoherentLoad));
        };
        auto dst = [&](int i) {
            const int r = i / CH;
            return reinterpret_cast<uint4*>(al + r * AP) + (i - r * CH);
        };
        for (int i0 = tid; i0 < total; i0 += 4 * NT) {
            const int ia = min(i0, total - 1), ib = min(i0 + NT, total - 1);
            const int ic = min(i0 + 2 * NT, total - 1), id = min(i0 + 3 * NT, total - 1);
            const uint4 va = ld(ia), vb = ld(ib), vc = ld(ic), vd = ld(id);
            *dst(ia) = va;
            *dst(ib) = vb;
            *dst(ic) = vc;
            *dst(id) = vd;
        }
    }
    __syncthreads();

    int cg = t0 / TPG, cr = t0 - (t0 / TPG) * TPG;
    auto compute = [&](int t, auto S) {
        constexpr int SL = decltype(S)::value;
        uint4 ev, od;
        unpack_signed16(*reinterpret_cast<const uint4*>(al + aoff + t * 64), ev, od);
        const v4i aev = v4i{static_cast<int>(ev.x), static_cast<int>(ev.y), static_cast<int>(ev.z), static_cast<int>(ev.w)};
        const v4i aod = v4i{static_cast<int>(od.x), static_cast<int>(od.y), static_cast<int>(od.z), static_cast<int>(od.w)};
        uint32_t szv = 0;
        if constexpr (SZ) szv = sz[zoff + (G1 ? t : cg)];
        if constexpr (ASYM) {
            const uint32_t zp = szv >> 16;
            unpack_asym(bbuf[SL], 0x80808080u - zp * 0x01010101u, ev, od);
        } else {
            unpack_signed16(bbuf[SL], ev, od);
        }
        const v4i bev = v4i{static_cast<int>(ev.x), static_cast<int>(ev.y), static_cast<int>(ev.z), static_cast<int>(ev.w)};
        const v4i bod = v4i{static_cast<int>(od.x), static_cast<int>(od.y), static_cast<int>(od.z), static_cast<int>(od.w)};
        if constexpr (G1) {
            // one tile per weight group: the group sum starts from a zero
            // register operand and is folded into fp32 at once
            const float sw = h2f(static_cast<uint16_t>(szv & 0xFFFFu));
            v4i q = __builtin_amdgcn_mfma_i32_16x16x64_i8(aev, bev, zc, 0, 0, 0);
            q = __builtin_amdgcn_mfma_i32_16x16x64_i8(aod, bod, q, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) facc[r] = fmaf(static_cast<float>(q[r]), sw, facc[r]);
            return;
        }
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aev, bev, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aod, bod, acc, 0, 0, 0);
        const bool group_end = (++cr == TPG);
        if constexpr (MODE == kLdGroup) {
            if (group_end || t + 1 == t1) {
                const float sw = h2f(static_cast<uint16_t>(szv & 0xFFFFu));
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    facc[r] = fmaf(static_cast<float>(acc[r]), sw, facc[r]);
                    acc[r] = 0;
                }
            }
        }
        if (group_end) {
            cr = 0;
            ++cg;
        }
    };

    // whole groups of D tiles with no branch around a step and the step's
    // load kept ahead of its arithmetic (as in the decode GEMM), then the
    // last tiles, whose loads are in flight; tile t uses slot (t - t0) % D
    if (t0 < t1) {
        int t = t0;
        for (; t + D <= t1; t += D) {
            static_for<0, D>([&](auto U) {
                constexpr int u = decltype(U)::value;
                issue(std::integral_constant<int, (u + D - 1) % D>{});
                __builtin_amdgcn_sched_barrier(0);
                compute(t + u, std::integral_constant<int, u>{});
            });
        }
        static_for<0, D - 1>([&](auto U) {
            constexpr int u = decltype(U)::value;
            if (t + u < t1) compute(t + u, std::integral_constant<int, u>{});
        });
    }

    // ---- add the waves' partial sums in LDS, in wave order ------------------
    __syncthreads();                                  // the staged data is dead
    float* red = reinterpret_cast<float*>(lds);       // [NW][4][64]
#pragma unroll
    for (int r = 0; r < 4; ++r)
        red[(wave * 4 + r) * 64 + lane] = (MODE == kLdGroup) ? facc[r] : __int_as_float(acc[r]);
    __syncthreads();
    constexpr float kUnshift = ASYM ? (1.0f / 16.0f) : (1.0f / 256.0f);
    if (tid < 4 * 64) {
        const int r = tid >> 6;
        const int l = tid & 63;
        const int gm = 4 * (l >> 4) + r;
        const int gn = n0 + (l & 15);
        if (gm < M && gn < N) {
            float v;
            if constexpr (MODE == kLdGroup) {
                v = 0.0f;
#pragma unroll
                for (int w = 0; w < NW; ++w) v += red[(w * 4 + r) * 64 + l];
            } else {
                int sum = 0;
#pragma unroll
                for (int w = 0; w < NW; ++w) sum += __float_as_int(red[(w * 4 + r) * 64 + l]);
                v = static_cast<float>(sum) * h2f(p.s_w[gn]);
            }
            // the token scale, like the codes, with a device-coherent load
            const float sxm = __hip_atomic_load(&p.s_x[gm], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            p.Y[static_cast<size_t>(gm) * N + gn] = f2h(v * sxm * kUnshift);
        }
    }
}

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

std::atomic<uint32_t> g_epoch{0};

// LDS bytes of the consumer part: scale table + staged activations (the
// reduction buffer reuses them and is smaller)
size_t consumer_lds(int M, int K, int group_size, bool asym) {
    const int G = K / group_size;
    const bool sz = (group_size != K) || asym;
    const size_t szb = sz ? static_cast<size_t>(16) * (G + 1) * 4 : 0;
    const size_t red = static_cast<size_t>(kLdWaves) * 4 * 64 * 4;
    const size_t need = szb + static_cast<size_t>(M) * (K / 2 + 16);
    return need > red ? need : red;
}

// dry: only report the resident workgroups of the device at this LDS size
template <int N1, bool ASYM, int MODE, bool G1>
hipError_t launch_t(const LdArgs& a, hipStream_t stream, bool dry, int* cap) {
    using C = LdCfg<N1>;
    auto* kern = &k_linear_dec<N1, ASYM, MODE, G1>;
    size_t lds = consumer_lds(a.M, C::K, a.group_size, ASYM);
    if (lds < static_cast<size_t>(C::PROD_LDS)) lds = C::PROD_LDS;
    static bool raised[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) dev = 63;
    if (!raised[dev]) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kLdLdsMax);
        if (e != hipSuccess) return e;
        raised[dev] = true;
    }
    if (dry) {
        // resident workgroups: VGPR-limited waves per SIMD (512 registers,
        // granule 8) and the CU's LDS, four SIMDs per CU
        hipFuncAttributes fa;
        e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kern));
        if (e != hipSuccess) return e;
        const int regs = ((fa.numRegs > 0 ? fa.numRegs : 1) + 7) / 8 * 8;
        int waves_simd = 512 / regs;
        if (waves_simd > 8) waves_simd = 8;
        const int by_regs = (4 * waves_simd) / kLdWaves;
        const int by_lds = static_cast<int>(static_cast<size_t>(kLdLdsCU) / (lds + fa.sharedSizeBytes));
        const int n = by_regs < by_lds ? by_regs : by_lds;
        *cap = n * device_cu_count();
        return hipSuccess;
    }
    const int units = a.M * C::RB;
    const int grid = ceil_div(a.N, 16) > units ? ceil_div(a.N, 16) : units;
    kern<<<dim3(grid), dim3(kLdThreads), lds, stream>>>(a);
    return hipGetLastError();
}

using LdLaunch = hipError_t (*)(const LdArgs&, hipStream_t, bool, int*);

template <int N1>
LdLaunch pick_mode(bool asym, int K, int group_size) {
    if (group_size == K) return asym ? &launch_t<N1, true, kLdChan, false> : &launch_t<N1, false, kLdChan, false>;
    if (group_size == kLdBK)
        return asym ? &launch_t<N1, true, kLdGroup, true> : &launch_t<N1, false, kLdGroup, true>;
    return asym ? &launch_t<N1, true, kLdGroup, false> : &launch_t<N1, false, kLdGroup, false>;
}

LdLaunch pick(int n1, bool asym, int K, int group_size) {
    switch (n1) {
        case 64: return pick_mode<64>(asym, K, group_size);
        case 224: return pick_mode<224>(asym, K, group_size);
        default: return nullptr;
    }
}

}  // namespace

size_t linear_decode_workspace_bytes(int M, int n1, int n2) {
    const size_t K = static_cast<size_t>(n1) * n2;
    return align256(K / 2 * M) + align256(sizeof(float) * M);
}

// 0: supported; 1: shape not covered; 2: too much LDS; 3: producers exceed the
// resident capacity of the device (*cap) or it could not be queried
int linear_decode_check(int M, int n1, int n2, int N, int K, int group_size, bool asym, int* capp) {
    if (n2 != kLdN2 || M < 1 || M > 16 || pick(n1, asym, K, group_size) == nullptr) return 1;
    if (consumer_lds(M, K, group_size, asym) > static_cast<size_t>(kLdLdsMax)) return 2;
    LdArgs a{};
    a.M = M;
    a.N = N;
    a.group_size = group_size;
    int cap = -1;
    const hipError_t e = pick(n1, asym, K, group_size)(a, nullptr, true, &cap);
    *capp = e == hipSuccess ? cap : -static_cast<int>(e);
    if (e != hipSuccess || M * (n1 / 16) > cap) return 3;
    return 0;
}

hipError_t linear_decode_launch(const uint16_t* X, int M, int n1, int n2, const float* P1,
                                const float* P2, ActQuant aq, const GemmArgs& g, void* ws,
                                uint32_t* sync, hipStream_t stream) {
    const size_t K = static_cast<size_t>(n1) * n2;
    char* q = static_cast<char*>(ws);
    LdArgs a{};
    a.X = X;
    a.P1 = P1;
    a.P2 = P2;
    a.aq = aq;
    a.Wq = g.Wq;
    a.s_w = g.s_w;
    a.z_w = g.z_w;
    a.Y = g.Y;
    a.Xq = reinterpret_cast<uint8_t*>(q);
    q += align256(K / 2 * M);
    a.s_x = reinterpret_cast<float*>(q);
    a.sync = reinterpret_cast<uint64_t*>(sync);
    a.M = M;
    a.N = g.N;
    a.group_size = g.group_size;
    uint32_t ep = ++g_epoch;
    if (ep == 0) ep = ++g_epoch;                      // 0 would match a zeroed buffer
    a.epoch = ep;
    LdLaunch f = pick(n1, g.asym, g.K, g.group_size);
    if (f == nullptr) return hipErrorInvalidValue;
    int cap = 0;
    return f(a, stream, false, &cap);
}

}  // namespace w4a4
