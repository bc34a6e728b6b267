// Online activation path: Kronecker transform, per-token scale, INT4
// quantization and nibble packing.
//
// FlatQuant: Flatness Matters for LLM Quantization — section Kronecker 分解
// (activation factor P1^T ×1 X̃ ×2 P2, equal to x·(P1 ⊗ P2) for a row-major
// reshape), section 额外可学习组件 (diag(c) before the transform, clip α_a),
// section 高效 Kernel 设计 (transform and quantize one token tile on chip).
// FRM-PTQ page, section 初步介绍 (uniform quantizer, here symmetric 4-bit).
//
// Fused path (n1, n2 multiples of 16, n1 <= 128, n2 in {16, 32, 64, 128},
// no diag(c)): one kernel, persistent workgroups of max(4, n2/16) waves, one
// token (or 2-4 tokens when n2 <= 32) per workgroup iteration, each wave
// owning one 16-column block of its token, everything on chip:
//   stage 1  T = X̄ · P2 on v_mfma_f32_16x16x32_f16.  X̄ is fp16 and exact as
//            an operand; P2 is split into fp16 hi + lo (two MFMAs), after a
//            power-of-two prescale putting max|P2| in [1, 2).  The wave's P2
//            fragments stay in VGPRs for the life of the workgroup.
//   stage 2  Z = P1^T · T.  T never leaves the accumulators: its fp32 values,
//            prescaled per wave by a power of two so max|T| is in
//            [2^14, 2^15), are split into fp16 hi + lo and used directly as
//            the B operand (the k order of the MFMA is chosen to match the
//            accumulator layout).  P1 hi/lo fragments live in LDS, in the
//            same k order.  Three MFMAs: hi*hi + hi*lo + lo*hi, i.e. about 22
//            significant bits per product and fp32 accumulation.
//   quant    per-token absmax by DPP wave reductions + LDS, t = z * (1/s),
//            round half to even,
//            nibble pairs formed across neighbouring lanes, packed bytes
//            staged in LDS and written with coalesced 16-byte stores.
// Power-of-two scalings are exact and undone before quantization.
//
// Split path (any n1, n2 up to 256, and diag(c)): three stream-ordered fp32
// FMA kernels with a workspace holding T = X̄·P2 and Z = P1^T·T:
//   stage1  one block per (token m, row r of X̄): T[m, r, :]
//   stage2  one thread per element of Z, block absmax -> atomicMax per token
//   quant   8 codes per thread -> one packed 32-bit store
#include "common.hpp"
#include "internal.hpp"

namespace w4a4 {

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kSplitThreads = 256;

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

__global__ __launch_bounds__(256) void k_tq_stage1(const uint16_t* __restrict__ X, int K,
                                                   int n2, const float* __restrict__ P2,
                                                   const float* __restrict__ c,
                                                   float* __restrict__ T,
                                                   uint32_t* __restrict__ amax) {
    __shared__ float xs[W4A4_MAX_FACTOR];
    const int m = blockIdx.x;
    const int r = blockIdx.y;
    const size_t base = static_cast<size_t>(m) * K + static_cast<size_t>(r) * n2;
    for (int j = threadIdx.x; j < n2; j += blockDim.x) {
        float v = h2f(X[base + j]);
        if (c) v *= c[static_cast<size_t>(r) * n2 + j];
        xs[j] = v;
    }
    if (r == 0 && threadIdx.x == 0) amax[m] = 0u;
    __syncthreads();
    for (int j = threadIdx.x; j < n2; j += blockDim.x) {
        float acc = 0.0f;
        for (int q = 0; q < n2; ++q) acc = fmaf(xs[q], P2[static_cast<size_t>(q) * n2 + j], acc);
        T[base + j] = acc;
    }
}

__global__ __launch_bounds__(256) void k_tq_stage2(const float* __restrict__ T, int K, int n1,
                                                   int n2, const float* __restrict__ P1,
                                                   float* __restrict__ Z,
                                                   uint32_t* __restrict__ amax) {
    __shared__ float red[kSplitThreads / 64];
    const int m = blockIdx.x;
    const int e = blockIdx.y * blockDim.x + threadIdx.x;
    float v = 0.0f;
    if (e < K) {
        const int i = e / n2;
        const int j = e - i * n2;
        const float* Tm = T + static_cast<size_t>(m) * K;
        float acc = 0.0f;
        for (int r = 0; r < n1; ++r)
            acc = fmaf(P1[static_cast<size_t>(r) * n1 + i], Tm[static_cast<size_t>(r) * n2 + j], acc);
        Z[static_cast<size_t>(m) * K + e] = acc;
        v = fabsf(acc);
    }
    v = wave_max(v);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = red[0];
        for (int w = 1; w < static_cast<int>(blockDim.x >> 6); ++w) b = fmaxf(b, red[w]);
        // non-negative floats order like their bit patterns
        atomicMax(&amax[m], __float_as_uint(b));
    }
}

__global__ __launch_bounds__(256) void k_tq_quant(const float* __restrict__ Z, int K, ActQuant aq,
                                                  const uint32_t* __restrict__ amax, int nparts,
                                                  uint8_t* __restrict__ Xq,
                                                  float* __restrict__ s_x) {
    const int m = blockIdx.x;
    const int idx = blockIdx.y * blockDim.x + threadIdx.x;
    const int e0 = idx * 8;
    const int ec = min(e0, K - 8);
    // this thread's 8 values (loaded before the scale is known)
    float z[8];
    const float* zp = Z + static_cast<size_t>(m) * K + ec;
#pragma unroll
    for (int t = 0; t < 8; ++t) z[t] = zp[t];
    float s;
    if (aq.steps == nullptr) {
        // the token's absmax: the largest of its partial maxima (bit patterns
        // of non-negative floats order like the floats), reduced by the
        // workgroup
        __shared__ float red[4];
        float ab = 0.0f;
        for (int q = threadIdx.x; q < nparts; q += 256)
            ab = fmaxf(ab, __uint_as_float(amax[static_cast<size_t>(m) * nparts + q]));
        ab = wave_max(ab);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ab;
        __syncthreads();
        ab = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        s = aq.alpha * ab / aq.qmax;
    } else {
        s = aq.per_channel ? 1.0f : aq.steps[0];
    }
    if (idx == 0) s_x[m] = s;
    if (e0 >= K) return;
    uint32_t word = 0;
    if (aq.steps != nullptr && aq.per_channel) {
        const v4f st0 = *reinterpret_cast<const v4f*>(aq.steps + ec);
        const v4f st1 = *reinterpret_cast<const v4f*>(aq.steps + ec + 4);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            word |= quant_nibble_magic(z[t], __builtin_amdgcn_rcpf(st0[t]), aq.qmax) << (4 * t);
            word |= quant_nibble_magic(z[t + 4], __builtin_amdgcn_rcpf(st1[t]), aq.qmax) << (4 * (t + 4));
        }
    } else {
        const bool zero = !(s > 0.0f);
        const float inv = zero ? 0.0f : 1.0f / s;
#pragma unroll
        for (int t = 0; t < 8; ++t) word |= quant_nibble(z[t], inv, zero, aq.qmax) << (4 * t);
    }
    reinterpret_cast<uint32_t*>(Xq + static_cast<size_t>(m) * (K / 2))[idx] = word;
}


// Static per-channel steps through a buffer resource: the per-lane part of
// a channel's byte offset sits in one VGPR and the part fixed at compile
// time in the scalar offset, so a batch of step loads needs no 64-bit
// address registers (reads past K return 0 and are never used).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t steps_rsrc(const float* steps, int K) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(steps), 0, K * 4, 0x00020000);
}

// Per-token group sums of the codes for the zero-point correction of the
// GEMM (asymmetric weights, groups of 128 codes): 16 * Σ_{k in g} q[m,k] as
// fp16 (|16 S| <= 16384, exact), the values the GEMM's own pre-pass would
// write.  A group is 64 packed bytes, i.e. four consecutive 16-byte chunks of
// the token's packed row; the four lanes that store them add their chunk
// sums (the chunk index is the lane index plus a multiple of 64, so a group
// sits in four consecutive lanes, all active or all inactive).
__device__ __forceinline__ int nibble_sum(uint32_t w) {
    // two's complement nibbles: the unsigned nibble sum less 16 per negative code
    const uint32_t u = (w & 0x0F0F0F0Fu) + ((w >> 4) & 0x0F0F0F0Fu);
    return static_cast<int>((u * 0x01010101u) >> 24) - 16 * __builtin_popcount(w & 0x88888888u);
}

__device__ __forceinline__ void store_group_sum(const uint4& v, int chunk, uint16_t* srow) {
    int sum = nibble_sum(v.x) + nibble_sum(v.y) + nibble_sum(v.z) + nibble_sum(v.w);
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    if ((chunk & 3) == 0) srow[chunk >> 2] = f2h(static_cast<float>(16 * sum));
}

// ===========================================================================
// Fused MFMA path
// ===========================================================================

template <int N1, int N2>
struct FusedCfg {
    static_assert(N1 % 16 == 0 && N2 % 16 == 0, "factors must be multiples of 16");
    static constexpr int K = N1 * N2;
    static constexpr int RB = N1 / 16;           // 16-row blocks of X̄, T and Z
    static constexpr int CB = N2 / 16;           // 16-column blocks, one wave each
    static constexpr int KS1 = (N2 + 31) / 32;   // stage-1 MFMA k-steps
    static constexpr int KS2 = (N1 + 31) / 32;   // stage-2 MFMA k-steps
    static constexpr int NW = CB < 4 ? 4 : CB;   // waves per workgroup
    static constexpr int NT = NW * 64;           // threads per workgroup
    static constexpr int TPI = NW / CB;          // tokens per workgroup iteration
    static_assert(NW % CB == 0 && NW <= 8, "unsupported n2");
    static constexpr int P1F = RB * KS2 * 64 * 8;  // fp16 elements of one P1 fragment set
    // X̄ staging: token rows padded so that the 16 rows one MFMA operand
    // read touches fall in distinct LDS banks.  Rows of 256 bytes take 32
    // bytes of padding: with 16 the bank-conflict counter showed 4 cycles per
    // ds_read_b128 of this pattern (16 rows x 4 chunks), with 32 none.
    static constexpr int XROW = N2 * 2 + ((N2 * 2) % 256 == 0 ? 32 : 16);   // bytes per staged row
    static constexpr int XSLOT = N1 * XROW;        // bytes per staged token
    static constexpr int XCH = K / 8;              // 16-byte chunks per token in HBM
    static constexpr int XLD = (TPI * XCH + NT - 1) / NT;  // chunks per thread per tile
};

// PC: static per-channel steps (a separate instantiation, so that the
// per-token paths carry none of its registers)
template <int N1, int N2, bool PC>
__global__ __launch_bounds__((FusedCfg<N1, N2>::NT)) void k_tq_fused(const uint16_t* __restrict__ X, int M,
                                                  const float* __restrict__ P1,
                                                  const float* __restrict__ P2, ActQuant aq,
                                                  uint8_t* __restrict__ Xq,
                                                  float* __restrict__ s_x,
                                                  float* __restrict__ Zout,
                                                  uint16_t* __restrict__ S16, int Gp) {
    using C = FusedCfg<N1, N2>;
    constexpr int K = C::K;
    __shared__ __align__(16) _Float16 p1hi[C::P1F];
    __shared__ __align__(16) _Float16 p1lo[C::P1F];
    __shared__ __align__(16) uint8_t qbuf[C::TPI * K / 2];
    __shared__ __align__(16) uint8_t xs[2][C::TPI * C::XSLOT];
    constexpr int NT = C::NT;
    __shared__ float red[2 * C::NW];
    __shared__ float tok_s[C::TPI];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int li = lane & 15;

    // ---- power-of-two prescale of the factors ------------------------------
    float m1 = 0.0f, m2 = 0.0f;
#pragma unroll
    for (int i = 0; i < (N1 * N1 + NT - 1) / NT; ++i) {
        const int e = tid + i * NT;
        if (e < N1 * N1) m1 = fmaxf(m1, fabsf(P1[e]));
    }
#pragma unroll
    for (int i = 0; i < (N2 * N2 + NT - 1) / NT; ++i) {
        const int e = tid + i * NT;
        if (e < N2 * N2) m2 = fmaxf(m2, fabsf(P2[e]));
    }
    m1 = wave_max(m1);
    m2 = wave_max(m2);
    if (lane == 0) {
        red[wave] = m1;
        red[C::NW + wave] = m2;
    }
    __syncthreads();
    m1 = 0.0f;
    m2 = 0.0f;
#pragma unroll
    for (int w = 0; w < C::NW; ++w) {
        m1 = fmaxf(m1, red[w]);
        m2 = fmaxf(m2, red[C::NW + w]);
    }
    const int e1 = m1 > 0.0f ? -ilog2f(m1) : 0;   // max|P1 * 2^e1| in [1, 2)
    const int e2 = m2 > 0.0f ? -ilog2f(m2) : 0;

    // ---- P1 fragments (stage-2 A operand) into LDS ---------------------------
    // fragment (ob, s), lane (gg, ii), element e holds P1[rho][16*ob + ii],
    // rho = 32s + 4gg + e (e < 4) or 32s + 16 + 4gg + (e - 4) (e >= 4): the
    // rows of T that the stage-1 accumulators of lane group gg hold.
#pragma unroll
    for (int i = 0; i < (C::P1F + NT - 1) / NT; ++i) {
        const int idx = tid + i * NT;
        if (idx >= C::P1F) break;
        const int e = idx & 7;
        const int ln = (idx >> 3) & 63;
        const int slot = idx >> 9;
        const int sk = slot % C::KS2;
        const int ob = slot / C::KS2;
        const int gg = ln >> 4, ii = ln & 15;
        const int rho = 32 * sk + (e < 4 ? 4 * gg + e : 16 + 4 * gg + (e - 4));
        const float v = rho < N1 ? ldexpf(P1[rho * N1 + 16 * ob + ii], e1) : 0.0f;
        {
            const F16Pair hl = split_f16(v);
            p1hi[idx] = hl.hi;
            p1lo[idx] = hl.lo;
        }
    }

    // ---- P2 fragments (stage-1 B operand) of this wave's 16 columns ---------
    const int tslot = wave / C::CB;
    const int cb = wave % C::CB;
    v8h p2hi[C::KS1], p2lo[C::KS1];
#pragma unroll
    for (int ks = 0; ks < C::KS1; ++ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int kk = 32 * ks + 8 * g + e;
            const float v = kk < N2 ? ldexpf(P2[kk * N2 + 16 * cb + li], e2) : 0.0f;
            {
                const F16Pair hl = split_f16(v);
                p2hi[ks][e] = hl.hi;
                p2lo[ks][e] = hl.lo;
            }
        }
    }
    // ---- X̄ tiles: HBM -> registers (next tile) -> LDS (double buffer) --------
    uint4 xr[C::XLD];
    auto load_tile = [&](int b) {
#pragma unroll
        for (int i = 0; i < C::XLD; ++i) {
            const int c = tid + i * NT;
            const int t = c / C::XCH;
            if (c < C::TPI * C::XCH && b + t < M)
                xr[i] = reinterpret_cast<const uint4*>(X + static_cast<size_t>(b) * K)[c];
            else
                xr[i] = make_uint4(0, 0, 0, 0);
        }
    };
    auto stage_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < C::XLD; ++i) {
            const int c = tid + i * NT;
            if (c < C::TPI * C::XCH) {
                const int t = c / C::XCH;
                const int cc = c - t * C::XCH;
                const int row = cc / (N2 / 8);
                const int col = cc - row * (N2 / 8);
                *reinterpret_cast<uint4*>(&xs[buf][t * C::XSLOT + row * C::XROW + col * 16]) = xr[i];
            }
        }
    };
    const int stride = gridDim.x * C::TPI;
    int base = blockIdx.x * C::TPI;
    if (base < M) load_tile(base);
    stage_tile(0);
    // the token loop reuses red[] and reads xs[0] after this barrier
    __syncthreads();

    for (int it = 0; base < M; base += stride, ++it) {
        const int buf = it & 1;
        if (base + stride < M) load_tile(base + stride);   // in flight during compute
        const int m = base + tslot;
        const bool valid = m < M;
        v4f Z[C::RB];
        float wmax = 0.0f;
        int unscale = 0;
        if (valid) {
            const uint8_t* xt = &xs[buf][tslot * C::XSLOT];
            // stage 1: T[:, cb] = X̄ · P2'[:, cb]
            v4f T[C::RB];
#pragma unroll
            for (int rb = 0; rb < C::RB; ++rb) {
                v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int ks = 0; ks < C::KS1; ++ks) {
                    v8h a;
                    if (32 * ks + 8 * g < N2)
                        a = *reinterpret_cast<const v8h*>(xt + (16 * rb + li) * C::XROW +
                                                          (32 * ks + 8 * g) * 2);
                    else
                        a = v8h{0, 0, 0, 0, 0, 0, 0, 0};
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, p2hi[ks], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, p2lo[ks], acc, 0, 0, 0);
                }
                T[rb] = acc;
            }
            // per-wave power-of-two prescale of T into the fp16 range
            float tm = 0.0f;
#pragma unroll
            for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
                for (int r = 0; r < 4; ++r) tm = fmaxf(tm, fabsf(T[rb][r]));
            tm = wave_max(tm);
            const int et = tm > 0.0f ? 14 - ilog2f(tm) : 0;
            // stage-2 B operand: accumulator rows 4g+r of blocks 2s and 2s+1
            v8h bh[C::KS2], bl[C::KS2];
#pragma unroll
            for (int sk = 0; sk < C::KS2; ++sk) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int rb = 2 * sk + (e >> 2);
                    const float v = rb < C::RB ? ldexpf(T[rb < C::RB ? rb : 0][e & 3], et) : 0.0f;
                    {
                        const F16Pair hl = split_f16(v);
                        bh[sk][e] = hl.hi;
                        bl[sk][e] = hl.lo;
                    }
                }
            }
            // stage 2, transposed: Zᵀ = T'ᵀ · P1' with the split T as the A
            // operand in its accumulators' own k order and the P1 fragments
            // as the B operand (the fragment's rows rho are that order), so
            // lane (g, li) of tile ob holds 2^-unscale Z[16 ob + li][16 cb +
            // 4 g + r]: four consecutive channels of one row
            unscale = -(e1 + e2 + et);
#pragma unroll
            for (int ob = 0; ob < C::RB; ++ob) {
                v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int sk = 0; sk < C::KS2; ++sk) {
                    const int off = ((ob * C::KS2 + sk) * 64 + lane) * 8;
                    const v8h ah = *reinterpret_cast<const v8h*>(p1hi + off);
                    const v8h al = *reinterpret_cast<const v8h*>(p1lo + off);
                    z = __builtin_amdgcn_mfma_f32_16x16x32_f16(bh[sk], al, z, 0, 0, 0);
                    z = __builtin_amdgcn_mfma_f32_16x16x32_f16(bl[sk], ah, z, 0, 0, 0);
                    z = __builtin_amdgcn_mfma_f32_16x16x32_f16(bh[sk], ah, z, 0, 0, 0);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) wmax = fmaxf(wmax, fabsf(z[r]));
                Z[ob] = z;
            }
        }
        // ---- per-token absmax and scale ---------------------------------------
        // (each wave's power of two is applied to its maximum: exact)
        wmax = ldexpf(wave_max(wmax), unscale);
        if (lane == 0) red[wave] = wmax;
        __syncthreads();
        float amax = 0.0f;
#pragma unroll
        for (int w = 0; w < C::CB; ++w) amax = fmaxf(amax, red[tslot * C::CB + w]);
        // static steps: the token scale is the tensor's step (or 1 with
        // per-channel steps); the reduction above is then unused
        const float s_static = PC ? 1.0f : (aq.steps ? aq.steps[0] : 0.0f);
        const float s = aq.steps ? s_static : aq.alpha * amax / aq.qmax;
        if (tid < C::TPI) {
            float a2 = 0.0f;
            for (int w = 0; w < C::CB; ++w) a2 = fmaxf(a2, red[tid * C::CB + w]);
            tok_s[tid] = aq.steps ? s_static : aq.alpha * a2 / aq.qmax;
        }
        if (valid) {
            if (Zout != nullptr) {
                float* zo = Zout + static_cast<size_t>(m) * K;
#pragma unroll
                for (int ob = 0; ob < C::RB; ++ob) {
                    v4f zz;
#pragma unroll
                    for (int r = 0; r < 4; ++r) zz[r] = ldexpf(Z[ob][r], unscale);
                    *reinterpret_cast<v4f*>(zo + (16 * ob + li) * N2 + 16 * cb + 4 * g) = zz;
                }
            } else {
                // the wave's power of two goes into the quantizer's multiplier
                // (exact, so the codes are those of the unscaled values)
                const float inv = s > 0.0f ? ldexpf(1.0f / s, unscale) : 0.0f;
                uint8_t* qb = qbuf + tslot * (K / 2);
                const __amdgpu_buffer_rsrc_t srs = steps_rsrc(aq.steps, K);
                const int svoff = (li * N2 + 16 * cb + 4 * g) * 4;
#pragma unroll
                for (int ob = 0; ob < C::RB; ++ob) {
                    v4f rst;
                    if (PC) {
                        // this row block's four steps only (one 16-byte load):
                        // no batch of all the token's step loads competing
                        // for registers
                        asm volatile("" ::: "memory");
                        rst = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                                           srs, svoff, 16 * ob * N2 * 4, 0));
                    }
                    uint32_t w = 0;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint32_t nib =
                            PC ? quant_nibble_magic(ldexpf(Z[ob][r], unscale),
                                                    __builtin_amdgcn_rcpf(rst[r]), aq.qmax)
                               : quant_nibble_magic(Z[ob][r], inv, aq.qmax);
                        w |= nib << (4 * r);
                    }
                    const int k0 = (16 * ob + li) * N2 + 16 * cb + 4 * g;
                    *reinterpret_cast<uint16_t*>(qb + (k0 >> 1)) = static_cast<uint16_t>(w);
                }
            }
        }
        __syncthreads();
        // ---- coalesced store of the packed rows and the scales ----------------
        if (Zout == nullptr) {
            constexpr int CH = K / 32;     // 16-byte chunks per token row
            for (int c = tid; c < C::TPI * CH; c += NT) {
                const int t = c / CH;
                const int mm = base + t;
                if (mm < M) {
                    const uint4 v = reinterpret_cast<const uint4*>(qbuf)[c];
                    reinterpret_cast<uint4*>(Xq + static_cast<size_t>(mm) * (K / 2))[c - t * CH] = v;
                    if (S16 != nullptr) store_group_sum(v, c - t * CH, S16 + static_cast<size_t>(mm) * Gp);
                }
            }
            if (tid < C::TPI && base + tid < M) s_x[base + tid] = tok_s[tid];
            // the padding groups of the sums rows: zero
            if (S16 != nullptr && tid < C::TPI * (Gp - K / 128) && base + tid / (Gp - K / 128) < M) {
                const int t = tid / (Gp - K / 128);
                S16[static_cast<size_t>(base + t) * Gp + K / 128 + (tid - t * (Gp - K / 128))] = 0;
            }
        }
        // the buffer written here was last read one iteration ago, before two
        // barriers; the barrier below publishes it for the next iteration
        if (base + stride < M) stage_tile(buf ^ 1);
        __syncthreads();
    }
}

template <int N1, int N2, bool PC>
hipError_t launch_fused_k(const uint16_t* X, int M, const float* P1, const float* P2, ActQuant aq,
                          uint8_t* Xq, float* s_x, float* Z, uint16_t* S16, int Gp,
                          hipStream_t stream) {
    using C = FusedCfg<N1, N2>;
    // persistent grid: as many workgroups as fit on the device at once, so the
    // per-workgroup fragment setup is paid once per resident workgroup
    static int per_cu = 0;
    if (per_cu == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_tq_fused<N1, N2, PC>, C::NT, 0) !=
                hipSuccess || n < 1)
            n = 1;
        per_cu = n;
    }
    const int units = (M + C::TPI - 1) / C::TPI;
    const int cap = per_cu * device_cu_count();
    const int grid = units < cap ? units : cap;
    k_tq_fused<N1, N2, PC><<<grid, C::NT, 0, stream>>>(X, M, P1, P2, aq, Xq, s_x, Z, S16, Gp);
    return hipGetLastError();
}

// c: unused (the token-batched kernel has no diag(c); fused_for does not
// offer it for a layer with c)
template <int N1, int N2>
hipError_t launch_fused(const uint16_t* X, int M, const float* P1, const float* P2, const float* c,
                        ActQuant aq, uint8_t* Xq, float* s_x, float* Z, uint16_t* S16, int Gp,
                        hipStream_t stream) {
    (void)c;
    if (aq.steps != nullptr && aq.per_channel && Xq != nullptr)
        return launch_fused_k<N1, N2, true>(X, M, P1, P2, aq, Xq, s_x, Z, S16, Gp, stream);
    return launch_fused_k<N1, N2, false>(X, M, P1, P2, aq, Xq, s_x, Z, S16, Gp, stream);
}

// ===========================================================================
// Wave-per-token MFMA path (n1, n2 <= 64): one wave transforms, quantizes
// and packs a whole token with no workgroup barrier.  The workgroup stages
// the split P2 (stage-1 B operand) and P1 (stage-2 B operand) fragments in
// LDS once; each wave then walks its own tokens:
//   stage 1  T = X̄ · P2 as in the fused path, X̄ fragments loaded straight
//            from HBM one token ahead;
//   stage 2  computed transposed, Zᵀ = Tᵀ · P1: the split T accumulators are
//            the A operand in their own k order and the P1 fragments of the
//            fused path become the B operand, so each lane ends up holding
//            four consecutive channels of a row of Z;
//   quant    wave absmax (DPP), 4 codes -> 16 bits per lane and tile,
//            assembled in the wave's LDS slice and written as 16-byte rows.
// ===========================================================================
template <int N1, int N2>
struct WaveCfg {
    static_assert(N1 % 16 == 0 && N2 % 16 == 0 && N1 <= 64 && N2 <= 64, "small factors");
    static constexpr int K = N1 * N2;
    static constexpr int RB = N1 / 16;           // 16-row blocks of Z (rows i)
    static constexpr int CB = N2 / 16;           // 16-column blocks of Z (columns j)
    static constexpr int KS1 = (N2 + 31) / 32;   // stage-1 k-steps
    static constexpr int KS2 = (N1 + 31) / 32;   // stage-2 k-steps
    static constexpr int NW = 8;                 // waves per workgroup
    static constexpr int NT = NW * 64;
    static constexpr int FRAG = 64 * 8;          // fp16 per fragment
    static constexpr int P2F = KS1 * CB * FRAG;  // fp16 per P2 fragment set
    static constexpr int P1F = KS2 * RB * FRAG;  // fp16 per P1 fragment set
    static constexpr int QB = K / 2;             // packed bytes per token
    static_assert(QB % 16 == 0, "whole 16-byte chunks per token");
};

// HC: the per-channel scale diag(c) multiplies the activations before the
// transform.  x ⊙ c is no longer an fp16 number, so the stage-1 A operand is
// split like the factors: c is prescaled by a power of two (|c'| < 1, so
// |x c'| stays in fp16's range), x·c' is formed in fp32 and split into fp16
// hi + lo, and stage 1 takes hi·P2hi + hi·P2lo + lo·P2hi.
template <int N1, int N2, bool PC, bool HC>
__global__ __launch_bounds__((WaveCfg<N1, N2>::NT)) void k_tq_wave(const uint16_t* __restrict__ X, int M,
                                                                const float* __restrict__ P1,
                                                                const float* __restrict__ P2,
                                                                const float* __restrict__ cvec, ActQuant aq,
                                                                uint8_t* __restrict__ Xq,
                                                                float* __restrict__ s_x,
                                                                float* __restrict__ Zout,
                                                                uint16_t* __restrict__ S16, int Gp) {
    using C = WaveCfg<N1, N2>;
    constexpr int K = C::K;
    constexpr int NT = C::NT;
    __shared__ __align__(16) _Float16 p2hi[C::P2F];
    __shared__ __align__(16) _Float16 p2lo[C::P2F];
    __shared__ __align__(16) _Float16 p1hi[C::P1F];
    __shared__ __align__(16) _Float16 p1lo[C::P1F];
    __shared__ __align__(16) uint8_t qbuf[C::NW][C::QB];
    __shared__ float red[3 * C::NW];
    // static per-channel steps: their reciprocals, rows of n2 padded by 4 so
    // the 16 rows one quarter-wave reads fall in distinct banks
    constexpr int SROW = N2 + 4;
    __shared__ __align__(16) float rstep[PC ? N1 * SROW : 4];
    // diag(c), prescaled, in the k order of the token
    __shared__ __align__(16) float cs[HC ? K : 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int li = lane & 15;

    // ---- this wave's tokens ------------------------------------------------------
    auto load_x = [&](int m, v8h (&xa)[C::RB][C::KS1]) {
        const uint16_t* xt = X + static_cast<size_t>(min(m, M - 1)) * K;
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
            for (int ks = 0; ks < C::KS1; ++ks) {
                if (32 * ks + 8 * g < N2)
                    xa[rb][ks] = *reinterpret_cast<const v8h*>(xt + (16 * rb + li) * N2 + 32 * ks + 8 * g);
                else
                    xa[rb][ks] = v8h{0, 0, 0, 0, 0, 0, 0, 0};
            }
    };
    const int stride = gridDim.x * C::NW;
    int m = blockIdx.x * C::NW + wave;
    v8h xa[C::RB][C::KS1], xn[C::RB][C::KS1];
    load_x(m, xa);                  // first token in flight during the setup

    // ---- fragments into LDS ----------------------------------------------------
    // P2 fragment (ks, cb), lane (gg, ii), element e: P2[32 ks + 8 gg + e][16 cb + ii].
    // P1 fragment (sk, ob), lane (gg, ii), element e: P1[rho][16 ob + ii] with
    // rho = 32 sk + 4 gg + e (e < 4) or 32 sk + 16 + 4 gg + (e - 4): the rows
    // of T held by accumulator lane group gg.  Every factor element appears
    // once (padding elements are zero), so the fragment values also give the
    // power-of-two prescales; all loads are issued before the first wait.
    constexpr int L2N = (C::P2F + NT - 1) / NT;
    constexpr int L1N = (C::P1F + NT - 1) / NT;
    float v2[L2N], v1[L1N];
    float m1 = 0.0f, m2 = 0.0f;
#pragma unroll
    for (int i = 0; i < L2N; ++i) {
        const int idx = tid + i * NT;
        const int e = idx & 7;
        const int ln = (idx >> 3) & 63;
        const int slot = idx >> 9;
        const int cb = slot % C::CB;
        const int ks = slot / C::CB;
        const int kk = 32 * ks + 8 * (ln >> 4) + e;
        const bool in = idx < C::P2F && kk < N2;
        v2[i] = P2[in ? kk * N2 + 16 * cb + (ln & 15) : 0];
        if (!in) v2[i] = 0.0f;
        m2 = fmaxf(m2, fabsf(v2[i]));
    }
#pragma unroll
    for (int i = 0; i < L1N; ++i) {
        const int idx = tid + i * NT;
        const int e = idx & 7;
        const int ln = (idx >> 3) & 63;
        const int slot = idx >> 9;
        const int ob = slot % C::RB;
        const int sk = slot / C::RB;
        const int gg = ln >> 4;
        const int rho = 32 * sk + (e < 4 ? 4 * gg + e : 16 + 4 * gg + (e - 4));
        const bool in = idx < C::P1F && rho < N1;
        v1[i] = P1[in ? rho * N1 + 16 * ob + (ln & 15) : 0];
        if (!in) v1[i] = 0.0f;
        m1 = fmaxf(m1, fabsf(v1[i]));
    }
    // static per-channel steps, loaded with the fragments (clamped, so the
    // load count is fixed)
    constexpr int SLN = PC ? (K / 4 + NT - 1) / NT : 0;
    v4f stv[SLN > 0 ? SLN : 1];
#pragma unroll
    for (int i = 0; i < SLN; ++i)
        stv[i] = reinterpret_cast<const v4f*>(aq.steps)[min(tid + i * NT, K / 4 - 1)];
    constexpr int CLN = HC ? (K / 4 + NT - 1) / NT : 0;
    v4f cv[CLN > 0 ? CLN : 1];
    float m3 = 0.0f;
#pragma unroll
    for (int i = 0; i < CLN; ++i) {
        cv[i] = reinterpret_cast<const v4f*>(cvec)[min(tid + i * NT, K / 4 - 1)];
        m3 = fmaxf(m3, fmaxf(fmaxf(fabsf(cv[i][0]), fabsf(cv[i][1])), fmaxf(fabsf(cv[i][2]), fabsf(cv[i][3]))));
    }
    m1 = wave_max(m1);
    m2 = wave_max(m2);
    if constexpr (HC) m3 = wave_max(m3);
    if (lane == 0) {
        red[wave] = m1;
        red[C::NW + wave] = m2;
        if constexpr (HC) red[2 * C::NW + wave] = m3;
    }
    __syncthreads();
    m1 = 0.0f;
    m2 = 0.0f;
    m3 = 0.0f;
#pragma unroll
    for (int w = 0; w < C::NW; ++w) {
        m1 = fmaxf(m1, red[w]);
        m2 = fmaxf(m2, red[C::NW + w]);
        if constexpr (HC) m3 = fmaxf(m3, red[2 * C::NW + w]);
    }
    const int e1 = m1 > 0.0f ? -ilog2f(m1) : 0;
    const int e2 = m2 > 0.0f ? -ilog2f(m2) : 0;
    const int ec = m3 > 0.0f ? -ilog2f(m3) - 1 : 0;   // max|c 2^ec| < 1
#pragma unroll
    for (int i = 0; i < CLN; ++i) {
        const int c4 = tid + i * NT;
        if (c4 < K / 4)
            *reinterpret_cast<v4f*>(cs + 4 * c4) =
                v4f{ldexpf(cv[i][0], ec), ldexpf(cv[i][1], ec), ldexpf(cv[i][2], ec), ldexpf(cv[i][3], ec)};
    }
#pragma unroll
    for (int i = 0; i < L2N; ++i) {
        const int idx = tid + i * NT;
        if (idx < C::P2F) {
            const float v = ldexpf(v2[i], e2);
            {
                const F16Pair hl = split_f16(v);
                p2hi[idx] = hl.hi;
                p2lo[idx] = hl.lo;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < L1N; ++i) {
        const int idx = tid + i * NT;
        if (idx < C::P1F) {
            const float v = ldexpf(v1[i], e1);
            {
                const F16Pair hl = split_f16(v);
                p1hi[idx] = hl.hi;
                p1lo[idx] = hl.lo;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < SLN; ++i) {
        const int c4 = tid + i * NT;
        if (c4 < K / 4) {
            const int r = (4 * c4) / N2, j = (4 * c4) % N2;
            *reinterpret_cast<v4f*>(rstep + r * SROW + j) =
                v4f{__builtin_amdgcn_rcpf(stv[i][0]), __builtin_amdgcn_rcpf(stv[i][1]),
                    __builtin_amdgcn_rcpf(stv[i][2]), __builtin_amdgcn_rcpf(stv[i][3])};
        }
    }
    __syncthreads();

    uint8_t* qb = qbuf[wave];
    // one token: xa holds its X̄ fragments
    auto token = [&](int m) __attribute__((always_inline)) {
        // an offset the compiler cannot see through: the fragment reads stay
        // LDS reads in the loop instead of 128 loop-invariant registers, which
        // lets two waves share a SIMD
        int fo = 0;
        asm volatile("" : "+s"(fo));

        // with diag(c): the A operand x ⊙ c' as fp16 hi + lo (x fp16, c' fp32)
        v8h xlo[HC ? C::RB : 1][HC ? C::KS1 : 1];
        if constexpr (HC) {
#pragma unroll
            for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
                for (int ks = 0; ks < C::KS1; ++ks) {
                    if (32 * ks + 8 * g >= N2) {
                        xlo[rb][ks] = v8h{0, 0, 0, 0, 0, 0, 0, 0};
                        continue;
                    }
                    const float* cp = cs + (16 * rb + li) * N2 + 32 * ks + 8 * g + fo;
                    const v4f c0 = *reinterpret_cast<const v4f*>(cp);
                    const v4f c1 = *reinterpret_cast<const v4f*>(cp + 4);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float v = static_cast<float>(xa[rb][ks][e]) * (e < 4 ? c0[e] : c1[e - 4]);
                        const F16Pair hl = split_f16(v);
                        xa[rb][ks][e] = hl.hi;
                        xlo[rb][ks][e] = hl.lo;
                    }
                }
        }
        // stage 1: T = X̄ · P2'
        v4f T[C::RB][C::CB];
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
#pragma unroll
            for (int rb = 0; rb < C::RB; ++rb) T[rb][cb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < C::KS1; ++ks) {
                const int off = ((ks * C::CB + cb) * 64 + lane) * 8 + fo;
                const v8h bh = *reinterpret_cast<const v8h*>(p2hi + off);
                const v8h bl = *reinterpret_cast<const v8h*>(p2lo + off);
#pragma unroll
                for (int rb = 0; rb < C::RB; ++rb) {
                    if constexpr (HC)
                        T[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xlo[rb][ks], bh, T[rb][cb], 0, 0, 0);
                    T[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[rb][ks], bh, T[rb][cb], 0, 0, 0);
                    T[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[rb][ks], bl, T[rb][cb], 0, 0, 0);
                }
            }
        }
        // power-of-two prescale of T into the fp16 range, then Tᵀ fragments:
        // A operand of k-step sk for column block cb = accumulator rows 4g+r
        // of row blocks 2 sk and 2 sk + 1
        float tm = 0.0f;
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r) tm = fmaxf(tm, fabsf(T[rb][cb][r]));
        tm = wave_max(tm);
        const int et = tm > 0.0f ? 14 - ilog2f(tm) : 0;
        v8h ah[C::KS2][C::CB], al[C::KS2][C::CB];
#pragma unroll
        for (int sk = 0; sk < C::KS2; ++sk)
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int rb = 2 * sk + (e >> 2);
                    const float v = rb < C::RB ? ldexpf(T[rb < C::RB ? rb : 0][cb][e & 3], et) : 0.0f;
                    {
                        const F16Pair hl = split_f16(v);
                        ah[sk][cb][e] = hl.hi;
                        al[sk][cb][e] = hl.lo;
                    }
                }
        // stage 2: Zᵀ = T'ᵀ · P1'  (tile (cb, ob): rows j, columns i)
        v4f Z[C::RB][C::CB];
#pragma unroll
        for (int ob = 0; ob < C::RB; ++ob) {
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb) Z[ob][cb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int sk = 0; sk < C::KS2; ++sk) {
                const int off = ((sk * C::RB + ob) * 64 + lane) * 8 + fo;
                const v8h bh = *reinterpret_cast<const v8h*>(p1hi + off);
                const v8h bl = *reinterpret_cast<const v8h*>(p1lo + off);
#pragma unroll
                for (int cb = 0; cb < C::CB; ++cb) {
                    Z[ob][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[sk][cb], bh, Z[ob][cb], 0, 0, 0);
                    Z[ob][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[sk][cb], bl, Z[ob][cb], 0, 0, 0);
                    Z[ob][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[sk][cb], bh, Z[ob][cb], 0, 0, 0);
                }
            }
        }
        // lane (g, li) of tile (ob, cb) holds 2^-unscale * Z[16 ob + li][16 cb + 4 g + r];
        // the power of two is folded into the scale and the quantizer's
        // multiplier (exact, so the codes are those of the unscaled values)
        const int unscale = -(e1 + e2 + et + ec);
        float zmax = 0.0f;
#pragma unroll
        for (int ob = 0; ob < C::RB; ++ob)
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r) zmax = fmaxf(zmax, fabsf(Z[ob][cb][r]));
        if (Zout != nullptr) {
#pragma unroll
            for (int ob = 0; ob < C::RB; ++ob)
#pragma unroll
                for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) Z[ob][cb][r] = ldexpf(Z[ob][cb][r], unscale);
            float* zo = Zout + static_cast<size_t>(m) * K;
#pragma unroll
            for (int ob = 0; ob < C::RB; ++ob)
#pragma unroll
                for (int cb = 0; cb < C::CB; ++cb)
                    *reinterpret_cast<v4f*>(zo + (16 * ob + li) * N2 + 16 * cb + 4 * g) = Z[ob][cb];
        } else {
            float s;
            if (PC)
                s = 1.0f;
            else if (aq.steps == nullptr)
                s = aq.alpha * ldexpf(wave_max(zmax), unscale) / aq.qmax;
            else
                s = aq.steps[0];
            const float inv = s > 0.0f ? ldexpf(1.0f / s, unscale) : 0.0f;
            if (PC) {
                // one step per channel: the lane's four consecutive channels
#pragma unroll
                for (int ob = 0; ob < C::RB; ++ob)
#pragma unroll
                    for (int cb = 0; cb < C::CB; ++cb) {
                        const int k0 = (16 * ob + li) * N2 + 16 * cb + 4 * g;
                        const v4f rs = *reinterpret_cast<const v4f*>(
                            rstep + (16 * ob + li) * SROW + 16 * cb + 4 * g + fo);
                        uint32_t w = 0;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            w |= quant_nibble_magic(ldexpf(Z[ob][cb][r], unscale), rs[r], aq.qmax) << (4 * r);
                        *reinterpret_cast<uint16_t*>(qb + k0 / 2) = static_cast<uint16_t>(w);
                    }
            } else {
#pragma unroll
                for (int ob = 0; ob < C::RB; ++ob)
#pragma unroll
                    for (int cb = 0; cb < C::CB; ++cb) {
                        uint32_t w = 0;
#pragma unroll
                        for (int r = 0; r < 4; ++r) w |= quant_nibble_magic(Z[ob][cb][r], inv, aq.qmax) << (4 * r);
                        *reinterpret_cast<uint16_t*>(qb + ((16 * ob + li) * N2 + 16 * cb + 4 * g) / 2) =
                            static_cast<uint16_t>(w);
                    }
            }
            // the wave's LDS slice is read back by the same wave: LDS operations
            // of one wave complete in order
            uint4* dst = reinterpret_cast<uint4*>(Xq + static_cast<size_t>(m) * (K / 2));
#pragma unroll
            for (int c = lane; c < C::QB / 16; c += 64) {
                const uint4 v = reinterpret_cast<const uint4*>(qb)[c];
                dst[c] = v;
                if (S16 != nullptr) store_group_sum(v, c, S16 + static_cast<size_t>(m) * Gp);
            }
            if (lane == 0) s_x[m] = s;
            // the padding groups of the sums row: zero
            if (S16 != nullptr && lane < Gp - K / 128) S16[static_cast<size_t>(m) * Gp + K / 128 + lane] = 0;
        }
    };
    // every token but the wave's last has the next one in flight (an
    // unconditional load inside the token loop: a branch there would make the
    // compiler wait for it before stage 1); the last token loads nothing more
    for (; m + stride < M; m += stride) {
        load_x(m + stride, xn);
        token(m);
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
            for (int ks = 0; ks < C::KS1; ++ks) xa[rb][ks] = xn[rb][ks];
    }
    if (m < M) token(m);
}

template <int N1, int N2, bool PC, bool HC>
hipError_t launch_wave_k(const uint16_t* X, int M, const float* P1, const float* P2, const float* c,
                         ActQuant aq, uint8_t* Xq, float* s_x, float* Z, uint16_t* S16, int Gp,
                         hipStream_t stream) {
    using C = WaveCfg<N1, N2>;
    // persistent grid: as many workgroups as fit on the device at once, so
    // the fragment setup is paid once per resident workgroup
    static int per_cu = 0;
    if (per_cu == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_tq_wave<N1, N2, PC, HC>, C::NT, 0) !=
                hipSuccess || n < 1)
            n = 1;
        per_cu = n;
    }
    const int units = (M + C::NW - 1) / C::NW;
    const int cap = per_cu * device_cu_count();
    const int grid = units < cap ? units : cap;
    k_tq_wave<N1, N2, PC, HC><<<grid, C::NT, 0, stream>>>(X, M, P1, P2, c, aq, Xq, s_x, Z, S16, Gp);
    return hipGetLastError();
}

template <int N1, int N2>
hipError_t launch_wave(const uint16_t* X, int M, const float* P1, const float* P2, const float* c,
                       ActQuant aq, uint8_t* Xq, float* s_x, float* Z, uint16_t* S16, int Gp,
                       hipStream_t stream) {
    const bool pc = aq.steps != nullptr && aq.per_channel && Xq != nullptr;
    if (c != nullptr)
        return pc ? launch_wave_k<N1, N2, true, true>(X, M, P1, P2, c, aq, Xq, s_x, Z, S16, Gp, stream)
                  : launch_wave_k<N1, N2, false, true>(X, M, P1, P2, c, aq, Xq, s_x, Z, S16, Gp, stream);
    return pc ? launch_wave_k<N1, N2, true, false>(X, M, P1, P2, c, aq, Xq, s_x, Z, S16, Gp, stream)
              : launch_wave_k<N1, N2, false, false>(X, M, P1, P2, c, aq, Xq, s_x, Z, S16, Gp, stream);
}

// S16 / Gp: the per-token group sums of the codes (see store_group_sum),
// written only when S16 is not null (quantizing calls with K a multiple of
// 128 and Gp >= K / 128)
using FusedFn = hipError_t (*)(const uint16_t*, int, const float*, const float*, const float*,
                               ActQuant, uint8_t*, float*, float*, uint16_t*, int, hipStream_t);

// (n1, n2) pairs with a fused (or wave-per-token) instantiation; with
// diag(c) only the wave-per-token kernels apply
FusedFn fused_for(int n1, int n2, bool has_c) {
#define W4A4_FUSED(a, b) \
    if (n1 == a && n2 == b) return has_c ? nullptr : &launch_fused<a, b>;
#define W4A4_WAVE(a, b) \
    if (n1 == a && n2 == b) return &launch_wave<a, b>;
    W4A4_WAVE(16, 16)
    W4A4_WAVE(32, 32)
    W4A4_WAVE(16, 64)
    W4A4_WAVE(32, 64)
    W4A4_WAVE(64, 64)
    W4A4_FUSED(32, 128)
    W4A4_FUSED(64, 128)
    W4A4_FUSED(96, 128)
    W4A4_FUSED(112, 128)
    W4A4_FUSED(128, 128)
    W4A4_FUSED(128, 64)
#undef W4A4_FUSED
#undef W4A4_WAVE
    return nullptr;
}

// ===========================================================================
// Column-block MFMA path: factors whose P1 fragments do not fit one LDS (n1
// above 128), and few tokens.  The unit of work is one token m and one
// 16-column block cb of Z, computed by one wave with the arithmetic of the
// fused path (stage 1 on X̄ fp16 and split P2, stage 2 on split T and split
// P1, power-of-two prescales).  The 16-row blocks of Z (stage-2 outputs) are
// split into `parts` ranges, one per grid row.  A workgroup of 8 waves is one
// token and one range: it stages the token's X̄ (rows padded by 16 bytes) and
// the P1 fragments of its range in LDS, with every load issued before the
// first wait, and its waves are the token's 8 column blocks; each redoes
// stage 1 for its block (parts > 1 spreads a handful of tokens over many
// CUs).  Z goes to the workspace in fp32 with one absmax per (unit,
// part); k_tq_quant then takes each token's largest partial maximum.
// ===========================================================================
constexpr int kColsWaves = 8;
constexpr int kColsLdsMax = 159 * 1024;       // dynamic LDS of one workgroup

template <int N1, int N2>
struct ColsCfg {
    // n1 a multiple of 32: every fragment row rho is a row of P1
    static_assert(N1 % 32 == 0 && N2 % 32 == 0, "factors: multiples of 32");
    static constexpr int K = N1 * N2;
    static constexpr int RB = N1 / 16;           // 16-row blocks of T and Z
    static constexpr int CB = N2 / 16;           // 16-column blocks (units per token)
    static constexpr int KS1 = N2 / 32;          // stage-1 MFMA k-steps
    static constexpr int KS2 = (N1 + 31) / 32;   // stage-2 MFMA k-steps
    static constexpr int FRAG = 64 * 8;          // fp16 elements of one fragment
    static constexpr int FRAG_BYTES = 2 * FRAG * 2;   // hi + lo
    // staged X̄ row, bytes: padded as in the fused path (32 bytes for rows
    // of 256 bytes: no bank conflict in the stage-1 operand reads)
    static constexpr int XROW = N2 * 2 + ((N2 * 2) % 256 == 0 ? 32 : 16);
    // the staged token, rounded up to whole 64-lane copies of 16 bytes
    static constexpr int XCOPIES = (N1 * (XROW / 16) + 63) / 64;
    static constexpr int XBYTES = XCOPIES * 1024;
    // row blocks of P1 fragments that fit beside the staged token
    static constexpr int MAX_RBP = (kColsLdsMax - XBYTES) / (KS2 * FRAG_BYTES);
    static_assert(CB == kColsWaves, "one wave per 16-column block of a token");
    static_assert(MAX_RBP >= 1, "staged token too large");
};

// row blocks per part and number of parts for M tokens (every part non-empty)
template <int N1, int N2>
void cols_parts(int M, int* rbp, int* parts) {
    using C = ColsCfg<N1, N2>;
    const int max_rbp = C::MAX_RBP;
    // about 8 waves per CU over 256 CUs
    const long units = static_cast<long>(M) * C::CB;
    long want = (2048 + units - 1) / units;
    if (want < 1) want = 1;
    if (want > C::RB) want = C::RB;
    int r = static_cast<int>((C::RB + want - 1) / want);
    if (r > max_rbp) r = max_rbp;
    *rbp = r;
    *parts = (C::RB + r - 1) / r;
}

template <int N1, int N2>
__global__ __launch_bounds__(kColsWaves * 64) void k_tq_cols(const uint16_t* __restrict__ X, int M,
                                                             const float* __restrict__ P1,
                                                             const float* __restrict__ P2, int rbp,
                                                             int parts, float* __restrict__ Zf,
                                                             uint32_t* __restrict__ amax) {
    using C = ColsCfg<N1, N2>;
    constexpr int K = C::K;
    constexpr int NT = kColsWaves * 64;
    extern __shared__ __align__(16) _Float16 cl[];
    __shared__ float red[kColsWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int li = lane & 15;
    const int part = blockIdx.y;
    const int ob0 = part * rbp;
    const int nob = min(C::RB - ob0, rbp);
    const int nf = nob * C::KS2;
    _Float16* p1hi = cl;
    _Float16* p1lo = cl + nf * C::FRAG;
    uint8_t* xs = reinterpret_cast<uint8_t*>(cl + 2 * nf * C::FRAG);
    const int m = blockIdx.x;                        // this workgroup's token

    // ---- this wave's P2 columns and the token's X̄ (to LDS): their loads are
    //      issued together with P1's, before the first wait -------------------
    const int cb = wave;                             // this wave's column block
    float p2v[C::KS1][8];
#pragma unroll
    for (int ks = 0; ks < C::KS1; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) p2v[ks][e] = P2[(32 * ks + 8 * g + e) * N2 + 16 * cb + li];
    // the token's X̄ goes to LDS by direct copies: 16-byte slot s holds row
    // s / RS, chunk s % RS (RS = XROW / 16); the chunks past the row's N2 / 8
    // and the slots past the token are padding (copied from the token's
    // first chunk, never read)
    {
        constexpr int RS = C::XROW / 16;
        const uint16_t* xb = X + static_cast<size_t>(m) * C::K;
        for (int j = wave; j < C::XCOPIES; j += kColsWaves) {
            const int s = j * 64 + lane;
            const int r = s / RS;
            const int c = s - r * RS;
            const uint32_t off = (r < N1 && c < N2 / 8) ? static_cast<uint32_t>(r * N2 * 2 + c * 16) : 0u;
            dma16_async_sv(xb, off, xs + j * 1024);
        }
    }

    // ---- P1 fragments of row blocks ob0 .. ob0+nob-1 into LDS ----------------
    // fragment (ob, sk), lane (gg, ii), element e holds P1[rho][16*ob + ii],
    // rho = 32 sk + 4 gg + e (e < 4) or 32 sk + 16 + 4 gg + (e - 4): the rows
    // of T that the stage-1 accumulators of lane group gg hold.  The part's
    // columns are read as 16-byte row pieces (rows rho, 4 columns each, all
    // loads issued before the first wait), its max |P1| gives the power-of-
    // two prescale, and each piece is scattered to 4 fragment lanes.
    // Every load of the kernel (P2 columns, X̄, P1 pieces) is issued before
    // the first use of any: a piece load guarded by its own use, or an X̄
    // load sunk next to its LDS store, would wait for memory once per load.
    // A batch of pieces past the part (a uniform test) is skipped; inside a
    // batch the index is clamped.
    constexpr int MAXI = (N1 * 4 * C::MAX_RBP + NT - 1) / NT;
    const int pieces = N1 * 4 * nob;                 // 16-byte pieces of the part
    float4 pv[MAXI];
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        if (i * NT < pieces) {
            const int idx = min(tid + i * NT, pieces - 1);
            const int rho = idx / (4 * nob);
            const int c4 = idx - rho * (4 * nob);
            pv[i] = *reinterpret_cast<const float4*>(P1 + static_cast<size_t>(rho) * N1 + 16 * ob0 + 4 * c4);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    float m1 = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        if (tid + i * NT < pieces)
            m1 = fmaxf(m1, fmaxf(fmaxf(fabsf(pv[i].x), fabsf(pv[i].y)),
                                 fmaxf(fabsf(pv[i].z), fabsf(pv[i].w))));
    }
    m1 = wave_max(m1);
    if (lane == 0) red[wave] = m1;
    // this wave's copies of X̄ have landed; after the barrier every wave's have
    wait_vmcnt<0>();
    __syncthreads();
    m1 = 0.0f;
#pragma unroll
    for (int w = 0; w < kColsWaves; ++w) m1 = fmaxf(m1, red[w]);
    const int e1 = m1 > 0.0f ? -ilog2f(m1) : 0;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        const int idx = tid + i * NT;
        if (idx < pieces) {
            const int rho = idx / (4 * nob);
            const int c4 = idx - rho * (4 * nob);
            const int sk = rho >> 5;
            const int rr = rho & 31;
            const int gg = (rr & 15) >> 2;
            const int e = (rr & 3) + ((rr >> 4) << 2);
            const float vv[4] = {pv[i].x, pv[i].y, pv[i].z, pv[i].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = 4 * c4 + q;             // column inside the part
                const int f = (col >> 4) * C::KS2 + sk;
                const int off = (f * 64 + gg * 16 + (col & 15)) * 8 + e;
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

    // ---- P2 fragments of this wave's 16 columns, prescaled per wave ----------
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

    // ---- stage 1: T[:, cb] = X̄ · P2'[:, cb] ----------------------------------
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
    // stage-2 B operand: accumulator rows 4g+r of blocks 2s and 2s+1
    v8h bh[C::KS2], bl[C::KS2];
#pragma unroll
    for (int sk = 0; sk < C::KS2; ++sk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int rb = 2 * sk + (e >> 2);
            const float v = rb < C::RB ? ldexpf(T[rb < C::RB ? rb : 0][e & 3], et) : 0.0f;
            {
                const F16Pair hl = split_f16(v);
                bh[sk][e] = hl.hi;
                bl[sk][e] = hl.lo;
            }
        }

    // ---- stage 2 for this part's row blocks ----------------------------------
    const int unscale = -(e1 + e2 + et);
    float wmax = 0.0f;
    float* zo = Zf + static_cast<size_t>(m) * K + 16 * cb + li;
    for (int j = 0; j < nob; ++j) {
        v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int sk = 0; sk < C::KS2; ++sk) {
            const int off = ((j * C::KS2 + sk) * 64 + lane) * 8;
            const v8h ah = *reinterpret_cast<const v8h*>(p1hi + off);
            const v8h al = *reinterpret_cast<const v8h*>(p1lo + off);
            z = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh[sk], z, 0, 0, 0);
            z = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl[sk], z, 0, 0, 0);
            z = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh[sk], z, 0, 0, 0);
        }
        const int row0 = 16 * (ob0 + j) + 4 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v = ldexpf(z[r], unscale);
            wmax = fmaxf(wmax, fabsf(v));
            zo[(row0 + r) * N2] = v;
        }
    }
    wmax = wave_max(wmax);
    if (lane == 0) amax[(static_cast<size_t>(m) * C::CB + cb) * parts + part] = __float_as_uint(wmax);
}

template <int N1, int N2>
size_t cols_ws_bytes(int M) {
    int rbp, parts;
    cols_parts<N1, N2>(M, &rbp, &parts);
    return align256(sizeof(float) * static_cast<size_t>(M) * N1 * N2) +
           align256(sizeof(uint32_t) * static_cast<size_t>(M) * ColsCfg<N1, N2>::CB * parts);
}

template <int N1, int N2>
hipError_t launch_cols(const uint16_t* X, int M, const float* P1, const float* P2, ActQuant aq,
                       uint8_t* Xq, float* s_x, float* Z, void* ws, hipStream_t stream) {
    using C = ColsCfg<N1, N2>;
    int rbp, parts;
    cols_parts<N1, N2>(M, &rbp, &parts);
    char* p = static_cast<char*>(ws);
    float* Zw = Z != nullptr ? Z : reinterpret_cast<float*>(p);
    p += align256(sizeof(float) * static_cast<size_t>(M) * C::K);
    uint32_t* amax = reinterpret_cast<uint32_t*>(p);
    const size_t lds = static_cast<size_t>(rbp) * C::KS2 * C::FRAG_BYTES + C::XBYTES;
    if (lds > 64 * 1024) {
        // more than the default dynamic LDS limit: raise it once per device
        static bool raised[64] = {};
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= 64 || !raised[dev]) {
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_tq_cols<N1, N2>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, kColsLdsMax);
            if (e != hipSuccess) return e;
            if (dev >= 0 && dev < 64) raised[dev] = true;
        }
    }
    const dim3 grid(M, parts);
    k_tq_cols<N1, N2><<<grid, kColsWaves * 64, lds, stream>>>(X, M, P1, P2, rbp, parts, Zw, amax);
    if (Z == nullptr)
        k_tq_quant<<<dim3(M, ceil_div(C::K / 8, 256)), dim3(256), 0, stream>>>(
            Zw, C::K, aq, amax, C::CB * parts, Xq, s_x);
    return hipGetLastError();
}

struct ColsFns {
    hipError_t (*launch)(const uint16_t*, int, const float*, const float*, ActQuant, uint8_t*, float*,
                         float*, void*, hipStream_t);
    size_t (*ws_bytes)(int);
};

// (n1, n2) pairs with a column-block instantiation
const ColsFns* cols_for(int n1, int n2) {
#define W4A4_COLS(a, b)                                                   \
    if (n1 == a && n2 == b) {                                             \
        static const ColsFns f{&launch_cols<a, b>, &cols_ws_bytes<a, b>}; \
        return &f;                                                        \
    }
    W4A4_COLS(160, 128)
    W4A4_COLS(192, 128)
    W4A4_COLS(224, 128)
    W4A4_COLS(256, 128)
#undef W4A4_COLS
    return nullptr;
}

}  // namespace

TqPath tq_select_path(int M, int n1, int n2, bool has_c) {
    (void)M;
    if (fused_for(n1, n2, has_c) != nullptr) return TqPath::Fused;
    if (!has_c && cols_for(n1, n2) != nullptr) return TqPath::Cols;
    return TqPath::Split;
}

size_t tq_workspace_bytes(int M, int n1, int n2, bool has_c) {
    const size_t K = static_cast<size_t>(n1) * n2;
    switch (tq_select_path(M, n1, n2, has_c)) {
        case TqPath::Fused:
            return 0;
        case TqPath::Cols:
            return cols_for(n1, n2)->ws_bytes(M);
        default:
            return 2 * align256(sizeof(float) * K * M) + align256(sizeof(uint32_t) * M);
    }
}

hipError_t tq_launch(const uint16_t* X, int M, int n1, int n2, const float* P1,
                     const float* P2, const float* c, ActQuant aq, bool quantize,
                     uint8_t* Xq, float* s_x, float* Z, void* ws, size_t ws_bytes,
                     hipStream_t stream, uint16_t* S16, int Gp, bool* sums_written) {
    (void)ws_bytes;
    if (sums_written != nullptr) *sums_written = false;
    if (M == 0) return hipSuccess;
    const TqPath path = tq_select_path(M, n1, n2, c != nullptr);
    if (path == TqPath::Fused) {
        const int K = n1 * n2;
        const bool sums = quantize && S16 != nullptr && K % 128 == 0 && Gp >= K / 128 &&
                          Gp - K / 128 < 64;
        const hipError_t e = fused_for(n1, n2, c != nullptr)(
            X, M, P1, P2, c, aq, quantize ? Xq : nullptr, s_x, quantize ? nullptr : Z,
            sums ? S16 : nullptr, sums ? Gp : 0, stream);
        if (e == hipSuccess && sums && sums_written != nullptr) *sums_written = true;
        return e;
    }
    if (path == TqPath::Cols)
        return cols_for(n1, n2)->launch(X, M, P1, P2, aq, Xq, s_x, quantize ? nullptr : Z, ws,
                                        stream);
    const int K = n1 * n2;
    char* p = static_cast<char*>(ws);
    float* T = reinterpret_cast<float*>(p);
    p += align256(sizeof(float) * static_cast<size_t>(K) * M);
    float* Zw = reinterpret_cast<float*>(p);
    p += align256(sizeof(float) * static_cast<size_t>(K) * M);
    uint32_t* amax = reinterpret_cast<uint32_t*>(p);
    float* Zout = quantize ? Zw : Z;

    k_tq_stage1<<<dim3(M, n1), dim3(n2 >= 256 ? 256 : ((n2 + 63) / 64) * 64), 0, stream>>>(
        X, K, n2, P2, c, T, amax);
    k_tq_stage2<<<dim3(M, ceil_div(K, kSplitThreads)), dim3(kSplitThreads), 0, stream>>>(
        T, K, n1, n2, P1, Zout, amax);
    if (quantize) {
        k_tq_quant<<<dim3(M, ceil_div(K / 8, 256)), dim3(256), 0, stream>>>(Zw, K, aq, amax, 1,
                                                                           Xq, s_x);
    }
    return hipGetLastError();
}

}  // namespace w4a4
