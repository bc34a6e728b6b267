// Decode attention over the INT4 KV cache (one query token per sequence).
//
// FlatQuant: Flatness Matters for LLM Quantization, sections 核心思想 and
// Transformer 集成: the key cache holds Q(k·P_h) per head, so the query takes
// the inverse transpose, (q·P_h^-T)·(k·P_h)^T = q·k^T; the value cache holds
// Q(v·P_v) and the attention output stays in the P_v basis (P_v^-1 belongs to
// the output projection's weights).  Softmax attention with grouped query
// heads (head h reads KV head h / G) is the textbook definition.
//
// Three launches:
//   1. q~ = q · P_h^-T · (sm_scale · log2 e), fp32 (k_rows_xform, kv_cache.hip);
//   2. k_attn_partial: one workgroup per (chunk of C positions, KV head,
//      sequence); four waves stream 32-token tiles of packed keys and values
//      from HBM into registers (the next tile's loads in flight while the
//      current one is computed) and run both products on MFMA with exact
//      operands.  Online softmax in base 2; the waves' states are merged in
//      LDS and one partial record per workgroup is written;
//   3. k_attn_combine merges the chunks of each (sequence, KV head).
//
// Arithmetic of the two products (fp16 MFMA, v_mfma_f32_16x16x32_f16):
//   codes enter as q or 16 q, exact in fp16 (nib8_h8x16); q~ is scaled by a
//   power of two per head into [1, 2), and the value weights
//   p'_t = p_t * s_v[t] by one power of two per chunk into (0, 2); both are
//   split into fp16 hi + lo, so every product is exact and only the fp32
//   accumulation rounds.  The running maximum of the online softmax is
//   raised only when a tile exceeds it by more than 2^10 (weights up to 2^10
//   stay exact in the split), so O is rarely rescaled.
#include "common.hpp"
#include "internal.hpp"

namespace w4a4 {

namespace {

constexpr int kHd = 128;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kGMax = 16;             // query heads per KV head (MFMA columns)

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Eight signed nibbles (nibble j = element j) as fp16 MFMA operand slots in
// the order 0, 4, 1, 5, 2, 6, 3, 7.  Each nibble stays where it is inside
// its 16-bit half: flipping its top bit gives the offset-binary u = q + 8,
// and OR-ing the exponent of 1024 gives 1024 + u (bits 0-3) or 1024 + 16 u
// (bits 4-7), both exact; subtracting 1032 or 1152 leaves q or 16 q.  So
// slots 2, 3, 6, 7 carry 16 q, and the other operand puts a factor 16 on
// slots 0, 1, 4, 5 instead (kSlotScale): every product is 16 q b.
__device__ __forceinline__ v8h nib8_h8x16(uint32_t w) {
    const uint32_t w8 = w >> 8;
    const v4u r = {(w & 0x000F000Fu) ^ 0x64086408u, (w & 0x00F000F0u) ^ 0x64806480u,
                   (w8 & 0x000F000Fu) ^ 0x64086408u, (w8 & 0x00F000F0u) ^ 0x64806480u};
    const _Float16 a = static_cast<_Float16>(1032.0f);
    const _Float16 b = static_cast<_Float16>(1152.0f);
    return __builtin_bit_cast(v8h, r) - v8h{a, a, b, b, a, a, b, b};
}
constexpr float kSlotScale[8] = {16.0f, 16.0f, 1.0f, 1.0f, 16.0f, 16.0f, 1.0f, 1.0f};

__device__ __forceinline__ float pow2i(int e) { return __builtin_ldexpf(1.0f, e); }


// ---------------------------------------------------------------------------
// Partial attention of one chunk.  Lane l of a wave: c16 = l % 16, q4 = l / 16.
//  - score product S^T[token, g] = K[token, :] · q~[g, :]^T: A = key rows,
//    B = q~ (column g = c16).  A 32-token tile is two 16-row products whose
//    row r holds token 8*(r/4) + 4*s + r%4 (s = product index), so lane l ends
//    with tokens 8*q4 .. 8*q4+7 of column g = c16;
//  - value product O^T[ch, g] += V^T[ch, tokens] · P'^T[tokens, g]: A = value
//    words (row c16 <-> channel 4*c16 + db%4 + 64*(db/4) for block db), B =
//    the lane's own weights; the output column is again g = c16, so the
//    softmax state of column g lives in the lanes that hold its O.
// Contraction slots follow the nibble order 0, 4, 1, 5, 2, 6, 3, 7 on both
// operands.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void
k_attn_partial(AttnArgs a) {
    // dynamic LDS: the q~ operands during the tile loop, then the waves' O
    // rows g < G for the merge (attn_partial_lds bytes)
    extern __shared__ __align__(16) uint8_t dyn[];
    __shared__ float sm[kWaves][kGMax];
    __shared__ float sl[kWaves][kGMax];
    __shared__ float svmax[kWaves];

    const int c = blockIdx.x;
    const int hk = blockIdx.y;
    const int b = blockIdx.z;
    const int C = a.chunk;
    int L = a.lengths[b];
    L = L < 0 ? 0 : (L > a.max_seq ? a.max_seq : L);
    const int t_begin = c * C;
    if (t_begin >= L) return;
    const int t_end = min(L, t_begin + C);
    const int G = a.heads_q / a.heads_kv;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int c16 = lane & 15;
    const int q4 = lane >> 4;
    const size_t bh = static_cast<size_t>(b) * a.heads_kv + hk;
    const float* ksc = a.k_scale + bh * a.max_seq + 8 * q4;
    const float* vsc = a.v_scale + bh * a.max_seq + 8 * q4;
    const int tau0 = 8 * (c16 >> 2) + (c16 & 3);      // key row of product s: tau0 + 4 s
    const uint8_t* kbase = a.k_cache + (bh * a.max_seq + tau0) * (kHd / 2) + 16 * q4;
    const uint32_t* vbase = a.v_cache + (bh * (a.max_seq / 8) + q4) * kHd + 4 * c16;

    // Tile data is loaded one operand at a time: each operand's registers
    // take the next tile's load as soon as the current tile has consumed them,
    // so the loads of tile n+1 overlap the rest of tile n without a second
    // register set.
    auto kptr = [&](int t) { return kbase + static_cast<size_t>(t) * (kHd / 2); };
    auto vptr = [&](int t) { return vbase + static_cast<size_t>(t / 8) * kHd; };

    int t0 = t_begin + 32 * w;
    const int tf = t0 < t_end ? t0 : t_begin;  // first tile, in flight during the setup
    uint4 k0 = *reinterpret_cast<const uint4*>(kptr(tf));
    uint4 k1 = *reinterpret_cast<const uint4*>(kptr(tf) + 4 * (kHd / 2));
    float4 sk0 = *reinterpret_cast<const float4*>(ksc + tf);
    float4 sk1 = *reinterpret_cast<const float4*>(ksc + tf + 4);
    float4 sv0 = *reinterpret_cast<const float4*>(vsc + tf);
    float4 sv1 = *reinterpret_cast<const float4*>(vsc + tf + 4);
    uint4 v0 = *reinterpret_cast<const uint4*>(vptr(tf));
    uint4 v1 = *reinterpret_cast<const uint4*>(vptr(tf) + 64);

    // chunk-wide power of two that brings the value scales into (0, 2)
    float vm = 0.0f;
    {
        const float* vs0 = a.v_scale + bh * a.max_seq;
        for (int t = t_begin + tid; t < t_end; t += kThreads) vm = fmaxf(vm, fabsf(vs0[t]));
    }

    // q~ of column g = c16 as fp16 hi/lo B operands, scaled by a per-column
    // power of two into [1, 2)
    const int g = c16;
    const bool gval = g < G;
    const float* qrow =
        a.qt + (static_cast<size_t>(b) * a.heads_q + hk * G + (gval ? g : 0)) * kHd + 32 * q4;
    float qv[4][8];
    float qmax = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const float4 x0 = *reinterpret_cast<const float4*>(qrow + 8 * ks);
        const float4 x1 = *reinterpret_cast<const float4*>(qrow + 8 * ks + 4);
        const float e8[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        constexpr int nu[8] = {0, 4, 1, 5, 2, 6, 3, 7};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            qv[ks][j] = gval ? e8[nu[j]] : 0.0f;
            qmax = fmaxf(qmax, fabsf(qv[ks][j]));
        }
    }
    qmax = fmaxf(qmax, __shfl_xor(qmax, 16));
    qmax = fmaxf(qmax, __shfl_xor(qmax, 32));
    vm = wave_max(vm);
    if (lane == 0) svmax[w] = vm;
    const int eq = qmax > 0.0f ? ilog2f(qmax) : 0;
    const float fq = pow2i(-eq);
    const float uq = pow2i(eq - 4);         // the slot factor 16 comes off here
    // the B operands live in LDS (one copy per workgroup, read per tile), not
    // in 32 registers per lane: that keeps the kernel at four waves per SIMD
    v8h (*sq)[4][64] = reinterpret_cast<v8h (*)[4][64]>(dyn);
    if (w == 0) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            v8h hv, lv;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const F16Pair hl = split_f16(qv[ks][j] * (fq * kSlotScale[j]));
                hv[j] = hl.hi;
                lv[j] = hl.lo;
            }
            sq[0][ks][lane] = hv;
            sq[1][ks][lane] = lv;
        }
    }

    __syncthreads();
    vm = fmaxf(fmaxf(svmax[0], svmax[1]), fmaxf(svmax[2], svmax[3]));
    const int ev = vm > 0.0f ? ilog2f(vm) : 0;
    const float fv = pow2i(-ev);
    const float fv16 = pow2i(4 - ev);       // with the slot factor 16 (even i)

    float m = -__builtin_inff();
    float lp = 0.0f;      // sum of p over the lane's tokens (rescaled with m)
    v4f O[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) O[db] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // one 32-token tile; MASK: the tile crosses t_end (only the last one can)
    auto tile = [&](auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int tn = t0 + 32 * kWaves < t_end ? t0 + 32 * kWaves : t0;   // next (or again)

        // scores; the compiler barrier keeps the q~ operand reads inside the loop
        __asm__ volatile("" ::: "memory");
        v8h qh[4], ql[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            qh[ks] = sq[0][ks][lane];
            ql[ks] = sq[1][ks][lane];
        }
        const uint32_t kw[2][4] = {{k0.x, k0.y, k0.z, k0.w}, {k1.x, k1.y, k1.z, k1.w}};
        v4f acc[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            acc[s] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const v8h ka = nib8_h8x16(kw[s][ks]);
                acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qh[ks], acc[s], 0, 0, 0);
                acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, ql[ks], acc[s], 0, 0, 0);
            }
        }
        k0 = *reinterpret_cast<const uint4*>(kptr(tn));
        k1 = *reinterpret_cast<const uint4*>(kptr(tn) + 4 * (kHd / 2));
        const float skv[2][4] = {{sk0.x, sk0.y, sk0.z, sk0.w}, {sk1.x, sk1.y, sk1.z, sk1.w}};
        const int nval = t_end - t0 - 8 * q4;          // lane's tokens below t_end
        float x[2][4];
        float mx = -__builtin_inff();
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[s][i] = acc[s][i] * (uq * skv[s][i]);
                if (MASK && !(4 * s + i < nval)) x[s][i] = -__builtin_inff();
                mx = fmaxf(mx, x[s][i]);
            }
        sk0 = *reinterpret_cast<const float4*>(ksc + tn);
        sk1 = *reinterpret_cast<const float4*>(ksc + tn + 4);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (__any(mx > m + 10.0f)) {
            const float mn = fmaxf(m, mx);
            const float al = __builtin_amdgcn_exp2f(m - mn);
            lp *= al;
#pragma unroll
            for (int db = 0; db < 8; ++db) O[db] *= al;
            m = mn;
        }
        // weights p' = p * s_v * 2^-ev (times the slot factor) as fp16 hi/lo
        const float svv[2][4] = {{sv0.x, sv0.y, sv0.z, sv0.w}, {sv1.x, sv1.y, sv1.z, sv1.w}};
        v8h ph, pl;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const float p = __builtin_amdgcn_exp2f(x[s][i] - m);
                lp += p;
                float pv = p * (svv[s][i] * (i & 1 ? fv : fv16));
                // past t_end the scale may be anything: the weight is zero
                if (MASK && !(4 * s + i < nval)) pv = 0.0f;
                const F16Pair hl = split_f16(pv);
                ph[2 * i + s] = hl.hi;
                pl[2 * i + s] = hl.lo;
            }
        sv0 = *reinterpret_cast<const float4*>(vsc + tn);
        sv1 = *reinterpret_cast<const float4*>(vsc + tn + 4);
        const uint32_t vw[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const v8h va = nib8_h8x16(vw[db]);
            O[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, ph, O[db], 0, 0, 0);
            O[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pl, O[db], 0, 0, 0);
        }
        v0 = *reinterpret_cast<const uint4*>(vptr(tn));
        v1 = *reinterpret_cast<const uint4*>(vptr(tn) + 64);
    };
    for (; t0 + 32 <= t_end; t0 += 32 * kWaves) tile(std::false_type{});
    if (t0 < t_end) tile(std::true_type{});

    // column totals over the four lane groups; the chunk's value scale
    // exponent goes back in here (a power of two, exact)
    lp += __shfl_xor(lp, 16);
    lp += __shfl_xor(lp, 32);
    const float unv = pow2i(ev - 4);
    if (q4 == 0) {
        sm[w][c16] = m;
        sl[w][c16] = lp;
    }
    __syncthreads();                         // every wave is done with sq
    float* so = reinterpret_cast<float*>(dyn);     // [kWaves][G][kHd]
    if (c16 < G) {
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                so[(w * G + c16) * kHd + 16 * q4 + 4 * i + (db & 3) + 64 * (db >> 2)] =
                    O[db][i] * unv;
    }
    __syncthreads();
    // merge the four waves
    const int nch = (a.max_seq + C - 1) / C;
    float* rec = a.part + ((bh * nch) + c) * static_cast<size_t>(G) * (kHd + 2);
    for (int it = tid; it < G * kHd; it += kThreads) {
        const int gg = it / kHd;
        const int d = it % kHd;
        float M = sm[0][gg];
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, sm[ww][gg]);
        float o = 0.0f, l = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float f = __builtin_amdgcn_exp2f(sm[ww][gg] - M);
            o += f * so[(ww * G + gg) * kHd + d];
            l += f * sl[ww][gg];
        }
        rec[2 * G + gg * kHd + d] = o;
        if (d == 0) {
            rec[gg] = M;
            rec[G + gg] = l;
        }
    }
}

// ---------------------------------------------------------------------------
// Merge the chunk records of one (sequence, KV head); fp16 output.  A thread
// owns output elements (g, d); for up to 16 chunks it issues all its loads
// (m_c, l_c and O_c[g][d] of every chunk) at once, so the merge costs one
// memory round trip.
// ---------------------------------------------------------------------------
constexpr int kCombineFast = 16;

__global__ __launch_bounds__(kThreads) void k_attn_combine(AttnArgs a) {
    const int hk = blockIdx.x;
    const int b = blockIdx.y;
    const int C = a.chunk;
    const int G = a.heads_q / a.heads_kv;
    int L = a.lengths[b];
    L = L < 0 ? 0 : (L > a.max_seq ? a.max_seq : L);
    const int nc = (L + C - 1) / C;
    const int nch = (a.max_seq + C - 1) / C;
    const size_t bh = static_cast<size_t>(b) * a.heads_kv + hk;
    const size_t rs = static_cast<size_t>(G) * (kHd + 2);
    const float* rec0 = a.part + bh * nch * rs;
    uint16_t* out = a.out + (static_cast<size_t>(b) * a.heads_q + hk * G) * kHd;
    for (int it = threadIdx.x; it < G * kHd; it += kThreads) {
        const int gg = it / kHd;
        const int d = it % kHd;
        float r = 0.0f;
        if (nc > 0 && nc <= kCombineFast) {
            float mc[kCombineFast], lc[kCombineFast], oc[kCombineFast];
#pragma unroll
            for (int cc = 0; cc < kCombineFast; ++cc) {
                const float* rc = rec0 + (cc < nc ? cc : 0) * rs;
                mc[cc] = rc[gg];
                lc[cc] = rc[G + gg];
                oc[cc] = rc[2 * G + gg * kHd + d];
            }
            float M = -__builtin_inff();
#pragma unroll
            for (int cc = 0; cc < kCombineFast; ++cc)
                if (cc < nc) M = fmaxf(M, mc[cc]);
            float num = 0.0f, den = 0.0f;
#pragma unroll
            for (int cc = 0; cc < kCombineFast; ++cc)
                if (cc < nc) {
                    const float f = __builtin_amdgcn_exp2f(mc[cc] - M);
                    num += f * oc[cc];
                    den += f * lc[cc];
                }
            r = num / den;
        } else if (nc > 0) {
            float M = -__builtin_inff();
            for (int cc = 0; cc < nc; ++cc) M = fmaxf(M, rec0[cc * rs + gg]);
            float num = 0.0f, den = 0.0f;
            for (int cc = 0; cc < nc; ++cc) {
                const float* rc = rec0 + cc * rs;
                const float f = __builtin_amdgcn_exp2f(rc[gg] - M);
                num += f * rc[2 * G + gg * kHd + d];
                den += f * rc[G + gg];
            }
            r = num / den;
        }
        out[it] = f2h(r);
    }
}

}  // namespace

size_t attn_partial_lds(int G) {
    const size_t q = 2 * 4 * 64 * sizeof(v8h);
    const size_t o = static_cast<size_t>(kWaves) * G * kHd * sizeof(float);
    return q > o ? q : o;
}

int attn_chunk(int batch, int heads_kv, int max_seq) {
    // the largest power of two (<= 1024) that still gives about 8 workgroups
    // per compute unit
    const int cus = device_cu_count();
    int C = 1024;
    while (C > 128 &&
           static_cast<long>((max_seq + C - 1) / C) * batch * heads_kv < 8L * cus)
        C /= 2;
    return C;
}

size_t attn_partial_bytes(int batch, int heads_q, int heads_kv, int max_seq, int chunk) {
    const size_t nch = static_cast<size_t>((max_seq + chunk - 1) / chunk);
    const size_t G = static_cast<size_t>(heads_q / heads_kv);
    return static_cast<size_t>(batch) * heads_kv * nch * G * (kHd + 2) * sizeof(float);
}

hipError_t attn_decode_launch(const AttnArgs& a, hipStream_t stream) {
    if (a.batch == 0) return hipSuccess;
    const int nch = (a.max_seq + a.chunk - 1) / a.chunk;
    const size_t lds = attn_partial_lds(a.heads_q / a.heads_kv);
    k_attn_partial<<<dim3(nch, a.heads_kv, a.batch), kThreads, lds, stream>>>(a);
    k_attn_combine<<<dim3(a.heads_kv, a.batch), kThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace w4a4
