// INT4 KV cache: per-head transform, per-head symmetric INT4 quantization and
// packing of new keys and values into the caches.
//
// FlatQuant: Flatness Matters for LLM Quantization, section Transformer 集成:
// the key cache and the value cache each get a transform applied per head,
// P_h and P_v (full d x d matrices, not Kronecker-factored).  FPTQuant page,
// sections 核心贡献 and 实验结果: INT4 KV cache (W4A4KV4).  The quantizer is
// the activations' one (FRM-PTQ page, 初步介绍, z = 0; FlatQuant's clip α),
// one scale per head vector of each token.
//
// Cache layout (one layer, head size 128):
//   keys   uint8  [batch][heads][max_seq][64]     two codes per byte, low
//                                                 nibble = even channel
//   values uint32 [batch][heads][max_seq/8][128]  nibble j of a word = token
//                                                 8*block + j of that channel
//   scales float  [batch][heads][max_seq]         one per head vector
// Keys are laid out for the score product (contraction over channels), values
// for the probability-value product (contraction over tokens): the decode
// attention kernel reads both as MFMA operands with no transpose.
#include "common.hpp"
#include "internal.hpp"

namespace w4a4 {

namespace {

constexpr int kHd = 128;       // head size
constexpr int kTile = 32;      // positions per work unit (aligned to 32)
constexpr int kThreads = 256;

struct Seg {
    int seq, p, n, t0;         // n clipped to the cache; 0 = skipped
};

__device__ __forceinline__ Seg load_seg(const KvAppendArgs& a, int i) {
    Seg s;
    s.seq = a.seg_seq[i];
    s.p = a.seg_start[i];
    s.t0 = a.cu_tokens[i];
    const int t1 = a.cu_tokens[i + 1];
    int n = t1 - s.t0;
    const bool ok = s.seq >= 0 && s.seq < a.batch && s.p >= 0 && s.p < a.max_seq && n > 0 &&
                    s.t0 >= 0 && t1 <= a.tokens;
    s.n = ok ? min(n, a.max_seq - s.p) : 0;
    return s;
}

// aligned 32-position tiles a segment touches
__device__ __forceinline__ int seg_tiles(const Seg& s) {
    return s.n > 0 ? (s.p + s.n - 1) / kTile - s.p / kTile + 1 : 0;
}

// Work unit u -> (segment, tile within the segment) by a block-wide prefix sum
// over the segments' tile counts.  Returns false when u is past the last tile.
__device__ bool find_unit(const KvAppendArgs& a, int u, int* seg, int* tile) {
    __shared__ int sc[kThreads];
    __shared__ int found_seg, found_tile;
    const int tid = threadIdx.x;
    if (tid == 0) found_seg = -1;
    __syncthreads();
    int base = 0;
    for (int b0 = 0; b0 < a.segments; b0 += kThreads) {
        const int i = b0 + tid;
        const int t = i < a.segments ? seg_tiles(load_seg(a, i)) : 0;
        sc[tid] = t;
        __syncthreads();
        for (int off = 1; off < kThreads; off <<= 1) {
            const int v = tid >= off ? sc[tid - off] : 0;
            __syncthreads();
            sc[tid] += v;
            __syncthreads();
        }
        const int incl = sc[tid];
        const int excl = incl - t;
        if (t > 0 && u >= base + excl && u < base + incl) {
            found_seg = i;
            found_tile = u - base - excl;
        }
        const int total = sc[kThreads - 1];
        __syncthreads();
        if (found_seg >= 0) break;
        base += total;
    }
    *seg = found_seg;
    *tile = found_tile;
    return found_seg >= 0;
}

// ---------------------------------------------------------------------------
// Z[r][:] = xs[r][:] · Pm for r < rows (rows <= 32), in place, fp32.  Thread:
// column e = tid % 128 and half dh = tid / 128 of the contraction.  The
// thread's 64 matrix entries (pcol_load, issued before the rows are loaded so
// that the two loads overlap) stay in registers and serve every row; the two
// halves are added through LDS.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void pcol_load(const float* __restrict__ Pm, float (&p)[64]) {
    const int e = threadIdx.x & (kHd - 1);
    const int dh = threadIdx.x >> 7;
#pragma unroll
    for (int i = 0; i < 64; ++i) p[i] = Pm[(64 * dh + i) * kHd + e];
}

__device__ __forceinline__ void rows_times(float (*xs)[kHd], int rows, const float (&p)[64]) {
    const int tid = threadIdx.x;
    const int e = tid & (kHd - 1);
    const int dh = tid >> 7;
    float acc[kTile];
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
        acc[r] = 0.0f;
        if (r < rows) {
            const float4* xr = reinterpret_cast<const float4*>(&xs[r][64 * dh]);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float4 x = xr[j];
                acc[r] = fmaf(x.x, p[4 * j], acc[r]);
                acc[r] = fmaf(x.y, p[4 * j + 1], acc[r]);
                acc[r] = fmaf(x.z, p[4 * j + 2], acc[r]);
                acc[r] = fmaf(x.w, p[4 * j + 3], acc[r]);
            }
        }
    }
    __syncthreads();
    if (dh == 1) {
#pragma unroll
        for (int r = 0; r < kTile; ++r)
            if (r < rows) xs[r][e] = acc[r];
    }
    __syncthreads();
    if (dh == 0) {
#pragma unroll
        for (int r = 0; r < kTile; ++r)
            if (r < rows) xs[r][e] += acc[r];
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// One workgroup: one 32-position tile of one segment, heads
// [blockIdx.y * hpw, +hpw), keys (blockIdx.z == 0) or values (== 1).
// Rows (position, head) are processed in batches of at most 32, each batch
// holding whole heads so that a value word's 8 tokens are written together.
// The transform runs in fp32 (fp16 inputs are exact in fp32).  The LDS
// holds the batch's inputs, then its Z, then its codes.
// ---------------------------------------------------------------------------
template <bool PER_HEAD>
__global__ __launch_bounds__(kThreads) void k_kv_append(KvAppendArgs a) {
    __shared__ float xs[kTile][kHd];     // inputs, then Z
    __shared__ uint8_t cs[kTile][kHd];   // codes as nibbles
    const int tid = threadIdx.x;
    int seg, tile;
    if (!find_unit(a, blockIdx.x, &seg, &tile)) return;
    const bool isv = blockIdx.z == 1;
    const uint16_t* X = isv ? a.v : a.k;
    const float* P = isv ? a.P_v : a.P_h;
    const float alpha = isv ? a.alpha_v : a.alpha_k;
    float* scale = isv ? a.v_scale : a.k_scale;
    const Seg s = load_seg(a, seg);
    const int P0 = (s.p / kTile + tile) * kTile;
    const int lo = max(P0, s.p);
    const int hi = min(P0 + kTile, s.p + s.n);
    const int npos = hi - lo;                       // >= 1
    const int h0 = blockIdx.y * a.hpw;
    const int nh = min(a.hpw, a.heads - h0);
    if (nh <= 0) return;
    // heads per batch: with per-head matrices one head, so that the rows of a
    // batch share their matrix
    const int hpb = PER_HEAD ? 1 : max(1, min(nh, kTile / npos));
    const int H = a.heads;

    float p[64];
    if (!PER_HEAD) pcol_load(P, p);
    for (int hb = 0; hb < nh; hb += hpb) {
        const int bh = min(hpb, nh - hb);
        if (PER_HEAD) pcol_load(P + static_cast<size_t>(h0 + hb) * kHd * kHd, p);
        const int rows = bh * npos;                 // row r: head hb + r / npos, position lo + r % npos
        // load the rows (16 halves per thread-iteration)
        for (int c = tid; c < rows * (kHd / 8); c += kThreads) {
            const int r = c / (kHd / 8);
            const int col = (c % (kHd / 8)) * 8;
            const int h = h0 + hb + r / npos;
            const int tok = s.t0 + (lo + r % npos - s.p);
            const uint4 w = *reinterpret_cast<const uint4*>(
                X + (static_cast<size_t>(tok) * H + h) * kHd + col);
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xs[r][col + 2 * i] = h2f(static_cast<uint16_t>(ww[i] & 0xFFFFu));
                xs[r][col + 2 * i + 1] = h2f(static_cast<uint16_t>(ww[i] >> 16));
            }
        }
        __syncthreads();
        // Z = X · P of the batch's head (every row of a batch shares it)
        rows_times(xs, rows, p);
        // quantize: one wave per row, two channels per lane
        const int lane = tid & 63;
        const int wv = tid >> 6;
        for (int r = wv; r < rows; r += kThreads / 64) {
            const float z0 = xs[r][lane];
            const float z1 = xs[r][lane + 64];
            const float m = wave_max(fmaxf(fabsf(z0), fabsf(z1)));
            const float sc = alpha * m / 7.0f;
            const bool zero = !(sc > 0.0f);
            const float inv = zero ? 0.0f : 1.0f / sc;
            cs[r][lane] = static_cast<uint8_t>(quant_nibble(z0, inv, zero));
            cs[r][lane + 64] = static_cast<uint8_t>(quant_nibble(z1, inv, zero));
            if (lane == 0) {
                const int h = h0 + hb + r / npos;
                const int pos = lo + r % npos;
                scale[(static_cast<size_t>(s.seq) * H + h) * a.max_seq + pos] = sc;
            }
        }
        __syncthreads();
        if (!isv) {
            // keys: one 32-bit word (8 codes) per thread-iteration
            for (int c = tid; c < rows * (kHd / 8); c += kThreads) {
                const int r = c / (kHd / 8);
                const int dw = c % (kHd / 8);
                uint32_t word = 0;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    word |= static_cast<uint32_t>(cs[r][8 * dw + j]) << (4 * j);
                const int h = h0 + hb + r / npos;
                const int pos = lo + r % npos;
                reinterpret_cast<uint32_t*>(
                    a.k_cache + ((static_cast<size_t>(s.seq) * H + h) * a.max_seq + pos) *
                                    (kHd / 2))[dw] = word;
            }
        } else {
            // values: one word per (head, 8-token block, channel); tokens of
            // the block outside [lo, hi) keep their stored nibbles
            const int fb = (lo - P0) / 8;
            const int nb = (hi - 1 - P0) / 8 - fb + 1;
            for (int c = tid; c < bh * nb * kHd; c += kThreads) {
                const int hl = c / (nb * kHd);
                const int blk = fb + (c / kHd) % nb;
                const int ch = c % kHd;
                const int h = h0 + hb + hl;
                uint32_t* dst = a.v_cache +
                                ((static_cast<size_t>(s.seq) * H + h) * (a.max_seq / 8) +
                                 P0 / 8 + blk) * kHd + ch;
                uint32_t keep = 0;
                uint32_t word = 0;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int pos = P0 + 8 * blk + j;
                    if (pos >= lo && pos < hi)
                        word |= static_cast<uint32_t>(cs[hl * npos + pos - lo][ch]) << (4 * j);
                    else
                        keep |= 0xFu << (4 * j);
                }
                if (keep) word |= *dst & keep;
                *dst = word;
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// y[h] = scale * q[h] · M for the query heads [blockIdx.x * rw, +rw) of
// sequence blockIdx.y, fp32 out.  rw = G with per-head matrices (the heads of
// one KV head), else up to 8 heads sharing the one matrix.
// ---------------------------------------------------------------------------
template <bool PER_HEAD>
__global__ __launch_bounds__(kThreads) void k_rows_xform(const uint16_t* __restrict__ q,
                                                         int heads_q, int G, int rw,
                                                         const float* __restrict__ M,
                                                         float scale, float* __restrict__ out) {
    __shared__ float xs[kTile][kHd];
    const int h0 = blockIdx.x * rw;
    const int rows = min(rw, heads_q - h0);
    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const size_t row0 = static_cast<size_t>(b) * heads_q + h0;
    float p[64];
    pcol_load(M + (PER_HEAD ? static_cast<size_t>(h0 / G) * kHd * kHd : 0), p);
    for (int c = tid; c < rows * kHd; c += kThreads) xs[c / kHd][c % kHd] = h2f(q[row0 * kHd + c]);
    __syncthreads();
    rows_times(xs, rows, p);
    for (int c = tid; c < rows * kHd; c += kThreads) out[row0 * kHd + c] = xs[c / kHd][c % kHd] * scale;
}

}  // namespace

int kv_append_hpw(int tokens, int segments, int heads) {
    // decode-like calls (about one token per segment): all heads of a token in
    // one workgroup, so the transform matrix is read once per token
    return (tokens <= 2 * segments) ? min(heads, 8) : 1;
}

hipError_t kv_append_launch(const KvAppendArgs& a, bool per_head, hipStream_t stream) {
    if (a.tokens == 0 || a.segments == 0) return hipSuccess;
    const long units = static_cast<long>(a.tokens) / kTile + 2L * a.segments + 1;
    dim3 grid(static_cast<unsigned>(units), ceil_div(a.heads, a.hpw), 2);
    if (per_head)
        k_kv_append<true><<<grid, kThreads, 0, stream>>>(a);
    else
        k_kv_append<false><<<grid, kThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t rows_xform_launch(const uint16_t* q, int batch, int heads_q, int heads_kv,
                             const float* M, bool per_head, float scale, float* out,
                             hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    const int G = heads_q / heads_kv;
    // 8 heads per workgroup (one KV head's G with per-head matrices): enough
    // workgroups to cover the chip for decode batches
    const int rw = per_head ? G : min(heads_q, 8);
    dim3 grid(ceil_div(heads_q, rw), batch);
    if (per_head)
        k_rows_xform<true><<<grid, kThreads, 0, stream>>>(q, heads_q, G, rw, M, scale, out);
    else
        k_rows_xform<false><<<grid, kThreads, 0, stream>>>(q, heads_q, G, rw, M, scale, out);
    return hipGetLastError();
}

}  // namespace w4a4
