// Offline weight preparation: merge of the inverse transform and RTN INT4
// quantization with nibble packing.
//
// FlatQuant: Flatness Matters for LLM Quantization, section Kronecker 分解:
// the weight-side factor P1^-1 ×1 W̃ ×2 (P2^-1)^T; section 额外可学习组件:
// diag(c) undone on the weights, clipping threshold α_w.
// FRM-PTQ page, section 初步介绍: Q(W) = clamp(round(W/s) + z, 0, 2^b - 1),
// and the page's group-wise (multi-granularity) weight quantization.
// MergeQuant page, 关键设计 item 2: per-channel static activation steps are
// folded into the weights of the linear layer (step migration).
#include "common.hpp"
#include "internal.hpp"

namespace w4a4 {

namespace {

static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// ---------------------------------------------------------------------------
// Gauss-Jordan inversion with partial pivoting, float64, one workgroup.
// A is [n, 2n] in global memory: [P | I] -> [I | P^-1].  Pivot magnitudes are
// recorded so the host can reject singular factors.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_invert(const float* __restrict__ P, int n,
                                                  double* __restrict__ A,
                                                  double* __restrict__ minpiv) {
    __shared__ double sval[1024];
    __shared__ int sidx[1024];
    __shared__ int piv_row;
    const int tid = threadIdx.x;
    const int w = 2 * n;
    for (int e = tid; e < n * w; e += blockDim.x) {
        const int r = e / w, col = e % w;
        A[e] = (col < n) ? static_cast<double>(P[r * n + col]) : (col - n == r ? 1.0 : 0.0);
    }
    double mp = __builtin_inf();
    __syncthreads();
    for (int k = 0; k < n; ++k) {
        // pivot search in column k, rows k..n-1
        double best = -1.0;
        int bi = k;
        for (int r = k + tid; r < n; r += blockDim.x) {
            const double v = fabs(A[r * w + k]);
            if (v > best) { best = v; bi = r; }
        }
        sval[tid] = best;
        sidx[tid] = bi;
        __syncthreads();
        for (int s = blockDim.x / 2; s > 0; s >>= 1) {
            if (tid < s) {
                const double o = sval[tid + s];
                const int oi = sidx[tid + s];
                if (o > sval[tid] || (o == sval[tid] && oi < sidx[tid])) {
                    sval[tid] = o;
                    sidx[tid] = oi;
                }
            }
            __syncthreads();
        }
        if (tid == 0) piv_row = sidx[0];
        mp = fmin(mp, sval[0]);
        __syncthreads();
        const int pr = piv_row;
        if (pr != k) {
            for (int col = tid; col < w; col += blockDim.x) {
                const double t = A[k * w + col];
                A[k * w + col] = A[pr * w + col];
                A[pr * w + col] = t;
            }
        }
        __syncthreads();
        const double pv = A[k * w + k];
        __syncthreads();
        if (pv != 0.0) {
            for (int col = tid; col < w; col += blockDim.x) A[k * w + col] /= pv;
        }
        __syncthreads();
        for (int e = tid; e < n * w; e += blockDim.x) {
            const int r = e / w, col = e % w;
            if (r != k && col != k) A[e] -= A[r * w + k] * A[k * w + col];
        }
        __syncthreads();
        for (int r = tid; r < n; r += blockDim.x)
            if (r != k) A[r * w + k] = 0.0;
        __syncthreads();
    }
    if (tid == 0) *minpiv = mp;
}

// Copy the inverse out of [I | P^-1] as a dense n x n matrix, optionally
// transposed, so the merge kernel reads it with unit stride.
__global__ __launch_bounds__(256) void k_extract_inverse(const double* __restrict__ A, int n,
                                                         bool transpose,
                                                         double* __restrict__ out) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= n * n) return;
    const int r = e / n, col = e % n;
    const double v = A[r * 2 * n + n + col];
    out[transpose ? col * n + r : e] = v;
}

// [I | P^-1] -> (P^-1)^T as fp32 (one rounding from fp64)
__global__ __launch_bounds__(256) void k_extract_inverse_t32(const double* __restrict__ A, int n,
                                                             float* __restrict__ out) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= n * n) return;
    const int r = e / n, col = e % n;
    out[col * n + r] = static_cast<float>(A[r * 2 * n + n + col]);
}

// ---------------------------------------------------------------------------
// Merge: Wt[n] = P1inv · (W̄[n] / c) · P2inv^T in float64, rounded to fp32.
// One persistent workgroup per row slot; U = W̄·P2inv^T lives in a float64
// slice of the workspace owned by the workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_merge(const float* __restrict__ W, int N, int n1,
                                               int n2, const double* __restrict__ P1inv,
                                               const double* __restrict__ P2invT,
                                               const float* __restrict__ c,
                                               double* __restrict__ Uws,
                                               float* __restrict__ Wt) {
    const int K = n1 * n2;
    double* U = Uws + static_cast<size_t>(blockIdx.x) * K;
    for (int row = blockIdx.x; row < N; row += gridDim.x) {
        const float* wr = W + static_cast<size_t>(row) * K;
        // U[i, j] = Σ_q (W̄[i,q]/c) · P2inv[j, q]   (P2invT[q, j] = P2inv[j, q])
        for (int e = threadIdx.x; e < K; e += blockDim.x) {
            const int i = e / n2, j = e % n2;
            double acc = 0.0;
            for (int q = 0; q < n2; ++q) {
                double v = static_cast<double>(wr[i * n2 + q]);
                if (c) v /= static_cast<double>(c[i * n2 + q]);
                acc = fma(v, P2invT[q * n2 + j], acc);
            }
            U[e] = acc;
        }
        __syncthreads();
        // Wt[i, j] = Σ_r P1inv[i, r] · U[r, j]
        float* out = Wt + static_cast<size_t>(row) * K;
        for (int e = threadIdx.x; e < K; e += blockDim.x) {
            const int i = e / n2, j = e % n2;
            double acc = 0.0;
            for (int r = 0; r < n1; ++r) acc = fma(P1inv[i * n1 + r], U[r * n2 + j], acc);
            out[e] = static_cast<float>(acc);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Pack: one workgroup per (row, group).  Range reduction in fp32 (exact for
// min / max), scale arithmetic in float64, direct float64 -> fp16 rounding,
// codes from the stored fp16 scale with float64 division.  qmax = 2^(b-1) - 1
// and umax = 2^b - 1 for b-bit codes (b = 4 or 3), one code per nibble.
// ---------------------------------------------------------------------------
template <bool ASYM>
__global__ __launch_bounds__(256) void k_pack(const float* __restrict__ Wt, int K,
                                              int group_size, float alpha, double qmax,
                                              double umax, uint8_t* __restrict__ Wq,
                                              uint16_t* __restrict__ s_w,
                                              uint16_t* __restrict__ z_w) {
    __shared__ float rmin[4], rmax[4];
    __shared__ double s_sh, z_sh;
    const int row = blockIdx.x;
    const int g = blockIdx.y;
    const int G = K / group_size;
    const float* v = Wt + static_cast<size_t>(row) * K + static_cast<size_t>(g) * group_size;
    float lo = __builtin_inff(), hi = -__builtin_inff();
    for (int e = threadIdx.x; e < group_size; e += blockDim.x) {
        lo = fminf(lo, v[e]);
        hi = fmaxf(hi, v[e]);
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    if ((threadIdx.x & 63) == 0) {
        rmin[threadIdx.x >> 6] = lo;
        rmax[threadIdx.x >> 6] = hi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float mn = rmin[0], mx = rmax[0];
        for (int w = 1; w < static_cast<int>(blockDim.x >> 6); ++w) {
            mn = fminf(mn, rmin[w]);
            mx = fmaxf(mx, rmax[w]);
        }
        const double a = static_cast<double>(alpha);
        uint16_t sbits;
        double z = 0.0;
        if (!ASYM) {
            const double amax = fmax(fabs(static_cast<double>(mn)), fabs(static_cast<double>(mx)));
            sbits = f64_to_f16_rne(a * amax / qmax);
        } else {
            const double dlo = a * fmin(static_cast<double>(mn), 0.0);
            const double dhi = a * fmax(static_cast<double>(mx), 0.0);
            sbits = f64_to_f16_rne((dhi - dlo) / umax);
            const double s = f16_bits_to_f64(sbits);
            if (s > 0.0) z = fmin(fmax(__builtin_rint(-dlo / s), 0.0), umax);
        }
        const double s = f16_bits_to_f64(sbits);
        s_w[static_cast<size_t>(row) * G + g] = sbits;
        if (ASYM) z_w[static_cast<size_t>(row) * G + g] = f64_to_f16_rne(z);
        s_sh = s;
        z_sh = z;
    }
    __syncthreads();
    const double s = s_sh;
    const double z = z_sh;
    const bool zero = !(s > 0.0);
    uint8_t* out = Wq + static_cast<size_t>(row) * (K / 2) + static_cast<size_t>(g) * (group_size / 2);
    for (int p = threadIdx.x; p < group_size / 2; p += blockDim.x) {
        uint32_t byte = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const double t = static_cast<double>(v[2 * p + h]) / (zero ? 1.0 : s);
            int q;
            if (ASYM)
                q = zero ? 0 : static_cast<int>(fmin(fmax(__builtin_rint(t) + z, 0.0), umax));
            else
                q = zero ? 0 : static_cast<int>(fmin(fmax(__builtin_rint(t), -qmax - 1.0), qmax));
            byte |= (static_cast<uint32_t>(q) & 0xFu) << (4 * h);
        }
        out[p] = static_cast<uint8_t>(byte);
    }
}

// ---------------------------------------------------------------------------
// Step migration: Wm[n, k] = Wt[n, k] * steps[k].  One fp32 multiply is the
// correctly rounded product, so the result is exactly fp32(Wt * step).
// Grid-stride over 4-element chunks (K % 4 == 0); in place is allowed.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_migrate(const float* Wt, int K, size_t chunks,
                                                 const float* __restrict__ steps, float* Wm) {
    const int kc = K / 4;
    for (size_t c = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < chunks;
         c += static_cast<size_t>(gridDim.x) * blockDim.x) {
        const int k4 = static_cast<int>(c % kc);
        float4 w = reinterpret_cast<const float4*>(Wt)[c];
        const float4 st = reinterpret_cast<const float4*>(steps)[k4];
        w.x *= st.x;
        w.y *= st.y;
        w.z *= st.z;
        w.w *= st.w;
        reinterpret_cast<float4*>(Wm)[c] = w;
    }
}

constexpr int kMergeBlocks = 256;

}  // namespace

size_t merge_workspace_bytes(int n1, int n2, int K) {
    return align256(sizeof(double) * 2 * n1 * n1) + align256(sizeof(double) * 2 * n2 * n2) +
           align256(sizeof(double) * n1 * n1) + align256(sizeof(double) * n2 * n2) +
           align256(sizeof(double) * 2) +
           align256(sizeof(double) * static_cast<size_t>(K) * kMergeBlocks);
}

hipError_t merge_launch(const float* W, int N, int K, int n1, int n2, const float* P1,
                        const float* P2, const float* c, float* Wt, void* ws,
                        hipStream_t stream, bool* singular) {
    char* p = static_cast<char*>(ws);
    double* A1 = reinterpret_cast<double*>(p);
    p += align256(sizeof(double) * 2 * n1 * n1);
    double* A2 = reinterpret_cast<double*>(p);
    p += align256(sizeof(double) * 2 * n2 * n2);
    double* P1inv = reinterpret_cast<double*>(p);
    p += align256(sizeof(double) * n1 * n1);
    double* P2invT = reinterpret_cast<double*>(p);
    p += align256(sizeof(double) * n2 * n2);
    double* piv = reinterpret_cast<double*>(p);
    p += align256(sizeof(double) * 2);
    double* U = reinterpret_cast<double*>(p);
    k_invert<<<1, 1024, 0, stream>>>(P1, n1, A1, piv);
    k_invert<<<1, 1024, 0, stream>>>(P2, n2, A2, piv + 1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    double hp[2];
    e = hipMemcpyAsync(hp, piv, sizeof(hp), hipMemcpyDeviceToHost, stream);
    if (e != hipSuccess) return e;
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return e;
    *singular = !(hp[0] > 1e-300) || !(hp[1] > 1e-300);
    if (*singular) return hipSuccess;
    k_extract_inverse<<<ceil_div(n1 * n1, 256), 256, 0, stream>>>(A1, n1, false, P1inv);
    k_extract_inverse<<<ceil_div(n2 * n2, 256), 256, 0, stream>>>(A2, n2, true, P2invT);
    const int blocks = N < kMergeBlocks ? N : kMergeBlocks;
    if (blocks > 0) k_merge<<<blocks, 256, 0, stream>>>(W, N, n1, n2, P1inv, P2invT, c, U, Wt);
    (void)K;
    return hipGetLastError();
}

size_t invert_t_workspace_bytes(int n, int count) {
    return align256(sizeof(double) * 2 * n * n) + align256(sizeof(double) * count);
}

hipError_t invert_t_launch(const float* P, int n, int count, float* out, void* ws,
                           hipStream_t stream, bool* singular) {
    double* A = static_cast<double*>(ws);
    double* piv = reinterpret_cast<double*>(static_cast<char*>(ws) +
                                            align256(sizeof(double) * 2 * n * n));
    for (int i = 0; i < count; ++i) {
        k_invert<<<1, 1024, 0, stream>>>(P + static_cast<size_t>(i) * n * n, n, A, piv + i);
        k_extract_inverse_t32<<<ceil_div(n * n, 256), 256, 0, stream>>>(
            A, n, out + static_cast<size_t>(i) * n * n);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    double hp[64];
    *singular = false;
    for (int i0 = 0; i0 < count; i0 += 64) {
        const int c = count - i0 < 64 ? count - i0 : 64;
        e = hipMemcpyAsync(hp, piv + i0, sizeof(double) * c, hipMemcpyDeviceToHost, stream);
        if (e != hipSuccess) return e;
        e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return e;
        for (int i = 0; i < c; ++i)
            if (!(hp[i] > 1e-300)) *singular = true;
    }
    return hipSuccess;
}

hipError_t migrate_steps_launch(const float* Wt, int N, int K, const float* steps, float* Wm,
                                hipStream_t stream) {
    const size_t chunks = static_cast<size_t>(N) * (K / 4);
    if (chunks == 0) return hipSuccess;
    const size_t want = (chunks + 255) / 256;
    const int blocks = static_cast<int>(want < 8192 ? want : 8192);
    k_migrate<<<blocks, 256, 0, stream>>>(Wt, K, chunks, steps, Wm);
    return hipGetLastError();
}

hipError_t pack_weights_launch(const float* Wt, int N, int K, int group_size, bool asym,
                               float alpha_w, int bits, uint8_t* Wq, uint16_t* s_w,
                               uint16_t* z_w, hipStream_t stream) {
    const double qmax = static_cast<double>((1 << (bits - 1)) - 1);
    const double umax = static_cast<double>((1 << bits) - 1);
    const int G = K / group_size;
    dim3 grid(N, G);
    const int threads = group_size >= 256 ? 256 : ((group_size + 63) / 64) * 64;
    if (asym)
        k_pack<true><<<grid, threads, 0, stream>>>(Wt, K, group_size, alpha_w, qmax, umax, Wq, s_w, z_w);
    else
        k_pack<false><<<grid, threads, 0, stream>>>(Wt, K, group_size, alpha_w, qmax, umax, Wq, s_w, z_w);
    return hipGetLastError();
}

}  // namespace w4a4
