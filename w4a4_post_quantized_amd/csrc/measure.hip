// Measurement aid: the HBM read rate that one launch of a given size
// reaches on this device (the ceiling the decode GEMM's bandwidth is read
// against).  Every lane streams 16-byte loads, eight in flight, over a
// persistent grid; the XOR of all 32-bit words is kept so the loads cannot
// be dropped.
#include "common.hpp"
#include "internal.hpp"

namespace w4a4 {

namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeDepth = 8;                  // 16-byte loads in flight per lane

__global__ __launch_bounds__(kProbeThreads) void k_read_probe(const uint4* __restrict__ p,
                                                              size_t n16,
                                                              uint32_t* __restrict__ out) {
    const size_t stride = static_cast<size_t>(gridDim.x) * kProbeThreads;
    size_t i = static_cast<size_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
    uint32_t x = 0;
    for (; i + (kProbeDepth - 1) * stride < n16; i += kProbeDepth * stride) {
        uint4 v[kProbeDepth];
#pragma unroll
        for (int d = 0; d < kProbeDepth; ++d) v[d] = p[i + d * stride];
#pragma unroll
        for (int d = 0; d < kProbeDepth; ++d) x ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = p[i];
        x ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    // one atomic per workgroup: the waves' words meet in LDS first
    for (int o = 32; o >= 1; o >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), o));
    __shared__ uint32_t red[kProbeThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t y = 0;
#pragma unroll
        for (int w = 0; w < kProbeThreads / 64; ++w) y ^= red[w];
        atomicXor(out, y);
    }
}

}  // namespace

hipError_t read_probe_launch(const void* buf, size_t bytes, uint32_t* out, hipStream_t stream) {
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    // a persistent grid of two workgroups per CU (each lane then streams
    // bytes / (CUs x 1024 x 16) loads; small reads get fewer workgroups)
    const size_t want = (n16 + kProbeThreads * kProbeDepth - 1) / (kProbeThreads * kProbeDepth);
    const size_t cap = static_cast<size_t>(device_cu_count()) * 2;
    const unsigned grid = static_cast<unsigned>(want < cap ? want : cap);
    k_read_probe<<<grid, kProbeThreads, 0, stream>>>(static_cast<const uint4*>(buf), n16, out);
    return hipGetLastError();
}

}  // namespace w4a4
