// Device helpers shared by the gfx950 kernels of libw4a4.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "w4a4.h"

namespace w4a4 {

// ---------------------------------------------------------------------------
// fp16 <-> float
// ---------------------------------------------------------------------------
__device__ __forceinline__ float h2f(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// float -> fp16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f2h(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// double -> fp16 bits with ONE rounding (nearest, ties to even).  A
// conversion through float32 could round twice; the weight scales must match
// a direct conversion bit for bit.  Values at or above 65520 give +-inf.
__host__ __device__ inline uint16_t f64_to_f16_rne(double x) {
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const uint16_t sign = static_cast<uint16_t>((b >> 48) & 0x8000u);
    const uint64_t a = b & 0x7FFFFFFFFFFFFFFFull;
    if (a >= 0x7FF0000000000000ull) {                       // inf or nan
        return sign | (a > 0x7FF0000000000000ull ? 0x7E00u : 0x7C00u);
    }
    const int E = static_cast<int>(a >> 52) - 1023;
    if (E >= 16) return sign | 0x7C00u;                      // >= 65536
    if (E < -25) return sign;                                // < 2^-25: to zero
    const uint64_t man = a & 0x000FFFFFFFFFFFFFull;
    uint64_t res, rem, half;
    if (E >= -14) {                                          // normal fp16
        res = (static_cast<uint64_t>(E + 15) << 10) | (man >> 42);
        rem = man & ((1ull << 42) - 1);
        half = 1ull << 41;
    } else {                                                 // subnormal fp16
        const uint64_t full = man | (1ull << 52);
        const int shift = 28 - E;                            // 43 .. 53
        res = full >> shift;
        rem = full & ((1ull << shift) - 1);
        half = 1ull << (shift - 1);
    }
    if (rem > half || (rem == half && (res & 1u))) res += 1; // carry may give inf
    return sign | static_cast<uint16_t>(res);
}

__host__ __device__ inline double f16_bits_to_f64(uint16_t h) {
    const int s = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1F;
    const int m = h & 0x3FF;
    double v;
    if (e == 0) {
        v = static_cast<double>(m) * 5.9604644775390625e-08;  // 2^-24
    } else if (e == 31) {
        v = m ? __builtin_nan("") : __builtin_inf();
    } else {
        v = static_cast<double>(1024 + m) * __builtin_ldexp(1.0, e - 25);
    }
    return s ? -v : v;
}

// ---------------------------------------------------------------------------
// reductions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
    return v;
}

// round half to even, clamp to the signed 4-bit range, as a nibble
__device__ __forceinline__ uint32_t quant_nibble(float z, float inv_or_s, bool zero) {
    float t = z / inv_or_s;
    float r = __builtin_rintf(t);
    r = fminf(fmaxf(r, -8.0f), 7.0f);
    int q = zero ? 0 : static_cast<int>(r);
    return static_cast<uint32_t>(q) & 0xFu;
}

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace w4a4
