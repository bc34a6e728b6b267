// Device helpers shared by the gfx950 kernels of libw4a4.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

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
// wave-level data movement and reductions (DPP, no LDS round trip)
// ---------------------------------------------------------------------------
// DPP controls (GFX9 encoding): quad_perm [1,0,3,2] swaps neighbours, quad_perm
// [2,3,0,1] swaps pairs, row_half_mirror reverses each 8 lanes, row_mirror
// reverses each 16 lanes.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}

// value of lane (l ^ 1)
__device__ __forceinline__ uint32_t lane_xor1(uint32_t v) {
    return static_cast<uint32_t>(dpp_i<kDppXor1>(static_cast<int>(v)));
}

// max over the 16 lanes of each row, in every lane of the row
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<kDppXor1>(v));
    v = fmaxf(v, dpp_f<kDppXor2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppMirror>(v));
    return v;
}
__device__ __forceinline__ float row16_min(float v) {
    v = fminf(v, dpp_f<kDppXor1>(v));
    v = fminf(v, dpp_f<kDppXor2>(v));
    v = fminf(v, dpp_f<kDppHalfMirror>(v));
    v = fminf(v, dpp_f<kDppMirror>(v));
    return v;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// max over the wave (64 lanes), wave-uniform result
__device__ __forceinline__ float wave_max(float v) {
    v = row16_max(v);
    return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)),
                 fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

__device__ __forceinline__ float wave_min(float v) {
    v = row16_min(v);
    return fminf(fminf(readlane_f(v, 0), readlane_f(v, 16)),
                 fminf(readlane_f(v, 32), readlane_f(v, 48)));
}

// t = z * inv_s (inv_s = 1/s of the token), round half to even, clamp to the
// signed range [-qmax - 1, qmax] (qmax = 7 for 4-bit codes, 3 for 3-bit), as a
// nibble; zero scale gives code 0
__device__ __forceinline__ uint32_t quant_nibble(float z, float inv_s, bool zero,
                                                 float qmax = 7.0f) {
    float r = __builtin_rintf(z * inv_s);
    r = fminf(fmaxf(r, -qmax - 1.0f), qmax);
    int q = zero ? 0 : static_cast<int>(r);
    return static_cast<uint32_t>(q) & 0xFu;
}

// The same code as quant_nibble for finite z: the product is clamped to
// [-qmax - 1, qmax] (v_med3) and rounded half to even by adding 1.5 * 2^23, whose
// float lands the integer in the low mantissa bits (two's complement in the
// low nibble).  A zero scale passes inv_s = 0 and gives code 0.
__device__ __forceinline__ uint32_t quant_nibble_magic(float z, float inv_s, float qmax = 7.0f) {
    const float t = __builtin_amdgcn_fmed3f(z * inv_s, -qmax - 1.0f, qmax);
    return __float_as_uint(t + 12582912.0f) & 0xFu;
}

// x = hi + lo in fp16 for MFMA operands.  hi is x with its float mantissa
// cut to fp16's 11 significant bits, so the conversion of hi to fp16 is exact
// (for |x| in fp16's normal range) whatever instruction and rounding the
// compiler picks for it; the packed and the scalar fp16 conversions have
// been seen to round a value very close to a rounding tie differently, and a
// hi converted twice must be the same number in both places.  lo = x - hi is
// exact in fp32 (at most 13 bits) and rounds once: |x - hi - lo| <= 2^-22 |x|.
struct F16Pair {
    _Float16 hi, lo;
};
__device__ __forceinline__ F16Pair split_f16(float x) {
    const float h = __uint_as_float(__float_as_uint(x) & 0xFFFFE000u);
    return {static_cast<_Float16>(h), static_cast<_Float16>(x - h)};
}

// floor(log2(x)) for a positive normal float
__device__ __forceinline__ int ilog2f(float x) {
    return static_cast<int>((__float_as_uint(x) >> 23) & 0xFFu) - 127;
}

// ---------------------------------------------------------------------------
// Packed 4-bit codes -> int8 MFMA operands
// ---------------------------------------------------------------------------
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

// unsigned nibbles u -> bytes u in [0, 15]
__device__ __forceinline__ void unpack_unsigned(const uint4& w, uint4& ev, uint4& od) {
    ev.x = w.x & 0x0F0F0F0Fu;
    ev.y = w.y & 0x0F0F0F0Fu;
    ev.z = w.z & 0x0F0F0F0Fu;
    ev.w = w.w & 0x0F0F0F0Fu;
    od.x = (w.x >> 4) & 0x0F0F0F0Fu;
    od.y = (w.y >> 4) & 0x0F0F0F0Fu;
    od.z = (w.z >> 4) & 0x0F0F0F0Fu;
    od.w = (w.w >> 4) & 0x0F0F0F0Fu;
}

// calls f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time
// ---------------------------------------------------------------------------
// direct-to-LDS copies and their synchronisation
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// 16-byte global -> LDS copy of one lane; the LDS address of lane l is
// lds_wave_base + 16 * l (the hardware adds the lane offset).
__device__ __forceinline__ void dma16(const void* src, uint8_t* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base,
                                     16, 0, 0);
}

// The same copy issued from inline assembly.  The compiler does not model it
// as a pending LDS write, so it inserts no wait for all outstanding copies
// before the next LDS read (which it must do for the builtin, not knowing
// which LDS bytes the copy writes); the caller orders copies and reads with
// its own s_waitcnt and barrier.  No output registers; the address registers
// are read at issue.  lds_wave_base must be wave-uniform.
__device__ __forceinline__ void dma16_async(const void* src, const uint8_t* lds_wave_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
            (const __attribute__((address_space(3))) uint8_t*)lds_wave_base)));
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(m0)
                 : "memory", "m0");
}

// Copies from a wave-uniform 64-bit base (scalar registers) and a per-lane
// 32-bit byte offset, issued like dma16_async: the compiler does not see
// them, the caller's s_waitcnt counts them.  The wave's LDS destination is a
// 32-bit LDS byte address (wave-uniform; the value m0 takes).  Taken from a
// __shared__ array cast to the LDS address space plus scalar offsets, it
// stays in scalar registers, where a generic LDS pointer is carried in a
// vector register pair and converted (readfirstlane, null test) at every
// copy.
__device__ __forceinline__ uint32_t lds_addr(const __attribute__((address_space(3))) uint8_t* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// the base is wave-uniform by contract; readfirstlane puts it in scalar
// registers where the compiler cannot prove it.  The builtin returns a signed
// int: each half goes through uint32_t before widening, so the low half is
// zero-extended
__device__ __forceinline__ uint64_t uniform_base(const void* base) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32)));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// 16 bytes per lane; the LDS address of lane l is lds_m0 + 16 * l
__device__ __forceinline__ void dma16_async_sv(const void* base, uint32_t off, uint32_t lds_m0) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_m0);
    const uint64_t bs = uniform_base(base);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(bs), "s"(m0)
                 : "memory", "m0");
}

// 4 bytes per lane; the LDS address of lane l is lds_m0 + 4 * l
__device__ __forceinline__ void dma4_async_sv(const void* base, uint32_t off, uint32_t lds_m0) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_m0);
    const uint64_t bs = uniform_base(base);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" : : "v"(off), "s"(bs), "s"(m0)
                 : "memory", "m0");
}

// the same with the destination as a generic pointer to the wave's LDS base
__device__ __forceinline__ void dma16_async_sv(const void* base, uint32_t off, const uint8_t* lds_wave_base) {
    dma16_async_sv(base, off, lds_addr((const __attribute__((address_space(3))) uint8_t*)lds_wave_base));
}

__device__ __forceinline__ void dma4_async_sv(const void* base, uint32_t off, const uint8_t* lds_wave_base) {
    dma4_async_sv(base, off, lds_addr((const __attribute__((address_space(3))) uint8_t*)lds_wave_base));
}

// Workgroup barrier without a memory fence; the compiler-only fences keep
// LDS accesses from being moved across it.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Compute units of the current device (cached per device ordinal).
inline int device_cu_count() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n < 1)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

}  // namespace w4a4
