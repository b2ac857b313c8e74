// common.h — internal helpers shared by the HIP sources of libvw4 (not public).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "vw4.h"

namespace vw4 {

// Thread-local error message, returned by vw4_last_error().
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

#define VW4_REQUIRE(cond, code, ...)      \
    do {                                  \
        if (!(cond)) {                    \
            ::vw4::set_error(__VA_ARGS__); \
            return (code);                \
        }                                 \
    } while (0)

// Checks the launch that was just enqueued.
int check_launch(const char* what);

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// ---------------------------------------------------------------------------
// Device-side number-format helpers.
// ---------------------------------------------------------------------------
// Compute units of the current device (cached per device; 256 if unknown).
static inline int device_cus() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

// binary32 -> bfloat16, round to nearest even, NaN kept quiet (upper 16 bits
// with the quiet bit set).  On gfx950 the compiler's conversion is one
// v_cvt_pk_bf16_f32, which gives exactly these bits for every one of the 2^32
// inputs in the default (IEEE, denormals kept) mode: checked exhaustively on
// MI355X against the integer form (u + 0x7fff + ((u >> 16) & 1)) >> 16.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

typedef __attribute__((ext_vector_type(2))) float vw4_f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 vw4_bf16x2;

// Two conversions in one instruction: lo in bits 0..15, hi in bits 16..31.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((vw4_f32x2){lo, hi}, vw4_bf16x2));
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return (float)v;
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
    _Float16 v = (_Float16)f;  // v_cvt_f16_f32, round to nearest even
    uint16_t h;
    __builtin_memcpy(&h, &v, 2);
    return h;
}

// Order-preserving key of a binary32 (ascending floats -> ascending keys);
// -0.0 is folded onto +0.0 so that equal floats share one key.
// Lane k's value of v, for every lane (k uniform): one wavefront walking a
// per-lane array in order without a round trip through LDS.
__device__ __forceinline__ double readlane_f64(double v, int k) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, k);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), k);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ uint32_t f32_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_f32(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

// RMSNorm sums of squares are kept per chunk of NORM_CHUNK columns
// ([M][ceil(D / NORM_CHUNK)] floats, summed in chunk order by every consumer).
constexpr int NORM_CHUNK = 256;

// Wavefront (64-lane) reductions via cross-lane moves.
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Sum over the S partial slices of element (m, c), slice order.  The loads
// of 8 slices are issued together (a chain of dependent loads would pay one
// memory latency per slice).
__device__ __forceinline__ float sum_parts(const float* __restrict__ part, int S, int M, int64_t ldp, int m,
                                           int64_t c) {
    float s = 0.0f;
    const int64_t stride = (int64_t)M * ldp;
    const float* p = part + (int64_t)m * ldp + c;
    for (int k0 = 0; k0 < S; k0 += 8) {
        float v[8];
        // slice index clamped instead of the load predicated: no branch
        // separates the loads (a branch would make the compiler wait for each)
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = p[(int64_t)(k0 + i < S ? k0 + i : S - 1) * stride];
#pragma unroll
        for (int i = 0; i < 8; ++i) s += (k0 + i < S) ? v[i] : 0.0f;
    }
    return s;
}

}  // namespace vw4
