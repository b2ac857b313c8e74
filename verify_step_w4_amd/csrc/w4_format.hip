// w4_format.hip — the W4 weight format: quantiser (host and device), packing
// into the kernel layout and back, plus the library's error plumbing.
//
// Format (hazakura.dev, "mtplx——M5 Maxで63tok/s…", section "4層のアーキテクチャ",
// Layer 0 names a 4-bit LM head; the group size, symmetry and fp16 scale are
// the workload's): per row n and 64-element group g along K,
//     scale = fp16_rne(absmax / 7)          (binary32 division, then RNE to fp16)
//     c_k   = clamp(rint(w_k / scale), -7, 7)  with the *rounded* scale, half-even
//     an all-zero (or fp16-underflowing) group gets scale 0 and codes 0.
//
// Packed layout (what w4_skinny_gemm streams), built for the matrix-core
// GEMM: rows are padded to a multiple of 64 and grouped in tiles of 64 rows;
// tile t and K-group g own a 2 KiB block at (t * G + g) * 2048 bytes.  Lane
// l = 16 kq + i (kq, i = 0..3, 0..15) of a wavefront owns 8 dwords of it,
// dword d = 2 nb + s at byte ((t * G + g) * 2 + d / 4) * 1024 + l * 16 +
// (d % 4) * 4 (so each of the lane's two 16-byte loads is part of one
// contiguous 1 KiB wavefront load); that dword holds row t * 64 + 16 nb + i,
// k = 64 g + 32 s + 8 kq + j (j = 0..7), which is exactly one 8-element
// operand of v_mfma_f32_16x16x32_bf16 for lane l.  Inside the dword the code
// nibble u = c + 8 of element j sits at bit 4 * (j / 2) for even j and
// 16 + 4 * (j / 2) for odd j, so ((dword >> 4i) & 0x000F000F) is the element
// pair (2i, 2i + 1), one per 16-bit half.
// Scales: fp16 [t][g][i][nb] (lane l reads its four row scales as 8 bytes).
#include <math.h>
#include <stdarg.h>

#include "common.h"

namespace vw4 {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_error("%s: launch failed: %s", what, hipGetErrorString(e));
        return VW4_EHIP;
    }
    return VW4_OK;
}

// ---------------------------------------------------------------------------
// Quantiser arithmetic, one group of 64.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int quant_code(float w, float sf) {
    if (sf == 0.0f) return 0;
    float r = rintf(w / sf);  // correctly rounded binary32 division, half-even rint
    r = fminf(fmaxf(r, -7.0f), 7.0f);
    return (int)r;
}

// One wavefront per (row, group): lane k holds w[n][64g + k].
// Returns the code of this lane; *scale_bits receives the group's fp16 scale.
__device__ __forceinline__ int quant_group_wave(float w, uint16_t* scale_bits) {
    float a = fabsf(w);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    const float s32 = a / 7.0f;
    const uint16_t s16 = f32_to_f16_bits(s32);
    const float sf = f16_bits_to_f32(s16);
    *scale_bits = s16;
    return quant_code(w, sf);
}

// Packed-layout position of nibble j (0..7) inside its dword.
__host__ __device__ __forceinline__ int packed_nibble_shift(int j) {
    return (j & 1) ? 16 + 4 * (j >> 1) : 4 * (j >> 1);
}

// Dword index (in the packed codes) holding row n, k = 8 * (k / 8) .. +8.
__host__ __device__ __forceinline__ int64_t packed_dword(int64_t n, int64_t k, int64_t G) {
    const int64_t t = n >> 6, g = k >> 6;
    const int nb = (int)((n >> 4) & 3), i = (int)(n & 15);
    const int s = (int)((k >> 5) & 1), kq = (int)((k >> 3) & 3);
    const int lane = kq * 16 + i, d = nb * 2 + s;
    return ((((t * G + g) * 2 + (d >> 2)) * 1024 + lane * 16) >> 2) + (d & 3);
}

// Index (in fp16 units) of the scale of row n, group g.
__host__ __device__ __forceinline__ int64_t packed_scale(int64_t n, int64_t g, int64_t G) {
    return (((n >> 6) * G + g) * 16 + (n & 15)) * 4 + ((n >> 4) & 3);
}

__global__ __launch_bounds__(256) void quantize_canonical_kernel(const float* __restrict__ w, int64_t N,
                                                                 int64_t K, uint8_t* __restrict__ codes,
                                                                 uint16_t* __restrict__ scales) {
    const int64_t G = K / 64;
    const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (n, g) index
    const int lane = threadIdx.x & 63;
    if (wid >= N * G) return;
    const int64_t n = wid / G, g = wid % G;
    const float v = w[n * K + g * 64 + lane];
    uint16_t sb;
    const int c = quant_group_wave(v, &sb);
    const uint32_t u = (uint32_t)(c + 8);
    const uint32_t hi = __shfl_down(u, 1, 64);
    if ((lane & 1) == 0) codes[n * (K / 2) + g * 32 + (lane >> 1)] = (uint8_t)(u | (hi << 4));
    if (lane == 0) scales[n * G + g] = sb;
}

__global__ __launch_bounds__(256) void quantize_packed_kernel(const float* __restrict__ w, int64_t N, int64_t K,
                                                              int64_t Npad, uint32_t* __restrict__ packed,
                                                              uint16_t* __restrict__ pscales) {
    const int64_t G = K / 64;
    const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (wid >= Npad * G) return;
    const int64_t n = wid / G, g = wid % G;
    int c = 0;
    uint16_t sb = 0;
    if (n < N) {
        const float v = w[n * K + g * 64 + lane];
        c = quant_group_wave(v, &sb);
    }
    // gather the 8 codes of this lane's dword into lane (lane & ~7)
    const uint32_t u = (uint32_t)(c + 8) << packed_nibble_shift(lane & 7);
    uint32_t word = u;
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) word |= __shfl_xor(word, off, 64);
    if ((lane & 7) == 0) packed[packed_dword(n, g * 64 + lane, G)] = word;
    if (lane == 0) pscales[packed_scale(n, g, G)] = sb;
}

// One thread per (padded row, group): canonical 32 bytes + scale -> packed.
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ codes,
                                                   const uint16_t* __restrict__ scales, int64_t N, int64_t K,
                                                   int64_t Npad, uint32_t* __restrict__ packed,
                                                   uint16_t* __restrict__ pscales) {
    const int64_t G = K / 64;
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= Npad * G) return;
    const int64_t n = id / G, g = id % G;
    const uint8_t* src = codes + n * (K / 2) + g * 32;
    for (int o = 0; o < 8; ++o) {          // the 8 runs of 8 k of the group
        uint32_t word = 0;
        for (int j = 0; j < 8; ++j) {
            const int k = o * 8 + j;       // k within the group
            uint32_t u = 8;
            if (n < N) {
                const uint8_t b = src[k >> 1];
                u = (k & 1) ? (b >> 4) : (b & 15u);
            }
            word |= u << packed_nibble_shift(j);
        }
        packed[packed_dword(n, g * 64 + o * 8, G)] = word;
    }
    pscales[packed_scale(n, g, G)] = (n < N) ? scales[n * G + g] : (uint16_t)0;
}

// W8: one u8 code u = c + 128 per element (row n, k at codes[n * K + k]).
// The high and low nibbles of u go to two planes, each in the W4 packed
// layout above; padding rows get u = 128 (code 0) and scale 0.
__global__ __launch_bounds__(256) void pack8_kernel(const uint8_t* __restrict__ codes,
                                                    const uint16_t* __restrict__ scales, int64_t N, int64_t K,
                                                    int64_t Npad, uint32_t* __restrict__ hi, uint32_t* __restrict__ lo,
                                                    uint16_t* __restrict__ pscales) {
    const int64_t G = K / 64;
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= Npad * G) return;
    const int64_t n = id / G, g = id % G;
    const uint8_t* src = codes + n * K + g * 64;
    for (int o = 0; o < 8; ++o) {
        uint32_t wh = 0, wl = 0;
        for (int j = 0; j < 8; ++j) {
            const uint32_t u = (n < N) ? src[o * 8 + j] : 128u;
            wh |= (u >> 4) << packed_nibble_shift(j);
            wl |= (u & 15u) << packed_nibble_shift(j);
        }
        const int64_t d = packed_dword(n, g * 64 + o * 8, G);
        hi[d] = wh;
        lo[d] = wl;
    }
    pscales[packed_scale(n, g, G)] = (n < N) ? scales[n * G + g] : (uint16_t)0;
}

// W6: one u8 code u = c + 32 per element.  The low 4 bits go to a plane in
// the W4 packed layout; the high 2 bits to a 2-bit plane with the same lane
// mapping: per tile and K-group 1 KiB, lane l = 16 kq + i owning 16 bytes,
// dword nb holding row 16 nb + i at k = 32 s + 8 kq + j in bits
// 8 s + 2 (j / 2) + 16 (j % 2).  Padding rows get u = 32 (code 0), scale 0.
__global__ __launch_bounds__(256) void pack6_kernel(const uint8_t* __restrict__ codes,
                                                    const uint16_t* __restrict__ scales, int64_t N, int64_t K,
                                                    int64_t Npad, uint32_t* __restrict__ hi, uint32_t* __restrict__ lo,
                                                    uint16_t* __restrict__ pscales) {
    const int64_t G = K / 64;
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= Npad * G) return;
    const int64_t n = id / G, g = id % G;
    const uint8_t* src = codes + n * K + g * 64;
    for (int o = 0; o < 8; ++o) {
        uint32_t wl = 0;
        for (int j = 0; j < 8; ++j) {
            const uint32_t u = (n < N) ? src[o * 8 + j] : 32u;
            wl |= (u & 15u) << packed_nibble_shift(j);
        }
        lo[packed_dword(n, g * 64 + o * 8, G)] = wl;
    }
    const int64_t t = n >> 6;
    const int i = (int)(n & 15), nb = (int)((n >> 4) & 3);
    for (int kq = 0; kq < 4; ++kq) {
        uint32_t wh = 0;
        for (int s = 0; s < 2; ++s)
            for (int j = 0; j < 8; ++j) {
                const uint32_t u = (n < N) ? src[32 * s + 8 * kq + j] : 32u;
                wh |= (u >> 4) << (8 * s + 2 * (j >> 1) + 16 * (j & 1));
            }
        hi[((t * G + g) * 64 + kq * 16 + i) * 4 + nb] = wh;
    }
    pscales[packed_scale(n, g, G)] = (n < N) ? scales[n * G + g] : (uint16_t)0;
}

// W5: one u8 code u = c + 16 per element.  The low 4 bits go to a plane in
// the W4 packed layout; the high bit to a 1-bit plane with the same lane
// mapping: per tile and K-group 512 bytes, lane l = 16 kq + i owning 8 bytes,
// dword d holding rows 16 nb + i of the two row blocks nb = 2 d, 2 d + 1, the
// bit of k = 32 s + 8 kq + j at 4 (2 (nb & 1) + s) + j / 2 + 16 (j % 2).  The
// thread of an even row block writes the dword of both of its blocks.
// Padding rows get u = 16 (code 0), scale 0.
__global__ __launch_bounds__(256) void pack5_kernel(const uint8_t* __restrict__ codes,
                                                    const uint16_t* __restrict__ scales, int64_t N, int64_t K,
                                                    int64_t Npad, uint32_t* __restrict__ hi, uint32_t* __restrict__ lo,
                                                    uint16_t* __restrict__ pscales) {
    const int64_t G = K / 64;
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= Npad * G) return;
    const int64_t n = id / G, g = id % G;
    const uint8_t* src = codes + n * K + g * 64;
    for (int o = 0; o < 8; ++o) {
        uint32_t wl = 0;
        for (int j = 0; j < 8; ++j) {
            const uint32_t u = (n < N) ? src[o * 8 + j] : 16u;
            wl |= (u & 15u) << packed_nibble_shift(j);
        }
        lo[packed_dword(n, g * 64 + o * 8, G)] = wl;
    }
    const int64_t t = n >> 6;
    const int i = (int)(n & 15), nb = (int)((n >> 4) & 3);
    if ((nb & 1) == 0) {
        for (int kq = 0; kq < 4; ++kq) {
            uint32_t wh = 0;
            for (int b = 0; b < 2; ++b) {
                const int64_t row = n + 16 * b;   // row blocks nb, nb + 1 of the same tile
                for (int s = 0; s < 2; ++s)
                    for (int j = 0; j < 8; ++j) {
                        const uint32_t u = (row < N) ? codes[row * K + g * 64 + 32 * s + 8 * kq + j] : 16u;
                        wh |= ((u >> 4) & 1u) << (4 * (2 * b + s) + (j >> 1) + 16 * (j & 1));
                    }
            }
            hi[((t * G + g) * 64 + kq * 16 + i) * 2 + (nb >> 1)] = wh;
        }
    }
    pscales[packed_scale(n, g, G)] = (n < N) ? scales[n * G + g] : (uint16_t)0;
}

// The 2-bit plane (the layout of W6's high plane, W3's low plane and W2's
// only plane) for row n and K-group g: field (u >> shift) & 3 of each code,
// or, with sign_mag, the sign-magnitude form of c = u - 1 in {-1, 0, 1} (bit 0
// = (c != 0), bit 1 = (c < 0)); padding rows take u = pad_u.  One thread per
// (n, g) writes its row's four dwords (one per kq).
__device__ __forceinline__ void write_plane2(const uint8_t* __restrict__ codes, int64_t N, int64_t K, int64_t n,
                                             int64_t g, int shift, uint32_t pad_u, bool sign_mag,
                                             uint32_t* __restrict__ plane) {
    const int64_t G = K / 64, t = n >> 6;
    const int i = (int)(n & 15), nb = (int)((n >> 4) & 3);
    const uint8_t* src = codes + n * K + g * 64;
    for (int kq = 0; kq < 4; ++kq) {
        uint32_t wd = 0;
        for (int s = 0; s < 2; ++s)
            for (int j = 0; j < 8; ++j) {
                const uint32_t u = (n < N) ? src[32 * s + 8 * kq + j] : pad_u;
                const uint32_t f = sign_mag ? (uint32_t)(u != 1u) | ((uint32_t)(u == 0u) << 1) : (u >> shift) & 3u;
                wd |= f << (8 * s + 2 * (j >> 1) + 16 * (j & 1));
            }
        plane[((t * G + g) * 64 + kq * 16 + i) * 4 + nb] = wd;
    }
}

// The 1-bit plane (the layout of W5's and W3's high planes) for row n and
// K-group g: bit (u >> shift) & 1 of each code.  The thread of an even row
// block writes the dwords of its block and the next (rows n and n + 16).
__device__ __forceinline__ void write_plane1(const uint8_t* __restrict__ codes, int64_t N, int64_t K, int64_t n,
                                             int64_t g, int shift, uint32_t pad_u, uint32_t* __restrict__ plane) {
    const int64_t G = K / 64, t = n >> 6;
    const int i = (int)(n & 15), nb = (int)((n >> 4) & 3);
    if (nb & 1) return;
    for (int kq = 0; kq < 4; ++kq) {
        uint32_t wd = 0;
        for (int b = 0; b < 2; ++b) {
            const int64_t row = n + 16 * b;
            for (int s = 0; s < 2; ++s)
                for (int j = 0; j < 8; ++j) {
                    const uint32_t u = (row < N) ? codes[row * K + g * 64 + 32 * s + 8 * kq + j] : pad_u;
                    wd |= ((u >> shift) & 1u) << (4 * (2 * b + s) + (j >> 1) + 16 * (j & 1));
                }
        }
        plane[((t * G + g) * 64 + kq * 16 + i) * 2 + (nb >> 1)] = wd;
    }
}

// W3: u = c + 4 = 4 hi + lo; lo (2 bits) to a 2-bit plane, hi (1 bit) to a
// 1-bit plane.  W2: c = u - 1 in sign-magnitude to one 2-bit plane.  Padding
// rows get code 0.
__global__ __launch_bounds__(256) void pack3_kernel(const uint8_t* __restrict__ codes,
                                                    const uint16_t* __restrict__ scales, int64_t N, int64_t K,
                                                    int64_t Npad, uint32_t* __restrict__ hi, uint32_t* __restrict__ lo,
                                                    uint16_t* __restrict__ pscales) {
    const int64_t G = K / 64;
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= Npad * G) return;
    const int64_t n = id / G, g = id % G;
    write_plane2(codes, N, K, n, g, 0, 4u, false, lo);
    write_plane1(codes, N, K, n, g, 2, 4u, hi);
    pscales[packed_scale(n, g, G)] = (n < N) ? scales[n * G + g] : (uint16_t)0;
}

__global__ __launch_bounds__(256) void pack2_kernel(const uint8_t* __restrict__ codes,
                                                    const uint16_t* __restrict__ scales, int64_t N, int64_t K,
                                                    int64_t Npad, uint32_t* __restrict__ plane,
                                                    uint16_t* __restrict__ pscales) {
    const int64_t G = K / 64;
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= Npad * G) return;
    const int64_t n = id / G, g = id % G;
    write_plane2(codes, N, K, n, g, 0, 1u, true, plane);
    pscales[packed_scale(n, g, G)] = (n < N) ? scales[n * G + g] : (uint16_t)0;
}

// 16-bit float weights (bf16 or fp16 bit patterns, [N][K] row-major) to the
// operand-tiled layout: per 64-row tile and K-group 8 KiB, word 2 nb + s of
// lane l = 16 kq + i (16-byte index ((t G + g) * 8 + 2 nb + s) * 64 + l)
// holding row 16 nb + i at k = 32 s + 8 kq + 0..7.  One thread per (n, g)
// writes its row's eight 16-byte words; padding rows are zero.
__global__ __launch_bounds__(256) void pack16_kernel(const uint16_t* __restrict__ w, int64_t N, int64_t K,
                                                     int64_t Npad, uint4* __restrict__ out) {
    const int64_t G = K / 64;
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= Npad * G) return;
    const int64_t n = id / G, g = id % G, t = n >> 6;
    const int i = (int)(n & 15), nb = (int)((n >> 4) & 3);
    for (int s = 0; s < 2; ++s)
        for (int kq = 0; kq < 4; ++kq) {
            uint32_t d[4];
            for (int p = 0; p < 4; ++p) {
                const int64_t k = g * 64 + 32 * s + 8 * kq + 2 * p;
                const uint32_t lo = (n < N) ? w[n * K + k] : 0u, hi = (n < N) ? w[n * K + k + 1] : 0u;
                d[p] = lo | (hi << 16);
            }
            out[((t * G + g) * 8 + 2 * nb + s) * 64 + 16 * kq + i] = make_uint4(d[0], d[1], d[2], d[3]);
        }
}

__global__ __launch_bounds__(256) void unpack_kernel(const uint32_t* __restrict__ packed,
                                                     const uint16_t* __restrict__ pscales, int64_t N, int64_t K,
                                                     uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
    const int64_t G = K / 64;
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= N * G) return;
    const int64_t n = id / G, g = id % G;
    uint8_t* dst = codes + n * (K / 2) + g * 32;
    for (int o = 0; o < 8; ++o) {
        const uint32_t word = packed[packed_dword(n, g * 64 + o * 8, G)];
        for (int jp = 0; jp < 4; ++jp) {
            const uint32_t lo = (word >> packed_nibble_shift(2 * jp)) & 15u;
            const uint32_t hi = (word >> packed_nibble_shift(2 * jp + 1)) & 15u;
            dst[o * 4 + jp] = (uint8_t)(lo | (hi << 4));
        }
    }
    scales[n * G + g] = pscales[packed_scale(n, g, G)];
}

static int check_shape(int64_t N, int64_t K) {
    VW4_REQUIRE(N >= 1 && N <= (int64_t)1 << 31, VW4_EINVAL, "N=%lld out of range", (long long)N);
    VW4_REQUIRE(K >= 64 && K % 64 == 0 && K <= 65536, VW4_EINVAL, "K=%lld must be a multiple of 64 in [64, 65536]",
                (long long)K);
    return VW4_OK;
}

static int64_t pad64(int64_t N) { return (N + 63) / 64 * 64; }

// Host binary32 -> binary16 (round to nearest even) from the bit layout.
static uint16_t host_f32_to_f16(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    const uint32_t sign = (x >> 16) & 0x8000u;
    const uint32_t ax = x & 0x7fffffffu;
    if (ax > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);
    if (ax >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);  // >= 65520 rounds to inf
    if (ax < 0x38800000u) {                                     // below 2^-14: subnormal result
        if (ax < 0x33000000u) return (uint16_t)sign;            // below 2^-25: rounds to 0
        const uint32_t e = ax >> 23;                            // 102..112
        const uint32_t m = (ax & 0x7fffffu) | 0x800000u;
        const uint32_t shift = 126u - e;                        // 14..24
        uint32_t r = m >> shift;
        const uint32_t rem = m & ((1u << shift) - 1u), halfway = 1u << (shift - 1u);
        if (rem > halfway || (rem == halfway && (r & 1u))) ++r;
        return (uint16_t)(sign | r);
    }
    uint32_t r = (ax - 0x38000000u) >> 13;                       // rebias 127 -> 15
    const uint32_t rem = ax & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (r & 1u))) ++r;
    return (uint16_t)(sign | r);
}

static float host_f16_to_f32(uint16_t h) {
    const uint32_t s = (uint32_t)(h & 0x8000u) << 16, e = (h >> 10) & 31u, m = h & 1023u;
    float v;
    if (e == 0) v = ldexpf((float)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexpf((float)(1024u + m), (int)e - 25);
    uint32_t b;
    memcpy(&b, &v, 4);
    b |= s;
    memcpy(&v, &b, 4);
    return v;
}

}  // namespace vw4

using namespace vw4;

extern "C" {

const char* vw4_version(void) { return "vw4 0.1.0 (gfx950)"; }

const char* vw4_last_error(void) { return g_err; }

int vw4_w4_quantize_host(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales) {
    int rc = check_shape(N, K);
    if (rc) return rc;
    VW4_REQUIRE(w && codes && scales, VW4_EINVAL, "null pointer");
    const int64_t G = K / 64;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float* wg = w + n * K + g * 64;
            float a = 0.0f;
            for (int k = 0; k < 64; ++k) a = fmaxf(a, fabsf(wg[k]));
            const uint16_t s16 = host_f32_to_f16(a / 7.0f);
            const float sf = host_f16_to_f32(s16);
            scales[n * G + g] = s16;
            uint8_t* dst = codes + n * (K / 2) + g * 32;
            for (int k = 0; k < 64; k += 2) {
                int c0 = 0, c1 = 0;
                if (sf != 0.0f) {
                    c0 = (int)fminf(fmaxf(rintf(wg[k] / sf), -7.0f), 7.0f);
                    c1 = (int)fminf(fmaxf(rintf(wg[k + 1] / sf), -7.0f), 7.0f);
                }
                dst[k >> 1] = (uint8_t)((c0 + 8) | ((c1 + 8) << 4));
            }
        }
    }
    return VW4_OK;
}

int vw4_w8_quantize_host(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales) {
    int rc = check_shape(N, K);
    if (rc) return rc;
    VW4_REQUIRE(w && codes && scales, VW4_EINVAL, "null pointer");
    const int64_t G = K / 64;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float* wg = w + n * K + g * 64;
            float a = 0.0f;
            for (int k = 0; k < 64; ++k) a = fmaxf(a, fabsf(wg[k]));
            const uint16_t s16 = host_f32_to_f16(a / 127.0f);
            const float sf = host_f16_to_f32(s16);
            scales[n * G + g] = s16;
            for (int k = 0; k < 64; ++k) {
                const int c = sf != 0.0f ? (int)fminf(fmaxf(rintf(wg[k] / sf), -127.0f), 127.0f) : 0;
                codes[n * K + g * 64 + k] = (uint8_t)(c + 128);
            }
        }
    }
    return VW4_OK;
}

int vw4_w8_pack(const uint8_t* codes_dev, const uint16_t* scales_dev, int64_t N, int64_t K, uint8_t* hi_dev,
                uint8_t* lo_dev, uint16_t* packed_scales_dev, void* stream) {
    int rc = check_shape(N, K);
    if (rc) return rc;
    VW4_REQUIRE(codes_dev && scales_dev && hi_dev && lo_dev && packed_scales_dev, VW4_EINVAL, "null pointer");
    VW4_REQUIRE(aligned(hi_dev, 16) && aligned(lo_dev, 16), VW4_EINVAL, "packed planes must be 16-byte aligned");
    const int64_t Np = pad64(N), total = Np * (K / 64);
    hipLaunchKernelGGL(pack8_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                       codes_dev, scales_dev, N, K, Np, (uint32_t*)hi_dev, (uint32_t*)lo_dev, packed_scales_dev);
    return check_launch("vw4_w8_pack");
}

int vw4_w6_quantize_host(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales) {
    int rc = check_shape(N, K);
    if (rc) return rc;
    VW4_REQUIRE(w && codes && scales, VW4_EINVAL, "null pointer");
    const int64_t G = K / 64;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float* wg = w + n * K + g * 64;
            float a = 0.0f;
            for (int k = 0; k < 64; ++k) a = fmaxf(a, fabsf(wg[k]));
            const uint16_t s16 = host_f32_to_f16(a / 31.0f);
            const float sf = host_f16_to_f32(s16);
            scales[n * G + g] = s16;
            for (int k = 0; k < 64; ++k) {
                const int c = sf != 0.0f ? (int)fminf(fmaxf(rintf(wg[k] / sf), -31.0f), 31.0f) : 0;
                codes[n * K + g * 64 + k] = (uint8_t)(c + 32);
            }
        }
    }
    return VW4_OK;
}

int vw4_w5_quantize_host(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales) {
    int rc = check_shape(N, K);
    if (rc) return rc;
    VW4_REQUIRE(w && codes && scales, VW4_EINVAL, "null pointer");
    const int64_t G = K / 64;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float* wg = w + n * K + g * 64;
            float a = 0.0f;
            for (int k = 0; k < 64; ++k) a = fmaxf(a, fabsf(wg[k]));
            const uint16_t s16 = host_f32_to_f16(a / 15.0f);
            const float sf = host_f16_to_f32(s16);
            scales[n * G + g] = s16;
            for (int k = 0; k < 64; ++k) {
                const int c = sf != 0.0f ? (int)fminf(fmaxf(rintf(wg[k] / sf), -15.0f), 15.0f) : 0;
                codes[n * K + g * 64 + k] = (uint8_t)(c + 16);
            }
        }
    }
    return VW4_OK;
}

size_t vw4_w5_hi_plane_bytes(int64_t N, int64_t K) {
    if (check_shape(N, K)) return 0;
    return (size_t)(pad64(N) * (K / 8));
}

int vw4_w5_pack(const uint8_t* codes_dev, const uint16_t* scales_dev, int64_t N, int64_t K, uint8_t* hi_dev,
                uint8_t* lo_dev, uint16_t* packed_scales_dev, void* stream) {
    int rc = check_shape(N, K);
    if (rc) return rc;
    VW4_REQUIRE(codes_dev && scales_dev && hi_dev && lo_dev && packed_scales_dev, VW4_EINVAL, "null pointer");
    VW4_REQUIRE(aligned(hi_dev, 16) && aligned(lo_dev, 16), VW4_EINVAL, "packed planes must be 16-byte aligned");
    const int64_t Np = pad64(N), total = Np * (K / 64);
    hipLaunchKernelGGL(pack5_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                       codes_dev, scales_dev, N, K, Np, (uint32_t*)hi_dev, (uint32_t*)lo_dev, packed_scales_dev);
    return check_launch("vw4_w5_pack");
}

// The b-bit symmetric recipe on the host: scale = fp16(absmax / qmax), codes
// against the rounded scale (binary32 division, half-even), clamped to
// [-qmax, qmax], stored as c + bias.
static int quantize_sym_host(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales, float qmax,
                             int bias) {
    int rc = check_shape(N, K);
    if (rc) return rc;
    VW4_REQUIRE(w && codes && scales, VW4_EINVAL, "null pointer");
    const int64_t G = K / 64;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float* wg = w + n * K + g * 64;
            float a = 0.0f;
            for (int k = 0; k < 64; ++k) a = fmaxf(a, fabsf(wg[k]));
            const uint16_t s16 = host_f32_to_f16(a / qmax);
            const float sf = host_f16_to_f32(s16);
            scales[n * G + g] = s16;
            for (int k = 0; k < 64; ++k) {
                const int c = sf != 0.0f ? (int)fminf(fmaxf(rintf(wg[k] / sf), -qmax), qmax) : 0;
                codes[n * K + g * 64 + k] = (uint8_t)(c + bias);
            }
        }
    }
    return VW4_OK;
}

int vw4_w3_quantize_host(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales) {
    return quantize_sym_host(w, N, K, codes, scales, 3.0f, 4);
}

int vw4_w2_quantize_host(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales) {
    return quantize_sym_host(w, N, K, codes, scales, 1.0f, 1);
}

size_t vw4_w3_hi_plane_bytes(int64_t N, int64_t K) {
    if (check_shape(N, K)) return 0;
    return (size_t)(pad64(N) * (K / 8));
}

size_t vw4_w3_lo_plane_bytes(int64_t N, int64_t K) {
    if (check_shape(N, K)) return 0;
    return (size_t)(pad64(N) * (K / 4));
}

size_t vw4_w2_packed_bytes(int64_t N, int64_t K) {
    if (check_shape(N, K)) return 0;
    return (size_t)(pad64(N) * (K / 4));
}

int vw4_w3_pack(const uint8_t* codes_dev, const uint16_t* scales_dev, int64_t N, int64_t K, uint8_t* hi_dev,
                uint8_t* lo_dev, uint16_t* packed_scales_dev, void* stream) {
    int rc = check_shape(N, K);
    if (rc) return rc;
    VW4_REQUIRE(codes_dev && scales_dev && hi_dev && lo_dev && packed_scales_dev, VW4_EINVAL, "null pointer");
    VW4_REQUIRE(aligned(hi_dev, 16) && aligned(lo_dev, 16), VW4_EINVAL, "packed planes must be 16-byte aligned");
    const int64_t Np = pad64(N), total = Np * (K / 64);
    hipLaunchKernelGGL(pack3_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                       codes_dev, scales_dev, N, K, Np, (uint32_t*)hi_dev, (uint32_t*)lo_dev, packed_scales_dev);
    return check_launch("vw4_w3_pack");
}

int vw4_w2_pack(const uint8_t* codes_dev, const uint16_t* scales_dev, int64_t N, int64_t K, uint8_t* packed_dev,
                uint16_t* packed_scales_dev, void* stream) {
    int rc = check_shape(N, K);
    if (rc) return rc;
    VW4_REQUIRE(codes_dev && scales_dev && packed_dev && packed_scales_dev, VW4_EINVAL, "null pointer");
    VW4_REQUIRE(aligned(packed_dev, 16), VW4_EINVAL, "packed plane must be 16-byte aligned");
    const int64_t Np = pad64(N), total = Np * (K / 64);
    hipLaunchKernelGGL(pack2_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                       codes_dev, scales_dev, N, K, Np, (uint32_t*)packed_dev, packed_scales_dev);
    return check_launch("vw4_w2_pack");
}

size_t vw4_w16_packed_bytes(int64_t N, int64_t K) {
    if (check_shape(N, K)) return 0;
    return (size_t)(pad64(N) * K * 2);
}

int vw4_w16_pack(const uint16_t* w_dev, int64_t N, int64_t K, uint8_t* packed_dev, void* stream) {
    int rc = check_shape(N, K);
    if (rc) return rc;
    VW4_REQUIRE(w_dev && packed_dev, VW4_EINVAL, "null pointer");
    VW4_REQUIRE(aligned(packed_dev, 16), VW4_EINVAL, "packed weights must be 16-byte aligned");
    const int64_t Np = pad64(N), total = Np * (K / 64);
    hipLaunchKernelGGL(pack16_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, (hipStream_t)stream, w_dev,
                       N, K, Np, (uint4*)packed_dev);
    return check_launch("vw4_w16_pack");
}

size_t vw4_w6_hi_plane_bytes(int64_t N, int64_t K) {
    if (check_shape(N, K)) return 0;
    return (size_t)(pad64(N) * (K / 4));
}

int vw4_w6_pack(const uint8_t* codes_dev, const uint16_t* scales_dev, int64_t N, int64_t K, uint8_t* hi_dev,
                uint8_t* lo_dev, uint16_t* packed_scales_dev, void* stream) {
    int rc = check_shape(N, K);
    if (rc) return rc;
    VW4_REQUIRE(codes_dev && scales_dev && hi_dev && lo_dev && packed_scales_dev, VW4_EINVAL, "null pointer");
    VW4_REQUIRE(aligned(hi_dev, 16) && aligned(lo_dev, 16), VW4_EINVAL, "packed planes must be 16-byte aligned");
    const int64_t Np = pad64(N), total = Np * (K / 64);
    hipLaunchKernelGGL(pack6_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                       codes_dev, scales_dev, N, K, Np, (uint32_t*)hi_dev, (uint32_t*)lo_dev, packed_scales_dev);
    return check_launch("vw4_w6_pack");
}

int vw4_w4_quantize(const float* w_dev, int64_t N, int64_t K, uint8_t* codes_dev, uint16_t* scales_dev,
                    void* stream) {
    int rc = check_shape(N, K);
    if (rc) return rc;
    VW4_REQUIRE(w_dev && codes_dev && scales_dev, VW4_EINVAL, "null pointer");
    const int64_t waves = N * (K / 64);
    hipLaunchKernelGGL(quantize_canonical_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                       (hipStream_t)stream, w_dev, N, K, codes_dev, scales_dev);
    return check_launch("vw4_w4_quantize");
}

size_t vw4_w4_packed_bytes(int64_t N, int64_t K, size_t* scale_bytes) {
    if (check_shape(N, K)) return 0;
    const int64_t Np = pad64(N);
    if (scale_bytes) *scale_bytes = (size_t)(Np * (K / 64) * 2);
    return (size_t)(Np * (K / 2));
}

int vw4_w4_pack(const uint8_t* codes_dev, const uint16_t* scales_dev, int64_t N, int64_t K, uint8_t* packed_dev,
                uint16_t* packed_scales_dev, void* stream) {
    int rc = check_shape(N, K);
    if (rc) return rc;
    VW4_REQUIRE(codes_dev && scales_dev && packed_dev && packed_scales_dev, VW4_EINVAL, "null pointer");
    VW4_REQUIRE(aligned(packed_dev, 16), VW4_EINVAL, "packed codes must be 16-byte aligned");
    const int64_t Np = pad64(N), total = Np * (K / 64);
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                       codes_dev, scales_dev, N, K, Np, (uint32_t*)packed_dev, packed_scales_dev);
    return check_launch("vw4_w4_pack");
}

int vw4_w4_unpack(const uint8_t* packed_dev, const uint16_t* packed_scales_dev, int64_t N, int64_t K,
                  uint8_t* codes_dev, uint16_t* scales_dev, void* stream) {
    int rc = check_shape(N, K);
    if (rc) return rc;
    VW4_REQUIRE(codes_dev && scales_dev && packed_dev && packed_scales_dev, VW4_EINVAL, "null pointer");
    VW4_REQUIRE(aligned(packed_dev, 16), VW4_EINVAL, "packed codes must be 16-byte aligned");
    const int64_t total = N * (K / 64);
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                       (const uint32_t*)packed_dev, packed_scales_dev, N, K, codes_dev, scales_dev);
    return check_launch("vw4_w4_unpack");
}

int vw4_w4_quantize_packed(const float* w_dev, int64_t N, int64_t K, uint8_t* packed_dev,
                           uint16_t* packed_scales_dev, void* stream) {
    int rc = check_shape(N, K);
    if (rc) return rc;
    VW4_REQUIRE(w_dev && packed_dev && packed_scales_dev, VW4_EINVAL, "null pointer");
    VW4_REQUIRE(aligned(packed_dev, 16), VW4_EINVAL, "packed codes must be 16-byte aligned");
    const int64_t Np = pad64(N), waves = Np * (K / 64);
    hipLaunchKernelGGL(quantize_packed_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                       (hipStream_t)stream, w_dev, N, K, Np, (uint32_t*)packed_dev, packed_scales_dev);
    return check_launch("vw4_w4_quantize_packed");
}

}  // extern "C"
