// w6_gemm.hip — the skinny GEMM on W6 weights (M = 1..8): a third weight
// format for the verify rows (gist.science, "BaseRT: …", section "メソドロジー",
// lists the quantisation formats its GEMV reads, Q2 ... Q8).
//
// y[m][n] = sum_g scale[n][g] * sum_{k in g} x[m][k] * c[n][k],  c in [-31, 31]
//
// The code u = c + 32 is split into a 2-bit high part and a 4-bit low part.
// The low plane is stored in the W4 packed layout (w4_format.hip); the high
// plane in a 2-bit layout with the same lane mapping: per tile and K-group,
// lane l owns 16 bytes, dword nb holding row 16 nb + i at k = 32 s + 8 kq + j
// (s = 0, 1; j = 0..7) in bits 8 s + 2 (j / 2) + 16 (j % 2), so
// ((dword >> (8 s + 2 p)) & 0x00030003) | 0x43004300 is the bf16 pair
// 128 + hi of elements (2p, 2p + 1).  With D_hi = sum x (128 + hi) and
// D_lo = sum x (128 + lo):  sum x c = 16 D_hi + D_lo - 2208 sum x; the chain
// of the high plane starts from x . (-138), so 16 (D_hi - 138 sum x) + D_lo
// is the group's sum.
// Products are exact in fp32 (bf16 x 8-bit integer), sums are fp32 in an
// order that depends only on (N, K): row m of an M-row call equals the
// one-row call bit for bit.
#include "common.h"

namespace vw4 {

namespace {

constexpr int W6_MAX_M = 8;
constexpr int W6_PF = 4;                       // groups in flight per lane
constexpr uint32_t NEG138_PAIR = 0xC30AC30Au;  // two bf16 -138.0
typedef uint32_t w6u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((ext_vector_type(8))) __bf16 w6bf16x8;
typedef __attribute__((ext_vector_type(4))) float w6f32x4;

__device__ __forceinline__ uint32_t w6_and_or(uint32_t v, uint32_t mask_s, uint32_t magic_v) {
    return __builtin_amdgcn_bitop3_b32(v, mask_s, magic_v, 0xEA);   // (v & mask) | magic
}

__device__ __forceinline__ w6bf16x8 w6_dequant8(uint32_t w, uint32_t kmask, uint32_t magic_v) {
    w6u32x4 r;
    r.x = w6_and_or(w, kmask, magic_v);
    r.y = w6_and_or(w >> 4, kmask, magic_v);
    r.z = w6_and_or(w >> 8, kmask, magic_v);
    r.w = w6_and_or(w >> 12, kmask, magic_v);
    return __builtin_bit_cast(w6bf16x8, r);
}

// 8 two-bit fields (k half s of one row block) -> the 8 bf16 values 128 + hi.
__device__ __forceinline__ w6bf16x8 w6_dequant8_2(uint32_t w, int s, uint32_t magic_v) {
    const uint32_t v = w >> (8 * s);
    w6u32x4 r;
    r.x = w6_and_or(v, 0x00030003u, magic_v);
    r.y = w6_and_or(v >> 2, 0x00030003u, magic_v);
    r.z = w6_and_or(v >> 4, 0x00030003u, magic_v);
    r.w = w6_and_or(v >> 6, 0x00030003u, magic_v);
    return __builtin_bit_cast(w6bf16x8, r);
}

__device__ __forceinline__ w6f32x4 w6_mfma(w6bf16x8 a, w6bf16x8 b, w6f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One K-group of one tile.  h: the lane's 16-byte load of the 2-bit high plane
// (dword nb = row block nb); la / lb: its two 16-byte loads of the low plane
// (row blocks 0, 1 and 2, 3); xa / xb: its activations for k halves 0 / 1;
// sc: its four row scales (fp16 pairs).
__device__ __forceinline__ void w6_group(w6u32x4 h, w6u32x4 la, w6u32x4 lb, w6u32x4 xa, w6u32x4 xb,
                                         uint2 sc, uint32_t kmask, uint32_t magic_v, w6f32x4 (&acc)[4]) {
    const w6bf16x8 a0 = __builtin_bit_cast(w6bf16x8, xa), a1 = __builtin_bit_cast(w6bf16x8, xb);
    const w6u32x4 nq = {NEG138_PAIR, NEG138_PAIR, NEG138_PAIR, NEG138_PAIR};
    const w6bf16x8 neg = __builtin_bit_cast(w6bf16x8, nq);
    const w6f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const w6f32x4 off = w6_mfma(a1, neg, w6_mfma(a0, neg, zero));
    const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
    const uint32_t lw[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
    const float f[4] = {f16_bits_to_f32((uint16_t)(sc.x & 0xffffu)), f16_bits_to_f32((uint16_t)(sc.x >> 16)),
                        f16_bits_to_f32((uint16_t)(sc.y & 0xffffu)), f16_bits_to_f32((uint16_t)(sc.y >> 16))};
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const w6f32x4 dh = w6_mfma(a1, w6_dequant8_2(hw[nb], 1, magic_v),
                                   w6_mfma(a0, w6_dequant8_2(hw[nb], 0, magic_v), off));
        const w6f32x4 dl = w6_mfma(a1, w6_dequant8(lw[2 * nb + 1], kmask, magic_v),
                                   w6_mfma(a0, w6_dequant8(lw[2 * nb], kmask, magic_v), zero));
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[nb][r] = fmaf(f[nb], fmaf(16.0f, dh[r], dl[r]), acc[nb][r]);
    }
}

// grid (ntiles, S_grid), one wavefront each: tile t, K-groups g0 .. g1 of
// slice s.  S_grid == 1 writes y; otherwise fp32 partials part[s][m][Npad].
__global__ __launch_bounds__(64) void w6_gemm_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                     const w6u32x4* __restrict__ whi,
                                                     const w6u32x4* __restrict__ wlo,
                                                     const uint16_t* __restrict__ spk, void* __restrict__ y,
                                                     int64_t ldy, int ydt, int M, int N, int G, int S_grid,
                                                     float* __restrict__ part, int64_t Npad, int to_part) {
    const int lane = threadIdx.x, kq = lane >> 4, i = lane & 15;
    const int t = blockIdx.x, s_idx = blockIdx.y;
    const int g0 = s_idx * G / S_grid, g1 = (s_idx + 1) * G / S_grid;
    const uint32_t kmask = 0x000F000Fu;
    const uint32_t magic_v = 0x43004300u;
    const int xr = i < M ? i : M - 1;            // A rows i >= M feed outputs that are never stored
    const w6u32x4* hbase = whi + (int64_t)t * G * 64 + lane;
    const w6u32x4* lbase = wlo + (int64_t)t * G * 128 + lane;
    const uint2* sbase = (const uint2*)spk + (int64_t)t * G * 16 + i;
    const w6u32x4* xbase = (const w6u32x4*)(x + (int64_t)xr * ldx) + kq;
    w6f32x4 acc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] = w6f32x4{0.f, 0.f, 0.f, 0.f};
    const int glast = g1 > g0 ? g1 - 1 : g0;
    w6u32x4 bh0[W6_PF], bl0[W6_PF], bl1[W6_PF], bx0[W6_PF], bx1[W6_PF];
    uint2 bs[W6_PF];
    auto issue = [&](int j, int gi) {
        bh0[j] = __builtin_nontemporal_load(hbase + (int64_t)gi * 64);
        bl0[j] = __builtin_nontemporal_load(lbase + (int64_t)gi * 128);
        bl1[j] = __builtin_nontemporal_load(lbase + (int64_t)gi * 128 + 64);
        bx0[j] = xbase[(int64_t)gi * 8];
        bx1[j] = xbase[(int64_t)gi * 8 + 4];
        bs[j] = sbase[(int64_t)gi * 16];
    };
    // g0 < G always (S_grid <= G): every address below is valid
#pragma unroll
    for (int j = 0; j < W6_PF; ++j) issue(j, min(g0 + j, glast));
    __builtin_amdgcn_sched_barrier(0);
    if (g0 < g1) {
        int g = g0;
        for (; g + W6_PF <= g1; g += W6_PF) {
#pragma unroll
            for (int j = 0; j < W6_PF; ++j) {
                w6_group(bh0[j], bl0[j], bl1[j], bx0[j], bx1[j], bs[j], kmask, magic_v, acc);
                __builtin_amdgcn_sched_barrier(0);
                issue(j, min(g + j + W6_PF, glast));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int j = 0; j < W6_PF - 1; ++j)
            if (g + j < g1) w6_group(bh0[j], bl0[j], bl1[j], bx0[j], bx1[j], bs[j], kmask, magic_v, acc);
    }
    // lane (kq, i) holds rows m = 4 kq + r of columns n = 64 t + 16 nb + i
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = 4 * kq + r;
        if (m >= M) break;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int n = t * 64 + nb * 16 + i;
            if (S_grid == 1 && !to_part) {
                if (n < N) {
                    if (ydt == VW4_F32) ((float*)y)[m * ldy + n] = acc[nb][r];
                    else ((uint16_t*)y)[m * ldy + n] = f32_to_bf16(acc[nb][r]);
                }
            } else {
                part[((int64_t)s_idx * M + m) * Npad + n] = acc[nb][r];
            }
        }
    }
}

// Sum of the S_grid partials in slice order.  grid (ntiles, M), 64 threads.
__global__ __launch_bounds__(64) void w6_reduce_kernel(const float* __restrict__ part, int S_grid, int M, int64_t Npad,
                                                       int N, void* __restrict__ y, int64_t ldy, int ydt) {
    const int n = blockIdx.x * 64 + threadIdx.x, m = blockIdx.y;
    if (n >= N) return;
    float s = 0.0f;
    for (int b = 0; b < S_grid; ++b) s += part[((int64_t)b * M + m) * Npad + n];
    if (ydt == VW4_F32) ((float*)y)[m * ldy + n] = s;
    else ((uint16_t*)y)[m * ldy + n] = f32_to_bf16(s);
}

struct W6Plan {
    int ntiles, G, S_grid;
    int64_t Npad;
    size_t ws_bytes;
};

// About two wavefronts per SIMD over the chip, at least four K-groups each,
// at most 8 partial slices.
W6Plan w6_plan(int M, int N, int K) {
    W6Plan p;
    p.G = K / 64;
    p.ntiles = (N + 63) / 64;
    p.Npad = (int64_t)p.ntiles * 64;
    const int want = 8 * device_cus();
    int S = (want + p.ntiles - 1) / p.ntiles;
    if (S > 8) S = 8;
    if (S > p.G / 4) S = p.G / 4;
    p.S_grid = S < 1 ? 1 : S;
    p.ws_bytes = p.S_grid > 1 ? ((size_t)p.S_grid * M * p.Npad * 4 + 255) / 256 * 256 : 0;
    return p;
}

}  // namespace

}  // namespace vw4

using namespace vw4;

extern "C" {

size_t vw4_w6_workspace_bytes(int32_t M, int32_t N, int32_t K) {
    if (M < 1 || M > W6_MAX_M || N < 1 || K < 64 || K % 64 || K > 65536) return 0;
    return w6_plan(M, N, K).ws_bytes;
}

int w6_skinny_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                   const uint16_t* scales_packed, void* y, int64_t ldy, int32_t y_dtype, int32_t M, int32_t N,
                   int32_t K, void* ws, size_t ws_bytes, void* stream) {
    VW4_REQUIRE(M >= 1 && M <= W6_MAX_M, VW4_EINVAL, "w6_skinny_gemm: M=%d must be in [1, 8]", M);
    VW4_REQUIRE(N >= 1, VW4_EINVAL, "w6_skinny_gemm: N=%d must be >= 1", N);
    VW4_REQUIRE(K >= 64 && K % 64 == 0 && K <= 65536, VW4_EINVAL,
                "w6_skinny_gemm: K=%d must be a multiple of 64 in [64, 65536]", K);
    VW4_REQUIRE(x && w_hi && w_lo && scales_packed && y, VW4_EINVAL, "w6_skinny_gemm: null pointer");
    VW4_REQUIRE(ldx >= K && ldx % 8 == 0 && aligned(x, 16), VW4_EINVAL,
                "w6_skinny_gemm: x needs ldx >= K, ldx %% 8 == 0 and 16-byte alignment");
    VW4_REQUIRE(aligned(w_hi, 16) && aligned(w_lo, 16) && aligned(scales_packed, 8), VW4_EINVAL,
                "w6_skinny_gemm: packed planes must be 16-byte and packed scales 8-byte aligned");
    VW4_REQUIRE(ldy >= N, VW4_EINVAL, "w6_skinny_gemm: ldy=%lld < N=%d", (long long)ldy, N);
    VW4_REQUIRE(y_dtype == VW4_F32 || y_dtype == VW4_BF16, VW4_EINVAL,
                "w6_skinny_gemm: y_dtype must be VW4_F32 or VW4_BF16");
    VW4_REQUIRE(aligned(y, y_dtype == VW4_F32 ? 4 : 2), VW4_EINVAL, "w6_skinny_gemm: y misaligned");
    const W6Plan p = w6_plan(M, N, K);
    float* part = nullptr;
    if (p.ws_bytes) {
        VW4_REQUIRE(ws && ws_bytes >= p.ws_bytes && aligned(ws, 256), VW4_EWORKSPACE,
                    "w6_skinny_gemm: needs a 256-byte aligned workspace of %zu bytes", p.ws_bytes);
        part = (float*)ws;
    }
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(w6_gemm_kernel, dim3(p.ntiles, p.S_grid), dim3(64), 0, st, x, ldx, (const w6u32x4*)w_hi,
                       (const w6u32x4*)w_lo, scales_packed, y, ldy, y_dtype, M, N, p.G, p.S_grid, part, p.Npad, 0);
    if (p.S_grid > 1)
        hipLaunchKernelGGL(w6_reduce_kernel, dim3(p.ntiles, M), dim3(64), 0, st, part, p.S_grid, M, p.Npad, N, y, ldy,
                           y_dtype);
    return check_launch("w6_skinny_gemm");
}

int vw4_w6_partials_layout(int32_t M, int32_t N, int32_t K, int32_t* S, int64_t* ldp) {
    VW4_REQUIRE(M >= 1 && M <= W6_MAX_M && N >= 1 && K >= 64 && K % 64 == 0 && K <= 65536, VW4_EINVAL,
                "vw4_w6_partials_layout: bad shape M=%d N=%d K=%d", M, N, K);
    const W6Plan p = w6_plan(M, N, K);
    if (S) *S = p.S_grid;
    if (ldp) *ldp = p.Npad;
    return VW4_OK;
}

int w6_skinny_gemm_partials(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                            const uint16_t* scales_packed, float* part, int32_t M, int32_t N, int32_t K,
                            void* stream) {
    VW4_REQUIRE(M >= 1 && M <= W6_MAX_M && N >= 1 && K >= 64 && K % 64 == 0 && K <= 65536, VW4_EINVAL,
                "w6_skinny_gemm_partials: bad shape M=%d N=%d K=%d", M, N, K);
    VW4_REQUIRE(x && w_hi && w_lo && scales_packed && part, VW4_EINVAL, "w6_skinny_gemm_partials: null pointer");
    VW4_REQUIRE(ldx >= K && ldx % 8 == 0 && aligned(x, 16), VW4_EINVAL,
                "w6_skinny_gemm_partials: x needs ldx >= K, ldx %% 8 == 0 and 16-byte alignment");
    VW4_REQUIRE(aligned(w_hi, 16) && aligned(w_lo, 16) && aligned(scales_packed, 8) && aligned(part, 16),
                VW4_EINVAL, "w6_skinny_gemm_partials: misaligned pointer");
    const W6Plan p = w6_plan(M, N, K);
    hipLaunchKernelGGL(w6_gemm_kernel, dim3(p.ntiles, p.S_grid), dim3(64), 0, (hipStream_t)stream, x, ldx,
                       (const w6u32x4*)w_hi, (const w6u32x4*)w_lo, scales_packed, (void*)part, p.Npad, VW4_F32, M, N,
                       p.G, p.S_grid, part, p.Npad, 1);
    return check_launch("w6_skinny_gemm_partials");
}

}  // extern "C"
