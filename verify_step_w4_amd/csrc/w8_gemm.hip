// w8_gemm.hip — the skinny GEMM on W8 weights (M = 1..8): a second weight
// format for the verify rows (gist.science, "BaseRT: …", section "メソドロジー",
// lists the quantisation formats its GEMV reads and names Q8).
//
// y[m][n] = sum_g scale[n][g] * sum_{k in g} x[m][k] * c[n][k],  c in [-127, 127]
//
// The code u = c + 128 is split into its high and low nibbles, each stored in
// the W4 packed layout (w4_format.hip), so the lane mapping, the bf16
// magic-number dequantisation (one v_bitop3 per pair: 128 + nibble) and the
// v_mfma_f32_16x16x32_bf16 operands are those of the W4 kernel, with two
// planes per group instead of one.  With D_hi = sum x (128 + hi) and
// D_lo = sum x (128 + lo):  sum x c = 16 D_hi + D_lo - 2304 sum x.  The chain
// of the high plane starts from x . (-144) (formed by the matrix cores from
// the same A operand), so 16 (D_hi - 144 sum x) + D_lo is the group's sum.
// Products are exact in fp32 (bf16 x 8-bit integer), sums are fp32 in an
// order that depends only on (N, K): row m of an M-row call equals the
// one-row call bit for bit.
#include "common.h"

namespace vw4 {

namespace {

constexpr int W8_MAX_M = 8;
constexpr int W8_PF = 4;                       // groups in flight per lane
constexpr uint32_t NEG144_PAIR = 0xC310C310u;  // two bf16 -144.0
typedef uint32_t w8u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((ext_vector_type(8))) __bf16 w8bf16x8;
typedef __attribute__((ext_vector_type(4))) float w8f32x4;

__device__ __forceinline__ uint32_t w8_and_or(uint32_t v, uint32_t mask_s, uint32_t magic_v) {
    return __builtin_amdgcn_bitop3_b32(v, mask_s, magic_v, 0xEA);   // (v & mask) | magic
}

__device__ __forceinline__ w8bf16x8 w8_dequant8(uint32_t w, uint32_t kmask, uint32_t magic_v) {
    w8u32x4 r;
    r.x = w8_and_or(w, kmask, magic_v);
    r.y = w8_and_or(w >> 4, kmask, magic_v);
    r.z = w8_and_or(w >> 8, kmask, magic_v);
    r.w = w8_and_or(w >> 12, kmask, magic_v);
    return __builtin_bit_cast(w8bf16x8, r);
}

__device__ __forceinline__ w8f32x4 w8_mfma(w8bf16x8 a, w8bf16x8 b, w8f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One K-group of one tile.  ha / hb: the lane's two 16-byte loads of the high
// plane (row blocks 0, 1 and 2, 3), la / lb of the low plane; xa / xb: its
// activations for k halves 0 / 1; sc: its four row scales (fp16 pairs).
__device__ __forceinline__ void w8_group(w8u32x4 ha, w8u32x4 hb, w8u32x4 la, w8u32x4 lb, w8u32x4 xa, w8u32x4 xb,
                                         uint2 sc, uint32_t kmask, uint32_t magic_v, w8f32x4 (&acc)[4]) {
    const w8bf16x8 a0 = __builtin_bit_cast(w8bf16x8, xa), a1 = __builtin_bit_cast(w8bf16x8, xb);
    const w8u32x4 nq = {NEG144_PAIR, NEG144_PAIR, NEG144_PAIR, NEG144_PAIR};
    const w8bf16x8 neg = __builtin_bit_cast(w8bf16x8, nq);
    const w8f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const w8f32x4 off = w8_mfma(a1, neg, w8_mfma(a0, neg, zero));
    const uint32_t hw[8] = {ha.x, ha.y, ha.z, ha.w, hb.x, hb.y, hb.z, hb.w};
    const uint32_t lw[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
    const float f[4] = {f16_bits_to_f32((uint16_t)(sc.x & 0xffffu)), f16_bits_to_f32((uint16_t)(sc.x >> 16)),
                        f16_bits_to_f32((uint16_t)(sc.y & 0xffffu)), f16_bits_to_f32((uint16_t)(sc.y >> 16))};
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const w8f32x4 dh = w8_mfma(a1, w8_dequant8(hw[2 * nb + 1], kmask, magic_v),
                                   w8_mfma(a0, w8_dequant8(hw[2 * nb], kmask, magic_v), off));
        const w8f32x4 dl = w8_mfma(a1, w8_dequant8(lw[2 * nb + 1], kmask, magic_v),
                                   w8_mfma(a0, w8_dequant8(lw[2 * nb], kmask, magic_v), zero));
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[nb][r] = fmaf(f[nb], fmaf(16.0f, dh[r], dl[r]), acc[nb][r]);
    }
}

// grid (ntiles, S_grid), one wavefront each: tile t, K-groups g0 .. g1 of
// slice s.  S_grid == 1 writes y; otherwise fp32 partials part[s][m][Npad].
__global__ __launch_bounds__(64) void w8_gemm_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                     const w8u32x4* __restrict__ whi,
                                                     const w8u32x4* __restrict__ wlo,
                                                     const uint16_t* __restrict__ spk, void* __restrict__ y,
                                                     int64_t ldy, int ydt, int M, int N, int G, int S_grid,
                                                     float* __restrict__ part, int64_t Npad, int to_part) {
    const int lane = threadIdx.x, kq = lane >> 4, i = lane & 15;
    const int t = blockIdx.x, s_idx = blockIdx.y;
    const int g0 = s_idx * G / S_grid, g1 = (s_idx + 1) * G / S_grid;
    const uint32_t kmask = 0x000F000Fu;
    const uint32_t magic_v = 0x43004300u;
    const int xr = i < M ? i : M - 1;            // A rows i >= M feed outputs that are never stored
    const w8u32x4* hbase = whi + (int64_t)t * G * 128 + lane;
    const w8u32x4* lbase = wlo + (int64_t)t * G * 128 + lane;
    const uint2* sbase = (const uint2*)spk + (int64_t)t * G * 16 + i;
    const w8u32x4* xbase = (const w8u32x4*)(x + (int64_t)xr * ldx) + kq;
    w8f32x4 acc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] = w8f32x4{0.f, 0.f, 0.f, 0.f};
    const int glast = g1 > g0 ? g1 - 1 : g0;
    w8u32x4 bh0[W8_PF], bh1[W8_PF], bl0[W8_PF], bl1[W8_PF], bx0[W8_PF], bx1[W8_PF];
    uint2 bs[W8_PF];
    auto issue = [&](int j, int gi) {
        bh0[j] = __builtin_nontemporal_load(hbase + (int64_t)gi * 128);
        bh1[j] = __builtin_nontemporal_load(hbase + (int64_t)gi * 128 + 64);
        bl0[j] = __builtin_nontemporal_load(lbase + (int64_t)gi * 128);
        bl1[j] = __builtin_nontemporal_load(lbase + (int64_t)gi * 128 + 64);
        bx0[j] = xbase[(int64_t)gi * 8];
        bx1[j] = xbase[(int64_t)gi * 8 + 4];
        bs[j] = sbase[(int64_t)gi * 16];
    };
    // g0 < G always (S_grid <= G): every address below is valid
#pragma unroll
    for (int j = 0; j < W8_PF; ++j) issue(j, min(g0 + j, glast));
    __builtin_amdgcn_sched_barrier(0);
    if (g0 < g1) {
        int g = g0;
        for (; g + W8_PF <= g1; g += W8_PF) {
#pragma unroll
            for (int j = 0; j < W8_PF; ++j) {
                w8_group(bh0[j], bh1[j], bl0[j], bl1[j], bx0[j], bx1[j], bs[j], kmask, magic_v, acc);
                __builtin_amdgcn_sched_barrier(0);
                issue(j, min(g + j + W8_PF, glast));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int j = 0; j < W8_PF - 1; ++j)
            if (g + j < g1) w8_group(bh0[j], bh1[j], bl0[j], bl1[j], bx0[j], bx1[j], bs[j], kmask, magic_v, acc);
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
__global__ __launch_bounds__(64) void w8_reduce_kernel(const float* __restrict__ part, int S_grid, int M, int64_t Npad,
                                                       int N, void* __restrict__ y, int64_t ldy, int ydt) {
    const int n = blockIdx.x * 64 + threadIdx.x, m = blockIdx.y;
    if (n >= N) return;
    float s = 0.0f;
    for (int b = 0; b < S_grid; ++b) s += part[((int64_t)b * M + m) * Npad + n];
    if (ydt == VW4_F32) ((float*)y)[m * ldy + n] = s;
    else ((uint16_t*)y)[m * ldy + n] = f32_to_bf16(s);
}

struct W8Plan {
    int ntiles, G, S_grid;
    int64_t Npad;
    size_t ws_bytes;
};

// About two wavefronts per SIMD over the chip, at least four K-groups each,
// at most 8 partial slices.
W8Plan w8_plan(int M, int N, int K) {
    W8Plan p;
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

size_t vw4_w8_workspace_bytes(int32_t M, int32_t N, int32_t K) {
    if (M < 1 || M > W8_MAX_M || N < 1 || K < 64 || K % 64 || K > 65536) return 0;
    return w8_plan(M, N, K).ws_bytes;
}

int w8_skinny_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                   const uint16_t* scales_packed, void* y, int64_t ldy, int32_t y_dtype, int32_t M, int32_t N,
                   int32_t K, void* ws, size_t ws_bytes, void* stream) {
    VW4_REQUIRE(M >= 1 && M <= W8_MAX_M, VW4_EINVAL, "w8_skinny_gemm: M=%d must be in [1, 8]", M);
    VW4_REQUIRE(N >= 1, VW4_EINVAL, "w8_skinny_gemm: N=%d must be >= 1", N);
    VW4_REQUIRE(K >= 64 && K % 64 == 0 && K <= 65536, VW4_EINVAL,
                "w8_skinny_gemm: K=%d must be a multiple of 64 in [64, 65536]", K);
    VW4_REQUIRE(x && w_hi && w_lo && scales_packed && y, VW4_EINVAL, "w8_skinny_gemm: null pointer");
    VW4_REQUIRE(ldx >= K && ldx % 8 == 0 && aligned(x, 16), VW4_EINVAL,
                "w8_skinny_gemm: x needs ldx >= K, ldx %% 8 == 0 and 16-byte alignment");
    VW4_REQUIRE(aligned(w_hi, 16) && aligned(w_lo, 16) && aligned(scales_packed, 8), VW4_EINVAL,
                "w8_skinny_gemm: packed planes must be 16-byte and packed scales 8-byte aligned");
    VW4_REQUIRE(ldy >= N, VW4_EINVAL, "w8_skinny_gemm: ldy=%lld < N=%d", (long long)ldy, N);
    VW4_REQUIRE(y_dtype == VW4_F32 || y_dtype == VW4_BF16, VW4_EINVAL,
                "w8_skinny_gemm: y_dtype must be VW4_F32 or VW4_BF16");
    VW4_REQUIRE(aligned(y, y_dtype == VW4_F32 ? 4 : 2), VW4_EINVAL, "w8_skinny_gemm: y misaligned");
    const W8Plan p = w8_plan(M, N, K);
    float* part = nullptr;
    if (p.ws_bytes) {
        VW4_REQUIRE(ws && ws_bytes >= p.ws_bytes && aligned(ws, 256), VW4_EWORKSPACE,
                    "w8_skinny_gemm: needs a 256-byte aligned workspace of %zu bytes", p.ws_bytes);
        part = (float*)ws;
    }
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(w8_gemm_kernel, dim3(p.ntiles, p.S_grid), dim3(64), 0, st, x, ldx, (const w8u32x4*)w_hi,
                       (const w8u32x4*)w_lo, scales_packed, y, ldy, y_dtype, M, N, p.G, p.S_grid, part, p.Npad, 0);
    if (p.S_grid > 1)
        hipLaunchKernelGGL(w8_reduce_kernel, dim3(p.ntiles, M), dim3(64), 0, st, part, p.S_grid, M, p.Npad, N, y, ldy,
                           y_dtype);
    return check_launch("w8_skinny_gemm");
}

int vw4_w8_partials_layout(int32_t M, int32_t N, int32_t K, int32_t* S, int64_t* ldp) {
    VW4_REQUIRE(M >= 1 && M <= W8_MAX_M && N >= 1 && K >= 64 && K % 64 == 0 && K <= 65536, VW4_EINVAL,
                "vw4_w8_partials_layout: bad shape M=%d N=%d K=%d", M, N, K);
    const W8Plan p = w8_plan(M, N, K);
    if (S) *S = p.S_grid;
    if (ldp) *ldp = p.Npad;
    return VW4_OK;
}

int w8_skinny_gemm_partials(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                            const uint16_t* scales_packed, float* part, int32_t M, int32_t N, int32_t K,
                            void* stream) {
    VW4_REQUIRE(M >= 1 && M <= W8_MAX_M && N >= 1 && K >= 64 && K % 64 == 0 && K <= 65536, VW4_EINVAL,
                "w8_skinny_gemm_partials: bad shape M=%d N=%d K=%d", M, N, K);
    VW4_REQUIRE(x && w_hi && w_lo && scales_packed && part, VW4_EINVAL, "w8_skinny_gemm_partials: null pointer");
    VW4_REQUIRE(ldx >= K && ldx % 8 == 0 && aligned(x, 16), VW4_EINVAL,
                "w8_skinny_gemm_partials: x needs ldx >= K, ldx %% 8 == 0 and 16-byte alignment");
    VW4_REQUIRE(aligned(w_hi, 16) && aligned(w_lo, 16) && aligned(scales_packed, 8) && aligned(part, 16),
                VW4_EINVAL, "w8_skinny_gemm_partials: misaligned pointer");
    const W8Plan p = w8_plan(M, N, K);
    hipLaunchKernelGGL(w8_gemm_kernel, dim3(p.ntiles, p.S_grid), dim3(64), 0, (hipStream_t)stream, x, ldx,
                       (const w8u32x4*)w_hi, (const w8u32x4*)w_lo, scales_packed, (void*)part, p.Npad, VW4_F32, M, N,
                       p.G, p.S_grid, part, p.Npad, 1);
    return check_launch("w8_skinny_gemm_partials");
}

}  // extern "C"
