// w4_gemm.hip — W4 skinny GEMM for the verify rows (M = 1..8).
//
// hazakura.dev, "mtplx——M5 Maxで63tok/s…", section "4層のアーキテクチャ", Layer 0:
// the verify pass is a matmul with a handful of rows (M = 3..6) that needed its
// own shader; gist.science, "BaseRT: …", section "メソドロジー": decode GEMVs
// dequantise inside the inner loop so weights are never materialised.
//
// y[m][n] = sum_g scale[n][g] * sum_{k in g} x[m][k] * c[n][k]
//
// MI355X design (bandwidth-bound: each weight byte is used M times at most):
//  * lane = output row.  A wavefront owns a tile of 64 rows and a slice of the
//    K groups; each lane streams its row's codes with 16-byte loads, and the
//    packed layout makes every wavefront load 1 KiB of contiguous HBM.
//  * The activations x are identical for all 64 lanes, so they are read with
//    scalar loads into SGPRs and feed v_dot2_f32_bf16 directly: no LDS traffic
//    and no cross-lane reduction in the inner loop.
//  * Dequantisation in registers: ((word >> 4i) & 0x000F000F) | 0x43004300 is a
//    pair of bf16 values 128 + u = 136 + c.  The constant 136 is removed once
//    per group by starting the group's accumulator at -136 * sum_{k in g} x[m][k]
//    (computed per workgroup in fp64 and rounded once), so the inner loop is
//    one AND-OR (plus a shift) per pair and M dot2 per pair.
//  * Split K: S_wg wavefronts of a workgroup take consecutive K slices of the
//    same tile and are reduced through LDS; when the tiles are too few to fill
//    the chip, S_grid workgroups per tile write fp32 partials to the workspace
//    and a second launch sums them in slice order.  The summation order
//    depends only on (N, K), never on M or on timing, so results are bitwise
//    reproducible and row m of an M-row call equals the one-row call.
#include <stdlib.h>

#include "common.h"

namespace vw4 {

constexpr int GEMM_MAX_M = 8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Constant address space: uniform loads through it become scalar (SGPR) loads.
typedef const __attribute__((address_space(4))) uint32_t cu32;
constexpr float GEMM_OFFSET = 136.0f;  // bf16 magic 128 plus the code bias 8
constexpr int PF = 4;                  // weight groups in flight per lane

// Marks an address as wavefront-uniform so that loads through it are scalar.
__device__ __forceinline__ cu32* uniform_ptr(cu32* p) {
    const uint64_t a = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return (cu32*)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                           false);
}

// (v & mask) | magic in one instruction: gfx950's three-input bitwise op with
// truth table 0xEA = (A & B) | C.  gfx9 VOP3 encodings take no literal
// constants and at most one SGPR, so the mask comes in an SGPR and the magic
// in a VGPR (the compiler would otherwise emit a v_and / v_or pair).
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t mask_s, uint32_t magic_v) {
    return __builtin_amdgcn_bitop3_b32(v, mask_s, magic_v, 0xEA);
}

template <int M>
__device__ __forceinline__ void gemm_dword(uint32_t word, cu32* const* xg, int xoff, uint32_t kmask,
                                           uint32_t kmagic, float (&ag)[M]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t pair = and_or(word >> (4 * i), kmask, kmagic);
#pragma unroll
        for (int m = 0; m < M; ++m) ag[m] = dot2_bf16(pair, xg[m][xoff + i], ag[m]);
    }
}

// One 64-element group of one row per lane: M partial sums started at
// -136 * sum(x) (xsg[m * ng]), 8 code dwords, then acc += scale * partial.
// Advances the activation pointers by one group.
template <int M>
__device__ __forceinline__ void gemm_group(u32x4 c0, u32x4 c1, uint32_t sbits, cu32** xp, const float* xsg, int ng,
                                           uint32_t kmask, uint32_t magic_v, float (&acc)[M]) {
    float ag[M];
#pragma unroll
    for (int m = 0; m < M; ++m) ag[m] = xsg[m * ng];
    gemm_dword<M>(c0.x, xp, 0, kmask, magic_v, ag);
    gemm_dword<M>(c0.y, xp, 4, kmask, magic_v, ag);
    gemm_dword<M>(c0.z, xp, 8, kmask, magic_v, ag);
    gemm_dword<M>(c0.w, xp, 12, kmask, magic_v, ag);
    gemm_dword<M>(c1.x, xp, 16, kmask, magic_v, ag);
    gemm_dword<M>(c1.y, xp, 20, kmask, magic_v, ag);
    gemm_dword<M>(c1.z, xp, 24, kmask, magic_v, ag);
    gemm_dword<M>(c1.w, xp, 28, kmask, magic_v, ag);
    const float sc = f16_bits_to_f32((uint16_t)sbits);
#pragma unroll
    for (int m = 0; m < M; ++m) {
        acc[m] = fmaf(sc, ag[m], acc[m]);
        xp[m] += 32;
    }
}

// Grouped (mixture-of-experts) launches: blockIdx.z is a slot; slots at or
// beyond *n_slots exit at once; slot s multiplies expert slot_expert[s]
// (weights at w_estride / s_estride per expert) with the activations at
// x + s * x_sstride into the partials at part + s * p_sstride.
struct GemmGroup {
    const int32_t* slot_expert;
    const int32_t* n_slots;   // NULL: plain (single-matrix) launch
    int64_t w_estride;        // u32x4 units
    int64_t s_estride;        // fp16 units
    int64_t x_sstride;        // bf16 elements
    int64_t p_sstride;        // floats
};

template <int M>
__global__ __launch_bounds__(256) void w4_gemm_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                      const u32x4* __restrict__ wpk,
                                                      const uint16_t* __restrict__ spk, void* __restrict__ y,
                                                      int64_t ldy, int ydt, int N, int G, int S_wg, int S_grid,
                                                      float* __restrict__ part, int64_t Npad, uint32_t kmask,
                                                      uint32_t kmagic, GemmGroup grp) {
    extern __shared__ float lds[];
    if (grp.n_slots) {
        const int slot = blockIdx.z;
        if (slot >= __builtin_amdgcn_readfirstlane(*grp.n_slots)) return;
        const int e = __builtin_amdgcn_readfirstlane(grp.slot_expert[slot]);
        wpk += (int64_t)e * grp.w_estride;
        spk += (int64_t)e * grp.s_estride;
        x += (int64_t)slot * grp.x_sstride;
        part += (int64_t)slot * grp.p_sstride;
        y = part;
    }
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int t = blockIdx.x;
    const int S = S_wg * S_grid;
    const int sw0 = blockIdx.y * S_wg;
    const int gw0 = (int)((int64_t)sw0 * G / S);
    const int gw1 = (int)((int64_t)(sw0 + S_wg) * G / S);
    const int ng = gw1 - gw0;
    float* xs = lds;                     // [M][ng]: -136 * sum of the group's x
    float* red = lds + M * ng;           // [S_wg][M][64]

    // Prologue: group sums of x for every group this workgroup touches.
    for (int i = tid; i < M * ng; i += blockDim.x) {
        const int m = i / ng, gg = i - m * ng;
        const uint4* xr = (const uint4*)(x + m * ldx + (int64_t)(gw0 + gg) * 64);
        double s = 0.0;
#pragma unroll 1
        for (int v = 0; v < 8; ++v) {
            const uint4 q = xr[v];
            const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s += (double)bf16_to_f32((uint16_t)(w4[e] & 0xffffu));
                s += (double)bf16_to_f32((uint16_t)(w4[e] >> 16));
            }
        }
        xs[m * ng + gg] = (float)(-(double)GEMM_OFFSET * s);
    }
    __syncthreads();

    const int s_idx = sw0 + wv;
    const int g0 = (int)((int64_t)s_idx * G / S);
    const int g1 = (int)((int64_t)(s_idx + 1) * G / S);

    // Activation rows of the current group, advanced by one group (32 dwords)
    // per iteration; kept wavefront-uniform so every x load is an s_load.
    cu32* xp[M];
#pragma unroll
    for (int m = 0; m < M; ++m) xp[m] = uniform_ptr((cu32*)(x + m * ldx) + g0 * 32);
    const uint32_t magic_v = kmagic;  // lives in a VGPR for and_or()

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.0f;

    // PF groups in flight per lane, each in its own registers: the main loop
    // consumes buffer i and refills it with the group PF further on (clamped to
    // the slice's last group, so every load address is valid and the loop body
    // has no branches); the last < PF groups are consumed after the loop.
    const u32x4* wbase = wpk + (int64_t)t * G * 128 + lane;
    const uint16_t* sbase = spk + (int64_t)t * G * 64 + lane;
    const int glast = g1 - 1;
    if (g0 < g1) {
        u32x4 b0[PF], b1[PF];
        uint32_t bs[PF];  // fp16 scale bits, one register each (packing two would force early waits)
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            const int gi = min(g0 + i, glast);
            b0[i] = __builtin_nontemporal_load(wbase + (int64_t)gi * 128);
            b1[i] = __builtin_nontemporal_load(wbase + (int64_t)gi * 128 + 64);
            bs[i] = sbase[(int64_t)gi * 64];
        }
        int g = g0;
        for (; g + PF <= g1; g += PF) {
#pragma unroll
            for (int i = 0; i < PF; ++i) {
                gemm_group<M>(b0[i], b1[i], bs[i], xp, xs + (g + i - gw0), ng, kmask, magic_v, acc);
                const int gn = min(g + i + PF, glast);
                // keep the refill right after its buffer's last use: the
                // scheduler would otherwise sink all refills to the loop end
                __builtin_amdgcn_sched_barrier(0);
                b0[i] = __builtin_nontemporal_load(wbase + (int64_t)gn * 128);
                b1[i] = __builtin_nontemporal_load(wbase + (int64_t)gn * 128 + 64);
                bs[i] = sbase[(int64_t)gn * 64];
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int i = 0; i < PF - 1; ++i)
            if (g + i < g1) gemm_group<M>(b0[i], b1[i], bs[i], xp, xs + (g + i - gw0), ng, kmask, magic_v, acc);
    }

    // Reduce the S_wg slices of this workgroup in slice order.
    float v[M];
    if (S_wg > 1) {
#pragma unroll
        for (int m = 0; m < M; ++m) red[(wv * M + m) * 64 + lane] = acc[m];
        __syncthreads();
        if (wv == 0) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                float s = red[m * 64 + lane];
                for (int w = 1; w < S_wg; ++w) s += red[(w * M + m) * 64 + lane];
                v[m] = s;
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < M; ++m) v[m] = acc[m];
    }

    const int n = t * 64 + lane;
    if (wv != 0) return;
    if (S_grid == 1) {
        if (n < N) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                if (ydt == VW4_F32) ((float*)y)[m * ldy + n] = v[m];
                else ((uint16_t*)y)[m * ldy + n] = f32_to_bf16(v[m]);
            }
        }
        return;
    }
    // Split across workgroups: fp32 partials; w4_gemm_reduce_kernel sums them.
#pragma unroll
    for (int m = 0; m < M; ++m) part[((int64_t)blockIdx.y * M + m) * Npad + n] = v[m];
}

// Sum of the S_grid partials of each output in slice order (a separate launch:
// on this part a dependent launch is cheaper than a device-wide atomic
// counter per workgroup).  grid = (ntiles, M), 64 threads.
__global__ __launch_bounds__(64) void w4_gemm_reduce_kernel(const float* __restrict__ part, int S_grid, int M,
                                                            int64_t Npad, int N, void* __restrict__ y, int64_t ldy,
                                                            int ydt) {
    const int n = blockIdx.x * 64 + threadIdx.x, m = blockIdx.y;
    if (n >= N) return;
    float s = 0.0f;
    for (int b0 = 0; b0 < S_grid; b0 += 8) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (b0 + i < S_grid) ? part[((int64_t)(b0 + i) * M + m) * Npad + n] : 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (b0 + i < S_grid) s += v[i];
    }
    if (ydt == VW4_F32) ((float*)y)[m * ldy + n] = s;
    else ((uint16_t*)y)[m * ldy + n] = f32_to_bf16(s);
}

struct GemmPlan {
    int ntiles, G, S_wg, S_grid;
    int64_t Npad;
    size_t ws_bytes;
    size_t lds_bytes;
};

// Split of K over wavefronts: enough wavefronts to cover the 256 CUs several
// times, at least two groups per wavefront.  Depends on (N, K) only.
// slots: matrices per launch (grouped launches spread the wave target over
// all of them).
static GemmPlan plan_gemm(int M, int N, int K, int slots = 1) {
    GemmPlan p;
    p.G = K / 64;
    p.ntiles = (N + 63) / 64;
    p.Npad = (int64_t)p.ntiles * 64;
    const int target_waves = 8192;
    const int units = p.ntiles * slots;
    int S = (target_waves + units - 1) / units;
    int maxS = p.G / 2 > 0 ? p.G / 2 : 1;
    if (S > maxS) S = maxS;
    if (S < 1) S = 1;
    p.S_wg = S < 4 ? S : 4;
    p.S_grid = (S + p.S_wg - 1) / p.S_wg;
    if (const char* e = getenv("VW4_GEMM_SPLIT")) {
        int a = 0, b = 0;
        if (sscanf(e, "%d,%d", &a, &b) == 2 && a >= 1 && a <= 4 && b >= 1 && a * b <= p.G) {
            p.S_wg = a;
            p.S_grid = b;
        }
    }
    const int S_all = p.S_wg * p.S_grid;
    const int ng_max = (int)(((int64_t)p.S_wg * p.G + S_all - 1) / S_all) + 1;
    p.lds_bytes = (size_t)M * ng_max * 4 + (p.S_wg > 1 ? (size_t)p.S_wg * M * 64 * 4 : 0);
    p.ws_bytes = 0;
    if (p.S_grid > 1) p.ws_bytes = ((size_t)p.S_grid * M * p.Npad * 4 + 255) / 256 * 256;
    return p;
}

template <int M>
static void launch_gemm(const GemmPlan& p, const uint16_t* x, int64_t ldx, const uint8_t* w, const uint16_t* s,
                        void* y, int64_t ldy, int ydt, int N, float* part, hipStream_t st) {
    hipLaunchKernelGGL(w4_gemm_kernel<M>, dim3(p.ntiles, p.S_grid), dim3(64 * p.S_wg), p.lds_bytes, st, x, ldx,
                       (const u32x4*)w, s, y, ldy, ydt, N, p.G, p.S_wg, p.S_grid, part, p.Npad, 0x000F000Fu,
                       0x43004300u, GemmGroup{});
    if (p.S_grid > 1)
        hipLaunchKernelGGL(w4_gemm_reduce_kernel, dim3(p.ntiles, M), dim3(64), 0, st, part, p.S_grid, M, p.Npad, N,
                           y, ldy, ydt);
}

int gemm_dispatch(const uint16_t* x, int64_t ldx, const uint8_t* w, const uint16_t* s, void* y, int64_t ldy,
                  int ydt, int M, int N, int K, void* ws, size_t ws_bytes, hipStream_t st) {
    VW4_REQUIRE(M >= 1 && M <= GEMM_MAX_M, VW4_EINVAL, "w4_skinny_gemm: M=%d must be in [1, 8]", M);
    VW4_REQUIRE(N >= 1, VW4_EINVAL, "w4_skinny_gemm: N=%d must be >= 1", N);
    VW4_REQUIRE(K >= 64 && K % 64 == 0 && K <= 65536, VW4_EINVAL,
                "w4_skinny_gemm: K=%d must be a multiple of 64 in [64, 65536]", K);
    VW4_REQUIRE(x && w && s && y, VW4_EINVAL, "w4_skinny_gemm: null pointer");
    VW4_REQUIRE(ldx >= K && ldx % 8 == 0 && aligned(x, 16), VW4_EINVAL,
                "w4_skinny_gemm: x needs ldx >= K, ldx %% 8 == 0 and 16-byte alignment");
    VW4_REQUIRE(aligned(w, 16) && aligned(s, 2), VW4_EINVAL, "w4_skinny_gemm: packed weights must be 16-byte aligned");
    VW4_REQUIRE(ldy >= N, VW4_EINVAL, "w4_skinny_gemm: ldy=%lld < N=%d", (long long)ldy, N);
    VW4_REQUIRE(ydt == VW4_F32 || ydt == VW4_BF16, VW4_EINVAL, "w4_skinny_gemm: y_dtype must be VW4_F32 or VW4_BF16");
    VW4_REQUIRE(aligned(y, ydt == VW4_F32 ? 4 : 2), VW4_EINVAL, "w4_skinny_gemm: y misaligned");
    const GemmPlan p = plan_gemm(M, N, K);
    float* part = nullptr;
    if (p.ws_bytes) {
        VW4_REQUIRE(ws && ws_bytes >= p.ws_bytes && aligned(ws, 256), VW4_EWORKSPACE,
                    "w4_skinny_gemm: needs a 256-byte aligned workspace of %zu bytes", p.ws_bytes);
        part = (float*)ws;
    }
    switch (M) {
        case 1: launch_gemm<1>(p, x, ldx, w, s, y, ldy, ydt, N, part, st); break;
        case 2: launch_gemm<2>(p, x, ldx, w, s, y, ldy, ydt, N, part, st); break;
        case 3: launch_gemm<3>(p, x, ldx, w, s, y, ldy, ydt, N, part, st); break;
        case 4: launch_gemm<4>(p, x, ldx, w, s, y, ldy, ydt, N, part, st); break;
        case 5: launch_gemm<5>(p, x, ldx, w, s, y, ldy, ydt, N, part, st); break;
        case 6: launch_gemm<6>(p, x, ldx, w, s, y, ldy, ydt, N, part, st); break;
        case 7: launch_gemm<7>(p, x, ldx, w, s, y, ldy, ydt, N, part, st); break;
        default: launch_gemm<8>(p, x, ldx, w, s, y, ldy, ydt, N, part, st); break;
    }
    return check_launch("w4_skinny_gemm");
}

// Partials form: the main kernel only (no reduction launch); part is the
// caller's [S_grid][M][Npad] fp32 buffer (per slot for grouped launches).
int gemm_partials(const uint16_t* x, int64_t ldx, const uint8_t* w, const uint16_t* s, float* part, int M, int N,
                  int K, hipStream_t st, const GemmGroup& grp = GemmGroup{}, int max_slots = 1) {
    VW4_REQUIRE(M >= 1 && M <= GEMM_MAX_M, VW4_EINVAL, "w4_skinny_gemm_partials: M=%d must be in [1, 8]", M);
    VW4_REQUIRE(N >= 1, VW4_EINVAL, "w4_skinny_gemm_partials: N=%d must be >= 1", N);
    VW4_REQUIRE(K >= 64 && K % 64 == 0 && K <= 65536, VW4_EINVAL,
                "w4_skinny_gemm_partials: K=%d must be a multiple of 64 in [64, 65536]", K);
    VW4_REQUIRE(x && w && s && part, VW4_EINVAL, "w4_skinny_gemm_partials: null pointer");
    VW4_REQUIRE(ldx >= K && ldx % 8 == 0 && aligned(x, 16), VW4_EINVAL,
                "w4_skinny_gemm_partials: x needs ldx >= K, ldx %% 8 == 0 and 16-byte alignment");
    VW4_REQUIRE(aligned(w, 16) && aligned(s, 2) && aligned(part, 4), VW4_EINVAL,
                "w4_skinny_gemm_partials: misaligned pointer");
    const GemmPlan p = plan_gemm(M, N, K, max_slots);
    // S_grid == 1 writes the product straight into part[0] with row stride Npad
    void* y = part;
    const int64_t ldy = p.Npad;
    float* pp = part;
    switch (M) {
#define VW4_CASE(MM)                                                                                               \
    case MM:                                                                                                       \
        hipLaunchKernelGGL(w4_gemm_kernel<MM>, dim3(p.ntiles, p.S_grid, max_slots), dim3(64 * p.S_wg), p.lds_bytes, st, x, ldx, \
                           (const u32x4*)w, s, y, ldy, VW4_F32, N, p.G, p.S_wg, p.S_grid, pp, p.Npad, 0x000F000Fu,   \
                           0x43004300u, grp);                                                                      \
        break;
        VW4_CASE(1) VW4_CASE(2) VW4_CASE(3) VW4_CASE(4) VW4_CASE(5) VW4_CASE(6) VW4_CASE(7) VW4_CASE(8)
#undef VW4_CASE
    }
    return check_launch("w4_skinny_gemm_partials");
}

int grouped_gemm_partials(const uint16_t* x, int64_t ldx, int64_t x_sstride, const uint8_t* w_bank,
                          int64_t w_estride_bytes, const uint16_t* s_bank, int64_t s_estride, const int32_t* slot_expert,
                          const int32_t* n_slots, int max_slots, float* part, int64_t p_sstride, int M, int N, int K,
                          hipStream_t st) {
    VW4_REQUIRE(slot_expert && n_slots && max_slots >= 1 && max_slots <= 65535, VW4_EINVAL,
                "w4_grouped_gemm: bad slot arguments");
    VW4_REQUIRE(w_estride_bytes % 16 == 0 && w_estride_bytes > 0 && s_estride > 0, VW4_EINVAL,
                "w4_grouped_gemm: expert strides must be positive, weights 16-byte multiples");
    VW4_REQUIRE(x_sstride % 8 == 0 && x_sstride >= 0 && p_sstride >= 0, VW4_EINVAL,
                "w4_grouped_gemm: bad slot strides");
    GemmGroup g;
    g.slot_expert = slot_expert;
    g.n_slots = n_slots;
    g.w_estride = w_estride_bytes / 16;
    g.s_estride = s_estride;
    g.x_sstride = x_sstride;
    g.p_sstride = p_sstride;
    return gemm_partials(x, ldx, w_bank, s_bank, part, M, N, K, st, g, max_slots);
}

int gemm_layout(int M, int N, int K, int* S, int64_t* ldp, int slots = 1) {
    VW4_REQUIRE(M >= 1 && M <= GEMM_MAX_M && N >= 1 && K >= 64 && K % 64 == 0 && K <= 65536, VW4_EINVAL,
                "vw4_gemm_partials_layout: bad shape M=%d N=%d K=%d", M, N, K);
    VW4_REQUIRE(slots >= 1 && slots <= 65535, VW4_EINVAL, "vw4_grouped_gemm_layout: max_slots=%d", slots);
    const GemmPlan p = plan_gemm(M, N, K, slots);
    if (S) *S = p.S_grid;
    if (ldp) *ldp = p.Npad;
    return VW4_OK;
}

size_t gemm_ws_bytes(int M, int N, int K) {
    if (M < 1 || M > GEMM_MAX_M || N < 1 || K < 64 || K % 64) return 0;
    return plan_gemm(M, N, K).ws_bytes;
}

}  // namespace vw4

extern "C" {

size_t vw4_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K) { return vw4::gemm_ws_bytes(M, N, K); }

int vw4_gemm_partials_layout(int32_t M, int32_t N, int32_t K, int32_t* S, int64_t* ldp) {
    int s = 0;
    int rc = vw4::gemm_layout(M, N, K, &s, ldp);
    if (S) *S = s;
    return rc;
}

int vw4_grouped_gemm_layout(int32_t M, int32_t N, int32_t K, int32_t max_slots, int32_t* S, int64_t* ldp) {
    int s = 0;
    int rc = vw4::gemm_layout(M, N, K, &s, ldp, max_slots);
    if (S) *S = s;
    return rc;
}

int w4_grouped_gemm(const uint16_t* x, int64_t ldx, int64_t x_sstride, const uint8_t* w_bank, int64_t w_estride,
                    const uint16_t* s_bank, int64_t s_estride, const int32_t* slot_expert, const int32_t* n_slots,
                    int32_t max_slots, float* part, int64_t p_sstride, int32_t M, int32_t N, int32_t K, void* stream) {
    if (max_slots >= 1 && max_slots <= 65535 && M >= 1 && M <= vw4::GEMM_MAX_M && N >= 1 && K >= 64 && K % 64 == 0) {
        int S = 0;
        int64_t ldp = 0;
        vw4::gemm_layout(M, N, K, &S, &ldp, max_slots);
        VW4_REQUIRE(p_sstride >= (int64_t)S * M * ldp, VW4_EINVAL,
                    "w4_grouped_gemm: p_sstride %lld < S * M * ldp = %lld", (long long)p_sstride,
                    (long long)((int64_t)S * M * ldp));
    }
    return vw4::grouped_gemm_partials(x, ldx, x_sstride, w_bank, w_estride, s_bank, s_estride, slot_expert, n_slots,
                                      max_slots, part, p_sstride, M, N, K, (hipStream_t)stream);
}

int w4_skinny_gemm_partials(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, const uint16_t* scales_packed,
                            float* part, int32_t M, int32_t N, int32_t K, void* stream) {
    return vw4::gemm_partials(x, ldx, w_packed, scales_packed, part, M, N, K, (hipStream_t)stream);
}

int w4_skinny_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, const uint16_t* scales_packed, void* y,
                   int64_t ldy, int32_t y_dtype, int32_t M, int32_t N, int32_t K, void* ws, size_t ws_bytes,
                   void* stream) {
    return vw4::gemm_dispatch(x, ldx, w_packed, scales_packed, y, ldy, y_dtype, M, N, K, ws, ws_bytes,
                              (hipStream_t)stream);
}

}  // extern "C"
