// w4_gemm.hip — W4 skinny GEMM for the verify rows (M = 1..8).
//
// hazakura.dev, "mtplx——M5 Maxで63tok/s…", section "4層のアーキテクチャ", Layer 0:
// the verify pass is a matmul with a handful of rows (M = 3..6) that needed its
// own shader; gist.science, "BaseRT: …", section "メソドロジー": decode GEMVs
// dequantise inside the inner loop so weights are never materialised.
//
// y[m][n] = sum_g scale[n][g] * sum_{k in g} x[m][k] * c[n][k]
//
// MI355X design.  The op is bound by HBM: every weight byte is read once and
// used by M <= 8 rows.  On gfx950, though, forming those products on the
// vector ALU (v_dot2_f32_bf16, 2 MACs per lane-op) plus the dequantisation
// costs about 24 lane-ops per 4 bytes of weights at M = 4, more than the
// chip issues at full HBM speed.  So the multiplies go to the matrix cores
// and the vector ALU only dequantises:
//  * A wavefront owns a tile of 64 rows and a slice of the K groups.  Per
//    64-element group, lane l = 16 kq + i loads 32 bytes (two 16-byte loads,
//    each part of a contiguous 1 KiB wavefront load): the 8 code nibbles of
//    rows 16 nb + i (nb = 0..3) at k = 32 s + 8 kq .. +8 (s = 0, 1), exactly
//    its B operand (W^T, column = row of W) of v_mfma_f32_16x16x32_bf16.
//  * The A operand is the activations: lane l supplies x[i][32 s + 8 kq .. +8]
//    (for i >= M any valid row: those output rows are not stored), read once
//    per group from L2.  D[m][n] lands in
//    lane (kq, i) as rows m = 4 kq .. +4, column n = 16 nb + i.
//  * Dequantisation in registers: ((word >> 4j) & 0x000F000F) | 0x43004300 is
//    a pair of bf16 values 128 + u = 136 + c (one v_bitop3 per pair).  The
//    constant is removed by one more product per group: the C input of the
//    four row blocks' products is x . (-136), which the matrix cores form from
//    the same A operand.  Then acc += scale[n] * D, per row.
//  * Split K: S_wg wavefronts of a workgroup take consecutive K slices of the
//    same tile and are reduced through LDS; when the tiles are too few to fill
//    the chip, S_grid workgroups per tile write fp32 partials and the consumer
//    (or a second launch) sums them in slice order.  Every summation order
//    depends only on (N, K): results are bitwise reproducible and row m of an
//    M-row call equals the one-row call (the matrix core computes each output
//    from its own row of A).
#include <stdlib.h>

#include <mutex>

#include "common.h"

namespace vw4 {

constexpr int GEMM_MAX_M = 8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
constexpr int PF = 4;                  // groups in flight per lane
constexpr int NORM_MAX_K = 64 * NORM_CHUNK;  // NORM mode: at most 64 chunk sums per row
constexpr uint32_t NEG136_PAIR = 0xC308C308u;  // two bf16 -136.0

// (v & mask) | magic in one instruction: gfx950's three-input bitwise op with
// truth table 0xEA = (A & B) | C.  gfx9 VOP3 encodings take no literal
// constants and at most one SGPR, so the mask comes in an SGPR and the magic
// in a VGPR (the compiler would otherwise emit a v_and / v_or pair).
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t mask_s, uint32_t magic_v) {
    return __builtin_amdgcn_bitop3_b32(v, mask_s, magic_v, 0xEA);
}

// 8 code nibbles -> the 8 bf16 values 128 + u of one MFMA operand.
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, uint32_t kmask, uint32_t magic_v) {
    u32x4 r;
    r.x = and_or(w, kmask, magic_v);
    r.y = and_or(w >> 4, kmask, magic_v);
    r.z = and_or(w >> 8, kmask, magic_v);
    r.w = and_or(w >> 12, kmask, magic_v);
    return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One K-group of one tile: wa / wb = the lane's two 16-byte code loads (row
// blocks 0, 1 and 2, 3), xa / xb = its activations for k halves 0 / 1, sc =
// its four row scales (fp16 pairs).
__device__ __forceinline__ void gemm_group(u32x4 wa, u32x4 wb, u32x4 xa, u32x4 xb, uint2 sc, uint32_t kmask,
                                           uint32_t magic_v, f32x4 (&acc)[4]) {
    const bf16x8 a0 = __builtin_bit_cast(bf16x8, xa), a1 = __builtin_bit_cast(bf16x8, xb);
    const u32x4 nq = {NEG136_PAIR, NEG136_PAIR, NEG136_PAIR, NEG136_PAIR};
    const bf16x8 neg = __builtin_bit_cast(bf16x8, nq);
    f32x4 off = {0.f, 0.f, 0.f, 0.f};
    off = mfma16(a0, neg, off);
    off = mfma16(a1, neg, off);
    f32x4 d[4];
    d[0] = mfma16(a1, dequant8(wa.y, kmask, magic_v), mfma16(a0, dequant8(wa.x, kmask, magic_v), off));
    d[1] = mfma16(a1, dequant8(wa.w, kmask, magic_v), mfma16(a0, dequant8(wa.z, kmask, magic_v), off));
    d[2] = mfma16(a1, dequant8(wb.y, kmask, magic_v), mfma16(a0, dequant8(wb.x, kmask, magic_v), off));
    d[3] = mfma16(a1, dequant8(wb.w, kmask, magic_v), mfma16(a0, dequant8(wb.z, kmask, magic_v), off));
    const float f[4] = {f16_bits_to_f32((uint16_t)(sc.x & 0xffffu)), f16_bits_to_f32((uint16_t)(sc.x >> 16)),
                        f16_bits_to_f32((uint16_t)(sc.y & 0xffffu)), f16_bits_to_f32((uint16_t)(sc.y >> 16))};
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[nb][r] = fmaf(f[nb], d[nb][r], acc[nb][r]);
}

// Eight activations of one row: h = bf16((r * inv) * gamma) per element, the
// standalone normalisation's arithmetic in its order.
__device__ __forceinline__ u32x4 norm8(u32x4 r, u32x4 g, float inv) {
    u32x4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float rl = __uint_as_float(r[e] << 16), rh = __uint_as_float(r[e] & 0xffff0000u);
        const float gl = __uint_as_float(g[e] << 16), gh = __uint_as_float(g[e] & 0xffff0000u);
        h[e] = f32x2_to_bf16x2(rl * inv * gl, rh * inv * gh);
    }
    return h;
}

// Grouped (mixture-of-experts) launches: blockIdx.z is a slot; slots at or
// beyond *n_slots exit at once; slot s multiplies expert slot_expert[s]
// (weights at w_estride / s_estride per expert) with the activations at
// x + s * x_sstride into the partials at part + s * p_sstride (SwiGLU
// epilogue: into y + s * y_sstride).
struct GemmGroup {
    const int32_t* slot_expert;
    const int32_t* n_slots;   // NULL: plain (single-matrix) launch
    int64_t w_estride;        // u32x4 units
    int64_t s_estride;        // fp16 units
    int64_t x_sstride;        // bf16 elements
    int64_t p_sstride;        // floats
    int64_t y_sstride;        // bf16 elements (SwiGLU epilogue)
};

// RMSNorm folded into the activation load: A = h = bf16(r * inv * gamma), with
// inv = 1 / sqrt(sum(ssq) / K + eps) from the per-chunk sums of squares of the
// residual rows (the same arithmetic, in the same order, as the standalone
// normalisation, so h is bitwise the same).
struct NormIn {
    const uint16_t* resid;    // [M][K] bf16
    const uint16_t* gamma;    // [K] bf16
    const float* ssq;         // [M][nch]
    int nch;
    float eps;
};

// Modes: NORM = the activations are h = bf16(rmsnorm(resid) * gamma), formed
// in registers from the residual rows and gamma as each group is consumed;
// SWIGLU = the matrix holds gate and up rows interleaved per 64-row tile
// (rows 64 t .. +32: gate features 32 t .. +32; rows 64 t + 32 .. +32: the up
// rows of the same features) and the workgroup, which then covers all of K
// (S_grid == 1), writes y[m][f] = bf16(silu(gate) * up) directly.
template <bool NORM, bool SWIGLU>
__global__ __launch_bounds__(256) void w4_gemm_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                      const u32x4* __restrict__ wpk,
                                                      const uint16_t* __restrict__ spk, void* __restrict__ y,
                                                      int64_t ldy, int ydt, int M, int N, int G, int S_wg,
                                                      int S_grid, float* __restrict__ part, int64_t Npad,
                                                      uint32_t kmask, uint32_t kmagic, GemmGroup grp, NormIn nrm) {
    __shared__ float red[4][16][64];     // [wavefront][4 nb + r][lane]
    if (grp.n_slots) {
        const int slot = blockIdx.z;
        if (slot >= __builtin_amdgcn_readfirstlane(*grp.n_slots)) return;
        const int e = __builtin_amdgcn_readfirstlane(grp.slot_expert[slot]);
        wpk += (int64_t)e * grp.w_estride;
        spk += (int64_t)e * grp.s_estride;
        x += (int64_t)slot * grp.x_sstride;
        part += (int64_t)slot * grp.p_sstride;
        y = SWIGLU ? (void*)((uint16_t*)y + (int64_t)slot * grp.y_sstride) : (void*)part;
    }
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, kq = lane >> 4, i = lane & 15;
    const int t = blockIdx.x;
    const int S = S_wg * S_grid;
    const int s_idx = blockIdx.y * S_wg + wv;
    const int g0 = s_idx * G / S;               // S * G < 2^31: 32-bit division
    const int g1 = (s_idx + 1) * G / S;
    const int K = G * 64;
    const uint32_t magic_v = kmagic;  // lives in a VGPR for and_or()
    const int xr = i < M ? i : M - 1;  // A rows i >= M feed output rows that are never stored
    if (NORM) {                        // A rows: the residual rows (row stride K)
        x = nrm.resid;
        ldx = K;
    }

    // per-lane streams, advanced by one group per step
    const u32x4* wbase = wpk + (int64_t)t * G * 128 + lane;                  // + g * 128 (+ 64: second half)
    const uint2* sbase = (const uint2*)spk + (int64_t)t * G * 16 + i;         // + g * 16
    const u32x4* xbase = (const u32x4*)(x + (int64_t)xr * ldx) + kq;          // + g * 8 (+ 4: k half 1)
    const u32x4* gbase = (const u32x4*)nrm.gamma + kq;                        // NORM: + g * 8 (+ 4)

    f32x4 acc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // NORM, part 1: the per-chunk sums of squares of the residual rows (chunk
    // = lane; row and chunk indexes clamped rather than the loads predicated,
    // so that no branch separates them from their use) are requested before
    // the weights.  Loads complete in issue order: waiting for these does not
    // wait for the weight stream behind them.
    float sv[GEMM_MAX_M];
    if (NORM) {
        const int lc = lane < nrm.nch ? lane : nrm.nch - 1;
#pragma unroll
        for (int m = 0; m < GEMM_MAX_M; ++m) sv[m] = nrm.ssq[(int64_t)(m < M ? m : M - 1) * nrm.nch + lc];
    }
    __builtin_amdgcn_sched_barrier(0);

    // PF groups in flight per lane, each in its own registers: the main loop
    // consumes buffer j and refills it with the group PF further on (clamped to
    // the slice's last group, so every load address is valid and the loop body
    // has no branches); the last < PF groups are consumed after the loop.
    const int glast = g1 > g0 ? g1 - 1 : g0;
    u32x4 bw0[PF], bw1[PF], bx0[PF], bx1[PF], bg0[PF], bg1[PF];
    uint2 bs[PF];
    auto issue = [&](int j, int gi) {
        bw0[j] = __builtin_nontemporal_load(wbase + (int64_t)gi * 128);
        bw1[j] = __builtin_nontemporal_load(wbase + (int64_t)gi * 128 + 64);
        bx0[j] = xbase[(int64_t)gi * 8];
        bx1[j] = xbase[(int64_t)gi * 8 + 4];
        if (NORM) {
            bg0[j] = gbase[(int64_t)gi * 8];
            bg1[j] = gbase[(int64_t)gi * 8 + 4];
        }
        bs[j] = sbase[(int64_t)gi * 16];
    };
    // g0 < G always (S <= G), so these addresses are valid even for an empty slice
#pragma unroll
    for (int j = 0; j < PF; ++j) issue(j, min(g0 + j, glast));
    __builtin_amdgcn_sched_barrier(0);

    // NORM, part 2: the chunk sums (at most 64: K <= 64 * NORM_CHUNK) added in
    // chunk order (lane values read back one by one), then this lane's row
    // factor, computed as the standalone normalisation computes it
    float inv = 1.0f;
    if (NORM) {
        float tot[GEMM_MAX_M];
#pragma unroll
        for (int m = 0; m < GEMM_MAX_M; ++m) tot[m] = 0.0f;
        for (int e = 0; e < nrm.nch; ++e)
#pragma unroll
            for (int m = 0; m < GEMM_MAX_M; ++m)
                tot[m] += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sv[m]), e));
        float tr = tot[0];
#pragma unroll
        for (int m = 1; m < GEMM_MAX_M; ++m) tr = xr == m ? tot[m] : tr;
        inv = 1.0f / sqrtf(tr / (float)K + nrm.eps);
    }

    auto consume = [&](int j) {
        if (NORM) {
            bx0[j] = norm8(bx0[j], bg0[j], inv);
            bx1[j] = norm8(bx1[j], bg1[j], inv);
        }
        gemm_group(bw0[j], bw1[j], bx0[j], bx1[j], bs[j], kmask, magic_v, acc);
    };
    if (g0 < g1) {
        int g = g0;
        for (; g + PF <= g1; g += PF) {
#pragma unroll
            for (int j = 0; j < PF; ++j) {
                consume(j);
                // keep the refill right after its buffer's last use: the
                // scheduler would otherwise sink all refills to the loop end
                __builtin_amdgcn_sched_barrier(0);
                issue(j, min(g + j + PF, glast));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int j = 0; j < PF - 1; ++j)
            if (g + j < g1) consume(j);
    }

    // Reduce the S_wg slices of this workgroup in slice order.
    if (S_wg > 1) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wv][nb * 4 + r][lane] = acc[nb][r];
        __syncthreads();
        if (wv != 0) return;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = red[0][nb * 4 + r][lane];
                for (int w = 1; w < S_wg; ++w) v += red[w][nb * 4 + r][lane];
                acc[nb][r] = v;
            }
    }

    // lane (kq, i) holds rows m = 4 kq + r of columns n = 64 t + 16 nb + i
    if (SWIGLU) {
        const int F = N / 2;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * kq + r;
            if (m >= M) break;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int f = t * 32 + nb * 16 + i;
                const float gt = acc[nb][r], up = acc[nb + 2][r];
                const float sg = gt / (1.0f + expf(-gt));
                if (f < F) ((uint16_t*)y)[m * ldy + f] = f32_to_bf16(sg * up);
            }
        }
        return;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = 4 * kq + r;
        if (m >= M) break;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int n = t * 64 + nb * 16 + i;
            if (S_grid == 1) {
                if (n < N) {
                    if (ydt == VW4_F32) ((float*)y)[m * ldy + n] = acc[nb][r];
                    else ((uint16_t*)y)[m * ldy + n] = f32_to_bf16(acc[nb][r]);
                }
            } else {
                // split across workgroups: fp32 partials, summed by the consumer
                part[((int64_t)blockIdx.y * M + m) * Npad + n] = acc[nb][r];
            }
        }
    }
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
};

// Split of K over wavefronts: about 2048 wavefronts (two per SIMD), at least
// four groups per wavefront and at most 8 partial slices; one wavefront per
// workgroup, except that very wide matrices (one slice) pair two wavefronts
// per tile through LDS.  Measured on MI355X over the 27B-class shapes: more
// wavefronts only add per-wavefront start-up and partial traffic.  Depends on
// (N, K) only.  slots: matrices per launch (grouped launches spread the
// wavefront target over all of them).
static GemmPlan plan_gemm(int M, int N, int K, int slots = 1) {
    GemmPlan p;
    p.G = K / 64;
    p.ntiles = (N + 63) / 64;
    p.Npad = (int64_t)p.ntiles * 64;
    const int target_waves = 2048;
    const int units = p.ntiles * slots;
    int S = (target_waves + units - 1) / units;
    int maxS = p.G / 4 < 8 ? p.G / 4 : 8;
    if (maxS < 1) maxS = 1;
    if (S > maxS) S = maxS;
    if (S < 1) S = 1;
    p.S_wg = 1;
    p.S_grid = S;
    if (S == 1 && units >= 1024 && p.G >= 8) {
        // Many tiles, one slice each: S_wg wavefronts per workgroup split K.
        // S_wg in 2..4 is chosen so that the last round of resident workgroups
        // is as full as possible (units / resident just below a whole number):
        // the kernel holds 4 wavefronts per SIMD (16 per CU) and at most 10
        // workgroups per CU (16 KiB of static LDS each).  Measured on the
        // 151936 x 5120 LM head: 3 per workgroup (1.85 rounds) is 3-5% faster
        // than 2 (1.16 rounds) and 4 (2.32 rounds).
        const int ncu = device_cus();
        double best = -1.0;
        for (int w = 2; w <= 4; ++w) {
            const int per_cu = 16 / w < 10 ? 16 / w : 10;
            const double rounds = (double)units / ((double)per_cu * ncu);
            const double fill = rounds / ceil(rounds);
            if (fill > best + 1e-9) {
                best = fill;
                p.S_wg = w;
            }
        }
    }
    if (const char* e = getenv("VW4_GEMM_SPLIT")) {
        int a = 0, b = 0;
        if (sscanf(e, "%d,%d", &a, &b) == 2 && a >= 1 && a <= 4 && b >= 1 && a * b <= p.G) {
            p.S_wg = a;
            p.S_grid = b;
        }
    }
    p.ws_bytes = 0;
    if (p.S_grid > 1) p.ws_bytes = ((size_t)p.S_grid * M * p.Npad * 4 + 255) / 256 * 256;
    return p;
}

template <bool NORM, bool SWIGLU>
static int launch_kernel(const GemmPlan& p, int slots, hipStream_t st, const uint16_t* x, int64_t ldx,
                         const uint8_t* w, const uint16_t* s, void* y, int64_t ldy, int ydt, int M, int N, float* part,
                         const GemmGroup& grp, const NormIn& nrm) {
    hipLaunchKernelGGL((w4_gemm_kernel<NORM, SWIGLU>), dim3(p.ntiles, p.S_grid, slots), dim3(64 * p.S_wg), 0, st,
                       x, ldx, (const u32x4*)w, s, y, ldy, ydt, M, N, p.G, p.S_wg, p.S_grid, part, p.Npad,
                       0x000F000Fu, 0x43004300u, grp, nrm);
    return VW4_OK;
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
    VW4_REQUIRE(aligned(w, 16) && aligned(s, 8), VW4_EINVAL,
                "w4_skinny_gemm: packed codes must be 16-byte and packed scales 8-byte aligned");
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
    const int rc = launch_kernel<false, false>(p, 1, st, x, ldx, w, s, y, ldy, ydt, M, N, part, GemmGroup{},
                                               NormIn{});
    if (rc) return rc;
    if (p.S_grid > 1)
        hipLaunchKernelGGL(w4_gemm_reduce_kernel, dim3(p.ntiles, M), dim3(64), 0, st, part, p.S_grid, M, p.Npad, N,
                           y, ldy, ydt);
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
    VW4_REQUIRE(aligned(w, 16) && aligned(s, 8) && aligned(part, 4), VW4_EINVAL,
                "w4_skinny_gemm_partials: misaligned pointer");
    const GemmPlan p = plan_gemm(M, N, K, max_slots);
    // S_grid == 1 writes the product straight into part[0] with row stride Npad
    const int rc = launch_kernel<false, false>(p, max_slots, st, x, ldx, w, s, part, p.Npad, VW4_F32, M, N, part,
                                               grp, NormIn{});
    if (rc) return rc;
    return check_launch("w4_skinny_gemm_partials");
}

// The partials form with the activations normalised on the fly:
// h = bf16(rmsnorm(resid) * gamma) (sums of squares from vw4_add_sumsq).
int gemm_rmsnorm_partials(const uint16_t* resid, const uint16_t* gamma, const float* ssq, float eps,
                          const uint8_t* w, const uint16_t* s, float* part, int M, int N, int K, hipStream_t st) {
    VW4_REQUIRE(M >= 1 && M <= GEMM_MAX_M && N >= 1 && K >= 64 && K % 64 == 0 && K <= NORM_MAX_K, VW4_EINVAL,
                "w4_skinny_gemm_rmsnorm_partials: bad shape M=%d N=%d K=%d (K <= %d)", M, N, K, NORM_MAX_K);
    VW4_REQUIRE(resid && gamma && ssq && w && s && part, VW4_EINVAL, "w4_skinny_gemm_rmsnorm_partials: null pointer");
    VW4_REQUIRE(aligned(resid, 16) && aligned(gamma, 16) && aligned(w, 16) && aligned(s, 8) && aligned(part, 4),
                VW4_EINVAL, "w4_skinny_gemm_rmsnorm_partials: misaligned pointer");
    VW4_REQUIRE(eps >= 0.0f, VW4_EINVAL, "w4_skinny_gemm_rmsnorm_partials: eps must be >= 0");
    const GemmPlan p = plan_gemm(M, N, K);
    const NormIn nrm{resid, gamma, ssq, (K + NORM_CHUNK - 1) / NORM_CHUNK, eps};
    const int rc = launch_kernel<true, false>(p, 1, st, nullptr, K, w, s, part, p.Npad, VW4_F32, M, N, part,
                                              GemmGroup{}, nrm);
    if (rc) return rc;
    return check_launch("w4_skinny_gemm_rmsnorm_partials");
}

// SwiGLU epilogue: one slice of K per tile, S_wg wavefronts per workgroup.
// One wavefront per tile as soon as the tiles alone give one per CU: measured
// on MI355X at M = 4, gate|up 34816 x 5120 (544 tiles) takes 21.5 us with one
// wavefront per tile against 24.7 with four (the LDS reduction and the
// uneven 2-3 four-wavefront workgroups per CU cost more than the longer
// per-wavefront K stream), and the grouped 30 x 1536 x 2048 (720 tiles) 12.1
// against 15.0 with three.  Fewer tiles: up to 4 wavefronts split K.
static GemmPlan plan_swiglu(int N, int K, int slots) {
    GemmPlan p;
    p.G = K / 64;
    p.ntiles = (N + 63) / 64;
    p.Npad = (int64_t)p.ntiles * 64;
    const int units = p.ntiles * slots;
    const int ncu = device_cus();
    int swg = (ncu + units - 1) / units;
    if (swg > 4) swg = 4;
    if (swg > p.G) swg = p.G;
    p.S_wg = swg < 1 ? 1 : swg;
    p.S_grid = 1;
    p.ws_bytes = 0;
    return p;
}

int gemm_swiglu(const uint16_t* x, int64_t ldx, const NormIn* nrm, const uint8_t* w, const uint16_t* s, uint16_t* a,
                int64_t lda, int M, int F, int K, hipStream_t st, const GemmGroup& grp, int slots) {
    VW4_REQUIRE(M >= 1 && M <= GEMM_MAX_M && F >= 32 && F % 32 == 0 && K >= 64 && K % 64 == 0 && K <= 65536,
                VW4_EINVAL, "w4 GEMM + SwiGLU: bad shape M=%d F=%d K=%d (F must be a multiple of 32)", M, F, K);
    VW4_REQUIRE(w && s && a && lda >= F, VW4_EINVAL, "w4 GEMM + SwiGLU: bad output or null pointer");
    VW4_REQUIRE(aligned(w, 16) && aligned(s, 8) && aligned(a, 2), VW4_EINVAL, "w4 GEMM + SwiGLU: misaligned pointer");
    const GemmPlan p = plan_swiglu(2 * F, K, slots);
    int rc;
    if (nrm) {
        VW4_REQUIRE(nrm->resid && nrm->gamma && nrm->ssq && aligned(nrm->resid, 16) && aligned(nrm->gamma, 16),
                    VW4_EINVAL, "w4 GEMM + SwiGLU: bad normalisation inputs");
        VW4_REQUIRE(K <= NORM_MAX_K, VW4_EINVAL, "w4 GEMM + SwiGLU: normalised rows need K <= %d", NORM_MAX_K);
        rc = launch_kernel<true, true>(p, slots, st, nullptr, K, w, s, a, lda, VW4_BF16, M, 2 * F, nullptr, grp,
                                       *nrm);
    } else {
        VW4_REQUIRE(x && ldx >= K && ldx % 8 == 0 && aligned(x, 16), VW4_EINVAL,
                    "w4 GEMM + SwiGLU: x needs ldx >= K, ldx %% 8 == 0 and 16-byte alignment");
        rc = launch_kernel<false, true>(p, slots, st, x, ldx, w, s, a, lda, VW4_BF16, M, 2 * F, nullptr, grp,
                                        NormIn{});
    }
    if (rc) return rc;
    return check_launch("w4 GEMM + SwiGLU");
}

int grouped_gemm_partials(const uint16_t* x, int64_t ldx, int64_t x_sstride, const uint8_t* w_bank,
                          int64_t w_estride_bytes, const uint16_t* s_bank, int64_t s_estride, const int32_t* slot_expert,
                          const int32_t* n_slots, int max_slots, float* part, int64_t p_sstride, int M, int N, int K,
                          hipStream_t st) {
    VW4_REQUIRE(slot_expert && n_slots && max_slots >= 1 && max_slots <= 65535, VW4_EINVAL,
                "w4_grouped_gemm: bad slot arguments");
    VW4_REQUIRE(w_estride_bytes % 16 == 0 && w_estride_bytes > 0 && s_estride > 0 && s_estride % 4 == 0, VW4_EINVAL,
                "w4_grouped_gemm: expert strides must be positive, weights 16-byte and scales 8-byte multiples");
    VW4_REQUIRE(x_sstride % 8 == 0 && x_sstride >= 0 && p_sstride >= 0, VW4_EINVAL,
                "w4_grouped_gemm: bad slot strides");
    GemmGroup g{};
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

int w4_skinny_gemm_rmsnorm_partials(const uint16_t* resid, const uint16_t* gamma, const void* norm_ws, float eps,
                                    const uint8_t* w_packed, const uint16_t* scales_packed, float* part, int32_t M,
                                    int32_t N, int32_t K, void* stream) {
    return vw4::gemm_rmsnorm_partials(resid, gamma, (const float*)norm_ws, eps, w_packed, scales_packed, part, M, N,
                                      K, (hipStream_t)stream);
}

int w4_skinny_gemm_rmsnorm_swiglu(const uint16_t* resid, const uint16_t* gamma, const void* norm_ws, float eps,
                                  const uint8_t* w_packed, const uint16_t* scales_packed, uint16_t* a, int64_t lda,
                                  int32_t M, int32_t F, int32_t K, void* stream) {
    const vw4::NormIn nrm{resid, gamma, (const float*)norm_ws, (K + vw4::NORM_CHUNK - 1) / vw4::NORM_CHUNK, eps};
    VW4_REQUIRE(eps >= 0.0f, VW4_EINVAL, "w4_skinny_gemm_rmsnorm_swiglu: eps must be >= 0");
    return vw4::gemm_swiglu(nullptr, K, &nrm, w_packed, scales_packed, a, lda, M, F, K, (hipStream_t)stream,
                            vw4::GemmGroup{}, 1);
}

int w4_skinny_gemm_swiglu(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, const uint16_t* scales_packed,
                          uint16_t* a, int64_t lda, int32_t M, int32_t F, int32_t K, void* stream) {
    return vw4::gemm_swiglu(x, ldx, nullptr, w_packed, scales_packed, a, lda, M, F, K, (hipStream_t)stream,
                            vw4::GemmGroup{}, 1);
}

int w4_grouped_gemm_swiglu(const uint16_t* x, int64_t ldx, int64_t x_sstride, const uint8_t* w_bank,
                           int64_t w_estride, const uint16_t* s_bank, int64_t s_estride, const int32_t* slot_expert,
                           const int32_t* n_slots, int32_t max_slots, uint16_t* a, int64_t a_sstride, int32_t M,
                           int32_t F, int32_t K, void* stream) {
    VW4_REQUIRE(slot_expert && n_slots && max_slots >= 1 && max_slots <= 65535, VW4_EINVAL,
                "w4_grouped_gemm_swiglu: bad slot arguments");
    VW4_REQUIRE(w_estride % 16 == 0 && w_estride > 0 && s_estride > 0 && s_estride % 4 == 0, VW4_EINVAL,
                "w4_grouped_gemm_swiglu: expert strides must be positive, weights 16-byte and scales 8-byte multiples");
    VW4_REQUIRE(x_sstride % 8 == 0 && x_sstride >= 0 && a_sstride >= (int64_t)M * F, VW4_EINVAL,
                "w4_grouped_gemm_swiglu: bad slot strides");
    vw4::GemmGroup g{};
    g.slot_expert = slot_expert;
    g.n_slots = n_slots;
    g.w_estride = w_estride / 16;
    g.s_estride = s_estride;
    g.x_sstride = x_sstride;
    g.y_sstride = a_sstride;
    return vw4::gemm_swiglu(x, ldx, nullptr, w_bank, s_bank, a, F, M, F, K, (hipStream_t)stream, g, max_slots);
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

// ---------------------------------------------------------------------------
// The allocation-free form of w4_skinny_gemm.  Its split-K partial sums live
// in a file-scope device array instead of a caller workspace: every GPU the
// library runs on holds one copy of VW4_NOALLOC_SCRATCH_BYTES until the
// process ends.  The largest split-K workspace the plan asks for at M <= 8 is
// 8 * 8 * 32768 * 4 bytes (S * Npad stays below 4096 * 64), so every shape
// the plan produces fits.  Host code never passes the array's name to a
// kernel: it is a host-side stand-in; the device address of each GPU's copy
// comes from hipGetSymbolAddress, taken once per device on the first call
// made with that device current.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[VW4_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex noalloc_mu;
void* noalloc_ptr[NOALLOC_MAX_DEVICES];

// Device address of the current device's scratch copy, or nullptr (with the
// error message set) if it cannot be had.
void* noalloc_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) {
        vw4::set_error("w4_skinny_gemm_noalloc: no current device (or device index >= %d)", NOALLOC_MAX_DEVICES);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(noalloc_mu);
    if (!noalloc_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            vw4::set_error("w4_skinny_gemm_noalloc: hipGetSymbolAddress of the scratch array failed on device %d: %s",
                           dev, hipGetErrorString(e));
            return nullptr;
        }
        noalloc_ptr[dev] = p;
    }
    return noalloc_ptr[dev];
}
}  // namespace

extern "C" {

size_t vw4_noalloc_scratch_bytes(void) { return VW4_NOALLOC_SCRATCH_BYTES; }

int w4_skinny_gemm_noalloc(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, const uint16_t* scales_packed,
                           void* y, int64_t ldy, int32_t y_dtype, int32_t M, int32_t N, int32_t K, void* stream) {
    const size_t need = vw4::gemm_ws_bytes(M, N, K);
    VW4_REQUIRE(need <= VW4_NOALLOC_SCRATCH_BYTES, VW4_EWORKSPACE,
                "w4_skinny_gemm_noalloc: the split-K partials need %zu bytes, more than the %zu-byte scratch array",
                need, (size_t)VW4_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (need) {
        ws = noalloc_scratch();
        if (!ws) return VW4_EHIP;
    }
    return vw4::gemm_dispatch(x, ldx, w_packed, scales_packed, y, ldy, y_dtype, M, N, K, ws,
                              need ? (size_t)VW4_NOALLOC_SCRATCH_BYTES : 0, (hipStream_t)stream);
}

}  // extern "C"
