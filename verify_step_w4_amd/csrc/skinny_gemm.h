// skinny_gemm.h — the skinny GEMM for the verify rows (M = 1..8), shared by
// every weight format (internal to libvw4, not public).
//
// hazakura.dev, "mtplx——M5 Maxで63tok/s…", section "4層のアーキテクチャ", Layer 0:
// the verify pass is a matmul with a handful of rows (M = 3..6) that needed its
// own shader; gist.science, "BaseRT: …", section "メソドロジー": decode GEMVs
// dequantise inside the inner loop so weights are never materialised, with one
// GEMV per quantisation format (Q2 ... Q8).
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
//    64-element group, lane l = 16 kq + i loads 16-byte words of each code
//    plane, each part of a contiguous wavefront load: in the 4-bit plane
//    layout, the 8 code nibbles of rows 16 nb + i (nb = 0..3) at k = 32 s +
//    8 kq .. +8 (s = 0, 1), exactly its B operand (W^T, column = row of W) of
//    v_mfma_f32_16x16x32_bf16.
//  * The A operand is the activations: lane l supplies x[i][32 s + 8 kq .. +8]
//    (for i >= M any valid row: those output rows are not stored), read once
//    per group from L2.  D[m][n] lands in lane (kq, i) as rows m = 4 kq .. +4,
//    column n = 16 nb + i.
//  * Dequantisation in registers: ((word >> 4j) & 0x000F000F) | 0x43004300 is
//    a pair of bf16 values 128 + u (one v_bitop3 per pair); a 2-bit field the
//    same with mask 0x00030003.  The constant is removed by one more product
//    per group: the C input of the row blocks' products is x . (-offset), which
//    the matrix cores form from the same A operand.  Then acc += scale[n] * D.
//  * Formats are plane decoders: W4 (one 4-bit plane) below; the others in
//    skinny_formats.h.  Everything else -- lane mapping, pipeline, split plan,
//    epilogues, reduction -- is one kernel template.
//  * Split K: S_wg wavefronts of a workgroup take consecutive K slices of the
//    same tile and are reduced through LDS; when the tiles are too few to fill
//    the chip, S_grid workgroups per tile write fp32 partials and the consumer
//    (or a second launch) sums them in slice order.  Every summation order
//    depends only on (N, K): results are bitwise reproducible and row m of an
//    M-row call equals the one-row call (the matrix core computes each output
//    from its own row of A).
#pragma once

#include "common.h"

namespace vw4 {
namespace sg {

constexpr int MAX_M = 8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
constexpr int PF = 4;                          // groups in flight per lane (default)
constexpr int NORM_MAX_K = 64 * NORM_CHUNK;    // NORM mode: at most 64 chunk sums per row

// (v & mask) | magic in one instruction: gfx950's three-input bitwise op with
// truth table 0xEA = (A & B) | C.  gfx9 VOP3 encodings take no literal
// constants and at most one SGPR, so the mask comes in an SGPR and the magic
// in a VGPR (the compiler would otherwise emit a v_and / v_or pair).
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t mask_s, uint32_t magic_v) {
    return __builtin_amdgcn_bitop3_b32(v, mask_s, magic_v, 0xEA);
}

// 8 code nibbles (4-bit plane word) -> the 8 bf16 values 128 + u of one MFMA operand.
__device__ __forceinline__ bf16x8 nib8(uint32_t w, uint32_t kmask, uint32_t magic_v) {
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

// The constant operand: 8 copies of one bf16 value (pair = two copies).
__device__ __forceinline__ bf16x8 pair8(uint32_t pair) {
    const u32x4 q = {pair, pair, pair, pair};
    return __builtin_bit_cast(bf16x8, q);
}

__device__ __forceinline__ void scales4(uint2 sc, float (&f)[4]) {
    f[0] = f16_bits_to_f32((uint16_t)(sc.x & 0xffffu));
    f[1] = f16_bits_to_f32((uint16_t)(sc.x >> 16));
    f[2] = f16_bits_to_f32((uint16_t)(sc.y & 0xffffu));
    f[3] = f16_bits_to_f32((uint16_t)(sc.y >> 16));
}

// Base pointers of a matrix's code planes (p1 unused by one-plane formats).
struct Planes {
    const u32x4* p0;
    const u32x4* p1;
};

// Per-format options, read through these traits: PF_GROUPS (groups in flight
// per lane, default PF) and NO_SCALES (a format without group scales: the
// kernel loads none and the decoder ignores its scale argument).
template <class...>
using void_t = void;
template <class F, class = void>
struct FmtPF {
    static constexpr int v = PF;
};
template <class F>
struct FmtPF<F, void_t<decltype(F::PF_GROUPS)>> {
    static constexpr int v = F::PF_GROUPS;
};
template <class F, class = void>
struct FmtScaled {
    static constexpr bool v = true;
};
template <class F>
struct FmtScaled<F, void_t<decltype(F::NO_SCALES)>> {
    static constexpr bool v = false;
};

// ---------------------------------------------------------------------------
// Plane decoders.  Each gives NW, the 16-byte words a lane loads per group;
// base(), the lane's word pointers of tile t (G groups per row); load(), the
// words of group g; group(), acc += scale * sum_k x * c for the lane's four
// row blocks from those words and the A operands a0 / a1 (k halves 0 / 1);
// expert(), the planes of expert e of a stacked bank (w_estride: the 4-bit
// plane's stride in 16-byte units).
// ---------------------------------------------------------------------------

// W4: c in [-7, 7] stored as u = c + 8 in one 4-bit plane (the packed layout of
// vw4_w4_pack): word 0 holds row blocks 0, 1, word 1 row blocks 2, 3, dword
// 2 nb' + s of a word = k half s of its row block nb'.  The folded offset:
// 136 = 128 + 8.
struct FmtW4 {
    static constexpr int NW = 2;
    static constexpr uint32_t NEG_PAIR = 0xC308C308u;   // two bf16 -136.0
    __device__ static void base(const Planes& P, int64_t t, int G, int lane, const u32x4*& b0, const u32x4*& b1) {
        b0 = P.p0 + t * G * 128 + lane;
        b1 = b0;
    }
    __device__ static void load(u32x4 (&w)[NW], const u32x4* b0, const u32x4*, int64_t g) {
        w[0] = __builtin_nontemporal_load(b0 + g * 128);
        w[1] = __builtin_nontemporal_load(b0 + g * 128 + 64);
    }
    __device__ static void group(const u32x4 (&w)[NW], bf16x8 a0, bf16x8 a1, uint2 sc, uint32_t kmask,
                                 uint32_t magic_v, f32x4 (&acc)[4]) {
        const bf16x8 neg = pair8(NEG_PAIR);
        f32x4 off = {0.f, 0.f, 0.f, 0.f};
        off = mfma16(a0, neg, off);
        off = mfma16(a1, neg, off);
        const u32x4 wa = w[0], wb = w[1];
        f32x4 d[4];
        d[0] = mfma16(a1, nib8(wa.y, kmask, magic_v), mfma16(a0, nib8(wa.x, kmask, magic_v), off));
        d[1] = mfma16(a1, nib8(wa.w, kmask, magic_v), mfma16(a0, nib8(wa.z, kmask, magic_v), off));
        d[2] = mfma16(a1, nib8(wb.y, kmask, magic_v), mfma16(a0, nib8(wb.x, kmask, magic_v), off));
        d[3] = mfma16(a1, nib8(wb.w, kmask, magic_v), mfma16(a0, nib8(wb.z, kmask, magic_v), off));
        float f[4];
        scales4(sc, f);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[nb][r] = fmaf(f[nb], d[nb][r], acc[nb][r]);
    }
    __host__ __device__ static Planes expert(Planes P, int64_t e, int64_t w_estride) {
        P.p0 += e * w_estride;
        return P;
    }
};

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
    int64_t w_estride;        // u32x4 units of the 4-bit plane
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
template <class Fmt, bool NORM, bool SWIGLU>
__global__ __launch_bounds__(256) void skinny_gemm_kernel(const uint16_t* __restrict__ x, int64_t ldx, Planes planes,
                                                          const uint16_t* __restrict__ spk, void* __restrict__ y,
                                                          int64_t ldy, int ydt, int M, int N, int G, int S_wg,
                                                          int S_grid, float* __restrict__ part, int64_t Npad,
                                                          uint32_t kmask, uint32_t kmagic, GemmGroup grp,
                                                          NormIn nrm) {
    constexpr int PFL = FmtPF<Fmt>::v;
    __shared__ float red[4][16][64];     // [wavefront][4 nb + r][lane]
    if (grp.n_slots) {
        const int slot = blockIdx.z;
        if (slot >= __builtin_amdgcn_readfirstlane(*grp.n_slots)) return;
        const int e = __builtin_amdgcn_readfirstlane(grp.slot_expert[slot]);
        planes = Fmt::expert(planes, e, grp.w_estride);
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
    const u32x4 *wb0, *wb1;
    Fmt::base(planes, t, G, lane, wb0, wb1);
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
    float sv[MAX_M];
    if (NORM) {
        const int lc = lane < nrm.nch ? lane : nrm.nch - 1;
#pragma unroll
        for (int m = 0; m < MAX_M; ++m) sv[m] = nrm.ssq[(int64_t)(m < M ? m : M - 1) * nrm.nch + lc];
    }
    __builtin_amdgcn_sched_barrier(0);

    // PFL groups in flight per lane, each in its own registers: the main loop
    // consumes buffer j and refills it with the group PFL further on (clamped to
    // the slice's last group, so every load address is valid and the loop body
    // has no branches); the last < PFL groups are consumed after the loop.
    const int glast = g1 > g0 ? g1 - 1 : g0;
    u32x4 bw[PFL][Fmt::NW], bx0[PFL], bx1[PFL], bg0[PFL], bg1[PFL];
    uint2 bs[PFL];
    auto issue = [&](int j, int gi) {
        Fmt::load(bw[j], wb0, wb1, gi);
        bx0[j] = xbase[(int64_t)gi * 8];
        bx1[j] = xbase[(int64_t)gi * 8 + 4];
        if (NORM) {
            bg0[j] = gbase[(int64_t)gi * 8];
            bg1[j] = gbase[(int64_t)gi * 8 + 4];
        }
        if (FmtScaled<Fmt>::v) bs[j] = sbase[(int64_t)gi * 16];
        else bs[j] = uint2{0u, 0u};
    };
    // g0 < G always (S <= G), so these addresses are valid even for an empty
    // slice.  The prologue issues group by group, in the order the loop
    // refills: the wait counts at the loop head then leave PFL - 1 groups in
    // flight.  (Prologue loads split around a branch -- weight words in one
    // block, activations and scales in the next -- made the compiler wait for
    // most of the prefetch at every loop head: 14 % slower on the 27B layer.)
#pragma unroll
    for (int j = 0; j < PFL; ++j) issue(j, min(g0 + j, glast));
    __builtin_amdgcn_sched_barrier(0);

    // NORM, part 2: the chunk sums (at most 64: K <= 64 * NORM_CHUNK) added in
    // chunk order (lane values read back one by one), then this lane's row
    // factor, computed as the standalone normalisation computes it
    float inv = 1.0f;
    if (NORM) {
        float tot[MAX_M];
#pragma unroll
        for (int m = 0; m < MAX_M; ++m) tot[m] = 0.0f;
        for (int e = 0; e < nrm.nch; ++e)
#pragma unroll
            for (int m = 0; m < MAX_M; ++m)
                tot[m] += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sv[m]), e));
        float tr = tot[0];
#pragma unroll
        for (int m = 1; m < MAX_M; ++m) tr = xr == m ? tot[m] : tr;
        inv = 1.0f / sqrtf(tr / (float)K + nrm.eps);
    }

    auto consume = [&](int j) {
        if (NORM) {
            bx0[j] = norm8(bx0[j], bg0[j], inv);
            bx1[j] = norm8(bx1[j], bg1[j], inv);
        }
        Fmt::group(bw[j], __builtin_bit_cast(bf16x8, bx0[j]), __builtin_bit_cast(bf16x8, bx1[j]), bs[j], kmask,
                   magic_v, acc);
    };
    // (an empty slice, g0 == g1, runs neither loop; no branch guards them, so
    // that the prologue's loads stay together ahead of the loop)
    int g = g0;
    for (; g + PFL <= g1; g += PFL) {
#pragma unroll
        for (int j = 0; j < PFL; ++j) {
            consume(j);
            // keep the refill right after its buffer's last use: the
            // scheduler would otherwise sink all refills to the loop end
            __builtin_amdgcn_sched_barrier(0);
            issue(j, min(g + j + PFL, glast));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int j = 0; j < PFL - 1; ++j)
        if (g + j < g1) consume(j);

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
static __global__ __launch_bounds__(64) void skinny_gemm_reduce_kernel(const float* __restrict__ part, int S_grid,
                                                                       int M, int64_t Npad, int N,
                                                                       void* __restrict__ y, int64_t ldy, int ydt) {
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

// Split of K over wavefronts (every format): about 2048 wavefronts (two per
// SIMD), at least four groups per wavefront and at most 8 partial slices;
// one wavefront per workgroup, except that very wide matrices (one slice)
// pair 2-4 wavefronts per tile through LDS.  Depends on (N, K) only.  slots:
// matrices per launch (grouped launches spread the wavefront target over all
// of them).  Defined in w4_gemm.hip.
GemmPlan plan_gemm(int M, int N, int K, int slots = 1);
// The plan of a gate|up GEMM with the SwiGLU epilogue (N = 2 F rows): one K slice
// per tile (S_grid == 1), S_wg wavefronts per workgroup.
GemmPlan plan_swiglu(int N, int K, int slots = 1);

// The plain call of any format: validated, one launch (plus the reduction
// launch of split plans).  w0 / w1: the format's planes (w1 unused for W4).
template <class Fmt>
int skinny_gemm_run(const char* name, const uint16_t* x, int64_t ldx, const uint8_t* w0, const uint8_t* w1,
                    const uint16_t* s, void* y, int64_t ldy, int ydt, int M, int N, int K, void* ws, size_t ws_bytes,
                    hipStream_t st) {
    VW4_REQUIRE(M >= 1 && M <= MAX_M, VW4_EINVAL, "%s: M=%d must be in [1, 8]", name, M);
    VW4_REQUIRE(N >= 1, VW4_EINVAL, "%s: N=%d must be >= 1", name, N);
    VW4_REQUIRE(K >= 64 && K % 64 == 0 && K <= 65536, VW4_EINVAL, "%s: K=%d must be a multiple of 64 in [64, 65536]",
                name, K);
    VW4_REQUIRE(x && w0 && w1 && s && y, VW4_EINVAL, "%s: null pointer", name);
    VW4_REQUIRE(ldx >= K && ldx % 8 == 0 && aligned(x, 16), VW4_EINVAL,
                "%s: x needs ldx >= K, ldx %% 8 == 0 and 16-byte alignment", name);
    VW4_REQUIRE(aligned(w0, 16) && aligned(w1, 16) && aligned(s, 8), VW4_EINVAL,
                "%s: packed codes must be 16-byte and packed scales 8-byte aligned", name);
    VW4_REQUIRE(ldy >= N, VW4_EINVAL, "%s: ldy=%lld < N=%d", name, (long long)ldy, N);
    VW4_REQUIRE(ydt == VW4_F32 || ydt == VW4_BF16, VW4_EINVAL, "%s: y_dtype must be VW4_F32 or VW4_BF16", name);
    VW4_REQUIRE(aligned(y, ydt == VW4_F32 ? 4 : 2), VW4_EINVAL, "%s: y misaligned", name);
    const GemmPlan p = plan_gemm(M, N, K);
    float* part = nullptr;
    if (p.ws_bytes) {
        VW4_REQUIRE(ws && ws_bytes >= p.ws_bytes && aligned(ws, 256), VW4_EWORKSPACE,
                    "%s: needs a 256-byte aligned workspace of %zu bytes", name, p.ws_bytes);
        part = (float*)ws;
    }
    const Planes P{(const u32x4*)w0, (const u32x4*)w1};
    hipLaunchKernelGGL((skinny_gemm_kernel<Fmt, false, false>), dim3(p.ntiles, p.S_grid, 1), dim3(64 * p.S_wg), 0, st,
                       x, ldx, P, s, y, ldy, ydt, M, N, p.G, p.S_wg, p.S_grid, part, p.Npad, 0x000F000Fu, 0x43004300u,
                       GemmGroup{}, NormIn{});
    if (p.S_grid > 1)
        hipLaunchKernelGGL(skinny_gemm_reduce_kernel, dim3(p.ntiles, M), dim3(64), 0, st, part, p.S_grid, M, p.Npad,
                           N, y, ldy, ydt);
    return check_launch(name);
}

// The partials form of any format: the main kernel only; part is the caller's
// [S_grid][M][Npad] fp32 buffer (S_grid == 1: the product, row stride Npad).
template <class Fmt>
int skinny_gemm_partials_run(const char* name, const uint16_t* x, int64_t ldx, const uint8_t* w0, const uint8_t* w1,
                             const uint16_t* s, float* part, int M, int N, int K, hipStream_t st,
                             const GemmGroup& grp = GemmGroup{}, int max_slots = 1) {
    VW4_REQUIRE(M >= 1 && M <= MAX_M, VW4_EINVAL, "%s: M=%d must be in [1, 8]", name, M);
    VW4_REQUIRE(N >= 1, VW4_EINVAL, "%s: N=%d must be >= 1", name, N);
    VW4_REQUIRE(K >= 64 && K % 64 == 0 && K <= 65536, VW4_EINVAL, "%s: K=%d must be a multiple of 64 in [64, 65536]",
                name, K);
    VW4_REQUIRE(x && w0 && w1 && s && part, VW4_EINVAL, "%s: null pointer", name);
    VW4_REQUIRE(ldx >= K && ldx % 8 == 0 && aligned(x, 16), VW4_EINVAL,
                "%s: x needs ldx >= K, ldx %% 8 == 0 and 16-byte alignment", name);
    VW4_REQUIRE(aligned(w0, 16) && aligned(w1, 16) && aligned(s, 8) && aligned(part, 4), VW4_EINVAL,
                "%s: misaligned pointer", name);
    const GemmPlan p = plan_gemm(M, N, K, max_slots);
    const Planes P{(const u32x4*)w0, (const u32x4*)w1};
    hipLaunchKernelGGL((skinny_gemm_kernel<Fmt, false, false>), dim3(p.ntiles, p.S_grid, max_slots),
                       dim3(64 * p.S_wg), 0, st, x, ldx, P, s, (void*)part, p.Npad, VW4_F32, M, N, p.G, p.S_wg,
                       p.S_grid, part, p.Npad, 0x000F000Fu, 0x43004300u, grp, NormIn{});
    return check_launch(name);
}

// Gate|up projection of any format with the SwiGLU in its epilogue: the
// matrix holds 2 F rows in the gate/up-interleaved order of the SWIGLU mode;
// a[m][f] = bf16(silu(g) * u), row stride lda >= F.
template <class Fmt>
int skinny_gemm_swiglu_run(const char* name, const uint16_t* x, int64_t ldx, const uint8_t* w0, const uint8_t* w1,
                           const uint16_t* s, uint16_t* a, int64_t lda, int M, int F, int K, hipStream_t st) {
    VW4_REQUIRE(M >= 1 && M <= MAX_M && F >= 32 && F % 32 == 0 && K >= 64 && K % 64 == 0 && K <= 65536, VW4_EINVAL,
                "%s: bad shape M=%d F=%d K=%d (F must be a multiple of 32)", name, M, F, K);
    VW4_REQUIRE(x && w0 && w1 && s && a && lda >= F, VW4_EINVAL, "%s: bad output or null pointer", name);
    VW4_REQUIRE(ldx >= K && ldx % 8 == 0 && aligned(x, 16), VW4_EINVAL,
                "%s: x needs ldx >= K, ldx %% 8 == 0 and 16-byte alignment", name);
    VW4_REQUIRE(aligned(w0, 16) && aligned(w1, 16) && aligned(s, 8) && aligned(a, 2), VW4_EINVAL,
                "%s: misaligned pointer", name);
    const GemmPlan p = plan_swiglu(2 * F, K, 1);
    const Planes P{(const u32x4*)w0, (const u32x4*)w1};
    hipLaunchKernelGGL((skinny_gemm_kernel<Fmt, false, true>), dim3(p.ntiles, 1, 1), dim3(64 * p.S_wg), 0, st, x,
                       ldx, P, s, (void*)a, lda, VW4_BF16, M, 2 * F, p.G, p.S_wg, p.S_grid, (float*)nullptr, p.Npad,
                       0x000F000Fu, 0x43004300u, GemmGroup{}, NormIn{});
    return check_launch(name);
}

}  // namespace sg
}  // namespace vw4
