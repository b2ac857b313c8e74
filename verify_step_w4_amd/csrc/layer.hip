// layer.hip — decoder-layer calls of the verify forward: residual add +
// RMSNorm, rotary embedding + KV-cache append, SwiGLU, grouped-query decode
// attention for the M verify rows (matrix cores).
//
// hazakura.dev, "mtplx——M5 Maxで63tok/s…", section "4層のアーキテクチャ", Layer 1:
// target and drafter share one checkpoint and its KV cache, and all drafts are
// scored in one forward pass of M = D + 1 rows.  gist.science, "BaseRT: …",
// section "メソドロジー": decode-step operator sequences are fused so that short
// kernels do not pay extra memory round trips and launches; attention is
// computed tile by tile with an online softmax (O(n) memory).
//
// Every call here consumes the split-K partial sums of the W4 GEMM that feeds
// it (sum over slices in slice order, fp32), so the GEMM needs no reduction
// launch of its own.  Rounding points: activations are stored as bf16 after
// every op (round to nearest even), arithmetic is fp32.
#include <math.h>
#include <stdlib.h>

#include "common.h"

namespace vw4 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4v;

// ---------------------------------------------------------------------------
// residual add + RMSNorm.  Chunk sums of squares: a chunk is NCOL = 256
// columns; lane l of one wavefront holds columns 4 l .. 4 l + 3 (zero past
// D), its value is v0^2 + v1^2 + v2^2 + v3^2 as the explicit fma chain below,
// and the wavefront adds the 64 lane values (wave_sum).  The total is the sum
// of the chunk sums in chunk order.  Every kernel forms them this way, so all
// paths give bitwise the same h:
//   - add_sumsq_kernel: resid += partials (bf16), chunk sums -> ws[m][chunk];
//     then rmsnorm_apply_kernel (or the W4 GEMM's NORM mode) applies them;
//   - add_rmsnorm_fused_kernel: one launch, out of place; every workgroup
//     forms all of its row's chunk sums itself (reading the whole row, mostly
//     from L2) and writes its own chunk of resid_out and h.
// ---------------------------------------------------------------------------
constexpr int NCOL = NORM_CHUNK;   // columns per chunk
constexpr int NMAXCH = 256; // chunks per row at most (D <= 65536)

__device__ __forceinline__ float chunk_sumsq(const float (&v)[4]) {
    return wave_sum(fmaf(v[3], v[3], fmaf(v[2], v[2], fmaf(v[1], v[1], v[0] * v[0]))));
}

// grid (ceil(D / NCOL), M), one wavefront per chunk.
__global__ __launch_bounds__(64) void add_sumsq_kernel(uint16_t* __restrict__ resid, const float* __restrict__ part,
                                                       int S, int64_t ldp, int M, int D, float* __restrict__ ssq) {
    const int ch = blockIdx.x, m = blockIdx.y, lane = threadIdx.x;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int d = ch * NCOL + 4 * lane + e;
        v[e] = 0.0f;
        if (d < D) {
            uint16_t* r = resid + (int64_t)m * D + d;
            v[e] = bf16_to_f32(*r);
            if (part) {
                v[e] += sum_parts(part, S, M, ldp, m, d);
                const uint16_t rb = f32_to_bf16(v[e]);
                *r = rb;
                v[e] = bf16_to_f32(rb);
            }
        }
    }
    const float q = chunk_sumsq(v);
    if (lane == 0) ssq[(int64_t)m * gridDim.x + ch] = q;
}

// One launch: resid_out = bf16(resid_in + sum_s part) and h for chunk
// blockIdx.x of row blockIdx.y.  nw = blockDim.x / 64 wavefronts, nw * CPW >=
// nch (at most CPW - 1 idle slots in all); wavefront w forms the sums of
// chunks w, w + nw, ... (CPW each).  All loads are issued before any is used
// (row and slice indexes clamped, no branches between them).  SS = number of
// partial slices (0: no add).
constexpr int FN_MAXW = 11, FN_MAXCH = 32;
template <int SS, int CPW>
__global__ __launch_bounds__(FN_MAXW * 64) void add_rmsnorm_fused_kernel(
    const uint16_t* __restrict__ rin, const float* __restrict__ part, int64_t ldp, const uint16_t* __restrict__ gamma,
    float eps, int M, int D, uint16_t* __restrict__ rout, uint16_t* __restrict__ h) {
    __shared__ float s_ssq[FN_MAXCH];
    const int ch = blockIdx.x, m = blockIdx.y, nch = gridDim.x;
    const int nw = blockDim.x >> 6;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int own_j = ch / nw, own_w = ch % nw;
    uint2 rr[CPW];
    f32x4 pp[CPW][SS > 0 ? SS : 1];
    // gamma of this workgroup's own chunk (used by its owner wavefront)
    const int gcol = ch * NCOL + 4 * lane < D ? ch * NCOL + 4 * lane : D - 4;
    const uint2 gg = *(const uint2*)(gamma + gcol);
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
        int c = w + nw * j;
        c = c < nch ? c : nch - 1;
        int col = c * NCOL + 4 * lane;
        col = col < D ? col : D - 4;                      // D % 4 == 0
        rr[j] = *(const uint2*)(rin + (int64_t)m * D + col);
#pragma unroll
        for (int s = 0; s < SS; ++s) pp[j][s] = *(const f32x4*)(part + ((int64_t)s * M + m) * ldp + col);
    }
    float own[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
        const int c = w + nw * j;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float x = bf16_to_f32((uint16_t)((e < 2 ? rr[j].x : rr[j].y) >> (16 * (e & 1))));
            if (SS > 0) {
                float sp = 0.0f;
#pragma unroll
                for (int s = 0; s < SS; ++s) sp += pp[j][s][e];
                x = bf16_to_f32(f32_to_bf16(x + sp));
            }
            v[e] = (c < nch && c * NCOL + 4 * lane + e < D) ? x : 0.0f;
        }
        const float q = chunk_sumsq(v);
        if (c < nch && lane == 0) s_ssq[c] = q;
        if (j == own_j && w == own_w) {
#pragma unroll
            for (int e = 0; e < 4; ++e) own[e] = v[e];
        }
    }
    __syncthreads();
    if (w != own_w) return;
    float tot = 0.0f;
    for (int c = 0; c < nch; ++c) tot += s_ssq[c];      // chunk order
    const float inv = 1.0f / sqrtf(tot / (float)D + eps);
    const int col = ch * NCOL + 4 * lane;
    if (col >= D) return;
    const float g[4] = {bf16_to_f32((uint16_t)(gg.x & 0xffffu)), bf16_to_f32((uint16_t)(gg.x >> 16)),
                        bf16_to_f32((uint16_t)(gg.y & 0xffffu)), bf16_to_f32((uint16_t)(gg.y >> 16))};
    uint2 ro, ho;
    ro.x = f32x2_to_bf16x2(own[0], own[1]);
    ro.y = f32x2_to_bf16x2(own[2], own[3]);
    ho.x = f32x2_to_bf16x2(own[0] * inv * g[0], own[1] * inv * g[1]);
    ho.y = f32x2_to_bf16x2(own[2] * inv * g[2], own[3] * inv * g[3]);
    *(uint2*)(rout + (int64_t)m * D + col) = ro;
    *(uint2*)(h + (int64_t)m * D + col) = ho;
}

// The MoE block's combine fused into the one-launch add + RMSNorm: the row
// added to resid_in is y[m][c] = sum_t weights[m][t] * (sum over the S slices
// of slot row_slot[m][t]'s partials), formed exactly as moe_combine_kernel
// forms it (the slices summed over 8 clamped slots in slice order, 0 added
// past S, as sum_parts does; the experts in selection order), then added as
// the single-slice partial of add_rmsnorm_fused_kernel (0 + y).  So
// resid_out and h are bitwise those of vw4_moe_combine followed by
// vw4_add_rmsnorm_out.  Layout and ownership as add_rmsnorm_fused_kernel;
// topk <= 8, S * 8 * CPW <= 32 four-float loads per lane.
template <int S, int CPW>
__global__ __launch_bounds__(FN_MAXW * 64) void moe_add_rmsnorm_kernel(
    const uint16_t* __restrict__ rin, const float* __restrict__ part, int64_t ldp, int64_t p_sstride,
    const int32_t* __restrict__ row_slot, const float* __restrict__ weights, int topk,
    const uint16_t* __restrict__ gamma, float eps, int M, int D, uint16_t* __restrict__ rout,
    uint16_t* __restrict__ h) {
    constexpr int TK = 8;
    __shared__ float s_ssq[FN_MAXCH];
    const int ch = blockIdx.x, m = blockIdx.y, nch = gridDim.x;
    const int nw = blockDim.x >> 6;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int own_j = ch / nw, own_w = ch % nw;
    int64_t sbase[TK];
    float wt[TK];
#pragma unroll
    for (int t = 0; t < TK; ++t) {
        const int tt = t < topk ? t : topk - 1;
        sbase[t] = (int64_t)row_slot[m * topk + tt] * p_sstride;
        wt[t] = weights[m * topk + tt];
    }
    uint2 rr[CPW];
    f32x4 pp[CPW][TK][S];
    const int gcol = ch * NCOL + 4 * lane < D ? ch * NCOL + 4 * lane : D - 4;
    const uint2 gg = *(const uint2*)(gamma + gcol);
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
        int c = w + nw * j;
        c = c < nch ? c : nch - 1;
        int col = c * NCOL + 4 * lane;
        col = col < D ? col : D - 4;                      // D % 4 == 0
        rr[j] = *(const uint2*)(rin + (int64_t)m * D + col);
#pragma unroll
        for (int t = 0; t < TK; ++t)
#pragma unroll
            for (int k = 0; k < S; ++k)
                pp[j][t][k] = *(const f32x4*)(part + sbase[t] + ((int64_t)k * M + m) * ldp + col);
    }
    float own[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
        const int c = w + nw * j;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float acc = 0.0f;
#pragma unroll
            for (int t = 0; t < TK; ++t) {
                float sv = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) sv += (i < S) ? pp[j][t][i < S ? i : S - 1][e] : 0.0f;
                if (t < topk) acc += wt[t] * sv;
            }
            float sp = 0.0f;
            sp += acc;
            float x = bf16_to_f32((uint16_t)((e < 2 ? rr[j].x : rr[j].y) >> (16 * (e & 1))));
            x = bf16_to_f32(f32_to_bf16(x + sp));
            v[e] = (c < nch && c * NCOL + 4 * lane + e < D) ? x : 0.0f;
        }
        const float q = chunk_sumsq(v);
        if (c < nch && lane == 0) s_ssq[c] = q;
        if (j == own_j && w == own_w) {
#pragma unroll
            for (int e = 0; e < 4; ++e) own[e] = v[e];
        }
    }
    __syncthreads();
    if (w != own_w) return;
    float tot = 0.0f;
    for (int c = 0; c < nch; ++c) tot += s_ssq[c];      // chunk order
    const float inv = 1.0f / sqrtf(tot / (float)D + eps);
    const int col = ch * NCOL + 4 * lane;
    if (col >= D) return;
    const float g[4] = {bf16_to_f32((uint16_t)(gg.x & 0xffffu)), bf16_to_f32((uint16_t)(gg.x >> 16)),
                        bf16_to_f32((uint16_t)(gg.y & 0xffffu)), bf16_to_f32((uint16_t)(gg.y >> 16))};
    uint2 ro, ho;
    ro.x = f32x2_to_bf16x2(own[0], own[1]);
    ro.y = f32x2_to_bf16x2(own[2], own[3]);
    ho.x = f32x2_to_bf16x2(own[0] * inv * g[0], own[1] * inv * g[1]);
    ho.y = f32x2_to_bf16x2(own[2] * inv * g[2], own[3] * inv * g[3]);
    *(uint2*)(rout + (int64_t)m * D + col) = ro;
    *(uint2*)(h + (int64_t)m * D + col) = ho;
}

__global__ __launch_bounds__(NCOL) void rmsnorm_apply_kernel(const uint16_t* __restrict__ resid,
                                                             const uint16_t* __restrict__ gamma, float eps, int D,
                                                             const float* __restrict__ ssq, int nch,
                                                             uint16_t* __restrict__ h) {
    __shared__ float s_ssq[NMAXCH];
    __shared__ float s_tot;
    const int ch = blockIdx.x, m = blockIdx.y, d = ch * NCOL + threadIdx.x;
    // this thread's row value and gain are requested together with the chunk
    // sums (one memory round trip)
    const bool live = d < D;
    const float r = live ? bf16_to_f32(resid[(int64_t)m * D + d]) : 0.0f;
    const float gm = live ? bf16_to_f32(gamma[d]) : 0.0f;
    for (int k = threadIdx.x; k < nch; k += NCOL) s_ssq[k] = ssq[(int64_t)m * nch + k];  // loads in parallel
    __syncthreads();
    if (threadIdx.x == 0) {
        float tot = 0.0f;
        for (int k = 0; k < nch; ++k) tot += s_ssq[k];  // chunk order
        s_tot = tot;
    }
    __syncthreads();
    if (!live) return;
    const float inv = 1.0f / sqrtf(s_tot / (float)D + eps);
    h[(int64_t)m * D + d] = f32_to_bf16(r * inv * gm);
}

// ---------------------------------------------------------------------------
// rotary embedding of q and k + KV append.  grid = (nq + 2 nkv, M), hd/2 threads.
// ---------------------------------------------------------------------------
__global__ void rope_kv_kernel(const float* __restrict__ part, int S, int64_t ldp, int M, int nq, int nkv, int hd,
                               int L, double theta, uint16_t* __restrict__ q_out, uint16_t* __restrict__ Kc,
                               uint16_t* __restrict__ Vb, int64_t Lmax) {
    const int hh = blockIdx.x, m = blockIdx.y, d = threadIdx.x, half = hd / 2;
    const int64_t c0 = (int64_t)hh * hd;
    const int64_t pos = (int64_t)L + m;
    const bool vhead = hh >= nq + nkv;
    // With S <= 8 the 2 S partial loads are all issued (slice index clamped,
    // no branch between them) before the angle is computed, so the fp64 math
    // runs while they are in flight; the sums are in slice order either way.
    float pa[8], pb[8];
    const float* p = part + (int64_t)m * ldp + c0 + d;
    const int64_t pst = (int64_t)M * ldp;
    if (S <= 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t k = i < S ? i : S - 1;
            pa[i] = p[k * pst];
            pb[i] = p[k * pst + half];
        }
    }
    // angle = pos * theta^(-2d/hd), in fp64 so that large positions keep their
    // accuracy; the rotation itself in fp32 (value heads need none)
    double sd = 0.0, cd = 1.0;
    if (!vhead) {
        const double ang = (double)pos * pow(theta, -2.0 * (double)d / (double)hd);
        sincos(ang, &sd, &cd);
    }
    float a = 0.0f, b = 0.0f;
    if (S <= 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a += i < S ? pa[i] : 0.0f;
            b += i < S ? pb[i] : 0.0f;
        }
    } else {
        a = sum_parts(part, S, M, ldp, m, c0 + d);
        b = sum_parts(part, S, M, ldp, m, c0 + d + half);
    }
    if (vhead) {  // value head: append as is
        const int kv = hh - nq - nkv;
        // blocked: [kv][position / 32][dim][position % 32]
        uint16_t* dst = Vb + (int64_t)kv * hd * Lmax + (pos >> 5) * hd * 32 + (pos & 31);
        dst[(int64_t)d * 32] = f32_to_bf16(a);
        dst[(int64_t)(d + half) * 32] = f32_to_bf16(b);
        return;
    }
    const float c = (float)cd, s = (float)sd;
    const float ra = a * c - b * s, rb = b * c + a * s;
    if (hh < nq) {
        uint16_t* dst = q_out + ((int64_t)m * nq + hh) * hd;
        dst[d] = f32_to_bf16(ra);
        dst[d + half] = f32_to_bf16(rb);
    } else {
        const int kv = hh - nq;
        uint16_t* dst = Kc + ((int64_t)kv * Lmax + pos) * hd;
        dst[d] = f32_to_bf16(ra);
        dst[d + half] = f32_to_bf16(rb);
    }
}

// ---------------------------------------------------------------------------
// SwiGLU.  grid = (ceil(F / 256), M), 256 threads.
// ---------------------------------------------------------------------------
// Grouped launches (n_slots != NULL): blockIdx.z is a slot with its own
// partials (p_sstride floats apart) and output (a_sstride elements apart);
// slots at or beyond *n_slots exit at once.
__global__ __launch_bounds__(256) void swiglu_kernel(const float* __restrict__ part, int S, int64_t ldp, int M, int F,
                                                     uint16_t* __restrict__ a, int64_t p_sstride, int64_t a_sstride,
                                                     const int32_t* __restrict__ n_slots) {
    const int j = blockIdx.x * 256 + threadIdx.x, m = blockIdx.y;
    if (j >= F) return;
    if (n_slots) {
        if ((int)blockIdx.z >= *n_slots) return;
        part += (int64_t)blockIdx.z * p_sstride;
        a += (int64_t)blockIdx.z * a_sstride;
    }
    const float g = sum_parts(part, S, M, ldp, m, j);
    const float u = sum_parts(part, S, M, ldp, m, (int64_t)F + j);
    const float sg = g / (1.0f + expf(-g));
    a[(int64_t)m * F + j] = f32_to_bf16(sg * u);
}

// ---------------------------------------------------------------------------
// Grouped-query decode attention on the matrix cores.
//
// KV cache layout: K [nkv][Lmax][128] (a position is one 256-byte row) and V
// in 32-position blocks, transposed inside each block: Vb [nkv][Lmax / 32]
// [128][32] (a block is 8 KiB, one row of 32 positions per head dimension).
// Both contractions read 16-byte runs straight into MFMA operands, and a
// 32-position tile of K or V is one contiguous 8 KiB run (measured: a fully
// transposed V [128][Lmax], whose tile is 128 pieces of 64 bytes 2 * Lmax
// bytes apart, costs 8-9% of the kernel's time at 8k-32k positions).
//
// grid = (nkv, nparts), 4 wavefronts.  The context is cut into whole
// 32-position tiles; the fewer than 32 positions past the last whole tile are
// left to attn_combine_kernel, so that a context just past a multiple of the
// tile count does not give one wavefront a second tile (measured: about 2 us
// per launch).  Workgroup (h, c) owns a contiguous
// range of 32-position tiles of KV head h and all QN = G * M queries that read
// it (query j: head h * G + j / M, row j % M; row m sees positions
// 0 .. L + m).  Wavefront w takes tiles w, w + 4, ... of the range; the next
// tile's K rows are requested once the scores have consumed the current ones,
// its V rows once P.V has.  Per tile, with
// v_mfma_f32_16x16x32_bf16 (A: lane l = row l % 16, k 8 (l / 16) .. +8;
// B: lane l = column l % 16, same k; D: lane l = column l % 16, rows
// 4 (l / 16) .. +4):
//   S^T[pos][query] = K[pos][:] . Q[query][:]   (A = K rows, B = queries),
//     the 16 A rows of block b being positions 8 (i / 4) + 4 b + i % 4, so
//     that lane (g, i) ends up holding query i at positions 8 g .. 8 g + 7;
//   online softmax in base 2 (scores pre-scaled by log2(e) / sqrt(128));
//   O[query][dim] += P[query][pos] . V[pos][dim]  (A = those 8 probabilities
//     as a bf16 head plus a bf16 tail, two products, so P keeps about 16
//     bits; B = 16 bytes of a Vb row).
// The four wavefronts merge pairwise in LDS ((w0 + w2) + (w1 + w3)), and the
// workgroup writes one partial (m, l, o) per query; attn_combine_kernel
// merges the partials in chunk order, then the remainder positions.
// ---------------------------------------------------------------------------
constexpr int AHD = 128;       // head dim handled
constexpr int AQN = 48;        // max queries per KV head (G * M)
constexpr int AT = 32;         // positions per tile
constexpr int AWV = 4;         // wavefronts per workgroup


struct AttnPart {   // per (kv head, query, chunk): max (base 2), sum
    float m, l;
};

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *(const u32x4v*)p);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct AttnTile {
    bf16x8 k[2][4];   // K rows of the two 16-position blocks, 4 steps of 32 dims
    bf16x8 v[8];      // Vb rows of the 8 16-dim blocks, positions 8 g .. +8
};

__device__ __forceinline__ void attn_load_k(AttnTile& T, const uint16_t* Kh, int64_t ctx, int64_t t0, int g, int i) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        int64_t pos = t0 + 8 * (i >> 2) + 4 * b + (i & 3);
        pos = pos < ctx ? pos : ctx - 1;               // rows past the context are masked later
#pragma unroll
        for (int s = 0; s < 4; ++s) T.k[b][s] = ld_bf16x8(Kh + pos * AHD + 32 * s + 8 * g);
    }
}

// Element (position p, dimension dim) of one KV head's blocked value cache;
// 8 positions from an 8-aligned p are 16 contiguous bytes.
__device__ __forceinline__ int64_t vb_at(int64_t p, int dim) {
    return ((p >> 5) * AHD + dim) * 32 + (p & 31);
}

__device__ __forceinline__ void attn_load_v(AttnTile& T, const uint16_t* Vh, int64_t Lmax, int64_t ctx, int64_t t0,
                                            int g, int i) {
    const int64_t p8 = t0 + 8 * g;
    if (p8 + 8 <= ctx) {
#pragma unroll
        for (int db = 0; db < 8; ++db) T.v[db] = ld_bf16x8(Vh + vb_at(p8, db * 16 + i));
    } else {
        // The context ends inside (or before) these 8 positions.  The 16 bytes
        // are read from an 8-aligned start at most (ctx - 1) rounded down, which
        // lies inside the cache (Lmax % 32 == 0), and the positions at or past
        // ctx are zeroed in registers (their probabilities are 0, and 0 * NaN
        // would not be).
        const int64_t last8 = (ctx - 1) & ~(int64_t)7;
        const int64_t pl = p8 < last8 ? p8 : last8;
        const int64_t nv64 = ctx - p8;
        const int nv = nv64 < 0 ? 0 : (int)nv64;
        u32x4v keep;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            keep[w] = (2 * w < nv ? 0x0000ffffu : 0u) | (2 * w + 1 < nv ? 0xffff0000u : 0u);
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const u32x4v raw = *(const u32x4v*)(Vh + vb_at(pl, db * 16 + i));
            T.v[db] = __builtin_bit_cast(bf16x8, raw & keep);
        }
    }
}

// One tile: scores from T.k, then (once T.k is consumed) the next tile's K
// rows are requested; softmax; P.V from T.v, then the next tile's V rows.
template <int NQB>
__device__ __forceinline__ void attn_tile(AttnTile& T, const bf16x8 (&qop)[NQB][4], const int64_t (&lim)[NQB],
                                          int64_t t0, int g, int i, float sl2e, float (&mrun)[NQB], float (&lrun)[NQB],
                                          f32x4 (&o)[NQB][8], bool more, int64_t tn0, const uint16_t* Kh,
                                          const uint16_t* Vh, int64_t Lmax, int64_t ctx) {
    f32x4 sc[NQB][2];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        sc[qb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        sc[qb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            sc[qb][0] = mfma16(T.k[0][s], qop[qb][s], sc[qb][0]);
            sc[qb][1] = mfma16(T.k[1][s], qop[qb][s], sc[qb][1]);
        }
    }
    if (more) attn_load_k(T, Kh, ctx, tn0, g, i);
    bf16x8 pv[NQB], pw[NQB];   // p = pv + pw to about 2^-17 (bf16 head and tail)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        float v[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            v[r] = sc[qb][0][r] * sl2e;
            v[4 + r] = sc[qb][1][r] * sl2e;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (t0 + 8 * g + e > lim[qb]) v[e] = -INFINITY;
            mx = fmaxf(mx, v[e]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mnew = fmaxf(mrun[qb], mx);
        const float mu = (mnew == -INFINITY) ? 0.0f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(mrun[qb] - mu);
        float ps = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(v[e] - mu);
            ps += p;
            const __bf16 hi = (__bf16)p;
            pv[qb][e] = hi;
            pw[qb][e] = (__bf16)(p - (float)hi);
        }
        lrun[qb] = lrun[qb] * alpha + ps;
        mrun[qb] = mnew;
        // O rows are queries 4 g + r; their factor lives in lane 16 g + 4 g + r
        float a4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) a4[r] = __shfl(alpha, 20 * g + r, 64);
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[qb][db][r] *= a4[r];
    }
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            o[qb][db] = mfma16(pv[qb], T.v[db], o[qb][db]);
            o[qb][db] = mfma16(pw[qb], T.v[db], o[qb][db]);
        }
    if (more) attn_load_v(T, Vh, Lmax, ctx, tn0, g, i);
}

// Merge another wavefront's state (LDS slot) into this one's registers.
template <int NQB>
__device__ __forceinline__ void attn_merge(const float* Wo, const float* Wm, const float* Wl, int lane, int g, int i,
                                           float (&mrun)[NQB], float (&lrun)[NQB], f32x4 (&o)[NQB][8]) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const float mb = Wm[qb * 16 + i], lb = Wl[qb * 16 + i];
        const float mx = fmaxf(mrun[qb], mb);
        const float mu = (mx == -INFINITY) ? 0.0f : mx;
        const float fa = __builtin_amdgcn_exp2f(mrun[qb] - mu), fb = __builtin_amdgcn_exp2f(mb - mu);
        lrun[qb] = fa * lrun[qb] + fb * lb;
        mrun[qb] = mx;
        float fa4[4], fb4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            fa4[r] = __shfl(fa, 20 * g + r, 64);
            fb4[r] = __shfl(fb, 20 * g + r, 64);
        }
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                o[qb][db][r] = fa4[r] * o[qb][db][r] + fb4[r] * Wo[((qb * 8 + db) * 4 + r) * 64 + lane];
    }
}

template <int NQB>
__device__ __forceinline__ void attn_store(float* Wo, float* Wm, float* Wl, int lane, int g, int i,
                                           const float (&mrun)[NQB], const float (&lrun)[NQB],
                                           const f32x4 (&o)[NQB][8]) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        if (g == 0) {
            Wm[qb * 16 + i] = mrun[qb];
            Wl[qb * 16 + i] = lrun[qb];
        }
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) Wo[((qb * 8 + db) * 4 + r) * 64 + lane] = o[qb][db][r];
    }
}

template <int NQB>
__device__ __forceinline__ void attn_body(const uint16_t* __restrict__ q, const uint16_t* __restrict__ Kc,
                                          const uint16_t* __restrict__ Vb, int64_t Lmax, int64_t L, int M, int nq,
                                          int G, int ntiles, float sl2e, float* __restrict__ ws_o,
                                          AttnPart* __restrict__ ws_ml) {
    constexpr int OSZ = NQB * 8 * 4 * 64;                  // one wavefront's o, lane-major
    __shared__ float Wo[2][OSZ];
    __shared__ float Wm[2][NQB * 16], Wl[2][NQB * 16];
    const int QN = G * M;
    const int h = blockIdx.x, c = blockIdx.y, nparts = gridDim.y;
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, i = lane & 15;
    const int64_t ctx = L + M;
    const int tb = c * ntiles / nparts, te = (c + 1) * ntiles / nparts;   // ntiles < 2^24: 32-bit division
    const uint16_t* Kh = Kc + (int64_t)h * Lmax * AHD;
    const uint16_t* Vh = Vb + (int64_t)h * AHD * Lmax;

    bf16x8 qop[NQB][4];
    int64_t lim[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int j = qb * 16 + i;
        if (j < QN) {
            const int row = j % M, head = h * G + j / M;
            const uint16_t* qp = q + ((int64_t)row * nq + head) * AHD;
#pragma unroll
            for (int s = 0; s < 4; ++s) qop[qb][s] = ld_bf16x8(qp + 32 * s + 8 * g);
            lim[qb] = L + row;
        } else {
            const bf16x8 z = {};
#pragma unroll
            for (int s = 0; s < 4; ++s) qop[qb][s] = z;
            lim[qb] = -1;
        }
    }
    float mrun[NQB], lrun[NQB];
    f32x4 o[NQB][8];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        mrun[qb] = -INFINITY;
        lrun[qb] = 0.0f;
#pragma unroll
        for (int db = 0; db < 8; ++db) o[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // one tile of registers: the next tile's K (V) rows are requested as soon
    // as the current ones have been consumed
    AttnTile T;
    int t = tb + wv;
    if (t < te) {
        attn_load_k(T, Kh, ctx, (int64_t)t * AT, g, i);
        attn_load_v(T, Vh, Lmax, ctx, (int64_t)t * AT, g, i);
    }
    for (; t < te; t += AWV) {
        const int tn = t + AWV;
        attn_tile<NQB>(T, qop, lim, (int64_t)t * AT, g, i, sl2e, mrun, lrun, o, tn < te, (int64_t)tn * AT, Kh, Vh,
                       Lmax, ctx);
    }
    // row sums over the four lanes that share a query
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        lrun[qb] += __shfl_xor(lrun[qb], 16, 64);
        lrun[qb] += __shfl_xor(lrun[qb], 32, 64);
    }
    // (w0 + w2) and (w1 + w3), then their sum, in wavefront 0
    if (wv >= 2) attn_store<NQB>(Wo[wv - 2], Wm[wv - 2], Wl[wv - 2], lane, g, i, mrun, lrun, o);
    __syncthreads();
    if (wv < 2) attn_merge<NQB>(Wo[wv], Wm[wv], Wl[wv], lane, g, i, mrun, lrun, o);
    __syncthreads();
    if (wv == 1) attn_store<NQB>(Wo[0], Wm[0], Wl[0], lane, g, i, mrun, lrun, o);
    __syncthreads();
    if (wv != 0) return;
    attn_merge<NQB>(Wo[0], Wm[0], Wl[0], lane, g, i, mrun, lrun, o);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int j = qb * 16 + i;
        if (g == 0 && j < QN) {
            AttnPart ap;
            ap.m = mrun[qb];
            ap.l = lrun[qb];
            ws_ml[((int64_t)h * QN + j) * nparts + c] = ap;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int jr = qb * 16 + 4 * g + r;
            if (jr < QN) {
                float* dst = ws_o + (((int64_t)h * QN + jr) * nparts + c) * AHD + i;
#pragma unroll
                for (int db = 0; db < 8; ++db) dst[db * 16] = o[qb][db][r];
            }
        }
    }
}

// Up to 32 queries per KV head: at most 256 registers per lane, so that two
// workgroups could share a CU (the plan launches about one per CU).  More
// queries: one workgroup per CU, no spills.
template <int NQB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ Kc, const uint16_t* __restrict__ Vb, int64_t Lmax,
    int64_t L, int M, int nq, int G, int ntiles, float sl2e, float* __restrict__ ws_o, AttnPart* __restrict__ ws_ml) {
    attn_body<NQB>(q, Kc, Vb, Lmax, L, M, nq, G, ntiles, sl2e, ws_o, ws_ml);
}

__global__ __launch_bounds__(256) void attn_mfma_wide_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ Kc, const uint16_t* __restrict__ Vb, int64_t Lmax,
    int64_t L, int M, int nq, int G, int ntiles, float sl2e, float* __restrict__ ws_o, AttnPart* __restrict__ ws_ml) {
    attn_body<3>(q, Kc, Vb, Lmax, L, M, nq, G, ntiles, sl2e, ws_o, ws_ml);
}

// Merge the chunk partials of one (kv head, query) and add the positions
// past the last whole tile (r0 .. ctx - 1, fewer than 32), which the tile
// kernel leaves out so that its workgroups stay balanced: grid = (QN, nkv),
// AHD threads.  The remainder is one more partial (scores and softmax in
// fp32, base 2), merged after the chunks in position order.  NPM >= nparts
// is the number of partial slots each thread loads (16, 32 or 64).
template <int NPM>
__global__ __launch_bounds__(AHD) void attn_combine_kernel(
    const float* __restrict__ ws_o, const AttnPart* __restrict__ ws_ml, int nparts, int QN, int M, int nq, int G,
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const uint16_t* __restrict__ Kc,
    const uint16_t* __restrict__ Vb, int64_t Lmax, int64_t L, int64_t r0, int64_t ctx, float sl2e) {
    __shared__ float s_f[64], s_l[64], s_sc[AT];
    __shared__ float s_mr;
    const int j = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
    const int row = j % M, head = h * G + j / M;
    const int64_t lim = L + row;                      // last position this query sees
    const int nr = (int)(ctx - r0);                   // 0 .. AT - 1
    const int64_t base = ((int64_t)h * QN + j) * nparts;
    // One memory round trip: the remainder's operands first (so that its
    // scores can be formed while the rest is in flight), then the partial
    // outputs and the chunk maxima and sums.
    // Remainder scores: thread 4 k + qt takes dims 32 qt .. +32 of position
    // r0 + k.  Its values of dimension d, positions r0 .. r0 + 31, come in
    // 8-position pieces whose start is clamped to the last 8-aligned start
    // before ctx (inside the cache: Lmax % 32 == 0); positions at or past ctx
    // are never used.
    // Every address is clamped to a valid one instead of the load being
    // predicated, so that no branch separates the loads and each wait covers
    // only the loads it needs.
    const int k = d >> 2, qt = d & 3;
    u32x4v kv[4], qv[4], vv[4];
    {
        const int64_t pk = r0 + k < ctx ? r0 + k : ctx - 1;
        const u32x4v* kp = (const u32x4v*)(Kc + ((int64_t)h * Lmax + pk) * AHD + 32 * qt);
        const u32x4v* qp = (const u32x4v*)(q + ((int64_t)row * nq + head) * AHD + 32 * qt);
        const int64_t last8 = (ctx - 1) & ~(int64_t)7;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kv[e] = kp[e];
            qv[e] = qp[e];
            const int64_t p8 = r0 + 8 * e < last8 ? r0 + 8 * e : last8;
            vv[e] = *(const u32x4v*)(Vb + (int64_t)h * AHD * Lmax + vb_at(p8, d));
        }
    }
    // (then up to 40 of the partial outputs: the wait counter counts at most
    // 63 loads, so with NPM = 64 the remainder's scores are formed before the
    // last 24 issue)
    constexpr int NP1 = NPM < 40 ? NPM : 40;
    __builtin_amdgcn_sched_barrier(0);
    // lanes d >= nparts repeat the last chunk: the maximum is unchanged and
    // the sums below stop at nparts
    const AttnPart ap = ws_ml[base + (d < nparts ? d : nparts - 1)];
    float o[NPM];
#pragma unroll
    for (int c = 0; c < NP1; ++c) o[c] = ws_o[(base + (c < nparts ? c : nparts - 1)) * AHD + d];
    __builtin_amdgcn_sched_barrier(0);
    // (unconditional: with nr == 0 every score is -inf and nothing is added;
    // a branch here would let the compiler sink the loads above into it)
    float mr = -INFINITY, lr = 0.0f, orr = 0.0f;
    {
        float sc = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                sc = fmaf(__uint_as_float(qv[e][w] << 16), __uint_as_float(kv[e][w] << 16), sc);
                sc = fmaf(__uint_as_float(qv[e][w] & 0xffff0000u), __uint_as_float(kv[e][w] & 0xffff0000u), sc);
            }
        sc += __shfl_xor(sc, 1, 64);
        sc += __shfl_xor(sc, 2, 64);
        if (qt == 0) s_sc[k] = (k < nr && r0 + k <= lim) ? sc * sl2e : -INFINITY;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = NP1; c < NPM; ++c) o[c] = ws_o[(base + (c < nparts ? c : nparts - 1)) * AHD + d];
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        for (int e = 0; e < nr; ++e) mr = fmaxf(mr, s_sc[e]);
        const float mru = (mr == -INFINITY) ? 0.0f : mr;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int w = 0; w < 4; ++w)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int e = 8 * c + 2 * w + hf;
                    if (e < nr) {
                        const float p = __builtin_amdgcn_exp2f(s_sc[e] - mru);
                        const float v = __uint_as_float(hf ? (vv[c][w] & 0xffff0000u) : (vv[c][w] << 16));
                        lr += p;
                        orr = fmaf(p, v, orr);
                    }
                }
    }
    // chunk maxima and sums: one chunk per thread (nparts <= 64)
    if (d < 64) {
        float mx = fmaxf(ap.m, mr);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        s_f[d] = (ap.m == -INFINITY) ? 0.0f : exp2f(ap.m - mx);
        s_l[d] = ap.l;
        if (d == 0) s_mr = (mr == -INFINITY) ? 0.0f : exp2f(mr - mx);
    }
    __syncthreads();
    float lt = 0.0f, ot = 0.0f;
#pragma unroll
    for (int c = 0; c < NPM; ++c) {
        if (c < nparts) {
            lt += s_f[c] * s_l[c];
            ot += s_f[c] * o[c];
        }
    }
    const float fr = s_mr;
    lt += fr * lr;
    ot += fr * orr;
    out[((int64_t)row * nq + head) * AHD + d] = f32_to_bf16(ot / lt);
}

struct AttnPlan {
    int QN, ntiles, nparts;
    size_t off_o, off_ml, total;
};

constexpr int ATTN_MAX_PARTS = 64;

// Whole 32-position tiles split evenly over nparts workgroups per KV head:
// about one workgroup per compute unit over all KV heads, and at least two
// tiles per workgroup (measured on MI355X from 512 to 32768 positions, M = 1
// and 4: one workgroup per CU beats two, and fewer partials make the merge
// cheaper).  The workspace is sized for ATTN_MAX_PARTS partials, so that its
// size does not depend on the device or the tuning.
static AttnPlan attn_plan(int M, int nq, int nkv, int64_t ctx) {
    AttnPlan p;
    p.QN = (nq / nkv) * M;
    p.ntiles = (int)(ctx / AT);                     // whole tiles; the rest goes to the combine
    int np = (p.ntiles + 1) / 2;
    int cap = device_cus() / nkv;
    cap = cap < 1 ? 1 : (cap > ATTN_MAX_PARTS ? ATTN_MAX_PARTS : cap);
    np = np > cap ? cap : np;
    if (const char* e = getenv("VW4_ATTN_TILES")) {  // tuning override: tiles per workgroup
        const int v = atoi(e);
        if (v >= 1 && v <= 1 << 20) np = (p.ntiles + v - 1) / v;
    }
    p.nparts = np < 1 ? 1 : (np > ATTN_MAX_PARTS ? ATTN_MAX_PARTS : np);
    size_t o = 0;
    p.off_o = o;
    o += (size_t)nkv * p.QN * ATTN_MAX_PARTS * AHD * sizeof(float);
    o = (o + 255) / 256 * 256;
    p.off_ml = o;
    o += (size_t)nkv * p.QN * ATTN_MAX_PARTS * sizeof(AttnPart);
    p.total = (o + 255) / 256 * 256;
    return p;
}

}  // namespace vw4

using namespace vw4;

extern "C" {

size_t vw4_norm_workspace_bytes(int32_t M, int32_t D) {
    if (M < 1 || M > 64 || D < 1 || D > 65536) return 0;
    return ((size_t)M * ((D + NCOL - 1) / NCOL) * sizeof(float) + 255) / 256 * 256;
}

int vw4_add_rmsnorm(uint16_t* resid, const float* part, int32_t S, int64_t ldp, const uint16_t* gamma, float eps,
                    int32_t M, int32_t D, uint16_t* h, void* ws, size_t ws_bytes, void* stream) {
    VW4_REQUIRE(resid && gamma && h, VW4_EINVAL, "vw4_add_rmsnorm: null pointer");
    VW4_REQUIRE(M >= 1 && M <= 64 && D >= 1 && D <= 65536, VW4_EINVAL, "vw4_add_rmsnorm: bad shape M=%d D=%d", M, D);
    VW4_REQUIRE(!part || (S >= 1 && ldp >= D), VW4_EINVAL, "vw4_add_rmsnorm: bad partial layout");
    VW4_REQUIRE(eps >= 0.0f, VW4_EINVAL, "vw4_add_rmsnorm: eps must be >= 0");
    const size_t need = vw4_norm_workspace_bytes(M, D);
    VW4_REQUIRE(ws && ws_bytes >= need, VW4_EWORKSPACE, "vw4_add_rmsnorm: needs a workspace of %zu bytes", need);
    const int nch = (D + NCOL - 1) / NCOL;
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(add_sumsq_kernel, dim3(nch, M), dim3(64), 0, st, resid, part, S, ldp, M, D, (float*)ws);
    hipLaunchKernelGGL(rmsnorm_apply_kernel, dim3(nch, M), dim3(NCOL), 0, st, resid, gamma, eps, D, (const float*)ws,
                       nch, h);
    return check_launch("vw4_add_rmsnorm");
}

int vw4_add_sumsq(uint16_t* resid, const float* part, int32_t S, int64_t ldp, int32_t M, int32_t D, void* ws,
                  size_t ws_bytes, void* stream) {
    VW4_REQUIRE(resid, VW4_EINVAL, "vw4_add_sumsq: null pointer");
    VW4_REQUIRE(M >= 1 && M <= 64 && D >= 1 && D <= 65536, VW4_EINVAL, "vw4_add_sumsq: bad shape M=%d D=%d", M, D);
    VW4_REQUIRE(!part || (S >= 1 && ldp >= D), VW4_EINVAL, "vw4_add_sumsq: bad partial layout");
    const size_t need = vw4_norm_workspace_bytes(M, D);
    VW4_REQUIRE(ws && ws_bytes >= need, VW4_EWORKSPACE, "vw4_add_sumsq: needs a workspace of %zu bytes", need);
    const int nch = (D + NCOL - 1) / NCOL;
    hipLaunchKernelGGL(add_sumsq_kernel, dim3(nch, M), dim3(64), 0, (hipStream_t)stream, resid, part, S, ldp, M, D,
                       (float*)ws);
    return check_launch("vw4_add_sumsq");
}

static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const char *pa = (const char*)a, *pb = (const char*)b;
    return pa < pb + nb && pb < pa + na;
}

int vw4_add_rmsnorm_out(const uint16_t* resid_in, const float* part, int32_t S, int64_t ldp, const uint16_t* gamma,
                        float eps, int32_t M, int32_t D, uint16_t* resid_out, uint16_t* h, void* stream) {
    VW4_REQUIRE(resid_in && gamma && resid_out && h, VW4_EINVAL, "vw4_add_rmsnorm_out: null pointer");
    VW4_REQUIRE(M >= 1 && M <= 64 && D >= 4 && D % 4 == 0 && D <= FN_MAXCH * NCOL, VW4_EINVAL,
                "vw4_add_rmsnorm_out: need 1 <= M <= 64, D %% 4 == 0, 4 <= D <= %d (M=%d D=%d)", FN_MAXCH * NCOL,
                M, D);
    VW4_REQUIRE(!part || (S >= 1 && S <= 8 && ldp >= D && ldp % 4 == 0 && aligned(part, 16)), VW4_EINVAL,
                "vw4_add_rmsnorm_out: partials need 1 <= S <= 8, ldp >= D, ldp %% 4 == 0, 16-byte alignment");
    VW4_REQUIRE(aligned(resid_in, 8) && aligned(resid_out, 8) && aligned(h, 8) && aligned(gamma, 8), VW4_EINVAL,
                "vw4_add_rmsnorm_out: resid_in, resid_out, h and gamma need 8-byte alignment");
    VW4_REQUIRE(eps >= 0.0f, VW4_EINVAL, "vw4_add_rmsnorm_out: eps must be >= 0");
    const size_t nb = (size_t)M * D * 2;
    VW4_REQUIRE(!overlaps(resid_in, nb, resid_out, nb) && !overlaps(resid_in, nb, h, nb) &&
                    !overlaps(resid_out, nb, h, nb),
                VW4_EINVAL, "vw4_add_rmsnorm_out: resid_in, resid_out and h must not overlap");
    // Chunks per wavefront: 1 up to 8 chunks, 2 up to 16, then 3 (at most 11
    // wavefronts).  Measured at D = 5120 (20 chunks) after the o and down
    // GEMMs: 7 wavefronts of 3 chunks beat 10 of 2 and 5 of 4, and 8 of 4
    // (12 clamped duplicate slots) by 0.7-0.9 us.
    const int nch = (D + NCOL - 1) / NCOL;
    const int cpw = nch <= 8 ? 1 : (nch <= 16 ? 2 : 3);
    const int nw = (nch + cpw - 1) / cpw;
    const dim3 grid(nch, M), blk(nw * 64);
    hipStream_t st = (hipStream_t)stream;
    const int ss = part ? S : 0;
    switch (ss * 3 + (cpw - 1)) {
#define VW4_FN_CASE(n)                                                                                        \
    case 3 * n:                                                                                             \
        hipLaunchKernelGGL((add_rmsnorm_fused_kernel<n, 1>), grid, blk, 0, st, resid_in, part, ldp, gamma, eps, M, \
                           D, resid_out, h);                                                                \
        break;                                                                                              \
    case 3 * n + 1:                                                                                         \
        hipLaunchKernelGGL((add_rmsnorm_fused_kernel<n, 2>), grid, blk, 0, st, resid_in, part, ldp, gamma, eps, M, \
                           D, resid_out, h);                                                                \
        break;                                                                                              \
    case 3 * n + 2:                                                                                         \
        hipLaunchKernelGGL((add_rmsnorm_fused_kernel<n, 3>), grid, blk, 0, st, resid_in, part, ldp, gamma, eps, M, \
                           D, resid_out, h);                                                                \
        break;
        VW4_FN_CASE(0) VW4_FN_CASE(1) VW4_FN_CASE(2) VW4_FN_CASE(3) VW4_FN_CASE(4) VW4_FN_CASE(5) VW4_FN_CASE(6)
        VW4_FN_CASE(7) VW4_FN_CASE(8)
#undef VW4_FN_CASE
    }
    return check_launch("vw4_add_rmsnorm_out");
}

int vw4_moe_add_rmsnorm(const uint16_t* resid_in, const float* part, int32_t S, int64_t ldp, int64_t p_sstride,
                        const int32_t* row_slot, const float* weights, int32_t topk, const uint16_t* gamma, float eps,
                        int32_t M, int32_t D, uint16_t* resid_out, uint16_t* h, void* stream) {
    VW4_REQUIRE(resid_in && part && row_slot && weights && gamma && resid_out && h, VW4_EINVAL,
                "vw4_moe_add_rmsnorm: null pointer");
    VW4_REQUIRE(M >= 1 && M <= 64 && D >= 4 && D % 4 == 0 && D <= FN_MAXCH * NCOL, VW4_EINVAL,
                "vw4_moe_add_rmsnorm: need 1 <= M <= 64, D %% 4 == 0, 4 <= D <= %d", FN_MAXCH * NCOL);
    VW4_REQUIRE(S >= 1 && ldp >= D && ldp % 4 == 0 && p_sstride >= (int64_t)S * M * ldp && p_sstride % 4 == 0 &&
                    aligned(part, 16),
                VW4_EINVAL, "vw4_moe_add_rmsnorm: bad partial layout (ldp, slot stride %% 4 == 0, 16-byte aligned)");
    VW4_REQUIRE(aligned(resid_in, 8) && aligned(resid_out, 8) && aligned(h, 8) && aligned(gamma, 8), VW4_EINVAL,
                "vw4_moe_add_rmsnorm: resid_in, resid_out, h and gamma need 8-byte alignment");
    VW4_REQUIRE(eps >= 0.0f, VW4_EINVAL, "vw4_moe_add_rmsnorm: eps must be >= 0");
    const size_t nb = (size_t)M * D * 2;
    VW4_REQUIRE(!overlaps(resid_in, nb, resid_out, nb) && !overlaps(resid_in, nb, h, nb) &&
                    !overlaps(resid_out, nb, h, nb),
                VW4_EINVAL, "vw4_moe_add_rmsnorm: resid_in, resid_out and h must not overlap");
    const int nch = (D + NCOL - 1) / NCOL;
    const int cpw = nch <= 8 ? 1 : (nch <= 16 ? 2 : 3);
    VW4_REQUIRE(topk >= 1 && topk <= 8 && S * 8 * cpw <= 32, VW4_EUNSUPPORTED,
                "vw4_moe_add_rmsnorm: topk=%d, S=%d at D=%d (built: topk <= 8, S * 8 * chunks per wavefront <= 32)",
                topk, S, D);
    const int nw = (nch + cpw - 1) / cpw;
    const dim3 grid(nch, M), blk(nw * 64);
    hipStream_t st = (hipStream_t)stream;
    switch (S * 4 + cpw) {
#define VW4_MN_CASE(s, c)                                                                                            \
    case s * 4 + c:                                                                                                \
        hipLaunchKernelGGL((moe_add_rmsnorm_kernel<s, c>), grid, blk, 0, st, resid_in, part, ldp, p_sstride, row_slot, \
                           weights, topk, gamma, eps, M, D, resid_out, h);                                         \
        break;
        VW4_MN_CASE(1, 1) VW4_MN_CASE(2, 1) VW4_MN_CASE(3, 1) VW4_MN_CASE(4, 1) VW4_MN_CASE(1, 2) VW4_MN_CASE(2, 2)
#undef VW4_MN_CASE
    }
    return check_launch("vw4_moe_add_rmsnorm");
}

int vw4_rope_kv_append(const float* part, int32_t S, int64_t ldp, int32_t M, int32_t nq, int32_t nkv, int32_t hd,
                       int32_t L, float theta, uint16_t* q_out, uint16_t* Kc, uint16_t* Vb, int64_t Lmax,
                       void* stream) {
    VW4_REQUIRE(part && q_out && Kc && Vb, VW4_EINVAL, "vw4_rope_kv_append: null pointer");
    VW4_REQUIRE(M >= 1 && M <= 64 && nq >= 1 && nkv >= 1 && hd >= 2 && hd % 2 == 0 && hd <= 2048, VW4_EINVAL,
                "vw4_rope_kv_append: bad shape");
    VW4_REQUIRE(S >= 1 && ldp >= (int64_t)(nq + 2 * nkv) * hd, VW4_EINVAL, "vw4_rope_kv_append: bad partial layout");
    VW4_REQUIRE(L >= 0 && (int64_t)L + M <= Lmax, VW4_EINVAL, "vw4_rope_kv_append: L + M exceeds the cache");
    VW4_REQUIRE(Lmax % 32 == 0, VW4_EINVAL, "vw4_rope_kv_append: Lmax must be a multiple of 32");
    VW4_REQUIRE(theta > 0.0f, VW4_EINVAL, "vw4_rope_kv_append: theta must be > 0");
    hipLaunchKernelGGL(rope_kv_kernel, dim3(nq + 2 * nkv, M), dim3(hd / 2), 0, (hipStream_t)stream, part, S, ldp, M,
                       nq, nkv, hd, L, (double)theta, q_out, Kc, Vb, Lmax);
    return check_launch("vw4_rope_kv_append");
}

int vw4_swiglu(const float* part, int32_t S, int64_t ldp, int32_t M, int32_t F, uint16_t* a, void* stream) {
    VW4_REQUIRE(part && a, VW4_EINVAL, "vw4_swiglu: null pointer");
    VW4_REQUIRE(M >= 1 && M <= 64 && F >= 1 && S >= 1 && ldp >= 2 * (int64_t)F, VW4_EINVAL, "vw4_swiglu: bad shape");
    hipLaunchKernelGGL(swiglu_kernel, dim3((F + 255) / 256, M), dim3(256), 0, (hipStream_t)stream, part, S, ldp, M, F,
                       a, (int64_t)0, (int64_t)0, (const int32_t*)nullptr);
    return check_launch("vw4_swiglu");
}

int vw4_grouped_swiglu(const float* part, int32_t S, int64_t ldp, int64_t p_sstride, int32_t M, int32_t F,
                       uint16_t* a, int64_t a_sstride, const int32_t* n_slots, int32_t max_slots, void* stream) {
    VW4_REQUIRE(part && a && n_slots, VW4_EINVAL, "vw4_grouped_swiglu: null pointer");
    VW4_REQUIRE(M >= 1 && M <= 64 && F >= 1 && S >= 1 && ldp >= 2 * (int64_t)F, VW4_EINVAL,
                "vw4_grouped_swiglu: bad shape");
    VW4_REQUIRE(max_slots >= 1 && max_slots <= 65535 && p_sstride >= (int64_t)S * M * ldp &&
                    a_sstride >= (int64_t)M * F,
                VW4_EINVAL, "vw4_grouped_swiglu: bad slot count or strides");
    hipLaunchKernelGGL(swiglu_kernel, dim3((F + 255) / 256, M, max_slots), dim3(256), 0, (hipStream_t)stream, part, S,
                       ldp, M, F, a, p_sstride, a_sstride, n_slots);
    return check_launch("vw4_grouped_swiglu");
}

size_t vw4_attn_workspace_bytes(int32_t M, int32_t nq, int32_t nkv, int32_t hd, int64_t ctx) {
    if (M < 1 || nq < 1 || nkv < 1 || nq % nkv || hd != AHD || ctx < 1) return 0;
    return attn_plan(M, nq, nkv, ctx).total;
}

int vw4_decode_attn(const uint16_t* q, const uint16_t* Kc, const uint16_t* Vb, int64_t Lmax, int64_t L, int32_t M,
                    int32_t nq, int32_t nkv, int32_t hd, uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
    VW4_REQUIRE(q && Kc && Vb && out, VW4_EINVAL, "vw4_decode_attn: null pointer");
    VW4_REQUIRE(hd == AHD, VW4_EUNSUPPORTED, "vw4_decode_attn: head dim %d (only 128 is built)", hd);
    VW4_REQUIRE(M >= 1 && nq >= 1 && nkv >= 1 && nq % nkv == 0, VW4_EINVAL, "vw4_decode_attn: bad head counts");
    const int QN = (nq / nkv) * M;
    VW4_REQUIRE(QN <= AQN, VW4_EUNSUPPORTED, "vw4_decode_attn: (nq/nkv)*M = %d > %d", QN, AQN);
    VW4_REQUIRE(L >= 0 && L + M <= Lmax, VW4_EINVAL, "vw4_decode_attn: L + M exceeds the cache");
    VW4_REQUIRE(L + M < ((int64_t)1 << 29), VW4_EUNSUPPORTED, "vw4_decode_attn: context of 2^29 or more positions");
    VW4_REQUIRE(Lmax % 32 == 0, VW4_EINVAL, "vw4_decode_attn: Lmax must be a multiple of 32");
    VW4_REQUIRE(aligned(Kc, 16) && aligned(Vb, 16) && aligned(q, 16), VW4_EINVAL, "vw4_decode_attn: misaligned");
    const AttnPlan p = attn_plan(M, nq, nkv, L + M);
    VW4_REQUIRE(ws && ws_bytes >= p.total && aligned(ws, 256), VW4_EWORKSPACE,
                "vw4_decode_attn: needs a 256-byte aligned workspace of %zu bytes", p.total);
    hipStream_t st = (hipStream_t)stream;
    float* wo = (float*)((char*)ws + p.off_o);
    AttnPart* wml = (AttnPart*)((char*)ws + p.off_ml);
    const float sl2e = 1.4426950408889634f / sqrtf((float)hd);
    const int G = nq / nkv;
    const dim3 grid(nkv, p.nparts);
    switch ((QN + 15) / 16) {
        case 1:
            hipLaunchKernelGGL(attn_mfma_kernel<1>, grid, dim3(256), 0, st, q, Kc, Vb, Lmax, L, M, nq, G, p.ntiles,
                               sl2e, wo, wml);
            break;
        case 2:
            hipLaunchKernelGGL(attn_mfma_kernel<2>, grid, dim3(256), 0, st, q, Kc, Vb, Lmax, L, M, nq, G, p.ntiles,
                               sl2e, wo, wml);
            break;
        default:
            hipLaunchKernelGGL(attn_mfma_wide_kernel, grid, dim3(256), 0, st, q, Kc, Vb, Lmax, L, M, nq, G, p.ntiles,
                               sl2e, wo, wml);
            break;
    }
    // the merge loads only as many partial slots as the plan can produce
    const int64_t r0 = (int64_t)p.ntiles * AT;
    if (p.nparts <= 16)
        hipLaunchKernelGGL(attn_combine_kernel<16>, dim3(QN, nkv), dim3(AHD), 0, st, wo, wml, p.nparts, QN, M, nq, G,
                           out, q, Kc, Vb, Lmax, L, r0, L + M, sl2e);
    else if (p.nparts <= 32)
        hipLaunchKernelGGL(attn_combine_kernel<32>, dim3(QN, nkv), dim3(AHD), 0, st, wo, wml, p.nparts, QN, M, nq, G,
                           out, q, Kc, Vb, Lmax, L, r0, L + M, sl2e);
    else
        hipLaunchKernelGGL(attn_combine_kernel<ATTN_MAX_PARTS>, dim3(QN, nkv), dim3(AHD), 0, st, wo, wml, p.nparts,
                           QN, M, nq, G, out, q, Kc, Vb, Lmax, L, r0, L + M, sl2e);
    return check_launch("vw4_decode_attn");
}

}  // extern "C"
