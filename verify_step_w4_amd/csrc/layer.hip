// layer.hip — decoder-layer calls of the verify forward: residual add +
// RMSNorm, rotary embedding + KV-cache append, SwiGLU, grouped-query decode
// attention for the M verify rows.
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

#include "common.h"

namespace vw4 {

// ---------------------------------------------------------------------------
// residual add + RMSNorm in two launches over many workgroups:
//   1. grid (ceil(D / NCOL), M): resid += partials (rounded to bf16), and the
//      chunk's sum of squares of the rounded residual -> ws[m][chunk]
//   2. grid (ceil(D / NCOL), M): total (chunk order) -> scale, h = bf16(...)
// ---------------------------------------------------------------------------
constexpr int NCOL = 256;   // columns per workgroup (one per thread)
constexpr int NMAXCH = 256; // chunks per row at most (D <= 65536)

__global__ __launch_bounds__(NCOL) void add_sumsq_kernel(uint16_t* __restrict__ resid, const float* __restrict__ part,
                                                         int S, int64_t ldp, int M, int D, float* __restrict__ ssq) {
    __shared__ float red[NCOL / 64];
    const int ch = blockIdx.x, m = blockIdx.y, d = ch * NCOL + threadIdx.x;
    float v = 0.0f;
    if (d < D) {
        uint16_t* r = resid + (int64_t)m * D + d;
        v = bf16_to_f32(*r);
        if (part) {
            v += sum_parts(part, S, M, ldp, m, d);
            const uint16_t rb = f32_to_bf16(v);
            *r = rb;
            v = bf16_to_f32(rb);
        }
    }
    float sq = wave_sum(v * v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sq;
    __syncthreads();
    if (threadIdx.x == 0) ssq[(int64_t)m * gridDim.x + ch] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(NCOL) void rmsnorm_apply_kernel(const uint16_t* __restrict__ resid,
                                                             const uint16_t* __restrict__ gamma, float eps, int D,
                                                             const float* __restrict__ ssq, int nch,
                                                             uint16_t* __restrict__ h) {
    __shared__ float s_ssq[NMAXCH];
    __shared__ float s_tot;
    const int ch = blockIdx.x, m = blockIdx.y, d = ch * NCOL + threadIdx.x;
    for (int k = threadIdx.x; k < nch; k += NCOL) s_ssq[k] = ssq[(int64_t)m * nch + k];  // loads in parallel
    __syncthreads();
    if (threadIdx.x == 0) {
        float tot = 0.0f;
        for (int k = 0; k < nch; ++k) tot += s_ssq[k];  // chunk order
        s_tot = tot;
    }
    __syncthreads();
    if (d >= D) return;
    const float inv = 1.0f / sqrtf(s_tot / (float)D + eps);
    const float r = bf16_to_f32(resid[(int64_t)m * D + d]);
    h[(int64_t)m * D + d] = f32_to_bf16(r * inv * bf16_to_f32(gamma[d]));
}

// ---------------------------------------------------------------------------
// rotary embedding of q and k + KV append.  grid = (nq + 2 nkv, M), hd/2 threads.
// ---------------------------------------------------------------------------
__global__ void rope_kv_kernel(const float* __restrict__ part, int S, int64_t ldp, int M, int nq, int nkv, int hd,
                               int L, double theta, uint16_t* __restrict__ q_out, uint16_t* __restrict__ Kc,
                               uint16_t* __restrict__ Vc, int64_t Lmax) {
    const int hh = blockIdx.x, m = blockIdx.y, d = threadIdx.x, half = hd / 2;
    const int64_t c0 = (int64_t)hh * hd;
    const float a = sum_parts(part, S, M, ldp, m, c0 + d);
    const float b = sum_parts(part, S, M, ldp, m, c0 + d + half);
    const int64_t pos = (int64_t)L + m;
    if (hh >= nq + nkv) {  // value head: append as is
        const int kv = hh - nq - nkv;
        uint16_t* dst = Vc + ((int64_t)kv * Lmax + pos) * hd;
        dst[d] = f32_to_bf16(a);
        dst[d + half] = f32_to_bf16(b);
        return;
    }
    // angle = pos * theta^(-2d/hd), in fp64 so that large positions keep their
    // accuracy; the rotation itself in fp32
    const double ang = (double)pos * pow(theta, -2.0 * (double)d / (double)hd);
    double sd, cd;
    sincos(ang, &sd, &cd);
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
// Grouped-query decode attention.
//
// grid = (nkv, nchunks), 256 threads (4 wavefronts).  Workgroup (h, c) owns
// context positions [c * CP, (c + 1) * CP) of KV head h and all QN = G * M
// queries that read it (G = nq / nkv query heads, M rows); query j is head
// h * G + j / M, row j % M.  Per 64-position tile, a wavefront:
//   1. lane = position: loads its key row (16 x 16 B) and forms the QN scores
//      with v_dot2_f32_bf16, the query rows coming through scalar loads
//      (identical for all lanes);
//   2. masks positions > L + row, takes the tile max per query (wave
//      reduction), p = exp(s - max), and stores p to LDS;
//   3. lane = pair of dims: accumulates p * v over the tile's positions, the p
//      row of each position read back from LDS as a broadcast;
// with an online softmax across the wavefront's tiles.  The 4 wavefronts'
// (max, sum, o) are merged in LDS and the workgroup writes one partial per
// query; attn_combine_kernel merges the chunks (log-sum-exp weights, chunk
// order).
// ---------------------------------------------------------------------------
constexpr int AHD = 128;       // head dim handled
constexpr int AQN = 64;        // max queries per KV head (G * M)
constexpr int ATILE = 64;      // positions per wavefront tile

typedef const __attribute__((address_space(4))) uint32_t acu32;

__device__ __forceinline__ acu32* uniform_ptr_a(acu32* p) {
    const uint64_t a = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return (acu32*)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

struct AttnPart {   // per (kv head, chunk, query): max, sum, then o[AHD]
    float m, l;
};

template <int QN>
__global__ __launch_bounds__(256) void attn_chunk_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ Kc,
                                                         const uint16_t* __restrict__ Vc, int64_t Lmax, int64_t L, int M,
                                                         int nq, int G, int CP, float scale, float* __restrict__ ws_o,
                                                         AttnPart* __restrict__ ws_ml) {
    // p values of the current tile per wavefront during the loop; the
    // wavefronts' o accumulators at the merge (same storage)
    constexpr int PSZ = 4 * ATILE * QN, WSZ = 4 * QN * AHD;
    __shared__ float smem[PSZ > WSZ ? PSZ : WSZ];
    __shared__ float Wm[4][QN], Wl[4][QN];
    float(*P)[ATILE][QN] = (float(*)[ATILE][QN])smem;
    float(*Wo)[QN][AHD] = (float(*)[QN][AHD])smem;
    const int h = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int64_t ctx = L + M;                                  // filled cache positions
    const int64_t p0 = (int64_t)c * CP, p1 = min(ctx, p0 + CP);
    const uint16_t* Kh = Kc + (int64_t)h * Lmax * AHD;
    const uint16_t* Vh = Vc + (int64_t)h * Lmax * AHD;

    float mrun[QN], lrun[QN], o0[QN], o1[QN];
#pragma unroll
    for (int j = 0; j < QN; ++j) { mrun[j] = -INFINITY; lrun[j] = 0.0f; o0[j] = 0.0f; o1[j] = 0.0f; }

    for (int64_t t0 = p0 + (int64_t)wv * ATILE; t0 < p1; t0 += 4 * ATILE) {
        const int64_t pos = t0 + lane;
        const bool valid = pos < p1;
        // 1. scores for this lane's position
        uint32_t kr[AHD / 2];
        const uint4* kp = (const uint4*)(Kh + (valid ? pos : p0) * AHD);
#pragma unroll
        for (int v = 0; v < AHD / 8; ++v) {
            const uint4 w = kp[v];
            kr[4 * v] = w.x; kr[4 * v + 1] = w.y; kr[4 * v + 2] = w.z; kr[4 * v + 3] = w.w;
        }
        float s[QN];
#pragma unroll
        for (int j = 0; j < QN; ++j) {
            const int row = j % M, head = h * G + j / M;
            acu32* qp = uniform_ptr_a((acu32*)(q + ((int64_t)row * nq + head) * AHD));
            float acc = 0.0f;
#pragma unroll
            for (int t = 0; t < AHD / 2; ++t) acc = dot2bf(kr[t], qp[t], acc);
            const bool vis = valid && pos <= L + row;
            s[j] = vis ? acc * scale : -INFINITY;
        }
        // 2. tile max, probabilities, online-softmax rescale
#pragma unroll
        for (int j = 0; j < QN; ++j) {
            float mx = s[j];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
            const float mnew = fmaxf(mrun[j], mx);
            const float pj = (s[j] == -INFINITY) ? 0.0f : expf(s[j] - mnew);
            const float alpha = (mrun[j] == -INFINITY) ? 0.0f : expf(mrun[j] - mnew);
            float ls = pj;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) ls += __shfl_xor(ls, off, 64);
            lrun[j] = lrun[j] * alpha + ls;
            o0[j] *= alpha;
            o1[j] *= alpha;
            mrun[j] = mnew;
            P[wv][lane][j] = pj;
        }
        // (LDS accesses of one wavefront execute in order: its reads below see
        // the writes above without a workgroup barrier)
        __builtin_amdgcn_wave_barrier();
        // 3. p * v with lane = dims (2 * lane, 2 * lane + 1); V rows loaded 8 at a time
        const int ntile = (int)min((int64_t)ATILE, p1 - t0);
        for (int u0 = 0; u0 < ntile; u0 += 8) {
            uint32_t vv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                vv[e] = (u0 + e < ntile) ? *((const uint32_t*)(Vh + (t0 + u0 + e) * AHD) + lane) : 0u;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (u0 + e >= ntile) break;
                const float v0 = bf16_to_f32((uint16_t)(vv[e] & 0xffffu)), v1 = bf16_to_f32((uint16_t)(vv[e] >> 16));
#pragma unroll
                for (int j = 0; j < QN; ++j) {
                    const float pj = P[wv][u0 + e][j];
                    o0[j] = fmaf(pj, v0, o0[j]);
                    o1[j] = fmaf(pj, v1, o1[j]);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();  // every wavefront is done with P before it is reused as Wo
    // merge the 4 wavefronts of the workgroup
#pragma unroll
    for (int j = 0; j < QN; ++j) {
        if (lane == 0) { Wm[wv][j] = mrun[j]; Wl[wv][j] = lrun[j]; }
        Wo[wv][j][2 * lane] = o0[j];
        Wo[wv][j][2 * lane + 1] = o1[j];
    }
    __syncthreads();
    const int nparts = gridDim.y;
    for (int idx = tid; idx < QN * AHD; idx += 256) {
        const int j = idx / AHD, d = idx % AHD;
        float mx = -INFINITY;
        for (int w = 0; w < 4; ++w) mx = fmaxf(mx, Wm[w][j]);
        float lt = 0.0f, ot = 0.0f;
        for (int w = 0; w < 4; ++w) {
            const float f = (Wm[w][j] == -INFINITY) ? 0.0f : expf(Wm[w][j] - mx);
            lt += f * Wl[w][j];
            ot += f * Wo[w][j][d];
        }
        const int64_t pi = ((int64_t)h * QN + j) * nparts + c;
        ws_o[pi * AHD + d] = ot;
        if (d == 0) { AttnPart ap; ap.m = mx; ap.l = lt; ws_ml[pi] = ap; }
    }
}

// Merge the chunk partials of one (kv head, query): grid = (QN, nkv), AHD threads.
__global__ __launch_bounds__(AHD) void attn_combine_kernel(const float* __restrict__ ws_o,
                                                           const AttnPart* __restrict__ ws_ml, int nparts, int QN, int M,
                                                           int nq, int G, uint16_t* __restrict__ out) {
    __shared__ float s_f[64], s_l[64];
    const int j = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
    const int64_t base = ((int64_t)h * QN + j) * nparts;
    // chunk maxima and sums: one chunk per thread (nparts <= 64), loads in parallel
    if (d < 64) {
        const AttnPart ap = (d < nparts) ? ws_ml[base + d] : AttnPart{-INFINITY, 0.0f};
        float mx = ap.m;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        s_f[d] = (ap.m == -INFINITY) ? 0.0f : expf(ap.m - mx);
        s_l[d] = ap.l;
    }
    __syncthreads();
    float o[64];
#pragma unroll
    for (int c = 0; c < 64; ++c) o[c] = (c < nparts) ? ws_o[(base + c) * AHD + d] : 0.0f;
    float lt = 0.0f, ot = 0.0f;
#pragma unroll
    for (int c = 0; c < 64; ++c) {
        if (c < nparts) {
            lt += s_f[c] * s_l[c];
            ot += s_f[c] * o[c];
        }
    }
    const int row = j % M, head = h * G + j / M;
    out[((int64_t)row * nq + head) * AHD + d] = f32_to_bf16(ot / lt);
}

struct AttnPlan {
    int QN, CP, nparts;
    size_t off_o, off_ml, total;
};

static AttnPlan attn_plan(int M, int nq, int nkv, int64_t ctx) {
    AttnPlan p;
    p.QN = (nq / nkv) * M;
    // chunks of >= 256 positions, at most 64 per KV head
    int64_t cp = 256;
    while ((ctx + cp - 1) / cp > 64) cp += 256;
    p.CP = (int)cp;
    p.nparts = (int)((ctx + cp - 1) / cp);
    size_t o = 0;
    p.off_o = o;
    o += (size_t)nkv * p.QN * p.nparts * AHD * sizeof(float);
    o = (o + 255) / 256 * 256;
    p.off_ml = o;
    o += (size_t)nkv * p.QN * p.nparts * sizeof(AttnPart);
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
    hipLaunchKernelGGL(add_sumsq_kernel, dim3(nch, M), dim3(NCOL), 0, st, resid, part, S, ldp, M, D, (float*)ws);
    hipLaunchKernelGGL(rmsnorm_apply_kernel, dim3(nch, M), dim3(NCOL), 0, st, resid, gamma, eps, D, (const float*)ws,
                       nch, h);
    return check_launch("vw4_add_rmsnorm");
}

int vw4_rope_kv_append(const float* part, int32_t S, int64_t ldp, int32_t M, int32_t nq, int32_t nkv, int32_t hd,
                       int32_t L, float theta, uint16_t* q_out, uint16_t* Kc, uint16_t* Vc, int64_t Lmax,
                       void* stream) {
    VW4_REQUIRE(part && q_out && Kc && Vc, VW4_EINVAL, "vw4_rope_kv_append: null pointer");
    VW4_REQUIRE(M >= 1 && M <= 64 && nq >= 1 && nkv >= 1 && hd >= 2 && hd % 2 == 0 && hd <= 2048, VW4_EINVAL,
                "vw4_rope_kv_append: bad shape");
    VW4_REQUIRE(S >= 1 && ldp >= (int64_t)(nq + 2 * nkv) * hd, VW4_EINVAL, "vw4_rope_kv_append: bad partial layout");
    VW4_REQUIRE(L >= 0 && (int64_t)L + M <= Lmax, VW4_EINVAL, "vw4_rope_kv_append: L + M exceeds the cache");
    VW4_REQUIRE(theta > 0.0f, VW4_EINVAL, "vw4_rope_kv_append: theta must be > 0");
    hipLaunchKernelGGL(rope_kv_kernel, dim3(nq + 2 * nkv, M), dim3(hd / 2), 0, (hipStream_t)stream, part, S, ldp, M,
                       nq, nkv, hd, L, (double)theta, q_out, Kc, Vc, Lmax);
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

int vw4_decode_attn(const uint16_t* q, const uint16_t* Kc, const uint16_t* Vc, int64_t Lmax, int64_t L, int32_t M,
                    int32_t nq, int32_t nkv, int32_t hd, uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
    VW4_REQUIRE(q && Kc && Vc && out, VW4_EINVAL, "vw4_decode_attn: null pointer");
    VW4_REQUIRE(hd == AHD, VW4_EUNSUPPORTED, "vw4_decode_attn: head dim %d (only 128 is built)", hd);
    VW4_REQUIRE(M >= 1 && nq >= 1 && nkv >= 1 && nq % nkv == 0, VW4_EINVAL, "vw4_decode_attn: bad head counts");
    const int QN = (nq / nkv) * M;
    VW4_REQUIRE(QN <= AQN, VW4_EUNSUPPORTED, "vw4_decode_attn: (nq/nkv)*M = %d > %d", QN, AQN);
    VW4_REQUIRE(L >= 0 && L + M <= Lmax, VW4_EINVAL, "vw4_decode_attn: L + M exceeds the cache");
    VW4_REQUIRE(aligned(Kc, 16) && aligned(Vc, 16) && aligned(q, 4), VW4_EINVAL, "vw4_decode_attn: misaligned");
    const AttnPlan p = attn_plan(M, nq, nkv, L + M);
    VW4_REQUIRE(ws && ws_bytes >= p.total && aligned(ws, 256), VW4_EWORKSPACE,
                "vw4_decode_attn: needs a 256-byte aligned workspace of %zu bytes", p.total);
    hipStream_t st = (hipStream_t)stream;
    float* wo = (float*)((char*)ws + p.off_o);
    AttnPart* wml = (AttnPart*)((char*)ws + p.off_ml);
    const float scale = 1.0f / sqrtf((float)hd);
    const int G = nq / nkv;
    const dim3 grid(nkv, p.nparts);
#define VW4_ATTN(QQ)                                                                                              \
    case QQ:                                                                                                      \
        hipLaunchKernelGGL(attn_chunk_kernel<QQ>, grid, dim3(256), 0, st, q, Kc, Vc, Lmax, L, M, nq, G, p.CP, scale, \
                           wo, wml);                                                                              \
        break;
    switch (QN) {
        VW4_ATTN(1) VW4_ATTN(2) VW4_ATTN(3) VW4_ATTN(4) VW4_ATTN(5) VW4_ATTN(6) VW4_ATTN(8) VW4_ATTN(10)
        VW4_ATTN(12) VW4_ATTN(15) VW4_ATTN(16) VW4_ATTN(20) VW4_ATTN(24) VW4_ATTN(25) VW4_ATTN(30) VW4_ATTN(32)
        VW4_ATTN(35) VW4_ATTN(40)
        default:
            set_error("vw4_decode_attn: G*M = %d has no compiled variant", QN);
            return VW4_EUNSUPPORTED;
    }
#undef VW4_ATTN
    hipLaunchKernelGGL(attn_combine_kernel, dim3(QN, nkv), dim3(AHD), 0, st, wo, wml, p.nparts, QN, M, nq, G, out);
    return check_launch("vw4_decode_attn");
}

}  // extern "C"
