// moe.hip — mixture-of-experts calls of the MoE-shaped verify step: router
// top-k with slot assignment, and the weighted combine of the expert outputs.
//
// gist.science, "BaseRT: Best-in-Class LLM Inference on Apple Silicon via
// Native Metal", section "結果": mixture-of-experts models (Qwen3-30B-A3B
// class: 128 experts, 8 active per token) are among the workloads of the
// decode runtime.  Each verify row is routed on its own: its router logits
// pick the top-k experts (largest logit first, the lower index first on equal
// logits), and the softmax weights of the chosen experts are renormalised to
// sum to one.
//
// Device-side slot list.  The distinct experts chosen by any row get slots
// 0 .. n_slots-1 in ascending expert order; the grouped W4 GEMM and the
// grouped SwiGLU launch max_slots slots and the ones at or beyond n_slots
// exit at once, so the host never reads the routing (the step stays
// capturable as a graph).  Every slot computes all M rows of its expert; the
// combine reads row m of slot row_slot[m][t] only.
#include <math.h>

#include "common.h"

namespace vw4 {

constexpr int MOE_MAX_E = 1024;
constexpr int MOE_MAX_K = 64;
constexpr int MOE_MAX_M = 16;
constexpr int MOE_KPL = MOE_MAX_E / 64;  // experts per lane

// One workgroup of 4 wavefronts; wavefront w routes rows w, w + 4, ...
// Selection key: the order-preserving fp32 key << 32 | ~index, unique per
// expert, so the top-k are the k largest keys and their order is the
// selection order.  With E <= MOE_RANK_E the keys go to LDS and every expert
// counts the keys above its own (its rank) in parallel; otherwise k rounds of
// a wavefront maximum pick them one by one.
constexpr int MOE_RANK_E = 256;
template <int KR>   // keys per lane ranked: E <= 64 * KR (rank path), 0: wavefront-maximum rounds
__global__ __launch_bounds__(256) void moe_route_kernel(const float* __restrict__ logits, int M, int E, int topk,
                                                        int32_t* __restrict__ experts, float* __restrict__ weights,
                                                        int32_t* __restrict__ slot_expert,
                                                        int32_t* __restrict__ n_slots, int32_t* __restrict__ row_slot) {
    __shared__ int32_t slot_of[MOE_MAX_E];
    __shared__ int32_t sel[MOE_MAX_M * MOE_MAX_K];
    __shared__ float sel_l[MOE_MAX_M * MOE_MAX_K];   // their logits (from the keys)
    __shared__ uint64_t s_key[4][MOE_RANK_E];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int e = tid; e < E; e += 256) slot_of[e] = 0;
    constexpr bool by_rank = KR > 0;
    // every wavefront runs the same number of row rounds (barriers inside)
    for (int m0 = 0; m0 < M; m0 += 4) {
        const int m = m0 + w;
        const bool live = m < M;
        const float* l = logits + (int64_t)(live ? m : 0) * E;
        uint64_t key[MOE_KPL];
#pragma unroll
        for (int i = 0; i < MOE_KPL; ++i) {
            const int e = lane + 64 * i;
            key[i] = e < E ? ((uint64_t)f32_key(l[e]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e) : 0;
        }
        if (by_rank) {
#pragma unroll
            for (int i = 0; i < KR; ++i)
                if (lane + 64 * i < E) s_key[w][lane + 64 * i] = key[i];
        }
        __syncthreads();
        if (live && by_rank) {
            int r[KR > 0 ? KR : 1];
#pragma unroll
            for (int i = 0; i < KR; ++i) r[i] = 0;
            int e2 = 0;
            for (; e2 + 2 <= E; e2 += 2) {     // two keys per LDS read
                const uint64_t k2a = s_key[w][e2], k2b = s_key[w][e2 + 1];
#pragma unroll
                for (int i = 0; i < KR; ++i) r[i] += (k2a > key[i] ? 1 : 0) + (k2b > key[i] ? 1 : 0);
            }
            if (e2 < E) {
#pragma unroll
                for (int i = 0; i < KR; ++i) r[i] += s_key[w][e2] > key[i] ? 1 : 0;
            }
#pragma unroll
            for (int i = 0; i < KR; ++i) {
                const int e = lane + 64 * i;
                if (e < E && r[i] < topk) {
                    sel[m * MOE_MAX_K + r[i]] = e;
                    sel_l[m * MOE_MAX_K + r[i]] = key_f32((uint32_t)(key[i] >> 32));
                    slot_of[e] = 1;
                }
            }
        } else if (live) {
            for (int t = 0; t < topk; ++t) {
                uint64_t best = 0;
#pragma unroll
                for (int i = 0; i < MOE_KPL; ++i) best = key[i] > best ? key[i] : best;
                uint64_t wb = best;
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) {
                    const uint64_t o = __shfl_xor(wb, off, 64);
                    wb = o > wb ? o : wb;
                }
                const int e = (int)(0xFFFFFFFFu - (uint32_t)wb);
#pragma unroll
                for (int i = 0; i < MOE_KPL; ++i)
                    if (key[i] == wb) key[i] = 0;
                if (lane == 0) {
                    sel[m * MOE_MAX_K + t] = e;
                    sel_l[m * MOE_MAX_K + t] = key_f32((uint32_t)(wb >> 32));
                    slot_of[e] = 1;
                }
            }
        }
        __syncthreads();
        if (live) {
            // weights: exp(l_e - l_top) in fp64 (l_top = the largest logit,
            // chosen first), normalised over the chosen experts in selection order
            const double top = (double)sel_l[m * MOE_MAX_K];
            const double pe = lane < topk ? exp((double)sel_l[m * MOE_MAX_K + lane] - top) : 0.0;
            double den = 0.0;
            for (int t = 0; t < topk; ++t) den += __shfl(pe, t, 64);
            if (lane < topk) weights[m * topk + lane] = (float)(pe / den);
        }
    }
    __syncthreads();
    // slots in ascending expert order: wavefront 0 counts the chosen experts
    // 64 at a time (ballot + popcount)
    if (w == 0) {
        int base = 0;
        for (int e0 = 0; e0 < E; e0 += 64) {
            const int e = e0 + lane;
            const bool chosen = e < E && slot_of[e] != 0;
            const uint64_t mask = __ballot(chosen);
            if (chosen) {
                const int s = base + __popcll(mask & ((1ull << lane) - 1ull));
                slot_expert[s] = e;
                slot_of[e] = s;
            }
            base += __popcll(mask);
        }
        if (lane == 0) *n_slots = base;
    }
    __syncthreads();
    for (int i = tid; i < M * topk; i += 256) {
        const int e = sel[(i / topk) * MOE_MAX_K + i % topk];
        experts[i] = e;
        row_slot[i] = slot_of[e];
    }
}

// y[m][d] = sum_t weights[m][t] * sum_s part[row_slot[m][t]][s][m][d]
// (experts in selection order, slices in slice order, fp32).
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ part, int S, int64_t ldp,
                                                          int64_t p_sstride, const int32_t* __restrict__ row_slot,
                                                          const float* __restrict__ weights, int M, int topk, int D,
                                                          float* __restrict__ y, int64_t ldy) {
    const int d = blockIdx.x * 256 + threadIdx.x, m = blockIdx.y;
    if (d >= D) return;
    float acc = 0.0f;
    for (int t0 = 0; t0 < topk; t0 += 8) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = t0 + i < topk
                       ? sum_parts(part + (int64_t)row_slot[m * topk + t0 + i] * p_sstride, S, M, ldp, m, d)
                       : 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (t0 + i < topk) acc += weights[m * topk + t0 + i] * v[i];
    }
    y[(int64_t)m * ldy + d] = acc;
}

}  // namespace vw4

using namespace vw4;

extern "C" {

int vw4_moe_route(const float* logits, int32_t M, int32_t E, int32_t topk, int32_t* experts, float* weights,
                  int32_t* slot_expert, int32_t* n_slots, int32_t* row_slot, void* stream) {
    VW4_REQUIRE(logits && experts && weights && slot_expert && n_slots && row_slot, VW4_EINVAL,
                "vw4_moe_route: null pointer");
    VW4_REQUIRE(M >= 1 && M <= MOE_MAX_M && E >= 1 && E <= MOE_MAX_E && topk >= 1 && topk <= MOE_MAX_K && topk <= E,
                VW4_EINVAL, "vw4_moe_route: need 1 <= M <= %d, 1 <= topk <= min(E, %d), E <= %d", MOE_MAX_M,
                MOE_MAX_K, MOE_MAX_E);
    hipStream_t st = (hipStream_t)stream;
    if (E <= 64)
        hipLaunchKernelGGL(moe_route_kernel<1>, dim3(1), dim3(256), 0, st, logits, M, E, topk, experts, weights,
                           slot_expert, n_slots, row_slot);
    else if (E <= 128)
        hipLaunchKernelGGL(moe_route_kernel<2>, dim3(1), dim3(256), 0, st, logits, M, E, topk, experts, weights,
                           slot_expert, n_slots, row_slot);
    else if (E <= MOE_RANK_E)
        hipLaunchKernelGGL(moe_route_kernel<4>, dim3(1), dim3(256), 0, st, logits, M, E, topk, experts, weights,
                           slot_expert, n_slots, row_slot);
    else
        hipLaunchKernelGGL(moe_route_kernel<0>, dim3(1), dim3(256), 0, st, logits, M, E, topk, experts, weights,
                           slot_expert, n_slots, row_slot);
    return check_launch("vw4_moe_route");
}

int vw4_moe_combine(const float* part, int32_t S, int64_t ldp, int64_t p_sstride, const int32_t* row_slot,
                    const float* weights, int32_t M, int32_t topk, int32_t D, float* y, int64_t ldy, void* stream) {
    VW4_REQUIRE(part && row_slot && weights && y, VW4_EINVAL, "vw4_moe_combine: null pointer");
    VW4_REQUIRE(M >= 1 && M <= 64 && topk >= 1 && D >= 1 && S >= 1 && ldp >= D && ldy >= D &&
                    p_sstride >= (int64_t)S * M * ldp,
                VW4_EINVAL, "vw4_moe_combine: bad shape or strides");
    hipLaunchKernelGGL(moe_combine_kernel, dim3((D + 255) / 256, M), dim3(256), 0, (hipStream_t)stream, part, S, ldp,
                       p_sstride, row_slot, weights, M, topk, D, y, ldy);
    return check_launch("vw4_moe_combine");
}

}  // extern "C"
