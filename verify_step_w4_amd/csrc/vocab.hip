// vocab.hip — verify_logits: LM-head GEMM of the verify rows, then the
// temperature / top-p statistics of every row.
//
// devtrends.cc, "Apple Silicon上でローカルLLMを最大2倍高速化するMTPLX", section
// "2つ目のモデル不要！MTPの裏技": the target distribution is sampled at
// temperature 0.6 with top_p 0.95, and the verify step must reproduce it exactly.
//
// Definition computed (per row of fp32 logits z, temperature T, top_p):
//   m = max z;  e_j = exp((z_j - m)/T) (fp64);  E = sum e_j
//   tau = the largest logit t with  sum_{z_j >= t} e_j >= top_p * E
//       (= the logit at which the prefix of the vocabulary sorted by
//        (logit desc, index asc) first reaches top_p * E)
//   kept set = { j : z_j >= tau },  Z = sum over the kept set,  log_z = log Z.
//   T == 0: greedy (argmax, lowest index on ties); top_p >= 1: everything kept.
//
// MI355X design: no sort.  Each row is split over P workgroups; tau is found
// by a radix descent on the order-preserving 32-bit key of the logits with
// fp64 mass histograms (11 + 11 + 10 key bits, one kernel per level, LDS
// histograms per workgroup).  Each level's workgroup histograms are combined
// by the last workgroup of the row to arrive (integer counter), in workgroup
// order.  A final pass recomputes E, Z, the mass strictly above tau and n_kept
// with fixed-order reductions, so every statistic is reproducible bit for bit;
// the histogram atomics only steer the descent and can matter only when the
// boundary mass is within rounding of top_p * E, which the final pass flags.
#include <math.h>

#include "common.h"

namespace vw4 {

constexpr int VT = 256;            // threads per workgroup
constexpr int VCHUNK = 4096;       // logits per workgroup (grown for huge V)
constexpr int VMAXP = 64;          // workgroups per row at most
constexpr int L1BITS = 11, L2BITS = 11, L3BITS = 10;
constexpr int HBINS = 2048;

struct RowState {
    float m;            // row max
    int32_t argmax;
    double E;           // sum of e over the row (descent target base)
    double target;      // top_p * E
    double above;       // mass of keys above the current prefix range
    uint32_t prefix;    // key prefix fixed so far
    uint32_t done;      // 1: statistics already final (T == 0 or non-finite)
    uint32_t flags;
    uint32_t pad;
};

struct WgPart {            // per-workgroup partial results
    float m;
    int32_t argmax;
    uint32_t bad;
    uint32_t n;
    double E;
    double Z;
    double gt;
    float mn;
    uint32_t pad;
};

struct VocabLayout {
    int P, chunk;
    size_t off_state, off_part, off_hist, off_cnt, total;
};

static VocabLayout vocab_layout(int rows, int V) {
    VocabLayout L;
    int P = ceil_div(V, VCHUNK);
    int chunk = VCHUNK;
    if (P > VMAXP) {
        chunk = ceil_div(ceil_div(V, VMAXP), VT) * VT;
        P = ceil_div(V, chunk);
    }
    L.P = P;
    L.chunk = chunk;
    size_t o = 0;
    L.off_state = o;
    o += (size_t)rows * sizeof(RowState);
    o = (o + 255) / 256 * 256;
    L.off_part = o;
    o += (size_t)rows * P * sizeof(WgPart);
    o = (o + 255) / 256 * 256;
    L.off_hist = o;
    o += (size_t)rows * P * HBINS * sizeof(double);
    L.off_cnt = o;
    o += (size_t)rows * 4 * sizeof(uint32_t);
    L.total = (o + 255) / 256 * 256;
    return L;
}

// ---------------------------------------------------------------------------
// Block-level helpers (256 threads, fixed combination order).
// ---------------------------------------------------------------------------
__device__ __forceinline__ double block_sum_f64(double v, double* sh) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    double s = sh[0] + sh[1] + sh[2] + sh[3];
    __syncthreads();
    return s;
}

__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, uint32_t* sh) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    uint32_t s = sh[0] + sh[1] + sh[2] + sh[3];
    __syncthreads();
    return s;
}

// Exclusive suffix sum over threads: returns sum_{t' > t} v_{t'}.
__device__ __forceinline__ double block_suffix_excl_f64(double v, double* sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    double s = v;  // inclusive suffix within the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double t = __shfl_down(s, off, 64);
        if (lane + off < 64) s += t;
    }
    if (lane == 0) sh[w] = s;
    __syncthreads();
    double later = 0.0;
    for (int w2 = 3; w2 > w; --w2) later += sh[w2];
    double ex = __shfl_down(s, 1, 64);
    if (lane == 63) ex = 0.0;
    __syncthreads();
    return ex + later;
}

// Last workgroup of a row to finish (release/acquire around an integer counter).
__device__ __forceinline__ bool arrive_last(uint32_t* cnt, uint32_t total, int* sh_flag) {
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) *sh_flag = (atomicAdd(cnt, 1u) == total - 1u);
    __syncthreads();
    const bool last = *sh_flag != 0;
    if (last) __threadfence();
    return last;
}

// Find, among HBINS combined bins (8 per thread, ascending key), the largest
// bin b with  above + sum_{b' >= b} H[b'] >= target.  Returns b (or -1) and
// the mass above it in *new_above.  nb = number of valid bins.
__device__ int descend_bins(const double* H, int nb, double above, double target, double* new_above, double* sh,
                            int* shi) {
    const int per = HBINS / VT;  // 8
    const int b0 = threadIdx.x * per;
    double mine = 0.0;
    for (int i = 0; i < per; ++i)
        if (b0 + i < nb) mine += H[b0 + i];
    const double later = block_suffix_excl_f64(mine, sh);
    if (threadIdx.x == 0) *shi = -1;
    __syncthreads();
    double cum = above + later;  // mass of all bins above this thread's range
    for (int i = per - 1; i >= 0; --i) {
        const int b = b0 + i;
        if (b >= nb) continue;
        const double h = H[b];
        if (cum < target && cum + h >= target) {
            *shi = b;  // exactly one bin can satisfy this (cum is monotone)
            sh[8] = cum;
        }
        cum += h;
    }
    __syncthreads();
    const int b = *shi;
    *new_above = (b >= 0) ? sh[8] : above;
    __syncthreads();
    return b;
}

// ---------------------------------------------------------------------------
// Level 1: max / argmax / non-finite check, local e relative to the
// workgroup max, level-1 histogram; the last workgroup combines.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(VT) void stats_level1_kernel(const float* __restrict__ logits, int V, int chunk, int P,
                                                          float temperature, float top_p, char* __restrict__ ws,
                                                          VocabLayout L, vw4_rowstat* __restrict__ stats) {
    __shared__ double hist[HBINS];
    __shared__ double shd[16];
    __shared__ float shf[4];
    __shared__ int shi[4];
    __shared__ int sflag;
    const int w = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
    const float* z = logits + (int64_t)r * V;
    const int c0 = w * chunk, c1 = min(V, c0 + chunk);
    RowState* state = (RowState*)(ws + L.off_state) + r;
    WgPart* parts = (WgPart*)(ws + L.off_part) + (int64_t)r * P;
    double* hists = (double*)(ws + L.off_hist) + (int64_t)r * P * HBINS;
    uint32_t* cnt = (uint32_t*)(ws + L.off_cnt) + r * 4;
    const double T = (double)temperature;

    float lm = -INFINITY;
    int li = 0x7fffffff;
    uint32_t bad = 0;
    for (int j = c0 + tid; j < c1; j += VT) {
        const float v = z[j];
        if (!isfinite(v)) bad = 1;
        if (v > lm || (v == lm && j < li)) { lm = v; li = j; }
    }
    // block max with lowest index on ties
    for (int off = 32; off > 0; off >>= 1) {
        const float om = __shfl_xor(lm, off, 64);
        const int oi = __shfl_xor(li, off, 64);
        if (om > lm || (om == lm && oi < li)) { lm = om; li = oi; }
    }
    if ((tid & 63) == 0) { shf[tid >> 6] = lm; shi[tid >> 6] = li; }
    __syncthreads();
    float m_w = shf[0];
    int a_w = shi[0];
    for (int k = 1; k < 4; ++k)
        if (shf[k] > m_w || (shf[k] == m_w && shi[k] < a_w)) { m_w = shf[k]; a_w = shi[k]; }
    __syncthreads();
    const uint32_t bad_w = block_sum_u32(bad, (uint32_t*)shi) != 0;

    double E_w = 0.0;
    const bool need_mass = T > 0.0 && !bad_w && top_p < 1.0f;
    if (T > 0.0 && !bad_w) {
        for (int b = tid; b < HBINS; b += VT) hist[b] = 0.0;
        __syncthreads();
        double es = 0.0;
        for (int j = c0 + tid; j < c1; j += VT) {
            const float v = z[j];
            const double e = exp(((double)v - (double)m_w) / T);
            es += e;
            if (need_mass) atomicAdd(&hist[f32_key(v) >> (32 - L1BITS)], e);
        }
        E_w = block_sum_f64(es, shd);
        if (need_mass)
            for (int b = tid; b < HBINS; b += VT) hists[(int64_t)w * HBINS + b] = hist[b];
    }
    if (tid == 0) {
        WgPart p;
        p.m = m_w; p.argmax = a_w; p.bad = bad_w; p.n = 0; p.E = E_w; p.Z = 0; p.gt = 0; p.mn = 0; p.pad = 0;
        parts[w] = p;
    }
    if (!arrive_last(&cnt[0], (uint32_t)P, &sflag)) return;

    // ---- last workgroup of the row: combine in workgroup order ----
    float m = parts[0].m;
    int a = parts[0].argmax;
    uint32_t anybad = parts[0].bad;
    for (int k = 1; k < P; ++k) {
        anybad |= parts[k].bad;
        if (parts[k].m > m) { m = parts[k].m; a = parts[k].argmax; }  // chunks ascend: first max is lowest index
    }
    if (tid == 0) cnt[0] = 0u;
    if (anybad || T == 0.0) {
        if (tid == 0) {
            vw4_rowstat s;
            s.max_logit = anybad ? NAN : m;
            s.tau = s.max_logit;
            s.log_z = 0.0;
            s.argmax = anybad ? -1 : a;
            s.n_kept = anybad ? 0 : 1;
            s.flags = anybad ? VW4_FLAG_NONFINITE : 0u;
            s.pad = 0;
            stats[r] = s;
            RowState st = {};
            st.m = m; st.argmax = a; st.done = 1; st.flags = s.flags;
            *state = st;
        }
        return;
    }
    __shared__ double fk[VMAXP];  // rescale factors exp((m_k - m)/T) of the workgroup partials
    for (int k = tid; k < P; k += VT) fk[k] = exp(((double)parts[k].m - (double)m) / T);
    __syncthreads();
    double E = 0.0;
    for (int k = 0; k < P; ++k) E += fk[k] * parts[k].E;
    const double target = (double)top_p * E;
    RowState st = {};
    st.m = m; st.argmax = a; st.E = E; st.target = target; st.done = 0; st.flags = 0;
    if (!need_mass) {
        st.prefix = 0; st.above = 0.0;
        if (tid == 0) *state = st;
        return;
    }
    // combined level-1 histogram, then the descent
    for (int b = tid; b < HBINS; b += VT) {
        double h = 0.0;
        for (int k = 0; k < P; ++k) h += fk[k] * hists[(int64_t)k * HBINS + b];
        hist[b] = h;
    }
    __syncthreads();
    double above;
    int b1 = descend_bins(hist, 1 << L1BITS, 0.0, target, &above, shd, &shi[0]);
    if (b1 < 0) {  // rounding left the target unreached: take the lowest non-empty bin
        for (int b = 0; b < HBINS; ++b) if (hist[b] > 0.0) { b1 = b; break; }
        above = 0.0;
        for (int b = b1 + 1; b < HBINS; ++b) above += hist[b];
        st.flags |= VW4_FLAG_TOPP_TIE;
    }
    st.prefix = (uint32_t)b1;
    st.above = above;
    if (tid == 0) *state = st;
}

// Levels 2 and 3: histogram of the next key bits among the logits whose key
// matches the prefix fixed so far; the last workgroup extends the prefix.
template <int SHIFT, int BITS>
__global__ __launch_bounds__(VT) void stats_level_kernel(const float* __restrict__ logits, int V, int chunk, int P,
                                                         float temperature, char* __restrict__ ws, VocabLayout L,
                                                         int cnt_slot) {
    __shared__ double hist[HBINS];
    __shared__ double shd[16];
    __shared__ int shi[4];
    __shared__ int sflag;
    const int w = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
    RowState* state = (RowState*)(ws + L.off_state) + r;
    const RowState st = *state;
    if (st.done || st.target <= 0.0) return;
    const float* z = logits + (int64_t)r * V;
    const int c0 = w * chunk, c1 = min(V, c0 + chunk);
    double* hists = (double*)(ws + L.off_hist) + (int64_t)r * P * HBINS;
    uint32_t* cnt = (uint32_t*)(ws + L.off_cnt) + r * 4 + cnt_slot;
    const double T = (double)temperature;
    const int nb = 1 << BITS;
    for (int b = tid; b < nb; b += VT) hist[b] = 0.0;
    __syncthreads();
    for (int j = c0 + tid; j < c1; j += VT) {
        const float v = z[j];
        const uint32_t k = f32_key(v);
        if ((k >> (SHIFT + BITS)) == st.prefix)
            atomicAdd(&hist[(k >> SHIFT) & (uint32_t)(nb - 1)], exp(((double)v - (double)st.m) / T));
    }
    __syncthreads();
    for (int b = tid; b < nb; b += VT) hists[(int64_t)w * HBINS + b] = hist[b];
    if (!arrive_last(cnt, (uint32_t)P, &sflag)) return;
    if (tid == 0) *cnt = 0u;
    for (int b = tid; b < HBINS; b += VT) {
        double h = 0.0;
        if (b < nb)
            for (int k = 0; k < P; ++k) h += hists[(int64_t)k * HBINS + b];
        hist[b] = h;
    }
    __syncthreads();
    double above;
    int bb = descend_bins(hist, nb, st.above, st.target, &above, shd, &shi[0]);
    RowState ns = st;
    if (bb < 0) {
        for (int b = 0; b < nb; ++b) if (hist[b] > 0.0) { bb = b; break; }
        if (bb < 0) bb = 0;
        above = st.above;
        for (int b = bb + 1; b < nb; ++b) above += hist[b];
        ns.flags |= VW4_FLAG_TOPP_TIE;
    }
    ns.prefix = (st.prefix << BITS) | (uint32_t)bb;
    ns.above = above;
    if (tid == 0) *state = ns;
}

// Final pass: fixed-order sums over the row with the global max and the
// selected cutoff; writes the row statistics.
__global__ __launch_bounds__(VT) void stats_final_kernel(const float* __restrict__ logits, int V, int chunk, int P,
                                                         float temperature, float top_p, char* __restrict__ ws,
                                                         VocabLayout L, vw4_rowstat* __restrict__ stats) {
    __shared__ double shd[16];
    __shared__ uint32_t shu[4];
    __shared__ float shf[4];
    __shared__ int sflag;
    const int w = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
    RowState* state = (RowState*)(ws + L.off_state) + r;
    const RowState st = *state;
    if (st.done) return;
    const float* z = logits + (int64_t)r * V;
    const int c0 = w * chunk, c1 = min(V, c0 + chunk);
    WgPart* parts = (WgPart*)(ws + L.off_part) + (int64_t)r * P;
    uint32_t* cnt = (uint32_t*)(ws + L.off_cnt) + r * 4 + 3;
    const double T = (double)temperature;
    const bool keep_all = !(top_p < 1.0f);
    const float tau = keep_all ? -INFINITY : key_f32(st.prefix);
    double se = 0.0, sz = 0.0, sg = 0.0;
    uint32_t n = 0;
    float mn = INFINITY;
    for (int j = c0 + tid; j < c1; j += VT) {
        const float v = z[j];
        const double e = exp(((double)v - (double)st.m) / T);
        se += e;
        mn = fminf(mn, v);
        if (v >= tau) { sz += e; ++n; }
        if (v > tau) sg += e;
    }
    se = block_sum_f64(se, shd);
    sz = block_sum_f64(sz, shd);
    sg = block_sum_f64(sg, shd);
    n = block_sum_u32(n, shu);
    for (int off = 32; off > 0; off >>= 1) mn = fminf(mn, __shfl_xor(mn, off, 64));
    if ((tid & 63) == 0) shf[tid >> 6] = mn;
    __syncthreads();
    mn = fminf(fminf(shf[0], shf[1]), fminf(shf[2], shf[3]));
    if (tid == 0) {
        WgPart p = parts[w];
        p.E = se; p.Z = sz; p.gt = sg; p.n = n; p.mn = mn;
        parts[w] = p;
    }
    if (!arrive_last(cnt, (uint32_t)P, &sflag)) return;
    if (tid != 0) return;
    *cnt = 0u;
    double E = 0.0, Z = 0.0, G = 0.0;
    uint32_t nk = 0;
    float rmin = INFINITY;
    for (int k = 0; k < P; ++k) {
        E += parts[k].E; Z += parts[k].Z; G += parts[k].gt; nk += parts[k].n;
        rmin = fminf(rmin, parts[k].mn);
    }
    uint32_t flags = st.flags;
    if (!keep_all) {
        const double Pt = (double)top_p * E;
        if (fabs(Z - Pt) < 1e-9 * E || fabs(G - Pt) < 1e-9 * E || !(G < Pt && Z >= Pt)) flags |= VW4_FLAG_TOPP_TIE;
    }
    vw4_rowstat s;
    s.max_logit = st.m;
    s.tau = keep_all ? rmin : tau;
    s.log_z = log(Z);
    s.argmax = st.argmax;
    s.n_kept = (int32_t)nk;
    s.flags = flags;
    s.pad = 0;
    stats[r] = s;
}

int gemm_dispatch(const uint16_t* x, int64_t ldx, const uint8_t* w, const uint16_t* s, void* y, int64_t ldy, int ydt,
                  int M, int N, int K, void* ws, size_t ws_bytes, hipStream_t st);
size_t gemm_ws_bytes(int M, int N, int K);

}  // namespace vw4

using namespace vw4;

extern "C" {

size_t vw4_workspace_bytes(int32_t rows, int32_t V) {
    if (rows < 1 || rows > 64 || V < 1 || V > (1 << 24)) return 0;
    return vocab_layout(rows, V).total;
}

int verify_logits(const uint16_t* hidden, int64_t ldh, const uint8_t* lm_packed, const uint16_t* lm_scales, int32_t rows,
                  int32_t V, int32_t d, float temperature, float top_p, float* logits, vw4_rowstat* stats, void* ws,
                  size_t ws_bytes, void* stream) {
    VW4_REQUIRE(rows >= 1 && rows <= 64, VW4_EINVAL, "verify_logits: rows=%d must be in [1, 64]", rows);
    VW4_REQUIRE(V >= 1 && V <= (1 << 24), VW4_EINVAL, "verify_logits: V=%d out of range", V);
    VW4_REQUIRE(isfinite(temperature) && temperature >= 0.0f, VW4_EINVAL, "verify_logits: temperature must be >= 0");
    VW4_REQUIRE(top_p > 0.0f && top_p <= 1.0f, VW4_EINVAL, "verify_logits: top_p must be in (0, 1]");
    VW4_REQUIRE(logits && stats, VW4_EINVAL, "verify_logits: null logits/stats");
    const VocabLayout L = vocab_layout(rows, V);
    VW4_REQUIRE(ws && ws_bytes >= L.total && aligned(ws, 256), VW4_EWORKSPACE,
                "verify_logits: needs a 256-byte aligned workspace of %zu bytes", L.total);
    hipStream_t st = (hipStream_t)stream;
    if (hidden) {
        VW4_REQUIRE(rows <= 8, VW4_EINVAL, "verify_logits: the LM-head GEMM takes at most 8 rows");
        VW4_REQUIRE(lm_packed && lm_scales, VW4_EINVAL, "verify_logits: null LM-head weights");
        // The GEMM's split-K scratch lives after the statistics' workspace.
        const size_t gws = gemm_ws_bytes(rows, V, d);
        VW4_REQUIRE(ws_bytes >= L.total + gws, VW4_EWORKSPACE,
                    "verify_logits: needs %zu workspace bytes with the LM-head GEMM", L.total + gws);
        int rc = gemm_dispatch(hidden, ldh, lm_packed, lm_scales, logits, V, VW4_F32, rows, V, d,
                               gws ? (char*)ws + L.total : nullptr, gws, st);
        if (rc) return rc;
    }
    const dim3 grid(L.P, rows);
    hipLaunchKernelGGL(stats_level1_kernel, grid, dim3(VT), 0, st, logits, V, L.chunk, L.P, temperature, top_p,
                       (char*)ws, L, stats);
    if (temperature > 0.0f) {
        if (top_p < 1.0f) {
            hipLaunchKernelGGL((stats_level_kernel<L3BITS, L2BITS>), grid, dim3(VT), 0, st, logits, V, L.chunk, L.P,
                               temperature, (char*)ws, L, 1);
            hipLaunchKernelGGL((stats_level_kernel<0, L3BITS>), grid, dim3(VT), 0, st, logits, V, L.chunk, L.P,
                               temperature, (char*)ws, L, 2);
        }
        hipLaunchKernelGGL(stats_final_kernel, grid, dim3(VT), 0, st, logits, V, L.chunk, L.P, temperature, top_p,
                           (char*)ws, L, stats);
    }
    return check_launch("verify_logits");
}

}  // extern "C"
