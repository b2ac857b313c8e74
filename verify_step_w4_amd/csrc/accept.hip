// accept.hip — spec_accept: Leviathan–Chen acceptance of the drafts, residual
// resampling at the first rejection, bonus token when every draft survives.
//
// hazakura.dev, "mtplx——M5 Maxで63tok/s…", section "4層のアーキテクチャ", Layer 2
// (probability-ratio acceptance -> residual correction -> bonus token) and
// section "mtplxの数字——本当なの？" (Leviathan–Chen rejection at T = 0.6, output
// law identical to the target); devtrends.cc, "…MTPLX", section
// "2つ目のモデル不要！MTPの裏技" (exact rejection sampling with residual correction).
//
// Per problem (M = D + 1 rows):
//   u_acc[i], u_res[i] from Philox4x64-10 (Salmon et al., SC'11),
//     key (seed, 0), counter (step, i, 0, 0): u = (r >> 11) * 2^-53 of words 0, 1
//   for i < D: accept x_i iff u_acc[i] * q_i(x_i) < p_i(x_i); first failure -> k
//   r = max(0, p_k - q_k) if k < D, r = p_D if k == D;  R = sum r
//   y = min{ j : C_j > u_res[k] * R },  C the running sum in index order
// p_i(j) = exp((z_ij - m_i)/T - log_z_i) on the kept set (z_ij >= tau_i), 0
// elsewhere; T == 0 makes p_i one-hot at the argmax.
//
// MI355X design: one launch.  Problem b's residual row is split over P
// workgroups (grid = (B, P)); every workgroup redoes the D accept tests (D <= 7
// scalar fp64 evaluations) so no extra launch is needed for them, computes
// fp64 chunk sums of r in a fixed order, and the last workgroup of the problem
// (integer counter) locates the chunk holding u * R, rescans that chunk with a
// block-wide fp64 prefix sum in index order, and writes the tokens.
#include <math.h>

#include "common.h"

namespace vw4 {

constexpr int AT = 256;          // threads per workgroup for large vocabularies
constexpr int ACHUNK = 4096;     // vocabulary entries per workgroup
constexpr int AMAXP = 64;
constexpr int AMAXD = 7;

struct AcceptPart {
    double r;       // chunk sum of the residual r
    double p;       // chunk sum of p_k (fallback when R == 0)
    int32_t last_r; // last index in the chunk with r > 0 (-1 if none)
    int32_t last_p; // last index with p_k > 0
};

struct AcceptLayout {
    int P, chunk, threads;
    size_t off_part, off_cnt, total;
};

static AcceptLayout accept_layout(int B, int V) {
    AcceptLayout L;
    if (V <= 1024) {
        L.P = 1;
        L.chunk = V;
        L.threads = 64;
    } else {
        L.threads = AT;
        L.chunk = ACHUNK;
        L.P = ceil_div(V, ACHUNK);
        if (L.P > AMAXP) {
            L.chunk = ceil_div(ceil_div(V, AMAXP), AT) * AT;
            L.P = ceil_div(V, L.chunk);
        }
    }
    size_t o = 0;
    L.off_part = o;
    o += (size_t)B * L.P * sizeof(AcceptPart);
    o = (o + 255) / 256 * 256;
    L.off_cnt = o;
    o += (size_t)B * sizeof(uint32_t);
    L.total = (o + 255) / 256 * 256;
    return L;
}

// ---------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): each round multiplies
// counter words 0 and 2 by the round multipliers (64x64 -> 128 bits), xors the
// high halves with the other two words and the round key, and permutes; the
// key advances by the Weyl increments between rounds.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void philox4x64_10(uint64_t k0, uint64_t k1, uint64_t c[4]) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
        const uint64_t hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
        const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
        k0 += W0;
        k1 += W1;
    }
}

__device__ __forceinline__ double unit53(uint64_t r) { return (double)(r >> 11) * 0x1.0p-53; }

__device__ __forceinline__ double p_of(const float* __restrict__ z, const vw4_rowstat& s, double T, int j) {
    if (T == 0.0) return (j == s.argmax) ? 1.0 : 0.0;
    const float v = z[j];
    if (!(v >= s.tau)) return 0.0;
    return exp(((double)v - (double)s.max_logit) / T - s.log_z);
}

template <int NT>
__device__ __forceinline__ double blk_sum(double v, double* sh) {
    v = wave_sum(v);
    if (NT == 64) return v;
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    double s = sh[0];
    for (int k = 1; k < NT / 64; ++k) s += sh[k];
    __syncthreads();
    return s;
}

template <int NT>
__device__ __forceinline__ int blk_max_i(int v, int* sh) {
    for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
    if (NT == 64) return v;
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    int s = sh[0];
    for (int k = 1; k < NT / 64; ++k) s = max(s, sh[k]);
    __syncthreads();
    return s;
}

// Exclusive prefix sum over threads in thread order (fixed combination order).
template <int NT>
__device__ __forceinline__ double blk_prefix_excl(double v, double* sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    double s = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double t = __shfl_up(s, off, 64);
        if (lane >= off) s += t;
    }
    double ex = __shfl_up(s, 1, 64);
    if (lane == 0) ex = 0.0;
    if (NT == 64) return ex;
    if (lane == 63) sh[w] = s;
    __syncthreads();
    double before = 0.0;
    for (int k = 0; k < w; ++k) before += sh[k];
    __syncthreads();
    return ex + before;
}

template <int NT>
__global__ __launch_bounds__(NT) void spec_accept_kernel(const float* __restrict__ logits, int64_t lstride,
                                                         const vw4_rowstat* __restrict__ stats, int64_t sstride,
                                                         const float* __restrict__ q, int64_t qstride,
                                                         const int32_t* __restrict__ draft, int D, int V,
                                                         float temperature, uint64_t seed, uint64_t step0, int chunk,
                                                         int P, int32_t* __restrict__ out_tokens,
                                                         int32_t* __restrict__ out_nacc, uint32_t* __restrict__ out_flags,
                                                         AcceptPart* __restrict__ parts, uint32_t* __restrict__ cnts) {
    __shared__ double sh[8];
    __shared__ int shi[8];
    __shared__ int s_last, s_y;
    __shared__ double s_u[2 * (AMAXD + 1)];
    const int64_t b = blockIdx.x;
    const int w = blockIdx.y, tid = threadIdx.x;
    const float* zb = logits + b * lstride;
    const vw4_rowstat* sb = stats + b * sstride;
    const float* qb = q ? q + b * qstride : nullptr;
    const int32_t* db = draft + b * D;
    const double T = (double)temperature;

    // uniforms of rows 0..D (thread i computes row i)
    if (tid <= D) {
        uint64_t c[4] = {step0 + (uint64_t)b, (uint64_t)tid, 0, 0};
        philox4x64_10(seed, 0, c);
        s_u[2 * tid] = unit53(c[0]);
        s_u[2 * tid + 1] = unit53(c[1]);
    }
    __syncthreads();

    uint32_t flags = 0;
    bool bad = false;
    for (int i = 0; i <= D; ++i) {
        const uint32_t f = sb[i].flags;
        if (f & VW4_FLAG_NONFINITE) bad = true;
        if (f & VW4_FLAG_TOPP_TIE) flags |= VW4_FLAG_TOPP_TIE;
    }
    if (bad) {
        if (w == 0 && tid <= D) out_tokens[b * (D + 1) + tid] = -1;
        if (w == 0 && tid == 0) {
            out_nacc[b] = -1;
            out_flags[b] = VW4_FLAG_NONFINITE;
        }
        return;
    }
    // accept tests (identical in every workgroup and thread)
    int k = D;
    for (int i = 0; i < D; ++i) {
        const int x = db[i];
        if (x < 0 || x >= V) { k = i; break; }  // malformed draft id: rejected, never dereferenced
        const double pi = p_of(zb + (int64_t)i * V, sb[i], T, x);
        const double qi = (double)qb[(int64_t)i * V + x];
        const double u = s_u[2 * i];
        if (qi > 0.0 && fabs(u - pi / qi) < 1e-5) flags |= VW4_FLAG_ACCEPT_TIE;
        if (!(u * qi < pi)) { k = i; break; }
    }
    const float* zk = zb + (int64_t)k * V;
    const vw4_rowstat sk = sb[k];
    const float* qk = (k < D) ? qb + (int64_t)k * V : nullptr;

    // chunk sums of r and p_k in a fixed order
    const int c0 = w * chunk, c1 = min(V, c0 + chunk);
    double sr = 0.0, sp = 0.0;
    int lr = -1, lp = -1;
    for (int j = c0 + tid; j < c1; j += NT) {
        const double pj = p_of(zk, sk, T, j);
        double rj = pj;
        if (qk) rj = fmax(0.0, pj - (double)qk[j]);
        sr += rj;
        sp += pj;
        if (rj > 0.0) lr = j;
        if (pj > 0.0) lp = j;
    }
    sr = blk_sum<NT>(sr, sh);
    sp = blk_sum<NT>(sp, sh);
    lr = blk_max_i<NT>(lr, shi);
    lp = blk_max_i<NT>(lp, shi);
    AcceptPart* pb = parts + b * P;
    if (tid == 0) {
        AcceptPart a;
        a.r = sr; a.p = sp; a.last_r = lr; a.last_p = lp;
        pb[w] = a;
    }
    if (P > 1) {
        __threadfence();
        __syncthreads();
        if (tid == 0) s_last = (atomicAdd(&cnts[b], 1u) == (uint32_t)(P - 1));
        __syncthreads();
        if (!s_last) return;
        __threadfence();
        if (tid == 0) cnts[b] = 0u;
    } else {
        __syncthreads();
    }

    // ---- last workgroup of problem b: locate u * R and sample ----
    bool use_p = false;
    double R = 0.0;
    for (int c = 0; c < P; ++c) R += pb[c].r;
    if (!(R > 0.0)) {
        use_p = true;
        flags |= VW4_FLAG_R_ZERO;
        R = 0.0;
        for (int c = 0; c < P; ++c) R += pb[c].p;
    }
    const double target = s_u[2 * k + 1] * R;
    int wc = -1;
    double before = 0.0, cum = 0.0;
    int last_any = -1;
    for (int c = 0; c < P; ++c) {
        const double m = use_p ? pb[c].p : pb[c].r;
        const int lst = use_p ? pb[c].last_p : pb[c].last_r;
        if (lst >= 0) last_any = lst;
        if (wc < 0 && cum + m > target) { wc = c; before = cum; }
        cum += m;
    }
    int y = -1;
    double cprev = 0.0, cy = 0.0;
    bool found = false;
    if (wc >= 0) {
        // rescan chunk wc: thread t owns a contiguous run of the chunk
        const int a0 = wc * chunk, a1 = min(V, a0 + chunk);
        const int per = (a1 - a0 + NT - 1) / NT;
        const int j0 = a0 + tid * per, j1 = min(a1, j0 + per);
        double mine = 0.0;
        for (int j = j0; j < j1; ++j) {
            const double pj = p_of(zk, sk, T, j);
            mine += (use_p || !qk) ? pj : fmax(0.0, pj - (double)qk[j]);
        }
        double run = before + blk_prefix_excl<NT>(mine, sh);
        int cand = 0x7fffffff;
        double cp = 0.0, cc = 0.0;
        for (int j = j0; j < j1; ++j) {
            const double pj = p_of(zk, sk, T, j);
            const double rj = (use_p || !qk) ? pj : fmax(0.0, pj - (double)qk[j]);
            const double nxt = run + rj;
            if (nxt > target) { cand = j; cp = run; cc = nxt; break; }
            run = nxt;
        }
        // lowest candidate index wins
        int best = cand;
        for (int off = 32; off > 0; off >>= 1) best = min(best, __shfl_xor(best, off, 64));
        if (NT > 64) {
            if ((tid & 63) == 0) shi[tid >> 6] = best;
            __syncthreads();
            best = shi[0];
            for (int q2 = 1; q2 < NT / 64; ++q2) best = min(best, shi[q2]);
        }
        if (tid == 0) s_y = 0x7fffffff;
        __syncthreads();
        if (cand != 0x7fffffff && cand == best) {
            s_y = cand;
            sh[6] = cp;
            sh[7] = cc;
        }
        __syncthreads();
        if (s_y != 0x7fffffff) {
            found = true;
            y = s_y;
            cprev = sh[6];
            cy = sh[7];
        }
    }
    if (tid != 0) return;
    if (!found) {
        // u * R at (or past) the end of the located chunk, or of the whole row:
        // only rounding puts it there, so it is a boundary case
        y = (wc >= 0) ? (use_p ? pb[wc].last_p : pb[wc].last_r) : last_any;
        flags |= VW4_FLAG_CDF_TIE;
    } else if (fabs(target - cprev) < 1e-9 * R || fabs(target - cy) < 1e-9 * R) {
        flags |= VW4_FLAG_CDF_TIE;
    }
    int32_t* tb = out_tokens + b * (D + 1);
    for (int i = 0; i < k; ++i) tb[i] = db[i];
    tb[k] = y;
    for (int i = k + 1; i <= D; ++i) tb[i] = -1;
    out_nacc[b] = k;
    out_flags[b] = flags;
}

}  // namespace vw4

using namespace vw4;

extern "C" {

size_t vw4_accept_workspace_bytes(int32_t B, int32_t V) {
    if (B < 1 || B > (1 << 24) || V < 1 || V > (1 << 24)) return 0;
    return accept_layout(B, V).total;
}

int spec_accept(const float* logits, int64_t logits_bstride, const vw4_rowstat* stats, int64_t stats_bstride,
                const float* q, int64_t q_bstride, const int32_t* draft, int32_t B, int32_t D, int32_t V,
                float temperature, uint64_t seed, uint64_t step0, int32_t* out_tokens, int32_t* out_n_acc,
                uint32_t* out_flags, void* ws, size_t ws_bytes, void* stream) {
    VW4_REQUIRE(B >= 1 && B <= (1 << 24), VW4_EINVAL, "spec_accept: B=%d out of range", B);
    VW4_REQUIRE(D >= 0 && D <= AMAXD, VW4_EINVAL, "spec_accept: D=%d must be in [0, 7]", D);
    VW4_REQUIRE(V >= 1 && V <= (1 << 24), VW4_EINVAL, "spec_accept: V=%d out of range", V);
    VW4_REQUIRE(isfinite(temperature) && temperature >= 0.0f, VW4_EINVAL, "spec_accept: temperature must be >= 0");
    VW4_REQUIRE(logits && stats && out_tokens && out_n_acc && out_flags, VW4_EINVAL, "spec_accept: null pointer");
    VW4_REQUIRE(D == 0 || (q && draft), VW4_EINVAL, "spec_accept: q and draft are required when D > 0");
    VW4_REQUIRE(logits_bstride >= 0 && stats_bstride >= 0 && q_bstride >= 0, VW4_EINVAL,
                "spec_accept: negative batch stride");
    const AcceptLayout L = accept_layout(B, V);
    VW4_REQUIRE(ws && ws_bytes >= L.total && aligned(ws, 256), VW4_EWORKSPACE,
                "spec_accept: needs a 256-byte aligned workspace of %zu bytes", L.total);
    AcceptPart* parts = (AcceptPart*)((char*)ws + L.off_part);
    uint32_t* cnts = (uint32_t*)((char*)ws + L.off_cnt);
    hipStream_t st = (hipStream_t)stream;
    const dim3 grid((unsigned)B, (unsigned)L.P);
    if (L.threads == 64)
        hipLaunchKernelGGL(spec_accept_kernel<64>, grid, dim3(64), 0, st, logits, logits_bstride, stats, stats_bstride,
                           q, q_bstride, draft ? draft : (const int32_t*)out_tokens, D, V, temperature, seed, step0,
                           L.chunk, L.P, out_tokens, out_n_acc, out_flags, parts, cnts);
    else
        hipLaunchKernelGGL(spec_accept_kernel<AT>, grid, dim3(AT), 0, st, logits, logits_bstride, stats, stats_bstride,
                           q, q_bstride, draft ? draft : (const int32_t*)out_tokens, D, V, temperature, seed, step0,
                           L.chunk, L.P, out_tokens, out_n_acc, out_flags, parts, cnts);
    return check_launch("spec_accept");
}

}  // extern "C"
