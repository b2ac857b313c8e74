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
// MI355X design: problem b's residual row is split over P workgroups
// (grid = (B, P)); every workgroup redoes the D accept tests (D <= 7 scalar
// fp64 evaluations) and stores fixed-order fp64 chunk sums of r.  A second
// launch (one workgroup per problem) locates the chunk holding u * R, rescans
// it with a block-wide fp64 prefix sum in index order and writes the tokens.
// Kernel boundaries, not device-wide atomics, separate the phases (an atomic
// counter costs tens of ns per arriving workgroup on this part).  Vocabularies
// of at most 1024 entries use one 64-lane workgroup per problem, up to 16384
// one 512-lane workgroup, each in one launch; so does T == 0, whose outcome
// needs no pass over the vocabulary.
#include <math.h>

#include "common.h"

namespace vw4 {

constexpr int AT = 256;          // threads per workgroup for large vocabularies
constexpr int AT1 = 512;         // one workgroup per problem up to AT1 * 32 entries
constexpr int ASH = 2 * (AT1 / 64) + 4;  // block-reduction scratch (two values per wavefront)
constexpr int ACHUNK = 4096;     // vocabulary entries per workgroup
constexpr int AMAXP = 64;
constexpr int AMAXD = 7;
constexpr int AU = 16;  // elements per thread loaded together (one latency per tile)

struct AcceptPart {
    double r;       // chunk sum of the residual r
    double p;       // chunk sum of p_k (fallback when R == 0)
    int32_t last_r; // last index in the chunk with r > 0 (-1 if none)
    int32_t last_p; // last index with p_k > 0
};

// Problems per call whose residual masses the chunk kernel keeps for the
// finishing workgroup (P * chunk doubles each, 1.2 MB at V = 151936): with
// them the finish loads the located chunk's masses instead of recomputing
// them (16 fp64 exponentials per thread on one CU).  Larger batches recompute;
// both read the same values in the same order.
constexpr int AKEEP_B = 8;

struct AcceptLayout {
    int P, chunk, threads;
    bool keep_r;
    size_t off_part, off_state, off_r, total;
};

static AcceptLayout accept_layout(int B, int V) {
    AcceptLayout L;
    if (V <= 1024) {
        L.P = 1;
        L.chunk = V;
        L.threads = 64;
    } else if (V <= AT1 * 32) {
        L.P = 1;
        L.chunk = V;
        L.threads = AT1;
    } else {
        L.threads = AT;
        L.chunk = ACHUNK;
        L.P = ceil_div(V, ACHUNK);
        if (L.P > AMAXP) {
            L.chunk = ceil_div(ceil_div(V, AMAXP), AT) * AT;
            L.P = ceil_div(V, L.chunk);
        }
    }
    L.keep_r = L.P > 1 && L.chunk <= AT * AU && B <= AKEEP_B;
    size_t o = 0;
    L.off_part = o;
    o += (size_t)B * L.P * sizeof(AcceptPart);
    o = (o + 255) / 256 * 256;
    L.off_state = o;
    o += (size_t)B * 64;
    o = (o + 255) / 256 * 256;
    L.off_r = o;
    if (L.keep_r) o += (size_t)B * L.P * L.chunk * sizeof(double);
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

// Target probability of token j whose logit is v.
__device__ __forceinline__ double p_val(float v, const vw4_rowstat& s, double T, int j) {
    if (T == 0.0) return (j == s.argmax) ? 1.0 : 0.0;
    if (!(v >= s.tau)) return 0.0;
    return exp(((double)v - (double)s.max_logit) / T - s.log_z);
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

// State every workgroup of a problem derives identically: uniforms, flags
// from the row statistics, and the first rejection k.
struct ProblemState {
    int k;
    uint32_t flags;
    bool bad;
};
// What the finishing workgroup needs from the chunk kernel, in one load:
// the decision state, the statistics of the resampled row k and its uniform.
struct ProblemSlot {
    ProblemState ps;
    int32_t pad0;
    vw4_rowstat sk;
    double u_res;
    double pad1;
};
static_assert(sizeof(ProblemSlot) == 64, "ProblemSlot is 64 bytes");

template <int NT>
__device__ __forceinline__ ProblemState problem_state(const float* __restrict__ zb, const vw4_rowstat* __restrict__ sb,
                                                      const float* __restrict__ qb, const int32_t* __restrict__ db,
                                                      int D, int V, double T, uint64_t seed, uint64_t step,
                                                      uint64_t row0, uint64_t cstream, double* s_u,
                                                      vw4_rowstat* s_st) {
    __shared__ double s_p[AMAXD + 1], s_q[AMAXD + 1];
    __shared__ int s_ok[AMAXD + 1];
    // thread i (<= D): row i's uniforms, statistics, and p_i(x_i), q_i(x_i) --
    // all rows' loads in flight together
    if (threadIdx.x <= D) {
        const int i = threadIdx.x;
        uint64_t c[4] = {step, row0 + (uint64_t)i, cstream, 0};
        philox4x64_10(seed, 0, c);
        s_u[2 * i] = unit53(c[0]);
        s_u[2 * i + 1] = unit53(c[1]);
        const vw4_rowstat st = sb[i];
        s_st[i] = st;
        if (i < D) {
            const int x = db[i];
            const bool ok = x >= 0 && x < V;  // a malformed draft id is rejected, never dereferenced
            s_ok[i] = ok;
            s_p[i] = ok ? p_val(zb[(int64_t)i * V + x], st, T, x) : 0.0;
            s_q[i] = ok ? (double)qb[(int64_t)i * V + x] : 0.0;
        }
    }
    __syncthreads();
    ProblemState ps;
    ps.flags = 0;
    ps.bad = false;
    for (int i = 0; i <= D; ++i) {
        const uint32_t f = s_st[i].flags;
        if (f & VW4_FLAG_NONFINITE) ps.bad = true;
        if (f & VW4_FLAG_TOPP_TIE) ps.flags |= VW4_FLAG_TOPP_TIE;
    }
    ps.k = D;
    if (ps.bad) return ps;
    for (int i = 0; i < D; ++i) {
        if (!s_ok[i]) { ps.k = i; break; }
        const double pi = s_p[i], qi = s_q[i], u = s_u[2 * i];
        if (qi > 0.0 && fabs(u - pi / qi) < 1e-5) ps.flags |= VW4_FLAG_ACCEPT_TIE;
        if (!(u * qi < pi)) { ps.k = i; break; }
    }
    return ps;
}

// Chunk w of the residual row of problem b: fixed-order sums of r and p_k.
// rout (if set) receives each entry's mass r (chunk-relative index); qout
// (if set) the row's p(j) as binary32 (the draft distribution draft_sample
// returns, written here instead of by a launch of its own).
template <int NT>
__device__ __forceinline__ AcceptPart chunk_sums(const float* __restrict__ zk, const vw4_rowstat& sk,
                                                 const float* __restrict__ qk, double T, int c0, int c1, double* sh,
                                                 int* shi, double* __restrict__ rout, float* __restrict__ qout) {
    double sr = 0.0, sp = 0.0;
    int lr = -1, lp = -1;
    for (int base = c0; base < c1; base += NT * AU) {
        // all loads of the tile issued together (clamped indices, no branches);
        // slots past the chunk end are masked below
        float zv[AU], qv[AU];
#pragma unroll
        for (int u = 0; u < AU; ++u) zv[u] = zk[min(base + u * NT + (int)threadIdx.x, c1 - 1)];
        if (qk) {
#pragma unroll
            for (int u = 0; u < AU; ++u) qv[u] = qk[min(base + u * NT + (int)threadIdx.x, c1 - 1)];
        } else {
#pragma unroll
            for (int u = 0; u < AU; ++u) qv[u] = 0.0f;
        }
#pragma unroll
        for (int u = 0; u < AU; ++u) {
            const int j = base + u * NT + threadIdx.x;
            if (j < c1) {
                const double pj = p_val(zv[u], sk, T, j);
                const double rj = qk ? fmax(0.0, pj - (double)qv[u]) : pj;
                if (rout) rout[j - c0] = rj;
                if (qout) qout[j] = (float)pj;
                sr += rj;
                sp += pj;
                if (rj > 0.0) lr = j;
                if (pj > 0.0) lp = j;
            }
        }
    }
    // the four block reductions in one pass: wavefront reductions (fixed
    // xor trees), one barrier, then the wavefronts' values combined in
    // wavefront order (the maxima are order-free)
    double r = wave_sum(sr), p = wave_sum(sp);
    for (int off = 32; off > 0; off >>= 1) {
        lr = max(lr, __shfl_xor(lr, off, 64));
        lp = max(lp, __shfl_xor(lp, off, 64));
    }
    if (NT > 64) {
        constexpr int NW = NT / 64;
        const int w = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) {
            sh[w] = r;
            sh[NW + w] = p;
            shi[w] = lr;
            shi[NW + w] = lp;
        }
        __syncthreads();
        r = sh[0];
        p = sh[NW];
        lr = shi[0];
        lp = shi[NW];
        for (int k = 1; k < NW; ++k) {
            r += sh[k];
            p += sh[NW + k];
            lr = max(lr, shi[k]);
            lp = max(lp, shi[NW + k]);
        }
        __syncthreads();
    }
    AcceptPart a;
    a.r = r;
    a.p = p;
    a.last_r = lr;
    a.last_p = lp;
    return a;
}

// Locate u * R among the chunk sums, rescan the chunk that holds it and
// write the outputs of problem b.  pb: the P chunk parts (in LDS or global).
// rkept (if set): the chunk kernel's masses r of this problem, [P][chunk].
template <int NT>
__device__ void finish_problem(const float* __restrict__ zk, const vw4_rowstat& sk, const float* __restrict__ qk,
                               const int32_t* __restrict__ db, const AcceptPart* pb, int P, int chunk, int D, int V,
                               double T, const ProblemState& ps, const double* s_u, int32_t* __restrict__ tb,
                               int32_t* __restrict__ nacc_b, uint32_t* __restrict__ flags_b, double* sh, int* shi,
                               const double* __restrict__ rkept) {
    __shared__ int s_y;
    const int k = ps.k;
    uint32_t flags = ps.flags;
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
    const bool resid = !use_p && qk != nullptr;
    int y = -1;
    double cprev = 0.0, cy = 0.0;
    bool found = false;
    if (wc >= 0) {
        // rescan chunk wc: thread t owns a contiguous run, prefix sums in index order
        const int a0 = wc * chunk, a1 = min(V, a0 + chunk);
        const int per = (a1 - a0 + NT - 1) / NT;
        const int j0 = a0 + threadIdx.x * per, j1 = min(a1, j0 + per);
        int cand = 0x7fffffff;
        double cp = 0.0, cc = 0.0;
        if (per <= AU) {
            // the whole run in registers: one load, the masses computed once
            // (or, kept by the chunk kernel, loaded: the same values)
            double rv[AU];
            double mine = 0.0;
            const double* rw = (rkept && !use_p) ? rkept + (int64_t)wc * chunk - a0 : nullptr;
            if (rw) {
#pragma unroll
                for (int u = 0; u < AU; ++u) rv[u] = (j0 + u < j1) ? rw[j0 + u] : 0.0;
#pragma unroll
                for (int u = 0; u < AU; ++u)
                    if (j0 + u < j1) mine += rv[u];
            } else {
                float zv[AU], qv[AU];
#pragma unroll
                for (int u = 0; u < AU; ++u) {
                    zv[u] = (j0 + u < j1) ? zk[j0 + u] : 0.0f;
                    qv[u] = (resid && j0 + u < j1) ? qk[j0 + u] : 0.0f;
                }
#pragma unroll
                for (int u = 0; u < AU; ++u) {
                    rv[u] = 0.0;
                    if (j0 + u < j1) {
                        const double pj = p_val(zv[u], sk, T, j0 + u);
                        rv[u] = resid ? fmax(0.0, pj - (double)qv[u]) : pj;
                        mine += rv[u];
                    }
                }
            }
            double run = before + blk_prefix_excl<NT>(mine, sh);
            for (int u = 0; u < AU; ++u) {
                if (j0 + u >= j1) break;
                const double nxt = run + rv[u];
                if (nxt > target) { cand = j0 + u; cp = run; cc = nxt; break; }
                run = nxt;
            }
        } else {
        // this thread's residual masses, computed once (runs of up to AU per pass)
        double mine = 0.0;
        for (int t0 = j0; t0 < j1; t0 += AU) {
            float zv[AU], qv[AU];
#pragma unroll
            for (int u = 0; u < AU; ++u) {
                zv[u] = (t0 + u < j1) ? zk[t0 + u] : 0.0f;
                qv[u] = (resid && t0 + u < j1) ? qk[t0 + u] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < AU; ++u) {
                if (t0 + u >= j1) break;
                const double pj = p_val(zv[u], sk, T, t0 + u);
                mine += resid ? fmax(0.0, pj - (double)qv[u]) : pj;
            }
        }
        double run = before + blk_prefix_excl<NT>(mine, sh);
        for (int t0 = j0; t0 < j1 && cand == 0x7fffffff; t0 += AU) {
            float zv[AU], qv[AU];
#pragma unroll
            for (int u = 0; u < AU; ++u) {
                zv[u] = (t0 + u < j1) ? zk[t0 + u] : 0.0f;
                qv[u] = (resid && t0 + u < j1) ? qk[t0 + u] : 0.0f;
            }
            for (int u = 0; u < AU; ++u) {
                if (t0 + u >= j1) break;
                const double pj = p_val(zv[u], sk, T, t0 + u);
                const double rj = resid ? fmax(0.0, pj - (double)qv[u]) : pj;
                const double nxt = run + rj;
                if (nxt > target) { cand = t0 + u; cp = run; cc = nxt; break; }
                run = nxt;
            }
        }
        }
        int best = cand;
        for (int off = 32; off > 0; off >>= 1) best = min(best, __shfl_xor(best, off, 64));
        if (NT > 64) {
            if ((threadIdx.x & 63) == 0) shi[threadIdx.x >> 6] = best;
            __syncthreads();
            best = shi[0];
            for (int q2 = 1; q2 < NT / 64; ++q2) best = min(best, shi[q2]);
        }
        if (threadIdx.x == 0) s_y = 0x7fffffff;
        __syncthreads();
        if (cand != 0x7fffffff && cand == best) {
            s_y = cand;
            sh[NT / 64 + 1] = cp;
            sh[NT / 64 + 2] = cc;
        }
        __syncthreads();
        if (s_y != 0x7fffffff) {
            found = true;
            y = s_y;
            cprev = sh[NT / 64 + 1];
            cy = sh[NT / 64 + 2];
        }
    }
    if (threadIdx.x != 0) return;
    if (!found) {
        // u * R at (or past) the end of the located chunk, or of the whole row:
        // only rounding puts it there, so it is a boundary case
        y = (wc >= 0) ? (use_p ? pb[wc].last_p : pb[wc].last_r) : last_any;
        flags |= VW4_FLAG_CDF_TIE;
    } else if (fabs(target - cprev) < 1e-9 * R || fabs(target - cy) < 1e-9 * R) {
        flags |= VW4_FLAG_CDF_TIE;
    }
    for (int i = 0; i < k; ++i) tb[i] = db[i];
    tb[k] = y;
    for (int i = k + 1; i <= D; ++i) tb[i] = -1;
    *nacc_b = k;
    *flags_b = flags;
}

struct AcceptArgs {
    const float* logits;
    int64_t lstride;
    const vw4_rowstat* stats;
    int64_t sstride;
    const float* q;
    int64_t qstride;
    const int32_t* draft;
    int D, V;
    float temperature;
    uint64_t seed, step0;
    int chunk, P;
    int32_t* out_tokens;
    int32_t* out_nacc;
    uint32_t* out_flags;
    AcceptPart* parts;
    ProblemSlot* states;   // per problem, written by workgroup 0 of the chunk kernel
    double* rkept;         // [B][P][chunk] masses r kept for the finish, or null
    float* q_out;          // draft_sample (B = 1, D = 0): p of the row as binary32, or null
    const uint64_t* step_dev;  // if set, the first problem's step is read here (graph replays)
    uint64_t row0, cstream;    // Philox counter words 1 (row offset) and 2 (stream): 0 for verify
};

__device__ __forceinline__ uint64_t first_step(const AcceptArgs& a) { return a.step_dev ? *a.step_dev : a.step0; }

__device__ __forceinline__ void write_bad(const AcceptArgs& a, int64_t b) {
    if (threadIdx.x <= a.D) a.out_tokens[b * (a.D + 1) + threadIdx.x] = -1;
    if (threadIdx.x == 0) {
        a.out_nacc[b] = -1;
        a.out_flags[b] = VW4_FLAG_NONFINITE;
    }
}

// grid (B, P).  With P == 1 the workgroup finishes its problem itself;
// otherwise it stores its chunk sums for accept_finish_kernel.
template <int NT>
__global__ __launch_bounds__(NT) void accept_chunk_kernel(AcceptArgs a) {
    __shared__ double sh[ASH];
    __shared__ int shi[ASH];
    __shared__ double s_u[2 * (AMAXD + 1)];
    __shared__ AcceptPart s_part;
    __shared__ vw4_rowstat s_st[AMAXD + 1];
    const int64_t b = blockIdx.x;
    const int w = blockIdx.y;
    const float* zb = a.logits + b * a.lstride;
    const vw4_rowstat* sb = a.stats + b * a.sstride;
    const float* qb = a.q ? a.q + b * a.qstride : nullptr;
    const int32_t* db = a.draft + b * a.D;
    const double T = (double)a.temperature;
    const ProblemState ps =
        problem_state<NT>(zb, sb, qb, db, a.D, a.V, T, a.seed, first_step(a) + (uint64_t)b, a.row0, a.cstream, s_u, s_st);
    if (ps.bad) {
        if (a.q_out) {  // the same values p_val gives for this row's statistics
            const int c0 = w * a.chunk, c1 = min(a.V, c0 + a.chunk);
            for (int j = c0 + (int)threadIdx.x; j < c1; j += NT) a.q_out[j] = (float)p_val(zb[j], s_st[0], T, j);
        }
        if (w == 0) write_bad(a, b);
        return;
    }
    const int k = ps.k;
    const float* zk = zb + (int64_t)k * a.V;
    const vw4_rowstat sk = s_st[k];
    const float* qk = (k < a.D) ? qb + (int64_t)k * a.V : nullptr;
    const int c0 = w * a.chunk, c1 = min(a.V, c0 + a.chunk);
    double* rout = (a.P > 1 && a.rkept) ? a.rkept + (b * a.P + w) * (int64_t)a.chunk : nullptr;
    const AcceptPart part = chunk_sums<NT>(zk, sk, qk, T, c0, c1, sh, shi, rout, a.q_out);
    if (a.P > 1) {
        if (threadIdx.x == 0) {
            a.parts[b * a.P + w] = part;
            if (w == 0) {
                ProblemSlot slot;
                slot.ps = ps;
                slot.pad0 = 0;
                slot.sk = sk;
                slot.u_res = s_u[2 * k + 1];
                slot.pad1 = 0.0;
                a.states[b] = slot;
            }
        }
        return;
    }
    if (threadIdx.x == 0) s_part = part;
    __syncthreads();
    finish_problem<NT>(zk, sk, qk, db, &s_part, 1, a.chunk, a.D, a.V, T, ps, s_u, a.out_tokens + b * (a.D + 1),
                       a.out_nacc + b, a.out_flags + b, sh, shi, nullptr);
}

// grid (B): combine the P chunk sums of problem b and sample its token.
template <int NT>
__global__ __launch_bounds__(NT) void accept_finish_kernel(AcceptArgs a) {
    __shared__ double sh[ASH];
    __shared__ int shi[ASH];
    __shared__ double s_u[2 * (AMAXD + 1)];
    __shared__ AcceptPart sp[AMAXP];
    const int64_t b = blockIdx.x;
    const float* zb = a.logits + b * a.lstride;
    const vw4_rowstat* sb = a.stats + b * a.sstride;
    const float* qb = a.q ? a.q + b * a.qstride : nullptr;
    const int32_t* db = a.draft + b * a.D;
    const double T = (double)a.temperature;
    __shared__ ProblemSlot s_slot;
    // the accept decisions, the resampled row's statistics and its uniform
    // come from the chunk kernel, loaded together with the chunk sums
    if (threadIdx.x == 0) s_slot = a.states[b];
    for (int c = threadIdx.x; c < a.P; c += NT) sp[c] = a.parts[b * a.P + c];
    __syncthreads();
    const ProblemState ps = s_slot.ps;
    if (ps.bad) return;  // outputs written by the chunk kernel
    const int k = ps.k;
    if (threadIdx.x == 0) s_u[2 * k + 1] = s_slot.u_res;
    __syncthreads();
    (void)sb;
    const float* zk = zb + (int64_t)k * a.V;
    const vw4_rowstat sk = s_slot.sk;
    const float* qk = (k < a.D) ? qb + (int64_t)k * a.V : nullptr;
    finish_problem<NT>(zk, sk, qk, db, sp, a.P, a.chunk, a.D, a.V, T, ps, s_u, a.out_tokens + b * (a.D + 1),
                       a.out_nacc + b, a.out_flags + b, sh, shi,
                       a.rkept ? a.rkept + b * a.P * (int64_t)a.chunk : nullptr);
}

// T == 0: every target row is one-hot at its argmax a_i, so the outcome of the
// general algorithm is known without a pass over the vocabulary.  Draft i is
// accepted iff it is a_i (u * q < 1 always holds there); the residual row
// k < D is max(0, 1 - q_k(a_k)) at a_k and 0 elsewhere (R == 0 falls back to
// p_k, the same token); the bonus row samples a_D.  The CDF-boundary flag of
// the general path reduces to u_res * R within 1e-9 * R of 0 or of R, the two
// ends of the only nonzero mass.  grid (B), one wavefront per problem.
__global__ __launch_bounds__(64) void accept_greedy_kernel(AcceptArgs a) {
    __shared__ double s_u[2 * (AMAXD + 1)];
    __shared__ vw4_rowstat s_st[AMAXD + 1];
    const int64_t b = blockIdx.x;
    const float* zb = a.logits + b * a.lstride;
    const vw4_rowstat* sb = a.stats + b * a.sstride;
    const float* qb = a.q ? a.q + b * a.qstride : nullptr;
    const int32_t* db = a.draft + b * a.D;
    const ProblemState ps =
        problem_state<64>(zb, sb, qb, db, a.D, a.V, 0.0, a.seed, first_step(a) + (uint64_t)b, a.row0, a.cstream, s_u, s_st);
    if (ps.bad) {
        write_bad(a, b);
        return;
    }
    if (threadIdx.x != 0) return;
    const int k = ps.k;
    const int32_t y = s_st[k].argmax;
    uint32_t flags = ps.flags;
    double R = 1.0;
    if (k < a.D) {
        R = fmax(0.0, 1.0 - (double)qb[(int64_t)k * a.V + y]);
        if (!(R > 0.0)) {
            flags |= VW4_FLAG_R_ZERO;
            R = 1.0;
        }
    }
    const double target = s_u[2 * k + 1] * R;
    if (fabs(target) < 1e-9 * R || fabs(target - R) < 1e-9 * R) flags |= VW4_FLAG_CDF_TIE;
    int32_t* tb = a.out_tokens + b * (a.D + 1);
    for (int i = 0; i < k; ++i) tb[i] = db[i];
    tb[k] = y;
    for (int i = k + 1; i <= a.D; ++i) tb[i] = -1;
    a.out_nacc[b] = k;
    a.out_flags[b] = flags;
}

__global__ void step_advance_kernel(uint64_t* step, uint64_t inc) { *step += inc; }

static int spec_accept_impl(const float* logits, int64_t logits_bstride, const vw4_rowstat* stats,
                            int64_t stats_bstride, const float* q, int64_t q_bstride, const int32_t* draft, int32_t B,
                            int32_t D, int32_t V, float temperature, uint64_t seed, uint64_t step0,
                            const uint64_t* step_dev, int32_t* out_tokens, int32_t* out_n_acc, uint32_t* out_flags,
                            void* ws, size_t ws_bytes, void* stream, uint64_t row0 = 0, uint64_t cstream = 0,
                            float* q_out = nullptr) {
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
    AcceptArgs a;
    a.logits = logits; a.lstride = logits_bstride; a.stats = stats; a.sstride = stats_bstride;
    a.q = q; a.qstride = q_bstride;
    a.draft = draft ? draft : (const int32_t*)out_tokens;  // D == 0: never read
    a.D = D; a.V = V; a.temperature = temperature; a.seed = seed; a.step0 = step0;
    a.chunk = L.chunk; a.P = L.P;
    a.out_tokens = out_tokens; a.out_nacc = out_n_acc; a.out_flags = out_flags;
    a.parts = (AcceptPart*)((char*)ws + L.off_part);
    a.states = (ProblemSlot*)((char*)ws + L.off_state);
    a.rkept = L.keep_r ? (double*)((char*)ws + L.off_r) : nullptr;
    a.step_dev = step_dev;
    a.row0 = row0; a.cstream = cstream;
    a.q_out = q_out;
    hipStream_t st = (hipStream_t)stream;
    if (temperature == 0.0f) {
        hipLaunchKernelGGL(accept_greedy_kernel, dim3((unsigned)B), dim3(64), 0, st, a);
        return check_launch("spec_accept");
    }
    const dim3 grid((unsigned)B, (unsigned)L.P);
    if (L.threads == 64) {
        hipLaunchKernelGGL(accept_chunk_kernel<64>, grid, dim3(64), 0, st, a);
    } else if (L.threads == AT1) {
        hipLaunchKernelGGL(accept_chunk_kernel<AT1>, grid, dim3(AT1), 0, st, a);
    } else {
        hipLaunchKernelGGL(accept_chunk_kernel<AT>, grid, dim3(AT), 0, st, a);
        if (L.P > 1) hipLaunchKernelGGL(accept_finish_kernel<AT>, dim3((unsigned)B), dim3(AT), 0, st, a);
    }
    return check_launch("spec_accept");
}


// q[j] = p(j) of one warped row as binary32 (the draft distribution the
// verify's ratio test reads); grid over V, 256 threads.
__global__ __launch_bounds__(256) void draft_q_kernel(const float* __restrict__ z, const vw4_rowstat* __restrict__ st,
                                                      int V, double T, float* __restrict__ q) {
    const vw4_rowstat s = *st;
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j < V) q[j] = (float)p_val(z[j], s, T, j);
}

static size_t draft_ws_tail(int V) { return (accept_layout(1, V).total + 255) / 256 * 256; }

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
    return spec_accept_impl(logits, logits_bstride, stats, stats_bstride, q, q_bstride, draft, B, D, V, temperature,
                            seed, step0, nullptr, out_tokens, out_n_acc, out_flags, ws, ws_bytes, stream);
}

int spec_accept_ex(const float* logits, int64_t logits_bstride, const vw4_rowstat* stats, int64_t stats_bstride,
                   const float* q, int64_t q_bstride, const int32_t* draft, int32_t B, int32_t D, int32_t V,
                   float temperature, uint64_t seed, const uint64_t* step_dev, int32_t* out_tokens,
                   int32_t* out_n_acc, uint32_t* out_flags, void* ws, size_t ws_bytes, void* stream) {
    VW4_REQUIRE(step_dev && aligned(step_dev, 8), VW4_EINVAL, "spec_accept_ex: step_dev must be an 8-byte aligned device pointer");
    return spec_accept_impl(logits, logits_bstride, stats, stats_bstride, q, q_bstride, draft, B, D, V, temperature,
                            seed, 0, step_dev, out_tokens, out_n_acc, out_flags, ws, ws_bytes, stream);
}

size_t vw4_draft_workspace_bytes(int32_t V) {
    if (V < 1 || V > (1 << 24)) return 0;
    return draft_ws_tail(V) + 256;
}

int draft_sample(const float* logits, const vw4_rowstat* stats, int32_t V, float temperature, uint64_t seed,
                 const uint64_t* step_dev, uint64_t step, int32_t depth, float* q_out, int32_t* token_out,
                 uint32_t* flags_out, void* ws, size_t ws_bytes, void* stream) {
    VW4_REQUIRE(logits && stats && token_out && flags_out, VW4_EINVAL, "draft_sample: null pointer");
    VW4_REQUIRE(V >= 1 && V <= (1 << 24), VW4_EINVAL, "draft_sample: V=%d out of range", V);
    VW4_REQUIRE(depth >= 0 && depth <= 1023, VW4_EINVAL, "draft_sample: depth=%d out of range", depth);
    VW4_REQUIRE(!step_dev || aligned(step_dev, 8), VW4_EINVAL, "draft_sample: step_dev must be 8-byte aligned");
    VW4_REQUIRE(isfinite(temperature) && temperature >= 0.0f, VW4_EINVAL, "draft_sample: temperature must be >= 0");
    const size_t tail = draft_ws_tail(V);
    VW4_REQUIRE(ws && ws_bytes >= tail + 256 && aligned(ws, 256), VW4_EWORKSPACE,
                "draft_sample: needs a 256-byte aligned workspace of %zu bytes", tail + 256);
    hipStream_t st = (hipStream_t)stream;
    // T > 0: the sampling pass writes q as it forms p; T == 0 samples without
    // a pass over the vocabulary, so q (one-hot) gets a launch of its own
    if (q_out && temperature == 0.0f) {
        hipLaunchKernelGGL(draft_q_kernel, dim3((unsigned)ceil_div(V, 256)), dim3(256), 0, st, logits, stats, V,
                           (double)temperature, q_out);
        const int rc = check_launch("draft_sample");
        if (rc != VW4_OK) return rc;
    }
    int32_t* n_acc = (int32_t*)((char*)ws + tail);
    return spec_accept_impl(logits, 0, stats, 0, nullptr, 0, nullptr, 1, 0, V, temperature, seed, step, step_dev,
                            token_out, n_acc, flags_out, ws, tail, stream, (uint64_t)depth, 1,
                            temperature > 0.0f ? q_out : nullptr);
}

int vw4_step_advance(uint64_t* step_dev, uint64_t inc, void* stream) {
    VW4_REQUIRE(step_dev && aligned(step_dev, 8), VW4_EINVAL, "vw4_step_advance: step_dev must be 8-byte aligned");
    hipLaunchKernelGGL(step_advance_kernel, dim3(1), dim3(1), 0, (hipStream_t)stream, step_dev, inc);
    return check_launch("vw4_step_advance");
}

}  // extern "C"
