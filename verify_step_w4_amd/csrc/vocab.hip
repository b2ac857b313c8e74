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
// MI355X design.  No sort: tau is found by a radix descent on the
// order-preserving 32-bit key of the logits.  Each row is split over P
// workgroups.  Phases communicate only through kernel boundaries (a device-wide
// atomic counter costs tens of ns per arriving workgroup on this part, a
// dependent launch about 1.7 us), and every cross-workgroup combination is a
// fixed-order sum, so all statistics are reproducible bit for bit:
//   1. per chunk: local max m_w, e_j relative to m_w (stored, fp64), E_w, and a
//      mass histogram of the top 11 key bits (LDS), stored with its 64 coarse
//      sums (32 bins each)
//   2. per chunk: combine the chunks' coarse sums (rescaled by exp((m_w - m)/T),
//      chunk order), descend them to the coarse bin holding the cutoff, then
//      combine and descend only that coarse bin's 32 histogram bins: the
//      level-1 cutoff bin (workgroup 0 publishes it); histogram of the next 11
//      key bits inside it, with its coarse sums
//   3. per chunk: the same two-step descent of level 2 from the published
//      level-1 result; fixed-order mass and count above the 22-bit key prefix
//      of the cutoff; counts of the last 10 key bits inside it, published as a
//      short list of the non-empty bins (the dense counts only when the list
//      overflows its 256-byte record)
//   4. per row: with the 10-bit counts every bin is one float value, so its mass
//      is count * exp((z - m)/T) exactly; finish the descent, tau, Z, n_kept.
// The LDS histogram atomics and the coarse sums only steer steps 2 and 3; the
// final decision in step 4 uses fixed-order sums and flags (VW4_FLAG_TOPP_TIE)
// any row whose boundary mass lies within 1e-9 * E of top_p * E, which is also
// where a steering sum could pick a neighbouring bin.
#include <math.h>

#include "common.h"

namespace vw4 {

constexpr int VT = 256;        // threads per workgroup
constexpr int VCHUNK = 4096;   // logits per workgroup (grown for huge V)
constexpr int VMAXP = 64;      // workgroups per row at most
constexpr int L1BITS = 11, L2BITS = 11, L3BITS = 10;
constexpr int HB = 2048;       // histogram bins of levels 1 and 2
constexpr int HB3 = 1024;      // bins of level 3
constexpr int NC = 64;         // coarse bins per level (HB / NC = 32 histogram bins each)
constexpr int FPC = HB / NC;   // histogram bins per coarse bin

struct ChunkPart {   // per-workgroup results of phase 1
    float m;
    int32_t argmax;
    uint32_t bad;
    float mn;
    double E;        // sum of exp((z - m_w)/T) over the chunk
};

struct ChunkSums {   // per-workgroup results of phase 5
    double above;    // mass of keys above the 22-bit cutoff prefix
    uint32_t n_above;
    uint32_t pad;    // the 22-bit prefix
};

// Phase-5 record of one chunk (REC uint32 words, 256 bytes): its ChunkSums
// (words 0-3), the number nz of non-empty level-3 bins (word 4), and the
// first REC_CAP of them as (count << 10 | bin) entries.  When nz > REC_CAP
// the chunk's dense counts are written as well.  A chunk holds at most
// 2^18 logits (V <= 2^24 over at most 64 chunks), so a count fits 22 bits.
constexpr int REC = 64, REC_HEAD = 5, REC_CAP = REC - REC_HEAD;
static_assert(sizeof(ChunkSums) == 16, "ChunkSums fills record words 0-3");

// The level-1 cutoff bin and the mass above it, as the level-2 pass found
// them (every workgroup of a row finds the same; workgroup 0 publishes).
struct Steer {
    int32_t b;
    int32_t pad;
    double above;
};

struct VocabLayout {
    int P, chunk, V, rows;
    size_t off_part, off_e, off_h1p, off_h1c, off_h2p, off_h2c, off_steer, off_rec, off_c3, total;
};

static size_t al256(size_t o) { return (o + 255) / 256 * 256; }

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
    L.V = V;
    L.rows = rows;
    size_t o = 0;
    L.off_part = o; o = al256(o + (size_t)rows * P * sizeof(ChunkPart));
    L.off_e = o;    o = al256(o + (size_t)rows * V * sizeof(double));
    L.off_h1p = o;  o = al256(o + (size_t)rows * P * HB * sizeof(double));
    L.off_h1c = o;  o = al256(o + (size_t)rows * P * NC * sizeof(double));
    L.off_h2p = o;  o = al256(o + (size_t)rows * P * HB * sizeof(double));
    L.off_h2c = o;  o = al256(o + (size_t)rows * P * NC * sizeof(double));
    L.off_steer = o; o = al256(o + (size_t)rows * sizeof(Steer));
    L.off_rec = o;  o = al256(o + (size_t)rows * P * REC * sizeof(uint32_t));
    L.off_c3 = o;   o = al256(o + (size_t)rows * P * HB3 * sizeof(uint32_t));
    L.total = o;
    return L;
}

struct RowView {     // pointers of one row inside the workspace
    ChunkPart* part;
    double* e;
    double* h1p;     // [P][HB] chunk histograms of level 1
    double* h1c;     // [P][NC] their coarse sums
    double* h2p;
    double* h2c;
    Steer* steer;
    uint32_t* rec;
    uint32_t* c3;
};

__device__ __forceinline__ RowView row_view(char* ws, const VocabLayout& L, int r) {
    RowView v;
    v.part = (ChunkPart*)(ws + L.off_part) + (int64_t)r * L.P;
    v.e = (double*)(ws + L.off_e) + (int64_t)r * L.V;
    v.h1p = (double*)(ws + L.off_h1p) + (int64_t)r * L.P * HB;
    v.h1c = (double*)(ws + L.off_h1c) + (int64_t)r * L.P * NC;
    v.h2p = (double*)(ws + L.off_h2p) + (int64_t)r * L.P * HB;
    v.h2c = (double*)(ws + L.off_h2c) + (int64_t)r * L.P * NC;
    v.steer = (Steer*)(ws + L.off_steer) + r;
    v.rec = (uint32_t*)(ws + L.off_rec) + (int64_t)r * L.P * REC;
    v.c3 = (uint32_t*)(ws + L.off_c3) + (int64_t)r * L.P * HB3;
    return v;
}

// ---------------------------------------------------------------------------
// Block helpers (VT = 256 threads, fixed combination order).
// ---------------------------------------------------------------------------
__device__ __forceinline__ double block_sum_f64(double v, double* sh) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    const double s = (sh[0] + sh[1]) + (sh[2] + sh[3]);
    __syncthreads();
    return s;
}

__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, uint32_t* sh) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    const uint32_t s = sh[0] + sh[1] + sh[2] + sh[3];
    __syncthreads();
    return s;
}

// Exclusive suffix sum over threads: sum_{t' > t} v_{t'}.
__device__ __forceinline__ double block_suffix_excl_f64(double v, double* sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    double s = v;
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

// Elements base + u*VT + threadIdx.x (u < VU) of a chunk ending at c1, loaded
// together before any is used: one memory latency per tile instead of one per
// element.  Out-of-range slots are left unread.
constexpr int VU = 16;
template <typename T>
__device__ __forceinline__ void load_tile(const T* __restrict__ src, int base, int c1, T (&v)[VU]) {
#pragma unroll
    for (int u = 0; u < VU; ++u) {
        const int j = base + u * VT + threadIdx.x;
        v[u] = (j < c1) ? src[j] : T(0);
    }
}

// Row max / argmax (lowest index) / non-finite / min over the P chunk parts.
struct RowMax {
    float m, mn;
    int32_t argmax;
    uint32_t bad;
};

// Stage the P chunk parts in LDS with one load per thread (independent loads:
// a dependent chain of global loads costs a full memory latency per part).
__device__ __forceinline__ void stage_parts(const ChunkPart* __restrict__ part, int P, ChunkPart* sp) {
    for (int k = threadIdx.x; k < P; k += blockDim.x) sp[k] = part[k];
    __syncthreads();
}

// Row header by one wavefront, lane k holding chunk part k (P <= 64), for
// the 1024-thread finishing kernel, where the whole-block loops over the parts
// cost one LDS round trip per part in each of 16 wavefronts.  The max, its
// argmax and the non-finite flag come from a lane reduction: a pure selection,
// exact, with ties to the lowest chunk as in the scan in chunk order (only
// non-finite rows, whose header is not used, could differ).  The minimum and
// E = sum_k f_k E_k are the scan's own chains in chunk order (fminf, and one
// fused multiply-add per chunk), operands taken lane by lane.
__device__ __forceinline__ RowMax wave_combine_max(const ChunkPart* sp, int P) {
    const int lane = threadIdx.x & 63;
    const bool in = lane < P;
    const ChunkPart& q = sp[in ? lane : 0];
    float m = in ? q.m : -INFINITY;
    int32_t a = in ? q.argmax : 0, k = in ? lane : 0x7fffffff;
    uint32_t bad = in ? q.bad : 0u;
    for (int off = 32; off > 0; off >>= 1) {
        const float om = __shfl_xor(m, off, 64);
        const int32_t ok = __shfl_xor(k, off, 64), oa = __shfl_xor(a, off, 64);
        if (om > m || (om == m && ok < k)) { m = om; k = ok; a = oa; }
        bad |= __shfl_xor(bad, off, 64);
    }
    // the minimum folded in chunk order (fminf of signed zeros may depend on order)
    const int32_t mnl = __float_as_int(q.mn);
    float mn = INFINITY;
    for (int c = 0; c < P; ++c) mn = fminf(mn, __int_as_float(__builtin_amdgcn_readlane(mnl, c)));
    RowMax r;
    r.m = m; r.mn = mn; r.argmax = a; r.bad = bad;
    return r;
}

__device__ __forceinline__ double wave_combine_E(const ChunkPart* sp, int P, float m, double T) {
    const int lane = threadIdx.x & 63;
    const ChunkPart& q = sp[lane < P ? lane : 0];
    const double f = exp(((double)q.m - (double)m) / T), e = q.E;
    double E = 0.0;
    for (int k = 0; k < P; ++k) E = fma(readlane_f64(f, k), readlane_f64(e, k), E);
    return E;
}

// The row max and E for the level passes, where they only steer: wavefront 0
// reduces the chunk parts (lane k holds part k, P <= 64; the max is a pure
// selection, the same as a scan in chunk order), and the result is broadcast
// through LDS.  The factors f[k] = exp((m_k - m)/T) are formed in fp64 as in
// every pass; E is their fixed-tree sum, which may differ from the
// chunk-order chain of the finishing pass in the last bits.
__device__ __forceinline__ RowMax steer_max(const ChunkPart* sp, int P, RowMax* s_mx) {
    if (threadIdx.x < 64) {
        const RowMax h = wave_combine_max(sp, P);
        if (threadIdx.x == 0) *s_mx = h;
    }
    __syncthreads();
    return *s_mx;
}

__device__ __forceinline__ double steer_E(const ChunkPart* sp, int P, float m, double T, double* f, double* s_E) {
    for (int k = threadIdx.x; k < P; k += blockDim.x) f[k] = exp(((double)sp[k].m - (double)m) / T);
    __syncthreads();
    if (threadIdx.x < 64) {
        const double e = wave_sum((int)threadIdx.x < P ? f[threadIdx.x] * sp[threadIdx.x].E : 0.0);
        if (threadIdx.x == 0) *s_E = e;
    }
    __syncthreads();
    return *s_E;
}

// Descend nb combined bins (ascending key, HB/VT = 8 per thread, this
// thread's slice in h): the largest bin b with
// above + sum_{b' >= b} H[b'] >= target, and the mass above it.  If rounding
// leaves the target beyond every bin, the lowest non-empty bin (-1 if all are
// empty); the finishing pass flags such a row.
__device__ int descend(const double (&h)[HB / VT], int nb, double above, double target, double* new_above,
                       double* sh, int* shi) {
    const int per = HB / VT;
    const int b0 = threadIdx.x * per;
    double mine = 0.0;
#pragma unroll
    for (int i = 0; i < per; ++i) mine += h[i];
    const double later = block_suffix_excl_f64(mine, sh);
    if (threadIdx.x == 0) *shi = -1;
    __syncthreads();
    double cum = above + later;
#pragma unroll
    for (int i = per - 1; i >= 0; --i) {
        if (cum < target && cum + h[i] >= target && b0 + i < nb) {
            *shi = b0 + i;
            sh[8] = cum;
        }
        cum += h[i];
    }
    __syncthreads();
    int b = *shi;
    double na = (b >= 0) ? sh[8] : above;
    __syncthreads();
    if (b < 0) {
        // target beyond the histogram's total (rounding, or top_p within an ulp
        // of 1): keep the lowest non-empty bin; the finishing pass flags it
        if (threadIdx.x == 0) *shi = 0x7fffffff;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < per; ++i)
            if (h[i] > 0.0) atomicMin(shi, b0 + i);
        __syncthreads();
        b = *shi;
        if (b == 0x7fffffff) b = -1;
        double mass_above = 0.0;
#pragma unroll
        for (int i = 0; i < per; ++i)
            if (b0 + i > b) mass_above += h[i];
        na = above + block_sum_f64(mass_above, sh);
    }
    *new_above = na;
    return b;
}

// Coarse sums of a chunk histogram in LDS: coarse bin c is the sum of bins
// c*FPC .. c*FPC + FPC - 1, four threads of 8 bins each (the reading order
// rotated by c against LDS bank conflicts), then combined pairwise; written to
// dst[c].  A fixed order: the sums are the same at every call.
__device__ __forceinline__ void write_coarse(const double* hist, double* __restrict__ dst) {
    const int c = threadIdx.x >> 2, q = threadIdx.x & 3;
    double a = 0.0;
#pragma unroll
    for (int i = 0; i < FPC / 4; ++i) a += hist[c * FPC + q * (FPC / 4) + ((i + c) & (FPC / 4 - 1))];
    a += __shfl_xor(a, 1, 64);
    a += __shfl_xor(a, 2, 64);
    if (q == 0) dst[c] = a;
}
static_assert(VT == 4 * NC && VT == 8 * FPC && FPC % 4 == 0 && VMAXP % 8 == 0,
              "four threads per coarse bin, eight per histogram bin of a coarse bin");

// The P chunks' coarse sums [P][NC]: the loads issued together (load_coarse,
// early, so that they travel with the kernel's other loads), then stored in
// LDS (commit_coarse).
constexpr int SC_U = VMAXP * NC / VT;
__device__ __forceinline__ void load_coarse(const double* __restrict__ hc, int P, double (&v)[SC_U]) {
    const int n = P * NC;
#pragma unroll
    for (int u = 0; u < SC_U; ++u) v[u] = hc[min((int)threadIdx.x + u * VT, n - 1)];
}

__device__ __forceinline__ void commit_coarse(const double (&v)[SC_U], int P, double* s_c) {
    const int n = P * NC;
#pragma unroll
    for (int u = 0; u < SC_U; ++u)
        if ((int)threadIdx.x + u * VT < n) s_c[threadIdx.x + u * VT] = v[u];
    __syncthreads();
}

// One level's cutoff bin from the chunk histograms hp [P][HB] and their coarse
// sums (in LDS, s_c [P][NC]): combine the coarse sums over the chunks in
// chunk order (times f[k] if f is set), descend to the coarse bin c holding
// the target, then load, combine and descend only the FPC histogram bins of c.
// Returns the bin (or -1 as descend does) and the mass above it.  Where
// rounding makes the coarse and the fine sums disagree about the crossing
// (a target within rounding of a coarse boundary), descend's fallback keeps a
// bin and the finishing pass, whose sums are exact in a fixed order, flags
// the row.  s_c is reused for the fine bins.
__device__ int steer(const double* __restrict__ hp, double* s_c, const double* f, int P, double above,
                     double target, double* new_above, double* s_bins, double* sh, int* shi) {
    const int tid = threadIdx.x;
    // coarse bin tid / 4 over chunk slots 16 (tid % 4) .. +16, then the four
    // partial sums pairwise (the reads of a run issued together)
    {
        const int cb = tid >> 2, q = tid & 3;
        double a = 0.0;
        if (f) {
#pragma unroll
            for (int u = 0; u < VMAXP / 4; ++u) {
                const int k = q * (VMAXP / 4) + u;
                if (k < P) a += f[k] * s_c[k * NC + cb];
            }
        } else {
#pragma unroll
            for (int u = 0; u < VMAXP / 4; ++u) {
                const int k = q * (VMAXP / 4) + u;
                if (k < P) a += s_c[k * NC + cb];
            }
        }
        a += __shfl_xor(a, 1, 64);
        a += __shfl_xor(a, 2, 64);
        if (q == 0) s_bins[cb] = a;
    }
    __syncthreads();
    double h[HB / VT];
#pragma unroll
    for (int i = 0; i < HB / VT; ++i) h[i] = (tid < NC / (HB / VT)) ? s_bins[tid * (HB / VT) + i] : 0.0;
    double above_c;
    const int c = descend(h, NC, above, target, &above_c, sh, shi);
    if (c < 0) {
        *new_above = above_c;
        return -1;
    }
    // the fine bins of c from every chunk, loads issued together
    constexpr int SF_U = VMAXP * FPC / VT;
    double v[SF_U];
    const int n = P * FPC;
#pragma unroll
    for (int u = 0; u < SF_U; ++u) {
        const int i = min(tid + u * VT, n - 1);
        v[u] = hp[(int64_t)(i / FPC) * HB + c * FPC + i % FPC];
    }
#pragma unroll
    for (int u = 0; u < SF_U; ++u)
        if (tid + u * VT < n) s_c[tid + u * VT] = v[u];
    __syncthreads();
    // bin tid / 8 of c over chunk slots 8 (tid % 8) .. +8, then the eight
    // partial sums pairwise
    {
        const int fb = tid >> 3, q = tid & 7;
        double a = 0.0;
        if (f) {
#pragma unroll
            for (int u = 0; u < VMAXP / 8; ++u) {
                const int k = q * (VMAXP / 8) + u;
                if (k < P) a += f[k] * s_c[k * FPC + fb];
            }
        } else {
#pragma unroll
            for (int u = 0; u < VMAXP / 8; ++u) {
                const int k = q * (VMAXP / 8) + u;
                if (k < P) a += s_c[k * FPC + fb];
            }
        }
        a += __shfl_xor(a, 1, 64);
        a += __shfl_xor(a, 2, 64);
        a += __shfl_xor(a, 4, 64);
        if (q == 0) s_bins[fb] = a;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < HB / VT; ++i) h[i] = (tid < FPC / (HB / VT)) ? s_bins[tid * (HB / VT) + i] : 0.0;
    double above_f;
    const int bf = descend(h, FPC, above_c, target, &above_f, sh, shi);
    *new_above = above_f;
    return bf < 0 ? -1 : c * FPC + bf;
}

// ---------------------------------------------------------------------------
// Phase 1: chunk max / argmax / min / non-finite; e relative to the chunk max;
// level-1 histogram.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(VT) void vs_chunk_kernel(const float* __restrict__ logits, float temperature,
                                                      float top_p, char* __restrict__ ws, VocabLayout L) {
    __shared__ double hist[HB];
    __shared__ double shd[16];
    __shared__ float shf[8];
    __shared__ int shi[8];
    const int w = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
    const RowView rv = row_view(ws, L, r);
    const float* z = logits + (int64_t)r * L.V;
    const int c0 = w * L.chunk, c1 = min(L.V, c0 + L.chunk);
    const double T = (double)temperature;

    float lm = -INFINITY, lmn = INFINITY;
    int li = 0x7fffffff;
    uint32_t bad = 0;
    // the first tile (the whole chunk unless V is huge) stays in registers for
    // both passes
    float v0[VU];
    load_tile(z, c0, c1, v0);
    for (int base = c0; base < c1; base += VT * VU) {
        float v[VU];
        if (base == c0) {
#pragma unroll
            for (int u = 0; u < VU; ++u) v[u] = v0[u];
        } else {
            load_tile(z, base, c1, v);
        }
#pragma unroll
        for (int u = 0; u < VU; ++u) {
            const int j = base + u * VT + tid;
            if (j < c1) {
                if (!isfinite(v[u])) bad = 1;
                lmn = fminf(lmn, v[u]);
                if (v[u] > lm || (v[u] == lm && j < li)) { lm = v[u]; li = j; }
            }
        }
    }
    for (int off = 32; off > 0; off >>= 1) {
        const float om = __shfl_xor(lm, off, 64);
        const int oi = __shfl_xor(li, off, 64);
        if (om > lm || (om == lm && oi < li)) { lm = om; li = oi; }
        lmn = fminf(lmn, __shfl_xor(lmn, off, 64));
    }
    if ((tid & 63) == 0) { shf[tid >> 6] = lm; shi[tid >> 6] = li; shf[4 + (tid >> 6)] = lmn; }
    __syncthreads();
    float m_w = shf[0];
    int a_w = shi[0];
    for (int k = 1; k < 4; ++k)
        if (shf[k] > m_w || (shf[k] == m_w && shi[k] < a_w)) { m_w = shf[k]; a_w = shi[k]; }
    const float mn_w = fminf(fminf(shf[4], shf[5]), fminf(shf[6], shf[7]));
    __syncthreads();
    const uint32_t bad_w = block_sum_u32(bad, (uint32_t*)shi) != 0;

    double E_w = 0.0;
    if (T > 0.0 && !bad_w) {
        const bool hist_on = top_p < 1.0f;
        if (hist_on) {
            for (int b = tid; b < HB; b += VT) hist[b] = 0.0;
            __syncthreads();
        }
        double es = 0.0;
        for (int base = c0; base < c1; base += VT * VU) {
            float v[VU];
            if (base == c0) {
#pragma unroll
                for (int u = 0; u < VU; ++u) v[u] = v0[u];
            } else {
                load_tile(z, base, c1, v);
            }
#pragma unroll
            for (int u = 0; u < VU; ++u) {
                const int j = base + u * VT + tid;
                if (j < c1) {
                    const double e = exp(((double)v[u] - (double)m_w) / T);
                    es += e;
                    if (hist_on) {
                        rv.e[j] = e;
                        atomicAdd(&hist[f32_key(v[u]) >> (32 - L1BITS)], e);
                    }
                }
            }
        }
        E_w = block_sum_f64(es, shd);
        if (hist_on) {
            for (int b = tid; b < HB; b += VT) rv.h1p[(int64_t)w * HB + b] = hist[b];
            write_coarse(hist, rv.h1c + (int64_t)w * NC);
        }
    }
    if (tid == 0) {
        ChunkPart p;
        p.m = m_w; p.argmax = a_w; p.bad = bad_w; p.mn = mn_w; p.E = E_w;
        rv.part[w] = p;
    }
}

// Phase 3: level-2 histogram of the chunk's logits inside the level-1 cutoff bin.
__global__ __launch_bounds__(VT) void vs_level2_kernel(const float* __restrict__ logits, float temperature,
                                                       float top_p, char* __restrict__ ws, VocabLayout L) {
    __shared__ double hist[HB];
    __shared__ double shd[16];
    __shared__ int shi[4];
    __shared__ ChunkPart sp[VMAXP];
    __shared__ double f[VMAXP];
    __shared__ double s_c[VMAXP * NC];
    __shared__ double s_bins[NC];
    const int w = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
    const RowView rv = row_view(ws, L, r);
    const float* z = logits + (int64_t)r * L.V;
    const int c0 = w * L.chunk, c1 = min(L.V, c0 + L.chunk);
    // every independent load first (one memory round trip): the chunk's first
    // tile of logits and e, the level-1 coarse sums, the chunk parts
    float v0[VU];
    double e0[VU], cv[SC_U];
    load_tile(z, c0, c1, v0);
    load_tile((const double*)rv.e, c0, c1, e0);
    load_coarse(rv.h1c, L.P, cv);
    stage_parts(rv.part, L.P, sp);
    commit_coarse(cv, L.P, s_c);
    __shared__ RowMax s_mx;
    __shared__ double s_E;
    const RowMax mx = steer_max(sp, L.P, &s_mx);
    if (mx.bad || !(temperature > 0.0f)) return;
    const double T = (double)temperature;
    const double E = steer_E(sp, L.P, mx.m, T, f, &s_E);
    const double target = (double)top_p * E;
    double above1;
    const int b1 = steer(rv.h1p, s_c, f, L.P, 0.0, target, &above1, s_bins, shd, shi);
    if (w == 0 && tid == 0) {
        Steer st;
        st.b = b1; st.pad = 0; st.above = above1;
        *rv.steer = st;
    }
    const double fw = f[w];
    for (int b = tid; b < HB; b += VT) hist[b] = 0.0;
    __syncthreads();
    if (b1 >= 0) {
        for (int base = c0; base < c1; base += VT * VU) {
            float v[VU];
            double ev[VU];
            if (base == c0) {
#pragma unroll
                for (int u = 0; u < VU; ++u) { v[u] = v0[u]; ev[u] = e0[u]; }
            } else {
                load_tile(z, base, c1, v);
                load_tile((const double*)rv.e, base, c1, ev);
            }
#pragma unroll
            for (int u = 0; u < VU; ++u) {
                if (base + u * VT + tid < c1) {
                    const uint32_t k = f32_key(v[u]);
                    if ((k >> (32 - L1BITS)) == (uint32_t)b1) atomicAdd(&hist[(k >> L3BITS) & (HB - 1)], ev[u] * fw);
                }
            }
        }
    }
    __syncthreads();
    for (int b = tid; b < HB; b += VT) rv.h2p[(int64_t)w * HB + b] = hist[b];
    write_coarse(hist, rv.h2c + (int64_t)w * NC);
}

// Phase 5: fixed-order mass/count above the 22-bit cutoff prefix and the
// level-3 counts inside it.
__global__ __launch_bounds__(VT) void vs_level3_kernel(const float* __restrict__ logits, float temperature,
                                                       float top_p, char* __restrict__ ws, VocabLayout L) {
    __shared__ uint32_t cnt[HB3];
    __shared__ double shd[16];
    __shared__ uint32_t shu[4];
    __shared__ int shi[4];
    __shared__ ChunkPart sp[VMAXP];
    __shared__ double f[VMAXP];
    __shared__ uint32_t s_nz;
    __shared__ double s_c[VMAXP * NC];
    __shared__ double s_bins[NC];
    const int w = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
    const RowView rv = row_view(ws, L, r);
    const float* z = logits + (int64_t)r * L.V;
    const int c0 = w * L.chunk, c1 = min(L.V, c0 + L.chunk);
    // every independent load first (one memory round trip): the tiles, the
    // level-1 cutoff the level-2 pass published, the level-2 coarse sums
    float v0[VU];
    double e0[VU], cv[SC_U];
    load_tile(z, c0, c1, v0);
    load_tile((const double*)rv.e, c0, c1, e0);
    const Steer st1 = *rv.steer;
    load_coarse(rv.h2c, L.P, cv);
    stage_parts(rv.part, L.P, sp);
    commit_coarse(cv, L.P, s_c);
    __shared__ RowMax s_mx;
    __shared__ double s_E;
    const RowMax mx = steer_max(sp, L.P, &s_mx);
    if (mx.bad || !(temperature > 0.0f)) return;
    const double T = (double)temperature;
    const double E = steer_E(sp, L.P, mx.m, T, f, &s_E);
    const double target = (double)top_p * E;
    const int b1 = st1.b;
    const double above1 = st1.above;
    double above2 = 0.0;
    const int b2 = (b1 >= 0) ? steer(rv.h2p, s_c, nullptr, L.P, above1, target, &above2, s_bins, shd, shi) : -1;
    const double fw = f[w];
    for (int b = tid; b < HB3; b += VT) cnt[b] = 0u;
    if (tid == 0) s_nz = 0u;
    __syncthreads();
    // without a usable steering bin (only rounding can cause this) the prefix
    // is placed above every key: nothing is "above", all counts land in bins
    // the finishing pass treats as a flagged boundary case
    const uint32_t prefix = (b1 >= 0 && b2 >= 0) ? (((uint32_t)b1 << L2BITS) | (uint32_t)b2) : 0x3fffffu;
    double sa = 0.0;
    uint32_t na = 0;
    for (int base = c0; base < c1; base += VT * VU) {
        float v[VU];
        double ev[VU];
        if (base == c0) {
#pragma unroll
            for (int u = 0; u < VU; ++u) { v[u] = v0[u]; ev[u] = e0[u]; }
        } else {
            load_tile(z, base, c1, v);
            load_tile((const double*)rv.e, base, c1, ev);
        }
#pragma unroll
        for (int u = 0; u < VU; ++u) {
            if (base + u * VT + tid < c1) {
                const uint32_t k = f32_key(v[u]);
                const uint32_t hi = k >> L3BITS;
                if (hi > prefix) { sa += ev[u] * fw; ++na; }
                else if (hi == prefix) atomicAdd(&cnt[k & (HB3 - 1)], 1u);
            }
        }
    }
    sa = block_sum_f64(sa, shd);
    na = block_sum_u32(na, shu);
    // the non-empty bins into the chunk's record (slots taken in any order:
    // the finishing pass only adds integer counts per bin)
    uint32_t* rec = rv.rec + (int64_t)w * REC;
    for (int b = tid; b < HB3; b += VT) {
        const uint32_t c = cnt[b];
        if (c) {
            const uint32_t slot = atomicAdd(&s_nz, 1u);
            if (slot < (uint32_t)REC_CAP) rec[REC_HEAD + slot] = (c << 10) | (uint32_t)b;
        }
    }
    __syncthreads();
    const uint32_t nz = s_nz;
    if (nz > (uint32_t)REC_CAP)
        for (int b = tid; b < HB3; b += VT) rv.c3[(int64_t)w * HB3 + b] = cnt[b];
    if (tid == 0) {
        ChunkSums s;
        s.above = sa; s.n_above = na; s.pad = prefix;
        *(ChunkSums*)rec = s;
        rec[4] = nz;
    }
}

// Phase 6: per row (HB3 = 1024 threads): finish and write the statistics.
__global__ __launch_bounds__(HB3) void vs_finish_kernel(float temperature, float top_p, char* __restrict__ ws,
                                                        VocabLayout L, vw4_rowstat* __restrict__ stats) {
    __shared__ double sh[HB3 / 64 + 4];
    __shared__ int s_b;
    __shared__ double s_cum;
    __shared__ ChunkPart sp[VMAXP];
    __shared__ __align__(16) uint32_t s_rec[VMAXP * REC];
    __shared__ uint32_t s_cnt[HB3];
    const int r = blockIdx.x, tid = threadIdx.x;
    const RowView rv = row_view(ws, L, r);
    // every independent load first (one memory round trip): the chunk parts
    // and the chunks' phase-5 records (at most VMAXP * REC / HB3 = 4 words per
    // thread, clamped loads issued together)
    const bool topp = top_p < 1.0f && temperature > 0.0f;
    if (topp) {
        const int nrec = L.P * REC;
        uint32_t rw[VMAXP * REC / HB3];
#pragma unroll
        for (int u = 0; u < VMAXP * REC / HB3; ++u) rw[u] = rv.rec[min(tid + u * HB3, nrec - 1)];
#pragma unroll
        for (int u = 0; u < VMAXP * REC / HB3; ++u)
            if (tid + u * HB3 < nrec) s_rec[tid + u * HB3] = rw[u];
        s_cnt[tid] = 0u;
    }
    for (int k = tid; k < L.P; k += blockDim.x) sp[k] = rv.part[k];
    __syncthreads();
    const double T = (double)temperature;
    // the level-3 counts of all chunks, bin by bin: the record entries, or the
    // dense counts of a chunk whose record overflowed (rare: its 22-bit prefix
    // bin then holds more than REC_CAP distinct values).  Records of a row
    // that stopped early (non-finite, T == 0) are never used.
    if (topp) {
        bool dense = false;
        for (int i = tid; i < L.P * REC; i += HB3) {
            const int k = i / REC, j = i % REC;
            const uint32_t nz = s_rec[k * REC + 4];
            if (j >= REC_HEAD && (uint32_t)(j - REC_HEAD) < nz) {
                if (nz <= (uint32_t)REC_CAP) atomicAdd(&s_cnt[s_rec[i] & (HB3 - 1)], s_rec[i] >> 10);
                else dense = true;
            }
        }
        if (__syncthreads_or(dense)) {
            for (int k = 0; k < L.P; ++k)
                if (s_rec[k * REC + 4] > (uint32_t)REC_CAP)
                    atomicAdd(&s_cnt[tid], rv.c3[(int64_t)k * HB3 + tid]);
        }
    }
    // the row header, by wavefront 0: max, E, and the mass and count above the
    // cutoff prefix summed over the chunks in chunk order
    __shared__ RowMax s_mx;
    __shared__ double s_E, s_above;
    __shared__ uint32_t s_na;
    if (tid < 64) {
        const RowMax h = wave_combine_max(sp, L.P);
        double E = 0.0, above = 0.0;
        uint32_t na = 0;
        if (!h.bad && T > 0.0) {
            E = wave_combine_E(sp, L.P, h.m, T);
            if (topp) {
                const ChunkSums* sk = (const ChunkSums*)&s_rec[min(tid, L.P - 1) * REC];
                const double a = sk->above;
                for (int k = 0; k < L.P; ++k) above += readlane_f64(a, k);
                na = (tid < L.P) ? sk->n_above : 0u;
                for (int off = 32; off > 0; off >>= 1) na += __shfl_xor(na, off, 64);
            }
        }
        if (tid == 0) { s_mx = h; s_E = E; s_above = above; s_na = na; }
    }
    __syncthreads();
    const RowMax mx = s_mx;
    vw4_rowstat s;
    s.max_logit = mx.m;
    s.argmax = mx.argmax;
    s.pad = 0;
    if (mx.bad || !(T > 0.0)) {
        if (tid == 0) {
            s.max_logit = mx.bad ? NAN : mx.m;
            s.tau = s.max_logit;
            s.log_z = 0.0;
            s.argmax = mx.bad ? -1 : mx.argmax;
            s.n_kept = mx.bad ? 0 : 1;
            s.flags = mx.bad ? VW4_FLAG_NONFINITE : 0u;
            stats[r] = s;
        }
        return;
    }
    const double E = s_E;
    if (!(top_p < 1.0f)) {
        if (tid == 0) {
            s.tau = mx.mn;
            s.log_z = log(E);
            s.n_kept = L.V;
            s.flags = 0;
            stats[r] = s;
        }
        return;
    }
    const double target = (double)top_p * E;
    const double above = s_above;
    const uint32_t n_above = s_na;
    const uint32_t prefix = ((const ChunkSums*)&s_rec[0])->pad;
    // level-3 bin b (thread b): one float value, mass = count * e(value)
    const uint32_t c = s_cnt[tid];
    const float zb = key_f32((prefix << L3BITS) | (uint32_t)tid);
    const double eb = (c && prefix != 0x3fffffu) ? exp(((double)zb - (double)mx.m) / T) : 0.0;
    const double mass = (double)c * eb;
    // suffix sums over the bins above each thread's bin (fixed tree order)
    const int lane = tid & 63, wv = tid >> 6;
    double sfx = mass;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double t = __shfl_down(sfx, off, 64);
        if (lane + off < 64) sfx += t;
    }
    if (lane == 0) sh[wv] = sfx;
    if (tid == 0) s_b = -1;
    __syncthreads();
    double later = 0.0;
    for (int w2 = HB3 / 64 - 1; w2 > wv; --w2) later += sh[w2];
    double ex = __shfl_down(sfx, 1, 64);
    if (lane == 63) ex = 0.0;
    const double cum_above = above + later + ex;  // mass of every key above this bin
    if (c && cum_above < target && cum_above + mass >= target) { s_b = tid; s_cum = cum_above; }
    __syncthreads();
    uint32_t flags = 0;
    int b3 = s_b;
    double G = s_cum;
    if (b3 < 0) {
        // steering missed the boundary by rounding: keep the nearest bin and flag it
        flags |= VW4_FLAG_TOPP_TIE;
        __shared__ int s_lo, s_hi;
        if (tid == 0) { s_lo = 0x7fffffff; s_hi = -1; }
        __syncthreads();
        if (c) { atomicMin(&s_lo, tid); atomicMax(&s_hi, tid); }
        __syncthreads();
        b3 = (above >= target) ? s_hi : s_lo;
        if (b3 < 0 || b3 >= HB3) b3 = 0;
        G = 0.0;
    }
    // Z = mass above + bins >= b3, in bin order from the top
    __syncthreads();
    const double mine = (tid >= b3) ? mass : 0.0;
    double zsum = wave_sum(mine);
    uint32_t nmine = (tid >= b3) ? c : 0u;
    uint32_t nsum = wave_sum(nmine);
    __shared__ double shz[HB3 / 64];
    __shared__ uint32_t shn[HB3 / 64];
    if (lane == 0) { shz[wv] = zsum; shn[wv] = nsum; }
    __syncthreads();
    if (tid != 0) return;
    double Zin = 0.0;
    uint32_t nin = 0;
    for (int k = HB3 / 64 - 1; k >= 0; --k) { Zin += shz[k]; nin += shn[k]; }
    const double Z = above + Zin;
    if (!(flags & VW4_FLAG_TOPP_TIE)) {
        if (fabs(Z - target) < 1e-9 * E || fabs(G - target) < 1e-9 * E) flags |= VW4_FLAG_TOPP_TIE;
    }
    s.tau = key_f32((prefix << L3BITS) | (uint32_t)b3);
    s.log_z = log(Z);
    s.n_kept = (int32_t)(n_above + nin);
    s.flags = flags;
    stats[r] = s;
}

// ---------------------------------------------------------------------------
// V <= RT * RU: one workgroup per row does every phase in LDS (one launch).
// The arithmetic is that of the chunked path with a single chunk: e relative
// to the row max, fixed-order block sums, the same three-level descent and
// the same finish and flags.
// ---------------------------------------------------------------------------
constexpr int RT = 1024, RNW = RT / 64, RU = 16;
constexpr int RHPT = HB / RT;            // level-1/2 bins per thread

__device__ __forceinline__ double row_sum_f64(double v, double* sh) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < RNW; ++k) s += sh[k];           // wavefront order
    __syncthreads();
    return s;
}

__device__ __forceinline__ uint32_t row_sum_u32(uint32_t v, uint32_t* sh) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t s = 0;
#pragma unroll
    for (int k = 0; k < RNW; ++k) s += sh[k];
    __syncthreads();
    return s;
}

// Exclusive suffix sum over the RT threads (fixed order).
__device__ __forceinline__ double row_suffix_excl(double v, double* sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    double s = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double t = __shfl_down(s, off, 64);
        if (lane + off < 64) s += t;
    }
    if (lane == 0) sh[w] = s;
    __syncthreads();
    double later = 0.0;
    for (int w2 = RNW - 1; w2 > w; --w2) later += sh[w2];
    double ex = __shfl_down(s, 1, 64);
    if (lane == 63) ex = 0.0;
    __syncthreads();
    return ex + later;
}

// Descend the HB bins in hist (LDS; thread t owns bins RHPT t .. +RHPT): the
// largest bin b with above + sum_{b' >= b} H[b'] >= target, -1 if none (then
// the lowest non-empty bin, as in the chunked path).
__device__ int row_descend(const double* hist, double above, double target, double* new_above, double* sh,
                           int* shi) {
    const int b0 = threadIdx.x * RHPT;
    double h[RHPT], mine = 0.0;
#pragma unroll
    for (int i = 0; i < RHPT; ++i) {
        h[i] = hist[b0 + i];
        mine += h[i];
    }
    const double later = row_suffix_excl(mine, sh);
    if (threadIdx.x == 0) shi[0] = -1;
    __syncthreads();
    double cum = above + later;
#pragma unroll
    for (int i = RHPT - 1; i >= 0; --i) {
        if (cum < target && cum + h[i] >= target) {
            shi[0] = b0 + i;
            sh[RNW] = cum;
        }
        cum += h[i];
    }
    __syncthreads();
    int b = shi[0];
    double na = (b >= 0) ? sh[RNW] : above;
    __syncthreads();
    if (b < 0) {
        if (threadIdx.x == 0) shi[0] = 0x7fffffff;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < RHPT; ++i)
            if (h[i] > 0.0) atomicMin(&shi[0], b0 + i);
        __syncthreads();
        b = shi[0];
        if (b == 0x7fffffff) b = -1;
        double mass_above = 0.0;
#pragma unroll
        for (int i = 0; i < RHPT; ++i)
            if (b0 + i > b) mass_above += h[i];
        na = above + row_sum_f64(mass_above, sh);
    }
    *new_above = na;
    return b;
}

__global__ __launch_bounds__(RT) void vs_row_kernel(const float* __restrict__ logits, float temperature, float top_p,
                                                    int V, vw4_rowstat* __restrict__ stats) {
    __shared__ double hist[HB];
    __shared__ uint32_t cnt[HB3];
    __shared__ double sh[RNW + 4];
    __shared__ float shf[2 * RNW];
    __shared__ int shi[RNW + 4];
    const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const float* z = logits + (int64_t)r * V;
    float v[RU];
#pragma unroll
    for (int u = 0; u < RU; ++u) {
        const int j = u * RT + tid;
        v[u] = (j < V) ? z[j] : 0.0f;
    }
    // max (lowest index on ties), min, non-finite
    float lm = -INFINITY, lmn = INFINITY;
    int li = 0x7fffffff;
    uint32_t bad = 0;
#pragma unroll
    for (int u = 0; u < RU; ++u) {
        const int j = u * RT + tid;
        if (j < V) {
            if (!isfinite(v[u])) bad = 1;
            lmn = fminf(lmn, v[u]);
            if (v[u] > lm || (v[u] == lm && j < li)) { lm = v[u]; li = j; }
        }
    }
    for (int off = 32; off > 0; off >>= 1) {
        const float om = __shfl_xor(lm, off, 64);
        const int oi = __shfl_xor(li, off, 64);
        if (om > lm || (om == lm && oi < li)) { lm = om; li = oi; }
        lmn = fminf(lmn, __shfl_xor(lmn, off, 64));
    }
    if (lane == 0) { shf[wv] = lm; shi[wv] = li; shf[RNW + wv] = lmn; }
    __syncthreads();
    float m = shf[0], mn = shf[RNW];
    int am = shi[0];
    for (int k = 1; k < RNW; ++k) {
        if (shf[k] > m || (shf[k] == m && shi[k] < am)) { m = shf[k]; am = shi[k]; }
        mn = fminf(mn, shf[RNW + k]);
    }
    __syncthreads();
    const bool isbad = row_sum_u32(bad, (uint32_t*)shi) != 0;
    const double T = (double)temperature;
    vw4_rowstat s;
    s.max_logit = m;
    s.argmax = am;
    s.pad = 0;
    if (isbad || !(T > 0.0)) {
        if (tid == 0) {
            s.max_logit = isbad ? NAN : m;
            s.tau = s.max_logit;
            s.log_z = 0.0;
            s.argmax = isbad ? -1 : am;
            s.n_kept = isbad ? 0 : 1;
            s.flags = isbad ? VW4_FLAG_NONFINITE : 0u;
            stats[r] = s;
        }
        return;
    }
    double e[RU], es = 0.0;
#pragma unroll
    for (int u = 0; u < RU; ++u) {
        e[u] = (u * RT + tid < V) ? exp(((double)v[u] - (double)m) / T) : 0.0;
        es += e[u];
    }
    const double E = row_sum_f64(es, sh);
    if (!(top_p < 1.0f)) {
        if (tid == 0) {
            s.tau = mn;
            s.log_z = log(E);
            s.n_kept = V;
            s.flags = 0;
            stats[r] = s;
        }
        return;
    }
    const double target = (double)top_p * E;
    // level 1
    for (int b = tid; b < HB; b += RT) hist[b] = 0.0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < RU; ++u)
        if (u * RT + tid < V) atomicAdd(&hist[f32_key(v[u]) >> (32 - L1BITS)], e[u]);
    __syncthreads();
    double above1, above2 = 0.0;
    const int b1 = row_descend(hist, 0.0, target, &above1, sh, shi);
    // level 2
    for (int b = tid; b < HB; b += RT) hist[b] = 0.0;
    __syncthreads();
    if (b1 >= 0) {
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            if (u * RT + tid < V) {
                const uint32_t k = f32_key(v[u]);
                if ((k >> (32 - L1BITS)) == (uint32_t)b1) atomicAdd(&hist[(k >> L3BITS) & (HB - 1)], e[u]);
            }
        }
    }
    __syncthreads();
    const int b2 = (b1 >= 0) ? row_descend(hist, above1, target, &above2, sh, shi) : -1;
    const uint32_t prefix = (b1 >= 0 && b2 >= 0) ? (((uint32_t)b1 << L2BITS) | (uint32_t)b2) : 0x3fffffu;
    // level 3: counts inside the prefix, mass and count above it
    for (int b = tid; b < HB3; b += RT) cnt[b] = 0u;
    __syncthreads();
    double sa = 0.0;
    uint32_t na = 0;
#pragma unroll
    for (int u = 0; u < RU; ++u) {
        if (u * RT + tid < V) {
            const uint32_t k = f32_key(v[u]);
            const uint32_t hi = k >> L3BITS;
            if (hi > prefix) { sa += e[u]; ++na; }
            else if (hi == prefix) atomicAdd(&cnt[k & (HB3 - 1)], 1u);
        }
    }
    const double above = row_sum_f64(sa, sh);
    const uint32_t n_above = row_sum_u32(na, (uint32_t*)shi);
    // finish (thread b = level-3 bin b): one float value per bin, mass = count * e(value)
    static_assert(RT == HB3, "one thread per level-3 bin");
    const uint32_t c = cnt[tid];
    const float zb = key_f32((prefix << L3BITS) | (uint32_t)tid);
    const double eb = (c && prefix != 0x3fffffu) ? exp(((double)zb - (double)m) / T) : 0.0;
    const double mass = (double)c * eb;
    const double cum_above = above + row_suffix_excl(mass, sh);  // mass of every key above this bin
    __shared__ int s_b;
    __shared__ double s_cum;
    if (tid == 0) s_b = -1;
    __syncthreads();
    if (c && cum_above < target && cum_above + mass >= target) { s_b = tid; s_cum = cum_above; }
    __syncthreads();
    uint32_t flags = 0;
    int b3 = s_b;
    double G = s_cum;
    if (b3 < 0) {
        // steering missed the boundary by rounding: keep the nearest bin and flag it
        flags |= VW4_FLAG_TOPP_TIE;
        __shared__ int s_lo, s_hi;
        if (tid == 0) { s_lo = 0x7fffffff; s_hi = -1; }
        __syncthreads();
        if (c) { atomicMin(&s_lo, tid); atomicMax(&s_hi, tid); }
        __syncthreads();
        b3 = (above >= target) ? s_hi : s_lo;
        if (b3 < 0 || b3 >= HB3) b3 = 0;
        G = 0.0;
    }
    __syncthreads();
    // Z = mass above + bins >= b3 (block sum in wavefront order)
    const double Zin = row_sum_f64((tid >= b3) ? mass : 0.0, sh);
    const uint32_t nin = row_sum_u32((tid >= b3) ? c : 0u, (uint32_t*)shi);
    if (tid != 0) return;
    const double Z = above + Zin;
    if (!(flags & VW4_FLAG_TOPP_TIE)) {
        if (fabs(Z - target) < 1e-9 * E || fabs(G - target) < 1e-9 * E) flags |= VW4_FLAG_TOPP_TIE;
    }
    s.tau = key_f32((prefix << L3BITS) | (uint32_t)b3);
    s.log_z = log(Z);
    s.n_kept = (int32_t)(n_above + nin);
    s.flags = flags;
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
    if (V <= RT * RU) {
        hipLaunchKernelGGL(vs_row_kernel, dim3(rows), dim3(RT), 0, st, logits, temperature, top_p, V, stats);
        return check_launch("verify_logits");
    }
    char* w = (char*)ws;
    const dim3 grid(L.P, rows);
    hipLaunchKernelGGL(vs_chunk_kernel, grid, dim3(VT), 0, st, logits, temperature, top_p, w, L);
    if (temperature > 0.0f && top_p < 1.0f) {
        hipLaunchKernelGGL(vs_level2_kernel, grid, dim3(VT), 0, st, logits, temperature, top_p, w, L);
        hipLaunchKernelGGL(vs_level3_kernel, grid, dim3(VT), 0, st, logits, temperature, top_p, w, L);
    }
    hipLaunchKernelGGL(vs_finish_kernel, dim3(rows), dim3(HB3), 0, st, temperature, top_p, w, L, stats);
    return check_launch("verify_logits");
}

}  // extern "C"
