/*
 * oracle.c — plain, slow, obviously-correct CPU oracle for the batched verify
 * step of MTP self-speculative decoding.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * path (verify_step_w4_amd/csrc); the two meet only through the seeded input
 * generators.
 *
 * Every floating-point result is computed in IEEE binary64 from the exact
 * values of the binary16/bfloat16/binary32 inputs, sequentially and in the
 * order the definition states.  No blocking, no fusion, no reordering.
 *
 * Sources followed (cited by page title and section):
 *  [mtplx/4層]   hazakura.dev, "mtplx——M5 Maxで63tok/s、Apple SiliconのローカルLLMが
 *                2倍以上速くなる日", section "4層のアーキテクチャ": Layer 0 (small-M matmul
 *                shader change, 4-bit LM head) and Layer 2 (draft -> one parallel
 *                verify -> probability-ratio acceptance -> residual correction ->
 *                bonus token).
 *  [mtplx/数字]  same page, section "mtplxの数字——本当なの？" (table row
 *                "max_diff = 0.0"; Leviathan–Chen ratio rejection at T=0.6, not greedy).
 *  [MTPLX/裏技]  devtrends.cc, "Apple Silicon上でローカルLLMを最大2倍高速化するMTPLX",
 *                section "2つ目のモデル不要！MTPの裏技" (all drafts verified in one
 *                forward pass; exact rejection sampling with residual correction;
 *                temperature 0.6 / top_p 0.95 give the same distribution as plain
 *                step-by-step sampling).
 *  [BaseRT/方法] gist.science, "BaseRT: Best-in-Class LLM Inference on Apple Silicon
 *                via Native Metal", technical summary, section "メソドロジー"
 *                (dequantisation inside the GEMV inner loop; FlashAttention with
 *                online softmax).
 *  The pages fix neither the weight format, the warp order, the tie rules nor
 *  the random-number generator; the readings used here are listed beside each
 *  function and in the design notes of the repository.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* Number formats, written from the IEEE 754 / bfloat16 bit layouts.         */
/* ------------------------------------------------------------------------ */

/* bfloat16 is the top half of a binary32. */
static double bf16_value(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double f16_value(uint16_t h) {
    int s = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)f, -24);              /* subnormal */
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(1024 + f), e - 25);           /* (1.f) * 2^(e-15) */
    return s ? -v : v;
}

/* binary32 -> binary16, round to nearest, ties to even.  The binary32 value is
 * exact in binary64, and scaling by a power of two is exact, so rint() in the
 * default rounding mode performs the single IEEE rounding. */
EXPORT uint16_t oracle_f32_to_f16(float f) {
    uint32_t ub;
    memcpy(&ub, &f, 4);
    uint16_t sign = (uint16_t)((ub >> 16) & 0x8000u);
    double x = fabs((double)f);
    if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
    if (x == 0.0) return sign;
    if (x < ldexp(1.0, -14)) {                     /* subnormal range, ulp 2^-24 */
        double q = rint(x * ldexp(1.0, 24));       /* 0 .. 1024 (1024 = min normal) */
        return (uint16_t)(sign | (uint16_t)q);
    }
    int e;
    (void)frexp(x, &e);                            /* x = f * 2^e, f in [0.5, 1) */
    e -= 1;                                        /* x in [2^e, 2^(e+1)) */
    double m = rint(ldexp(x, 10 - e));             /* 1024 .. 2048 */
    if (m == 2048.0) { m = 1024.0; e += 1; }
    if (e + 15 >= 31) return (uint16_t)(sign | 0x7c00u);   /* overflow -> inf */
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(m - 1024.0));
}

EXPORT double oracle_f16_value(uint16_t h) { return f16_value(h); }

/* binary64 -> bfloat16 (1 sign, 8 exponent bits with bias 127, 7 fraction
 * bits), one rounding to nearest, ties to even; overflow -> inf. */
EXPORT uint16_t oracle_bf16_round(double v) {
    uint16_t sign = (uint16_t)(signbit(v) ? 0x8000u : 0u);
    double x = fabs(v);
    if (isnan(v)) return (uint16_t)(sign | 0x7fc0u);
    if (isinf(v)) return (uint16_t)(sign | 0x7f80u);   /* infinities are exact */
    if (x == 0.0) return sign;
    if (x < ldexp(1.0, -126)) {                    /* subnormal, ulp 2^-133 */
        double q = rint(x * ldexp(1.0, 133));      /* 0 .. 128 (128 = min normal) */
        return (uint16_t)(sign | (uint16_t)q);
    }
    int e;
    (void)frexp(x, &e);
    e -= 1;                                        /* x in [2^e, 2^(e+1)) */
    double m = rint(ldexp(x, 7 - e));              /* 128 .. 256 */
    if (m == 256.0) { m = 128.0; e += 1; }
    if (e + 127 >= 255) return (uint16_t)(sign | 0x7f80u);
    return (uint16_t)(sign | (uint16_t)((e + 127) << 7) | (uint16_t)(m - 128.0));
}

EXPORT double oracle_bf16_value(uint16_t h) { return bf16_value(h); }

/* ------------------------------------------------------------------------ */
/* (a1) W4 weight format: symmetric int4, group 64 along K, fp16 scales.    */
/* Reading (the pages say only "4-bit", [mtplx/4層] Layer 0): codes in       */
/* [-7, 7]; scale = fp16(absmax / 7) rounded to nearest-even; codes use the  */
/* rounded scale; round half to even; clamp; an all-zero (or underflowing)   */
/* group gets scale 0 and codes 0.  Canonical storage: u8 codes[N][K/2]      */
/* holding u = c + 8, even k in the low nibble; f16 scales[N][K/64].          */
/* ------------------------------------------------------------------------ */
EXPORT void oracle_w4_quantize(const float* w, int64_t N, int64_t K,
                               uint8_t* codes, uint16_t* scales) {
    const int64_t G = K / 64;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float* wg = w + n * K + g * 64;
            float a = 0.0f;
            for (int k = 0; k < 64; ++k) {
                float v = fabsf(wg[k]);
                if (v > a) a = v;
            }
            float s32 = a / 7.0f;                       /* binary32 division */
            uint16_t s16 = oracle_f32_to_f16(s32);
            float sf = (float)f16_value(s16);
            scales[n * G + g] = s16;
            for (int k = 0; k < 64; ++k) {
                int c = 0;
                if (sf != 0.0f) {
                    float r = rintf(wg[k] / sf);        /* binary32 division, half-even */
                    if (r > 7.0f) r = 7.0f;
                    if (r < -7.0f) r = -7.0f;
                    c = (int)r;
                }
                int64_t kk = g * 64 + k;
                uint8_t* byte = codes + n * (K / 2) + kk / 2;
                uint8_t u = (uint8_t)(c + 8);
                if ((kk & 1) == 0) *byte = (uint8_t)((*byte & 0xF0u) | u);
                else               *byte = (uint8_t)((*byte & 0x0Fu) | (u << 4));
            }
        }
    }
}

/* Integer code of element (n, k) from the canonical layout. */
static int code_at(const uint8_t* codes, int64_t K, int64_t n, int64_t k) {
    uint8_t b = codes[n * (K / 2) + k / 2];
    int u = (k & 1) ? (b >> 4) : (b & 15);
    return u - 8;
}

EXPORT int oracle_w4_code(const uint8_t* codes, int64_t K, int64_t n, int64_t k) {
    return code_at(codes, K, n, k);
}

/* ------------------------------------------------------------------------ */
/* (a2/a3) W4 skinny GEMM: y[m][n] = sum_k x[m][k] * c[n][k] * s[n][k/64].   */
/* The definition of a matmul over the dequantised matrix ([BaseRT/方法]:     */
/* dequantisation is part of the product, weights are never materialised).  */
/* fp64, sequential in k.  Rows n are independent, so they are split over     */
/* host threads; each output is still one sequential sum.                     */
/* ------------------------------------------------------------------------ */
EXPORT void oracle_w4_gemm(const uint16_t* x_bf16, int64_t M, int64_t K,
                           const uint8_t* codes, const uint16_t* scales, int64_t N,
                           double* y /* [M][N] */) {
    const int64_t G = K / 64;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double xv = bf16_value(x_bf16[m * K + k]);
                double c = (double)code_at(codes, K, n, k);
                double s = f16_value(scales[n * G + k / 64]);
                acc += xv * c * s;
            }
            y[m * N + n] = acc;
        }
    }
}

/* Selected outputs only (for spot checks of very large products). */
EXPORT void oracle_w4_gemm_at(const uint16_t* x_bf16, int64_t K, const uint8_t* codes_row,
                              const uint16_t* scales_row, double* out) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        uint8_t b = codes_row[k / 2];
        int c = ((k & 1) ? (b >> 4) : (b & 15)) - 8;
        acc += bf16_value(x_bf16[k]) * (double)c * f16_value(scales_row[k / 64]);
    }
    *out = acc;
}

/* ------------------------------------------------------------------------ */
/* Compensated (Neumaier) summation helper: s is the running sum, c the       */
/* running compensation; the sum is s + c.                                    */
/* ------------------------------------------------------------------------ */
static void kahan_add(double* s, double* c, double v) {
    double t = *s + v;
    if (fabs(*s) >= fabs(v)) *c += (*s - t) + v;
    else                     *c += (v - t) + *s;
    *s = t;
}

/* ------------------------------------------------------------------------ */
/* (a4) Temperature + top-p warp of one row of fp32 logits.                   */
/* [MTPLX/裏技]: sampling at temperature 0.6 and top_p 0.95 ("nucleus").     */
/* Reading (pages silent): temperature first, then top-p on the tempered     */
/* distribution; the kept set is the smallest prefix of the vocabulary       */
/* sorted by (logit descending, index ascending) whose mass reaches          */
/* top_p * E, widened to every token whose logit equals the cutoff logit     */
/* tau; top_p >= 1 keeps everything; T == 0 is greedy (argmax, lowest index   */
/* on ties).                                                                  */
/* ------------------------------------------------------------------------ */
typedef struct {
    double m;         /* max logit */
    double tau;       /* cutoff logit (kept set: z >= tau) */
    double E;         /* sum of exp((z - m)/T) over the whole row */
    double Z;         /* sum over the kept set */
    double log_z;
    double P;         /* top_p * E */
    double S_at;      /* sorted prefix mass including the cutoff position */
    double S_before;  /* sorted prefix mass before the cutoff position */
    int64_t argmax;
    int64_t n_kept;
    int64_t k_star;   /* cutoff position in the sorted order */
    uint32_t flags;   /* bit0: non-finite logit; bit1: top-p boundary within 1e-9*E */
    uint32_t pad;
} oracle_warp_t;

static const float* g_sort_z;   /* comparator context (single-threaded use) */
static int cmp_desc(const void* a, const void* b) {
    int64_t i = *(const int64_t*)a, j = *(const int64_t*)b;
    float zi = g_sort_z[i], zj = g_sort_z[j];
    if (zi > zj) return -1;
    if (zi < zj) return 1;
    return (i < j) ? -1 : (i > j);
}

EXPORT void oracle_warp(const float* z, int64_t V, float temperature, float top_p,
                        oracle_warp_t* st, double* p /* nullable, [V] */) {
    memset(st, 0, sizeof(*st));
    for (int64_t j = 0; j < V; ++j)
        if (!isfinite(z[j])) { st->flags |= 1u; st->argmax = -1; st->n_kept = 0; return; }
    int64_t a = 0;
    for (int64_t j = 1; j < V; ++j) if (z[j] > z[a]) a = j;
    st->argmax = a;
    st->m = (double)z[a];
    const double T = (double)temperature;
    if (T == 0.0) {
        st->tau = st->m; st->E = 1.0; st->Z = 1.0; st->log_z = 0.0; st->P = 1.0;
        st->n_kept = 1; st->k_star = 0; st->S_at = 1.0; st->S_before = 0.0;
        if (p) { for (int64_t j = 0; j < V; ++j) p[j] = 0.0; p[a] = 1.0; }
        return;
    }
    double* e = (double*)malloc((size_t)V * sizeof(double));
    double es = 0.0, ec = 0.0;
    for (int64_t j = 0; j < V; ++j) {
        e[j] = exp(((double)z[j] - st->m) / T);
        kahan_add(&es, &ec, e[j]);
    }
    st->E = es + ec;
    const double P = (double)top_p * st->E;
    st->P = P;
    if ((double)top_p >= 1.0) {
        double mn = (double)z[0];
        for (int64_t j = 1; j < V; ++j) if ((double)z[j] < mn) mn = (double)z[j];
        st->tau = mn; st->n_kept = V; st->k_star = V - 1;
        st->Z = st->E; st->S_at = st->E; st->S_before = st->E;
    } else {
        int64_t* ord = (int64_t*)malloc((size_t)V * sizeof(int64_t));
        for (int64_t j = 0; j < V; ++j) ord[j] = j;
        g_sort_z = z;
        qsort(ord, (size_t)V, sizeof(int64_t), cmp_desc);
        double ps = 0.0, pc = 0.0, before = 0.0;
        int64_t ks = V - 1;
        for (int64_t k = 0; k < V; ++k) {
            before = ps + pc;
            kahan_add(&ps, &pc, e[ord[k]]);
            if (ps + pc >= P) { ks = k; break; }
        }
        st->k_star = ks;
        st->S_at = ps + pc;
        st->S_before = before;
        st->tau = (double)z[ord[ks]];
        double zs = 0.0, zc = 0.0;
        int64_t nk = 0;
        for (int64_t j = 0; j < V; ++j)
            if ((double)z[j] >= st->tau) { kahan_add(&zs, &zc, e[j]); ++nk; }
        st->Z = zs + zc;
        st->n_kept = nk;
        if (fabs(st->S_at - P) < 1e-9 * st->E || fabs(st->S_before - P) < 1e-9 * st->E)
            st->flags |= 2u;
        free(ord);
    }
    st->log_z = log(st->Z);
    if (p) {
        for (int64_t j = 0; j < V; ++j)
            p[j] = ((double)z[j] >= st->tau) ? e[j] / st->Z : 0.0;
    }
    free(e);
}

/* ------------------------------------------------------------------------ */
/* (a5) Philox4x64-10, from Salmon, Moraes, Dror, Shaw, "Parallel Random     */
/* Numbers: As Easy as 1, 2, 3" (SC'11): ten rounds, each two 64x64->128     */
/* products of counter words with the round multipliers, the high halves     */
/* xored with the round key and the other words, then a word permutation;   */
/* the key advances by the Weyl constants between rounds.                    */
/* The pages name no generator; the reading is: key = (seed, 0),             */
/* counter = (step, row, stream, 0), u = (r >> 11) * 2^-53.                   */
/* ------------------------------------------------------------------------ */
EXPORT void oracle_philox4x64_10(const uint64_t key[2], const uint64_t ctr[4], uint64_t out[4]) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
    uint64_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint64_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += W0; k1 += W1; }
        unsigned __int128 p0 = (unsigned __int128)M0 * c0;
        unsigned __int128 p1 = (unsigned __int128)M1 * c2;
        uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
        uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
        uint64_t n0 = hi1 ^ c1 ^ k0;
        uint64_t n1 = lo1;
        uint64_t n2 = hi0 ^ c3 ^ k1;
        uint64_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static double u53(uint64_t r) { return (double)(r >> 11) * ldexp(1.0, -53); }

/* Uniforms of one verify problem: u_acc[i] = first word, u_res[i] = second
 * word of the block at counter (step, i, 0, 0), for rows i = 0..D. */
EXPORT void oracle_verify_uniforms(uint64_t seed, uint64_t step, int32_t D,
                                   double* u_acc, double* u_res) {
    const uint64_t key[2] = {seed, 0};
    for (int32_t i = 0; i <= D; ++i) {
        uint64_t ctr[4] = {step, (uint64_t)i, 0, 0}, out[4];
        oracle_philox4x64_10(key, ctr, out);
        u_acc[i] = u53(out[0]);
        u_res[i] = u53(out[1]);
    }
}

/* ------------------------------------------------------------------------ */
/* (a6/a7) Leviathan–Chen acceptance with residual resampling and a bonus    */
/* token ([mtplx/4層] Layer 2; [MTPLX/裏技]; [mtplx/数字]).                    */
/* For i < D in order: accept draft x_i iff u_acc[i] * q_i(x_i) < p_i(x_i)    */
/* (the ratio test min(1, p/q) written without a division).  At the first     */
/* rejection k, sample from r = max(0, p_k - q_k) / sum(r); if all D drafts   */
/* are accepted, sample the bonus token from p_D.  Sampling is the inverse    */
/* CDF in vocabulary-index order: y = min{ j : C_j > u_res[k] * R }.         */
/* Readings: q is used as given (fp32, not renormalised); R <= 0 falls back  */
/* to p_k (flag bit4); flags: bit2 accept test with |u - p/q| < 1e-5;         */
/* bit3 CDF boundary within 1e-9 * R; bit0 non-finite logits; bit1 a row's   */
/* top-p boundary was flagged.                                               */
/* ------------------------------------------------------------------------ */
static double p_of(const float* z, const oracle_warp_t* st, float temperature, int64_t x) {
    const double T = (double)temperature;
    if (T == 0.0) return (x == st->argmax) ? 1.0 : 0.0;
    if ((double)z[x] < st->tau) return 0.0;
    return exp(((double)z[x] - st->m) / T) / st->Z;
}

EXPORT void oracle_accept_with_uniforms(const float* z /* [D+1][V] */,
                                        const oracle_warp_t* st /* [D+1] */,
                                        const float* q /* [D][V] */,
                                        const int32_t* draft /* [D] */,
                                        int32_t D, int64_t V, float temperature,
                                        const double* u_acc, const double* u_res,
                                        int32_t* tokens /* [D+1] */, int32_t* n_acc,
                                        uint32_t* flags) {
    uint32_t f = 0;
    for (int32_t i = 0; i <= D; ++i) {
        if (st[i].flags & 1u) {
            for (int32_t t = 0; t <= D; ++t) tokens[t] = -1;
            *n_acc = -1;
            *flags = 1u;
            return;
        }
        if (st[i].flags & 2u) f |= 2u;
    }
    int32_t k = D;
    for (int32_t i = 0; i < D; ++i) {
        int64_t x = draft[i];
        double pi = p_of(z + (int64_t)i * V, &st[i], temperature, x);
        double qi = (double)q[(int64_t)i * V + x];
        if (qi > 0.0 && fabs(u_acc[i] - pi / qi) < 1e-5) f |= 4u;
        if (u_acc[i] * qi < pi) { tokens[i] = draft[i]; continue; }
        k = i;
        break;
    }
    const float* zk = z + (int64_t)k * V;
    double* r = (double*)malloc((size_t)V * sizeof(double));
    double rs = 0.0, rc = 0.0;
    for (int64_t j = 0; j < V; ++j) {
        double pj = p_of(zk, &st[k], temperature, j);
        double v = pj;
        if (k < D) {
            double d = pj - (double)q[(int64_t)k * V + j];
            v = d > 0.0 ? d : 0.0;
        }
        r[j] = v;
        kahan_add(&rs, &rc, v);
    }
    double R = rs + rc;
    if (!(R > 0.0)) {
        f |= 16u;
        rs = 0.0; rc = 0.0;
        for (int64_t j = 0; j < V; ++j) { r[j] = p_of(zk, &st[k], temperature, j); kahan_add(&rs, &rc, r[j]); }
        R = rs + rc;
    }
    const double target = u_res[k] * R;
    double cs = 0.0, cc = 0.0, prev = 0.0, cy = 0.0;
    int64_t y = -1, last_pos = -1;
    for (int64_t j = 0; j < V; ++j) {
        if (r[j] > 0.0) last_pos = j;
        prev = cs + cc;
        kahan_add(&cs, &cc, r[j]);
        if (cs + cc > target) { y = j; cy = cs + cc; break; }
    }
    if (y < 0) { y = last_pos; f |= 8u; }   /* u*R rounded up to R: boundary case */
    else if (fabs(target - prev) < 1e-9 * R || fabs(target - cy) < 1e-9 * R) f |= 8u;
    free(r);
    tokens[k] = (int32_t)y;
    for (int32_t t = k + 1; t <= D; ++t) tokens[t] = -1;
    *n_acc = k;
    *flags = f;
}

/* One verify problem end to end from logits: warp every row, draw the
 * uniforms from Philox, run the accept/resample loop. */
EXPORT void oracle_spec_accept(const float* z, const float* q, const int32_t* draft,
                               int32_t D, int64_t V, float temperature, float top_p,
                               uint64_t seed, uint64_t step, oracle_warp_t* st /* [D+1] */,
                               int32_t* tokens, int32_t* n_acc, uint32_t* flags) {
    for (int32_t i = 0; i <= D; ++i) oracle_warp(z + (int64_t)i * V, V, temperature, top_p, &st[i], NULL);
    double u_acc[64], u_res[64];
    oracle_verify_uniforms(seed, step, D, u_acc, u_res);
    oracle_accept_with_uniforms(z, st, q, draft, D, V, temperature, u_acc, u_res, tokens, n_acc, flags);
}

/* Many problems sharing one set of logits, stats and q (the tiny-vocabulary
 * distribution trials); problem b uses step0 + b and its own drafts. */
EXPORT void oracle_spec_accept_trials(const float* z, const float* q, const int32_t* drafts /* [B][D] */,
                                      int64_t B, int32_t D, int64_t V, float temperature, float top_p,
                                      uint64_t seed, uint64_t step0,
                                      int32_t* tokens /* [B][D+1] */, int32_t* n_acc, uint32_t* flags) {
    oracle_warp_t st[64];
    for (int32_t i = 0; i <= D; ++i) oracle_warp(z + (int64_t)i * V, V, temperature, top_p, &st[i], NULL);
    #pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        double u_acc[64], u_res[64];
        oracle_verify_uniforms(seed, step0 + (uint64_t)b, D, u_acc, u_res);
        oracle_accept_with_uniforms(z, st, q, drafts + b * D, D, V, temperature, u_acc, u_res,
                                    tokens + b * (D + 1), n_acc + b, flags + b);
    }
}

/* ------------------------------------------------------------------------ */
/* (a8) Decoder-layer glue, bf16 storage and binary32 rounding points are    */
/* NOT modelled here: each function returns the exact fp64 value of the      */
/* operation on its (bf16) inputs; the caller compares with a tolerance.     */
/* RMSNorm: y = x / sqrt(mean(x^2) + eps) * gamma.                            */
/* ------------------------------------------------------------------------ */
EXPORT void oracle_rmsnorm(const uint16_t* x_bf16, const uint16_t* gamma_bf16, int64_t M, int64_t D,
                           double eps, double* y) {
    for (int64_t m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int64_t d = 0; d < D; ++d) { double v = bf16_value(x_bf16[m * D + d]); ss += v * v; }
        double inv = 1.0 / sqrt(ss / (double)D + eps);
        for (int64_t d = 0; d < D; ++d)
            y[m * D + d] = bf16_value(x_bf16[m * D + d]) * inv * bf16_value(gamma_bf16[d]);
    }
}

/* SwiGLU: silu(g) * u with silu(g) = g / (1 + exp(-g)). */
static double swiglu1(double g, double u) { return g / (1.0 + exp(-g)) * u; }

EXPORT void oracle_swiglu(const uint16_t* g_bf16, const uint16_t* u_bf16, int64_t n, double* y) {
    for (int64_t i = 0; i < n; ++i) y[i] = swiglu1(bf16_value(g_bf16[i]), bf16_value(u_bf16[i]));
}

/* The same on unrounded gate/up values (a GEMM's fp64 output handed on
 * without an intermediate bf16 store). */
EXPORT void oracle_swiglu_f64(const double* g, const double* u, int64_t n, double* y) {
    for (int64_t i = 0; i < n; ++i) y[i] = swiglu1(g[i], u[i]);
}

/* Rotary embedding, rotate-half convention (RoFormer), base theta:
 * for d < H/2, angle = pos * theta^(-2d/H);
 * out[d] = x[d] cos - x[d+H/2] sin, out[d+H/2] = x[d+H/2] cos + x[d] sin. */
EXPORT void oracle_rope(const double* x, int64_t H, int64_t pos, double theta, double* out) {
    int64_t h2 = H / 2;
    for (int64_t d = 0; d < h2; ++d) {
        double ang = (double)pos * pow(theta, -2.0 * (double)d / (double)H);
        double c = cos(ang), s = sin(ang);
        double a = x[d], b = x[d + h2];
        out[d] = a * c - b * s;
        out[d + h2] = b * c + a * s;
    }
}

/* (a9) GQA decode attention for M query rows over a bf16 KV cache.
 * q: fp64 [M][Hq][Dh] (already rotated); K, V: bf16 [Hkv][Lc][Dh], where
 * Lc >= L + M and positions L..L+M-1 hold the rows' own keys/values.
 * Row i attends positions 0..L+i; head h reads kv head h / (Hq/Hkv).
 * out: fp64 [M][Hq][Dh]. */
EXPORT void oracle_decode_attn(const double* q, const uint16_t* Kc, const uint16_t* Vc,
                               int64_t M, int64_t Hq, int64_t Hkv, int64_t Dh, int64_t L, int64_t Lc,
                               double* out) {
    const int64_t grp = Hq / Hkv;
    const double scale = 1.0 / sqrt((double)Dh);
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t h = 0; h < Hq; ++h) {
            const int64_t kh = h / grp;
            const int64_t n = L + i + 1;
            double* s = (double*)malloc((size_t)n * sizeof(double));
            double mx = -INFINITY;
            for (int64_t j = 0; j < n; ++j) {
                double dot = 0.0;
                for (int64_t d = 0; d < Dh; ++d)
                    dot += q[(i * Hq + h) * Dh + d] * bf16_value(Kc[(kh * Lc + j) * Dh + d]);
                s[j] = dot * scale;
                if (s[j] > mx) mx = s[j];
            }
            double den = 0.0;
            for (int64_t j = 0; j < n; ++j) { s[j] = exp(s[j] - mx); den += s[j]; }
            for (int64_t d = 0; d < Dh; ++d) {
                double acc = 0.0;
                for (int64_t j = 0; j < n; ++j) acc += s[j] * bf16_value(Vc[(kh * Lc + j) * Dh + d]);
                out[(i * Hq + h) * Dh + d] = acc / den;
            }
            free(s);
        }
    }
}

/* (a10) MoE router: softmax over E router logits, top-k by probability with
 * ties to the lower expert index, weights renormalised to sum to one.
 * Reading: no shared expert; the router logits are given. */
EXPORT void oracle_moe_route(const float* logits, int64_t M, int64_t E, int64_t topk,
                             int32_t* experts /* [M][topk] */, double* weights /* [M][topk] */) {
    for (int64_t m = 0; m < M; ++m) {
        const float* l = logits + m * E;
        double mx = -INFINITY;
        for (int64_t e = 0; e < E; ++e) if ((double)l[e] > mx) mx = (double)l[e];
        double* pr = (double*)malloc((size_t)E * sizeof(double));
        double den = 0.0;
        for (int64_t e = 0; e < E; ++e) { pr[e] = exp((double)l[e] - mx); den += pr[e]; }
        for (int64_t e = 0; e < E; ++e) pr[e] /= den;
        char* used = (char*)calloc((size_t)E, 1);
        double tot = 0.0;
        for (int64_t t = 0; t < topk; ++t) {
            /* highest probability == highest logit (softmax is increasing);
             * the fp32 logits decide, ties go to the lower index */
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e)
                if (!used[e] && (best < 0 || l[e] > l[best])) best = e;
            used[best] = 1;
            experts[m * topk + t] = (int32_t)best;
            weights[m * topk + t] = pr[best];
            tot += pr[best];
        }
        for (int64_t t = 0; t < topk; ++t) weights[m * topk + t] /= tot;
        free(pr);
        free(used);
    }
}

/* ------------------------------------------------------------------------ */
/* The draft side of the cycle.  [mtplx/4層] Layer 1: the drafter is the MTP   */
/* head inside the same checkpoint; Layer 0: it has a 4-bit LM head of its    */
/* own; Layer 2: each cycle drafts, then verifies.  The pages do not describe */
/* the head's inside.  Reading (the common MTP head): the hidden row h of the */
/* last processed position and the embedding e of the next token are each    */
/* RMS-normalised with a gain of their own, concatenated [h ; e], projected   */
/* back to d by a W4 matrix, passed through one decoder layer, the final norm */
/* and the (shared, W4) LM head; D drafts apply the head D times, each time   */
/* feeding its own output row and the token it just drew.                     */
/* ------------------------------------------------------------------------ */

/* Projection input of one draft: [rmsnorm(h) * gamma_h ; rmsnorm(e) * gamma_e],
 * the exact fp64 values (the caller rounds to bfloat16). */
EXPORT void oracle_mtp_input(const uint16_t* h_bf16, const uint16_t* e_bf16, const uint16_t* gamma_h,
                             const uint16_t* gamma_e, int64_t d, double eps, double* out /* [2d] */) {
    oracle_rmsnorm(h_bf16, gamma_h, 1, d, eps, out);
    oracle_rmsnorm(e_bf16, gamma_e, 1, d, eps, out + d);
}

/* Token embedding rows: out[i] = E[tokens[i]]; an id outside [0, V) gives a
 * row of zeros. */
EXPORT void oracle_embed_rows(const uint16_t* E, int64_t V, int64_t d, const int32_t* tokens, int64_t n,
                              uint16_t* out /* [n][d] */) {
    for (int64_t i = 0; i < n; ++i) {
        const int64_t t = tokens[i];
        if (t >= 0 && t < V) memcpy(out + i * d, E + t * d, (size_t)d * sizeof(uint16_t));
        else memset(out + i * d, 0, (size_t)d * sizeof(uint16_t));
    }
}

/* Uniform of draft depth `depth` in cycle `step`: Philox4x64-10 with key
 * (seed, 0) and counter (step, depth, 1, 0) -- the third word 1 keeps the
 * draft stream apart from the verify's, whose third word is 0 -- second
 * output word, 53 bits. */
EXPORT double oracle_draft_uniform(uint64_t seed, uint64_t step, int32_t depth) {
    const uint64_t key[2] = {seed, 0};
    uint64_t ctr[4] = {step, (uint64_t)depth, 1, 0}, out[4];
    oracle_philox4x64_10(key, ctr, out);
    return u53(out[1]);
}

/* One draft: q = the warped distribution of the draft logits z (the same
 * temperature / top-p reading as a verify row), written as binary32 for the
 * verify's ratio test; the token is drawn from that distribution (fp64, index
 * order, the inverse CDF of the acceptance step's sampler) at the draft
 * uniform.  Reading: the drafter samples with the target's temperature and
 * top-p. */
EXPORT void oracle_draft_sample(const float* z, int64_t V, float temperature, float top_p, uint64_t seed,
                                uint64_t step, int32_t depth, float* q_out /* nullable, [V] */,
                                oracle_warp_t* st, int32_t* token, uint32_t* flags) {
    double* p = (double*)calloc((size_t)V, sizeof(double));
    oracle_warp(z, V, temperature, top_p, st, p);
    if (q_out) for (int64_t j = 0; j < V; ++j) q_out[j] = (float)p[j];
    const double u_acc = 0.0, u_res = oracle_draft_uniform(seed, step, depth);
    int32_t n_acc;
    oracle_accept_with_uniforms(z, st, NULL, NULL, 0, V, temperature, &u_acc, &u_res, token, &n_acc, flags);
    free(p);
}

/* ------------------------------------------------------------------------ */
/* A second weight format for the skinny GEMM: W8.  [BaseRT/方法] lists the    */
/* quantisation formats the engine's GEMV reads (Q2 ... Q8) and names Q8; the */
/* pages give no layout.  Reading: the W4 recipe with 8-bit codes -- codes in */
/* [-127, 127]; scale = fp16(absmax / 127) rounded to nearest-even; codes use */
/* the rounded scale, rounded half to even and clamped; an all-zero group     */
/* gets scale 0 and codes 0.  Canonical storage: u8 codes[N][K] holding       */
/* u = c + 128; f16 scales[N][K/64].                                           */
/* ------------------------------------------------------------------------ */
EXPORT void oracle_w8_quantize(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales) {
    const int64_t G = K / 64;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float* wg = w + n * K + g * 64;
            float a = 0.0f;
            for (int k = 0; k < 64; ++k) {
                float v = fabsf(wg[k]);
                if (v > a) a = v;
            }
            uint16_t s16 = oracle_f32_to_f16(a / 127.0f);   /* binary32 division */
            float sf = (float)f16_value(s16);
            scales[n * G + g] = s16;
            for (int k = 0; k < 64; ++k) {
                int c = 0;
                if (sf != 0.0f) {
                    float r = rintf(wg[k] / sf);            /* binary32 division, half-even */
                    if (r > 127.0f) r = 127.0f;
                    if (r < -127.0f) r = -127.0f;
                    c = (int)r;
                }
                codes[n * K + g * 64 + k] = (uint8_t)(c + 128);
            }
        }
    }
}

/* y[m][n] = sum_k x[m][k] * c[n][k] * s[n][k/64], fp64, sequential in k. */
EXPORT void oracle_w8_gemm(const uint16_t* x_bf16, int64_t M, int64_t K, const uint8_t* codes,
                           const uint16_t* scales, int64_t N, double* y /* [M][N] */) {
    const int64_t G = K / 64;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += bf16_value(x_bf16[m * K + k]) * (double)((int)codes[n * K + k] - 128) *
                       f16_value(scales[n * G + k / 64]);
            y[m * N + n] = acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* A fourth weight format: W5 (the same BaseRT section lists Q2 ... Q8 among  */
/* the GEMV's formats; no layout).  Reading: the W4 recipe with 5-bit codes -- */
/* codes in [-15, 15]; scale = fp16(absmax / 15) rounded to nearest-even;     */
/* codes use the rounded scale, half-even, clamped; an all-zero group gets    */
/* scale 0 and codes 0.  Canonical storage: u8 codes[N][K] holding u = c + 16; */
/* f16 scales[N][K/64].                                                       */
/* ------------------------------------------------------------------------ */
EXPORT void oracle_w5_quantize(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales) {
    const int64_t G = K / 64;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float* wg = w + n * K + g * 64;
            float a = 0.0f;
            for (int k = 0; k < 64; ++k) {
                float v = fabsf(wg[k]);
                if (v > a) a = v;
            }
            uint16_t s16 = oracle_f32_to_f16(a / 15.0f);    /* binary32 division */
            float sf = (float)f16_value(s16);
            scales[n * G + g] = s16;
            for (int k = 0; k < 64; ++k) {
                int c = 0;
                if (sf != 0.0f) {
                    float r = rintf(wg[k] / sf);            /* binary32 division, half-even */
                    if (r > 15.0f) r = 15.0f;
                    if (r < -15.0f) r = -15.0f;
                    c = (int)r;
                }
                codes[n * K + g * 64 + k] = (uint8_t)(c + 16);
            }
        }
    }
}

/* y[m][n] = sum_k x[m][k] * c[n][k] * s[n][k/64], fp64, sequential in k. */
EXPORT void oracle_w5_gemm(const uint16_t* x_bf16, int64_t M, int64_t K, const uint8_t* codes,
                           const uint16_t* scales, int64_t N, double* y /* [M][N] */) {
    const int64_t G = K / 64;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += bf16_value(x_bf16[m * K + k]) * (double)((int)codes[n * K + k] - 16) *
                       f16_value(scales[n * G + k / 64]);
            y[m * N + n] = acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* The widest format of the same BaseRT list (Q2 ... FP16): unquantised fp16  */
/* weights, w[N][K] as IEEE binary16 bit patterns, no scales; and the same    */
/* with bf16 weights (the 16-bit float type of bf16 checkpoints).             */
/* y[m][n] = sum_k x[m][k] * w[n][k], fp64, sequential in k.                  */
/* ------------------------------------------------------------------------ */
EXPORT void oracle_f16_gemm(const uint16_t* x_bf16, int64_t M, int64_t K, const uint16_t* w_f16, int64_t N,
                            double* y /* [M][N] */) {
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += bf16_value(x_bf16[m * K + k]) * f16_value(w_f16[n * K + k]);
            y[m * N + n] = acc;
        }
    }
}

EXPORT void oracle_b16_gemm(const uint16_t* x_bf16, int64_t M, int64_t K, const uint16_t* w_bf16, int64_t N,
                            double* y /* [M][N] */) {
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += bf16_value(x_bf16[m * K + k]) * bf16_value(w_bf16[n * K + k]);
            y[m * N + n] = acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Two narrower weight formats: W3 and W2 (the same BaseRT section lists Q2   */
/* ... Q8 among the GEMV's formats; no layout).  Reading: the W4 recipe with  */
/* b-bit codes in [-(2^(b-1) - 1), 2^(b-1) - 1] -- W3: [-3, 3], scale =       */
/* fp16(absmax / 3); W2: [-1, 1], scale = fp16(absmax / 1) -- codes against   */
/* the rounded scale, half-even, clamped; an all-zero group gets scale 0 and  */
/* codes 0.  Canonical storage: u8 codes[N][K] holding u = c + 2^(b-1)        */
/* (W3: c + 4, W2: c + 1); f16 scales[N][K/64].                               */
/* ------------------------------------------------------------------------ */
EXPORT void oracle_w3_quantize(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales) {
    const int64_t G = K / 64;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float* wg = w + n * K + g * 64;
            float a = 0.0f;
            for (int k = 0; k < 64; ++k) {
                float v = fabsf(wg[k]);
                if (v > a) a = v;
            }
            uint16_t s16 = oracle_f32_to_f16(a / 3.0f);     /* binary32 division */
            float sf = (float)f16_value(s16);
            scales[n * G + g] = s16;
            for (int k = 0; k < 64; ++k) {
                int c = 0;
                if (sf != 0.0f) {
                    float r = rintf(wg[k] / sf);            /* binary32 division, half-even */
                    if (r > 3.0f) r = 3.0f;
                    if (r < -3.0f) r = -3.0f;
                    c = (int)r;
                }
                codes[n * K + g * 64 + k] = (uint8_t)(c + 4);
            }
        }
    }
}

EXPORT void oracle_w2_quantize(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales) {
    const int64_t G = K / 64;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float* wg = w + n * K + g * 64;
            float a = 0.0f;
            for (int k = 0; k < 64; ++k) {
                float v = fabsf(wg[k]);
                if (v > a) a = v;
            }
            uint16_t s16 = oracle_f32_to_f16(a);            /* absmax / 1 */
            float sf = (float)f16_value(s16);
            scales[n * G + g] = s16;
            for (int k = 0; k < 64; ++k) {
                int c = 0;
                if (sf != 0.0f) {
                    float r = rintf(wg[k] / sf);            /* binary32 division, half-even */
                    if (r > 1.0f) r = 1.0f;
                    if (r < -1.0f) r = -1.0f;
                    c = (int)r;
                }
                codes[n * K + g * 64 + k] = (uint8_t)(c + 1);
            }
        }
    }
}

/* y[m][n] = sum_k x[m][k] * (u[n][k] - bias) * s[n][k/64], fp64, sequential in k
 * (bias 4 for W3 codes, 1 for W2 codes). */
static void w_small_gemm(const uint16_t* x_bf16, int64_t M, int64_t K, const uint8_t* codes, int bias,
                         const uint16_t* scales, int64_t N, double* y) {
    const int64_t G = K / 64;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += bf16_value(x_bf16[m * K + k]) * (double)((int)codes[n * K + k] - bias) *
                       f16_value(scales[n * G + k / 64]);
            y[m * N + n] = acc;
        }
    }
}

EXPORT void oracle_w3_gemm(const uint16_t* x_bf16, int64_t M, int64_t K, const uint8_t* codes,
                           const uint16_t* scales, int64_t N, double* y /* [M][N] */) {
    w_small_gemm(x_bf16, M, K, codes, 4, scales, N, y);
}

EXPORT void oracle_w2_gemm(const uint16_t* x_bf16, int64_t M, int64_t K, const uint8_t* codes,
                           const uint16_t* scales, int64_t N, double* y /* [M][N] */) {
    w_small_gemm(x_bf16, M, K, codes, 1, scales, N, y);
}

/* ------------------------------------------------------------------------ */
/* A third weight format: W6 ([BaseRT/方法] lists Q2 ... Q8; no layout).       */
/* Reading: the W4 recipe with 6-bit codes -- codes in [-31, 31]; scale =     */
/* fp16(absmax / 31) rounded to nearest-even; codes use the rounded scale,    */
/* half-even, clamped; an all-zero group gets scale 0 and codes 0.  Canonical */
/* storage: u8 codes[N][K] holding u = c + 32; f16 scales[N][K/64].           */
/* ------------------------------------------------------------------------ */
EXPORT void oracle_w6_quantize(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales) {
    const int64_t G = K / 64;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float* wg = w + n * K + g * 64;
            float a = 0.0f;
            for (int k = 0; k < 64; ++k) {
                float v = fabsf(wg[k]);
                if (v > a) a = v;
            }
            uint16_t s16 = oracle_f32_to_f16(a / 31.0f);    /* binary32 division */
            float sf = (float)f16_value(s16);
            scales[n * G + g] = s16;
            for (int k = 0; k < 64; ++k) {
                int c = 0;
                if (sf != 0.0f) {
                    float r = rintf(wg[k] / sf);            /* binary32 division, half-even */
                    if (r > 31.0f) r = 31.0f;
                    if (r < -31.0f) r = -31.0f;
                    c = (int)r;
                }
                codes[n * K + g * 64 + k] = (uint8_t)(c + 32);
            }
        }
    }
}

/* y[m][n] = sum_k x[m][k] * c[n][k] * s[n][k/64], fp64, sequential in k. */
EXPORT void oracle_w6_gemm(const uint16_t* x_bf16, int64_t M, int64_t K, const uint8_t* codes,
                           const uint16_t* scales, int64_t N, double* y /* [M][N] */) {
    const int64_t G = K / 64;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += bf16_value(x_bf16[m * K + k]) * (double)((int)codes[n * K + k] - 32) *
                       f16_value(scales[n * G + k / 64]);
            y[m * N + n] = acc;
        }
    }
}
