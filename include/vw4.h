/*
 * vw4.h — C ABI of the batched-verify library for MI355X (gfx950).
 *
 * The library implements the verify half of multi-token-prediction
 * self-speculative decoding: the main model scores all M = D+1 rows (D drafts
 * plus the bonus position) in one pass, then the drafts are accepted or
 * corrected so that the emitted tokens follow the target distribution exactly.
 *   - hazakura.dev, "mtplx——M5 Maxで63tok/s、Apple SiliconのローカルLLMが2倍以上速くなる日",
 *     section "4層のアーキテクチャ": Layer 0 names the small-M (M = 3..6) matmul
 *     and the 4-bit LM head; Layer 2 names the cycle draft -> one parallel
 *     verify -> probability-ratio acceptance -> residual correction -> bonus token.
 *   - devtrends.cc, "Apple Silicon上でローカルLLMを最大2倍高速化するMTPLX",
 *     section "2つ目のモデル不要！MTPの裏技": the whole batch of drafts is verified
 *     in a single forward pass with Leviathan–Chen rejection sampling and
 *     residual correction; at temperature 0.6 / top_p 0.95 the output law is that
 *     of plain step-by-step sampling.
 *   - gist.science, "BaseRT: Best-in-Class LLM Inference on Apple Silicon via
 *     Native Metal", section "メソドロジー": dequantisation inside the GEMV inner
 *     loop; all decode buffers preallocated by the caller (zero allocation in the
 *     decode loop); FlashAttention-style online softmax.
 *
 * Conventions for every entry point:
 *   - Pointers named *_dev, and every array argument of a compute call, are
 *     device memory owned by the caller.  The library allocates nothing and
 *     keeps no pointer after returning.  Scratch memory comes from a caller
 *     workspace sized by the matching *_workspace_bytes() query (its contents
 *     need no initialisation and are dead after the call's kernels finish).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *     only enqueue work; results are valid once the stream reaches that point.
 *     Calls that share a workspace must not run concurrently.
 *   - Return codes: VW4_OK, or a negative error detected on the host before
 *     anything is enqueued (nothing is written in that case).  vw4_last_error()
 *     returns a thread-local message for the last failure.  Data-dependent
 *     conditions (non-finite logits, near-ties) are not errors: they set flag
 *     bits in the outputs.
 */
#ifndef VW4_H
#define VW4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported symbols (the library is built with hidden default visibility). */
#define VW4_API __attribute__((visibility("default")))

#define VW4_OK 0
#define VW4_EINVAL (-1)       /* bad shape, alignment or parameter */
#define VW4_EUNSUPPORTED (-2) /* valid request the library does not handle */
#define VW4_EHIP (-3)         /* HIP runtime or launch failure */
#define VW4_EWORKSPACE (-4)   /* workspace missing or too small */

/* Output dtypes of the GEMM. */
#define VW4_F32 0
#define VW4_BF16 1

/* Row flags (vw4_rowstat.flags) and problem flags (spec_accept out_flags). */
#define VW4_FLAG_NONFINITE 1u   /* a logit was NaN or infinite */
#define VW4_FLAG_TOPP_TIE 2u    /* top-p boundary mass within 1e-9 * E of top_p * E */
#define VW4_FLAG_ACCEPT_TIE 4u  /* an accept test had |u - p/q| < 1e-5 */
#define VW4_FLAG_CDF_TIE 8u     /* the sampled token's CDF boundary within 1e-9 * R of u * R */
#define VW4_FLAG_R_ZERO 16u     /* residual mass was zero; sampled from p instead */

/* Per-row statistics of the tempered, top-p-truncated target distribution.
 * For T > 0 the target is p_j = exp((z_j - max_logit)/T) / exp(log_z) for
 * z_j >= tau, else 0.  For T == 0 it is one-hot at argmax (tau = max_logit,
 * log_z = 0, n_kept = 1). */
typedef struct vw4_rowstat {
    float max_logit;   /* m = max_j z_j */
    float tau;         /* cutoff logit: the kept set is { j : z_j >= tau } */
    double log_z;      /* log of sum over the kept set of exp((z_j - m)/T) */
    int32_t argmax;    /* lowest index attaining the max */
    int32_t n_kept;    /* size of the kept set */
    uint32_t flags;    /* VW4_FLAG_NONFINITE | VW4_FLAG_TOPP_TIE */
    uint32_t pad;
} vw4_rowstat;

/* Library version string and the calling thread's last error message. */
VW4_API const char* vw4_version(void);
VW4_API const char* vw4_last_error(void);

/* ------------------------------------------------------------------------
 * W4 weight format (offline), for the 4-bit weights named on
 * hazakura.dev's mtplx page (section "4層のアーキテクチャ", Layer 0): symmetric
 * int4 codes c in [-7, 7], one fp16 scale per 64 consecutive elements along K,
 * scale = fp16_rne(absmax / 7), c = clamp(rint_half_even(w / scale), -7, 7)
 * with the rounded scale, all-zero groups get scale 0.
 *
 * Canonical layout: codes u8 [N][K/2] holding c + 8, even k in the low nibble;
 * scales f16 [N][K/64].  Kernel ("packed") layout, produced by vw4_w4_pack:
 * rows padded to a multiple of 64 and stored tile-major so that one wavefront
 * streams 64 rows with fully coalesced 16-byte loads; sizes from
 * vw4_w4_packed_bytes.  Requirements: K % 64 == 0, N >= 1, finite weights.
 * ------------------------------------------------------------------------ */

/* Quantise fp32 host weights w[N][K] into host canonical codes and scales. */
VW4_API int vw4_w4_quantize_host(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales);

/* Same arithmetic on the GPU: device w_dev[N][K] -> device canonical arrays. */
VW4_API int vw4_w4_quantize(const float* w_dev, int64_t N, int64_t K, uint8_t* codes_dev,
                    uint16_t* scales_dev, void* stream);

/* Bytes of the packed code array; *scale_bytes (if not NULL) receives the
 * bytes of the packed scale array.  Returns 0 for invalid shapes. */
VW4_API size_t vw4_w4_packed_bytes(int64_t N, int64_t K, size_t* scale_bytes);

/* Canonical (device) -> packed (device). */
VW4_API int vw4_w4_pack(const uint8_t* codes_dev, const uint16_t* scales_dev, int64_t N, int64_t K,
                uint8_t* packed_dev, uint16_t* packed_scales_dev, void* stream);

/* Packed (device) -> canonical (device); the inverse of vw4_w4_pack. */
VW4_API int vw4_w4_unpack(const uint8_t* packed_dev, const uint16_t* packed_scales_dev, int64_t N, int64_t K,
                  uint8_t* codes_dev, uint16_t* scales_dev, void* stream);

/* Quantise device fp32 weights straight into the packed layout (equals
 * vw4_w4_quantize followed by vw4_w4_pack, without the canonical copy). */
VW4_API int vw4_w4_quantize_packed(const float* w_dev, int64_t N, int64_t K, uint8_t* packed_dev,
                           uint16_t* packed_scales_dev, void* stream);

/* ------------------------------------------------------------------------
 * W4 skinny GEMM (hazakura.dev mtplx page, "4層のアーキテクチャ" Layer 0: the
 * small-M matmul of the verify pass; gist.science BaseRT summary, "メソドロジー":
 * dequantisation in the inner loop, weights never materialised).
 *   y[m][n] = sum_k x[m][k] * c[n][k] * scale[n][k/64]      0 <= m < M, 0 <= n < N
 * x: bf16 [M][ldx] (row stride ldx elements, ldx >= K, ldx % 8 == 0, 16-byte
 * aligned); w: packed codes/scales of an [N][K] matrix; y: fp32 or bf16 (RNE)
 * [M][ldy] with ldy >= N.  1 <= M <= 8, K % 64 == 0, K <= 65536.
 * Accumulation is fp32 in a fixed order that does not depend on M, so row m of
 * an M-row call equals the single-row call on x[m] bit for bit, and repeated
 * calls are bitwise reproducible.  ws may be NULL when
 * vw4_gemm_workspace_bytes() returns 0 for the shape.
 * ------------------------------------------------------------------------ */
VW4_API size_t vw4_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K);

VW4_API int w4_skinny_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, const uint16_t* scales_packed,
                   void* y, int64_t ldy, int32_t y_dtype, int32_t M, int32_t N, int32_t K,
                   void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * w4_skinny_gemm without a workspace, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, kernels and results as w4_skinny_gemm (bit for
 * bit); the split-K partial sums go to a static device array of
 * VW4_NOALLOC_SCRATCH_BYTES (8 MiB) that each GPU the library runs on holds
 * until the process ends.  The call allocates nothing (no hipMalloc, no
 * library allocator).  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (different streams, or host threads) race and give
 * undefined results; serialise them.  Nothing in the array needs to start at
 * zero.  Returns VW4_EWORKSPACE if a shape's partials exceed the array (no
 * shape with M <= 8 does), VW4_EHIP if the array's device address cannot be
 * obtained, else as w4_skinny_gemm.
 * ------------------------------------------------------------------------ */
#define VW4_NOALLOC_SCRATCH_BYTES (8u << 20)
VW4_API size_t vw4_noalloc_scratch_bytes(void);
VW4_API int w4_skinny_gemm_noalloc(const uint16_t* x, int64_t ldx, const uint8_t* w_packed,
                                   const uint16_t* scales_packed, void* y, int64_t ldy, int32_t y_dtype, int32_t M,
                                   int32_t N, int32_t K, void* stream);

/* ------------------------------------------------------------------------
 * verify_logits: LM head of the verify rows, then the temperature / top-p
 * statistics of every row (devtrends.cc MTPLX page, section
 * "2つ目のモデル不要！MTPの裏技": sampling at temperature 0.6, top_p 0.95).
 *   hidden (nullable): bf16 [rows][ldh]; lm_packed/lm_scales: packed W4 [V][d].
 *   If hidden != NULL: logits[rows][V] = w4 GEMM(hidden) (fp32), then stats.
 *   If hidden == NULL: logits is an INPUT and only the statistics are computed.
 * Statistics (one vw4_rowstat per row): m = max; for T > 0, e_j = exp((z_j - m)/T)
 * in fp64, E = sum e_j; the kept set is the smallest prefix of the vocabulary
 * sorted by (logit desc, index asc) whose mass reaches top_p * E, widened to
 * all tokens whose logit equals the cutoff tau; top_p >= 1 keeps all; T == 0
 * is greedy.  Requires 1 <= rows <= 64, 1 <= V <= 2^24, d % 64 == 0,
 * T >= 0 (finite), 0 < top_p <= 1.  Workspace: vw4_workspace_bytes(rows, V).
 * ------------------------------------------------------------------------ */
VW4_API size_t vw4_workspace_bytes(int32_t rows, int32_t V);

VW4_API int verify_logits(const uint16_t* hidden, int64_t ldh, const uint8_t* lm_packed, const uint16_t* lm_scales,
                  int32_t rows, int32_t V, int32_t d, float temperature, float top_p, float* logits,
                  vw4_rowstat* stats, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * spec_accept: Leviathan–Chen acceptance, residual resampling and bonus token
 * for B independent verify problems of M = D+1 rows each (hazakura.dev mtplx
 * page, "4層のアーキテクチャ" Layer 2 and "mtplxの数字——本当なの？"; devtrends.cc
 * MTPLX page, "2つ目のモデル不要！MTPの裏技").
 * Problem b reads logits + b*logits_bstride ([M][V] fp32), stats + b*stats_bstride
 * ([M] rowstats from verify_logits with the same temperature), q + b*q_bstride
 * ([D][V] fp32 draft distributions, used as given) and draft + b*D ([D] int32);
 * a stride of 0 shares one array between all problems.  With key (seed, 0) and
 * counter (step0 + b, i, 0, 0), Philox4x64-10 (Salmon et al., SC'11) gives the
 * row-i uniforms u_acc = (r0 >> 11) 2^-53 and u_res = (r1 >> 11) 2^-53.
 *   for i < D: accept draft x_i iff u_acc[i] * q_i(x_i) < p_i(x_i), else stop (k = i)
 *   k < D: sample y from max(0, p_k - q_k) / R; k == D: sample the bonus y from p_D
 *   sampling: y = min{ j : C_j > u_res[k] * R } with C the running sum in index order
 * Outputs: out_tokens[b][0..k] = x_0..x_{k-1}, y; the rest -1; out_n_acc[b] = k;
 * out_flags[b] = VW4_FLAG_* bits (a row flagged non-finite gives tokens -1 and
 * n_acc -1).  D = 0 is plain sampling of p_0 (one autoregressive step).
 * Requires 1 <= B <= 2^24, 0 <= D <= 7, 1 <= V <= 2^24, draft ids in [0, V).
 * Workspace: vw4_accept_workspace_bytes(B, V) (for V > 16384 and B <= 8 it
 * also holds the row's fp64 residual masses, 8 V bytes per problem, which the
 * sampling pass reads back instead of recomputing them).
 * ------------------------------------------------------------------------ */
VW4_API size_t vw4_accept_workspace_bytes(int32_t B, int32_t V);

/* As spec_accept, but the step of problem 0 is read from device memory
 * (*step_dev) when the kernels run, so that a captured graph of the verify step
 * (the pages' compiled-graph cache: hazakura.dev mtplx page,
 * "4層のアーキテクチャ" Layer 0, GraphBank) draws fresh uniforms on every replay;
 * vw4_step_advance(step_dev, inc) adds inc to it on the stream. */
VW4_API int spec_accept_ex(const float* logits, int64_t logits_bstride, const vw4_rowstat* stats,
                           int64_t stats_bstride, const float* q, int64_t q_bstride, const int32_t* draft, int32_t B,
                           int32_t D, int32_t V, float temperature, uint64_t seed, const uint64_t* step_dev,
                           int32_t* out_tokens, int32_t* out_n_acc, uint32_t* out_flags, void* ws, size_t ws_bytes,
                           void* stream);
VW4_API int vw4_step_advance(uint64_t* step_dev, uint64_t inc, void* stream);

VW4_API int spec_accept(const float* logits, int64_t logits_bstride, const vw4_rowstat* stats, int64_t stats_bstride,
                const float* q, int64_t q_bstride, const int32_t* draft, int32_t B, int32_t D, int32_t V,
                float temperature, uint64_t seed, uint64_t step0, int32_t* out_tokens, int32_t* out_n_acc,
                uint32_t* out_flags, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Decoder-layer calls of the verify forward (hazakura.dev mtplx page,
 * "4層のアーキテクチャ" Layer 1: target and drafter share one checkpoint and a
 * KV cache; gist.science BaseRT summary, "メソドロジー": decode-step operator
 * sequences fused so that short kernels do not pay extra round trips, and
 * attention computed tile by tile with an online softmax).  All tensors bf16
 * unless stated; M <= 8 verify rows at positions L .. L+M-1.
 *
 * Split GEMM outputs.  w4_skinny_gemm_partials writes the GEMM as S fp32
 * partial sums part[S][M][ldp] (S and ldp from vw4_gemm_partials_layout; the
 * output is the sum over S in slice order, and S == 1 means part[0] is the
 * product itself).  The layer calls below take such partials and fold the
 * reduction into their own pass, so no separate reduction launch is needed.
 * ------------------------------------------------------------------------ */
VW4_API int vw4_gemm_partials_layout(int32_t M, int32_t N, int32_t K, int32_t* S, int64_t* ldp);

VW4_API int w4_skinny_gemm_partials(const uint16_t* x, int64_t ldx, const uint8_t* w_packed,
                                    const uint16_t* scales_packed, float* part, int32_t M, int32_t N, int32_t K,
                                    void* stream);

/* resid[M][D] (bf16, in/out) += sum_s part[s][m][d] (fp32; part may be NULL to
 * skip the add), rounded to bf16; then h = bf16(rmsnorm(resid) * gamma):
 * h = r / sqrt(mean_d(r^2) + eps) * gamma.  D <= 65536, M <= 64.
 * Workspace: vw4_norm_workspace_bytes(M, D) (per-chunk sums of squares). */
VW4_API size_t vw4_norm_workspace_bytes(int32_t M, int32_t D);
VW4_API int vw4_add_rmsnorm(uint16_t* resid, const float* part, int32_t S, int64_t ldp, const uint16_t* gamma,
                            float eps, int32_t M, int32_t D, uint16_t* h, void* ws, size_t ws_bytes, void* stream);

/* vw4_add_rmsnorm in one launch, out of place: resid_out = bf16(resid_in +
 * sum_s part) (part may be NULL: resid_out = resid_in) and h = bf16(
 * rmsnorm(resid_out) * gamma), bitwise what vw4_add_rmsnorm gives.  Every
 * workgroup forms its row's sums of squares itself (the same chunk sums, in
 * the same order), so no second launch is needed; that is why the residual is
 * written to another buffer (other workgroups still read resid_in).
 * D % 4 == 0, 4 <= D <= 8192, M <= 64, S <= 8, ldp % 4 == 0; part 16-byte
 * aligned, the rest 8-byte aligned; resid_in, resid_out and h must not
 * overlap.  No workspace. */
VW4_API int vw4_add_rmsnorm_out(const uint16_t* resid_in, const float* part, int32_t S, int64_t ldp,
                                const uint16_t* gamma, float eps, int32_t M, int32_t D, uint16_t* resid_out,
                                uint16_t* h, void* stream);

/* The first half of vw4_add_rmsnorm alone: resid += sum_s part (bf16), and the
 * per-chunk sums of squares of the rounded rows into ws ([M][ceil(D / 256)]
 * floats, chunk order), for a GEMM that normalises its own activations. */
VW4_API int vw4_add_sumsq(uint16_t* resid, const float* part, int32_t S, int64_t ldp, int32_t M, int32_t D,
                          void* ws, size_t ws_bytes, void* stream);

/* w4_skinny_gemm_partials with the RMSNorm folded into the activation load
 * (gist.science BaseRT summary, "メソドロジー": operator sequences fused so
 * that short kernels do not pay an extra round trip): the activations are
 * h = bf16(resid / sqrt(mean(resid^2) + eps) * gamma), formed in registers
 * as each group of 64 columns is consumed, from resid [M][K] bf16, gamma [K]
 * bf16 and the sums of squares vw4_add_sumsq left in norm_ws; h is bitwise
 * what vw4_add_rmsnorm writes.  K <= 16384 (at most 64 chunk sums per row).
 * Partials layout as vw4_gemm_partials_layout(M, N, K). */
VW4_API int w4_skinny_gemm_rmsnorm_partials(const uint16_t* resid, const uint16_t* gamma, const void* norm_ws,
                                            float eps, const uint8_t* w_packed, const uint16_t* scales_packed,
                                            float* part, int32_t M, int32_t N, int32_t K, void* stream);

/* Gate|up projection with the SwiGLU in its epilogue, on given bf16
 * activations x [M][K] (row stride ldx): a[m][f] = bf16(silu(g) * u), the
 * matrix packed gate/up-interleaved as for w4_skinny_gemm_rmsnorm_swiglu. */
VW4_API int w4_skinny_gemm_swiglu(const uint16_t* x, int64_t ldx, const uint8_t* w_packed,
                                  const uint16_t* scales_packed, uint16_t* a, int64_t lda, int32_t M, int32_t F,
                                  int32_t K, void* stream);

/* Fused gate|up projection with the SwiGLU in its epilogue:
 * a[m][f] = bf16(silu(g) * u) (row stride lda >= F), g and u being rows of
 * one W4 matrix of 2F rows packed in gate/up-interleaved order: rows
 * 64 t .. 64 t + 31 are the gate rows of features 32 t .. 32 t + 31 and rows
 * 64 t + 32 .. 64 t + 63 the up rows of the same features (F % 32 == 0).
 * The activations are normalised as in w4_skinny_gemm_rmsnorm_partials
 * (K <= 16384). */
VW4_API int w4_skinny_gemm_rmsnorm_swiglu(const uint16_t* resid, const uint16_t* gamma, const void* norm_ws,
                                          float eps, const uint8_t* w_packed, const uint16_t* scales_packed,
                                          uint16_t* a, int64_t lda, int32_t M, int32_t F, int32_t K, void* stream);

/* vw4_moe_combine followed by vw4_add_rmsnorm_out (with the combined rows as
 * its single partial slice) in one launch: resid_out = bf16(resid_in + y) and
 * h = bf16(rmsnorm(resid_out) * gamma), y the weighted sum of the routed
 * experts' down-projection partials of vw4_moe_combine (gist.science BaseRT
 * summary, "メソドロジー": fused decode operator sequences; "結果": MoE models
 * of the Qwen3-30B-A3B class).  Bitwise the two calls' results.  Arguments as
 * the two calls (part [slot][S][M][ldp] fp32, slot stride p_sstride, 16-byte
 * aligned, ldp and p_sstride multiples of 4).  Built for topk <= 8 with
 * D <= 2048 and S <= 4, or D <= 4096 and S <= 2; VW4_EUNSUPPORTED otherwise. */
VW4_API int vw4_moe_add_rmsnorm(const uint16_t* resid_in, const float* part, int32_t S, int64_t ldp,
                                int64_t p_sstride, const int32_t* row_slot, const float* weights, int32_t topk,
                                const uint16_t* gamma, float eps, int32_t M, int32_t D, uint16_t* resid_out,
                                uint16_t* h, void* stream);

/* From the fused q|k|v projection (partials of [M][(nq + 2 nkv) * hd]): rotary
 * embedding (rotate-half, base theta, position L + m) of q and k; q -> q_out
 * [M][nq][hd]; k appended to the key cache Kc [nkv][Lmax][hd] and v to the
 * blocked value cache Vb [nkv][Lmax / 32][hd][32] (position p, dimension d at
 * [p / 32][d][p % 32]), both at positions L + m.  hd even, L + M <= Lmax,
 * Lmax % 32 == 0. */
VW4_API int vw4_rope_kv_append(const float* part, int32_t S, int64_t ldp, int32_t M, int32_t nq, int32_t nkv,
                               int32_t hd, int32_t L, float theta, uint16_t* q_out, uint16_t* Kc, uint16_t* Vb,
                               int64_t Lmax, void* stream);

/* a[M][F] = bf16(silu(g) * u) with g = part[.][m][0:F], u = part[.][m][F:2F]
 * (fused gate|up projection), silu(g) = g / (1 + exp(-g)). */
VW4_API int vw4_swiglu(const float* part, int32_t S, int64_t ldp, int32_t M, int32_t F, uint16_t* a, void* stream);

/* Grouped-query decode attention for M verify rows: query head h reads KV head
 * h / (nq / nkv); row m attends to positions 0 .. L + m of the cache (causal
 * inside the verify rows); softmax(q k^T / sqrt(hd)) v, computed tile by tile
 * with an online softmax (gist.science BaseRT summary, "メソドロジー") on the
 * matrix cores: bf16 products, fp32 accumulation, the probabilities of the
 * P.V product split into a bf16 head and tail (about 16 significant bits);
 * the fewer than 32 positions past the last whole 32-position tile are added
 * in the merge pass, in fp32.  q [M][nq][hd]; keys Kc [nkv][Lmax][hd]; values
 * in 32-position blocks, Vb [nkv][Lmax / 32][hd][32] (as vw4_rope_kv_append
 * writes them); out [M][nq * hd] bf16.  hd == 128, nq % nkv == 0,
 * (nq / nkv) * M <= 48, Lmax % 32 == 0, L + M < 2^29, q / Kc / Vb 16-byte
 * aligned.  Workspace: vw4_attn_workspace_bytes. */
VW4_API size_t vw4_attn_workspace_bytes(int32_t M, int32_t nq, int32_t nkv, int32_t hd, int64_t ctx);
VW4_API int vw4_decode_attn(const uint16_t* q, const uint16_t* Kc, const uint16_t* Vb, int64_t Lmax, int64_t L,
                            int32_t M, int32_t nq, int32_t nkv, int32_t hd, uint16_t* out, void* ws, size_t ws_bytes,
                            void* stream);

/* ------------------------------------------------------------------------
 * Mixture-of-experts calls of the MoE-shaped verify step (gist.science,
 * "BaseRT: Best-in-Class LLM Inference on Apple Silicon via Native Metal",
 * section "結果": MoE models of the Qwen3-30B-A3B class, 128 experts with 8
 * active).  Each verify row is routed on its own; the distinct experts chosen
 * by any row form device-side "slots", so no call reads the routing on the
 * host and the whole step can be captured as a HIP graph.
 * ------------------------------------------------------------------------ */

/* Router: per row m of logits [M][E] (fp32), the topk experts with the
 * largest logits (equal logits: lower index first) -> experts[M][topk] in that
 * order, and their softmax probabilities renormalised over the chosen ones ->
 * weights[M][topk] (fp64 arithmetic, stored fp32).  Slots: the distinct
 * chosen experts in ascending order -> slot_expert[0 .. *n_slots) (at most
 * min(E, M * topk) entries are written); row_slot[M][topk] = slot of
 * experts[m][t].  Limits: M <= 16, E <= 1024, topk <= min(E, 64).  Logits are
 * expected finite; non-finite ones still give valid indices. */
VW4_API int vw4_moe_route(const float* logits, int32_t M, int32_t E, int32_t topk, int32_t* experts, float* weights,
                          int32_t* slot_expert, int32_t* n_slots, int32_t* row_slot, void* stream);

/* Grouped W4 GEMM over the slots: for every slot s < *n_slots (device
 * value; launches cover max_slots slots and the rest exit), expert
 * e = slot_expert[s], part[s] = split-K partials (as w4_skinny_gemm_partials,
 * [S][M][ldp] from vw4_grouped_gemm_layout) of x_s . W_e^T with
 * x_s = x + s * x_sstride ([M][K], row stride ldx, bf16) and W_e the packed W4
 * matrix at w_bank + e * w_estride bytes with its packed scales at
 * s_bank + e * s_estride fp16 elements.  Slot s's partials start at
 * part + s * p_sstride floats, p_sstride >= S * M * ldp.  An [E * N][K] matrix
 * packed by vw4_w4_pack with N % 64 == 0 is such a bank with
 * w_estride = N * K / 2 and s_estride = N * K / 64.  x_sstride = 0 gives every
 * slot the same rows. */
VW4_API int vw4_grouped_gemm_layout(int32_t M, int32_t N, int32_t K, int32_t max_slots, int32_t* S, int64_t* ldp);
VW4_API int w4_grouped_gemm(const uint16_t* x, int64_t ldx, int64_t x_sstride, const uint8_t* w_bank,
                            int64_t w_estride, const uint16_t* s_bank, int64_t s_estride, const int32_t* slot_expert,
                            const int32_t* n_slots, int32_t max_slots, float* part, int64_t p_sstride, int32_t M,
                            int32_t N, int32_t K, void* stream);

/* Grouped gate|up projection with the SwiGLU in its epilogue: for every
 * slot s < *n_slots, a + s * a_sstride ([M][F] bf16) = bf16(silu(g) * u) of
 * expert slot_expert[s], whose [2F][K] matrix is packed gate/up-interleaved
 * as for w4_skinny_gemm_rmsnorm_swiglu; x, strides and banks as
 * w4_grouped_gemm. */
VW4_API int w4_grouped_gemm_swiglu(const uint16_t* x, int64_t ldx, int64_t x_sstride, const uint8_t* w_bank,
                                   int64_t w_estride, const uint16_t* s_bank, int64_t s_estride,
                                   const int32_t* slot_expert, const int32_t* n_slots, int32_t max_slots, uint16_t* a,
                                   int64_t a_sstride, int32_t M, int32_t F, int32_t K, void* stream);

/* vw4_swiglu per slot: slot s < *n_slots reads partials at
 * part + s * p_sstride and writes a + s * a_sstride ([M][F] bf16). */
VW4_API int vw4_grouped_swiglu(const float* part, int32_t S, int64_t ldp, int64_t p_sstride, int32_t M, int32_t F,
                               uint16_t* a, int64_t a_sstride, const int32_t* n_slots, int32_t max_slots,
                               void* stream);

/* y[m][d] (fp32, row stride ldy) = sum_t weights[m][t] * (expert output of
 * row m in slot row_slot[m][t]), the expert output being the sum of the slot's
 * down-projection partials part[slot][s][m][d] (S slices, row stride ldp,
 * slots p_sstride floats apart).  Experts in selection order, fp32. */
VW4_API int vw4_moe_combine(const float* part, int32_t S, int64_t ldp, int64_t p_sstride, const int32_t* row_slot,
                            const float* weights, int32_t M, int32_t topk, int32_t D, float* y, int64_t ldy,
                            void* stream);

/* ------------------------------------------------------------------------
 * The draft side of the cycle (hazakura.dev mtplx page, section
 * "4層のアーキテクチャ": Layer 1, the drafter is the MTP head inside the same
 * checkpoint; Layer 0, it has a 4-bit LM head; Layer 2, Draft -> Verify ->
 * ratio acceptance -> residual correction -> bonus token).  The pages do not
 * describe the head's inside; the common MTP head is built: the last hidden
 * row and the next token's embedding, each RMS-normalised with its own gain,
 * concatenated, projected back to d (a W4 GEMM), one decoder layer, the final
 * norm and the LM head.  All pointers are device memory owned by the caller.
 * ------------------------------------------------------------------------ */

/* out[i][0:d] (row stride ldo) = E[tokens[i]][0:d] (E: [V][d] bf16, row
 * stride lde), for i < n; an id outside [0, V) gives a row of zeros (ids are
 * read on the device, so a captured graph can take new ones).  d % 8 == 0,
 * strides multiples of 8, E and out 16-byte aligned, 1 <= n <= 65535. */
VW4_API int vw4_embed_rows(const uint16_t* E, int64_t lde, int32_t V, int32_t d, const int32_t* tokens, int32_t n,
                           uint16_t* out, int64_t ldo, void* stream);

/* Projection input of one draft, out[0:2d] (bf16):
 *   out[0:d]  = bf16(h_r * (1 / sqrt(mean(h_r^2) + eps)) * gamma_h), r = *h_row
 *               (0 if h_row is NULL; clamped to [0, h_rows)), h_r = h + r * ldh;
 *   out[d:2d] = the same of the embedding row E[*token] with gamma_e (a zero
 *               row for an id outside [0, V)).
 * Sums of squares in fp32.  8 <= d <= 8192, d % 8 == 0, strides multiples of
 * 8, h, E, gains and out 16-byte aligned. */
VW4_API int vw4_mtp_input(const uint16_t* h, int64_t ldh, int32_t h_rows, const int32_t* h_row, const uint16_t* E,
                          int64_t lde, int32_t V, const int32_t* token, const uint16_t* gamma_h,
                          const uint16_t* gamma_e, float eps, int32_t d, uint16_t* out, void* stream);

/* One draft token from draft logits [V] (fp32) and their rowstat (from
 * verify_logits with the target's temperature and top-p):
 *   q_out (nullable) [V] = p(j) as binary32, p the warped distribution (the
 *     q row the verify's spec_accept reads for this draft);
 *   *token_out = min{ j : C_j > u * R } (inverse CDF of p in index order, fp64),
 *     u = (r1 >> 11) 2^-53 of Philox4x64-10 with key (seed, 0) and counter
 *     (step, depth, 1, 0): the third word 1 keeps drafts apart from the verify's
 *     uniforms, whose third word is 0; step = *step_dev if step_dev is not NULL
 *     (read when the kernels run), else the step argument;
 *   *flags_out: VW4_FLAG_* bits (a non-finite row gives token -1).
 * T == 0 is greedy (argmax, q one-hot).  1 <= V <= 2^24, 0 <= depth <= 1023.
 * Workspace: vw4_draft_workspace_bytes(V), 256-byte aligned. */
VW4_API size_t vw4_draft_workspace_bytes(int32_t V);
VW4_API int draft_sample(const float* logits, const vw4_rowstat* stats, int32_t V, float temperature, uint64_t seed,
                         const uint64_t* step_dev, uint64_t step, int32_t depth, float* q_out, int32_t* token_out,
                         uint32_t* flags_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * A second weight format for the skinny GEMM: W8 (gist.science, "BaseRT: Best-
 * in-Class LLM Inference on Apple Silicon via Native Metal", section
 * "メソドロジー": the GEMV reads several quantisation formats, Q8 among them;
 * no layout is given).  Per row n and 64-element group g along K:
 *     scale = fp16_rne(absmax / 127);  c_k = clamp(rint(w_k / scale), -127, 127)
 * with the rounded scale, half-even; an all-zero group gets scale 0 and codes 0.
 * Canonical storage: u8 codes[N][K] holding u = c + 128, fp16 scales[N][K/64].
 * Kernel storage: the high and the low nibble of u as two planes, each in the
 * W4 packed layout (vw4_w4_packed_bytes(N, K) bytes per plane) with the W4
 * packed scales.
 * ------------------------------------------------------------------------ */

/* Host quantiser (host memory): w [N][K] fp32 -> codes [N][K], scales [N][K/64]. */
VW4_API int vw4_w8_quantize_host(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales);

/* Canonical codes and scales (device) -> the two packed nibble planes hi, lo
 * (16-byte aligned, vw4_w4_packed_bytes(N, K) bytes each) and the packed
 * scales; rows are padded to a multiple of 64 with code 0 and scale 0. */
VW4_API int vw4_w8_pack(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K, uint8_t* hi,
                        uint8_t* lo, uint16_t* packed_scales, void* stream);

/* y[M][N] (fp32 or bf16, row stride ldy) = x[M][K] (bf16, row stride ldx) .
 * deq(W8)^T, W8 given as its packed planes and scales.  1 <= M <= 8,
 * K % 64 == 0, K <= 65536; x 16-byte aligned with ldx % 8 == 0.  Workspace:
 * vw4_w8_workspace_bytes(M, N, K) (0: none needed), 256-byte aligned.
 * Sums are fp32 in an order fixed by (N, K). */
VW4_API size_t vw4_w8_workspace_bytes(int32_t M, int32_t N, int32_t K);
VW4_API int w8_skinny_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                           const uint16_t* scales_packed, void* y, int64_t ldy, int32_t y_dtype, int32_t M, int32_t N,
                           int32_t K, void* ws, size_t ws_bytes, void* stream);

/* The product as fp32 split-K partials for a consumer that sums them (the
 * decoder's RoPE, add + RMSNorm and SwiGLU calls take (part, S, ldp)):
 * part[s][m][n] (s < S, row stride ldp), S and ldp from
 * vw4_w8_partials_layout(M, N, K); columns n >= N of a row are padding.
 * part is caller-owned, S * M * ldp floats, 16-byte aligned. */
VW4_API int vw4_w8_partials_layout(int32_t M, int32_t N, int32_t K, int32_t* S, int64_t* ldp);
VW4_API int w8_skinny_gemm_partials(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                                    const uint16_t* scales_packed, float* part, int32_t M, int32_t N, int32_t K,
                                    void* stream);

/* ------------------------------------------------------------------------
 * Gate|up projection with the SwiGLU in the epilogue, in the formats other
 * than W4 (w4_skinny_gemm_swiglu above): a[m][f] = bf16(silu(g) * u), row
 * stride lda >= F, from one matrix of 2 F rows in the gate/up-interleaved
 * order of w4_skinny_gemm_rmsnorm_swiglu (rows 64 t .. 64 t + 31 the gate rows
 * of features 32 t .. 32 t + 31, rows 64 t + 32 .. 64 t + 63 their up rows;
 * F % 32 == 0), packed by the format's own pack.  x bf16 [M][ldx] (ldx >= K,
 * ldx % 8 == 0, 16-byte aligned), M in 1..8, K % 64 == 0 and K <= 65536.
 * Each GEMM's sums are fp32 in an order that depends only on (F, K).
 * VW4_EINVAL on a bad shape, a null or misaligned pointer.
 * ------------------------------------------------------------------------ */
VW4_API int w8_skinny_gemm_swiglu(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                                  const uint16_t* scales_packed, uint16_t* a, int64_t lda, int32_t M, int32_t F,
                                  int32_t K, void* stream);
VW4_API int w6_skinny_gemm_swiglu(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                                  const uint16_t* scales_packed, uint16_t* a, int64_t lda, int32_t M, int32_t F,
                                  int32_t K, void* stream);
VW4_API int w5_skinny_gemm_swiglu(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                                  const uint16_t* scales_packed, uint16_t* a, int64_t lda, int32_t M, int32_t F,
                                  int32_t K, void* stream);
VW4_API int w3_skinny_gemm_swiglu(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                                  const uint16_t* scales_packed, uint16_t* a, int64_t lda, int32_t M, int32_t F,
                                  int32_t K, void* stream);
VW4_API int w2_skinny_gemm_swiglu(const uint16_t* x, int64_t ldx, const uint8_t* w_packed,
                                  const uint16_t* scales_packed, uint16_t* a, int64_t lda, int32_t M, int32_t F,
                                  int32_t K, void* stream);
VW4_API int f16_skinny_gemm_swiglu(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, uint16_t* a,
                                   int64_t lda, int32_t M, int32_t F, int32_t K, void* stream);
VW4_API int bf16_skinny_gemm_swiglu(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, uint16_t* a,
                                    int64_t lda, int32_t M, int32_t F, int32_t K, void* stream);

/* ------------------------------------------------------------------------
 * Unquantised 16-bit float weights: the widest end of the same BaseRT list
 * (Q2 ... FP16), as fp16 and as bf16.  w[N][K] holds IEEE binary16 (fp16)
 * or bfloat16 bit patterns; there are no scales.
 *
 * vw4_w16_pack: w (device, [N][K] row-major) -> the operand-tiled layout
 * (vw4_w16_packed_bytes(N, K) = pad64(N) * K * 2 bytes, 16-byte aligned):
 * per 64-row tile t and K-group g 8 KiB, the 16-byte word
 * ((t * K/64 + g) * 8 + 2 nb + s) * 64 + 16 kq + i holding row
 * 64 t + 16 nb + i at k = 64 g + 32 s + 8 kq + 0..7; padding rows are zero.
 * The same pack serves both types.
 *
 * f16_skinny_gemm / bf16_skinny_gemm: y = x @ W^T with the conventions of
 * w4_skinny_gemm (x bf16 [M][ldx], ldx >= K, ldx % 8 == 0, 16-byte aligned;
 * y fp32 or bf16 [M][ldy]; M in 1..8, K % 64 == 0 and K <= 65536; a
 * workspace of at least vw4_{f16,bf16}_workspace_bytes(M, N, K) bytes,
 * 256-byte aligned, when that is not 0, else VW4_EWORKSPACE).  fp16 weights
 * are split exactly into two bf16 parts, so every product is exact in fp32;
 * sums are fp32.  The partials calls write S slices of [M][ldp] fp32 sums
 * (vw4_{f16,bf16}_partials_layout) that add up, in slice order, to y.
 * ------------------------------------------------------------------------ */
VW4_API size_t vw4_w16_packed_bytes(int64_t N, int64_t K);
VW4_API int vw4_w16_pack(const uint16_t* w, int64_t N, int64_t K, uint8_t* packed, void* stream);
VW4_API size_t vw4_f16_workspace_bytes(int32_t M, int32_t N, int32_t K);
VW4_API size_t vw4_bf16_workspace_bytes(int32_t M, int32_t N, int32_t K);
VW4_API int f16_skinny_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, void* y, int64_t ldy,
                            int32_t y_dtype, int32_t M, int32_t N, int32_t K, void* ws, size_t ws_bytes,
                            void* stream);
VW4_API int bf16_skinny_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, void* y, int64_t ldy,
                             int32_t y_dtype, int32_t M, int32_t N, int32_t K, void* ws, size_t ws_bytes,
                             void* stream);
VW4_API int vw4_f16_partials_layout(int32_t M, int32_t N, int32_t K, int32_t* S, int64_t* ldp);
VW4_API int vw4_bf16_partials_layout(int32_t M, int32_t N, int32_t K, int32_t* S, int64_t* ldp);
VW4_API int f16_skinny_gemm_partials(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, float* part,
                                     int32_t M, int32_t N, int32_t K, void* stream);
VW4_API int bf16_skinny_gemm_partials(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, float* part,
                                      int32_t M, int32_t N, int32_t K, void* stream);

/* ------------------------------------------------------------------------
 * The narrowest weight formats: W3 and W2 (the same BaseRT section lists Q2
 * ... Q8; no layout).  Per row n and 64-element group g: scale =
 * fp16_rne(absmax / qmax), c_k = clamp(rint(w_k / scale), -qmax, qmax) with
 * the rounded scale, half-even; an all-zero group gets scale 0 and codes 0.
 * W3: qmax 3, canonical u8 codes[N][K] holding u = c + 4; W2: qmax 1,
 * u = c + 1; fp16 scales[N][K/64].
 *
 * Kernel storage, W3: the high bit of u in the 1-bit plane of the W5 layout
 * (vw4_w3_hi_plane_bytes(N, K) = pad64(N) * K / 8 bytes), the low 2 bits in
 * a 2-bit plane (vw4_w3_lo_plane_bytes(N, K) = pad64(N) * K / 4 bytes: per
 * 64-row tile and K-group 1 KiB, lane l = 16 kq + i owning 16 bytes, dword
 * nb holding row 16 nb + i, the field of k = 32 s + 8 kq + j at bits
 * 8 s + 2 (j / 2) + 16 (j % 2)), and the W4 packed scales.  W2: c = u - 1
 * in sign-magnitude (field bit 0 = (c != 0), bit 1 = (c < 0)) in one 2-bit
 * plane of that layout (vw4_w2_packed_bytes(N, K) bytes) and the W4 packed
 * scales.  Padding rows hold code 0 and scale 0.  Planes are 16-byte
 * aligned.
 *
 * The quantisers run on the host (VW4_EINVAL on a bad shape or a null
 * pointer); the packs read device codes and scales and write device planes
 * on `stream`.  The GEMM calls behave as their W6 / W4 counterparts: x bf16
 * [M][ldx] (ldx >= K, ldx % 8 == 0, 16-byte aligned), y fp32 or bf16
 * [M][ldy], M in 1..8, K % 64 == 0 and K <= 65536; a workspace of at least
 * vw4_wN_workspace_bytes(M, N, K) bytes (256-byte aligned) when that is not
 * 0, else VW4_EWORKSPACE; the partials calls write S slices of [M][ldp]
 * fp32 sums (vw4_wN_partials_layout) that add up, in slice order, to y.
 * ------------------------------------------------------------------------ */
VW4_API int vw4_w3_quantize_host(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales);
VW4_API size_t vw4_w3_hi_plane_bytes(int64_t N, int64_t K);
VW4_API size_t vw4_w3_lo_plane_bytes(int64_t N, int64_t K);
VW4_API int vw4_w3_pack(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K, uint8_t* hi,
                        uint8_t* lo, uint16_t* packed_scales, void* stream);
VW4_API size_t vw4_w3_workspace_bytes(int32_t M, int32_t N, int32_t K);
VW4_API int w3_skinny_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                           const uint16_t* scales_packed, void* y, int64_t ldy, int32_t y_dtype, int32_t M, int32_t N,
                           int32_t K, void* ws, size_t ws_bytes, void* stream);
VW4_API int vw4_w3_partials_layout(int32_t M, int32_t N, int32_t K, int32_t* S, int64_t* ldp);
VW4_API int w3_skinny_gemm_partials(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                                    const uint16_t* scales_packed, float* part, int32_t M, int32_t N, int32_t K,
                                    void* stream);

VW4_API int vw4_w2_quantize_host(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales);
VW4_API size_t vw4_w2_packed_bytes(int64_t N, int64_t K);
VW4_API int vw4_w2_pack(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K, uint8_t* packed,
                        uint16_t* packed_scales, void* stream);
VW4_API size_t vw4_w2_workspace_bytes(int32_t M, int32_t N, int32_t K);
VW4_API int w2_skinny_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, const uint16_t* scales_packed,
                           void* y, int64_t ldy, int32_t y_dtype, int32_t M, int32_t N, int32_t K, void* ws,
                           size_t ws_bytes, void* stream);
VW4_API int vw4_w2_partials_layout(int32_t M, int32_t N, int32_t K, int32_t* S, int64_t* ldp);
VW4_API int w2_skinny_gemm_partials(const uint16_t* x, int64_t ldx, const uint8_t* w_packed,
                                    const uint16_t* scales_packed, float* part, int32_t M, int32_t N, int32_t K,
                                    void* stream);

/* ------------------------------------------------------------------------
 * A fourth weight format: W5 (the same BaseRT section lists Q2 ... Q8; no
 * layout).  Per row n and 64-element group g: scale = fp16_rne(absmax / 15),
 * c_k = clamp(rint(w_k / scale), -15, 15) with the rounded scale, half-even;
 * an all-zero group gets scale 0 and codes 0.  Canonical storage: u8
 * codes[N][K] holding u = c + 16, fp16 scales[N][K/64].  Kernel storage: the
 * low 4 bits of u in the W4 packed layout (vw4_w4_packed_bytes(N, K) bytes),
 * the high bit in a 1-bit plane of vw4_w5_hi_plane_bytes(N, K) bytes (per
 * 64-row tile and K-group 512 bytes; lane l = 16 kq + i owns 8 bytes, dword d
 * holding rows 16 nb + i of row blocks nb = 2 d and 2 d + 1, the bit of
 * k = 32 s + 8 kq + j at 4 (2 (nb & 1) + s) + j / 2 + 16 (j % 2)), and the W4
 * packed scales.  The calls below behave as their W6 counterparts.
 * ------------------------------------------------------------------------ */
VW4_API int vw4_w5_quantize_host(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales);
VW4_API size_t vw4_w5_hi_plane_bytes(int64_t N, int64_t K);
VW4_API int vw4_w5_pack(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K, uint8_t* hi,
                        uint8_t* lo, uint16_t* packed_scales, void* stream);
VW4_API size_t vw4_w5_workspace_bytes(int32_t M, int32_t N, int32_t K);
VW4_API int w5_skinny_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                           const uint16_t* scales_packed, void* y, int64_t ldy, int32_t y_dtype, int32_t M, int32_t N,
                           int32_t K, void* ws, size_t ws_bytes, void* stream);
VW4_API int vw4_w5_partials_layout(int32_t M, int32_t N, int32_t K, int32_t* S, int64_t* ldp);
VW4_API int w5_skinny_gemm_partials(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                                    const uint16_t* scales_packed, float* part, int32_t M, int32_t N, int32_t K,
                                    void* stream);

/* ------------------------------------------------------------------------
 * A third weight format: W6 (the same BaseRT section lists Q2 ... Q8; no
 * layout).  Per row n and 64-element group g: scale = fp16_rne(absmax / 31),
 * c_k = clamp(rint(w_k / scale), -31, 31) with the rounded scale, half-even;
 * an all-zero group gets scale 0 and codes 0.  Canonical storage: u8
 * codes[N][K] holding u = c + 32, fp16 scales[N][K/64].  Kernel storage: the
 * low 4 bits of u in the W4 packed layout (vw4_w4_packed_bytes(N, K) bytes),
 * the high 2 bits in a 2-bit plane of vw4_w6_hi_plane_bytes(N, K) bytes (per
 * 64-row tile and K-group 1 KiB; lane l = 16 kq + i owns 16 bytes, dword nb
 * holding row 16 nb + i at k = 32 s + 8 kq + j in bits 8 s + 2 (j / 2) +
 * 16 (j % 2)), and the W4 packed scales.
 * ------------------------------------------------------------------------ */
VW4_API int vw4_w6_quantize_host(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales);
VW4_API size_t vw4_w6_hi_plane_bytes(int64_t N, int64_t K);
VW4_API int vw4_w6_pack(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K, uint8_t* hi,
                        uint8_t* lo, uint16_t* packed_scales, void* stream);
/* As w8_skinny_gemm / w8_skinny_gemm_partials / vw4_w8_*_bytes, for W6 planes. */
VW4_API size_t vw4_w6_workspace_bytes(int32_t M, int32_t N, int32_t K);
VW4_API int w6_skinny_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                           const uint16_t* scales_packed, void* y, int64_t ldy, int32_t y_dtype, int32_t M, int32_t N,
                           int32_t K, void* ws, size_t ws_bytes, void* stream);
VW4_API int vw4_w6_partials_layout(int32_t M, int32_t N, int32_t K, int32_t* S, int64_t* ldp);
VW4_API int w6_skinny_gemm_partials(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                                    const uint16_t* scales_packed, float* part, int32_t M, int32_t N, int32_t K,
                                    void* stream);

/* ------------------------------------------------------------------------
 * Measurement: the plain streaming-read ceiling of the part (gist.science
 * BaseRT summary, "結果": decode is bound by memory bandwidth; the W4 GEMM's
 * achieved bandwidth is reported against it beside the published peak).
 * Reads `bytes` (a multiple of 16) at device pointer src with 16-byte
 * non-temporal loads, blocks workgroups of 256 threads in a grid-stride loop;
 * sink[b] (device, `blocks` words, caller-owned) receives the XOR of the
 * 32-bit words workgroup b read, so the XOR of all sink words equals the XOR
 * of the buffer's words.  1 <= blocks <= 2^20.  Enqueues only.
 * ------------------------------------------------------------------------ */
VW4_API int vw4_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VW4_H */
