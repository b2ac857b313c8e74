// w16_gemm.hip — the skinny GEMM on unquantised 16-bit float weights (M =
// 1..8): the widest end of the format list the GEMV reads (gist.science,
// "BaseRT: …", section "メソドロジー": Q2 ... FP16), as fp16 and as bf16.
//
// y[m][n] = sum_k x[m][k] * w[n][k]
//
// The weights sit in the operand-tiled layout of vw4_w16_pack, one 16-byte
// word per MFMA B operand.  bf16 weights feed the matrix cores as they are;
// fp16 weights are split exactly into two bf16 parts (hi = the weight
// truncated to 8 significant bits, lo = the rest, at most 3 bits), so both
// products with the bf16 activations are exact in fp32.  The kernel is the
// shared template of skinny_gemm.h (no group scales: the products accumulate
// straight into the matrix-core chains) and the split plan every format
// shares; sums are fp32 in an order that depends only on (N, K): row m of an
// M-row call equals the one-row call bit for bit.  The template's scale
// pointer is not read for these formats; the weights' pointer stands in.
#include "skinny_formats.h"

using namespace vw4;

namespace {

template <class Fmt>
int w16_gemm(const char* name, const uint16_t* x, int64_t ldx, const uint8_t* w, void* y, int64_t ldy,
             int32_t y_dtype, int32_t M, int32_t N, int32_t K, void* ws, size_t ws_bytes, void* stream) {
    return sg::skinny_gemm_run<Fmt>(name, x, ldx, w, w, (const uint16_t*)w, y, ldy, y_dtype, M, N, K, ws, ws_bytes,
                                    (hipStream_t)stream);
}

template <class Fmt>
int w16_partials(const char* name, const uint16_t* x, int64_t ldx, const uint8_t* w, float* part, int32_t M,
                 int32_t N, int32_t K, void* stream) {
    return sg::skinny_gemm_partials_run<Fmt>(name, x, ldx, w, w, (const uint16_t*)w, part, M, N, K,
                                             (hipStream_t)stream);
}

int w16_layout(const char* name, int32_t M, int32_t N, int32_t K, int32_t* S, int64_t* ldp) {
    VW4_REQUIRE(M >= 1 && M <= sg::MAX_M && N >= 1 && K >= 64 && K % 64 == 0 && K <= 65536, VW4_EINVAL,
                "%s: bad shape M=%d N=%d K=%d", name, M, N, K);
    const sg::GemmPlan p = sg::plan_gemm(M, N, K);
    if (S) *S = p.S_grid;
    if (ldp) *ldp = p.Npad;
    return VW4_OK;
}

size_t w16_ws(int32_t M, int32_t N, int32_t K) {
    if (M < 1 || M > sg::MAX_M || N < 1 || K < 64 || K % 64 || K > 65536) return 0;
    return sg::plan_gemm(M, N, K).ws_bytes;
}

}  // namespace

extern "C" {

size_t vw4_f16_workspace_bytes(int32_t M, int32_t N, int32_t K) { return w16_ws(M, N, K); }
size_t vw4_bf16_workspace_bytes(int32_t M, int32_t N, int32_t K) { return w16_ws(M, N, K); }

int f16_skinny_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, void* y, int64_t ldy, int32_t y_dtype,
                    int32_t M, int32_t N, int32_t K, void* ws, size_t ws_bytes, void* stream) {
    return w16_gemm<sg::FmtF16>("f16_skinny_gemm", x, ldx, w_packed, y, ldy, y_dtype, M, N, K, ws, ws_bytes, stream);
}

int bf16_skinny_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, void* y, int64_t ldy, int32_t y_dtype,
                     int32_t M, int32_t N, int32_t K, void* ws, size_t ws_bytes, void* stream) {
    return w16_gemm<sg::FmtB16>("bf16_skinny_gemm", x, ldx, w_packed, y, ldy, y_dtype, M, N, K, ws, ws_bytes, stream);
}

int vw4_f16_partials_layout(int32_t M, int32_t N, int32_t K, int32_t* S, int64_t* ldp) {
    return w16_layout("vw4_f16_partials_layout", M, N, K, S, ldp);
}

int vw4_bf16_partials_layout(int32_t M, int32_t N, int32_t K, int32_t* S, int64_t* ldp) {
    return w16_layout("vw4_bf16_partials_layout", M, N, K, S, ldp);
}

int f16_skinny_gemm_partials(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, float* part, int32_t M,
                             int32_t N, int32_t K, void* stream) {
    return w16_partials<sg::FmtF16>("f16_skinny_gemm_partials", x, ldx, w_packed, part, M, N, K, stream);
}

int bf16_skinny_gemm_partials(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, float* part, int32_t M,
                              int32_t N, int32_t K, void* stream) {
    return w16_partials<sg::FmtB16>("bf16_skinny_gemm_partials", x, ldx, w_packed, part, M, N, K, stream);
}

int f16_skinny_gemm_swiglu(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, uint16_t* a, int64_t lda,
                           int32_t M, int32_t F, int32_t K, void* stream) {
    return sg::skinny_gemm_swiglu_run<sg::FmtF16>("f16_skinny_gemm_swiglu", x, ldx, w_packed, w_packed,
                                                  (const uint16_t*)w_packed, a, lda, M, F, K, (hipStream_t)stream);
}

int bf16_skinny_gemm_swiglu(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, uint16_t* a, int64_t lda,
                            int32_t M, int32_t F, int32_t K, void* stream) {
    return sg::skinny_gemm_swiglu_run<sg::FmtB16>("bf16_skinny_gemm_swiglu", x, ldx, w_packed, w_packed,
                                                  (const uint16_t*)w_packed, a, lda, M, F, K, (hipStream_t)stream);
}

}  // extern "C"
