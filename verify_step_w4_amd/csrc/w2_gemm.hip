// w2_gemm.hip — the skinny GEMM on W2 weights (M = 1..8): the narrowest weight
// format for the verify rows (gist.science, "BaseRT: …", section "メソドロジー",
// lists the quantisation formats its GEMV reads, Q2 ... Q8).
//
// y[m][n] = sum_g scale[n][g] * sum_{k in g} x[m][k] * c[n][k],  c in [-1, 1]
//
// The code c sits sign-magnitude (bit 0 = (c != 0), bit 1 = (c < 0)) in one
// 2-bit plane with the lane mapping of the W4 layout: per 64-row tile and
// K-group 1 KiB, lane l = 16 kq + i owning 16 bytes, dword nb holding row
// 16 nb + i, the field of k = 32 s + 8 kq + j at bits 8 s + 2 (j / 2) +
// 16 (j % 2).  The kernel is the shared template of skinny_gemm.h with the W2
// plane decoder: a field moved to bits 14-15 is the bf16 value 2 c, so the
// matrix cores sum x . (2 c) with no offset term and the group adds
// (scale / 2) times that.  Products are exact in fp32; sums are fp32 in an
// order that depends only on (N, K): row m of an M-row call equals the
// one-row call bit for bit.
#include "skinny_formats.h"

using namespace vw4;

extern "C" {

size_t vw4_w2_workspace_bytes(int32_t M, int32_t N, int32_t K) {
    if (M < 1 || M > sg::MAX_M || N < 1 || K < 64 || K % 64 || K > 65536) return 0;
    return sg::plan_gemm(M, N, K).ws_bytes;
}

int w2_skinny_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, const uint16_t* scales_packed, void* y,
                   int64_t ldy, int32_t y_dtype, int32_t M, int32_t N, int32_t K, void* ws, size_t ws_bytes,
                   void* stream) {
    return sg::skinny_gemm_run<sg::FmtW2>("w2_skinny_gemm", x, ldx, w_packed, w_packed, scales_packed, y, ldy, y_dtype,
                                          M, N, K, ws, ws_bytes, (hipStream_t)stream);
}

int vw4_w2_partials_layout(int32_t M, int32_t N, int32_t K, int32_t* S, int64_t* ldp) {
    VW4_REQUIRE(M >= 1 && M <= sg::MAX_M && N >= 1 && K >= 64 && K % 64 == 0 && K <= 65536, VW4_EINVAL,
                "vw4_w2_partials_layout: bad shape M=%d N=%d K=%d", M, N, K);
    const sg::GemmPlan p = sg::plan_gemm(M, N, K);
    if (S) *S = p.S_grid;
    if (ldp) *ldp = p.Npad;
    return VW4_OK;
}

int w2_skinny_gemm_partials(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, const uint16_t* scales_packed,
                            float* part, int32_t M, int32_t N, int32_t K, void* stream) {
    return sg::skinny_gemm_partials_run<sg::FmtW2>("w2_skinny_gemm_partials", x, ldx, w_packed, w_packed,
                                                   scales_packed, part, M, N, K, (hipStream_t)stream);
}

int w2_skinny_gemm_swiglu(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, const uint16_t* scales_packed,
                          uint16_t* a, int64_t lda, int32_t M, int32_t F, int32_t K, void* stream) {
    return sg::skinny_gemm_swiglu_run<sg::FmtW2>("w2_skinny_gemm_swiglu", x, ldx, w_packed, w_packed, scales_packed, a,
                                                 lda, M, F, K, (hipStream_t)stream);
}

}  // extern "C"
