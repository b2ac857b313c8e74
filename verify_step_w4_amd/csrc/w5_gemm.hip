// w5_gemm.hip — the skinny GEMM on W5 weights (M = 1..8): a fourth weight
// format for the verify rows (gist.science, "BaseRT: …", section "メソドロジー",
// lists the quantisation formats its GEMV reads, Q2 ... Q8).
//
// y[m][n] = sum_g scale[n][g] * sum_{k in g} x[m][k] * c[n][k],  c in [-15, 15]
//
// The code u = c + 16 is split into a 1-bit high part and a 4-bit low part.
// The low plane is stored in the W4 packed layout (w4_format.hip); the high
// plane in a 1-bit layout with the same lane mapping: per tile and K-group,
// lane l owns 8 bytes, dword d holding rows 16 nb + i of row blocks
// nb = 2 d, 2 d + 1, the bit of k = 32 s + 8 kq + j at 4 (2 (nb & 1) + s) +
// j / 2 + 16 (j % 2).  The kernel is the shared template of skinny_gemm.h
// with the W5 plane decoder (D_hi = sum x (128 + hi), D_lo = sum x (128 +
// lo): sum x c = 16 (D_hi - 137 sum x) + D_lo), and the split plan every
// format shares.  Products are exact in fp32;
// sums are fp32 in an order that depends only on (N, K): row m of an M-row
// call equals the one-row call bit for bit.
#include "skinny_formats.h"

using namespace vw4;

extern "C" {

size_t vw4_w5_workspace_bytes(int32_t M, int32_t N, int32_t K) {
    if (M < 1 || M > sg::MAX_M || N < 1 || K < 64 || K % 64 || K > 65536) return 0;
    return sg::plan_gemm(M, N, K).ws_bytes;
}

int w5_skinny_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                   const uint16_t* scales_packed, void* y, int64_t ldy, int32_t y_dtype, int32_t M, int32_t N,
                   int32_t K, void* ws, size_t ws_bytes, void* stream) {
    return sg::skinny_gemm_run<sg::FmtW5>("w5_skinny_gemm", x, ldx, w_hi, w_lo, scales_packed, y, ldy, y_dtype, M, N,
                                          K, ws, ws_bytes, (hipStream_t)stream);
}

int vw4_w5_partials_layout(int32_t M, int32_t N, int32_t K, int32_t* S, int64_t* ldp) {
    VW4_REQUIRE(M >= 1 && M <= sg::MAX_M && N >= 1 && K >= 64 && K % 64 == 0 && K <= 65536, VW4_EINVAL,
                "vw4_w5_partials_layout: bad shape M=%d N=%d K=%d", M, N, K);
    const sg::GemmPlan p = sg::plan_gemm(M, N, K);
    if (S) *S = p.S_grid;
    if (ldp) *ldp = p.Npad;
    return VW4_OK;
}

int w5_skinny_gemm_partials(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                            const uint16_t* scales_packed, float* part, int32_t M, int32_t N, int32_t K,
                            void* stream) {
    return sg::skinny_gemm_partials_run<sg::FmtW5>("w5_skinny_gemm_partials", x, ldx, w_hi, w_lo, scales_packed, part,
                                                   M, N, K, (hipStream_t)stream);
}

int w5_skinny_gemm_swiglu(const uint16_t* x, int64_t ldx, const uint8_t* w_hi, const uint8_t* w_lo,
                          const uint16_t* scales_packed, uint16_t* a, int64_t lda, int32_t M, int32_t F, int32_t K,
                          void* stream) {
    return sg::skinny_gemm_swiglu_run<sg::FmtW5>("w5_skinny_gemm_swiglu", x, ldx, w_hi, w_lo, scales_packed, a,
                                                   lda, M, F, K, (hipStream_t)stream);
}

}  // extern "C"
