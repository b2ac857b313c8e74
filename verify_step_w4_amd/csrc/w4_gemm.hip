// w4_gemm.hip — W4 skinny GEMM for the verify rows (M = 1..8): the W4 entry
// points (plain, partials, grouped, SwiGLU epilogue, RMSNorm-on-load, the
// allocation-free form) and the split plan every format shares.  The kernel
// itself is the shared template of skinny_gemm.h with the W4 plane decoder.
//
// hazakura.dev, "mtplx——M5 Maxで63tok/s…", section "4層のアーキテクチャ", Layer 0:
// the verify pass is a matmul with a handful of rows (M = 3..6) that needed its
// own shader; gist.science, "BaseRT: …", section "メソドロジー": decode GEMVs
// dequantise inside the inner loop so weights are never materialised.
#include <math.h>
#include <stdlib.h>

#include <mutex>

#include "skinny_gemm.h"

namespace vw4 {

using sg::FmtW4;
using sg::GemmGroup;
using sg::GemmPlan;
using sg::NormIn;
using sg::plan_gemm;
constexpr int GEMM_MAX_M = sg::MAX_M;
constexpr int NORM_MAX_K = sg::NORM_MAX_K;

namespace sg {
// Split of K over wavefronts (every format): about 2048 wavefronts (two per SIMD), at least
// four groups per wavefront and at most 8 partial slices; one wavefront per
// workgroup, except that very wide matrices (one slice) pair two wavefronts
// per tile through LDS.  Measured on MI355X over the 27B-class shapes: more
// wavefronts only add per-wavefront start-up and partial traffic.  Depends on
// (N, K) only.  slots: matrices per launch (grouped launches spread the
// wavefront target over all of them).
GemmPlan plan_gemm(int M, int N, int K, int slots) {
    GemmPlan p;
    p.G = K / 64;
    p.ntiles = (N + 63) / 64;
    p.Npad = (int64_t)p.ntiles * 64;
    const int target_waves = 2048;
    const int units = p.ntiles * slots;
    int S = (target_waves + units - 1) / units;
    int maxS = p.G / 4 < 8 ? p.G / 4 : 8;
    if (maxS < 1) maxS = 1;
    if (S > maxS) S = maxS;
    if (S < 1) S = 1;
    p.S_wg = 1;
    p.S_grid = S;
    if (S == 1 && units >= 1024 && p.G >= 8) {
        // Many tiles, one slice each: S_wg wavefronts per workgroup split K.
        // S_wg in 2..4 is chosen so that the last round of resident workgroups
        // is as full as possible (units / resident just below a whole number):
        // the kernel holds 4 wavefronts per SIMD (16 per CU) and at most 10
        // workgroups per CU (16 KiB of static LDS each).  Measured on the
        // 151936 x 5120 LM head: 3 per workgroup (1.85 rounds) is 3-5% faster
        // than 2 (1.16 rounds) and 4 (2.32 rounds).
        const int ncu = device_cus();
        double best = -1.0;
        for (int w = 2; w <= 4; ++w) {
            const int per_cu = 16 / w < 10 ? 16 / w : 10;
            const double rounds = (double)units / ((double)per_cu * ncu);
            const double fill = rounds / ceil(rounds);
            if (fill > best + 1e-9) {
                best = fill;
                p.S_wg = w;
            }
        }
    }
    if (const char* e = getenv("VW4_GEMM_SPLIT")) {
        int a = 0, b = 0;
        if (sscanf(e, "%d,%d", &a, &b) == 2 && a >= 1 && a <= 4 && b >= 1 && a * b <= p.G) {
            p.S_wg = a;
            p.S_grid = b;
        }
    }
    p.ws_bytes = 0;
    if (p.S_grid > 1) p.ws_bytes = ((size_t)p.S_grid * M * p.Npad * 4 + 255) / 256 * 256;
    return p;
}


// SwiGLU epilogue: one slice of K per tile, S_wg wavefronts per workgroup.
// One wavefront per tile as soon as the tiles alone give one per CU: measured
// on MI355X at M = 4, gate|up 34816 x 5120 (544 tiles) takes 21.5 us with one
// wavefront per tile against 24.7 with four (the LDS reduction and the
// uneven 2-3 four-wavefront workgroups per CU cost more than the longer
// per-wavefront K stream), and the grouped 30 x 1536 x 2048 (720 tiles) 12.1
// against 15.0 with three.  Fewer tiles: up to 4 wavefronts split K.
GemmPlan plan_swiglu(int N, int K, int slots) {
    GemmPlan p;
    p.G = K / 64;
    p.ntiles = (N + 63) / 64;
    p.Npad = (int64_t)p.ntiles * 64;
    const int units = p.ntiles * slots;
    const int ncu = device_cus();
    int swg = (ncu + units - 1) / units;
    if (swg > 4) swg = 4;
    if (swg > p.G) swg = p.G;
    p.S_wg = swg < 1 ? 1 : swg;
    p.S_grid = 1;
    p.ws_bytes = 0;
    return p;
}

}  // namespace sg

template <bool NORM, bool SWIGLU>
static int launch_kernel(const GemmPlan& p, int slots, hipStream_t st, const uint16_t* x, int64_t ldx,
                         const uint8_t* w, const uint16_t* s, void* y, int64_t ldy, int ydt, int M, int N, float* part,
                         const GemmGroup& grp, const NormIn& nrm) {
    const sg::Planes P{(const sg::u32x4*)w, (const sg::u32x4*)w};
    hipLaunchKernelGGL((sg::skinny_gemm_kernel<FmtW4, NORM, SWIGLU>), dim3(p.ntiles, p.S_grid, slots),
                       dim3(64 * p.S_wg), 0, st, x, ldx, P, s, y, ldy, ydt, M, N, p.G, p.S_wg, p.S_grid, part, p.Npad,
                       0x000F000Fu, 0x43004300u, grp, nrm);
    return VW4_OK;
}

int gemm_dispatch(const uint16_t* x, int64_t ldx, const uint8_t* w, const uint16_t* s, void* y, int64_t ldy,
                  int ydt, int M, int N, int K, void* ws, size_t ws_bytes, hipStream_t st) {
    return sg::skinny_gemm_run<FmtW4>("w4_skinny_gemm", x, ldx, w, w, s, y, ldy, ydt, M, N, K, ws, ws_bytes, st);
}

// Partials form: the main kernel only (no reduction launch); part is the
// caller's [S_grid][M][Npad] fp32 buffer (per slot for grouped launches).
int gemm_partials(const uint16_t* x, int64_t ldx, const uint8_t* w, const uint16_t* s, float* part, int M, int N,
                  int K, hipStream_t st, const GemmGroup& grp = GemmGroup{}, int max_slots = 1) {
    return sg::skinny_gemm_partials_run<FmtW4>(grp.n_slots ? "w4_grouped_gemm" : "w4_skinny_gemm_partials", x, ldx,
                                               w, w, s, part, M, N, K, st, grp, max_slots);
}

// The partials form with the activations normalised on the fly:
// h = bf16(rmsnorm(resid) * gamma) (sums of squares from vw4_add_sumsq).
int gemm_rmsnorm_partials(const uint16_t* resid, const uint16_t* gamma, const float* ssq, float eps,
                          const uint8_t* w, const uint16_t* s, float* part, int M, int N, int K, hipStream_t st) {
    VW4_REQUIRE(M >= 1 && M <= GEMM_MAX_M && N >= 1 && K >= 64 && K % 64 == 0 && K <= NORM_MAX_K, VW4_EINVAL,
                "w4_skinny_gemm_rmsnorm_partials: bad shape M=%d N=%d K=%d (K <= %d)", M, N, K, NORM_MAX_K);
    VW4_REQUIRE(resid && gamma && ssq && w && s && part, VW4_EINVAL, "w4_skinny_gemm_rmsnorm_partials: null pointer");
    VW4_REQUIRE(aligned(resid, 16) && aligned(gamma, 16) && aligned(w, 16) && aligned(s, 8) && aligned(part, 4),
                VW4_EINVAL, "w4_skinny_gemm_rmsnorm_partials: misaligned pointer");
    VW4_REQUIRE(eps >= 0.0f, VW4_EINVAL, "w4_skinny_gemm_rmsnorm_partials: eps must be >= 0");
    const GemmPlan p = plan_gemm(M, N, K);
    const NormIn nrm{resid, gamma, ssq, (K + NORM_CHUNK - 1) / NORM_CHUNK, eps};
    const int rc = launch_kernel<true, false>(p, 1, st, nullptr, K, w, s, part, p.Npad, VW4_F32, M, N, part,
                                              GemmGroup{}, nrm);
    if (rc) return rc;
    return check_launch("w4_skinny_gemm_rmsnorm_partials");
}

int gemm_swiglu(const uint16_t* x, int64_t ldx, const NormIn* nrm, const uint8_t* w, const uint16_t* s, uint16_t* a,
                int64_t lda, int M, int F, int K, hipStream_t st, const GemmGroup& grp, int slots) {
    VW4_REQUIRE(M >= 1 && M <= GEMM_MAX_M && F >= 32 && F % 32 == 0 && K >= 64 && K % 64 == 0 && K <= 65536,
                VW4_EINVAL, "w4 GEMM + SwiGLU: bad shape M=%d F=%d K=%d (F must be a multiple of 32)", M, F, K);
    VW4_REQUIRE(w && s && a && lda >= F, VW4_EINVAL, "w4 GEMM + SwiGLU: bad output or null pointer");
    VW4_REQUIRE(aligned(w, 16) && aligned(s, 8) && aligned(a, 2), VW4_EINVAL, "w4 GEMM + SwiGLU: misaligned pointer");
    const GemmPlan p = sg::plan_swiglu(2 * F, K, slots);
    int rc;
    if (nrm) {
        VW4_REQUIRE(nrm->resid && nrm->gamma && nrm->ssq && aligned(nrm->resid, 16) && aligned(nrm->gamma, 16),
                    VW4_EINVAL, "w4 GEMM + SwiGLU: bad normalisation inputs");
        VW4_REQUIRE(K <= NORM_MAX_K, VW4_EINVAL, "w4 GEMM + SwiGLU: normalised rows need K <= %d", NORM_MAX_K);
        rc = launch_kernel<true, true>(p, slots, st, nullptr, K, w, s, a, lda, VW4_BF16, M, 2 * F, nullptr, grp,
                                       *nrm);
    } else {
        VW4_REQUIRE(x && ldx >= K && ldx % 8 == 0 && aligned(x, 16), VW4_EINVAL,
                    "w4 GEMM + SwiGLU: x needs ldx >= K, ldx %% 8 == 0 and 16-byte alignment");
        rc = launch_kernel<false, true>(p, slots, st, x, ldx, w, s, a, lda, VW4_BF16, M, 2 * F, nullptr, grp,
                                        NormIn{});
    }
    if (rc) return rc;
    return check_launch("w4 GEMM + SwiGLU");
}

int grouped_gemm_partials(const uint16_t* x, int64_t ldx, int64_t x_sstride, const uint8_t* w_bank,
                          int64_t w_estride_bytes, const uint16_t* s_bank, int64_t s_estride, const int32_t* slot_expert,
                          const int32_t* n_slots, int max_slots, float* part, int64_t p_sstride, int M, int N, int K,
                          hipStream_t st) {
    VW4_REQUIRE(slot_expert && n_slots && max_slots >= 1 && max_slots <= 65535, VW4_EINVAL,
                "w4_grouped_gemm: bad slot arguments");
    VW4_REQUIRE(w_estride_bytes % 16 == 0 && w_estride_bytes > 0 && s_estride > 0 && s_estride % 4 == 0, VW4_EINVAL,
                "w4_grouped_gemm: expert strides must be positive, weights 16-byte and scales 8-byte multiples");
    VW4_REQUIRE(x_sstride % 8 == 0 && x_sstride >= 0 && p_sstride >= 0, VW4_EINVAL,
                "w4_grouped_gemm: bad slot strides");
    GemmGroup g{};
    g.slot_expert = slot_expert;
    g.n_slots = n_slots;
    g.w_estride = w_estride_bytes / 16;
    g.s_estride = s_estride;
    g.x_sstride = x_sstride;
    g.p_sstride = p_sstride;
    return gemm_partials(x, ldx, w_bank, s_bank, part, M, N, K, st, g, max_slots);
}

int gemm_layout(int M, int N, int K, int* S, int64_t* ldp, int slots = 1) {
    VW4_REQUIRE(M >= 1 && M <= GEMM_MAX_M && N >= 1 && K >= 64 && K % 64 == 0 && K <= 65536, VW4_EINVAL,
                "vw4_gemm_partials_layout: bad shape M=%d N=%d K=%d", M, N, K);
    VW4_REQUIRE(slots >= 1 && slots <= 65535, VW4_EINVAL, "vw4_grouped_gemm_layout: max_slots=%d", slots);
    const GemmPlan p = plan_gemm(M, N, K, slots);
    if (S) *S = p.S_grid;
    if (ldp) *ldp = p.Npad;
    return VW4_OK;
}

size_t gemm_ws_bytes(int M, int N, int K) {
    if (M < 1 || M > GEMM_MAX_M || N < 1 || K < 64 || K % 64) return 0;
    return plan_gemm(M, N, K).ws_bytes;
}

}  // namespace vw4

extern "C" {

size_t vw4_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K) { return vw4::gemm_ws_bytes(M, N, K); }

int vw4_gemm_partials_layout(int32_t M, int32_t N, int32_t K, int32_t* S, int64_t* ldp) {
    int s = 0;
    int rc = vw4::gemm_layout(M, N, K, &s, ldp);
    if (S) *S = s;
    return rc;
}

int vw4_grouped_gemm_layout(int32_t M, int32_t N, int32_t K, int32_t max_slots, int32_t* S, int64_t* ldp) {
    int s = 0;
    int rc = vw4::gemm_layout(M, N, K, &s, ldp, max_slots);
    if (S) *S = s;
    return rc;
}

int w4_grouped_gemm(const uint16_t* x, int64_t ldx, int64_t x_sstride, const uint8_t* w_bank, int64_t w_estride,
                    const uint16_t* s_bank, int64_t s_estride, const int32_t* slot_expert, const int32_t* n_slots,
                    int32_t max_slots, float* part, int64_t p_sstride, int32_t M, int32_t N, int32_t K, void* stream) {
    if (max_slots >= 1 && max_slots <= 65535 && M >= 1 && M <= vw4::GEMM_MAX_M && N >= 1 && K >= 64 && K % 64 == 0) {
        int S = 0;
        int64_t ldp = 0;
        vw4::gemm_layout(M, N, K, &S, &ldp, max_slots);
        VW4_REQUIRE(p_sstride >= (int64_t)S * M * ldp, VW4_EINVAL,
                    "w4_grouped_gemm: p_sstride %lld < S * M * ldp = %lld", (long long)p_sstride,
                    (long long)((int64_t)S * M * ldp));
    }
    return vw4::grouped_gemm_partials(x, ldx, x_sstride, w_bank, w_estride, s_bank, s_estride, slot_expert, n_slots,
                                      max_slots, part, p_sstride, M, N, K, (hipStream_t)stream);
}

int w4_skinny_gemm_rmsnorm_partials(const uint16_t* resid, const uint16_t* gamma, const void* norm_ws, float eps,
                                    const uint8_t* w_packed, const uint16_t* scales_packed, float* part, int32_t M,
                                    int32_t N, int32_t K, void* stream) {
    return vw4::gemm_rmsnorm_partials(resid, gamma, (const float*)norm_ws, eps, w_packed, scales_packed, part, M, N,
                                      K, (hipStream_t)stream);
}

int w4_skinny_gemm_rmsnorm_swiglu(const uint16_t* resid, const uint16_t* gamma, const void* norm_ws, float eps,
                                  const uint8_t* w_packed, const uint16_t* scales_packed, uint16_t* a, int64_t lda,
                                  int32_t M, int32_t F, int32_t K, void* stream) {
    const vw4::NormIn nrm{resid, gamma, (const float*)norm_ws, (K + vw4::NORM_CHUNK - 1) / vw4::NORM_CHUNK, eps};
    VW4_REQUIRE(eps >= 0.0f, VW4_EINVAL, "w4_skinny_gemm_rmsnorm_swiglu: eps must be >= 0");
    return vw4::gemm_swiglu(nullptr, K, &nrm, w_packed, scales_packed, a, lda, M, F, K, (hipStream_t)stream,
                            vw4::GemmGroup{}, 1);
}

int w4_skinny_gemm_swiglu(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, const uint16_t* scales_packed,
                          uint16_t* a, int64_t lda, int32_t M, int32_t F, int32_t K, void* stream) {
    return vw4::gemm_swiglu(x, ldx, nullptr, w_packed, scales_packed, a, lda, M, F, K, (hipStream_t)stream,
                            vw4::GemmGroup{}, 1);
}

int w4_grouped_gemm_swiglu(const uint16_t* x, int64_t ldx, int64_t x_sstride, const uint8_t* w_bank,
                           int64_t w_estride, const uint16_t* s_bank, int64_t s_estride, const int32_t* slot_expert,
                           const int32_t* n_slots, int32_t max_slots, uint16_t* a, int64_t a_sstride, int32_t M,
                           int32_t F, int32_t K, void* stream) {
    VW4_REQUIRE(slot_expert && n_slots && max_slots >= 1 && max_slots <= 65535, VW4_EINVAL,
                "w4_grouped_gemm_swiglu: bad slot arguments");
    VW4_REQUIRE(w_estride % 16 == 0 && w_estride > 0 && s_estride > 0 && s_estride % 4 == 0, VW4_EINVAL,
                "w4_grouped_gemm_swiglu: expert strides must be positive, weights 16-byte and scales 8-byte multiples");
    VW4_REQUIRE(x_sstride % 8 == 0 && x_sstride >= 0 && a_sstride >= (int64_t)M * F, VW4_EINVAL,
                "w4_grouped_gemm_swiglu: bad slot strides");
    vw4::GemmGroup g{};
    g.slot_expert = slot_expert;
    g.n_slots = n_slots;
    g.w_estride = w_estride / 16;
    g.s_estride = s_estride;
    g.x_sstride = x_sstride;
    g.y_sstride = a_sstride;
    return vw4::gemm_swiglu(x, ldx, nullptr, w_bank, s_bank, a, F, M, F, K, (hipStream_t)stream, g, max_slots);
}

int w4_skinny_gemm_partials(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, const uint16_t* scales_packed,
                            float* part, int32_t M, int32_t N, int32_t K, void* stream) {
    return vw4::gemm_partials(x, ldx, w_packed, scales_packed, part, M, N, K, (hipStream_t)stream);
}

int w4_skinny_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, const uint16_t* scales_packed, void* y,
                   int64_t ldy, int32_t y_dtype, int32_t M, int32_t N, int32_t K, void* ws, size_t ws_bytes,
                   void* stream) {
    return vw4::gemm_dispatch(x, ldx, w_packed, scales_packed, y, ldy, y_dtype, M, N, K, ws, ws_bytes,
                              (hipStream_t)stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The allocation-free form of w4_skinny_gemm.  Its split-K partial sums live
// in a file-scope device array instead of a caller workspace: every GPU the
// library runs on holds one copy of VW4_NOALLOC_SCRATCH_BYTES until the
// process ends.  The largest split-K workspace the plan asks for at M <= 8 is
// 8 * 8 * 32768 * 4 bytes (S * Npad stays below 4096 * 64), so every shape
// the plan produces fits.  Host code never passes the array's name to a
// kernel: it is a host-side stand-in; the device address of each GPU's copy
// comes from hipGetSymbolAddress, taken once per device on the first call
// made with that device current.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[VW4_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex noalloc_mu;
void* noalloc_ptr[NOALLOC_MAX_DEVICES];

// Device address of the current device's scratch copy, or nullptr (with the
// error message set) if it cannot be had.
void* noalloc_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) {
        vw4::set_error("w4_skinny_gemm_noalloc: no current device (or device index >= %d)", NOALLOC_MAX_DEVICES);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(noalloc_mu);
    if (!noalloc_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            vw4::set_error("w4_skinny_gemm_noalloc: hipGetSymbolAddress of the scratch array failed on device %d: %s",
                           dev, hipGetErrorString(e));
            return nullptr;
        }
        noalloc_ptr[dev] = p;
    }
    return noalloc_ptr[dev];
}
}  // namespace

extern "C" {

size_t vw4_noalloc_scratch_bytes(void) { return VW4_NOALLOC_SCRATCH_BYTES; }

int w4_skinny_gemm_noalloc(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, const uint16_t* scales_packed,
                           void* y, int64_t ldy, int32_t y_dtype, int32_t M, int32_t N, int32_t K, void* stream) {
    const size_t need = vw4::gemm_ws_bytes(M, N, K);
    VW4_REQUIRE(need <= VW4_NOALLOC_SCRATCH_BYTES, VW4_EWORKSPACE,
                "w4_skinny_gemm_noalloc: the split-K partials need %zu bytes, more than the %zu-byte scratch array",
                need, (size_t)VW4_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (need) {
        ws = noalloc_scratch();
        if (!ws) return VW4_EHIP;
    }
    return vw4::gemm_dispatch(x, ldx, w_packed, scales_packed, y, ldy, y_dtype, M, N, K, ws,
                              need ? (size_t)VW4_NOALLOC_SCRATCH_BYTES : 0, (hipStream_t)stream);
}

}  // extern "C"
