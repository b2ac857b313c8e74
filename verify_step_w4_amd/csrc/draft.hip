// draft.hip — the inputs of the draft side of the cycle: token embedding rows
// (the target's verify rows) and the MTP head's projection input.
//
// hazakura.dev mtplx page, section "4層のアーキテクチャ", Layer 1: the drafter
// is the MTP head inside the same checkpoint, and Layer 2: each cycle drafts,
// then verifies.  The pages do not describe the head's inside; the common MTP
// head is used: the hidden row of the last processed position and the
// embedding of the next token, each RMS-normalised with its own gain,
// concatenated [h ; e] and projected back to the model width by a W4 matrix.
#include "common.h"

namespace vw4 {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4d;

// grid (n), 256 threads: row i of out = E[tokens[i]] (16-byte pieces), or
// zeros for an id outside [0, V).
__global__ __launch_bounds__(256) void embed_rows_kernel(const uint16_t* __restrict__ E, int64_t lde, int V, int d,
                                                         const int32_t* __restrict__ tokens,
                                                         uint16_t* __restrict__ out, int64_t ldo) {
    const int i = blockIdx.x;
    const int t = tokens[i];
    const bool ok = t >= 0 && t < V;
    const u32x4d* src = (const u32x4d*)(E + (int64_t)(ok ? t : 0) * lde);
    u32x4d* dst = (u32x4d*)(out + (int64_t)i * ldo);
    const u32x4d zero = {0u, 0u, 0u, 0u};
    for (int c = threadIdx.x; c < d / 8; c += 256) dst[c] = ok ? src[c] : zero;
}

constexpr int MI_THREADS = 256;
constexpr int MI_MAXV = 4;     // 16-byte pieces per thread: d <= 8 * 256 * 4 = 8192

// grid (2), 256 threads.  Workgroup 0 normalises the hidden row h[*h_row]
// (clamped to [0, h_rows)) with gamma_h into out[0:d]; workgroup 1 the
// embedding row E[*token] (zeros for an id outside [0, V)) with gamma_e into
// out[d:2d].  y = bf16(x * (1 / sqrt(mean(x^2) + eps)) * gamma), the sum of
// squares in fp32 per thread, then per wavefront, then in wavefront order.
__global__ __launch_bounds__(MI_THREADS) void mtp_input_kernel(
    const uint16_t* __restrict__ h, int64_t ldh, int h_rows, const int32_t* __restrict__ h_row,
    const uint16_t* __restrict__ E, int64_t lde, int V, const int32_t* __restrict__ token,
    const uint16_t* __restrict__ gamma_h, const uint16_t* __restrict__ gamma_e, float eps, int d,
    uint16_t* __restrict__ out) {
    __shared__ float s_w[MI_THREADS / 64];
    const int half = blockIdx.x, tid = threadIdx.x;
    const uint16_t* src;
    const uint16_t* gam;
    bool live = true;
    if (half == 0) {
        int r = h_row ? *h_row : 0;
        r = r < 0 ? 0 : (r >= h_rows ? h_rows - 1 : r);
        src = h + (int64_t)r * ldh;
        gam = gamma_h;
    } else {
        const int t = *token;
        live = t >= 0 && t < V;
        src = E + (int64_t)(live ? t : 0) * lde;
        gam = gamma_e;
    }
    const int nv = d / 8;
    u32x4d v[MI_MAXV], g[MI_MAXV];
#pragma unroll
    for (int k = 0; k < MI_MAXV; ++k) {
        const int c = tid + k * MI_THREADS;
        const int cc = c < nv ? c : nv - 1;     // clamped: every load issued, no branch between them
        v[k] = ((const u32x4d*)src)[cc];
        g[k] = ((const u32x4d*)gam)[cc];
    }
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < MI_MAXV; ++k) {
        const bool use = live && tid + k * MI_THREADS < nv;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float a = bf16_to_f32((uint16_t)(v[k][w] & 0xffffu)), b = bf16_to_f32((uint16_t)(v[k][w] >> 16));
            ss += use ? fmaf(a, a, b * b) : 0.0f;
        }
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) s_w[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.0f;
#pragma unroll
    for (int w = 0; w < MI_THREADS / 64; ++w) tot += s_w[w];
    const float inv = 1.0f / sqrtf(tot / (float)d + eps);
    u32x4d* dst = (u32x4d*)(out + (int64_t)half * d);
#pragma unroll
    for (int k = 0; k < MI_MAXV; ++k) {
        const int c = tid + k * MI_THREADS;
        if (c >= nv) break;
        u32x4d o;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float a = bf16_to_f32((uint16_t)(v[k][w] & 0xffffu)), b = bf16_to_f32((uint16_t)(v[k][w] >> 16));
            if (!live) a = b = 0.0f;
            const float ga = bf16_to_f32((uint16_t)(g[k][w] & 0xffffu)), gb = bf16_to_f32((uint16_t)(g[k][w] >> 16));
            o[w] = (uint32_t)f32_to_bf16(a * inv * ga) | ((uint32_t)f32_to_bf16(b * inv * gb) << 16);
        }
        dst[c] = o;
    }
}

}  // namespace vw4

using namespace vw4;

extern "C" {

int vw4_embed_rows(const uint16_t* E, int64_t lde, int32_t V, int32_t d, const int32_t* tokens, int32_t n,
                   uint16_t* out, int64_t ldo, void* stream) {
    VW4_REQUIRE(E && tokens && out, VW4_EINVAL, "vw4_embed_rows: null pointer");
    VW4_REQUIRE(V >= 1 && d >= 8 && d % 8 == 0 && n >= 1 && n <= 65535 && lde >= d && ldo >= d && lde % 8 == 0 &&
                    ldo % 8 == 0,
                VW4_EINVAL, "vw4_embed_rows: need d %% 8 == 0, 1 <= n <= 65535, strides >= d and multiples of 8");
    VW4_REQUIRE(aligned(E, 16) && aligned(out, 16) && aligned(tokens, 4), VW4_EINVAL,
                "vw4_embed_rows: E and out need 16-byte alignment");
    hipLaunchKernelGGL(embed_rows_kernel, dim3(n), dim3(256), 0, (hipStream_t)stream, E, lde, V, d, tokens, out, ldo);
    return check_launch("vw4_embed_rows");
}

int vw4_mtp_input(const uint16_t* h, int64_t ldh, int32_t h_rows, const int32_t* h_row, const uint16_t* E,
                  int64_t lde, int32_t V, const int32_t* token, const uint16_t* gamma_h, const uint16_t* gamma_e,
                  float eps, int32_t d, uint16_t* out, void* stream) {
    VW4_REQUIRE(h && E && token && gamma_h && gamma_e && out, VW4_EINVAL, "vw4_mtp_input: null pointer");
    VW4_REQUIRE(d >= 8 && d % 8 == 0 && d <= 8 * MI_THREADS * MI_MAXV && h_rows >= 1 && V >= 1 && ldh >= d &&
                    lde >= d && ldh % 8 == 0 && lde % 8 == 0,
                VW4_EINVAL, "vw4_mtp_input: need d %% 8 == 0, 8 <= d <= %d, strides >= d and multiples of 8 (d=%d)",
                8 * MI_THREADS * MI_MAXV, d);
    VW4_REQUIRE(aligned(h, 16) && aligned(E, 16) && aligned(gamma_h, 16) && aligned(gamma_e, 16) &&
                    aligned(out, 16),
                VW4_EINVAL, "vw4_mtp_input: h, E, gains and out need 16-byte alignment");
    VW4_REQUIRE(eps >= 0.0f, VW4_EINVAL, "vw4_mtp_input: eps must be >= 0");
    hipLaunchKernelGGL(mtp_input_kernel, dim3(2), dim3(MI_THREADS), 0, (hipStream_t)stream, h, ldh, h_rows, h_row, E,
                       lde, V, token, gamma_h, gamma_e, eps, d, out);
    return check_launch("vw4_mtp_input");
}

}  // extern "C"
