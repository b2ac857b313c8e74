// stream_read.hip — the plain streaming-read ceiling of the part.
//
// gist.science, "BaseRT: …", section "結果" (and qiita.com, "Apple Silicon向け
// LLM推論エンジンを開発して…", section "開発の背景"): decode of a large model is
// bound by memory bandwidth.  The W4 GEMM's achieved bandwidth is judged
// against the chip's published HBM peak and against what a kernel that only
// reads can reach on the same part; this call is that kernel.  Each thread
// reads 16-byte words with non-temporal loads in a grid-stride loop and XORs
// them; each workgroup writes the XOR of its threads' words, so the result
// can be checked and the loads cannot be dropped.
#include "common.h"

namespace vw4 {

typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4s* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    u32x4s a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // two loads in flight per thread per trip
    for (; j + nth < n16; j += 2 * nth) {
        a ^= __builtin_nontemporal_load(src + j);
        b ^= __builtin_nontemporal_load(src + j + nth);
    }
    if (j < n16) a ^= __builtin_nontemporal_load(src + j);
    a ^= b;
    uint32_t v = a.x ^ a.y ^ a.z ^ a.w;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v ^= (uint32_t)__shfl_xor((int)v, off, 64);
    __shared__ uint32_t wsum[4];
    const int wv = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) wsum[wv] = v;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = wsum[0] ^ wsum[1] ^ wsum[2] ^ wsum[3];
}

}  // namespace vw4

extern "C" int vw4_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, void* stream) {
    VW4_REQUIRE(src && sink, VW4_EINVAL, "vw4_stream_read: null pointer");
    VW4_REQUIRE(bytes >= 16 && bytes % 16 == 0 && vw4::aligned(src, 16), VW4_EINVAL,
                "vw4_stream_read: bytes must be a positive multiple of 16 and src 16-byte aligned");
    VW4_REQUIRE(blocks >= 1 && blocks <= (1 << 20), VW4_EINVAL, "vw4_stream_read: blocks=%d not in [1, 2^20]", blocks);
    hipLaunchKernelGGL(vw4::stream_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (const vw4::u32x4s*)src, (int64_t)(bytes / 16), sink);
    return vw4::check_launch("vw4_stream_read");
}
