// Measurement support: the ceilings this part sustains, reported beside the spec peaks so that each kernel's fraction
// can be read against both.
// - An MFMA-only loop of the FP8 block-scaled instruction. No memory traffic in the loop: each wave keeps 16
//   accumulators of 32 x 32 (the large-tile GEMM's register shape) and alternates two operand sets taken from caller
//   bytes (real quantized data toggles bits as a GEMM's operands do).
// - A streaming copy: 16-byte non-temporal loads and stores, four per thread per trip of a grid-stride loop.
#include "mxq_device.h"
#include "launch.h"

namespace mxq {

__global__ __launch_bounds__(256, 1) void mfma_probe_kernel(const uint8_t* __restrict__ ops, int64_t iters,
                                                            float* __restrict__ sink) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // 16 fragments of 32 bytes per lane: 8 per operand set, from ops[(wave * 64 + lane) * 512 ...]
    const v8i* src = reinterpret_cast<const v8i*>(ops + ((int64_t)(wave * 64 + lane)) * 512);
    v8i f[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) f[i] = src[i];
    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
    auto round = [&](int set) {                      // set is a constant after unrolling
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f[set + 4 + i], f[set + j], acc[i][j], 0, 0,
                                                                              0, 0x7F7F7F7F, 0, 0x7F7F7F7F);
    };
    int64_t it = 0;
    for (; it + 1 < iters; it += 2) {
        round(0);
        round(8);
    }
    if (it < iters) round(0);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) s += acc[i][j][e];
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

hipError_t launch_mfma_probe(const uint8_t* ops, int64_t iters, int blocks, float* sink, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ops, iters, sink);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void copy_probe_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                         int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256 * 4;
    for (int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x; i < n16; i += stride) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i + 256 * u < n16) v[u] = ldnt16(&src[i + 256 * u]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i + 256 * u < n16) stnt16(&dst[i + 256 * u], v[u]);
    }
}

hipError_t launch_copy_probe(const void* src, void* dst, int64_t bytes, int blocks, hipStream_t stream) {
    hipLaunchKernelGGL(copy_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), bytes / 16);
    return hipGetLastError();
}

}  // namespace mxq
