// Measurement support library (libmxq_probe.so, C ABI in include/mxq_probe.h): the ceilings this part sustains,
// reported beside the spec peaks so that each kernel's fraction can be read against both. It is not a step of the
// method and is built apart from libmxq.so.
// - An MFMA-only loop of the FP8 block-scaled instruction. No memory traffic in the loop: each wave keeps 16
//   accumulators of 32 x 32 (the large-tile GEMM's register shape) and alternates two operand sets taken from caller
//   bytes (real quantized data toggles bits as a GEMM's operands do).
// - A streaming copy and a streaming read: 16-byte non-temporal accesses, 4, 8 or 16 loads in flight per thread, over
//   a fixed grid that loops or over one workgroup per piece of the data.
// - A streaming read into LDS with the large-tile GEMM's copy instruction (buffer_load_dwordx4 ... lds), so that the
//   hardware counters' bytes per byte of that load path can be read off a transfer of known size.
#include <stdint.h>

#include "mxq_device.h"
#include "mxq_probe.h"

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

static hipError_t launch_mfma_probe(const uint8_t* ops, int64_t iters, int blocks, float* sink, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ops, iters, sink);
    return hipGetLastError();
}

// Copy: thread t of workgroup w handles the 16-byte chunks w * 256 U + t + 256 u (u < U), all U loads issued before
// the first store; LOOP makes the grid stride over the data (a fixed grid), otherwise one workgroup per 256 U chunks.
template <int U, bool LOOP>
__global__ __launch_bounds__(256) void copy_probe_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                         int64_t n16) {
    const int64_t stride = LOOP ? (int64_t)gridDim.x * 256 * U : n16;
    for (int64_t i = (int64_t)blockIdx.x * 256 * U + threadIdx.x; i < n16; i += stride) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i + 256 * u < n16) v[u] = ldnt16(&src[i + 256 * u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i + 256 * u < n16) stnt16(&dst[i + 256 * u], v[u]);
    }
}

// Read: the same walk with loads only; the xor of the words read leaves the workgroup as one 4-byte store, so the
// loads cannot be dropped and the stores add no measurable traffic.
template <int U, bool LOOP>
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
    __shared__ uint32_t part[4];
    const int64_t stride = LOOP ? (int64_t)gridDim.x * 256 * U : n16;
    uint32_t x = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 * U + threadIdx.x; i < n16; i += stride) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i + 256 * u < n16) v[u] = ldnt16(&src[i + 256 * u]);
            else v[u] = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// Read into LDS: workgroup w streams the 64 KiB pieces w, w + gridDim.x, ... Each wave moves its 16 KiB of a piece
// with 16 instructions that each land 1 KiB (lane l's 16 bytes at slot l), waits for them, then reads its own slots
// back and xors every word into the workgroup's sink word, so every byte is used and the result can be checked.
typedef int v4i __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256, 1) void read_lds_probe_kernel(const uint8_t* __restrict__ src, int64_t pieces,
                                                                uint32_t* __restrict__ sink) {
    __shared__ __attribute__((aligned(16))) uint4 buf[4096];          // 64 KiB: 16 KiB per wave
    __shared__ uint32_t part[4];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(&buf[wave * 1024]));
    uint32_t x = 0;
    for (int64_t p = blockIdx.x; p < pieces; p += gridDim.x) {
        const uint64_t base = reinterpret_cast<uint64_t>(src + p * 65536);
        const v4i rsrc = v4i{(int)__builtin_amdgcn_readfirstlane((uint32_t)base),
                             (int)(__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)) & 0xFFFFu), 65536,
                             0x00020000};
        const int voff = wave * 16384 + lane * 16;
        // the previous piece's reads of these slots have returned before the slots are refilled
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int c = 0; c < 16; ++c)
            asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                         :: "v"(voff + 1024 * c), "s"(rsrc), "{m0}"(lds0 + 1024 * c) : "memory");
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const uint4 v = buf[wave * 1024 + c * 64 + lane];
            x ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off, 64);
    if (lane == 0) part[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

template <int U>
static hipError_t launch_copy_u(const void* src, void* dst, int64_t n16, int blocks, hipStream_t stream) {
    const uint4* s = static_cast<const uint4*>(src);
    uint4* d = static_cast<uint4*>(dst);
    if (blocks > 0)
        hipLaunchKernelGGL((copy_probe_kernel<U, true>), dim3((unsigned)blocks), dim3(256), 0, stream, s, d, n16);
    else
        hipLaunchKernelGGL((copy_probe_kernel<U, false>), dim3((unsigned)((n16 + 256 * U - 1) / (256 * U))), dim3(256),
                           0, stream, s, d, n16);
    return hipGetLastError();
}

template <int U>
static hipError_t launch_read_u(const void* src, int64_t n16, int blocks, uint32_t* sink, hipStream_t stream) {
    const uint4* s = static_cast<const uint4*>(src);
    if (blocks > 0)
        hipLaunchKernelGGL((read_probe_kernel<U, true>), dim3((unsigned)blocks), dim3(256), 0, stream, s, n16, sink);
    else
        hipLaunchKernelGGL((read_probe_kernel<U, false>), dim3((unsigned)((n16 + 256 * U - 1) / (256 * U))), dim3(256),
                           0, stream, s, n16, sink);
    return hipGetLastError();
}

static hipError_t launch_read_lds(const void* src, int64_t pieces, int blocks, uint32_t* sink, hipStream_t stream) {
    hipLaunchKernelGGL(read_lds_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(src), pieces, sink);
    return hipGetLastError();
}

}  // namespace mxq

extern "C" {

mxq_status mxq_probe_mfma_fp8(const uint8_t* operand_bytes, int64_t iters, int64_t blocks, float* sink,
                              hipStream_t stream) {
    if (!operand_bytes || !sink) return MXQ_ERR_NULL;
    if (iters < 1 || blocks < 1 || blocks > 65536) return MXQ_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(operand_bytes) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u))
        return MXQ_ERR_ALIGN;
    return mxq::launch_mfma_probe(operand_bytes, iters, (int)blocks, sink, stream) == hipSuccess ? MXQ_OK
                                                                                                  : MXQ_ERR_HIP;
}

// Full-grid launches need (n16 + 256 U - 1) / (256 U) workgroups, below 2^31.
static bool probe_grid_ok(int64_t bytes, int64_t blocks, int64_t unroll) {
    if (blocks < 0 || blocks > 65536 || (unroll != 4 && unroll != 8 && unroll != 16)) return false;
    return blocks > 0 || bytes / 16 / (256 * unroll) < 0x7FFFFFFF;
}

mxq_status mxq_probe_copy(const void* src, void* dst, int64_t bytes, int64_t blocks, int64_t unroll,
                          hipStream_t stream) {
    if (bytes < 0 || (bytes & 15) || !probe_grid_ok(bytes, blocks, unroll)) return MXQ_ERR_SHAPE;
    if (bytes > 0 && (!src || !dst)) return MXQ_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(dst) & 15u)) return MXQ_ERR_ALIGN;
    if (bytes == 0) return MXQ_OK;
    const int64_t n16 = bytes / 16;
    hipError_t e = unroll == 4 ? mxq::launch_copy_u<4>(src, dst, n16, (int)blocks, stream)
                 : unroll == 8 ? mxq::launch_copy_u<8>(src, dst, n16, (int)blocks, stream)
                               : mxq::launch_copy_u<16>(src, dst, n16, (int)blocks, stream);
    return e == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

mxq_status mxq_probe_read(const void* src, int64_t bytes, int64_t blocks, int64_t unroll, uint32_t* sink,
                          hipStream_t stream) {
    if (bytes < 0 || (bytes & 15) || !probe_grid_ok(bytes, blocks, unroll)) return MXQ_ERR_SHAPE;
    if (!sink || (bytes > 0 && !src)) return MXQ_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return MXQ_ERR_ALIGN;
    if (bytes == 0) return MXQ_OK;
    const int64_t n16 = bytes / 16;
    hipError_t e = unroll == 4 ? mxq::launch_read_u<4>(src, n16, (int)blocks, sink, stream)
                 : unroll == 8 ? mxq::launch_read_u<8>(src, n16, (int)blocks, sink, stream)
                               : mxq::launch_read_u<16>(src, n16, (int)blocks, sink, stream);
    return e == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

mxq_status mxq_probe_read_lds(const void* src, int64_t bytes, int64_t blocks, uint32_t* sink, hipStream_t stream) {
    if (bytes < 0 || bytes % 65536 != 0 || blocks < 1 || blocks > 65536) return MXQ_ERR_SHAPE;
    if (!sink || (bytes > 0 && !src)) return MXQ_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return MXQ_ERR_ALIGN;
    return mxq::launch_read_lds(src, bytes / 65536, (int)blocks, sink, stream) == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

}  // extern "C"
