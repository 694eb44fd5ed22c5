// The single-GPU parts of the FP8 gradient all-reduce ("FP8-LM: Training FP8 Large Language Models", Section 3.4:
// the automatic scaling factor mu of Eq. 3 and the shared scaling factor of Eq. 4-6). Both are HBM-bound streams.
//
// Auto-scaled cast: g' = mu * g (one fp32 rounding), q = FP8(g') with saturation; the tensor's scale is mu. The codes
// at the format's maximum magnitude are counted (one 64-bit vector atomic add per workgroup); a one-thread finalize
// halves mu when their fraction exceeds 0.001 % and otherwise multiplies it by 2^(1/1000).
// Shared-scale requantize: s_g = min of the scales gathered from the ranks; every code is decoded, divided by its own
// scale, multiplied by s_g and re-encoded, each an fp32 rounding; the sum of N such tensors carries the scale N s_g.
#pragma clang fp contract(off)
#include "mxq_device.h"
#include "launch.h"

namespace mxq {

constexpr int GC_THREADS = 256;

template <int FMT>
__device__ __forceinline__ uint32_t fp8_max_code() { return FMT == FMT_E4M3 ? 0x7Eu : 0x7Bu; }

// ---------------------------------------------------------------------------------------- auto-scaled cast
__global__ void autoscale_prep_kernel(unsigned long long* __restrict__ count) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *count = 0ull;
}

template <int FMT>
__device__ __forceinline__ uint32_t cast_quad(float m, uint32_t p0, uint32_t p1, uint32_t& cnt) {
    constexpr float FMAX = FMT == FMT_E4M3 ? 448.0f : 57344.0f;
    const float a = clamp_keep_nan(bf16_lo(p0) * m, FMAX), b = clamp_keep_nan(bf16_hi(p0) * m, FMAX);
    const float c = clamp_keep_nan(bf16_lo(p1) * m, FMAX), d = clamp_keep_nan(bf16_hi(p1) * m, FMAX);
    const uint32_t w = cvt_f32_pair<FMT, true>(cvt_f32_pair<FMT, false>(0u, a, b), c, d);
#pragma unroll
    for (int e = 0; e < 4; ++e) cnt += ((w >> (8 * e)) & 0x7Fu) == fp8_max_code<FMT>() ? 1u : 0u;
    return w;
}

template <int FMT>
__global__ __launch_bounds__(GC_THREADS) void autoscale_cast_kernel(const uint16_t* __restrict__ g, int64_t n,
                                                                   const float* __restrict__ mu,
                                                                   uint8_t* __restrict__ q,
                                                                   unsigned long long* __restrict__ count) {
    __shared__ uint32_t red[GC_THREADS / 64];
    const float m = *mu;
    uint32_t cnt = 0;
    const int64_t chunks = n / 8, stride = (int64_t)gridDim.x * GC_THREADS;
    for (int64_t i = (int64_t)blockIdx.x * GC_THREADS + threadIdx.x; i < chunks; i += stride) {
        const uint4 v = ldnt16(g + 8 * i);
        const uint32_t lo = cast_quad<FMT>(m, v.x, v.y, cnt);
        const uint32_t hi = cast_quad<FMT>(m, v.z, v.w, cnt);
        stnt8(q + 8 * i, make_uint2(lo, hi));
    }
    if (blockIdx.x == 0) {
        for (int64_t i = chunks * 8 + threadIdx.x; i < n; i += GC_THREADS) {
            uint32_t c = 0;
            const uint32_t w = cast_quad<FMT>(m, (uint32_t)g[i], 0u, c);
            cnt += ((w & 0x7Fu) == fp8_max_code<FMT>()) ? 1u : 0u;
            q[i] = (uint8_t)(w & 0xFFu);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += (uint32_t)__shfl_xor((int)cnt, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long t = 0;
        for (int w = 0; w < GC_THREADS / 64; ++w) t += red[w];
        if (t) atomicAdd(count, t);
    }
}

__global__ void autoscale_finalize_kernel(const unsigned long long* __restrict__ count, int64_t n,
                                          float* __restrict__ mu, float* __restrict__ scale_out,
                                          unsigned long long* __restrict__ overflow_out) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        const float m = *mu;
        const unsigned long long c = *count;
        const double ratio = n > 0 ? (double)c / (double)n : 0.0;
        const float up = __uint_as_float(0x3F8016B9u);            // 2^(1/1000) rounded to fp32
        *mu = ratio > 1e-5 ? m * 0.5f : m * up;
        if (scale_out) *scale_out = m;
        *overflow_out = c;
    }
}

hipError_t launch_autoscale_cast(const uint16_t* g, int64_t n, int fmt, float* mu, uint8_t* q, float* scale_out,
                                 unsigned long long* overflow, unsigned long long* count, hipStream_t stream) {
    // one 8-value chunk per thread over a full grid (measured faster than a looping grid of 4096 workgroups)
    int64_t blocks = (n / 8 + GC_THREADS - 1) / GC_THREADS;
    if (blocks < 1) blocks = 1;
    if (blocks > (int64_t(1) << 30)) blocks = int64_t(1) << 30;
    hipLaunchKernelGGL(autoscale_prep_kernel, dim3(1), dim3(64), 0, stream, count);
    if (fmt == FMT_E4M3)
        hipLaunchKernelGGL(autoscale_cast_kernel<FMT_E4M3>, dim3((unsigned)blocks), dim3(GC_THREADS), 0, stream, g, n,
                           (const float*)mu, q, count);
    else
        hipLaunchKernelGGL(autoscale_cast_kernel<FMT_E5M2>, dim3((unsigned)blocks), dim3(GC_THREADS), 0, stream, g, n,
                           (const float*)mu, q, count);
    hipLaunchKernelGGL(autoscale_finalize_kernel, dim3(1), dim3(64), 0, stream, (const unsigned long long*)count, n, mu,
                       scale_out, overflow);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------- shared-scale requantize
// s_g = min of the gathered scales (a NaN entry makes it NaN); sum scale = N * s_g (one fp32 rounding).
__global__ __launch_bounds__(GC_THREADS) void min_scale_kernel(const float* __restrict__ scales, int N,
                                                              float* __restrict__ shared_out,
                                                              float* __restrict__ sum_out) {
    __shared__ float shm[GC_THREADS / 64];
    __shared__ int shn[GC_THREADS / 64];
    float m = __uint_as_float(0x7F800000u);
    int nan = 0;
    for (int i = threadIdx.x; i < N; i += GC_THREADS) {
        const float s = scales[i];
        if (s != s) nan = 1;
        else if (s < m) m = s;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        m = fminf(m, __shfl_xor(m, off, 64));
        nan |= __shfl_xor(nan, off, 64);
    }
    if ((threadIdx.x & 63) == 0) { shm[threadIdx.x >> 6] = m; shn[threadIdx.x >> 6] = nan; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < GC_THREADS / 64; ++w) { m = fminf(m, shm[w]); nan |= shn[w]; }
        const float sg = nan ? __uint_as_float(0x7FC00000u) : m;
        *shared_out = sg;
        if (sum_out) *sum_out = (float)N * sg;
    }
}

// Exact decode from the bit fields (OCP E4M3FN / E5M2).
template <int FMT>
__device__ __forceinline__ float fp8_decode(uint32_t c) {
    const uint32_t s = (c & 0x80u) << 24;
    if constexpr (FMT == FMT_E4M3) {
        const uint32_t e = (c >> 3) & 15u, m = c & 7u;
        if (e == 15u && m == 7u) return __uint_as_float(s | 0x7FC00000u);
        if (e == 0u) return __uint_as_float(s | __float_as_uint((float)m * 0.001953125f));    // m * 2^-9
        return __uint_as_float(s | ((e + 120u) << 23) | (m << 20));
    } else {
        const uint32_t e = (c >> 2) & 31u, m = c & 3u;
        if (e == 31u) return __uint_as_float(s | (m == 0u ? 0x7F800000u : 0x7FC00000u));
        if (e == 0u) return __uint_as_float(s | __float_as_uint((float)m * 1.52587890625e-05f));  // m * 2^-16
        return __uint_as_float(s | ((e + 112u) << 23) | (m << 21));
    }
}

// Saturating RNE encode with the NaN codes of the oracle's reading (E4M3 S.1111.111, E5M2 S.11111.10).
template <int FMT>
__device__ __forceinline__ uint32_t fp8_encode1(float u) {
    constexpr float FMAX = FMT == FMT_E4M3 ? 448.0f : 57344.0f;
    if (u != u) return ((__float_as_uint(u) >> 24) & 0x80u) | (FMT == FMT_E4M3 ? 0x7Fu : 0x7Eu);
    return cvt_f32_pair<FMT, false>(0u, clamp_keep_nan(u, FMAX), 0.0f) & 0xFFu;
}

// The output code depends on nothing but the input code (given s_in and s_g), so each workgroup first evaluates the
// element arithmetic once per possible code into a 256-byte LDS table (one code per thread), then streams the
// tensor through table lookups. The table spans 64 dwords, one per LDS bank, so the byte lookups never conflict.
template <int FIN, int FOUT>
__global__ __launch_bounds__(GC_THREADS) void requantize_kernel(const uint8_t* __restrict__ qin, int64_t n,
                                                               const float* __restrict__ s_in,
                                                               const float* __restrict__ s_g,
                                                               uint8_t* __restrict__ qout) {
    static_assert(GC_THREADS == 256, "one table entry per thread");
    __shared__ uint8_t lut[256];
    {
        const float si = *s_in, sg = *s_g;
        const float v = fp8_decode<FIN>(threadIdx.x);
        const float t = v / si;
        const float u = sg * t;
        lut[threadIdx.x] = (uint8_t)fp8_encode1<FOUT>(u);
    }
    __syncthreads();
    auto map4 = [&](uint32_t w) {
        return (uint32_t)lut[w & 0xFFu] | ((uint32_t)lut[(w >> 8) & 0xFFu] << 8) |
               ((uint32_t)lut[(w >> 16) & 0xFFu] << 16) | ((uint32_t)lut[w >> 24] << 24);
    };
    const int64_t chunks = n / 16, stride = (int64_t)gridDim.x * GC_THREADS;
    for (int64_t i = (int64_t)blockIdx.x * GC_THREADS + threadIdx.x; i < chunks; i += stride) {
        const uint4 v = ldnt16(qin + 16 * i);
        stnt16(qout + 16 * i, make_uint4(map4(v.x), map4(v.y), map4(v.z), map4(v.w)));
    }
    if (blockIdx.x == 0)
        for (int64_t i = chunks * 16 + threadIdx.x; i < n; i += GC_THREADS) qout[i] = lut[qin[i]];
}

hipError_t launch_requantize_shared(const uint8_t* q_in, int64_t n, int fmt_in, const float* scale_in,
                                    const float* scales, int nranks, int fmt_out, uint8_t* q_out, float* shared_out,
                                    float* sum_out, hipStream_t stream) {
    hipLaunchKernelGGL(min_scale_kernel, dim3(1), dim3(GC_THREADS), 0, stream, scales, nranks, shared_out, sum_out);
    if (n > 0) {
        // one 16-code chunk per thread; each workgroup's 256-entry table costs one evaluation per thread
        int64_t blocks = (n / 16 + GC_THREADS - 1) / GC_THREADS;
        if (blocks < 1) blocks = 1;
        if (blocks > (int64_t(1) << 30)) blocks = int64_t(1) << 30;
        const dim3 grid((unsigned)blocks), blk(GC_THREADS);
        const float* sg = shared_out;
        if (fmt_in == FMT_E4M3 && fmt_out == FMT_E4M3)
            hipLaunchKernelGGL((requantize_kernel<FMT_E4M3, FMT_E4M3>), grid, blk, 0, stream, q_in, n, scale_in, sg, q_out);
        else if (fmt_in == FMT_E4M3)
            hipLaunchKernelGGL((requantize_kernel<FMT_E4M3, FMT_E5M2>), grid, blk, 0, stream, q_in, n, scale_in, sg, q_out);
        else if (fmt_out == FMT_E4M3)
            hipLaunchKernelGGL((requantize_kernel<FMT_E5M2, FMT_E4M3>), grid, blk, 0, stream, q_in, n, scale_in, sg, q_out);
        else
            hipLaunchKernelGGL((requantize_kernel<FMT_E5M2, FMT_E5M2>), grid, blk, 0, stream, q_in, n, scale_in, sg, q_out);
    }
    return hipGetLastError();
}

}  // namespace mxq
