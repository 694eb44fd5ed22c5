/*
 * mxq_probe.h — C ABI of libmxq_probe.so, the measurement-support library that sits beside libmxq.so.
 *
 * None of these calls is a step of the FP8 / MXFP8 training numerics; they measure what this part sustains, so that
 * each kernel of libmxq.so can be read against the sustained ceiling as well as against the spec peak. Only the
 * benchmark and its tests load this library. Conventions are those of mxq.h: device pointers, work enqueued on
 * `stream`, host-side validation returning a status before anything is enqueued, no allocation, no synchronization.
 */
#ifndef MXQ_PROBE_H
#define MXQ_PROBE_H

#include "mxq.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * An MFMA-only loop of the block-scaled FP8 instruction (v_mfma_scale_f32_32x32x64_f8f6f4, unit scales) in the
 * large-tile GEMM's register shape. `blocks` workgroups of 256 threads each run iters * 16 instructions per wave, i.e.
 * blocks * 4 * iters * 16 * 131072 FLOP in all; there is no memory traffic in the loop. operand_bytes: device,
 * >= 131072 bytes (real quantized data gives a realistic bit toggle rate), 16-byte aligned. sink: device
 * float[blocks * 256], written. 1 <= blocks <= 65536, iters >= 1.
 */
mxq_status mxq_probe_mfma_fp8(const uint8_t* operand_bytes, int64_t iters, int64_t blocks, float* sink,
                              hipStream_t stream);

/*
 * A streaming device copy dst[0 .. bytes) = src[0 .. bytes) with 16-byte non-temporal loads and stores.
 * blocks > 0: a grid of `blocks` workgroups of 256 threads loops over the data, `unroll` (4, 8 or 16) 16-byte loads
 * in flight per thread per trip. blocks == 0: one workgroup per 256 x unroll chunks of 16 bytes (no loop).
 * Device pointers, 16-byte aligned, not overlapping; bytes % 16 == 0; 0 <= blocks <= 65536.
 */
mxq_status mxq_probe_copy(const void* src, void* dst, int64_t bytes, int64_t blocks, int64_t unroll,
                          hipStream_t stream);

/*
 * A streaming device read of src[0 .. bytes) (16-byte non-temporal loads, `unroll` in flight per thread, grid as in
 * mxq_probe_copy) whose only store is one 4-byte xor of the words read per workgroup, to sink[blockIdx] (sink: device
 * uint32[number of workgroups]; 65536 entries always suffice when blocks > 0, bytes / (4096 * unroll) + 1 when
 * blocks == 0). The HBM read rate the part sustains.
 */
mxq_status mxq_probe_read(const void* src, int64_t bytes, int64_t blocks, int64_t unroll, uint32_t* sink,
                          hipStream_t stream);

/*
 * A streaming read of src[0 .. bytes) into LDS with the large-tile GEMM's global-to-LDS copy instruction
 * (buffer_load_dwordx4 ... lds, 1 KiB per wave instruction): `blocks` workgroups of 256 threads loop over the 64 KiB
 * pieces of src, and workgroup w writes the xor of every 32-bit word it read to sink[w] (sink: device uint32[blocks]).
 * It gives the hardware counters' bytes per byte for that load path. bytes % 65536 == 0; src 16-byte aligned;
 * 1 <= blocks <= 65536. bytes == 0 writes sink[w] = 0.
 */
mxq_status mxq_probe_read_lds(const void* src, int64_t bytes, int64_t blocks, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MXQ_PROBE_H */
