/*
 * b2b_bench.h -- measurement instruments of libb2b.so (not part of the
 * cascade): the practical ceilings of the running MI355X's matrix cores and
 * HBM, against which the fused kernels' rates are reported beside the
 * datasheet peaks.  The pages state the benefit of fusion only as the memory
 * round trip it saves (page 1, "数据处理方法、装置、设备及介质", background and
 * detailed description); these kernels measure what that memory and the
 * matrix cores actually deliver, so that a kernel's rate can be read as a
 * fraction of what is reachable.
 *
 * Both calls only enqueue one kernel on `stream` and return; time them with
 * events on the same stream.  Errors: INVALID_VALUE for bad arguments,
 * NOT_SUPPORTED for a dtype without a matrix-core loop, HIP for a failed
 * launch.
 */
#ifndef B2B_BENCH_H_
#define B2B_BENCH_H_

#include "b2b.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Matrix cores alone: every wave runs `iters` rounds of independent chains
 * of the instruction the fused kernels use for `dtype` (fp16/bf16:
 * v_mfma_f32_16x16x32, 16 accumulators; fp64: v_mfma_f64_16x16x4, 8
 * accumulators), with no memory traffic inside the loop.
 *   workgroups  1..65536 workgroups of 256 threads (launch two per compute
 *               unit for two waves per SIMD)
 *   iters       1..2^24 rounds
 *   sink        device buffer of workgroups * 256 * 8 bytes: one value per
 *               thread, written at the end so the loop is not dropped
 *   flop        out (host): the floating-point operations the launch performs
 */
b2b_status_t b2b_bench_mfma(b2b_dtype_t dtype, int32_t workgroups, int64_t iters, void* sink, double* flop,
                            hipStream_t stream);

/*
 * HBM stream: dst[i] = src[i] over `bytes` bytes (a multiple of 64), 16-byte
 * loads and non-temporal 16-byte stores, as the fused kernels read A and
 * write D.  src and dst are device pointers, 16-byte aligned, not
 * overlapping; the traffic is 2 * bytes.
 *   workgroups  1..65536 workgroups of 256 threads, each walking the buffer
 *               with a grid stride
 */
b2b_status_t b2b_bench_copy(const void* src, void* dst, int64_t bytes, int32_t workgroups, hipStream_t stream);

/*
 * HBM stream with a read:write mix: dst[i] = src[i] ^ src[i + n] ^ ... over
 * 16-byte pieces, R = read_bytes / write_bytes read streams of n pieces each
 * (src holds them back to back) for the one written stream of n pieces.  Fed
 * a cascade's own A (read) and D (written) buffers, it moves exactly the
 * bytes the cascade must move to and from HBM, at the rate the memory system
 * gives a pure stream of that mix -- the cascade's practical memory roofline.
 * R = 1 is the copy above.
 *   src, dst     device pointers, 16-byte aligned, not overlapping
 *   read_bytes   R * write_bytes, 1 <= R <= 4
 *   write_bytes  a multiple of 64
 *   workgroups   1..65536 workgroups of 256 threads, grid stride
 */
b2b_status_t b2b_bench_stream(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes,
                              int32_t workgroups, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* B2B_BENCH_H_ */
