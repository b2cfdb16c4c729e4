/*
 * fa_probe.h -- measurement probes exported by libfa.so.  They are not part of
 * the attention method: they measure the two hardware limits the kernels are
 * priced against (bf16 MFMA throughput for the attention kernels, HBM read
 * bandwidth for the split-KV decode), so that measured ceilings can be
 * reported beside the published peaks.  The caller times the launch (for
 * example with events on `stream`) and divides the work below by the time.
 *
 * Conventions are those of fa.h: device pointers the caller owns, arguments
 * validated before any launch, asynchronous on `stream`, FA_* status codes.
 */
#ifndef FA_PROBE_H
#define FA_PROBE_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * bf16 MFMA throughput: `blocks` workgroups of 8 wavefronts; each wavefront
 * issues `iters` x 16 v_mfma_f32_32x32x16_bf16 on four independent
 * accumulator chains, operands in registers, no memory traffic in the loop.
 * Work: blocks * 8 * iters * 16 * 32768 FLOP.
 * sink: device float[blocks * 512], written once per thread (keeps the
 * accumulators live); its values carry no meaning.
 * Errors: FA_ERR_INVALID_ARG for blocks < 1, iters < 1 or a null sink.
 */
int fa_probe_mfma(int blocks, int iters, float* sink, hipStream_t stream);

/*
 * HBM read bandwidth: 256 workgroups of 512 threads read `bytes` from `buf`
 * once with 16-byte non-temporal loads, 4 in flight per thread, in a
 * grid-stride sweep (the pattern and hint of the decode's K/V stream).
 * Work: `bytes` read.  bytes must be a positive multiple of 16 * 512 * 256 * 4
 * (8 MiB); buf 16-byte aligned.
 * sink: device unsigned[256 * 512], written once per thread (an XOR of the
 * data read).
 * Errors: FA_ERR_INVALID_ARG for a bad size, alignment or null pointer.
 */
int fa_probe_hbm_read(const void* buf, size_t bytes, unsigned* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H */
