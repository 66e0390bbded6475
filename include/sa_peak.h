/*
 * sa_peak.h -- achievable-peak probes of the MI355X this library runs on.
 *
 * Measurement utilities, not part of the sparse-attention method: the
 * benchmark reports its kernels' rates against the published peaks and,
 * beside them, against what these plain kernels reach on the same GPU (a
 * streaming HBM read, and dense MFMA loops in bf16 and fp8).
 *
 * Every call is asynchronous on `stream` (a hipStream_t, NULL = the default
 * stream); time it with events on that stream.  Buffers are caller-owned
 * device memory.  Returns 0, or a negative sa_status (see sparse_attn.h) for
 * invalid arguments or a failed launch.
 */
#ifndef SA_PEAK_H
#define SA_PEAK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a multiple of 16, 16-byte aligned) from `src` once with
 * 16-byte non-temporal loads: each workgroup streams one contiguous slab,
 * each wave instruction covering 1 KB; `sink` [grid * 256] u32 receives one
 * XOR per thread so the loads cannot be dropped.  grid: workgroups of 256
 * threads (>= 1); 1024 measured fastest on MI355X. */
int32_t sa_peak_read(const void* src, size_t bytes, uint32_t* sink, int32_t grid, void* stream);

/* `grid` workgroups of 256 threads each run `iters` rounds of 8 independent
 * MFMA accumulations: dtype 1 = v_mfma_f32_16x16x32_bf16 (16384 flops
 * each), dtype 2 = v_mfma_scale_f32_16x16x128_f8f6f4 on fp8 (65536 flops
 * each).  Total flops = grid * 4 waves * iters * 8 * flops per MFMA.  `sink`
 * [grid * 256] f32 receives the accumulators' sums. */
int32_t sa_peak_mfma(int32_t dtype, int32_t iters, float* sink, int32_t grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SA_PEAK_H */
