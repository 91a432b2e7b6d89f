/*
 * pa_probe.h -- HBM read ceilings for the benchmark (libpa_probe.so).
 *
 * Not part of the paged-attention path: two loads-only kernels that read
 * exactly the bytes a decode call reads, so the benchmark can report what a
 * kernel that does nothing but load them reaches on the same GPU [P1 §04
 * table: decode is bound by memory bandwidth; P3 §1.2]. Every pointer is
 * device memory owned by the caller; calls are asynchronous on `stream` (a
 * hipStream_t passed as void*) and return 0, or -1 for invalid arguments or
 * a failed launch. Loads are streaming (nt), as in the decode kernels.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes (a multiple of 16) from src in one contiguous sweep,
 * `grid` workgroups of 512 threads each taking an equal contiguous share.
 * sink: device uint32 [grid * 512], written only in the (practically
 * impossible) case that the XOR of a thread's data is 0x9e3779b9. */
int pa_probe_read_linear(const void *src, size_t bytes, uint32_t *sink, int grid, void *stream);

/* Reads whole blocks of the two pools k_pool and v_pool (block_bytes each, a
 * multiple of 8 KiB) in the order of `blocks` (device int32 [num_blocks];
 * ids outside [0, pool_blocks) are skipped): the block sequence a decode
 * call walks, without the attention. `grid` workgroups of 512 threads each
 * take an equal contiguous share of the list, two blocks in flight. */
int pa_probe_read_blocks(const void *k_pool, const void *v_pool, int64_t pool_blocks,
                         int block_bytes, const int32_t *blocks, int64_t num_blocks,
                         uint32_t *sink, int grid, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
