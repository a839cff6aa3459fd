/* Gather-rate probe of the benchmark (libqsa_probe.so).
 *
 * Not part of the QSA layer's boundary (qsa.h) and used by no QSA entry
 * point: the benchmark calls it to measure, on the same GPU and in the same
 * run, the rate at which the sparse attention's 2 KiB micro-block gathers can
 * be served -- from a region that fits in the L2, uniformly at random from a
 * cache as large as the workload's, and along the attention's own selection
 * lists -- with the attention's arithmetic taken out.  This gives the
 * attention kernel (PyTorchKR post "Qwen3.8-Flash-Next, 1/9의 학습 비용으로 …",
 * section "QSA: 인덱서 자체의 비용을 줄이는 희소 어텐션": sparse core attention
 * over the selected micro-blocks) a measured ceiling beside the datasheet
 * peaks.
 */
#pragma once

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* For every row r < rows of idx (int32 [rows][list_len], device) and both KV
 * groups g = 0, 1: load, step by step, the K~ and V blocks named by the row's
 * ids -- 2 KiB at k_base + g*grp_stride + id*2048 and at
 * v_base + g*grp_stride + id*2048 (device memory the caller owns, at least
 * grp_stride + n_blocks*2048 bytes each) -- in `step` (2, 4 or 8) entries per
 * step; ids outside [0, n_blocks) read block 0, a tail of fewer than `step`
 * entries is skipped.  One wave per (row, group), four rows of one group per
 * 256-thread work-group, group 0's work-groups first, in launches of at most
 * launch_rows rows, asynchronous on `stream` (a hipStream_t).  pad_kib (0, 40,
 * 64 or 96) KiB of LDS per work-group caps the work-groups a CU holds.  Each
 * wave writes a checksum of what it loaded into sink (device, 65,536 uint32).
 * Returns 0, or a hipError_t code: 1 (invalid value) for a null pointer, a
 * negative size or an unsupported step / pad_kib, before anything is enqueued;
 * a failed launch's code otherwise. */
int qsa_probe_gather(void *stream, const void *k_base, const void *v_base, int64_t grp_stride, int64_t n_blocks,
                     const int32_t *idx, int64_t rows, int32_t list_len, int64_t launch_rows, int32_t step,
                     int32_t pad_kib, uint32_t *sink);

#ifdef __cplusplus
}
#endif
