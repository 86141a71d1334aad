/*
 * msa_probe.h -- a measurement aid built beside the decode library (libmsa_probe.so); not part
 * of the pass. It reads the index-K pages a decode call over full-length rows reads, through
 * the same block table and with the decode kernels' load pattern, and only folds the bytes
 * into one XOR word per thread: its time is the streaming ceiling of the decode kernels on
 * this GPU (how fast HBM serves that access pattern), against which their fixed costs (the
 * plan, the per-split ranking, publication and merge) are judged.
 */
#ifndef MSA_PROBE_H
#define MSA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_PROBE_SPLIT_PATTERN 0  /* the VALU decode kernel: pages in batches of 16 KiB */
#define MSA_PROBE_CHUNK_PATTERN 1  /* the verify kernel: 8 KiB chunks, two in flight per wave */

/*
 * Reads every page block_table[b][j], j < W, of `page_bytes` bytes (a multiple of 16 KiB: 32 KiB
 * for a bf16 page, 16 KiB for an FP8 page) from k_cache (device, 16-byte aligned). Grid:
 * ceil(W / blocks_per_wg) workgroups per row of 4 waves each, wave w reading every 4th block of
 * its workgroup's range. out: device uint32 [batch][ceil(W / blocks_per_wg)][256], one XOR fold
 * per thread. Every table entry must name a page of k_cache (not checked). Enqueued on `stream`
 * (a hipStream_t). Returns 0, -1 on invalid arguments, -4 if the launch fails.
 */
int32_t msa_probe_stream_pages(const void *k_cache, int32_t page_bytes, const int32_t *block_table,
                               int32_t batch, int32_t W, int32_t bt_stride, int32_t blocks_per_wg,
                               int32_t pattern, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_PROBE_H */
