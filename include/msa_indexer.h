/*
 * msa_indexer.h -- C ABI of the MI355X (gfx950) MiniMax-M3 lightning-indexer decode pass.
 *
 * The pass, for each decode row b (one decode token) and each of the 4 index heads h:
 *   1. scores every 128-token block j of the row's paged bf16 index-K cache as
 *      S[b][h][j] = max over the block's valid tokens t of sum_d q[b][h][d] * k[t][d],
 *      accumulated in fp32, with no scale applied;
 *   2. selects the top `topk` blocks, with the first `n_init` blocks and the last
 *      `n_local` blocks of the row always selected (pinned).
 * Variants: up to 4 query positions per row (speculative-decode verification,
 * msa_indexer_decode_multi), an FP8 E4M3 cache (msa_indexer_decode_fp8), and the selection
 * written as a 16-token page table (msa_indexer_decode_pages, msa_indexer_expand_pages).
 * Sources:
 *   - vLLM PR #57832 "context-parallel decode scoring for MiniMax-M3's sparse lightning
 *     indexer on ROCm": Problem (one index-K head shared by the 4 index heads, every
 *     block of the context scored), Solution (per-head top-k, packed int64 (score, block
 *     id) keys, exact merge of per-shard top-k, pinned init/sink and sliding-window
 *     blocks), CUDA graph capture (shapes from a bound, block counts and strides as
 *     runtime arguments, chunks past a row's end return at once).
 *   - SGLang PR #41488 "[AMD] Add opt-in MiniMax-M3 TP4 indexer context partitioning":
 *     Modifications (4 heads, dim 128, 128-token blocks, max scoring, top-16, initial /
 *     recent block priorities, every K tile scored for all heads while resident, 16
 *     candidates kept per shard).
 *   - TensorRT-LLM PR #17008 "MiniMax-M3 MSA: split the KV axis for the decode indexer
 *     proxy": Description and Changes (full-context max-score pass; split-KV to shorten
 *     the per-workgroup serial tile chain), Accuracy (each split's max seeded at -inf,
 *     so splitting the KV axis cannot change a score).
 *   - vLLM blog "Following the Bottleneck: Optimizing MiniMax M3 on AMD Instinct MI355X",
 *     section 2 (no positive score scale: it cannot change top-k order).
 *
 * Conventions for every entry point:
 *   - Pointers named q, k_cache, block_table, seq_lens, out_*, workspace are DEVICE
 *     pointers (hipMalloc'd memory of the current device). The caller owns every buffer;
 *     the library never allocates or frees memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). All work is
 *     enqueued on it and the call returns without synchronizing. Errors found on the
 *     device surface at the caller's next synchronization or through the workspace's
 *     error word (msa_indexer_read_error).
 *   - Grid and workspace sizes depend only on (batch, max_blocks_per_seq, topk,
 *     num_splits) and, for the multi-token and FP8 calls, qlen; never on seq_lens or
 *     block_table contents, so a call can be captured once in a HIP graph and replayed
 *     after seq_lens / block_table change on device.
 *   - Argument checks run on the host before any HIP call; a failed check returns a
 *     negative status and enqueues nothing. Nothing aborts.
 *   - Concurrent calls that share a workspace on one device race; give each stream its own.
 */
#ifndef MSA_INDEXER_H
#define MSA_INDEXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MSA_OK 0
#define MSA_ERR_INVALID_ARG (-1)         /* null/misaligned pointer, bad size or parameter */
#define MSA_ERR_WORKSPACE_TOO_SMALL (-2) /* workspace_bytes < msa_indexer_workspace_bytes(...) */
#define MSA_ERR_UNSUPPORTED (-3)         /* shape beyond what the library handles */
#define MSA_ERR_HIP (-4)                 /* the HIP runtime refused a launch */

/* Fixed model geometry (SGLang PR #41488, Modifications). */
#define MSA_INDEX_HEADS 4
#define MSA_HEAD_DIM 128
#define MSA_BLOCK_TOKENS 128

/* Limits of the library. */
#define MSA_MAX_TOPK 64
#define MSA_MAX_BLOCKS_PER_SEQ 16384     /* 2M tokens per row */
#define MSA_MAX_QUERY_LEN 4              /* query positions per row in the multi-token calls */

/* Block-scoring engines (msa_indexer_split_topk / msa_indexer_block_scores). */
#define MSA_ENGINE_DEFAULT 0                /* the VALU engine */
#define MSA_ENGINE_VALU 1                /* bf16 dot2 instructions + in-row DPP sums */
#define MSA_ENGINE_MFMA 2                /* v_mfma_f32_16x16x32_bf16, heads padded to 16 */

/* Device error bits, OR-ed into the workspace's error word by the kernels. */
#define MSA_DEVERR_PAGE_OUT_OF_RANGE 1u  /* a needed block_table entry was outside [0, num_pages) */

/*
 * Human-readable text for a status code. Never NULL. Every entry point reports a rejected
 * configuration as a status before it enqueues anything, as the pages' integration fails
 * unsupported configurations at startup instead of running them (vLLM PR #57832, Test Result).
 */
const char *msa_status_string(int32_t status);

/*
 * Number of KV splits S a call uses: num_splits > 0 asks for that many (the library
 * may use fewer so that no split is empty by construction); 0 picks S from batch and
 * max_blocks_per_seq. Returns a negative status on invalid arguments.
 * Split s of row b owns logical blocks [s*C, min((s+1)*C, nb_b)), C = ceil(W/S)
 * (TensorRT-LLM PR #17008, Changes: split the KV axis into contiguous tile ranges).
 */
int32_t msa_indexer_num_splits(int32_t batch, int32_t max_blocks_per_seq, int32_t topk,
                               int32_t num_splits);

/*
 * The plan a call with these arguments uses: S splits per row, C blocks per split, Lk =
 * min(topk, C) candidates kept per (split, head), and whether the merge runs inside the
 * split kernel (fused: one launch) or as a second launch. The single-token decode fuses
 * when topk <= 16 and the S lists of Lk keys, each rounded up to a power of two, hold at
 * most 1024 keys per head (e.g. 256 splits of 4 blocks), or when S <= 64 and S * Lk <=
 * 1024; otherwise it takes two launches. Any output pointer may be NULL.
 * Returns MSA_OK or a negative status. With num_splits = 0, topk <= 16 and batch *
 * max_blocks_per_seq >= 8192 the plan is the device plan: the kernel itself picks C (a
 * power of two from 4 to 64) and each workgroup's (row, split) from seq_lens, so that about
 * 512 workgroups cover the tokens actually present; *blocks_per_split is then 0 and *splits
 * is S = min(64, ceil(W/4)), which sizes the workspace (S * topk keys per row and head). A
 * row of nb blocks takes ceil(nb / C) splits of Lk = min(topk, C) keys per head, as many as
 * fit those keys and the merge (at most 1024 keys, lists rounded up to a power of two): at
 * topk = 16, up to 256 splits of 4 blocks, so that one long row among short ones is still
 * spread over the whole chip. The multi-token and FP8 calls use the same plan and merge in a
 * second launch, except with qlen = 1, topk <= 16 and either the device plan or lists short
 * enough that a row's merge is cheap (S lists of Lk keys rounded up to a power of two, at
 * most 4 * 64 / Lk2 lists): then the last split of each row merges it in the same launch.
 */
int32_t msa_indexer_plan(int32_t batch, int32_t max_blocks_per_seq, int32_t topk, int32_t num_splits,
                         int32_t *splits, int32_t *blocks_per_split, int32_t *candidates_per_split,
                         int32_t *fused);

/* Workspace layout (msa_indexer_workspace_bytes). */
#define MSA_WORKSPACE_HEADER_BYTES 256   /* the device error word first */
#define MSA_WORKSPACE_ROW_BYTES 4352     /* 17 counter lines of 256 B per row */

/*
 * Workspace bytes a call with these arguments needs (0 on invalid arguments): the persistent,
 * allocation-free buffer of vLLM PR #57832 (Problem and CUDA graph capture: buffers sized from
 * the launch bounds, reused by every replay), sized from (batch, max_blocks_per_seq, topk,
 * num_splits) only.
 * Layout of a buffer of N bytes (the size the caller passes as workspace_bytes):
 *   [0, 256)                           header; its first uint32 is the device error word;
 *   [256 + 4352 b, 256 + 4352 (b+1))   the counter lines of row b (uint32 [17][64]: line 0
 *                                      counts the row's finished splits, lines 1..16 count
 *                                      groups of 16 splits for rows of more than 128 splits);
 *   the last K bytes (256-aligned)     the per-split candidate keys, uint64 [batch][4][S * Lk]
 *                                      (each head's split lists one after another),
 *                                      K = this size minus 256 minus 4352 * batch.
 * The whole buffer must be zero before its first use (e.g. hipMemset once after allocation).
 * Every call leaves the counters at zero when it ends, and a row's counter lines sit at an
 * offset that depends on nothing but the row, while a call's keys fill the end of the buffer.
 * So one buffer can serve any sequence of calls, and graph replays, without being cleared
 * again, provided every call passes the buffer's full size N and N holds the largest batch's
 * counter lines plus the largest key region of those calls. Calls with the same
 * max_blocks_per_seq, topk and num_splits (and qlen, for msa_indexer_workspace_bytes_multi)
 * meet this whatever their batch sizes, with N the size the largest batch needs. The error
 * word only ever gains bits (msa_indexer_read_error takes and clears them).
 */
size_t msa_indexer_workspace_bytes(int32_t batch, int32_t max_blocks_per_seq, int32_t topk,
                                   int32_t num_splits);

/*
 * The whole decode pass: block scores, per-split top-k, exact merge (vLLM PR #57832, Solution:
 * every block scored, per-head top-k of packed (score, block id) keys, an exact merge of per-shard
 * top-k lists with the init/sink and sliding-window blocks pinned; SGLang PR #41488,
 * Modifications: max over each 128-token block, 4 heads scored from one read of each K tile;
 * TensorRT-LLM PR #17008, Changes and Accuracy: the KV axis split into contiguous tile ranges,
 * each range's maximum seeded at -inf, so the split count cannot change a score).
 * Beyond the plain form of this call (q, k_cache, block_table, seq_lens, sizes, topk, pins,
 * outputs, workspace, stream) it takes num_splits, the split-count knob TensorRT-LLM PR #17008
 * sweeps (Performance: num_kv_splits 1..32) and checks for invariance (Accuracy); 0 leaves the
 * choice to the library.
 *
 *   q            bf16 [batch][4][128], contiguous, 16-byte aligned: post-RoPE index queries,
 *                one decode token per row.
 *   k_cache      bf16 [num_pages][128 tokens][128 dims], contiguous, 16-byte aligned:
 *                the shared single-head index-K cache, one logical block per page.
 *   block_table  int32 [batch][bt_stride]: logical block j of row b lives in page
 *                block_table[b*bt_stride + j]. Only entries j < nb_b are read; each must
 *                lie in [0, num_pages). An entry outside is never dereferenced: its block
 *                scores -inf and the workspace error word gets MSA_DEVERR_PAGE_OUT_OF_RANGE.
 *   seq_lens     int32 [batch]: context tokens of row b (the decode token included).
 *                Values are clamped to [0, max_blocks_per_seq*128]; nb_b = ceil(len/128).
 *   batch >= 0 (0 is a successful no-op), 0 <= max_blocks_per_seq <= MSA_MAX_BLOCKS_PER_SEQ,
 *   bt_stride >= max_blocks_per_seq, num_pages >= 0.
 *   topk in [1, MSA_MAX_TOPK]; n_init, n_local >= 0 and n_init + n_local <= topk.
 *     Pinned blocks of row b: j < n_init and j >= nb_b - n_local (whole blocks; a partial
 *     last block counts). They are selected first, in score order.
 *   out_ids      int32 [batch][4][topk]: selected logical block ids of (b, h), in order
 *                (pinned first, then higher score, then lower id); slots past
 *                m = min(topk, nb_b) hold -1.
 *   out_scores   fp32 [batch][4][topk]: the selected blocks' scores (-0.0 reads as +0.0);
 *                slots past m hold -inf.
 *   workspace    device memory of at least msa_indexer_workspace_bytes(...) bytes, 256-byte
 *                aligned, zeroed once before its first use; workspace_bytes is its full size
 *                (see msa_indexer_workspace_bytes).
 *   num_splits   0 = automatic; see msa_indexer_num_splits.
 * When the plan is fused (msa_indexer_plan) this is one kernel launch: the last split of
 * each row to finish merges the row. Otherwise stage 1 and stage 2 are two launches.
 */
int32_t msa_indexer_decode(const void *q, const void *k_cache, const int32_t *block_table,
                           const int32_t *seq_lens, int32_t batch, int32_t max_blocks_per_seq,
                           int32_t bt_stride, int64_t num_pages, int32_t topk, int32_t n_init,
                           int32_t n_local, int32_t *out_ids, float *out_scores, void *workspace,
                           size_t workspace_bytes, int32_t num_splits, void *stream);

/* Limits of msa_indexer_decode_noalloc's scratch array (one per GPU). */
#define MSA_NOALLOC_SCRATCH_BYTES (16u << 20)  /* 16 MiB */
#define MSA_NOALLOC_MAX_BATCH 256

/*
 * msa_indexer_decode for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same pass and results,
 * with the library's own scratch array in place of the workspace. Allocates nothing (no
 * hipMalloc, hipFree or allocating library routine). The array is a file-scope device array of
 * MSA_NOALLOC_SCRATCH_BYTES on each GPU, held until the process ends: the first
 * MSA_WORKSPACE_HEADER_BYTES + MSA_NOALLOC_MAX_BATCH * MSA_WORKSPACE_ROW_BYTES bytes are the
 * row counters, the rest holds the keys. Calls with batch > MSA_NOALLOC_MAX_BATCH, or whose
 * keys (batch * S * 4 * Lk * 8 bytes for the call's plan) exceed the rest, return
 * MSA_ERR_WORKSPACE_TOO_SMALL and enqueue nothing; at the default plan this admits batch 256 at
 * up to 4096 blocks per row (a row's keys are at most 32 KiB under the device plan).
 * The first call on a device looks the array up and clears its counters on `stream`. Every
 * call on a GPU shares that GPU's array and leaves its counters at zero, so calls that overlap
 * on one GPU (concurrent streams, threads or processes' graphs) race: serialize them.
 *   error_flags  optional device uint32 (NULL: not kept): MSA_DEVERR_* bits are OR-ed into it,
 *                as into a workspace's error word; the caller reads and clears it.
 * Every other argument as in msa_indexer_decode.
 */
int32_t msa_indexer_decode_noalloc(const void *q, const void *k_cache, const int32_t *block_table,
                                   const int32_t *seq_lens, int32_t batch, int32_t max_blocks_per_seq,
                                   int32_t bt_stride, int64_t num_pages, int32_t topk, int32_t n_init,
                                   int32_t n_local, int32_t *out_ids, float *out_scores,
                                   uint32_t *error_flags, int32_t num_splits, void *stream);

/*
 * msa_indexer_decode with an explicit scoring engine (MSA_ENGINE_*): for measuring the
 * engines against each other on the whole pass. msa_indexer_decode uses MSA_ENGINE_DEFAULT,
 * which is the VALU engine (faster on MI355X, where the pass is bound by HBM bandwidth).
 */
int32_t msa_indexer_decode_engine(const void *q, const void *k_cache, const int32_t *block_table,
                                  const int32_t *seq_lens, int32_t batch,
                                  int32_t max_blocks_per_seq, int32_t bt_stride, int64_t num_pages,
                                  int32_t topk, int32_t n_init, int32_t n_local, int32_t *out_ids,
                                  float *out_scores, void *workspace, size_t workspace_bytes,
                                  int32_t num_splits, int32_t engine, void *stream);

/*
 * msa_indexer_decode that also writes the selection as a 16-token page table, for a
 * sparse-attention kernel that pages KV in 16-token pages while the indexer selects
 * 128-token blocks (vLLM blog "Following the Bottleneck", section 3 and Figure 5: each
 * selected block becomes the eight 16-token page entries of its physical block, and only
 * this table is built; the KV cache is not copied or moved).
 *   out_pages    int32 [batch][4][8*topk], 16-byte aligned. For (b, h), the selected blocks
 *                in ascending logical block order; the i-th, block j, gives entries
 *                8i .. 8i+7 = 8 * block_table[b*bt_stride + j] + t (t = 0..7). Entries past
 *                8 * m are -1.
 *   out_tokens   int32 [batch][4], 4-byte aligned: tokens in that table, the sum over the
 *                selected blocks of min(128, len_b - 128 j). Only the last block of a row can
 *                be partial, and it comes last when selected, so the table's first
 *                out_tokens entries' tokens are exactly the selected context.
 * Both must be non-null when batch > 0. num_pages must be at most 2^28 (so a 16-token page
 * id fits int32; MSA_ERR_UNSUPPORTED otherwise). `engine` as in msa_indexer_decode_engine;
 * every other argument as in msa_indexer_decode. The table is written by the same launch
 * that writes out_ids (the merging workgroup of each row), not by an extra pass.
 */
int32_t msa_indexer_decode_pages(const void *q, const void *k_cache, const int32_t *block_table,
                                 const int32_t *seq_lens, int32_t batch,
                                 int32_t max_blocks_per_seq, int32_t bt_stride, int64_t num_pages,
                                 int32_t topk, int32_t n_init, int32_t n_local, int32_t *out_ids,
                                 float *out_scores, int32_t *out_pages, int32_t *out_tokens,
                                 void *workspace, size_t workspace_bytes, int32_t num_splits,
                                 int32_t engine, void *stream);

/*
 * The page table of msa_indexer_decode_pages from given selections (vLLM blog "Following the
 * Bottleneck", section 3), e.g. a selection a previous layer made and later layers reuse.
 *   ids          int32 [batch][4][topk], 4-byte aligned: per (b, h), block ids in any order.
 *                An id outside [0, nb_b) stands for no block (so -1 padding is skipped) and
 *                is never looked up; a repeated id is expanded each time it appears.
 *   block_table, seq_lens, batch, max_blocks_per_seq, bt_stride as in msa_indexer_decode
 *                (block_table entries of selected blocks are copied, not range-checked).
 *   topk in [1, MSA_MAX_TOPK]; out_pages int32 [batch][4][8*topk] (16-byte aligned) and
 *   out_tokens int32 [batch][4] as in msa_indexer_decode_pages, counting each expanded id.
 * One launch of `batch` workgroups; no workspace. Entries are 8 * page + t modulo 2^32.
 */
int32_t msa_indexer_expand_pages(const int32_t *ids, const int32_t *block_table,
                                 const int32_t *seq_lens, int32_t batch,
                                 int32_t max_blocks_per_seq, int32_t bt_stride, int32_t topk,
                                 int32_t *out_pages, int32_t *out_tokens, void *stream);

/*
 * msa_indexer_expand_pages for the selections of a multi-token pass (the page-table builder
 * reused for speculative-decode verification, vLLM blog "Following the Bottleneck", section
 * 3): ids int32 [batch][qlen][4][topk] as msa_indexer_decode_multi writes them; selection
 * (b, p) uses block_table row b and position p's causal length L_p = max(0, len_b -
 * (qlen-1-p)) (len_b clamped to the table first) for its ids' range and its token count.
 * out_pages int32 [batch][qlen][4][8*topk] (16-byte aligned), out_tokens int32
 * [batch][qlen][4]. qlen in 1..MSA_MAX_QUERY_LEN; qlen = 1 is msa_indexer_expand_pages.
 */
int32_t msa_indexer_expand_pages_multi(const int32_t *ids, const int32_t *block_table,
                                       const int32_t *seq_lens, int32_t batch,
                                       int32_t max_blocks_per_seq, int32_t bt_stride, int32_t qlen,
                                       int32_t topk, int32_t *out_pages, int32_t *out_tokens,
                                       void *stream);

/*
 * Workspace bytes of msa_indexer_decode_multi and msa_indexer_decode_fp8 (0 on invalid
 * arguments): the layout of msa_indexer_workspace_bytes with keys uint64
 * [batch][qlen*4][S * Lk]. Zeroed once before its first use, like the single-token workspace,
 * and shareable with it under the same rule.
 */
size_t msa_indexer_workspace_bytes_multi(int32_t batch, int32_t max_blocks_per_seq, int32_t qlen,
                                         int32_t topk, int32_t num_splits);

/*
 * Multi-token decode: a row that verifies qlen draft tokens (speculative decoding) carries
 * qlen query positions, the last qlen tokens of its context (vLLM PR #57832, Test Plan:
 * query_len 4 verifies; vLLM blog "Following the Bottleneck", section 2: one workgroup per
 * request scores all draft positions from one read of the keys).
 *   q            bf16 [batch][qlen][4][128], contiguous, 16-byte aligned.
 *   qlen         1 .. MSA_MAX_QUERY_LEN.
 *   seq_lens     context tokens of row b, the qlen draft tokens included; clamped to
 *                [0, max_blocks_per_seq*128] first. Position p then sees the first
 *                L_p = max(0, len_b - (qlen-1-p)) tokens (the causal clamp
 *                min(q_end + offset_q, kv_len) of TensorRT-LLM PR #17008, Description).
 *   out_ids, out_scores  int32 / fp32 [batch][qlen][4][topk]: for every (b, p, h), exactly
 *                what msa_indexer_decode returns for query q[b][p] and length L_p (its own
 *                block count, pinned blocks and padding).
 *   workspace    at least msa_indexer_workspace_bytes_multi(...) bytes, 256-byte aligned.
 * Every other argument as in msa_indexer_decode. Each page is read once for all positions
 * and heads (MFMA: 4 positions x 4 heads fill the 16 rows of v_mfma_f32_16x16x32_bf16).
 * Two launches (one for qlen = 1 under the conditions msa_indexer_plan states): per-split
 * top-k of every (position, head), then one wave per (b, p, h) merging the splits' lists.
 * Under the device plan both launches derive the split width from seq_lens alike.
 */
int32_t msa_indexer_decode_multi(const void *q, const void *k_cache, const int32_t *block_table,
                                 const int32_t *seq_lens, int32_t batch,
                                 int32_t max_blocks_per_seq, int32_t bt_stride, int64_t num_pages,
                                 int32_t qlen, int32_t topk, int32_t n_init, int32_t n_local,
                                 int32_t *out_ids, float *out_scores, void *workspace,
                                 size_t workspace_bytes, int32_t num_splits, void *stream);

/*
 * Test and debugging aid for the multi-token pass: fp32 block scores
 * out[b][p][h][j], [batch][qlen][4][max_blocks_per_seq], -inf for blocks position p does not
 * see (j >= ceil(L_p / 128)) and for pages out of range. Same scoring code as
 * msa_indexer_decode_multi.
 */
int32_t msa_indexer_block_scores_multi(const void *q, const void *k_cache,
                                       const int32_t *block_table, const int32_t *seq_lens,
                                       int32_t batch, int32_t max_blocks_per_seq,
                                       int32_t bt_stride, int64_t num_pages, int32_t qlen,
                                       float *out, int32_t num_splits, void *stream);

/*
 * msa_indexer_decode_multi over an FP8 E4M3 index-K cache (SGLang PR #41488, Accuracy and
 * Speed Tests: BF16 queries, FP8 E4M3 index caches).
 *   k_cache      uint8 [num_pages][128 tokens][128 dims], 16-byte aligned: OCP FP8 E4M3
 *                codes (exponent bias 7, subnormals, no infinities; the NaN codes 0x7F and
 *                0xFF are outside the contract). A page is 16 KiB.
 *   k_scale      the cache's one positive scale: keys are k_scale * value(code). Must be
 *                finite and > 0 (MSA_ERR_INVALID_ARG otherwise). A positive scale cannot
 *                change the selection; it scales the reported scores.
 * Every other argument, the outputs and the workspace (msa_indexer_workspace_bytes_multi)
 * as in msa_indexer_decode_multi; qlen = 1 is the single-token pass over an FP8 cache (q
 * [batch][1][4][128] is the same memory as [batch][4][128]). Scores are fp32 sums of the
 * exact products q * value(code), times k_scale once per block maximum.
 */
int32_t msa_indexer_decode_fp8(const void *q, const void *k_cache, float k_scale,
                               const int32_t *block_table, const int32_t *seq_lens, int32_t batch,
                               int32_t max_blocks_per_seq, int32_t bt_stride, int64_t num_pages,
                               int32_t qlen, int32_t topk, int32_t n_init, int32_t n_local,
                               int32_t *out_ids, float *out_scores, void *workspace,
                               size_t workspace_bytes, int32_t num_splits, void *stream);

/*
 * Test and debugging aid: msa_indexer_block_scores_multi over an FP8 E4M3 cache with scale
 * k_scale (arguments as in msa_indexer_decode_fp8).
 */
int32_t msa_indexer_block_scores_fp8(const void *q, const void *k_cache, float k_scale,
                                     const int32_t *block_table, const int32_t *seq_lens,
                                     int32_t batch, int32_t max_blocks_per_seq, int32_t bt_stride,
                                     int64_t num_pages, int32_t qlen, float *out, int32_t num_splits,
                                     void *stream);

/*
 * Stage 1 of msa_indexer_decode alone (never fused): one workgroup per (row, split) scores its blocks
 * for all 4 heads from a single read of each page and writes each head's top-Lk
 * (Lk = min(topk, C)) candidate keys of the split, best first, into the workspace. `engine` picks the scoring
 * instructions (MSA_ENGINE_*). Other arguments as in msa_indexer_decode.
 * Key layout (vLLM PR #57832, Solution step 3: one sortable int64 per candidate):
 *   bit 63 pinned | bits 62..31 order-preserving image of the fp32 score | bits 30..0
 *   (2^31-1 - block id); keys compare as unsigned integers, larger is better.
 */
int32_t msa_indexer_split_topk(const void *q, const void *k_cache, const int32_t *block_table,
                               const int32_t *seq_lens, int32_t batch,
                               int32_t max_blocks_per_seq, int32_t bt_stride, int64_t num_pages,
                               int32_t topk, int32_t n_init, int32_t n_local, void *workspace,
                               size_t workspace_bytes, int32_t num_splits, int32_t engine,
                               void *stream);

/*
 * Stage 2 of msa_indexer_decode alone: per (row, head), the exact top-min(topk, nb_b) of
 * the union of the splits' candidates, decoded into out_ids / out_scores. Exact because a
 * block in the global top-k is in the top-k of its own split (vLLM PR #57832, Solution;
 * SGLang PR #41488, Modifications). Arguments as in msa_indexer_decode; the workspace
 * must hold stage 1's keys for the same (batch, max_blocks_per_seq, topk, num_splits).
 */
int32_t msa_indexer_merge(const int32_t *seq_lens, int32_t batch, int32_t max_blocks_per_seq,
                          int32_t topk, int32_t *out_ids, float *out_scores,
                          const void *workspace, size_t workspace_bytes, int32_t num_splits,
                          void *stream);

/*
 * Test and debugging aid: the full block-score matrix out[b][h][j], fp32
 * [batch][4][max_blocks_per_seq], -inf for j >= nb_b and for blocks whose page is out of
 * range, from the same scoring code as stage 1. It is the max-score output the pages compare
 * across split counts (TensorRT-LLM PR #17008, Accuracy: max_score bitwise identical for every
 * num_kv_splits). Besides the plain form (inputs, sizes, out, stream) it takes num_splits, to
 * reproduce that check, and engine, to score with either instruction path (the MFMA-versus-VALU
 * comparison); 0 and MSA_ENGINE_DEFAULT are the decode call's choices.
 */
int32_t msa_indexer_block_scores(const void *q, const void *k_cache, const int32_t *block_table,
                                 const int32_t *seq_lens, int32_t batch,
                                 int32_t max_blocks_per_seq, int32_t bt_stride,
                                 int64_t num_pages, float *out, int32_t num_splits,
                                 int32_t engine, void *stream);

/*
 * Takes the workspace's device error bits: a one-thread kernel on `stream` reads and clears
 * the error word in one atomic step (so it is ordered after every earlier call on the stream
 * and before every later one), then the bits are copied to *host_flags and the stream is
 * synchronized. workspace must be 256-byte aligned. Returns MSA_ERR_HIP if a HIP call fails.
 */
int32_t msa_indexer_read_error(void *workspace, uint32_t *host_flags, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_INDEXER_H */
