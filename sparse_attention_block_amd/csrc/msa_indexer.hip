// msa_indexer.hip -- MI355X (gfx950) kernels and C ABI of the MiniMax-M3 lightning-indexer
// decode pass. The ABI and the operation are documented in include/msa_indexer.h.
//
// Kernels:
//   split_kernel   single-token pass over a bf16 cache, grid (S, batch), 4 waves. A
//                  workgroup owns C = ceil(W/S) consecutive logical blocks of one row (the
//                  split-KV axis of TensorRT-LLM PR #17008, Changes). Each wave walks every
//                  4th block of the split: it reads the block's page once (32 KiB, 16 B per
//                  lane per load) and scores all four heads from those registers (SGLang PR
//                  #41488, Modifications: every K tile scored for all heads while resident).
//                  Block maxima go to LDS; then wave h ranks the split's keys for head h and
//                  writes its top-k, best first. Usually the row's last workgroup then merges
//                  the row (the fused plan).
//   verify_kernel  the same decomposition for 1..4 query positions per row and for FP8
//                  caches, on the MFMA engine (4 positions x 4 heads = 16 rows).
//   merge_kernel   one wave per (row, position, head): the exact top-min(k, nb) of the
//                  splits' sorted candidate lists (vLLM PR #57832, Solution: a global top-k
//                  block is in its own shard's top-k, so the merge of the per-shard lists is
//                  exact), for unfused plans and the verify kernel.
//   expand_kernel  16-token page tables of given selections.
// Grid and workspace depend only on host arguments (batch, W, topk, S, qlen); row lengths
// are read on the device, where the decode call's device plan also picks its split width,
// and splits past a row's end return at once (vLLM PR #57832, CUDA graph capture).

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "msa_indexer.h"

// The workspace of the allocation-free decode (msa_indexer_decode_noalloc): one copy of this
// array on every GPU the library runs on, held until the process ends, shared by every such
// call on that GPU. In host code the name stands for a host-side shadow, not device memory:
// host code only ever uses the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[MSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kHeads = MSA_INDEX_HEADS;
constexpr int kDim = MSA_HEAD_DIM;
constexpr int kBlock = MSA_BLOCK_TOKENS;
constexpr int kWaves = 4;                       // waves per split workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxSplitBlocks = 64;             // C <= 64: one split candidate per lane
// Verify kernel: 8 KiB chunks in flight per wave (two measured faster than three or four).
#ifndef MSA_CHUNK_BUFFERS
#define MSA_CHUNK_BUFFERS 2
#endif
constexpr int kChunkBuffers = MSA_CHUNK_BUFFERS;
constexpr int kSpreadMaxUnits = 5;              // spread layout: splits of up to 5 blocks read at once
constexpr int kMaxSplits = 256;                 // merge: at most 4 lists per lane
constexpr int kMaxMergeKeys = 4096;             // S * Lk keys of one (row, head) in LDS
constexpr int kMaxFusedKeys = 1024;             // fused merge: S * topk keys per head, 4 heads in LDS
constexpr size_t kHeaderBytes = 256;            // workspace header (error word first)
constexpr size_t kAlign = 256;
// Each counter gets a 256-byte line of its own: atomics on one cache line serialize like
// atomics on one address (measured ~10 ns each under contention), so counters sharing a
// line would queue behind each other. A row has a row counter and 16 group counters.
constexpr int kCounterLine = 64;                // uint32 per counter line (256 B)
constexpr int kCounterGroup = 16;               // workgroups per group counter
constexpr int kCounterTwoLevel = 128;           // rows of more splits count in two levels
constexpr int kCounterStride = kCounterLine * (1 + kMaxSplits / kCounterGroup);  // uint32 per row
constexpr int kPageElems = kBlock * kDim;       // elements per page (bf16: 32 KiB, E4M3: 16 KiB)

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Index-K pages are read exactly once per pass, so their loads carry the non-temporal
// hint: streaming them past the caches measured ~13% faster than plain loads on MI355X.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------------------
// Cross-lane helpers (DPP within 16-lane rows, readlane across rows).

// Every pattern used here reads a lane of the same row, so bound_ctrl (out-of-row reads
// give 0) never applies; setting it lets the compiler fold more moves into their adds.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, dpp_u32<CTRL>(__builtin_bit_cast(uint32_t, x)));
}

constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]: partner lane ^ 1
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]: partner lane ^ 2
constexpr int kQuadSwapMid = 0xD8;    // quad_perm [0,2,1,3]: lanes 1 and 2 of each quad swap
constexpr int kRowRor4 = 0x124;       // row_ror:4 (keeps lane & 3)
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i within each 8 lanes
constexpr int kRowMirror = 0x140;     // lane i <-> 15-i within each 16 lanes

__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_f32<kQuadSwap1>(x));
  x = fmaxf(x, dpp_f32<kQuadSwap2>(x));
  x = fmaxf(x, dpp_f32<kRowHalfMirror>(x));
  x = fmaxf(x, dpp_f32<kRowMirror>(x));
  return x;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  uint32_t lo = dpp_u32<CTRL>((uint32_t)x);
  uint32_t hi = dpp_u32<CTRL>((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int lane) {
  uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, lane);
  uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// Bitonic networks on 64-bit keys over the 64 lanes of a wave (all lanes active), best
// (largest) first. A step pairs each lane with a partner, and of the two the lane with the
// lower index keeps the larger key. Stage k (k = 2, 4, .., 64) sorts blocks of k lanes:
// its first step pairs a lane with its mirror in the block (lane ^ (k - 1)), which leaves
// two bitonic halves with every key of the first at least every key of the second, and
// the half-cleaner steps after it pair lane ^ j for j = k/4, .., 1. Partners within a
// 16-lane row come from DPP (lane ^ 4 as lane ^ 3 followed by lane ^ 7); the others from
// ds_bpermute.
constexpr int kQuadRev = 0x1B;  // quad_perm [3,2,1,0]: partner lane ^ 3
constexpr int kRowRor8 = 0x128; // row_ror:8: partner lane ^ 8 within each 16 lanes

__device__ __forceinline__ uint64_t bpermute_u64(uint64_t x, int src_lane) {
  const int lo = __builtin_amdgcn_ds_bpermute(src_lane << 2, (int)(uint32_t)x);
  const int hi = __builtin_amdgcn_ds_bpermute(src_lane << 2, (int)(uint32_t)(x >> 32));
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// The key of lane ^ X.
template <int X>
__device__ __forceinline__ uint64_t partner_u64(uint64_t x) {
  if constexpr (X == 1) return dpp_u64<kQuadSwap1>(x);
  else if constexpr (X == 2) return dpp_u64<kQuadSwap2>(x);
  else if constexpr (X == 3) return dpp_u64<kQuadRev>(x);
  else if constexpr (X == 4) return dpp_u64<kRowHalfMirror>(dpp_u64<kQuadRev>(x));
  else if constexpr (X == 7) return dpp_u64<kRowHalfMirror>(x);
  else if constexpr (X == 8) return dpp_u64<kRowRor8>(x);
  else if constexpr (X == 15) return dpp_u64<kRowMirror>(x);
  else return bpermute_u64(x, (int)(__lane_id() ^ X));
}

template <int X, int UPPER>
__device__ __forceinline__ uint64_t bitonic_step(uint64_t x, int lane) {
  const uint64_t p = partner_u64<X>(x);
  return ((p > x) != ((lane & UPPER) != 0)) ? p : x;
}

// Sorts each 16-lane row that holds a bitonic sequence.
__device__ __forceinline__ uint64_t bitonic_clean16(uint64_t x, int lane) {
  x = bitonic_step<8, 8>(x, lane);
  x = bitonic_step<4, 4>(x, lane);
  x = bitonic_step<2, 2>(x, lane);
  return bitonic_step<1, 1>(x, lane);
}

// Stage k of the network: sorts every block of k lanes whose halves are sorted.
template <int K>
__device__ __forceinline__ uint64_t bitonic_stage(uint64_t x, int lane) {
  x = bitonic_step<K - 1, K / 2>(x, lane);
  if constexpr (K >= 64) x = bitonic_step<16, 16>(x, lane);
  if constexpr (K >= 32) x = bitonic_step<8, 8>(x, lane);
  if constexpr (K >= 16) x = bitonic_step<4, 4>(x, lane);
  if constexpr (K >= 8) x = bitonic_step<2, 2>(x, lane);
  if constexpr (K >= 4) x = bitonic_step<1, 1>(x, lane);
  return x;
}

// Sorts lanes 0 .. n-1 of the wave (n uniform, at most 64; the other lanes must hold 0,
// which stays behind every key): lane r < n ends with the r-th largest. Stages stop at the
// first block size k >= n, so n candidates take 1 + 2 + .. + log2(k) steps.
__device__ __forceinline__ uint64_t sort_desc_first(uint64_t x, int lane, int n) {
  if (n > 1) x = bitonic_stage<2>(x, lane);
  if (n > 2) x = bitonic_stage<4>(x, lane);
  if (n > 4) x = bitonic_stage<8>(x, lane);
  if (n > 8) x = bitonic_stage<16>(x, lane);
  if (n > 16) x = bitonic_stage<32>(x, lane);
  if (n > 32) x = bitonic_stage<64>(x, lane);
  return x;
}

// sort_desc_first of T independent key sets at once, each step applied to all T before the
// next, so that their dependency chains overlap.
template <int T, int K>
__device__ __forceinline__ void bitonic_stage_all(uint64_t (&x)[T], int lane) {
#pragma unroll
  for (int t = 0; t < T; ++t) x[t] = bitonic_step<K - 1, K / 2>(x[t], lane);
  if constexpr (K >= 64) {
#pragma unroll
    for (int t = 0; t < T; ++t) x[t] = bitonic_step<16, 16>(x[t], lane);
  }
  if constexpr (K >= 32) {
#pragma unroll
    for (int t = 0; t < T; ++t) x[t] = bitonic_step<8, 8>(x[t], lane);
  }
  if constexpr (K >= 16) {
#pragma unroll
    for (int t = 0; t < T; ++t) x[t] = bitonic_step<4, 4>(x[t], lane);
  }
  if constexpr (K >= 8) {
#pragma unroll
    for (int t = 0; t < T; ++t) x[t] = bitonic_step<2, 2>(x[t], lane);
  }
  if constexpr (K >= 4) {
#pragma unroll
    for (int t = 0; t < T; ++t) x[t] = bitonic_step<1, 1>(x[t], lane);
  }
}

template <int T>
__device__ __forceinline__ void sort_desc_first_all(uint64_t (&x)[T], int lane, int n) {
  if (n > 1) bitonic_stage_all<T, 2>(x, lane);
  if (n > 2) bitonic_stage_all<T, 4>(x, lane);
  if (n > 4) bitonic_stage_all<T, 8>(x, lane);
  if (n > 8) bitonic_stage_all<T, 16>(x, lane);
  if (n > 16) bitonic_stage_all<T, 32>(x, lane);
  if (n > 32) bitonic_stage_all<T, 64>(x, lane);
}

// Largest value over the 64 lanes of a wave (all lanes active).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  x = umax64(x, dpp_u64<kQuadSwap1>(x));
  x = umax64(x, dpp_u64<kQuadSwap2>(x));
  x = umax64(x, dpp_u64<kRowHalfMirror>(x));
  x = umax64(x, dpp_u64<kRowMirror>(x));
  return umax64(umax64(readlane_u64(x, 0), readlane_u64(x, 16)),
                umax64(readlane_u64(x, 32), readlane_u64(x, 48)));
}

// ---------------------------------------------------------------------------------------
// Candidate keys (vLLM PR #57832, Solution step 3; SGLang PR #41488: score/ID ordering).
// bit 63: pinned; bits 62..31: order-preserving image of the fp32 score (-0 folded onto +0);
// bits 30..0: 2^31-1 - block id, so equal scores rank the lower id first. Unsigned
// comparison of keys is the selection order; 0 is below every real key.

__device__ __forceinline__ uint64_t make_key(float score, int j, bool pinned) {
  uint32_t u = __builtin_bit_cast(uint32_t, score);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)pinned << 63) | ((uint64_t)ord << 31) | (uint64_t)(0x7FFFFFFF - j);
}

__device__ __forceinline__ int key_id(uint64_t key) { return 0x7FFFFFFF - (int)(key & 0x7FFFFFFFu); }

__device__ __forceinline__ float key_score(uint64_t key) {
  const uint32_t ord = (uint32_t)(key >> 31);
  const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
  return __builtin_bit_cast(float, u);
}

// ---------------------------------------------------------------------------------------
// Block scoring. Both engines take one page (128 tokens x 128 dims bf16, 32 KiB) and leave
// the four heads' block maxima in every lane of row 0 (lanes 0..15) at least.

// VALU engine. Load i of a wave covers bytes [1024 i, 1024 i + 1024) of the page: lane l
// holds token 4i + l/16, dims 8(l%16) .. +7 (fully coalesced). Each lane forms partial dot
// products of its 8 dims with bf16 dot2 instructions (fp32 accumulate) for the four heads,
// the 16 lanes of a row reduce-scatter them (row_sum4_scatter) so that each lane ends with
// the row's full sum for one head, and each lane keeps a running max of its head; rows
// merge at the end.
struct QValu {
  uint32_t d[kHeads][4];  // this lane's 8 dims of each head, as 4 bf16 pairs
};

__device__ __forceinline__ void load_q_valu(const uint16_t* __restrict__ q, int b, int lane, QValu& r) {
  const int c = lane & 15;
#pragma unroll
  for (int h = 0; h < kHeads; ++h) {
    const uint4 v = *reinterpret_cast<const uint4*>(q + ((size_t)(b * kHeads + h) * kDim + c * 8));
    r.d[h][0] = v.x; r.d[h][1] = v.y; r.d[h][2] = v.z; r.d[h][3] = v.w;
  }
}

__device__ __forceinline__ float dot8(const uint4& k, const uint32_t (&qd)[4]) {
  float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.x),
                                            __builtin_bit_cast(bf16x2_t, qd[0]), 0.0f, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.y),
                                      __builtin_bit_cast(bf16x2_t, qd[1]), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.z),
                                      __builtin_bit_cast(bf16x2_t, qd[2]), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.w),
                                      __builtin_bit_cast(bf16x2_t, qd[3]), s, false);
  return s;
}

// The four heads' sums over a 16-lane row, one head per lane: lane l ends with the row
// sum of head 2 (l & 1) + ((l >> 1) & 1) (lanes 1 and 2 swapped against l & 3). Across
// lane ^ 1, a lane keeps two heads and sends the other two; across lane ^ 2 it keeps one;
// rotations of the row by 4 and 8 (which keep l & 3) add the four quads. 9 adds/selects
// and 5 DPP moves instead of 16 DPP adds for four separate row sums.
__device__ __forceinline__ float row_sum4_scatter(float p0, float p1, float p2, float p3, bool b0, bool b1) {
  const float a0 = (b0 ? p2 : p0) + dpp_f32<kQuadSwap1>(b0 ? p0 : p2);
  const float a1 = (b0 ? p3 : p1) + dpp_f32<kQuadSwap1>(b0 ? p1 : p3);
  float x = (b1 ? a1 : a0) + dpp_f32<kQuadSwap2>(b1 ? a0 : a1);
  x += dpp_f32<kRowRor4>(x);
  x += dpp_f32<kRowRor8>(x);
  return x;
}

// A page is scored in batches of 16 wave loads (16 KiB); the compiler schedules each
// batch's loads ahead of its arithmetic.
constexpr int kValuBatch = 16;

template <bool FULL>
__device__ __forceinline__ void valu_batch(const uint4* p, int i0, int nl, int valid, int lane,
                                           const QValu& qr, float& m) {
  const int row = lane >> 4;
  const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
  uint4 kv[kValuBatch];
#pragma unroll
  for (int i = 0; i < kValuBatch; ++i)
    kv[i] = (FULL || i0 + i < nl) ? load_stream(p + (i0 + i) * 64) : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < kValuBatch; ++i) {
    const bool ok = FULL || 4 * (i0 + i) + row < valid;
    const float x = row_sum4_scatter(dot8(kv[i], qr.d[0]), dot8(kv[i], qr.d[1]), dot8(kv[i], qr.d[2]),
                                     dot8(kv[i], qr.d[3]), b0, b1);
    m = ok ? fmaxf(m, x) : m;
  }
}

// The block maximum of head (lane & 3) in lanes 0..3 (and every lane with the same lane & 3).
__device__ __forceinline__ float score_block_valu(const uint16_t* __restrict__ page, int valid,
                                                  const QValu& qr, int lane) {
  const uint4* p = reinterpret_cast<const uint4*>(page) + lane;
  float m = -__builtin_inff();
  const int nl = (valid + 3) >> 2;  // wave loads that hold a valid token
  if (valid == kBlock) {
#pragma unroll
    for (int i0 = 0; i0 < 32; i0 += kValuBatch) valu_batch<true>(p, i0, nl, valid, lane, qr, m);
  } else {
    for (int i0 = 0; i0 < nl; i0 += kValuBatch) valu_batch<false>(p, i0, nl, valid, lane, qr, m);
  }
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  return dpp_f32<kQuadSwapMid>(m);  // lane l & 3 = h now holds head h
}

// Spread layout: wave w scores quarter w of a block, tokens 32 w .. 32 w + 31, which are wave
// loads 8 w .. 8 w + 7 of the page. The maximum over its first `vw` tokens (vw <= 0: none,
// -inf) of head (lane & 3), in lanes 0..3 (and every lane with the same lane & 3).
__device__ __forceinline__ float quarter_max(const uint4 (&kv)[8], int vw, const QValu& qr, int lane) {
  const int row = lane >> 4;
  const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
  float m = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float x = row_sum4_scatter(dot8(kv[i], qr.d[0]), dot8(kv[i], qr.d[1]), dot8(kv[i], qr.d[2]),
                                     dot8(kv[i], qr.d[3]), b0, b1);
    m = 4 * i + row < vw ? fmaxf(m, x) : m;
  }
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  return dpp_f32<kQuadSwapMid>(m);
}

// Loads a wave's quarter of a page (p: the page's first uint4 plus this lane's offset and
// the quarter's; only loads that hold one of the first vw tokens when not FULL).
template <bool FULL>
__device__ __forceinline__ void quarter_load(const uint4* p, int vw, uint4 (&kv)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) kv[i] = (FULL || 4 * i < vw) ? load_stream(p + i * 64) : make_uint4(0, 0, 0, 0);
}

// MFMA engine. v_mfma_f32_16x16x32_bf16 with A = q (rows = heads, padded 4 -> 16 with
// zeros) and B = K^T (columns = 16 tokens of a tile). Lane l supplies row/column l%16 and
// 8 consecutive k-slots of lane group g = l/16; A and B use the same slots, so any fixed
// assignment of dims to slots gives the exact dot product. Step s (of 4) covers dims
// [32 s, 32 s + 32): group g takes dims 32 s + 8 g .. +7, so the four groups of one token
// read 64 contiguous bytes. The 16x16 result puts column l%16 in lane l, rows 4(l/16)..+3,
// so lanes 0..15 hold the four heads' scores of their token. Each load instruction covers
// half of sixteen 128-byte lines, so these loads stay cacheable: the line's other half is
// read by the next instruction (with the streaming hint this pattern measured ~25% slower).
struct QMfma {
  bf16x8_t a[4];  // per k-step
};

__device__ __forceinline__ void load_q_mfma(const uint16_t* __restrict__ q, int b, int lane, QMfma& r) {
  const int m = lane & 15, g = lane >> 4;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (m < kHeads) v = *reinterpret_cast<const uint4*>(q + ((size_t)(b * kHeads + m) * kDim + s * 32 + g * 8));
    r.a[s] = __builtin_bit_cast(bf16x8_t, v);
  }
}

__device__ __forceinline__ void score_block_mfma(const uint16_t* __restrict__ page, int valid,
                                                 const QMfma& qr, int lane, float (&m)[kHeads]) {
  const int n = lane & 15, g = lane >> 4;
  // uint4 index of (token 16 t + n, step s, group g) = (16 t + n) * 16 + 4 s + g
  const uint4* p = reinterpret_cast<const uint4*>(page) + n * 16 + g;
#pragma unroll
  for (int h = 0; h < kHeads; ++h) m[h] = -__builtin_inff();
  if (valid == kBlock) {
    uint4 kv[8][4];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s) kv[t][s] = p[t * 256 + s * 4];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qr.a[s], __builtin_bit_cast(bf16x8_t, kv[t][s]), acc, 0, 0, 0);
#pragma unroll
      for (int h = 0; h < kHeads; ++h) m[h] = fmaxf(m[h], acc[h]);
    }
  } else {
    for (int t = 0; 16 * t < valid; ++t) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 kv = p[t * 256 + s * 4];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qr.a[s], __builtin_bit_cast(bf16x8_t, kv), acc, 0, 0, 0);
      }
      const bool ok = 16 * t + n < valid;
#pragma unroll
      for (int h = 0; h < kHeads; ++h) m[h] = ok ? fmaxf(m[h], acc[h]) : m[h];
    }
  }
  // Lanes 0..15 hold per-token maxima of the real heads; fold the 16 columns.
#pragma unroll
  for (int h = 0; h < kHeads; ++h) m[h] = row_max16(m[h]);
}

// ---------------------------------------------------------------------------------------
// Merge of split lists (vLLM PR #57832, Solution: a block in a head's global top-k is in
// the top-k of its own shard, so the top-k of the union of the shard lists is exact).

// Copies n keys src[f(e)], e < n, into dst[g(e)] with every one of a thread's loads in
// flight before it writes any (one memory round trip instead of one per key). The keys
// were written by other workgroups, possibly on other XCDs, so they are read with
// agent-scope atomic loads (device-coherent, never a stale L2 line).
template <typename SrcIndex, typename DstIndex>
__device__ __forceinline__ void stage_keys(const uint64_t* __restrict__ src, uint64_t* dst, int n,
                                           int tid, int nthreads, SrcIndex f, DstIndex g) {
  constexpr int kBatch = 16;
  for (int base = 0; base < n; base += kBatch * nthreads) {
    uint64_t v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int e = base + j * nthreads + tid;
      v[j] = e < n ? __hip_atomic_load(src + f(e), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int e = base + j * nthreads + tid;
      if (e < n) dst[g(e)] = v[j];
    }
  }
}

// One wave, all lanes active: the m largest keys of ns lists of Lk keys each (sorted best
// first, zero padded; list sp starts at lk[sp * stride]) held in LDS, by m rounds of "take
// the largest list head". Lane l owns lists l, l+64, l+128, l+192. Lane i < m returns the
// i-th key. Used when the lists are too many or too long for merge_top16.
__device__ __forceinline__ uint64_t merge_rounds(const uint64_t* lk, int ns, int Lk, int stride, int m,
                                                 int lane) {
  constexpr int kLists = kMaxSplits / 64;
  uint64_t head[kLists];
  int ptr[kLists];
#pragma unroll
  for (int r = 0; r < kLists; ++r) {
    const int sp = lane + 64 * r;
    ptr[r] = 0;
    head[r] = sp < ns ? lk[sp * stride] : 0;
  }
  uint64_t mine = 0;
  for (int i = 0; i < m; ++i) {
    uint64_t best = head[0];
#pragma unroll
    for (int r = 1; r < kLists; ++r) best = umax64(best, head[r]);
    const uint64_t w = wave_max_u64(best);
    if (lane == i) mine = w;
#pragma unroll
    for (int r = 0; r < kLists; ++r) {
      if (head[r] == w) {  // keys are distinct: exactly one list holds w
        const int sp = lane + 64 * r;
        ++ptr[r];
        head[r] = ptr[r] < Lk ? lk[sp * stride + ptr[r]] : 0;
      }
    }
  }
  return mine;
}

// Top 16 of sorted lists with a bitonic merge network held in registers (one wave, all
// lanes active): ns lists with ns * Lk2 <= 1024 (network_fits). Every list is best first
// with Lk <= 16 keys; rounded up to
// Lk2 = 2^lg >= Lk (zero padded), 16 / Lk2 lists share a 16-lane row, so a register holds
// 64 / Lk2 lists: lane l of register t reads element l % Lk2 of list
// t * (64 / Lk2) + l / Lk2. Each row is first sorted from its runs of Lk2 into 16 (the
// network's stages 2 Lk2 .. 16). Two sorted rows A and B of 16 merge into their top 16 as
// max(A[i], B[15 - i]), which is bitonic, followed by a half-cleaner (bitonic_clean16):
// registers merge pairwise in the same lane (B mirrored within its row; a register with
// no partner is left as it is), then the four rows of the last register merge with their
// mirrored neighbours (lane ^ 31, then lane ^ 63). Every row ends with the same 16 keys;
// lane i < 16 returns the i-th largest, and for m <= 16 the first m are the m largest of
// the union (the merge of vLLM PR #57832, Solution, with a network in place of repeated
// extraction). The lists may have been written by other workgroups on other XCDs, so they
// are read with agent-scope atomic loads (device-coherent), all in flight at once.
constexpr int kNetworkMaxM = 16;
constexpr int kNetworkKeys = 16 * 64;  // 16 registers of 64 lanes

__device__ __host__ __forceinline__ int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Whether merge_top16 takes ns lists of Lk keys for a top-`topk` selection.
__device__ __host__ __forceinline__ bool network_fits(int ns, int Lk, int topk) {
  return topk <= kNetworkMaxM && ns * pow2_at_least(Lk) <= kNetworkKeys;
}

// One level of the register tree: r[t] takes the top 16 of r[t] and r[t + HALF], t < HALF.
// The HALF merges are independent; each step is applied to all of them before the next, so
// their dependency chains overlap.
template <int HALF>
__device__ __forceinline__ void merge_level(uint64_t (&r)[16], int lane) {
#pragma unroll
  for (int t = 0; t < HALF; ++t) r[t] = umax64(r[t], partner_u64<15>(r[t + HALF]));
#pragma unroll
  for (int t = 0; t < HALF; ++t) r[t] = bitonic_step<8, 8>(r[t], lane);
#pragma unroll
  for (int t = 0; t < HALF; ++t) r[t] = bitonic_step<4, 4>(r[t], lane);
#pragma unroll
  for (int t = 0; t < HALF; ++t) r[t] = bitonic_step<2, 2>(r[t], lane);
#pragma unroll
  for (int t = 0; t < HALF; ++t) r[t] = bitonic_step<1, 1>(r[t], lane);
}

// Sorts each row of r[0 .. N) from its runs of 2^lg keys into 16 (stages 2^(lg+1) .. 16),
// the N registers step by step together.
template <int N>
__device__ __forceinline__ void sort_rows(uint64_t (&r)[16], int lg, int lane) {
  if (lg < 1) {
#pragma unroll
    for (int t = 0; t < N; ++t) r[t] = bitonic_stage<2>(r[t], lane);
  }
  if (lg < 2) {
#pragma unroll
    for (int t = 0; t < N; ++t) r[t] = bitonic_step<3, 2>(r[t], lane);
#pragma unroll
    for (int t = 0; t < N; ++t) r[t] = bitonic_step<1, 1>(r[t], lane);
  }
  if (lg < 3) {
#pragma unroll
    for (int t = 0; t < N; ++t) r[t] = bitonic_step<7, 4>(r[t], lane);
#pragma unroll
    for (int t = 0; t < N; ++t) r[t] = bitonic_step<2, 2>(r[t], lane);
#pragma unroll
    for (int t = 0; t < N; ++t) r[t] = bitonic_step<1, 1>(r[t], lane);
  }
#pragma unroll
  for (int t = 0; t < N; ++t) r[t] = bitonic_step<15, 8>(r[t], lane);
#pragma unroll
  for (int t = 0; t < N; ++t) r[t] = bitonic_step<4, 4>(r[t], lane);
#pragma unroll
  for (int t = 0; t < N; ++t) r[t] = bitonic_step<2, 2>(r[t], lane);
#pragma unroll
  for (int t = 0; t < N; ++t) r[t] = bitonic_step<1, 1>(r[t], lane);
}

// The 16 largest keys of registers r[0 .. R) (R <= 16; the registers past R hold zeros),
// whose 16-lane rows hold sorted runs of 2^lg keys: best first in lanes 0..15.
__device__ __forceinline__ uint64_t network_top16(uint64_t (&r)[16], int R, int lg, int lane) {
  // Registers past R hold zeros: sorting or merging them changes nothing, so the stages
  // below run on power-of-two register counts without a branch per register.
  if (lg < 4) {  // several lists per row: sort each row first
    if (R > 8) sort_rows<16>(r, lg, lane);
    else if (R > 4) sort_rows<8>(r, lg, lane);
    else if (R > 2) sort_rows<4>(r, lg, lane);
    else if (R > 1) sort_rows<2>(r, lg, lane);
    else sort_rows<1>(r, lg, lane);
  }
  if (R > 8) merge_level<8>(r, lane);
  if (R > 4) merge_level<4>(r, lane);
  if (R > 2) merge_level<2>(r, lane);
  if (R > 1) merge_level<1>(r, lane);
  uint64_t x = r[0];
  x = bitonic_clean16(umax64(x, partner_u64<31>(x)), lane);
  x = bitonic_clean16(umax64(x, partner_u64<63>(x)), lane);
  return x;
}

// The 16 largest keys of ns lists of Lk keys (each sorted best first, zero padded; list sp
// at lists[sp * list_stride], written by split sp, which owns blocks [sp * C, sp * C + C)),
// best first in lanes 0..15. Lists are padded to Lk2 = 2^ceil(log2 Lk) keys and 64 / Lk2
// of them share a register: lane l of register t holds element l % Lk2 of list
// t * 64 / Lk2 + l / Lk2.
// Many short lists (more than 8 registers of lists of at most 8 keys, e.g. 256 splits of 4
// blocks; more than 3 registers of lists of 2 to 8 keys; 2 or more of one-key lists) are
// pruned first: the 16th largest list head is at most the 16th largest key (the
// 16 best heads are 16 keys), and a list's keys are at most its head, so every key of the
// top 16 lies in one of the 16 lists with the best heads. The heads (at most 256, 4
// registers) are ranked first, and only those 16 lists (16 Lk2 keys, 1 or 2 registers) are
// read and merged: a second round of loads, but about a third of the network's steps
// (sorting 16 registers of short runs is its largest part). A head names its list: its
// block id divided by C (so lists of even splits, whose widths differ, are never pruned:
// prune = false).
// merge_top16 in two phases, for a caller that can issue the first round of loads before it
// needs their values: merge_issue reads every key (or, pruned, every list head) into r,
// merge_finish merges them.
struct MergeShape {
  int lg;       // log2 Lk2
  int R;        // registers that hold a list
  bool pruned;
};

__device__ __forceinline__ MergeShape merge_shape(int ns, int Lk, bool prune) {
  MergeShape m;
  m.lg = Lk <= 1 ? 0 : Lk <= 2 ? 1 : Lk <= 4 ? 2 : Lk <= 8 ? 3 : 4;
  const int per_reg = 64 >> m.lg;
  m.R = (ns + per_reg - 1) / per_reg;
  // Pruned: more than 8 registers of lists, or more than 3 of lists of 2 to 8 keys (measured
  // ahead there since the lists of one head lie together), or 2 or more registers of one-key
  // lists, whose heads are the keys (the ranking of the heads is then the answer).
  m.pruned = prune && m.lg < 4 && (m.R > 8 || (m.lg >= 1 && m.R > 3) || (m.lg == 0 && m.R >= 2));
  return m;
}

__device__ __forceinline__ void merge_issue(const uint64_t* __restrict__ lists, size_t list_stride, int ns,
                                            int Lk, const MergeShape& m, int lane, uint64_t (&r)[16]) {
  if (m.pruned) {
    const int RH = (ns + 63) / 64;  // registers of list heads, one head per lane
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int sp = t * 64 + lane;
      r[t] = (t < RH && sp < ns)
                 ? __hip_atomic_load(lists + sp * list_stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                 : 0;
    }
    return;
  }
  const int per_reg = 64 >> m.lg, sub = lane >> m.lg, e = lane & ((1 << m.lg) - 1);
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int sp = t * per_reg + sub;
    r[t] = (t < m.R && sp < ns && e < Lk)
               ? __hip_atomic_load(lists + sp * list_stride + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
               : 0;
  }
}

__device__ __forceinline__ uint64_t merge_finish(const uint64_t* __restrict__ lists, size_t list_stride, int ns,
                                                 int Lk, int C, const MergeShape& m, int lane,
                                                 uint64_t (&r)[16]) {
  if (!m.pruned) return network_top16(r, m.R, m.lg, lane);
  const int lg = m.lg, RH = (ns + 63) / 64;
  const int e = lane & ((1 << lg) - 1);
  uint64_t head;
  if (RH >= 2) {
    // Lanes pruned first, by the same argument with a lane's heads as its list: the 16 best
    // heads lie among the heads of the 16 lanes with the best maxima. Those lanes' heads
    // (at most 64) are gathered into one register, head t of the i-th best lane into lane
    // 4 i + t, and ranked there: two one-register networks instead of one over RH.
    uint64_t mx = r[0];
#pragma unroll
    for (int t = 1; t < 4; ++t) mx = t < RH ? umax64(mx, r[t]) : mx;
    uint64_t q[16] = {mx};
    const uint64_t best = network_top16(q, 1, 0, lane);         // lane i < 16: i-th best maximum
    const int holder = best != 0 ? (key_id(best) / C) & 63 : -1;  // the lane that holds it
    const int from = __shfl(holder, lane >> 2);
    uint64_t c = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint64_t v = bpermute_u64(r[t], from < 0 ? lane : from);
      c = (from >= 0 && (lane & 3) == t) ? v : c;
    }
    uint64_t g[16] = {c};
    head = network_top16(g, 1, 0, lane);
  } else {
    head = network_top16(r, RH, 0, lane);
  }
  if (lg == 0) return head;  // one key per list: the best heads are the best keys
  const int src = head != 0 ? key_id(head) / C : -1;  // lane i < 16: the list of the i-th best head
  const int R2 = max(1, (16 << lg) / 64);             // registers of the 16 lists' keys
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int i = (t * 64 + lane) >> lg;  // rank of the list this slot holds
    const int sp = t < R2 ? __shfl(src, i & 15) : -1;
    r[t] = (t < R2 && i < 16 && e < Lk && sp >= 0)
               ? __hip_atomic_load(lists + sp * list_stride + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
               : 0;
  }
  return network_top16(r, R2, lg, lane);
}

__device__ __forceinline__ uint64_t merge_top16(const uint64_t* __restrict__ lists, size_t list_stride,
                                                int ns, int Lk, int C, int lane, bool prune = true) {
  const MergeShape m = merge_shape(ns, Lk, prune);
  uint64_t r[16];
  merge_issue(lists, list_stride, ns, Lk, m, lane, r);
  return merge_finish(lists, list_stride, ns, Lk, C, m, lane, r);
}

__device__ __forceinline__ void write_selection(uint64_t mine, int m, int topk, int lane,
                                                int32_t* oid, float* osc) {
  if (lane < topk) {
    oid[lane] = lane < m ? key_id(mine) : -1;
    osc[lane] = lane < m ? key_score(mine) : -__builtin_inff();
  }
}

// ---------------------------------------------------------------------------------------
// 16-token page table of one (row, head), for a sparse-attention consumer that pages KV in
// 16-token pages (vLLM blog "Following the Bottleneck", section 3, Figure 5: each selected
// 128-token block stands for its physical block's eight 16-token pages; only the table is
// built, the cache stays in place). Lane i < topk holds block id `id`, `valid` when it names
// a block of the row. The valid blocks go out in ascending logical order, block i of that
// order as entries 8i .. 8i+7 = 8 * page + t (modulo 2^32); the remaining entries up to
// 8 topk are -1. *tokens = the valid blocks' tokens. All 64 lanes must be active.

__device__ __forceinline__ void emit_pages(int id, bool valid, int topk, int lane,
                                           const int32_t* __restrict__ btrow, int L,
                                           int32_t* __restrict__ pages, int32_t* __restrict__ tokens) {
  // Sorted descending, ~((id << 6) | lane) puts the valid lanes first in ascending
  // (id, lane) order (repeated ids keep one slot each) and the invalid ones (0) after:
  // slot i takes the i-th sorted entry.
  valid = valid && id >= 0 && id < (L + kBlock - 1) / kBlock;
  const uint64_t ord = valid ? ~(((uint64_t)(uint32_t)id << 6) | (uint64_t)lane) : 0;
  const uint64_t mine = sort_desc_first(ord, lane, topk);
  const int n = __popcll(__ballot(valid));
  if (lane < topk) {
    int4 lo = make_int4(-1, -1, -1, -1), hi = lo;
    if (lane < n && mine != 0) {
      const uint32_t p = (uint32_t)btrow[(int)(uint32_t)(~mine >> 6)] * 8u;
      lo = make_int4((int)p, (int)(p + 1), (int)(p + 2), (int)(p + 3));
      hi = make_int4((int)(p + 4), (int)(p + 5), (int)(p + 6), (int)(p + 7));
    }
    int4* dst = reinterpret_cast<int4*>(pages + (size_t)lane * 8);
    dst[0] = lo;
    dst[1] = hi;
  }
  // Each lane's count is at most 128: sum it bit by bit over the wave.
  const int cnt = valid ? min(kBlock, L - id * kBlock) : 0;
  int total = 0;
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) total += __popcll(__ballot((cnt >> bit) & 1)) << bit;
  if (lane == 0) *tokens = total;
}

// ---------------------------------------------------------------------------------------
// Stage 1.
//
// Row b gets ns = ceil(nb / C) workgroups; workgroup s owns the contiguous blocks
// [s*C, min((s+1)*C, nb)) (the split-KV decomposition of TensorRT-LLM PR #17008,
// Changes), wave w scoring every 4th of them. Each workgroup then ranks its blocks' keys
// per head and keeps the top Lk = min(topk, C). The last of the row's workgroups to
// finish resets the row's counter and, in the fused mode, merges the row.

enum Mode { kScores = 0, kSplit = 1, kFused = 2 };

// The most splits of C blocks a row may have under the device plan: its lists (ns *
// min(topk, C) keys per head) must fit the S * topk keys the workspace holds per row and
// head, and the merge network. At topk = 16, S = 64: 256, 128, 64, 64, 64 for C = 4 .. 64,
// i.e. rows of up to 1024 blocks at C <= 16, 2048 at 32 and 4096 at 64.
__device__ __host__ __forceinline__ int device_max_splits(int C, int S, int topk) {
  const int lk = min(topk, C);
  return min(S * topk / lk, kNetworkKeys / pow2_at_least(lk));
}

// The longest row (in blocks) that splits of 4 << t blocks may cover, t = 0 .. 4; computed
// on the host for the call's S and topk.
struct SplitLimits {
  int32_t blocks[5];
};

// The device plan's split width and splits per row in the case that every row is W blocks
// long, computed on the host with the arithmetic of device_split_width (C = 0: not under
// the device plan). See rows_full.
struct FullRowPlan {
  int32_t C, ns;
};

SplitLimits split_limits(int S, int topk) {
  SplitLimits l;
  for (int t = 0; t < 5; ++t) l.blocks[t] = device_max_splits(4 << t, S, topk) * (4 << t);
  return l;
}

struct SplitArgs {
  const uint16_t* q;
  const uint16_t* k;
  const int32_t* bt;
  const int32_t* lens;
  int32_t W, bt_stride;
  int64_t num_pages;
  int32_t S, C, Lk, topk, n_init, n_local;
  int32_t batch;
  int32_t device_plan;  // fused mode: C and each workgroup's (row, split) chosen on the device
  int32_t spread;       // VALU engine, not block-score mode: each wave scores a quarter of every block
  int32_t even;         // host plan: the first W - S (C - 1) splits of a row cover C blocks, the rest C - 1
  SplitLimits lim;      // device plan: per-row block limits of each split width
  FullRowPlan full;     // device plan: the plan when every row is W blocks long
  uint64_t* keys;       // [batch][4][S * LkMax] (list_offset)
  uint32_t* err;        // device error word (may be null)
  uint32_t* counters;   // [batch][kCounterStride]: row and group counters (count_in); zero between calls
  int32_t* out_ids;     // [batch][4][topk] (fused mode)
  float* out_scores;    // [batch][4][topk] (fused mode)
  int32_t* out_pages;   // [batch][4][8 topk] 16-token page table (fused mode; may be null)
  int32_t* out_tokens;  // [batch][4] tokens in that table (with out_pages)
  float* scores;        // [batch][4][W] (block-score mode)
};

__device__ __forceinline__ int row_tokens(const int32_t* lens, int b, int W) {
  const int L = lens[b];
  return L < 0 ? 0 : (L > W * kBlock ? W * kBlock : L);
}

// Tokens that query position p of Q sees in a row of L tokens (the row's last Q tokens are
// its query positions; TensorRT-LLM PR #17008, Description: the causal clamp).
__device__ __forceinline__ int causal_len(int L, int Q, int p) { return max(0, L - (Q - 1 - p)); }

// ---------------------------------------------------------------------------------------
// The device plan (the fused single-token pass, and the split passes of the multi-token and
// FP8 calls). The host launches a 1-D grid sized from its arguments alone; every workgroup
// then reads the row lengths and picks the same split width C: about 512 workgroups in all
// (measured best for uniform batches: 4..32 rows of 128K tokens), at least 4 blocks per
// split, and no more splits in any row than its lists can hold (device_max_splits: up to
// 256 at C = 4), so a long row among short ones still spreads over the chip. Row b takes
// max(1, ceil(nb_b / C)) consecutive workgroup ids (an empty row one, to write its
// padding); workgroups past the last row have nothing to do.
constexpr int kDeviceTarget = 512;     // workgroups the device plan aims at
constexpr int kDeviceMaxSplits = 64;   // splits per row at 16 or more blocks per split
// Tables of fewer blocks (batch x W) keep the host plan: the device plan's prologue (the
// row lengths read before any page) costs ~1 us, which only pays where a row can be long.
constexpr int64_t kDeviceMinBlocks = 8192;

// Inclusive prefix sum over the 64 lanes, without LDS: DPP adds within each 16-lane row (the
// lanes 1, 2 and 3 below, then 4 and 8 below with the bank masks that keep a row's lower lanes
// out), then the row broadcasts of lane 15 to rows 1 and 3 and of lane 31 to rows 2 and 3.
// Seven dependent adds, where a ballot per bit takes one ballot, two mbcnt and an add per bit.
template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ int dpp_or_zero(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, BANK_MASK, false);
}

__device__ __forceinline__ int wave_scan(int x) {
  int s = x + dpp_or_zero<0x111, 0xF, 0xF>(x);   // row_shr:1
  s += dpp_or_zero<0x112, 0xF, 0xF>(x);          // row_shr:2
  s += dpp_or_zero<0x113, 0xF, 0xF>(x);          // row_shr:3
  s += dpp_or_zero<0x114, 0xF, 0xE>(s);          // row_shr:4, lanes 4..15 of each row
  s += dpp_or_zero<0x118, 0xF, 0xC>(s);          // row_shr:8, lanes 8..15 of each row
  s += dpp_or_zero<0x142, 0xA, 0xF>(s);          // row_bcast:15 into rows 1 and 3
  s += dpp_or_zero<0x143, 0xC, 0xF>(s);          // row_bcast:31 into rows 2 and 3
  return s;
}

__device__ __forceinline__ int wave_sum(int x) { return __builtin_amdgcn_readlane(wave_scan(x), 63); }

// Largest of the 64 lanes' non-negative values.
__device__ __forceinline__ int wave_max_nonneg(int x) {
  uint32_t u = (uint32_t)x;
  u = max(u, dpp_u32<kQuadSwap1>(u));
  u = max(u, dpp_u32<kQuadSwap2>(u));
  u = max(u, dpp_u32<kRowHalfMirror>(u));
  u = max(u, dpp_u32<kRowMirror>(u));
  return (int)max(max((uint32_t)__builtin_amdgcn_readlane((int)u, 0), (uint32_t)__builtin_amdgcn_readlane((int)u, 16)),
                  max((uint32_t)__builtin_amdgcn_readlane((int)u, 32), (uint32_t)__builtin_amdgcn_readlane((int)u, 48)));
}

// Where the list of split s, task t (position-head p * 4 + h) of row b starts in the
// workspace keys: rows lie S * QH * LkMax keys apart (LkMax = the plan's Lk; topk under
// the device plan), a row's tasks S * LkMax keys apart, and a task's lists follow one another
// (this call's Lk = min(topk, C) keys each; at most S * LkMax keys in all). The merging wave
// of a task then reads its lists from consecutive lines: the heads of 256 lists of 4 lie in
// 64 lines of 128 bytes, not 256 (the agent-scope loads go to the memory side line by line).
__device__ __forceinline__ size_t list_offset(int b, int S, int QH, int LkMax, int s, int t, int Lk) {
  return ((size_t)b * QH + t) * S * LkMax + (size_t)s * Lk;
}

// Thread 0 of a workgroup that has published its lists (split s of the row's ns): whether it
// is the last of them, i.e. whether it merges the row. row points at the row's counter
// block: the row counter in its first 256-byte line, group counters in the next 16. A row of
// more than 128 splits counts in two levels, 16 splits per group counter and then the
// groups' last workgroups on the row counter, because increments of one line serialize:
// 256 workgroups finishing together on one counter cost ~1.2 us more than 16 groups (the
// second level adds one atomic round trip, which only pays past 128 splits). Every counter
// is back at zero when the call ends.
__device__ __forceinline__ bool count_in(uint32_t* row, int s, int ns) {
  if (ns > kCounterTwoLevel) {
    const int g = s / kCounterGroup;
    const int members = min(kCounterGroup, ns - g * kCounterGroup);
    uint32_t* group = row + kCounterLine * (1 + g);
    if (__hip_atomic_fetch_add(group, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != (uint32_t)(members - 1))
      return false;
    __hip_atomic_store(group, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ns = (ns + kCounterGroup - 1) / kCounterGroup;
  }
  if (__hip_atomic_fetch_add(row, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != (uint32_t)(ns - 1)) return false;
  __hip_atomic_store(row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

struct DevicePlan {
  int C, b, s;
  bool active;
  int L;  // the row's tokens (clamped), so the workgroup need not read its length again
};

// Wave-uniform: every lane of every wave computes the same plan. Lane l reads the lengths
// of rows l, l+64, ... (rows past the first 64 are read again in the second pass; they are
// cache hits); sums and prefix sums are DPP scans and the longest-row bounds ballots, without
// LDS.
__device__ __forceinline__ int device_blocks(const int32_t* lens, int batch, int W, int r) {
  return r < batch ? (row_tokens(lens, r, W) + kBlock - 1) / kBlock : 0;
}

// The split width C of the device plan (the same in every lane); nb0 = this lane's row's
// block count, device_blocks(lens, batch, W, lane). A row fits C = 4 << t when it has at
// most lim.blocks[t] blocks.
__device__ __forceinline__ int device_split_width(const int32_t* lens, int batch, int W, int lane, int nb0,
                                                  const SplitLimits& lim) {
  auto blocks = [&](int r) { return device_blocks(lens, batch, W, r); };
  int N = 0;
  bool over[5] = {false, false, false, false, false};  // a row does not fit splits of 4 << t blocks
  for (int r0 = 0; r0 < batch; r0 += 64) {
    const int nb = r0 == 0 ? nb0 : blocks(r0 + lane);
    N += wave_sum(nb);
#pragma unroll
    for (int t = 0; t < 5; ++t) over[t] = over[t] || __ballot(nb > lim.blocks[t]) != 0;
  }
  int C_min = 4;
#pragma unroll
  for (int t = 0; t < 5; ++t) C_min = over[t] ? (4 << (t + 1)) : C_min;
  return min(max(pow2_at_least(max(1, (N + kDeviceTarget - 1) / kDeviceTarget)), C_min), kMaxSplitBlocks);
}

// Whether every row (at most 64 of them) is W blocks long, given this lane's row's block
// count nb0. The plan is then the full-row plan the host computed (the same arithmetic as
// device_split_width over W-block rows), and the workgroups take it from one ballot instead
// of the general plan's ballot sums and prefix scans (0.7-1.1 us per call at the
// 32 x 1024-block benchmark shape).
__device__ __forceinline__ bool rows_full(int batch, int W, int lane, int nb0, const FullRowPlan& full) {
  return full.C > 0 && batch <= 64 && __ballot(lane < batch && nb0 != W) == 0;
}

// The device plan's split width (the same in every lane and every kernel of a call).
__device__ __forceinline__ int device_width(const int32_t* lens, int batch, int W, int lane, int nb0,
                                            const SplitLimits& lim, const FullRowPlan& full) {
  return rows_full(batch, W, lane, nb0, full) ? full.C : device_split_width(lens, batch, W, lane, nb0, lim);
}

__device__ __forceinline__ DevicePlan device_plan(const int32_t* lens, int batch, int W,
                                                  const SplitLimits& lim, const FullRowPlan& full,
                                                  int g, int lane) {
  auto tokens = [&](int r) { return r < batch ? row_tokens(lens, r, W) : 0; };
  const int L0 = tokens(lane);
  const int nb0 = (L0 + kBlock - 1) / kBlock;
  if (rows_full(batch, W, lane, nb0, full)) {
    const int b = g / full.ns;
    return DevicePlan{full.C, b, g - b * full.ns, b < batch, __builtin_amdgcn_readlane(L0, min(b, 63))};
  }
  const int C = device_split_width(lens, batch, W, lane, nb0, lim);
  const int log2C = __builtin_ctz(C);  // C is a power of two
  if (batch <= 64) {
    // The row with the most splits (the first such) takes workgroups 0, 1, .., the rows after
    // it follow in order and wrap around. Workgroups are dispatched in order, one per CU
    // until every CU holds one; a later one shares a CU with an earlier one, whose waves are
    // older and win the CU's arbitration, so it finishes later. The longest row, whose merge
    // also ends the call, then never waits for a second workgroup on its CUs.
    const int cnt = lane < batch ? max(1, (nb0 + C - 1) >> log2C) : 0;
    const int inclusive = wave_scan(cnt);
    const int total = __builtin_amdgcn_readlane(inclusive, 63);
    const int top = wave_max_nonneg(cnt);
    const int r0 = __builtin_ctzll(__ballot(lane < batch && cnt == top));
    const int shift = __builtin_amdgcn_readlane(inclusive, r0) - __builtin_amdgcn_readlane(cnt, r0);
    int gr = g;
    if (g < total) {
      gr = g + shift;
      if (gr >= total) gr -= total;
    }
    const uint64_t hit = __ballot(lane < batch && gr >= inclusive - cnt && gr < inclusive);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      return DevicePlan{C, l, gr - (__builtin_amdgcn_readlane(inclusive, l) - __builtin_amdgcn_readlane(cnt, l)),
                        true, __builtin_amdgcn_readlane(L0, l)};
    }
    return DevicePlan{C, 0, 0, false, 0};
  }
  int base = 0;
  for (int r0 = 0; r0 < batch; r0 += 64) {
    const int r = r0 + lane;
    const int L = r0 == 0 ? L0 : tokens(r);
    const int nb = (L + kBlock - 1) / kBlock;
    const int cnt = r < batch ? max(1, (nb + C - 1) >> log2C) : 0;
    const int inclusive = wave_scan(cnt);
    const int first = base + inclusive - cnt;
    const uint64_t hit = __ballot(r < batch && g >= first && g < first + cnt);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      return DevicePlan{C, r0 + l, g - __builtin_amdgcn_readlane(first, l), true, __builtin_amdgcn_readlane(L, l)};
    }
    base += __builtin_amdgcn_readlane(inclusive, 63);
  }
  return DevicePlan{C, 0, 0, false, 0};
}

// Block j of the row, held in cache page `page`: the maximum of head (lane & 3), valid in
// lanes 0..3.
// Entry j of a block-table row, read with a scalar load (wave-uniform j). The table is
// only read during a call, and the scalar cache starts each dispatch invalidated. A vector
// load here would count in the wave's vector memory counter, which completes in order: the
// wait for the page number would also wait for every chunk load issued before it, draining
// the pipeline at each block boundary; the scalar load waits on the LDS/scalar counter only.
__device__ __forceinline__ int table_entry(const int32_t* row, int j) {
  typedef const __attribute__((address_space(4))) int32_t* const_row_t;
  return ((const_row_t)row)[j];
}

template <int ENGINE>
__device__ __forceinline__ float score_page(const SplitArgs& a, int page, int j, int L, int lane,
                                            const void* qr) {
  const int valid = min(kBlock, L - j * kBlock);
  if (page < 0 || (int64_t)page >= a.num_pages) {
    if (a.err != nullptr && lane == 0) atomicOr(a.err, (uint32_t)MSA_DEVERR_PAGE_OUT_OF_RANGE);
    return -__builtin_inff();
  }
  const uint16_t* pg = a.k + (size_t)page * kPageElems;
  if constexpr (ENGINE == MSA_ENGINE_MFMA) {
    float m[kHeads];
    score_block_mfma(pg, valid, *static_cast<const QMfma*>(qr), lane, m);
    const int h = lane & 3;
    return h == 0 ? m[0] : h == 1 ? m[1] : h == 2 ? m[2] : m[3];
  } else {
    return score_block_valu(pg, valid, *static_cast<const QValu*>(qr), lane);
  }
}

// SPREAD (VALU engine, not block-score mode): the spread layout, each wave scoring a quarter of
// every block of the split (chosen on the host, SplitArgs::spread).
template <int ENGINE, int MODE, bool SPREAD>
__global__ __launch_bounds__(kThreads) void split_kernel(SplitArgs a) {
  static_assert(!SPREAD || (ENGINE == MSA_ENGINE_VALU && MODE != kScores), "spread: VALU engine, lists");
  extern __shared__ uint64_t lk[];  // fused mode: [S][4][Lk] lists of one row, then merge scratch
  __shared__ float sc[SPREAD ? kWaves : 1][kMaxSplitBlocks][kHeads];  // block maxima (spread: per quarter)
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr bool spread = SPREAD;
  int s = blockIdx.x, b = blockIdx.y, C = a.C;
  int Ldp = -1;  // the device plan's row length (clamped): no second read of it
  if (MODE == kFused && a.device_plan) {
    const DevicePlan dp = device_plan(a.lens, a.batch, a.W, a.lim, a.full, blockIdx.x, lane);
    if (!dp.active) return;
    s = dp.s;
    b = dp.b;
    C = dp.C;
    Ldp = dp.L;
  }
  // Even splits: the first `wide` = W - S (C - 1) splits of a row are C blocks long, the rest
  // C - 1. Workgroups start in the order of their linear id, the 256th ~1.6 us after the first,
  // so every row's wide splits take the first ids: they start earliest and end with the
  // narrow ones instead of after them.
  const int wide = a.W - a.S * (C - 1);
  if (MODE != kScores && a.even) {
    const int g = blockIdx.y * a.S + blockIdx.x;
    if (g < a.batch * wide) {
      b = g / wide;
      s = g - b * wide;
    } else {
      const int k = g - a.batch * wide, narrow = a.S - wide;
      b = k / narrow;
      s = wide + (k - b * narrow);
    }
  }
  const int Lk = min(a.topk, C);
  // The wave's first page number and the row's query are read together with the row
  // length rather than after it (the table row has W entries, so the read is in bounds
  // whatever the length); each page number after it is read while the page before it is
  // being scored.
  const int32_t* btrow = a.bt + (size_t)b * a.bt_stride;
  // The split's first block (with even splits, s (C - 1) + min(s, wide)).
  const int j_start = MODE != kScores && a.even ? s * (C - 1) + min(s, wide) : s * C;
  const int j_first = j_start + wave;
  int page = !spread && j_first < a.W ? btrow[j_first] : 0;
  // Spread layout: lane u < C holds the page number of the split's block j_start + u.
  const int pg_spread = spread && lane < C && j_start + lane < a.W ? btrow[j_start + lane] : -1;
  typename std::conditional<ENGINE == MSA_ENGINE_MFMA, QMfma, QValu>::type qr;
  if constexpr (ENGINE == MSA_ENGINE_MFMA) load_q_mfma(a.q, b, lane, qr);
  else load_q_valu(a.q, b, lane, qr);
  const int L = Ldp >= 0 ? Ldp : row_tokens(a.lens, b, a.W);
  const int nb = (L + kBlock - 1) / kBlock;

  if (MODE == kScores) {  // block scores out; -inf at and past the row's end
    const int j0 = s * C, j1 = min(j0 + C, nb);
    const int e0 = max(j0, nb), e1 = min(j0 + C, a.W);
    for (int idx = threadIdx.x; idx < (e1 - e0) * kHeads; idx += kThreads) {
      const int h = idx / (e1 - e0), j = e0 + idx % (e1 - e0);
      a.scores[((size_t)b * kHeads + h) * a.W + j] = -__builtin_inff();
    }
    if (j0 >= nb) return;
    for (int j = j0 + wave; j < j1; j += kWaves) {
      const int next = j + kWaves < j1 ? btrow[j + kWaves] : 0;
      const float m = score_page<ENGINE>(a, page, j, L, lane, &qr);
      if (lane < kHeads) a.scores[((size_t)b * kHeads + lane) * a.W + j] = m;
      page = next;
    }
    return;
  }

  // Workgroups that take part in this row (with even splits, those that start below nb).
  const int ns = !a.even ? (nb + C - 1) / C
                 : nb <= wide * C ? (nb + C - 1) / C : wide + (nb - wide * C + C - 2) / (C - 1);
  const int j0 = j_start;
  const int j1 = min(a.even ? (s + 1) * (C - 1) + min(s + 1, wide) : j0 + C, nb);
  if (s >= ns) {
    // An empty row has no workgroup to merge it: its first workgroup writes the padding.
    if (MODE == kFused && nb == 0 && s == 0) {
      if ((int)threadIdx.x < kHeads * a.topk) {
        const size_t o = (size_t)b * kHeads * a.topk + threadIdx.x;
        a.out_ids[o] = -1;
        a.out_scores[o] = -__builtin_inff();
      }
      if (a.out_pages != nullptr) {
        for (int e = threadIdx.x; e < kHeads * a.topk * 8; e += kThreads)
          a.out_pages[(size_t)b * kHeads * a.topk * 8 + e] = -1;
        if (threadIdx.x < kHeads) a.out_tokens[(size_t)b * kHeads + threadIdx.x] = 0;
      }
    }
    return;
  }
  if constexpr (SPREAD) {
    {
      // Wave w takes quarter w of each of the split's n blocks ("units" 0 .. n-1), read
      // through NB rotating register buffers of 8 wave loads: NB units in flight. Lane u holds
      // unit u's page number (read with the row length). A quarter past the block's valid
      // tokens scores -inf (quarter 0 of a block of the row always holds a token, so the
      // maximum over the four quarters is the block's). When every page is in range, each
      // unit is read whole whatever its valid tokens (in bounds: the page exists), so every
      // load of the steady state is issued unconditionally and the wait for a buffer leaves
      // the younger buffers' loads in flight (a load that may have been skipped would force
      // a wait for all of them). A page out of range is reported and its unit not read.
      constexpr int NB = 2;
      const int n = j1 - j0;
      const bool in_range = pg_spread >= 0 && (int64_t)pg_spread < a.num_pages;
      if (a.err != nullptr && lane < n && !in_range) atomicOr(a.err, (uint32_t)MSA_DEVERR_PAGE_OUT_OF_RANGE);
      const uint64_t okm = __ballot(lane < n && in_range);
      auto valid_of = [&](int u) { return min(32, min(kBlock, L - (j0 + u) * kBlock) - 32 * wave); };
      auto quarter_of = [&](int u) {
        const int pg = __builtin_amdgcn_readlane(pg_spread, u);
        return reinterpret_cast<const uint4*>(a.k + (size_t)pg * kPageElems) + wave * 512 + lane;
      };
      auto issue = [&](int u, uint4 (&kv)[8]) { quarter_load<true>(quarter_of(u), 32, kv); };
      auto score = [&](int u, const uint4 (&kv)[8]) {
        const float m = quarter_max(kv, valid_of(u), qr, lane);
        if (lane < kHeads) sc[wave][u][lane] = m;
      };
      uint4 buf[NB][8];
      if (okm == (n == 64 ? ~0ull : (1ull << n) - 1)) {
        if (n <= NB) {
          // All n units in flight at once, n a compile-time constant in each case (a load
          // under a branch here made the compiler wait for every earlier load first).
          auto all = [&](auto count) {
            constexpr int K = decltype(count)::value;
#pragma unroll
            for (int i = 0; i < K; ++i) issue(i, buf[i]);
#pragma unroll
            for (int i = 0; i < K; ++i) score(i, buf[i]);
          };
          if (n == 1) all(std::integral_constant<int, 1>{});
          else all(std::integral_constant<int, NB>{});
        } else if (n >= 4 && n <= kSpreadMaxUnits) {
          // Four or five units (even splits): the first four in flight at once, the fifth
          // issued as soon as the first is scored; n a compile-time constant in each case, in
          // straight-line code (a rotating loop of four buffers copies registers at its back
          // edge and needs twice the registers; a third case for three units spilled; all five
          // in flight measured slower).
          auto upto5 = [&](auto count) {
            constexpr int K = decltype(count)::value;
            uint4 kv[4][8];
#pragma unroll
            for (int i = 0; i < 4; ++i) issue(i, kv[i]);
            score(0, kv[0]);
            if constexpr (K == 5) {
              __builtin_amdgcn_sched_barrier(0);  // the fifth unit's loads after the first's use
              issue(4, kv[0]);
            }
#pragma unroll
            for (int i = 1; i < 4; ++i) score(i, kv[i]);
            if constexpr (K == 5) score(4, kv[0]);
          };
          if (n == 4) upto5(std::integral_constant<int, 4>{});
          else upto5(std::integral_constant<int, 5>{});
        } else {
#pragma unroll
          for (int i = 0; i < NB; ++i) issue(i, buf[i]);
          int u = 0;
          while (u + 2 * NB <= n) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
              score(u + i, buf[i]);
              issue(u + NB + i, buf[i]);
            }
            u += NB;
          }
          const int r = n - u - NB;  // units after the buffered ones: 0 .. NB-1
#pragma unroll
          for (int i = 0; i < NB; ++i) {
            score(u + i, buf[i]);
            if (i < r) issue(u + NB + i, buf[i]);
          }
#pragma unroll
          for (int i = 0; i < NB; ++i)
            if (i < r) score(u + NB + i, buf[i]);
        }
      } else {
        for (int u = 0; u < n; ++u) {
          const int vw = ((okm >> u) & 1) ? valid_of(u) : 0;
          quarter_load<false>(quarter_of(u), vw, buf[0]);
          const float m = quarter_max(buf[0], vw, qr, lane);
          if (lane < kHeads) sc[wave][u][lane] = m;
        }
      }
    }
  }
  if constexpr (!SPREAD) {
    for (int j = j0 + wave; j < j1; j += kWaves) {
      const int next = j + kWaves < j1 ? btrow[j + kWaves] : 0;
      const float m = score_page<ENGINE>(a, page, j, L, lane, &qr);
      if (lane < kHeads) sc[0][j - j0][lane] = m;
      page = next;
    }
  }
  __syncthreads();

  // Wave h sorts the split's keys of head h (one per lane, 0 past the split's blocks) and
  // keeps the first Lk: the split's list, best first, zero padded.
  const int n = j1 - j0;
  const int h = wave;
  uint64_t key = 0;
  if (lane < n) {
    const int jj = j0 + lane;
    float v = sc[0][lane][h];
    if constexpr (SPREAD) v = fmaxf(fmaxf(v, sc[1 % kWaves][lane][h]), fmaxf(sc[2 % kWaves][lane][h], sc[3 % kWaves][lane][h]));
    key = make_key(v, jj, jj < a.n_init || jj >= nb - a.n_local);
  }
  key = sort_desc_first(key, lane, n);
  if (MODE == kFused && ns == 1) {
    // The row's only split: its sorted keys are the selection (m <= n of them), so it is
    // written at once, without the publication, count and reload of the lists.
    const int m = min(a.topk, nb);
    const size_t o = ((size_t)b * kHeads + h) * a.topk;
    write_selection(key, m, a.topk, lane, a.out_ids + o, a.out_scores + o);
    if (a.out_pages != nullptr)
      emit_pages(key_id(key), lane < m, a.topk, lane, btrow, L, a.out_pages + o * 8,
                 a.out_tokens + (size_t)b * kHeads + h);
    return;
  }
  // Agent-scope atomic stores: written through to the device-coherent level, so the
  // row's last workgroup can read them from any XCD without an L2 writeback.
  uint64_t* out = a.keys + list_offset(b, a.S, kHeads, a.Lk, s, h, Lk);
  if (lane < Lk) __hip_atomic_store(out + lane, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // Publish this workgroup's lists and count it in. Every wave waits until its list
  // stores have completed (reached the device-coherent level) before the barrier, so the
  // counter increment after it cannot overtake them (and a group's last workgroup counts
  // the group in only after every member has). A release fence would do the same plus a
  // writeback of the whole L2, which measured ~0.17 us per workgroup here; the lists are
  // the only data other workgroups read. The last workgroup leaves the counters at zero
  // for the next call (and for graph replays).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) s_last = count_in(a.counters + (size_t)b * kCounterStride, s, ns);
  __syncthreads();
  if (!s_last) return;
  if (MODE != kFused) return;

  // Head h's lists of row b are one contiguous range [s][i] of the workspace, the heads
  // S * LkMax keys apart. Wave h merges head h's lists straight from it with the network;
  // otherwise the lists are staged in LDS as [s][h][i], each workgroup's four lists with one
  // pad key after them so that lanes reading list s (stride 4 Lk + 1 keys) fall on different
  // banks.
  const uint64_t* row_keys = a.keys + list_offset(b, a.S, kHeads, a.Lk, 0, 0, Lk);
  const size_t head_stride = (size_t)a.S * a.Lk;
  const int m = min(a.topk, nb);
  uint64_t mine;
  if (network_fits(ns, Lk, a.topk)) {
    mine = merge_top16(row_keys + h * head_stride, (size_t)Lk, ns, Lk, C, lane, !a.even);
  } else {
    const int row_len = kHeads * Lk, stride = row_len + 1;
    stage_keys(row_keys, lk, ns * row_len, threadIdx.x, kThreads,
               [row_len, Lk, head_stride](int e) {
                 const int sp = e / row_len, r = e % row_len;
                 return (size_t)(r / Lk) * head_stride + (size_t)sp * Lk + r % Lk;
               },
               [row_len](int e) { return e + e / row_len; });
    __syncthreads();
    mine = merge_rounds(lk + h * Lk, ns, Lk, stride, m, lane);
  }
  const size_t o = ((size_t)b * kHeads + h) * a.topk;
  write_selection(mine, m, a.topk, lane, a.out_ids + o, a.out_scores + o);
  if (a.out_pages != nullptr)
    emit_pages(key_id(mine), lane < m, a.topk, lane, btrow, L, a.out_pages + o * 8,
               a.out_tokens + (size_t)b * kHeads + h);
}

// ---------------------------------------------------------------------------------------
// Stage 2 on its own: one wave per (row, position-head task), grid (Q*4, batch). Keys are
// [batch][Q*4][S * LkMax] (list_offset); Q = 1 is the single-token layout [batch][4][S * LkMax].

struct MergeArgs {
  const int32_t* lens;
  int32_t W, Q, S, C, Lk, topk;
  int32_t batch;
  int32_t device_plan;  // C (and Lk = min(topk, C)) chosen on the device, as the split pass did
  SplitLimits lim;
  FullRowPlan full;     // device plan: the plan when every row is W blocks long
  const uint64_t* keys;
  int32_t* out_ids;     // [batch][Q][4][topk]
  float* out_scores;
  const int32_t* bt;    // with out_pages (Q = 1): the block table and its row stride
  int32_t bt_stride;
  int32_t* out_pages;   // may be null
  int32_t* out_tokens;
};

// LDS for the lists when merge_rounds may run: topk above 16, or more than 64 splits (with
// at most 64 splits and topk <= 16 the lists always fit merge_top16).
size_t merge_lds_bytes(int S, int Lk, int topk) {
  return S <= 64 && topk <= kNetworkMaxM ? 0 : (size_t)S * (Lk + 1) * sizeof(uint64_t);
}

__global__ __launch_bounds__(64) void merge_kernel(MergeArgs a) {
  extern __shared__ uint64_t lk[];  // merge_rounds: [ns][Lk + 1] lists
  const int task = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int p = task >> 2;
  const int QH = a.Q * kHeads;
  // Where the lists lie depends on the row's length and, under the device plan, on every row's
  // (one memory round trip). The lists are complete (the split launch has ended), so the first
  // round of loads is issued at once for a full row under the full-row plan the host computed
  // (the decode case of uniform batches), alongside the lengths, and kept if the row takes that
  // plan; otherwise the lists are read once the plan is known. The lengths are read first, so
  // that the waits for them do not wait for the list loads.
  const int L = row_tokens(a.lens, b, a.W);
  int raw0 = a.lens[min(lane, a.batch - 1)];  // row `lane`'s length, unclamped (batch >= 1)
  const int Cg = a.device_plan ? a.full.C : a.C;
  const int Lkg = a.device_plan ? min(a.topk, Cg) : a.Lk;
  const int nsg = Cg > 0 ? (a.W + Cg - 1) / Cg : 0;
  const bool guess = Cg > 0 && network_fits(nsg, Lkg, a.topk);
  MergeShape shape = merge_shape(nsg, Lkg, true);
  uint64_t r[16];
  if (guess) merge_issue(a.keys + list_offset(b, a.S, QH, a.Lk, 0, task, Lkg), (size_t)Lkg, nsg, Lkg, shape, lane, r);
  asm volatile("" : "+v"(raw0));  // keeps the length's first use (and its wait) after the list loads
  const int nb = (L + kBlock - 1) / kBlock;
  const int Lp = causal_len(L, a.Q, p);
  const int m = min(a.topk, (Lp + kBlock - 1) / kBlock);
  // device_blocks(lens, batch, W, lane) from the length read above
  const int nb0 = lane < a.batch ? (min(max(raw0, 0), a.W * kBlock) + kBlock - 1) / kBlock : 0;
  const int C = a.device_plan ? device_width(a.lens, a.batch, a.W, lane, nb0, a.lim, a.full) : a.C;
  const int ns = (nb + C - 1) / C;
  const int Lk = a.device_plan ? min(a.topk, C) : a.Lk, stride = Lk + 1;
  const uint64_t* src = a.keys + list_offset(b, a.S, QH, a.Lk, 0, task, Lk);
  uint64_t mine;
  if (guess && C == Cg && ns == nsg) {
    mine = merge_finish(src, (size_t)Lk, ns, Lk, C, shape, lane, r);
  } else if (network_fits(ns, Lk, a.topk)) {
    mine = merge_top16(src, (size_t)Lk, ns, Lk, C, lane);
  } else {
    stage_keys(src, lk, ns * Lk, lane, 64, [](int e) { return e; },
               [Lk, stride](int e) { return (e / Lk) * stride + e % Lk; });
    __syncthreads();
    mine = merge_rounds(lk, ns, Lk, stride, m, lane);
  }
  const size_t o = ((size_t)b * QH + task) * a.topk;
  write_selection(mine, m, a.topk, lane, a.out_ids + o, a.out_scores + o);
  if (a.out_pages != nullptr)
    emit_pages(key_id(mine), lane < m, a.topk, lane, a.bt + (size_t)b * a.bt_stride, Lp,
               a.out_pages + o * 8, a.out_tokens + (size_t)b * QH + task);
}

// ---------------------------------------------------------------------------------------
// Page tables of given selections: one workgroup per row, wave h for head h.

struct ExpandArgs {
  const int32_t* ids;   // [batch][Q][4][topk]
  const int32_t* bt;
  const int32_t* lens;
  int32_t W, bt_stride, topk, Q;
  int32_t* out_pages;   // [batch][Q][4][8 topk]
  int32_t* out_tokens;  // [batch][Q][4]
};

// Workgroup r = b*Q + p: selection (b, p), block-table row b, position p's causal length.
__global__ __launch_bounds__(kThreads) void expand_kernel(ExpandArgs a) {
  const int r = blockIdx.x, b = r / a.Q, p = r % a.Q;
  const int h = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int L = causal_len(row_tokens(a.lens, b, a.W), a.Q, p);
  const int nb = (L + kBlock - 1) / kBlock;
  const size_t bh = (size_t)r * kHeads + h;
  const int id = lane < a.topk ? a.ids[bh * a.topk + lane] : -1;
  emit_pages(id, id >= 0 && id < nb, a.topk, lane, a.bt + (size_t)b * a.bt_stride, L,
             a.out_pages + bh * a.topk * 8, a.out_tokens + bh);
}

// ---------------------------------------------------------------------------------------
// Multi-token decode: a row verifying Q <= 4 draft tokens carries Q query positions, the
// last Q tokens of its context. All Q x 4 (position, head) query rows are scored from one
// read of each page (vLLM blog "Following the Bottleneck", section 2: one workgroup per
// request for all draft positions, reusing the key loads). Under the causal clamp of
// TensorRT-LLM PR #17008 (Description), position p sees the first L - (Q-1-p) tokens.
//
// The 16 query rows are exactly the A operand of v_mfma_f32_16x16x32_bf16: row m = 4p + h
// (rows from 4Q on are zero). The result puts token column l%16 in lane l with rows
// 4(l/16) .. +3, so lane group g = l/16 holds position g's four heads: the causal mask is a
// per-lane token bound.

struct QMulti {
  bf16x8_t a[4];  // per k-step, as QMfma
};

__device__ __forceinline__ void load_q_multi(const uint16_t* __restrict__ q, int b, int Q, int lane,
                                             QMulti& r) {
  const int m = lane & 15, g = lane >> 4;
  const int p = m >> 2, h = m & 3;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (p < Q)
      v = *reinterpret_cast<const uint4*>(q + ((size_t)((b * Q + p) * kHeads + h) * kDim + s * 32 + g * 8));
    r.a[s] = __builtin_bit_cast(bf16x8_t, v);
  }
}

// Streaming form for the verify kernel. The MFMA operand layout reads half of sixteen
// 128-byte lines per load instruction, which streams poorly. Here each wave instead reads
// its pages with the coalesced pattern of the VALU engine (load i: 1 KiB = tokens 4i .. 4i+3,
// lane l: token 4i + l/16, dims 8(l%16) .. +7, non-temporal), 32 tokens (8 loads) at a time,
// one chunk ahead, and passes each chunk through a private 8 KiB LDS region to reach the
// operand layout. 16-byte slot c of token t is stored at position c ^ (t % 16) of the token's
// 256-byte row, so neither the row-wise writes nor the column-wise operand reads (16 tokens,
// one slot each) put two lanes of a pass on the same banks.
// The same scheme serves FP8 E4M3 caches (one byte per element, 128-byte tokens, a 16 KiB
// page): a chunk is then 64 tokens, still 8 KiB and 8 loads, and the operand read of each
// lane is the 8 bytes of its 8 k-slots, widened to bf16 exactly (every E4M3 value is a bf16
// value) by v_cvt_scalef32_pk_bf16_fp8 with scale 1.
constexpr int kChunkLoads = 8;                 // 1 KiB wave loads per chunk
constexpr int kChunkSlots = kChunkLoads * 64;  // 16-byte slots per chunk (8 KiB)

template <bool FP8>
struct KvGeom {
  static constexpr int kTokenSlots = FP8 ? 8 : 16;              // 16-byte slots per token
  static constexpr int kChunkTokens = kChunkSlots / kTokenSlots;  // 64 or 32
  static constexpr int kTokensPerLoad = 64 / kTokenSlots;       // 8 or 4
  static constexpr size_t kPageBytes = (size_t)kBlock * kDim * (FP8 ? 1 : 2);
};

__device__ __forceinline__ void chunk_load(const uint8_t* __restrict__ page, int c, int lane,
                                           uint4 (&kv)[kChunkLoads]) {
  const uint4* p = reinterpret_cast<const uint4*>(page) + c * kChunkSlots + lane;
#pragma unroll
  for (int i = 0; i < kChunkLoads; ++i) kv[i] = load_stream(p + i * 64);
}

template <bool FP8>
__device__ __forceinline__ void chunk_to_lds(uint4* region, const uint4 (&kv)[kChunkLoads], int lane) {
  using G = KvGeom<FP8>;
  const int r = lane / G::kTokenSlots, c = lane % G::kTokenSlots;
#pragma unroll
  for (int i = 0; i < kChunkLoads; ++i) {
    const int t = G::kTokensPerLoad * i + r;
    region[t * G::kTokenSlots + (c ^ (t % G::kTokenSlots))] = kv[i];
  }
}

// Four E4M3 codes (one dword) to bf16 pairs, exactly.
__device__ __forceinline__ uint32_t e4m3_pair_lo(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false));
}
__device__ __forceinline__ uint32_t e4m3_pair_hi(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true));
}

// Operand of MFMA k-step s for the chunk token t in column l%16: the bf16 values of dims
// 32 s + 8 g .. +7 (g = l/16).
template <bool FP8>
__device__ __forceinline__ bf16x8_t chunk_operand(const uint4* region, int t, int s, int g) {
  if constexpr (FP8) {
    const int c = 2 * s + (g >> 1);
    const uint2 v = reinterpret_cast<const uint2*>(region)[(t * 8 + (c ^ (t & 7))) * 2 + (g & 1)];
    const uint4 w = make_uint4(e4m3_pair_lo(v.x), e4m3_pair_hi(v.x), e4m3_pair_lo(v.y), e4m3_pair_hi(v.y));
    return __builtin_bit_cast(bf16x8_t, w);
  } else {
    return __builtin_bit_cast(bf16x8_t, region[t * 16 + ((4 * s + g) ^ (t & 15))]);
  }
}

// Running maxima over one chunk: lane group g accumulates position g's four heads; token
// 16 tg + l%16 of the chunk is column l%16 of MFMA tg. ok_g: tokens of the chunk position g
// sees (>= the chunk size: all).
template <bool FP8>
__device__ __forceinline__ void chunk_mfma(const uint4* region, int ok_g, const QMulti& qr, int lane,
                                           float (&m)[kHeads]) {
  constexpr int TG = KvGeom<FP8>::kChunkTokens / 16;
  const int n = lane & 15, g = lane >> 4;
  // The token groups' accumulations are independent: k-step by k-step across the groups,
  // so each MFMA's latency overlaps the other groups' instead of stalling its own chain.
  f32x4_t acc[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) acc[tg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
      acc[tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qr.a[s], chunk_operand<FP8>(region, 16 * tg + n, s, g),
                                                        acc[tg], 0, 0, 0);
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const bool ok = 16 * tg + n < ok_g;
#pragma unroll
    for (int h = 0; h < kHeads; ++h) m[h] = fmaxf(m[h], ok ? acc[tg][h] : -__builtin_inff());
  }
}

// Inserts key k into each 16-lane row of x (sorted best first, zero padded, k the same in
// every lane of a row): a row's lanes below k's place keep their keys, the lane at its place
// takes k and the lanes after it take their predecessor's key, so the row's last key drops
// out. Zero keys change nothing.
__device__ __forceinline__ uint64_t row_insert(uint64_t x, uint64_t k, int lane) {
  constexpr int kRowShr1 = 0x111;  // row_shr:1: the key of lane - 1 within the row
  const uint64_t prev = dpp_u64<kRowShr1>(x);
  return x > k ? x : (((lane & 15) == 0 || prev > k) ? k : prev);
}

struct VerifyArgs {
  const uint16_t* q;    // [batch][Q][4][128]
  const uint8_t* k;     // bf16 or E4M3 pages
  float k_scale;        // E4M3 caches: keys are k_scale * value
  const int32_t* bt;
  const int32_t* lens;
  int32_t W, bt_stride;
  int64_t num_pages;
  int32_t Q, S, C, Lk, topk, n_init, n_local;
  int32_t batch;
  int32_t device_plan;  // split modes: C and each workgroup's (row, split) chosen on the device
  SplitLimits lim;
  FullRowPlan full;     // device plan: the plan when every row is W blocks long
  uint64_t* keys;       // [batch][Q*4][S * LkMax] (list_offset)
  uint32_t* err;        // device error word (may be null)
  float* scores;        // [batch][Q][4][W] (block-score mode)
  uint32_t* counters;   // fused mode: [batch][kCounterStride], zero between calls
  int32_t* out_ids;     // fused mode (Q = 1): [batch][4][topk]
  float* out_scores;
};


// Grid (S, batch), 4 waves; split s of row b owns blocks [s*C, min((s+1)*C, nb)), nb the
// last position's block count. kScores: block scores out. kSplit: per (position, head) the
// split's top Lk keys, best first, zero padded. kFused (one position, topk <= 16, lists that
// merge_top16 holds in at most 4 registers): kSplit, then the row's last workgroup merges
// the lists as split_kernel does.
template <int MODE, bool FP8, bool RUNNING>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void verify_kernel(VerifyArgs a) {
  using G = KvGeom<FP8>;
  __shared__ float sc[kMaxSplitBlocks][16];
  __shared__ uint4 stage[kWaves * kChunkSlots];  // one 8 KiB chunk region per wave
  __shared__ int s_last;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  int s = blockIdx.x, b = blockIdx.y, C = a.C, Lk = a.Lk, L;
  if (MODE != kScores && a.device_plan) {
    const DevicePlan dp = device_plan(a.lens, a.batch, a.W, a.lim, a.full, blockIdx.x, lane);
    if (!dp.active) return;
    s = dp.s;
    b = dp.b;
    C = dp.C;
    Lk = min(a.topk, C);
    L = dp.L;
  } else {
    L = row_tokens(a.lens, b, a.W);
  }
  const int nb = (L + kBlock - 1) / kBlock;
  const int Lg = g < a.Q ? causal_len(L, a.Q, g) : 0;
  const int32_t* btrow = a.bt + (size_t)b * a.bt_stride;
  const int j0 = s * C, j1 = min(j0 + C, nb);

  if (MODE == kScores) {  // blocks past the row's end: -inf for every position
    const int e0 = max(j0, nb), e1 = min(j0 + C, a.W), ne = e1 - e0;
    for (int idx = threadIdx.x; idx < ne * a.Q * kHeads; idx += kThreads) {
      const int r = idx / ne, j = e0 + idx % ne;
      a.scores[((size_t)b * a.Q * kHeads + r) * a.W + j] = -__builtin_inff();
    }
  }
  if (j0 >= nb) {
    // An empty row has no workgroup to merge it: its first workgroup writes the padding.
    if (MODE == kFused && nb == 0 && s == 0 && (int)threadIdx.x < a.Q * kHeads * a.topk) {
      const size_t o = (size_t)b * a.Q * kHeads * a.topk + threadIdx.x;
      a.out_ids[o] = -1;
      a.out_scores[o] = -__builtin_inff();
    }
    return;
  }
  QMulti qr;
  load_q_multi(a.q, b, a.Q, lane, qr);
  uint4* region = stage + wave * kChunkSlots;
  // RUNNING (three or four positions, topk <= 16; chosen on the host): each wave keeps the
  // top 16 of its own blocks per (position, head) as it goes: register h, row p (lanes 16 p ..
  // 16 p + 15) holds position p's keys of head h, best first. Its lanes hold position p's
  // block maxima (lane group p), so a block's keys are inserted where they are, and at the end
  // the four waves' lists merge in a few steps instead of the Q sorts of the split's keys
  // after the last block (bf16 four positions 164.4 -> 162.7 us, FP8 four positions 87.0 ->
  // 86.1 us). Fewer positions pay the same insertions for fewer sorts and keep the sorts.
  constexpr bool running = RUNNING && MODE != kScores;
  uint64_t top[kHeads] = {0, 0, 0, 0};
  const int nbp_g = (causal_len(L, a.Q, min(g, a.Q - 1)) + kBlock - 1) / kBlock;  // lane group g's position

  // The wave's blocks j0 + wave, j0 + wave + 4, ... as one stream of 32-token chunks: chunk
  // c of block j holds tokens 32c .. 32c+31; a block has ceil(vmax / 32) chunks, vmax the
  // tokens the last position sees. Blocks whose page is out of range score -inf, unread.
  auto emit = [&](int j, float (&m)[kHeads]) {
    if (FP8) {
#pragma unroll
      for (int h = 0; h < kHeads; ++h) m[h] *= a.k_scale;
    }
    if constexpr (running) {
      // A block past position g's end has no key.
      const bool real = g < a.Q && j < nbp_g;
      const bool pinned = j < a.n_init || j >= nbp_g - a.n_local;
#pragma unroll
      for (int h = 0; h < kHeads; ++h) top[h] = row_insert(top[h], real ? make_key(m[h], j, pinned) : 0, lane);
      return;
    }
    if ((lane & 15) == 0 && g < a.Q) {
      if (MODE == kScores) {
#pragma unroll
        for (int h = 0; h < kHeads; ++h) a.scores[((size_t)(b * a.Q + g) * kHeads + h) * a.W + j] = m[h];
      } else {
#pragma unroll
        for (int h = 0; h < kHeads; ++h) sc[j - j0][4 * g + h] = m[h];
      }
    }
  };
  // First block at or after j with a page in range (out-of-range ones are emitted as -inf);
  // its page in *page. Everything here is wave-uniform and kept in scalar registers.
  auto next_block = [&](int j, int& page) {
    for (; j < j1; j += kWaves) {
      page = table_entry(btrow, j);
      if (page >= 0 && (int64_t)page < a.num_pages) return j;
      if (a.err != nullptr && lane == 0) atomicOr(a.err, (uint32_t)MSA_DEVERR_PAGE_OUT_OF_RANGE);
      float m[kHeads];
#pragma unroll
      for (int h = 0; h < kHeads; ++h) m[h] = -__builtin_inff();
      emit(j, m);
    }
    return j;
  };
  auto chunks_of = [&](int j) { return (min(kBlock, L - j * kBlock) + G::kChunkTokens - 1) / G::kChunkTokens; };

  // A cursor over that stream: chunk c of block j (page pg, nch chunks); j >= j1 ends it.
  struct Cursor {
    int j, c, nch, page;
  };
  auto first = [&]() {
    Cursor u{0, 0, 0, 0};
    u.j = next_block(j0 + wave, u.page);
    u.nch = u.j < j1 ? chunks_of(u.j) : 0;
    return u;
  };
  auto advance = [&](const Cursor& u) {
    Cursor v = u;
    if (u.j >= j1) return v;
    if (++v.c < u.nch) return v;
    v.c = 0;
    v.j = next_block(u.j + kWaves, v.page);
    v.nch = v.j < j1 ? chunks_of(v.j) : 0;
    return v;
  };
  auto page_ptr = [&](const Cursor& u) { return a.k + (size_t)u.page * G::kPageBytes; };

  // kChunkBuffers register buffers, as many chunks in flight: the chunk in the oldest buffer
  // (landed) is copied to LDS, that buffer is refilled at once with the chunk kChunkBuffers
  // ahead, and the MFMAs of the copied chunk run while the younger chunks and that one load.
  float m[kHeads];
#pragma unroll
  for (int h = 0; h < kHeads; ++h) m[h] = -__builtin_inff();
  // ALWAYS: the chunk ahead is known to exist, so its load is issued without a branch.
  auto process = [&](auto always, const Cursor& cur, uint4 (&A)[kChunkLoads], const Cursor& ahead) {
    chunk_to_lds<FP8>(region, A, lane);
    if (decltype(always)::value || ahead.j < j1) chunk_load(page_ptr(ahead), ahead.c, lane, A);
    chunk_mfma<FP8>(region, Lg - cur.j * kBlock - cur.c * G::kChunkTokens, qr, lane, m);
    if (cur.c + 1 == cur.nch) {
#pragma unroll
      for (int h = 0; h < kHeads; ++h) m[h] = row_max16(m[h]);
      emit(cur.j, m);
#pragma unroll
      for (int h = 0; h < kHeads; ++h) m[h] = -__builtin_inff();
    }
  };
  const std::true_type always;
  const std::false_type if_any;
  // kChunkBuffers register buffers rotate through the wave's stream: cs[0 .. NB) are the
  // buffered chunks, cs[NB .. 2 NB) the chunks after them (a cursor past the stream: j >= j1).
  constexpr int NB = kChunkBuffers;
  Cursor cs[2 * NB];
  cs[0] = first();
  if (cs[0].j < j1) {
    uint4 buf[NB][kChunkLoads];
#pragma unroll
    for (int i = 1; i < NB; ++i) cs[i] = advance(cs[i - 1]);
    // Steady state, NB chunks per trip so that the buffers rotate without copies: while the
    // NB chunks after the buffered ones all exist, every refill is issued, and the loop is
    // entered only with every buffer loaded. The loads in flight then follow one fixed order
    // on every path into the loop head, so the compiler's wait for a buffer leaves the younger
    // buffers' loads in flight; where a load may have been skipped on some path, it has to
    // wait for all of them.
    if (cs[NB - 1].j < j1) {
#pragma unroll
      for (int i = 0; i < NB; ++i) chunk_load(page_ptr(cs[i]), cs[i].c, lane, buf[i]);
#pragma unroll
      for (int i = NB; i < 2 * NB; ++i) cs[i] = advance(cs[i - 1]);
      while (cs[2 * NB - 1].j < j1) {
#pragma unroll
        for (int i = 0; i < NB; ++i) process(always, cs[i], buf[i], cs[NB + i]);
#pragma unroll
        for (int i = 0; i < NB; ++i) cs[i] = cs[NB + i];
#pragma unroll
        for (int i = NB; i < 2 * NB; ++i) cs[i] = advance(cs[i - 1]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (cs[i].j < j1) chunk_load(page_ptr(cs[i]), cs[i].c, lane, buf[i]);
#pragma unroll
      for (int i = NB; i < 2 * NB; ++i) cs[i] = cs[NB - 1];
    }
    bool more = true;
    while (more) {  // the last chunks: refills only where a chunk remains
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (more) {
          process(if_any, cs[i], buf[i], cs[NB + i]);
          more = cs[i + 1].j < j1;
        }
      }
      if (more) {
#pragma unroll
        for (int i = 0; i < NB; ++i) cs[i] = cs[NB + i];
#pragma unroll
        for (int i = NB; i < 2 * NB; ++i) cs[i] = advance(cs[i - 1]);
      }
    }
  }
  if (MODE == kScores) return;
  if constexpr (running) {  // the wave's lists to its own staging region, which it alone has used
    uint64_t* own = reinterpret_cast<uint64_t*>(region);
#pragma unroll
    for (int h = 0; h < kHeads; ++h) own[h * 64 + lane] = top[h];
  }
  __syncthreads();

  const int h = wave;
  if constexpr (running) {
    // Wave h merges the four waves' lists of head h, every position's row at once: the split's
    // top 16 per (position, head), best first, in row p.
    uint64_t r[16];
#pragma unroll
    for (int w = 0; w < 16; ++w)
      r[w] = w < kWaves ? reinterpret_cast<const uint64_t*>(stage + w * kChunkSlots)[h * 64 + lane] : 0;
    merge_level<2>(r, lane);
    merge_level<1>(r, lane);
    const int i = lane & 15;
    if (g < a.Q) {
      if (MODE == kFused && nb <= C) {
        // The row's only split: each position's keys are its selection.
        const int m = min(a.topk, nbp_g);
        const size_t o = (((size_t)b * a.Q + g) * kHeads + h) * a.topk;
        if (i < a.topk) {
          a.out_ids[o + i] = i < m ? key_id(r[0]) : -1;
          a.out_scores[o + i] = i < m ? key_score(r[0]) : -__builtin_inff();
        }
      } else if (i < Lk) {
        uint64_t* out = a.keys + list_offset(b, a.S, a.Q * kHeads, a.Lk, s, 4 * g + h, Lk);
        if (MODE == kFused) __hip_atomic_store(out + i, r[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else out[i] = r[0];
      }
    }
    if (MODE != kFused || nb <= C) return;
  }

  // Wave h sorts head h's keys of every position (the positions side by side) and keeps the
  // first Lk. A block past position p's end has no key (0).
  const int n = j1 - j0;
  auto key_of = [&](int p) -> uint64_t {
    const int nbp = (causal_len(L, a.Q, p) + kBlock - 1) / kBlock;
    const int jj = j0 + lane;
    const bool real = lane < n && jj < nbp;
    return real ? make_key(sc[lane][4 * p + h], jj, jj < a.n_init || jj >= nbp - a.n_local) : 0;
  };
  auto publish = [&](int p, uint64_t key) {
    if (MODE == kFused && nb <= C) {
      // The row's only split: each position's sorted keys are its selection.
      const int nbp = (causal_len(L, a.Q, p) + kBlock - 1) / kBlock;
      const size_t o = (((size_t)b * a.Q + p) * kHeads + h) * a.topk;
      write_selection(key, min(a.topk, nbp), a.topk, lane, a.out_ids + o, a.out_scores + o);
      return;
    }
    uint64_t* out = a.keys + list_offset(b, a.S, a.Q * kHeads, a.Lk, s, 4 * p + h, Lk);
    if (MODE == kFused) {
      if (lane < Lk) __hip_atomic_store(out + lane, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      if (lane < Lk) out[lane] = key;
    }
  };
  if constexpr (running) {
    // published above
  } else if (a.Q == 1) {
    uint64_t k[1] = {key_of(0)};
    sort_desc_first_all<1>(k, lane, n);
    publish(0, k[0]);
  } else if (a.Q == 2) {
    uint64_t k[2] = {key_of(0), key_of(1)};
    sort_desc_first_all<2>(k, lane, n);
    publish(0, k[0]);
    publish(1, k[1]);
  } else {
    uint64_t k[4] = {key_of(0), key_of(1), key_of(2), a.Q > 3 ? key_of(3) : 0};
    sort_desc_first_all<4>(k, lane, n);
#pragma unroll
    for (int p = 0; p < 4; ++p)
      if (p < a.Q) publish(p, k[p]);
  }
  if (MODE != kFused || nb <= C) return;

  // Publication and the last workgroup's merge, as in split_kernel (one position: wave h
  // merges head h).
  const int ns = (nb + C - 1) / C;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) s_last = count_in(a.counters + (size_t)b * kCounterStride, s, ns);
  __syncthreads();
  if (!s_last) return;
  const uint64_t mine = merge_top16(a.keys + list_offset(b, a.S, kHeads, a.Lk, 0, h, Lk), (size_t)Lk,
                                    ns, Lk, C, lane);
  const size_t o = ((size_t)b * kHeads + h) * a.topk;
  write_selection(mine, min(a.topk, nb), a.topk, lane, a.out_ids + o, a.out_scores + o);
}

// The error word's bits, taken (read and cleared atomically) into the header's next word.
__global__ void take_error_kernel(uint32_t* hdr) {
  hdr[1] = __hip_atomic_exchange(hdr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------------------
// Host side.

struct Plan {
  int S, C, Lk;
  bool fused;
  bool device = false;  // C and the (row, split) of each workgroup are chosen on the device
  int grid = 0;         // device plan: workgroups launched (1-D)
  bool even = false;    // widths C and C - 1, the wide splits first; C = ceil(W / S), the widest
};

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

constexpr int64_t kSpreadBlocks = 256;  // single-block splits up to this many blocks per call
constexpr int kEvenWorkgroups = 256;      // even splits: one workgroup per CU

int pow2_ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Split plan from host arguments only. A row of W blocks gets S = ceil(W/C) workgroups
// (at most 256) of C blocks each (at most 64: one candidate per lane in the per-split
// ranking). Each workgroup keeps Lk = min(topk, C) candidates per head. Automatic C:
// about batch*W/1024 blocks per workgroup, at least 4: 32 at batch 32 x 1024 blocks,
// which keeps 4 workgroups of 4 waves on each of the 256 CUs. The merge is fused into
// the split kernel (the last workgroup of each row merges it) when the lists fit the merge
// network (topk <= 16 and S lists of Lk keys rounded up to a power of two hold at most 1024
// keys: up to 256 splits of 4 blocks, merged from the workspace), or when a row has at
// most 64 workgroups whose lists fit in LDS (S * Lk <= 1024 keys per head).
int32_t plan_from_width(int32_t W, int32_t topk, int C, Plan* p);

int32_t make_plan(int32_t batch, int32_t W, int32_t topk, int32_t num_splits, Plan* p) {
  if (batch < 0 || W < 0 || topk < 1 || topk > MSA_MAX_TOPK || num_splits < 0) return MSA_ERR_INVALID_ARG;
  if (W > MSA_MAX_BLOCKS_PER_SEQ) return MSA_ERR_UNSUPPORTED;
  if (W == 0) {
    *p = Plan{1, 1, topk, true};
    return MSA_OK;
  }
  int C;
  if (num_splits > 0) {
    C = ceil_div(W, num_splits);
  } else {
    C = pow2_ceil(std::max(1, ceil_div((int64_t)batch * W, 1024)));
    C = std::min(std::max(C, 4), kMaxSplitBlocks);
  }
  return plan_from_width(W, topk, C, p);
}

// The host plan with the smallest split width C >= C0 that the limits allow (W > 0).
int32_t plan_from_width(int32_t W, int32_t topk, int C, Plan* p) {
  for (;; ++C) {
    if (C > kMaxSplitBlocks) return MSA_ERR_UNSUPPORTED;
    const int S = ceil_div(W, C), Lk = std::min(topk, C);
    if (S <= kMaxSplits && (int64_t)S * Lk <= kMaxMergeKeys) {
      *p = Plan{S, C, Lk, network_fits(S, Lk, topk) || (S <= 64 && (int64_t)S * Lk <= kMaxFusedKeys)};
      return MSA_OK;
    }
  }
}

// The plan of msa_indexer_decode and of the multi-token and FP8 calls: with num_splits = 0,
// 0 < W <= 64 * 64, topk <= 16 and batch * W >= kDeviceMinBlocks the device plan (S =
// min(64, ceil(W/4)) sizes the workspace at S * topk keys per row and head; a row takes at
// most device_max_splits(C, S, topk) splits, at most ceil(W/4) in all; a grid that covers any
// lengths: with C >= N/512 the rows need at most N/C + batch <= 512 + batch workgroups, or
// ceil(batch*W/64) + batch when C is held at 64); otherwise the host plan above.
int32_t make_decode_plan(int32_t batch, int32_t W, int32_t topk, int32_t num_splits, Plan* p) {
  int32_t rc = make_plan(batch, W, topk, num_splits, p);
  if (rc != MSA_OK) return rc;
  if (num_splits == 0 && W > 0 && W <= kDeviceMaxSplits * kMaxSplitBlocks && topk <= kNetworkMaxM &&
      (int64_t)batch * W >= kDeviceMinBlocks) {
    const int64_t per_row = ceil_div(W, 4);
    const int64_t need = std::max<int64_t>(kDeviceTarget, ceil_div((int64_t)batch * W, kMaxSplitBlocks)) + batch;
    Plan d{(int)std::min<int64_t>(kDeviceMaxSplits, per_row), 0, topk, true};
    d.device = true;
    d.grid = (int)std::min<int64_t>((int64_t)batch * per_row, need);
    *p = d;
  }
  return MSA_OK;
}

// The single-token decode's plan (msa_indexer_decode and the calls built on it): the decode
// plan, except that a small table (batch * W <= 512 blocks) with the split count left automatic
// and the VALU engine splits into single blocks (at most 256 blocks in all) or pairs. The split
// kernel then reads it in the spread layout, the four waves of a workgroup taking the four
// quarters of each block with every load of the split in flight at once: four times the
// workgroups of 4-block splits, on as many more CUs (batch 1 x 64 blocks: 7.8 -> 6.4 us).
size_t row_key_bytes(int32_t W, int32_t topk, int32_t num_splits, int32_t Q);

int32_t make_single_plan(int32_t batch, int32_t W, int32_t topk, int32_t num_splits, int32_t engine,
                         Plan* p) {
  int32_t rc = make_decode_plan(batch, W, topk, num_splits, p);
  if (rc != MSA_OK || num_splits != 0 || p->device || engine == MSA_ENGINE_MFMA || W == 0) return rc;
  const int64_t blocks = (int64_t)batch * W;
  if (blocks <= 2 * kSpreadBlocks) {
    Plan t;
    if (plan_from_width(W, topk, blocks <= kSpreadBlocks ? 1 : 2, &t) == MSA_OK) *p = t;
    return MSA_OK;
  }
  // Even splits: where the plan's workgroups just exceed the CU count (some CUs would hold
  // two, and those end the call), rows of 4 to 64 (batch * S > 256) take S = 256 / batch
  // splits of C - 1 or C <= 5 blocks each, read in the spread layout, so every CU holds one
  // workgroup. Kept out of the pruned merge (S <= 64) and within the workspace's key bound.
  if (batch >= 4 && batch <= 64 && (int64_t)batch * p->S > kEvenWorkgroups) {
    const int S = kEvenWorkgroups / batch, C = (W + S - 1) / S, Lk = std::min(topk, C);
    if (S < p->S && C <= kSpreadMaxUnits && network_fits(S, Lk, topk) &&
        (size_t)S * Lk * kHeads * sizeof(uint64_t) <= row_key_bytes(W, topk, 0, 1)) {
      Plan e{S, C, Lk, true};
      e.even = true;
      *p = e;
    }
  }
  return MSA_OK;
}

// Workspace layout (the caller's buffer of ws_size bytes, 256-byte aligned):
//   [0, 256)                   header: the device error word, then the word read_error stages
//   [256 + 4352 b, + 4352)     row b's 17 counter lines (row counter, 16 group counters)
//   the last keys_bytes        keys uint64 [batch][Q*4][S * Lk] (list_offset), 256-byte aligned
// A row's counter lines sit at an offset that depends on nothing but the row, and a call's
// keys fill the end of the buffer. So calls that share one buffer and pass its full size
// never write keys over a counter line another of them counts on, whatever their batch sizes
// (for calls of one table width, topk, split count and qlen; in general when the buffer holds
// the largest batch's counter lines plus the largest key region). The counters return to zero
// at the end of every call; the keys need no initial state.
constexpr size_t kRowCounterBytes = kCounterStride * sizeof(uint32_t);  // 17 lines of 256 B

size_t counters_end(int32_t batch) { return kHeaderBytes + (size_t)batch * kRowCounterBytes; }

size_t keys_bytes(int32_t batch, int32_t Q, const Plan& p) {
  const size_t n = (size_t)batch * p.S * Q * kHeads * p.Lk * sizeof(uint64_t);
  return (n + kAlign - 1) / kAlign * kAlign;
}

// LDS for the fused merge when merge_rounds may run (as merge_lds_bytes, for all four heads).
size_t fused_lds_bytes(const Plan& p, int topk) {
  return network_fits(p.S, p.Lk, topk) ? 0 : (size_t)p.S * (kHeads * p.Lk + 1) * sizeof(uint64_t);
}
// (For the device plan p.S and p.Lk bound the per-call values: S splits, Lk <= topk.)

// Key bytes per row that a call with these (W, topk, num_splits, Q) may use at any batch size:
// an explicit split count fixes the width; the automatic one takes a width of 1 .. 64 blocks
// from the batch, or the device plan (S * topk keys per head). Sizing every call's workspace
// with this bound (workspace_bytes) is what lets calls of any batch share one buffer: a call of
// batch B writes at most B times this many key bytes at the buffer's end, which stay clear of
// the counter lines of any batch the buffer holds.
size_t row_key_bytes(int32_t W, int32_t topk, int32_t num_splits, int32_t Q) {
  size_t best = 0;
  auto consider = [&](const Plan& p) {
    best = std::max(best, (size_t)p.S * Q * kHeads * p.Lk * sizeof(uint64_t));
  };
  Plan p;
  if (W == 0 || num_splits > 0) {
    if (make_plan(1, W, topk, num_splits, &p) == MSA_OK) consider(p);
    return best;
  }
  for (int c0 = 1; c0 <= kMaxSplitBlocks; c0 *= 2)  // 1 and 2: the single-token decode's small tables
    if (plan_from_width(W, topk, c0, &p) == MSA_OK) consider(p);
  if (make_decode_plan(kDeviceMinBlocks, W, topk, 0, &p) == MSA_OK && p.device) consider(p);
  return best;
}

// Workspace bytes of a call (the size check of every call, and workspace_bytes).
size_t ws_bytes(int32_t batch, int32_t W, int32_t topk, int32_t num_splits, int32_t Q = 1) {
  const size_t kb = (size_t)batch * row_key_bytes(W, topk, num_splits, Q);
  return counters_end(batch) + (kb + kAlign - 1) / kAlign * kAlign;
}

// The error word, counters and keys of a call in a buffer of ws_size bytes whose keys take
// kb bytes (ws_size >= counters_end(batch) + kb, checked by the caller).
struct WsView {
  uint32_t* err;
  uint32_t* counters;
  uint64_t* keys;
};

WsView ws_view(void* ws, size_t ws_size, size_t kb) {
  if (ws == nullptr) return WsView{nullptr, nullptr, nullptr};
  char* w = static_cast<char*>(ws);
  return WsView{reinterpret_cast<uint32_t*>(w), reinterpret_cast<uint32_t*>(w + kHeaderBytes),
                reinterpret_cast<uint64_t*>(w + ((ws_size - kb) & ~(kAlign - 1)))};
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

int32_t check_inputs(const void* q, const void* k, const int32_t* bt, const int32_t* lens,
                     int32_t batch, int32_t W, int32_t bt_stride, int64_t num_pages) {
  if (batch < 0 || W < 0 || bt_stride < W || num_pages < 0) return MSA_ERR_INVALID_ARG;
  if (batch == 0) return MSA_OK;
  // The table and the cache may be null only when nothing can be read from them.
  if (!q || !lens || (!bt && W > 0) || (!k && num_pages > 0)) return MSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(bt, 4) || !aligned(lens, 4)) return MSA_ERR_INVALID_ARG;
  if (num_pages > (int64_t)1 << 31) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

int32_t check_select(int32_t topk, int32_t n_init, int32_t n_local) {
  if (topk < 1 || topk > MSA_MAX_TOPK) return MSA_ERR_INVALID_ARG;
  if (n_init < 0 || n_local < 0 || (int64_t)n_init + n_local > topk) return MSA_ERR_INVALID_ARG;
  return MSA_OK;
}

// hipGetLastError reports (and clears) the last error of any HIP call of this thread,
// including one left by other code before this library's call (another library's failed
// query, say). Each launch site clears that first, so the status it reads after its launch
// is its own launch's.
void clear_stale_error() { (void)hipGetLastError(); }

template <int MODE>
int32_t launch_split(const SplitArgs& a, int32_t batch, int32_t engine, size_t lds, hipStream_t st,
                     int device_grid = 0) {
  dim3 grid(a.S, batch), block(kThreads);
  if (device_grid > 0) grid = dim3(device_grid, 1);
  if (engine == MSA_ENGINE_DEFAULT) engine = MSA_ENGINE_VALU;
  clear_stale_error();
  if (engine == MSA_ENGINE_VALU && a.spread && MODE != kScores)
    hipLaunchKernelGGL((split_kernel<MSA_ENGINE_VALU, MODE == kScores ? kSplit : MODE, true>), grid, block, lds, st, a);
  else if (engine == MSA_ENGINE_VALU)
    hipLaunchKernelGGL((split_kernel<MSA_ENGINE_VALU, MODE, false>), grid, block, lds, st, a);
  else if (engine == MSA_ENGINE_MFMA)
    hipLaunchKernelGGL((split_kernel<MSA_ENGINE_MFMA, MODE, false>), grid, block, lds, st, a);
  else
    return MSA_ERR_INVALID_ARG;
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}

// The device plan at full rows (device_split_width with every row W blocks long).
FullRowPlan full_row_plan(bool device, int32_t batch, int32_t W, const SplitLimits& lim) {
  if (!device || W <= 0 || batch <= 0) return FullRowPlan{0, 1};
  int C_min = 4;
  for (int t = 0; t < 5; ++t)
    if (W > lim.blocks[t]) C_min = 4 << (t + 1);
  const int64_t per_wg = std::max<int64_t>(1, ((int64_t)batch * W + kDeviceTarget - 1) / kDeviceTarget);
  const int C = std::min(std::max(pow2_at_least((int)std::min<int64_t>(per_wg, 1 << 20)), C_min), kMaxSplitBlocks);
  return FullRowPlan{C, (W + C - 1) / C};
}

SplitArgs make_split_args(const void* q, const void* k, const int32_t* bt, const int32_t* lens,
                          int32_t W, int32_t bt_stride, int64_t num_pages, const Plan& p,
                          int32_t topk, int32_t n_init, int32_t n_local, const WsView& w, int32_t batch) {
  SplitArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.bt = bt;
  a.lens = lens;
  a.W = W;
  a.bt_stride = bt_stride;
  a.num_pages = num_pages;
  a.S = p.S;
  a.C = p.C;
  a.Lk = p.Lk;
  a.topk = topk;
  a.n_init = n_init;
  a.n_local = n_local;
  a.batch = batch;
  a.device_plan = p.device ? 1 : 0;
  a.spread = p.even || p.C % kWaves != 0 ? 1 : 0;
  a.even = p.even ? 1 : 0;
  a.lim = split_limits(p.S, topk);
  a.full = full_row_plan(p.device, batch, W, a.lim);
  a.err = w.err;
  a.counters = w.counters;
  a.keys = w.keys;
  a.out_ids = nullptr;
  a.out_scores = nullptr;
  a.out_pages = nullptr;
  a.out_tokens = nullptr;
  a.scores = nullptr;
  return a;
}

// Validates everything a decode-style call needs; fills the plan.
int32_t check_call(const void* q, const void* k, const int32_t* bt, const int32_t* lens,
                   int32_t batch, int32_t W, int32_t bt_stride, int64_t num_pages, int32_t topk,
                   int32_t n_init, int32_t n_local, const void* ws, size_t ws_size,
                   int32_t num_splits, Plan* p, bool decode = false, bool check_ws = true) {
  int32_t rc = check_inputs(q, k, bt, lens, batch, W, bt_stride, num_pages);
  if (rc != MSA_OK) return rc;
  if ((rc = check_select(topk, n_init, n_local)) != MSA_OK) return rc;
  rc = decode ? make_decode_plan(batch, W, topk, num_splits, p) : make_plan(batch, W, topk, num_splits, p);
  if (rc != MSA_OK) return rc;
  if (batch == 0 || !check_ws) return MSA_OK;
  if (!ws || !aligned(ws, kAlign)) return MSA_ERR_INVALID_ARG;
  if (ws_size < ws_bytes(batch, W, topk, num_splits)) return MSA_ERR_WORKSPACE_TOO_SMALL;
  return MSA_OK;
}

// Page-table outputs (both or neither): 16-byte aligned table, 4-byte aligned counts; the
// block table must be there to read pages from, and 8 * page must fit 32 bits.
int32_t check_pages(const int32_t* out_pages, const int32_t* out_tokens, const int32_t* bt,
                    int32_t W, int64_t num_pages) {
  if (!out_pages && !out_tokens) return MSA_OK;
  if (!out_pages || !out_tokens || !aligned(out_pages, 16) || !aligned(out_tokens, 4))
    return MSA_ERR_INVALID_ARG;
  if (W > 0 && !bt) return MSA_ERR_INVALID_ARG;
  if (num_pages > ((int64_t)1 << 28)) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

int32_t launch_merge(const uint64_t* keys, const int32_t* lens, int32_t W, int32_t Q, const Plan& p,
                     int32_t topk, int32_t* out_ids, float* out_scores, int32_t batch, hipStream_t st,
                     const int32_t* bt = nullptr, int32_t bt_stride = 0, int32_t* out_pages = nullptr,
                     int32_t* out_tokens = nullptr) {
  MergeArgs a;
  a.lens = lens;
  a.W = W;
  a.Q = Q;
  a.S = p.S;
  a.C = p.C;
  a.Lk = p.Lk;
  a.topk = topk;
  a.keys = keys;
  a.out_ids = out_ids;
  a.out_scores = out_scores;
  a.bt = bt;
  a.bt_stride = bt_stride;
  a.out_pages = out_pages;
  a.out_tokens = out_tokens;
  a.batch = batch;
  a.device_plan = p.device ? 1 : 0;
  a.lim = split_limits(p.S, topk);
  a.full = full_row_plan(p.device, batch, W, a.lim);
  clear_stale_error();
  hipLaunchKernelGGL(merge_kernel, dim3(Q * kHeads, batch), dim3(64), merge_lds_bytes(p.S, p.Lk, topk), st, a);
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}

int32_t merge_impl(const int32_t* lens, int32_t batch, int32_t W, int32_t topk, int32_t* out_ids,
                   float* out_scores, const void* ws, size_t ws_size, int32_t num_splits,
                   hipStream_t st, const int32_t* bt = nullptr, int32_t bt_stride = 0,
                   int32_t* out_pages = nullptr, int32_t* out_tokens = nullptr) {
  if (batch < 0 || W < 0) return MSA_ERR_INVALID_ARG;
  if (topk < 1 || topk > MSA_MAX_TOPK) return MSA_ERR_INVALID_ARG;
  Plan p;
  int32_t rc = make_plan(batch, W, topk, num_splits, &p);
  if (rc != MSA_OK) return rc;
  if (batch == 0) return MSA_OK;
  if (!lens || !out_ids || !out_scores || !ws) return MSA_ERR_INVALID_ARG;
  if (!aligned(lens, 4) || !aligned(out_ids, 4) || !aligned(out_scores, 4) || !aligned(ws, kAlign))
    return MSA_ERR_INVALID_ARG;
  if (ws_size < ws_bytes(batch, W, topk, num_splits)) return MSA_ERR_WORKSPACE_TOO_SMALL;
  const uint64_t* keys = ws_view(const_cast<void*>(ws), ws_size, keys_bytes(batch, 1, p)).keys;
  return launch_merge(keys, lens, W, 1, p, topk, out_ids, out_scores, batch, st, bt, bt_stride,
                      out_pages, out_tokens);
}



VerifyArgs make_verify_args(const void* q, const void* k, const int32_t* bt, const int32_t* lens,
                            int32_t W, int32_t bt_stride, int64_t num_pages, int32_t Q, const Plan& p,
                            int32_t topk, int32_t n_init, int32_t n_local, const WsView& w,
                            int32_t batch, float k_scale = 1.0f) {
  VerifyArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint8_t*>(k);
  a.k_scale = k_scale;
  a.bt = bt;
  a.lens = lens;
  a.W = W;
  a.bt_stride = bt_stride;
  a.num_pages = num_pages;
  a.Q = Q;
  a.S = p.S;
  a.C = p.C;
  a.Lk = p.Lk;
  a.topk = topk;
  a.n_init = n_init;
  a.n_local = n_local;
  a.err = w.err;
  a.keys = w.keys;
  a.counters = w.counters;
  a.scores = nullptr;
  a.out_ids = nullptr;
  a.out_scores = nullptr;
  a.batch = batch;
  a.device_plan = p.device ? 1 : 0;
  a.lim = split_limits(p.S, topk);
  a.full = full_row_plan(p.device, batch, W, a.lim);
  return a;
}

bool valid_scale(float k_scale) { return k_scale > 0.0f && k_scale <= 3.402823466e38f; }

// Whether a one-position pass merges in its own launch (the row's last workgroup merging,
// wave h head h): always under the device plan, whose rows have at most 256 splits of at most
// 16 keys (merge_top16 prunes what does not fit); under a host plan when each head's lists fit
// 4 registers (S lists of Lk keys, 64 / Lk2 per register). With more, the serial merge in the
// row's last workgroup measured slower than the merge kernel, which runs every (row, head) at
// once (FP8 at batch 32 x 128K: 32 lists of 16, 89.8 vs 88.7 us). Passes of several positions
// always merge in the merge kernel: one workgroup merging every position of a row in its tail
// (the positions side by side in the network) measured slower than the merge kernel's wave per
// (row, position, head) at every shape tried (bf16, 4 positions, batch 32 x 128K: 168.8 vs
// 166.2 us; batch 16 with one 128K row among 1K rows: 23.4 vs 16.1 us).
bool fuse_verify(const Plan& p, int topk, int qlen) {
  if (qlen > 1 || topk > kNetworkMaxM) return false;
  if (p.device) return true;
  if (p.S > 64) return false;
  int lk2 = 1;
  while (lk2 < p.Lk) lk2 <<= 1;
  return ceil_div(p.S, 64 / lk2) <= 4;
}

template <int MODE>
void launch_verify(const VerifyArgs& a, bool fp8, int32_t batch, hipStream_t st, int device_grid = 0) {
  const dim3 grid = device_grid > 0 ? dim3(device_grid, 1) : dim3(a.S, batch);
  // The running lists pay per block and save the sorts after the last one: measured ahead
  // with three or four positions at every shape tried (bf16 four positions at the benchmark
  // shape 165.1 -> 163.4 us, at 16 x 8700 tokens 12.4 -> 12.1 us), behind with two positions
  // on short splits (16 x 8700 tokens 11.5 -> 11.7 us).
  const bool running = MODE != kScores && a.Q >= 3 && a.topk <= kNetworkMaxM;
  clear_stale_error();
  if (fp8 && running)
    hipLaunchKernelGGL((verify_kernel<MODE, true, true>), grid, dim3(kThreads), 0, st, a);
  else if (fp8)
    hipLaunchKernelGGL((verify_kernel<MODE, true, false>), grid, dim3(kThreads), 0, st, a);
  else if (running)
    hipLaunchKernelGGL((verify_kernel<MODE, false, true>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((verify_kernel<MODE, false, false>), grid, dim3(kThreads), 0, st, a);
}

int32_t verify_decode_impl(const void* q, const void* k_cache, bool fp8, float k_scale,
                           const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                           int32_t W, int32_t bt_stride, int64_t num_pages, int32_t qlen,
                           int32_t topk, int32_t n_init, int32_t n_local, int32_t* out_ids,
                           float* out_scores, void* workspace, size_t workspace_bytes,
                           int32_t num_splits, hipStream_t st) {
  if (qlen < 1 || qlen > MSA_MAX_QUERY_LEN || !valid_scale(k_scale)) return MSA_ERR_INVALID_ARG;
  int32_t rc = check_inputs(q, k_cache, block_table, seq_lens, batch, W, bt_stride, num_pages);
  if (rc != MSA_OK) return rc;
  if ((rc = check_select(topk, n_init, n_local)) != MSA_OK) return rc;
  Plan p;
  if ((rc = make_decode_plan(batch, W, topk, num_splits, &p)) != MSA_OK) return rc;
  if (batch == 0) return MSA_OK;
  if (!out_ids || !out_scores || !aligned(out_ids, 4) || !aligned(out_scores, 4)) return MSA_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, kAlign)) return MSA_ERR_INVALID_ARG;
  if (workspace_bytes < ws_bytes(batch, W, topk, num_splits, qlen)) return MSA_ERR_WORKSPACE_TOO_SMALL;
  VerifyArgs a = make_verify_args(q, k_cache, block_table, seq_lens, W, bt_stride, num_pages, qlen,
                                  p, topk, n_init, n_local,
                                  ws_view(workspace, workspace_bytes, keys_bytes(batch, qlen, p)), batch,
                                  k_scale);
  const int grid = p.device ? p.grid : 0;
  if (fuse_verify(p, topk, qlen)) {  // one position, a cheap merge: in the same launch
    a.out_ids = out_ids;
    a.out_scores = out_scores;
    launch_verify<kFused>(a, fp8, batch, st, grid);
    return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
  }
  launch_verify<kSplit>(a, fp8, batch, st, grid);
  if (hipGetLastError() != hipSuccess) return MSA_ERR_HIP;
  return launch_merge(a.keys, seq_lens, W, qlen, p, topk, out_ids, out_scores, batch, st);
}

int32_t verify_scores_impl(const void* q, const void* k_cache, bool fp8, float k_scale,
                           const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                           int32_t W, int32_t bt_stride, int64_t num_pages, int32_t qlen, float* out,
                           int32_t num_splits, hipStream_t st) {
  if (qlen < 1 || qlen > MSA_MAX_QUERY_LEN || !valid_scale(k_scale)) return MSA_ERR_INVALID_ARG;
  int32_t rc = check_inputs(q, k_cache, block_table, seq_lens, batch, W, bt_stride, num_pages);
  if (rc != MSA_OK) return rc;
  Plan p;
  if ((rc = make_plan(batch, W, 16, num_splits, &p)) != MSA_OK) return rc;
  if (batch == 0 || W == 0) return MSA_OK;
  if (!out || !aligned(out, 4)) return MSA_ERR_INVALID_ARG;
  VerifyArgs a = make_verify_args(q, k_cache, block_table, seq_lens, W, bt_stride, num_pages, qlen, p,
                                  16, 0, 0, WsView{nullptr, nullptr, nullptr}, batch, k_scale);
  a.scores = out;
  launch_verify<kScores>(a, fp8, batch, st);
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}

// The allocation-free decode: the library's scratch array stands in for the workspace.
struct ScratchUse {
  uint32_t* err;  // the caller's device error word (may be null: bits are then not kept)
};

constexpr int kMaxDevices = 64;
constexpr size_t kNoallocBytes = MSA_NOALLOC_SCRATCH_BYTES;
constexpr int32_t kNoallocMaxBatch = MSA_NOALLOC_MAX_BATCH;

std::mutex g_scratch_mu;
char* g_scratch[kMaxDevices];  // the scratch array's device address, per device (null: not set up)

__global__ void zero_words_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// The scratch array's address on the current device. The first call on a device looks it up
// with that device current and clears the header and every counter line on `st` (the loader
// zero-fills the array too; the counters then return to zero at the end of every call).
int32_t scratch_on_current_device(hipStream_t st, char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return MSA_ERR_HIP;
    const size_t words = counters_end(kNoallocMaxBatch) / sizeof(uint32_t);
    clear_stale_error();
    hipLaunchKernelGGL(zero_words_kernel, dim3(256), dim3(256), 0, st, static_cast<uint32_t*>(ptr), words);
    if (hipGetLastError() != hipSuccess) return MSA_ERR_HIP;
    g_scratch[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch[dev];
  return MSA_OK;
}

int32_t decode_impl(const void* q, const void* k_cache, const int32_t* block_table,
                    const int32_t* seq_lens, int32_t batch, int32_t W, int32_t bt_stride,
                    int64_t num_pages, int32_t topk, int32_t n_init, int32_t n_local,
                    int32_t* out_ids, float* out_scores, int32_t* out_pages, int32_t* out_tokens,
                    void* workspace, size_t workspace_bytes, int32_t num_splits, int32_t engine,
                    hipStream_t st, const ScratchUse* scratch = nullptr) {
  // Check everything (outputs included) before the first HIP call.
  if (batch > 0 && (!out_ids || !out_scores || !aligned(out_ids, 4) || !aligned(out_scores, 4)))
    return MSA_ERR_INVALID_ARG;
  if (engine < MSA_ENGINE_DEFAULT || engine > MSA_ENGINE_MFMA) return MSA_ERR_INVALID_ARG;
  Plan p;
  int32_t rc = check_call(q, k_cache, block_table, seq_lens, batch, W, bt_stride, num_pages, topk,
                          n_init, n_local, workspace, workspace_bytes, num_splits, &p, true,
                          scratch == nullptr);
  if (rc != MSA_OK) return rc;
  if (batch > 0 && (rc = check_pages(out_pages, out_tokens, block_table, W, num_pages)) != MSA_OK)
    return rc;
  if (batch == 0) return MSA_OK;
  if ((rc = make_single_plan(batch, W, topk, num_splits, engine, &p)) != MSA_OK) return rc;
  const size_t kb = keys_bytes(batch, 1, p);
  WsView w;
  if (scratch != nullptr) {
    // The scratch keeps counter lines for kNoallocMaxBatch rows and the keys after them, a
    // fixed split, so no shape can lay keys over another's counters.
    if (batch > kNoallocMaxBatch || kb > kNoallocBytes - counters_end(kNoallocMaxBatch))
      return MSA_ERR_WORKSPACE_TOO_SMALL;
    char* base = nullptr;
    if ((rc = scratch_on_current_device(st, &base)) != MSA_OK) return rc;
    w = ws_view(base, kNoallocBytes, kb);
    w.err = scratch->err;
  } else {
    w = ws_view(workspace, workspace_bytes, kb);
  }
  SplitArgs a = make_split_args(q, k_cache, block_table, seq_lens, W, bt_stride, num_pages, p, topk,
                                n_init, n_local, w, batch);
  if (p.fused) {
    a.out_ids = out_ids;
    a.out_scores = out_scores;
    a.out_pages = out_pages;
    a.out_tokens = out_tokens;
    return launch_split<kFused>(a, batch, engine, fused_lds_bytes(p, topk), st, p.device ? p.grid : 0);
  }
  if ((rc = launch_split<kSplit>(a, batch, engine, 0, st)) != MSA_OK) return rc;
  return launch_merge(w.keys, seq_lens, W, 1, p, topk, out_ids, out_scores, batch, st, block_table,
                      bt_stride, out_pages, out_tokens);
}

}  // namespace

extern "C" {

const char* msa_status_string(int32_t status) {
  switch (status) {
    case MSA_OK: return "ok";
    case MSA_ERR_INVALID_ARG: return "invalid argument";
    case MSA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MSA_ERR_UNSUPPORTED: return "unsupported shape";
    case MSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int32_t msa_indexer_num_splits(int32_t batch, int32_t max_blocks_per_seq, int32_t topk,
                               int32_t num_splits) {
  Plan p;
  const int32_t rc = make_single_plan(batch, max_blocks_per_seq, topk, num_splits, MSA_ENGINE_DEFAULT, &p);
  return rc == MSA_OK ? p.S : rc;
}

int32_t msa_indexer_plan(int32_t batch, int32_t max_blocks_per_seq, int32_t topk,
                         int32_t num_splits, int32_t* splits, int32_t* blocks_per_split,
                         int32_t* candidates_per_split, int32_t* fused) {
  Plan p;
  const int32_t rc = make_single_plan(batch, max_blocks_per_seq, topk, num_splits, MSA_ENGINE_DEFAULT, &p);
  if (rc != MSA_OK) return rc;
  if (splits) *splits = p.S;
  if (blocks_per_split) *blocks_per_split = p.C;
  if (candidates_per_split) *candidates_per_split = p.Lk;
  if (fused) *fused = p.fused ? 1 : 0;
  return MSA_OK;
}

size_t msa_indexer_workspace_bytes(int32_t batch, int32_t max_blocks_per_seq, int32_t topk,
                                   int32_t num_splits) {
  Plan p;
  if (make_decode_plan(batch, max_blocks_per_seq, topk, num_splits, &p) != MSA_OK) return 0;
  return ws_bytes(batch, max_blocks_per_seq, topk, num_splits);
}

int32_t msa_indexer_split_topk(const void* q, const void* k_cache, const int32_t* block_table,
                               const int32_t* seq_lens, int32_t batch,
                               int32_t max_blocks_per_seq, int32_t bt_stride, int64_t num_pages,
                               int32_t topk, int32_t n_init, int32_t n_local, void* workspace,
                               size_t workspace_bytes, int32_t num_splits, int32_t engine,
                               void* stream) {
  Plan p;
  int32_t rc = check_call(q, k_cache, block_table, seq_lens, batch, max_blocks_per_seq, bt_stride,
                          num_pages, topk, n_init, n_local, workspace, workspace_bytes, num_splits, &p);
  if (rc != MSA_OK) return rc;
  if (engine < MSA_ENGINE_DEFAULT || engine > MSA_ENGINE_MFMA) return MSA_ERR_INVALID_ARG;
  if (batch == 0) return MSA_OK;
  const SplitArgs a = make_split_args(q, k_cache, block_table, seq_lens, max_blocks_per_seq, bt_stride,
                                      num_pages, p, topk, n_init, n_local,
                                      ws_view(workspace, workspace_bytes, keys_bytes(batch, 1, p)), batch);
  return launch_split<kSplit>(a, batch, engine, 0, static_cast<hipStream_t>(stream));
}

int32_t msa_indexer_merge(const int32_t* seq_lens, int32_t batch, int32_t max_blocks_per_seq,
                          int32_t topk, int32_t* out_ids, float* out_scores,
                          const void* workspace, size_t workspace_bytes, int32_t num_splits,
                          void* stream) {
  return merge_impl(seq_lens, batch, max_blocks_per_seq, topk, out_ids, out_scores, workspace,
                    workspace_bytes, num_splits, static_cast<hipStream_t>(stream));
}


int32_t msa_indexer_decode_engine(const void* q, const void* k_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, int32_t batch,
                                  int32_t max_blocks_per_seq, int32_t bt_stride,
                                  int64_t num_pages, int32_t topk, int32_t n_init,
                                  int32_t n_local, int32_t* out_ids, float* out_scores,
                                  void* workspace, size_t workspace_bytes, int32_t num_splits,
                                  int32_t engine, void* stream) {
  return decode_impl(q, k_cache, block_table, seq_lens, batch, max_blocks_per_seq, bt_stride,
                     num_pages, topk, n_init, n_local, out_ids, out_scores, nullptr, nullptr,
                     workspace, workspace_bytes, num_splits, engine, static_cast<hipStream_t>(stream));
}

int32_t msa_indexer_decode(const void* q, const void* k_cache, const int32_t* block_table,
                           const int32_t* seq_lens, int32_t batch, int32_t max_blocks_per_seq,
                           int32_t bt_stride, int64_t num_pages, int32_t topk, int32_t n_init,
                           int32_t n_local, int32_t* out_ids, float* out_scores, void* workspace,
                           size_t workspace_bytes, int32_t num_splits, void* stream) {
  return decode_impl(q, k_cache, block_table, seq_lens, batch, max_blocks_per_seq, bt_stride,
                     num_pages, topk, n_init, n_local, out_ids, out_scores, nullptr, nullptr,
                     workspace, workspace_bytes, num_splits, MSA_ENGINE_DEFAULT,
                     static_cast<hipStream_t>(stream));
}

int32_t msa_indexer_decode_noalloc(const void* q, const void* k_cache, const int32_t* block_table,
                                   const int32_t* seq_lens, int32_t batch, int32_t max_blocks_per_seq,
                                   int32_t bt_stride, int64_t num_pages, int32_t topk, int32_t n_init,
                                   int32_t n_local, int32_t* out_ids, float* out_scores,
                                   uint32_t* error_flags, int32_t num_splits, void* stream) {
  if (error_flags != nullptr && !aligned(error_flags, 4)) return MSA_ERR_INVALID_ARG;
  const ScratchUse use{error_flags};
  return decode_impl(q, k_cache, block_table, seq_lens, batch, max_blocks_per_seq, bt_stride,
                     num_pages, topk, n_init, n_local, out_ids, out_scores, nullptr, nullptr,
                     nullptr, kNoallocBytes, num_splits, MSA_ENGINE_DEFAULT,
                     static_cast<hipStream_t>(stream), &use);
}

int32_t msa_indexer_decode_pages(const void* q, const void* k_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, int32_t batch,
                                 int32_t max_blocks_per_seq, int32_t bt_stride, int64_t num_pages,
                                 int32_t topk, int32_t n_init, int32_t n_local, int32_t* out_ids,
                                 float* out_scores, int32_t* out_pages, int32_t* out_tokens,
                                 void* workspace, size_t workspace_bytes, int32_t num_splits,
                                 int32_t engine, void* stream) {
  if (batch > 0 && (!out_pages || !out_tokens)) return MSA_ERR_INVALID_ARG;
  return decode_impl(q, k_cache, block_table, seq_lens, batch, max_blocks_per_seq, bt_stride,
                     num_pages, topk, n_init, n_local, out_ids, out_scores, out_pages, out_tokens,
                     workspace, workspace_bytes, num_splits, engine, static_cast<hipStream_t>(stream));
}

int32_t msa_indexer_expand_pages(const int32_t* ids, const int32_t* block_table,
                                 const int32_t* seq_lens, int32_t batch,
                                 int32_t max_blocks_per_seq, int32_t bt_stride, int32_t topk,
                                 int32_t* out_pages, int32_t* out_tokens, void* stream) {
  return msa_indexer_expand_pages_multi(ids, block_table, seq_lens, batch, max_blocks_per_seq,
                                        bt_stride, 1, topk, out_pages, out_tokens, stream);
}

int32_t msa_indexer_expand_pages_multi(const int32_t* ids, const int32_t* block_table,
                                       const int32_t* seq_lens, int32_t batch,
                                       int32_t max_blocks_per_seq, int32_t bt_stride, int32_t qlen,
                                       int32_t topk, int32_t* out_pages, int32_t* out_tokens,
                                       void* stream) {
  if (batch < 0 || max_blocks_per_seq < 0 || bt_stride < max_blocks_per_seq) return MSA_ERR_INVALID_ARG;
  if (topk < 1 || topk > MSA_MAX_TOPK || qlen < 1 || qlen > MSA_MAX_QUERY_LEN) return MSA_ERR_INVALID_ARG;
  if (max_blocks_per_seq > MSA_MAX_BLOCKS_PER_SEQ) return MSA_ERR_UNSUPPORTED;
  if (batch == 0) return MSA_OK;
  if (!ids || !seq_lens || !out_pages || !out_tokens || (!block_table && max_blocks_per_seq > 0))
    return MSA_ERR_INVALID_ARG;
  if (!aligned(ids, 4) || !aligned(seq_lens, 4) || !aligned(block_table, 4) ||
      !aligned(out_pages, 16) || !aligned(out_tokens, 4))
    return MSA_ERR_INVALID_ARG;
  ExpandArgs a;
  a.ids = ids;
  a.bt = block_table;
  a.lens = seq_lens;
  a.W = max_blocks_per_seq;
  a.bt_stride = bt_stride;
  a.topk = topk;
  a.Q = qlen;
  a.out_pages = out_pages;
  a.out_tokens = out_tokens;
  clear_stale_error();
  hipLaunchKernelGGL(expand_kernel, dim3(batch * qlen), dim3(kThreads), 0, static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}

int32_t msa_indexer_block_scores(const void* q, const void* k_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, int32_t batch,
                                 int32_t max_blocks_per_seq, int32_t bt_stride,
                                 int64_t num_pages, float* out, int32_t num_splits,
                                 int32_t engine, void* stream) {
  int32_t rc = check_inputs(q, k_cache, block_table, seq_lens, batch, max_blocks_per_seq, bt_stride,
                            num_pages);
  if (rc != MSA_OK) return rc;
  if (engine < MSA_ENGINE_DEFAULT || engine > MSA_ENGINE_MFMA) return MSA_ERR_INVALID_ARG;
  Plan p;
  if ((rc = make_plan(batch, max_blocks_per_seq, 16, num_splits, &p)) != MSA_OK) return rc;
  if (batch == 0 || max_blocks_per_seq == 0) return MSA_OK;
  if (!out || !aligned(out, 4)) return MSA_ERR_INVALID_ARG;
  SplitArgs a = make_split_args(q, k_cache, block_table, seq_lens, max_blocks_per_seq, bt_stride,
                                num_pages, p, 16, 0, 0, WsView{nullptr, nullptr, nullptr}, batch);
  a.scores = out;
  return launch_split<kScores>(a, batch, engine, 0, static_cast<hipStream_t>(stream));
}

int32_t msa_indexer_read_error(void* workspace, uint32_t* host_flags, void* stream) {
  if (!workspace || !host_flags || !aligned(workspace, kAlign)) return MSA_ERR_INVALID_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t* hdr = static_cast<uint32_t*>(workspace);
  // Read and clear in one atomic step on the caller's stream (so a bit a kernel sets between
  // the read and the clear cannot be lost, and the clear is ordered before the stream's next
  // kernel), then copy the staged word out.
  clear_stale_error();
  hipLaunchKernelGGL(take_error_kernel, dim3(1), dim3(1), 0, st, hdr);
  if (hipGetLastError() != hipSuccess) return MSA_ERR_HIP;
  if (hipMemcpyAsync(host_flags, hdr + 1, sizeof(uint32_t), hipMemcpyDeviceToHost, st) != hipSuccess)
    return MSA_ERR_HIP;
  return hipStreamSynchronize(st) == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}

size_t msa_indexer_workspace_bytes_multi(int32_t batch, int32_t max_blocks_per_seq, int32_t qlen,
                                         int32_t topk, int32_t num_splits) {
  Plan p;
  if (qlen < 1 || qlen > MSA_MAX_QUERY_LEN) return 0;
  if (make_decode_plan(batch, max_blocks_per_seq, topk, num_splits, &p) != MSA_OK) return 0;
  return ws_bytes(batch, max_blocks_per_seq, topk, num_splits, qlen);
}

int32_t msa_indexer_decode_multi(const void* q, const void* k_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, int32_t batch,
                                 int32_t max_blocks_per_seq, int32_t bt_stride, int64_t num_pages,
                                 int32_t qlen, int32_t topk, int32_t n_init, int32_t n_local,
                                 int32_t* out_ids, float* out_scores, void* workspace,
                                 size_t workspace_bytes, int32_t num_splits, void* stream) {
  return verify_decode_impl(q, k_cache, false, 1.0f, block_table, seq_lens, batch, max_blocks_per_seq,
                            bt_stride, num_pages, qlen, topk, n_init, n_local, out_ids, out_scores,
                            workspace, workspace_bytes, num_splits, static_cast<hipStream_t>(stream));
}

int32_t msa_indexer_decode_fp8(const void* q, const void* k_cache, float k_scale,
                               const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                               int32_t max_blocks_per_seq, int32_t bt_stride, int64_t num_pages,
                               int32_t qlen, int32_t topk, int32_t n_init, int32_t n_local,
                               int32_t* out_ids, float* out_scores, void* workspace,
                               size_t workspace_bytes, int32_t num_splits, void* stream) {
  return verify_decode_impl(q, k_cache, true, k_scale, block_table, seq_lens, batch, max_blocks_per_seq,
                            bt_stride, num_pages, qlen, topk, n_init, n_local, out_ids, out_scores,
                            workspace, workspace_bytes, num_splits, static_cast<hipStream_t>(stream));
}

int32_t msa_indexer_block_scores_multi(const void* q, const void* k_cache, const int32_t* block_table,
                                       const int32_t* seq_lens, int32_t batch,
                                       int32_t max_blocks_per_seq, int32_t bt_stride,
                                       int64_t num_pages, int32_t qlen, float* out,
                                       int32_t num_splits, void* stream) {
  return verify_scores_impl(q, k_cache, false, 1.0f, block_table, seq_lens, batch, max_blocks_per_seq,
                            bt_stride, num_pages, qlen, out, num_splits, static_cast<hipStream_t>(stream));
}

int32_t msa_indexer_block_scores_fp8(const void* q, const void* k_cache, float k_scale,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     int32_t batch, int32_t max_blocks_per_seq, int32_t bt_stride,
                                     int64_t num_pages, int32_t qlen, float* out, int32_t num_splits,
                                     void* stream) {
  return verify_scores_impl(q, k_cache, true, k_scale, block_table, seq_lens, batch, max_blocks_per_seq,
                            bt_stride, num_pages, qlen, out, num_splits, static_cast<hipStream_t>(stream));
}

}  // extern "C"
