// msa_indexer.hip -- MI355X (gfx950) kernels and C ABI of the MiniMax-M3 lightning-indexer
// decode pass. The ABI and the operation are documented in include/msa_indexer.h.
//
// Two kernels per call:
//   split_kernel  grid (S, batch), 4 waves. A workgroup owns C = ceil(W/S) consecutive
//                 logical blocks of one row (the split-KV axis of TensorRT-LLM PR #17008,
//                 Changes). Each wave walks every 4th block of the split: it reads the
//                 block's page once (32 KiB, 16 B per lane per load) and scores all four
//                 heads from those registers (SGLang PR #41488, Modifications: every K tile
//                 scored for all heads while resident). Block maxima go to LDS; then wave h
//                 ranks the split's keys for head h and writes its top-k, best first.
//   merge_kernel  grid (4, batch), 1 wave per (row, head): the exact top-min(k, nb) of the
//                 splits' sorted candidate lists, by repeated extraction of the largest list
//                 head (vLLM PR #57832, Solution: a global top-k block is in its own shard's
//                 top-k, so the merge of the per-shard lists is exact).
// Grid and workspace depend only on (batch, W, topk, S); per-row lengths are read on the
// device and splits past a row's end return at once (vLLM PR #57832, CUDA graph capture).

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "msa_indexer.h"

namespace {

constexpr int kHeads = MSA_INDEX_HEADS;
constexpr int kDim = MSA_HEAD_DIM;
constexpr int kBlock = MSA_BLOCK_TOKENS;
constexpr int kWaves = 4;                       // waves per split workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxSplitBlocks = 64;             // C <= 64: one split candidate per lane
constexpr int kMaxSplits = 256;                 // merge: at most 4 lists per lane
constexpr int kMaxMergeKeys = 4096;             // S * topk keys of one (row, head) in LDS
constexpr size_t kHeaderBytes = 256;            // workspace header (error word first)
constexpr int kPageElems = kBlock * kDim;       // bf16 elements per page

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------
// Cross-lane helpers (DPP within 16-lane rows, readlane across rows).

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, dpp_u32<CTRL>(__builtin_bit_cast(uint32_t, x)));
}

constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]: partner lane ^ 1
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]: partner lane ^ 2
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i within each 8 lanes
constexpr int kRowMirror = 0x140;     // lane i <-> 15-i within each 16 lanes

// Sum over the 16 lanes of each row; every lane of the row ends with the same value
// (each step adds a pair in the same order on both partners).
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f32<kQuadSwap1>(x);
  x += dpp_f32<kQuadSwap2>(x);
  x += dpp_f32<kRowHalfMirror>(x);
  x += dpp_f32<kRowMirror>(x);
  return x;
}

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
// products of its 8 dims with bf16 dot2 instructions (fp32 accumulate), the 16 lanes of a
// row are summed with DPP, and the running max is kept per row; rows merge at the end.
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

__device__ __forceinline__ void score_block_valu(const uint16_t* __restrict__ page, int valid,
                                                 const QValu& qr, int lane, float (&m)[kHeads]) {
  const uint4* p = reinterpret_cast<const uint4*>(page) + lane;
#pragma unroll
  for (int h = 0; h < kHeads; ++h) m[h] = -__builtin_inff();
  if (valid == kBlock) {
    uint4 kv[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) kv[i] = p[i * 64];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
#pragma unroll
      for (int h = 0; h < kHeads; ++h) m[h] = fmaxf(m[h], row_sum16(dot8(kv[i], qr.d[h])));
    }
  } else {
    const int row = lane >> 4;
    for (int i = 0; 4 * i < valid; ++i) {
      const uint4 kv = p[i * 64];
      const bool ok = 4 * i + row < valid;
#pragma unroll
      for (int h = 0; h < kHeads; ++h) {
        const float s = row_sum16(dot8(kv, qr.d[h]));
        m[h] = ok ? fmaxf(m[h], s) : m[h];
      }
    }
  }
#pragma unroll
  for (int h = 0; h < kHeads; ++h) {
    m[h] = fmaxf(m[h], __shfl_xor(m[h], 16));
    m[h] = fmaxf(m[h], __shfl_xor(m[h], 32));
  }
}

// MFMA engine. v_mfma_f32_16x16x32_bf16 with A = q (rows = heads, padded 4 -> 16 with
// zeros) and B = K^T (columns = 16 tokens of a tile). Lane l supplies row/column l%16 and
// 8 consecutive k-slots of lane group g = l/16; A and B use the same slots, so any fixed
// assignment of dims to slots gives the exact dot product. Step s (of 4) covers dims
// [32 s, 32 s + 32): group g takes dims 32 s + 8 g .. +7, so the four groups of one token
// read 64 contiguous bytes. The 16x16 result puts column l%16 in lane l, rows 4(l/16)..+3,
// so lanes 0..15 hold the four heads' scores of their token.
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
// Stage 1: scores + per-split top-k.

struct SplitArgs {
  const uint16_t* q;
  const uint16_t* k;
  const int32_t* bt;
  const int32_t* lens;
  int32_t W, bt_stride;
  int64_t num_pages;
  int32_t S, C, topk, n_init, n_local;
  uint64_t* keys;       // [batch][S][4][topk]
  uint32_t* err;        // device error word (may be null)
  float* scores;        // [batch][4][W] (block-score mode only)
};

__device__ __forceinline__ int row_tokens(const int32_t* lens, int b, int W) {
  const int L = lens[b];
  return L < 0 ? 0 : (L > W * kBlock ? W * kBlock : L);
}

template <int ENGINE, bool SCORES>
__global__ __launch_bounds__(kThreads) void split_kernel(SplitArgs a) {
  const int s = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int L = row_tokens(a.lens, b, a.W);
  const int nb = (L + kBlock - 1) / kBlock;
  const int j0 = s * a.C;
  const int j1 = min(j0 + a.C, nb);

  if (SCORES) {  // -inf for this split's blocks at or past the row's end
    const int e0 = max(j0, nb), e1 = min(j0 + a.C, a.W);
    for (int idx = threadIdx.x; idx < (e1 - e0) * kHeads; idx += kThreads) {
      const int h = idx / (e1 - e0), j = e0 + idx % (e1 - e0);
      a.scores[((size_t)b * kHeads + h) * a.W + j] = -__builtin_inff();
    }
  }
  if (j0 >= nb) return;

  __shared__ float sc[kMaxSplitBlocks][kHeads];

  typename std::conditional<ENGINE == MSA_ENGINE_MFMA, QMfma, QValu>::type qr;
  if constexpr (ENGINE == MSA_ENGINE_MFMA) load_q_mfma(a.q, b, lane, qr);
  else load_q_valu(a.q, b, lane, qr);

  const int32_t* btrow = a.bt + (size_t)b * a.bt_stride;
  for (int j = j0 + wave; j < j1; j += kWaves) {
    const int page = btrow[j];
    const int valid = min(kBlock, L - j * kBlock);
    float m[kHeads];
    if (page < 0 || (int64_t)page >= a.num_pages) {
#pragma unroll
      for (int h = 0; h < kHeads; ++h) m[h] = -__builtin_inff();
      if (a.err != nullptr && lane == 0) atomicOr(a.err, (uint32_t)MSA_DEVERR_PAGE_OUT_OF_RANGE);
    } else {
      const uint16_t* pg = a.k + (size_t)page * kPageElems;
      if constexpr (ENGINE == MSA_ENGINE_MFMA) score_block_mfma(pg, valid, qr, lane, m);
      else score_block_valu(pg, valid, qr, lane, m);
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < kHeads; ++h) sc[j - j0][h] = m[h];
    }
  }
  __syncthreads();

  const int n = j1 - j0;
  if (SCORES) {
    for (int idx = threadIdx.x; idx < n * kHeads; idx += kThreads) {
      const int h = idx / n, jj = idx % n;
      a.scores[((size_t)b * kHeads + h) * a.W + j0 + jj] = sc[jj][h];
    }
    return;
  }

  // Wave h ranks the split's keys of head h: rank = number of larger keys (keys are
  // distinct), so the keys of rank < topk land in best-first order.
  const int h = wave;
  uint64_t key = 0;
  if (lane < n) {
    const int j = j0 + lane;
    key = make_key(sc[lane][h], j, j < a.n_init || j >= nb - a.n_local);
  }
  int rank = 0;
  for (int i = 0; i < n; ++i) rank += readlane_u64(key, i) > key ? 1 : 0;
  uint64_t* out = a.keys + ((size_t)(b * a.S + s) * kHeads + h) * a.topk;
  const int cnt = min(a.topk, n);
  if (lane < n && rank < a.topk) out[rank] = key;
  if (lane >= cnt && lane < a.topk) out[lane] = 0;
}

// ---------------------------------------------------------------------------------------
// Stage 2: exact merge of the split lists.

struct MergeArgs {
  const int32_t* lens;
  int32_t W, S, C, topk;
  const uint64_t* keys;
  int32_t* out_ids;
  float* out_scores;
};

__global__ __launch_bounds__(64) void merge_kernel(MergeArgs a) {
  extern __shared__ uint64_t lk[];  // [ns][topk]
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int L = row_tokens(a.lens, b, a.W);
  const int nb = (L + kBlock - 1) / kBlock;
  const int m = min(a.topk, nb);
  const int ns = (nb + a.C - 1) / a.C;

  for (int idx = lane; idx < ns * a.topk; idx += 64) {
    const int s = idx / a.topk, i = idx % a.topk;
    lk[idx] = a.keys[((size_t)(b * a.S + s) * kHeads + h) * a.topk + i];
  }
  __syncthreads();

  constexpr int kLists = kMaxSplits / 64;
  uint64_t head[kLists];
  int ptr[kLists];
#pragma unroll
  for (int r = 0; r < kLists; ++r) {
    const int s = lane + 64 * r;
    ptr[r] = 0;
    head[r] = s < ns ? lk[s * a.topk] : 0;
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
      if (head[r] == w) {
        const int s = lane + 64 * r;
        ++ptr[r];
        head[r] = ptr[r] < a.topk ? lk[s * a.topk + ptr[r]] : 0;
      }
    }
  }
  if (lane < a.topk) {
    const size_t o = ((size_t)b * kHeads + h) * a.topk + lane;
    a.out_ids[o] = lane < m ? key_id(mine) : -1;
    a.out_scores[o] = lane < m ? key_score(mine) : -__builtin_inff();
  }
}

// ---------------------------------------------------------------------------------------
// Host side.

struct Plan {
  int S, C;
};

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

int pow2_ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Split plan from host arguments only. Automatic: C ~ batch*W/1024 blocks per split
// (about 4 waves x 4 KiB pages per SIMD of the chip), within [4, 64].
int32_t make_plan(int32_t batch, int32_t W, int32_t topk, int32_t num_splits, Plan* p) {
  if (batch < 0 || W < 0 || topk < 1 || topk > MSA_MAX_TOPK || num_splits < 0) return MSA_ERR_INVALID_ARG;
  if (W > MSA_MAX_BLOCKS_PER_SEQ) return MSA_ERR_UNSUPPORTED;
  if (W == 0) { p->S = 1; p->C = 1; return MSA_OK; }
  int cmin = 1;
  cmin = std::max(cmin, ceil_div((int64_t)W * topk, kMaxMergeKeys));
  cmin = std::max(cmin, ceil_div(W, kMaxSplits));
  int C;
  if (num_splits > 0) {
    C = ceil_div(W, num_splits);
  } else {
    C = pow2_ceil(std::max(1, ceil_div((int64_t)batch * W, 1024)));
    C = std::min(std::max(C, 4), kMaxSplitBlocks);
  }
  C = std::max(C, cmin);
  if (C > kMaxSplitBlocks) return MSA_ERR_UNSUPPORTED;
  p->C = C;
  p->S = ceil_div(W, C);
  return MSA_OK;
}

size_t ws_bytes(int32_t batch, const Plan& p, int32_t topk) {
  return kHeaderBytes + (size_t)batch * p.S * kHeads * topk * sizeof(uint64_t);
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

template <bool SCORES>
int32_t launch_split(const SplitArgs& a, int32_t batch, int32_t engine, hipStream_t st) {
  dim3 grid(a.S, batch), block(kThreads);
  if (engine == MSA_ENGINE_DEFAULT) engine = MSA_ENGINE_VALU;
  if (engine == MSA_ENGINE_VALU)
    hipLaunchKernelGGL((split_kernel<MSA_ENGINE_VALU, SCORES>), grid, block, 0, st, a);
  else if (engine == MSA_ENGINE_MFMA)
    hipLaunchKernelGGL((split_kernel<MSA_ENGINE_MFMA, SCORES>), grid, block, 0, st, a);
  else
    return MSA_ERR_INVALID_ARG;
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}

int32_t split_topk_impl(const void* q, const void* k, const int32_t* bt, const int32_t* lens,
                        int32_t batch, int32_t W, int32_t bt_stride, int64_t num_pages,
                        int32_t topk, int32_t n_init, int32_t n_local, void* ws, size_t ws_size,
                        int32_t num_splits, int32_t engine, hipStream_t st) {
  int32_t rc = check_inputs(q, k, bt, lens, batch, W, bt_stride, num_pages);
  if (rc != MSA_OK) return rc;
  if ((rc = check_select(topk, n_init, n_local)) != MSA_OK) return rc;
  if (engine < MSA_ENGINE_DEFAULT || engine > MSA_ENGINE_MFMA) return MSA_ERR_INVALID_ARG;
  Plan p;
  if ((rc = make_plan(batch, W, topk, num_splits, &p)) != MSA_OK) return rc;
  if (batch == 0) return MSA_OK;
  if (!ws || !aligned(ws, 256)) return MSA_ERR_INVALID_ARG;
  if (ws_size < ws_bytes(batch, p, topk)) return MSA_ERR_WORKSPACE_TOO_SMALL;
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
  a.topk = topk;
  a.n_init = n_init;
  a.n_local = n_local;
  a.err = static_cast<uint32_t*>(ws);
  a.keys = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + kHeaderBytes);
  a.scores = nullptr;
  return launch_split<false>(a, batch, engine, st);
}

int32_t merge_impl(const int32_t* lens, int32_t batch, int32_t W, int32_t topk, int32_t* out_ids,
                   float* out_scores, const void* ws, size_t ws_size, int32_t num_splits,
                   hipStream_t st) {
  if (batch < 0 || W < 0) return MSA_ERR_INVALID_ARG;
  if (topk < 1 || topk > MSA_MAX_TOPK) return MSA_ERR_INVALID_ARG;
  Plan p;
  int32_t rc = make_plan(batch, W, topk, num_splits, &p);
  if (rc != MSA_OK) return rc;
  if (batch == 0) return MSA_OK;
  if (!lens || !out_ids || !out_scores || !ws) return MSA_ERR_INVALID_ARG;
  if (!aligned(lens, 4) || !aligned(out_ids, 4) || !aligned(out_scores, 4) || !aligned(ws, 256))
    return MSA_ERR_INVALID_ARG;
  if (ws_size < ws_bytes(batch, p, topk)) return MSA_ERR_WORKSPACE_TOO_SMALL;
  MergeArgs a;
  a.lens = lens;
  a.W = W;
  a.S = p.S;
  a.C = p.C;
  a.topk = topk;
  a.keys = reinterpret_cast<const uint64_t*>(static_cast<const char*>(ws) + kHeaderBytes);
  a.out_ids = out_ids;
  a.out_scores = out_scores;
  const size_t lds = (size_t)p.S * topk * sizeof(uint64_t);
  hipLaunchKernelGGL(merge_kernel, dim3(kHeads, batch), dim3(64), lds, st, a);
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
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
  const int32_t rc = make_plan(batch, max_blocks_per_seq, topk, num_splits, &p);
  return rc == MSA_OK ? p.S : rc;
}

size_t msa_indexer_workspace_bytes(int32_t batch, int32_t max_blocks_per_seq, int32_t topk,
                                   int32_t num_splits) {
  Plan p;
  if (make_plan(batch, max_blocks_per_seq, topk, num_splits, &p) != MSA_OK) return 0;
  return ws_bytes(batch, p, topk);
}

int32_t msa_indexer_split_topk(const void* q, const void* k_cache, const int32_t* block_table,
                               const int32_t* seq_lens, int32_t batch,
                               int32_t max_blocks_per_seq, int32_t bt_stride, int64_t num_pages,
                               int32_t topk, int32_t n_init, int32_t n_local, void* workspace,
                               size_t workspace_bytes, int32_t num_splits, int32_t engine,
                               void* stream) {
  return split_topk_impl(q, k_cache, block_table, seq_lens, batch, max_blocks_per_seq, bt_stride,
                         num_pages, topk, n_init, n_local, workspace, workspace_bytes, num_splits,
                         engine, static_cast<hipStream_t>(stream));
}

int32_t msa_indexer_merge(const int32_t* seq_lens, int32_t batch, int32_t max_blocks_per_seq,
                          int32_t topk, int32_t* out_ids, float* out_scores,
                          const void* workspace, size_t workspace_bytes, int32_t num_splits,
                          void* stream) {
  return merge_impl(seq_lens, batch, max_blocks_per_seq, topk, out_ids, out_scores, workspace,
                    workspace_bytes, num_splits, static_cast<hipStream_t>(stream));
}

int32_t msa_indexer_decode(const void* q, const void* k_cache, const int32_t* block_table,
                           const int32_t* seq_lens, int32_t batch, int32_t max_blocks_per_seq,
                           int32_t bt_stride, int64_t num_pages, int32_t topk, int32_t n_init,
                           int32_t n_local, int32_t* out_ids, float* out_scores, void* workspace,
                           size_t workspace_bytes, int32_t num_splits, void* stream) {
  // Check everything (outputs included) before the first launch.
  if (batch > 0 && (!out_ids || !out_scores || !aligned(out_ids, 4) || !aligned(out_scores, 4)))
    return MSA_ERR_INVALID_ARG;
  int32_t rc = split_topk_impl(q, k_cache, block_table, seq_lens, batch, max_blocks_per_seq,
                               bt_stride, num_pages, topk, n_init, n_local, workspace,
                               workspace_bytes, num_splits, MSA_ENGINE_DEFAULT,
                               static_cast<hipStream_t>(stream));
  if (rc != MSA_OK) return rc;
  return merge_impl(seq_lens, batch, max_blocks_per_seq, topk, out_ids, out_scores, workspace,
                    workspace_bytes, num_splits, static_cast<hipStream_t>(stream));
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
  SplitArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.bt = block_table;
  a.lens = seq_lens;
  a.W = max_blocks_per_seq;
  a.bt_stride = bt_stride;
  a.num_pages = num_pages;
  a.S = p.S;
  a.C = p.C;
  a.topk = 16;
  a.n_init = 0;
  a.n_local = 0;
  a.keys = nullptr;
  a.err = nullptr;
  a.scores = out;
  return launch_split<true>(a, batch, engine, static_cast<hipStream_t>(stream));
}

int32_t msa_indexer_read_error(void* workspace, uint32_t* host_flags, void* stream) {
  if (!workspace || !host_flags) return MSA_ERR_INVALID_ARG;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return MSA_ERR_HIP;
  if (hipMemcpy(host_flags, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess)
    return MSA_ERR_HIP;
  if (hipMemset(workspace, 0, sizeof(uint32_t)) != hipSuccess) return MSA_ERR_HIP;
  return MSA_OK;
}

}  // extern "C"
