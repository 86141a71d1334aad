// stream_probe.hip -- a measurement aid beside the decode library (libmsa_probe.so): reads
// the index-K pages a decode call over full-length rows reads, through the same shuffled block
// table, with the decode kernels' load pattern, and does nothing with the bytes but fold them
// into one XOR word per lane (so the loads cannot be dropped). Its time is the streaming
// ceiling the decode kernels are measured against: what HBM gives this access pattern.
//
// Both patterns split row b into contiguous ranges of C blocks, one workgroup of 4 waves per
// range, wave w taking every 4th block of its range (the decode's split-KV decomposition), and
// read a page with 1 KiB wave loads of 16 bytes per lane, non-temporal:
//   kSplitPattern   the VALU decode kernel's: each page in batches of 16 loads (16 KiB),
//                   one batch landing before the next is issued;
//   kChunkPattern   the verify kernel's (multi-token and FP8 passes): a wave's pages as one
//                   stream of 8 KiB chunks (8 loads), two chunks in flight.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "msa_probe.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void fold(uint4& x, const uint4& v) {
  x.x ^= v.x;
  x.y ^= v.y;
  x.z ^= v.z;
  x.w ^= v.w;
}

struct ProbeArgs {
  const uint8_t* k;
  const int32_t* bt;
  int32_t W, bt_stride, C, loads_per_page;  // loads_per_page: page bytes / 1 KiB
  uint32_t* out;                            // [batch][S][256]
};

constexpr int kBatch = 16;  // split pattern: loads per batch
constexpr int kChunk = 8;   // chunk pattern: loads per chunk

template <int PATTERN>
__global__ __launch_bounds__(256) void probe_kernel(ProbeArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = blockIdx.x, b = blockIdx.y;
  const int j0 = s * a.C, j1 = min(j0 + a.C, a.W);
  const int32_t* btrow = a.bt + (size_t)b * a.bt_stride;
  const size_t page_bytes = (size_t)a.loads_per_page * 1024;
  uint4 x = make_uint4(0, 0, 0, 0);
  if (PATTERN == MSA_PROBE_SPLIT_PATTERN) {
    for (int j = j0 + wave; j < j1; j += 4) {
      const uint4* p = reinterpret_cast<const uint4*>(a.k + (size_t)btrow[j] * page_bytes) + lane;
      for (int i0 = 0; i0 < a.loads_per_page; i0 += kBatch) {
        uint4 v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) v[i] = load_stream(p + (i0 + i) * 64);
#pragma unroll
        for (int i = 0; i < kBatch; ++i) fold(x, v[i]);
      }
    }
  } else {
    // The wave's chunks, in order: chunk c is chunk c % cpp of its (c / cpp)-th block.
    const int cpp = a.loads_per_page / kChunk;
    const int nblk = j1 > j0 + wave ? (j1 - j0 - wave + 3) / 4 : 0;
    const int n = nblk * cpp;
    auto ptr = [&](int c) {
      const int j = j0 + wave + 4 * (c / cpp);
      return reinterpret_cast<const uint4*>(a.k + (size_t)btrow[j] * page_bytes) + (c % cpp) * kChunk * 64 + lane;
    };
    auto load = [&](int c, uint4 (&v)[kChunk]) {
      if (c < n) {
        const uint4* p = ptr(c);
#pragma unroll
        for (int i = 0; i < kChunk; ++i) v[i] = load_stream(p + i * 64);
      }
    };
    auto take = [&](const uint4 (&v)[kChunk]) {
#pragma unroll
      for (int i = 0; i < kChunk; ++i) fold(x, v[i]);
    };
    uint4 A[kChunk], B[kChunk];
    load(0, A);
    load(1, B);
    for (int c = 0; c < n; c += 2) {
      take(A);
      load(c + 2, A);
      if (c + 1 >= n) break;
      take(B);
      load(c + 3, B);
    }
  }
  a.out[((size_t)b * gridDim.x + s) * 256 + threadIdx.x] = x.x ^ x.y ^ x.z ^ x.w;
}

}  // namespace

extern "C" int32_t msa_probe_stream_pages(const void* k_cache, int32_t page_bytes,
                                          const int32_t* block_table, int32_t batch, int32_t W,
                                          int32_t bt_stride, int32_t blocks_per_wg, int32_t pattern,
                                          uint32_t* out, void* stream) {
  if (!k_cache || !block_table || !out || batch <= 0 || W <= 0 || bt_stride < W || blocks_per_wg <= 0)
    return -1;
  if (page_bytes <= 0 || page_bytes % (1024 * kBatch) != 0) return -1;  // whole batches and chunks
  if (pattern != MSA_PROBE_SPLIT_PATTERN && pattern != MSA_PROBE_CHUNK_PATTERN) return -1;
  if (reinterpret_cast<uintptr_t>(k_cache) % 16 != 0) return -1;
  ProbeArgs a;
  a.k = static_cast<const uint8_t*>(k_cache);
  a.bt = block_table;
  a.W = W;
  a.bt_stride = bt_stride;
  a.C = blocks_per_wg;
  a.loads_per_page = page_bytes / 1024;
  a.out = out;
  const dim3 grid((W + blocks_per_wg - 1) / blocks_per_wg, batch);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (pattern == MSA_PROBE_SPLIT_PATTERN)
    hipLaunchKernelGGL(probe_kernel<MSA_PROBE_SPLIT_PATTERN>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(probe_kernel<MSA_PROBE_CHUNK_PATTERN>, grid, dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
