// Realized attention cost per (query block, KV chunk).
//
// Split-KV page, Abstract: KV chunks are balanced by their realized attention
// cost.  Unit: visible (query, context key) pairs of one head, in int64:
//   counts[b][c]  = B * |[start_c, start_c + len_c) ∩ [ctx_begin_b, anchor_b)|
//   chunk_cost[c] = sum_b counts[b][c]
// One thread owns one chunk and walks the blocks, so every counts row is written
// with coalesced stores and chunk_cost needs no atomics.  Workgroup 0 also checks
// every block's range and writes mask_err (0 or 1) itself, so the flag needs no
// clearing beforehand.
#include <hip/hip_runtime.h>

#include "bsx_internal.h"

namespace bsx {
namespace {

__device__ inline void clamp_range(int64_t lo, int64_t hi, int64_t S, int64_t* clo,
                                   int64_t* chi) {
  lo = lo < 0 ? 0 : (lo > S ? S : lo);
  hi = hi < lo ? lo : (hi > S ? S : hi);
  *clo = lo;
  *chi = hi;
}

__global__ __launch_bounds__(256) void cost_kernel(CostParams p) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (blockIdx.x == 0) {
    int bad = 0;
    for (int b = threadIdx.x; b < p.n_blocks; b += blockDim.x) {
      const int64_t lo = p.ctx_begin[b], hi = p.anchor[b];
      bad |= (lo < 0) | (lo > hi) | (hi > p.ctx_len);
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) *p.mask_err = bad ? 1 : 0;
  }
  if (c >= p.n_chunks) return;
  const ChunkEntry ce = reinterpret_cast<const ChunkEntry*>(p.table.base())[c];
  const int64_t c0 = ce.start;
  const int64_t c1 = c0 + ce.len;
  int64_t total = 0;
  for (int b = 0; b < p.n_blocks; ++b) {
    int64_t lo, hi;
    clamp_range(p.ctx_begin[b], p.anchor[b], p.ctx_len, &lo, &hi);
    const int64_t a = lo > c0 ? lo : c0;
    const int64_t z = hi < c1 ? hi : c1;
    const int64_t n = z > a ? (z - a) * p.block_size : 0;
    if (p.counts) p.counts[int64_t(b) * p.n_chunks + c] = n;
    total += n;
  }
  p.chunk_cost[c] = total;
}

}  // namespace

hipError_t launch_cost(const CostParams& p, hipStream_t stream) {
  const int blocks = p.n_chunks > 0 ? (p.n_chunks + 255) / 256 : 1;
  hipLaunchKernelGGL(cost_kernel, dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace bsx
