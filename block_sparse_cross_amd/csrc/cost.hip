// Realized attention cost per (query block, KV chunk).
//
// Split-KV page, Abstract: KV chunks are balanced by their realized attention
// cost.  Unit: visible (query, context key) pairs of one head, in int64:
//   counts[b][c]  = B * |[start_c, start_c + len_c) ∩ [ctx_begin_b, anchor_b)|
//   chunk_cost[c] = sum_b counts[b][c]
// A workgroup owns 64 chunks; its four waves take every fourth block, reading the
// block ranges from LDS (staged 256 at a time with coalesced loads), so each lane
// walks only a quarter of the blocks with no dependent global loads.  Counts rows
// are written with coalesced stores; the four partial chunk sums meet in LDS, so
// chunk_cost needs no atomics.  Workgroup 0 also checks every block's range and
// writes mask_err (0 or 1) itself, so the flag needs no clearing beforehand.
#include <hip/hip_runtime.h>

#include "bsx_internal.h"

namespace bsx {
namespace {

constexpr int kThreads = 256;
constexpr int kChunksPerWg = 64;

__global__ __launch_bounds__(kThreads) void cost_kernel(CostParams p) {
  __shared__ int64_t s_lo[kThreads], s_hi[kThreads];
  __shared__ int64_t s_part[4][kChunksPerWg];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x * kChunksPerWg + lane;
  const bool c_ok = c < p.n_chunks;
  int64_t c0 = 0, c1 = 0;
  if (c_ok) {
    const ChunkEntry ce = reinterpret_cast<const ChunkEntry*>(p.table.base())[c];
    c0 = ce.start;
    c1 = c0 + ce.len;
  }
  int bad = 0;
  int64_t total = 0;
  for (int b0 = 0; b0 < p.n_blocks; b0 += kThreads) {
    const int b = b0 + tid;
    if (b < p.n_blocks) {
      int64_t lo = p.ctx_begin[b], hi = p.anchor[b];
      bad |= (lo < 0) | (lo > hi) | (hi > p.ctx_len);
      lo = lo < 0 ? 0 : (lo > p.ctx_len ? p.ctx_len : lo);
      hi = hi < lo ? lo : (hi > p.ctx_len ? p.ctx_len : hi);
      s_lo[tid] = lo;
      s_hi[tid] = hi;
    }
    __syncthreads();
    const int nb = p.n_blocks - b0 < kThreads ? p.n_blocks - b0 : kThreads;
    for (int i = wave; i < nb; i += 4) {
      const int64_t a = s_lo[i] > c0 ? s_lo[i] : c0;
      const int64_t z = s_hi[i] < c1 ? s_hi[i] : c1;
      const int64_t n = z > a ? (z - a) * p.block_size : 0;
      if (c_ok && p.counts) p.counts[int64_t(b0 + i) * p.n_chunks + c] = n;
      total += n;
    }
    __syncthreads();
  }
  s_part[wave][lane] = total;
  bad = __syncthreads_or(bad);
  if (blockIdx.x == 0 && tid == 0) *p.mask_err = bad ? 1 : 0;
  if (wave == 0 && c_ok)
    p.chunk_cost[c] = s_part[0][lane] + s_part[1][lane] + s_part[2][lane] + s_part[3][lane];
}

}  // namespace

hipError_t launch_cost(const CostParams& p, hipStream_t stream) {
  const int blocks = p.n_chunks > 0 ? (p.n_chunks + kChunksPerWg - 1) / kChunksPerWg : 1;
  hipLaunchKernelGGL(cost_kernel, dim3(blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace bsx
