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
// Launches over many blocks split them into groups along the grid's second
// dimension (otherwise a few thousand chunks would give only tens of workgroups);
// each group leaves its chunk sums and flag in the workspace and a small second pass
// adds them.
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
  // this workgroup's blocks: group blockIdx.y of `span` blocks
  const int b_begin = int(blockIdx.y) * p.span;
  const int b_end = p.n_blocks - b_begin < p.span ? p.n_blocks : b_begin + p.span;
  int bad = 0;
  int64_t total = 0;
  for (int b0 = b_begin; b0 < b_end; b0 += kThreads) {
    const int b = b0 + tid;
    if (b < b_end) {
      int64_t lo = p.ctx_begin[b], hi = p.anchor[b];
      bad |= (lo < 0) | (lo > hi) | (hi > p.ctx_len);
      lo = lo < 0 ? 0 : (lo > p.ctx_len ? p.ctx_len : lo);
      hi = hi < lo ? lo : (hi > p.ctx_len ? p.ctx_len : hi);
      s_lo[tid] = lo;
      s_hi[tid] = hi;
    }
    __syncthreads();
    const int nb = b_end - b0 < kThreads ? b_end - b0 : kThreads;
    for (int i = wave; i < nb; i += 4) {
      const int64_t a = s_lo[i] > c0 ? s_lo[i] : c0;
      const int64_t z = s_hi[i] < c1 ? s_hi[i] : c1;
      const int64_t n = z > a ? (z - a) * p.block_size : 0;
      // counts are written once and not read back here: non-temporal stores
      if (c_ok && p.counts) __builtin_nontemporal_store(n, p.counts + int64_t(b0 + i) * p.n_chunks + c);
      total += n;
    }
    __syncthreads();
  }
  s_part[wave][lane] = total;
  bad = __syncthreads_or(bad);
  const int64_t sum = s_part[0][lane] + s_part[1][lane] + s_part[2][lane] + s_part[3][lane];
  if (!p.part) {
    if (blockIdx.x == 0 && tid == 0) *p.mask_err = bad ? 1 : 0;
    if (wave == 0 && c_ok) p.chunk_cost[c] = sum;
  } else {
    if (blockIdx.x == 0 && tid == 0) p.bad[blockIdx.y] = bad;
    if (wave == 0 && c_ok) p.part[int64_t(blockIdx.y) * p.n_chunks + c] = sum;
  }
}

// Adds the block groups' chunk sums (exact integer sums) and their mask flags.
__global__ __launch_bounds__(kThreads) void cost_sum_kernel(CostParams p, int n_groups) {
  const int c = blockIdx.x * kThreads + threadIdx.x;
  if (c < p.n_chunks) {
    int64_t t = 0;
    for (int g = 0; g < n_groups; ++g) t += p.part[int64_t(g) * p.n_chunks + c];
    p.chunk_cost[c] = t;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    int any = 0;
    for (int g = 0; g < n_groups; ++g) any |= p.bad[g];
    *p.mask_err = any ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_cost(const CostParams& p, hipStream_t stream) {
  const int blocks = p.n_chunks > 0 ? (p.n_chunks + kChunksPerWg - 1) / kChunksPerWg : 1;
  const int groups = p.part ? (p.n_blocks + p.span - 1) / p.span : 1;
  hipLaunchKernelGGL(cost_kernel, dim3(blocks, groups), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !p.part) return e;
  const int sum_blocks = p.n_chunks > 0 ? (p.n_chunks + kThreads - 1) / kThreads : 1;
  hipLaunchKernelGGL(cost_sum_kernel, dim3(sum_blocks), dim3(kThreads), 0, stream, p, groups);
  return hipGetLastError();
}

}  // namespace bsx
