// Exact merge of partial (O, LSE) pairs.
//
// Split-KV page, Abstract: the context-parallel method is exact while moving only
// query-sized tensors.  With normalized partials the exact combination is
//   LSE = M + log sum_p exp(LSE_p - M),   O = sum_p exp(LSE_p - LSE) O_p,
// M = max_p LSE_p; partials with LSE_p = -inf are skipped without reading O_p.
//
// Bandwidth-bound: the kernel streams every finite partial row once.  A workgroup
// owns kRowsPerWg consecutive rows (few, so thousands of workgroups keep enough
// loads in flight).  Phase 1: 16 lane groups split the partials, each lane keeps
// an online (max, sum) for one row from coalesced LSE loads, and the partial sums
// meet in LDS.  Phase 2: the weights exp(LSE_p - LSE) of up to kPartsPerPass
// partials go to LDS, so the O loads that follow depend on nothing in flight;
// head_dim/4 lanes per row each own one float4 of the row and accumulate the
// weighted partial rows with the part loop unrolled (several 16-byte loads in
// flight per lane).  A partial with zero weight (LSE = -inf) is never loaded.
#include <hip/hip_runtime.h>

#include <math.h>

#include "bsx_internal.h"

namespace bsx {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWg = 16;
constexpr int kGroups = kThreads / kRowsPerWg;  // partial groups in phase 1
constexpr int kUnroll = 8;
constexpr int kPartsPerPass = 128;

__global__ __launch_bounds__(kThreads) void lse_merge_kernel(int n_parts, int64_t n_rows,
                                                             int head_dim,
                                                             const float* __restrict__ o_parts,
                                                             const float* __restrict__ lse_parts,
                                                             float* __restrict__ o_out,
                                                             float* __restrict__ lse_out) {
  __shared__ float sh_m[kGroups][kRowsPerWg];
  __shared__ float sh_s[kGroups][kRowsPerWg];
  __shared__ float sh_lse[kRowsPerWg];
  __shared__ float sh_w[kPartsPerPass][kRowsPerWg];
  const int tid = threadIdx.x;
  const int64_t row0 = int64_t(blockIdx.x) * kRowsPerWg;

  // Phase 1: online max/sum of exp over this group's share of the partials.
  {
    const int i = tid % kRowsPerWg, grp = tid / kRowsPerWg;
    const int64_t row = row0 + i;
    float m = -INFINITY, s = 0.f;
    if (row < n_rows) {
      for (int p = grp; p < n_parts; p += kGroups) {
        const float x = lse_parts[int64_t(p) * n_rows + row];
        if (x == -INFINITY) continue;
        if (x > m) {
          s = s * expf(m - x) + 1.f;
          m = x;
        } else {
          s += expf(x - m);
        }
      }
    }
    sh_m[grp][i] = m;
    sh_s[grp][i] = s;
  }
  __syncthreads();
  if (tid < kRowsPerWg) {
    float m = -INFINITY;
    for (int w = 0; w < kGroups; ++w) m = fmaxf(m, sh_m[w][tid]);
    float lse = -INFINITY;
    if (m != -INFINITY) {
      float s = 0.f;
      for (int w = 0; w < kGroups; ++w)
        if (sh_m[w][tid] != -INFINITY) s += sh_s[w][tid] * expf(sh_m[w][tid] - m);
      lse = m + logf(s);
    }
    sh_lse[tid] = lse;
    const int64_t row = row0 + tid;
    if (row < n_rows) lse_out[row] = lse;
  }
  __syncthreads();

  // Phase 2: weighted sum of the finite partial rows, kPartsPerPass partials at a
  // time; with more partials than that, later passes add to the row written so far.
  const int tpr = head_dim >> 2;              // lanes per row, one float4 each
  const int rows_per_pass = kThreads / tpr;
  const int sub = tid / tpr, col = (tid % tpr) * 4;
  for (int p0 = 0; p0 < n_parts; p0 += kPartsPerPass) {
    const int np = n_parts - p0 < kPartsPerPass ? n_parts - p0 : kPartsPerPass;
    __syncthreads();  // previous weights are no longer read
    for (int idx = tid; idx < np * kRowsPerWg; idx += kThreads) {
      const int pp = idx / kRowsPerWg, i = idx % kRowsPerWg;
      const int64_t row = row0 + i;
      float w = 0.f;
      if (row < n_rows && sh_lse[i] != -INFINITY) {
        const float x = lse_parts[int64_t(p0 + pp) * n_rows + row];
        if (x != -INFINITY) w = expf(x - sh_lse[i]);
      }
      sh_w[pp][i] = w;
    }
    __syncthreads();
    if (sub >= rows_per_pass) continue;
    for (int r = sub; r < kRowsPerWg; r += rows_per_pass) {
      const int64_t row = row0 + r;
      if (row >= n_rows) break;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      if (p0 > 0) acc = *reinterpret_cast<const float4*>(o_out + row * head_dim + col);
      const float* op = o_parts + row * head_dim + col;
      const int64_t ostride = n_rows * int64_t(head_dim);
      int pp = 0;
      for (; pp + kUnroll <= np; pp += kUnroll) {
        float w[kUnroll];
        float4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          w[u] = sh_w[pp + u][r];
          v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (w[u] != 0.f)
            v[u] = *reinterpret_cast<const float4*>(op + int64_t(p0 + pp + u) * ostride);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          acc.x = fmaf(w[u], v[u].x, acc.x);
          acc.y = fmaf(w[u], v[u].y, acc.y);
          acc.z = fmaf(w[u], v[u].z, acc.z);
          acc.w = fmaf(w[u], v[u].w, acc.w);
        }
      }
      for (; pp < np; ++pp) {
        const float w = sh_w[pp][r];
        if (w == 0.f) continue;
        const float4 v = *reinterpret_cast<const float4*>(op + int64_t(p0 + pp) * ostride);
        acc.x = fmaf(w, v.x, acc.x);
        acc.y = fmaf(w, v.y, acc.y);
        acc.z = fmaf(w, v.z, acc.z);
        acc.w = fmaf(w, v.w, acc.w);
      }
      *reinterpret_cast<float4*>(o_out + row * head_dim + col) = acc;
    }
  }
}

}  // namespace

hipError_t launch_lse_merge(int32_t n_parts, int64_t n_rows, int32_t head_dim,
                            const float* o_parts, const float* lse_parts, float* o_out,
                            float* lse_out, hipStream_t stream) {
  const int64_t blocks = (n_rows + kRowsPerWg - 1) / kRowsPerWg;
  hipLaunchKernelGGL(lse_merge_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, n_parts,
                     n_rows, head_dim, o_parts, lse_parts, o_out, lse_out);
  return hipGetLastError();
}

}  // namespace bsx
