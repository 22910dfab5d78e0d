// Exact merge of partial (O, LSE) pairs.
//
// Split-KV page, Abstract: the context-parallel method is exact while moving only
// query-sized tensors.  With normalized partials the exact combination is
//   LSE = M + log sum_p exp(LSE_p - M),   O = sum_p exp(LSE_p - LSE) O_p,
// M = max_p LSE_p; partials with LSE_p = -inf are skipped without reading O_p.
//
// Bandwidth-bound: every finite partial row is streamed once, with non-temporal
// loads and stores (read-once data need not displace the caches).  A workgroup owns
// kRowsPerWg consecutive rows.  Phase 1: the partial LSEs of those rows are read
// once into LDS while lane groups keep an online (max, sum) per row; the group sums
// meet in LDS and give each row's LSE.  Phase 2: the LDS values become weights
// exp(LSE_p - LSE) (0 for an empty partial); head_dim/4 lanes per row each own one
// float4 column, and every lane accumulates kRowsPerThread rows at once, so each
// partial is read as one contiguous piece of kRowsPerWg rows.  The loads of the next
// kUnroll partials are issued before the current ones are consumed.  A merge too small
// to fill the chip twice over with 32-row workgroups (the training step's: 17 sets of
// 32K rows) runs 16-row workgroups with four partials in flight per row instead: its
// time is one workgroup's chain of dependent loads, not the memory system's rate.
#include <hip/hip_runtime.h>

#include <math.h>

#include "bsx_internal.h"

namespace bsx {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kPartsPerPass = kMergeBf16MaxParts;  // weights held in LDS at once
constexpr int64_t kSmallMergeWgs = 1024;  // 32-row workgroups in two rounds of four per CU

__device__ inline f32x4 load_nt(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}

// Stores a merged row piece: f32 as is, or rounded to bf16 (nearest, ties to even).
template <bool kBf16>
__device__ inline void store_row(void* o_out, int64_t at, f32x4 v) {
  if constexpr (kBf16) {
    typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
    const bf16x4v b = {static_cast<__bf16>(v.x), static_cast<__bf16>(v.y),
                       static_cast<__bf16>(v.z), static_cast<__bf16>(v.w)};
    __builtin_nontemporal_store(__builtin_bit_cast(uint64_t, b),
                                reinterpret_cast<uint64_t*>(static_cast<__bf16*>(o_out) + at));
  } else {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(static_cast<float*>(o_out) + at));
  }
}

// kBf16: the merged O is written as bf16; launched only when one pass of weights covers
// every partial (the f32 path adds later passes to the rows written so far).
// kRowsPerThread rows per lane, kRowsPerWg per workgroup, kUnroll partials in flight.
template <bool kBf16, int kRowsPerThread, int kRowsPerWg, int kUnroll>
__global__ __launch_bounds__(kThreads) void lse_merge_kernel(int n_parts, int64_t n_rows,
                                                             int head_dim,
                                                             const float* __restrict__ o_parts,
                                                             const float* __restrict__ lse_parts,
                                                             void* __restrict__ o_out,
                                                             float* __restrict__ lse_out) {
  constexpr int kGroups = kThreads / kRowsPerWg;  // lane groups of phase 1
  static_assert(kThreads % kRowsPerWg == 0, "phase 1 needs whole lane groups");
  __shared__ float sh_m[kGroups][kRowsPerWg];
  __shared__ float sh_s[kGroups][kRowsPerWg];
  __shared__ float sh_lse[kRowsPerWg];
  __shared__ float sh_w[kPartsPerPass][kRowsPerWg];  // partial LSEs, then weights
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
        if (p < kPartsPerPass) sh_w[p][i] = x;
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
    for (int g = 0; g < kGroups; ++g) m = fmaxf(m, sh_m[g][tid]);
    float lse = -INFINITY;
    if (m != -INFINITY) {
      float s = 0.f;
      for (int g = 0; g < kGroups; ++g)
        if (sh_m[g][tid] != -INFINITY) s += sh_s[g][tid] * expf(sh_m[g][tid] - m);
      lse = m + logf(s);
    }
    sh_lse[tid] = lse;
    const int64_t row = row0 + tid;
    if (row < n_rows) lse_out[row] = lse;
  }
  __syncthreads();

  // Phase 2: weighted sum of the finite partial rows, kPartsPerPass partials at a
  // time; with more partials than that, later passes reload their LSEs and add to
  // the rows written so far.
  const int tpr = head_dim >> 2;  // lanes per row, one float4 each
  const int rows_per_pass = kThreads / tpr;
  const int sub = tid / tpr, col = (tid % tpr) * 4;
  const int64_t pstride = n_rows * int64_t(head_dim);
  for (int p0 = 0; p0 < n_parts; p0 += kPartsPerPass) {
    const int np = n_parts - p0 < kPartsPerPass ? n_parts - p0 : kPartsPerPass;
    if (p0 > 0) __syncthreads();  // the previous pass's weights are no longer read
    for (int idx = tid; idx < np * kRowsPerWg; idx += kThreads) {
      const int pp = idx / kRowsPerWg, i = idx % kRowsPerWg;
      const int64_t row = row0 + i;
      float x = -INFINITY;
      if (row < n_rows) x = p0 == 0 ? sh_w[pp][i] : lse_parts[int64_t(p0 + pp) * n_rows + row];
      sh_w[pp][i] = (x == -INFINITY || sh_lse[i] == -INFINITY) ? 0.f : expf(x - sh_lse[i]);
    }
    __syncthreads();
    if (sub >= rows_per_pass) continue;
    for (int rb = sub; rb < kRowsPerWg; rb += rows_per_pass * kRowsPerThread) {
      int r[kRowsPerThread];
      bool live[kRowsPerThread];
      f32x4 acc[kRowsPerThread];
      const float* src[kRowsPerThread];
#pragma unroll
      for (int k = 0; k < kRowsPerThread; ++k) {
        r[k] = rb + k * rows_per_pass;
        live[k] = r[k] < kRowsPerWg && row0 + r[k] < n_rows;
        if (!live[k]) r[k] = 0;  // keeps LDS and pointer arithmetic in range
        const int64_t off = (row0 + r[k]) * head_dim + col;
        acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!kBf16 && live[k] && p0 > 0)
          acc[k] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(o_out) + off);
        src[k] = o_parts + int64_t(p0) * pstride + off;
      }
      // loads of partial q for every owned row, or zeros where not needed
      auto fetch = [&](int q, f32x4* v) {
#pragma unroll
        for (int k = 0; k < kRowsPerThread; ++k)
          v[k] = (live[k] && q < np && sh_w[q][r[k]] != 0.f) ? load_nt(src[k] + q * pstride)
                                                              : f32x4{0.f, 0.f, 0.f, 0.f};
      };
      f32x4 cur[kUnroll][kRowsPerThread];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) fetch(u, cur[u]);
      for (int pp = 0; pp < np; pp += kUnroll) {
        f32x4 nxt[kUnroll][kRowsPerThread];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) fetch(pp + kUnroll + u, nxt[u]);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
          for (int k = 0; k < kRowsPerThread; ++k) {
            const float w = pp + u < np ? sh_w[pp + u][r[k]] : 0.f;
            if (w == 0.f) continue;  // an empty partial's O may hold anything
            acc[k].x = fmaf(w, cur[u][k].x, acc[k].x);
            acc[k].y = fmaf(w, cur[u][k].y, acc[k].y);
            acc[k].z = fmaf(w, cur[u][k].z, acc[k].z);
            acc[k].w = fmaf(w, cur[u][k].w, acc[k].w);
          }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
          for (int k = 0; k < kRowsPerThread; ++k) cur[u][k] = nxt[u][k];
      }
#pragma unroll
      for (int k = 0; k < kRowsPerThread; ++k)
        if (live[k]) store_row<kBf16>(o_out, (row0 + r[k]) * head_dim + col, acc[k]);
    }
  }
}

}  // namespace

hipError_t launch_lse_merge(int32_t n_parts, int64_t n_rows, int32_t head_dim,
                            const float* o_parts, const float* lse_parts, bool out_bf16,
                            void* o_out, float* lse_out, hipStream_t stream) {
  if (out_bf16 && n_parts > kPartsPerPass) return hipErrorInvalidValue;
  const bool small = (n_rows + 31) / 32 <= kSmallMergeWgs;
  const int64_t blocks = small ? (n_rows + 15) / 16 : (n_rows + 31) / 32;
  const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
  if (small && out_bf16)
    hipLaunchKernelGGL((lse_merge_kernel<true, 2, 16, 4>), grid, block, 0, stream, n_parts,
                       n_rows, head_dim, o_parts, lse_parts, o_out, lse_out);
  else if (small)
    hipLaunchKernelGGL((lse_merge_kernel<false, 2, 16, 4>), grid, block, 0, stream, n_parts,
                       n_rows, head_dim, o_parts, lse_parts, o_out, lse_out);
  else if (out_bf16)
    hipLaunchKernelGGL((lse_merge_kernel<true, 4, 32, 2>), grid, block, 0, stream, n_parts,
                       n_rows, head_dim, o_parts, lse_parts, o_out, lse_out);
  else
    hipLaunchKernelGGL((lse_merge_kernel<false, 4, 32, 2>), grid, block, 0, stream, n_parts,
                       n_rows, head_dim, o_parts, lse_parts, o_out, lse_out);
  return hipGetLastError();
}

}  // namespace bsx
