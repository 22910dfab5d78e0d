// Forward partials for f32 inputs, in f32 arithmetic throughout (no reduced
// precision anywhere): the reference-precision variant of the attention kernel.
//
// Attention is softmax(Q K^T / sqrt(d)) V (Flash-dLLM page, "Method 1: I/O-Aware
// Fused KV-Cache Kernel"), taken per output slot over the keys of the slot's chunks
// that the row may see, with an online (running max / running sum) softmax, and
// emitted as a normalized partial with its natural-log LSE.
//
// Both products run on the f32 matrix cores (v_mfma_f32_16x16x4f32: f32 products,
// f32 accumulation; CDNA4 has no reduced-precision f32 mode).  Work item: one
// workgroup per (16-row tile of one KV head's query rows, KV head, slot).  Query rows
// of KV head g are r = q * G + (h - g * G) for the G query heads h of the group, so
// the rows of a tile share every K/V tile they read.  Four waves split the keys: wave w
// takes keys [16 w, 16 w + 16) of every 64-key tile (one MFMA block) and keeps its own
// online softmax state for the 16 rows; the four quarters of a row are combined once,
// through LDS, at the end (the exact LSE-weighted combination of partial softmaxes).
// Small tiles keep many CUs busy: one workgroup's two products are bound by its CU's
// matrix rate, so the rows are spread over as many workgroups as there are 16-row tiles.
//
// Scores are formed transposed, S^T = K Q^T, so that lane l's scores and its output
// accumulators all belong to one query row (row l % 16 of the wave): the four 16-lane
// groups hold different keys of that row, and the online softmax exchanges only the
// row maximum (and, once at the end, the row sum) between them.
//
// MFMA 16x16x4 f32 operand layout (lane l, c = l % 16, k = l / 16): A[c][k],
// B[k][c]; D[4k + i][c] in register i.
//   S^T = K Q^T:  A[c][k] = K[key c][d], B[k][c] = Q[row c][d], d = 32k + s for the
//                 s-th of 32 products, so a lane reads 32 contiguous dims of a key.
//                 Register i of the result is the score of key 4k + i for row c.
//   O^T = V^T P^T: one product per i: A[c][k] = V[key 4k + i][dim(c, n)],
//                 B[k][c] = P[row c][key 4k + i], with dim(c, n) = 4c + 64(n / 4) +
//                 n % 4 for the n-th of 8 output blocks (two 16-byte V reads per lane).
//                 Register i' of block n is O[row c][dim(4k + i', n)].
// K/V tiles of 64 keys are staged in LDS (row pitch 132 floats: conflict-free
// 16-byte reads for both operand patterns), the next tile prefetched into registers
// while the current one is multiplied.
#include <hip/hip_runtime.h>

#include <math.h>

#include "bsx_internal.h"
#include "fwd_common.h"

namespace bsx {
namespace {

constexpr int D = 128;
constexpr int ROWS = 16;  // rows per workgroup
constexpr int KT = 64;    // keys per staged tile: one 16-key MFMA block per wave
constexpr int THREADS = 256;
constexpr int KP = D + 4;  // LDS row pitch in floats (16-byte aligned)
constexpr int LOADS = KT * D / 4 / THREADS;  // float4 loads of K (and of V) per thread
constexpr float kLn2 = 0.6931471805599453f;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(THREADS) void fwd_f32_kernel(FwdParams, int n_tiles) {
  const BSX_KARG FwdParams& p = kernel_arg0<FwdParams>();
  // staged K then V tile; at the end, the accumulators of waves 1..3
  constexpr int NW = THREADS / 64;
  __shared__ __align__(16) float smem[2 * KT * KP];
  __shared__ float xm[NW * 64], xl[NW * 64];
  static_assert(2 * KT * KP >= 32 * NW * 64, "the waves' accumulators fit the staging buffer");
  float* const sk = smem;
  float* const sv = smem + KT * KP;

  const int tid = threadIdx.x;
  int bid = blockIdx.x;
  const int tile = bid % n_tiles;
  bid /= n_tiles;
  const int g = bid % p.n_kv_heads;
  const int slot = bid / p.n_kv_heads;
  const bool is_self = p.has_self && slot == p.n_slots;
  const int G = p.n_q_heads / p.n_kv_heads;
  const int64_t n_q = int64_t(p.n_blocks) * p.block_size;
  const int64_t n_rows = n_q * G;

  const int wave = tid >> 6, lane = tid & 63;
  const int c = lane & 15, kq = lane >> 4;
  const int64_t r = int64_t(tile) * ROWS + c;
  const bool row_ok = r < n_rows;
  const int64_t qi = row_ok ? r / G : 0;
  const int h = g * G + int(row_ok ? r % G : 0);
  int64_t lo = 0, hi = 0;
  if (row_ok)
    visible_range(p.anchor, p.ctx_begin, p.ctx_len, p.block_size, is_self, qi / p.block_size,
                  &lo, &hi);
  const bool live = row_ok && lo < hi;

  // union of the live rows' ranges (every wave holds all 16 rows)
  int64_t mlo = live ? lo : INT64_MAX, mhi = live ? hi : INT64_MIN;
  for (int off = 8; off >= 1; off >>= 1) {
    const int64_t a = __shfl_xor(mlo, off), b = __shfl_xor(mhi, off);
    mlo = a < mlo ? a : mlo;
    mhi = b > mhi ? b : mhi;
  }

  // this lane's 32 query dims [32 kq, 32 kq + 32) of row c
  float qv[32];
  {
    const float* qrow = static_cast<const float*>(p.q) + (qi * p.n_q_heads + h) * D + 32 * kq;
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      const float4 t = row_ok ? *reinterpret_cast<const float4*>(qrow + i)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
      qv[i] = t.x;
      qv[i + 1] = t.y;
      qv[i + 2] = t.z;
      qv[i + 3] = t.w;
    }
  }
  f32x4 acc[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  const float* kb = static_cast<const float*>(is_self ? p.k_self : p.k);
  const float* vb = static_cast<const float*>(is_self ? p.v_self : p.v);
  const int64_t kstride = int64_t(p.n_kv_heads) * D;

  SegmentWalk walk;
  walk.init(p.table.dev ? p.table.dev : (const char*)(p.table.words), p.entries_off, slot,
            is_self, mlo, mhi, p.entries_order);
  bool have = mlo < mhi && walk.next();
  int64_t p0 = have ? walk.seg0 : 0;

  // prefetch registers: thread t stages float4 t + 256 j of the tile (key = idx / 32)
  float4 kpre[LOADS], vpre[LOADS];
  int nvalid = 0;
  int64_t l0 = 0;
  auto fetch = [&]() {
    nvalid = int(walk.seg1 - p0 < KT ? walk.seg1 - p0 : KT);
    l0 = walk.local0 + (p0 - walk.seg0);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int idx = tid + THREADS * j;
      const int key = idx >> 5, c4 = idx & 31;
      kpre[j] = vpre[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (key < nvalid) {
        const int64_t off = (l0 + key) * kstride + int64_t(g) * D + 4 * c4;
        kpre[j] = *reinterpret_cast<const float4*>(kb + off);
        vpre[j] = *reinterpret_cast<const float4*>(vb + off);
      }
    }
  };
  if (have) fetch();

  while (have) {
    const int64_t cur_p0 = p0;
    const int cur_nvalid = nvalid;
    __syncthreads();  // the previous tile is no longer read
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int idx = tid + THREADS * j;
      const int key = idx >> 5, c4 = idx & 31;
      *reinterpret_cast<float4*>(sk + key * KP + 4 * c4) = kpre[j];
      *reinterpret_cast<float4*>(sv + key * KP + 4 * c4) = vpre[j];
    }
    __syncthreads();

    // next tile: advance the walk and prefetch while this one is multiplied
    p0 += KT;
    if (p0 >= walk.seg1) {
      have = walk.next();
      if (have) p0 = walk.seg0;
    }
    if (have) fetch();

    // scores: st[i] is key 16 wave + 4 kq + i of the tile, for row c
    f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      const float* kr = sk + (16 * wave + c) * KP + 32 * kq;
#pragma unroll
      for (int i = 0; i < 32; i += 4) {
        const float4 kk = *reinterpret_cast<const float4*>(kr + i);
        st = mfma4(kk.x, qv[i], st);
        st = mfma4(kk.y, qv[i + 1], st);
        st = mfma4(kk.z, qv[i + 2], st);
        st = mfma4(kk.w, qv[i + 3], st);
      }
    }
    float s[4];
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = 16 * wave + 4 * kq + i;
      const int64_t pos = cur_p0 + key;
      const bool vis = key < cur_nvalid && pos >= lo && pos < hi;
      s[i] = vis ? st[i] * p.scale_log2 : -INFINITY;
      mt = fmaxf(mt, s[i]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = exp2f(s[i] - m_use);
      psum += s[i];
    }
    lsum = lsum * alpha + psum;
    m = m_new;
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] *= alpha;

#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* vr = sv + (16 * wave + 4 * kq + i) * KP + 4 * c;
      const float4 va = *reinterpret_cast<const float4*>(vr);
      const float4 vc = *reinterpret_cast<const float4*>(vr + 64);
      acc[0] = mfma4(va.x, s[i], acc[0]);
      acc[1] = mfma4(va.y, s[i], acc[1]);
      acc[2] = mfma4(va.z, s[i], acc[2]);
      acc[3] = mfma4(va.w, s[i], acc[3]);
      acc[4] = mfma4(vc.x, s[i], acc[4]);
      acc[5] = mfma4(vc.y, s[i], acc[5]);
      acc[6] = mfma4(vc.z, s[i], acc[6]);
      acc[7] = mfma4(vc.w, s[i], acc[7]);
    }
  }

  // combine the key quarters of each row: waves 1..3 hand (m, l, acc) to wave 0
  __syncthreads();  // the last tile is no longer read
  if (wave > 0) {
    const int xi = wave * 64 + lane;
    xm[xi] = m;
    xl[xi] = lsum;
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) smem[(4 * n + i) * (NW * 64) + xi] = acc[n][i];
  }
  __syncthreads();
  if (wave > 0) return;
  {
    float mm = m;
#pragma unroll
    for (int w = 1; w < NW; ++w) mm = fmaxf(mm, xm[w * 64 + lane]);
    const float mu = mm == -INFINITY ? 0.f : mm;
    const float a0 = exp2f(m - mu);
    lsum *= a0;
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] *= a0;
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const int xi = w * 64 + lane;
      const float aw = exp2f(xm[xi] - mu);
      lsum += xl[xi] * aw;
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[n][i] += smem[(4 * n + i) * (NW * 64) + xi] * aw;
    }
    m = mm;
  }

  float ltot = lsum + __shfl_xor(lsum, 16);
  ltot += __shfl_xor(ltot, 32);
  if (!row_ok) return;
  const int64_t orow = (int64_t(slot) * n_q + qi) * p.n_q_heads + h;
  if (kq == 0) p.lse_part[orow] = ltot > 0.f ? (m + log2f(ltot)) * kLn2 : -INFINITY;
  if (ltot > 0.f) {
    const float inv = 1.f / ltot;
    float* op = p.o_part + orow * D;
    // register i' of block n is dim 4 (4 kq + i') + 64 (n / 4) + n % 4
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int half = 0; half < 2; ++half)
        *reinterpret_cast<float4*>(op + 16 * kq + 4 * i + 64 * half) =
            make_float4(acc[4 * half][i] * inv, acc[4 * half + 1][i] * inv,
                        acc[4 * half + 2][i] * inv, acc[4 * half + 3][i] * inv);
  }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream) {
  const int G = p.n_q_heads / p.n_kv_heads;
  const int64_t n_rows = int64_t(p.n_blocks) * p.block_size * G;
  const int64_t n_tiles = (n_rows + ROWS - 1) / ROWS;
  const int64_t n_out = int64_t(p.n_slots) + p.has_self;
  const int64_t grid = n_tiles * p.n_kv_heads * n_out;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fwd_f32_kernel, dim3(unsigned(grid)), dim3(THREADS), 0, stream, p,
                     int(n_tiles));
  return hipGetLastError();
}

}  // namespace bsx
