// Forward partials for f32 inputs, in f32 arithmetic throughout (no reduced
// precision anywhere): the reference-precision variant of the attention kernel.
//
// Attention is softmax(Q K^T / sqrt(d)) V (Flash-dLLM page, "Method 1: I/O-Aware
// Fused KV-Cache Kernel"), taken per output slot over the keys of the slot's chunks
// that the row may see, with an online (running max / running sum) softmax, and
// emitted as a normalized partial with its natural-log LSE.
//
// Work item: one workgroup per (64-row tile of one KV head's query rows, KV head,
// slot).  Query rows of KV head g are r = q * G + (h - g * G) for the G query heads
// h of the group, so the rows of a tile share every K/V tile they read.  Four
// lanes own one row: lane u holds query dims and output dims [32u, 32u + 32), the
// dot products are reduced across the four lanes, and each lane keeps the whole
// row's scores, so the softmax needs no further exchange.  K/V tiles of 32 keys
// are staged in LDS with a padded layout (no bank conflicts for the 4-way split).
#include <hip/hip_runtime.h>

#include <math.h>

#include "bsx_internal.h"
#include "fwd_common.h"

namespace bsx {
namespace {

constexpr int D = 128;
constexpr int ROWS = 64;
constexpr int KT = 32;
constexpr int THREADS = 256;
constexpr int QUARTER = D / 4;        // dims per lane
constexpr int PAD_Q = QUARTER + 1;    // padded quarter row in LDS
constexpr int ROW_PITCH = 4 * PAD_Q;  // 132 floats per staged key
constexpr float kLn2 = 0.6931471805599453f;

__global__ __launch_bounds__(THREADS) void fwd_f32_kernel(FwdParams, int n_tiles) {
  const BSX_KARG FwdParams& p = kernel_arg0<FwdParams>();
  __shared__ float sk[KT * ROW_PITCH];
  __shared__ float sv[KT * ROW_PITCH];
  __shared__ int64_t red_lo[THREADS / 64], red_hi[THREADS / 64];

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

  const int j = tid >> 2, u = tid & 3;
  const int64_t r = int64_t(tile) * ROWS + j;
  const bool row_ok = r < n_rows;
  const int64_t qi = row_ok ? r / G : 0;
  const int h = g * G + int(row_ok ? r % G : 0);
  int64_t lo = 0, hi = 0;
  if (row_ok)
    visible_range(p.anchor, p.ctx_begin, p.ctx_len, p.block_size, is_self, qi / p.block_size,
                  &lo, &hi);
  const bool live = row_ok && lo < hi;

  // union of the live rows' ranges
  int64_t mlo = live ? lo : INT64_MAX, mhi = live ? hi : INT64_MIN;
  for (int off = 32; off >= 1; off >>= 1) {
    const int64_t a = __shfl_xor(mlo, off), b = __shfl_xor(mhi, off);
    mlo = a < mlo ? a : mlo;
    mhi = b > mhi ? b : mhi;
  }
  if ((tid & 63) == 0) {
    red_lo[tid >> 6] = mlo;
    red_hi[tid >> 6] = mhi;
  }
  __syncthreads();
  for (int w = 0; w < THREADS / 64; ++w) {
    mlo = red_lo[w] < mlo ? red_lo[w] : mlo;
    mhi = red_hi[w] > mhi ? red_hi[w] : mhi;
  }

  const float* qrow = static_cast<const float*>(p.q) + (qi * p.n_q_heads + h) * D + QUARTER * u;
  float qv[QUARTER];
#pragma unroll
  for (int i = 0; i < QUARTER; ++i) qv[i] = row_ok ? qrow[i] : 0.f;
  float acc[QUARTER];
#pragma unroll
  for (int i = 0; i < QUARTER; ++i) acc[i] = 0.f;
  float m = -INFINITY, l = 0.f;

  const float* kb = static_cast<const float*>(is_self ? p.k_self : p.k);
  const float* vb = static_cast<const float*>(is_self ? p.v_self : p.v);
  const int64_t kstride = int64_t(p.n_kv_heads) * D;

  SegmentWalk walk;
  walk.init(p.table.dev ? p.table.dev : (const char*)(p.table.words),
            p.entries_off, slot, is_self, mlo, mhi, p.entries_order);
  while (mlo < mhi && walk.next()) {
    for (int64_t p0 = walk.seg0; p0 < walk.seg1; p0 += KT) {
      const int nvalid = int(walk.seg1 - p0 < KT ? walk.seg1 - p0 : KT);
      const int64_t l0 = walk.local0 + (p0 - walk.seg0);
      __syncthreads();  // the previous tile is no longer read
      for (int idx = tid; idx < KT * (D / 4); idx += THREADS) {
        const int key = idx / (D / 4), c4 = idx % (D / 4);
        float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
        if (key < nvalid) {
          const int64_t off = (l0 + key) * kstride + int64_t(g) * D + 4 * c4;
          kk = *reinterpret_cast<const float4*>(kb + off);
          vv = *reinterpret_cast<const float4*>(vb + off);
        }
        const int dst = key * ROW_PITCH + (c4 / 8) * PAD_Q + (c4 % 8) * 4;
        sk[dst] = kk.x; sk[dst + 1] = kk.y; sk[dst + 2] = kk.z; sk[dst + 3] = kk.w;
        sv[dst] = vv.x; sv[dst + 1] = vv.y; sv[dst + 2] = vv.z; sv[dst + 3] = vv.w;
      }
      __syncthreads();

      float s[KT];
#pragma unroll
      for (int key = 0; key < KT; ++key) {
        const float* kr = sk + key * ROW_PITCH + u * PAD_Q;
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < QUARTER; ++i) part = fmaf(qv[i], kr[i], part);
        part += __shfl_xor(part, 1);
        part += __shfl_xor(part, 2);
        const int64_t pos = p0 + key;
        const bool vis = key < nvalid && pos >= lo && pos < hi;
        s[key] = vis ? part * p.scale_log2 : -INFINITY;
      }
      float mt = -INFINITY;
#pragma unroll
      for (int key = 0; key < KT; ++key) mt = fmaxf(mt, s[key]);
      const float m_new = fmaxf(m, mt);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m - m_use);
      float psum = 0.f;
#pragma unroll
      for (int key = 0; key < KT; ++key) {
        s[key] = exp2f(s[key] - m_use);
        psum += s[key];
      }
      l = l * alpha + psum;
      m = m_new;
#pragma unroll
      for (int i = 0; i < QUARTER; ++i) acc[i] *= alpha;
#pragma unroll
      for (int key = 0; key < KT; ++key) {
        const float* vr = sv + key * ROW_PITCH + u * PAD_Q;
#pragma unroll
        for (int i = 0; i < QUARTER; ++i) acc[i] = fmaf(s[key], vr[i], acc[i]);
      }
    }
  }

  if (!row_ok) return;
  const int64_t orow = (int64_t(slot) * n_q + qi) * p.n_q_heads + h;
  if (u == 0) p.lse_part[orow] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  if (l > 0.f) {
    const float inv = 1.f / l;
    float* op = p.o_part + orow * D + QUARTER * u;
#pragma unroll
    for (int i = 0; i < QUARTER; i += 4)
      *reinterpret_cast<float4*>(op + i) =
          make_float4(acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv);
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
