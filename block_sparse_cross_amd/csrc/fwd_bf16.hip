// Forward partials for bf16 inputs on CDNA4 matrix cores (gfx950).
//
// Attention is softmax(Q K^T / sqrt(d)) V (Flash-dLLM page, "Method 1: I/O-Aware
// Fused KV-Cache Kernel"), taken per output slot over the visible keys of the
// slot's chunks (Split-KV page, Abstract: per-chunk / per-rank partials combined
// by an exact merge), emitted as a normalized partial plus natural-log LSE.
//
// Work item: one workgroup (4 waves) per (128-row tile of KV head g's query rows,
// g, slot).  Rows of head g are r = q * G + (h - g * G), so one K/V tile staged in
// LDS serves the G query heads of the GQA group and every query of the tile's
// draft blocks.  Each wave owns 32 rows.
//
// Orientation: the wave computes S^T = K Q^T and O^T += V^T P^T with
// v_mfma_f32_32x32x16_bf16, so a query row is a lane column of every accumulator:
// lanes c and c + 32 hold row c, the softmax row max/sum needs one exchange
// between the two half-waves, and the per-row rescale of O is a per-lane scalar.
//   S^T:  A = K tile (keys x d) from LDS, B = Q^T (d x rows) kept in registers.
//   O^T:  A = V^T tile (d x keys) from LDS, B = P^T (keys x rows) taken straight
//         from the S^T accumulator after the softmax (bf16).
// The accumulator holds keys {0-3, 8-11, 16-19, 24-27} + 4 * half of each 32-key
// block in a lane, so V^T is stored with bits 2 and 3 of the key index swapped
// inside each 16-key group; then each PV operand is one 16-byte LDS read.
//
// Memory path: K/V tiles of 64 keys are loaded with 16-byte coalesced global reads
// into registers one tile ahead, V is transposed in registers (v_perm_b32), and
// both are written to a double-buffered, XOR-swizzled LDS stage (conflict-free
// MFMA operand reads); one barrier per tile.  Only the first/last tile of a
// segment and tiles on a row-range boundary take the per-element mask; keys
// outside every row's range are never loaded (block-sparse skip).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "bsx_internal.h"
#include "fwd_common.h"

namespace bsx {
namespace {

constexpr int D = 128;
constexpr int ROWS = 128;
constexpr int KT = 64;
constexpr int THREADS = 256;
constexpr int K_BYTES = KT * D * 2;   // K tile: 64 keys x 256 B
constexpr int V_BYTES = KT * D * 2;   // V^T tile: 128 dims x 128 B
constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// LDS byte offset of the 16-byte chunk `ch` (0..15) of key row `key` in a K tile.
__device__ inline int k_off(int key, int ch) { return key * 256 + ((ch ^ (key & 7)) << 4); }
// LDS byte offset of the 16-byte chunk `ch` (0..7) of dim row `d` in a V^T tile.
__device__ inline int vt_off(int d, int ch) { return d * 128 + ((ch ^ ((d ^ (d >> 3)) & 7)) << 4); }
// Stored position of key w (0..15) inside its 16-key group: bits 2 and 3 swapped.
__device__ inline int vt_pos(int w) { return (w & 3) | ((w & 4) << 1) | ((w & 8) >> 1); }

struct Tile {
  int64_t p0;     // first position
  int64_t l0;     // local row of p0
  int nvalid;     // keys of the tile inside the segment
};

struct TileWalk {
  SegmentWalk seg;
  int64_t p0;
  __device__ bool first() {
    if (!seg.next()) return false;
    p0 = seg.seg0;
    return true;
  }
  __device__ bool advance() {
    p0 += KT;
    if (p0 < seg.seg1) return true;
    if (!seg.next()) return false;
    p0 = seg.seg0;
    return true;
  }
  __device__ Tile tile() const {
    Tile t;
    t.p0 = p0;
    t.l0 = seg.local0 + (p0 - seg.seg0);
    const int64_t n = seg.seg1 - p0;
    t.nvalid = int(n < KT ? n : KT);
    return t;
  }
};

__global__ __launch_bounds__(THREADS, 2) void fwd_bf16_kernel(FwdParams p, int n_tiles) {
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE_BYTES];
  __shared__ int64_t red[4][4];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;

  int bid = blockIdx.x;
  const int tile_id = n_tiles - 1 - (bid % n_tiles);
  bid /= n_tiles;
  const int g = bid % p.n_kv_heads;
  const int slot = bid / p.n_kv_heads;
  const bool is_self = p.has_self && slot == p.n_slots;
  const int G = p.n_q_heads / p.n_kv_heads;
  const int64_t n_q = int64_t(p.n_blocks) * p.block_size;
  const int64_t n_rows = n_q * G;

  // ---- this lane's query row and its visible range
  const int64_t r = int64_t(tile_id) * ROWS + wave * 32 + col;
  const bool row_ok = r < n_rows;
  const int64_t qi = row_ok ? r / G : 0;
  const int h = g * G + int(row_ok ? r % G : 0);
  int64_t lo = 0, hi = 0;
  if (row_ok) visible_range(p, is_self, qi / p.block_size, &lo, &hi);
  const bool live = row_ok && lo < hi;

  // ---- workgroup-wide union [mlo, mhi) and intersection [Lmax, Hmin) of live ranges
  {
    int64_t a = live ? lo : INT64_MAX, b = live ? hi : INT64_MIN;
    int64_t c = live ? lo : INT64_MIN, e = live ? hi : INT64_MAX;
    for (int off = 16; off >= 1; off >>= 1) {
      const int64_t a2 = __shfl_xor(a, off), b2 = __shfl_xor(b, off);
      const int64_t c2 = __shfl_xor(c, off), e2 = __shfl_xor(e, off);
      a = a2 < a ? a2 : a;
      b = b2 > b ? b2 : b;
      c = c2 > c ? c2 : c;
      e = e2 < e ? e2 : e;
    }
    if (lane == 0) {
      red[wave][0] = a;
      red[wave][1] = b;
      red[wave][2] = c;
      red[wave][3] = e;
    }
  }
  __syncthreads();
  int64_t mlo = INT64_MAX, mhi = INT64_MIN, lmax = INT64_MIN, hmin = INT64_MAX;
  for (int w = 0; w < 4; ++w) {
    mlo = red[w][0] < mlo ? red[w][0] : mlo;
    mhi = red[w][1] > mhi ? red[w][1] : mhi;
    lmax = red[w][2] > lmax ? red[w][2] : lmax;
    hmin = red[w][3] < hmin ? red[w][3] : hmin;
  }

  const int64_t orow = (int64_t(slot) * n_q + qi) * p.n_q_heads + h;

  TileWalk walk;
  walk.seg.init(p, slot, is_self, mlo, mhi);
  bool have = mlo < mhi && walk.first();
  if (!have) {
    if (row_ok && half == 0) p.lse_part[orow] = -INFINITY;
    return;
  }

  // ---- Q^T fragments: lane (half, col) holds dims 16t + 8*half .. +8 of its row
  bf16x8 qf[8];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + (qi * p.n_q_heads + h) * D;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row_ok) x = *reinterpret_cast<const u32x4*>(qrow + 16 * t + 8 * half);
      qf[t] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const uint16_t* kbase = static_cast<const uint16_t*>(is_self ? p.k_self : p.k);
  const uint16_t* vbase = static_cast<const uint16_t*>(is_self ? p.v_self : p.v);
  const int64_t kstride = int64_t(p.n_kv_heads) * D;
  const int64_t gofs = int64_t(g) * D;

  // staging registers: K rows (tid>>4) + 16i, chunk tid&15; V keys 4*(tid>>4)+i, dims 8*(tid&15)
  u32x4 kr[4], vr[4];
  const int ld_row = tid >> 4, ld_ch = tid & 15;

  auto load_tile = [&](const Tile& t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = ld_row + 16 * i;
      kr[i] = u32x4{0u, 0u, 0u, 0u};
      if (key < t.nvalid)
        kr[i] = *reinterpret_cast<const u32x4*>(kbase + (t.l0 + key) * kstride + gofs + 8 * ld_ch);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = 4 * ld_row + i;
      vr[i] = u32x4{0u, 0u, 0u, 0u};
      if (key < t.nvalid)
        vr[i] = *reinterpret_cast<const u32x4*>(vbase + (t.l0 + key) * kstride + gofs + 8 * ld_ch);
    }
  };

  auto store_tile = [&](int stage) {
    char* kb = smem + stage * STAGE_BYTES;
    char* vb = kb + K_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = ld_row + 16 * i;
      *reinterpret_cast<u32x4*>(kb + k_off(key, ld_ch)) = kr[i];
    }
    // V: keys 4*ld_row .. +3 of dims 8*ld_ch .. +7 -> V^T rows d, stored positions sp .. sp+3
    const int k4 = 4 * ld_row;
    const int sp = (k4 & ~15) | vt_pos(k4 & 15);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t w0 = __builtin_amdgcn_perm(vr[1][e >> 1], vr[0][e >> 1], sel);
      const uint32_t w1 = __builtin_amdgcn_perm(vr[3][e >> 1], vr[2][e >> 1], sel);
      const int d = 8 * ld_ch + e;
      *reinterpret_cast<u32x2*>(vb + vt_off(d, sp >> 3) + ((sp & 7) << 1)) = u32x2{w0, w1};
    }
  };

  f32x16 acc_o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc_o[db][v] = 0.f;
  float m = -INFINITY, lsum = 0.f;
  const float c2 = p.scale_log2;

  Tile cur = walk.tile();
  load_tile(cur);
  store_tile(0);
  __syncthreads();
  int stage = 0;

  while (have) {
    const bool have_next = walk.advance();
    Tile nxt = cur;
    if (have_next) {
      nxt = walk.tile();
      load_tile(nxt);
    }

    // ---- S^T = K Q^T for the two 32-key blocks of the tile
    const char* kb = smem + stage * STAGE_BYTES;
    const char* vb = kb + K_BYTES;
    f32x16 s[2];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[b2][v] = 0.f;
      const int key = b2 * 32 + col;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kb + k_off(key, 2 * t + half));
        s[b2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[t],
                                                         s[b2], 0, 0, 0);
      }
    }

    // ---- mask (boundary tiles only), online softmax in base 2
    const bool full = cur.nvalid == KT && cur.p0 >= lmax && cur.p0 + KT <= hmin;
    if (!full) {
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = b2 * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          const int64_t pos = cur.p0 + key;
          const bool vis = key < cur.nvalid && pos >= lo && pos < hi;
          s[b2][v] = vis ? s[b2][v] : -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int v = 0; v < 16; ++v) mt = fmaxf(mt, s[b2][v]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m, mt * c2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    float psum = 0.f;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[b2][v], c2, -m_use));
        s[b2][v] = e;
        psum += e;
      }
    lsum = lsum * alpha + psum;
    m = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc_o[db][v] *= alpha;
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = static_cast<__bf16>(s[u >> 1][8 * (u & 1) + e]);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = db * 32 + col;
        const u32x4 a = *reinterpret_cast<const u32x4*>(vb + vt_off(d, 2 * u + half));
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pf,
                                                             acc_o[db], 0, 0, 0);
      }
    }

    if (have_next) store_tile(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    cur = nxt;
    have = have_next;
  }

  // ---- normalize and write this lane's half of the row
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (!row_ok) return;
  const bool has_keys = live && ltot > 0.f;
  if (half == 0) p.lse_part[orow] = has_keys ? (m + __log2f(ltot)) * kLn2 : -INFINITY;
  if (!has_keys) return;
  const float inv = 1.f / ltot;
  float* op = p.o_part + orow * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = db * 32 + 8 * a + 4 * half;
      *reinterpret_cast<float4*>(op + d0) =
          make_float4(acc_o[db][4 * a] * inv, acc_o[db][4 * a + 1] * inv,
                      acc_o[db][4 * a + 2] * inv, acc_o[db][4 * a + 3] * inv);
    }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  const int G = p.n_q_heads / p.n_kv_heads;
  const int64_t n_rows = int64_t(p.n_blocks) * p.block_size * G;
  const int64_t n_tiles = (n_rows + ROWS - 1) / ROWS;
  const int64_t n_out = int64_t(p.n_slots) + p.has_self;
  const int64_t grid = n_tiles * p.n_kv_heads * n_out;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fwd_bf16_kernel, dim3(unsigned(grid)), dim3(THREADS), 0, stream, p,
                     int(n_tiles));
  return hipGetLastError();
}

}  // namespace bsx
