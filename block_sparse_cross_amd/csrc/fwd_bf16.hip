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
//   O^T:  A = V^T (d x keys), read from the row-major V tile with the gfx950
//         transpose load ds_read_b64_tr_b16, B = P^T (keys x rows) taken straight
//         from the S^T accumulator after the softmax (bf16).
// The S^T accumulator holds keys {0-3, 8-11, 16-19, 24-27} + 4 * half of each
// 32-key block in a lane; the V^T operand is read in that same key order, so P^T
// never moves between lanes.
//
// Memory path: K/V rows of a 64-key tile are read with 16-byte buffer loads from a
// per-tile scalar base (keys past the segment end fall outside the buffer range
// and read as zero), one tile ahead of the compute, and written to a
// double-buffered LDS stage with padded rows: the K operand reads (b128, 16 rows
// at one chunk) are free of bank conflicts on the 64-bank LDS, the V transpose reads
// (4 rows x 4 chunks) two-way conflicted (about a tenth of LDS cycles; a layout
// without the conflict measured no faster); one barrier per tile.  Only tiles that cross a segment end or some row's range take
// the per-element mask; keys outside every row's range are never loaded.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "bsx_internal.h"
#include "fwd_common.h"
#include "mfma_common.h"

namespace bsx {
namespace {

constexpr int D = 128;
constexpr int ROWS = kFwdRows;
constexpr int KT = kFwdKeyTile;
constexpr int THREADS = 256;
constexpr int K_PITCH = 272;                 // bytes per staged K row (256 + 16 pad)
constexpr int V_PITCH = 288;                 // bytes per staged V row (256 + 32 pad)
constexpr int K_BYTES = KT * K_PITCH;
constexpr int V_BYTES = KT * V_PITCH;
constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;

// The two values of a query row held by lanes l and l ^ 32, as (a, b) in either order:
// v_permlane32_swap exchanges the upper half-wave of its first operand with the lower
// half-wave of its second, so with two copies of x every lane ends up holding x of
// both half-waves.  A VALU exchange, unlike a shuffle through LDS (ds_bpermute), which
// would queue behind the tile's operand reads.
__device__ inline void half_pair(float x, float* a, float* b) {
  float u = x, w = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(u), "+v"(w));
  *a = u;
  *b = w;
}

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

__global__ __launch_bounds__(THREADS, 2) void fwd_bf16_kernel(FwdParams, int n_tiles, int n_pairs) {
  const BSX_KARG FwdParams& p = kernel_arg0<FwdParams>();
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE_BYTES];
  __shared__ int64_t red[4][4];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;

  // Workgroup i runs on XCD i % 8.  With at least 8 (KV head, slot) pairs, all row
  // tiles of a pair go to the same XCD (pairs are dealt to the XCDs in rounds of 8,
  // alternating direction) so they share that XCD's L2 copy of the slot's K/V.  With a launch order, items run heaviest first (per XCD
  // when pairs keep their XCD); without one, pairs run one after another.
  int pair, tile_id, pj = 0;
  bool empty_item = false;
  if (p.order) {
    int code = p.order[blockIdx.x];
    if (code == -1) return;
    empty_item = code < -1;  // marked by the order pass: the item visits no key tile
    if (empty_item) code = -2 - code;
    pair = code / n_tiles;
    tile_id = code - pair * n_tiles;
    if (p.piece) pj = p.piece[blockIdx.x];
  } else if (n_pairs >= kXcds) {
    const int xcd = blockIdx.x % kXcds;
    const int j = blockIdx.x / kXcds;
    pair = pair_of_xcd_round(j / n_tiles, xcd);
    tile_id = n_tiles - 1 - (j % n_tiles);
    if (pair >= n_pairs) return;
  } else {
    // fewer pairs than XCDs: items go round-robin over all XCDs (a pair's K/V is then
    // cached by several L2s, which beats leaving XCDs idle)
    pair = blockIdx.x / n_tiles;
    tile_id = n_tiles - 1 - blockIdx.x % n_tiles;
  }
  const int g = pair % p.n_kv_heads;
  const int slot = pair / p.n_kv_heads;
  const bool is_self = p.has_self && slot == p.n_slots;
  const int G = p.n_q_heads / p.n_kv_heads;
  const int64_t n_q = int64_t(p.n_blocks) * p.block_size;
  const int64_t n_rows = n_q * G;

  // ---- this lane's query row and its visible range
  const int64_t r = int64_t(tile_id) * ROWS + wave * 32 + col;
  const bool row_ok = r < n_rows;
  const int64_t qi = row_ok ? r / G : 0;
  const int h = g * G + int(row_ok ? r % G : 0);
  if (empty_item) {  // (a split launch marks no item)
    if (row_ok && half == 0) p.lse_part[(int64_t(slot) * n_q + qi) * p.n_q_heads + h] = -INFINITY;
    return;
  }
  // the lane's block range: the raw ctx_begin / anchor loads go out first, the Q loads
  // next, and the range is formed after both are in flight (the scheduling barrier
  // keeps the wait for the range from moving ahead of the Q loads)
  const int64_t blk = qi / p.block_size;
  int64_t raw_a = 0, raw_z = 0;
  if (row_ok && !is_self) {
    raw_a = p.ctx_begin[blk];
    raw_z = p.anchor[blk];
  }

  // ---- Q^T fragments: lane (half, col) holds dims 16t + 8*half .. +8 of its row
  bf16x8 qf[8];
  {
    // uniform base at the tile's first query; rows past the end read as zero
    const int64_t q0 = int64_t(tile_id) * ROWS / G;
    const int64_t q_bytes = (n_q - q0) * p.n_q_heads * D * 2;
    const __amdgpu_buffer_rsrc_t qr =
        make_rsrc(static_cast<const uint16_t*>(p.q) + q0 * p.n_q_heads * D,
                  uint32_t(q_bytes < 0xffffffffll ? q_bytes : 0xffffffffll));
    const uint32_t qoff =
        row_ok ? uint32_t(((qi - q0) * p.n_q_heads + h) * D * 2) + 16 * half : 0x80000000u;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      qf[t] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, qoff + 32 * t,
                                                                               0, 0));
  }
  __builtin_amdgcn_sched_barrier(0);
  // visible range [lo, hi) of the lane's row (the same clamping as visible_range)
  int64_t lo = 0, hi = 0;
  if (row_ok) {
    if (is_self) {
      lo = blk * p.block_size;
      hi = lo + p.block_size;
    } else {
      lo = raw_a < 0 ? 0 : (raw_a > p.ctx_len ? p.ctx_len : raw_a);
      hi = raw_z < lo ? lo : (raw_z > p.ctx_len ? p.ctx_len : raw_z);
    }
  }
  const bool live = row_ok && lo < hi;

  // ---- workgroup-wide union [mlo, mhi) and intersection [lmax, hmin) of live ranges
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
  // (an LDS-only barrier: the Q loads stay in flight while the walk starts and the first
  // K / V tile loads; the first MFMA waits for them)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  int64_t mlo = INT64_MAX, mhi = INT64_MIN, lmax = INT64_MIN, hmin = INT64_MAX;
  for (int w = 0; w < 4; ++w) {
    mlo = red[w][0] < mlo ? red[w][0] : mlo;
    mhi = red[w][1] > mhi ? red[w][1] : mhi;
    lmax = red[w][2] > lmax ? red[w][2] : lmax;
    hmin = red[w][3] < hmin ? red[w][3] : hmin;
  }
  mlo = uniform64(mlo);
  mhi = uniform64(mhi);
  lmax = uniform64(lmax);
  hmin = uniform64(hmin);

  const int64_t orow = (int64_t(slot) * n_q + qi) * p.n_q_heads + h;

  // A split item's piece pj covers tiles [pj P, pj P + P) of the walk and writes a
  // normalized partial of its own (slot sb + pj of part_o / part_lse).
  const ConstI32s split_tab = reinterpret_cast<ConstI32s>(const_bytes(p.split));  // scalar loads
  const int sb = p.split ? split_tab[4 + pair * n_tiles + tile_id] : -1;
  const int P = p.split ? split_tab[0] : 0;
  const int64_t prow = (int64_t(sb + pj) * ROWS + wave * 32 + col);  // split: partial row
  TileWalk walk;
  walk.seg.init(p.table.dev ? p.table.dev : (const char*)(p.table.words),
                p.entries_off, slot, is_self, mlo, mhi, p.entries_order);
  bool have = mlo < mhi && walk.first();
  int left = INT32_MAX;  // tiles this workgroup may still take
  if (have && sb >= 0) {
    int64_t skip = int64_t(pj) * P;
    while (skip > 0) {
      const int64_t in_seg = (walk.seg.seg1 - walk.p0 + KT - 1) / KT;
      if (skip < in_seg) {
        walk.p0 += skip * KT;
        break;
      }
      skip -= in_seg;
      if (!walk.seg.next()) {
        have = false;
        break;
      }
      walk.p0 = walk.seg.seg0;
    }
    left = P;
  }
  if (!have) {
    if (row_ok && half == 0) {
      if (sb >= 0)
        p.part_lse[prow] = -INFINITY;
      else
        p.lse_part[orow] = -INFINITY;
    }
    return;
  }

  const uint16_t* kbase = static_cast<const uint16_t*>(is_self ? p.k_self : p.k);
  const uint16_t* vbase = static_cast<const uint16_t*>(is_self ? p.v_self : p.v);
  const int64_t kstride = int64_t(p.n_kv_heads) * D;      // elements between key rows
  const uint32_t row_bytes = uint32_t(kstride * 2);
  const int64_t gofs = int64_t(g) * D;

  // staging: thread loads key rows ld_row + 16 i, 16-byte chunk ld_ch, of K and V
  const int ld_row = tid >> 4, ld_ch = tid & 15;
  const uint32_t ld_off = uint32_t(ld_row) * row_bytes + uint32_t(ld_ch) * 16;
  u32x4 kr[4], vr[4];

  auto load_tile = [&](const Tile& t) {
    // the buffer ends after the tile's last valid key: rows beyond it read as zero
    const uint32_t bytes = uint32_t(t.nvalid - 1) * row_bytes + D * 2;
    const __amdgpu_buffer_rsrc_t kb = make_rsrc(kbase + t.l0 * kstride + gofs, bytes);
    const __amdgpu_buffer_rsrc_t vb = make_rsrc(vbase + t.l0 * kstride + gofs, bytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kr[i] = __builtin_amdgcn_raw_buffer_load_b128(kb, ld_off + uint32_t(16 * i) * row_bytes, 0, 0);
      vr[i] = __builtin_amdgcn_raw_buffer_load_b128(vb, ld_off + uint32_t(16 * i) * row_bytes, 0, 0);
    }
  };

  auto store_tile = [&](int stage) {
    char* kb = smem + stage * STAGE_BYTES;
    char* vb = kb + K_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(kb + (ld_row + 16 * i) * K_PITCH + ld_ch * 16) = kr[i];
      *reinterpret_cast<u32x4*>(vb + (ld_row + 16 * i) * V_PITCH + ld_ch * 16) = vr[i];
    }
  };

  // per-lane LDS read offsets (everything else is an immediate)
  const int k_rd = col * K_PITCH + half * 16;
  const int tj = lane & 15, tg = lane >> 4;
  const int v_rd = (4 * half + (tj >> 2)) * V_PITCH + (16 * (tg & 1) + 4 * (tj & 3)) * 2;

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
    const bool have_next = --left > 0 && walk.advance();
    Tile nxt = cur;
    if (have_next) {
      nxt = walk.tile();
      load_tile(nxt);
    }

    const char* kb = smem + stage * STAGE_BYTES;
    const char* vb = kb + K_BYTES;

    // ---- S^T = K Q^T for the two 32-key blocks of the tile
    f32x16 s[2];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[b2][v] = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kb + k_rd + b2 * 32 * K_PITCH + 32 * t);
        s[b2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[t],
                                                         s[b2], 0, 0, 0);
      }
    }

    // ---- mask (boundary tiles only), online softmax in base 2
    const bool full = cur.nvalid == KT && cur.p0 >= lmax && cur.p0 + KT <= hmin;
    if (!full) {
      const int64_t dl = lo - cur.p0, dh = hi - cur.p0;
      const int lo_rel = int(dl < -1 ? -1 : (dl > KT ? KT : dl));
      const int hi_rel = int(dh < -1 ? -1 : (dh > KT ? KT : dh));
      const int lim = hi_rel < cur.nvalid ? hi_rel : cur.nvalid;
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = b2 * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          s[b2][v] = (key >= lo_rel && key < lim) ? s[b2][v] : -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int v = 0; v < 16; ++v) mt = fmaxf(mt, s[b2][v]);
    {
      float ma, mb;
      half_pair(mt, &ma, &mb);
      mt = fmaxf(ma, mb) * c2;
    }
    // Lazy rescale: keep the reference max until a tile exceeds it by more than
    // kRescaleSlack (base 2), so exp2 results stay <= 2^kRescaleSlack and the
    // accumulator is rescaled only when the reference moves.
    const bool bump = mt > m + kRescaleSlack;
    if (__any(bump)) {
      // rows that do not move keep alpha = 1 (also when their reference is still -inf)
      const float alpha = bump ? __builtin_amdgcn_exp2f(m - mt) : 1.f;  // 0 when m = -inf
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc_o[db][v] *= alpha;
      m = bump ? mt : m;
    }
    const float m_use = m == -INFINITY ? 0.f : m;
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[b2][v], c2, -m_use));
        s[b2][v] = e;
        ps[v & 3] += e;
      }
    lsum += (ps[0] + ps[1]) + (ps[2] + ps[3]);

    // ---- O^T += V^T P^T: V^T operand = two transpose loads of 4 keys x 16 dims
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = static_cast<__bf16>(s[u >> 1][8 * (u & 1) + e]);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const char* va = vb + v_rd + 16 * u * V_PITCH + db * 64;
        const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(va));
        const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(va + 8 * V_PITCH));
        const bf16x8 a = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf, acc_o[db], 0, 0, 0);
      }
    }

    if (have_next) store_tile(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    cur = nxt;
    have = have_next;
  }

  // ---- normalize.  The rows go out through LDS so that every store writes whole
  // 512-byte rows (the accumulator holds 16 bytes of a row per lane): each wave puts its
  // 32 rows in a 16 KB piece of the (now idle) stages, row r's 16-byte chunk c at slot
  // c ^ r (conflict-free lane-per-row writes and row-per-32-lanes reads), with each
  // row's destination next to them (-1: a row without keys, whose O is not written).
  float la, lb;
  half_pair(lsum, &la, &lb);
  const float ltot = la + lb;
  const bool has_keys = row_ok && live && ltot > 0.f;
  const float lse_out = has_keys ? (m + __log2f(ltot)) * kLn2 : -INFINITY;
  if (row_ok && half == 0) {
    if (sb >= 0)
      p.part_lse[prow] = lse_out;
    else
      p.lse_part[orow] = lse_out;
  }
  const float inv = has_keys ? 1.f / ltot : 0.f;
  static_assert(4 * 32 * D * 4 + 4 * 32 * 8 <= 2 * STAGE_BYTES, "four waves' rows fit the stages");
  char* tb = smem + wave * (32 * D * 4);
  int64_t* s_dst = reinterpret_cast<int64_t*>(smem + 4 * 32 * D * 4) + wave * 32;
  if (half == 0) s_dst[col] = has_keys ? (sb >= 0 ? prow : orow) * D : -1;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int c = 8 * db + 2 * a + half;  // dims 4c .. 4c + 3
      *reinterpret_cast<float4*>(tb + col * (D * 4) + ((c ^ col) * 16)) =
          make_float4(acc_o[db][4 * a] * inv, acc_o[db][4 * a + 1] * inv,
                      acc_o[db][4 * a + 2] * inv, acc_o[db][4 * a + 3] * inv);
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's rows are in LDS
  float* base = sb >= 0 ? p.part_o : p.o_part;
  const int c = lane & 31;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 2 * i + (lane >> 5);
    const int64_t at = s_dst[r];
    if (at >= 0)
      *reinterpret_cast<float4*>(base + at + 4 * c) =
          *reinterpret_cast<const float4*>(tb + r * (D * 4) + ((c ^ r) * 16));
  }
}

}  // namespace


hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  const int G = p.n_q_heads / p.n_kv_heads;
  const int64_t n_rows = int64_t(p.n_blocks) * p.block_size * G;
  const int64_t n_tiles = (n_rows + ROWS - 1) / ROWS;
  const int64_t n_out = int64_t(p.n_slots) + p.has_self;
  const int64_t n_pairs = int64_t(p.n_kv_heads) * n_out;
  const int64_t grid =
      p.piece ? fwd_split_layout(p.n_blocks, p.block_size, p.n_q_heads, p.n_kv_heads,
                                 int32_t(n_out)).grid
              : fwd_bf16_grid(p.n_blocks, p.block_size, p.n_q_heads, p.n_kv_heads, int32_t(n_out));
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fwd_bf16_kernel, dim3(unsigned(grid)), dim3(THREADS), 0, stream, p,
                     int(n_tiles), int(n_pairs));
  return hipGetLastError();
}

}  // namespace bsx
