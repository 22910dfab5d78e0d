// Backward pass of the draft-query block-sparse attention (bf16 inputs, gfx950).
//
// The training workload needs dQ, dK, dV of O = softmax(Q K^T / sqrt(d)) V (the
// attention formula of the Flash-dLLM page, "Method 1: I/O-Aware Fused KV-Cache
// Kernel") under the draft-block mask (Split-KV page, Abstract).  With the merged
// forward results (O, LSE), per query row r and visible key k:
//   P = exp(s - LSE),  D_r = sum_d dO_r O_r,  dS = P (dO_r . v_k - D_r),
//   dQ_r = scale sum_k dS k_k,  dK_k = scale sum_r dS q_r,  dV_k = sum_r P dO_r,
// where dK/dV sum over the query heads of the key's KV head.  Restricted to a chunk
// subset (one rank's local keys) this gives exact local dK/dV and that share of dQ.
//
// Three kernels, no atomics (results are deterministic):
//   delta: D_r = rowsum(dO * O), stored with the row's log2-domain LSE; the same
//          launch flags the key tiles no draft block sees and plans the dQ split.
//   dkdv:  key-major.  A workgroup owns 64 local keys of one KV head, 32 per wave
//          pair, and walks the draft blocks whose range reaches its keys, 32 query
//          rows at a time streamed into LDS.  In a pair one wave computes P and dV,
//          the other dP, dS and dK (P passes through LDS).  S = Q K^T and
//          dP = dO V^T put keys in lane columns, so the mask is one predicate per
//          lane; dV^T += dO^T P and dK^T += Q^T dS read dO^T / Q^T with LDS
//          transpose loads.  The draft blocks' own keys are extra tiles whose only
//          rows are their block's.
//   dq:    query-major, shaped like the forward kernel: 128 rows per workgroup,
//          K/V tiles of 64 keys in LDS; S^T = K Q^T and dP^T = V dO^T put rows in
//          lane columns, dQ^T += K^T dS^T reads K^T with transpose loads.  The
//          plan cuts each row tile's key walk into pieces of P tiles (about
//          kDqTargetWgs workgroups in all: draft blocks see very different context
//          lengths); a row tile of one piece writes dQ directly, the pieces of a split
//          row tile write partial sums that a reduce kernel adds in piece order.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "bsx_internal.h"
#include "fwd_common.h"
#include "mfma_common.h"

namespace bsx {
namespace {

constexpr int D = 128;
constexpr int THREADS = 256;
constexpr int KV_KEYS = 64;   // keys per dK / dV workgroup (and per flagged key tile)
constexpr int QROWS = kDqRows;  // query rows per dQ workgroup (row tile)
constexpr int KT = 64;          // keys per dQ K / V tile
typedef float f32x4v __attribute__((ext_vector_type(4)));
constexpr float kLog2e = 1.4426950408889634f;

// log2-domain LSE of a row; rows with no visible key get +inf so that P = 0.
__device__ inline float row_lse2(float lse) {
  return lse == -INFINITY ? INFINITY : lse * kLog2e;
}

// ---------------------------------------------------------------- dQ split plan
// One workgroup, the first of the row-statistics launch (the plan needs only the block
// ranges and the chunk list, so it costs no launch of its own).  w_t = key tiles of row
// tile t's context walk (the dQ kernel's own union of its rows' ranges over all local
// chunks); P = max(kDqMinPieceTiles, ceil(sum w / target)); count_t = max(1,
// ceil(w_t / P)) pieces.  Pieces are listed row tile by row tile; split row tiles
// (count_t > 1) get consecutive partial slots from sbase_t.  Header: P, number of
// pieces, number of split row tiles.
constexpr int kWaves = THREADS / 64;
constexpr int PLAN_LDS_TILES = 512;    // plans up to this many row tiles ...
constexpr int PLAN_LDS_ENTRIES = 512;  // ... and chunks work from LDS
struct PlanLds {
  ChunkEntry ent[PLAN_LDS_ENTRIES];
  int64_t lo[PLAN_LDS_TILES], hi[PLAN_LDS_TILES];
  int32_t tiles[PLAN_LDS_TILES];
  int64_t w[kWaves];
  int scan[3][kWaves];
};

__device__ void dq_plan_workgroup(const BSX_KARG BwdParams& p, int n_tiles, int cap, int target,
                                  PlanLds& s) {
  const int tid = threadIdx.x;
  const int Hkv = p.n_kv_heads, G = p.n_q_heads / Hkv;
  const int64_t n_rows = int64_t(p.n_blocks) * p.block_size * G;
  const char* table = p.table.dev ? p.table.dev : (const char*)(p.table.words);
  const ChunkEntry* ent = reinterpret_cast<const ChunkEntry*>(table);
  int32_t* plan = p.dq_plan;
  int32_t* count = plan + 4;
  int32_t* sbase = count + n_tiles;
  int32_t* piece_tile = sbase + n_tiles;
  int32_t* piece_j = piece_tile + cap;
  int32_t* multi_tile = piece_j + cap;

  // each thread owns a contiguous run of row tiles
  const int per = (n_tiles + THREADS - 1) / THREADS;
  const int t0 = tid * per < n_tiles ? tid * per : n_tiles;
  const int t1 = t0 + per < n_tiles ? t0 + per : n_tiles;
  auto span = [&](int t, int64_t* mlo, int64_t* mhi) {
    const int64_t r0 = int64_t(t) * QROWS;
    const int64_t r1 = r0 + QROWS < n_rows ? r0 + QROWS : n_rows;
    row_span_union(p.anchor, p.ctx_begin, p.ctx_len, p.block_size, G, false, r0, r1, mlo, mhi);
  };
  // key tiles of the walk over the chunk list E cut to [lo, hi): a sorted, disjoint list
  // is bisected to its first entry ending after lo and walked only while entries start
  // before hi; any other list is walked whole
  auto walk_len = [&](const ChunkEntry* E, int64_t lo, int64_t hi) -> int64_t {
    if (!(lo < hi)) return 0;
    if (p.entries_order < 2) return walk_tiles(E, 0, p.n_entries, lo, hi, KT);
    int e = 0, b = p.n_entries;
    while (e < b) {
      const int mid = (e + b) >> 1;
      if (E[mid].start + int64_t(E[mid].len) > lo) b = mid; else e = mid + 1;
    }
    int64_t w = 0;
    for (; e < p.n_entries && E[e].start < hi; ++e) w += walk_tiles(E, e, e + 1, lo, hi, KT);
    return w;
  };
  int64_t wsum = 0;
  const bool lds_ent = p.n_entries <= PLAN_LDS_ENTRIES;
  if (lds_ent)
    for (int e = tid; e < p.n_entries; e += THREADS) s.ent[e] = ent[e];
  const bool small = n_tiles <= PLAN_LDS_TILES && lds_ent;
  if (small) {
    // small plan: ranges, entries and the walk lengths in LDS
    for (int t = tid; t < n_tiles; t += THREADS) {
      span(t, &s.lo[t], &s.hi[t]);
      s.tiles[t] = 0;
    }
    __syncthreads();
    if (p.entries_order >= 2) {
      for (int t = tid; t < n_tiles; t += THREADS)
        s.tiles[t] = int32_t(walk_len(s.ent, s.lo[t], s.hi[t]));
    } else {
      // (row tile, entry) pairs spread over all lanes (at most 2^18 of them here)
      const int n_pairs = n_tiles * p.n_entries;
      for (int i = tid; i < n_pairs; i += THREADS) {
        const int t = i / p.n_entries, e = i - t * p.n_entries;
        const int64_t w = walk_tiles(s.ent, e, e + 1, s.lo[t], s.hi[t], KT);
        if (w) atomicAdd(&s.tiles[t], int(w));
      }
    }
    __syncthreads();
    for (int t = t0; t < t1; ++t) wsum += s.tiles[t];
  } else {
    if (lds_ent) __syncthreads();  // the LDS copy of the list is complete
    const ChunkEntry* E = lds_ent ? s.ent : ent;
    for (int t = t0; t < t1; ++t) {
      int64_t mlo, mhi;
      span(t, &mlo, &mhi);
      const int64_t w = walk_len(E, mlo, mhi);
      count[t] = int32_t(w < INT32_MAX ? w : INT32_MAX);
      wsum += w;
    }
  }
  // W: wave sums, then the sum of the wave totals (one barrier)
  const int lane = tid & 63, wv = tid >> 6;
  for (int off = 32; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off);
  if (lane == 0) s.w[wv] = wsum;
  __syncthreads();
  int64_t W = 0;
  for (int i = 0; i < kWaves; ++i) W += s.w[i];
  int64_t P = (W + target - 1) / target;
  P = P < kDqMinPieceTiles ? kDqMinPieceTiles : P;

  int own[3] = {0, 0, 0};  // pieces, partial slots, split row tiles
  for (int t = t0; t < t1; ++t) {
    const int64_t w = small ? s.tiles[t] : count[t];
    const int c = int(w > P ? (w + P - 1) / P : 1);
    count[t] = c;
    own[0] += c;
    own[1] += c > 1 ? c : 0;
    own[2] += c > 1 ? 1 : 0;
  }
  // exclusive scans of the three per-thread totals: inclusive scans within each wave,
  // then the wave totals (one barrier)
  int incl[3];
  for (int k = 0; k < 3; ++k) {
    incl[k] = own[k];
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl[k], off);
      if (lane >= off) incl[k] += y;
    }
    if (lane == 63) s.scan[k][wv] = incl[k];
  }
  __syncthreads();
  int before[3] = {0, 0, 0}, total[3] = {0, 0, 0};
  for (int i = 0; i < kWaves; ++i)
    for (int k = 0; k < 3; ++k) {
      before[k] += i < wv ? s.scan[k][i] : 0;
      total[k] += s.scan[k][i];
    }
  int at = before[0] + incl[0] - own[0], slot = before[1] + incl[1] - own[1],
      mi = before[2] + incl[2] - own[2];
  for (int t = t0; t < t1; ++t) {
    const int c = count[t];
    for (int j = 0; j < c; ++j) {
      piece_tile[at + j] = t;
      piece_j[at + j] = j;
    }
    at += c;
    if (c > 1) {
      sbase[t] = slot;
      slot += c;
      multi_tile[mi++] = t;
    } else {
      sbase[t] = -1;
    }
  }
  if (tid == 0) {
    plan[0] = int32_t(P);
    plan[1] = total[0];
    plan[2] = total[2];
    plan[3] = 0;
  }
}

// ---------------------------------------------------------------- row statistics
// Workgroups [0, plan_wgs) (none or one): the dQ split plan.  The next seen_wgs:
// tile_seen[t] for the 64-key local tiles t, THREADS tiles each: 1 when the context
// range [ctx_begin, anchor) of some draft block holds the position of one of the
// tile's keys (a key's gradients are sums over the rows that see it, so an unseen
// tile's dK and dV are zero).  These come first so that their longer chains of loads
// overlap the rest.  The other workgroups: stats[r] = (log2-domain LSE,
// D_r = rowsum(dO * O)) of query row r = q * H_q + h.
constexpr int kSeenLdsBlocks = 1024;  // block ranges staged in LDS per pass
constexpr int kSeenLdsEntries = 512;  // chunk tables up to this size are read from LDS
struct SeenLds {
  int64_t lo[kSeenLdsBlocks], hi[kSeenLdsBlocks];
  int64_t est[kSeenLdsEntries];
  uint32_t elen[kSeenLdsEntries], eoff[kSeenLdsEntries];
};
union DeltaLds {  // the plan and the tile flags run in different workgroups
  PlanLds plan;
  SeenLds seen;
};

__global__ __launch_bounds__(THREADS) void bwd_delta_kernel(BwdParams, int64_t n_rows,
                                                            int plan_wgs, int seen_wgs,
                                                            int n_ctx_tiles, int n_tiles, int cap,
                                                            int target) {
  const BSX_KARG BwdParams& p = kernel_arg0<BwdParams>();
  __shared__ __attribute__((aligned(16))) DeltaLds lds;
  const int wg = int(blockIdx.x);
  if (wg < plan_wgs) {
    dq_plan_workgroup(p, n_tiles, cap, target, lds.plan);
    return;
  }
  if (wg - plan_wgs >= seen_wgs) {
    const float* o = p.o;
    const uint16_t* d_o = static_cast<const uint16_t*>(p.d_o);
    const int64_t row =
        int64_t(wg - plan_wgs - seen_wgs) * (THREADS / 32) + (threadIdx.x >> 5);
    const int c = (threadIdx.x & 31) * 4;
    float acc = 0.f;
    if (row < n_rows) {
      const float4 ov = *reinterpret_cast<const float4*>(o + row * D + c);
      const uint2 dv = *reinterpret_cast<const uint2*>(d_o + row * D + c);
      acc = fmaf(ov.x, __uint_as_float(dv.x << 16), acc);
      acc = fmaf(ov.y, __uint_as_float(dv.x & 0xffff0000u), acc);
      acc = fmaf(ov.z, __uint_as_float(dv.y << 16), acc);
      acc = fmaf(ov.w, __uint_as_float(dv.y & 0xffff0000u), acc);
    }
    for (int off = 16; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if ((threadIdx.x & 31) == 0 && row < n_rows)
      reinterpret_cast<float2*>(p.stats)[row] = make_float2(row_lse2(p.lse[row]), acc);
    return;
  }
  // ---- key tile flags
  int64_t* s_lo = lds.seen.lo;
  int64_t* s_hi = lds.seen.hi;
  int64_t* s_est = lds.seen.est;
  uint32_t* s_elen = lds.seen.elen;
  uint32_t* s_eoff = lds.seen.eoff;
  const int t = (wg - plan_wgs) * THREADS + int(threadIdx.x);
  const bool own = t < n_ctx_tiles;
  const char* table = p.table.dev ? p.table.dev : (const char*)(p.table.words);
  const ChunkEntry* ent = reinterpret_cast<const ChunkEntry*>(table);
  // a small chunk table is copied to LDS with the first pass's block ranges (one round
  // trip): the search and the walk below then read no global memory one load at a time
  const int n_ent = p.n_entries;
  const bool lds_ent = n_ent <= kSeenLdsEntries;
  if (lds_ent) {
    for (int e = threadIdx.x; e < n_ent; e += THREADS) {
      s_est[e] = ent[e].start;
      s_elen[e] = ent[e].len;
      s_eoff[e] = ent[e].local_off;
    }
  }
  auto e_start = [&](int e) { return lds_ent ? s_est[e] : ent[e].start; };
  auto e_len = [&](int e) { return int64_t(lds_ent ? s_elen[e] : ent[e].len); };
  auto e_off = [&](int e) { return int64_t(lds_ent ? s_eoff[e] : ent[e].local_off); };
  // the tile's key rows [r0, r1) cut into at most a few position segments: the first
  // chunk holding row r0 (local offsets increase along the list) and those after it
  const int64_t r0 = int64_t(t) * KV_KEYS;
  const int64_t r1 = r0 + KV_KEYS < p.n_local ? r0 + KV_KEYS : p.n_local;
  int e0 = 0;
  bool seen = false;
  for (int b0 = 0; b0 < p.n_blocks; b0 += kSeenLdsBlocks) {
    const int nb = p.n_blocks - b0 < kSeenLdsBlocks ? p.n_blocks - b0 : kSeenLdsBlocks;
    __syncthreads();  // the previous pass is done with the staged ranges
    for (int i = threadIdx.x; i < nb; i += THREADS)
      visible_range(p.anchor, p.ctx_begin, p.ctx_len, p.block_size, false, b0 + i, &s_lo[i],
                    &s_hi[i]);
    __syncthreads();
    if (!own || seen) continue;
    if (b0 == 0) {
      int lo = 0, hi = n_ent - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (e_off(mid) <= r0) lo = mid; else hi = mid - 1;
      }
      e0 = lo;
    }
    for (int e = e0; e < n_ent && !seen; ++e) {
      const int64_t off = e_off(e), len = e_len(e);
      if (off >= r1) break;
      const int64_t a_row = r0 > off ? r0 : off;
      const int64_t z_row = r1 < off + len ? r1 : off + len;
      if (a_row >= z_row) continue;
      const int64_t a = e_start(e) + (a_row - off), z = e_start(e) + (z_row - off);
      for (int i = 0; i < nb; ++i)
        if (s_lo[i] < s_hi[i] && s_lo[i] < z && s_hi[i] > a) {
          seen = true;
          break;
        }
    }
  }
  if (own) p.tile_seen[t] = seen ? 1 : 0;
}

// ---------------------------------------------------------------- dK / dV
// A workgroup owns KV_KEYS local keys of one KV head as two wave pairs of 32 keys.
// The two waves of a pair split the work of the pair's keys by role:
//   role A (even wave): S = Q K^T -> P (masked, bf16) -> dV^T += dO^T P,
//   role B (odd wave):  dP = dO V^T, then with A's P: dS = P (dP - D) -> dK^T += Q^T dS,
// so each wave holds one 32 x 128 f32 accumulator and one of K / V as operands (two
// workgroups fit a CU).  P crosses from A to B through LDS once per step, as the
// bf16 values the dV product uses (dS is formed from those same values).
// The Q / dO rows of a step (32 query rows of one draft block) and their row
// statistics stream into four LDS stages with direct-to-LDS loads issued two steps
// ahead; one barrier per step publishes both A's P and the stage of the next step.
// Key positions come from a binary search of the chunk table (from an LDS copy when
// the table is small); the prologue's barriers wait for LDS traffic only, so the K / V
// operand loads arrive while the window of draft blocks is compacted.
constexpr int RS = 32;        // query rows per step
constexpr int DQ_LDS_ENTRIES = 256;  // chunk lists up to this long are searched in LDS by dQ
constexpr int ROW_B = D * 2;  // staged Q / dO row: 16 chunks of 16 bytes
constexpr int WIN = 128;      // draft blocks compacted per window
constexpr int XP_BYTES = 2048;  // one pair's P of one step: [u][lane] x 16 bytes
constexpr int SEARCH_LDS = 256;  // chunk tables up to this size are searched in LDS

// One stage.  Slot c of row r holds global chunk c ^ swz(r), so the b128 row reads
// and the transpose reads of the operands are free of bank conflicts.
struct DkdvStage {
  char q[RS * ROW_B];
  char d_o[RS * ROW_B];
  float lse2[RS];
  float delta[RS];
};

// Joins the workgroup barrier once at most N vector-memory loads of this wave are in
// flight and its LDS accesses are done.  Unlike __syncthreads it leaves the younger
// direct-to-LDS prefetches outstanding.
template <int N>
__device__ inline void wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Workgroup barrier for LDS traffic only: vector-memory loads in flight (the K / V
// operands, prefetches) stay outstanding, unlike __syncthreads.
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;

// LDS chunk swizzle of staged row r: slot c of the row holds global chunk c ^ swz(r).
// The LDS serves 64 banks of 4 bytes: a b128 operand read covers 16 rows at one chunk
// (conflict-free when swz is a bijection on r mod 16) and a transpose read 4 aligned
// rows x 4 adjacent chunks (conflict-free when bits 2-3 of swz differ over the 4
// rows); the low 4 bits of r rotated by two satisfy both.
__device__ inline int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// x / G for the query-head group size G and 0 <= x < 2^32 / G: the high word of
// x * ceil(2^32 / G).  With ceil(2^32 / G) = (2^32 + e) / G, 0 <= e < G, the product
// adds x e / 2^32 < 1 to x / G's fractional part, which stays below 1 (G = 1 apart).
struct DivByG {
  uint32_t m;
  bool one;
  __device__ explicit DivByG(int G)
      : m(G > 1 ? uint32_t(((uint64_t(1) << 32) + uint64_t(G) - 1) / uint64_t(G)) : 0u),
        one(G == 1) {}
  __device__ int operator()(int x) const {
    return one ? x : int(__umulhi(uint32_t(x), m));
  }
};

// The P exchange.  Written as LDS instructions the compiler does not track: it
// would otherwise make every access to these buffers (which no direct-to-LDS load
// targets) wait for all direct-to-LDS prefetches in flight.  The writes complete
// before the next wait_barrier (lgkmcnt(0)); the reads wait for their own data.
__device__ inline void xp_write(char* at, bf16x8 a, bf16x8 b) {
  const uint32_t addr = uint32_t(reinterpret_cast<uintptr_t>(at));
  asm volatile("ds_write_b128 %0, %1\n\tds_write_b128 %0, %2 offset:1024" ::"v"(addr),
               "v"(__builtin_bit_cast(u32x4, a)), "v"(__builtin_bit_cast(u32x4, b))
               : "memory");
}
__device__ inline void xp_read(const char* at, bf16x8* a, bf16x8* b) {
  const uint32_t addr = uint32_t(reinterpret_cast<uintptr_t>(at));
  u32x4 x, y;
  asm volatile(
      "ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:1024\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(x), "=&v"(y)
      : "v"(addr)
      : "memory");
  *a = __builtin_bit_cast(bf16x8, x);
  *b = __builtin_bit_cast(bf16x8, y);
}

__global__ __launch_bounds__(THREADS, 2) void bwd_dkdv_kernel(BwdParams, int n_ctx_tiles,
                                                              int self_tiles_per_block) {
  const BSX_KARG BwdParams& p = kernel_arg0<BwdParams>();
  // four stages as distinct arrays: loads into one provably never alias reads of another
  __shared__ __attribute__((aligned(16))) DkdvStage stg0;
  __shared__ __attribute__((aligned(16))) DkdvStage stg1;
  __shared__ __attribute__((aligned(16))) DkdvStage stg2;
  __shared__ __attribute__((aligned(16))) DkdvStage stg3;
  __shared__ __attribute__((aligned(16))) char xp0[2 * XP_BYTES];  // P of even steps
  __shared__ __attribute__((aligned(16))) char xp1[2 * XP_BYTES];  // P of odd steps
  __shared__ int s_blocks[WIN];
  __shared__ int64_t s_blo[WIN], s_bhi[WIN];
  __shared__ int s_wcount[4];
  __shared__ int64_t s_red[2][2];
  __shared__ uint32_t s_eoff[SEARCH_LDS];  // a small chunk table: local offsets ...
  __shared__ int64_t s_estart[SEARCH_LDS];  // ... and context starts

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform copies
  const int pair = wave_u >> 1;
  const bool role_b = (wave_u & 1) != 0;
  const int Hkv = p.n_kv_heads, Hq = p.n_q_heads, G = Hq / Hkv, B = p.block_size;
  const int g = blockIdx.x % Hkv;
  const int t = blockIdx.x / Hkv;
  const bool is_self = t >= n_ctx_tiles;
  const char* table = p.table.dev ? p.table.dev : (const char*)(p.table.words);
  const ChunkEntry* ent = reinterpret_cast<const ChunkEntry*>(table);

  // ---- this lane's key (both half-waves hold the same key column)
  int self_block = 0;
  int64_t key0, key_end;  // tile's first key row, end of the key rows it may use
  if (!is_self) {
    key0 = int64_t(t) * KV_KEYS;
    key_end = p.n_local;
  } else {
    const int st = t - n_ctx_tiles;
    self_block = st / self_tiles_per_block;
    key0 = int64_t(self_block) * B + int64_t(st % self_tiles_per_block) * KV_KEYS;
    key_end = int64_t(self_block + 1) * B;
  }
  const int kk = pair * 32 + col;
  const int64_t krow = key0 + kk;
  const bool kvalid = krow < key_end;
  const bool pair_live = __any(kvalid);  // same in both waves of a pair

  // ---- context keys no draft block sees: their dK and dV rows are zero.  Tile t pairs
  // with its mirror n - 1 - t: when exactly one of the two is seen, the seen tile's
  // workgroup also writes the other's zero rows after its own (the unseen tiles of a
  // packed batch cluster at the back, so their zero stores then overlap computing
  // workgroups instead of trailing them); otherwise each unseen tile writes its own.
  auto zero_tile = [&](int tt) {
    const int64_t k0 = int64_t(tt) * KV_KEYS;
    const int64_t rows = p.n_local - k0 < KV_KEYS ? p.n_local - k0 : KV_KEYS;
    const int c4 = (tid & 31) * 4;
#pragma unroll
    for (int i = 0; i < KV_KEYS / (THREADS / 32); ++i) {
      const int r = (tid >> 5) + i * (THREADS / 32);
      if (r < rows) {
        const int64_t at = ((k0 + r) * Hkv + g) * D + c4;
        // (whole lines, written once: streamed past the caches)
        __builtin_nontemporal_store(f32x4v{0.f, 0.f, 0.f, 0.f}, reinterpret_cast<f32x4v*>(p.dk + at));
        __builtin_nontemporal_store(f32x4v{0.f, 0.f, 0.f, 0.f}, reinterpret_cast<f32x4v*>(p.dv + at));
      }
    }
  };
  bool zero_mirror = false;
  const int t_mirror = n_ctx_tiles - 1 - t;
  if (!is_self) {
    const bool seen = p.tile_seen[t] != 0;
    const bool mirror_seen = t_mirror != t && p.tile_seen[t_mirror] != 0;
    if (!seen) {
      if (!mirror_seen) zero_tile(t);  // else the mirror tile's workgroup writes them
      return;
    }
    zero_mirror = t_mirror != t && !mirror_seen;
  }

  // ---- the first window's block ranges start loading (raw values, used later), a
  // small chunk table goes to LDS
  const int scan_begin = is_self ? self_block : 0;
  const int scan_end = is_self ? self_block + 1 : p.n_blocks;
  int64_t raw_a = 0, raw_z = 0;  // a block's ctx_begin and anchor
  bool in_win = false;
  auto load_ranges = [&](int w0) {
    const int b = w0 + tid;
    in_win = tid < WIN && b < scan_end;
    if (in_win && !is_self) {
      raw_a = p.ctx_begin[b];
      raw_z = p.anchor[b];
    }
  };
  // visible range of the lane's block of the window, [blo, bhi)
  int64_t blo = 0, bhi = 0;
  auto finish_ranges = [&](int w0) {
    if (!in_win) return;
    if (is_self) {
      blo = int64_t(w0 + tid) * B;
      bhi = blo + B;
    } else {
      int64_t a = raw_a, z = raw_z;
      a = a < 0 ? 0 : (a > p.ctx_len ? p.ctx_len : a);
      z = z < a ? a : (z > p.ctx_len ? p.ctx_len : z);
      blo = a;
      bhi = z;
    }
  };
  load_ranges(scan_begin);
  const int n_ent = p.n_entries;
  const bool lds_table = !is_self && n_ent <= SEARCH_LDS;
  if (lds_table) {
    for (int e = tid; e < n_ent; e += THREADS) {
      const ChunkEntry c = ent[e];
      s_eoff[e] = c.local_off;
      s_estart[e] = c.start;
    }
  }
  lds_barrier();

  // ---- context position of the key (role A applies the mask): the last chunk whose
  // local offset is at most the key's row
  int64_t kpos = krow;
  if (!is_self && kvalid && !role_b) {
    int lo = 0, hi = n_ent - 1;
    if (lds_table) {
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (int64_t(s_eoff[mid]) <= krow) lo = mid; else hi = mid - 1;
      }
      kpos = s_estart[lo] + (krow - int64_t(s_eoff[lo]));
    } else {
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (int64_t(ent[mid].local_off) <= krow) lo = mid; else hi = mid - 1;
      }
      kpos = ent[lo].start + (krow - int64_t(ent[lo].local_off));
    }
  }

  // ---- K (role A) or V (role B) rows of this lane's key: MFMA B operands, dims
  // 16 i + 8 half .. + 8; rows past the tile's end read as zero; they
  // arrive while the window is compacted
  const int64_t kstride = int64_t(Hkv) * D;
  const uint32_t row_bytes = uint32_t(kstride * 2);
  const int64_t nrows_tile = key_end - key0 < KV_KEYS ? key_end - key0 : KV_KEYS;
  const void* kv_src = is_self ? (role_b ? p.v_self : p.k_self) : (role_b ? p.v : p.k);
  bf16x8 kf[8];
  {
    const uint32_t bytes = nrows_tile > 0 ? uint32_t(nrows_tile) * row_bytes : 0u;
    const __amdgpu_buffer_rsrc_t kr =
        make_rsrc(static_cast<const uint16_t*>(kv_src) + key0 * kstride + int64_t(g) * D, bytes);
    const uint32_t off = uint32_t(kk) * row_bytes + 16 * half;
#pragma unroll
    for (int i = 0; i < 8; ++i) kf[i] = as_bf16x8(buffer_load16(kr, off + 32 * i));
  }

  // ---- position range of the workgroup's keys (from the role-A waves)
  if (!role_b) {
    int64_t a = kvalid ? kpos : INT64_MAX, b = kvalid ? kpos : INT64_MIN;
    for (int off = 16; off >= 1; off >>= 1) {
      const int64_t a2 = __shfl_xor(a, off), b2 = __shfl_xor(b, off);
      a = a2 < a ? a2 : a;
      b = b2 > b ? b2 : b;
    }
    if (lane == 0) {
      s_red[pair][0] = a;
      s_red[pair][1] = b;
    }
  }
  lds_barrier();
  int64_t pmin = s_red[0][0] < s_red[1][0] ? s_red[0][0] : s_red[1][0];
  int64_t pmax = s_red[0][1] > s_red[1][1] ? s_red[0][1] : s_red[1][1];
  pmin = uniform64(pmin);
  pmax = uniform64(pmax);

  f32x16 acc[4];  // dV^T (role A) or unscaled dK^T (role B): rows d, columns keys
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = zero16();
  const float c2 = p.scale_log2;
  const int nr = B * G;  // query rows of one draft block
  const int nsub = (nr + RS - 1) / RS;
  // operand reads of a stage: b128 row read of row col, chunk 2 i + half, at
  // (k_rd ^ 32 i); transpose read of rows 16 u + 8 hi + 4 half + tj / 4, chunk
  // 4 db + c0, at (tr_rd[hi] ^ 64 db) + 4096 u
  const int k_rd = col * ROW_B + 16 * (half ^ swz(col));
  int tr_rd[2];
  {
    const int tj = lane & 15, tg = lane >> 4;
#pragma unroll
    for (int hi2 = 0; hi2 < 2; ++hi2) {
      const int rr = 8 * hi2 + 4 * half + (tj >> 2);
      const int c0 = 2 * (tg & 1) + ((tj & 3) >> 1);
      tr_rd[hi2] = rr * ROW_B + 16 * (c0 ^ swz(rr)) + 8 * (tj & 1);
    }
  }
  // staging: wave w fills rows 8 w .. 8 w + 7 of Q and of dO, four rows per load
  // (lane: row 8 w + 4 i + lane / 16, slot lane % 16 <- chunk slot ^ swz(row), where
  // swz(row) = ((lane / 16) << 2) | (2 (w & 1) + i));
  // wave 0 also loads the 32 rows' statistics (lane: row lane % 32, field lane / 32)
  const uint32_t ld_chunk = uint32_t(((lane & 15) ^ ((lane >> 4) << 2) ^ (2 * (wave & 1))) * 16);
  const DivByG div_g(G);  // rows of a block are < B G, far below 2^32 / G
  const int blk_elems = B * Hq * D;
  const uint32_t blk_bytes = uint32_t(blk_elems) * 2u;
  const uint32_t blk_stat_bytes = uint32_t(B * Hq) * 8u;

  for (int wb = scan_begin; wb < scan_end && pmin <= pmax; wb += WIN) {
    // ordered compaction of the hit blocks of this window (and their ranges)
    if (wb != scan_begin) load_ranges(wb);
    finish_ranges(wb);
    const bool hit = in_win && (is_self || (blo < bhi && blo <= pmax && bhi > pmin));
    const uint64_t ball = __ballot(hit);
    lds_barrier();  // the previous window is done with s_blocks, the stages and P
    if (lane == 0) s_wcount[wave] = __popcll(ball);
    lds_barrier();
    int before = 0, total = 0;
    for (int w = 0; w < 4; ++w) {
      before += w < wave ? s_wcount[w] : 0;
      total += s_wcount[w];
    }
    if (hit) {
      const int at = before + __popcll(ball & ((uint64_t(1) << lane) - 1));
      s_blocks[at] = wb + tid;
      s_blo[at] = blo;
      s_bhi[at] = bhi;
    }
    lds_barrier();
    const int nseq = total * nsub;
    if (nseq == 0) continue;

    // loads of the next step in issue order into `dst`
    int ib = 0, isub = 0;
    auto issue = [&](DkdvStage& dst) {
      const int blk = __builtin_amdgcn_readfirstlane(s_blocks[ib]);
      const int64_t q0 = int64_t(blk) * B;  // the block's first query
      const __amdgpu_buffer_rsrc_t qr =
          make_rsrc(static_cast<const uint16_t*>(p.q) + q0 * Hq * D, blk_bytes);
      const __amdgpu_buffer_rsrc_t dr =
          make_rsrc(static_cast<const uint16_t*>(p.d_o) + q0 * Hq * D, blk_bytes);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int rr = isub * RS + 8 * wave + 4 * i + (lane >> 4);  // row within the block
        const int qq = div_g(rr);
        const uint32_t off = rr < nr ? uint32_t(((qq * Hq + g * G + (rr - qq * G)) * D) * 2) +
                                           (ld_chunk ^ uint32_t(16 * i))
                                     : 0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            qr, (lds_void*)(dst.q + (8 * wave_u + 4 * i) * ROW_B), 16, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            dr, (lds_void*)(dst.d_o + (8 * wave_u + 4 * i) * ROW_B), 16, off, 0, 0, 0);
      }
      if (wave_u == 0) {
        const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.stats + q0 * Hq * 2, blk_stat_bytes);
        const int rr = isub * RS + col;
        const int qq = div_g(rr);
        const uint32_t off =
            rr < nr ? uint32_t(((qq * Hq + g * G + (rr - qq * G)) * 2 + half) * 4) : 0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_void*)(dst.lse2), 4, off, 0, 0, 0);
      }
      if (++isub == nsub) {
        isub = 0;
        ++ib;
      }
    };

    int j = 0, cb = 0, csub = 0;  // step computed next, its block index and sub-tile
    // One step computes on stage `cur` and loads step j + 3 into `nx`; the barrier in
    // its middle publishes A's P (buffer `xpb`) and the stage of step j + 1.
    auto step = [&](DkdvStage& cur, DkdvStage& nx, char* xpb) -> bool {
      char* xpp = xpb + pair * XP_BYTES;
      f32x16 s;  // set in the role that is live (a zero start in its first product)
      bf16x8 pb[2];
      bf16x4 tr[2][4][2];  // phase-2 transpose operands, read before the barrier
      float4 st4[4];       // A: log2 LSE (+inf for an invisible key); B: D
      if (pair_live && !role_b) {
        u32x4 opd[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          opd[i] = *reinterpret_cast<const u32x4*>(cur.q + (k_rd ^ (32 * i)));
#pragma unroll
        for (int a = 0; a < 4; ++a)
          st4[a] = *reinterpret_cast<const float4*>(cur.lse2 + 8 * a + 4 * half);
        __builtin_amdgcn_sched_barrier(0);
        s = zero16();
#pragma unroll
        for (int i = 0; i < 8; ++i) s = mfma_bf16(as_bf16x8(opd[i]), kf[i], s);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            tr[u][db][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4*)(cur.d_o + ((tr_rd[0] ^ (64 * db)) + 4096 * u)));
            tr[u][db][1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4*)(cur.d_o + ((tr_rd[1] ^ (64 * db)) + 4096 * u)));
          }
        // an invisible key gets P = exp2(x - inf) = 0
        const int64_t vlo = s_blo[cb], vhi = s_bhi[cb];
        const float koff = (kvalid & (kpos >= vlo) & (kpos < vhi)) ? 0.f : INFINITY;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float lv[4] = {st4[a].x + koff, st4[a].y + koff, st4[a].z + koff, st4[a].w + koff};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * a + e;
            s[v] = __builtin_amdgcn_exp2f(fmaf(s[v], c2, -lv[e]));
          }
        }
        pb[0] = pack_bf16(s, 0);
        pb[1] = pack_bf16(s, 1);
        xp_write(xpp + lane * 16, pb[0], pb[1]);
      }
      if (pair_live && role_b) {
        u32x4 opd[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          opd[i] = *reinterpret_cast<const u32x4*>(cur.d_o + (k_rd ^ (32 * i)));
        __builtin_amdgcn_sched_barrier(0);
        s = zero16();
#pragma unroll
        for (int i = 0; i < 8; ++i) s = mfma_bf16(as_bf16x8(opd[i]), kf[i], s);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            tr[u][db][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4*)(cur.q + ((tr_rd[0] ^ (64 * db)) + 4096 * u)));
            tr[u][db][1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4*)(cur.q + ((tr_rd[1] ^ (64 * db)) + 4096 * u)));
          }
#pragma unroll
        for (int a = 0; a < 4; ++a)
          st4[a] = *reinterpret_cast<const float4*>(cur.delta + 8 * a + 4 * half);
      }
      if (j + 2 < nseq) {
        if (wave_u == 0) wait_barrier<5>(); else wait_barrier<4>();
      } else {
        wait_barrier<0>();
      }
      if (j + 3 < nseq) issue(nx);
      if (pair_live && role_b) {
        xp_read(xpp + lane * 16, &pb[0], &pb[1]);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float dd[4] = {st4[a].x, st4[a].y, st4[a].z, st4[a].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * a + e;
            s[v] = static_cast<float>(pb[v >> 3][v & 7]) * (s[v] - dd[e]);  // dS
          }
        }
        pb[0] = pack_bf16(s, 0);
        pb[1] = pack_bf16(s, 1);
      }
      if (pair_live) {
        // A: dV^T += dO^T P;  B: dK^T += Q^T dS
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const bf16x4 lo4 = tr[u][db][0], hi4 = tr[u][db][1];
            const bf16x8 a = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
            acc[db] = mfma_bf16(a, pb[u], acc[db]);
          }
      }
      if (++csub == nsub) {
        csub = 0;
        ++cb;
      }
      return ++j < nseq;
    };

    // prologue: steps 0 .. 2 in flight, step 0 published
    issue(stg0);
    if (nseq > 1) issue(stg1);
    if (nseq > 2) issue(stg2);
    if (nseq > 2) {
      if (wave_u == 0) wait_barrier<10>(); else wait_barrier<8>();
    } else if (nseq > 1) {
      if (wave_u == 0) wait_barrier<5>(); else wait_barrier<4>();
    } else {
      wait_barrier<0>();
    }
    while (step(stg0, stg3, xp0) && step(stg1, stg0, xp1) && step(stg2, stg1, xp0) &&
           step(stg3, stg2, xp1)) {
    }
  }

  // ---- dV (role A) or dK (role B) of the pair's 32 keys, through LDS so that whole
  // 512-byte rows go out per store (the accumulator holds 16 bytes of a row per lane,
  // rows 4 KB apart).  Each wave uses one stage: row r, 16-byte chunk c at slot c ^ r,
  // so the lane-per-row writes and the row-per-32-lanes reads are conflict-free.
  lds_barrier();  // every wave is done with the stages
  char* tb = reinterpret_cast<char*>(wave_u == 0 ? &stg0 : wave_u == 1 ? &stg1 : wave_u == 2 ? &stg2 : &stg3);
  static_assert(32 * D * 4 <= int(sizeof(DkdvStage)), "a wave's rows fit one stage");
  const float sc = role_b ? p.scale : 1.f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int c = 8 * db + 2 * a + half;  // dims 4c .. 4c + 3
      *reinterpret_cast<float4*>(tb + col * (D * 4) + ((c ^ col) * 16)) =
          make_float4(acc[db][4 * a] * sc, acc[db][4 * a + 1] * sc, acc[db][4 * a + 2] * sc,
                      acc[db][4 * a + 3] * sc);
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's rows are in LDS
  float* dst = role_b ? (is_self ? p.dk_self : p.dk) : (is_self ? p.dv_self : p.dv);
  const int c = lane & 31;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 2 * i + (lane >> 5);
    const float4 v = *reinterpret_cast<const float4*>(tb + r * (D * 4) + ((c ^ r) * 16));
    const int64_t key = key0 + pair * 32 + r;
    if (key < key_end) *reinterpret_cast<float4*>(dst + (key * Hkv + g) * D + 4 * c) = v;
  }
  if (zero_mirror) zero_tile(t_mirror);
}

// ---------------------------------------------------------------- dQ
constexpr int ROW_BYTES = D * 2;         // staged K / V row: 16 chunks of 16 bytes
constexpr int TILE_BYTES = KT * ROW_BYTES;

__global__ __launch_bounds__(THREADS, 2) void bwd_dq_kernel(BwdParams, int n_tiles, int cap) {
  const BSX_KARG BwdParams& p = kernel_arg0<BwdParams>();
  // two stages of K and V tiles, four distinct arrays: the direct-to-LDS loads into
  // one stage provably never alias the operand reads of the other
  __shared__ __attribute__((aligned(16))) char lds_k0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char lds_v0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char lds_k1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char lds_v1[TILE_BYTES];
  __shared__ int64_t red[4][4];
  // the chunk list, when it is short: a workgroup finds where its walk starts from LDS
  __shared__ __attribute__((aligned(16))) ChunkEntry s_ent[DQ_LDS_ENTRIES];
  __shared__ int64_t s_dst[4][32];  // destinations of the rows (epilogue)

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;
  const int Hkv = p.n_kv_heads, Hq = p.n_q_heads, G = Hq / Hkv, B = p.block_size;
  const int g = blockIdx.x % Hkv;
  const int piece = blockIdx.x / Hkv;
  const int64_t n_q = int64_t(p.n_blocks) * B;
  const int64_t n_rows = n_q * G;
  const char* table = p.table.dev ? p.table.dev : (const char*)(p.table.words);
  const ChunkEntry* ent = reinterpret_cast<const ChunkEntry*>(table);
  const bool lds_ent = p.n_entries <= DQ_LDS_ENTRIES;
  static_assert(DQ_LDS_ENTRIES == THREADS, "one chunk entry per thread");
  // this thread's entry (start, len): buffer loads (a generic-pointer load would make
  // every later wait include it), written to LDS once Q / dO are in flight
  int64_t my_start = 0;
  uint32_t my_len = 0, my_loff = 0;
  if (lds_ent) {
    const __amdgpu_buffer_rsrc_t er = make_rsrc(ent, uint32_t(p.n_entries) * 16u);
    my_start = __builtin_bit_cast(int64_t, __builtin_amdgcn_raw_buffer_load_b64(er, uint32_t(tid) * 16u, 0, 0));
    my_len = __builtin_amdgcn_raw_buffer_load_b32(er, uint32_t(tid) * 16u + 8u, 0, 0);
    my_loff = __builtin_amdgcn_raw_buffer_load_b32(er, uint32_t(tid) * 16u + 12u, 0, 0);
  }

  // this workgroup's piece: key tiles [j P, j P + P) of row tile tile_id's walk
  const int32_t* plan = p.dq_plan;
  const int P = plan[0];
  if (piece >= plan[1]) return;
  const int32_t* count = plan + 4;
  const int32_t* sbase = count + n_tiles;
  const int32_t* piece_tile = sbase + n_tiles;
  const int32_t* piece_j = piece_tile + cap;
  const int tile_id = piece_tile[piece];
  const int pj = piece_j[piece];
  const bool split = count[tile_id] > 1;

  const int64_t r = int64_t(tile_id) * QROWS + wave * 32 + col;
  const bool row_ok = r < n_rows;
  const int64_t qi = row_ok ? r / G : 0;
  const int h = g * G + int(row_ok ? r % G : 0);
  const int64_t blk = qi / B;
  const float2 stat = row_ok ? reinterpret_cast<const float2*>(p.stats)[qi * Hq + h]
                             : make_float2(INFINITY, 0.f);
  const float lse2 = stat.x, dlt = stat.y;

  // the context range of the lane's block (issued before the Q / dO loads, so the range
  // reduction waits for these alone)
  int64_t ctx_lo = 0, ctx_hi = 0;
  if (row_ok) visible_range(p.anchor, p.ctx_begin, p.ctx_len, B, false, blk, &ctx_lo, &ctx_hi);

  // Q^T and dO^T fragments of this lane's row (dims 16t + 8*half .. +8)
  bf16x8 qf[8], dof[8];
  {
    const int64_t q0 = int64_t(tile_id) * QROWS / G;
    const int64_t bytes = (n_q - q0) * Hq * D * 2;
    const uint32_t nb = uint32_t(bytes < 0xffffffffll ? bytes : 0xffffffffll);
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(static_cast<const uint16_t*>(p.q) + q0 * Hq * D, nb);
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(static_cast<const uint16_t*>(p.d_o) + q0 * Hq * D, nb);
    const uint32_t off = row_ok ? uint32_t(((qi - q0) * Hq + h) * D * 2) + 16 * half : 0x80000000u;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      qf[t] = as_bf16x8(buffer_load16(qr, off + 32 * t));
      dof[t] = as_bf16x8(buffer_load16(dr, off + 32 * t));
    }
  }
  if (lds_ent && tid < p.n_entries) {  // published by the range barriers below
    s_ent[tid].start = my_start;
    s_ent[tid].len = my_len;
    s_ent[tid].local_off = my_loff;
  }

  f32x16 dq[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) dq[db] = zero16();
  const float c2 = p.scale_log2;
  const int64_t kstride = int64_t(Hkv) * D;
  const uint32_t row_bytes = uint32_t(kstride * 2);
  const int64_t gofs = int64_t(g) * D;
  // Direct-to-LDS staging: wave w fills rows 16w .. 16w + 15 of a tile, four rows per
  // instruction, one 16-byte chunk per lane; slot c of LDS row r holds global chunk
  // c ^ swz(r), so the b128 and transpose operand reads below are conflict-free.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t ld_row_off = uint32_t(16 * wave + (lane >> 4)) * row_bytes;
  // (row 16w + 4i + lane / 16: swz = ((lane / 16) << 2) | i)
  const uint32_t ld_chunk = uint32_t(((lane & 15) ^ ((lane >> 4) << 2)) * 16);
  // b128 read of key row col [+32], chunk 2t + half: address (k_rd ^ 32t) [+ 8192]
  const int k_rd = col * ROW_BYTES + 16 * (half ^ swz(col));
  // transpose read (rows 16u + 8hi + 4half + j/4, chunk 4db + c0): (tr_rd[hi] ^ 64db) + 4096u
  const int tj = lane & 15, tg = lane >> 4;
  int tr_rd[2];
#pragma unroll
  for (int hi2 = 0; hi2 < 2; ++hi2) {
    const int rr = 8 * hi2 + 4 * half + (tj >> 2);
    const int c0 = 2 * (tg & 1) + ((tj & 3) >> 1);
    tr_rd[hi2] = rr * ROW_BYTES + 16 * (c0 ^ swz(rr)) + 8 * (tj & 1);
  }

  // phase 0: local context chunks; phase 1: the draft blocks' own keys
  for (int phase = 0; phase < (p.has_self && pj == 0 ? 2 : 1); ++phase) {
    const bool is_self = phase == 1;
    int64_t lo = ctx_lo, hi = ctx_hi;
    if (row_ok && is_self)
      visible_range(p.anchor, p.ctx_begin, p.ctx_len, B, true, blk, &lo, &hi);
    const bool live = row_ok && lo < hi;
    {
      int64_t a = live ? lo : INT64_MAX, b = live ? hi : INT64_MIN;
      int64_t c = live ? lo : INT64_MIN, e = live ? hi : INT64_MAX;
      for (int off = 16; off >= 1; off >>= 1) {
        const int64_t a2 = __shfl_xor(a, off), b2 = __shfl_xor(b, off);
        const int64_t c3 = __shfl_xor(c, off), e2 = __shfl_xor(e, off);
        a = a2 < a ? a2 : a;
        b = b2 > b ? b2 : b;
        c = c3 > c ? c3 : c;
        e = e2 < e ? e2 : e;
      }
      // (LDS-only barriers: the Q / dO loads stay in flight while the walk starts and the
      // first K / V tile loads; the first MFMA waits for them)
      lds_barrier();  // previous phase is done with `red` (and the stages)
      if (lane == 0) {
        red[wave][0] = a;
        red[wave][1] = b;
        red[wave][2] = c;
        red[wave][3] = e;
      }
    }
    lds_barrier();
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

    // the context walk of piece pj starts pj * P tiles in; the self walk is one piece.
    // With the list in LDS the start (chunk entry, tile within its segment) is found
    // there: bisection to the first chunk that ends after mlo when the list is sorted
    // and disjoint, then whole chunks skipped by their tile counts.
    int e_start = -1;
    int64_t skip_in = 0;
    if (!is_self && lds_ent && mlo < mhi) {
      int e = 0;
      if (p.entries_order >= 2) {
        int b1 = p.n_entries;
        while (e < b1) {
          const int mid = (e + b1) >> 1;
          if (s_ent[mid].start + int64_t(s_ent[mid].len) > mlo) b1 = mid; else e = mid + 1;
        }
      }
      int64_t skip = int64_t(pj) * P;
      for (; e < p.n_entries; ++e) {
        const int64_t st = s_ent[e].start;
        if (p.entries_order >= 1 && st >= mhi) break;
        const int64_t a = st > mlo ? st : mlo;
        const int64_t en = st + int64_t(s_ent[e].len);
        const int64_t z = en < mhi ? en : mhi;
        if (a >= z) continue;
        const int64_t w = (z - a + KT - 1) / KT;
        if (skip < w) {
          e_start = e;
          skip_in = skip;
          break;
        }
        skip -= w;
      }
      if (e_start < 0) continue;  // the piece is past the walk's end
    }
    SegmentWalk walk;
    if (is_self) {
      walk.init(nullptr, 0, 0, true, mlo, mhi);
      if (!(mlo < mhi) || !walk.next()) continue;
    } else if (e_start >= 0) {
      // the first segment from the LDS copy; later segments come from the list itself
      walk.init_range(ent, e_start + 1, p.n_entries, mlo, mhi, p.entries_order >= 1 ? 1 : 0);
      const int64_t st = s_ent[e_start].start;
      const int64_t en = st + int64_t(s_ent[e_start].len);
      walk.seg0 = st > mlo ? st : mlo;
      walk.seg1 = en < mhi ? en : mhi;
      walk.local0 = int64_t(s_ent[e_start].local_off) + (walk.seg0 - st);
    } else {
      walk.init_range(ent, 0, p.n_entries, mlo, mhi, p.entries_order);
      if (!(mlo < mhi) || !walk.next()) continue;
    }
    int64_t p0 = walk.seg0 + skip_in * KT;
    int left = is_self ? INT32_MAX : P;
    if (!is_self && e_start < 0) {
      int64_t skip = int64_t(pj) * P;
      bool found = true;
      while (skip > 0) {
        const int64_t seg_tiles = (walk.seg1 - walk.seg0 + KT - 1) / KT;
        if (skip < seg_tiles) break;
        skip -= seg_tiles;
        if (!walk.next()) {
          found = false;
          break;
        }
      }
      if (!found) continue;
      p0 = walk.seg0 + skip * KT;
    }
    const uint16_t* kbase = static_cast<const uint16_t*>(is_self ? p.k_self : p.k);
    const uint16_t* vbase = static_cast<const uint16_t*>(is_self ? p.v_self : p.v);

    auto tile_of = [&](int64_t pos0, int64_t* l0, int* nvalid) {
      *l0 = walk.local0 + (pos0 - walk.seg0);
      const int64_t n = walk.seg1 - pos0;
      *nvalid = int(n < KT ? n : KT);
    };
    // the buffers end after the tile's last valid key: rows beyond it read as zero
    auto dma_tile = [&](int64_t l0, int nvalid, char* kdst, char* vdst) {
      const uint32_t bytes = uint32_t(nvalid - 1) * row_bytes + D * 2;
      const __amdgpu_buffer_rsrc_t kb = make_rsrc(kbase + l0 * kstride + gofs, bytes);
      const __amdgpu_buffer_rsrc_t vb = make_rsrc(vbase + l0 * kstride + gofs, bytes);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t off = ld_row_off + uint32_t(4 * i) * row_bytes + (ld_chunk ^ uint32_t(16 * i));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            kb, (lds_void*)(kdst + (16 * wave_u + 4 * i) * ROW_BYTES), 16, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            vb, (lds_void*)(vdst + (16 * wave_u + 4 * i) * ROW_BYTES), 16, off, 0, 0, 0);
      }
    };
    // dS for one staged tile and its contribution dQ^T += K^T dS^T
    auto compute_tile = [&](const char* kb, const char* vb, int64_t t_p0, int t_n) {
      f32x16 sv[2], dp[2];
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2) {
        sv[b2] = zero16();
        dp[b2] = zero16();
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int o = (k_rd ^ (32 * t)) + b2 * 32 * ROW_BYTES;
          sv[b2] = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(kb + o)), qf[t], sv[b2]);
          dp[b2] = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(vb + o)), dof[t], dp[b2]);
        }
      }
      const bool full = t_n == KT && t_p0 >= lmax && t_p0 + KT <= hmin;
      int lo_h = -4 * half, lim_h = KT - 4 * half;
      if (!full) {
        const int64_t dl = lo - t_p0, dh = hi - t_p0;
        const int lo_rel = int(dl < -1 ? -1 : (dl > KT ? KT : dl));
        const int hi_rel = int(dh < -1 ? -1 : (dh > KT ? KT : dh));
        lo_h = lo_rel - 4 * half;
        lim_h = (hi_rel < t_n ? hi_rel : t_n) - 4 * half;
      }
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          // key = kb16 + 4 * half; bounds shifted by the lane's half instead
          const int kb16 = b2 * 32 + 8 * (v >> 2) + (v & 3);
          const bool vis = live && kb16 >= lo_h && kb16 < lim_h;
          const float pv = vis ? __builtin_amdgcn_exp2f(fmaf(sv[b2][v], c2, -lse2)) : 0.f;
          sv[b2][v] = pv * (dp[b2][v] - dlt);  // dS
        }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 sb = pack_bf16(sv[u >> 1], u & 1);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(kb + ((tr_rd[0] ^ (64 * db)) + 4096 * u)));
          const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(kb + ((tr_rd[1] ^ (64 * db)) + 4096 * u)));
          const bf16x8 a = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
          dq[db] = mfma_bf16(a, sb, dq[db]);
        }
      }
    };

    int64_t cur_p0 = p0, cur_l0;
    int cur_n;
    tile_of(cur_p0, &cur_l0, &cur_n);
    dma_tile(cur_l0, cur_n, lds_k0, lds_v0);
    __syncthreads();  // also waits for the direct-to-LDS loads
    // One step computes the tile in (kb, vb) while the next tile streams into
    // (kn, vn); the barrier at its end publishes that tile and retires this one.
    auto step = [&](const char* kb, const char* vb, char* kn, char* vn) {
      int64_t nxt_p0 = cur_p0 + KT, nxt_l0 = 0;
      int nxt_n = 0;
      bool have_next = --left > 0;
      if (have_next && nxt_p0 >= walk.seg1) {
        have_next = walk.next();
        nxt_p0 = have_next ? walk.seg0 : 0;
      }
      if (have_next) {
        tile_of(nxt_p0, &nxt_l0, &nxt_n);
        dma_tile(nxt_l0, nxt_n, kn, vn);
      }
      compute_tile(kb, vb, cur_p0, cur_n);
      __syncthreads();
      cur_p0 = nxt_p0;
      cur_l0 = nxt_l0;
      cur_n = nxt_n;
      return have_next;
    };
    while (step(lds_k0, lds_v0, lds_k1, lds_v1) && step(lds_k1, lds_v1, lds_k0, lds_v0)) {
    }
  }

  // ---- the rows go out through LDS so that every store writes whole 512-byte rows (the
  // accumulator holds 16 bytes of a row per lane): wave w puts its 32 rows in tile
  // buffer w, row r's 16-byte chunk c at slot c ^ r, with each row's destination in
  // s_dst (-1: past the last row).  A split row tile's piece writes its unscaled
  // partial sum, [slot][row in tile][d]; otherwise dQ = scale * sum.
  lds_barrier();  // every wave is done with the tile buffers
  char* tb = wave_u == 0 ? lds_k0 : wave_u == 1 ? lds_v0 : wave_u == 2 ? lds_k1 : lds_v1;
  static_assert(32 * D * 4 <= TILE_BYTES, "a wave's rows fit one tile buffer");
  const float sc = split ? 1.f : p.scale;
  float* base = split ? p.dq_part : p.dq;
  if (half == 0)
    s_dst[wave][col] =
        !row_ok ? -1
                : split ? ((int64_t(sbase[tile_id] + pj) * Hkv + g) * QROWS + wave * 32 + col) * D
                        : (qi * Hq + h) * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int c = 8 * db + 2 * a + half;  // dims 4c .. 4c + 3
      *reinterpret_cast<float4*>(tb + col * (D * 4) + ((c ^ col) * 16)) =
          make_float4(dq[db][4 * a] * sc, dq[db][4 * a + 1] * sc, dq[db][4 * a + 2] * sc,
                      dq[db][4 * a + 3] * sc);
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's rows are in LDS
  const int c = lane & 31;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 2 * i + (lane >> 5);
    const int64_t at = s_dst[wave][r];
    if (at >= 0)
      *reinterpret_cast<float4*>(base + at + 4 * c) =
          *reinterpret_cast<const float4*>(tb + r * (D * 4) + ((c ^ r) * 16));
  }
}

// ---------------------------------------------------------------- dQ reduce
// dQ of a split row tile = scale * sum of its pieces' partials.  One workgroup per
// (split row tile, KV head, 8-row group): its four 64-lane groups each add a fixed
// quarter of the pieces in piece order, and the four sums are added in group order,
// so the result is deterministic.  A long walk splits into many pieces (tens), and
// one lane adding all of them one after another would set the kernel's time.  Each
// load instruction of a lane group reads 1 KB contiguous (two rows, 16 bytes a lane).
constexpr int RED_ROWS = 8;
constexpr int RED_SPLIT = THREADS / (RED_ROWS * 8);  // lane groups per row group

__global__ __launch_bounds__(THREADS) void bwd_dq_reduce_kernel(BwdParams, int n_tiles, int cap) {
  const BSX_KARG BwdParams& p = kernel_arg0<BwdParams>();
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  __shared__ f32x4v s_part[RED_SPLIT - 1][4][RED_ROWS * 8];  // lane-minor: conflict-free
  const int Hkv = p.n_kv_heads, Hq = p.n_q_heads, G = Hq / Hkv;
  constexpr int kGroups = QROWS / RED_ROWS;
  const int g = blockIdx.x % Hkv;
  const int rg = (blockIdx.x / Hkv) % kGroups;
  const int m = blockIdx.x / (Hkv * kGroups);
  const int32_t* plan = p.dq_plan;
  if (m >= plan[2]) return;
  const int32_t* count = plan + 4;
  const int32_t* sbase = count + n_tiles;
  const int32_t* multi_tile = sbase + n_tiles + 2 * int64_t(cap);
  const int t = multi_tile[m];
  const int c = count[t], s0 = sbase[t];
  const int k = threadIdx.x >> 6;  // lane group: pieces [c k / 4, c (k + 1) / 4)
  const int li = threadIdx.x & 63;
  const int c4 = (li & 31) * 4;     // dims c4 .. c4 + 3 of rows 2 i + li / 32 (i < 4)
  const int64_t n_rows = int64_t(p.n_blocks) * p.block_size * G;
  const int64_t rbase = int64_t(t) * QROWS + rg * RED_ROWS;
  f32x4v acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4v{0.f, 0.f, 0.f, 0.f};
  const int j0 = c * k / RED_SPLIT, j1 = c * (k + 1) / RED_SPLIT;
  for (int j = j0; j < j1; ++j) {
    const float* src = p.dq_part + ((int64_t(s0 + j) * Hkv + g) * QROWS + rg * RED_ROWS) * D + c4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 2 * i + (li >> 5);
      if (rbase + row < n_rows)
        acc[i] += __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(src + row * D));
    }
  }
  if (k > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s_part[k - 1][i][li] = acc[i];
  }
  __syncthreads();
  if (k > 0) return;
#pragma unroll
  for (int q = 0; q < RED_SPLIT - 1; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += s_part[q][i][li];
  const float sc = p.scale;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = rbase + 2 * i + (li >> 5);
    if (r >= n_rows) continue;
    const int64_t qi = r / G;
    const int h = g * G + int(r % G);
    *reinterpret_cast<float4*>(p.dq + (qi * Hq + h) * D + c4) =
        make_float4(acc[i].x * sc, acc[i].y * sc, acc[i].z * sc, acc[i].w * sc);
  }
}

}  // namespace


hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream) {
  const int64_t n_q = int64_t(p.n_blocks) * p.block_size;
  const int64_t n_rows = n_q * p.n_q_heads;
  const int64_t n_ctx_tiles = (p.n_local + KV_KEYS - 1) / KV_KEYS;
  const DqLayout l = bwd_dq_layout(p.n_blocks, p.block_size, p.n_q_heads, p.n_kv_heads);
  const int64_t target = (kDqTargetWgs + p.n_kv_heads - 1) / p.n_kv_heads;
  const int64_t q_grid = l.cap * p.n_kv_heads;
  if (q_grid > 0x7fffffff || l.cap > 0x7fffffff || l.n_tiles > 0x7fffffff)
    return hipErrorInvalidValue;
  {
    const int64_t plan_wgs = l.n_tiles > 0 ? 1 : 0;
    const int64_t delta_wgs = (n_rows + (THREADS / 32) - 1) / (THREADS / 32);
    const int64_t seen_wgs = (n_ctx_tiles + THREADS - 1) / THREADS;
    const int64_t grid = plan_wgs + seen_wgs + delta_wgs;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (grid > 0) {
      hipLaunchKernelGGL(bwd_delta_kernel, dim3(unsigned(grid)), dim3(THREADS), 0, stream, p,
                         n_rows, int(plan_wgs), int(seen_wgs), int(n_ctx_tiles), int(l.n_tiles),
                         int(l.cap), int(target));
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  const int self_tiles = (p.block_size + KV_KEYS - 1) / KV_KEYS;
  const int64_t kv_grid =
      (n_ctx_tiles + (p.has_self ? int64_t(p.n_blocks) * self_tiles : 0)) * p.n_kv_heads;
  if (kv_grid > 0x7fffffff) return hipErrorInvalidValue;
  if (kv_grid > 0) {
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(unsigned(kv_grid)), dim3(THREADS), 0, stream, p,
                       int(n_ctx_tiles), self_tiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (l.n_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_dq_kernel, dim3(unsigned(q_grid)), dim3(THREADS), 0, stream, p,
                     int(l.n_tiles), int(l.cap));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dq_reduce_kernel,
                     dim3(unsigned(l.n_tiles * p.n_kv_heads * (QROWS / RED_ROWS))), dim3(THREADS),
                     0, stream, p, int(l.n_tiles), int(l.cap));
  return hipGetLastError();
}

}  // namespace bsx
