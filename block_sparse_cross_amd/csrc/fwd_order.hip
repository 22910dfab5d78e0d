// Launch order of the bf16 forward: heaviest work items first.
//
// A forward item (kFwdRows query rows of one KV head, one output slot) visits a
// data-dependent number of key tiles: the slot's chunks cut to the union of the
// rows' visible ranges (Split-KV page, Abstract: realized per-chunk cost under the
// block-sparse mask).  Items vary from zero to all of a slot's tiles, so the
// natural launch order leaves the last round of workgroups running on a fraction
// of the chip.  This pass counts each item's tiles and sorts the workgroups of
// each XCD by that count, largest first (longest-processing-time order), keeping
// every item on the XCD the natural order gives it (its slot's K/V stays in that
// XCD's L2).  Items that visit no tile come last and are marked, so their
// workgroups skip straight to writing an empty partial.  The order changes no result,
// only the schedule.
//
// One workgroup of 1024 threads per sorted list (one list per XCD, or one list when
// items go round-robin over the XCDs): every workgroup counts the per-(row tile,
// slot) tiles into LDS, then counting-sorts its list's slots on the clamped count
// (one LDS histogram per wave, so atomics meet only within a wave; suffix sums;
// scatter; equal counts keep no particular order).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "bsx_internal.h"
#include "fwd_common.h"

namespace bsx {
namespace {

constexpr int kThreads = 1024;
static_assert(sizeof(ChunkEntry) == 16 && offsetof(ChunkEntry, len) == 8,
              "chunk entries are read as four words: start (two), len, local offset");
constexpr int kKeys = 64;   // sort key: 0 = no item, else 1 + min(tiles, 62)
constexpr int kWaves = kThreads / 64;
constexpr int kTableLdsWords = 4096;  // chunk tables up to 16 KiB are read from LDS
constexpr int kRangeLdsBlocks = 1024;  // block ranges of launches up to this size, too

__global__ __launch_bounds__(kThreads) void fwd_order_kernel(FwdParams, int32_t* order,
                                                             int n_tiles, int n_pairs, int grid) {
  const BSX_KARG FwdParams& p = kernel_arg0<FwdParams>();
  __shared__ uint16_t work[kOrderMaxItems];
  // exact tile counts of split launches (at most kSplitMaxItems items): pieces are cut
  // from these, so they must not saturate like the 16-bit sort keys above
  __shared__ int32_t work_exact[kSplitMaxItems];
  __shared__ int32_t pos[1][kKeys][kWaves];
  const int tid = threadIdx.x;
  const int n_out = p.n_slots + p.has_self;
  const int G = p.n_q_heads / p.n_kv_heads;
  const int64_t n_rows = int64_t(p.n_blocks) * p.block_size * G;
  __shared__ __attribute__((aligned(16))) uint32_t s_table[kTableLdsWords];
  __shared__ int64_t s_blo[kRangeLdsBlocks], s_bhi[kRangeLdsBlocks];
  // the chunk table and every block's visible range, copied to LDS when they fit (one
  // round trip; every lane walks them below)
  // (a table in the kernel arguments is copied whole, so the copy need not wait for
  // the entry count: one round trip instead of two)
  const char* table = p.table.dev ? p.table.dev : (const char*)(p.table.words);
  static_assert(kInlineBytes <= int(sizeof(s_table)), "an inline table fits the LDS copy");
  const int64_t table_bytes =
      p.table.dev ? p.entries_off + int64_t(reinterpret_cast<const int32_t*>(table)[p.n_slots]) * 16
                  : kInlineBytes;
  const bool lds_table = table_bytes <= int64_t(sizeof(s_table));
  const bool lds_ranges = p.n_blocks <= kRangeLdsBlocks;
  if (lds_table) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(table);
    for (int i = tid; i < int(table_bytes / 4); i += kThreads) s_table[i] = src[i];
  }
  if (lds_ranges) {
    for (int b = tid; b < p.n_blocks; b += kThreads)
      visible_range(p.anchor, p.ctx_begin, p.ctx_len, p.block_size, false, b, &s_blo[b], &s_bhi[b]);
  }
  if (lds_table || lds_ranges) __syncthreads();
  if (lds_table) table = reinterpret_cast<const char*>(s_table);
  const int32_t* slot_ptr = reinterpret_cast<const int32_t*>(table);
  const ChunkEntry* ent = reinterpret_cast<const ChunkEntry*>(table + p.entries_off);

  // ---- key tiles visited by each (row tile, slot) item
  const int n_items = n_tiles * n_out;
  for (int it = tid; it < n_items; it += kThreads) {
    const int tile = it / n_out, slot = it % n_out;
    const bool is_self = p.has_self && slot == p.n_slots;
    const int64_t r0 = int64_t(tile) * kFwdRows;
    const int64_t r1 = r0 + kFwdRows < n_rows ? r0 + kFwdRows : n_rows;
    int64_t mlo = INT64_MAX, mhi = INT64_MIN;
    if (lds_ranges && !is_self) {
      // the union of the ranges of the blocks of rows [r0, r1), from LDS
      const int64_t b0 = r0 / G / p.block_size, b1 = (r1 - 1) / G / p.block_size;
      for (int64_t b = b0; b <= b1; ++b) {
        if (s_blo[b] < s_bhi[b]) {
          mlo = s_blo[b] < mlo ? s_blo[b] : mlo;
          mhi = s_bhi[b] > mhi ? s_bhi[b] : mhi;
        }
      }
    } else {
      row_span_union(p.anchor, p.ctx_begin, p.ctx_len, p.block_size, G, is_self, r0, r1, &mlo,
                     &mhi);
    }
    int64_t tiles = 0;
    if (mlo < mhi) {
      if (is_self) {
        tiles = (mhi - mlo + kFwdKeyTile - 1) / kFwdKeyTile;
      } else if (lds_table) {
        // the same walk, reading the LDS copy through the LDS array itself (through the
        // generic table pointer every entry would be a flat load)
        int e0 = int(s_table[slot]);
        const int e1 = int(s_table[slot + 1]);
        const uint32_t* w = s_table + p.entries_off / 4;
        auto start_of = [&](int e) {
          return int64_t(uint64_t(w[4 * e]) | (uint64_t(w[4 * e + 1]) << 32));
        };
        if (p.entries_order >= 2) {  // disjoint and sorted: bisect to the first entry ending after mlo
          int b = e1;
          while (e0 < b) {
            const int mid = (e0 + b) >> 1;
            if (start_of(mid) + int64_t(w[4 * mid + 2]) > mlo)
              b = mid;
            else
              e0 = mid + 1;
          }
        }
        for (int e = e0; e < e1; ++e) {
          const int64_t start = start_of(e);
          if (p.entries_order >= 1 && start >= mhi) break;  // sorted: no later entry reaches mhi
          const int64_t a = start > mlo ? start : mlo;
          const int64_t end = start + int64_t(w[4 * e + 2]);
          const int64_t z = end < mhi ? end : mhi;
          if (a < z) tiles += (z - a + kFwdKeyTile - 1) / kFwdKeyTile;
        }
      } else {
        tiles = walk_tiles(ent, slot_ptr[slot], slot_ptr[slot + 1], mlo, mhi, kFwdKeyTile);
      }
    }
    work[it] = uint16_t(tiles < 0xffff ? tiles : 0xffff);
    // a local buffer below 2^32 keys has below 2^26 tiles: the count fits int32
    if (p.split && it < kSplitMaxItems) work_exact[it] = int32_t(tiles);
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  if (p.split) {
    if (blockIdx.x > 0) return;  // (launched with one workgroup)
    // ---- split launch (fewer pairs than XCDs, at most kThreads items): thread c owns
    // item c = pair * n_tiles + tile.  P = max(min tiles, ceil(sum / target)); an item
    // of w > P tiles becomes ceil(w / P) pieces, each of P tiles but the last.
    __shared__ int64_t s_sum[kThreads];
    __shared__ int s_scan[3][kThreads];
    int32_t* piece = const_cast<int32_t*>(p.piece);
    int32_t* split = const_cast<int32_t*>(p.split);
    const int n_codes = n_pairs * n_tiles;
    const int c = tid;
    int w = 0;
    if (c < n_codes) w = work_exact[(c % n_tiles) * n_out + (c / n_tiles) / p.n_kv_heads];
    s_sum[tid] = w;
    __syncthreads();
    for (int off = kThreads / 2; off > 0; off >>= 1) {
      if (tid < off) s_sum[tid] += s_sum[tid + off];
      __syncthreads();
    }
    int64_t P = (s_sum[0] + kSplitTargetPieces - 1) / kSplitTargetPieces;
    P = P < kSplitMinPieceTiles ? kSplitMinPieceTiles : P;
    const int pc = c < n_codes ? (w > P ? int((w + P - 1) / P) : 1) : 0;
    const int own[3] = {pc, pc > 1 ? pc : 0, pc > 1 ? 1 : 0};
    for (int k = 0; k < 3; ++k) s_scan[k][tid] = own[k];
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      int v[3];
      for (int k = 0; k < 3; ++k) v[k] = tid >= off ? s_scan[k][tid - off] : 0;
      __syncthreads();
      for (int k = 0; k < 3; ++k) s_scan[k][tid] += v[k];
      __syncthreads();
    }
    const int slot0 = s_scan[1][tid] - own[1], list_at = s_scan[2][tid] - own[2];
    if (c < n_codes) {
      split[4 + c] = pc > 1 ? slot0 : -1;
      split[4 + n_codes + c] = pc;
      if (pc > 1) split[4 + 2 * n_codes + list_at] = c;
    }
    const int total = s_scan[0][kThreads - 1];
    if (tid == 0) {
      split[0] = int32_t(P);
      split[1] = total;
      split[2] = s_scan[2][kThreads - 1];
      split[3] = 0;
    }
    // counting sort of the pieces by their tile count, longest first (one list)
    auto piece_key = [&](int j) {
      const int64_t pw = pc > 1 ? (w - int64_t(j) * P < P ? w - int64_t(j) * P : P) : w;
      return 1 + int(pw < kKeys - 2 ? pw : kKeys - 2);
    };
    for (int i = tid; i < kKeys * kWaves; i += kThreads) (&pos[0][0][0])[i] = 0;
    __syncthreads();
    for (int j = 0; j < pc; ++j) atomicAdd(&pos[0][piece_key(j)][wave], 1);
    __syncthreads();
    if (wave == 0) {
      const int key = kKeys - 1 - lane;
      int sum = 0;
      for (int q = 0; q < kWaves; ++q) sum += pos[0][key][q];
      int incl = sum;
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      int acc = incl - sum;
      for (int q = 0; q < kWaves; ++q) {
        const int cnt = pos[0][key][q];
        pos[0][key][q] = acc;
        acc += cnt;
      }
    }
    __syncthreads();
    for (int j = 0; j < pc; ++j) {
      const int at = atomicAdd(&pos[0][piece_key(j)][wave], 1);
      order[at] = c;
      piece[at] = j;
    }
    for (int i = total + tid; i < grid; i += kThreads) {
      order[i] = -1;
      piece[i] = 0;
    }
    return;
  }

  // ---- workgroup slot bid holds, in the natural order, item (pair, tile) below.  With
  // fewer pairs than XCDs, slots are one list (items round-robin over XCDs, nx = 1);
  // otherwise each XCD's slots are sorted separately (nx = kXcds).
  const bool per_xcd_lists = n_pairs >= kXcds;
  const int nx = per_xcd_lists ? kXcds : 1;
  const int per_xcd = (n_pairs + kXcds - 1) / kXcds;
  const int n_bids = per_xcd_lists ? kXcds * per_xcd * n_tiles : n_pairs * n_tiles;
  auto key_of = [&](int bid, int* code) {
    const int xcd = per_xcd_lists ? bid % kXcds : 0;
    const int j = per_xcd_lists ? bid / kXcds : bid;
    const int pair = per_xcd_lists ? pair_of_xcd_round(j / n_tiles, xcd) : j / n_tiles;
    const int tile = n_tiles - 1 - j % n_tiles;
    if (pair >= n_pairs) {
      *code = -1;
      return 0;
    }
    const int w = work[tile * n_out + pair / p.n_kv_heads];
    // an item that visits no tile is marked (-2 - item): its workgroup only writes the
    // rows' empty-partial LSE
    *code = w > 0 ? pair * n_tiles + tile : -2 - (pair * n_tiles + tile);
    return 1 + (w < kKeys - 2 ? w : kKeys - 2);
  };
  static_assert(kKeys == 64, "one key per lane in the prefix pass");
  // workgroup `list` sorts the slots of XCD list `list` (bid % nx == list)
  const int list = blockIdx.x;
  if (list >= nx) return;
  const int list_len = n_bids / nx;  // n_bids is a multiple of kXcds with per-XCD lists
  for (int i = tid; i < kKeys * kWaves; i += kThreads) (&pos[0][0][0])[i] = 0;
  __syncthreads();
  for (int j = tid; j < list_len; j += kThreads) {
    int code;
    const int key = key_of(j * nx + list, &code);
    atomicAdd(&pos[0][key][wave], 1);
  }
  __syncthreads();
  if (wave == 0) {
    const int key = kKeys - 1 - lane;
    int own = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) own += pos[0][key][w];
    int incl = own;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    int acc = incl - own;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int c = pos[0][key][w];
      pos[0][key][w] = acc;
      acc += c;
    }
  }
  __syncthreads();
  for (int j = tid; j < list_len; j += kThreads) {
    int code;
    const int key = key_of(j * nx + list, &code);
    const int at = atomicAdd(&pos[0][key][wave], 1);
    order[at * nx + list] = code;
  }
}

// ---- combine the pieces of each split item (exact LSE merge of normalized partials):
// LSE = M + log sum_j exp(LSE_j - M), O = sum_j exp(LSE_j - LSE) O_j over pieces with
// finite LSE.  One workgroup per (split item, 32 of its rows); a lane owns 16 columns.
constexpr int kMergeRows = 32;

__global__ __launch_bounds__(256) void fwd_piece_merge_kernel(FwdParams, int n_tiles, int n_codes) {
  const BSX_KARG FwdParams& p = kernel_arg0<FwdParams>();
  const int32_t* split = p.split;
  const int m = blockIdx.x / (kFwdRows / kMergeRows);
  const int rg = blockIdx.x % (kFwdRows / kMergeRows);
  if (m >= split[2]) return;
  const int code = split[4 + 2 * n_codes + m];
  const int pc = split[4 + n_codes + code], sb = split[4 + code];
  const int pair = code / n_tiles, tile = code % n_tiles;
  const int G = p.n_q_heads / p.n_kv_heads;
  const int g = pair % p.n_kv_heads, slot = pair / p.n_kv_heads;
  const int64_t n_q = int64_t(p.n_blocks) * p.block_size;
  const int row = rg * kMergeRows + (threadIdx.x >> 3), d0 = (threadIdx.x & 7) * 16;
  const int64_t r = int64_t(tile) * kFwdRows + row;
  if (r >= n_q * G) return;
  float mx = -INFINITY;
  for (int j = 0; j < pc; ++j) mx = fmaxf(mx, p.part_lse[int64_t(sb + j) * kFwdRows + row]);
  const int64_t qi = r / G;
  const int h = g * G + int(r % G);
  const int64_t orow = (int64_t(slot) * n_q + qi) * p.n_q_heads + h;
  if (mx == -INFINITY) {
    if ((threadIdx.x & 7) == 0) p.lse_part[orow] = -INFINITY;
    return;
  }
  float ssum = 0.f;
  for (int j = 0; j < pc; ++j) {
    const float l = p.part_lse[int64_t(sb + j) * kFwdRows + row];
    if (l != -INFINITY) ssum += expf(l - mx);
  }
  const float lse = mx + logf(ssum);
  float4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < pc; ++j) {
    const float l = p.part_lse[int64_t(sb + j) * kFwdRows + row];
    if (l == -INFINITY) continue;  // an empty piece's O is never read
    const float wgt = expf(l - lse);
    const float* src = p.part_o + (int64_t(sb + j) * kFwdRows + row) * 128 + d0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 x = *reinterpret_cast<const float4*>(src + 4 * i);
      acc[i].x = fmaf(wgt, x.x, acc[i].x);
      acc[i].y = fmaf(wgt, x.y, acc[i].y);
      acc[i].z = fmaf(wgt, x.z, acc[i].z);
      acc[i].w = fmaf(wgt, x.w, acc[i].w);
    }
  }
  float* dst = p.o_part + orow * 128 + d0;
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<float4*>(dst + 4 * i) = acc[i];
  if ((threadIdx.x & 7) == 0) p.lse_part[orow] = lse;
}

}  // namespace


hipError_t launch_fwd_order(const FwdParams& p, int32_t* order, hipStream_t stream) {
  const int G = p.n_q_heads / p.n_kv_heads;
  const int64_t n_rows = int64_t(p.n_blocks) * p.block_size * G;
  const int64_t n_tiles = (n_rows + kFwdRows - 1) / kFwdRows;
  const int64_t n_out = int64_t(p.n_slots) + p.has_self;
  if (n_tiles * n_out > kOrderMaxItems) return hipErrorInvalidValue;
  const int64_t n_pairs = int64_t(p.n_kv_heads) * n_out;
  int64_t grid = fwd_bf16_grid(p.n_blocks, p.block_size, p.n_q_heads, p.n_kv_heads,
                               int32_t(n_out));
  if (p.split) {
    const FwdSplitLayout l = fwd_split_layout(p.n_blocks, p.block_size, p.n_q_heads,
                                              p.n_kv_heads, int32_t(n_out));
    if (!l.split_capable || !p.piece) return hipErrorInvalidValue;
    grid = l.grid;
  }
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  // one workgroup per sorted list: per XCD when pairs keep their XCD, else one
  const int lists = (!p.split && n_pairs >= kXcds) ? kXcds : 1;
  hipLaunchKernelGGL(fwd_order_kernel, dim3(lists), dim3(kThreads), 0, stream, p, order,
                     int(n_tiles), int(n_pairs), int(grid));
  return hipGetLastError();
}

}  // namespace bsx

namespace bsx {

hipError_t launch_fwd_piece_merge(const FwdParams& p, hipStream_t stream) {
  const int64_t n_out = int64_t(p.n_slots) + p.has_self;
  const FwdSplitLayout l = fwd_split_layout(p.n_blocks, p.block_size, p.n_q_heads,
                                            p.n_kv_heads, int32_t(n_out));
  if (!l.split_capable || !p.split) return hipErrorInvalidValue;
  const int G = p.n_q_heads / p.n_kv_heads;
  const int64_t n_tiles = (int64_t(p.n_blocks) * p.block_size * G + kFwdRows - 1) / kFwdRows;
  hipLaunchKernelGGL(fwd_piece_merge_kernel, dim3(unsigned(l.n_codes * (kFwdRows / kMergeRows))),
                     dim3(256), 0, stream, p, int(n_tiles), int(l.n_codes));
  return hipGetLastError();
}

}  // namespace bsx
