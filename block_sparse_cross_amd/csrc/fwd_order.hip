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
// XCD's L2).  The order changes no result, only the schedule.
//
// One workgroup of 1024 threads: per-(row tile, slot) tile counts go to LDS, then a
// counting sort on the clamped count per XCD (one LDS histogram per wave, so atomics
// meet only within a wave; suffix sums; scatter; equal counts keep no particular order).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "bsx_internal.h"
#include "fwd_common.h"

namespace bsx {
namespace {

constexpr int kThreads = 1024;
constexpr int kKeys = 64;   // sort key: 0 = no item, else 1 + min(tiles, 62)
constexpr int kWaves = kThreads / 64;
constexpr int kTableLdsWords = 4096;  // chunk tables up to 16 KiB are read from LDS

__global__ __launch_bounds__(kThreads) void fwd_order_kernel(FwdParams, int32_t* order,
                                                             int n_tiles, int n_pairs) {
  const BSX_KARG FwdParams& p = kernel_arg0<FwdParams>();
  __shared__ uint16_t work[kOrderMaxItems];
  __shared__ int32_t pos[kXcds][kKeys][kWaves];
  const int tid = threadIdx.x;
  const int n_out = p.n_slots + p.has_self;
  const int G = p.n_q_heads / p.n_kv_heads;
  const int64_t n_rows = int64_t(p.n_blocks) * p.block_size * G;
  __shared__ __attribute__((aligned(16))) uint32_t s_table[kTableLdsWords];
  // the chunk table, copied to LDS when it fits: every lane walks it below
  const char* table = p.table.dev ? p.table.dev : (const char*)(p.table.words);
  const int64_t table_bytes =
      p.entries_off + int64_t(reinterpret_cast<const int32_t*>(table)[p.n_slots]) * 16;
  if (table_bytes <= int64_t(sizeof(s_table))) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(table);
    for (int i = tid; i < int(table_bytes / 4); i += kThreads) s_table[i] = src[i];
    __syncthreads();
    table = reinterpret_cast<const char*>(s_table);
  }
  const int32_t* slot_ptr = reinterpret_cast<const int32_t*>(table);
  const ChunkEntry* ent = reinterpret_cast<const ChunkEntry*>(table + p.entries_off);

  // ---- key tiles visited by each (row tile, slot) item
  const int n_items = n_tiles * n_out;
  for (int it = tid; it < n_items; it += kThreads) {
    const int tile = it / n_out, slot = it % n_out;
    const bool is_self = p.has_self && slot == p.n_slots;
    const int64_t r0 = int64_t(tile) * kFwdRows;
    const int64_t r1 = r0 + kFwdRows < n_rows ? r0 + kFwdRows : n_rows;
    int64_t mlo, mhi;
    row_span_union(p.anchor, p.ctx_begin, p.ctx_len, p.block_size, G, is_self, r0, r1, &mlo, &mhi);
    int64_t tiles = 0;
    if (mlo < mhi)
      tiles = is_self ? (mhi - mlo + kFwdKeyTile - 1) / kFwdKeyTile
                      : walk_tiles(ent, slot_ptr[slot], slot_ptr[slot + 1], mlo, mhi, kFwdKeyTile);
    work[it] = uint16_t(tiles < 0xffff ? tiles : 0xffff);
  }
  __syncthreads();

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
    const int pair = per_xcd_lists ? (j / n_tiles) * kXcds + xcd : j / n_tiles;
    const int tile = n_tiles - 1 - j % n_tiles;
    if (pair >= n_pairs) {
      *code = -1;
      return 0;
    }
    *code = pair * n_tiles + tile;
    const int w = work[tile * n_out + pair / p.n_kv_heads];
    return 1 + (w < kKeys - 2 ? w : kKeys - 2);
  };
  static_assert(kKeys == 64, "one key per lane in the prefix pass");
  const int wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < kXcds * kKeys * kWaves; i += kThreads) (&pos[0][0][0])[i] = 0;
  __syncthreads();
  for (int bid = tid; bid < n_bids; bid += kThreads) {
    int code;
    const int key = key_of(bid, &code);
    atomicAdd(&pos[bid % nx][key][wave], 1);
  }
  __syncthreads();
  if (wave < nx) {
    const int x = wave, key = kKeys - 1 - lane;
    int own = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) own += pos[x][key][w];
    int incl = own;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    int acc = incl - own;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int c = pos[x][key][w];
      pos[x][key][w] = acc;
      acc += c;
    }
  }
  __syncthreads();
  for (int bid = tid; bid < n_bids; bid += kThreads) {
    int code;
    const int key = key_of(bid, &code);
    const int x = bid % nx;
    const int at = atomicAdd(&pos[x][key][wave], 1);
    order[at * nx + x] = code;
  }
}

}  // namespace

hipError_t launch_fwd_order(const FwdParams& p, int32_t* order, hipStream_t stream) {
  const int G = p.n_q_heads / p.n_kv_heads;
  const int64_t n_rows = int64_t(p.n_blocks) * p.block_size * G;
  const int64_t n_tiles = (n_rows + kFwdRows - 1) / kFwdRows;
  const int64_t n_out = int64_t(p.n_slots) + p.has_self;
  if (n_tiles * n_out > kOrderMaxItems) return hipErrorInvalidValue;
  const int64_t n_pairs = int64_t(p.n_kv_heads) * n_out;
  if (fwd_bf16_grid(p.n_blocks, p.block_size, p.n_q_heads, p.n_kv_heads, int32_t(n_out)) >
      0x7fffffff)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(fwd_order_kernel, dim3(1), dim3(kThreads), 0, stream, p, order,
                     int(n_tiles), int(n_pairs));
  return hipGetLastError();
}

}  // namespace bsx
