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
// counting sort on the clamped count per XCD (LDS histogram, suffix sums, scatter
// with LDS atomics; items of equal count keep no particular order).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "bsx_internal.h"
#include "fwd_common.h"

namespace bsx {
namespace {

constexpr int kThreads = 1024;
constexpr int kKeys = 256;  // sort key: 0 = no item, else 1 + min(tiles, 254)

__global__ __launch_bounds__(kThreads) void fwd_order_kernel(FwdParams, int32_t* order,
                                                             int n_tiles, int n_pairs) {
  const BSX_KARG FwdParams& p = kernel_arg0<FwdParams>();
  __shared__ uint16_t work[kOrderMaxItems];
  __shared__ int32_t pos[kXcds][kKeys];
  const int tid = threadIdx.x;
  const int n_out = p.n_slots + p.has_self;
  const int G = p.n_q_heads / p.n_kv_heads;
  const int64_t n_rows = int64_t(p.n_blocks) * p.block_size * G;
  const char* table = p.table.dev ? p.table.dev : (const char*)(p.table.words);
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
  for (int i = tid; i < kXcds * kKeys; i += kThreads) (&pos[0][0])[i] = 0;
  __syncthreads();

  // ---- workgroup slot bid holds, in the natural order, item (pair, tile) below
  const int per_xcd = (n_pairs + kXcds - 1) / kXcds;
  const int64_t n_bids = int64_t(kXcds) * per_xcd * n_tiles;
  auto key_of = [&](int64_t bid, int* code) {
    const int xcd = int(bid % kXcds);
    const int64_t j = bid / kXcds;
    const int pair = int(j / n_tiles) * kXcds + xcd;
    const int tile = n_tiles - 1 - int(j % n_tiles);
    if (pair >= n_pairs) {
      *code = -1;
      return 0;
    }
    *code = pair * n_tiles + tile;
    const int w = work[tile * n_out + pair / p.n_kv_heads];
    return 1 + (w < kKeys - 2 ? w : kKeys - 2);
  };
  for (int64_t bid = tid; bid < n_bids; bid += kThreads) {
    int code;
    const int key = key_of(bid, &code);
    atomicAdd(&pos[bid % kXcds][key], 1);
  }
  __syncthreads();

  // ---- start of each key's run: items with larger keys come first (suffix sums).
  // One wave per XCD; lane l owns keys 255 - 4l .. 252 - 4l.
  static_assert(kKeys == 4 * 64, "one wave of 64 lanes, four keys each");
  if (tid < kXcds * 64) {
    const int x = tid >> 6, l = tid & 63;
    int c[4], own = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = pos[x][kKeys - 1 - (4 * l + q)];
      own += c[q];
    }
    int incl = own;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (l >= off) incl += y;
    }
    int acc = incl - own;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pos[x][kKeys - 1 - (4 * l + q)] = acc;
      acc += c[q];
    }
  }
  __syncthreads();

  for (int64_t bid = tid; bid < n_bids; bid += kThreads) {
    int code;
    const int key = key_of(bid, &code);
    const int x = int(bid % kXcds);
    const int at = atomicAdd(&pos[x][key], 1);
    order[int64_t(at) * kXcds + x] = code;
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
  hipLaunchKernelGGL(fwd_order_kernel, dim3(1), dim3(kThreads), 0, stream, p, order,
                     int(n_tiles), int(n_pairs));
  return hipGetLastError();
}

}  // namespace bsx
