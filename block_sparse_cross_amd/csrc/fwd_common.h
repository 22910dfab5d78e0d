// Device helpers shared by the forward attention kernels: the visibility rule
// and the walk over a slot's key segments.
//
// Visibility (Split-KV page, Abstract: anchor-sampled draft blocks cross-attend
// the context under a block-sparse mask): the queries of block b see the context
// positions [ctx_begin[b], anchor[b]) and the B keys of their own draft block.
// In the self slot, "positions" are draft-key rows, so block b sees [b*B, b*B+B).
#pragma once

#include <hip/hip_runtime.h>

#include "bsx_internal.h"

namespace bsx {

// The kernel's first argument, read in place from the kernarg segment (where it
// sits at offset 0) through a constant-address-space reference: its fields load
// with scalar instructions as wave-uniform values.  Naming the by-value parameter
// instead would make the compiler copy the whole struct, inline chunk table
// included, to scratch.
#if defined(__HIP_DEVICE_COMPILE__)
#define BSX_KARG __attribute__((address_space(4)))
#else
#define BSX_KARG
#endif
template <typename T>
__device__ inline const BSX_KARG T& kernel_arg0() {
#if defined(__HIP_DEVICE_COMPILE__)
  return *(const BSX_KARG T*)__builtin_amdgcn_kernarg_segment_ptr();
#else
  return *static_cast<const T*>(nullptr);  // host pass: never executed
#endif
}

// Wave-uniform copies of values read through a generic pointer (chunk tables live
// either in the kernarg segment or in device memory, so the compiler cannot prove
// their loads uniform; descriptors built from them must be scalar).
__device__ inline int32_t uniform32(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline int64_t uniform_i64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x)));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x) >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

// Visible range of block `blk` in the slot's position space, clamped to [0, S].
__device__ inline void visible_range(const int64_t* anchor, const int64_t* ctx_begin,
                                     int64_t S, int block_size, bool self_slot, int64_t blk,
                                     int64_t* lo, int64_t* hi) {
  if (self_slot) {
    *lo = blk * block_size;
    *hi = *lo + block_size;
    return;
  }
  int64_t a = ctx_begin[blk], z = anchor[blk];
  a = a < 0 ? 0 : (a > S ? S : a);
  z = z < a ? a : (z > S ? S : z);
  *lo = a;
  *hi = z;
}

// Union [*mlo, *mhi) of the visible ranges of the query rows [r0, r1) of one KV
// head (row r is query r / G), per lane (no wave-uniform assumption); empty when no
// row sees anything (*mlo >= *mhi).
__device__ inline void row_span_union(const int64_t* anchor, const int64_t* ctx_begin, int64_t S,
                                      int block_size, int G, bool self_slot, int64_t r0,
                                      int64_t r1, int64_t* mlo, int64_t* mhi) {
  *mlo = INT64_MAX;
  *mhi = INT64_MIN;
  const int64_t b0 = r0 / G / block_size, b1 = (r1 - 1) / G / block_size;
  for (int64_t b = b0; b <= b1; ++b) {
    int64_t lo, hi;
    visible_range(anchor, ctx_begin, S, block_size, self_slot, b, &lo, &hi);
    if (lo < hi) {
      *mlo = lo < *mlo ? lo : *mlo;
      *mhi = hi > *mhi ? hi : *mhi;
    }
  }
}

// Key tiles of `key_tile` positions a walk over entries [e0, e1) cut to [mlo, mhi)
// visits (each segment is tiled from its first position), per lane.
__device__ inline int64_t walk_tiles(const ChunkEntry* ent, int e0, int e1, int64_t mlo,
                                     int64_t mhi, int key_tile) {
  int64_t tiles = 0;
  if (!(mlo < mhi)) return 0;
  for (int e = e0; e < e1; ++e) {
    const int64_t a = ent[e].start > mlo ? ent[e].start : mlo;
    const int64_t end = ent[e].start + int64_t(ent[e].len);
    const int64_t z = end < mhi ? end : mhi;
    if (a < z) tiles += (z - a + key_tile - 1) / key_tile;
  }
  return tiles;
}

// Walks the key segments a workgroup must visit for one slot: each segment is a
// run of positions [seg0, seg1) stored at local rows local0 .. local0 + (seg1 - seg0),
// already cut to the union [minlo, maxhi) of the ranges its rows can see.
// The walk reads the chunk table through constant-address-space pointers: the table
// is not written while a kernel walks it, and its entry reads (wave-uniform) become
// scalar loads, which wait for nothing but themselves (through a generic pointer
// they are flat loads, and waiting for one waits for every load in flight).
typedef const __attribute__((address_space(4))) char* ConstBytes;
typedef const __attribute__((address_space(4))) int32_t* ConstI32s;
typedef const __attribute__((address_space(4))) ChunkEntry* ConstEntries;
__device__ inline ConstBytes const_bytes(const void* ptr) {
  return reinterpret_cast<ConstBytes>(reinterpret_cast<uintptr_t>(ptr));
}

struct SegmentWalk {
  ConstEntries ent;
  int e;
  int e_end;
  int64_t minlo;
  int64_t maxhi;
  bool self_slot;
  bool sorted;  // entries sorted by start: the walk ends at the first start >= maxhi
  int64_t seg0;
  int64_t seg1;
  int64_t local0;

  // table: slot_ptr (int32) at byte 0, ChunkEntry list at entries_off; order: the
  // order of each slot's entries (0 any, 1 sorted by start, 2 sorted and disjoint)
  __device__ void init(const void* table_ptr, uint32_t entries_off, int slot, bool is_self,
                       int64_t lo, int64_t hi, int order = 0) {
    self_slot = is_self;
    minlo = lo;
    maxhi = hi;
    sorted = order >= 1;
    if (is_self) {
      ent = nullptr;
      e = 0;
      e_end = 1;
    } else {
      const ConstBytes table = const_bytes(table_ptr);
      const ConstI32s slot_ptr = reinterpret_cast<ConstI32s>(table);
      ent = reinterpret_cast<ConstEntries>(table + entries_off);
      e = uniform32(slot_ptr[slot]);
      e_end = uniform32(slot_ptr[slot + 1]);
      if (order >= 2) skip_to_first();
    }
  }

  // entry fields, wave-uniform
  __device__ int64_t start_of(int i) const { return uniform_i64(ent[i].start); }
  __device__ int64_t len_of(int i) const {
    return int64_t(uniform32(int32_t(ent[i].len))) & 0xffffffffll;
  }

  // Disjoint entries sorted by start: their ends increase too, so the first entry that
  // ends after minlo is found by bisection.
  __device__ void skip_to_first() {
    int a = e, b = e_end;
    while (a < b) {
      const int mid = (a + b) >> 1;
      if (start_of(mid) + len_of(mid) > minlo)
        b = mid;
      else
        a = mid + 1;
    }
    e = a;
  }

  // Walks entries [e0, e1) of an explicit list (all chunks, for the backward pass);
  // order as for init.
  __device__ void init_range(const ChunkEntry* list, int e0, int e1, int64_t lo, int64_t hi,
                             int order = 0) {
    self_slot = false;
    sorted = order >= 1;
    minlo = lo;
    maxhi = hi;
    ent = reinterpret_cast<ConstEntries>(const_bytes(list));
    e = e0;
    e_end = e1;
    if (order >= 2) skip_to_first();
  }

  // Advances to the next non-empty segment; false when the slot is exhausted.
  __device__ bool next() {
    if (self_slot) {
      if (e >= e_end) return false;
      e = e_end;
      seg0 = minlo;
      seg1 = maxhi;
      local0 = minlo;
      return seg0 < seg1;
    }
    while (e < e_end) {
      const int i = e++;
      const int64_t start = start_of(i);
      if (sorted && start >= maxhi) {  // no later entry reaches the range
        e = e_end;
        return false;
      }
      const int64_t len = len_of(i);
      const int64_t loff = int64_t(uniform32(int32_t(ent[i].local_off))) & 0xffffffffll;
      const int64_t a = start > minlo ? start : minlo;
      const int64_t z = start + len < maxhi ? start + len : maxhi;
      if (a < z) {
        seg0 = a;
        seg1 = z;
        local0 = loff + (a - start);
        return true;
      }
    }
    return false;
  }
};


}  // namespace bsx
