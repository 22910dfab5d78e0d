// Internal declarations shared by the host API (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace bsx {

// One KV chunk as the kernels see it: packed positions [start, start + len) stored
// at local rows [local_off, local_off + len) of the local K/V buffer.
struct ChunkEntry {
  int64_t start;
  uint32_t len;
  uint32_t local_off;
};

// A small host-built table passed by value in the kernel arguments, so a launch
// needs no separate copy.  Tables larger than kInlineBytes live in the caller's
// workspace instead (`dev` non-null), filled by launch_upload on the same stream.
constexpr int kInlineBytes = 2816;
struct ChunkTable {
  const char* dev;
  uint32_t words[kInlineBytes / 4];
#ifdef __HIPCC__
  __device__ const char* base() const {
    return dev ? dev : reinterpret_cast<const char*>(words);
  }
#endif
};

// bf16 forward work decomposition: one workgroup per (kFwdRows query rows of a KV
// head, KV head, slot), keys visited in tiles of kFwdKeyTile; workgroup i runs on
// XCD i % kXcds (MI355X dispatches workgroups round-robin over its 8 XCDs).
constexpr int kFwdRows = 128;
constexpr int kFwdKeyTile = 64;
constexpr int kXcds = 8;
// (KV head, slot) pair that XCD x runs in round `round` of the natural launch order:
// rounds alternate direction over the XCDs, so a run of pairs whose work falls (or
// rises) with the pair index, such as LPT bins filled heaviest first, is spread
// evenly over the XCDs instead of piling its heavier half onto half of them.
__host__ __device__ inline int pair_of_xcd_round(int round, int xcd) {
  return round * kXcds + ((round & 1) ? kXcds - 1 - xcd : xcd);
}
// The launch-order pass handles at most this many (row tile, output slot) items.
constexpr int kOrderMaxItems = 32768;
// Launches with fewer (KV head, slot) pairs than XCDs and fewer items than this may
// split long items into pieces (about kSplitTargetPieces in all) that the piece
// merge combines.
constexpr int kSplitMaxItems = 1024;
constexpr int kSplitTargetPieces = 1536;
constexpr int kSplitMinPieceTiles = 16;

// Forward problem as handed to the kernels.  The table holds slot_ptr[n_slots + 1]
// (int32) at byte 0 and the non-empty chunks grouped by slot, in chunk index order,
// at byte entries_off: slot s owns entries [slot_ptr[s], slot_ptr[s + 1]).
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* k_self;
  const void* v_self;
  const int64_t* anchor;
  const int64_t* ctx_begin;
  float* o_part;
  float* lse_part;
  int64_t ctx_len;
  int64_t n_local;
  int32_t n_blocks;
  int32_t block_size;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t n_slots;    // context slots; the self slot, when present, is index n_slots
  int32_t has_self;
  float scale;        // softmax scale
  float scale_log2;   // scale * log2(e)
  uint32_t entries_off;
  // order of each slot's chunk entries: 0 any, 1 sorted by start, 2 sorted and
  // disjoint (so their ends increase too)
  int32_t entries_order;
  const int32_t* order;  // bf16 launch order (workgroup -> item), or null: natural order
  // split launches (order pass output, else null): piece index per workgroup, and
  // split[0] = tiles per piece P, split[4 + code] = first partial slot of item `code`
  // (-1: not split); pieces of split items write normalized partials to part_o
  // [slot][kFwdRows][head_dim] and part_lse [slot][kFwdRows]
  const int32_t* piece;
  const int32_t* split;
  float* part_o;
  float* part_lse;
  ChunkTable table;
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* k_self;
  const void* v_self;
  const float* o;
  const float* lse;
  const void* d_o;
  const int64_t* anchor;
  const int64_t* ctx_begin;
  float* dq;
  float* dk;
  float* dv;
  float* dk_self;
  float* dv_self;
  float* stats;               // workspace [N_q][H_q][2]: log2-domain LSE, rowsum(dO * O)
  // workspace [ceil(n_local / 64)]: 1 when some draft block sees a key of the 64-key
  // local tile, else 0 (written by the first backward kernel)
  int32_t* tile_seen;
  int32_t* dq_plan;           // workspace: dQ work split (bwd_dq_layout)
  float* dq_part;             // workspace: partial dQ of split row tiles
  int64_t ctx_len;
  int64_t n_local;
  int32_t n_entries;
  // the chunk list's order: 0 any, 1 sorted by start, 2 sorted and disjoint
  int32_t entries_order;
  int32_t n_blocks;
  int32_t block_size;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t has_self;
  float scale;
  float scale_log2;
  ChunkTable table;           // every non-empty chunk, in chunk index order
};

struct CostParams {
  const int64_t* anchor;
  const int64_t* ctx_begin;
  int64_t* counts;          // may be null
  int64_t* chunk_cost;
  int32_t* mask_err;
  int64_t ctx_len;
  int32_t n_blocks;
  int32_t block_size;
  int32_t n_chunks;
  ChunkTable table;         // ChunkEntry per chunk, every chunk, in index order
  // Launches with many blocks split them into groups of `span` blocks (gridDim.y groups):
  // each group writes its chunk sums to part[group][n_chunks] and its mask flag to
  // bad[group], and a second pass adds them.  Null when one group covers every block.
  int64_t* part;
  int32_t* bad;
  int32_t span;
};
// Workgroups the cost launch aims for when it splits the blocks into groups.
constexpr int kCostTargetWgs = 2048;
// Most block groups a launch over n_chunks chunks uses (sizes its workspace).
inline int32_t cost_max_groups(int32_t n_chunks) {
  const int32_t n_cg = n_chunks > 64 ? (n_chunks + 63) / 64 : 1;
  return (kCostTargetWgs + n_cg - 1) / n_cg;
}

// Largest payload one upload launch carries in its kernel arguments.
constexpr int kUploadWords = kInlineBytes / 4;

hipError_t launch_upload(const uint32_t* host_words, size_t n_words, uint32_t* dst,
                         hipStream_t stream);
hipError_t launch_cost(const CostParams& p, hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream);
// Workgroups of the bf16 forward launch (the length of its launch-order array).
int64_t fwd_bf16_grid(int32_t n_blocks, int32_t block_size, int32_t n_q_heads,
                      int32_t n_kv_heads, int32_t n_out);
// Forward launch layout when items may be split (else split_capable is false):
// the grid, and the workspace of the order pass's split tables and the partials.
struct FwdSplitLayout {
  bool split_capable;
  int64_t grid;           // workgroups: items + kSplitTargetPieces
  int64_t n_codes;        // item codes: pairs x row tiles
  int64_t part_slots;     // partial slots of split items
  size_t piece_bytes;     // int32 [grid]
  size_t split_bytes;     // int32: header[4], sbase[n_codes], pcount[n_codes], list[n_codes]
  size_t part_o_bytes;    // f32 [part_slots][kFwdRows][128]
  size_t part_lse_bytes;  // f32 [part_slots][kFwdRows]
};
FwdSplitLayout fwd_split_layout(int32_t n_blocks, int32_t block_size, int32_t n_q_heads,
                                int32_t n_kv_heads, int32_t n_out);
// Fills `order` (grid entries) with the forward's workgroup -> item map, heaviest
// first (within each XCD when pairs keep their XCD); with p.piece/p.split non-null
// (split launches) also the pieces and split tables.  p.order is ignored.
hipError_t launch_fwd_order(const FwdParams& p, int32_t* order, hipStream_t stream);
// Combines the pieces of each split item into o_part / lse_part (split launches).
hipError_t launch_fwd_piece_merge(const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);
// Partials one merge pass weighs at once; a bf16 merged output needs a single pass.
constexpr int kMergeBf16MaxParts = 128;
hipError_t launch_lse_merge(int32_t n_parts, int64_t n_rows, int32_t head_dim,
                            const float* o_parts, const float* lse_parts, bool out_bf16,
                            void* o_out, float* lse_out, hipStream_t stream);
// dQ work split: the row tiles (kDqRows query rows of one KV head) are cut into
// pieces of P key tiles, P chosen so the launch has about kDqTargetWgs workgroups:
// about 1.75 rounds of the chip's 512 dQ workgroup slots (two per CU).  Fewer, longer
// pieces pay fewer workgroup prologues and leave fewer partials to write and reduce;
// a count just past a whole number of rounds leaves a thin last round.
constexpr int kDqRows = 128;
constexpr int kDqTargetWgs = 896;
constexpr int kDqMinPieceTiles = 8;
struct DqLayout {
  int64_t n_tiles;        // row tiles per KV head
  int64_t cap;            // bound on the number of pieces
  int64_t part_slots;     // bound on the pieces of split row tiles
  size_t plan_bytes;      // int32: header[4], count[n_tiles], sbase[n_tiles],
                          // piece_tile[cap], piece_j[cap], multi_tile[n_tiles]
  size_t part_bytes;      // f32: part_slots x H_kv x kDqRows x 128
};
DqLayout bwd_dq_layout(int32_t n_blocks, int32_t block_size, int32_t n_q_heads,
                       int32_t n_kv_heads);
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream);

// The current device's copy of the no-allocation scratch array (BSX_NOALLOC_SCRATCH_BYTES,
// 256-byte aligned), its address looked up once per device; null with *err set when the
// device or the lookup fails.
void* noalloc_scratch(hipError_t* err);

}  // namespace bsx
