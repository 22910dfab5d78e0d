// Host-side launch layouts of the attention kernels: grid sizes and the workspace
// pieces the host reserves for them.  Plain host code (no kernels), so the host
// logic of the library can also be built and checked without a GPU compiler.
#include "bsx_internal.h"

namespace bsx {

int64_t fwd_bf16_grid(int32_t n_blocks, int32_t block_size, int32_t n_q_heads,
                      int32_t n_kv_heads, int32_t n_out) {
  const int64_t n_rows = int64_t(n_blocks) * block_size * (n_q_heads / n_kv_heads);
  const int64_t n_tiles = (n_rows + kFwdRows - 1) / kFwdRows;
  const int64_t n_pairs = int64_t(n_kv_heads) * n_out;
  if (n_pairs < kXcds) return n_pairs * n_tiles;  // round-robin over XCDs
  const int64_t per_xcd = (n_pairs + kXcds - 1) / kXcds;
  return kXcds * per_xcd * n_tiles;
}

FwdSplitLayout fwd_split_layout(int32_t n_blocks, int32_t block_size, int32_t n_q_heads,
                                int32_t n_kv_heads, int32_t n_out) {
  FwdSplitLayout l{};
  if (n_kv_heads < 1 || n_blocks < 1 || block_size < 1 || n_out < 1) return l;
  const int64_t n_rows = int64_t(n_blocks) * block_size * (n_q_heads / n_kv_heads);
  const int64_t n_tiles = (n_rows + kFwdRows - 1) / kFwdRows;
  const int64_t n_pairs = int64_t(n_kv_heads) * n_out;
  l.n_codes = n_pairs * n_tiles;
  l.split_capable = n_pairs < kXcds && l.n_codes <= kSplitMaxItems;
  if (!l.split_capable) return l;
  // sum_i ceil(w_i / P) <= sum_i (w_i / P + 1) <= kSplitTargetPieces + n_codes pieces
  l.grid = l.n_codes + kSplitTargetPieces;
  // pieces of split items: each has w > P, so ceil(w / P) < 2 w / P, summing below 2 x target
  l.part_slots = 2 * int64_t(kSplitTargetPieces);
  l.piece_bytes = sizeof(int32_t) * size_t(l.grid);
  l.split_bytes = sizeof(int32_t) * size_t(4 + 3 * l.n_codes);
  l.part_o_bytes = sizeof(float) * size_t(l.part_slots) * kFwdRows * 128;
  l.part_lse_bytes = sizeof(float) * size_t(l.part_slots) * kFwdRows;
  return l;
}

DqLayout bwd_dq_layout(int32_t n_blocks, int32_t block_size, int32_t n_q_heads,
                       int32_t n_kv_heads) {
  DqLayout l{};
  if (n_kv_heads < 1 || n_blocks < 1 || block_size < 1) return l;
  const int64_t n_rows = int64_t(n_blocks) * block_size * (n_q_heads / n_kv_heads);
  const int64_t target = (kDqTargetWgs + n_kv_heads - 1) / n_kv_heads;
  l.n_tiles = (n_rows + kDqRows - 1) / kDqRows;
  l.cap = target + l.n_tiles;
  l.part_slots = 2 * target < l.cap ? 2 * target : l.cap;
  l.plan_bytes = sizeof(int32_t) * size_t(4 + 3 * l.n_tiles + 2 * l.cap);
  l.part_bytes = sizeof(float) * size_t(l.part_slots) * n_kv_heads * kDqRows * 128;
  return l;
}

}  // namespace bsx
