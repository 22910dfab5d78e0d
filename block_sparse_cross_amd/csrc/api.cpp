// Host side of libbsx: argument checks, LPT planning, per-call work descriptors,
// and kernel launches.  Every entry point validates all of its arguments before
// touching the HIP runtime, so argument errors never launch anything.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <numeric>
#include <queue>
#include <string>
#include <vector>

#include "../../include/bsx.h"
#include "bsx_internal.h"

namespace {

// Text of the last error on this thread (a fixed buffer: reporting an error allocates
// nothing).
thread_local char g_last_error[512];

bsx_status fail(bsx_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

bsx_status ok() {
  g_last_error[0] = '\0';
  return BSX_OK;
}

bsx_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(BSX_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int kMaxBlockSize = 256;
constexpr int kHeadDim = 128;

// Checks the fields every attention call relies on.
bsx_status check_shape(const bsx_shape* s, bool need_heads) {
  if (!s) return fail(BSX_E_INVALID, "shape is NULL");
  if (s->n_blocks < 0) return fail(BSX_E_INVALID, "n_blocks = %d < 0", s->n_blocks);
  if (s->block_size < 1 || s->block_size > kMaxBlockSize)
    return fail(BSX_E_INVALID, "block_size = %d outside [1, %d]", s->block_size, kMaxBlockSize);
  if (s->ctx_len < 0) return fail(BSX_E_INVALID, "ctx_len = %lld < 0", (long long)s->ctx_len);
  if (s->ctx_len > (int64_t(1) << 40))
    return fail(BSX_E_INVALID, "ctx_len = %lld exceeds 2^40", (long long)s->ctx_len);
  if ((int64_t)s->n_blocks * s->block_size > (int64_t(1) << 24))
    return fail(BSX_E_INVALID, "n_blocks * block_size exceeds 2^24 queries");
  if (!need_heads) return ok();
  if (s->n_kv_heads < 1) return fail(BSX_E_INVALID, "n_kv_heads = %d < 1", s->n_kv_heads);
  if (s->n_q_heads < s->n_kv_heads || s->n_q_heads % s->n_kv_heads != 0)
    return fail(BSX_E_INVALID, "n_q_heads = %d is not a positive multiple of n_kv_heads = %d",
                s->n_q_heads, s->n_kv_heads);
  if (s->n_q_heads > 1024) return fail(BSX_E_INVALID, "n_q_heads = %d > 1024", s->n_q_heads);
  if (s->dtype != BSX_F32 && s->dtype != BSX_BF16)
    return fail(BSX_E_INVALID, "dtype = %d is not BSX_F32 or BSX_BF16", s->dtype);
  if (s->head_dim < 1) return fail(BSX_E_INVALID, "head_dim = %d < 1", s->head_dim);
  if (s->head_dim != kHeadDim)
    return fail(BSX_E_UNSUPPORTED, "head_dim = %d (only %d is implemented)", s->head_dim,
                kHeadDim);
  if (!std::isfinite(s->scale)) return fail(BSX_E_INVALID, "scale is not finite");
  return ok();
}

// Checks a chunk table; on success *n_local is the local K/V length.
bsx_status check_chunks(const bsx_shape* s, const bsx_chunks* c, bool need_slots,
                        int64_t* n_local) {
  if (!c) return fail(BSX_E_INVALID, "chunks is NULL");
  if (c->n_chunks < 0) return fail(BSX_E_INVALID, "n_chunks = %d < 0", c->n_chunks);
  if (c->n_chunks > (1 << 20)) return fail(BSX_E_INVALID, "n_chunks = %d > 2^20", c->n_chunks);
  if (c->n_chunks > 0 && (!c->start || !c->len))
    return fail(BSX_E_INVALID, "chunk start/len arrays are NULL");
  int64_t total = 0;
  for (int32_t i = 0; i < c->n_chunks; ++i) {
    const int64_t st = c->start[i], ln = c->len[i];
    if (ln < 0) return fail(BSX_E_INVALID, "chunk %d: len = %lld < 0", i, (long long)ln);
    if (st < 0 || st > s->ctx_len || ln > s->ctx_len - st)
      return fail(BSX_E_INVALID, "chunk %d: [%lld, %lld) is not inside [0, %lld)", i,
                  (long long)st, (long long)(st + ln), (long long)s->ctx_len);
    total += ln;
  }
  if (need_slots) {
    if (c->n_slots < (c->n_chunks > 0 ? 1 : 0) || c->n_slots > (1 << 20))
      return fail(BSX_E_INVALID, "n_slots = %d is out of range", c->n_slots);
    if (!c->slot) {
      if (c->n_slots != c->n_chunks)
        return fail(BSX_E_INVALID, "slot is NULL but n_slots (%d) != n_chunks (%d)", c->n_slots,
                    c->n_chunks);
    } else {
      for (int32_t i = 0; i < c->n_chunks; ++i)
        if (c->slot[i] < 0 || c->slot[i] >= c->n_slots)
          return fail(BSX_E_INVALID, "chunk %d: slot %d outside [0, %d)", i, c->slot[i],
                      c->n_slots);
    }
  }
  if (total >= (int64_t(1) << 32))
    return fail(BSX_E_UNSUPPORTED, "local K/V buffer of %lld keys (at most 2^32 - 1)",
                (long long)total);
  if (n_local) *n_local = total;
  return ok();
}

// Per-call descriptor of the forward pass: slot_ptr[n_slots + 1] (int32), then the
// non-empty chunks grouped by slot in chunk index order (ChunkEntry, 16-byte aligned).
struct FwdLayout {
  size_t ptr_bytes;
  size_t entries_off;
  size_t total;
};

FwdLayout fwd_layout(int32_t n_slots, int32_t n_chunks) {
  FwdLayout l;
  l.ptr_bytes = sizeof(int32_t) * (size_t(n_slots) + 1);
  l.entries_off = align_up(l.ptr_bytes, 16);
  l.total = l.entries_off + sizeof(bsx::ChunkEntry) * size_t(n_chunks);
  return l;
}

// Places a host-built table inline in the kernel arguments when it fits, else
// uploads it to the workspace on `stream` and points the kernels there.
hipError_t place_table(const uint32_t* words, size_t n_words, void* ws, hipStream_t stream,
                       bsx::ChunkTable* t) {
  std::memset(t, 0, sizeof(*t));
  if (n_words * 4 <= size_t(bsx::kInlineBytes)) {
    if (n_words) std::memcpy(t->words, words, n_words * 4);
    t->dev = nullptr;
    return hipSuccess;
  }
  t->dev = static_cast<const char*>(ws);
  return bsx::launch_upload(words, n_words, static_cast<uint32_t*>(ws), stream);
}

hipError_t place_table(const std::vector<uint32_t>& words, void* ws, hipStream_t stream,
                       bsx::ChunkTable* t) {
  return place_table(words.data(), words.size(), ws, stream, t);
}

// Storage the forward descriptor is built in, provided by the caller (the builder
// itself allocates nothing).
struct FwdDescStorage {
  int64_t* off;            // [n_chunks]
  int32_t* ptr;            // [n_slots + 1]
  int32_t* fill;           // [n_slots]
  bsx::ChunkEntry* ent;    // [n_chunks]
  bsx::ChunkEntry* tmp;    // [n_chunks]
  uint32_t* words;         // [fwd_desc_words(n_slots, n_chunks)]
};

size_t fwd_desc_words(int32_t n_slots, int32_t n_chunks) {
  return align_up(fwd_layout(n_slots, n_chunks).total, 4) / 4;
}

// Stable sort of a[0, n) by start (bottom-up merge sort through tmp).
void sort_by_start(bsx::ChunkEntry* a, int32_t n, bsx::ChunkEntry* tmp) {
  bsx::ChunkEntry* src = a;
  bsx::ChunkEntry* dst = tmp;
  for (int32_t width = 1; width < n; width *= 2) {
    for (int32_t lo = 0; lo < n; lo += 2 * width) {
      const int32_t mid = std::min(lo + width, n), hi = std::min(lo + 2 * width, n);
      int32_t i = lo, j = mid, k = lo;
      while (i < mid && j < hi) dst[k++] = src[j].start < src[i].start ? src[j++] : src[i++];
      while (i < mid) dst[k++] = src[i++];
      while (j < hi) dst[k++] = src[j++];
    }
    std::swap(src, dst);
  }
  if (src != a) std::memcpy(a, src, sizeof(bsx::ChunkEntry) * size_t(n));
}

// Each slot's entries are sorted by start (ties keep chunk index order); *order is 2
// when every slot's entries are also disjoint, else 1.  Kernels walking a slot stop at
// its first entry past their range, and bisect to their first entry when disjoint.
// Returns the descriptor's length in 32-bit words (in st.words).
size_t build_fwd_descriptor(const bsx_chunks* c, const FwdDescStorage& st, int32_t* n_entries,
                            int32_t* order) {
  const int32_t nc = c->n_chunks, ns = c->n_slots;
  const FwdLayout l = fwd_layout(ns, nc);
  int64_t acc = 0;
  for (int32_t i = 0; i < nc; ++i) {
    st.off[i] = acc;
    acc += c->len[i];
  }
  for (int32_t s = 0; s <= ns; ++s) st.ptr[s] = 0;
  for (int32_t i = 0; i < nc; ++i)
    if (c->len[i] > 0) st.ptr[(c->slot ? c->slot[i] : i) + 1]++;
  for (int32_t s = 0; s < ns; ++s) st.ptr[s + 1] += st.ptr[s];
  for (int32_t s = 0; s < ns; ++s) st.fill[s] = st.ptr[s];
  for (int32_t i = 0; i < nc; ++i) {
    if (c->len[i] <= 0) continue;
    const int32_t s = c->slot ? c->slot[i] : i;
    st.ent[st.fill[s]++] = bsx::ChunkEntry{c->start[i], uint32_t(c->len[i]), uint32_t(st.off[i])};
  }
  bool disjoint = true;
  for (int32_t s = 0; s < ns; ++s) {
    bsx::ChunkEntry* b = st.ent + st.ptr[s];
    const int32_t n = st.ptr[s + 1] - st.ptr[s];
    sort_by_start(b, n, st.tmp);
    for (int32_t j = 0; j + 1 < n; ++j)
      if (b[j].start + int64_t(b[j].len) > b[j + 1].start) disjoint = false;
  }
  *order = disjoint ? 2 : 1;
  const size_t used = l.entries_off + sizeof(bsx::ChunkEntry) * size_t(st.ptr[ns]);
  const size_t n_words = align_up(used, 4) / 4;
  std::memset(st.words, 0, n_words * 4);
  std::memcpy(st.words, st.ptr, l.ptr_bytes);
  if (st.ptr[ns] > 0)
    std::memcpy(reinterpret_cast<char*>(st.words) + l.entries_off, st.ent,
                sizeof(bsx::ChunkEntry) * size_t(st.ptr[ns]));
  *n_entries = st.ptr[ns];
  return n_words;
}

float resolve_scale(const bsx_shape* s) {
  return s->scale > 0.f ? s->scale : 1.0f / std::sqrt(float(s->head_dim));
}

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace

extern "C" {

int bsx_abi_version(void) { return BSX_ABI_VERSION; }

const char* bsx_last_error(void) { return g_last_error; }

const char* bsx_status_string(int status) {
  switch (status) {
    case BSX_OK: return "BSX_OK";
    case BSX_E_INVALID: return "BSX_E_INVALID";
    case BSX_E_UNSUPPORTED: return "BSX_E_UNSUPPORTED";
    case BSX_E_WORKSPACE: return "BSX_E_WORKSPACE";
    case BSX_E_DEVICE: return "BSX_E_DEVICE";
    default: return "unknown bsx_status";
  }
}

bsx_status bsx_validate_mask(const bsx_shape* shape, const int64_t* anchor,
                             const int64_t* ctx_begin) {
  bsx_status st = check_shape(shape, false);
  if (st != BSX_OK) return st;
  if (shape->n_blocks > 0 && (!anchor || !ctx_begin))
    return fail(BSX_E_INVALID, "anchor/ctx_begin is NULL");
  for (int32_t b = 0; b < shape->n_blocks; ++b) {
    const int64_t lo = ctx_begin[b], hi = anchor[b];
    if (lo < 0 || lo > hi || hi > shape->ctx_len)
      return fail(BSX_E_INVALID, "block %d: context range [%lld, %lld) is not inside [0, %lld]",
                  b, (long long)lo, (long long)hi, (long long)shape->ctx_len);
  }
  return ok();
}

bsx_status bsx_mask_from_anchors(const bsx_shape* shape, const int64_t* anchor_global,
                                 const int64_t* sample_start, int64_t* ctx_begin,
                                 int64_t* anchor) {
  bsx_status st = check_shape(shape, false);
  if (st != BSX_OK) return st;
  if (shape->n_blocks > 0 && (!anchor_global || !ctx_begin || !anchor))
    return fail(BSX_E_INVALID, "anchor_global/ctx_begin/anchor is NULL");
  // check every block first, so that nothing is written on error
  for (int32_t b = 0; b < shape->n_blocks; ++b) {
    const int64_t lo = sample_start ? sample_start[b] : 0, hi = anchor_global[b];
    if (lo < 0 || lo > hi || hi > shape->ctx_len)
      return fail(BSX_E_INVALID,
                  "block %d: anchor %lld with sample start %lld is not inside [0, %lld]", b,
                  (long long)hi, (long long)lo, (long long)shape->ctx_len);
  }
  for (int32_t b = 0; b < shape->n_blocks; ++b) {
    ctx_begin[b] = sample_start ? sample_start[b] : 0;
    anchor[b] = anchor_global[b];
  }
  return ok();
}

bsx_status bsx_lpt(int32_t n_items, const int64_t* cost, int32_t n_bins, int32_t* bin_of,
                   int64_t* bin_load, int64_t* makespan, double* imbalance) {
  if (n_items < 0) return fail(BSX_E_INVALID, "n_items = %d < 0", n_items);
  if (n_bins < 1) return fail(BSX_E_INVALID, "n_bins = %d < 1", n_bins);
  if (n_items > 0 && (!cost || !bin_of)) return fail(BSX_E_INVALID, "cost/bin_of is NULL");
  for (int32_t i = 0; i < n_items; ++i)
    if (cost[i] < 0) return fail(BSX_E_INVALID, "cost[%d] = %lld < 0", i, (long long)cost[i]);
  std::vector<int32_t> order(n_items);
  std::iota(order.begin(), order.end(), 0);
  std::sort(order.begin(), order.end(), [cost](int32_t a, int32_t b) {
    return cost[a] != cost[b] ? cost[a] > cost[b] : a < b;
  });
  std::vector<int64_t> load(n_bins, 0);
  // least loaded bin first, ties to the lower index: a min-heap on (load, index)
  typedef std::pair<int64_t, int32_t> Bin;
  std::priority_queue<Bin, std::vector<Bin>, std::greater<Bin>> heap;
  for (int32_t j = 0; j < n_bins; ++j) heap.push(Bin(0, j));
  int64_t total = 0;
  for (int32_t i : order) {
    const int32_t best = heap.top().second;
    heap.pop();
    bin_of[i] = best;
    load[best] += cost[i];
    total += cost[i];
    heap.push(Bin(load[best], best));
  }
  const int64_t ms = *std::max_element(load.begin(), load.end());
  if (bin_load) std::copy(load.begin(), load.end(), bin_load);
  if (makespan) *makespan = ms;
  if (imbalance)
    *imbalance = total > 0 ? double(ms) / (double(total) / double(n_bins)) - 1.0 : 0.0;
  return ok();
}

bsx_status bsx_place(int32_t mode, int32_t n_items, const int64_t* cost, int32_t n_bins,
                     int32_t* bin_of, int64_t* bin_load, int64_t* makespan, double* imbalance) {
  if (mode == BSX_PLACE_LPT)
    return bsx_lpt(n_items, cost, n_bins, bin_of, bin_load, makespan, imbalance);
  if (mode != BSX_PLACE_CONTIGUOUS && mode != BSX_PLACE_ZIGZAG && mode != BSX_PLACE_ROUND_ROBIN)
    return fail(BSX_E_INVALID, "placement mode %d is not one of 0..3", mode);
  if (n_items < 0) return fail(BSX_E_INVALID, "n_items = %d < 0", n_items);
  if (n_bins < 1) return fail(BSX_E_INVALID, "n_bins = %d < 1", n_bins);
  if (n_items > 0 && (!cost || !bin_of)) return fail(BSX_E_INVALID, "cost/bin_of is NULL");
  for (int32_t i = 0; i < n_items; ++i)
    if (cost[i] < 0) return fail(BSX_E_INVALID, "cost[%d] = %lld < 0", i, (long long)cost[i]);
  const int64_t n = n_items, P = n_bins;
  std::vector<int64_t> load(size_t(n_bins), 0);
  int64_t total = 0;
  for (int64_t i = 0; i < n; ++i) {
    int64_t b;
    if (mode == BSX_PLACE_CONTIGUOUS) {
      b = i * P / n;
    } else if (mode == BSX_PLACE_ZIGZAG) {
      const int64_t run = i * 2 * P / n;
      b = run < P ? run : 2 * P - 1 - run;
    } else {
      b = i % P;
    }
    bin_of[i] = int32_t(b);
    load[size_t(b)] += cost[i];
    total += cost[i];
  }
  const int64_t ms = *std::max_element(load.begin(), load.end());
  if (bin_load) std::copy(load.begin(), load.end(), bin_load);
  if (makespan) *makespan = ms;
  if (imbalance)
    *imbalance = total > 0 ? double(ms) / (double(total) / double(n_bins)) - 1.0 : 0.0;
  return ok();
}

// Cost workspace: the chunk table (when it is not inline), then for launches over many
// blocks the block groups' chunk sums and mask flags.
static size_t cost_table_bytes(int32_t n_chunks) {
  return align_up(sizeof(bsx::ChunkEntry) * size_t(n_chunks < 0 ? 0 : n_chunks), 256) + 256;
}

size_t bsx_cost_workspace(int32_t n_chunks) {
  const size_t nc = size_t(n_chunks < 0 ? 0 : n_chunks);
  const size_t groups = size_t(bsx::cost_max_groups(n_chunks < 0 ? 0 : n_chunks));
  return cost_table_bytes(n_chunks) + align_up(sizeof(int64_t) * groups * nc, 256) +
         align_up(sizeof(int32_t) * groups, 256);
}

bsx_status bsx_cost(const bsx_shape* shape, const int64_t* anchor, const int64_t* ctx_begin,
                    const bsx_chunks* chunks, int64_t* counts, int64_t* chunk_cost,
                    int32_t* mask_err, void* ws, size_t ws_bytes, void* stream) {
  bsx_status st = check_shape(shape, false);
  if (st != BSX_OK) return st;
  st = check_chunks(shape, chunks, false, nullptr);
  if (st != BSX_OK) return st;
  if (!mask_err) return fail(BSX_E_INVALID, "mask_err is NULL");
  if (shape->n_blocks > 0 && (!anchor || !ctx_begin))
    return fail(BSX_E_INVALID, "anchor/ctx_begin is NULL");
  if (chunks->n_chunks > 0 && !chunk_cost) return fail(BSX_E_INVALID, "chunk_cost is NULL");
  const size_t need = bsx_cost_workspace(chunks->n_chunks);
  if (!ws || ws_bytes < need)
    return fail(BSX_E_WORKSPACE, "workspace of %zu bytes is smaller than %zu", ws_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<uint32_t> words(size_t(chunks->n_chunks) * 4);
  for (int32_t i = 0; i < chunks->n_chunks; ++i) {
    const bsx::ChunkEntry e{chunks->start[i], uint32_t(chunks->len[i]), 0u};
    std::memcpy(&words[size_t(i) * 4], &e, sizeof(e));
  }
  bsx::CostParams p{};
  hipError_t e = place_table(words, ws, s, &p.table);
  if (e != hipSuccess) return device_status(e, "cost descriptor upload");
  p.anchor = anchor;
  p.ctx_begin = ctx_begin;
  p.counts = counts;
  p.chunk_cost = chunk_cost;
  p.mask_err = mask_err;
  p.ctx_len = shape->ctx_len;
  p.n_blocks = shape->n_blocks;
  p.block_size = shape->block_size;
  p.n_chunks = chunks->n_chunks;
  // enough block groups to fill the chip, each a whole number of 256-block rounds
  const int32_t rounds = (shape->n_blocks + 255) / 256;
  const int32_t max_groups = bsx::cost_max_groups(chunks->n_chunks);
  const int32_t want = rounds < max_groups ? rounds : max_groups;
  p.span = shape->n_blocks > 0 ? shape->n_blocks : 1;
  p.part = nullptr;
  p.bad = nullptr;
  if (want > 1) {
    const int32_t per = (rounds + want - 1) / want;  // rounds per group
    p.span = per * 256;
    char* base = static_cast<char*>(ws) + cost_table_bytes(chunks->n_chunks);
    p.part = reinterpret_cast<int64_t*>(base);
    p.bad = reinterpret_cast<int32_t*>(
        base + align_up(sizeof(int64_t) * size_t(max_groups) * size_t(chunks->n_chunks), 256));
  }
  return device_status(bsx::launch_cost(p, s), "cost kernel");
}

// Forward workspace: the chunk table (when it is not inline), then for bf16 launches
// the launch order (int32 per workgroup) and, for launches that may split items, the
// piece list, the split tables and the pieces' partials.  Laid out for a given
// number of output slots; bsx_fwd_workspace covers both with and without a self slot.
struct FwdWs {
  size_t order_off = 0, piece_off = 0, split_off = 0, part_o_off = 0, part_lse_off = 0;
  bool order = false, split = false;
  size_t total = 0;
};

// allow_split: launches with few (KV head, slot) pairs may cut long items into pieces,
// which needs room for the pieces' partials; without it such launches run unsplit.
FwdWs fwd_ws_layout(const bsx_shape* shape, const bsx_chunks* chunks, int64_t n_out,
                    bool allow_split = true) {
  FwdWs w;
  w.total = align_up(fwd_layout(chunks->n_slots, chunks->n_chunks).total, 256);
  if (!shape || shape->dtype != BSX_BF16 || shape->n_kv_heads < 1 || shape->n_blocks < 1 ||
      n_out < 1)
    return w;
  const int64_t n_rows = int64_t(shape->n_blocks) * shape->block_size *
                         (shape->n_q_heads / shape->n_kv_heads);
  const int64_t n_tiles = (n_rows + bsx::kFwdRows - 1) / bsx::kFwdRows;
  if (n_tiles * n_out > bsx::kOrderMaxItems) return w;
  const bsx::FwdSplitLayout sl = bsx::fwd_split_layout(
      shape->n_blocks, shape->block_size, shape->n_q_heads, shape->n_kv_heads, int32_t(n_out));
  const bool split = allow_split && sl.split_capable;
  const int64_t grid = split ? sl.grid
                             : bsx::fwd_bf16_grid(shape->n_blocks, shape->block_size,
                                                  shape->n_q_heads, shape->n_kv_heads,
                                                  int32_t(n_out));
  w.order = true;
  w.order_off = w.total;
  w.total += align_up(sizeof(int32_t) * size_t(grid), 256);
  if (split) {
    w.split = true;
    w.piece_off = w.total;
    w.total += align_up(sl.piece_bytes, 256);
    w.split_off = w.total;
    w.total += align_up(sl.split_bytes, 256);
    w.part_o_off = w.total;
    w.total += align_up(sl.part_o_bytes, 256);
    w.part_lse_off = w.total;
    w.total += align_up(sl.part_lse_bytes, 256);
  }
  return w;
}

// Argument checks of a forward call (all but the workspace).  *n_local is the local
// K/V length; *empty is true when there is nothing to compute.
bsx_status check_fwd_args(const bsx_shape* shape, const void* q, const void* k, const void* v,
                          const void* k_self, const void* v_self, const int64_t* anchor,
                          const int64_t* ctx_begin, const bsx_chunks* chunks,
                          const float* o_part, const float* lse_part, int64_t* n_local,
                          bool* empty) {
  bsx_status st = check_shape(shape, true);
  if (st != BSX_OK) return st;
  st = check_chunks(shape, chunks, true, n_local);
  if (st != BSX_OK) return st;
  if ((k_self == nullptr) != (v_self == nullptr))
    return fail(BSX_E_INVALID, "k_self and v_self must both be given or both be NULL");
  const int64_t n_out = int64_t(chunks->n_slots) + (k_self != nullptr);
  *empty = shape->n_blocks == 0 || n_out == 0;
  if (*empty) return ok();
  if (!q || !anchor || !ctx_begin || !o_part || !lse_part)
    return fail(BSX_E_INVALID, "q/anchor/ctx_begin/o_part/lse_part is NULL");
  if (*n_local > 0 && (!k || !v)) return fail(BSX_E_INVALID, "k/v is NULL");
  return ok();
}

// Builds the forward descriptor in `st` and launches the forward pass; `ws` holds the
// pieces of layout `w` (the table when it is not inline, the launch order, the split
// tables).
bsx_status launch_forward(const bsx_shape* shape, const void* q, const void* k, const void* v,
                          const void* k_self, const void* v_self, const int64_t* anchor,
                          const int64_t* ctx_begin, const bsx_chunks* chunks, int64_t n_local,
                          float* o_part, float* lse_part, const FwdDescStorage& st,
                          const FwdWs& w, void* ws, hipStream_t s) {
  int32_t n_entries = 0, entries_order = 0;
  const size_t n_words = build_fwd_descriptor(chunks, st, &n_entries, &entries_order);
  const FwdLayout l = fwd_layout(chunks->n_slots, chunks->n_chunks);
  const int has_self = k_self != nullptr;

  bsx::FwdParams p{};
  hipError_t e = place_table(st.words, n_words, ws, s, &p.table);
  if (e != hipSuccess) return device_status(e, "forward descriptor upload");
  p.entries_off = uint32_t(l.entries_off);
  p.entries_order = entries_order;
  p.q = q;
  p.k = k;
  p.v = v;
  p.k_self = k_self;
  p.v_self = v_self;
  p.anchor = anchor;
  p.ctx_begin = ctx_begin;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.ctx_len = shape->ctx_len;
  p.n_local = n_local;
  p.n_blocks = shape->n_blocks;
  p.block_size = shape->block_size;
  p.n_q_heads = shape->n_q_heads;
  p.n_kv_heads = shape->n_kv_heads;
  p.n_slots = chunks->n_slots;
  p.has_self = has_self;
  p.scale = resolve_scale(shape);
  p.scale_log2 = p.scale * kLog2e;
  p.order = nullptr;
  p.piece = nullptr;
  p.split = nullptr;
  p.part_o = nullptr;
  p.part_lse = nullptr;
  if (shape->dtype == BSX_BF16) {
    // The launch-order pass (heaviest items first on each XCD, empty items dropped)
    // costs one small launch and pays for itself even when items are at most one chunk
    // long (measured on 16 one-chunk LPT bins).  Launches with few items may also split
    // long items into pieces (merged afterwards).
    char* base = static_cast<char*>(ws);
    if (w.order) {
      int32_t* order = reinterpret_cast<int32_t*>(base + w.order_off);
      if (w.split) {
        p.piece = reinterpret_cast<int32_t*>(base + w.piece_off);
        p.split = reinterpret_cast<int32_t*>(base + w.split_off);
        p.part_o = reinterpret_cast<float*>(base + w.part_o_off);
        p.part_lse = reinterpret_cast<float*>(base + w.part_lse_off);
      }
      e = bsx::launch_fwd_order(p, order, s);
      if (e != hipSuccess) return device_status(e, "forward launch-order kernel");
      p.order = order;
    }
    e = bsx::launch_fwd_bf16(p, s);
    if (e == hipSuccess && p.split) e = bsx::launch_fwd_piece_merge(p, s);
  } else {
    e = bsx::launch_fwd_f32(p, s);
  }
  return device_status(e, "forward kernel");
}

size_t bsx_fwd_workspace(const bsx_shape* shape, const bsx_chunks* chunks) {
  if (!chunks || chunks->n_chunks < 0 || chunks->n_slots < 0) return 0;
  const size_t with_self = fwd_ws_layout(shape, chunks, int64_t(chunks->n_slots) + 1).total;
  const size_t without = fwd_ws_layout(shape, chunks, chunks->n_slots).total;
  return with_self > without ? with_self : without;
}

bsx_status bsx_attn_fwd(const bsx_shape* shape, const void* q, const void* k, const void* v,
                        const void* k_self, const void* v_self, const int64_t* anchor,
                        const int64_t* ctx_begin, const bsx_chunks* chunks, float* o_part,
                        float* lse_part, void* ws, size_t ws_bytes, void* stream) {
  int64_t n_local = 0;
  bool empty = false;
  bsx_status st = check_fwd_args(shape, q, k, v, k_self, v_self, anchor, ctx_begin, chunks,
                                 o_part, lse_part, &n_local, &empty);
  if (st != BSX_OK || empty) return st;
  const size_t need = bsx_fwd_workspace(shape, chunks);
  if (!ws || ws_bytes < need)
    return fail(BSX_E_WORKSPACE, "workspace of %zu bytes is smaller than %zu", ws_bytes, need);
  const int32_t nc = chunks->n_chunks, ns = chunks->n_slots;
  std::vector<int64_t> off(size_t(nc) + 1);
  std::vector<int32_t> ptr(size_t(ns) + 1), fill(size_t(ns) + 1);
  std::vector<bsx::ChunkEntry> ent(size_t(nc) + 1), tmp(size_t(nc) + 1);
  std::vector<uint32_t> words(fwd_desc_words(ns, nc) + 1);
  const FwdDescStorage storage{off.data(), ptr.data(), fill.data(), ent.data(), tmp.data(),
                               words.data()};
  const int64_t n_out = int64_t(ns) + (k_self != nullptr);
  return launch_forward(shape, q, k, v, k_self, v_self, anchor, ctx_begin, chunks, n_local,
                        o_part, lse_part, storage, fwd_ws_layout(shape, chunks, n_out), ws,
                        static_cast<hipStream_t>(stream));
}

bsx_status bsx_attn_fwd_noalloc(const bsx_shape* shape, const void* q, const void* k,
                                const void* v, const void* k_self, const void* v_self,
                                const int64_t* anchor, const int64_t* ctx_begin,
                                const bsx_chunks* chunks, float* o_part, float* lse_part,
                                void* stream) {
  int64_t n_local = 0;
  bool empty = false;
  bsx_status st = check_fwd_args(shape, q, k, v, k_self, v_self, anchor, ctx_begin, chunks,
                                 o_part, lse_part, &n_local, &empty);
  if (st != BSX_OK || empty) return st;
  constexpr int32_t kMax = BSX_NOALLOC_MAX_CHUNKS;
  if (chunks->n_chunks > kMax || chunks->n_slots > kMax)
    return fail(BSX_E_UNSUPPORTED,
                "bsx_attn_fwd_noalloc takes at most %d chunks and %d slots (got %d, %d)", kMax,
                kMax, chunks->n_chunks, chunks->n_slots);
  const int64_t n_out = int64_t(chunks->n_slots) + (k_self != nullptr);
  const FwdWs w = fwd_ws_layout(shape, chunks, n_out, /*allow_split=*/false);
  if (w.total > size_t(BSX_NOALLOC_SCRATCH_BYTES))
    return fail(BSX_E_UNSUPPORTED,
                "this forward needs %zu bytes of scratch; bsx_attn_fwd_noalloc has %zu",
                w.total, size_t(BSX_NOALLOC_SCRATCH_BYTES));
  // descriptor storage on the stack, sized for the largest table this entry point takes
  int64_t off[kMax];
  int32_t ptr[kMax + 1], fill[kMax + 1];
  bsx::ChunkEntry ent[kMax], tmp[kMax];
  uint32_t words[(16 * (kMax + 1) + 16 * kMax) / 4 + 4];
  static_assert(sizeof(words) / 4 >= (sizeof(int32_t) * (kMax + 1) + 15) / 16 * 4 + 4 * kMax,
                "descriptor words of the largest table fit");
  const FwdDescStorage storage{off, ptr, fill, ent, tmp, words};
  hipError_t e = hipSuccess;
  void* scratch = bsx::noalloc_scratch(&e);
  if (!scratch) return device_status(e == hipSuccess ? hipErrorInvalidDevice : e,
                                     "scratch address of the current device");
  return launch_forward(shape, q, k, v, k_self, v_self, anchor, ctx_begin, chunks, n_local,
                        o_part, lse_part, storage, w, scratch, static_cast<hipStream_t>(stream));
}

bsx_status bsx_lse_merge(int32_t n_parts, int64_t n_rows, int32_t head_dim,
                         const float* o_parts, const float* lse_parts, int32_t out_dtype,
                         void* o_out, float* lse_out, void* stream) {
  if (n_parts < 1 || n_parts > 4096)
    return fail(BSX_E_INVALID, "n_parts = %d outside [1, 4096]", n_parts);
  if (n_rows < 0) return fail(BSX_E_INVALID, "n_rows = %lld < 0", (long long)n_rows);
  if (head_dim < 4 || head_dim > 512 || head_dim % 4 != 0)
    return fail(BSX_E_INVALID, "head_dim = %d is not a multiple of 4 in [4, 512]", head_dim);
  if (out_dtype != BSX_F32 && out_dtype != BSX_BF16)
    return fail(BSX_E_INVALID, "out_dtype = %d is not BSX_F32 or BSX_BF16", out_dtype);
  if (out_dtype == BSX_BF16 && n_parts > bsx::kMergeBf16MaxParts)
    return fail(BSX_E_UNSUPPORTED, "a bf16 merged output takes at most %d partials (got %d)",
                bsx::kMergeBf16MaxParts, n_parts);
  if (n_rows == 0) return ok();
  if (!o_parts || !lse_parts || !o_out || !lse_out)
    return fail(BSX_E_INVALID, "a merge pointer is NULL");
  return device_status(bsx::launch_lse_merge(n_parts, n_rows, head_dim, o_parts, lse_parts,
                                             out_dtype == BSX_BF16, o_out, lse_out,
                                             static_cast<hipStream_t>(stream)),
                       "merge kernel");
}

// Key-tile flags of the backward: one int32 per 64 local keys.
size_t bwd_seen_bytes(const bsx_chunks* chunks) {
  int64_t n_local = 0;
  for (int32_t i = 0; i < chunks->n_chunks; ++i)
    if (chunks->len && chunks->len[i] > 0) n_local += chunks->len[i];
  return sizeof(int32_t) * size_t((n_local + 63) / 64);
}

size_t bsx_bwd_workspace(const bsx_shape* shape, const bsx_chunks* chunks) {
  if (!shape || !chunks || chunks->n_chunks < 0 || shape->n_blocks < 0 || shape->block_size < 0 ||
      shape->n_q_heads < 0)
    return 0;
  const size_t ent = align_up(sizeof(bsx::ChunkEntry) * size_t(chunks->n_chunks), 256);
  const size_t delta = align_up(
      2 * sizeof(float) * size_t(shape->n_blocks) * shape->block_size * shape->n_q_heads, 256);
  const bsx::DqLayout l = bsx::bwd_dq_layout(shape->n_blocks, shape->block_size,
                                             shape->n_q_heads, shape->n_kv_heads);
  return ent + delta + align_up(l.plan_bytes, 256) + align_up(l.part_bytes, 256) +
         align_up(bwd_seen_bytes(chunks), 256) + 256;
}

bsx_status bsx_attn_bwd(const bsx_shape* shape, const void* q, const void* k, const void* v,
                        const void* k_self, const void* v_self, const float* o,
                        const float* lse, const void* d_o, const int64_t* anchor,
                        const int64_t* ctx_begin, const bsx_chunks* chunks, float* dq,
                        float* dk, float* dv, float* dk_self, float* dv_self, void* ws,
                        size_t ws_bytes, void* stream) {
  bsx_status st = check_shape(shape, true);
  if (st != BSX_OK) return st;
  int64_t n_local = 0;
  st = check_chunks(shape, chunks, false, &n_local);
  if (st != BSX_OK) return st;
  if (shape->dtype != BSX_BF16)
    return fail(BSX_E_UNSUPPORTED, "the backward pass takes bf16 inputs only");
  if ((k_self == nullptr) != (v_self == nullptr))
    return fail(BSX_E_INVALID, "k_self and v_self must both be given or both be NULL");
  const int has_self = k_self != nullptr;
  if (has_self && (!dk_self || !dv_self))
    return fail(BSX_E_INVALID, "dk_self/dv_self is NULL while k_self is given");
  if (shape->n_blocks > 0 && (!q || !o || !lse || !d_o || !anchor || !ctx_begin || !dq))
    return fail(BSX_E_INVALID, "q/o/lse/d_o/anchor/ctx_begin/dq is NULL");
  if (n_local > 0 && (!k || !v || !dk || !dv)) return fail(BSX_E_INVALID, "k/v/dk/dv is NULL");
  const size_t need = bsx_bwd_workspace(shape, chunks);
  if (!ws || ws_bytes < need)
    return fail(BSX_E_WORKSPACE, "workspace of %zu bytes is smaller than %zu", ws_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // local offsets of the non-empty chunks, in chunk index order
  std::vector<bsx::ChunkEntry> ent;
  int64_t acc = 0;
  for (int32_t i = 0; i < chunks->n_chunks; ++i) {
    if (chunks->len[i] > 0)
      ent.push_back(bsx::ChunkEntry{chunks->start[i], uint32_t(chunks->len[i]), uint32_t(acc)});
    acc += chunks->len[i];
  }
  // the list stays in chunk index order (local offsets increase along it); walks over
  // it may stop early or bisect when it also happens to be sorted by start / disjoint
  int32_t entries_order = 2;
  for (size_t i = 0; i + 1 < ent.size(); ++i) {
    if (ent[i].start > ent[i + 1].start) {
      entries_order = 0;
      break;
    }
    if (ent[i].start + int64_t(ent[i].len) > ent[i + 1].start) entries_order = 1;
  }
  std::vector<uint32_t> words(ent.size() * sizeof(bsx::ChunkEntry) / 4);
  if (!ent.empty()) std::memcpy(words.data(), ent.data(), ent.size() * sizeof(bsx::ChunkEntry));
  bsx::BwdParams p{};
  hipError_t e = place_table(words, ws, s, &p.table);
  if (e != hipSuccess) return device_status(e, "backward descriptor upload");
  const size_t ent_bytes = align_up(sizeof(bsx::ChunkEntry) * size_t(chunks->n_chunks), 256);
  p.q = q;
  p.k = k;
  p.v = v;
  p.k_self = k_self;
  p.v_self = v_self;
  p.o = o;
  p.lse = lse;
  p.d_o = d_o;
  p.anchor = anchor;
  p.ctx_begin = ctx_begin;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dk_self = dk_self;
  p.dv_self = dv_self;
  p.stats = reinterpret_cast<float*>(static_cast<char*>(ws) + ent_bytes);
  const size_t delta_bytes = align_up(
      2 * sizeof(float) * size_t(shape->n_blocks) * shape->block_size * shape->n_q_heads, 256);
  const bsx::DqLayout dl = bsx::bwd_dq_layout(shape->n_blocks, shape->block_size,
                                              shape->n_q_heads, shape->n_kv_heads);
  p.dq_plan = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + ent_bytes + delta_bytes);
  p.dq_part = reinterpret_cast<float*>(static_cast<char*>(ws) + ent_bytes + delta_bytes +
                                       align_up(dl.plan_bytes, 256));
  p.tile_seen = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + ent_bytes + delta_bytes +
                                           align_up(dl.plan_bytes, 256) +
                                           align_up(dl.part_bytes, 256));
  p.ctx_len = shape->ctx_len;
  p.n_local = n_local;
  p.n_entries = int32_t(ent.size());
  p.entries_order = entries_order;
  p.n_blocks = shape->n_blocks;
  p.block_size = shape->block_size;
  p.n_q_heads = shape->n_q_heads;
  p.n_kv_heads = shape->n_kv_heads;
  p.has_self = has_self;
  p.scale = resolve_scale(shape);
  p.scale_log2 = p.scale * kLog2e;
  return device_status(bsx::launch_bwd_bf16(p, s), "backward kernels");
}

}  // extern "C"
