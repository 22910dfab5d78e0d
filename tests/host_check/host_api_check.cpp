// Host-only check of libbsx's host logic (argument validation, LPT and placement,
// chunk-table descriptors, workspace layouts), built with g++ under AddressSanitizer
// and UndefinedBehaviorSanitizer.  The kernel launchers are replaced by stubs that
// decode every descriptor the host built and compare it with the call's arguments;
// "device" buffers are host allocations of exactly the size the *_workspace queries
// return, and the stubs touch every byte the kernels would, so an overrun of a
// workspace layout is a sanitizer error.  No GPU and no HIP runtime are involved.
#include <algorithm>
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <random>
#include <vector>

#include "bsx.h"
#include "bsx_internal.h"

// ---------------------------------------------------------------- failure reporting
static int g_fail = 0;
#define CHECK(cond)                                                              \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "CHECK failed at line %d: %s\n", __LINE__, #cond);    \
      ++g_fail;                                                                  \
      if (g_fail > 20) std::exit(1);                                             \
    }                                                                            \
  } while (0)

extern "C" const char* hipGetErrorString(hipError_t) { return "stubbed HIP error"; }

// ---------------------------------------------------------------- expectations
// What the call under test was given, for the stubs to compare against.
struct Expect {
  std::vector<int64_t> start, len;
  std::vector<int32_t> slot;  // empty: slot i
  int32_t n_slots = 0;
  int64_t n_local = 0;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  int n_fwd_calls = 0, n_order_calls = 0, n_bwd_calls = 0, n_cost_calls = 0;
};
static Expect g_exp;

static void touch(const void* p, size_t bytes) {
  // a write of every byte: out of bounds of the allocation -> ASan report
  if (bytes) std::memset(const_cast<void*>(p), 0xA5, bytes);
}

static bool in_ws(const void* p, size_t bytes) {
  const char* c = static_cast<const char*>(p);
  return c >= g_exp.ws && c + bytes <= g_exp.ws + g_exp.ws_bytes;
}

static const char* table_base(const bsx::ChunkTable& t) {
  return t.dev ? t.dev : reinterpret_cast<const char*>(t.words);
}

namespace bsx {

hipError_t launch_upload(const uint32_t* host_words, size_t n_words, uint32_t* dst,
                         hipStream_t) {
  CHECK(in_ws(dst, n_words * 4));
  std::memcpy(dst, host_words, n_words * 4);
  return hipSuccess;
}

hipError_t launch_cost(const CostParams& p, hipStream_t) {
  ++g_exp.n_cost_calls;
  const char* t = table_base(p.table);
  CHECK(p.n_chunks == int32_t(g_exp.start.size()));
  for (int32_t i = 0; i < p.n_chunks; ++i) {
    ChunkEntry e;
    std::memcpy(&e, t + 16 * size_t(i), sizeof(e));
    CHECK(e.start == g_exp.start[i] && int64_t(e.len) == g_exp.len[i]);
  }
  if (p.part) {
    const int32_t groups = (p.n_blocks + p.span - 1) / p.span;
    CHECK(groups <= cost_max_groups(p.n_chunks));
    CHECK(in_ws(p.part, sizeof(int64_t) * size_t(groups) * p.n_chunks));
    CHECK(in_ws(p.bad, sizeof(int32_t) * size_t(groups)));
    touch(p.part, sizeof(int64_t) * size_t(groups) * p.n_chunks);
    touch(p.bad, sizeof(int32_t) * size_t(groups));
  }
  return hipSuccess;
}

// The forward descriptor: slot_ptr[n_slots + 1], then each slot's non-empty chunks
// sorted by start, with their local offsets.
static void check_fwd_table(const FwdParams& p) {
  const char* t = table_base(p.table);
  const int32_t* ptr = reinterpret_cast<const int32_t*>(t);
  CHECK(p.n_slots == g_exp.n_slots);
  CHECK(ptr[0] == 0);
  std::vector<int64_t> off(g_exp.start.size());
  int64_t acc = 0;
  for (size_t i = 0; i < off.size(); ++i) {
    off[i] = acc;
    acc += g_exp.len[i];
  }
  CHECK(acc == p.n_local);
  bool disjoint = true;
  for (int32_t s = 0; s < p.n_slots; ++s) {
    CHECK(ptr[s + 1] >= ptr[s]);
    // expected entries of slot s, in chunk index order
    std::vector<ChunkEntry> want;
    for (size_t i = 0; i < off.size(); ++i) {
      const int32_t si = g_exp.slot.empty() ? int32_t(i) : g_exp.slot[i];
      if (si == s && g_exp.len[i] > 0)
        want.push_back(ChunkEntry{g_exp.start[i], uint32_t(g_exp.len[i]), uint32_t(off[i])});
    }
    CHECK(ptr[s + 1] - ptr[s] == int32_t(want.size()));
    std::vector<ChunkEntry> got(size_t(ptr[s + 1] - ptr[s]));
    if (!got.empty())
      std::memcpy(got.data(), t + p.entries_off + 16 * size_t(ptr[s]), 16 * got.size());
    for (size_t j = 0; j + 1 < got.size(); ++j) {
      CHECK(got[j].start <= got[j + 1].start);
      if (got[j].start + int64_t(got[j].len) > got[j + 1].start) disjoint = false;
    }
    // the same multiset (the sort is stable, so ties keep chunk index order)
    std::stable_sort(want.begin(), want.end(),
                     [](const ChunkEntry& a, const ChunkEntry& b) { return a.start < b.start; });
    for (size_t j = 0; j < got.size() && j < want.size(); ++j)
      CHECK(got[j].start == want[j].start && got[j].len == want[j].len &&
            got[j].local_off == want[j].local_off);
  }
  CHECK(p.entries_order == (disjoint ? 2 : 1));
}

hipError_t launch_fwd_order(const FwdParams& p, int32_t* order, hipStream_t) {
  ++g_exp.n_order_calls;
  check_fwd_table(p);
  const int64_t n_out = int64_t(p.n_slots) + p.has_self;
  const FwdSplitLayout sl = fwd_split_layout(p.n_blocks, p.block_size, p.n_q_heads,
                                             p.n_kv_heads, int32_t(n_out));
  const int64_t grid = p.split ? sl.grid
                               : fwd_bf16_grid(p.n_blocks, p.block_size, p.n_q_heads,
                                               p.n_kv_heads, int32_t(n_out));
  CHECK(in_ws(order, sizeof(int32_t) * size_t(grid)));
  touch(order, sizeof(int32_t) * size_t(grid));
  if (p.split) {
    CHECK(sl.split_capable);
    touch(p.piece, sl.piece_bytes);
    touch(p.split, sl.split_bytes);
    touch(p.part_o, sl.part_o_bytes);
    touch(p.part_lse, sl.part_lse_bytes);
    CHECK(in_ws(p.piece, sl.piece_bytes) && in_ws(p.split, sl.split_bytes));
    CHECK(in_ws(p.part_o, sl.part_o_bytes) && in_ws(p.part_lse, sl.part_lse_bytes));
  }
  return hipSuccess;
}

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t) {
  ++g_exp.n_fwd_calls;
  check_fwd_table(p);
  // the launch-order pass runs unless it would exceed its item limit
  const int64_t n_rows = int64_t(p.n_blocks) * p.block_size * (p.n_q_heads / p.n_kv_heads);
  const int64_t items = (n_rows + kFwdRows - 1) / kFwdRows * (int64_t(p.n_slots) + p.has_self);
  CHECK((p.order != nullptr) == (items <= kOrderMaxItems));
  return hipSuccess;
}

hipError_t launch_fwd_piece_merge(const FwdParams& p, hipStream_t) {
  CHECK(p.split != nullptr && p.part_o != nullptr);
  return hipSuccess;
}

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t) {
  ++g_exp.n_fwd_calls;
  check_fwd_table(p);
  CHECK(p.order == nullptr);
  return hipSuccess;
}

hipError_t launch_lse_merge(int32_t, int64_t, int32_t, const float*, const float*, bool, void*,
                            float*, hipStream_t) {
  return hipSuccess;
}

// The backward's chunk list: every non-empty chunk in chunk index order with its
// local offset; the order flag says whether the list is sorted (and disjoint).
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t) {
  ++g_exp.n_bwd_calls;
  const char* t = table_base(p.table);
  std::vector<ChunkEntry> want;
  int64_t acc = 0;
  for (size_t i = 0; i < g_exp.start.size(); ++i) {
    if (g_exp.len[i] > 0)
      want.push_back(ChunkEntry{g_exp.start[i], uint32_t(g_exp.len[i]), uint32_t(acc)});
    acc += g_exp.len[i];
  }
  CHECK(p.n_entries == int32_t(want.size()) && p.n_local == acc);
  bool sorted = true, disjoint = true;
  for (int32_t e = 0; e < p.n_entries; ++e) {
    ChunkEntry c;
    std::memcpy(&c, t + 16 * size_t(e), sizeof(c));
    CHECK(c.start == want[e].start && c.len == want[e].len && c.local_off == want[e].local_off);
    if (e + 1 < p.n_entries) {
      if (want[e].start > want[e + 1].start) sorted = false;
      if (want[e].start + int64_t(want[e].len) > want[e + 1].start) disjoint = false;
    }
  }
  CHECK(p.entries_order == (!sorted ? 0 : disjoint ? 2 : 1));
  const size_t rows = size_t(p.n_blocks) * p.block_size * p.n_q_heads;
  const DqLayout l = bwd_dq_layout(p.n_blocks, p.block_size, p.n_q_heads, p.n_kv_heads);
  touch(p.stats, 2 * sizeof(float) * rows);
  touch(p.dq_plan, l.plan_bytes);
  touch(p.dq_part, l.part_bytes);
  touch(p.tile_seen, sizeof(int32_t) * size_t((p.n_local + 63) / 64));
  CHECK(in_ws(p.stats, 2 * sizeof(float) * rows) && in_ws(p.dq_plan, l.plan_bytes));
  CHECK(in_ws(p.dq_part, l.part_bytes));
  CHECK(in_ws(p.tile_seen, sizeof(int32_t) * size_t((p.n_local + 63) / 64)));
  return hipSuccess;
}

// The no-allocation scratch: a host buffer of the declared size stands in for the
// device array, so the layouts of bsx_attn_fwd_noalloc are checked against its bounds.
static std::vector<char> g_scratch(BSX_NOALLOC_SCRATCH_BYTES);
void* noalloc_scratch(hipError_t* err) {
  *err = hipSuccess;
  g_exp.ws = g_scratch.data();
  g_exp.ws_bytes = g_scratch.size();
  return g_scratch.data();
}

}  // namespace bsx

// ---------------------------------------------------------------- helpers
static std::mt19937_64 g_rng(12345);
static int64_t rnd(int64_t lo, int64_t hi) {  // [lo, hi]
  return lo + int64_t(g_rng() % uint64_t(hi - lo + 1));
}

struct Buf {  // a fake device buffer of exactly n bytes (heap, so ASan guards its ends)
  std::vector<char>* v;
  explicit Buf(size_t n) : v(new std::vector<char>(n ? n : 1)) {}
  ~Buf() { delete v; }
  void* p() { return v->data(); }
};

static bsx_shape make_shape(int32_t nb, int32_t B, int32_t hq, int32_t hk, int64_t S,
                            int32_t dtype) {
  bsx_shape s;
  s.n_blocks = nb;
  s.block_size = B;
  s.n_q_heads = hq;
  s.n_kv_heads = hk;
  s.head_dim = 128;
  s.dtype = dtype;
  s.ctx_len = S;
  s.scale = 0.f;
  return s;
}

// LPT against a direct transcription of its rule (longest first, least loaded bin,
// ties by index) computed with a linear scan instead of a heap.
static void check_lpt(int n, int P) {
  std::vector<int64_t> cost(static_cast<size_t>(n));
  for (auto& c : cost) c = rnd(0, 3) == 0 ? 0 : rnd(0, 1000) * rnd(1, 1 << 20);
  std::vector<int32_t> bin(static_cast<size_t>(n));
  std::vector<int64_t> load(static_cast<size_t>(P));
  int64_t ms = -1;
  double imb = -1;
  CHECK(bsx_lpt(n, cost.data(), P, bin.data(), load.data(), &ms, &imb) == BSX_OK);
  std::vector<int> order(static_cast<size_t>(n));
  for (int i = 0; i < n; ++i) order[size_t(i)] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return cost[size_t(a)] > cost[size_t(b)]; });
  std::vector<int64_t> l2(static_cast<size_t>(P), 0);
  for (int i : order) {
    int best = 0;
    for (int j = 1; j < P; ++j)
      if (l2[size_t(j)] < l2[size_t(best)]) best = j;
    CHECK(bin[size_t(i)] == best);
    l2[size_t(best)] += cost[size_t(i)];
  }
  CHECK(l2 == load);
  for (int mode = 0; mode < 4; ++mode)
    CHECK(bsx_place(mode, n, cost.data(), P, bin.data(), load.data(), &ms, &imb) == BSX_OK);
}

// A random chunk table; returns n_local.
static int64_t random_chunks(int64_t S, int n, int n_slots, bool slots, bsx_chunks* c) {
  g_exp.start.assign(size_t(n), 0);
  g_exp.len.assign(size_t(n), 0);
  g_exp.slot.clear();
  int64_t total = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t st = rnd(0, S);
    const int64_t ln = rnd(0, 5) == 0 ? 0 : rnd(0, S - st);
    g_exp.start[size_t(i)] = st;
    g_exp.len[size_t(i)] = ln;
    total += ln;
  }
  if (slots) {
    g_exp.slot.resize(size_t(n));
    for (auto& s : g_exp.slot) s = int32_t(rnd(0, n_slots - 1));
  }
  g_exp.n_slots = slots ? n_slots : n;
  g_exp.n_local = total;
  c->n_chunks = n;
  c->n_slots = g_exp.n_slots;
  c->start = g_exp.start.data();
  c->len = g_exp.len.data();
  c->slot = slots ? g_exp.slot.data() : nullptr;
  return total;
}

int main() {
  void* const D = reinterpret_cast<void*>(0x1000);  // never dereferenced by the stubs

  // ---- LPT and placements
  for (int it = 0; it < 200; ++it) check_lpt(int(rnd(0, 300)), int(rnd(1, 70)));
  CHECK(bsx_lpt(3, nullptr, 2, nullptr, nullptr, nullptr, nullptr) == BSX_E_INVALID);
  CHECK(bsx_place(9, 0, nullptr, 1, nullptr, nullptr, nullptr, nullptr) == BSX_E_INVALID);

  // ---- mask helpers
  {
    bsx_shape s = make_shape(3, 16, 8, 2, 100, BSX_BF16);
    int64_t an[3] = {5, 100, 37}, st[3] = {0, 50, 40}, b[3] = {-7, -7, -7}, a[3] = {-7, -7, -7};
    CHECK(bsx_mask_from_anchors(&s, an, st, b, a) == BSX_E_INVALID);  // block 2: 40 > 37
    CHECK(b[0] == -7 && a[0] == -7);  // nothing written on error
    int64_t st2[3] = {0, 50, 10};
    CHECK(bsx_mask_from_anchors(&s, an, st2, b, a) == BSX_OK);
    CHECK(b[1] == 50 && a[1] == 100 && b[2] == 10 && a[2] == 37);
    CHECK(bsx_validate_mask(&s, a, b) == BSX_OK);
    a[2] = 101;
    CHECK(bsx_validate_mask(&s, a, b) == BSX_E_INVALID);
    CHECK(std::strlen(bsx_last_error()) > 0);
  }

  // ---- cost, forward and backward descriptors over random chunk tables
  for (int it = 0; it < 300; ++it) {
    const int64_t S = rnd(1, 1 << 22);
    const int n = int(rnd(0, it % 3 == 0 ? 400 : 40));  // > 176 chunks: uploaded tables
    const int n_slots = int(rnd(1, 20));
    const bool slots = rnd(0, 1) == 1;
    bsx_chunks c;
    random_chunks(S, n, n_slots, slots, &c);
    const int32_t hk = int32_t(1) << rnd(0, 3);
    const int32_t hq = hk * int32_t(rnd(1, 8));
    const int32_t nb = int32_t(rnd(0, 300));
    const int32_t B = int32_t(rnd(1, 256));
    const int32_t dtype = rnd(0, 3) == 0 ? BSX_F32 : BSX_BF16;
    bsx_shape s = make_shape(nb, B, hq, hk, S, dtype);

    {  // cost
      const size_t need = bsx_cost_workspace(n);
      Buf ws(need);
      g_exp.ws = static_cast<char*>(ws.p());
      g_exp.ws_bytes = need;
      const bsx_status st = bsx_cost(&s, static_cast<int64_t*>(D), static_cast<int64_t*>(D), &c,
                                     static_cast<int64_t*>(D), static_cast<int64_t*>(D),
                                     static_cast<int32_t*>(D), ws.p(), need, nullptr);
      CHECK(st == BSX_OK || nb * int64_t(B) > (int64_t(1) << 24));
      if (need > 0)
        CHECK(bsx_cost(&s, static_cast<int64_t*>(D), static_cast<int64_t*>(D), &c,
                       static_cast<int64_t*>(D), static_cast<int64_t*>(D),
                       static_cast<int32_t*>(D), ws.p(), need - 1, nullptr) != BSX_OK);
    }
    for (int self = 0; self < 2; ++self) {  // forward, with and without draft keys
      const size_t need = bsx_fwd_workspace(&s, &c);
      Buf ws(need);
      g_exp.ws = static_cast<char*>(ws.p());
      g_exp.ws_bytes = need;
      const bsx_status st =
          bsx_attn_fwd(&s, D, D, D, self ? D : nullptr, self ? D : nullptr,
                       static_cast<int64_t*>(D), static_cast<int64_t*>(D), &c,
                       static_cast<float*>(D), static_cast<float*>(D), ws.p(), need, nullptr);
      CHECK(st == BSX_OK);
    }
    if (n <= BSX_NOALLOC_MAX_CHUNKS && c.n_slots <= BSX_NOALLOC_MAX_CHUNKS) {
      // the same forward without a workspace, in the fixed scratch
      const int before = g_exp.n_fwd_calls;
      const bsx_status st =
          bsx_attn_fwd_noalloc(&s, D, D, D, D, D, static_cast<int64_t*>(D),
                               static_cast<int64_t*>(D), &c, static_cast<float*>(D),
                               static_cast<float*>(D), nullptr);
      CHECK(st == BSX_OK && (nb == 0 || g_exp.n_fwd_calls == before + 1));
    }
    if (dtype == BSX_BF16) {  // backward
      const size_t need = bsx_bwd_workspace(&s, &c);
      Buf ws(need);
      g_exp.ws = static_cast<char*>(ws.p());
      g_exp.ws_bytes = need;
      float* F = static_cast<float*>(D);
      const bsx_status st = bsx_attn_bwd(&s, D, D, D, D, D, F, F, D, static_cast<int64_t*>(D),
                                         static_cast<int64_t*>(D), &c, F, F, F, F, F, ws.p(),
                                         need, nullptr);
      CHECK(st == BSX_OK);
    }
  }
  CHECK(g_exp.n_fwd_calls > 100 && g_exp.n_bwd_calls > 50 && g_exp.n_cost_calls > 100);
  CHECK(g_exp.n_order_calls > 50);

  // ---- argument errors launch nothing
  {
    const int before = g_exp.n_fwd_calls;
    bsx_chunks c;
    random_chunks(1000, 4, 2, true, &c);
    bsx_shape s = make_shape(2, 16, 8, 2, 1000, BSX_BF16);
    s.head_dim = 64;
    CHECK(bsx_attn_fwd(&s, D, D, D, nullptr, nullptr, static_cast<int64_t*>(D),
                       static_cast<int64_t*>(D), &c, static_cast<float*>(D),
                       static_cast<float*>(D), D, 1 << 20, nullptr) == BSX_E_UNSUPPORTED);
    s.head_dim = 128;
    g_exp.slot[0] = 7;
    CHECK(bsx_attn_fwd(&s, D, D, D, nullptr, nullptr, static_cast<int64_t*>(D),
                       static_cast<int64_t*>(D), &c, static_cast<float*>(D),
                       static_cast<float*>(D), D, 1 << 20, nullptr) == BSX_E_INVALID);
    CHECK(g_exp.n_fwd_calls == before);
    CHECK(bsx_lse_merge(129, 10, 128, static_cast<float*>(D), static_cast<float*>(D), BSX_BF16,
                        D, static_cast<float*>(D), nullptr) == BSX_E_UNSUPPORTED);
    bsx_chunks big;
    random_chunks(100000, BSX_NOALLOC_MAX_CHUNKS + 1, 4, true, &big);
    s.ctx_len = 100000;
    CHECK(bsx_attn_fwd_noalloc(&s, D, D, D, nullptr, nullptr, static_cast<int64_t*>(D),
                               static_cast<int64_t*>(D), &big, static_cast<float*>(D),
                               static_cast<float*>(D), nullptr) == BSX_E_UNSUPPORTED);
    CHECK(g_exp.n_fwd_calls == before);
  }

  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host check OK\n");
  return 0;
}
