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
//   delta: D_r = rowsum(dO * O).
//   dkdv:  key-major.  A workgroup owns 128 local keys of one KV head (32 per wave,
//          K/V rows kept in registers as MFMA operands) and walks the draft blocks
//          whose range reaches its keys, 32 query rows at a time staged in LDS.
//          S = Q K^T and dP = dO V^T put keys in lane columns, so the mask is one
//          predicate per lane; dV^T += dO^T P and dK^T += Q^T dS read dO^T / Q^T
//          with LDS transpose loads.  The draft blocks' own keys are extra tiles
//          whose only rows are their block's.
//   dq:    query-major, shaped like the forward kernel: 128 rows per workgroup,
//          K/V tiles of 64 keys in LDS; S^T = K Q^T and dP^T = V dO^T put rows in
//          lane columns, dQ^T += K^T dS^T reads K^T with transpose loads.
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
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- delta
__global__ __launch_bounds__(THREADS) void bwd_delta_kernel(const float* __restrict__ o,
                                                            const uint16_t* __restrict__ d_o,
                                                            float* __restrict__ delta,
                                                            int64_t n_rows) {
  const int64_t row = int64_t(blockIdx.x) * (THREADS / 32) + (threadIdx.x >> 5);
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
  if ((threadIdx.x & 31) == 0 && row < n_rows) delta[row] = acc;
}

// log2-domain LSE of a row; rows with no visible key get +inf so that P = 0.
__device__ inline float row_lse2(float lse) {
  return lse == -INFINITY ? INFINITY : lse * kLog2e;
}

// ---------------------------------------------------------------- dK / dV
constexpr int KV_KEYS = 128;   // keys per workgroup (32 per wave)
constexpr int RS = 32;         // query rows per staged sub-tile
constexpr int RP = 272;        // LDS pitch (bytes) of a staged Q / dO row

__global__ __launch_bounds__(THREADS, 1) void bwd_dkdv_kernel(BwdParams, int n_ctx_tiles,
                                                              int self_tiles_per_block) {
  const BSX_KARG BwdParams& p = kernel_arg0<BwdParams>();
  __shared__ __attribute__((aligned(16))) char sq[RS * RP];
  __shared__ __attribute__((aligned(16))) char sdo[RS * RP];
  __shared__ __attribute__((aligned(16))) float s_lse2[RS];
  __shared__ __attribute__((aligned(16))) float s_delta[RS];
  __shared__ int s_blocks[THREADS];
  __shared__ int s_wcount[4];
  __shared__ int64_t s_red[4][2];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;
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
  const int kk = wave * 32 + col;
  const int64_t krow = key0 + kk;
  const bool kvalid = krow < key_end;
  int64_t kpos = krow;
  if (!is_self && kvalid) {
    int lo = 0, hi = p.n_entries - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (int64_t(ent[mid].local_off) <= krow) lo = mid; else hi = mid - 1;
    }
    kpos = ent[lo].start + (krow - int64_t(ent[lo].local_off));
  }

  // ---- position range of the workgroup's keys
  {
    int64_t a = kvalid ? kpos : INT64_MAX, b = kvalid ? kpos : INT64_MIN;
    for (int off = 16; off >= 1; off >>= 1) {
      const int64_t a2 = __shfl_xor(a, off), b2 = __shfl_xor(b, off);
      a = a2 < a ? a2 : a;
      b = b2 > b ? b2 : b;
    }
    if (lane == 0) {
      s_red[wave][0] = a;
      s_red[wave][1] = b;
    }
  }
  __syncthreads();
  int64_t pmin = INT64_MAX, pmax = INT64_MIN;
  for (int w = 0; w < 4; ++w) {
    pmin = s_red[w][0] < pmin ? s_red[w][0] : pmin;
    pmax = s_red[w][1] > pmax ? s_red[w][1] : pmax;
  }
  pmin = uniform64(pmin);
  pmax = uniform64(pmax);

  // ---- K / V rows of this lane's key as MFMA B operands (dims 16t + 8*half .. +8)
  const int64_t kstride = int64_t(Hkv) * D;
  const uint32_t row_bytes = uint32_t(kstride * 2);
  const int64_t nrows_tile = key_end - key0 < KV_KEYS ? key_end - key0 : KV_KEYS;
  const uint16_t* kbase = static_cast<const uint16_t*>(is_self ? p.k_self : p.k);
  const uint16_t* vbase = static_cast<const uint16_t*>(is_self ? p.v_self : p.v);
  bf16x8 kf[8], vf[8];
  {
    const uint32_t bytes = nrows_tile > 0 ? uint32_t(nrows_tile) * row_bytes : 0u;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + key0 * kstride + int64_t(g) * D, bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + key0 * kstride + int64_t(g) * D, bytes);
    const uint32_t off = uint32_t(kk) * row_bytes + 16 * half;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kf[i] = as_bf16x8(buffer_load16(kr, off + 32 * i));
      vf[i] = as_bf16x8(buffer_load16(vr, off + 32 * i));
    }
  }

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }
  const float c2 = p.scale_log2;
  const int64_t n_q = int64_t(p.n_blocks) * B;
  const int q_rd = col * RP + half * 16;          // b128 row reads of Q / dO
  const int tr_rd = tr_lane_offset(lane, RP);     // transpose reads of Q^T / dO^T
  const int ld_row = tid >> 3, ld_ch = (tid & 7) * 2;  // staging: row, first of 2 chunks

  // ---- walk the draft blocks whose visible range reaches these keys
  const int scan_begin = is_self ? self_block : 0;
  const int scan_end = is_self ? self_block + 1 : p.n_blocks;
  for (int wb = scan_begin; wb < scan_end && pmin <= pmax; wb += THREADS) {
    // ordered compaction of the hit blocks of this window into s_blocks
    const int b = wb + tid;
    bool hit = false;
    if (b < scan_end) {
      if (is_self) {
        hit = true;
      } else {
        int64_t lo, hi;
        visible_range(p.anchor, p.ctx_begin, p.ctx_len, B, false, b, &lo, &hi);
        hit = lo < hi && lo <= pmax && hi > pmin;
      }
    }
    const uint64_t ball = __ballot(hit);
    if (lane == 0) s_wcount[wave] = __popcll(ball);
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < 4; ++w) {
      before += w < wave ? s_wcount[w] : 0;
      total += s_wcount[w];
    }
    if (hit) s_blocks[before + __popcll(ball & ((uint64_t(1) << lane) - 1))] = b;
    __syncthreads();

    for (int i = 0; i < total; ++i) {
      const int blk = s_blocks[i];
      int64_t lo, hi;
      visible_range(p.anchor, p.ctx_begin, p.ctx_len, B, is_self, blk, &lo, &hi);
      const bool key_vis = kvalid && kpos >= lo && kpos < hi;
      const bool wave_on = __any(key_vis);
      const int64_t r0 = int64_t(blk) * B * G;
      const int nr = B * G;
      for (int rs = 0; rs < nr; rs += RS) {
        // stage rows r0 + rs .. + RS of Q, dO, LSE, D
        {
          const int rr = rs + ld_row;
          const bool ok = rr < nr;
          const int64_t r = r0 + rr;
          const int64_t q = ok ? r / G : 0;
          const int h = g * G + int(ok ? r % G : 0);
          const int64_t base = (q * Hq + h) * D;
          const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + base;
          const uint16_t* drow = static_cast<const uint16_t*>(p.d_o) + base;
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int ch = ld_ch + c;
            u32x4 qv = {0u, 0u, 0u, 0u}, dv4 = {0u, 0u, 0u, 0u};
            if (ok) {
              qv = *reinterpret_cast<const u32x4*>(qrow + ch * 8);
              dv4 = *reinterpret_cast<const u32x4*>(drow + ch * 8);
            }
            *reinterpret_cast<u32x4*>(sq + ld_row * RP + ch * 16) = qv;
            *reinterpret_cast<u32x4*>(sdo + ld_row * RP + ch * 16) = dv4;
          }
          if ((tid & 7) == 0) {
            s_lse2[ld_row] = ok && q < n_q ? row_lse2(p.lse[q * Hq + h]) : INFINITY;
            s_delta[ld_row] = ok && q < n_q ? p.delta[q * Hq + h] : 0.f;
          }
        }
        __syncthreads();
        if (wave_on) {
          f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            sacc = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(sq + q_rd + 32 * k)),
                             kf[k], sacc);
            dpacc = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(sdo + q_rd + 32 * k)),
                              vf[k], dpacc);
          }
          f32x16 pm, ds;
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const float4 l4 = *reinterpret_cast<const float4*>(s_lse2 + 8 * a + 4 * half);
            const float4 d4 = *reinterpret_cast<const float4*>(s_delta + 8 * a + 4 * half);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
            const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int v = 4 * a + e;
              const float pv =
                  key_vis ? __builtin_amdgcn_exp2f(fmaf(sacc[v], c2, -lv[e])) : 0.f;
              pm[v] = pv;
              ds[v] = pv * (dpacc[v] - dd[e]);
            }
          }
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const bf16x8 pb = pack_bf16(pm, u);
            const bf16x8 sb = pack_bf16(ds, u);
#pragma unroll
            for (int db = 0; db < 4; ++db) {
              dv[db] = mfma_bf16(tr_operand(sdo + tr_rd, RP, u, db * 64), pb, dv[db]);
              dk[db] = mfma_bf16(tr_operand(sq + tr_rd, RP, u, db * 64), sb, dk[db]);
            }
          }
        }
        __syncthreads();
      }
    }
  }

  if (!kvalid) return;
  float* dkrow = (is_self ? p.dk_self : p.dk) + (krow * Hkv + g) * D;
  float* dvrow = (is_self ? p.dv_self : p.dv) + (krow * Hkv + g) * D;
  const float sc = p.scale;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = db * 32 + 8 * a + 4 * half;
      *reinterpret_cast<float4*>(dkrow + d0) =
          make_float4(dk[db][4 * a] * sc, dk[db][4 * a + 1] * sc, dk[db][4 * a + 2] * sc,
                      dk[db][4 * a + 3] * sc);
      *reinterpret_cast<float4*>(dvrow + d0) =
          make_float4(dv[db][4 * a], dv[db][4 * a + 1], dv[db][4 * a + 2], dv[db][4 * a + 3]);
    }
}

// ---------------------------------------------------------------- dQ
constexpr int QROWS = 128;
constexpr int KT = 64;
constexpr int TP = 272;                  // LDS pitch (bytes) of staged K / V rows
constexpr int TILE_BYTES = KT * TP;
constexpr int STAGE_BYTES = 2 * TILE_BYTES;

__global__ __launch_bounds__(THREADS, 1) void bwd_dq_kernel(BwdParams, int n_tiles) {
  const BSX_KARG BwdParams& p = kernel_arg0<BwdParams>();
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE_BYTES];
  __shared__ int64_t red[4][4];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;
  const int Hkv = p.n_kv_heads, Hq = p.n_q_heads, G = Hq / Hkv, B = p.block_size;
  const int g = blockIdx.x % Hkv;
  const int tile_id = blockIdx.x / Hkv;
  const int64_t n_q = int64_t(p.n_blocks) * B;
  const int64_t n_rows = n_q * G;
  const char* table = p.table.dev ? p.table.dev : (const char*)(p.table.words);
  const ChunkEntry* ent = reinterpret_cast<const ChunkEntry*>(table);

  const int64_t r = int64_t(tile_id) * QROWS + wave * 32 + col;
  const bool row_ok = r < n_rows;
  const int64_t qi = row_ok ? r / G : 0;
  const int h = g * G + int(row_ok ? r % G : 0);
  const int64_t blk = qi / B;
  const float lse2 = row_ok ? row_lse2(p.lse[qi * Hq + h]) : INFINITY;
  const float dlt = row_ok ? p.delta[qi * Hq + h] : 0.f;

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

  f32x16 dq[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) dq[db] = zero16();
  const float c2 = p.scale_log2;
  const int64_t kstride = int64_t(Hkv) * D;
  const uint32_t row_bytes = uint32_t(kstride * 2);
  const int64_t gofs = int64_t(g) * D;
  const int ld_row = tid >> 4, ld_ch = tid & 15;
  const uint32_t ld_off = uint32_t(ld_row) * row_bytes + uint32_t(ld_ch) * 16;
  const int k_rd = col * TP + half * 16;
  const int tr_rd = tr_lane_offset(lane, TP);

  // phase 0: local context chunks; phase 1: the draft blocks' own keys
  for (int phase = 0; phase < (p.has_self ? 2 : 1); ++phase) {
    const bool is_self = phase == 1;
    int64_t lo = 0, hi = 0;
    if (row_ok)
      visible_range(p.anchor, p.ctx_begin, p.ctx_len, B, is_self, blk, &lo, &hi);
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
      __syncthreads();  // previous phase is done with `red` and the stages
      if (lane == 0) {
        red[wave][0] = a;
        red[wave][1] = b;
        red[wave][2] = c;
        red[wave][3] = e;
      }
    }
    __syncthreads();
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

    SegmentWalk walk;
    if (is_self) {
      walk.init(nullptr, 0, 0, true, mlo, mhi);
    } else {
      walk.init_range(ent, 0, p.n_entries, mlo, mhi);
    }
    if (!(mlo < mhi) || !walk.next()) continue;
    int64_t p0 = walk.seg0;
    const uint16_t* kbase = static_cast<const uint16_t*>(is_self ? p.k_self : p.k);
    const uint16_t* vbase = static_cast<const uint16_t*>(is_self ? p.v_self : p.v);

    u32x4 kr[4], vr[4];
    auto tile_of = [&](int64_t pos0, int64_t* l0, int* nvalid) {
      *l0 = walk.local0 + (pos0 - walk.seg0);
      const int64_t n = walk.seg1 - pos0;
      *nvalid = int(n < KT ? n : KT);
    };
    auto load_tile = [&](int64_t l0, int nvalid) {
      const uint32_t bytes = uint32_t(nvalid - 1) * row_bytes + D * 2;
      const __amdgpu_buffer_rsrc_t kb = make_rsrc(kbase + l0 * kstride + gofs, bytes);
      const __amdgpu_buffer_rsrc_t vb = make_rsrc(vbase + l0 * kstride + gofs, bytes);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kr[i] = buffer_load16(kb, ld_off + uint32_t(16 * i) * row_bytes);
        vr[i] = buffer_load16(vb, ld_off + uint32_t(16 * i) * row_bytes);
      }
    };
    auto store_tile = [&](int stage) {
      char* kb = smem + stage * STAGE_BYTES;
      char* vb = kb + TILE_BYTES;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<u32x4*>(kb + (ld_row + 16 * i) * TP + ld_ch * 16) = kr[i];
        *reinterpret_cast<u32x4*>(vb + (ld_row + 16 * i) * TP + ld_ch * 16) = vr[i];
      }
    };

    int64_t cur_p0 = p0, cur_l0;
    int cur_n;
    tile_of(cur_p0, &cur_l0, &cur_n);
    load_tile(cur_l0, cur_n);
    store_tile(0);
    __syncthreads();
    int stage = 0;
    bool have = true;
    while (have) {
      // next tile of the walk
      int64_t nxt_p0 = cur_p0 + KT, nxt_l0 = 0;
      int nxt_n = 0;
      bool have_next = true;
      if (nxt_p0 >= walk.seg1) {
        have_next = walk.next();
        nxt_p0 = have_next ? walk.seg0 : 0;
      }
      if (have_next) {
        tile_of(nxt_p0, &nxt_l0, &nxt_n);
        load_tile(nxt_l0, nxt_n);
      }

      const char* kb = smem + stage * STAGE_BYTES;
      const char* vb = kb + TILE_BYTES;
      f32x16 s[2], dp[2];
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2) {
        s[b2] = zero16();
        dp[b2] = zero16();
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int o = k_rd + b2 * 32 * TP + 32 * t;
          s[b2] = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(kb + o)), qf[t], s[b2]);
          dp[b2] = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(vb + o)), dof[t], dp[b2]);
        }
      }
      const bool full = cur_n == KT && cur_p0 >= lmax && cur_p0 + KT <= hmin;
      int lo_rel = 0, lim = KT;
      if (!full) {
        const int64_t dl = lo - cur_p0, dh = hi - cur_p0;
        lo_rel = int(dl < -1 ? -1 : (dl > KT ? KT : dl));
        const int hi_rel = int(dh < -1 ? -1 : (dh > KT ? KT : dh));
        lim = hi_rel < cur_n ? hi_rel : cur_n;
      }
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = b2 * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          const bool vis = live && (full || (key >= lo_rel && key < lim));
          const float pv = vis ? __builtin_amdgcn_exp2f(fmaf(s[b2][v], c2, -lse2)) : 0.f;
          s[b2][v] = pv * (dp[b2][v] - dlt);  // dS
        }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 sb = pack_bf16(s[u >> 1], u & 1);
#pragma unroll
        for (int db = 0; db < 4; ++db)
          dq[db] = mfma_bf16(tr_operand(kb + tr_rd, TP, u, db * 64), sb, dq[db]);
      }

      if (have_next) store_tile(stage ^ 1);
      __syncthreads();
      stage ^= 1;
      cur_p0 = nxt_p0;
      cur_l0 = nxt_l0;
      cur_n = nxt_n;
      have = have_next;
    }
  }

  if (!row_ok) return;
  float* op = p.dq + (qi * Hq + h) * D;
  const float sc = p.scale;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = db * 32 + 8 * a + 4 * half;
      *reinterpret_cast<float4*>(op + d0) =
          make_float4(dq[db][4 * a] * sc, dq[db][4 * a + 1] * sc, dq[db][4 * a + 2] * sc,
                      dq[db][4 * a + 3] * sc);
    }
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream) {
  const int64_t n_q = int64_t(p.n_blocks) * p.block_size;
  const int64_t n_rows = n_q * p.n_q_heads;
  if (n_rows > 0) {
    const int64_t blocks = (n_rows + (THREADS / 32) - 1) / (THREADS / 32);
    hipLaunchKernelGGL(bwd_delta_kernel, dim3(unsigned(blocks)), dim3(THREADS), 0, stream, p.o,
                       static_cast<const uint16_t*>(p.d_o), p.delta, n_rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t n_ctx_tiles = (p.n_local + KV_KEYS - 1) / KV_KEYS;
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
  const int G = p.n_q_heads / p.n_kv_heads;
  const int64_t q_tiles = (n_q * G + QROWS - 1) / QROWS;
  const int64_t q_grid = q_tiles * p.n_kv_heads;
  if (q_grid > 0x7fffffff) return hipErrorInvalidValue;
  if (q_grid > 0) {
    hipLaunchKernelGGL(bwd_dq_kernel, dim3(unsigned(q_grid)), dim3(THREADS), 0, stream, p,
                       int(q_tiles));
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace bsx
