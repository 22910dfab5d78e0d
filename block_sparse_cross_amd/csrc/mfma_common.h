// Shared gfx950 helpers of the bf16 matrix-core kernels: vector types, buffer
// resources, wave-uniform values, and the LDS transpose read.
//
// Conventions for v_mfma_f32_32x32x16_bf16 (D = A B + C, M = N = 32, K = 16):
//   A operand: lane l holds A[m = l % 32][k = 8 * (l / 32) .. + 8]
//   B operand: lane l holds B[k = 8 * (l / 32) .. + 8][n = l % 32]
//   D:         lane l holds column n = l % 32, rows 8 * (v / 4) + 4 * (l / 32) + v % 4
//              for accumulator element v = 0 .. 15.
// A product whose K dimension is the row index of an accumulator therefore takes
// its 8 k-values per lane from elements v = 8u .. 8u + 7 of that accumulator, i.e.
// rows 16u + 8 * (e / 4) + 4 * half + e % 4 for e = 0 .. 7; the matching operand is
// read from LDS in that same row order with two transpose loads of 4 rows each.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ inline int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x)));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x) >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

// Raw buffer resource over [base, base + bytes): loads past the end read as zero.
// `base` and `bytes` must be the same in every lane; they are moved to scalar
// registers explicitly, because after a divergent branch the compiler may no
// longer prove them uniform and would wrap each load in a per-lane loop.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const int64_t b = uniform64(reinterpret_cast<int64_t>(base));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(b), (short)0, (int)n,
                                           0x00020000);
}

__device__ inline u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ inline bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ inline f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int v = 0; v < 16; ++v) z[v] = 0.f;
  return z;
}

// Transposed A operand (32 columns x 8 rows of a row-major bf16 LDS tile) for the
// k-block `u`: `base` is the lane's address from tr_lane_offset, `pitch` the row
// pitch in bytes, `col_bytes` the byte offset of the 32-column block.
__device__ inline bf16x8 tr_operand(const char* base, int pitch, int u, int col_bytes) {
  const char* a = base + 16 * u * pitch + col_bytes;
  const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a));
  const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a + 8 * pitch));
  return bf16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane j supplies the address of
// 4 consecutive elements of row j / 4, columns 4 * (j % 4) .. + 3, of a 4 x 16 block,
// and lane i receives column i of that block.  This is the lane's byte offset for
// rows 4 * half + (j / 4) (and + 8 for the second read) and columns
// 16 * (group % 2) + 4 * (j % 4) of a 32-column block.
__device__ inline int tr_lane_offset(int lane, int pitch) {
  const int j = lane & 15, grp = lane >> 4, half = lane >> 5;
  return (4 * half + (j >> 2)) * pitch + (16 * (grp & 1) + 4 * (j & 3)) * 2;
}

__device__ inline bf16x8 pack_bf16(const f32x16& s, int u) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(s[8 * u + e]);
  return r;
}

}  // namespace bsx
