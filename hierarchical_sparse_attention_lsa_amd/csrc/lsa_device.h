// Device-side helpers shared by the LSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsa {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Round-half-even of the exact quotient s / n (n > 0), for signed s.
__device__ __forceinline__ int rhe_div(int s, int n) {
  int q = s / n;
  int r = s - q * n;
  if (r < 0) { q -= 1; r += n; }
  const int twice = 2 * r;
  return q + ((twice > n) | ((twice == n) & (q & 1)));
}

// int8 x int8 -> int32, 16x16 output tile, 64-deep contraction.  Lane l
// supplies row (l % 16) of A and column (l % 16) of B, bytes
// 16*(l/16) .. +15 of the 64-deep dot product (same split for A and B, so
// the contraction is complete whatever the hardware's k order).  Output:
// lane l holds D[4*(l/16) + v][l % 16], v = 0..3.
__device__ __forceinline__ v4i mfma_i8_16x16x64(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// bf16 x bf16 -> f32, 16x16 tile, 32-deep: lane l supplies row/col (l % 16),
// elements 8*(l/16) .. +7.
__device__ __forceinline__ v4f mfma_bf16_16x16x32(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// bf16 x bf16 -> f32, 16x16 tile, 16-deep: lane l supplies row/col (l % 16),
// elements 4*(l/16) .. +3.
__device__ __forceinline__ v4f mfma_bf16_16x16x16(v4s a, v4s b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// float -> bf16 bits, round to nearest even (inputs are finite here).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ long long shfl_xor_i64(long long v, int m) {
  int lo = __shfl_xor((int)(v & 0xffffffffll), m);
  int hi = __shfl_xor((int)(v >> 32), m);
  return ((long long)hi << 32) | (unsigned int)lo;
}

// Wave-wide inclusive scans on DPP lane moves (VALU, no LDS crossbar):
// shifts by 1, 2, 4, 8 inside each 16-lane row, then row 1 and 3 take the
// last lane of the row before (row_bcast:15) and rows 2 and 3 lane 31
// (row_bcast:31).  Lanes whose source is outside the row, or whose row is
// masked off, receive `id`.  Every lane of the wave must be active.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_move(int id, int x) {
  return __builtin_amdgcn_update_dpp(id, x, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ long long dpp_move(long long id, long long x) {
  const int lo = dpp_move<CTRL, ROWS>((int)(id & 0xffffffffll), (int)(x & 0xffffffffll));
  const int hi = dpp_move<CTRL, ROWS>((int)(id >> 32), (int)(x >> 32));
  return ((long long)hi << 32) | (unsigned int)lo;
}
template <class T, class Op>
__device__ __forceinline__ T wave_incl_scan(T x, T id, Op op) {
  x = op(x, dpp_move<0x111, 0xf>(id, x));
  x = op(x, dpp_move<0x112, 0xf>(id, x));
  x = op(x, dpp_move<0x114, 0xf>(id, x));
  x = op(x, dpp_move<0x118, 0xf>(id, x));
  x = op(x, dpp_move<0x142, 0xa>(id, x));
  x = op(x, dpp_move<0x143, 0xc>(id, x));
  return x;
}
__device__ __forceinline__ int lane63(int x) { return __builtin_amdgcn_readlane(x, 63); }
__device__ __forceinline__ long long lane63(long long x) {
  const int lo = __builtin_amdgcn_readlane((int)(x & 0xffffffffll), 63);
  const int hi = __builtin_amdgcn_readlane((int)(x >> 32), 63);
  return ((long long)hi << 32) | (unsigned int)lo;
}

// Exclusive prefix sum over a wave; returns the wave total in *total.
__device__ __forceinline__ int wave_excl_scan(int x, int* total) {
  const int s = wave_incl_scan(x, 0, [](int a, int b) { return a + b; });
  *total = lane63(s);
  return s - x;
}

}  // namespace lsa
