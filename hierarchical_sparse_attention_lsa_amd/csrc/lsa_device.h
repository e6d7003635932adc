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

// Exclusive prefix sum over a wave; returns the wave total in *total.
__device__ __forceinline__ int wave_excl_scan(int x, int* total) {
  const int l = lane_id();
  int s = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(s, d);
    if (l >= d) s += y;
  }
  *total = __shfl(s, 63);
  return s - x;
}

}  // namespace lsa
