// Stochastic rounding of the SGD step onto E's storage grid (FP8 E4M3FN or bf16), shared by
// the chunked GEMM's SGD epilogue and the whole-row SGD product. The uniform of element
// (v, d) is 16 bits of a Philox-4x32-10 block keyed by the caller's seed: counter
// (d / 8, v low, v high, 0), half-word d % 8, so any thread layout draws the same bits.
#pragma once
#include "common.h"

namespace cl {

// Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011): four 32-bit counter words, a
// two-word key bumped by the Weyl constants between rounds, two 32x32 -> 64-bit products
// per round.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0], p1 = (uint64_t)0xCD9E8D57u * c[2];   // one v_mad_u64_u32 each
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
  }
}

// Stochastic rounding of y onto a storage grid given its neighbours in magnitude,
// lo_m <= |y| < lo_m + step (lo_m, step, |y| - lo_m exact): y goes to the upper neighbour
// on the real line when u step < y - lo, u = h / 2^16. Zero results are +0.
// (y on the grid: frac = 0 keeps lo_m = |y| on both sides, since u step < step)
__device__ __forceinline__ float sr_pick(float y, float lo_m, float step, uint32_t h) {
  const float m = __builtin_fabsf(y);
  const float frac = m - lo_m;
  const float us = (float)h * (1.0f / 65536.0f) * step;
  const bool up = y >= 0.0f ? us < frac : !(us < step - frac);   // magnitude rounds up
  const float mag = up ? lo_m + step : lo_m;
  return mag == 0.0f ? 0.0f : __builtin_copysignf(mag, y);
}
// OCP E4M3FN: saturate to +-448; spacing 2^-9 below 2^-6, else 3 mantissa bits
__device__ __forceinline__ float sr_fp8(float y, uint32_t h) {
  y = __builtin_amdgcn_fmed3f(y, -kFp8Max, kFp8Max);
  const float m = __builtin_fabsf(y);
  const uint32_t b = __float_as_uint(m);
  const bool sub = m < 0.015625f;
  const float lo_m = sub ? __builtin_floorf(m * 512.0f) * (1.0f / 512.0f) : __uint_as_float(b & 0xFFF00000u);
  const float step = sub ? 1.0f / 512.0f : __uint_as_float((b & 0x7F800000u) - (3u << 23));
  return sr_pick(y, lo_m, step, h);
}
// bf16: 7 stored mantissa bits (finite, normal magnitudes)
__device__ __forceinline__ float sr_bf16(float y, uint32_t h) {
  const uint32_t b = __float_as_uint(__builtin_fabsf(y)) & 0xFFFF0000u;
  const float lo_m = __uint_as_float(b);
  return sr_pick(y, lo_m, __uint_as_float(b + 0x10000u) - lo_m, h);
}

// the 16 uniforms of columns d0 .. d0 + 15 (d0 a multiple of 16) of item v: half-word j of hw
__device__ __forceinline__ void sr_uniforms16(uint64_t seed, int64_t v, int64_t d0, uint32_t (&hw)[8]) {
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  uint32_t c0[4] = {(uint32_t)(d0 >> 3), (uint32_t)v, (uint32_t)((uint64_t)v >> 32), 0u};
  uint32_t c1[4] = {(uint32_t)(d0 >> 3) + 1u, (uint32_t)v, (uint32_t)((uint64_t)v >> 32), 0u};
  philox4x32_10(c0, k0, k1);
  philox4x32_10(c1, k0, k1);
#pragma unroll
  for (int q = 0; q < 4; ++q) { hw[q] = c0[q]; hw[4 + q] = c1[q]; }
}
__device__ __forceinline__ uint32_t sr_h16(const uint32_t (&hw)[8], int j) {
  return (j & 1) ? (hw[j >> 1] >> 16) : (hw[j >> 1] & 0xFFFFu);
}

}  // namespace cl
