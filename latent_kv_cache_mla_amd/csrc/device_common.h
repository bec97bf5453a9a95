// device_common.h — small device helpers shared by the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// OCP e4m3fn code -> fp32 from the field definitions: exponent bias 7,
// exponent field 0 = subnormal m/8 * 2^-6, S.1111.111 = NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v = (e == 0) ? static_cast<float>(m) * (1.0f / 512.0f)
                     : __uint_as_float(((e + 120u) << 23) | (m << 20));
  if (e == 15u && m == 7u) v = __uint_as_float(0x7FC00000u);
  return (c & 0x80u) ? -v : v;
}

// floor(a / d) for 0 <= a, 0 < d: a double-precision estimate corrected to
// the exact integer (the integer division it replaces is a long instruction
// sequence on this hardware)
__device__ __forceinline__ int64_t floordiv_dev(int64_t a, int64_t d) {
  int64_t q = static_cast<int64_t>(static_cast<double>(a) / static_cast<double>(d));
  while (q > 0 && q * d > a) --q;
  while ((q + 1) * d <= a) ++q;
  return q;
}

// range_begin and range_of_page of partition.h, with floordiv_dev
__device__ __forceinline__ int64_t range_begin_dev(int64_t g, int64_t P, int64_t G) {
  return floordiv_dev(g * P, G);
}
__device__ __forceinline__ int64_t range_of_page_dev(int64_t x, int64_t P, int64_t G) {
  const int64_t g = floordiv_dev((x + 1) * G + P - 1, P) - 1;
  return g < G - 1 ? g : G - 1;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// RoPE angle of pair k at position pos, in double precision so that large
// positions keep their phase (pos * theta^(-2k/d)).
__device__ __forceinline__ void rope_cs(int pos, int k, int d, double theta, float* c, float* s) {
  const double ang = static_cast<double>(pos) * pow(theta, -2.0 * k / d);
  double sd, cd;
  sincos(ang, &sd, &cd);
  *c = static_cast<float>(cd);
  *s = static_cast<float>(sd);
}

// Effective length of sequence b: negative lengths count as empty and no
// sequence may extend past its block-table row (so the table is never read
// out of bounds, whatever the device contents).
__device__ __forceinline__ int clamp_len(int s, int max_blocks) {
  s = s < 0 ? 0 : s;
  const int cap = max_blocks * 64;
  return s > cap ? cap : s;
}

}  // namespace mla
