// Device helpers shared by the digit forms of decode activations (int8 and fp6 digits).
#pragma once

#include "common.hpp"

namespace f2i {

constexpr int kDigitHeader = 64;     // bytes before the digits: int32 [B, m, S_0 .. S_{B-1}]

// Power-of-two exponent S with amax * 2^S in [2^21, 2^22) (0 for an all-zero column).
__device__ __forceinline__ int digit_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127;   // floor(log2 amax), normal
  return 21 - (e < -126 ? -126 : e);
}

// Eight consecutive activations as fp32 (bf16 widened exactly).
template <typename XT> struct Load8x;
template <> struct Load8x<float> {
  __device__ static void run(const float* p, float* v) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};
template <> struct Load8x<uint16_t> {
  __device__ static void run(const uint16_t* p, float* v) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  }
};

// max |x[0..len)| over a workgroup of NT threads (order-free, exact); len % 8 == 0.  Thread
// tid's first eight values are left in keep[] (the caller reuses them when len <= 8 * NT).
template <typename XT, int NT>
__device__ __forceinline__ float column_amax(const XT* __restrict__ xb, int len, float keep[8],
                                             float* s_max) {
  float amax = 0.f;
  for (int j = threadIdx.x * 8; j < len; j += NT * 8) {
    float v[8];
    Load8x<XT>::run(xb + j, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) { amax = fmaxf(amax, fabsf(v[e])); keep[e] = v[e]; }
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & (kWave - 1)) == 0) s_max[threadIdx.x / kWave] = amax;
  __syncthreads();
  amax = 0.f;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) amax = fmaxf(amax, s_max[w]);
  return amax;
}

}  // namespace f2i
