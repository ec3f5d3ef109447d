// Device helpers and internal launcher declarations shared by the library's HIP sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace f2i {

constexpr int kWave = 64;

// bf16 <-> fp32.  bf16 is the upper half of an fp32 bit pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (quiet NaN kept).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Stores one fp32 value as the output dtype.
__device__ __forceinline__ void store_out(float* y, int64_t idx, float v) { y[idx] = v; }
__device__ __forceinline__ void store_out(uint16_t* y, int64_t idx, float v) { y[idx] = f32_to_bf16_rne(v); }

}  // namespace f2i

// ---- internal launchers (host side), implemented in the .hip files ----
namespace f2i {
// One GEMV of a grouped launch (all items share m, T, B and the dtypes).
struct GemvItem {
  const void* packed;
  const float* scales;
  const void* x;
  void* y;
  int n;
};
constexpr int kMaxGroup = 48;   // items per launch; the table travels in the kernel arguments
struct GemvGroup {
  int count;
  int tile_start[kMaxGroup + 1];   // first 16-row tile of each item; [count] = total tiles
  GemvItem items[kMaxGroup];
};
hipError_t launch_gemv_mfma_group(const GemvGroup& grp, int m, int T, int B, int y_bf16, hipStream_t s);
hipError_t launch_quantize(const float* R, int n, int m, int T, uint8_t* packed, float* scales,
                           double* scales64, uint8_t* codes, hipStream_t s);
hipError_t launch_pack(const uint8_t* codes, int n, int m, int T, uint8_t* packed, hipStream_t s);
hipError_t launch_gemv_valu(const uint8_t* packed, const float* scales, int n, int m, int T,
                            const void* x, int x_bf16, int B, void* y, int y_bf16, hipStream_t s);
hipError_t launch_gemv_mfma(const uint8_t* packed, const float* scales, int n, int m, int T,
                            const void* x, int B, void* y, int y_bf16, void* unused, hipStream_t s);
hipError_t launch_gemv_i8(const uint8_t* packed, const float* scales, int n, int m, int T,
                          const void* x, int B, void* y, int y_bf16, hipStream_t s);
hipError_t launch_act_quant(const void* x, int x_bf16, int N, int two_m, int8_t* q, float* delta,
                            hipStream_t s);
hipError_t launch_gemm(const uint8_t* packed, const float* scales, int n, int m, int T,
                       const int8_t* q, const float* delta, int N, void* y, int y_mode,
                       hipStream_t s);
}  // namespace f2i
