// Dequantize a packed layer back to its real form: R^ = realform(sum_t U~(t), sum_t W~(t)).
//
// Sources: zhichai.net reading note, "Step 2" dequantization (w^ = s_re b_re + i s_im b_im) and
// "Step 3" (the layer is the sum of its T stage terms); "Step 1" / ModelScope card "Fairy2i-W2",
// "Method" (the widely-linear map y = U x + W conj(x) of a real layer R).  Expanding U x +
// W conj(x) with x = a + ib gives the real blocks
//     R11 = Re U + Re W   R12 = Im W - Im U   R21 = Im U + Im W   R22 = Re U - Re W.
// This is the forward pass of quantization-aware training (fake quantization) and a third
// route to the layer's map, next to the decode GEMV and the prefill GEMM.
//
// One workgroup of 256 threads per complex row i; thread l handles columns 4l.., 4l+1024.., so
// every packed word read gives it codes j..j+3 in one shift and one mask, and each of the four
// blocks is written with one 16-byte (fp32) or 8-byte (bf16) store.  Per (j, stage) the sums
// run over t in order in fp32: Re U = sum_t (code re-axis ? +-s_re(t) : 0), and likewise.
#include "common.hpp"

namespace f2i {

template <typename OT> struct Store4;
// The real form is written once and not read back by this kernel: non-temporal stores.
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef unsigned v2u_t __attribute__((ext_vector_type(2)));
template <> struct Store4<float> {
  __device__ static void run(float* p, const float* v) {
    __builtin_nontemporal_store(v4f_t{v[0], v[1], v[2], v[3]}, reinterpret_cast<v4f_t*>(p));
  }
};
template <> struct Store4<uint16_t> {
  __device__ static void run(uint16_t* p, const float* v) {
    __builtin_nontemporal_store(
        v2u_t{(uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16),
              (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16)},
        reinterpret_cast<v2u_t*>(p));
  }
};

template <typename OT>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ packed,
                                                 const float* __restrict__ scales, int n, int m, int T,
                                                 OT* __restrict__ R) {
  const int i = blockIdx.x;
  const uint32_t* __restrict__ words = reinterpret_cast<const uint32_t*>(packed);
  const float* __restrict__ sc = scales + (int64_t)i * T * 4;
  const int64_t ld = 2 * (int64_t)m;
  OT* __restrict__ r11 = R + (int64_t)i * ld;             // row i:   [R11 | R12]
  OT* __restrict__ r21 = R + (int64_t)(n + i) * ld;       // row n+i: [R21 | R22]
  for (int j = 4 * threadIdx.x; j < m; j += 4 * 256) {
    float ur[4] = {0.f, 0.f, 0.f, 0.f}, ui[4] = {0.f, 0.f, 0.f, 0.f};
    float wr[4] = {0.f, 0.f, 0.f, 0.f}, wi[4] = {0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int M = 0; M < 2; ++M) {
        const float s_re = sc[(t * 2 + M) * 2], s_im = sc[(t * 2 + M) * 2 + 1];
        const uint32_t w = words[tiled_word(i, t * 2 + M, j >> 4, m, T)];
        const uint32_t k4 = (w >> (2 * ((j & 15) >> 2))) & 0x03030303u;   // codes j..j+3 in bytes
        float* re = M == 0 ? ur : wr;
        float* im = M == 0 ? ui : wi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t k = (k4 >> (8 * e)) & 3u;
          re[e] += k == 0 ? s_re : k == 2 ? -s_re : 0.f;
          im[e] += k == 1 ? s_im : k == 3 ? -s_im : 0.f;
        }
      }
    }
    float b11[4], b12[4], b21[4], b22[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      b11[e] = ur[e] + wr[e];
      b12[e] = wi[e] - ui[e];
      b21[e] = ui[e] + wi[e];
      b22[e] = ur[e] - wr[e];
    }
    Store4<OT>::run(r11 + j, b11);
    Store4<OT>::run(r11 + m + j, b12);
    Store4<OT>::run(r21 + j, b21);
    Store4<OT>::run(r21 + m + j, b22);
  }
}

hipError_t launch_dequant(const uint8_t* packed, const float* scales, int n, int m, int T, void* R,
                          int r_bf16, hipStream_t s) {
  if (r_bf16)
    hipLaunchKernelGGL(k_dequant<uint16_t>, dim3(n), dim3(256), 0, s, packed, scales, n, m, T,
                       static_cast<uint16_t*>(R));
  else
    hipLaunchKernelGGL(k_dequant<float>, dim3(n), dim3(256), 0, s, packed, scales, n, m, T,
                       static_cast<float*>(R));
  return hipGetLastError();
}

}  // namespace f2i
