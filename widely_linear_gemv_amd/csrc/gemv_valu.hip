// Decode GEMV on the vector ALUs: y = sum_t U~(t) x + W~(t) conj(x) with every code an add,
// a subtract or a real/imaginary swap with sign -- no weight multiplications.
//
// Sources: ModelScope card "Fairy2i-W2", "Method" (y = U x + W conj(x)); zhichai.net reading
// note, "Step 2" dequantization (s_re b_re + i s_im b_im) and "Industry implications:
// multiplication-free inference" (B_re, B_im in {-1, 0, 1}; a product with +-i swaps real and
// imaginary parts with a sign flip); 36Kr article, parallel stages (the T terms are data
// independent and summed).
//
// One wave per complex row.  Lane l reads packed words l, l+64, ... of each (stage, matrix)
// plane -- 16 codes each (code p of a word in bits 8*(p%4) + 2*(p/4)), found through the
// tiled word order of the packed form -- and the 16 matching x values.  For each code it negates
// the (a, b) pair when the sign bit is set and adds it to the real-axis or imaginary-axis
// accumulator; the scales of that plane multiply the accumulated sums once per lane, and the
// wave reduces the per-lane outputs with cross-lane adds at the end.  All sums are fp32.
// This kernel is exact up to fp32 rounding for fp32 and bf16 x and is the reference GPU path;
// the MFMA kernel is the fast path for bf16 x.
#include "common.hpp"

namespace f2i {

constexpr int kSegWords = 8;      // packed words per lane and row segment (64 * 8 * 16 = 8192 columns)

template <typename XT> struct XLoad;
template <> struct XLoad<float> {
  __device__ static void load16(const float* p, float* v) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float4 f = reinterpret_cast<const float4*>(p)[h];
      v[4 * h] = f.x; v[4 * h + 1] = f.y; v[4 * h + 2] = f.z; v[4 * h + 3] = f.w;
    }
  }
};
template <> struct XLoad<uint16_t> {
  __device__ static void load16(const uint16_t* p, float* v) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 w = reinterpret_cast<const uint4*>(p)[h];
      v[8 * h + 0] = bf16_lo(w.x); v[8 * h + 1] = bf16_hi(w.x);
      v[8 * h + 2] = bf16_lo(w.y); v[8 * h + 3] = bf16_hi(w.y);
      v[8 * h + 4] = bf16_lo(w.z); v[8 * h + 5] = bf16_hi(w.z);
      v[8 * h + 6] = bf16_lo(w.w); v[8 * h + 7] = bf16_hi(w.w);
    }
  }
};

template <typename XT, typename YT, int NB>
__global__ __launch_bounds__(256) void k_gemv_valu(const uint8_t* __restrict__ packed,
                                                   const float* __restrict__ scales, int n, int m,
                                                   int T, const XT* __restrict__ x, int B,
                                                   YT* __restrict__ y) {
  const int lane = threadIdx.x & (kWave - 1);
  const int i = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (i >= n) return;                       // the whole wave leaves together
  const int dw_plane = m / 16;
  const uint32_t* __restrict__ words = reinterpret_cast<const uint32_t*>(packed);
  const int64_t xs = 2 * (int64_t)m;        // x row stride
  const int64_t ys = 2 * (int64_t)n;

  for (int b0 = 0; b0 < B; b0 += NB) {
    float yr[NB], yi[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) { yr[b] = 0.f; yi[b] = 0.f; }
    for (int t = 0; t < T; ++t) {
      for (int M = 0; M < 2; ++M) {
        const int64_t so = (((int64_t)i * T + t) * 2 + M) * 2;
        const float s_re = scales[so], s_im = scales[so + 1];
        // Segments of kSegWords words per lane (8192 columns): each segment's axis sums are
        // applied to the scales and added to the outputs, so no fp32 sum of a long row runs over
        // more than 128 codes or m / 8192 segments in series.  Rows of up to 8192 columns are
        // one segment.
        for (int q0 = 0; q0 < dw_plane; q0 += kWave * kSegWords) {
          const int q1 = min(dw_plane, q0 + kWave * kSegWords);
          // per-axis sums of +-a and +-b (a = Re x, b = Im x) over this segment's codes
          float ra[NB], rb[NB], ia[NB], ib[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) { ra[b] = rb[b] = ia[b] = ib[b] = 0.f; }
          for (int q = q0 + lane; q < q1; q += kWave) {
            const uint32_t w = words[tiled_word(i, t * 2 + M, q, m, T)];
            const int j0 = q * 16;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              const int bb = b0 + b < B ? b0 + b : B - 1;    // padded columns repeat the last one
              float xa[16], xb[16];
              XLoad<XT>::load16(x + bb * xs + j0, xa);
              XLoad<XT>::load16(x + bb * xs + m + j0, xb);
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const uint32_t k = (w >> (8 * (r & 3) + 2 * (r >> 2))) & 3u;   // code j0 + r
                const uint32_t sgn = (k & 2u) << 30;          // code 2 or 3: negate
                const float va = __uint_as_float(__float_as_uint(xa[r]) ^ sgn);
                const float vb = __uint_as_float(__float_as_uint(xb[r]) ^ sgn);
                const bool on_im = (k & 1u) != 0;              // code 1 or 3: imaginary axis
                ra[b] += on_im ? 0.f : va;
                rb[b] += on_im ? 0.f : vb;
                ia[b] += on_im ? va : 0.f;
                ib[b] += on_im ? vb : 0.f;
              }
            }
          }
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            if (M == 0) {   // U x:       Re = s_re*ra - s_im*ib ; Im = s_re*rb + s_im*ia
              yr[b] += s_re * ra[b] - s_im * ib[b];
              yi[b] += s_re * rb[b] + s_im * ia[b];
            } else {        // W conj(x): Re = s_re*ra + s_im*ib ; Im = s_im*ia - s_re*rb
              yr[b] += s_re * ra[b] + s_im * ib[b];
              yi[b] += s_im * ia[b] - s_re * rb[b];
            }
          }
        }
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float vr = wave_sum(yr[b]);
      const float vi = wave_sum(yi[b]);
      if (lane == 0 && b0 + b < B) {
        store_out(y, (int64_t)(b0 + b) * ys + i, vr);
        store_out(y, (int64_t)(b0 + b) * ys + n + i, vi);
      }
    }
  }
}

hipError_t launch_gemv_valu(const uint8_t* packed, const float* scales, int n, int m, int T,
                            const void* x, int x_bf16, int B, void* y, int y_bf16, hipStream_t s) {
  const dim3 block(256), grid((n + 3) / 4);
#define F2I_GEMV_VALU(XT, YT, NB)                                                              \
  hipLaunchKernelGGL((k_gemv_valu<XT, YT, NB>), grid, block, 0, s, packed, scales, n, m, T,   \
                     static_cast<const XT*>(x), B, static_cast<YT*>(y))
  const bool wide = B >= 4;
  if (!x_bf16 && !y_bf16) { if (wide) F2I_GEMV_VALU(float, float, 4); else F2I_GEMV_VALU(float, float, 1); }
  else if (!x_bf16 && y_bf16) { if (wide) F2I_GEMV_VALU(float, uint16_t, 4); else F2I_GEMV_VALU(float, uint16_t, 1); }
  else if (x_bf16 && !y_bf16) { if (wide) F2I_GEMV_VALU(uint16_t, float, 4); else F2I_GEMV_VALU(uint16_t, float, 1); }
  else { if (wide) F2I_GEMV_VALU(uint16_t, uint16_t, 4); else F2I_GEMV_VALU(uint16_t, uint16_t, 1); }
#undef F2I_GEMV_VALU
  return hipGetLastError();
}

}  // namespace f2i
