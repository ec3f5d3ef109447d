// Prefill: per-token int8 activations and the ternary-plane int8 MFMA GEMM.
//
// Sources: zhichai.net reading note, "Industry implications: multiplication-free inference"
// (B_re, B_im in {-1, 0, 1}: the product reduces to additions, subtractions and skips);
// ModelScope card "Fairy2i-W2", "Method" (y = U x + W conj(x), each matrix a sum of T
// quantized terms); 36Kr article, parallel stages.  The per-token int8 activation format is
// not on the pages; it is the plainest way to run the batched product on integer matrix
// cores, and its rounding is fixed exactly (see the header).
//
// GEMM: output rows are (complex row i, stage t, matrix M, plane), output columns are
// (token, component a = Re x or b = Im x).  Each wave owns 16 complex rows and 8*NF tokens.
// Per 64-column step a lane reads one 32-bit code word per (t, M) -- 16 codes of its row --
// spreads the codes into bytes with a shift and a mask (the packed layout puts codes
// b, b+4, b+8, b+12 in byte b), and maps each byte through a 4-entry table with v_perm_b32
// into the int8 planes B_re and B_im.  Each plane and 16-column activation fragment feeds one
// v_mfma_i32_16x16x64_i8; every sum is exact in int32 (|P| <= 127 m).  The epilogue applies
// the fp32 scales once per accumulated sum and the token's delta once per output.
#include "common.hpp"

namespace f2i {

typedef int v4i __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ act quant ----

template <typename XT> struct Load8;
template <> struct Load8<float> {
  __device__ static void run(const float* p, float* v) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};
template <> struct Load8<uint16_t> {
  __device__ static void run(const uint16_t* p, float* v) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  }
};

// One workgroup per token: amax (order-free, exact), delta = amax / 127 (IEEE fp32 divide),
// q = clamp(rint(x / delta)) with rint rounding half to even.
template <typename XT>
__global__ __launch_bounds__(256) void k_act_quant(const XT* __restrict__ x, int two_m,
                                                   int8_t* __restrict__ q,
                                                   float* __restrict__ delta) {
  __shared__ float s_max[256 / kWave];
  const int tok = blockIdx.x;
  const XT* __restrict__ xr = x + (int64_t)tok * two_m;
  int8_t* __restrict__ qr = q + (int64_t)tok * two_m;
  float amax = 0.f;
  for (int j = threadIdx.x * 8; j < two_m; j += 256 * 8) {
    float v[8];
    Load8<XT>::run(xr + j, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & (kWave - 1)) == 0) s_max[threadIdx.x / kWave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float d = amax / 127.0f;
  for (int j = threadIdx.x * 8; j < two_m; j += 256 * 8) {
    float v[8];
    Load8<XT>::run(xr + j, v);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int qi = 0;
      if (d != 0.f) qi = (int)fminf(fmaxf(rintf(v[e] / d), -127.f), 127.f);
      const uint32_t byte = (uint32_t)(qi & 0xFF);
      if (e < 4) lo |= byte << (8 * e); else hi |= byte << (8 * (e - 4));
    }
    *reinterpret_cast<uint2*>(qr + j) = make_uint2(lo, hi);
  }
  if (threadIdx.x == 0) delta[tok] = d;
}

hipError_t launch_act_quant(const void* x, int x_bf16, int N, int two_m, int8_t* q, float* delta,
                            hipStream_t s) {
  if (x_bf16)
    hipLaunchKernelGGL(k_act_quant<uint16_t>, dim3(N), dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), two_m, q, delta);
  else
    hipLaunchKernelGGL(k_act_quant<float>, dim3(N), dim3(256), 0, s,
                       static_cast<const float*>(x), two_m, q, delta);
  return hipGetLastError();
}

// ----------------------------------------------------------------------- GEMM ----

// 16 codes (one packed word) -> int8 planes B_re and B_im in column order.
__device__ __forceinline__ void decode_planes(uint32_t D, v4i& re, v4i& im) {
  constexpr uint32_t lo2 = 0x03030303u;
  constexpr uint32_t kRe = 0x00FF0001u;   // code 0 -> +1, 1 -> 0, 2 -> -1, 3 -> 0
  constexpr uint32_t kIm = 0xFF000100u;   // code 0 -> 0, 1 -> +1, 2 -> 0, 3 -> -1
  const uint32_t k0 = D & lo2, k1 = (D >> 2) & lo2, k2 = (D >> 4) & lo2, k3 = (D >> 6) & lo2;
  re = v4i{(int)__builtin_amdgcn_perm(0u, kRe, k0), (int)__builtin_amdgcn_perm(0u, kRe, k1),
           (int)__builtin_amdgcn_perm(0u, kRe, k2), (int)__builtin_amdgcn_perm(0u, kRe, k3)};
  im = v4i{(int)__builtin_amdgcn_perm(0u, kIm, k0), (int)__builtin_amdgcn_perm(0u, kIm, k1),
           (int)__builtin_amdgcn_perm(0u, kIm, k2), (int)__builtin_amdgcn_perm(0u, kIm, k3)};
}

enum { kOutF32 = 0, kOutBF16 = 1, kOutRaw = 2 };

// Workgroup = 4 waves = 2 row blocks x 2 token blocks (16 complex rows x 8*NF tokens each).
template <int TT, int NF, int MODE>
__global__ __launch_bounds__(256) void k_gemm(const uint8_t* __restrict__ packed,
                                              const float* __restrict__ scales, int n, int m,
                                              const int8_t* __restrict__ q,
                                              const float* __restrict__ delta, int N,
                                              void* __restrict__ yv) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15;          // A row / B column inside a 16x16 tile
  const int g = lane >> 4;          // 16-column group of the 64-column step
  const int i0 = (blockIdx.x * 2 + (wave & 1)) * 16;
  const int tok0 = (blockIdx.y * 2 + (wave >> 1)) * (8 * NF);
  if (i0 >= n || tok0 >= N) return;   // whole wave; no workgroup barrier below

  const int dw_plane = m / 16;
  const int ia = i0 + r;
  const bool a_ok = ia < n;
  const uint32_t* __restrict__ arow =
      reinterpret_cast<const uint32_t*>(packed) + (int64_t)(a_ok ? ia : 0) * (TT * 2 * dw_plane);
  const int64_t two_m = 2 * (int64_t)m;

  const int8_t* bptr[NF];
  bool b_ok[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int tok = tok0 + 8 * f + (r >> 1);
    b_ok[f] = tok < N;
    bptr[f] = q + (int64_t)(b_ok[f] ? tok : 0) * two_m + (r & 1) * (int64_t)m + 16 * g;
  }

  v4i acc[TT][2][2][NF];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int M = 0; M < 2; ++M)
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[t][M][p][f] = v4i{0, 0, 0, 0};

  const int ksteps = m / 64;
  for (int kk = 0; kk < ksteps; ++kk) {
    v4i A[TT][2][2];
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int M = 0; M < 2; ++M) {
        const uint32_t D = a_ok ? arow[(t * 2 + M) * dw_plane + 4 * kk + g] : 0u;
        decode_planes(D, A[t][M][0], A[t][M][1]);
      }
    v4i Bf[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f)
      Bf[f] = b_ok[f] ? *reinterpret_cast<const v4i*>(bptr[f] + 64 * kk) : v4i{0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int M = 0; M < 2; ++M)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int f = 0; f < NF; ++f)
            acc[t][M][p][f] =
                __builtin_amdgcn_mfma_i32_16x16x64_i8(A[t][M][p], Bf[f], acc[t][M][p][f], 0, 0, 0);
  }

  // C layout of a 16x16 tile: lane holds rows 4g..4g+3 of column r.
  const int comp = r & 1;
  if constexpr (MODE == kOutRaw) {
    int* __restrict__ P = static_cast<int*>(yv);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int tok = tok0 + 8 * f + (r >> 1);
      if (!b_ok[f]) continue;
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int M = 0; M < 2; ++M)
#pragma unroll
          for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = i0 + 4 * g + e;
              if (i < n)
                P[((((int64_t)(t * 2 + M) * 2 + p) * 2 + comp) * N + tok) * n + i] =
                    acc[t][M][p][f][e];
            }
    }
  } else {
    const int64_t ys = 2 * (int64_t)n;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = i0 + 4 * g + e;
      const bool i_ok = i < n;
      float s[TT][2][2];
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int M = 0; M < 2; ++M)
#pragma unroll
          for (int ax = 0; ax < 2; ++ax)
            s[t][M][ax] = i_ok ? scales[(((int64_t)i * TT + t) * 2 + M) * 2 + ax] : 0.f;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        float vre = 0.f, vim = 0.f;
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const float PUr = (float)acc[t][0][0][f][e], PUi = (float)acc[t][0][1][f][e];
          const float PWr = (float)acc[t][1][0][f][e], PWi = (float)acc[t][1][1][f][e];
          if (comp == 0) {   // column a = Re x
            vre += s[t][0][0] * PUr + s[t][1][0] * PWr;
            vim += s[t][0][1] * PUi + s[t][1][1] * PWi;
          } else {           // column b = Im x
            vre += s[t][1][1] * PWi - s[t][0][1] * PUi;
            vim += s[t][0][0] * PUr - s[t][1][0] * PWr;
          }
        }
        vre += __shfl_xor(vre, 1);   // lanes r and r^1 hold columns a and b of one token
        vim += __shfl_xor(vim, 1);
        const int tok = tok0 + 8 * f + (r >> 1);
        if (b_ok[f] && i_ok) {
          const float d = delta[tok];
          if (MODE == kOutF32) {
            float* __restrict__ y = static_cast<float*>(yv);
            if (comp == 0) y[(int64_t)tok * ys + i] = d * vre;
            else y[(int64_t)tok * ys + n + i] = d * vim;
          } else {
            uint16_t* __restrict__ y = static_cast<uint16_t*>(yv);
            if (comp == 0) y[(int64_t)tok * ys + i] = f32_to_bf16_rne(d * vre);
            else y[(int64_t)tok * ys + n + i] = f32_to_bf16_rne(d * vim);
          }
        }
      }
    }
  }
}

template <int TT>
static void launch_gemm_t(const uint8_t* packed, const float* scales, int n, int m,
                          const int8_t* q, const float* delta, int N, void* y, int mode,
                          hipStream_t s) {
  constexpr int NF = TT <= 2 ? 4 : 2;
  const dim3 grid((n + 31) / 32, (N + 16 * NF - 1) / (16 * NF)), block(256);
  if (mode == kOutF32)
    hipLaunchKernelGGL((k_gemm<TT, NF, kOutF32>), grid, block, 0, s, packed, scales, n, m, q, delta, N, y);
  else if (mode == kOutBF16)
    hipLaunchKernelGGL((k_gemm<TT, NF, kOutBF16>), grid, block, 0, s, packed, scales, n, m, q, delta, N, y);
  else
    hipLaunchKernelGGL((k_gemm<TT, NF, kOutRaw>), grid, block, 0, s, packed, scales, n, m, q, delta, N, y);
}

hipError_t launch_gemm(const uint8_t* packed, const float* scales, int n, int m, int T,
                       const int8_t* q, const float* delta, int N, void* y, int y_mode,
                       hipStream_t s) {
  switch (T) {
    case 1: launch_gemm_t<1>(packed, scales, n, m, q, delta, N, y, y_mode, s); break;
    case 2: launch_gemm_t<2>(packed, scales, n, m, q, delta, N, y, y_mode, s); break;
    case 3: launch_gemm_t<3>(packed, scales, n, m, q, delta, N, y, y_mode, s); break;
    default: launch_gemm_t<4>(packed, scales, n, m, q, delta, N, y, y_mode, s); break;
  }
  return hipGetLastError();
}

}  // namespace f2i
