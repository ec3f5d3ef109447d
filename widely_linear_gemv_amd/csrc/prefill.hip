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
// (token, component a = Re x or b = Im x).  A workgroup owns 16 complex rows and 8 waves of 8*NF
// tokens.  Per 64-column step the workgroup decodes the tile's code words once: a shift and a
// mask spread four codes into four bytes (the packed layout puts codes b, b+4, b+8, b+12 in
// byte b) and v_perm_b32 maps each byte through a 4-entry table into the int8 planes B_re and
// B_im, written to LDS.  Each plane fragment and 16-column activation fragment feeds one
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

enum { kOutF32 = 0, kOutBF16 = 1, kOutRaw = 2 };

constexpr int kGemmWaves = 8;      // waves per workgroup, each with its own 8*NF tokens

// Workgroup = 16 complex rows x (8 waves x 8*NF tokens).  Per 64-column step the workgroup
// decodes the tile's codes once -- one half word (8 codes) per thread -- into int8 planes in a
// double-buffered LDS tile [plane = (t, M, re/im)][row][64]; every wave then reads the 4T plane
// fragments from LDS and multiplies them with its own activation fragments (prefetched one
// step ahead from global memory), NF column fragments per plane fragment.
template <int TT, int NF, int MODE>
__global__ __launch_bounds__(64 * kGemmWaves) void k_gemm(const uint8_t* __restrict__ packed,
                                                          const float* __restrict__ scales, int n, int m,
                                                          const int8_t* __restrict__ q,
                                                          const float* __restrict__ delta, int N,
                                                          void* __restrict__ yv) {
  constexpr int kPlanes = TT * 4;                  // (t, M, re/im)
  constexpr int KS = 2;                            // 64-column MFMA sub-steps per pipeline step
  __shared__ __align__(16) int8_t s_a[2][kPlanes][16][64 * KS];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int r = lane & 15;          // A row / B column inside a 16x16 tile
  const int g = lane >> 4;          // 16-column group of the 64-column step
  const int i0 = blockIdx.x * 16;
  const int tok0 = (blockIdx.y * kGemmWaves + wave) * (8 * NF);
  const int dw_plane = m / 16;
  const int64_t two_m = 2 * (int64_t)m;
  const int ksteps = (m + 64 * KS - 1) / (64 * KS);   // a partial last step is zero-filled

  // decode assignment: half word h = ((row * 2T + tm) * 4KS + wq) * 2 + hh
  constexpr int kHalves = 16 * TT * 2 * 4 * KS * 2;
  constexpr int kPerThread = (kHalves + 64 * kGemmWaves - 1) / (64 * kGemmWaves);
  const uint32_t* __restrict__ words = reinterpret_cast<const uint32_t*>(packed);
  uint32_t wreg[kPerThread];
  auto load_words = [&](int kk) {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int h = tid + u * 64 * kGemmWaves;
      const int rr = h / (TT * 2 * 8 * KS), tm = (h / (8 * KS)) % (TT * 2), wq = (h / 2) % (4 * KS);
      const int i = i0 + rr;
      const int word = 4 * KS * kk + wq;
      wreg[u] = (h < kHalves && i < n && word < dw_plane)
          ? words[(int64_t)i * (TT * 2 * dw_plane) + tm * dw_plane + word] : 0u;
    }
  };
  auto decode_to_lds = [&](int buf) {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int h = tid + u * 64 * kGemmWaves;
      if (h >= kHalves) continue;
      const int rr = h / (TT * 2 * 8 * KS), tm = (h / (8 * KS)) % (TT * 2), wq = (h / 2) % (4 * KS), hh = h % 2;
      constexpr uint32_t lo2 = 0x03030303u;
      constexpr uint32_t kRe = 0x00FF0001u;   // code 0 -> +1, 1 -> 0, 2 -> -1, 3 -> 0
      constexpr uint32_t kIm = 0xFF000100u;   // code 0 -> 0, 1 -> +1, 2 -> 0, 3 -> -1
      const uint32_t w = wreg[u];
      const uint32_t ka = (w >> (4 * hh)) & lo2;        // codes 16wq + 8hh + 0..3
      const uint32_t kb = (w >> (4 * hh + 2)) & lo2;    // codes 16wq + 8hh + 4..7
      const int col = 16 * wq + 8 * hh;
      *reinterpret_cast<uint2*>(&s_a[buf][tm * 2 + 0][rr][col]) =
          make_uint2(__builtin_amdgcn_perm(0u, kRe, ka), __builtin_amdgcn_perm(0u, kRe, kb));
      *reinterpret_cast<uint2*>(&s_a[buf][tm * 2 + 1][rr][col]) =
          make_uint2(__builtin_amdgcn_perm(0u, kIm, ka), __builtin_amdgcn_perm(0u, kIm, kb));
    }
  };

  const int8_t* bptr[NF];
  bool b_ok[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int tok = tok0 + 8 * f + (r >> 1);
    b_ok[f] = tok < N;
    bptr[f] = q + (int64_t)(b_ok[f] ? tok : 0) * two_m + (r & 1) * (int64_t)m + 16 * g;
  }
  v4i bcur[KS][NF], bnxt[KS][NF];
  auto load_b = [&](int kk, v4i (&b)[KS][NF]) {
#pragma unroll
    for (int u = 0; u < KS; ++u)
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int col = 64 * (KS * kk + u);
        b[u][f] = (b_ok[f] && col < m) ? *reinterpret_cast<const v4i*>(bptr[f] + col) : v4i{0, 0, 0, 0};
      }
  };

  v4i acc[kPlanes][NF];
#pragma unroll
  for (int p = 0; p < kPlanes; ++p)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[p][f] = v4i{0, 0, 0, 0};

  load_words(0);
  load_b(0, bcur);
  decode_to_lds(0);
  __syncthreads();
  for (int kk = 0; kk < ksteps; ++kk) {
    const int buf = kk & 1;
    const bool more = kk + 1 < ksteps;
    if (more) { load_words(kk + 1); load_b(kk + 1, bnxt); }
#pragma unroll
    for (int u = 0; u < KS; ++u)
#pragma unroll
      for (int p = 0; p < kPlanes; ++p) {
        const v4i a = *reinterpret_cast<const v4i*>(&s_a[buf][p][r][64 * u + 16 * g]);
#pragma unroll
        for (int f = 0; f < NF; ++f)
          acc[p][f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bcur[u][f], acc[p][f], 0, 0, 0);
      }
    if (more) {
      decode_to_lds(buf ^ 1);
#pragma unroll
      for (int u = 0; u < KS; ++u)
#pragma unroll
        for (int f = 0; f < NF; ++f) bcur[u][f] = bnxt[u][f];
    }
    __syncthreads();
  }

  // C layout of a 16x16 tile: lane holds rows 4g..4g+3 of column r.  Plane index p = (t*2+M)*2+re/im.
  const int comp = r & 1;
  if (tok0 >= N) return;
  if constexpr (MODE == kOutRaw) {
    int* __restrict__ P = static_cast<int*>(yv);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int tok = tok0 + 8 * f + (r >> 1);
      if (!b_ok[f]) continue;
#pragma unroll
      for (int p = 0; p < kPlanes; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i0 + 4 * g + e;
          if (i < n) P[(((int64_t)p * 2 + comp) * N + tok) * n + i] = acc[p][f][e];
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
          const float PUr = (float)acc[(t * 2 + 0) * 2 + 0][f][e], PUi = (float)acc[(t * 2 + 0) * 2 + 1][f][e];
          const float PWr = (float)acc[(t * 2 + 1) * 2 + 0][f][e], PWi = (float)acc[(t * 2 + 1) * 2 + 1][f][e];
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
  constexpr int tok_per_wg = kGemmWaves * 8 * NF;
  const dim3 grid((n + 15) / 16, (N + tok_per_wg - 1) / tok_per_wg), block(64 * kGemmWaves);
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
