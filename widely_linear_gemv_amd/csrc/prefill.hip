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
// (token, component a = Re x or b = Im x).  A workgroup owns 8 tiles of 16 complex rows (one per
// wave) and 8*NF tokens.  The activations of each 256-column chunk are staged once per workgroup
// in LDS and shared by its 8 waves; each wave decodes its own tile's code words in registers: a
// shift and a mask spread four codes into four bytes (the packed layout puts codes b, b+4, b+8,
// b+12 in byte b) and v_perm_b32 maps each byte through a 4-entry table into the int8 planes B_re
// and B_im.  Each plane fragment and 16-column activation fragment feeds one
// v_mfma_i32_16x16x64_i8; every sum is exact in int32 (|P| <= 127 m).  The epilogue applies the
// fp32 scales once per accumulated sum and the token's delta once per output.
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
// q = clamp(rint(x / delta)) with rint rounding half to even.  KEEP > 0: the token's values stay
// in registers between the two passes (two_m <= 2048 KEEP, eight per thread and group), so x is
// read once; KEEP == 0 reads them again in the second pass (from cache).
template <typename XT, int KEEP>
__global__ __launch_bounds__(256) void k_act_quant(const XT* __restrict__ x, int two_m,
                                                   int8_t* __restrict__ q,
                                                   float* __restrict__ delta) {
  __shared__ float s_max[256 / kWave];
  const int tok = blockIdx.x;
  const XT* __restrict__ xr = x + (int64_t)tok * two_m;
  int8_t* __restrict__ qr = q + (int64_t)tok * two_m;
  constexpr int NK = KEEP > 0 ? KEEP : 1;
  float keep[NK][8];
  float amax = 0.f;
  if constexpr (KEEP > 0) {
#pragma unroll
    for (int c = 0; c < KEEP; ++c) {
      const int j = (threadIdx.x + 256 * c) * 8;
      if (j < two_m) {
        Load8<XT>::run(xr + j, keep[c]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) keep[c][e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(keep[c][e]));
    }
  } else {
    for (int j = threadIdx.x * 8; j < two_m; j += 256 * 8) {
      float v[8];
      Load8<XT>::run(xr + j, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & (kWave - 1)) == 0) s_max[threadIdx.x / kWave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float d = amax / 127.0f;
  auto quantize8 = [&](const float (&v)[8], int j) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int qi = 0;
      if (d != 0.f) qi = (int)fminf(fmaxf(rintf(v[e] / d), -127.f), 127.f);
      const uint32_t byte = (uint32_t)(qi & 0xFF);
      if (e < 4) lo |= byte << (8 * e); else hi |= byte << (8 * (e - 4));
    }
    *reinterpret_cast<uint2*>(qr + j) = make_uint2(lo, hi);
  };
  if constexpr (KEEP > 0) {
#pragma unroll
    for (int c = 0; c < KEEP; ++c) {
      const int j = (threadIdx.x + 256 * c) * 8;
      if (j < two_m) quantize8(keep[c], j);
    }
  } else {
    for (int j = threadIdx.x * 8; j < two_m; j += 256 * 8) {
      float v[8];
      Load8<XT>::run(xr + j, v);
      quantize8(v, j);
    }
  }
  if (threadIdx.x == 0) delta[tok] = d;
}

template <typename XT>
static void launch_act_quant_t(const XT* x, int N, int two_m, int8_t* q, float* delta, hipStream_t s) {
  const dim3 grid(N), block(256);
  if (two_m <= 2048) hipLaunchKernelGGL((k_act_quant<XT, 1>), grid, block, 0, s, x, two_m, q, delta);
  else if (two_m <= 4096) hipLaunchKernelGGL((k_act_quant<XT, 2>), grid, block, 0, s, x, two_m, q, delta);
  else if (two_m <= 8192) hipLaunchKernelGGL((k_act_quant<XT, 4>), grid, block, 0, s, x, two_m, q, delta);
  else if (two_m <= 16384) hipLaunchKernelGGL((k_act_quant<XT, 8>), grid, block, 0, s, x, two_m, q, delta);
  else hipLaunchKernelGGL((k_act_quant<XT, 0>), grid, block, 0, s, x, two_m, q, delta);
}

hipError_t launch_act_quant(const void* x, int x_bf16, int N, int two_m, int8_t* q, float* delta,
                            hipStream_t s) {
  if (x_bf16) launch_act_quant_t(static_cast<const uint16_t*>(x), N, two_m, q, delta, s);
  else launch_act_quant_t(static_cast<const float*>(x), N, two_m, q, delta, s);
  return hipGetLastError();
}

// ----------------------------------------------------------------------- GEMM ----

enum { kOutF32 = 0, kOutBF16 = 1, kOutRaw = 2 };

constexpr int kGemmWaves = 8;      // waves per workgroup, one 16-row tile each

// Epilogue of a 16-row x 8*NF-token wave tile: acc[p][f] with plane p = (t*2+M)*2 + re/im and
// column fragment f = 2 tg + comp (tokens tok0 + 16 tg + r, component comp: a = Re x, b = Im x).
// A lane holds both components of its tokens, so it forms Re y and Im y of its four rows alone:
//   Re y = sum_t  sU_re P_U,re(a) - sU_im P_U,im(b) + sW_re P_W,re(a) + sW_im P_W,im(b)
//   Im y = sum_t  sU_re P_U,re(b) + sU_im P_U,im(a) + sW_im P_W,im(a) - sW_re P_W,re(b)
// (U x + W conj(x) with each term's two axis scales), times the token's delta.
template <int TT, int NF, int MODE>
__device__ __forceinline__ void gemm_epilogue(const v4i (&acc)[TT * 4][NF], const float* __restrict__ scales,
                                              int n, int N, const float* __restrict__ delta,
                                              void* __restrict__ yv, int i0, int tok0, int r, int g) {
  constexpr int kPlanes = TT * 4;
  constexpr int NT = NF / 2;                 // groups of 16 tokens

  // C layout of a 16x16 tile: lane holds rows 4g..4g+3 of column r.  Each lane stores its four
  // consecutive rows with one 16-byte (8-byte for bf16) store when n is a multiple of 4, which
  // keeps every store row-aligned; otherwise it stores them one by one.
  if (tok0 >= N) return;
  const int ib = i0 + 4 * g;                 // first of this lane's four rows
  const bool vec = (n % 4) == 0;
  if constexpr (MODE == kOutRaw) {
    int* __restrict__ P = static_cast<int*>(yv);
#pragma unroll
    for (int tg = 0; tg < NT; ++tg) {
      const int tok = tok0 + 16 * tg + r;
      if (tok >= N || ib >= n) continue;
#pragma unroll
      for (int comp = 0; comp < 2; ++comp)
#pragma unroll
        for (int p = 0; p < kPlanes; ++p) {
          int* dst = P + (((int64_t)p * 2 + comp) * N + tok) * n + ib;
          if (vec) {
            *reinterpret_cast<v4i*>(dst) = acc[p][2 * tg + comp];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (ib + e < n) dst[e] = acc[p][2 * tg + comp][e];
          }
        }
    }
  } else {
#pragma clang fp contract(fast)
    const int64_t ys = 2 * (int64_t)n;
    float s[4][TT][2][2];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int M = 0; M < 2; ++M)
#pragma unroll
          for (int ax = 0; ax < 2; ++ax)
            s[e][t][M][ax] = ib + e < n ? scales[(((int64_t)(ib + e) * TT + t) * 2 + M) * 2 + ax] : 0.f;
#pragma unroll
    for (int tg = 0; tg < NT; ++tg) {
      const int tok = tok0 + 16 * tg + r;
      const bool ok = tok < N;
      const float d = delta[ok ? tok : 0];
      float ore[4], oim[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float vre = 0.f, vim = 0.f;
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const int u = (t * 2 + 0) * 2, w = (t * 2 + 1) * 2;
          const float Ura = (float)acc[u][2 * tg][e], Uia = (float)acc[u + 1][2 * tg][e];
          const float Wra = (float)acc[w][2 * tg][e], Wia = (float)acc[w + 1][2 * tg][e];
          const float Urb = (float)acc[u][2 * tg + 1][e], Uib = (float)acc[u + 1][2 * tg + 1][e];
          const float Wrb = (float)acc[w][2 * tg + 1][e], Wib = (float)acc[w + 1][2 * tg + 1][e];
          vre += s[e][t][0][0] * Ura - s[e][t][0][1] * Uib + s[e][t][1][0] * Wra + s[e][t][1][1] * Wib;
          vim += s[e][t][0][0] * Urb + s[e][t][0][1] * Uia + s[e][t][1][1] * Wia - s[e][t][1][0] * Wrb;
        }
        ore[e] = d * vre;
        oim[e] = d * vim;
      }
      if (!ok || ib >= n) continue;
      const int64_t off = (int64_t)tok * ys + ib;
      if (MODE == kOutF32) {
        float* __restrict__ y = static_cast<float*>(yv) + off;
        if (vec) {
          *reinterpret_cast<float4*>(y) = make_float4(ore[0], ore[1], ore[2], ore[3]);
          *reinterpret_cast<float4*>(y + n) = make_float4(oim[0], oim[1], oim[2], oim[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (ib + e < n) y[e] = ore[e], y[n + e] = oim[e];
        }
      } else {
        uint16_t* __restrict__ y = static_cast<uint16_t*>(yv) + off;
        if (vec) {
          *reinterpret_cast<uint2*>(y) =
              make_uint2((uint32_t)f32_to_bf16_rne(ore[0]) | ((uint32_t)f32_to_bf16_rne(ore[1]) << 16),
                         (uint32_t)f32_to_bf16_rne(ore[2]) | ((uint32_t)f32_to_bf16_rne(ore[3]) << 16));
          *reinterpret_cast<uint2*>(y + n) =
              make_uint2((uint32_t)f32_to_bf16_rne(oim[0]) | ((uint32_t)f32_to_bf16_rne(oim[1]) << 16),
                         (uint32_t)f32_to_bf16_rne(oim[2]) | ((uint32_t)f32_to_bf16_rne(oim[3]) << 16));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (ib + e < n) y[e] = f32_to_bf16_rne(ore[e]), y[n + e] = f32_to_bf16_rne(oim[e]);
        }
      }
    }
  }
}

// Workgroup = 8 tiles of 16 complex rows (wave w takes tile 8 blockIdx.x + w) x 8*NF tokens.  Per
// 256-column chunk (the chunk of the packed form) the workgroup copies into one of two LDS buffers,
// with direct global-to-LDS buffer loads (no registers on the way): each wave its own tile's 2T
// code planes (1 KB each, lane l's 16 bytes at 16 l as in the packed form), and all waves together
// the tokens' activations, 256 columns of int8 per row, 1 KB (4 rows) per copy.  Row 16 f + r holds
// column r of token fragment f: token 16 (f/2) + r, component f & 1 (a = Re x, b = Im x), so
// a lane's accumulators hold both components of its tokens.  Within an activation row, 16-byte
// segment sg sits in slot sg ^ (row % 16), so the 16 lanes that read one fragment (16 rows, same
// columns) hit 16 different slots, each its own group of LDS banks.  Every wave
// then runs the chunk's four 64-column MFMA steps: lane (r, g) decodes word s of its row r,
// 64-column group g for each plane (columns 64g + 16s .. +15, the k order of the decode GEMVs)
// and multiplies both ternary planes with the NF activation fragments it reads at the same
// columns.  The next chunk's copies are issued before the current chunk is multiplied; each chunk
// ends with a wait for this wave's copies and the workgroup's one barrier.
//
// No load is predicated: codes and activations are read through buffer resources sized to the
// tiles and tokens that exist, so reads past n or N return 0 (those outputs are never stored);
// activation columns past m and code groups past m read as 0 (offset past every range).
typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int TT, int NF, int MODE>
__global__ __launch_bounds__(64 * kGemmWaves) void k_gemm(const uint8_t* __restrict__ packed,
                                                          const float* __restrict__ scales, int n, int m,
                                                          const int8_t* __restrict__ q,
                                                          const float* __restrict__ delta, int N,
                                                          void* __restrict__ yv) {
  constexpr int kPlanes = TT * 4;                  // (t, M, re/im)
  constexpr int kWords = TT * 2;                   // code planes (t, M)
  constexpr int kActBytes = NF * 4096;             // 16 NF activation rows of 256 bytes
  constexpr int kCodeBytes = kGemmWaves * kWords * 1024;
  static_assert(2 * (kCodeBytes + kActBytes) <= 160 * 1024, "two buffers fit in LDS");
  __shared__ __align__(16) uint8_t s_lds[2][kCodeBytes + kActBytes];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform: keeps the buffer resources scalar
  const int r = lane & 15;          // A row / B column inside a 16x16 tile
  const int g = lane >> 4;          // 64-column group of the chunk
  const int tiles = (n + 15) / 16;
  const int tile = blockIdx.x * kGemmWaves + wave;
  const int i0 = tile * 16;
  const int tok0 = blockIdx.y * (8 * NF);
  const int64_t two_m = 2 * (int64_t)m;
  const int nchunk = (m + 255) / 256;
  const int64_t tile_bytes = (int64_t)16 * TT * 2 * (m / 4);
  const __amdgpu_buffer_rsrc_t rsrc_w =
      range_rsrc(packed + (int64_t)min(tile, tiles - 1) * tile_bytes, tile < tiles ? tile_bytes : 0);
  const __amdgpu_buffer_rsrc_t rsrc_q =
      range_rsrc(q + (int64_t)min(tok0, N) * two_m, (int64_t)max(N - tok0, 0) * two_m);

  v4i acc[kPlanes][NF];
#pragma unroll
  for (int p = 0; p < kPlanes; ++p)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[p][f] = v4i{0, 0, 0, 0};

  // chunk c into buffer b: this wave's planes, then activation blocks wave, wave + 8, ...
  auto stage = [&](int c, int b) {
    uint8_t* base = s_lds[b];
    const int groups = min(4, (m - 256 * c) >> 6);
    const bool ok_w = g < groups;
#pragma unroll
    for (int P = 0; P < kWords; ++P)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc_w, (lds_ptr_t)(base + (wave * kWords + P) * 1024), 16,
          ok_w ? (uint32_t)(c * kWords * 1024 + P * groups * 256 + lane * 16) : kNoLoad, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < (4 * NF + kGemmWaves - 1) / kGemmWaves; ++k) {
      const int blk = wave + kGemmWaves * k;        // activation rows 4 blk .. 4 blk + 3
      if (blk >= 4 * NF) break;
      const int R = 4 * blk + (lane >> 4), slot = lane & 15, sg = slot ^ (R & 15);
      const bool ok = 256 * c + 16 * sg < m;        // row R = 16 f + r: fragment f's column r
      const int tok = 16 * (R >> 5) + (R & 15), comp = (R >> 4) & 1;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc_q, (lds_ptr_t)(base + kCodeBytes + blk * 1024), 16,
          ok ? (uint32_t)(tok * two_m + comp * m + 256 * c + 16 * sg) : kNoLoad, 0, 0, 0);
    }
  };
  constexpr uint32_t lo2 = 0x03030303u;
  constexpr uint32_t kRe = 0x00FF0001u;   // code 0 -> +1, 1 -> 0, 2 -> -1, 3 -> 0
  constexpr uint32_t kIm = 0xFF000100u;   // code 0 -> 0, 1 -> +1, 2 -> 0, 3 -> -1
  auto compute = [&](int b) {
    const uint8_t* base = s_lds[b];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4i bf[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) {       // column r: token 16 (f/2) + r, component f & 1 -> row 16 f + r
        const int R = 16 * f + r;
        bf[f] = *reinterpret_cast<const v4i*>(base + kCodeBytes + R * 256 + 16 * ((4 * g + s) ^ r));
      }
#pragma unroll
      for (int tm = 0; tm < kWords; ++tm) {
        const uint32_t x = *reinterpret_cast<const uint32_t*>(base + (wave * kWords + tm) * 1024 + lane * 16 + 4 * s);
        const uint32_t k0 = x & lo2, k1 = (x >> 2) & lo2, k2 = (x >> 4) & lo2, k3 = (x >> 6) & lo2;
        const v4i re = v4i{(int)__builtin_amdgcn_perm(0u, kRe, k0), (int)__builtin_amdgcn_perm(0u, kRe, k1),
                           (int)__builtin_amdgcn_perm(0u, kRe, k2), (int)__builtin_amdgcn_perm(0u, kRe, k3)};
        const v4i im = v4i{(int)__builtin_amdgcn_perm(0u, kIm, k0), (int)__builtin_amdgcn_perm(0u, kIm, k1),
                           (int)__builtin_amdgcn_perm(0u, kIm, k2), (int)__builtin_amdgcn_perm(0u, kIm, k3)};
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          acc[tm * 2 + 0][f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(re, bf[f], acc[tm * 2 + 0][f], 0, 0, 0);
          acc[tm * 2 + 1][f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(im, bf[f], acc[tm * 2 + 1][f], 0, 0, 0);
        }
      }
    }
  };

  stage(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int c = 0; c < nchunk; ++c) {
    if (c + 1 < nchunk) stage(c + 1, (c + 1) & 1);   // its buffer's last readers passed the previous barrier
    compute(c & 1);
    __builtin_amdgcn_s_waitcnt(0);                  // this wave's copies of chunk c + 1 have landed
    __syncthreads();
  }

  if (tile < tiles) gemm_epilogue<TT, NF, MODE>(acc, scales, n, N, delta, yv, i0, tok0, r, g);
}

template <int TT>
static void launch_gemm_t(const uint8_t* packed, const float* scales, int n, int m,
                          const int8_t* q, const float* delta, int N, void* y, int mode,
                          hipStream_t s) {
  constexpr int NF = TT <= 2 ? 4 : 2;   // accumulators: 4T planes x NF fragments x 4 registers
  constexpr int tok_per_wg = 8 * NF;
  const int tiles = (n + 15) / 16;
  const dim3 grid((tiles + kGemmWaves - 1) / kGemmWaves, (N + tok_per_wg - 1) / tok_per_wg),
      block(64 * kGemmWaves);
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
