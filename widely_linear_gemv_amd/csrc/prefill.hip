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

constexpr int kGemmWaves = 8;      // waves per workgroup (two per SIMD), each with its own 8*NF tokens
constexpr int kAhead = 3;          // plane fragments read from LDS ahead of their MFMAs

// Workgroup = 16 complex rows x (8 waves x 8*NF tokens).  Per 128-column step the workgroup
// decodes the tile's codes once -- one half word (8 codes) per thread -- into int8 planes in a
// double-buffered LDS tile [plane = (t, M, re/im)][row][128 + pad]; every wave then reads the
// 4T plane fragments from LDS (one read ahead of the MFMAs that use it) and multiplies them with
// its own activation fragments, which are loaded from global memory one step ahead into a
// ping-pong register pair, NF column fragments per plane fragment.
//
// No load is predicated: codes and activations are read through buffer resources sized to the
// rows and tokens that exist, so reads past n or N return 0 (and those outputs are never stored);
// columns past m (at most one 64-column half of the last step) get zero planes from the decoder,
// so whatever activations sit there add nothing.
// Epilogue of a 16-row x 8*NF-token wave tile: acc[p][f] with plane p = (t*2+M)*2 + re/im and
// column fragment f (tokens tok0 + 8f + r/2, component r & 1).
template <int TT, int NF, int MODE>
__device__ __forceinline__ void gemm_epilogue(const v4i (&acc)[TT * 4][NF], const float* __restrict__ scales,
                                              int n, int N, const float* __restrict__ delta,
                                              void* __restrict__ yv, int i0, int tok0, int r, int g) {
  constexpr int kPlanes = TT * 4;
  bool b_ok[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) b_ok[f] = tok0 + 8 * f + (r >> 1) < N;

  // C layout of a 16x16 tile: lane holds rows 4g..4g+3 of column r.  Plane index p = (t*2+M)*2+re/im.
  // Each lane stores its four consecutive rows with one 16-byte (8-byte for bf16) store when n is
  // a multiple of 4, which keeps every store row-aligned; otherwise it stores them one by one.
  const int comp = r & 1;
  if (tok0 >= N) return;
  const int ib = i0 + 4 * g;                 // first of this lane's four rows
  const bool vec = (n % 4) == 0;
  if constexpr (MODE == kOutRaw) {
    int* __restrict__ P = static_cast<int*>(yv);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int tok = tok0 + 8 * f + (r >> 1);
      if (!b_ok[f] || ib >= n) continue;
#pragma unroll
      for (int p = 0; p < kPlanes; ++p) {
        int* dst = P + (((int64_t)p * 2 + comp) * N + tok) * n + ib;
        if (vec) {
          *reinterpret_cast<v4i*>(dst) = acc[p][f];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (ib + e < n) dst[e] = acc[p][f][e];
        }
      }
    }
  } else {
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
    for (int f = 0; f < NF; ++f) {
      const int tok = tok0 + 8 * f + (r >> 1);
      const float d = delta[b_ok[f] ? tok : 0];
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float vre = 0.f, vim = 0.f;
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const float PUr = (float)acc[(t * 2 + 0) * 2 + 0][f][e], PUi = (float)acc[(t * 2 + 0) * 2 + 1][f][e];
          const float PWr = (float)acc[(t * 2 + 1) * 2 + 0][f][e], PWi = (float)acc[(t * 2 + 1) * 2 + 1][f][e];
          if (comp == 0) {   // column a = Re x
            vre += s[e][t][0][0] * PUr + s[e][t][1][0] * PWr;
            vim += s[e][t][0][1] * PUi + s[e][t][1][1] * PWi;
          } else {           // column b = Im x
            vre += s[e][t][1][1] * PWi - s[e][t][0][1] * PUi;
            vim += s[e][t][0][0] * PUr - s[e][t][1][0] * PWr;
          }
        }
        vre += __shfl_xor(vre, 1);   // lanes r and r^1 hold columns a and b of one token
        vim += __shfl_xor(vim, 1);
        o[e] = d * (comp == 0 ? vre : vim);   // lane a stores Re y, lane b stores Im y
      }
      if (!b_ok[f] || ib >= n) continue;
      const int64_t off = (int64_t)tok * ys + (comp == 0 ? 0 : n) + ib;
      if (MODE == kOutF32) {
        float* __restrict__ y = static_cast<float*>(yv) + off;
        if (vec) {
          *reinterpret_cast<float4*>(y) = make_float4(o[0], o[1], o[2], o[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (ib + e < n) y[e] = o[e];
        }
      } else {
        uint16_t* __restrict__ y = static_cast<uint16_t*>(yv) + off;
        if (vec) {
          *reinterpret_cast<uint2*>(y) =
              make_uint2((uint32_t)f32_to_bf16_rne(o[0]) | ((uint32_t)f32_to_bf16_rne(o[1]) << 16),
                         (uint32_t)f32_to_bf16_rne(o[2]) | ((uint32_t)f32_to_bf16_rne(o[3]) << 16));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (ib + e < n) y[e] = f32_to_bf16_rne(o[e]);
        }
      }
    }
  }
}

// Raw buffer resource over [base, base + bytes): loads at offsets past the end return 0.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int nrec = (int)min(max(bytes, (int64_t)0), (int64_t)0x7FFFFFF0);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
}

template <int TT, int NF, int MODE>
__global__ __launch_bounds__(64 * kGemmWaves) void k_gemm(const uint8_t* __restrict__ packed,
                                                          const float* __restrict__ scales, int n, int m,
                                                          const int8_t* __restrict__ q,
                                                          const float* __restrict__ delta, int N,
                                                          void* __restrict__ yv) {
  constexpr int kPlanes = TT * 4;                  // (t, M, re/im)
  constexpr int KS = 2;                            // 64-column MFMA sub-steps per pipeline step
  constexpr int kRow = 64 * KS + 16;               // LDS row pitch: 16 pad bytes spread the rows over the banks
  __shared__ __align__(16) int8_t s_a[2][kPlanes][16][kRow];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform: keeps the buffer resources scalar
  const int r = lane & 15;          // A row / B column inside a 16x16 tile
  const int g = lane >> 4;          // 16-column group of the 64-column step
  const int i0 = blockIdx.x * 16;
  const int tok0 = (blockIdx.y * kGemmWaves + wave) * (8 * NF);
  const int dw_plane = m / 16;
  const int64_t two_m = 2 * (int64_t)m;
  const int ksteps = (m + 64 * KS - 1) / (64 * KS);

  // decode assignment: half word h = ((row * 2T + tm) * 4KS + wq) * 2 + hh.  The tile's code
  // words are read through a buffer resource over this workgroup's tile of the packed form (the
  // last tile's padding rows hold code 0; their outputs are never stored).  Step kk covers
  // words 8kk .. 8kk+7 of each row and plane: chunk kk/2, 64-column groups 2(kk%2) and 2(kk%2)+1.
  static_assert(KS == 2, "a step is half a 256-column chunk of the packed form");
  constexpr int kHalves = 16 * TT * 2 * 4 * KS * 2;
  constexpr int kPerThread = (kHalves + 64 * kGemmWaves - 1) / (64 * kGemmWaves);
  const int64_t tile_bytes = (int64_t)16 * TT * 2 * dw_plane * 4;
  const __amdgpu_buffer_rsrc_t rsrc_w = make_rsrc(packed + (int64_t)blockIdx.x * tile_bytes, tile_bytes);
  int woff[kPerThread], wtm[kPerThread];
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int h = min(tid + u * 64 * kGemmWaves, kHalves - 1);
    const int rr = h / (TT * 2 * 8 * KS), tm = (h / (8 * KS)) % (TT * 2), wq = (h / 2) % (4 * KS);
    woff[u] = (wq >> 2) * 64 + rr * 4 + (wq & 3);      // group within the step, row, word
    wtm[u] = tm;
  }
  uint32_t wreg[kPerThread];
  auto load_words = [&](int kk) {
    const int c = kk >> 1;
    const int groups = min(4, (m - 256 * c) >> 6);
    const int base = c * (TT * 2) * 256 + (kk & 1) * 128;
#pragma unroll
    for (int u = 0; u < kPerThread; ++u)
      wreg[u] = __builtin_amdgcn_raw_buffer_load_b32(rsrc_w, 4 * (base + wtm[u] * groups * 64 + woff[u]), 0, 0);
  };
  auto decode_to_lds = [&](int buf, int kk) {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int h = tid + u * 64 * kGemmWaves;
      if (kHalves % (64 * kGemmWaves) != 0 && h >= kHalves) continue;
      const int rr = h / (TT * 2 * 8 * KS), tm = (h / (8 * KS)) % (TT * 2), wq = (h / 2) % (4 * KS), hh = h % 2;
      constexpr uint32_t lo2 = 0x03030303u;
      constexpr uint32_t kRe = 0x00FF0001u;   // code 0 -> +1, 1 -> 0, 2 -> -1, 3 -> 0
      constexpr uint32_t kIm = 0xFF000100u;   // code 0 -> 0, 1 -> +1, 2 -> 0, 3 -> -1
      const bool in_m = 4 * KS * kk + wq < dw_plane;
      const uint32_t w = wreg[u];
      const uint32_t ka = (w >> (4 * hh)) & lo2;        // codes 16wq + 8hh + 0..3
      const uint32_t kb = (w >> (4 * hh + 2)) & lo2;    // codes 16wq + 8hh + 4..7
      const int col = 16 * wq + 8 * hh;
      uint2 re = make_uint2(__builtin_amdgcn_perm(0u, kRe, ka), __builtin_amdgcn_perm(0u, kRe, kb));
      uint2 im = make_uint2(__builtin_amdgcn_perm(0u, kIm, ka), __builtin_amdgcn_perm(0u, kIm, kb));
      if (!in_m) re = im = make_uint2(0u, 0u);
      *reinterpret_cast<uint2*>(&s_a[buf][tm * 2 + 0][rr][col]) = re;
      *reinterpret_cast<uint2*>(&s_a[buf][tm * 2 + 1][rr][col]) = im;
    }
  };

  // Activations: one buffer resource over this wave's tokens, so tokens past N read 0.  Lane
  // (r, g) reads 16 columns 16g.. of component r&1 of token 8f + r/2.
  const __amdgpu_buffer_rsrc_t rsrc_q =
      make_rsrc(q + (int64_t)min(tok0, N) * two_m, (int64_t)max(N - tok0, 0) * two_m);
  const int voff_q = (int)((r >> 1) * two_m + (r & 1) * m + 16 * g);
  // B fragments of 64-column sub-step j (= KS * step + u) into one register slot.
  auto load_b = [&](int j, v4i (&b)[NF]) {
#pragma unroll
    for (int f = 0; f < NF; ++f)
      b[f] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                 rsrc_q, voff_q + (int)(8 * f * two_m) + 64 * j, 0, 0));
  };

  v4i acc[kPlanes][NF];
#pragma unroll
  for (int p = 0; p < kPlanes; ++p)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[p][f] = v4i{0, 0, 0, 0};

  // One pipeline step (KS = 2 sub-steps of 64 columns) on LDS buffer `buf`.  Activations use
  // two register slots, one per sub-step, each loaded one sub-step ahead of its MFMAs; the next
  // step's code words are loaded at the top and decoded into the other LDS buffer at the end,
  // followed by the step's one barrier.  Loads and decode run unconditionally (the last step
  // reloads in-range data and decodes zero planes nobody reads), so every path into a step has
  // the same loads in flight and the compiler's load counters wait only for the operands due.
  static_assert(KS == 2, "two activation slots, one per sub-step");
  v4i b0[NF], b1[NF];
  auto step = [&](int kk, int buf) {
    const int kn = min(kk + 1, ksteps - 1);
    load_b(KS * kk + 1, b1);
    load_words(kn);
    // Plane fragments x = (u, p) are read kAhead fragments ahead of the MFMAs that use them; the
    // scheduling barriers keep those LDS reads in flight under the MFMAs (the scheduler would
    // otherwise sink each read to its use and expose the LDS latency once per fragment).
    constexpr int NX = KS * kPlanes;
    auto lds_a = [&](int x) {
      return *reinterpret_cast<const v4i*>(&s_a[buf][x % kPlanes][r][64 * (x / kPlanes) + 16 * g]);
    };
    v4i a[kAhead + 1];
#pragma unroll
    for (int x = 0; x < kAhead; ++x) a[x] = lds_a(x);
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      const int u = x / kPlanes, p = x % kPlanes;
      if (x == kPlanes) load_b(KS * kn, b0);   // sub-step 0 of the next step, under sub-step 1
      if (x + kAhead < NX) a[(x + kAhead) % (kAhead + 1)] = lds_a(x + kAhead);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < NF; ++f)
        acc[p][f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[x % (kAhead + 1)], u == 0 ? b0[f] : b1[f], acc[p][f], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    decode_to_lds(buf ^ 1, kk + 1);
    __syncthreads();
  };

  load_words(0);
  load_b(0, b0);
  decode_to_lds(0, 0);
  __syncthreads();
  int kk = 0;
  for (; kk + 1 < ksteps; kk += 2) {
    step(kk, 0);
    step(kk + 1, 1);
  }
  if (kk < ksteps) step(kk, 0);

  gemm_epilogue<TT, NF, MODE>(acc, scales, n, N, delta, yv, i0, tok0, r, g);
}

template <int TT>
static void launch_gemm_t(const uint8_t* packed, const float* scales, int n, int m,
                          const int8_t* q, const float* delta, int N, void* y, int mode,
                          hipStream_t s) {
  constexpr int NF = TT <= 2 ? 4 : 2;   // accumulators: 4T planes x NF fragments x 4 registers
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
