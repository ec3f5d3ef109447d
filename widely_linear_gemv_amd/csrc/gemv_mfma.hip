// Decode GEMV on the matrix cores: y = sum_t U~(t) x + W~(t) conj(x), bf16 x, fp32 sums.
//
// Sources: ModelScope card "Fairy2i-W2", "Method" (y = U x + W conj(x)); zhichai.net reading
// note, "Step 2" dequantization and "Industry implications: multiplication-free inference"
// (B_re, B_im in {-1, 0, 1}; products reduce to additions, subtractions, skips); 36Kr article,
// parallel stages.
//
// The arithmetic is still add / subtract / skip: every weight factor is +-1 or 0 and x enters
// unchanged as bf16, so every product is exact and only the fp32 additions inside the MFMA
// round.  It runs on v_mfma_f32_16x16x32_bf16 because on gfx950 a VALU add costs a lane-cycle
// per code per batch column -- several times what an HBM-bound stream of 2-bit codes allows --
// while one MFMA consumes 512 code-planes in 16 cycles.
//
//  * A operand (16 rows x 32 columns, bf16): 16 complex output rows, one plane (B_re or B_im)
//    per MFMA.  A packed word holds code 4d+b in bits 8b+2d (axis bit) and 8b+2d+1 (sign bit).
//    Shifting the word left by 14-(8b+2d) puts that code's two bits at bits 14-15 and the code
//    two places later at bits 30-31, so
//        im = (w << sh) & 0xC000C000     gives two bf16 values s*2.0 (axis = imaginary) or +-0
//        re = im ^ 0x40004000            gives the real-axis plane
//    -- 1.5 VALU operations per code for both planes.  Element order inside a lane is
//    (0, 2, 1, 3, 4, 6, 5, 7) of each 8-code group; the B operand is permuted to match.
//  * K assignment: a workgroup handles 16 rows; its 4 waves take 256-column chunks in turn.  In a
//    chunk, lane group g owns columns 64g..64g+63 (one 16-byte load of 4 words per plane) and at
//    MFMA step s = 0..7 contributes columns 64g+8s .. 64g+8s+7.
//  * B operand (32 x 16, bf16): columns are (batch b, component a = Re x or b = Im x); 8 batch
//    columns per MFMA, two column groups for B > 8.  Each lane loads 8 consecutive bf16 of x and
//    swaps elements 1,2 and 5,6 with v_perm_b32.
//  * One 16x16 fp32 accumulator per (stage, matrix, plane, column group).  The epilogue applies
//    the fp32 scales (and the factor 1/2 of the +-2 encoding) once per accumulated sum, adds the
//    a and b columns of a batch entry across two lanes, and sums the four waves through LDS in a
//    fixed order.
#include "common.hpp"

namespace f2i {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kChunk = 256;        // columns per wave work unit
constexpr int kGemvWaves = 4;

// Eight codes (h = which half of the word) of one packed word -> A operands of both planes.
template <int H>
__device__ __forceinline__ void decode_bf16(uint32_t w, v4u& re, v4u& im) {
  constexpr uint32_t kKeep = 0xC000C000u, kFlip = 0x40004000u;
  // dword q = 2d' + b holds codes (4d'+b, 4d'+b+2) of this half; shift = 14 - (8b + 2(2H+d'))
  const uint32_t t0 = w << (14 - 4 * H);        // b = 0, d' = 0
  const uint32_t t1 = w << (6 - 4 * H);         // b = 1, d' = 0
  const uint32_t t2 = w << (12 - 4 * H);        // b = 0, d' = 1
  const uint32_t t3 = w << (4 - 4 * H);         // b = 1, d' = 1
  im = v4u{t0 & kKeep, t1 & kKeep, t2 & kKeep, t3 & kKeep};
  re = v4u{im[0] ^ kFlip, im[1] ^ kFlip, im[2] ^ kFlip, im[3] ^ kFlip};
}

// x[j0 .. j0+7] (bf16) -> B operand in element order (0, 2, 1, 3, 4, 6, 5, 7).
__device__ __forceinline__ v4u load_b(const uint16_t* p) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  return v4u{__builtin_amdgcn_perm(w.y, w.x, 0x05040100u), __builtin_amdgcn_perm(w.y, w.x, 0x07060302u),
             __builtin_amdgcn_perm(w.w, w.z, 0x05040100u), __builtin_amdgcn_perm(w.w, w.z, 0x07060302u)};
}

template <int TT, int CG, typename YT>
__global__ __launch_bounds__(64 * kGemvWaves) void k_gemv_mfma(
    const uint8_t* __restrict__ packed, const float* __restrict__ scales, int n, int m,
    const uint16_t* __restrict__ x, int B, YT* __restrict__ y) {
  __shared__ float s_y[kGemvWaves][16][2][16];   // [wave][batch][re/im][row]
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int i0 = blockIdx.x * 16;
  const int ia = i0 + r;
  const bool a_ok = ia < n;
  const int dw_plane = m / 16;
  const uint32_t* __restrict__ arow =
      reinterpret_cast<const uint32_t*>(packed) + (int64_t)(a_ok ? ia : 0) * (TT * 2 * dw_plane);
  // B column of this lane: batch b = 8*cg + (r >> 1), component r & 1
  const int comp = r & 1;
  const uint16_t* xb[CG];
  bool b_ok[CG];
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) {
    const int b = cg * 8 + (r >> 1);
    b_ok[cg] = b < B;
    xb[cg] = x + (int64_t)(b_ok[cg] ? b : 0) * 2 * m + comp * m;
  }

  v4f acc[TT][2][2][CG];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int M = 0; M < 2; ++M)
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int cg = 0; cg < CG; ++cg) acc[t][M][p][cg] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nchunk = (m + kChunk - 1) / kChunk;
  for (int c = wave; c < nchunk; c += kGemvWaves) {
    const int jg = c * kChunk + 64 * g;            // first column of this lane group
    const bool k_ok = jg < m;                      // m % 64 == 0: a group is all in or all out
    uint4 wd[TT][2];
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int M = 0; M < 2; ++M)
        wd[t][M] = (a_ok && k_ok)
            ? *reinterpret_cast<const uint4*>(arow + (t * 2 + M) * dw_plane + jg / 16)
            : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      v4u bv[CG];
#pragma unroll
      for (int cg = 0; cg < CG; ++cg)
        bv[cg] = (b_ok[cg] && k_ok) ? load_b(xb[cg] + jg + 8 * s) : v4u{0u, 0u, 0u, 0u};
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int M = 0; M < 2; ++M) {
          const uint4 q = wd[t][M];
          const uint32_t w = (s >> 1) == 0 ? q.x : (s >> 1) == 1 ? q.y : (s >> 1) == 2 ? q.z : q.w;
          v4u are, aim;
          if (s & 1) decode_bf16<1>(w, are, aim); else decode_bf16<0>(w, are, aim);
#pragma unroll
          for (int cg = 0; cg < CG; ++cg) {
            acc[t][M][0][cg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(v8bf, are), __builtin_bit_cast(v8bf, bv[cg]), acc[t][M][0][cg], 0, 0, 0);
            acc[t][M][1][cg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(v8bf, aim), __builtin_bit_cast(v8bf, bv[cg]), acc[t][M][1][cg], 0, 0, 0);
          }
        }
    }
  }

  // Epilogue.  C tile: lane holds rows 4g..4g+3 of column r = 2*bl + comp.
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = 4 * g + e;
    const int i = i0 + row;
    float sc[TT][4];
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q)                 // sUr, sUi, sWr, sWi, halved for the +-2 code
        sc[t][q] = i < n ? 0.5f * scales[((int64_t)i * TT + t) * 4 + q] : 0.f;
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      float vre = 0.f, vim = 0.f;
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const float CUr = acc[t][0][0][cg][e], CUi = acc[t][0][1][cg][e];
        const float CWr = acc[t][1][0][cg][e], CWi = acc[t][1][1][cg][e];
        if (comp == 0) {    // a = Re x:  Re += sUr*P(U,re) + sWr*P(W,re) ; Im += sUi*P(U,im) + sWi*P(W,im)
          vre += sc[t][0] * CUr + sc[t][2] * CWr;
          vim += sc[t][1] * CUi + sc[t][3] * CWi;
        } else {            // b = Im x:  Re += sWi*P(W,im) - sUi*P(U,im) ; Im += sUr*P(U,re) - sWr*P(W,re)
          vre += sc[t][3] * CWi - sc[t][1] * CUi;
          vim += sc[t][0] * CUr - sc[t][2] * CWr;
        }
      }
      vre += __shfl_xor(vre, 1);
      vim += __shfl_xor(vim, 1);
      if (comp == 0) {
        s_y[wave][cg * 8 + (r >> 1)][0][row] = vre;
        s_y[wave][cg * 8 + (r >> 1)][1][row] = vim;
      }
    }
  }
  __syncthreads();
  const int64_t ys = 2 * (int64_t)n;
  for (int idx = threadIdx.x; idx < 16 * 2 * 16; idx += 64 * kGemvWaves) {
    const int row = idx & 15, part = (idx >> 4) & 1, b = idx >> 5;
    const int i = i0 + row;
    if (b < B && i < n) {
      float v = s_y[0][b][part][row];
#pragma unroll
      for (int w = 1; w < kGemvWaves; ++w) v += s_y[w][b][part][row];
      store_out(y, (int64_t)b * ys + (part ? n + i : i), v);
    }
  }
}

template <int TT, typename YT>
static void launch_t(const uint8_t* packed, const float* scales, int n, int m, const void* x,
                     int B, void* y, hipStream_t s) {
  const dim3 grid((n + 15) / 16), block(64 * kGemvWaves);
  const uint16_t* xx = static_cast<const uint16_t*>(x);
  if (B <= 8)
    hipLaunchKernelGGL((k_gemv_mfma<TT, 1, YT>), grid, block, 0, s, packed, scales, n, m, xx, B, static_cast<YT*>(y));
  else
    hipLaunchKernelGGL((k_gemv_mfma<TT, 2, YT>), grid, block, 0, s, packed, scales, n, m, xx, B, static_cast<YT*>(y));
}

hipError_t launch_gemv_mfma(const uint8_t* packed, const float* scales, int n, int m, int T,
                            const void* x, int B, void* y, int y_bf16, void*, hipStream_t s) {
  if (y_bf16) {
    switch (T) {
      case 1: launch_t<1, uint16_t>(packed, scales, n, m, x, B, y, s); break;
      case 2: launch_t<2, uint16_t>(packed, scales, n, m, x, B, y, s); break;
      case 3: launch_t<3, uint16_t>(packed, scales, n, m, x, B, y, s); break;
      default: launch_t<4, uint16_t>(packed, scales, n, m, x, B, y, s); break;
    }
  } else {
    switch (T) {
      case 1: launch_t<1, float>(packed, scales, n, m, x, B, y, s); break;
      case 2: launch_t<2, float>(packed, scales, n, m, x, B, y, s); break;
      case 3: launch_t<3, float>(packed, scales, n, m, x, B, y, s); break;
      default: launch_t<4, float>(packed, scales, n, m, x, B, y, s); break;
    }
  }
  return hipGetLastError();
}

}  // namespace f2i
