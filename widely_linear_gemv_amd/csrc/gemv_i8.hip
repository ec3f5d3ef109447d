// Decode GEMV for batch 1-2 on the int8 matrix cores: y = sum_t U~(t) x + W~(t) conj(x).
//
// Sources: ModelScope card "Fairy2i-W2", "Method" (y = U x + W conj(x)); zhichai.net reading
// note, "Step 2" dequantization and "Industry implications: multiplication-free inference"
// (B_re, B_im in {-1, 0, 1}; products reduce to additions, subtractions, skips); 36Kr article,
// parallel stages.
//
// Weight planes are int8 {-1, 0, +1}; x enters as an exact integer: every bf16 value of a batch
// column is scaled by one power of two 2^S (chosen so that max|x| * 2^S < 2^22) and rounded to
// an integer X, which is split into three signed int8 digits X = l0 + 2^8 l1 + 2^16 l2.  All
// products and sums are then exact int32 arithmetic (v_mfma_i32_16x16x64_i8); the only rounding
// is X itself (relative 2^-23 of the column maximum; none for bf16 values within 2^14 of it)
// and the fp32 epilogue.  Why not bf16 MFMA here: on gfx950 MFMA and VALU time add, and this
// form costs half the MFMA cycles and ~0.94 instead of ~1.5 VALU operations per code.
//
//  * Codes -> planes: the packed word of 16 codes holds code 4d+b in bits 8b+2d..8b+2d+1, so
//    (w >> 2d) & 0x03030303 puts codes 4d..4d+3 in bytes 0..3 (column order), and v_perm_b32
//    maps each byte through the 4-entry tables {+1, 0, -1, 0} (B_re) and {0, +1, 0, -1} (B_im).
//  * K assignment: a workgroup owns 16 complex rows; its waves take 256-column chunks in turn.
//    In a chunk lane group g owns columns 64g..64g+63 (one 16-byte load of 4 packed words per
//    plane) and at MFMA step s = 0..3 contributes columns 64g+16s..64g+16s+15.
//  * x digits live in LDS, converted once per workgroup: column c = 8b + 4comp + l of the MFMA
//    (batch b, component a = Re x / b = Im x, digit l, slot 3 empty), row stride m + 16 bytes.
//  * Epilogue: each lane scales its int32 sums by 2^(8l-S) and the fp32 axis scales, then the
//    digits and components of a batch column are summed across lanes (xor 1, 2, 4) and the waves
//    through LDS in a fixed order.
#include "common.hpp"

namespace f2i {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kI8Chunk = 256;
constexpr int kI8MaxWaves = 8;
constexpr int kI8Stride = 16;       // LDS row padding (bytes) against bank conflicts

__device__ __forceinline__ void decode_i8(uint32_t w, v4i& re, v4i& im) {
  constexpr uint32_t lo2 = 0x03030303u;
  constexpr uint32_t kRe = 0x00FF0001u;   // code 0 -> +1, 1 -> 0, 2 -> -1, 3 -> 0
  constexpr uint32_t kIm = 0xFF000100u;   // code 0 -> 0, 1 -> +1, 2 -> 0, 3 -> -1
  const uint32_t k0 = w & lo2, k1 = (w >> 2) & lo2, k2 = (w >> 4) & lo2, k3 = (w >> 6) & lo2;
  re = v4i{(int)__builtin_amdgcn_perm(0u, kRe, k0), (int)__builtin_amdgcn_perm(0u, kRe, k1),
           (int)__builtin_amdgcn_perm(0u, kRe, k2), (int)__builtin_amdgcn_perm(0u, kRe, k3)};
  im = v4i{(int)__builtin_amdgcn_perm(0u, kIm, k0), (int)__builtin_amdgcn_perm(0u, kIm, k1),
           (int)__builtin_amdgcn_perm(0u, kIm, k2), (int)__builtin_amdgcn_perm(0u, kIm, k3)};
}

// Power-of-two exponent S with amax * 2^S < 2^22 (0 for an all-zero column).
__device__ __forceinline__ int digit_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127;   // floor(log2 amax), normal
  return 21 - (e < -126 ? -126 : e);
}

template <int TT, typename YT>
__global__ __launch_bounds__(64 * kI8MaxWaves) void k_gemv_i8(
    const uint8_t* __restrict__ packed, const float* __restrict__ scales, int n, int m,
    const uint16_t* __restrict__ x, int B, YT* __restrict__ y) {
  extern __shared__ __align__(16) int8_t s_x[];          // [16 columns][m + 16]
  __shared__ float s_sc[16][TT][4];
  __shared__ float s_y[kI8MaxWaves][2][2][16];             // [wave][batch][re/im][row]
  __shared__ float s_max[kI8MaxWaves][2];
  const int nw = blockDim.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int i0 = blockIdx.x * 16;
  const int ia = i0 + r;
  const bool a_ok = ia < n;
  const int dw_plane = m / 16;
  const int ld = m + kI8Stride;
  const uint32_t* __restrict__ arow =
      reinterpret_cast<const uint32_t*>(packed) + (int64_t)(a_ok ? ia : 0) * (TT * 2 * dw_plane);
  const int nchunk = (m + kI8Chunk - 1) / kI8Chunk;

  // 1. issue the code loads of the first chunk before anything else
  uint4 wd[TT][2];
  auto load_codes = [&](int c) {
    const int jg = c * kI8Chunk + 64 * g;
    const bool k_ok = a_ok && jg < m;
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int M = 0; M < 2; ++M)
        wd[t][M] = k_ok ? *reinterpret_cast<const uint4*>(arow + (t * 2 + M) * dw_plane + jg / 16)
                        : make_uint4(0u, 0u, 0u, 0u);
  };
  if (wave < nchunk) load_codes(wave);

  // 2. scales of the tile -> LDS
  for (int idx = threadIdx.x; idx < 16 * TT * 4; idx += blockDim.x) {
    const int row = idx / (TT * 4), rest = idx % (TT * 4);
    const int i = i0 + row;
    s_sc[row][rest / 4][rest % 4] = i < n ? scales[(int64_t)i * TT * 4 + rest] : 0.f;
  }

  // 3. x -> exact int8 digits in LDS.  Pass one: column maxima.
  const int per_b = 2 * m;                        // values per batch column
  float amax[2] = {0.f, 0.f};
  for (int b = 0; b < B; ++b)
    for (int j = threadIdx.x * 8; j < per_b; j += blockDim.x * 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(x + (int64_t)b * per_b + j);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) amax[b] = fmaxf(amax[b], fmaxf(fabsf(bf16_lo(w4[h])), fabsf(bf16_hi(w4[h]))));
    }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) amax[b] = fmaxf(amax[b], __shfl_xor(amax[b], off));
    if (lane == 0) s_max[wave][b] = amax[b];
  }
  __syncthreads();
  int S[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float mx = 0.f;
    for (int w = 0; w < nw; ++w) mx = fmaxf(mx, s_max[w][b]);
    S[b] = digit_exponent(mx);
  }
  // Pass two: digits.  Column c = 8b + 4comp + l; slots l = 3 and batches >= B are zero.
  for (int idx = threadIdx.x * 8; idx < 2 * per_b; idx += blockDim.x * 8) {
    const int b = idx / per_b, j2 = idx % per_b;       // j2 in [0, 2m): comp = j2 / m
    const int comp = j2 / m, j = j2 % m;
    uint32_t dg[3][2] = {{0, 0}, {0, 0}, {0, 0}};
    if (b < B) {
      const uint4 v = *reinterpret_cast<const uint4*>(x + (int64_t)b * per_b + j2);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xv = (e & 1) ? bf16_hi(w4[e >> 1]) : bf16_lo(w4[e >> 1]);
        const int X = (int)rintf(ldexpf(xv, S[b]));    // |X| < 2^22, exact scaling
        const int l0 = ((X + 128) & 255) - 128;
        const int X1 = (X - l0) >> 8;
        const int l1 = ((X1 + 128) & 255) - 128;
        const int l2 = (X1 - l1) >> 8;
        const int sh = 8 * (e & 3);
        dg[0][e >> 2] |= (uint32_t)(l0 & 255) << sh;
        dg[1][e >> 2] |= (uint32_t)(l1 & 255) << sh;
        dg[2][e >> 2] |= (uint32_t)(l2 & 255) << sh;
      }
    }
#pragma unroll
    for (int l = 0; l < 3; ++l)
      *reinterpret_cast<uint2*>(s_x + (int64_t)(8 * b + 4 * comp + l) * ld + j) = make_uint2(dg[l][0], dg[l][1]);
  }
  // zero the empty columns (l = 3 of every (b, comp)) once; they are never written above
  for (int idx = threadIdx.x * 8; idx < 4 * m; idx += blockDim.x * 8) {
    const int q = idx / m, j = idx % m;                // q = 2b + comp
    *reinterpret_cast<uint2*>(s_x + (int64_t)(4 * q + 3) * ld + j) = make_uint2(0u, 0u);
  }
  __syncthreads();

  // 4. main loop
  v4i acc[TT][2][2];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int M = 0; M < 2; ++M) { acc[t][M][0] = v4i{0, 0, 0, 0}; acc[t][M][1] = v4i{0, 0, 0, 0}; }
  const int8_t* xcol = s_x + (int64_t)r * ld;          // B column r of this lane
  for (int c = wave; c < nchunk; c += nw) {
    const int jg = c * kI8Chunk + 64 * g;
    const bool k_ok = jg < m;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const v4i bv = k_ok ? *reinterpret_cast<const v4i*>(xcol + jg + 16 * s) : v4i{0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int M = 0; M < 2; ++M) {
          const uint4 q = wd[t][M];
          const uint32_t w = s == 0 ? q.x : s == 1 ? q.y : s == 2 ? q.z : q.w;
          v4i are, aim;
          decode_i8(w, are, aim);
          acc[t][M][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(are, bv, acc[t][M][0], 0, 0, 0);
          acc[t][M][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aim, bv, acc[t][M][1], 0, 0, 0);
        }
    }
    if (c + nw < nchunk) load_codes(c + nw);
  }

  // 5. epilogue.  Lane holds rows 4g..4g+3 of column r = 8b + 4comp + l.
  const int bl = r >> 3, comp = (r >> 2) & 1, l = r & 3;
  const float wdig = ldexpf(1.0f, 8 * l - (bl < 2 ? S[bl] : 0));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = 4 * g + e;
    float vre = 0.f, vim = 0.f;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const float sUr = s_sc[row][t][0], sUi = s_sc[row][t][1];
      const float sWr = s_sc[row][t][2], sWi = s_sc[row][t][3];
      const float CUr = (float)acc[t][0][0][e], CUi = (float)acc[t][0][1][e];
      const float CWr = (float)acc[t][1][0][e], CWi = (float)acc[t][1][1][e];
      if (comp == 0) {    // a = Re x:  Re += sUr*P(U,re) + sWr*P(W,re) ; Im += sUi*P(U,im) + sWi*P(W,im)
        vre += sUr * CUr + sWr * CWr;
        vim += sUi * CUi + sWi * CWi;
      } else {            // b = Im x:  Re += sWi*P(W,im) - sUi*P(U,im) ; Im += sUr*P(U,re) - sWr*P(W,re)
        vre += sWi * CWi - sUi * CUi;
        vim += sUr * CUr - sWr * CWr;
      }
    }
    vre *= wdig;
    vim *= wdig;
#pragma unroll
    for (int off = 1; off <= 4; off <<= 1) {   // digits (1, 2) and components (4)
      vre += __shfl_xor(vre, off);
      vim += __shfl_xor(vim, off);
    }
    if ((r & 7) == 0) {
      s_y[wave][bl][0][row] = vre;
      s_y[wave][bl][1][row] = vim;
    }
  }
  __syncthreads();
  const int64_t ys = 2 * (int64_t)n;
  for (int idx = threadIdx.x; idx < 2 * 2 * 16; idx += blockDim.x) {
    const int row = idx & 15, part = (idx >> 4) & 1, b = idx >> 5;
    const int i = i0 + row;
    if (b < B && i < n) {
      float v = s_y[0][b][part][row];
      for (int w = 1; w < nw; ++w) v += s_y[w][b][part][row];
      store_out(y, (int64_t)b * ys + (part ? n + i : i), v);
    }
  }
}

size_t gemv_i8_lds_bytes(int m) { return (size_t)16 * (m + kI8Stride); }

hipError_t launch_gemv_i8(const uint8_t* packed, const float* scales, int n, int m, int T,
                          const void* x, int B, void* y, int y_bf16, hipStream_t s) {
  const int nchunk = (m + kI8Chunk - 1) / kI8Chunk;
  const int nw = nchunk < kI8MaxWaves ? nchunk : kI8MaxWaves;
  const dim3 grid((n + 15) / 16), block(64 * nw);
  const size_t lds = gemv_i8_lds_bytes(m);
  const uint16_t* xx = static_cast<const uint16_t*>(x);
#define F2I_GEMV_I8(TT, YT)                                                                       \
  do {                                                                                            \
    auto kern = k_gemv_i8<TT, YT>;                                                                \
    if (lds > 65536) {                                                                            \
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),                     \
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);   \
      if (e != hipSuccess) return e;                                                              \
    }                                                                                             \
    hipLaunchKernelGGL(kern, grid, block, lds, s, packed, scales, n, m, xx, B, static_cast<YT*>(y)); \
  } while (0)
  if (y_bf16) {
    switch (T) {
      case 1: F2I_GEMV_I8(1, uint16_t); break;
      case 2: F2I_GEMV_I8(2, uint16_t); break;
      case 3: F2I_GEMV_I8(3, uint16_t); break;
      default: F2I_GEMV_I8(4, uint16_t); break;
    }
  } else {
    switch (T) {
      case 1: F2I_GEMV_I8(1, float); break;
      case 2: F2I_GEMV_I8(2, float); break;
      case 3: F2I_GEMV_I8(3, float); break;
      default: F2I_GEMV_I8(4, float); break;
    }
  }
#undef F2I_GEMV_I8
  return hipGetLastError();
}

}  // namespace f2i
