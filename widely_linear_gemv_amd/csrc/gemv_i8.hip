// Decode GEMV for batch 1-2 on the int8 matrix cores: y = sum_t U~(t) x + W~(t) conj(x).
//
// Sources: ModelScope card "Fairy2i-W2", "Method" (y = U x + W conj(x)); zhichai.net reading
// note, "Step 2" dequantization and "Industry implications: multiplication-free inference"
// (B_re, B_im in {-1, 0, 1}; products reduce to additions, subtractions, skips); 36Kr article,
// parallel stages.
//
// Weight planes are int8 {-1, 0, +1}; x enters as an exact integer.  A separate pass turns x
// into its digit form once: each batch column b is scaled by one power of two 2^S_b (chosen so
// that max|x_b| 2^S_b lies in [2^21, 2^22)) and rounded to an integer X, split into three signed
// int8 digits X = d0 + 2^8 d1 + 2^16 d2.  All products and sums of the GEMV are then exact
// int32 arithmetic (v_mfma_i32_16x16x64_i8); the only roundings are X itself (none for a bf16
// value no more than 2^14 below its column maximum) and the fp32 epilogue.  Against the bf16
// matrix-core form this halves the MFMA cycles per code (64 columns per instruction instead of
// 32) and needs ~0.94 instead of ~1.5 VALU operations per code for the planes; on gfx950 the
// two add up on a SIMD, so their sum sets the speed once the codes stream at full bandwidth.
//
//  * Digit form (one buffer per x): int32 header [B, m, S_0, S_1] in the first 64 bytes, then
//    int8 [B][2][4][m] -- batch column, component (a = Re x, b = Im x), digit slot (3 = zero).
//  * Codes -> planes: the packed word of 16 codes holds code 4d+b in bits 8b+2d..8b+2d+1, so
//    (w >> 2d) & 0x03030303 puts codes 4d..4d+3 in bytes 0..3 (column order), and v_perm_b32
//    maps each byte through the 4-entry tables {+1, 0, -1, 0} (B_re) and {0, +1, 0, -1} (B_im).
//  * B operand: MFMA column c = 8b + 4comp + l holds digit l of component comp of batch entry
//    b; lane (c, g) loads the 16 digits of its k-group straight from the digit form.
//  * K assignment and grouping as in the bf16 kernel: one wave owns a 16-row tile of one item
//    of a grouped or strided call and streams its 256-column chunks, one 1 KB load per plane, prefetching
//    the next chunk's codes and digits while the current one is decoded and multiplied.  In a
//    chunk lane group g owns columns 64g..64g+63 and at MFMA step s contributes columns
//    64g+16s..+15.
//  * Epilogue: each lane scales its int32 sums by 2^(8l - S_b) and the fp32 axis scales, and
//    the digits and components of a batch entry are summed across its 8 lanes on DPP lane
//    permutes (group_sum).
#include "common.hpp"
#include "digits.hpp"

namespace f2i {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kI8Chunk = 256;

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

// ------------------------------------------------------------------ digit form of x ----

// One workgroup of 1024 threads per batch column: max |x| (order-free, exact), S, then the
// digits of all 2m values and the zero slot.  For 2m <= 8192 every thread keeps its 8 values in
// registers between the two passes; longer columns are read twice.
constexpr int kDigitThreads = 1024;

template <typename XT>
__global__ __launch_bounds__(kDigitThreads) void k_x_digits(const XT* __restrict__ x, int m, int B,
                                                            uint8_t* __restrict__ blob) {
  __shared__ float s_max[kDigitThreads / kWave];
  const int b = blockIdx.x;
  const XT* __restrict__ xb = x + (int64_t)b * 2 * m;
  const int stride = kDigitThreads * 8;
  const bool one_pass = 2 * m <= stride;
  float keep[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float amax = column_amax<XT, kDigitThreads>(xb, 2 * m, keep, s_max);
  const int S = digit_exponent(amax);
  // 2^S as two exact power-of-two factors (S can exceed the fp32 exponent range for tiny columns)
  const float f1 = ldexpf(1.0f, S / 2), f2 = ldexpf(1.0f, S - S / 2);
  int* hdr = reinterpret_cast<int*>(blob);
  if (threadIdx.x == 0) {
    if (b == 0) { hdr[0] = B; hdr[1] = m; }
    hdr[2 + b] = S;
  }
  int8_t* __restrict__ dg = reinterpret_cast<int8_t*>(blob + kDigitHeader) + (int64_t)b * 8 * m;
  for (int j2 = threadIdx.x * 8; j2 < 2 * m; j2 += stride) {
    const int comp = j2 / m, j = j2 % m;         // m % 64 == 0: 8 values never straddle comps
    float v[8];
    if (one_pass) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = keep[e];
    } else {
      Load8x<XT>::run(xb + j2, v);
    }
    uint32_t d[3][2] = {{0u, 0u}, {0u, 0u}, {0u, 0u}};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int X = (int)rintf((v[e] * f1) * f2);     // |X| <= 2^22, scaling exact
      const int l0 = ((X + 128) & 255) - 128;
      const int X1 = (X - l0) >> 8;
      const int l1 = ((X1 + 128) & 255) - 128;
      const int l2 = (X1 - l1) >> 8;
      const int sh = 8 * (e & 3);
      d[0][e >> 2] |= (uint32_t)(l0 & 255) << sh;
      d[1][e >> 2] |= (uint32_t)(l1 & 255) << sh;
      d[2][e >> 2] |= (uint32_t)(l2 & 255) << sh;
    }
    int8_t* base = dg + (int64_t)comp * 4 * m + j;
#pragma unroll
    for (int l = 0; l < 3; ++l) *reinterpret_cast<uint2*>(base + (int64_t)l * m) = make_uint2(d[l][0], d[l][1]);
    *reinterpret_cast<uint2*>(base + (int64_t)3 * m) = make_uint2(0u, 0u);
  }
}

size_t x_digits_bytes(int64_t m, int64_t B) { return (size_t)kDigitHeader + (size_t)B * 8 * (size_t)m; }

hipError_t launch_x_digits(const void* x, int x_bf16, int m, int B, void* blob, hipStream_t s) {
  if (x_bf16)
    hipLaunchKernelGGL(k_x_digits<uint16_t>, dim3(B), dim3(kDigitThreads), 0, s, static_cast<const uint16_t*>(x), m, B,
                       static_cast<uint8_t*>(blob));
  else
    hipLaunchKernelGGL(k_x_digits<float>, dim3(B), dim3(kDigitThreads), 0, s, static_cast<const float*>(x), m, B,
                       static_cast<uint8_t*>(blob));
  return hipGetLastError();
}

// ------------------------------------------------------------------------- GEMV ----

template <int TT, int NW, typename YT>
__global__ __launch_bounds__(kWave * NW) void k_gemv_i8(const GemvGroup grp, int m, int B) {
  int tile;
  const GemvItem it = locate_item<YT>(grp, blockIdx.x, tile);
  const int n = it.n;
  const uint8_t* __restrict__ packed = static_cast<const uint8_t*>(it.packed);
  const float* __restrict__ scales = it.scales;
  const uint8_t* __restrict__ blob = static_cast<const uint8_t*>(it.x);
  YT* __restrict__ y = static_cast<YT*>(it.y);

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
  const int r = lane & 15, g = lane >> 4;
  const int i0 = tile * 16;
  const int64_t tile_bytes = (int64_t)16 * TT * 2 * (m / 4);
  // The tile's codes and the digit form through buffer resources: batch entries past B read 0,
  // and so does every load of a lane group past column m (offset kNoLoad).
  const __amdgpu_buffer_rsrc_t rsrc_a = range_rsrc(packed + (int64_t)tile * tile_bytes, tile_bytes);
  const __amdgpu_buffer_rsrc_t rsrc_x = range_rsrc(blob + kDigitHeader, (int64_t)B * 8 * m);
  const uint32_t voff_x = (uint32_t)(r * m);          // column r = 8b + 4comp + l -> slot r

  v4i acc[TT][2][2];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int M = 0; M < 2; ++M) { acc[t][M][0] = v4i{0, 0, 0, 0}; acc[t][M][1] = v4i{0, 0, 0, 0}; }

  const int nchunk = (m + kI8Chunk - 1) / kI8Chunk;
  // Operands of one chunk: every plane's 16-row x 256-column block (1 KB when the chunk is full:
  // lane l = 16g + r takes row r, columns 64g..64g+63) and the digits of every MFMA step.
  struct Chunk { uint4 w[TT][2]; v4i x[4]; };
  auto load_chunk = [&](int c, Chunk& ch) {
    const int groups = min(4, (m - kI8Chunk * c) >> 6);
    const bool k_ok = g < groups;
    const uint32_t cbase = (uint32_t)c * (TT * 2) * 1024;
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int M = 0; M < 2; ++M)
        ch.w[t][M] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
            rsrc_a, k_ok ? cbase + (uint32_t)((t * 2 + M) * groups * 256 + lane * 16) : kNoLoad, 0, kStreamLoad));
    const int jg = c * kI8Chunk + 64 * g;            // first column of this lane group
#pragma unroll
    for (int s = 0; s < 4; ++s)
      ch.x[s] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
          rsrc_x, k_ok ? voff_x + (uint32_t)(jg + 16 * s) : kNoLoad, 0, 0));
  };
  auto compute_chunk = [&](const Chunk& ch) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int M = 0; M < 2; ++M) {
          const uint4 q = ch.w[t][M];
          const uint32_t w = s == 0 ? q.x : s == 1 ? q.y : s == 2 ? q.z : q.w;
          v4i are, aim;
          decode_i8(w, are, aim);
          acc[t][M][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(are, ch.x[s], acc[t][M][0], 0, 0, 0);
          acc[t][M][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aim, ch.x[s], acc[t][M][1], 0, 0, 0);
        }
  };
  // The chunks stream through two operand sets; the scheduling barriers keep each prefetch
  // ahead of the compute it overlaps (the scheduler would otherwise sink the loads to their
  // use).  The prefetch is unconditional, so every path has the same loads in flight; one past
  // the last chunk has a negative group count and loads at the out-of-range offset (reads nothing).
  __shared__ float s_sc[NW][16 * TT * 4];
  TileScales<TT> tsc;
  tsc.load(scales, i0, n, lane);               // ahead of the first chunk's loads
  {
    Chunk c0, c1;
    int c = wave;                                  // wave w takes chunks w, w + NW, ...
    load_chunk(c, c0);
    tsc.park(s_sc[wave], lane);
    for (; c + NW < nchunk; c += 2 * NW) {
      load_chunk(c + NW, c1);
      __builtin_amdgcn_sched_barrier(0);
      compute_chunk(c0);
      load_chunk(c + 2 * NW, c0);
      __builtin_amdgcn_sched_barrier(0);
      compute_chunk(c1);
    }
    if (c < nchunk) compute_chunk(c0);
  }

  // Epilogue.  Lane holds rows 4g..4g+3 of column r = 8b + 4comp + l.  With several waves per
  // tile their sums meet in LDS and are added in wave order.
  __shared__ float s_y[NW > 1 ? NW : 1][2][2][16];      // [wave][batch][re/im][row]
  const int bl = r >> 3, comp = (r >> 2) & 1, l = r & 3;
  const int* hdr = reinterpret_cast<const int*>(blob);
  const int S = bl < B ? hdr[2 + bl] : 0;
  const float wdig = ldexpf(1.0f, 8 * l - S);
  const int64_t ys = 2 * (int64_t)n;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = i0 + 4 * g + e;
    const float* sc = &s_sc[wave][(4 * g + e) * TT * 4];
    float vre = 0.f, vim = 0.f;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const float sUr = sc[4 * t], sUi = sc[4 * t + 1], sWr = sc[4 * t + 2], sWi = sc[4 * t + 3];
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
    vre = group_sum<8>(vre);                    // digits (lanes ^ 1, ^ 2) and components (^ 4)
    vim = group_sum<8>(vim);
    if (NW > 1) {
      if ((r & 7) == 0) { s_y[wave][bl][0][4 * g + e] = vre; s_y[wave][bl][1][4 * g + e] = vim; }
    } else if ((r & 7) == 0 && bl < B && i < n) {
      store_out(y, (int64_t)bl * ys + i, vre);
      store_out(y, (int64_t)bl * ys + n + i, vim);
    }
  }
  if constexpr (NW > 1) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < 2 * 2 * 16; idx += kWave * NW) {
      const int row = idx & 15, part = (idx >> 4) & 1, b = idx >> 5;
      const int i = i0 + row;
      if (b < B && i < n) {
        float v = s_y[0][b][part][row];
        for (int w = 1; w < NW; ++w) v += s_y[w][b][part][row];
        store_out(y, (int64_t)b * ys + (part ? n + i : i), v);
      }
    }
  }
}

template <int TT, typename YT>
static void launch_i8_t(const GemvGroup& group, int m, int B, hipStream_t s) {
  GemvGroup grp = group;
  grp.units_per_item = grp.tiles_per_item;        // one workgroup per tile
  const int tiles = group_tiles(grp);
  const dim3 grid(tiles);
  switch (gemv_waves_per_tile(tiles, m)) {
    case 8: hipLaunchKernelGGL((k_gemv_i8<TT, 8, YT>), grid, dim3(8 * kWave), 0, s, grp, m, B); break;
    case 4: hipLaunchKernelGGL((k_gemv_i8<TT, 4, YT>), grid, dim3(4 * kWave), 0, s, grp, m, B); break;
    case 2: hipLaunchKernelGGL((k_gemv_i8<TT, 2, YT>), grid, dim3(2 * kWave), 0, s, grp, m, B); break;
    default: hipLaunchKernelGGL((k_gemv_i8<TT, 1, YT>), grid, dim3(kWave), 0, s, grp, m, B); break;
  }
}

hipError_t launch_gemv_i8_group(const GemvGroup& grp, int m, int T, int B, int y_bf16, hipStream_t s) {
  if (y_bf16) {
    switch (T) {
      case 1: launch_i8_t<1, uint16_t>(grp, m, B, s); break;
      case 2: launch_i8_t<2, uint16_t>(grp, m, B, s); break;
      case 3: launch_i8_t<3, uint16_t>(grp, m, B, s); break;
      default: launch_i8_t<4, uint16_t>(grp, m, B, s); break;
    }
  } else {
    switch (T) {
      case 1: launch_i8_t<1, float>(grp, m, B, s); break;
      case 2: launch_i8_t<2, float>(grp, m, B, s); break;
      case 3: launch_i8_t<3, float>(grp, m, B, s); break;
      default: launch_i8_t<4, float>(grp, m, B, s); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_gemv_i8(const uint8_t* packed, const float* scales, int n, int m, int T,
                          const void* digits, int B, void* y, int y_bf16, hipStream_t s) {
  GemvGroup grp;
  grp.count = 1;
  grp.tile_start[0] = 0;
  grp.tile_start[1] = (n + 15) / 16;
  grp.items[0] = GemvItem{packed, scales, digits, y, n};
  return launch_gemv_i8_group(grp, m, T, B, y_bf16, s);
}

}  // namespace f2i
