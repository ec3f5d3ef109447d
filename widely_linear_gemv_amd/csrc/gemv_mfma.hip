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
//  * K assignment: a workgroup handles 16 rows; its waves (up to 8) take 256-column chunks in
//    turn.  In a chunk, lane group g owns columns 64g..64g+63 (one 16-byte load of 4 words per
//    plane) and at MFMA step s = 0..7 contributes columns 64g+8s .. 64g+8s+7.  All loads of a
//    chunk (codes of every plane, x of every step) are issued before the first MFMA, and the
//    rows' scales are staged in LDS at kernel start: a small layer is one memory round trip.
//  * Grouped launches: one grid covers the row tiles of several GEMVs of the same m (for
//    example the q, k and v projections that share x); each workgroup finds its GEMV by binary
//    search over the first-tile table passed in the kernel arguments.
//  * B operand (32 x 16, bf16): columns are (batch b, component a = Re x or b = Im x); 8 batch
//    columns per MFMA, two column groups for B > 8.  Each lane loads 8 consecutive bf16 of x and
//    swaps elements 1,2 and 5,6 with v_perm_b32.
//  * One 16x16 fp32 accumulator per (stage, matrix, plane, column group).  The epilogue applies
//    the fp32 scales (and the factor 1/2 of the +-2 encoding) once per accumulated sum, adds the
//    a and b columns of a batch entry across two lanes, and sums the waves through LDS in a
//    fixed order.
#include "common.hpp"

namespace f2i {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kChunk = 256;        // columns per wave work unit
constexpr int kMaxWaves = 8;       // upper bound of waves per 16-row tile (LDS sizing)
constexpr int kWavesPerTile = 4;   // waves per tile; each streams its chunks with prefetch

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

// x[j0 .. j0+7] (bf16, as loaded) -> B operand in element order (0, 2, 1, 3, 4, 6, 5, 7).
__device__ __forceinline__ v4u permute_b(uint4 w) {
  return v4u{__builtin_amdgcn_perm(w.y, w.x, 0x05040100u), __builtin_amdgcn_perm(w.y, w.x, 0x07060302u),
             __builtin_amdgcn_perm(w.w, w.z, 0x05040100u), __builtin_amdgcn_perm(w.w, w.z, 0x07060302u)};
}

// Workgroup tile -> GEMV item: first tile of every item (tile_start[count] = total tiles).
__device__ __forceinline__ int find_item(const GemvGroup& g, int tile) {
  int lo = 0, hi = g.count - 1;
  while (lo < hi) {                       // last item with tile_start <= tile
    const int mid = (lo + hi + 1) >> 1;
    if (g.tile_start[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int TT, int CG, typename YT>
__global__ __launch_bounds__(64 * kMaxWaves) void k_gemv_mfma(const GemvGroup grp, int m, int B) {
  __shared__ float s_sc[16][TT][4];              // halved scales of the tile's rows
  __shared__ float s_y[kMaxWaves][16][2][16];    // [wave][batch][re/im][row]
  const int item = find_item(grp, blockIdx.x);
  const GemvItem it = grp.items[item];
  const int n = it.n;
  const uint8_t* __restrict__ packed = static_cast<const uint8_t*>(it.packed);
  const float* __restrict__ scales = it.scales;
  const uint16_t* __restrict__ x = static_cast<const uint16_t*>(it.x);
  YT* __restrict__ y = static_cast<YT*>(it.y);

  const int nw = blockDim.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int i0 = (blockIdx.x - grp.tile_start[item]) * 16;
  const int ia = i0 + r;
  const bool a_ok = ia < n;
  const int dw_plane = m / 16;
  const uint32_t* __restrict__ arow =
      reinterpret_cast<const uint32_t*>(packed) + (int64_t)(a_ok ? ia : 0) * (TT * 2 * dw_plane);

  // Scales of the 16 rows go to LDS now, so the epilogue needs no global round trip.
  for (int idx = threadIdx.x; idx < 16 * TT * 4; idx += blockDim.x) {
    const int row = idx / (TT * 4), rest = idx % (TT * 4);
    const int i = i0 + row;
    s_sc[row][rest / 4][rest % 4] = i < n ? 0.5f * scales[(int64_t)i * TT * 4 + rest] : 0.f;
  }

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
  constexpr bool kPrefetch = CG == 1;              // two column groups need the registers
  uint4 wd[TT][2], xr[8][CG];                      // operands of the chunk being computed
  auto load_chunk = [&](int c, uint4 (&w)[TT][2], uint4 (&xx)[8][CG]) {
    const int jg = c * kChunk + 64 * g;            // first column of this lane group
    const bool k_ok = c < nchunk && jg < m;        // m % 64 == 0: a group is all in or all out
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int M = 0; M < 2; ++M)
        w[t][M] = (a_ok && k_ok)
            ? *reinterpret_cast<const uint4*>(arow + (t * 2 + M) * dw_plane + jg / 16)
            : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int cg = 0; cg < CG; ++cg)
        xx[s][cg] = (b_ok[cg] && k_ok) ? *reinterpret_cast<const uint4*>(xb[cg] + jg + 8 * s)
                                       : make_uint4(0u, 0u, 0u, 0u);
  };
  load_chunk(wave, wd, xr);
  for (int c = wave; c < nchunk; c += nw) {
    // prefetch the next chunk of this wave while the current one is decoded and multiplied
    uint4 wn[TT][2], xn[8][CG];
    if (kPrefetch && c + nw < nchunk) load_chunk(c + nw, wn, xn);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      v4u bv[CG];
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) bv[cg] = permute_b(xr[s][cg]);
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
    if (!kPrefetch) {
      if (c + nw < nchunk) load_chunk(c + nw, wd, xr);
    } else if (c + nw < nchunk) {
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int M = 0; M < 2; ++M) wd[t][M] = wn[t][M];
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int cg = 0; cg < CG; ++cg) xr[s][cg] = xn[s][cg];
    }
  }
  __syncthreads();                                 // s_sc is ready

  // Epilogue.  C tile: lane holds rows 4g..4g+3 of column r = 2*bl + comp.
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = 4 * g + e;
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      float vre = 0.f, vim = 0.f;
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const float sUr = s_sc[row][t][0], sUi = s_sc[row][t][1];
        const float sWr = s_sc[row][t][2], sWi = s_sc[row][t][3];
        const float CUr = acc[t][0][0][cg][e], CUi = acc[t][0][1][cg][e];
        const float CWr = acc[t][1][0][cg][e], CWi = acc[t][1][1][cg][e];
        if (comp == 0) {    // a = Re x:  Re += sUr*P(U,re) + sWr*P(W,re) ; Im += sUi*P(U,im) + sWi*P(W,im)
          vre += sUr * CUr + sWr * CWr;
          vim += sUi * CUi + sWi * CWi;
        } else {            // b = Im x:  Re += sWi*P(W,im) - sUi*P(U,im) ; Im += sUr*P(U,re) - sWr*P(W,re)
          vre += sWi * CWi - sUi * CUi;
          vim += sUr * CUr - sWr * CWr;
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
  for (int idx = threadIdx.x; idx < 16 * 2 * 16; idx += blockDim.x) {
    const int row = idx & 15, part = (idx >> 4) & 1, b = idx >> 5;
    const int i = i0 + row;
    if (b < B && i < n) {
      float v = s_y[0][b][part][row];
      for (int w = 1; w < nw; ++w) v += s_y[w][b][part][row];
      store_out(y, (int64_t)b * ys + (part ? n + i : i), v);
    }
  }
}

template <int TT, typename YT>
static void launch_t(const GemvGroup& grp, int m, int B, hipStream_t s) {
  const int nchunk = (m + kChunk - 1) / kChunk;
  const int nw = nchunk < kWavesPerTile ? nchunk : kWavesPerTile;
  const dim3 grid(grp.tile_start[grp.count]), block(64 * nw);
  if (B <= 8)
    hipLaunchKernelGGL((k_gemv_mfma<TT, 1, YT>), grid, block, 0, s, grp, m, B);
  else
    hipLaunchKernelGGL((k_gemv_mfma<TT, 2, YT>), grid, block, 0, s, grp, m, B);
}

hipError_t launch_gemv_mfma_group(const GemvGroup& grp, int m, int T, int B, int y_bf16, hipStream_t s) {
  if (y_bf16) {
    switch (T) {
      case 1: launch_t<1, uint16_t>(grp, m, B, s); break;
      case 2: launch_t<2, uint16_t>(grp, m, B, s); break;
      case 3: launch_t<3, uint16_t>(grp, m, B, s); break;
      default: launch_t<4, uint16_t>(grp, m, B, s); break;
    }
  } else {
    switch (T) {
      case 1: launch_t<1, float>(grp, m, B, s); break;
      case 2: launch_t<2, float>(grp, m, B, s); break;
      case 3: launch_t<3, float>(grp, m, B, s); break;
      default: launch_t<4, float>(grp, m, B, s); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_gemv_mfma(const uint8_t* packed, const float* scales, int n, int m, int T,
                            const void* x, int B, void* y, int y_bf16, void*, hipStream_t s) {
  GemvGroup grp;
  grp.count = 1;
  grp.tile_start[0] = 0;
  grp.tile_start[1] = (n + 15) / 16;
  grp.items[0] = GemvItem{packed, scales, x, y, n};
  return launch_gemv_mfma_group(grp, m, T, B, y_bf16, s);
}

}  // namespace f2i
