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
//  * K assignment: one wave owns a 16-row tile and streams its 256-column chunks, the next
//    chunk's loads in flight while the current one is multiplied.  The packed form stores a
//    tile's (chunk, plane) block as 16 rows x 64-column groups of 16 bytes in [group][row]
//    order, so each plane of a chunk is one 1 KB load with lane l = 16g + r taking row r,
//    columns 64g..64g+63; at MFMA step s = 0..7 lane group g contributes columns
//    64g+8s .. 64g+8s+7.
//  * Grouped launches: one grid covers the row tiles of several GEMVs of the same m (for
//    example the q, k and v projections that share x); each workgroup finds its GEMV by binary
//    search over the first-tile table passed in the kernel arguments, or, for a strided batch of
//    same-shape GEMVs, by one division (operands at fixed strides, no table).
//  * B operand (32 x 16, bf16): columns are (batch b, component a = Re x or b = Im x); 8 batch
//    columns per MFMA, two column groups for B > 8.  Each lane loads 8 consecutive bf16 of x and
//    swaps elements 1,2 and 5,6 with v_perm_b32.
//  * One 16x16 fp32 accumulator per (stage, matrix, plane, column group).  The epilogue applies
//    the fp32 scales (and the factor 1/2 of the +-2 encoding) once per accumulated sum and adds
//    the a and b columns of a batch entry across two lanes.
//  * Large launches at batch 3-16 (k_gemv_mfma_sx): a workgroup takes 8 consecutive tiles of one
//    item, one per wave, and stages each chunk's x -- the same for all 8 -- once in LDS, already
//    permuted into the B-operand order; the waves read their B operands from there.  Loading x
//    per wave costs as many bytes as the codes at B = 4 and four times as many at B = 16, and
//    holding two chunks of it in registers leaves one wave per SIMD; shared, it costs neither.
#include "common.hpp"

namespace f2i {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kChunk = 256;        // columns per chunk of the packed form
// Long rows (the LONG kernels, rows of more than kFlushChunks chunks): a wave's accumulators take
// at most kFlushChunks of its chunks (8 MFMA steps each) before their sums are applied to the
// scales and added to per-lane output partials; the accumulators then restart from zero.  Each
// fp32 sum so runs over at most 256 MFMA steps plus one output partial per kFlushChunks chunks,
// instead of m / 32 steps in series, which keeps the rounding of the longest accepted rows (2^22
// columns) within the fp32 tolerance.  Rows of up to 8192 columns (every LLaMA-2-7B shape) take
// the plain kernels, whose registers the flush would otherwise crowd.
constexpr int kFlushChunks = 32;

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

template <int TT, int CG>
__device__ __forceinline__ void combine_row(const v4f (&acc)[TT][2][2][CG], const float* sc, int e, int cg,
                                            int comp, float& vre, float& vim) {
  vre = 0.f;
  vim = 0.f;
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const float sUr = 0.5f * sc[4 * t], sUi = 0.5f * sc[4 * t + 1];
    const float sWr = 0.5f * sc[4 * t + 2], sWi = 0.5f * sc[4 * t + 3];
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
}

// Applies the accumulated sums of every row and column group to the tile's scales, adds them to
// the output partials and clears the accumulators (long rows; see kFlushChunks).
template <int TT, int CG>
__device__ __forceinline__ void flush_partials(v4f (&acc)[TT][2][2][CG], const float* s_scw, int g, int comp,
                                               float (&ypart)[4][CG][2], bool& flushed) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      float vre, vim;
      combine_row<TT, CG>(acc, &s_scw[(4 * g + e) * TT * 4], e, cg, comp, vre, vim);
      ypart[e][cg][0] = flushed ? ypart[e][cg][0] + vre : vre;
      ypart[e][cg][1] = flushed ? ypart[e][cg][1] + vim : vim;
    }
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int M = 0; M < 2; ++M)
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int cg = 0; cg < CG; ++cg) acc[t][M][p][cg] = v4f{0.f, 0.f, 0.f, 0.f};
  flushed = true;
}

// At most eight batch columns (CG = 1) the hint of two waves per SIMD keeps every accumulator in
// the arch registers: without it the allocator placed some of them in the accumulation registers
// and moved them back and forth every iteration (12-80 moves per 64-130 MFMAs at T = 2), taking
// 240 registers where 148 do (three waves per SIMD); with two column groups the same hint spills.
template <int TT, int CG, int NW, typename YT, bool LONG>
__global__ __launch_bounds__(kWave * NW, CG == 1 ? 2 : 1) void k_gemv_mfma(const GemvGroup grp, int m, int B) {
  int tile;
  const GemvItem it = locate_item<YT>(grp, blockIdx.x, tile);
  const int n = it.n;
  const uint8_t* __restrict__ packed = static_cast<const uint8_t*>(it.packed);
  const float* __restrict__ scales = it.scales;
  const uint16_t* __restrict__ x = static_cast<const uint16_t*>(it.x);
  YT* __restrict__ y = static_cast<YT*>(it.y);

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
  const int r = lane & 15, g = lane >> 4;
  const int i0 = tile * 16;
  const int64_t tile_bytes = (int64_t)16 * TT * 2 * (m / 4);
  // The tile's codes and x through buffer resources: batch entries past B read 0, and so does
  // every load of a lane group past column m (offset kNoLoad).
  const __amdgpu_buffer_rsrc_t rsrc_a = range_rsrc(packed + (int64_t)tile * tile_bytes, tile_bytes);
  const __amdgpu_buffer_rsrc_t rsrc_x = range_rsrc(x, (int64_t)B * 2 * m * 2);

  // B column of this lane: batch b = 8*cg + (r >> 1), component r & 1
  const int comp = r & 1;
  uint32_t voff_x[CG];
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) voff_x[cg] = (uint32_t)(((cg * 8 + (r >> 1)) * 2 * m + comp * m) * 2);

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
  // Operands of one chunk: every plane's 16-row x 256-column block (1 KB when the chunk is
  // full: lane l = 16g + r takes bytes 16l.., i.e. row r, columns 64g..64g+63) and x of every
  // MFMA step.
  struct Chunk { uint4 w[TT][2]; uint4 x[8][CG]; };
  auto load_chunk = [&](int c, Chunk& ch) {
    const int groups = min(4, (m - kChunk * c) >> 6);
    const bool k_ok = g < groups;
    const uint32_t cbase = (uint32_t)c * (TT * 2) * 1024;
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int M = 0; M < 2; ++M)
        ch.w[t][M] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
            rsrc_a, k_ok ? cbase + (uint32_t)((t * 2 + M) * groups * 256 + lane * 16) : kNoLoad, 0, kStreamLoad));
    const int jg = c * kChunk + 64 * g;            // first column of this lane group
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int cg = 0; cg < CG; ++cg)
        ch.x[s][cg] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
            rsrc_x, k_ok ? voff_x[cg] + (uint32_t)((jg + 8 * s) * 2) : kNoLoad, 0, 0));
  };
  auto compute_chunk = [&](const Chunk& ch) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      v4u bv[CG];
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) bv[cg] = permute_b(ch.x[s][cg]);
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int M = 0; M < 2; ++M) {
          const uint4 q = ch.w[t][M];
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
  };
  // The chunks stream through two operand sets: the next chunk's loads are issued before the
  // current one is decoded and multiplied.  The scheduling barriers keep each prefetch ahead of
  // the compute it overlaps (the scheduler would otherwise sink the loads to their use).  The
  // prefetch is unconditional, so every path has the same loads in flight; one past the last
  // chunk has a negative group count and loads at the out-of-range offset (reads nothing).
  __shared__ float s_sc[NW][16 * TT * 4];
  float ypart[4][CG][2];                         // output partials of long rows
  bool flushed = false;
  TileScales<TT> tsc;
  tsc.load(scales, i0, n, lane);               // ahead of the first chunk's loads
  {
    Chunk c0, c1;
    int c = wave;                                  // wave w takes chunks w, w + NW, ...
    int pairs = 0;
    load_chunk(c, c0);
    tsc.park(s_sc[wave], lane);
    for (; c + NW < nchunk; c += 2 * NW) {
      load_chunk(c + NW, c1);
      __builtin_amdgcn_sched_barrier(0);
      compute_chunk(c0);
      load_chunk(c + 2 * NW, c0);
      __builtin_amdgcn_sched_barrier(0);
      compute_chunk(c1);
      if constexpr (LONG) {
        if (++pairs == kFlushChunks / 2 && c + 2 * NW < nchunk) {   // wave-uniform
          pairs = 0;
          flush_partials<TT, CG>(acc, s_sc[wave], g, comp, ypart, flushed);
        }
      }
    }
    if (c < nchunk) compute_chunk(c0);
  }

  // Epilogue.  C tile: lane holds rows 4g..4g+3 of column r = 2*bl + comp.  Scales are halved
  // (the planes carry +-2).  With several waves per tile their sums meet in LDS and are added
  // in wave order.
  __shared__ float s_y[NW > 1 ? NW : 1][16][2][16];     // [wave][batch][re/im][row]
  const int64_t ys = 2 * (int64_t)n;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = i0 + 4 * g + e;
    const float* sc = &s_sc[wave][(4 * g + e) * TT * 4];
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      float vre, vim;
      combine_row<TT, CG>(acc, sc, e, cg, comp, vre, vim);
      if (LONG && flushed) {
        vre = ypart[e][cg][0] + vre;
        vim = ypart[e][cg][1] + vim;
      }
      vre = group_sum<2>(vre);
      vim = group_sum<2>(vim);
      const int b = cg * 8 + (r >> 1);
      if (NW > 1) {
        if (comp == 0) { s_y[wave][b][0][4 * g + e] = vre; s_y[wave][b][1][4 * g + e] = vim; }
      } else if (comp == 0 && b < B && i < n) {
        store_out(y, (int64_t)b * ys + i, vre);
        store_out(y, (int64_t)b * ys + n + i, vim);
      }
    }
  }
  if constexpr (NW > 1) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < 8 * CG * 2 * 16; idx += kWave * NW) {
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

constexpr int kSxWaves = 8;             // tiles (waves) per workgroup of the shared-x kernel
constexpr int kSxPitch = 2 * kChunk + 16;  // LDS bytes per (batch, component) row of a chunk's x

// Shared-x form for large launches.  grp.tile_start (units_per_item in a strided batch) counts
// workgroups of kSxWaves tiles here, so a workgroup never spans two items (their x differ); tiles
// past an item's last read no codes and store nothing.  Per chunk the workgroup stages x[b][comp][256 columns] (bf16, permuted per 8
// columns) in one of two LDS buffers, one 16-byte unit per thread and column group, and waits
// once; codes are loaded one chunk ahead as in k_gemv_mfma.
template <int TT, int CG, typename YT, bool LONG>
__global__ __launch_bounds__(kWave * kSxWaves) void k_gemv_mfma_sx(const GemvGroup grp, int m, int B) {
  constexpr int kXRows = 16 * CG;                 // (batch, component) rows of the B operand
  constexpr int kSeg = kXRows * (2 * kChunk / 16) / (kWave * kSxWaves);   // 16-byte units per thread
  static_assert(kSeg * kWave * kSxWaves == kXRows * (2 * kChunk / 16), "whole units per thread");
  __shared__ __align__(16) uint8_t s_x[2][kXRows * kSxPitch];
  int unit;
  const GemvItem it = locate_item<YT>(grp, blockIdx.x, unit);
  const int n = it.n;
  const uint8_t* __restrict__ packed = static_cast<const uint8_t*>(it.packed);
  const float* __restrict__ scales = it.scales;
  const uint16_t* __restrict__ x = static_cast<const uint16_t*>(it.x);
  YT* __restrict__ y = static_cast<YT*>(it.y);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform
  const int r = lane & 15, g = lane >> 4;
  const int comp = r & 1;
  const int tiles = (n + 15) / 16;
  const int tile = kSxWaves * unit + wave;
  const int i0 = tile * 16;
  const int64_t tile_bytes = (int64_t)16 * TT * 2 * (m / 4);
  const __amdgpu_buffer_rsrc_t rsrc_a =
      range_rsrc(packed + (int64_t)min(tile, tiles - 1) * tile_bytes, tile < tiles ? tile_bytes : 0);
  const __amdgpu_buffer_rsrc_t rsrc_x = range_rsrc(x, (int64_t)B * 2 * m * 2);

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
  // staging unit e = tid + 512 k: row e / 32 (batch row / 2, component row & 1), columns 8 (e % 32)
  auto load_x = [&](int c, uint4 (&st)[kSeg]) {
#pragma unroll
    for (int k = 0; k < kSeg; ++k) {
      const int e = tid + kWave * kSxWaves * k, row = e >> 5, u = e & 31;
      const bool ok = kChunk * c + 8 * u < m;
      st[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
          rsrc_x, ok ? (uint32_t)((row * m + kChunk * c + 8 * u) * 2) : kNoLoad, 0, 0));
    }
  };
  auto store_x = [&](int buf, const uint4 (&st)[kSeg]) {
#pragma unroll
    for (int k = 0; k < kSeg; ++k) {
      const int e = tid + kWave * kSxWaves * k, row = e >> 5, u = e & 31;
      *reinterpret_cast<v4u*>(&s_x[buf][row * kSxPitch + 16 * u]) = permute_b(st[k]);
    }
  };
  auto load_w = [&](int c, uint4 (&w)[TT][2]) {
    const int groups = min(4, (m - kChunk * c) >> 6);
    const bool k_ok = g < groups;
    const uint32_t cbase = (uint32_t)c * (TT * 2) * 1024;
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int M = 0; M < 2; ++M)
        w[t][M] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
            rsrc_a, k_ok ? cbase + (uint32_t)((t * 2 + M) * groups * 256 + lane * 16) : kNoLoad, 0, kStreamLoad));
  };
  auto compute_chunk = [&](int buf, const uint4 (&wc)[TT][2]) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      v4u bv[CG];
#pragma unroll
      for (int cg = 0; cg < CG; ++cg)   // column r: batch 8 cg + r/2, component r & 1; columns 64g + 8s ..
        bv[cg] = *reinterpret_cast<const v4u*>(&s_x[buf][((cg * 8 + (r >> 1)) * 2 + comp) * kSxPitch + (64 * g + 8 * s) * 2]);
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int M = 0; M < 2; ++M) {
          const uint4 q = wc[t][M];
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
  };

  __shared__ float s_sc[kSxWaves][16 * TT * 4];
  float ypart[4][CG][2];                         // output partials of long rows
  bool flushed = false;
  TileScales<TT> tsc;
  tsc.load(scales, i0, n, lane);               // ahead of the first chunk's loads
  uint4 w0[TT][2], w1[TT][2];
  uint4 st[kSeg];
  load_w(0, w0);
  load_x(0, st);
  store_x(0, st);
  tsc.park(s_sc[wave], lane);
  __syncthreads();
  for (int c = 0; c < nchunk; ++c) {
    const int cn = c + 1;   // past the last chunk every load takes the out-of-range offset
    load_w(cn, w1);
    load_x(cn, st);
    __builtin_amdgcn_sched_barrier(0);
    compute_chunk(c & 1, w0);
    store_x((c & 1) ^ 1, st);                // its last readers passed the previous barrier
    if constexpr (LONG) {
      if ((c & (kFlushChunks - 1)) == kFlushChunks - 1 && c + 1 < nchunk)
        flush_partials<TT, CG>(acc, s_sc[wave], g, comp, ypart, flushed);
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TT; ++t) { w0[t][0] = w1[t][0]; w0[t][1] = w1[t][1]; }
  }
  if (tile >= tiles) return;

  const int64_t ys = 2 * (int64_t)n;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = i0 + 4 * g + e;
    const float* sc = &s_sc[wave][(4 * g + e) * TT * 4];
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      float vre, vim;
      combine_row<TT, CG>(acc, sc, e, cg, comp, vre, vim);
      if (LONG && flushed) {
        vre = ypart[e][cg][0] + vre;
        vim = ypart[e][cg][1] + vim;
      }
      vre = group_sum<2>(vre);
      vim = group_sum<2>(vim);
      const int b = cg * 8 + (r >> 1);
      if (comp == 0 && b < B && i < n) {
        store_out(y, (int64_t)b * ys + i, vre);
        store_out(y, (int64_t)b * ys + n + i, vim);
      }
    }
  }
}

template <int TT, int CG, typename YT, bool LONG>
static void launch_cg(const GemvGroup& group, int m, int B, hipStream_t s) {
  GemvGroup grp = group;
  const int tiles = group_tiles(grp);
  int nw = gemv_waves_per_tile(tiles, m);
  if (LONG && nw > 1) nw = 4;              // long rows have more than 4 chunks
  if (nw == 1 && B >= 3) {                 // large launch, batch 3-16: shared x
    int blocks = 0;
    if (grp.batch > 0) {
      grp.units_per_item = (grp.tiles_per_item + kSxWaves - 1) / kSxWaves;
      blocks = grp.batch * grp.units_per_item;
    } else {
      for (int k = 0; k < grp.count; ++k) {
        grp.tile_start[k] = blocks;
        blocks += ((grp.items[k].n + 15) / 16 + kSxWaves - 1) / kSxWaves;
      }
      grp.tile_start[grp.count] = blocks;
    }
    hipLaunchKernelGGL((k_gemv_mfma_sx<TT, CG, YT, LONG>), dim3(blocks), dim3(kSxWaves * kWave), 0, s, grp, m, B);
    return;
  }
  grp.units_per_item = grp.tiles_per_item;        // one workgroup per tile
  const dim3 grid(tiles);
  if constexpr (LONG) {
    if (nw == 4) hipLaunchKernelGGL((k_gemv_mfma<TT, CG, 4, YT, true>), grid, dim3(4 * kWave), 0, s, grp, m, B);
    else hipLaunchKernelGGL((k_gemv_mfma<TT, CG, 1, YT, true>), grid, dim3(kWave), 0, s, grp, m, B);
    return;
  }
  switch (nw) {
    case 8: hipLaunchKernelGGL((k_gemv_mfma<TT, CG, 8, YT, false>), grid, dim3(8 * kWave), 0, s, grp, m, B); break;
    case 4: hipLaunchKernelGGL((k_gemv_mfma<TT, CG, 4, YT, false>), grid, dim3(4 * kWave), 0, s, grp, m, B); break;
    case 2: hipLaunchKernelGGL((k_gemv_mfma<TT, CG, 2, YT, false>), grid, dim3(2 * kWave), 0, s, grp, m, B); break;
    default: hipLaunchKernelGGL((k_gemv_mfma<TT, CG, 1, YT, false>), grid, dim3(kWave), 0, s, grp, m, B); break;
  }
}

template <int TT, typename YT>
static void launch_t(const GemvGroup& grp, int m, int B, hipStream_t s) {
  const bool long_rows = (m + kChunk - 1) / kChunk > kFlushChunks;
  if (B <= 8) {
    if (long_rows) launch_cg<TT, 1, YT, true>(grp, m, B, s);
    else launch_cg<TT, 1, YT, false>(grp, m, B, s);
  } else {
    if (long_rows) launch_cg<TT, 2, YT, true>(grp, m, B, s);
    else launch_cg<TT, 2, YT, false>(grp, m, B, s);
  }
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
