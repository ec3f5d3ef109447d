// Decode GEMV for batch 3-16 on the scaled matrix cores: fp4 code planes times bf16 x split into
// two fp8 parts.  y = sum_t U~(t) x + W~(t) conj(x).
//
// Sources: ModelScope card "Fairy2i-W2", "Method" (y = U x + W conj(x)); zhichai.net reading
// note, "Step 2" dequantization and "Industry implications: multiplication-free inference"
// (B_re, B_im in {-1, 0, 1}; products reduce to additions, subtractions, skips); 36Kr article,
// parallel stages.
//
//  * A operand: the u = B_re + B_im and v = B_re - B_im planes as fp4 +-6 straight from the packed
//    words (f4planes.hpp), six ALU operations per 16 codes -- a quarter of the bf16 kernel's
//    decode work, which is what limits that kernel at these batch sizes.
//  * B operand: x in fp8 e4m3 with one E8M0 scale per 32-column block (the columns one fp4 A lane
//    holds at one MFMA step).  For each (batch entry, component, block) with max |x| = M, E = floor(log2 M) - 7 (clamped to [-127, 127]),
//    xs = x 2^-E (exact) has |xs| < 256; hi = rne_e4m3(xs) and lo = rne_e4m3(xs - hi).  A bf16 x
//    has 8 significant bits, so xs - hi is exact in fp32 and has at most 4; lo is exact whenever
//    |x| >= 2^-10 M, and otherwise off by at most half of e4m3's smallest subnormal, 2^-10 2^E
//    <= 2^-17 M.  hi and lo are separate MFMA columns under the same block scale, so every
//    product is +-6 hi 2^E or +-6 lo 2^E, exact in fp32; the sums round in fp32.
//  * v_mfma_scale_f32_16x16x128_f8f6f4, A fp4 (scale 2^0), B fp8 with the scale of K block kb of
//    column n in lane 16 kb + n.  Columns n = 4b' + 2comp + part
//    (b' = batch entry within the column group, comp a = Re x / b = Im x, part hi / lo): four
//    batch entries per 16-column group, CG groups for B <= 4 CG.  Per chunk of 256 columns: 2 K
//    steps x 2T matrices x 2 planes x CG MFMAs of 128 columns, the fp8 rate's cycles, which is as
//    many as the bf16 kernel's at B = 8 and 16 and half at B = 4.
//  * A workgroup takes 8 consecutive tiles of one item (one wave each, the codes of the next chunk
//    in flight while the current one is multiplied) and stages each chunk's x once, already split
//    and in B-operand order, in one of two LDS buffers; the 512 threads split the chunk's
//    (batch, component, block) quarters between them (four neighbouring lanes share a block and
//    take its maximum on DPP).
#include "common.hpp"
#include "f4planes.hpp"

namespace f2i {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kF8Chunk = 256;
// Tiles (waves) per workgroup: eight, or four where the accumulators and operands of a wave need
// more than the 256 registers a wave has at two waves per SIMD (T * column groups >= 8).
template <int TT, int CG>
constexpr int f8_waves() { return TT * CG >= 8 ? 4 : 8; }
constexpr int kF8Rec = 32;                   // bytes of one lane's B operand (32 fp8 values)

// With fp8 B operands (eight registers, read over several passes) the instruction must not write
// its result into registers of its operands: measured on this part, a destination that reused a dying B
// operand's first four registers corrupted the products of K >= 32.  The compiler gives a dying
// operand's registers to the destination, so every A and B operand is kept live past the MFMAs
// that read it by empty uses that also read each such MFMA's result (so none can move below them).
template <typename V>
__device__ __forceinline__ void keep_live_after(const V& v, const v4f& after) {
#if __HIP_DEVICE_COMPILE__                           // the constraints name GPU registers
  asm volatile("" ::"v"(v), "v"(after));
#endif
}

template <int CG, int NWV>
struct F8Stage {
  // LDS of one chunk: records [step s][column group][half][lane] of 16 bytes (a lane's 32 bytes as
  // two planes, so the lanes of a 16-byte read are consecutive: conflict-free), then the
  // block-scale bytes [s][column group][lane].
  static constexpr int kRecBytes = 2 * CG * kWave * kF8Rec;
  static constexpr int kBytes = kRecBytes + 2 * CG * kWave;
  // Work items per chunk: (batch entry, component, block, quarter), 4 CG * 2 * 8 * 4 of them.
  static constexpr int kItems = 4 * CG * 2 * 8 * 4;
  static constexpr int kPerThread = (kItems + kWave * NWV - 1) / (kWave * NWV);
};

// One workgroup: tiles W unit .. W unit + W - 1 of one item (W = f8_waves).  x is bf16 [B][2m].
template <int TT, int CG, typename YT>
__global__ __launch_bounds__((kWave * f8_waves<TT, CG>())) void k_gemv_f8x(const GemvGroup grp, int m, int B) {
  constexpr int kF8Waves = f8_waves<TT, CG>();
  using St = F8Stage<CG, kF8Waves>;
  __shared__ __align__(16) uint8_t s_x[2][St::kBytes];
  __shared__ float s_sc[kF8Waves][16 * TT * 4];
  int unit;
  const GemvItem it = locate_item<YT>(grp, blockIdx.x, unit);
  const int n = it.n;
  const uint8_t* __restrict__ packed = static_cast<const uint8_t*>(it.packed);
  const float* __restrict__ scales = it.scales;
  YT* __restrict__ y = static_cast<YT*>(it.y);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform
  const int r = lane & 15, g = lane >> 4;
  const int tiles = (n + 15) / 16;
  const int tile = kF8Waves * unit + wave;
  const int i0 = tile * 16;
  const int64_t tile_bytes = (int64_t)16 * TT * 2 * (m / 4);
  const __amdgpu_buffer_rsrc_t rsrc_a =
      range_rsrc(packed + (int64_t)min(tile, tiles - 1) * tile_bytes, tile < tiles ? tile_bytes : 0);
  const __amdgpu_buffer_rsrc_t rsrc_x = range_rsrc(it.x, (int64_t)B * 2 * m * 2);
  const int nchunk = (m + kF8Chunk - 1) / kF8Chunk;

  v4f acc[TT][2][2][CG];                        // [stage][U/W][u/v plane][column group]
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int M = 0; M < 2; ++M)
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int cg = 0; cg < CG; ++cg) acc[t][M][p][cg] = v4f{0.f, 0.f, 0.f, 0.f};

  // Staging.  Item e: quarter k = e & 3 (elements 8k .. 8k + 7) of the A-side block blk = e >> 2:
  // step s = blk & 1, A lane group g = (blk >> 1) & 3, component comp = (blk >> 3) & 1, batch entry
  // b = blk >> 4 -- the 32 columns 64g + 32s + (0..31) that lane group g's fp4 A operand holds
  // (K = 32g + (0..31)); quarter k is columns 64g + 32s + 16(k >> 1) + 4(k & 1) + {0..3} and the same
  // + 8, interleaved in the element order f4_column gives A, loaded as two 8-byte pieces.  The block
  // scale of K block g of column n sits in lane 16g + n.  With fp8 B a lane of group G holds K =
  // 16G + (0..15) in elements 0-15 and 64 + 16G + (0..15) in 16-31 (both measured on this part),
  // so A element q of group g is element 16(g >> 1) + (q & 15) of B lane group 2(g & 1) + (q >> 4).
  struct XPiece { uint2 p[St::kPerThread][2]; };
  auto load_x = [&](int c, XPiece& xp) {
#pragma unroll
    for (int k2 = 0; k2 < St::kPerThread; ++k2) {
      const int e = tid + kWave * kF8Waves * k2;
      const int k = e & 3, blk = e >> 2;
      const int s = blk & 1, g = (blk >> 1) & 3, comp = (blk >> 3) & 1, b = blk >> 4;
      const int col = kF8Chunk * c + 64 * g + 32 * s + 16 * (k >> 1) + 4 * (k & 1);
      const bool ok = e < St::kItems && b < B && kF8Chunk * c + 64 * g < m;
      const uint32_t off = (uint32_t)(((b * 2 + comp) * m + col) * 2);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        xp.p[k2][h] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
            rsrc_x, ok ? off + 16 * h : kNoLoad, 0, 0));
    }
  };
  auto store_x = [&](int buf, const XPiece& xp) {
    uint8_t* rec = s_x[buf];
    uint8_t* scb = s_x[buf] + St::kRecBytes;
#pragma unroll
    for (int k2 = 0; k2 < St::kPerThread; ++k2) {
      const int e = tid + kWave * kF8Waves * k2;
      const int k = e & 3, blk = e >> 2;
      const int s = blk & 1, g = (blk >> 1) & 3, comp = (blk >> 3) & 1, b = blk >> 4;
      // element 2j of the quarter is value j of the first piece, element 2j + 1 value j of the second
      float v[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w0 = j < 2 ? xp.p[k2][0].x : xp.p[k2][0].y, w1 = j < 2 ? xp.p[k2][1].x : xp.p[k2][1].y;
        v[2 * j] = (j & 1) ? bf16_hi(w0) : bf16_lo(w0);
        v[2 * j + 1] = (j & 1) ? bf16_hi(w1) : bf16_lo(w1);
      }
      float mx = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(v[j]));
      mx = fmaxf(mx, dpp_read<0xB1>(mx));                 // the block's four quarters: lane ^ 1
      mx = fmaxf(mx, dpp_read<0x4E>(mx));                 // lane ^ 2
      // E = floor(log2 M) - 7, so that |x| 2^-E < 256 (e4m3 holds up to 448); 0 for an empty block
      const int eM = (int)((__float_as_uint(mx) >> 23) & 0xFF);   // biased exponent (0: zero or subnormal)
      int E = mx > 0.f ? (eM == 0 ? -126 : eM - 127) - 7 : 0;   // in [-133, 120]
      E = E < -127 ? -127 : E;                          // the smallest E8M0 scale, 2^-127
      const float f = __uint_as_float((uint32_t)(127 - E) << 23);   // 2^-E, a normal float
      uint32_t hi[2] = {0u, 0u}, lo[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float a0 = v[j] * f, a1 = v[j + 1] * f;    // exact: a power of two, no overflow
        const int h8 = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
        const float r0 = a0 - __builtin_amdgcn_cvt_f32_fp8(h8, 0);
        const float r1 = a1 - __builtin_amdgcn_cvt_f32_fp8(h8, 1);
        const int l8 = __builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false);
        hi[j >> 2] |= ((uint32_t)h8 & 0xFFFFu) << (16 * ((j >> 1) & 1));
        lo[j >> 2] |= ((uint32_t)l8 & 0xFFFFu) << (16 * ((j >> 1) & 1));
      }
      if (e < St::kItems) {
        const int cg = b >> 2, nh = 4 * (b & 3) + 2 * comp;      // column of hi; lo is nh + 1
        const int l_rec = 16 * (2 * (g & 1) + (k >> 1)) + nh;     // B lane holding this quarter
        const int at = 16 * (g >> 1) + 8 * (k & 1);               // its byte offset in that record
        uint8_t* base = rec + ((s * CG + cg) * kWave) * kF8Rec + (at >> 4) * (kWave * 16) + (at & 15);
        *reinterpret_cast<uint2*>(base + l_rec * 16) = make_uint2(hi[0], hi[1]);
        *reinterpret_cast<uint2*>(base + (l_rec + 1) * 16) = make_uint2(lo[0], lo[1]);
        if (k == 0) {
          const uint32_t sb = (uint32_t)(127 + E);
          *reinterpret_cast<uint16_t*>(scb + (s * CG + cg) * kWave + 16 * g + nh) = (uint16_t)(sb | (sb << 8));
        }
      }
    }
  };
  auto load_w = [&](int c, uint4 (&w)[TT][2]) {
    const int groups = min(4, (m - kF8Chunk * c) >> 6);
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
    const uint8_t* rec = s_x[buf];
    const uint8_t* scb = s_x[buf] + St::kRecBytes;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v8i xb[CG];
      int sb[CG];
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
        const uint8_t* p = rec + ((s * CG + cg) * kWave) * kF8Rec + lane * 16;
        const uint4 lo = *reinterpret_cast<const uint4*>(p);
        const uint4 hi = *reinterpret_cast<const uint4*>(p + kWave * 16);
        xb[cg] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sb[cg] = scb[(s * CG + cg) * kWave + lane];
      }
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int M = 0; M < 2; ++M) {
          const uint4 q = wc[t][M];
          v8i pu, pv;
          decode_f4(s == 0 ? q.x : q.z, s == 0 ? q.y : q.w, pu, pv);
#pragma unroll
          for (int cg = 0; cg < CG; ++cg) {
            // A fp4 (scale 2^0), B fp8 e4m3 with the lane's block scale
            acc[t][M][0][cg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                pu, xb[cg], acc[t][M][0][cg], 4, 0, 0, 127, 0, sb[cg]);
            acc[t][M][1][cg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                pv, xb[cg], acc[t][M][1][cg], 4, 0, 0, 127, 0, sb[cg]);
          }
#pragma unroll
          for (int cg = 0; cg < CG; ++cg) {
            keep_live_after(pu, acc[t][M][0][cg]);
            keep_live_after(pv, acc[t][M][1][cg]);
          }
        }
#pragma unroll
      for (int cg = 0; cg < CG; ++cg)
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int M = 0; M < 2; ++M)
#pragma unroll
            for (int p = 0; p < 2; ++p) keep_live_after(xb[cg], acc[t][M][p][cg]);
    }
  };

  TileScales<TT> tsc;
  tsc.load(scales, i0, n, lane);               // ahead of the first chunk's loads
  // Codes stream one chunk ahead of the multiply (two ahead measured slower: 4096 x 4096 pool at
  // B = 4, 247 -> 260 us).
  uint4 w0[TT][2], w1[TT][2];
  XPiece xp;
  load_w(0, w0);
  load_x(0, xp);
  store_x(0, xp);
  tsc.park(s_sc[wave], lane);
  __syncthreads();
  for (int c = 0; c < nchunk; ++c) {
    const int cn = c + 1;   // past the last chunk every load takes the out-of-range offset
    load_w(cn, w1);
    load_x(cn, xp);
    __builtin_amdgcn_sched_barrier(0);
    compute_chunk(c & 1, w0);
    store_x((c & 1) ^ 1, xp);                // its last readers passed the previous barrier
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TT; ++t) { w0[t][0] = w1[t][0]; w0[t][1] = w1[t][1]; }
  }
  if (tile >= tiles) return;

  // Epilogue.  Lane holds rows 4g .. 4g + 3 of column r = 4b' + 2comp + part.  Axis sums (times 6)
  // P = (Su + Sv) / 2, Q = (Su - Sv) / 2, the widely-linear combination with the fp32 scales, the
  // factor 1/6, and the sum over a batch entry's four columns (components, hi and lo parts).
  const int comp = (r >> 1) & 1;
  const int64_t ys = 2 * (int64_t)n;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = i0 + 4 * g + e;
    const float* sc = &s_sc[wave][(4 * g + e) * TT * 4];
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      float vre = 0.f, vim = 0.f;
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const float sUr = sc[4 * t], sUi = sc[4 * t + 1], sWr = sc[4 * t + 2], sWi = sc[4 * t + 3];
        const float PU = (acc[t][0][0][cg][e] + acc[t][0][1][cg][e]) * 0.5f;
        const float QU = (acc[t][0][0][cg][e] - acc[t][0][1][cg][e]) * 0.5f;
        const float PW = (acc[t][1][0][cg][e] + acc[t][1][1][cg][e]) * 0.5f;
        const float QW = (acc[t][1][0][cg][e] - acc[t][1][1][cg][e]) * 0.5f;
        if (comp == 0) {    // a = Re x
          vre += sUr * PU + sWr * PW;
          vim += sUi * QU + sWi * QW;
        } else {            // b = Im x
          vre += sWi * QW - sUi * QU;
          vim += sUr * PU - sWr * PW;
        }
      }
      vre *= 1.0f / 6.0f;
      vim *= 1.0f / 6.0f;
      vre = group_sum<4>(vre);
      vim = group_sum<4>(vim);
      const int b = 4 * cg + (r >> 2);
      if ((r & 3) == 0 && b < B && i < n) {
        store_out(y, (int64_t)b * ys + i, vre);
        store_out(y, (int64_t)b * ys + n + i, vim);
      }
    }
  }
}

template <int TT, int CG, typename YT>
static void launch_f8x_cg(const GemvGroup& group, int m, int B, hipStream_t s) {
  constexpr int kF8Waves = f8_waves<TT, CG>();
  GemvGroup grp = group;
  int blocks = 0;
  if (grp.batch > 0) {
    grp.units_per_item = (grp.tiles_per_item + kF8Waves - 1) / kF8Waves;
    blocks = grp.batch * grp.units_per_item;
  } else {
    for (int k = 0; k < grp.count; ++k) {
      grp.tile_start[k] = blocks;
      blocks += ((grp.items[k].n + 15) / 16 + kF8Waves - 1) / kF8Waves;
    }
    grp.tile_start[grp.count] = blocks;
  }
  hipLaunchKernelGGL((k_gemv_f8x<TT, CG, YT>), dim3(blocks), dim3(kF8Waves * kWave), 0, s, grp, m, B);
}

template <int TT, typename YT>
static void launch_f8x_t(const GemvGroup& grp, int m, int B, hipStream_t s) {
  if (B <= 4) launch_f8x_cg<TT, 1, YT>(grp, m, B, s);
  else if (B <= 8) launch_f8x_cg<TT, 2, YT>(grp, m, B, s);
  else launch_f8x_cg<TT, 4, YT>(grp, m, B, s);
}

template <typename YT>
static void launch_f8x_y(const GemvGroup& grp, int m, int T, int B, hipStream_t s) {
  switch (T) {
    case 1: launch_f8x_t<1, YT>(grp, m, B, s); break;
    case 2: launch_f8x_t<2, YT>(grp, m, B, s); break;
    case 3: launch_f8x_t<3, YT>(grp, m, B, s); break;
    default: launch_f8x_t<4, YT>(grp, m, B, s); break;
  }
}

hipError_t launch_gemv_f8x_group(const GemvGroup& grp, int m, int T, int B, int y_bf16, hipStream_t s) {
  if (y_bf16) launch_f8x_y<uint16_t>(grp, m, T, B, s);
  else launch_f8x_y<float>(grp, m, T, B, s);
  return hipGetLastError();
}

}  // namespace f2i
