// Decode GEMV for batch 1-2 on the fp4 x fp6 matrix cores: y = sum_t U~(t) x + W~(t) conj(x).
//
// Sources: ModelScope card "Fairy2i-W2", "Method" (y = U x + W conj(x)); zhichai.net reading
// note, "Step 2" dequantization and "Industry implications: multiplication-free inference"
// (B_re, B_im in {-1, 0, 1}; products reduce to additions, subtractions, skips); 36Kr article,
// parallel stages.
//
//  * Sum and difference planes.  With u = B_re + B_im and v = B_re - B_im every codeword gives
//    u, v in {+1, -1}: code 0 (+1) u = v = +1; code 1 (+i) u = +1, v = -1; code 2 (-1)
//    u = v = -1; code 3 (-i) u = -1, v = +1.  So u is negative exactly when the code's high bit
//    is set and v when its two bits differ, and B_re = (u + v) / 2, B_im = (u - v) / 2: the sums
//    over the u and v planes give both axis sums of a stage.
//  * fp4 (e2m1) planes straight from the packed words.  The planes are held as +-6, the fp4
//    value whose nibble is 0b s111 (sign s in bit 3, all other bits set), so setting the low three
//    bits of every nibble turns a sign bit into an operand.  Nibble j of a packed word holds two
//    codes, one in its bits 0-1 and one in bits 2-3 (high bits in 1 and 3): w | 0x77777777 is the
//    u plane of the eight codes in the upper halves, (w << 2) | 0x77777777 that of the lower
//    halves, and the same two forms on w ^ (w << 1) give the v plane -- six ALU operations per
//    16 codes (v_lshl_or_b32 and v_bitop3_b32 fuse the shifts and xors), no table lookups.  The
//    plane's k order (which column each nibble is) is fixed by this; the fp6 digit form of x is
//    stored in the same order.
//  * x in fp6 digit form: X = rne(x 2^S) exactly as for the int8 digit form (S with
//    max|x| 2^S in [2^21, 2^22)), written with eight balanced base-8 digits d_l in [-4, 3], all
//    exact in fp6 e2m3.  MFMA column c = 8 comp + l holds digit l of component comp (a = Re x,
//    b = Im x); each batch entry has its own MFMAs.
//  * v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales takes 128 columns per instruction at the
//    issue rate of the int8 16x16x64 form.  Every product is +-6d and every partial sum an
//    integer of magnitude at most 24m < 2^24 (m <= 2^19), so the fp32 accumulation is exact;
//    Su + Sv is even and below 2^25, so the halving is exact too.  The factor 6 leaves in the
//    epilogue's digit weight; the only roundings are X itself and the fp32 epilogue.
//  * Streaming as in the int8 kernel: one wave per 16-row tile of one item of a grouped or strided call
//    (or NW waves splitting the 256-column chunks for small launches), one 1 KB load per plane
//    and chunk, the next chunk prefetched while the current one is decoded and multiplied.  In
//    a chunk lane l = 16g + r holds row r, columns 64g..64g+63 (four words); MFMA step s < 2
//    takes words 2s and 2s+1.  Large batch-1 launches end on tiles split over four waves, whose
//    exact integer accumulators are added before the epilogue (k_gemv_f4_mixed): the outputs
//    are those of one wave per tile, bit for bit, and the launch's tail is short-lived waves.
#include "common.hpp"
#include "digits.hpp"

namespace f2i {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kF4Chunk = 256;
constexpr int kF6Record = 32;        // bytes per (chunk, step, batch entry, lane): 24 of digits + 8 zero

// Column (within its 256-column chunk) of element q < 32 of the fp4 plane of lane group g at MFMA
// step s: word 2s + q/16 of the lane's four words; in that word, the upper (h = 1) or lower
// (h = 0) code of nibble j.  Code p of a word sits in bits 8(p % 4) + 2(p / 4), so nibble j holds
// codes p = 4(2(j % 2)) + j/2 (lower) and p + 4 (upper).
__host__ __device__ __forceinline__ int f4_column(int g, int s, int q) {
  const int wd = 2 * s + (q >> 4), h = (q >> 3) & 1, j = q & 7;
  return 64 * g + 16 * wd + 4 * (2 * (j & 1) + h) + (j >> 1);
}

constexpr uint32_t kLow3 = 0x77777777u;     // the non-sign bits of every nibble: fp4 +-6

// u and v planes (fp4 +-6) of one packed word: [lower halves, upper halves] of its nibbles.
__device__ __forceinline__ void decode_f4_word(uint32_t w, uint32_t& u_lo, uint32_t& u_hi,
                                               uint32_t& v_lo, uint32_t& v_hi) {
  const uint32_t w1 = w << 1;
  u_hi = w | kLow3;
  u_lo = (w << 2) | kLow3;                                    // v_lshl_or_b32
  v_hi = __builtin_amdgcn_bitop3_b32(w, w1, kLow3, 0xBE);     // (w ^ w1) | kLow3
  v_lo = ((w ^ w1) << 2) | kLow3;
}

__device__ __forceinline__ void decode_f4(uint32_t w0, uint32_t w1, v8i& u, v8i& v) {
  uint32_t a0, a1, b0, b1, c0, c1, d0, d1;
  decode_f4_word(w0, a0, a1, c0, c1);
  decode_f4_word(w1, b0, b1, d0, d1);
  u = v8i{(int)a0, (int)a1, (int)b0, (int)b1, 0, 0, 0, 0};
  v = v8i{(int)c0, (int)c1, (int)d0, (int)d1, 0, 0, 0, 0};
}

// fp6 e2m3 bits of an integer d in [-4, 4]: magnitudes 0, 1, 2, 3, 4 -> 0x00, 0x08, 0x10, 0x14,
// 0x18; sign in bit 5.
__device__ __forceinline__ uint32_t fp6_int(int d) {
  const int a = d < 0 ? -d : d;
  const uint32_t mag = (uint32_t)(0x1814100800ull >> (8 * a)) & 0xFFu;
  return d < 0 ? (mag | 0x20u) : mag;
}

// ------------------------------------------------------------------ fp6 digit form of x ----
//
// int32 header [B, m, S_0, S_1] in the first 64 bytes, then records of 32 bytes ordered
// [chunk c][step s < 2][batch b][lane 16g + col]: the 32 fp6 values (6 bits each, element q at bits
// 6q..6q+5) of digit l = col % 8 of component col / 8 of x_b, for the columns f4_column(g, s, q) of
// chunk c; bytes 24..31 are zero, and so are the records of 64-column groups past m.

// One workgroup of 256 threads per (256-column chunk, batch entry): all of them read the whole
// column (2m values, from L2 after the first workgroup) for max |x| and S -- the same value in
// every workgroup, as the maximum is order-free.  Then four neighbouring threads share one work
// item, 8 columns (a quarter of a record's elements) of one component in one (half s, lane group
// g): each takes two of the columns and all eight of their digits, and the four 12-bit pieces
// of each digit's 48 bits are merged across the four lanes; each lane stores two digits' pieces.
constexpr int kF6Threads = 256;

template <typename XT>
__device__ __forceinline__ float x_value(const XT* p);
template <> __device__ __forceinline__ float x_value<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float x_value<uint16_t>(const uint16_t* p) {
  return __uint_as_float((uint32_t)*p << 16);
}

template <typename XT>
__global__ __launch_bounds__(kF6Threads) void k_x_digits_f6(const XT* __restrict__ x, int m, int B,
                                                            uint8_t* __restrict__ blob) {
  __shared__ float s_max[kF6Threads / kWave];
  const int c = blockIdx.x, b = blockIdx.y;
  const XT* __restrict__ xb = x + (int64_t)b * 2 * m;
  const int item = threadIdx.x >> 2, part = threadIdx.x & 3;    // part: columns 2 part, 2 part + 1
  const int quarter = item & 3, comp = (item >> 2) & 1, g = (item >> 3) & 3, s = (item >> 5) & 1;
  const bool present = kF4Chunk * c + 64 * g < m;
  float xv[2] = {0.f, 0.f};                  // this thread's two values, loaded before the max pass
  if (present) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
      xv[jj] = x_value(xb + (int64_t)comp * m + kF4Chunk * c + f4_column(g, s, 8 * quarter + 2 * part + jj));
  }
  float keep[8];
  const float amax = column_amax<XT, kF6Threads>(xb, 2 * m, keep, s_max);
  const int S = digit_exponent(amax);
  const float f1 = ldexpf(1.0f, S / 2), f2 = ldexpf(1.0f, S - S / 2);   // 2^S, exact in two steps
  int* hdr = reinterpret_cast<int*>(blob);
  if (c == 0 && threadIdx.x == 0) {
    if (b == 0) { hdr[0] = B; hdr[1] = m; }
    hdr[2 + b] = S;
  }
  uint32_t bits[8] = {0, 0, 0, 0, 0, 0, 0, 0};                   // 12 bits per digit
  if (present) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      int X = (int)rintf((xv[jj] * f1) * f2);                     // |X| <= 2^22
#pragma unroll
      for (int l = 0; l < 8; ++l) {
        const int d = ((X + 4) & 7) - 4;
        X = (X - d) >> 3;
        bits[l] |= fp6_int(d) << (6 * jj);
      }
    }
  }
  // digit l's 48 bits: piece of lane part at bits 12 part; lanes 4 item .. 4 item + 3 merge them
  uint64_t full[8];
#pragma unroll
  for (int l = 0; l < 8; ++l) {
    uint64_t v = (uint64_t)bits[l] << (12 * part);
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    lo |= __shfl_xor(lo, 1);
    hi |= __shfl_xor(hi, 1);
    lo |= __shfl_xor(lo, 2);
    hi |= __shfl_xor(hi, 2);
    full[l] = ((uint64_t)hi << 32) | lo;
  }
#pragma unroll
  for (int l = 0; l < 8; ++l) {
    if ((l >> 1) != part) continue;                              // this lane stores digits 2 part, 2 part + 1
    const int lane = 16 * g + 8 * comp + l;
    uint8_t* rec = blob + kDigitHeader + ((((int64_t)c * 2 + s) * B + b) * 64 + lane) * kF6Record;
    uint16_t* r16 = reinterpret_cast<uint16_t*>(rec + 6 * quarter);
    r16[0] = (uint16_t)full[l];
    r16[1] = (uint16_t)(full[l] >> 16);
    r16[2] = (uint16_t)(full[l] >> 32);
    if (quarter == 3) *reinterpret_cast<uint2*>(rec + 24) = make_uint2(0u, 0u);
  }
}

size_t x_digits_f6_bytes(int64_t m, int64_t B) {
  return (size_t)kDigitHeader + (size_t)((m + kF4Chunk - 1) / kF4Chunk) * 2 * (size_t)B * 64 * kF6Record;
}

hipError_t launch_x_digits_f6(const void* x, int x_bf16, int m, int B, void* blob, hipStream_t s) {
  const dim3 grid((m + kF4Chunk - 1) / kF4Chunk, B);
  if (x_bf16)
    hipLaunchKernelGGL(k_x_digits_f6<uint16_t>, grid, dim3(kF6Threads), 0, s,
                       static_cast<const uint16_t*>(x), m, B, static_cast<uint8_t*>(blob));
  else
    hipLaunchKernelGGL(k_x_digits_f6<float>, grid, dim3(kF6Threads), 0, s,
                       static_cast<const float*>(x), m, B, static_cast<uint8_t*>(blob));
  return hipGetLastError();
}

// ------------------------------------------------------------------------- GEMV ----

// One unit (a 16-row tile of one item) streamed by NW cooperating waves; `wave` is this wave's
// index among them, s_scw its own LDS slot for the tile's scales, s_y the NW waves' partial outputs.
// EXACT (NW = 4, one batch entry): the waves first add their accumulators through LDS (s_acc,
// 16 T x 64 floats per wave) -- exact, since every partial and total is an integer below 2^24 --
// and wave w then runs the single-wave epilogue for rows 4g + w, so the outputs are bit-identical
// to one wave streaming the whole unit.
template <int TT, int NW, int BT, typename YT, bool EXACT = false>
__device__ __forceinline__ void gemv_f4_tile(const GemvGroup& grp, int m, int B, int unit, int wave,
                                             float* __restrict__ s_scw, float (*s_y)[BT][2][16],
                                             float* __restrict__ s_acc = nullptr) {
  static_assert(!EXACT || (NW == 4 && BT == 1), "the exact split is for four waves and one batch entry");
  int tile;
  const GemvItem it = locate_item<YT>(grp, unit, tile);
  const int n = it.n;
  const uint8_t* __restrict__ packed = static_cast<const uint8_t*>(it.packed);
  const float* __restrict__ scales = it.scales;
  const uint8_t* __restrict__ blob = static_cast<const uint8_t*>(it.x);
  YT* __restrict__ y = static_cast<YT*>(it.y);

  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15, g = lane >> 4;
  const int i0 = tile * 16;
  const int nchunk = (m + kF4Chunk - 1) / kF4Chunk;
  const int64_t tile_bytes = (int64_t)16 * TT * 2 * (m / 4);
  const __amdgpu_buffer_rsrc_t rsrc_a = range_rsrc(packed + (int64_t)tile * tile_bytes, tile_bytes);
  const __amdgpu_buffer_rsrc_t rsrc_x =
      range_rsrc(blob + kDigitHeader, (int64_t)nchunk * 2 * B * 64 * kF6Record);

  v4f acc[TT][2][2][BT];                    // [stage][U/W][u/v plane][batch entry]
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int M = 0; M < 2; ++M)
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int b = 0; b < BT; ++b) acc[t][M][p][b] = v4f{0.f, 0.f, 0.f, 0.f};

  struct Chunk { uint4 w[TT][2]; v8i x[2][BT]; };     // codes; fp6 digit operands per step
  auto load_chunk = [&](int c, Chunk& ch) {
    const int groups = min(4, (m - kF4Chunk * c) >> 6);
    const bool k_ok = g < groups;
    const uint32_t cbase = (uint32_t)c * (TT * 2) * 1024;
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int M = 0; M < 2; ++M)
        ch.w[t][M] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
            rsrc_a, k_ok ? cbase + (uint32_t)((t * 2 + M) * groups * 256 + lane * 16) : kNoLoad, 0, kStreamLoad));
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const bool ok = k_ok && b < B;
        const uint32_t off = (uint32_t)((((c * 2 + s) * B + b) * 64 + lane) * kF6Record);
        const v4i lo = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
            rsrc_x, ok ? off : kNoLoad, 0, 0));
        const v2i hi = __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(
            rsrc_x, ok ? off + 16 : kNoLoad, 0, 0));
        ch.x[s][b] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, 0, 0};
      }
  };
  auto compute_chunk = [&](const Chunk& ch) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int M = 0; M < 2; ++M) {
          const uint4 q = ch.w[t][M];
          v8i pu, pv;
          decode_f4(s == 0 ? q.x : q.z, s == 0 ? q.y : q.w, pu, pv);
#pragma unroll
          for (int b = 0; b < BT; ++b) {
            acc[t][M][0][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                pu, ch.x[s][b], acc[t][M][0][b], 4, 2, 0, 127, 0, 127);   // A fp4, B fp6 e2m3, scales 2^0
            acc[t][M][1][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                pv, ch.x[s][b], acc[t][M][1][b], 4, 2, 0, 127, 0, 127);
          }
        }
    }
  };
  // Operand sets stream through registers: chunk c + (D - 1) NW is loaded before chunk c is
  // multiplied, with D = 3 sets for one batch entry and T <= 2 and D = 2 otherwise (where operands
  // and accumulators take more registers).  The scheduling barriers keep each prefetch ahead of
  // the compute it overlaps (the scheduler would otherwise sink the loads to their use).  Every
  // prefetch is issued, so every path has the same loads in flight; one past the last chunk has a
  // negative group count and so loads at the out-of-range offset, which reads nothing.
  TileScales<TT> tsc;
  tsc.load(scales, i0, n, lane);               // ahead of the first chunk's loads
  if constexpr (BT == 1 && TT <= 2) {
    Chunk c0, c1, c2;
    int c = wave;                                  // wave w takes chunks w, w + NW, ...
    load_chunk(c, c0);
    load_chunk(c + NW, c1);
    tsc.park(s_scw, lane);
    for (; c + 2 * NW < nchunk; c += 3 * NW) {
      load_chunk(c + 2 * NW, c2);
      __builtin_amdgcn_sched_barrier(0);
      compute_chunk(c0);
      load_chunk(c + 3 * NW, c0);
      __builtin_amdgcn_sched_barrier(0);
      compute_chunk(c1);
      load_chunk(c + 4 * NW, c1);
      __builtin_amdgcn_sched_barrier(0);
      compute_chunk(c2);
    }
    if (c < nchunk) compute_chunk(c0);
    if (c + NW < nchunk) compute_chunk(c1);
  } else {
    Chunk c0, c1;
    int c = wave;
    load_chunk(c, c0);
    tsc.park(s_scw, lane);
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

  // Epilogue.  Lane holds rows 4g..4g+3 of column r = 8 comp + l.  Axis sums (times 6)
  // P = (Su + Sv) / 2, Q = (Su - Sv) / 2 (exact), then the widely-linear combination with the
  // fp32 scales, the digit weight 2^(3l - S_b) / 6, and the sum over digits (xor 1, 2, 4) and
  // components (xor 8).
  if constexpr (EXACT) {
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int M = 0; M < 2; ++M)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s_acc[((wave * TT * 4 + (t * 2 + M) * 2 + p) * 4 + e) * kWave + lane] = acc[t][M][p][0][e];
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int M = 0; M < 2; ++M)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          float v = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) v += s_acc[((w * TT * 4 + (t * 2 + M) * 2 + p) * 4 + wave) * kWave + lane];
          acc[t][M][p][0][wave & 3] = v;    // this wave's rows: e = wave
        }
  }
  const int comp = r >> 3, l = r & 7;
  const int* hdr = reinterpret_cast<const int*>(blob);
  const int64_t ys = 2 * (int64_t)n;
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    const int S = b < B ? hdr[2 + b] : 0;
    const float wdig = ldexpf(1.0f / 6.0f, 3 * l - S);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (EXACT && e != wave) continue;
      const int i = i0 + 4 * g + e;
      const float* sc = &s_scw[(4 * g + e) * TT * 4];
      float vre = 0.f, vim = 0.f;
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const float sUr = sc[4 * t], sUi = sc[4 * t + 1], sWr = sc[4 * t + 2], sWi = sc[4 * t + 3];
        const float PU = (acc[t][0][0][b][e] + acc[t][0][1][b][e]) * 0.5f;
        const float QU = (acc[t][0][0][b][e] - acc[t][0][1][b][e]) * 0.5f;
        const float PW = (acc[t][1][0][b][e] + acc[t][1][1][b][e]) * 0.5f;
        const float QW = (acc[t][1][0][b][e] - acc[t][1][1][b][e]) * 0.5f;
        if (comp == 0) {    // a = Re x
          vre += sUr * PU + sWr * PW;
          vim += sUi * QU + sWi * QW;
        } else {            // b = Im x
          vre += sWi * QW - sUi * QU;
          vim += sUr * PU - sWr * PW;
        }
      }
      vre *= wdig;
      vim *= wdig;
#pragma unroll
      for (int off = 1; off <= 8; off <<= 1) {
        vre += __shfl_xor(vre, off);
        vim += __shfl_xor(vim, off);
      }
      if (NW > 1 && !EXACT) {
        if (r == 0) { s_y[wave][b][0][4 * g + e] = vre; s_y[wave][b][1][4 * g + e] = vim; }
      } else if (r == 0 && b < B && i < n) {
        store_out(y, (int64_t)b * ys + i, vre);
        store_out(y, (int64_t)b * ys + n + i, vim);
      }
    }
  }
  if constexpr (NW > 1 && !EXACT) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < BT * 2 * 16; idx += kWave * NW) {
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

template <int TT, int NW, int BT, typename YT>
__global__ __launch_bounds__(kWave * NW, (BT == 1 && TT <= 3) ? 3 : 1) void k_gemv_f4(const GemvGroup grp, int m, int B) {
  __shared__ float s_sc[NW][16 * TT * 4];
  __shared__ float s_y[NW > 1 ? NW : 1][BT][2][16];     // [wave][batch][re/im][row]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
  gemv_f4_tile<TT, NW, BT, YT>(grp, m, B, blockIdx.x, wave, s_sc[wave], s_y);
}

// Large batch-1 launches in two granularities.  The first nA workgroups take four units each,
// one wave per unit (the fastest form while the chip is full); the rest take one unit each, its
// chunks split over the four waves.  Workgroups start in index order, so the units that finish a
// launch are the short-lived ones: the launch's tail, where fewer and fewer waves remain in
// flight, lasts about a quarter as long.  Both forms give the single-wave kernel's outputs bit for
// bit (the split one adds its waves' exact integer accumulators before the epilogue).
template <int TT, typename YT>
__global__ __launch_bounds__(kWave * 4, 3) void k_gemv_f4_mixed(const GemvGroup grp, int m, int nA) {
  __shared__ float s_sc[4][16 * TT * 4];
  __shared__ float s_y[4][1][2][16];
  __shared__ float s_acc[4 * 16 * TT * kWave];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
  if ((int)blockIdx.x < nA)
    gemv_f4_tile<TT, 1, 1, YT>(grp, m, 1, 4 * (int)blockIdx.x + wave, 0, s_sc[wave], s_y);
  else
    gemv_f4_tile<TT, 4, 1, YT, true>(grp, m, 1, 4 * nA + ((int)blockIdx.x - nA), wave, s_sc[wave], s_y, s_acc);
}

// Mixed-granularity launches: units left to the one-unit-per-workgroup form at the end, and the
// smallest launch that uses them (measured on the 1 GiB pool, 32768 tiles: tails of 256-2048 tiles
// within 1 % of each other and ~2 % faster than 3072-6144; launches of 6144 tiles ran slower in
// this form, 16512 unchanged).
constexpr int kF4TailTiles = 1536;
constexpr int kF4MixedMinTiles = 12288;

template <int TT, int BT, typename YT>
static void launch_f4_t(const GemvGroup& group, int m, int B, hipStream_t s) {
  GemvGroup grp = group;
  grp.units_per_item = grp.tiles_per_item;        // one workgroup per tile
  const int tiles = group_tiles(grp);
  if constexpr (BT == 1 && TT <= 3) {
    if (gemv_waves_per_tile(tiles, m) == 1 && tiles >= kF4MixedMinTiles) {
      const int nA = (tiles - kF4TailTiles) / 4;          // four units per workgroup
      hipLaunchKernelGGL((k_gemv_f4_mixed<TT, YT>), dim3(nA + (tiles - 4 * nA)), dim3(4 * kWave), 0, s, grp, m, nA);
      return;
    }
  }
  const dim3 grid(tiles);
  switch (gemv_waves_per_tile(tiles, m)) {
    case 8: hipLaunchKernelGGL((k_gemv_f4<TT, 8, BT, YT>), grid, dim3(8 * kWave), 0, s, grp, m, B); break;
    case 4: hipLaunchKernelGGL((k_gemv_f4<TT, 4, BT, YT>), grid, dim3(4 * kWave), 0, s, grp, m, B); break;
    case 2: hipLaunchKernelGGL((k_gemv_f4<TT, 2, BT, YT>), grid, dim3(2 * kWave), 0, s, grp, m, B); break;
    default: hipLaunchKernelGGL((k_gemv_f4<TT, 1, BT, YT>), grid, dim3(kWave), 0, s, grp, m, B); break;
  }
}

template <int TT, typename YT>
static void launch_f4_b(const GemvGroup& grp, int m, int B, hipStream_t s) {
  if (B == 1) launch_f4_t<TT, 1, YT>(grp, m, B, s);
  else launch_f4_t<TT, 2, YT>(grp, m, B, s);
}

template <typename YT>
static void launch_f4_y(const GemvGroup& grp, int m, int T, int B, hipStream_t s) {
  switch (T) {
    case 1: launch_f4_b<1, YT>(grp, m, B, s); break;
    case 2: launch_f4_b<2, YT>(grp, m, B, s); break;
    case 3: launch_f4_b<3, YT>(grp, m, B, s); break;
    default: launch_f4_b<4, YT>(grp, m, B, s); break;
  }
}

hipError_t launch_gemv_f4_group(const GemvGroup& grp, int m, int T, int B, int y_bf16, hipStream_t s) {
  if (y_bf16) launch_f4_y<uint16_t>(grp, m, T, B, s);
  else launch_f4_y<float>(grp, m, T, B, s);
  return hipGetLastError();
}

hipError_t launch_gemv_f4(const uint8_t* packed, const float* scales, int n, int m, int T,
                          const void* digits, int B, void* y, int y_bf16, hipStream_t s) {
  GemvGroup grp;
  grp.count = 1;
  grp.tile_start[0] = 0;
  grp.tile_start[1] = (n + 15) / 16;
  grp.items[0] = GemvItem{packed, scales, digits, y, n};
  return launch_gemv_f4_group(grp, m, T, B, y_bf16, s);
}

}  // namespace f2i
