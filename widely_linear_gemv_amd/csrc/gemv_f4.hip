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
//  * bf16 x without a digit-form buffer: each workgroup builds the records it multiplies in LDS
//    (build_f4_records: same S, X and digits as k_x_digits_f6, held as fp4, which represents
//    every digit exactly, so the outputs equal the two-call form bit for bit).  Large launches keep their workgroups resident (k_gemv_f4_persist), so a
//    workgroup builds once and then streams many tiles; small launches build once per tile.
//  * Streaming as in the int8 kernel: one wave per 16-row tile of one item of a grouped or strided call
//    (or NW waves splitting the 256-column chunks for small launches), one 1 KB load per plane
//    and chunk, the next chunk prefetched while the current one is decoded and multiplied.  In
//    a chunk lane l = 16g + r holds row r, columns 64g..64g+63 (four words); MFMA step s < 2
//    takes words 2s and 2s+1.  Large batch-1 launches end on tiles split over four waves, whose
//    exact integer accumulators are added before the epilogue (k_gemv_f4_mixed): the outputs
//    are those of one wave per tile, bit for bit, and the launch's tail is short-lived waves.
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "digits.hpp"
#include "f4planes.hpp"

namespace f2i {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kF4Chunk = 256;
constexpr int kF6Record = 32;        // bytes per (chunk, step, batch entry, lane): 24 of digits + 8 zero

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

// ------------------------------------------- fp4 digit records built on chip (bf16 x) ----
//
// The fp4 GEMV on bf16 x without a digit-form buffer: each workgroup makes the records its waves
// multiply -- the same X = rne(x 2^S), with the same S and digits as k_x_digits_f6 -- in LDS, once,
// and its waves read their B operands from there.  The digits d in [-4, 3] are exact in fp4 e2m1
// too (0, +-1, +-2, +-3, -4), so these records hold them as fp4: 16 bytes (the 32 values, element
// q in bits 4q..4q+3), ordered [chunk][step][b][lane] as in the digit form, and the MFMAs that
// read them take B as fp4.  Every product +-6d and every sum are the integers of the fp6 form, so
// the outputs equal the two-call form's bit for bit.  The digits come from Y = X + kDigitBias,
// whose plain base-8 digits are the balanced digits plus 4 (X is within +-2^22, so
// 0 <= Y < 8^8); a v_perm_b32 maps four such digits at once to their fp4 codes (one per byte),
// and two such words interleave into a word of eight nibbles.
constexpr int kRecBytes = 16;
constexpr int kDigitBias = 9586980;                 // 4 (8^8 - 1) / 7
constexpr uint32_t kF4CodesLo = 0x0A0C0D0Eu;       // fp4 e2m1 of the digits -4, -3, -2, -1
constexpr uint32_t kF4CodesHi = 0x05040200u;       // and of 0, 1, 2, 3

// LDS bytes of the records of a row of m columns and B batch entries.
__host__ __device__ inline int f4_record_bytes(int m, int B) {
  return ((m + kF4Chunk - 1) / kF4Chunk) * 2 * B * kWave * kRecBytes;
}

// LDS bytes of the per-chunk, per-batch-entry exponents of the per-wave records (16-byte aligned).
__host__ __device__ inline int f4_local_exp_bytes(int m, int B) { return (((m + kF4Chunk - 1) / kF4Chunk) * B * 4 + 15) & ~15; }

// LDS bytes of the staged bf16 x of B batch entries (2m values each).
__host__ __device__ inline int f4_xstage_bytes(int m, int B) { return 4 * m * B; }

// Maximum over the 64 lanes of a wave (exact, so the order is free): DPP within each row of 16
// lanes, then the four rows' results.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_read<0xB1>(v));                 // lane ^ 1
  v = fmaxf(v, dpp_read<0x4E>(v));                 // lane ^ 2
  v = fmaxf(v, dpp_read<0x141>(v));                // row_half_mirror
  v = fmaxf(v, dpp_read<0x140>(v));                // row_mirror: every lane holds its row's maximum
  const int iv = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// The four 3-bit digits of a 12-bit value, one per byte (digit i in the low bits of byte i).
__device__ __forceinline__ uint32_t spread_digits(uint32_t v) {
  v = (v | (v << 10)) & 0x003F003Fu;                // digits 0-1 in bits 0-5, digits 2-3 in bits 16-21
  return (v | (v << 5)) & 0x07070707u;              // each digit at the bottom of its own byte
}

// 4 x 4 byte transpose: byte t of out[i] is byte i of in[t].
__device__ __forceinline__ void transpose_bytes(const uint32_t in[4], uint32_t out[4]) {
  const uint32_t u0 = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);   // in0.0 in1.0 in0.1 in1.1
  const uint32_t u1 = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);   // in0.2 in1.2 in0.3 in1.3
  const uint32_t u2 = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
  const uint32_t u3 = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(u2, u0, 0x05040100u);                     // u0.0 u0.1 u2.0 u2.1
  out[1] = __builtin_amdgcn_perm(u2, u0, 0x07060302u);                     // u0.2 u0.3 u2.2 u2.3
  out[2] = __builtin_amdgcn_perm(u3, u1, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(u3, u1, 0x07060302u);
}

// Half of the eight digit records of one (chunk, step, batch entry, lane group, component): its
// 16 columns' bf16 values u (in column order, elements 16h .. 16h + 15 of the records) at exponent
// S; writes 8 bytes of digit l's record at dst0 + l kRecBytes for every l.  Each column's Y is
// formed once, then its digits 0-3 and 4-7 as fp4 codes, one per byte.  X = rne(x 2^S): x f1 f2 is
// exact and below 2^22 in magnitude, so adding 1.5 2^23 in the same fma rounds it to the integer in
// the sum's low bits (ties to even, as rintf).
__device__ __forceinline__ void build_record_half(const uint4 u[2], int S, uint8_t* dst0) {
  const float f1 = ldexpf(1.0f, S / 2), f2 = ldexpf(1.0f, S - S / 2);   // 2^S, exact in two steps
  uint32_t cl[16], ch[16];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t wd[4] = {u[k].x, u[k].y, u[k].z, u[k].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xv = (e & 1) ? bf16_hi(wd[e >> 1]) : bf16_lo(wd[e >> 1]);
      const uint32_t y = __float_as_uint(__builtin_fmaf(xv * f1, f2, 12582912.0f)) -
                         (0x4B400000u - (uint32_t)kDigitBias);
      cl[8 * k + e] = __builtin_amdgcn_perm(kF4CodesHi, kF4CodesLo, spread_digits(y & 0xFFFu));
      ch[8 * k + e] = __builtin_amdgcn_perm(kF4CodesHi, kF4CodesLo, spread_digits(y >> 12));
    }
  }
  // Dword j of digit l's half: nibble k is element 8j + k, so byte t pairs elements 8j + 2t and
  // 8j + 2t + 1; the pairs of all four digits of a word, transposed, give four digits' dwords at once.
  uint32_t dw[2][8];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint32_t pl[4], ph[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c0 = f4_column(0, 0, 8 * j + 2 * t), c1 = f4_column(0, 0, 8 * j + 2 * t + 1);
      pl[t] = cl[c0] | (cl[c1] << 4);
      ph[t] = ch[c0] | (ch[c1] << 4);
    }
    transpose_bytes(pl, &dw[j][0]);
    transpose_bytes(ph, &dw[j][4]);
  }
#pragma unroll
  for (int l = 0; l < 8; ++l) *reinterpret_cast<uint2*>(dst0 + l * kRecBytes) = make_uint2(dw[0][l], dw[1][l]);
}

// Workgroup-collective: reads x (bf16 [B][2m]), takes S_b of every batch entry (each thread
// computes it; s_S[b] keeps a copy for the epilogue), then builds every record into s_rec.
// kStage: x is copied into s_x on the first pass and the records are built from that copy;
// otherwise they read x again from global memory (from L2: every workgroup of the launch reads the
// same x), which leaves the workgroup only the records' LDS.  s_red holds one float per wave and
// batch entry.  In two parts: load_x() issues the loads of the first (usually the only) batch of x
// into registers, build() does the rest and ends with a barrier.  Every wave of the workgroup calls
// both, once each, in that order; a wave may issue its first code loads between them, and since a
// wave's loads complete in issue order, build()'s wait for x then does not wait for those code
// loads, which stream while the records are built.
template <bool kStage>
struct F4RecordBuild {
  static constexpr bool kLocal = false;               // one exponent S_b per batch entry
  static constexpr int kBatch = 8;                    // 16-byte units of x in flight per thread
  const uint16_t* x;
  int m, B;
  uint8_t* s_rec;
  uint16_t* s_x;
  int* s_S;
  float* s_red;
  uint4 v[kBatch];

  __device__ __forceinline__ int units() const { return (2 * m * B) / 8; }   // 16-byte units of x (8 values each)
  __device__ __forceinline__ void load_batch(int u0) {
    const int nthr = blockDim.x, nu = units();
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int u = u0 + k * nthr;
      v[k] = u < nu ? reinterpret_cast<const uint4*>(x)[u] : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void load_x() {
    load_batch(threadIdx.x);
    __builtin_amdgcn_sched_barrier(0);                // issued before the caller's next loads
  }
  __device__ __forceinline__ void build();
};

// No record build (the operands come from the digit form, or the records are already built).
struct NoRecordBuild {
  static constexpr bool kLocal = false;
  __device__ __forceinline__ void load_x() {}
  __device__ __forceinline__ void build() {}
};

template <bool kStage>
__device__ __forceinline__ void F4RecordBuild<kStage>::build() {
  __builtin_amdgcn_sched_barrier(0);                  // the caller's loads stay ahead of the build
  const int tid = threadIdx.x, nthr = blockDim.x, nwave = nthr / kWave;
  const int nu = units();
  const int per_b = (2 * m) / 8;
  float amax[2] = {0.f, 0.f};
  auto take = [&](int u0) {                           // stage and take the maxima of a loaded batch
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int u = u0 + k * nthr;
      if (u < nu) {
        if constexpr (kStage) reinterpret_cast<uint4*>(s_x)[u] = v[k];
        const uint32_t wd[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
        float mx = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(wd[e])), fabsf(bf16_hi(wd[e]))));
        if (u < per_b) amax[0] = fmaxf(amax[0], mx); else amax[1] = fmaxf(amax[1], mx);
      }
    }
  };
  take(tid);                                          // the batch load_x issued: outside the loop, so
  for (int u0 = tid + kBatch * nthr; u0 < nu; u0 += kBatch * nthr) {   // its waits count x alone
    load_batch(u0);
    take(u0);
  }
  amax[0] = wave_max(amax[0]);
  if (B > 1) amax[1] = wave_max(amax[1]);
  if ((tid & (kWave - 1)) == 0) {
    s_red[tid / kWave] = amax[0];
    s_red[nwave + tid / kWave] = amax[1];
  }
  __syncthreads();
  int S[2] = {0, 0};                                  // max |x_b| is order-free, so exact
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if (b < B) {
      float mx = 0.f;
      for (int w = 0; w < nwave; ++w) mx = fmaxf(mx, s_red[b * nwave + w]);
      S[b] = digit_exponent(mx);
    }
  }
  if (tid < B) s_S[tid] = tid == 0 ? S[0] : S[1];     // read by the epilogue, after the last barrier
  // Records in halves: an item is 16 consecutive columns of one (chunk, step, batch entry, lane
  // group, component) -- elements 16h .. 16h + 15 of that record -- and all eight of its digits,
  // so each column's Y is formed once; element q = 16h + e is column f4_column(0, 0, e) of the
  // half, and the half of digit l's record is its dwords 2h and 2h + 1 (elements 8j .. 8j + 7 of
  // the half in dword 2h + j).
  const int nitem = ((m + kF4Chunk - 1) / kF4Chunk) * 2 * B * 16;
  for (int item = tid; item < nitem; item += nthr) {
    const int h = item & 1, comp = (item >> 1) & 1, g = (item >> 2) & 3, blk = item >> 4;
    const int b = blk % B, cs = blk / B, s = cs & 1, c = cs >> 1;
    uint8_t* dst0 = s_rec + (((c * 2 + s) * B + b) * kWave + 16 * g + 8 * comp) * kRecBytes + 8 * h;
    if (kF4Chunk * c + 64 * g < m) {
      const uint4* src = reinterpret_cast<const uint4*>((kStage ? s_x : x) + (int64_t)b * 2 * m + (int64_t)comp * m +
                                                       kF4Chunk * c + 64 * g + 32 * s + 16 * h);
      const uint4 u[2] = {src[0], src[1]};
      build_record_half(u, b == 0 ? S[0] : S[1], dst0);
    } else {
#pragma unroll
      for (int l = 0; l < 8; ++l) *reinterpret_cast<uint2*>(dst0 + l * kRecBytes) = make_uint2(0u, 0u);
    }
  }
  __syncthreads();
}

// The whole build at once (for callers with no loads to put between its parts).
template <bool kStage>
__device__ __forceinline__ void build_f4_records(const uint16_t* x, int m, int B, uint8_t* s_rec, uint16_t* s_x,
                                                 int* s_S, float* s_red) {
  F4RecordBuild<kStage> bld{x, m, B, s_rec, s_x, s_S, s_red, {}};
  bld.load_x();
  bld.build();
}

// Per-wave records with one exponent per chunk and batch entry (bf16 x): wave w of the NW waves that
// split a tile builds the records of its own chunks c = w, w + NW, ... and nothing else, each at
// its chunk's own exponent S_c (max over the chunk's 512 values of |x| 2^S_c in [2^21, 2^22)).
// There is no workgroup-wide step: the wave reads only its chunks of x, reduces their maxima on
// DPP and writes records that only it reads (LDS accesses of one wave complete in order).  The
// chunk's MFMAs then take 2^-S_c as their block scales (2^-floor(S_c/2) on A, the rest on B; S_c
// lies in [-106, 147], so both fit E8M0), so the digit sums of every chunk enter the fp32
// accumulators at one common scale and the epilogue applies only the digit weight.  Against one
// exponent per row, each chunk's X keeps 22 bits below its own maximum (never fewer), and the sums
// across chunks round in fp32.  A pass covers 64 items (halves of a chunk's records), one per lane:
// two of the wave's chunks at batch 1, one chunk's two batch entries at batch 2.
template <int BT>
struct F4LocalBuild {
  static constexpr bool kLocal = true;
  static constexpr int kPre = 4;                      // passes whose x loads are issued up front
  const uint16_t* x;                                  // bf16 [BT][2m]
  int m, nw, wave;
  uint8_t* s_rec;
  int* s_Sc;                                          // one exponent per chunk and batch entry
  uint4 v[kPre][2];                                   // this lane's items: 16 columns of x per pass
  __device__ __forceinline__ int nchunk() const { return (m + kF4Chunk - 1) / kF4Chunk; }
  // A pass covers 64 half-records: two of the wave's chunks at batch 1, one chunk's two batch
  // entries at batch 2 (lanes 32-63 take the second).
  __device__ __forceinline__ int passes() const {
    const int cpw = wave < nchunk() ? (nchunk() - wave + nw - 1) / nw : 0;
    return BT == 1 ? (cpw + 1) / 2 : cpw;
  }
  __device__ __forceinline__ int lane() const { return threadIdx.x & (kWave - 1); }
  __device__ __forceinline__ int chunk_of(int pass) const {
    return BT == 1 ? wave + nw * (2 * pass + (lane() >> 5)) : wave + nw * pass;
  }
  __device__ __forceinline__ int batch_of() const { return BT == 1 ? 0 : lane() >> 5; }
  __device__ __forceinline__ bool present(int c, int g) const { return c < nchunk() && kF4Chunk * c + 64 * g < m; }
  // Range-checked buffer loads (absent columns read the out-of-range offset, which returns 0):
  // no branch, so the passes' loads issue back to back with no wait between them.
  __device__ __forceinline__ void load_pass(int pass, uint4 (&u)[2]) const {
    const __amdgpu_buffer_rsrc_t rs = range_rsrc(x + (int64_t)batch_of() * 2 * m, (int64_t)4 * m);
    const int c = chunk_of(pass);
    const int item = lane() & 31, h = item & 1, comp = (item >> 1) & 1, g = (item >> 2) & 3, s = item >> 4;
    const uint32_t off = present(c, g) ? (uint32_t)(2 * (comp * m + kF4Chunk * c + 64 * g + 32 * s + 16 * h)) : kNoLoad;
    u[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    u[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off == kNoLoad ? kNoLoad : off + 16, 0, 0));
  }
  // The x loads of the first kPre passes (all of them for rows of up to 8192 columns split over
  // four or more waves), so that later passes do not wait for a load of their own.
  __device__ __forceinline__ void load_x() {
    const int np = passes();
#pragma unroll
    for (int p = 0; p < kPre; ++p)
      if (p < np) load_pass(p, v[p]);
    __builtin_amdgcn_sched_barrier(0);                // issued before the caller's next loads
  }
  __device__ __forceinline__ void build_pass(int pass, const uint4 (&u)[2]) {
    const int item = lane() & 31, h = item & 1, comp = (item >> 1) & 1, g = (item >> 2) & 3, s = item >> 4;
    float mx = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t wd[4] = {u[k].x, u[k].y, u[k].z, u[k].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(wd[e])), fabsf(bf16_hi(wd[e]))));
    }
    mx = fmaxf(mx, dpp_read<0xB1>(mx));               // lane ^ 1
    mx = fmaxf(mx, dpp_read<0x4E>(mx));               // lane ^ 2
    mx = fmaxf(mx, dpp_read<0x141>(mx));              // row_half_mirror
    mx = fmaxf(mx, dpp_read<0x140>(mx));              // row_mirror: every lane holds its row's maximum
    const int iv = __builtin_bit_cast(int, mx);
    const float m0 = fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 0)),
                           __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 16)));
    const float m1 = fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 32)),
                           __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 48)));
    const int S0 = digit_exponent(m0), S1 = digit_exponent(m1);
    const int c = chunk_of(pass);
    if (c < nchunk()) {
      uint8_t* dst0 = s_rec + (((c * 2 + s) * BT + batch_of()) * kWave + 16 * g + 8 * comp) * kRecBytes + 8 * h;
      if (present(c, g)) {
        build_record_half(u, lane() < 32 ? S0 : S1, dst0);
      } else {
#pragma unroll
        for (int l = 0; l < 8; ++l) *reinterpret_cast<uint2*>(dst0 + l * kRecBytes) = make_uint2(0u, 0u);
      }
    }
    if (lane() == 0) {
      if constexpr (BT == 1) {
        s_Sc[wave + nw * 2 * pass] = S0;
        if (wave + nw * (2 * pass + 1) < nchunk()) s_Sc[wave + nw * (2 * pass + 1)] = S1;
      } else {
        s_Sc[2 * (wave + nw * pass)] = S0;             // [chunk][batch entry]
        s_Sc[2 * (wave + nw * pass) + 1] = S1;
      }
    }
  }
  __device__ __forceinline__ void build() {
    __builtin_amdgcn_sched_barrier(0);                // the caller's loads stay ahead of the build
    const int np = passes();
#pragma unroll
    for (int p = 0; p < kPre; ++p)
      if (p < np) build_pass(p, v[p]);
    for (int p = kPre; p < np; ++p) {                 // rows longer than the up-front loads cover
      uint4 u[2];
      load_pass(p, u);
      build_pass(p, u);
    }
  }
};

// ------------------------------------------------------------------------- GEMV ----

// The epilogue's sum over a row's 16 lanes (digits and components): DPP permutes (group_sum) for
// one batch entry per tile, and for two at T <= 2 (there they cost no registers, and against lane
// shuffles through LDS they saved ~1 us per small batch-2 launch: 32-layer decode step on the
// digit form 1220 -> 1092 us).  Two entries at T > 2: lane shuffles, which the compiler schedules
// with fewer live registers there (with DPP those kernels took 16-48 more and lost a wave per SIMD).
template <int BT, int TT>
__device__ __forceinline__ void row_sums(float& vre, float& vim) {
  if constexpr (BT == 1 || TT <= 2) {
    vre = group_sum<16>(vre);
    vim = group_sum<16>(vim);
  } else {
#pragma unroll
    for (int off = 1; off <= 8; off <<= 1) {
      vre += __shfl_xor(vre, off);
      vim += __shfl_xor(vim, off);
    }
  }
}

// One unit (a 16-row tile of one item) streamed by NW cooperating waves; `wave` is this wave's
// index among them, s_scw its own LDS slot for the tile's scales, s_y the NW waves' partial outputs.
// EXACT (NW = 4, one batch entry): the waves first add their accumulators through LDS (s_acc,
// 16 T x 64 floats per wave) -- exact, since every partial and total is an integer below 2^24 --
// and wave w then runs the single-wave epilogue for rows 4g + w, so the outputs are bit-identical
// to one wave streaming the whole unit.
// FUSED: x is bf16 [B][2m] (not its digit form); the operands are the workgroup's records in s_rec
// and S_b in s_S, built either before the waves call this function or by bld, which the function
// calls (every wave, once) with the tile's scale and first code loads between its two parts.
template <int TT, int NW, int BT, typename YT, bool EXACT = false, bool FUSED = false,
          typename Build = NoRecordBuild>
__device__ __forceinline__ void gemv_f4_tile(const GemvGroup& grp, int m, int B, int unit, int wave,
                                             float* __restrict__ s_scw, float (*s_y)[BT][2][16],
                                             float* __restrict__ s_acc = nullptr,
                                             const uint8_t* __restrict__ s_rec = nullptr,
                                             const int* __restrict__ s_S = nullptr, Build bld = {}) {
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

  // codes; fp6 digit operands per step (from the digit form; FUSED reads them from LDS instead)
  struct Chunk { uint4 w[TT][2]; v8i x[FUSED ? 1 : 2][FUSED ? 1 : BT]; int c; };
  auto load_chunk = [&](int c, Chunk& ch) {
    const int groups = min(4, (m - kF4Chunk * c) >> 6);
    const bool k_ok = g < groups;
    const uint32_t cbase = (uint32_t)c * (TT * 2) * 1024;
    ch.c = c;
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int M = 0; M < 2; ++M)
        ch.w[t][M] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
            rsrc_a, k_ok ? cbase + (uint32_t)((t * 2 + M) * groups * 256 + lane * 16) : kNoLoad, 0, kStreamLoad));
    if constexpr (FUSED) return;
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
        ch.x[FUSED ? 0 : s][FUSED ? 0 : b] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, 0, 0};
      }
  };
  auto compute_chunk = [&](const Chunk& ch) {
    // block scales (E8M0, 127 = 2^0): 2^-S for per-chunk records (Build::kLocal; one S per chunk
    // and batch entry), else 2^0
    int sca[BT], scb[BT];
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      sca[b] = 127;
      scb[b] = 127;
      if constexpr (Build::kLocal) {
        const int S = __builtin_amdgcn_readfirstlane(bld.s_Sc[ch.c * BT + b]);
        sca[b] = 127 - (S >> 1);
        scb[b] = 127 - (S - (S >> 1));
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v8i xs[BT];                          // this step's B operands
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        if constexpr (FUSED) {
          if (b < B) {
            const uint4 rr = *reinterpret_cast<const uint4*>(s_rec + (((ch.c * 2 + s) * B + b) * kWave + lane) * kRecBytes);
            xs[b] = v8i{(int)rr.x, (int)rr.y, (int)rr.z, (int)rr.w, 0, 0, 0, 0};
          } else {
            xs[b] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
          }
        } else {
          xs[b] = ch.x[FUSED ? 0 : s][FUSED ? 0 : b];
        }
      }
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int M = 0; M < 2; ++M) {
          const uint4 q = ch.w[t][M];
          v8i pu, pv;
          decode_f4(s == 0 ? q.x : q.z, s == 0 ? q.y : q.w, pu, pv);
#pragma unroll
          for (int b = 0; b < BT; ++b) {
            // A fp4; B fp6 e2m3 (digit form) or fp4 (records in LDS)
            acc[t][M][0][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                pu, xs[b], acc[t][M][0][b], 4, FUSED ? 4 : 2, 0, sca[b], 0, scb[b]);
            acc[t][M][1][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                pv, xs[b], acc[t][M][1][b], 4, FUSED ? 4 : 2, 0, sca[b], 0, scb[b]);
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
  bld.load_x();
  tsc.load(scales, i0, n, lane);               // ahead of the first chunk's loads
  if constexpr (BT == 1 && TT <= 2) {
    Chunk c0, c1, c2;
    int c = wave;                                  // wave w takes chunks w, w + NW, ...
    load_chunk(c, c0);
    load_chunk(c + NW, c1);
    bld.build();
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
  } else if constexpr (BT == 2 || FUSED) {
    // One chunk per iteration, the prefetched set copied into place at its end (16 moves per
    // chunk).  With the loop unrolled over two sets instead, the register allocator moves the
    // accumulators between register ranges every iteration (64-192 accumulator moves per 32-96
    // MFMAs at batch 2), which also raised the batch-2 kernels from 164-168 to 212-228 registers
    // (two waves per SIMD instead of three).
    Chunk cur, nxt;
    int c = wave;
    load_chunk(c, cur);
    bld.build();
    tsc.park(s_scw, lane);
    for (; c < nchunk; c += NW) {
      load_chunk(c + NW, nxt);
      __builtin_amdgcn_sched_barrier(0);
      compute_chunk(cur);
      cur = nxt;
    }
  } else {
    Chunk c0, c1;
    int c = wave;
    load_chunk(c, c0);
    bld.build();
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
  // fp32 scales, the digit weight 2^(3l - S_b) / 6, and the sum over digits and components: the
  // 16 lanes of a row, on DPP lane permutes (group_sum).
  if constexpr (EXACT) {
    if constexpr (FUSED) __syncthreads();        // s_acc shares LDS with the records: all waves are past them
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
    const int S = Build::kLocal || b >= B ? 0 : (FUSED ? s_S[b] : hdr[2 + b]);   // kLocal: in the MFMA scales
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
      row_sums<BT, TT>(vre, vim);
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

// One wave of a resident workgroup on bf16 x: it takes units first, first + stride, ... (below
// tiles) and streams their (unit, chunk) steps as one sequence, with the operand sets in flight
// running on across unit boundaries (so no unit starts with an empty pipeline); at a unit's last
// chunk it runs that unit's epilogue.  B operands come from the workgroup's records in LDS; each
// unit's scales are loaded while the unit streams and parked in s_scw before its epilogue.  The
// arithmetic per unit is that of gemv_f4_tile with one wave, so the outputs are identical.
// bld builds the records (every wave calls it once), with the first unit's scale and code loads
// issued between its two parts.
template <int TT, int BT, typename YT, typename Build>
__device__ __forceinline__ void gemv_f4_stream(const GemvGroup& grp, int m, int B, int first, int stride, int tiles,
                                               float* __restrict__ s_scw, const uint8_t* __restrict__ s_rec,
                                               const int* __restrict__ s_S, Build bld) {
  if (first >= tiles) {
    bld.load_x();
    bld.build();
    return;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15, g = lane >> 4;
  const int nchunk = (m + kF4Chunk - 1) / kF4Chunk;
  const int64_t tile_bytes = (int64_t)16 * TT * 2 * (m / 4);
  const int nunits = (tiles - 1 - first) / stride + 1;
  const int total = nunits * nchunk;

  v4f acc[TT][2][2][BT];
  auto clear = [&]() {
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int M = 0; M < 2; ++M)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int b = 0; b < BT; ++b) acc[t][M][p][b] = v4f{0.f, 0.f, 0.f, 0.f};
  };
  clear();

  // code stream of unit k of this wave (an empty range past the last unit: loads return 0)
  auto unit_rsrc = [&](int k) {
    int tile = 0;
    const GemvItem it = locate_item<YT>(grp, first + min(k, nunits - 1) * stride, tile);
    return range_rsrc(static_cast<const uint8_t*>(it.packed) + (int64_t)tile * tile_bytes, k < nunits ? tile_bytes : 0);
  };
  struct Chunk { uint4 w[TT][2]; };
  int lk = 0, lc = 0;                                  // unit and chunk of the next load
  __amdgpu_buffer_rsrc_t lrs = unit_rsrc(0);
  auto load_next = [&](Chunk& ch) {
    const int groups = min(4, (m - kF4Chunk * lc) >> 6);
    const bool k_ok = g < groups;
    const uint32_t cbase = (uint32_t)lc * (TT * 2) * 1024;
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int M = 0; M < 2; ++M)
        ch.w[t][M] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
            lrs, k_ok ? cbase + (uint32_t)((t * 2 + M) * groups * 256 + lane * 16) : kNoLoad, 0, kStreamLoad));
    if (++lc == nchunk) {
      lc = 0;
      lrs = unit_rsrc(++lk);
    }
  };

  TileScales<TT> tsc;
  auto load_scales = [&](int k) {
    int tile = 0;
    const GemvItem it = locate_item<YT>(grp, first + k * stride, tile);
    tsc.load(it.scales, tile * 16, it.n, lane);
  };
  const int comp = r >> 3, l = r & 7;
  auto epilogue = [&](int k) {
    tsc.park(s_scw, lane);
    if (k + 1 < nunits) load_scales(k + 1);           // the next unit's scales, a whole unit ahead
    int tile = 0;
    const GemvItem it = locate_item<YT>(grp, first + k * stride, tile);
    const int n = it.n, i0 = tile * 16;
    YT* __restrict__ y = static_cast<YT*>(it.y);
    const int64_t ys = 2 * (int64_t)n;
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      const int S = b < B ? s_S[b] : 0;
      const float wdig = ldexpf(1.0f / 6.0f, 3 * l - S);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
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
        row_sums<BT, TT>(vre, vim);
        if (r == 0 && b < B && i < n) {
          store_out(y, (int64_t)b * ys + i, vre);
          store_out(y, (int64_t)b * ys + n + i, vim);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();                   // the scales are read before the next park
    clear();
  };

  int ck = 0, cc = 0;                                  // unit and chunk of the next compute
  auto compute_next = [&](const Chunk& ch) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v8i xs[BT];
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        if (b < B) {
          const uint4 rr = *reinterpret_cast<const uint4*>(s_rec + (((cc * 2 + s) * B + b) * kWave + lane) * kRecBytes);
          xs[b] = v8i{(int)rr.x, (int)rr.y, (int)rr.z, (int)rr.w, 0, 0, 0, 0};
        } else {
          xs[b] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        }
      }
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
                pu, xs[b], acc[t][M][0][b], 4, 4, 0, 127, 0, 127);   // A and B fp4, scales 2^0
            acc[t][M][1][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                pv, xs[b], acc[t][M][1][b], 4, 4, 0, 127, 0, 127);
          }
        }
    }
    if (++cc == nchunk) {
      epilogue(ck);
      cc = 0;
      ++ck;
    }
  };

  bld.load_x();
  load_scales(0);
  if constexpr (BT == 1 && TT <= 2) {                  // three operand sets in flight
    Chunk c0, c1, c2;
    load_next(c0);
    load_next(c1);
    bld.build();
    int st = 0;
    for (; st + 2 < total; st += 3) {
      load_next(c2);
      __builtin_amdgcn_sched_barrier(0);
      compute_next(c0);
      load_next(c0);
      __builtin_amdgcn_sched_barrier(0);
      compute_next(c1);
      load_next(c1);
      __builtin_amdgcn_sched_barrier(0);
      compute_next(c2);
    }
    if (st < total) compute_next(c0);
    if (st + 1 < total) compute_next(c1);
  } else {                                            // two
    Chunk c0, c1;
    load_next(c0);
    bld.build();
    int st = 0;
    for (; st + 1 < total; st += 2) {
      load_next(c1);
      __builtin_amdgcn_sched_barrier(0);
      compute_next(c0);
      load_next(c0);
      __builtin_amdgcn_sched_barrier(0);
      compute_next(c1);
    }
    if (st < total) compute_next(c0);
  }
}

template <int TT, int NW, int BT, typename YT, bool FUSED>
__global__ __launch_bounds__(kWave * NW, (BT == 1 && TT <= 3) ? 3 : 1) void k_gemv_f4(const GemvGroup grp, int m, int B) {
  __shared__ float s_sc[NW][16 * TT * 4];
  __shared__ float s_y[NW > 1 ? NW : 1][BT][2][16];     // [wave][batch][re/im][row]
  __shared__ int s_S[2];
  __shared__ float s_red[2 * NW];
  extern __shared__ __align__(16) uint8_t s_dyn[];       // FUSED: records, then the staged x
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
  if constexpr (FUSED) {
    int tile;
    const GemvItem it = locate_item<YT>(grp, blockIdx.x, tile);
    const F4RecordBuild<true> bld{static_cast<const uint16_t*>(it.x), m, B, s_dyn,
                                  reinterpret_cast<uint16_t*>(s_dyn + f4_record_bytes(m, B)), s_S, s_red, {}};
    gemv_f4_tile<TT, NW, BT, YT, false, true>(grp, m, B, blockIdx.x, wave, s_sc[wave], s_y, nullptr, s_dyn, s_S, bld);
  } else {
    gemv_f4_tile<TT, NW, BT, YT, false, false>(grp, m, B, blockIdx.x, wave, s_sc[wave], s_y);
  }
}

// Small launches on bf16 x (NW > 1 waves per tile, batch 1-2): each wave builds the records of its
// own chunks at per-chunk exponents (F4LocalBuild), so no wave waits on another before its first
// MFMA; the waves meet once, to add their partial outputs.
template <int TT, int NW, int BT, typename YT>
__global__ __launch_bounds__(kWave * NW, (BT == 1 && TT <= 3) ? 3 : 1) void k_gemv_f4_local(const GemvGroup grp, int m) {
  static_assert(NW > 1, "the waves of a tile split its chunks");
  __shared__ float s_sc[NW][16 * TT * 4];
  __shared__ float s_y[NW][BT][2][16];                  // [wave][batch][re/im][row]
  extern __shared__ __align__(16) uint8_t s_dyn[];       // records, then one exponent per chunk
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
  int tile;
  const GemvItem it = locate_item<YT>(grp, blockIdx.x, tile);
  const F4LocalBuild<BT> bld{static_cast<const uint16_t*>(it.x), m, NW, wave, s_dyn,
                             reinterpret_cast<int*>(s_dyn + f4_record_bytes(m, BT)), {}};
  gemv_f4_tile<TT, NW, BT, YT, false, true>(grp, m, BT, blockIdx.x, wave, s_sc[wave], s_y, nullptr, s_dyn, nullptr, bld);
}

// Large batch-1 launches in two granularities.  The first nA workgroups take four units each,
// one wave per unit (the fastest form while the chip is full); the rest take one unit each, its
// chunks split over the four waves.  Workgroups start in index order, so the units that finish a
// launch are the short-lived ones: the launch's tail, where fewer and fewer waves remain in
// flight, lasts about a quarter as long.  Both forms give the single-wave kernel's outputs bit for
// bit (the split one adds its waves' exact integer accumulators before the epilogue).  FUSED: the
// four tiles of a workgroup share one set of records; the split form's accumulator exchange reuses
// their LDS once every wave is past its last chunk.  (Every item of a launch shares x.)
template <int TT, typename YT, bool FUSED>
__global__ __launch_bounds__(kWave * 4, 3) void k_gemv_f4_mixed(const GemvGroup grp, int m, int nA) {
  __shared__ float s_sc[4][16 * TT * 4];
  __shared__ float s_y[4][1][2][16];
  __shared__ float s_acc_own[FUSED ? 1 : 4 * 16 * TT * kWave];
  __shared__ int s_S[2];
  __shared__ float s_red[8];
  extern __shared__ __align__(16) uint8_t s_dyn[];       // FUSED: records and staged x; then s_acc
  float* s_acc = FUSED ? reinterpret_cast<float*>(s_dyn) : s_acc_own;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
  if constexpr (FUSED)
    build_f4_records<true>(static_cast<const uint16_t*>(grp.items[0].x), m, 1, s_dyn,
                           reinterpret_cast<uint16_t*>(s_dyn + f4_record_bytes(m, 1)), s_S, s_red);
  if ((int)blockIdx.x < nA)
    gemv_f4_tile<TT, 1, 1, YT, false, FUSED>(grp, m, 1, 4 * (int)blockIdx.x + wave, 0, s_sc[wave], s_y, nullptr,
                                             s_dyn, s_S);
  else
    gemv_f4_tile<TT, 4, 1, YT, true, FUSED>(grp, m, 1, 4 * nA + ((int)blockIdx.x - nA), wave, s_sc[wave], s_y,
                                            s_acc, s_dyn, s_S);
}

// FUSED launches of one wave per tile (at least 1536 tiles): workgroups of four waves stay resident
// for the whole launch, build one set of records, and each wave then streams tiles
// 4 blockIdx + wave, then 4 gridDim more, ... (the grid is the number of workgroups the chip holds
// at once) as one sequence (gemv_f4_stream), so the records are built once per resident workgroup
// rather than once per four tiles and no tile starts with an empty pipeline.
template <int TT, int BT, typename YT>
__global__ __launch_bounds__(kWave * 4, (BT == 1 && TT <= 3) ? 3 : 1) void k_gemv_f4_persist(const GemvGroup grp, int m, int B) {
  __shared__ float s_sc[4][16 * TT * 4];
  __shared__ int s_S[2];
  __shared__ float s_red[8];
  extern __shared__ __align__(16) uint8_t s_dyn[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
  const uint16_t* x = static_cast<const uint16_t*>(grp.items[0].x);
  const int tiles = group_tiles(grp);
  if constexpr (BT == 1) {
    const F4RecordBuild<true> bld{x, m, B, s_dyn, reinterpret_cast<uint16_t*>(s_dyn + f4_record_bytes(m, B)), s_S,
                                  s_red, {}};
    gemv_f4_stream<TT, BT, YT>(grp, m, B, 4 * (int)blockIdx.x + wave, 4 * (int)gridDim.x, tiles, s_sc[wave], s_dyn, s_S,
                               bld);
  } else {
    // batch 2 builds without the staged copy of x (the records alone let three workgroups share a
    // CU), before its tile loop
    build_f4_records<false>(x, m, B, s_dyn, nullptr, s_S, s_red);
    // batch 2: one tile at a time (the streaming form's registers would halve its occupancy;
    // measured 5139 against 4832 GB/s on the 1 GiB attention pool)
    for (int unit = 4 * (int)blockIdx.x + wave; unit < tiles; unit += 4 * (int)gridDim.x)
      gemv_f4_tile<TT, 1, BT, YT, false, true>(grp, m, B, unit, 0, s_sc[wave], nullptr, nullptr, s_dyn, s_S);
  }
}

// Mixed-granularity launches: units left to the one-unit-per-workgroup form at the end, and the
// smallest launch that uses them (measured on the 1 GiB pool, 32768 tiles: tails of 256-2048 tiles
// within 1 % of each other and ~2 % faster than 3072-6144; launches of 6144 tiles ran slower in
// this form, 16512 unchanged).
constexpr int kF4TailTiles = 1536;
constexpr int kF4MixedMinTiles = 12288;

// Most dynamic LDS a launch on bf16 x can take with BT batch entries per tile: records (and the
// staged x, if kept) of m B <= 8192 columns, the most the C ABI accepts on this path.
constexpr int kF4FusedMaxCols = 8192;
static size_t f4_fused_lds_max(int BT, bool stage) {
  const int m = kF4FusedMaxCols / BT;
  return (size_t)f4_record_bytes(m, BT) + (stage ? (size_t)f4_xstage_bytes(m, BT) : 0);
}

// Host-side launch state of one kernel, per device and guarded by a mutex (callers may launch
// from several threads or devices): whether its dynamic-LDS limit has been raised there, and how
// many of its workgroups the device holds at once with a given dynamic LDS.
constexpr int kMaxLaunchDevices = 64;
struct KernelLaunchState {
  std::mutex mu;
  bool lds_set[kMaxLaunchDevices] = {};
  size_t resident_lds[kMaxLaunchDevices] = {};
  int resident[kMaxLaunchDevices] = {};
};

static int current_device() {
  int dev = 0;
  return hipGetDevice(&dev) == hipSuccess ? dev : 0;
}

// Dynamic LDS above 64 KB needs a kernel attribute; it is set once per kernel and device, to the
// most any of its launches can take, so later launches with larger rows are covered too.
template <typename K>
static void lds_launch_prepare(K kernel, size_t max_bytes, KernelLaunchState& st) {
  if (max_bytes <= 65536) return;
  const int dev = current_device();
  std::lock_guard<std::mutex> lock(st.mu);
  if (dev >= 0 && dev < kMaxLaunchDevices && st.lds_set[dev]) return;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)max_bytes);
  if (dev >= 0 && dev < kMaxLaunchDevices) st.lds_set[dev] = true;
}

// Workgroups of `threads` threads and `lds` bytes of dynamic LDS that the current device holds at
// once (at least one per CU).
template <typename K>
static int resident_workgroups(K kernel, int threads, size_t lds, KernelLaunchState& st) {
  const int dev = current_device();
  std::lock_guard<std::mutex> lock(st.mu);
  const bool cached = dev >= 0 && dev < kMaxLaunchDevices;
  if (cached && st.resident[dev] > 0 && st.resident_lds[dev] == lds) return st.resident[dev];
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel), threads, lds) !=
          hipSuccess || per_cu < 1)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  if (cached) {
    st.resident[dev] = per_cu * cus;
    st.resident_lds[dev] = lds;
  }
  return per_cu * cus;
}

// Waves per tile of the per-wave-record launches: as the other small launches, except that long
// rows (16 chunks or more) in launches of at most 256 tiles split over eight waves, so each wave
// builds fewer records before its first MFMA (32-layer step, 4096 x 11008 projection: 8.2 ->
// 7.9 us per launch; at 2048 columns eight waves were slower, 4.46 -> 5.0 us).
static int f4_local_waves_per_tile(int tiles, int m) {
  const int nchunk = (m + kF4Chunk - 1) / kF4Chunk;
  return nchunk >= 16 && tiles <= 256 ? 8 : gemv_waves_per_tile(tiles, m);
}

template <int TT, int BT, typename YT, bool FUSED>
static void launch_f4_t(const GemvGroup& group, int m, int B, hipStream_t s) {
  GemvGroup grp = group;
  grp.units_per_item = grp.tiles_per_item;        // one workgroup per tile
  const int tiles = group_tiles(grp);
  const size_t rec = FUSED ? (size_t)f4_record_bytes(m, B) + f4_xstage_bytes(m, B) : 0;
  if constexpr (FUSED) {
    if (gemv_waves_per_tile(tiles, m) == 1) {             // resident workgroups, four tiles at a time
      const size_t lds = BT == 1 ? rec : (size_t)f4_record_bytes(m, B);
      static KernelLaunchState st;
      lds_launch_prepare(k_gemv_f4_persist<TT, BT, YT>, f4_fused_lds_max(BT, BT == 1), st);
      const int grid = std::min((tiles + 3) / 4, resident_workgroups(k_gemv_f4_persist<TT, BT, YT>, 4 * kWave, lds, st));
      hipLaunchKernelGGL((k_gemv_f4_persist<TT, BT, YT>), dim3(grid), dim3(4 * kWave), lds, s, grp, m, B);
      return;
    }
  }
  if constexpr (BT == 1 && TT <= 3) {
    if (gemv_waves_per_tile(tiles, m) == 1 && tiles >= kF4MixedMinTiles) {
      const int nA = (tiles - kF4TailTiles) / 4;          // four units per workgroup
      const size_t lds = FUSED ? std::max(rec, (size_t)4 * 16 * TT * kWave * sizeof(float)) : 0;
      static KernelLaunchState st;
      lds_launch_prepare(k_gemv_f4_mixed<TT, YT, FUSED>,
                         FUSED ? std::max(f4_fused_lds_max(1, true), (size_t)4 * 16 * TT * kWave * sizeof(float)) : 0,
                         st);
      hipLaunchKernelGGL((k_gemv_f4_mixed<TT, YT, FUSED>), dim3(nA + (tiles - 4 * nA)), dim3(4 * kWave), lds, s, grp,
                         m, nA);
      return;
    }
  }
  const dim3 grid(tiles);
  if constexpr (FUSED) {                                  // small launches: per-wave records
    const size_t lds = (size_t)f4_record_bytes(m, BT) + f4_local_exp_bytes(m, BT);
    const size_t lds_max = (size_t)f4_record_bytes(kF4FusedMaxCols / BT, BT) + f4_local_exp_bytes(kF4FusedMaxCols / BT, BT);
    switch (f4_local_waves_per_tile(tiles, m)) {
#define F2I_F4_LOCAL_CASE(NWV)                                                                        \
      {                                                                                                 \
        static KernelLaunchState st;                                                                    \
        lds_launch_prepare(k_gemv_f4_local<TT, NWV, BT, YT>, lds_max, st);                              \
        hipLaunchKernelGGL((k_gemv_f4_local<TT, NWV, BT, YT>), grid, dim3(NWV * kWave), lds, s, grp, m); \
      }                                                                                                 \
      return;
      case 8: F2I_F4_LOCAL_CASE(8)
      case 4: F2I_F4_LOCAL_CASE(4)
      default: F2I_F4_LOCAL_CASE(2)
#undef F2I_F4_LOCAL_CASE
    }
  } else {
  switch (gemv_waves_per_tile(tiles, m)) {
#define F2I_F4_CASE(NWV)                                                                               \
    {                                                                                                    \
      static KernelLaunchState st;                                                                       \
      lds_launch_prepare(k_gemv_f4<TT, NWV, BT, YT, FUSED>, FUSED ? f4_fused_lds_max(BT, true) : 0, st);    \
      hipLaunchKernelGGL((k_gemv_f4<TT, NWV, BT, YT, FUSED>), grid, dim3(NWV * kWave), rec, s, grp, m, B); \
    }                                                                                                    \
    break;
    case 8: F2I_F4_CASE(8)
    case 4: F2I_F4_CASE(4)
    case 2: F2I_F4_CASE(2)
    default: F2I_F4_CASE(1)
#undef F2I_F4_CASE
  }
  }
}

template <int TT, typename YT, bool FUSED>
static void launch_f4_b(const GemvGroup& grp, int m, int B, hipStream_t s) {
  if (B == 1) launch_f4_t<TT, 1, YT, FUSED>(grp, m, B, s);
  else launch_f4_t<TT, 2, YT, FUSED>(grp, m, B, s);
}

template <typename YT, bool FUSED>
static void launch_f4_y(const GemvGroup& grp, int m, int T, int B, hipStream_t s) {
  switch (T) {
    case 1: launch_f4_b<1, YT, FUSED>(grp, m, B, s); break;
    case 2: launch_f4_b<2, YT, FUSED>(grp, m, B, s); break;
    case 3: launch_f4_b<3, YT, FUSED>(grp, m, B, s); break;
    default: launch_f4_b<4, YT, FUSED>(grp, m, B, s); break;
  }
}

hipError_t launch_gemv_f4_group(const GemvGroup& grp, int m, int T, int B, int y_bf16, int x_bf16, hipStream_t s) {
  if (x_bf16) {
    if (y_bf16) launch_f4_y<uint16_t, true>(grp, m, T, B, s);
    else launch_f4_y<float, true>(grp, m, T, B, s);
  } else {
    if (y_bf16) launch_f4_y<uint16_t, false>(grp, m, T, B, s);
    else launch_f4_y<float, false>(grp, m, T, B, s);
  }
  return hipGetLastError();
}

hipError_t launch_gemv_f4(const uint8_t* packed, const float* scales, int n, int m, int T,
                          const void* x, int B, void* y, int y_bf16, int x_bf16, hipStream_t s) {
  GemvGroup grp;
  grp.count = 1;
  grp.tile_start[0] = 0;
  grp.tile_start[1] = (n + 15) / 16;
  grp.items[0] = GemvItem{packed, scales, x, y, n};
  return launch_gemv_f4_group(grp, m, T, B, y_bf16, x_bf16, s);
}

int gemv_f4_record_bytes(int m, int B) { return f4_record_bytes(m, B); }

}  // namespace f2i
