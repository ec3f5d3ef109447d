// Device helpers and internal launcher declarations shared by the library's HIP sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace f2i {

constexpr int kWave = 64;

// bf16 <-> fp32.  bf16 is the upper half of an fp32 bit pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (quiet NaN kept).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Sum of v over aligned groups of N lanes (N = 2, 4, 8 or 16, within a 16-lane row), every lane
// of a group ending with the total, on DPP lane permutes (a VALU operand modifier: no LDS
// traffic).  The steps pair lanes as an xor butterfly over offsets 1, 2, 4, 8 does -- quad
// permutes for 1 and 2; then, with the values already uniform across each quad (half-row),
// the half-row mirror (lane 7 - i) and the row mirror (lane 15 - i) meet the same partner groups
// as offsets 4 and 8 -- and IEEE addition is commutative, so the sums are the butterfly's bit
// for bit and equal in every lane of the group.
template <int CTRL>
__device__ __forceinline__ float dpp_read(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  // No contraction into these adds: fusing a caller's multiply into the first one would leave
  // the two lanes of a pair with differently rounded sums.
#pragma clang fp contract(off)
  static_assert(N == 2 || N == 4 || N == 8 || N == 16, "groups of 2, 4, 8 or 16 lanes");
  v += dpp_read<0xB1>(v);                          // quad_perm [1, 0, 3, 2]: lane ^ 1
  if constexpr (N >= 4) v += dpp_read<0x4E>(v);    // quad_perm [2, 3, 0, 1]: lane ^ 2
  if constexpr (N >= 8) v += dpp_read<0x141>(v);   // row_half_mirror: quad 0 <-> 1, 2 <-> 3
  if constexpr (N >= 16) v += dpp_read<0x140>(v);  // row_mirror: half-row 0 <-> 1
  return v;
}

// Stores one fp32 value as the output dtype.
__device__ __forceinline__ void store_out(float* y, int64_t idx, float v) { y[idx] = v; }
__device__ __forceinline__ void store_out(uint16_t* y, int64_t idx, float v) { y[idx] = f32_to_bf16_rne(v); }

}  // namespace f2i

// ---- internal launchers (host side), implemented in the .hip files ----
namespace f2i {
// One GEMV of a grouped launch (all items share m, T, B and the dtypes).
struct GemvItem {
  const void* packed;
  const float* scales;
  const void* x;
  void* y;
  int n;
};
// Packed form: 16-code words ordered per 16-row tile as [chunk of 256 columns][plane P = 2t+M]
// [64-column group < G_c][row][word < 4], tiles one after another, the last tile padded with
// rows of code 0.  Word index of word wq (columns 16wq .. 16wq+15) of plane P of row i:
__host__ __device__ __forceinline__ int64_t tiled_word(int i, int P, int wq, int m, int T) {
  const int c = wq >> 4, g = (wq >> 2) & 3, w = wq & 3;
  const int groups = min(4, (m - 256 * c) >> 6);        // 64-column groups in chunk c
  return (int64_t)(i >> 4) * 16 * (2 * T) * (m >> 4)    // 16 rows x 2T planes x m/16 words
       + (int64_t)c * (2 * T) * 256                      // full chunks before c
       + P * groups * 64 + g * 64 + (i & 15) * 4 + w;
}
__host__ __device__ __forceinline__ int padded_rows(int n) { return (n + 15) & ~15; }

// Waves per 16-row tile of the matrix-core GEMVs: one wave streams a whole tile when there are
// enough tiles to fill the chip (about 1536 waves); a smaller launch splits each tile's chunks
// over 4 waves (2 when there are fewer than 4 chunks), and a launch of under 64 tiles over up to
// 8.  Measured on the LLaMA-2-7B projection groups (128-688 tiles), 4 waves beat 8 by 0-36 %.
inline int gemv_waves_per_tile(int tiles, int m) {
  const int nchunk = (m + 255) / 256;
  if (tiles >= 1536 || nchunk < 2) return 1;
  if (nchunk < 4) return 2;
  return tiles < 64 && nchunk >= 8 ? 8 : 4;
}

constexpr int kMaxGroup = 48;   // items per launch; the table travels in the kernel arguments
struct GemvGroup {
  int count;
  int tile_start[kMaxGroup + 1];   // first 16-row tile of each item; [count] = total tiles
  GemvItem items[kMaxGroup];
  // Strided batch (batch > 0) instead of the table: items[0] is matrix 0, and matrix k's packed
  // form, scales and output lie k * packed_stride bytes, k * scales_stride floats and k * y_stride
  // output elements further on.  Every matrix has tiles_per_item tiles; a launcher sets
  // units_per_item to its workgroups per matrix.
  int batch = 0;
  int tiles_per_item = 0;
  int units_per_item = 0;
  int64_t packed_stride = 0, scales_stride = 0, y_stride = 0;
};
// 16-row tiles of a launch.
__host__ __device__ inline int group_tiles(const GemvGroup& g) {
  return g.batch > 0 ? g.batch * g.tiles_per_item : g.tile_start[g.count];
}
// Buffer resource over [base, base + bytes): loads at offsets past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const void* base, int64_t bytes) {
  const int nrec = (int)min(max(bytes, (int64_t)0), (int64_t)0x7FFFFF00);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
}
constexpr uint32_t kNoLoad = 0x80000000u;   // buffer offset past every range: the load returns 0
// Cache policy of loads whose data is read once (the decode GEMVs' code stream): non-temporal at
// device scope (sc1 nt), so the stream does not displace the reused x operands from the per-CU
// vector cache.  Measured +4-6 % on the fp4 GEMV; results are unaffected.
constexpr int kStreamLoad = 18;

// Scales of one 16-row tile, [row][t][M][axis] fp32 (16 x 4T floats; rows past n read as 0).
// A GEMV issues the load ahead of its operand stream (lane l takes floats lT .. lT + T - 1) and
// parks the values in LDS once they arrive, so its epilogue waits on no memory round trip.
template <int TT>
struct TileScales {
  float v[TT];
  __device__ __forceinline__ void load(const float* scales, int i0, int n, int lane) {
    const __amdgpu_buffer_rsrc_t rs =
        range_rsrc(scales + (int64_t)i0 * TT * 4, (int64_t)(min(n, i0 + 16) - i0) * TT * 16);
#pragma unroll
    for (int q = 0; q < TT; ++q)
      v[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)((lane * TT + q) * 4), 0, 0));
  }
  // lds: this wave's 16 x 4T floats
  __device__ __forceinline__ void park(float* lds, int lane) const {
#pragma unroll
    for (int q = 0; q < TT; ++q) lds[lane * TT + q] = v[q];
    __builtin_amdgcn_wave_barrier();
  }
};

// Workgroup -> item of a grouped launch: the last item whose first workgroup (tile_start, in the
// launch's own unit of tiles or tile groups) is at or before `block`.
__device__ __forceinline__ int find_item(const GemvGroup& g, int block) {
  int lo = 0, hi = g.count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (g.tile_start[mid] <= block) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Item of workgroup `block` of a grouped or strided-batch launch, and the workgroup's index within
// that item (`unit`, in the launch's own unit: tiles, or groups of tiles).
template <typename YT>
__device__ __forceinline__ GemvItem locate_item(const GemvGroup& g, int block, int& unit) {
  if (g.batch > 0) {
    const int k = block / g.units_per_item;
    unit = block - k * g.units_per_item;
    GemvItem it = g.items[0];
    it.packed = static_cast<const uint8_t*>(it.packed) + (int64_t)k * g.packed_stride;
    it.scales += (int64_t)k * g.scales_stride;
    it.y = static_cast<YT*>(it.y) + (int64_t)k * g.y_stride;
    return it;
  }
  const int k = find_item(g, block);
  unit = block - g.tile_start[k];
  return g.items[k];
}

hipError_t launch_gemv_mfma_group(const GemvGroup& grp, int m, int T, int B, int y_bf16, hipStream_t s);
hipError_t launch_quantize(const void* R, int r_bf16, int n, int m, int T, uint8_t* packed, float* scales,
                           double* scales64, uint8_t* codes, hipStream_t s);
// One matrix of a grouped quantize launch (every item has the same n, m, T and R dtype).
struct QuantItem {
  const void* R;
  uint8_t* packed;
  float* scales;
  double* scales64;    // may be null
  uint8_t* codes;      // may be null
};
constexpr int kMaxQuantItems = 32;   // items per launch; the table travels in the kernel arguments
struct QuantGroup {
  int count;
  QuantItem items[kMaxQuantItems];
};
hipError_t launch_quantize_group(const QuantGroup& grp, int r_bf16, int n, int m, int T, hipStream_t s);
size_t quantize_tensor_workspace_bytes(int64_t n);
hipError_t launch_quantize_tensor(const void* R, int r_bf16, int n, int m, int T, void* ws, uint8_t* packed,
                                  float* scales, double* scales64, uint8_t* codes, hipStream_t s);
hipError_t launch_pack(const uint8_t* codes, int n, int m, int T, uint8_t* packed, hipStream_t s);
hipError_t launch_gemv_valu(const uint8_t* packed, const float* scales, int n, int m, int T,
                            const void* x, int x_bf16, int B, void* y, int y_bf16, hipStream_t s);
hipError_t launch_gemv_mfma(const uint8_t* packed, const float* scales, int n, int m, int T,
                            const void* x, int B, void* y, int y_bf16, void* unused, hipStream_t s);
hipError_t launch_gemv_i8(const uint8_t* packed, const float* scales, int n, int m, int T,
                          const void* digits, int B, void* y, int y_bf16, hipStream_t s);
hipError_t launch_gemv_i8_group(const GemvGroup& grp, int m, int T, int B, int y_bf16, hipStream_t s);
// x_bf16: x is bf16 [B][2m] and each workgroup builds its digit records on chip; otherwise x
// is the digit form made by launch_x_digits_f6.
hipError_t launch_gemv_f4(const uint8_t* packed, const float* scales, int n, int m, int T,
                          const void* x, int B, void* y, int y_bf16, int x_bf16, hipStream_t s);
hipError_t launch_gemv_f4_group(const GemvGroup& grp, int m, int T, int B, int y_bf16, int x_bf16, hipStream_t s);
// Batch 3-16 on bf16 x: fp4 code planes times x split into two fp8 parts under per-block scales.
hipError_t launch_gemv_f8x_group(const GemvGroup& grp, int m, int T, int B, int y_bf16, hipStream_t s);
int gemv_f4_record_bytes(int m, int B);     // LDS bytes of the on-chip records (x_bf16 launches)
size_t x_digits_f6_bytes(int64_t m, int64_t B);
hipError_t launch_x_digits_f6(const void* x, int x_bf16, int m, int B, void* blob, hipStream_t s);
size_t x_digits_bytes(int64_t m, int64_t B);
hipError_t launch_x_digits(const void* x, int x_bf16, int m, int B, void* blob, hipStream_t s);
hipError_t launch_dequant(const uint8_t* packed, const float* scales, int n, int m, int T, void* R,
                          int r_bf16, hipStream_t s);
hipError_t launch_act_quant(const void* x, int x_bf16, int N, int two_m, int8_t* q, float* delta,
                            hipStream_t s);
hipError_t launch_gemm(const uint8_t* packed, const float* scales, int n, int m, int T,
                       const int8_t* q, const float* delta, int N, void* y, int y_mode,
                       hipStream_t s);
}  // namespace f2i
