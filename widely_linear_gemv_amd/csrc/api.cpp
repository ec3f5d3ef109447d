// C ABI of libfairy2i.so: argument checks, status codes, dispatch to the HIP launchers.
// The operations themselves are specified in include/fairy2i.h.
#include "fairy2i.h"

#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>

#include "common.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return FAIRY2I_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(FAIRY2I_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxRows = int64_t(1) << 28;   // complex rows n
constexpr int64_t kMaxCols = int64_t(1) << 22;   // complex columns m
constexpr int64_t kMaxTokens = int64_t(1) << 20;

int check_stages(int T) {
  if (T < 1 || T > 4) return fail(FAIRY2I_ERR_STAGES, "T = %d, must be in [1, 4]", T);
  return FAIRY2I_OK;
}

// The fp4 GEMV's fp32 sums stay exact integers up to 24 m < 2^24.
constexpr int64_t kMaxColsF4 = int64_t(1) << 19;

int check_f4_cols(int kernel, int64_t m) {
  if (kernel == FAIRY2I_GEMV_MFMA_F4 && m > kMaxColsF4)
    return fail(FAIRY2I_ERR_SHAPE, "m = %lld: the fp4 MFMA GEMV takes m <= %lld", (long long)m,
                (long long)kMaxColsF4);
  return FAIRY2I_OK;
}

int check_nm(int64_t n, int64_t m) {
  if (n < 1 || n > kMaxRows) return fail(FAIRY2I_ERR_SHAPE, "n = %lld out of range", (long long)n);
  if (m < 64 || m > kMaxCols || m % 64 != 0)
    return fail(FAIRY2I_ERR_SHAPE, "m = %lld: need m >= 64 and m %% 64 == 0", (long long)m);
  return FAIRY2I_OK;
}

size_t align16(size_t v) { return (v + 15) & ~size_t(15); }

// Kernels with one 256-thread workgroup per row (quantizers, dequantize) address at most
// 2^24 - 1 workgroups per launch (2^32 work-items).
constexpr int64_t kMaxRowLaunch = (int64_t(1) << 24) - 1;
int check_row_launch(int64_t n) {
  if ((n + 15) / 16 * 16 > kMaxRowLaunch)
    return fail(FAIRY2I_ERR_SHAPE, "n = %lld: one launch covers at most %lld rows", (long long)n,
                (long long)(kMaxRowLaunch / 16 * 16));
  return FAIRY2I_OK;
}

}  // namespace

extern "C" {

int fairy2i_abi_version(void) { return FAIRY2I_ABI_VERSION; }

const char* fairy2i_last_error(void) { return g_err; }

const char* fairy2i_status_string(int status) {
  switch (status) {
    case FAIRY2I_OK: return "ok";
    case FAIRY2I_ERR_NULL: return "null pointer";
    case FAIRY2I_ERR_SHAPE: return "bad shape";
    case FAIRY2I_ERR_STAGES: return "bad stage count";
    case FAIRY2I_ERR_DTYPE: return "bad dtype";
    case FAIRY2I_ERR_ALIGN: return "misaligned pointer";
    case FAIRY2I_ERR_WORKSPACE: return "workspace too small";
    case FAIRY2I_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

static int quantize_any(const void* R, int r_bf16, int64_t two_n, int64_t two_m, int T, uint8_t* packed,
                        float* scales, double* scales64, uint8_t* codes, hipStream_t stream) {
  if (!R || !packed || !scales) return fail(FAIRY2I_ERR_NULL, "R, packed and scales are required");
  if (int s = check_stages(T)) return s;
  if (two_n < 2 || two_n % 2 || two_m < 2 || two_m % 2)
    return fail(FAIRY2I_ERR_SHAPE, "R is %lld x %lld; both sizes must be even",
                (long long)two_n, (long long)two_m);
  const int64_t n = two_n / 2, m = two_m / 2;
  if (int s = check_nm(n, m)) return s;
  if (int s = check_row_launch(n)) return s;
  if (2 * T * m > 65536)
    return fail(FAIRY2I_ERR_SHAPE, "2*T*m = %lld exceeds 65536", (long long)(2 * T * m));
  if (!aligned(R, r_bf16 ? 2 : 4) || !aligned(packed, 16) || !aligned(scales, 4) ||
      (scales64 && !aligned(scales64, 8)) || (codes && !aligned(codes, 16)))
    return fail(FAIRY2I_ERR_ALIGN, "R needs 4 (fp32) or 2 (bf16), scales 4, scales64 8, packed/codes 16-byte alignment");
  return hip_status(f2i::launch_quantize(R, r_bf16, (int)n, (int)m, T, packed, scales, scales64, codes, stream),
                    "quantize launch");
}

int fairy2i_quantize(const float* R, int64_t two_n, int64_t two_m, int T, uint8_t* packed,
                     float* scales, double* scales64, uint8_t* codes, hipStream_t stream) {
  return quantize_any(R, 0, two_n, two_m, T, packed, scales, scales64, codes, stream);
}

int fairy2i_quantize_bf16(const uint16_t* R, int64_t two_n, int64_t two_m, int T, uint8_t* packed,
                          float* scales, double* scales64, uint8_t* codes, hipStream_t stream) {
  return quantize_any(R, 1, two_n, two_m, T, packed, scales, scales64, codes, stream);
}

int fairy2i_quantize_grouped(int count, const void* const* R, int R_dtype, int64_t two_n, int64_t two_m, int T,
                             uint8_t* const* packed, float* const* scales, double* const* scales64,
                             uint8_t* const* codes, hipStream_t stream) {
  if (count < 0) return fail(FAIRY2I_ERR_SHAPE, "count = %d", count);
  if (count > 0 && (!R || !packed || !scales)) return fail(FAIRY2I_ERR_NULL, "R, packed and scales arrays are required");
  if (R_dtype != FAIRY2I_F32 && R_dtype != FAIRY2I_BF16)
    return fail(FAIRY2I_ERR_DTYPE, "R_dtype %d: need F32 or BF16", R_dtype);
  if (int s = check_stages(T)) return s;
  if (two_n < 2 || two_n % 2 || two_m < 2 || two_m % 2)
    return fail(FAIRY2I_ERR_SHAPE, "R is %lld x %lld; both sizes must be even",
                (long long)two_n, (long long)two_m);
  const int64_t n = two_n / 2, m = two_m / 2;
  if (int s = check_nm(n, m)) return s;
  if (2 * T * m > 65536)
    return fail(FAIRY2I_ERR_SHAPE, "2*T*m = %lld exceeds 65536", (long long)(2 * T * m));
  const int64_t rows = (n + 15) / 16 * 16;
  if (std::min(count, f2i::kMaxQuantItems) * rows > kMaxRowLaunch)
    return fail(FAIRY2I_ERR_SHAPE, "%d layers of %lld rows exceed one launch's %lld workgroups",
                std::min(count, f2i::kMaxQuantItems), (long long)rows, (long long)kMaxRowLaunch);
  const int bf16 = R_dtype == FAIRY2I_BF16;
  for (int k = 0; k < count; ++k) {
    if (!R[k] || !packed[k] || !scales[k]) return fail(FAIRY2I_ERR_NULL, "layer %d: R, packed and scales are required", k);
    const double* s64 = scales64 ? scales64[k] : nullptr;
    const uint8_t* cd = codes ? codes[k] : nullptr;
    if (!aligned(R[k], bf16 ? 2 : 4) || !aligned(packed[k], 16) || !aligned(scales[k], 4) ||
        (s64 && !aligned(s64, 8)) || (cd && !aligned(cd, 16)))
      return fail(FAIRY2I_ERR_ALIGN, "layer %d: R needs 4 (fp32) or 2 (bf16), scales 4, scales64 8, "
                  "packed/codes 16-byte alignment", k);
  }
  for (int k0 = 0; k0 < count; k0 += f2i::kMaxQuantItems) {
    f2i::QuantGroup grp;
    grp.count = std::min(count - k0, f2i::kMaxQuantItems);
    for (int k = 0; k < grp.count; ++k)
      grp.items[k] = f2i::QuantItem{R[k0 + k], packed[k0 + k], scales[k0 + k],
                                    scales64 ? scales64[k0 + k] : nullptr, codes ? codes[k0 + k] : nullptr};
    if (int s = hip_status(f2i::launch_quantize_group(grp, bf16, (int)n, (int)m, T, stream), "grouped quantize launch"))
      return s;
  }
  return ok();
}

size_t fairy2i_quantize_tensor_workspace_bytes(int64_t n, int64_t m, int T) {
  (void)m;
  (void)T;
  if (n < 1 || n > kMaxRows) return 0;
  return f2i::quantize_tensor_workspace_bytes(n);
}

int fairy2i_quantize_tensor(const void* R, int R_dtype, int64_t two_n, int64_t two_m, int T,
                            void* workspace, size_t workspace_bytes, uint8_t* packed, float* scales,
                            double* scales64, uint8_t* codes, hipStream_t stream) {
  if (!R || !packed || !scales || !workspace)
    return fail(FAIRY2I_ERR_NULL, "R, workspace, packed and scales are required");
  if (R_dtype != FAIRY2I_F32 && R_dtype != FAIRY2I_BF16)
    return fail(FAIRY2I_ERR_DTYPE, "R_dtype %d: need F32 or BF16", R_dtype);
  if (int s = check_stages(T)) return s;
  if (two_n < 2 || two_n % 2 || two_m < 2 || two_m % 2)
    return fail(FAIRY2I_ERR_SHAPE, "R is %lld x %lld; both sizes must be even",
                (long long)two_n, (long long)two_m);
  const int64_t n = two_n / 2, m = two_m / 2;
  if (int s = check_nm(n, m)) return s;
  if (int s = check_row_launch(n)) return s;
  if (2 * m > 65536) return fail(FAIRY2I_ERR_SHAPE, "m = %lld exceeds 32768", (long long)m);
  const size_t need = f2i::quantize_tensor_workspace_bytes(n);
  if (workspace_bytes < need)
    return fail(FAIRY2I_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
  const int bf16 = R_dtype == FAIRY2I_BF16;
  if (!aligned(R, bf16 ? 2 : 4) || !aligned(workspace, 16) || !aligned(packed, 16) || !aligned(scales, 4) ||
      (scales64 && !aligned(scales64, 8)) || (codes && !aligned(codes, 16)))
    return fail(FAIRY2I_ERR_ALIGN, "R needs 4 (fp32) or 2 (bf16), scales 4, scales64 8, workspace/packed/codes 16-byte alignment");
  return hip_status(f2i::launch_quantize_tensor(R, bf16, (int)n, (int)m, T, workspace, packed, scales,
                                                scales64, codes, stream),
                    "per-tensor quantize launch");
}

int fairy2i_pack(const uint8_t* codes, int64_t n, int64_t m, int T, uint8_t* packed,
                 hipStream_t stream) {
  if (!codes || !packed) return fail(FAIRY2I_ERR_NULL, "codes and packed are required");
  if (int s = check_stages(T)) return s;
  if (int s = check_nm(n, m)) return s;
  if (!aligned(codes, 16) || !aligned(packed, 16))
    return fail(FAIRY2I_ERR_ALIGN, "codes and packed need 16-byte alignment");
  return hip_status(f2i::launch_pack(codes, (int)n, (int)m, T, packed, stream), "pack launch");
}

// Checks the dtype / algorithm / batch combination of a GEMV call and resolves AUTO and MFMA to
// the kernel that runs.  Returns minus the status (with the message recorded) on a bad combination.
// The fp4 GEMV on bf16 x builds each row's digit records in LDS (fp4, 16 bytes per record): at
// most 32 chunks of 256 columns over the batch entries (64 KB).  AUTO takes it for launches of at
// least kF4FusedMinTiles tiles, whose workgroups stay resident and build the records once for many
// tiles (those workgroups need one x for the launch).  In smaller launches at batch 1 each wave
// builds the records of its own chunks only; per launch, 32 distinct T = 2 layers in a graph,
// bf16 / fp4 us: m = 2048 16 tiles 5.08 / 5.00, 256 tiles 5.94 / 4.77, 1535 tiles 21.06 / 14.76;
// m = 4096, 5504 and 8192 faster at every size (8192, 1535 tiles: 58.76 / 44.35); m = 1024 16 tiles
// 3.85 / 4.09, 64 tiles 4.11 / 4.11, 128 tiles 4.23 / 4.18, 1535 tiles 12.56 / 10.84; m = 512
// slower up to 128 tiles and at 1535.  At batch 2 the per-tile build and the second batch entry's
// operands make it slower than bf16 at every small size measured (m = 512 to 4096, 16 to 1535
// tiles).
constexpr int kMaxF4FusedColumns = 8192;
constexpr int64_t kF4FusedMinTiles = 1536;
constexpr int64_t kF4FusedSmallMinM = 2048;          // any launch size from here
constexpr int64_t kF4FusedShortMinM = 1024;          // and from kF4FusedShortMinTiles tiles from here
constexpr int64_t kF4FusedShortMinTiles = 128;
static bool f4_records_fit(int64_t m, int64_t B) { return m * B <= kMaxF4FusedColumns; }
static bool f4_fused_small_wins(int64_t B, int64_t m, int64_t tiles) {
  return B == 1 && (m >= kF4FusedSmallMinM || (m >= kF4FusedShortMinM && tiles >= kF4FusedShortMinTiles));
}

// At batch 3-4 the fp4 kernel on x split into two fp8 parts beats the bf16 kernel on large
// launches (1 GiB pools, bf16 / fp4 x fp8 us: 4096 x 4096 at B = 3 337.7 / 262.9, B = 4 316.4 /
// 247.2; 11008 x 4096 B = 4 301.6 / 252.4; 4096 x 11008 B = 4 289.1 / 250.5); at B = 8 the two are
// within 3 % either way and at B = 16 it takes twice as long (its four column groups need four-wave
// workgroups); in the decode step's small launches (4-23 MB) its eight-tile workgroups leave most
// of the chip idle (B = 8: 18.9 against 11.4 us per q/k/v launch).
constexpr int64_t kF4x8MinTiles = 1536;
constexpr int64_t kF4x8MaxM = int64_t(1) << 19;
static bool f4x8_wins(int64_t B, int64_t m, int64_t tiles) {
  return B >= 3 && B <= 4 && tiles >= kF4x8MinTiles && m <= kF4x8MaxM;
}

static int gemv_kernel(int x_dtype, int y_dtype, int algo, int64_t B, int64_t m, int64_t tiles = 0,
                       bool shared_x = true) {
  if (x_dtype != FAIRY2I_F32 && x_dtype != FAIRY2I_BF16 && x_dtype != FAIRY2I_X_DIGITS &&
      x_dtype != FAIRY2I_X_DIGITS_F6)
    return -fail(FAIRY2I_ERR_DTYPE, "x_dtype %d: need F32, BF16, X_DIGITS or X_DIGITS_F6", x_dtype);
  if (y_dtype != FAIRY2I_F32 && y_dtype != FAIRY2I_BF16)
    return -fail(FAIRY2I_ERR_DTYPE, "y_dtype %d: need F32 or BF16", y_dtype);
  if (algo < FAIRY2I_GEMV_AUTO || algo > FAIRY2I_GEMV_MFMA_F4)
    return -fail(FAIRY2I_ERR_DTYPE, "unknown GEMV algorithm %d", algo);
  if (B < 1 || B > 16) return -fail(FAIRY2I_ERR_SHAPE, "B = %lld: need 1 <= B <= 16", (long long)B);
  int kernel = algo;
  if (kernel == FAIRY2I_GEMV_AUTO)
    kernel = x_dtype == FAIRY2I_X_DIGITS    ? FAIRY2I_GEMV_MFMA_I8
           : x_dtype == FAIRY2I_X_DIGITS_F6 ? FAIRY2I_GEMV_MFMA_F4
           : x_dtype == FAIRY2I_BF16        ? ((B <= 2 && f4_records_fit(m, B) &&
                                                        (tiles >= kF4FusedMinTiles ? shared_x
                                                                                   : f4_fused_small_wins(B, m, tiles))) ||
                                                       f4x8_wins(B, m, tiles)
                                                   ? FAIRY2I_GEMV_MFMA_F4 : FAIRY2I_GEMV_MFMA_BF16)
                                            : FAIRY2I_GEMV_VALU;
  if (kernel == FAIRY2I_GEMV_MFMA) kernel = FAIRY2I_GEMV_MFMA_BF16;
  if (kernel == FAIRY2I_GEMV_MFMA_I8) {
    if (x_dtype != FAIRY2I_X_DIGITS)
      return -fail(FAIRY2I_ERR_DTYPE, "the int8 MFMA GEMV takes x in digit form (fairy2i_x_digits)");
    if (B > 2) return -fail(FAIRY2I_ERR_SHAPE, "B = %lld: the int8 MFMA GEMV takes B <= 2", (long long)B);
  } else if (kernel == FAIRY2I_GEMV_MFMA_F4) {
    if (x_dtype != FAIRY2I_X_DIGITS_F6 && x_dtype != FAIRY2I_BF16)
      return -fail(FAIRY2I_ERR_DTYPE, "the fp4 MFMA GEMV takes bf16 x or x in fp6 digit form (fairy2i_x_digits_f6)");
    if (B > 2 && x_dtype != FAIRY2I_BF16)
      return -fail(FAIRY2I_ERR_SHAPE, "B = %lld: the fp4 MFMA GEMV on a digit form takes B <= 2 (bf16 x: B <= 16)",
                   (long long)B);
    if (x_dtype == FAIRY2I_BF16 && B <= 2 && m > 0 && !f4_records_fit(m, B))
      return -fail(FAIRY2I_ERR_SHAPE, "m = %lld, B = %lld: the fp4 MFMA GEMV on bf16 x takes m * B <= %d "
                   "(its digit records are built in LDS); make the digit form with fairy2i_x_digits_f6",
                   (long long)m, (long long)B, kMaxF4FusedColumns);
    if (x_dtype == FAIRY2I_BF16 && B <= 2 && !shared_x && tiles >= kF4FusedMinTiles)
      return -fail(FAIRY2I_ERR_SHAPE, "the fp4 MFMA GEMV on bf16 x needs one x for every item of a launch of "
                   "%lld tiles or more (give the items' x as one digit form, or use the bf16 kernel)",
                   (long long)kF4FusedMinTiles);
  } else if (x_dtype == FAIRY2I_X_DIGITS) {
    return -fail(FAIRY2I_ERR_DTYPE, "x in digit form needs the int8 MFMA GEMV");
  } else if (x_dtype == FAIRY2I_X_DIGITS_F6) {
    return -fail(FAIRY2I_ERR_DTYPE, "x in fp6 digit form needs the fp4 MFMA GEMV");
  } else if (kernel == FAIRY2I_GEMV_MFMA_BF16 && x_dtype != FAIRY2I_BF16) {
    return -fail(FAIRY2I_ERR_DTYPE, "the bf16 MFMA GEMV takes bf16 x only");
  }
  return kernel;
}

size_t fairy2i_packed_bytes(int64_t n, int64_t m, int T) {
  if (n < 1 || m < 1 || T < 1) return 0;
  return (size_t)((n + 15) / 16) * 16 * (size_t)T * 2 * (size_t)(m / 4);
}

size_t fairy2i_x_digits_bytes(int64_t m, int64_t B) {
  if (m < 1 || B < 1) return 0;
  return f2i::x_digits_bytes(m, B);
}

int fairy2i_x_digits(const void* x, int x_dtype, int64_t m, int64_t B, void* digits, hipStream_t stream) {
  if (!x || !digits) return fail(FAIRY2I_ERR_NULL, "x and digits are required");
  if (x_dtype != FAIRY2I_F32 && x_dtype != FAIRY2I_BF16)
    return fail(FAIRY2I_ERR_DTYPE, "x_dtype %d: need F32 or BF16", x_dtype);
  if (m < 64 || m > kMaxCols || m % 64 != 0)
    return fail(FAIRY2I_ERR_SHAPE, "m = %lld: need m >= 64 and m %% 64 == 0", (long long)m);
  if (B < 1 || B > 2) return fail(FAIRY2I_ERR_SHAPE, "B = %lld: the digit form takes 1 <= B <= 2", (long long)B);
  if (!aligned(x, 16) || !aligned(digits, 16))
    return fail(FAIRY2I_ERR_ALIGN, "x and digits need 16-byte alignment");
  return hip_status(f2i::launch_x_digits(x, x_dtype == FAIRY2I_BF16, (int)m, (int)B, digits, stream),
                    "x digits launch");
}

size_t fairy2i_x_digits_f6_bytes(int64_t m, int64_t B) {
  if (m < 1 || B < 1) return 0;
  return f2i::x_digits_f6_bytes(m, B);
}

int fairy2i_x_digits_f6(const void* x, int x_dtype, int64_t m, int64_t B, void* digits, hipStream_t stream) {
  if (!x || !digits) return fail(FAIRY2I_ERR_NULL, "x and digits are required");
  if (x_dtype != FAIRY2I_F32 && x_dtype != FAIRY2I_BF16)
    return fail(FAIRY2I_ERR_DTYPE, "x_dtype %d: need F32 or BF16", x_dtype);
  if (m < 64 || m > kMaxCols || m % 64 != 0)
    return fail(FAIRY2I_ERR_SHAPE, "m = %lld: need m >= 64 and m %% 64 == 0", (long long)m);
  if (B < 1 || B > 2) return fail(FAIRY2I_ERR_SHAPE, "B = %lld: the fp6 digit form takes 1 <= B <= 2", (long long)B);
  if (!aligned(x, 16) || !aligned(digits, 16))
    return fail(FAIRY2I_ERR_ALIGN, "x and digits need 16-byte alignment");
  return hip_status(f2i::launch_x_digits_f6(x, x_dtype == FAIRY2I_BF16, (int)m, (int)B, digits, stream),
                    "x fp6 digits launch");
}

// The fp4 matrix-core GEMVs: batch 1-2 on a digit form or bf16 x (launch_gemv_f4_group); batch 3-16
// on bf16 x split into fp8 parts (launch_gemv_f8x_group).
static hipError_t launch_f4_family(const f2i::GemvGroup& grp, int64_t m, int T, int64_t B, int ybf, int x_dtype,
                                   hipStream_t stream) {
  if (B > 2) return f2i::launch_gemv_f8x_group(grp, (int)m, T, (int)B, ybf, stream);
  return f2i::launch_gemv_f4_group(grp, (int)m, T, (int)B, ybf, x_dtype == FAIRY2I_BF16, stream);
}

int fairy2i_gemv(const uint8_t* packed, const float* scales, int64_t n, int64_t m, int T,
                 const void* x, int x_dtype, int64_t B, void* y, int y_dtype, int algo,
                 hipStream_t stream) {
  if (!packed || !scales || !x || !y) return fail(FAIRY2I_ERR_NULL, "packed, scales, x and y are required");
  const int kernel = gemv_kernel(x_dtype, y_dtype, algo, B, m, (n + 15) / 16);
  if (kernel < 0) return -kernel;
  if (int s = check_stages(T)) return s;
  if (int s = check_nm(n, m)) return s;
  if (int s = check_f4_cols(kernel, m)) return s;
  if (!aligned(packed, 16) || !aligned(x, 16) || !aligned(y, 16) || !aligned(scales, 4))
    return fail(FAIRY2I_ERR_ALIGN, "packed, x and y need 16-byte alignment, scales 4");
  if (kernel == FAIRY2I_GEMV_MFMA_F4 && B > 2) {
    f2i::GemvGroup grp;
    grp.count = 1;
    grp.tile_start[0] = 0;
    grp.tile_start[1] = (int)((n + 15) / 16);
    grp.items[0] = f2i::GemvItem{packed, scales, x, y, (int)n};
    return hip_status(launch_f4_family(grp, m, T, B, y_dtype == FAIRY2I_BF16, x_dtype, stream),
                      "gemv (fp4 x fp8 mfma) launch");
  }
  if (kernel == FAIRY2I_GEMV_MFMA_F4)
    return hip_status(f2i::launch_gemv_f4(packed, scales, (int)n, (int)m, T, x, (int)B, y,
                                          y_dtype == FAIRY2I_BF16, x_dtype == FAIRY2I_BF16, stream),
                      "gemv (fp4 mfma) launch");
  if (kernel == FAIRY2I_GEMV_MFMA_I8)
    return hip_status(f2i::launch_gemv_i8(packed, scales, (int)n, (int)m, T, x, (int)B, y,
                                          y_dtype == FAIRY2I_BF16, stream),
                      "gemv (int8 mfma) launch");
  if (kernel == FAIRY2I_GEMV_MFMA_BF16)
    return hip_status(f2i::launch_gemv_mfma(packed, scales, (int)n, (int)m, T, x, (int)B, y,
                                            y_dtype == FAIRY2I_BF16, nullptr, stream),
                      "gemv (bf16 mfma) launch");
  return hip_status(f2i::launch_gemv_valu(packed, scales, (int)n, (int)m, T, x,
                                          x_dtype == FAIRY2I_BF16, (int)B, y,
                                          y_dtype == FAIRY2I_BF16, stream),
                    "gemv (valu) launch");
}

int fairy2i_gemv_grouped(const fairy2i_gemv_item* items, int count, int64_t m, int T, int x_dtype,
                         int64_t B, int y_dtype, int algo, hipStream_t stream) {
  if (!items) return fail(FAIRY2I_ERR_NULL, "items is required");
  if (count < 1) return fail(FAIRY2I_ERR_SHAPE, "count = %d: need at least one item", count);
  for (int k = 0; k < count; ++k)
    if (!items[k].packed || !items[k].scales || !items[k].x || !items[k].y)
      return fail(FAIRY2I_ERR_NULL, "item %d: packed, scales, x and y are required", k);
  int64_t all_tiles = 0;
  bool shared_x = true;
  for (int k = 0; k < count; ++k) {
    all_tiles += (items[k].n + 15) / 16;
    shared_x = shared_x && items[k].x == items[0].x;
  }
  const int kernel = gemv_kernel(x_dtype, y_dtype, algo, B, m, all_tiles, shared_x);
  if (kernel < 0) return -kernel;
  if (int s = check_stages(T)) return s;
  for (int k = 0; k < count; ++k)
    if (int s = check_nm(items[k].n, m)) return s;
  if (int s = check_f4_cols(kernel, m)) return s;
  for (int k = 0; k < count; ++k)
    if (!aligned(items[k].packed, 16) || !aligned(items[k].x, 16) || !aligned(items[k].y, 16) ||
        !aligned(items[k].scales, 4))
      return fail(FAIRY2I_ERR_ALIGN, "item %d: packed, x and y need 16-byte alignment, scales 4", k);
  if (kernel == FAIRY2I_GEMV_VALU) {
    for (int k = 0; k < count; ++k) {
      const fairy2i_gemv_item& it = items[k];
      int s = fairy2i_gemv(it.packed, it.scales, it.n, m, T, it.x, x_dtype, B, it.y, y_dtype, algo, stream);
      if (s != FAIRY2I_OK) return s;
    }
    return ok();
  }
  for (int k0 = 0; k0 < count; k0 += f2i::kMaxGroup) {
    f2i::GemvGroup grp;
    grp.count = count - k0 < f2i::kMaxGroup ? count - k0 : f2i::kMaxGroup;
    int tiles = 0;
    for (int k = 0; k < grp.count; ++k) {
      const fairy2i_gemv_item& it = items[k0 + k];
      grp.tile_start[k] = tiles;
      grp.items[k] = f2i::GemvItem{it.packed, it.scales, it.x, it.y, (int)it.n};
      tiles += (int)((it.n + 15) / 16);
    }
    grp.tile_start[grp.count] = tiles;
    const int ybf = y_dtype == FAIRY2I_BF16;
    hipError_t e = kernel == FAIRY2I_GEMV_MFMA_F4
                       ? launch_f4_family(grp, m, T, B, ybf, x_dtype, stream)
                 : kernel == FAIRY2I_GEMV_MFMA_I8 ? f2i::launch_gemv_i8_group(grp, (int)m, T, (int)B, ybf, stream)
                 : f2i::launch_gemv_mfma_group(grp, (int)m, T, (int)B, ybf, stream);
    if (e != hipSuccess) return hip_status(e, "gemv (grouped mfma) launch");
  }
  return ok();
}

int fairy2i_gemv_strided(const uint8_t* packed, int64_t packed_stride, const float* scales,
                         int64_t scales_stride, int64_t n, int64_t m, int T, const void* x,
                         int x_dtype, int64_t B, void* y, int64_t y_stride, int y_dtype,
                         int64_t batch, int algo, hipStream_t stream) {
  if (!packed || !scales || !x || !y) return fail(FAIRY2I_ERR_NULL, "packed, scales, x and y are required");
  const int kernel = gemv_kernel(x_dtype, y_dtype, algo, B, m, batch > 0 && n > 0 ? batch * ((n + 15) / 16) : 0);
  if (kernel < 0) return -kernel;
  if (int s = check_stages(T)) return s;
  if (int s = check_nm(n, m)) return s;
  if (int s = check_f4_cols(kernel, m)) return s;
  const int64_t tiles = (n + 15) / 16;
  if (batch < 1 || batch > (int64_t(1) << 30) / tiles)
    return fail(FAIRY2I_ERR_SHAPE, "batch = %lld: need 1 <= batch and batch * ceil(n/16) <= 2^30", (long long)batch);
  const int64_t y_elem = y_dtype == FAIRY2I_BF16 ? 2 : 4;
  if (packed_stride < 0 || scales_stride < 0 || y_stride < 0)
    return fail(FAIRY2I_ERR_SHAPE, "strides must be >= 0");
  if (batch > 1 && y_stride < 2 * n * B)
    return fail(FAIRY2I_ERR_SHAPE, "y_stride = %lld: outputs of different matrices overlap (need >= 2nB = %lld)",
                (long long)y_stride, (long long)(2 * n * B));
  if (!aligned(packed, 16) || !aligned(x, 16) || !aligned(y, 16) || !aligned(scales, 4) ||
      packed_stride % 16 != 0 || (y_stride * y_elem) % 16 != 0)
    return fail(FAIRY2I_ERR_ALIGN, "packed, x and y (and their strides) need 16-byte alignment, scales 4");
  if (kernel == FAIRY2I_GEMV_VALU) {
    for (int64_t k = 0; k < batch; ++k) {
      int s = fairy2i_gemv(packed + k * packed_stride, scales + k * scales_stride, n, m, T, x, x_dtype, B,
                           static_cast<uint8_t*>(y) + k * y_stride * y_elem, y_dtype, algo, stream);
      if (s != FAIRY2I_OK) return s;
    }
    return ok();
  }
  f2i::GemvGroup grp;
  grp.count = 1;
  grp.tile_start[0] = 0;
  grp.tile_start[1] = (int)tiles;
  grp.items[0] = f2i::GemvItem{packed, scales, x, y, (int)n};
  grp.batch = (int)batch;
  grp.tiles_per_item = (int)tiles;
  grp.packed_stride = packed_stride;
  grp.scales_stride = scales_stride;
  grp.y_stride = y_stride;
  const int ybf = y_dtype == FAIRY2I_BF16;
  hipError_t e = kernel == FAIRY2I_GEMV_MFMA_F4
                     ? launch_f4_family(grp, m, T, B, ybf, x_dtype, stream)
               : kernel == FAIRY2I_GEMV_MFMA_I8 ? f2i::launch_gemv_i8_group(grp, (int)m, T, (int)B, ybf, stream)
               : f2i::launch_gemv_mfma_group(grp, (int)m, T, (int)B, ybf, stream);
  return hip_status(e, "gemv (strided batch) launch");
}

int fairy2i_dequantize(const uint8_t* packed, const float* scales, int64_t n, int64_t m, int T,
                       void* R, int R_dtype, hipStream_t stream) {
  if (!packed || !scales || !R) return fail(FAIRY2I_ERR_NULL, "packed, scales and R are required");
  if (R_dtype != FAIRY2I_F32 && R_dtype != FAIRY2I_BF16)
    return fail(FAIRY2I_ERR_DTYPE, "R_dtype %d: need F32 or BF16", R_dtype);
  if (int s = check_stages(T)) return s;
  if (int s = check_nm(n, m)) return s;
  if (int s = check_row_launch(n)) return s;
  if (!aligned(packed, 16) || !aligned(R, 16) || !aligned(scales, 4))
    return fail(FAIRY2I_ERR_ALIGN, "packed and R need 16-byte alignment, scales 4");
  return hip_status(f2i::launch_dequant(packed, scales, (int)n, (int)m, T, R, R_dtype == FAIRY2I_BF16, stream),
                    "dequantize launch");
}

int fairy2i_act_quant(const void* x, int x_dtype, int64_t N, int64_t two_m, int8_t* q,
                      float* delta, hipStream_t stream) {
  if (!x || !q || !delta) return fail(FAIRY2I_ERR_NULL, "x, q and delta are required");
  if (x_dtype != FAIRY2I_F32 && x_dtype != FAIRY2I_BF16)
    return fail(FAIRY2I_ERR_DTYPE, "x_dtype %d: need F32 or BF16", x_dtype);
  if (N < 1 || N > kMaxTokens) return fail(FAIRY2I_ERR_SHAPE, "N = %lld out of range", (long long)N);
  if (two_m < 8 || two_m % 8 || two_m > 2 * kMaxCols)
    return fail(FAIRY2I_ERR_SHAPE, "row length %lld: need a positive multiple of 8", (long long)two_m);
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(delta, 4))
    return fail(FAIRY2I_ERR_ALIGN, "x and q need 16-byte alignment, delta 4");
  return hip_status(f2i::launch_act_quant(x, x_dtype == FAIRY2I_BF16, (int)N, (int)two_m, q, delta, stream),
                    "act_quant launch");
}

size_t fairy2i_gemm_workspace_bytes(int64_t n, int64_t m, int T, int64_t N, int x_dtype) {
  (void)n;
  (void)T;
  if (x_dtype == FAIRY2I_I8 || N < 1 || m < 1) return 0;
  return align16((size_t)N * 2 * (size_t)m) + align16((size_t)N * 4);
}

}  // extern "C"

// Argument checks of the prefill GEMM (null -> dtype -> stages -> shape -> alignment), shared by
// fairy2i_gemm and fairy2i_gemm_noalloc.
static int check_gemm(const uint8_t* packed, const float* scales, int64_t n, int64_t m, int T, const void* x,
                      int x_dtype, const float* x_scale, int64_t N, const void* y, int y_dtype) {
  if (!packed || !scales || !x || !y) return fail(FAIRY2I_ERR_NULL, "packed, scales, x and y are required");
  if (x_dtype == FAIRY2I_I8 && !x_scale)
    return fail(FAIRY2I_ERR_NULL, "x_scale (delta) is required with int8 x");
  if (x_dtype != FAIRY2I_F32 && x_dtype != FAIRY2I_BF16 && x_dtype != FAIRY2I_I8)
    return fail(FAIRY2I_ERR_DTYPE, "x_dtype %d: need F32, BF16 or I8", x_dtype);
  if (y_dtype != FAIRY2I_F32 && y_dtype != FAIRY2I_BF16 && y_dtype != FAIRY2I_I32)
    return fail(FAIRY2I_ERR_DTYPE, "y_dtype %d: need F32, BF16 or I32", y_dtype);
  if (int s = check_stages(T)) return s;
  if (int s = check_nm(n, m)) return s;
  if (N < 1 || N > kMaxTokens) return fail(FAIRY2I_ERR_SHAPE, "N = %lld out of range", (long long)N);
  if (!aligned(packed, 16) || !aligned(x, 16) || !aligned(y, 16) || !aligned(scales, 4) ||
      (x_scale && !aligned(x_scale, 4)))
    return fail(FAIRY2I_ERR_ALIGN, "packed, x, y, workspace need 16-byte alignment; scales, x_scale 4");
  return FAIRY2I_OK;
}

// The prefill GEMM's launches, with the activation workspace (int8 q, then delta) at `workspace`.
static int gemm_launch(const uint8_t* packed, const float* scales, int64_t n, int64_t m, int T, const void* x,
                       int x_dtype, float* x_scale, int64_t N, void* y, int y_dtype, void* workspace,
                       hipStream_t stream) {
  const int8_t* q = static_cast<const int8_t*>(x);
  const float* delta = x_scale;
  if (x_dtype != FAIRY2I_I8) {
    int8_t* qw = static_cast<int8_t*>(workspace);
    float* dw = x_scale ? x_scale
                        : reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                                   align16((size_t)N * 2 * (size_t)m));
    hipError_t e = f2i::launch_act_quant(x, x_dtype == FAIRY2I_BF16, (int)N, (int)(2 * m), qw, dw, stream);
    if (e != hipSuccess) return hip_status(e, "act_quant launch");
    q = qw;
    delta = dw;
  }
  const int mode = y_dtype == FAIRY2I_F32 ? 0 : (y_dtype == FAIRY2I_BF16 ? 1 : 2);
  return hip_status(f2i::launch_gemm(packed, scales, (int)n, (int)m, T, q, delta, (int)N, y, mode, stream),
                    "gemm launch");
}

// ---- the entry point that allocates nothing: its activation workspace is a static device array ----
//
// `scratch` is one array per GPU, reserved when the library's code object is loaded on that GPU and
// held until the process ends.  In host code its name stands for no device address: the address
// on the current device comes from hipGetSymbolAddress, taken once per device on the entry point's
// first call there and kept in g_scratch_ptr.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (looked up once per device).
int scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FAIRY2I_ERR_HIP, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(FAIRY2I_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FAIRY2I_OK;
}
}  // namespace

extern "C" {

size_t fairy2i_gemm_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

int fairy2i_gemm_noalloc(const uint8_t* packed, const float* scales, int64_t n, int64_t m, int T,
                         const void* x, int x_dtype, float* x_scale, int64_t N, void* y, int y_dtype,
                         hipStream_t stream) {
  if (int s = check_gemm(packed, scales, n, m, T, x, x_dtype, x_scale, N, y, y_dtype)) return s;
  const size_t need = fairy2i_gemm_workspace_bytes(n, m, T, N, x_dtype);
  if (need > kNoAllocScratchBytes)
    return fail(FAIRY2I_ERR_WORKSPACE,
                "N = %lld tokens of 2m = %lld need %zu bytes of activation workspace; the static scratch "
                "holds %zu (use fairy2i_gemm with a caller workspace)",
                (long long)N, (long long)(2 * m), need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    if (int s = scratch_on_current_device(&ws)) return s;
  }
  return gemm_launch(packed, scales, n, m, T, x, x_dtype, x_scale, N, y, y_dtype, ws, stream);
}

int fairy2i_gemm(const uint8_t* packed, const float* scales, int64_t n, int64_t m, int T,
                 const void* x, int x_dtype, float* x_scale, int64_t N, void* y, int y_dtype,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (int s = check_gemm(packed, scales, n, m, T, x, x_dtype, x_scale, N, y, y_dtype)) return s;
  if (workspace && !aligned(workspace, 16))
    return fail(FAIRY2I_ERR_ALIGN, "packed, x, y, workspace need 16-byte alignment; scales, x_scale 4");
  const size_t need = fairy2i_gemm_workspace_bytes(n, m, T, N, x_dtype);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(FAIRY2I_ERR_WORKSPACE, "GEMM needs %zu workspace bytes, got %zu", need,
                workspace ? workspace_bytes : size_t(0));
  return gemm_launch(packed, scales, n, m, T, x, x_dtype, x_scale, N, y, y_dtype, workspace, stream);
}

}  // extern "C"
