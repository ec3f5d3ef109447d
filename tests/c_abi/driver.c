/* The widely-linear path driven through the C ABI alone: plain C, the HIP runtime for device
 * memory, no Python and no torch.  Quantizes a layer, runs the decode GEMV on the VALU kernel
 * (fp32 x) and on the fp4 kernel (x in fp6 digit form, made by the library), and the prefill
 * GEMM with raw int32 output; checks a few documented argument errors.  Inputs and outputs are
 * raw little-endian files in one directory, so a test can compare them with its own reference.
 *
 *   fairy2i_c_driver DIR two_n two_m T B N
 *     in:  DIR/R.f32 [two_n][two_m]   DIR/x.f32 [B][two_m]   DIR/xp.f32 [N][two_m]
 *     out: DIR/packed.u8  DIR/scales.f32  DIR/scales64.f64  DIR/y_valu.f32  DIR/y_f4.f32
 *          DIR/p.i32 (GEMM accumulators [T][2][2][2][N][n])  DIR/delta.f32 [N]
 * Prints "ok" and exits 0 when every call returned FAIRY2I_OK (and every error check its
 * documented status); otherwise prints the failing call and the library's message. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fairy2i.h"

static int failed = 0;

#define CHECK_HIP(call)                                                                  \
  do {                                                                                   \
    hipError_t e_ = (call);                                                              \
    if (e_ != hipSuccess) {                                                              \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                         \
      exit(3);                                                                           \
    }                                                                                    \
  } while (0)

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: status %d (%s), expected %d: %s\n", what, got, fairy2i_status_string(got), want,
            fairy2i_last_error());
    failed = 1;
  }
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(2); }
  void* buf = malloc(bytes);
  if (!buf || fread(buf, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(2); }
  fclose(f);
  return buf;
}

static void write_file(const char* dir, const char* name, const void* buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(buf, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(2); }
  fclose(f);
}

/* device buffer of `bytes`, filled from host memory when src is not NULL */
static void* to_device(const void* src, size_t bytes) {
  void* d = NULL;
  CHECK_HIP(hipMalloc(&d, bytes));
  if (src) CHECK_HIP(hipMemcpy(d, src, bytes, hipMemcpyHostToDevice));
  return d;
}

static void fetch(const char* dir, const char* name, const void* dev, size_t bytes) {
  void* h = malloc(bytes);
  if (!h) exit(2);
  CHECK_HIP(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost));
  write_file(dir, name, h, bytes);
  free(h);
}

/* two device buffers hold the same bytes */
static void same_bytes(const void* a, const void* b, size_t bytes, const char* what) {
  void* ha = malloc(bytes);
  void* hb = malloc(bytes);
  if (!ha || !hb) exit(2);
  CHECK_HIP(hipMemcpy(ha, a, bytes, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hb, b, bytes, hipMemcpyDeviceToHost));
  if (memcmp(ha, hb, bytes) != 0) {
    fprintf(stderr, "%s: bytes differ\n", what);
    failed = 1;
  }
  free(ha);
  free(hb);
}

int main(int argc, char** argv) {
  if (argc != 7) {
    fprintf(stderr, "usage: %s DIR two_n two_m T B N\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  const int64_t two_n = atoll(argv[2]), two_m = atoll(argv[3]);
  const int T = atoi(argv[4]);
  const int64_t B = atoll(argv[5]), N = atoll(argv[6]);
  const int64_t n = two_n / 2, m = two_m / 2;
  if (fairy2i_abi_version() != 7) { fprintf(stderr, "ABI version %d\n", fairy2i_abi_version()); return 2; }

  const size_t r_bytes = (size_t)(two_n * two_m) * sizeof(float);
  const size_t x_bytes = (size_t)(B * two_m) * sizeof(float);
  const size_t xp_bytes = (size_t)(N * two_m) * sizeof(float);
  const size_t packed_bytes = fairy2i_packed_bytes(n, m, T);
  const size_t nscale = (size_t)(n * T * 4);
  const size_t y_bytes = (size_t)(B * two_n) * sizeof(float);
  const size_t p_bytes = (size_t)T * 8 * (size_t)N * (size_t)n * sizeof(int32_t);

  float* hR = (float*)read_file(dir, "R.f32", r_bytes);
  float* hx = (float*)read_file(dir, "x.f32", x_bytes);
  float* hxp = (float*)read_file(dir, "xp.f32", xp_bytes);
  void* R = to_device(hR, r_bytes);
  void* x = to_device(hx, x_bytes);
  void* xp = to_device(hxp, xp_bytes);
  void* packed = to_device(NULL, packed_bytes);
  void* scales = to_device(NULL, nscale * sizeof(float));
  void* scales64 = to_device(NULL, nscale * sizeof(double));
  void* y_valu = to_device(NULL, y_bytes);
  void* y_f4 = to_device(NULL, y_bytes);
  const size_t dig_bytes = fairy2i_x_digits_f6_bytes(m, B);
  void* digits = to_device(NULL, dig_bytes);
  void* p = to_device(NULL, p_bytes);
  void* delta = to_device(NULL, (size_t)N * sizeof(float));
  const size_t ws_bytes = fairy2i_gemm_workspace_bytes(n, m, T, N, FAIRY2I_F32);
  void* ws = ws_bytes ? to_device(NULL, ws_bytes) : NULL;
  hipStream_t s;
  CHECK_HIP(hipStreamCreate(&s));

  expect(fairy2i_quantize((const float*)R, two_n, two_m, T, (uint8_t*)packed, (float*)scales, (double*)scales64,
                          NULL, s), FAIRY2I_OK, "fairy2i_quantize");
  /* the same layer twice through the grouped call: both copies equal the single call */
  const void* g_R[2] = {R, R};
  uint8_t* g_packed[2] = {(uint8_t*)to_device(NULL, packed_bytes), (uint8_t*)to_device(NULL, packed_bytes)};
  float* g_scales[2] = {(float*)to_device(NULL, nscale * sizeof(float)), (float*)to_device(NULL, nscale * sizeof(float))};
  double* g_scales64[2] = {(double*)to_device(NULL, nscale * sizeof(double)), NULL};
  expect(fairy2i_quantize_grouped(2, g_R, FAIRY2I_F32, two_n, two_m, T, g_packed, g_scales, g_scales64, NULL, s),
         FAIRY2I_OK, "fairy2i_quantize_grouped");
  expect(fairy2i_gemv((const uint8_t*)packed, (const float*)scales, n, m, T, x, FAIRY2I_F32, B, y_valu, FAIRY2I_F32,
                      FAIRY2I_GEMV_VALU, s), FAIRY2I_OK, "fairy2i_gemv (VALU)");
  if (B <= 2) {
    expect(fairy2i_x_digits_f6(x, FAIRY2I_F32, m, B, digits, s), FAIRY2I_OK, "fairy2i_x_digits_f6");
    expect(fairy2i_gemv((const uint8_t*)packed, (const float*)scales, n, m, T, digits, FAIRY2I_X_DIGITS_F6, B, y_f4,
                        FAIRY2I_F32, FAIRY2I_GEMV_MFMA_F4, s), FAIRY2I_OK, "fairy2i_gemv (fp4)");
  }
  expect(fairy2i_gemm((const uint8_t*)packed, (const float*)scales, n, m, T, xp, FAIRY2I_F32, (float*)delta, N, p,
                      FAIRY2I_I32, ws, ws_bytes, s), FAIRY2I_OK, "fairy2i_gemm (int32)");

  /* documented argument errors: checked on the host, nothing is launched */
  expect(fairy2i_gemv(NULL, (const float*)scales, n, m, T, x, FAIRY2I_F32, B, y_valu, FAIRY2I_F32,
                      FAIRY2I_GEMV_VALU, s), FAIRY2I_ERR_NULL, "null packed");
  expect(fairy2i_gemv((const uint8_t*)packed, (const float*)scales, n, m, 5, x, FAIRY2I_F32, B, y_valu, FAIRY2I_F32,
                      FAIRY2I_GEMV_VALU, s), FAIRY2I_ERR_STAGES, "T = 5");
  expect(fairy2i_gemv((const uint8_t*)packed, (const float*)scales, n, m + 1, T, x, FAIRY2I_F32, B, y_valu,
                      FAIRY2I_F32, FAIRY2I_GEMV_VALU, s), FAIRY2I_ERR_SHAPE, "m not a multiple of 64");
  expect(fairy2i_gemv((const uint8_t*)packed, (const float*)scales, n, m, T, x, FAIRY2I_F32, B, y_valu, FAIRY2I_F32,
                      FAIRY2I_GEMV_MFMA_BF16, s), FAIRY2I_ERR_DTYPE, "bf16 kernel on fp32 x");

  CHECK_HIP(hipStreamSynchronize(s));
  for (int k = 0; k < 2; ++k) {
    same_bytes(g_packed[k], packed, packed_bytes, "grouped quantize: packed");
    same_bytes(g_scales[k], scales, nscale * sizeof(float), "grouped quantize: scales");
  }
  same_bytes(g_scales64[0], scales64, nscale * sizeof(double), "grouped quantize: scales64");
  fetch(dir, "packed.u8", packed, packed_bytes);
  fetch(dir, "scales.f32", scales, nscale * sizeof(float));
  fetch(dir, "scales64.f64", scales64, nscale * sizeof(double));
  fetch(dir, "y_valu.f32", y_valu, y_bytes);
  if (B <= 2) fetch(dir, "y_f4.f32", y_f4, y_bytes);
  fetch(dir, "p.i32", p, p_bytes);
  fetch(dir, "delta.f32", delta, (size_t)N * sizeof(float));

  CHECK_HIP(hipStreamDestroy(s));
  hipFree(R); hipFree(x); hipFree(xp); hipFree(packed); hipFree(scales); hipFree(scales64);
  hipFree(y_valu); hipFree(y_f4); hipFree(digits); hipFree(p); hipFree(delta);
  if (ws) hipFree(ws);
  for (int k = 0; k < 2; ++k) { hipFree(g_packed[k]); hipFree(g_scales[k]); }
  hipFree(g_scales64[0]);
  free(hR); free(hx); free(hxp);
  if (failed) return 1;
  printf("ok\n");
  return 0;
}
