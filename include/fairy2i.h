/*
 * fairy2i.h -- C ABI of libfairy2i.so, the MI355X (gfx950) hot path of Fairy2i-style
 * 2-bit widely-linear layers.
 *
 * What the library computes (sources are the pages this method is described on):
 *   - A real layer R (2n x 2m) is rewritten as y = U x + W conj(x) with U, W complex n x m
 *     (zhichai.net reading note "Fairy2i: Ultra-Low-Bit LLM Quantization Using Complex
 *     Weights {+-1, +-i}", "Step 1", Theorem 1 and its block closed form; ModelScope card
 *     "Fairy2i-W2", "Method", widely-linear transform).
 *   - Each of U, W is approximated by T residual stages of codes in {+1, i, -1, -i} with a
 *     real-axis and an imaginary-axis scale ("Step 2" projection and dequantization;
 *     "Step 3" residual recursion; card "Method").
 *   - The layer is applied without multiplying by weights: every code adds, subtracts or
 *     swaps real and imaginary parts ("Industry implications: multiplication-free
 *     inference"; 36Kr article, parallel stages).
 *
 * Conventions used by every call:
 *   - Every pointer argument is a DEVICE pointer owned by the caller, unless stated.
 *   - Each call checks its arguments on the host, enqueues its kernels on `stream` and
 *     returns; results are valid once the stream has reached that point.  The library never
 *     allocates device memory, keeps no pointer after returning and has no global state
 *     except a thread-local error message and the static device array of fairy2i_gemm_noalloc.
 *   - R x~ layout: R is fp32 row-major [2n][2m] (like nn.Linear.weight [out][in]);
 *     x~ = [Re x; Im x] and y~ = [Re y; Im y], i.e. a real vector of length 2m (2n) whose
 *     first half is the real part.  R's four quadrants are the blocks R11, R12, R21, R22.
 *   - Code k in {0,1,2,3} stands for i**k = (1, i, -1, -i).  Bit 0 is the axis (0 real,
 *     1 imaginary), bit 1 the sign.
 *   - packed form (fairy2i_packed_bytes(n, m, T) bytes): the codes of row i, stage t, matrix
 *     M (0 = U, 1 = W) -- plane P = 2t + M -- as little-endian 32-bit words of 16 codes.
 *     Word w of a (row, plane) holds codes j = 16w..16w+15; code 16w+p sits in bits
 *     8*(p%4) + 2*(p/4) .. +1, so byte b holds codes b, b+4, b+8, b+12 (one shift and one mask
 *     spread four codes into four bytes in j order).  Words are ordered per tile of 16 rows
 *     (the last tile padded with rows of code 0) as [chunk c of 256 columns][plane P]
 *     [64-column group g < G_c][row r < 16][word < 4], G_c = min(4, (m - 256c) / 64), tiles one
 *     after another: one (tile, chunk, plane) block is 16 rows x 64 columns per 256 bytes, the
 *     A operand of the matrix-core kernels as one contiguous load.  Four codes per byte:
 *     T*n*m/2 bytes per layer (T bits per real parameter of R) plus the padding rows.
 *   - scales: fp32 [n][T][2][2] = [row][stage][matrix][axis], axis 0 = real, 1 = imaginary.
 *   - Requirements: n >= 1, m >= 64 and m % 64 == 0, 1 <= T <= 4; pointers to packed, x, y,
 *     codes and workspaces 16-byte aligned; pointers to scales 4-byte aligned (8 for fp64).
 *   - Every call returns a fairy2i_status.  Nothing aborts or throws across the ABI.  Checks
 *     run in the order null -> dtype -> stages -> shape -> alignment -> workspace; launch
 *     failures return FAIRY2I_ERR_HIP.  fairy2i_last_error() gives the detail.
 *     Data-dependent preconditions (finite inputs, codes <= 3) are not checked.
 */
#ifndef FAIRY2I_H
#define FAIRY2I_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FAIRY2I_ABI_VERSION 7

typedef enum {
  FAIRY2I_OK = 0,
  FAIRY2I_ERR_NULL = 1,       /* a required pointer is NULL */
  FAIRY2I_ERR_SHAPE = 2,      /* n, m, batch or token count out of range */
  FAIRY2I_ERR_STAGES = 3,     /* T outside [1, 4] */
  FAIRY2I_ERR_DTYPE = 4,      /* unsupported dtype (or algorithm) combination */
  FAIRY2I_ERR_ALIGN = 5,      /* pointer not aligned as required */
  FAIRY2I_ERR_WORKSPACE = 6,  /* workspace NULL or smaller than the *_workspace_bytes call */
  FAIRY2I_ERR_HIP = 7         /* a HIP runtime call or kernel launch failed */
} fairy2i_status;

typedef enum {
  FAIRY2I_F32 = 0,
  FAIRY2I_BF16 = 1,
  FAIRY2I_I8 = 2,
  FAIRY2I_I32 = 3,
  FAIRY2I_X_DIGITS = 4,     /* decode-GEMV x as 22-bit integers in int8 digits (fairy2i_x_digits):
                             * each element off by at most 2^-22 of its column's max |x|, exact
                             * for bf16 values within 2^14 of that maximum */
  FAIRY2I_X_DIGITS_F6 = 5   /* the same integers in fp6 digits (fairy2i_x_digits_f6), same bound */
} fairy2i_dtype;

/* GEMV kernels.  AUTO picks MFMA_F4 for x in fp6 digit form, MFMA_I8 for x in int8 digit form,
 * MFMA_F4 or MFMA_BF16 for bf16 x (below) and VALU for fp32 x; MFMA means MFMA_BF16.
 *   VALU       fp32 add/sub/swap accumulation on the vector ALUs; fp32 or bf16 x.
 *   MFMA_BF16  codes decoded in registers to bf16 planes {+-2, 0}, multiplied with the unchanged
 *              bf16 x on v_mfma_f32_16x16x32_bf16: exact products, fp32 sums.  bf16 x.
 *   MFMA_I8    codes decoded to int8 planes {-1, 0, 1}, multiplied with x in digit form (made
 *              once per x by fairy2i_x_digits) on v_mfma_i32_16x16x64_i8: exact int32 sums,
 *              fp32 epilogue.  x_dtype FAIRY2I_X_DIGITS, B <= 2.  Half the MFMA cycles and
 *              ~2/3 of the VALU work per code of MFMA_BF16.
 *   MFMA_F4    codes read as fp4 planes of u = B_re + B_im and v = B_re - B_im (both +-1 for
 *              every codeword, eight bit operations per 16 codes), multiplied with x in fp6
 *              digit form on v_mfma_scale_f32_16x16x128_f8f6f4: exact integer sums in fp32, B_re
 *              and B_im sums as (u +- v) / 2, fp32 epilogue.  B <= 2.  x_dtype FAIRY2I_X_DIGITS_F6
 *              (the digit form made once by fairy2i_x_digits_f6 and shared by every GEMV that
 *              reads that x) or FAIRY2I_BF16: then the digits are built on chip from the bf16 x
 *              (m * B <= 8192; in a grouped call of 1536 tiles or more every item must have the
 *              same x).  In launches of 1536 tiles or more, and for m <= 256, each workgroup
 *              builds the same digits as fairy2i_x_digits_f6 (outputs identical bit for bit to
 *              the two-call form).  Smaller launches digitize each 256-column chunk of each batch
 *              entry at its own exponent (max over the chunk's 512 values of |x| 2^S_c in
 *              [2^21, 2^22)), each wave for the chunks it multiplies, and pass 2^-S_c to the
 *              MFMAs as block scales: every element is off by at most 2^-22 of its chunk's
 *              maximum (never more than the per-row form), the chunks' sums are added in fp32,
 *              and the outputs are not bit-identical to the two-call form.  The fastest decode
 *              kernel on gfx950: half the MFMA cycles and about half the VALU work per code of
 *              MFMA_I8.  At 3 <= B <= 16 (bf16 x only) the same fp4 planes multiply x split into
 *              two fp8 e4m3 parts, hi = rne(x 2^-E) and lo = rne(x 2^-E - hi), under one E8M0
 *              scale 2^E per 32 columns (the columns one fp4 lane holds at one MFMA step) with
 *              E = floor(log2 M) - 7 for the block's max |x| = M: every product exact, fp32 sums;
 *              each x entry is exact when |x| >= 2^-10 M and otherwise off by at most 2^-17 M
 *              (m <= 2^19).
 * AUTO with bf16 x takes MFMA_F4 at 3 <= B <= 4 for launches of at least 1536 16-row tiles (the
 * fp8 split above); and for launches of at least 1536 16-row tiles with B <= 2,
 * m * B <= 8192 and one x for the launch (resident workgroups build the digits once for many
 * tiles); for smaller launches at B = 1 with 2048 <= m <= 8192, or 1024 <= m < 2048 in launches
 * of at least 128 tiles (each wave builds the digits of its own chunks, which there costs less
 * than MFMA_BF16's work); and MFMA_BF16 otherwise. */
typedef enum {
  FAIRY2I_GEMV_AUTO = 0,
  FAIRY2I_GEMV_VALU = 1,
  FAIRY2I_GEMV_MFMA = 2,
  FAIRY2I_GEMV_MFMA_BF16 = 3,
  FAIRY2I_GEMV_MFMA_I8 = 4,
  FAIRY2I_GEMV_MFMA_F4 = 5
} fairy2i_gemv_algo;

/* Bytes of the packed form of an n x m complex layer with T stages:
 * ceil(n / 16) * 16 * T * 2 * m / 4 (0 for non-positive sizes). */
size_t fairy2i_packed_bytes(int64_t n, int64_t m, int T);

/* Quantize a real layer.  Widely-linear split (Theorem 1, "Step 1"), then for t < T:
 * projection to the nearest of {1, i, -1, -i} (first in that order on ties), per-row
 * per-stage per-matrix axis scales s = mean |Re r| (|Im r|) over the entries coded on that
 * axis (0 if none), residual r <- r - (s_re b_re + i s_im b_im) ("Step 2", "Step 3").
 * All arithmetic is fp64; the scale sums use a fixed order (256 partial sums over
 * j = l, l+256, ..., then a halving tree), so results do not depend on the launch.
 *   R        fp32 [two_n][two_m], read only.
 *   packed   out, the packed form (fairy2i_packed_bytes(n, m, T) bytes, padding rows zeroed).
 *   scales   out, fp32 [n][T][2][2] (round-to-nearest-even of the fp64 scales).
 *   scales64 optional out (NULL skips), fp64 [n][T][2][2].
 *   codes    optional out (NULL skips), uint8 [T][2][n][m], one code per byte.
 * Extra requirements: 2*T*m <= 65536 (codes of one row are staged on chip); ceil(n / 16) * 16
 * < 2^24 (one workgroup per row, one launch). */
int fairy2i_quantize(const float* R, int64_t two_n, int64_t two_m, int T,
                     uint8_t* packed, float* scales, double* scales64, uint8_t* codes,
                     hipStream_t stream);

/* fairy2i_quantize for a bf16 layer (checkpoints are commonly stored in bf16): R is bf16
 * [two_n][two_m] (raw bits, 2-byte aligned), widened exactly to fp64; everything else as
 * fairy2i_quantize, so a bf16 layer quantizes exactly like its fp32 widening. */
int fairy2i_quantize_bf16(const uint16_t* R, int64_t two_n, int64_t two_m, int T,
                          uint8_t* packed, float* scales, double* scales64, uint8_t* codes,
                          hipStream_t stream);

/* fairy2i_quantize on count layers of one shape, in as few launches as the per-launch table
 * allows (32 layers each): every layer is quantized exactly as by its own fairy2i_quantize call
 * (same codes, packed bytes and scales, bit for bit), but the layers' rows share launches, so a
 * stack of small layers fills the device instead of ending every launch on a partial round of
 * workgroups.  Arguments are host arrays of count device pointers:
 *   R         [count] layers [two_n][two_m], R_dtype FAIRY2I_F32 (4-byte aligned) or
 *             FAIRY2I_BF16 (raw bits, 2-byte aligned, widened exactly); read only.
 *   packed    [count] out, each fairy2i_packed_bytes(n, m, T) bytes, 16-byte aligned.
 *   scales    [count] out, each fp32 [n][T][2][2].
 *   scales64  NULL, or [count] optional outs (entries may be NULL), each fp64 [n][T][2][2].
 *   codes     NULL, or [count] optional outs (entries may be NULL), each uint8 [T][2][n][m],
 *             16-byte aligned.
 * count = 0 does nothing; count < 0 or more rows than one launch can address
 * (min(count, 32) * ceil(n / 16) * 16 >= 2^24) is FAIRY2I_ERR_SHAPE; a NULL array or R,
 * packed or scales entry is FAIRY2I_ERR_NULL.  Nothing is launched unless every argument
 * passes.  Extra requirement as fairy2i_quantize: 2*T*m <= 65536. */
int fairy2i_quantize_grouped(int count, const void* const* R, int R_dtype, int64_t two_n, int64_t two_m, int T,
                             uint8_t* const* packed, float* const* scales, double* const* scales64,
                             uint8_t* const* codes, hipStream_t stream);

/* Device workspace bytes of fairy2i_quantize_tensor for n complex rows: 40 n rounded up to a
 * multiple of 16, plus 128 (0 when n is out of range; m and T do not enter). */
size_t fairy2i_quantize_tensor_workspace_bytes(int64_t n, int64_t m, int T);

/* fairy2i_quantize with per-tensor axis scales, the other reading of the axis-wise scales of
 * "Step 2" (zhichai.net note; ModelScope card "Method"), whose granularity the pages leave open:
 * one (s_re, s_im) pair per stage and matrix, s_re the mean of |Re r| over every entry of the
 * matrix coded on the real axis (s_im likewise; 0 if none), residual as in fairy2i_quantize.
 * The row sums are those of fairy2i_quantize; the tensor sum combines them in the same fixed
 * order with rows in place of columns (256 partial sums over rows l, l+256, ..., halving tree),
 * so the result does not depend on the launch.  Counts are exact.
 *   R, R_dtype  [two_n][two_m], FAIRY2I_F32 (4-byte aligned) or FAIRY2I_BF16 (raw bits,
 *               2-byte aligned, widened exactly).
 *   workspace   device memory of at least fairy2i_quantize_tensor_workspace_bytes(n, m, T)
 *               bytes, 16-byte aligned, owned by the caller; its contents are ignored on entry
 *               and undefined on return.  Calls that share one workspace must not overlap.
 *   packed, scales, scales64, codes  as fairy2i_quantize; every row of scales (scales64) holds
 *               the same pairs, so every consumer of fairy2i_quantize's output takes them as is.
 * Runs as 2T + 1 launches on stream.  Extra requirements: m <= 32768, and n as for
 * fairy2i_quantize.  Error codes as
 * fairy2i_quantize, plus FAIRY2I_ERR_WORKSPACE for a short workspace and FAIRY2I_ERR_DTYPE
 * for another R_dtype. */
int fairy2i_quantize_tensor(const void* R, int R_dtype, int64_t two_n, int64_t two_m, int T,
                            void* workspace, size_t workspace_bytes, uint8_t* packed, float* scales,
                            double* scales64, uint8_t* codes, hipStream_t stream);

/* Pack one-byte codes uint8 [T][2][n][m] (values 0..3; higher bits are ignored) into the
 * packed form above, padding rows zeroed (ModelScope card "Model details": 2 bits per real
 * parameter at T=2).  packed: fairy2i_packed_bytes(n, m, T) bytes. */
int fairy2i_pack(const uint8_t* codes, int64_t n, int64_t m, int T, uint8_t* packed,
                 hipStream_t stream);

/* Digit form of decode-GEMV activations, the input of the MFMA_I8 kernel (exact integer
 * arithmetic on the int8 matrix cores; same sum as the ModelScope card "Method" y = U x +
 * W conj(x), with x held exactly as integers).  For each batch column b < B: one power of two
 * 2^S_b with max_j |x_b,j| 2^S_b in [2^21, 2^22) (S_b = 0 for an all-zero column), X =
 * round_half_even(x 2^S_b) -- exact for every bf16 value no more than 2^14 below the column
 * maximum; otherwise (smaller bf16 values, most fp32 values) off by at most 2^-22 of the column
 * maximum, so an output moves by at most that times the sum of |R^| over its row -- and X = d0 + 2^8 d1 + 2^16 d2
 * with signed int8 digits.
 *   x        [B][2m], x_dtype FAIRY2I_F32 or FAIRY2I_BF16, 16-byte aligned.  1 <= B <= 2.
 *   digits   out, fairy2i_x_digits_bytes(m, B) bytes, 16-byte aligned: int32 header
 *            [B, m, S_0, S_1] in the first 64 bytes, then int8 [B][2][4][m] (batch column,
 *            component Re x / Im x, digit slot; slot 3 is zero).
 * The digit form is tied to the m and B it was made with; pass the same m and B to the GEMV. */
size_t fairy2i_x_digits_bytes(int64_t m, int64_t B);
int fairy2i_x_digits(const void* x, int x_dtype, int64_t m, int64_t B, void* digits, hipStream_t stream);

/* fp6 digit form of decode-GEMV activations, the input of the MFMA_F4 kernel.  The same X_b =
 * round_half_even(x_b 2^S_b) as fairy2i_x_digits (same S_b, same rounding), written with eight
 * balanced base-8 digits X = sum_l 8^l d_l, d_l in [-4, 3], each stored as fp6 e2m3 (exact).
 *   x        [B][2m], x_dtype FAIRY2I_F32 or FAIRY2I_BF16, 16-byte aligned.  1 <= B <= 2.
 *   digits   out, fairy2i_x_digits_f6_bytes(m, B) = 64 + ceil(m / 256) * 4096 * B bytes,
 *            16-byte aligned: int32 header [B, m, S_0, S_1] in the first 64 bytes, then
 *            32-byte records ordered [256-column chunk][half][b][lane], each holding the 32 fp6
 *            digits (6 bits each, little-endian) that one lane of the MFMA_F4 kernel multiplies
 *            with its fp4 codes, in the column order those codes take in the packed words;
 *            every byte is written.
 * The form is tied to the m and B it was made with; pass the same m and B to the GEMV. */
size_t fairy2i_x_digits_f6_bytes(int64_t m, int64_t B);
int fairy2i_x_digits_f6(const void* x, int x_dtype, int64_t m, int64_t B, void* digits, hipStream_t stream);

/* Dequantize a packed layer to its real form (the fake-quantized layer of QAT and a third route
 * to the layer's map): U^ = sum_t (s_re(t) b_re(t) + i s_im(t) b_im(t)) and likewise W^
 * (zhichai.net note, "Step 2" dequantization and "Step 3" stage sum), then the real blocks of
 * y = U^ x + W^ conj(x) (Note "Step 1"; ModelScope card "Method"):
 *     R11 = Re U^ + Re W^   R12 = Im W^ - Im U^   R21 = Im U^ + Im W^   R22 = Re U^ - Re W^.
 * The stage sums run over t in order in fp32.
 *   packed, scales  as produced by fairy2i_quantize.
 *   R       out, [2n][2m] row-major, R_dtype FAIRY2I_F32 or FAIRY2I_BF16 (round to nearest even),
 *           16-byte aligned.
 * Extra requirement: n as for fairy2i_quantize (one workgroup per row). */
int fairy2i_dequantize(const uint8_t* packed, const float* scales, int64_t n, int64_t m, int T,
                       void* R, int R_dtype, hipStream_t stream);

/* Decode GEMV: y~[b] = sum_t U~(t) x[b] + W~(t) conj(x[b]) for b < B (ModelScope card "Method":
 * the widely-linear form y = U x + W conj(x), each matrix the sum of its T quantized terms;
 * zhichai.net note "Industry implications": with codes in {+-1, +-i} every product is an add,
 * subtract or real/imaginary swap with sign; 36Kr article: the stage terms are independent and
 * summed).  One accumulator per (stage, matrix, axis), so each scale multiplies an accumulated
 * sum, not a weight.
 *   packed, scales  as produced by fairy2i_quantize.
 *   x       [B][2m] with x_dtype FAIRY2I_F32 or FAIRY2I_BF16, or a digit form of such an x
 *           (x_dtype FAIRY2I_X_DIGITS or FAIRY2I_X_DIGITS_F6, made with the same m and B).
 *           1 <= B <= 16.
 *   y       out, [B][2n], y_dtype FAIRY2I_F32 or FAIRY2I_BF16 (round to nearest even).
 *   algo    fairy2i_gemv_algo; MFMA_BF16 requires x_dtype BF16, MFMA_I8 x_dtype X_DIGITS and
 *           B <= 2, MFMA_F4 x_dtype X_DIGITS_F6 (m <= 2^19: its fp32 sums stay exact integers)
 *           and B <= 2, or BF16 (B <= 2: m * B <= 8192; B > 2: m <= 2^19); VALU takes F32 or
 *           BF16.
 * Uses no workspace. */
int fairy2i_gemv(const uint8_t* packed, const float* scales, int64_t n, int64_t m, int T,
                 const void* x, int x_dtype, int64_t B, void* y, int y_dtype, int algo,
                 hipStream_t stream);

/* One GEMV of a grouped call.  packed, scales, x, y as for fairy2i_gemv; n complex rows. */
typedef struct {
  const uint8_t* packed;
  const float* scales;
  const void* x;
  void* y;
  int64_t n;
} fairy2i_gemv_item;

/* Grouped decode GEMV: `count` independent GEMVs that share m, T, B and the dtypes (for example
 * the q, k and v projections, which also share x; ModelScope card "Method": every linear layer
 * becomes a widely-linear layer).  The MFMA kernels cover all items' row tiles in one grid of
 * up to 48 items per launch, so a small layer does not pay a launch ramp and tail of its own;
 * VALU runs the items one after another.  Items that share x may share its digit form.
 *   items   HOST array of `count` items (read during the call only; the pointers in it are
 *           device pointers).  Each item is checked like a fairy2i_gemv call. */
int fairy2i_gemv_grouped(const fairy2i_gemv_item* items, int count, int64_t m, int T, int x_dtype,
                         int64_t B, int y_dtype, int algo, hipStream_t stream);

/* Strided-batch decode GEMV: `batch` GEMVs of one shape (n, m, T) that share x, with matrix k's
 * operands at constant strides from matrix 0's (for example q, k and v kept in one buffer, or
 * the layers of a stack stored back to back).  Same rows as fairy2i_gemv_grouped (ModelScope
 * card "Method"), but with no limit on the number of matrices per launch: the MFMA kernels run
 * the whole batch as one grid; VALU runs the matrices one after another.
 *   packed + k * packed_stride   matrix k's packed form; packed_stride in bytes, >= 0, a
 *                                multiple of 16.
 *   scales + k * scales_stride   its scales; scales_stride in floats, >= 0 (0: shared scales).
 *   y + k * y_stride             its output [B][2n]; y_stride in elements of y_dtype, at least
 *                                2nB when batch > 1 (outputs must not overlap), and a multiple
 *                                of 16 bytes.
 *   x, x_dtype, B, y_dtype, algo as for fairy2i_gemv; 1 <= batch and batch * ceil(n / 16)
 *   <= 2^30.  Uses no workspace. */
int fairy2i_gemv_strided(const uint8_t* packed, int64_t packed_stride, const float* scales,
                         int64_t scales_stride, int64_t n, int64_t m, int T, const void* x,
                         int x_dtype, int64_t B, void* y, int64_t y_stride, int y_dtype,
                         int64_t batch, int algo, hipStream_t stream);

/* Per-token int8 activations for the prefill GEMM (the pages fix no activation format; this is
 * the plainest integer form that lets the int8 matrix cores run the multiplication-free product
 * of the zhichai.net note, "Industry implications"): delta[tok] = fl32(max_j |x~_j| / 127),
 * q = clamp(round_half_even(fl32(x~ / delta)), -127, 127); delta == 0 gives q = 0.
 *   x      [N][two_m], x_dtype FAIRY2I_F32 or FAIRY2I_BF16.  q out int8 [N][two_m],
 *   delta  out fp32 [N]. */
int fairy2i_act_quant(const void* x, int x_dtype, int64_t N, int64_t two_m, int8_t* q,
                      float* delta, hipStream_t stream);

/* Workspace for fairy2i_gemm: int8 activations and their scales when x is not already int8. */
size_t fairy2i_gemm_workspace_bytes(int64_t n, int64_t m, int T, int64_t N, int x_dtype);

/* Prefill GEMM over N tokens.  Codes are decoded on chip into int8 planes B_re, B_im in
 * {-1, 0, 1} ("Industry implications"); int8 matrix cores accumulate
 * P[t][M][plane][comp][tok][i] = sum_j B_plane[i][j] * q[tok][comp*m + j] exactly in int32.
 *   x        [N][2m]; x_dtype BF16 / F32 (quantized per token inside, see fairy2i_act_quant)
 *            or I8 (already quantized).
 *   x_scale  delta [N] fp32: output when x is BF16/F32 (may be NULL), input when x is I8.
 *   y        y_dtype F32 / BF16: y~ [N][2n] = delta * the widely-linear combination of P
 *            with the fp32 scales.  y_dtype I32: the raw accumulators, int32
 *            [T][2][2][2][N][n] = [stage][matrix][plane][comp (0: Re x, 1: Im x)][tok][row].
 *   workspace  fairy2i_gemm_workspace_bytes(...) bytes, 16-byte aligned (NULL allowed if 0).
 *   1 <= N <= 1048576. */
int fairy2i_gemm(const uint8_t* packed, const float* scales, int64_t n, int64_t m, int T,
                 const void* x, int x_dtype, float* x_scale, int64_t N,
                 void* y, int y_dtype, void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/* fairy2i_gemm for callers that cannot allocate device memory -- code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc -- and so cannot pass a workspace.  Same
 * arguments, results and checks as fairy2i_gemm without the workspace: when x is BF16 / F32 its
 * per-token int8 activations and delta are staged in a static device array of the library (one
 * per GPU, fairy2i_gemm_noalloc_max_bytes() = 32 MiB, held from the first call on that GPU until
 * the process ends; the entry point and its kernels allocate nothing).  The call uses the array of
 * the calling thread's current device; `stream` must belong to that device.
 *   Limit: fairy2i_gemm_workspace_bytes(n, m, T, N, x_dtype) <= fairy2i_gemm_noalloc_max_bytes()
 *   (for example 2048 tokens of 2m <= 16380 reals); a larger call returns FAIRY2I_ERR_WORKSPACE.
 *   The array is shared by every call on a GPU and keeps the last call's contents (every byte a
 *   call reads it has written first): calls that overlap on one GPU -- on different streams or
 *   host threads without ordering -- race and must not be issued.  With x in I8 the array is not
 *   used. */
size_t fairy2i_gemm_noalloc_max_bytes(void);
int fairy2i_gemm_noalloc(const uint8_t* packed, const float* scales, int64_t n, int64_t m, int T,
                         const void* x, int x_dtype, float* x_scale, int64_t N,
                         void* y, int y_dtype, hipStream_t stream);

const char* fairy2i_status_string(int status);
const char* fairy2i_last_error(void);   /* thread-local detail of the last non-OK return */
int fairy2i_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FAIRY2I_H */
