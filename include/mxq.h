/*
 * mxq.h -- C ABI of the MI355X (gfx950) library for the online half of
 * block-aligned outlier rotation + MXFP4 quantization of LLM activations.
 *
 * Operation (DuQuant++ page, "DuQuant++: block-aligned rotation quantization
 * for MXFP4 activation outliers"):
 *   sec. 3.1   smoothing: X' = X * Lambda^-1, Lambda a per-channel factor
 *   sec. 3.2-3.3  rotation: X^ = X' * R, R = BlockDiag(R_b, ..., R_b) with one
 *              shared 32x32 orthogonal block R_b, so every 32-channel group g
 *              of a token row is rotated on its own: y_g = x'_g * R_b
 *   sec. 2.1   MXFP4: each 32-element group gets one shared scale from its
 *              largest magnitude and every element is rounded to the nearest
 *              4-bit float
 *   sec. 5.2 item 1  smoothing and rotation fused into one kernel in front of
 *              the MXFP4 linear layer (here quantization is fused in as well)
 *
 * MXFP4 convention (OCP Microscaling Formats v1.0, FP32-to-MX conversion):
 *   amax = max_n |y_n| over the 32 rotated values of the group
 *   e    = floor(log2 amax) - 2  (2 = largest exponent of E2M1), clamped to
 *          [-127, 127]; amax = 0 gives e = -127
 *   scale byte S = e + 127 (E8M0, bias 127).  0xFF (NaN) is never produced.
 *   element code = E2M1 value nearest to y_n / 2^e among
 *          {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}; a value exactly halfway
 *          goes to the even code (ties-to-even); |y_n / 2^e| > 6 saturates to
 *          +-6; zero results are always code 0x0 (never 0x8).
 *   Since amax / 2^e is in [4, 8), the largest element always encodes to 4 or
 *   6, and at most the top quarter of the range (6, 8) is clipped.
 *   code nibble: bit 3 sign, bits 2..0 magnitude code (values above by code
 *   0..7).  Packing: byte j of a group holds element 2j in its low nibble and
 *   element 2j+1 in its high nibble.
 *
 * Layouts (all row-major, dense unless a stride is given):
 *   x       [tokens][x_row_stride] elements, the first `channels` of a row used
 *   lambda  [channels] fp32
 *   r_hat   [32][32] bf16 bit patterns, y_n = sum_k x'_k * r_hat[k][n]
 *   codes   [tokens][channels / 2] bytes
 *   scales  [tokens][channels / 32] bytes
 *
 * Common rules for every call:
 *   - Every buffer is DEVICE memory owned by the caller; the library never
 *     allocates, frees or synchronizes.  `stream` is a hipStream_t passed as
 *     void* (NULL = the null stream).  Calls are asynchronous: results are
 *     valid once the caller has synchronized that stream.
 *   - Arguments are validated on the host before any HIP call; on error
 *     nothing is launched and nothing is written.  A launch failure returns
 *     MXQ_ERR_HIP.  Faults during execution surface at the caller's next sync.
 *   - tokens == 0 or channels == 0 is a valid empty call (returns MXQ_OK,
 *     launches nothing, pointers may be NULL).
 *   - Pointers x, codes, y_rot, y and lambda must be 16-byte aligned, and
 *     x_row_stride * sizeof(element) must be a multiple of 16 (MXQ_ERR_ALIGN).
 *     scales and r_hat need only their natural alignment.
 *   - Limits: channels % 32 == 0, tokens below 2^31, channels at most 2^28,
 *     and tokens * ceil(channels / 2048) below 2^31 (MXQ_ERR_SHAPE).
 *   - NaN or infinite inputs are outside the contract (no error is raised,
 *     the output for such a group is unspecified), and so are finite inputs
 *     whose smoothed or rotated fp32 values overflow (magnitude 2^128 or
 *     more; e.g. 32 values near the bf16 maximum under a spreading block).
 *   - The library holds no per-call state; calls are thread-safe.  Calls that
 *     write the same output buffers concurrently race, as with any kernel.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MXQ_OK = 0,
    MXQ_ERR_NULL = 1,   /* a required pointer is NULL                        */
    MXQ_ERR_SHAPE = 2,  /* negative size, channels % 32 != 0, or too large   */
    MXQ_ERR_DTYPE = 3,  /* dtype not supported by this entry point           */
    MXQ_ERR_ALIGN = 4,  /* pointer or row pitch not aligned as required      */
    MXQ_ERR_STRIDE = 5, /* x_row_stride < channels                           */
    MXQ_ERR_HIP = 6     /* the HIP runtime reported an error at launch       */
} mxq_status;

typedef enum { MXQ_BF16 = 0, MXQ_FP16 = 1, MXQ_FP32 = 2 } mxq_dtype;

typedef enum { MXQ_NORM_RMS = 0, MXQ_NORM_LAYER = 1 } mxq_norm_kind;

/* Smooth + rotate + MXFP4-quantize in one pass over x.
 * DuQuant++ page sec. 3.3 (online transform X * Lambda^-1 * R) and sec. 2.1
 * (MXFP4 encoding); the smoothing factor is that of sec. 3.1.
 *   x        BF16 or FP16 activations (MXQ_ERR_DTYPE otherwise)
 *   lambda   per-channel divisor, or NULL for no smoothing (same as all ones)
 *   r_hat    the shared 32x32 block in bf16
 *   codes, scales  outputs, fully overwritten
 * The rotation runs on the matrix cores with bf16 operands and fp32
 * accumulation.  Without lambda the activations enter as bf16 terms whose
 * sum is exactly x (bf16 x: 1 term; fp16 x: 2 terms), so the products are
 * exact and only the fp32 accumulation rounds.  With lambda, x' = x *
 * rcp(lambda) (rcp the hardware reciprocal, within 1 ulp; fp16 x times the
 * factor in one fused multiply, rounded once) enters as two bf16 terms, each
 * rounded to nearest: hi = bf16(x'), lo = bf16(x' - hi), |x' - hi - lo| <=
 * 2^-18 |x'|.  So every rotated value of a group g is within about
 * 2^-18 ||x'_g||_2 (lambda) or 0 (no lambda), plus the fp32 accumulation
 * error of its 32 terms, of the exact x'_g R.  That holds at every
 * magnitude: a group whose rotated maximum is below 2^-64 (whose bf16 terms
 * or products would fall below bf16's or fp32's normal range) is
 * recomputed, after the main pass over the rows, from x' * 2^k, k <= 64 a
 * power-of-two shift chosen from the group's largest |x'| (x * (factor *
 * 2^k) formed exactly in fp64, rounded to fp32 once, then split into 3 exact
 * bf16 terms), and encoded with its scale reduced by k; the y_rot output
 * (mxq_rotate_quant_ex) of a group below fp32's normal range is its value
 * rounded to fp32.  Rows holding such groups cost a second pass; ordinary
 * data has none.
 * lambda entries must be finite normal fp32 values with |lambda| in
 * [2^-126, 2^126]; others give unspecified codes for their groups. */
mxq_status mxq_rotate_quant(const void *x, int32_t x_dtype, int64_t tokens, int64_t channels,
                            int64_t x_row_stride, const float *lambda, const uint16_t *r_hat,
                            uint8_t *codes, uint8_t *scales, void *stream);

/* Same kernel as mxq_rotate_quant; additionally stores the fp32 rotated
 * values y [tokens][channels] (dense) when y_rot is not NULL.  Codes and
 * scales are bit-identical to those of mxq_rotate_quant.  Meant for tests and
 * error studies: the extra store costs 4 bytes per element. */
mxq_status mxq_rotate_quant_ex(const void *x, int32_t x_dtype, int64_t tokens, int64_t channels,
                               int64_t x_row_stride, const float *lambda, const uint16_t *r_hat,
                               uint8_t *codes, uint8_t *scales, float *y_rot, void *stream);

/* Plain MXFP4 quantization of x (no smoothing, no rotation); DuQuant++ page
 * sec. 2.1.  x may be BF16, FP16 or FP32.  Bit-identical to mxq_rotate_quant
 * with lambda = NULL and r_hat = identity for BF16/FP16 input. */
mxq_status mxq_quant(const void *x, int32_t x_dtype, int64_t tokens, int64_t channels,
                     int64_t x_row_stride, uint8_t *codes, uint8_t *scales, void *stream);

/* Decode MXFP4 back to BF16 or FP32 y [tokens][channels] (dense):
 * y = (-1)^s * {0, .5, 1, 1.5, 2, 3, 4, 6}[m] * 2^(S - 127) (OCP MX v1.0
 * E2M1 and E8M0 tables).  All 16 codes are accepted (0x8 gives -0.0);
 * S = 0xFF gives NaN; values beyond the output type's range give +-inf.
 * Every finite result is exact in both output types.  The decoded tensor is
 * the rotated X^ of sec. 3.3, not the original activations. */
mxq_status mxq_dequant(const uint8_t *codes, const uint8_t *scales, int64_t tokens,
                       int64_t channels, void *y, int32_t y_dtype, void *stream);

/* Rotation by a block of another size, for the block-size ablation of the
 * DuQuant++ page (sec. 4.3: B = 16, 32, 64, 128 with MXFP4 groups kept 32
 * wide): every block of B channels of x / lambda is multiplied by the B x B
 * bf16 matrix r_block (row-major, y_n = sum_k x'_k r_block[k][n]), then
 * every 32-element group of the result is MXFP4-encoded as in
 * mxq_rotate_quant.  block must be 16, 32, 64 or 128 and divide channels
 * (MXQ_ERR_SHAPE otherwise); y_rot may be NULL or fp32 [tokens][channels].
 * B = 32 is mxq_rotate_quant itself (the call goes to its kernel); other
 * sizes follow the same arithmetic, layout and error rules: the product runs
 * on the matrix cores with the bf16 terms of x' that mxq_rotate_quant uses
 * (exact without lambda, two rounded terms with it). */
mxq_status mxq_rotate_quant_block(const void *x, int32_t x_dtype, int64_t tokens, int64_t channels,
                                  int64_t x_row_stride, const float *lambda, const uint16_t *r_block,
                                  int32_t block, uint8_t *codes, uint8_t *scales, float *y_rot,
                                  void *stream);

/* Norm + smooth + rotate + MXFP4-quantize in one pass over x.
 * DuQuant++ page sec. 5.2 item 1: the per-channel 1/lambda folds into the
 * output of the norm in front of the linear layer, and the online steps run
 * as one kernel.  For every token row h of x (the norm's input):
 *   RMSNorm   (MXQ_NORM_RMS)    n_c = h_c / sqrt(sum_c h_c^2 / C + eps)
 *   LayerNorm (MXQ_NORM_LAYER)  n_c = (h_c - mu) / sqrt(sum_c (h_c - mu)^2 / C + eps),
 *                               mu = sum_c h_c / C (biased variance)
 *   a_c = n_c * gamma_c + beta_c,  x'_c = a_c / lambda_c
 * then the rotation and encoding of mxq_rotate_quant.
 *   x        BF16 or FP16, [tokens][x_row_stride], channels <= 16384
 *   gamma    fp32 [channels], required; beta fp32 [channels] or NULL (zero);
 *   lambda   fp32 [channels] or NULL (ones); eps finite and >= 0
 *            (MXQ_ERR_SHAPE if negative, infinite or NaN).  A row whose
 *            variance is zero (a row of zeros for RMSNorm, a constant row
 *            for LayerNorm) with eps = 0 is outside the contract (0 / 0).
 *            The per-channel factors gamma_c / lambda_c and beta_c / lambda_c,
 *            rounded to fp32, must each be 0 or of magnitude in
 *            [2^-64, 2^64); others give unspecified codes for their groups.
 *   y_rot    NULL, or fp32 [tokens][channels] receiving the rotated values
 * Arithmetic: row sums in fp32 per 128 values (exact products of the 16-bit
 * inputs on the matrix cores; LayerNorm's centred sums per 8 values on the
 * vector units, about a shift near the mean), accumulated and reduced in
 * fp64; the LayerNorm mean is subtracted as an fp32 pair (hi + lo), so its
 * error scales with the row's spread, not its mean; 1/sqrt in fp64,
 * rounded to fp32; x'_c = fma(n_c, gamma_c/lambda_c,
 * beta_c/lambda_c) in fp32 (the two factors formed once per block with IEEE
 * division); the product with the block as in mxq_rotate_quant with lambda
 * (two bf16 terms rounded to nearest, within 2^-18 |x'|).  Every finite 16-bit row is in range: a bf16 row whose fp32
 * sum of squares leaves [2^-80, 2^1000] (squares beyond fp32's range, or lost
 * below it) is scaled by a power of two 2^kr taken from its largest |h| and
 * its statistics retaken, with eps scaled by 2^(2 kr), which leaves the
 * normalized row unchanged; a group whose rotated maximum is below 2^-64 is
 * recomputed from x' * 2^k as in mxq_rotate_quant, with x' * 2^k formed as
 * fma(d * 2^k, gamma/lambda, (beta/lambda) * 2^k) from 1/sqrt in fp64 times
 * 2^k.  Such rows cost a second pass over the rows of their wave; ordinary
 * data has none.  Same layout, alignment (gamma, beta, lambda: 4 bytes) and
 * error rules as mxq_rotate_quant; norm_kind other than the two values gives
 * MXQ_ERR_DTYPE. */
mxq_status mxq_norm_rotate_quant(const void *x, int32_t x_dtype, int64_t tokens, int64_t channels,
                                 int64_t x_row_stride, int32_t norm_kind, const float *gamma,
                                 const float *beta, float eps, const float *lambda,
                                 const uint16_t *r_hat, uint8_t *codes, uint8_t *scales, float *y_rot,
                                 void *stream);

/* ---- the consumer: MXFP4 x MXFP4 linear layer ----------------------------
 * DuQuant++ page sec. 3.3 (weight absorption, W^ = R^T Lambda W, so that
 * (X Lambda^-1 R)(R^T Lambda W) = X W) and sec. 5.2 (the rotated MXFP4
 * activations feed an MXFP4 linear layer).
 *
 * mxq_absorb_quant: offline preparation of the weights.  w holds W^T, one
 *   row of `cols` = K input features per output feature (the usual linear
 *   layer layout [N][K], BF16 or FP16, row pitch w_row_stride elements).
 *   Each row is multiplied by lambda (per input feature, fp32; NULL = no
 *   smoothing), rotated group by group with the shared 32x32 block r_hat
 *   (same convention as mxq_rotate_quant: y_n = sum_k w'_k r_hat[k][n]) and
 *   MXFP4-encoded along K: codes [rows][cols/2], scales [rows][cols/32], the
 *   B operand of mxq_gemm_mxfp4.  The product w * lambda is rounded once to
 *   fp32 and then carried as two bf16 terms rounded to nearest, as x' is in
 *   mxq_rotate_quant (without lambda, exact terms).  Same rules, limits and
 *   errors as mxq_rotate_quant.
 *
 * mxq_gemm_mxfp4: y[m][n] = sum_k dq(A)[m][k] * dq(B)[n][k], where
 *   A = (a_codes [M][K/2], a_scales [M][K/32]) are quantized activations as
 *   written by mxq_rotate_quant (M tokens, K channels) and
 *   B = (b_codes [N][K/2], b_scales [N][K/32]) the quantized weights as
 *   written by mxq_absorb_quant.  y is [M][ldy] FP32 (y_dtype MXQ_FP32) or
 *   BF16 (MXQ_BF16, round-to-nearest-even of the fp32 result); only the first
 *   N entries of each row are written.  Runs on the scaled matrix cores
 *   (v_mfma_scale_f32_16x16x128_f8f6f4, E2M1 operands, E8M0 block scales):
 *   every product is exact and the sum is accumulated in fp32, so each FP32
 *   output is within 2 K 2^-24 sum_k |dq(A)[m][k] dq(B)[n][k]| of the exact
 *   value (much closer in practice) as long as products and partial sums stay
 *   in the fp32 normal range.  Scale bytes 0xFF (NaN) give NaN.
 *   Requirements: K % 128 == 0 and K <= 2^24, M and N below 2^31
 *   (MXQ_ERR_SHAPE); a_codes, b_codes 16-byte aligned, a_scales, b_scales
 *   2-byte aligned, y aligned to its element (MXQ_ERR_ALIGN); ldy >= N
 *   (MXQ_ERR_STRIDE).  M == 0 or N == 0 is an empty call; K == 0 writes
 *   zeros (the code and scale pointers may then be NULL). */
mxq_status mxq_absorb_quant(const void *w, int32_t w_dtype, int64_t rows, int64_t cols,
                            int64_t w_row_stride, const float *lambda, const uint16_t *r_hat,
                            uint8_t *codes, uint8_t *scales, void *stream);

mxq_status mxq_gemm_mxfp4(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                          const uint8_t *b_scales, int64_t M, int64_t N, int64_t K, void *y,
                          int32_t y_dtype, int64_t ldy, void *stream);

/* ---- fragment-tiled MXFP4 operands -----------------------------------------
 * A storage order of MXFP4 operands for the product above.  The DuQuant++
 * page fixes no memory layout: sec. 5.4 items 2-3 leave the weight format to
 * the target hardware and put the fused transform directly in front of the
 * MXFP4 linear layer, and sec. 5.2 item 1 asks for no extra pass over
 * intermediate tensors; here the quantizer can write the order in which the
 * matrix cores read, so no repacking pass sits between them.  An operand of R rows and K positions
 * (K % 128 == 0) is cut into records of 16 rows x 128 positions; record
 * (t, s) -- rows 16t..16t+15, positions 128s..128s+127 -- has index
 * t * (K/128) + s.  Its 64 slots follow the operand order of the
 * 16 x 16 x 128 scaled MFMA: slot l is row 16t + l % 16, group 4s + l / 16
 * (32 positions).  Codes: 1024-byte records, slot l's 16 code bytes (same
 * byte order as the row layout) at byte 16 l.  Scales: 64-byte records,
 * slot l's scale byte at byte l.  Buffers hold ceil(R/16) * (K/128)
 * records, i.e. ceil(R/16) * 16 * K/2 code bytes and ceil(R/16) * 16 * K/32
 * scale bytes.  Rows R..16*ceil(R/16)-1 are padding.
 *
 * mxq_tile_mxfp4: row layout (codes [rows][K/2], scales [rows][K/32]) to
 *   the tiled layout, padding rows written as zero bytes.  Meant for the
 *   weights, once, offline.  Requirements: K % 128 == 0, K <= 2^24,
 *   rows < 2^31 (MXQ_ERR_SHAPE); codes and tiled_codes 16-byte aligned
 *   (MXQ_ERR_ALIGN); rows == 0 or K == 0 is an empty call.  The output must
 *   not overlap the input.
 *
 * mxq_rotate_quant_tiled: mxq_rotate_quant with its codes and scales written
 *   in the tiled layout (bit-identical bytes, other positions); channels must
 *   be a multiple of 128 (MXQ_ERR_SHAPE) and tiled_scales 16-byte aligned
 *   (MXQ_ERR_ALIGN).  The codes of the padding rows of the last record row
 *   are not written; their scale bytes may be written as zero.  Other rules
 *   as mxq_rotate_quant.
 *
 * mxq_gemm_mxfp4_tiled: mxq_gemm_mxfp4 with both operands tiled (A from
 *   mxq_rotate_quant_tiled or mxq_tile_mxfp4, B from mxq_tile_mxfp4 of
 *   mxq_absorb_quant's output).  Outputs are bit-identical to those of
 *   mxq_gemm_mxfp4 on the same operands in the row layout; the contents of
 *   padding rows affect only outputs that are not written.  Same
 *   requirements, with a_tscales and b_tscales 4-byte aligned. */
mxq_status mxq_tile_mxfp4(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K,
                          uint8_t *tiled_codes, uint8_t *tiled_scales, void *stream);

mxq_status mxq_rotate_quant_tiled(const void *x, int32_t x_dtype, int64_t tokens, int64_t channels,
                                  int64_t x_row_stride, const float *lambda, const uint16_t *r_hat,
                                  uint8_t *tiled_codes, uint8_t *tiled_scales, void *stream);

mxq_status mxq_gemm_mxfp4_tiled(const uint8_t *a_tcodes, const uint8_t *a_tscales, const uint8_t *b_tcodes,
                                const uint8_t *b_tscales, int64_t M, int64_t N, int64_t K, void *y,
                                int32_t y_dtype, int64_t ldy, void *stream);

/* mxq_norm_rotate_quant_tiled: mxq_norm_rotate_quant with its codes and
 *   scales written in the tiled layout (bit-identical bytes, other
 *   positions); channels must be a multiple of 128 (MXQ_ERR_SHAPE) and
 *   tiled_scales 16-byte aligned (MXQ_ERR_ALIGN).  Short (decode-sized)
 *   batches store each row on its own; long batches stage a record row, or
 *   half of one, in LDS and store whole records.  The padding rows of the
 *   last record row are unspecified: they may be written as zeros or left
 *   untouched.  Other rules as mxq_norm_rotate_quant. */
mxq_status mxq_norm_rotate_quant_tiled(const void *x, int32_t x_dtype, int64_t tokens, int64_t channels,
                                       int64_t x_row_stride, int32_t norm_kind, const float *gamma,
                                       const float *beta, float eps, const float *lambda, const uint16_t *r_hat,
                                       uint8_t *tiled_codes, uint8_t *tiled_scales, void *stream);

/* ---- offline calibration of the shared block (DuQuant++ page sec. 3.2) ----
 * Greedy outlier-aware construction of the 32x32 block R_b, in fp64 as the
 * page advises (sec. 3 pitfalls, item 3), on the GPU.  Two calls:
 *
 * mxq_calib_worst_group: over the calibration activations x [tokens][stride]
 *   (BF16, FP16 or FP32; the first `channels` of each row), divided by lambda
 *   when lambda is not NULL (the search runs on X / Lambda, sec. 5.1 item 3),
 *   find the 32-channel group with the largest |value| (ties: lowest group)
 *   and copy that group's slice X_worst to x_worst [tokens][32] fp64.
 *   group (one int64) and linf (one double) receive the group index and its
 *   largest |value|.  All pointers are device memory.
 *
 * mxq_calib_givens: starting from R = I, repeat at most max_steps times (the
 *   page uses 128): d = the column of x_worst holding the largest |value|
 *   (ties: lowest column); for every other column j the Givens rotation
 *   G(d, j) with angle pi/4, which maps (x_d, x_j) to
 *   (c x_d - s x_j, s x_d + c x_j), c = s = sqrt(1/2); keep the j whose
 *   rotated tensor has the smallest largest |value| (ties: lowest j); if
 *   that value is not larger than the current one, R <- R G and
 *   x_worst <- x_worst G, else stop.  Outputs (device memory):
 *     x_worst      overwritten with x_worst * R
 *     r_block      [32][32] fp64, row-major, y = x * r_block
 *     linf_history [max_steps + 1] fp64: entry 0 the initial largest |value|,
 *                  entry i the value after step i (i <= *steps_done; the
 *                  sequence never increases); later entries untouched
 *     steps_done   one int32: number of rotations taken
 *     pairs        [max_steps][2] int32 (d, j) of each step taken, or NULL
 *   Every product and sum is a separately rounded fp64 operation in a fixed
 *   order: results are bit-reproducible.  Each step is two kernel launches.
 *
 * Both take a device workspace of at least mxq_calib_workspace_bytes(channels)
 * bytes (channels = 0 is enough for mxq_calib_givens), 256-byte aligned and
 * owned by the caller; calls sharing a workspace must not overlap.  Errors:
 * MXQ_ERR_DTYPE, MXQ_ERR_SHAPE (tokens <= 0, channels not a positive
 * multiple of 32, max_steps < 0), MXQ_ERR_NULL, MXQ_ERR_STRIDE, MXQ_ERR_ALIGN
 * (workspace too small or misaligned, fp64 outputs not 8-byte aligned), all
 * before any launch; MXQ_ERR_HIP on a launch failure. */
size_t mxq_calib_workspace_bytes(int64_t channels);

mxq_status mxq_calib_worst_group(const void *x, int32_t x_dtype, int64_t tokens, int64_t channels,
                                 int64_t x_row_stride, const float *lambda, double *x_worst, int64_t *group,
                                 double *linf, void *workspace, size_t workspace_bytes, void *stream);

mxq_status mxq_calib_givens(double *x_worst, int64_t tokens, int32_t max_steps, double *r_block,
                            double *linf_history, int32_t *steps_done, int32_t *pairs, void *workspace,
                            size_t workspace_bytes, void *stream);

/* mxq_calib_givens_angles: the same greedy search, except that every
 *   candidate j also chooses its angle (the page's step 3d asks for the
 *   rotation that lowers the largest |value| the most).  The angles form a
 *   grid of angle_grid = M entries (1 <= M <= 1024, MXQ_ERR_SHAPE otherwise):
 *   index 0 is pi/4, index k (1 <= k < M) the angle theta with
 *   tan(theta / 2) = k / M, i.e. c = (M^2 - k^2) / (M^2 + k^2) and
 *   s = 2 k M / (M^2 + k^2), each a correctly rounded fp64 division.  The
 *   largest |value| is periodic in theta with period pi/2, so the grid spans
 *   (0, pi/2) with gaps of at most 2 / M radians.  The pair (j, angle) with
 *   the smallest largest |value| wins (ties: lowest j, then lowest index).
 *   M = 1 is mxq_calib_givens bit for bit.  Extra output:
 *     angles       [max_steps] int32 grid index of each step's angle, or NULL
 *   Other arguments, outputs, rules and errors as mxq_calib_givens (the
 *   same workspace size serves both); each step is three kernel launches. */
mxq_status mxq_calib_givens_angles(double *x_worst, int64_t tokens, int32_t max_steps, int32_t angle_grid,
                                   double *r_block, double *linf_history, int32_t *steps_done, int32_t *pairs,
                                   int32_t *angles, void *workspace, size_t workspace_bytes, void *stream);

/* mxq_calib_worst_group_noalloc: mxq_calib_worst_group for callers that
 *   cannot allocate device memory -- code under HIP graph capture, tight
 *   serving loops, harnesses that forbid hipMalloc.  It takes no workspace
 *   and allocates nothing: the per-group maxima live in a device array of
 *   the library (64 KiB, one per GPU, held until the process ends), so
 *   channels is limited to 262144 (MXQ_ERR_SHAPE above that, before any HIP
 *   call).  Every call on one GPU shares that array; the call clears what it
 *   uses before reading it, and calls that overlap on one GPU (other
 *   streams, other threads) race.  The array's address is looked up on the
 *   first call on each device (MXQ_ERR_HIP if that fails).  Same outputs,
 *   bit for bit, and the same other rules and errors as
 *   mxq_calib_worst_group. */
mxq_status mxq_calib_worst_group_noalloc(const void *x, int32_t x_dtype, int64_t tokens, int64_t channels,
                                         int64_t x_row_stride, const float *lambda, double *x_worst,
                                         int64_t *group, double *linf, void *stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char *mxq_status_str(int32_t status);

/* Launch plan of the quantize kernels, a pure host function that touches no
 * device: for `tokens` x `channels` on a GPU with `cu_count` compute units it
 * writes {blocks, waves, tile_columns, row_step, waves_per_block} into
 * out[0..4].  Returns MXQ_ERR_SHAPE for shapes the entry points reject. */
mxq_status mxq_plan(int64_t tokens, int64_t channels, int32_t cu_count, int32_t *out);

/* Library ABI version: 1. */
int32_t mxq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
