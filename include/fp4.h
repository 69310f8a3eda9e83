/*
 * fp4.h -- C ABI of libfp4.so: the block-quantized linear layer on AMD
 * Instinct MI355X (gfx950).
 *
 * The layer is three GEMMs (Fprop Y = X W^T, Dgrad dX = dY W, Wgrad
 * dW = dY^T X), each run on MXFP4 operands: blocks of 32 elements that share
 * one E8M0 power-of-two exponent, each element an E2M1 4-bit float.  Before
 * quantization an operand may be rotated block-wise by a Hadamard transform,
 * plain (the same every step) or after seeded random sign flips.  A second
 * quantizer produces NVFP4 (16-element blocks, E4M3 block scales, an fp32
 * tensor scale) with a renormalization folded into the block scales by
 * stochastic rounding, or with stochastic rounding of every element.
 *
 * Pages this interface follows (title, then section):
 *   [AMD-MXFP4]  "Pretraining large language models with MXFP4 on Native FP4
 *                Hardware" (htx.com news item): "Что такое MXFP4" (the block
 *                format), "Поисковая экспериментальная работа: корень
 *                нестабильности" (the three GEMMs; stochastic rounding;
 *                randomized vs deterministic Hadamard), and the figure caption
 *                of section "Сквозная эффективность" (the transform "H16").
 *   [QUARTET-II] "Quartet II -- обучение в NVFP4 с точными несмещёнными
 *                градиентами" (Telegram post): NVFP4 with FP8 scales,
 *                renormalization folded into the scales by stochastic rounding.
 *   [NV-NVFP4]   "NVIDIA создала метод обучения нейросетей в 4-bit точности":
 *                "Как это работает" (16x16 random Hadamard transforms).
 *
 * Conventions shared by every entry point
 *   - Pointers are device pointers (hipMalloc / torch CUDA tensors) owned by
 *     the caller, 16-byte aligned, tensors contiguous row-major.  The library
 *     allocates nothing in these calls and keeps no state between calls,
 *     except the device workspace the caller passes to nvfp4_quantize.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on it and returns; results are ready when the stream is.
 *   - Arguments are validated before any HIP call.  The status code is the
 *     only error channel: nothing is printed, nothing is thrown across the ABI.
 *     A kernel fault surfaces at the caller's next synchronization.
 *   - Sizes are int64; every size must be > 0.  Non-contraction dimensions
 *     may have any size (tails are masked).
 *   - Calls are reentrant; concurrent calls on different streams are safe as
 *     long as their output buffers do not overlap.
 */
#ifndef FP4_H_
#define FP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP4_OK = 0,
    FP4_ERR_NULL = 1,    /* a required pointer is NULL                         */
    FP4_ERR_SHAPE = 2,   /* size <= 0, contraction not a multiple of the block, */
                         /* or a size whose byte count overflows int64          */
    FP4_ERR_ALIGN = 3,   /* a pointer is not 16-byte aligned                    */
    FP4_ERR_ENUM = 4,    /* unknown axis / Hadamard mode / size / rounding /    */
                         /* output type / flag                                  */
    FP4_ERR_LAUNCH = 5,  /* the HIP runtime refused a kernel launch             */
    FP4_ERR_WORKSPACE = 6 /* workspace missing or smaller than required         */
} fp4_status;

/* Which axis of x[rows, cols] the 32-element blocks run along (the GEMM
 * contraction axis of that operand). */
typedef enum {
    FP4_AXIS_COLS = 0,   /* blocks along cols (contiguous): an operand of R = rows
                            rows of C = cols elements                           */
    FP4_AXIS_ROWS = 1    /* blocks along rows (strided), i.e. quantize x^T: an
                            operand of R = cols rows of C = rows elements       */
} fp4_axis;

/* MXFP4 operand layouts, used by every MXFP4 entry point.  An operand has R
 * logical rows of C contraction elements (C % 32 == 0), nb = C / 32 blocks
 * per row.  Neither layout is the plain row-major [R, C/2] / [R, C/32]; the
 * tags below name them, so that a caller can check at compile time
 * (#if !FP4_CODE_LAYOUT_TILED32 ... #error) which layouts it was written for.
 *
 * Codes ("32-row tiled", FP4_CODE_LAYOUT_TILED32): the 16 code bytes of
 * block b of row r (two E2M1 codes per byte, the even element in the low
 * nibble) are at offset ((r / 32) * nb + b) * 512 + (r % 32) * 16, i.e. for
 * each group of 32 rows and each block one contiguous 512-byte chunk, an
 * array [ceil(R/32)][nb][32][16] of FP4_CODE_BYTES(R, C) bytes.  Two
 * consecutive chunks of a row group are exactly the operand of one
 * 32 x 32 x 64 scaled MFMA in lane order, so a GEMM loads each k-step of 32
 * rows as one contiguous kilobyte.  When R % 32 != 0 the rows of the last
 * group past R are padding: the quantizers do not write them and the GEMMs
 * use them only for output rows that are not stored.
 *
 * Scales ("k-grouped", FP4_SCALE_LAYOUT_KGROUPED): the E8M0 scales are
 * stored in groups of 8 consecutive blocks: the byte of block b of row r is
 * at offset ((b / 8) * R + r) * 8 + b % 8, i.e. an array [ceil(nb/8)][R][8]
 * of FP4_SCALE_BYTES(R, C) bytes.  One group is the 256-element contraction
 * slice a GEMM stage consumes, so a stage's scales for consecutive rows are
 * one contiguous run.  When nb % 8 != 0 the last group's bytes past block
 * nb - 1 are padding: the quantizers do not write them and the GEMMs ignore
 * them.
 *
 * Output buffers are raw pointers: the library cannot check their extent.
 * Codes and scales buffers must be at least FP4_CODE_BYTES(R, C) and
 * FP4_SCALE_BYTES(R, C) bytes for the (R, C) of the call (a smaller buffer
 * is written past its end). */
#define FP4_CODE_LAYOUT_TILED32 1
#define FP4_SCALE_LAYOUT_KGROUPED 1
#define FP4_CODE_BYTES(R, C) ((((int64_t)(R) + 31) / 32) * 16 * (int64_t)(C))
#define FP4_SCALE_BYTES(R, C) ((((int64_t)(C) / 32 + 7) / 8) * (int64_t)(R) * 8)

/* Block rotation applied before quantization, along the block axis.
 * [AMD-MXFP4, "Поисковая экспериментальная работа..."]: a Hadamard transform,
 * either deterministic (the same every step) or with random sign flips. */
typedef enum {
    FP4_HAD_NONE = 0,    /* no rotation                                          */
    FP4_HAD_DET = 1,     /* y = H_n x / sqrt(n), H_n Sylvester-ordered            */
    FP4_HAD_SIGNED = 2   /* y = H_n D x / sqrt(n), D = diag of n seeded signs     */
} fp4_hadamard;

typedef enum {
    FP4_RTN = 0,         /* nearest E2M1 value, ties to the even code            */
    FP4_SR = 1           /* stochastic rounding (Philox4x32-10 keyed by sr_seed) */
} fp4_rounding;

/*
 * fp4_hadamard_quantize -- rotate (optionally) and quantize bf16 x[rows, cols]
 * to MXFP4 along `axis`.  [AMD-MXFP4, "Что такое MXFP4"]: 32-element blocks,
 * one shared E8M0 exponent, E2M1 elements rounded to the nearest value.
 *
 * Per 32-element block along the axis (the logical row r of A = x or x^T):
 *   1. had != NONE: each had_n-element sub-block (had_n = 16 or 32) is
 *      rotated: a = D x (signs), butterflies with strides 1, 2, ..., had_n/2
 *      computing (a+b, a-b) in binary32, then one binary32 multiply by
 *      fl(1/sqrt(had_n)).  D: s_j = -1 iff bit j of word 0 of Philox4x32-10
 *      (key = sign_seed, counter = (0, 0, 1, 0)); all +1 for DET.
 *   2. e = clamp(floor(log2 max|y|) - 2, -127, 127) (max = 0 gives -127);
 *      scale byte = e + 127.  A block holding a NaN or an infinity (also one
 *      produced by the rotation) gets scale 0xFF and all-zero codes.
 *   3. v = y * 2^-e in binary32; code = E2M1(v) with saturation at +-6:
 *      RTN ties to even, or SR: round up iff (u >> 8) * 2^-24 < p, p the
 *      fractional position between the two neighbours, u = word (idx & 3) of
 *      Philox4x32-10(key = sr_seed, counter = (idx >> 2, 0, 0) as 32-bit words
 *      (lo, hi, 0, 0)), idx = r * C + c the element's position in [R, C].
 *   4. codes: two per byte, the even element in the low nibble.
 * Output layout: the tiled codes (FP4_CODE_BYTES(R, C) bytes) and the
 * k-grouped scales (FP4_SCALE_BYTES(R, C) bytes) of R rows of C elements,
 * with (R, C) = (rows, cols) for AXIS_COLS and (cols, rows) for AXIS_ROWS.
 * Requirements: C % 32 == 0; x, codes, scales 16-byte aligned.
 * had_n is ignored when had == FP4_HAD_NONE; sign_seed is ignored unless
 * SIGNED; sr_seed is ignored unless rnd == FP4_SR.  For Wgrad, quantize dY
 * and X with the same had / had_n / sign_seed so the rotations cancel in
 * dY^T X (and different sr_seeds).
 */
fp4_status fp4_hadamard_quantize(const void* x_bf16, int64_t rows, int64_t cols,
                                 fp4_axis axis, int had_n, fp4_hadamard had,
                                 uint64_t sign_seed, fp4_rounding rnd, uint64_t sr_seed,
                                 uint8_t* codes, uint8_t* scales_e8m0, void* stream);

/*
 * fp4_hadamard_quantize_dual -- both MXFP4 quantizations of bf16 x[rows, cols]
 * from one read of x: the "rows" output is exactly what
 *   fp4_hadamard_quantize(x, rows, cols, FP4_AXIS_ROWS, had_n_rows, had_rows,
 *                         sign_seed_rows, rnd_rows, sr_seed_rows, ...)
 * writes (x^T blocked along rows: the Wgrad operands) and the "cols" output
 * exactly what the same call with FP4_AXIS_COLS and the *_cols settings
 * writes (the Fprop / Dgrad operands).  [AMD-MXFP4, "Поисковая
 * экспериментальная работа: корень нестабильности"]: each operand of the
 * three GEMMs is quantized along its own contraction axis, the Wgrad pair
 * after the rotation; a training step needs X and dY both ways.
 * Requirements: rows % 32 == 0 and cols % 32 == 0; every pointer 16-byte
 * aligned; the two outputs must not overlap.  Errors as fp4_hadamard_quantize.
 */
fp4_status fp4_hadamard_quantize_dual(const void* x_bf16, int64_t rows, int64_t cols,
                                      int had_n_rows, fp4_hadamard had_rows, uint64_t sign_seed_rows,
                                      fp4_rounding rnd_rows, uint64_t sr_seed_rows,
                                      uint8_t* codes_rows, uint8_t* scales_rows, int had_n_cols,
                                      fp4_hadamard had_cols, uint64_t sign_seed_cols,
                                      fp4_rounding rnd_cols, uint64_t sr_seed_cols,
                                      uint8_t* codes_cols, uint8_t* scales_cols, void* stream);

/*
 * fp4_wgrad_quantize -- the two Wgrad operands in one call: exactly what
 *   fp4_hadamard_quantize(dy, T, N, FP4_AXIS_ROWS, had_n, had, sign_seed, rnd, sr_seed_dy, dytq, dyts)
 *   fp4_hadamard_quantize(x,  T, K, FP4_AXIS_ROWS, had_n, had, sign_seed, rnd, sr_seed_x,  xtq,  xts)
 * write, with one launch for both when the sizes allow it.  [AMD-MXFP4,
 * "Поисковая экспериментальная работа: корень нестабильности"]: Wgrad rotates
 * both operands along the token axis with the same transform, so this call
 * takes one rotation for the pair.
 * Requirements: T % 32 == 0; pointers 16-byte aligned; the outputs must not
 * overlap.  Errors as fp4_hadamard_quantize.
 */
fp4_status fp4_wgrad_quantize(const void* dy_bf16, const void* x_bf16, int64_t T, int64_t N,
                              int64_t K, int had_n, fp4_hadamard had, uint64_t sign_seed,
                              fp4_rounding rnd, uint64_t sr_seed_dy, uint64_t sr_seed_x,
                              uint8_t* dytq, uint8_t* dyts, uint8_t* xtq, uint8_t* xts, void* stream);

/*
 * The three scaled-FP4 GEMMs of a linear layer.  [AMD-MXFP4, "Поисковая
 * экспериментальная работа: корень нестабильности"]: Fprop Y = X W^T,
 * Dgrad dX = dY W, Wgrad dW = dY^T X, all in MXFP4 on native FP4 matrix
 * cores.  Each computes, in fp32 accumulation,
 *     C[m, n] = sum_k  e2m1(a[m,k]) 2^(sa[m,k/32]-127) * e2m1(b[n,k]) 2^(sb[n,k/32]-127)
 * over two MXFP4 operands stored along their contraction axis (tiled codes
 * and k-grouped scales, as fp4_hadamard_quantize writes them).  C is
 * written (overwritten, not accumulated) as row-major fp32.
 * Requirements: T, N, K > 0; the contraction size a multiple of 32 and
 * below 2^24; at most 2^24 - 1 output tiles of 256 x 256; all pointers
 * 16-byte aligned.  Otherwise FP4_ERR_SHAPE / FP4_ERR_ALIGN.
 */
/* Fprop:  xq/xs = quantize(X[T,K], AXIS_COLS), wq/ws = quantize(W[N,K], AXIS_COLS);
 *         y[T, N] = X W^T.  Contraction K. */
fp4_status fp4_gemm_fprop(const uint8_t* xq, const uint8_t* xs, const uint8_t* wq,
                          const uint8_t* ws, int64_t T, int64_t N, int64_t K,
                          float* y, void* stream);
/* Dgrad:  dyq/dys = quantize(dY[T,N], AXIS_COLS), wtq/wts = quantize(W[N,K], AXIS_ROWS);
 *         dx[T, K] = dY W.  Contraction N. */
fp4_status fp4_gemm_dgrad(const uint8_t* dyq, const uint8_t* dys, const uint8_t* wtq,
                          const uint8_t* wts, int64_t T, int64_t N, int64_t K,
                          float* dx, void* stream);
/* Wgrad:  dytq/dyts = quantize(dY[T,N], AXIS_ROWS), xtq/xts = quantize(X[T,K], AXIS_ROWS);
 *         dw[N, K] = dY^T X.  Contraction T. */
fp4_status fp4_gemm_wgrad(const uint8_t* dytq, const uint8_t* dyts, const uint8_t* xtq,
                          const uint8_t* xts, int64_t T, int64_t N, int64_t K,
                          float* dw, void* stream);

/* Output element type of fp4_gemm_mx. */
typedef enum {
    FP4_OUT_F32 = 0,     /* binary32                                              */
    FP4_OUT_BF16 = 1     /* bfloat16, rounded to nearest even from the fp32 result */
} fp4_out_dtype;

/*
 * fp4_gemm_mx -- the same scaled-FP4 product as the three role entry points,
 * C[m, n] = sum_k a[m, k] b[n, k] over MXFP4 operands aq/as [M, Kc] and
 * bq/bs [N, Kc] (tiled codes and k-grouped scales along the contraction, as
 * fp4_hadamard_quantize writes them), with two output options:
 *   out = FP4_OUT_F32 or FP4_OUT_BF16: the element type of C (row-major
 *         [M, N]); bf16 is the fp32 result rounded to nearest even (NaN ->
 *         0x7FC0).
 *   accumulate = 0: C is overwritten; 1: C = A B^T + C, the old value read
 *         from C (widened to fp32) and added to the fp32 product before the
 *         output rounding.
 * Fprop, Dgrad and Wgrad are fp4_gemm_mx(A, B) with the operands named in
 * their comments above, fp32 output and accumulate = 0.  [AMD-MXFP4,
 * "Поисковая экспериментальная работа: корень нестабильности"]: the three
 * GEMMs in MXFP4; gradient accumulation and a bf16 activation output are
 * what a training step adds around them.
 * Requirements as for the role entry points; out and accumulate outside
 * their values give FP4_ERR_ENUM.
 */
fp4_status fp4_gemm_mx(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                       int64_t M, int64_t N, int64_t Kc, void* c, fp4_out_dtype out,
                       int accumulate, void* stream);

/* Rounding of nvfp4_quantize.  [QUARTET-II] contrasts two ways to make the
 * quantized gradient unbiased: stochastic rounding of every FP4 element
 * (NVIDIA's recipe, also [NV-NVFP4, "Как это работает"]) and elements
 * rounded to nearest with a per-block renormalization put into the FP8
 * scales by stochastic rounding (Quartet II). */
typedef enum {
    NVFP4_RTN = 0,         /* elements to nearest, scales to nearest        */
    NVFP4_RENORM_SR = 1,   /* elements to nearest, renormalized scale by SR */
    NVFP4_ELEMENT_SR = 2   /* elements by SR, scales to nearest             */
} nvfp4_mode;

/*
 * nvfp4_quantize -- NVFP4 quantization of bf16 x[rows, cols] along cols in
 * 16-element blocks.  [QUARTET-II]: FP4 elements with FP8 (E4M3) block
 * scales; the renormalization factor of a rotated tensor is folded into the
 * FP8 scales by stochastic rounding, the elements themselves are rounded to
 * nearest (mode NVFP4_RENORM_SR); the alternative it compares against rounds
 * every element stochastically (NVFP4_ELEMENT_SR).  [NV-NVFP4, "Как это
 * работает"]: 16x16 random Hadamard transforms.
 *   1. y = 16-block transform of each row (had as in fp4_hadamard_quantize
 *      with had_n = 16; NONE, DET or SIGNED).
 *   2. A = max |y| over the tensor, or *amax_in (a device float) when
 *      amax_in != NULL.  s_t = fl(A / 2688) (6 * 448), 1 when A = 0;
 *      *tensor_scale = s_t (a device float).
 *   3. per block: s_b = E4M3_RNE(fl(m_b / fl(6 s_t))) saturating at 448;
 *      s_b = 0 gives all-zero codes and scale 0.  Otherwise
 *      v_i = y_i * fl(1 / fl(s_b s_t)), codes = E2M1 RTN of v_i; with
 *      NVFP4_ELEMENT_SR codes = E2M1 SR of v_i (the rule of
 *      fp4_hadamard_quantize: |v| >= 6 gives 6, else up iff
 *      (u >> 8) 2^-24 < p) with u = word (idx & 3) of
 *      Philox4x32-10(key = sr_seed, counter = (idx >> 2 as (lo, hi), 0, 0)),
 *      idx = r * cols + c, and the stored scale is s_b.
 *   4. NVFP4_RENORM_SR: num = sum y_i^2, den = sum y_i e2m1(code_i) as binary32
 *      fmaf chains in element order; if den > 0 the stored scale is
 *      E4M3_SR(fl(num / fl(s_t den))) with u = word (blk & 3) of
 *      Philox4x32-10(key = sr_seed, counter = (blk >> 2 as (lo, hi), 2, 0)),
 *      blk = r * cols/16 + c/16; otherwise s_b.
 * Layout: codes [rows, cols/2], scales_e4m3 [rows, cols/16].
 * workspace: device memory of nvfp4_workspace_bytes() bytes, used for the
 * tensor amax when amax_in == NULL (cleared by the library on `stream`);
 * may be NULL when amax_in != NULL.
 * Non-finite values (the pages are silent; this is the library's rule):
 *   - the computed A is NaN if any rotated element is NaN, else +Inf if any
 *     is infinite;
 *   - an A (computed or supplied) whose s_t is not a finite positive number
 *     (A NaN, infinite, negative, or so small that A / 2688 is zero) makes
 *     *tensor_scale the quiet NaN 0x7FC00000, every scale byte 0x7F (the
 *     E4M3 NaN) and every code zero;
 *   - otherwise a block holding a NaN or an infinity (also one produced by
 *     the rotation) gets scale 0x7F and zero codes;
 *   - a block whose fl(1 / fl(s_b s_t)) is infinite (A below about 2^-125)
 *     gets zero codes and scale s_b;
 *   - NVFP4_RENORM_SR keeps s_b when its target is NaN (sums that overflow)
 *     and saturates an infinite target at 448.
 * Requirements: cols % 16 == 0; pointers 16-byte aligned (tensor_scale and
 * amax_in 4-byte aligned).
 */
fp4_status nvfp4_quantize(const void* x_bf16, int64_t rows, int64_t cols, fp4_hadamard had,
                          uint64_t sign_seed, nvfp4_mode mode, uint64_t sr_seed,
                          const float* amax_in, uint8_t* codes, uint8_t* scales_e4m3,
                          float* tensor_scale, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Workspace bytes nvfp4_quantize needs for a [rows, cols] input. */
size_t nvfp4_workspace_bytes(int64_t rows, int64_t cols);

/*
 * nvfp4_quantize_noalloc -- nvfp4_quantize without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops, harnesses that forbid allocation).  Same arguments,
 * results and errors as nvfp4_quantize; the in-library tensor amax (when
 * amax_in == NULL) lives in a 256-byte array the library holds in device
 * memory, one per GPU, until the process ends.  Nothing is allocated or
 * freed by the call.
 *   - The scratch array holds the one-word amax of an input of any size;
 *     FP4_ERR_WORKSPACE if nvfp4_workspace_bytes(rows, cols) ever exceeded
 *     its 256 bytes.
 *   - Every call on one GPU shares that GPU's array (cleared by a kernel at
 *     the start of each two-pass call): calls that overlap on one GPU, e.g.
 *     on two streams, race on it and must be serialized by the caller.
 *   - FP4_ERR_LAUNCH also reports a failure to look up the array's device
 *     address (once per device, on the first call with it current).
 */
fp4_status nvfp4_quantize_noalloc(const void* x_bf16, int64_t rows, int64_t cols, fp4_hadamard had,
                                  uint64_t sign_seed, nvfp4_mode mode, uint64_t sr_seed,
                                  const float* amax_in, uint8_t* codes, uint8_t* scales_e4m3,
                                  float* tensor_scale, void* stream);

/* Static, NUL-terminated name of a status code. */
const char* fp4_status_string(fp4_status status);

#ifdef __cplusplus
}
#endif

#endif /* FP4_H_ */
