/*
 * snip.h -- C ABI of libsnip: quantizers, block-scaled GEMMs and the
 * quantized linear layer of a Llama-like block, for AMD MI355X (gfx950).
 *
 * What the operations compute (sources cited by page title and section):
 *   - "SNIP: An Adaptive Mixed Precision Framework for Subbyte LLM
 *     Training", Abstract and Fig. 5: every linear layer of the block
 *     (Fig. 4: Q, K, V, O, Gate, Up, Down) runs its forward GEMM and its two
 *     backward GEMMs in a per-layer precision (FP8 or FP4; BF16 baseline),
 *     and statistics of activations and gradients are gathered to judge the
 *     precision loss.
 *   - "FP4 All the Way" summary page, Outline: NVFP4 = blocks of 16 E2M1
 *     values sharing one E4M3 scale; round-to-nearest in the forward pass,
 *     stochastic rounding in back-propagation and update.
 *   - "Research on Mixed-Precision Training for LLMs", Core Techniques:
 *     stochastic rounding rounds up or down by proximity and keeps the
 *     expected value.
 *
 * Conventions
 *   Ownership   The caller allocates and owns every buffer: inputs, outputs,
 *               quantized codes/scales, statistics and workspace. The library
 *               never allocates device memory.
 *   Pointers    Arguments documented "device" are device addresses; "host"
 *               ones are host addresses. Device pointers must be 16-byte
 *               aligned; leading dimensions are in elements.
 *   Streams     `stream` is a hipStream_t passed as void* (NULL = the null
 *               stream). Calls enqueue work and return before it completes,
 *               except snip_layer_stats, which synchronises the stream.
 *   Errors      Every call returns an int status (SNIP_OK = 0 or a negative
 *               SNIP_E_* code). Arguments are validated on the host before
 *               any HIP call, so a rejected call has enqueued nothing.
 *               snip_last_error() returns a thread-local message for the
 *               last failure. No C++ exception crosses this interface.
 *   Threads     Calls hold no global mutable state (apart from the launch
 *               timing switch, snip_timing_*) and may be made from several
 *               threads; work enqueued on one stream is ordered.
 *   Workspace   Caller-provided device scratch of at least the size the
 *               matching snip_*_workspace() returns; its contents need no
 *               initialisation and are clobbered. Calls that overlap in time
 *               must not share a workspace.
 *
 * Number formats and rounding (the full definitions are in the design notes)
 *   SNIP_NVFP4     4-bit E2M1 codes {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6},
 *                  one E4M3 scale per 16 consecutive K elements, and a
 *                  power-of-two tensor scale 2^e: e is the smallest integer
 *                  with max|x| / 2^e <= 6 * 448. Block scale = E4M3 RNE of
 *                  blockmax|x / 2^e| / 6; element r = (x / 2^e) * fp32(1 / s).
 *   SNIP_FP8_E4M3  8-bit E4M3 ("fn": max 448, no infinities) codes and a
 *                  power-of-two tensor scale with max|x| / 2^e <= 448.
 *   SNIP_MXFP4     E2M1 codes, one E8M0 scale per 32 K elements,
 *                  scale exponent floor(log2 blockmax|x|) - 2.
 *   SNIP_BF16      no quantization (bf16 values, K-contiguous).
 *   SNIP_RNE       round to nearest, ties to even, saturating.
 *   SNIP_SR        stochastic rounding with 16 random bits per element from
 *                  Philox4x32-10: key (seed lo, seed hi), counter
 *                  (g lo, g hi, tensor_id, 0), g = idx >> 3, word (idx>>1)&3,
 *                  half idx & 1, idx = element index in the quantized
 *                  output layout (row * K + k). Round the magnitude up iff
 *                  R16 + floor(frac * 2^16) >= 2^16, frac being the position
 *                  of |r| between its two neighbouring representable values.
 */
#ifndef SNIP_H
#define SNIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define SNIP_OK            0
#define SNIP_E_NULL       -1  /* a required pointer is NULL                  */
#define SNIP_E_SHAPE      -2  /* a dimension is out of range or misaligned   */
#define SNIP_E_ALIGN      -3  /* a device pointer is not 16-byte aligned     */
#define SNIP_E_FORMAT     -4  /* unknown format / rounding / layout, or a mismatch */
#define SNIP_E_WORKSPACE  -5  /* workspace missing or too small              */
#define SNIP_E_HIP        -6  /* a HIP launch or API call failed             */
#define SNIP_E_NONFINITE  -7  /* statistics report non-finite inputs         */

/* ---- enums ------------------------------------------------------------ */
#define SNIP_BF16      0
#define SNIP_FP8_E4M3  1
#define SNIP_NVFP4     2
#define SNIP_MXFP4     3
/* FP4 design-space variants [FP4 All the Way, Outline: block size, scaling
 * format and rounding were explored]: E2M1 codes with another block size or
 * scale format than NVFP4 / MX-FP4. Quantizer only (snip_quantize); the
 * GEMM and layer calls reject them with SNIP_E_FORMAT. */
#define SNIP_FP4_E4M3_B32  4  /* E4M3 scale per 32, power-of-two tensor scale */
#define SNIP_FP4_E8M0_B16  5  /* E8M0 scale per 16 (MX rule)                  */
#define SNIP_FP4_BF16_B16  6  /* BF16 scale per 16: bf16_RNE(blockmax / 6)    */
#define SNIP_FP4_BF16_B32  7  /* BF16 scale per 32                            */

#define SNIP_RNE       0
#define SNIP_SR        1

#define SNIP_ROWWISE   0  /* blocks along each row: [R, C] -> [R, C]        */
#define SNIP_COLWISE   1  /* blocks along each column: [R, C] -> [C, R]     */
#define SNIP_BOTHWISE  2  /* launch records only: one pass writing both      */

/* ---- descriptors ------------------------------------------------------ */

/* A quantized operand: `rows` rows of `k` elements, K-contiguous.
 * Host struct describing caller-owned device buffers:
 *   codes       device. NVFP4/MXFP4: u8[rows][k/2], element k in the low
 *               nibble when k is even, bit 3 of a nibble = sign.
 *               FP8: u8[rows][k]. BF16: bf16[rows][k].
 *               The FP4 variants (formats 4..7): as NVFP4.
 *   scales      device. NVFP4: E4M3 u8[rows][k/16]; MXFP4: E8M0 u8[rows][k/32];
 *               FP4_E4M3_B32: E4M3 u8[rows][k/32]; FP4_E8M0_B16: E8M0
 *               u8[rows][k/16]; FP4_BF16_B16 / _B32: bf16 bits
 *               u16[rows][k/16] / [k/32]; NULL for FP8 and BF16.
 *   tensor_exp  device int32: exponent e of the tensor scale 2^e for NVFP4,
 *               FP8 and FP4_E4M3_B32 (written by snip_quantize); unused (may
 *               be NULL) for the other formats. */
typedef struct snip_qtensor {
  int32_t  format;
  int32_t  reserved;
  int64_t  rows;
  int64_t  k;
  void*    codes;
  void*    scales;
  int32_t* tensor_exp;
} snip_qtensor;

/* Per-tensor statistics of one quantize pass (device memory, 24 bytes):
 *   sum_err2    sum over finite elements of (Q(x) - x)^2 (fp64 total)
 *   sum_x2      sum over finite elements of x^2
 *   amax        max |x| over the finite elements of the tensor quantized:
 *               the tensor-scale input, or, when a max was supplied
 *               (amax_in), the tensor's own max, so that a delayed-scaling
 *               caller can pass it to the next step
 *   n_nonfinite number of NaN / Inf inputs (their blocks' codes are
 *               unspecified) */
typedef struct snip_stats {
  double   sum_err2;
  double   sum_x2;
  float    amax;
  uint32_t n_nonfinite;
} snip_stats;

/* Host-side report derived from one snip_stats record. */
typedef struct snip_tensor_report {
  double   sum_err2;
  double   sum_x2;
  double   rel_mse;      /* sum_err2 / sum_x2 (0 when both are 0)            */
  double   norm_ratio;   /* ||x|| / ||Q(x) - x|| (+inf when the error is 0)  */
  float    amax;
  uint32_t n_nonfinite;
  int32_t  below_sqrt3;  /* 1 when ||x|| < sqrt(3) * ||Q(x) - x||: the regime
                            where learning on quantized gradients loses
                            efficiency ("FP4 All the Way", Outline)         */
  int32_t  reserved;
} snip_tensor_report;

/* ---- quantizer -------------------------------------------------------- */

/* Quantize one bf16 row-major tensor x[rows][cols] (leading dimension ld).
 * [FP4 All the Way, Outline] (formats, RTN/SR); [SNIP, Abstract] (stats).
 *   x          device bf16, 16-byte aligned, ld >= cols, ld % 8 == 0
 *   rows, cols > 0, cols % 16 == 0. ROWWISE: K = cols (MXFP4: cols % 32 == 0).
 *              COLWISE: K = rows, rows % 16 == 0 (MXFP4: % 32 == 0).
 *   layout     SNIP_ROWWISE -> out is [rows][cols]; SNIP_COLWISE -> out is
 *              [cols][rows] (the transpose, blocks along the source rows).
 *   format, rounding  as above (BF16 ignores rounding and copies/transposes;
 *              the FP4 variants need cols (ROWWISE) or rows (COLWISE) to be a
 *              multiple of their block).
 *   seed, tensor_id   random stream for SNIP_SR (ignored for SNIP_RNE).
 *   amax_in    device float or NULL. NULL: the tensor max is computed from x
 *              (an extra read pass). Non-NULL: used as max|x| for the tensor
 *              scale (delayed scaling; elements beyond it saturate); stats
 *              still reports x's own max.
 *   out        host descriptor of caller-owned device buffers; out->format,
 *              out->rows and out->k must match the call.
 *   stats      device snip_stats or NULL.
 *   ws         device workspace of snip_quantize_workspace() bytes.
 * Errors: NULL, SHAPE, ALIGN, FORMAT, WORKSPACE, HIP. */
int snip_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld,
                  int layout, int format, int rounding,
                  uint64_t seed, uint32_t tensor_id, const float* amax_in,
                  const snip_qtensor* out, snip_stats* stats,
                  void* ws, size_t ws_bytes, void* stream);

/* ---- block-scaled GEMM ------------------------------------------------- */

/* c[M][N] (fp32, leading dimension ldc, overwritten) = A . B^T, with
 * A = dequant(a) [M][K] and B = dequant(b) [N][K]; M = a->rows, N = b->rows,
 * K = a->k = b->k. [SNIP, Fig. 5]: the GEMMs of a linear layer.
 *   a, b       host descriptors; same format; K % 128 == 0; M, N > 0;
 *              each operand's codes below 4 GiB (rows x K x bytes per
 *              element), else SHAPE -- the same limit holds for every GEMM
 *              operand of the layer calls below.
 *              NVFP4 (code x block scale) and FP8 codes are decoded exactly
 *              to fp16 and run on the fp16 MFMA; MXFP4 runs on the gfx950
 *              scaled 4-bit MFMA with its E8M0 block scales in the
 *              instruction; BF16 on the bf16 MFMA. Accumulation is fp32;
 *              the tensor scales 2^(ea + eb) are applied in the epilogue.
 *   c          device fp32, ldc >= N.
 *   ws         may be NULL when ws_bytes == 0 (no workspace needed).
 * Errors: NULL, SHAPE, ALIGN, FORMAT, HIP. */
int snip_qgemm(const snip_qtensor* a, const snip_qtensor* b, float* c, int64_t ldc,
               void* ws, size_t ws_bytes, void* stream);

/* GEMM whose output is also quantized in the same launch: c = A . B^T as
 * snip_qgemm, and the row-wise quantization of c (blocks along N) in
 * out->format, as snip_quantize(..., SNIP_ROWWISE, out->format, rounding,
 * seed, tensor_id, amax_in, ...) would quantize a tensor holding c's fp32
 * values: the layer output becomes the next GEMM's quantized operand
 * without another read of it. [SNIP, Fig. 5]: a linear layer's output is
 * the input of the next layer; [FP4 All the Way, Outline]: forward
 * operands with nearest rounding, gradients with stochastic rounding.
 *   a, b, c, ldc  as snip_qgemm; a and b are FP8_E4M3 or NVFP4; ldc % 4 == 0.
 *   rounding      SNIP_RNE or SNIP_SR (Philox stream seed / tensor_id,
 *                 element index row * N + col).
 *   amax_in       device float, required: the tensor max that sets the
 *                 tensor scale (delayed scaling: c's own max is known only
 *                 after the launch; stats->amax reports it for the next call).
 *                 Values beyond it saturate.
 *   out           host descriptor, format NVFP4 or FP8_E4M3, rows = M,
 *                 k = N; N % 16 == 0.
 *   stats         device snip_stats or NULL: Sum (Q(c) - c)^2, Sum c^2,
 *                 max|c| and the non-finite count of c.
 *   ws            device, snip_qgemm_qout_workspace() bytes.
 * Errors: NULL, SHAPE, ALIGN, FORMAT, WORKSPACE, HIP. */
int snip_qgemm_qout(const snip_qtensor* a, const snip_qtensor* b, float* c, int64_t ldc,
                    int rounding, uint64_t seed, uint32_t tensor_id, const float* amax_in,
                    const snip_qtensor* out, snip_stats* stats, void* ws, size_t ws_bytes,
                    void* stream);

/* ---- quantized linear layer --------------------------------------------- */

/* Forward: y[T][out] (fp32) = Q_rne(x) . Q_rne(w)^T. [SNIP, Fig. 5];
 * [FP4 All the Way, Outline] (round-to-nearest forward).
 *   x          device bf16 [T][in]; w device bf16 [out][in] (contiguous).
 *   T, in, out > 0; in % 128 == 0 (the GEMM's K); T, out any.
 *   format     the layer's GEMM format from the plan.
 *   seed, layer_id  random-stream namespace (tensor ids 8*layer_id + {0,1};
 *              RTN draws no random bits).
 *   y          device fp32 [T][out].
 *   stats2     device snip_stats[2] = {X, W} or NULL.
 *   ws         device, snip_linear_fwd_workspace() bytes.
 * Errors: NULL, SHAPE, ALIGN, FORMAT, WORKSPACE, HIP. */
int snip_linear_fwd(const void* x, const void* w, int64_t T, int64_t in, int64_t out,
                    int format, uint64_t seed, uint32_t layer_id,
                    float* y, snip_stats* stats2, void* ws, size_t ws_bytes, void* stream);

/* Backward: dx[T][in] = Q_sr(dy) . Q_sr(w^T)^T   (K = out, fmt_dgrad)
 *           dw[out][in] = Q_sr(dy^T) . Q_sr(x^T)^T (K = T, fmt_wgrad)
 * [SNIP, Fig. 5]; [FP4 All the Way, Outline] (stochastic rounding in
 * back-propagation and update).
 *   dy         device bf16 [T][out]; x [T][in]; w [out][in] (contiguous).
 *   out % 128 == 0 and in % 16 == 0 when dx is computed; T % 128 == 0 and
 *   in % 16 == 0, out % 16 == 0 when dw is computed.
 *   tensor ids 8*layer_id + {2: dY row-wise, 3: W column-wise,
 *              4: dY column-wise, 5: X column-wise}.
 *   fwd_stats2 device snip_stats[2] = {X, W} written by snip_linear_fwd on the
 *              same x and w, or NULL. When given, their amax fields serve as
 *              max|x| and max|w| and the two tensors are not re-read for it.
 *   dx, dw     device fp32 or NULL (NULL skips that GEMM and its operands).
 *   stats4     device snip_stats[4] = {dY, W^T, dY^T, X^T} or NULL
 *              (entries of a skipped GEMM are left untouched).
 *   ws         device, snip_linear_bwd_workspace() bytes.
 * Errors: NULL, SHAPE, ALIGN, FORMAT, WORKSPACE, HIP. */
int snip_linear_bwd(const void* dy, const void* x, const void* w,
                    int64_t T, int64_t in, int64_t out,
                    int fmt_dgrad, int fmt_wgrad, uint64_t seed, uint32_t layer_id,
                    const snip_stats* fwd_stats2, float* dx, float* dw, snip_stats* stats4,
                    void* ws, size_t ws_bytes, void* stream);

/* ---- fused quantizers: one read of a tensor, both layouts -------------- */

/* Quantize one bf16 tensor x[rows][cols] row-wise and column-wise from a
 * single read of x: out_row receives exactly what snip_quantize(...,
 * SNIP_ROWWISE, format, rounding_row, seed, tensor_id_row, ...) writes and
 * out_col exactly what snip_quantize(..., SNIP_COLWISE, format,
 * rounding_col, seed, tensor_id_col, ...) writes (same codes, scales and
 * tensor exponent). [FP4 All the Way, Outline]: a tensor is quantized with
 * nearest rounding for the forward GEMM and stochastic rounding for the
 * backward ones; [SNIP, Fig. 5]: X, W and dY each feed two GEMMs, along
 * different dimensions.
 *   x          device bf16, 16-byte aligned, ld >= cols, ld % 8 == 0.
 *   format     SNIP_NVFP4, SNIP_FP8_E4M3 or SNIP_MXFP4 (BF16: FORMAT error).
 *   rows, cols > 0, both multiples of 16 (MXFP4: of 32).
 *   amax_in    as for snip_quantize.
 *   out_row    host descriptor, [rows][cols]; out_col [cols][rows].
 *   stats2     device snip_stats[2] = {row-wise, column-wise} or NULL.
 *   ws         device, snip_quantize_dual_workspace() bytes.
 * Errors: NULL, SHAPE, ALIGN, FORMAT, WORKSPACE, HIP. */
int snip_quantize_dual(const void* x, int64_t rows, int64_t cols, int64_t ld, int format,
                       int rounding_row, int rounding_col, uint64_t seed,
                       uint32_t tensor_id_row, uint32_t tensor_id_col, const float* amax_in,
                       const snip_qtensor* out_row, const snip_qtensor* out_col,
                       snip_stats* stats2, void* ws, size_t ws_bytes, void* stream);

/* Forward that also emits the backward operands built from x and w, so
 * that each of them is read once per training step:
 *   y[T][out] = Q_rne(x) . Q_rne(w)^T        (as snip_linear_fwd), and
 *   wt = Q_sr(w) column-wise, [in][out]      (tensor id 8*layer_id + 3),
 *   xt = Q_sr(x) column-wise, [in][T]        (tensor id 8*layer_id + 5):
 * byte for byte the operands snip_linear_bwd builds for the B sides of its
 * dgrad and wgrad GEMMs when fmt_dgrad = fmt_wgrad = format.
 * [SNIP, Fig. 5]; [FP4 All the Way, Outline].
 *   x          device bf16 [T][in]; w device bf16 [out][in] (contiguous).
 *   format     NVFP4, FP8_E4M3 or MXFP4, for all three GEMMs of the layer.
 *   T, in, out multiples of 128.
 *   amax_x, amax_w  device float each, or NULL. NULL: that tensor's max is
 *              computed from it (a read pass before quantizing). Non-NULL:
 *              used as max|x| for the tensor scale of both layouts (delayed
 *              scaling; elements beyond it saturate) and the pre-pass is
 *              skipped. The pointer may be the amax field of an earlier
 *              call's statistics record, including one that this call
 *              overwrites: it is read before the statistics are written.
 *   wt, xt     host descriptors of caller-owned device buffers in `format`
 *              (rows in, k = out; rows in, k = T); the caller keeps them
 *              until snip_linear_bwd_saved.
 *   stats4     device snip_stats[4] = {X, W, W^T, X^T} or NULL. The amax
 *              field is always max|x| of the tensor quantized now.
 *   ws         device, snip_linear_fwd_save_workspace() bytes.
 * Errors: NULL, SHAPE, ALIGN, FORMAT, WORKSPACE, HIP. */
int snip_linear_fwd_save(const void* x, const void* w, int64_t T, int64_t in, int64_t out,
                         int format, uint64_t seed, uint32_t layer_id,
                         const float* amax_x, const float* amax_w, float* y,
                         const snip_qtensor* wt, const snip_qtensor* xt, snip_stats* stats4,
                         void* ws, size_t ws_bytes, void* stream);

/* Backward from the saved operands: dy is read once and quantized both ways
 * (row-wise SR, tensor id 8*layer_id + 2; column-wise SR, id
 * 8*layer_id + 4), then
 *   dx[T][in]   = Q_sr(dy) . (wt)^T      (K = out)
 *   dw[out][in] = Q_sr(dy^T) . (xt)^T    (K = T)
 * identical to snip_linear_bwd with fmt_dgrad = fmt_wgrad = wt->format.
 * [SNIP, Fig. 5]; [FP4 All the Way, Outline].
 *   dy         device bf16 [T][out].
 *   wt, xt     as written by snip_linear_fwd_save (same format; wt [in][out],
 *              xt [in][T]); T, in, out multiples of 128.
 *   amax_dy    device float or NULL: a supplied max for dy, as amax_x of
 *              snip_linear_fwd_save.
 *   dx, dw     device fp32 or NULL (NULL skips that GEMM).
 *   stats2     device snip_stats[2] = {dY, dY^T} or NULL (amax: max|dy|).
 *   ws         device, snip_linear_bwd_saved_workspace() bytes.
 * Errors: NULL, SHAPE, ALIGN, FORMAT, WORKSPACE, HIP. */
int snip_linear_bwd_saved(const void* dy, const snip_qtensor* wt, const snip_qtensor* xt,
                          int64_t T, int64_t in, int64_t out, uint64_t seed, uint32_t layer_id,
                          const float* amax_dy, float* dx, float* dw, snip_stats* stats2,
                          void* ws, size_t ws_bytes, void* stream);

/* ---- allocation-free forward ------------------------------------------- */

/* Bytes of the static device scratch array behind
 * snip_linear_fwd_save_noalloc (held on every GPU the library runs on until
 * the process ends). */
#define SNIP_NOALLOC_SCRATCH_BYTES (32u << 20)

/* snip_linear_fwd_save without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving or training loops, harnesses that forbid hipMalloc): the
 * quantized row-wise X and W, the tensor-max and statistics partials and
 * any split-K partials live in the library's static scratch array instead
 * of a caller workspace. Same arguments (minus ws, ws_bytes), same results
 * byte for byte as snip_linear_fwd_save. Allocates nothing: no hipMalloc,
 * no allocating library call.
 *   Limit      the layer's workspace (snip_linear_fwd_save_workspace) must
 *              fit in SNIP_NOALLOC_SCRATCH_BYTES, else SNIP_E_WORKSPACE
 *              (checked before any HIP call). Layers up to the
 *              TinyLlama-1B shapes (T = 4096, 2048 -> 5632) fit.
 *   Sharing    every call on one GPU uses that GPU's one array, whose
 *              contents the last call leaves behind (nothing in it needs
 *              initialising: each call writes before it reads). Calls that
 *              overlap in time on one GPU (other streams, other threads)
 *              race on it and must be serialised by the caller.
 *   Set-up     the first call on a device looks up the array's device
 *              address there (hipGetSymbolAddress, with that device
 *              current); make it outside graph capture.
 *   stream     its device is the one whose array is used.
 * Errors: NULL, SHAPE, ALIGN, FORMAT, WORKSPACE (layer too large), HIP. */
int snip_linear_fwd_save_noalloc(const void* x, const void* w, int64_t T, int64_t in, int64_t out,
                                 int format, uint64_t seed, uint32_t layer_id,
                                 const float* amax_x, const float* amax_w, float* y,
                                 const snip_qtensor* wt, const snip_qtensor* xt, snip_stats* stats4,
                                 void* stream);

/* Synchronise `stream`, copy n device statistics records to the host and
 * derive the report of each. [SNIP, Abstract] (statistics for the precision
 * decision); [FP4 All the Way, Outline] (sqrt(3) threshold).
 *   dev_stats  device snip_stats[n]; host_out host snip_tensor_report[n].
 * Returns SNIP_E_NONFINITE (after filling host_out) when any record counts
 * non-finite inputs. Errors: NULL, SHAPE, HIP, NONFINITE. */
int snip_layer_stats(const snip_stats* dev_stats, int n, snip_tensor_report* host_out,
                     void* stream);

/* ---- sizing and diagnostics -------------------------------------------- */

/* Workspace bytes for the calls above (0 on invalid arguments). */
size_t snip_quantize_workspace(int64_t rows, int64_t cols, int layout, int format);
size_t snip_qgemm_workspace(int64_t M, int64_t N, int64_t K, int format);
size_t snip_linear_fwd_workspace(int64_t T, int64_t in, int64_t out, int format);
size_t snip_linear_bwd_workspace(int64_t T, int64_t in, int64_t out,
                                 int fmt_dgrad, int fmt_wgrad);
size_t snip_quantize_dual_workspace(int64_t rows, int64_t cols, int format);
size_t snip_linear_fwd_save_workspace(int64_t T, int64_t in, int64_t out, int format);
size_t snip_linear_bwd_saved_workspace(int64_t T, int64_t in, int64_t out, int format);
/* format: the operands' format (the output format does not change it). */
size_t snip_qgemm_qout_workspace(int64_t M, int64_t N, int64_t K, int format);

/* Workspace bytes of any of the calls above, by operation code: the one
 * sizing entry of the boundary, equal to the per-call helper of that call.
 *   op       SNIP_OP_* below; M, N, K as listed there (K is ignored by the
 *            quantizers); format: the call's format (for SNIP_OP_LINEAR_BWD
 *            both fmt_dgrad and fmt_wgrad).
 * Returns 0 on an unknown op or invalid arguments. */
#define SNIP_OP_QUANTIZE          0  /* M = rows, N = cols                       */
#define SNIP_OP_QGEMM             1  /* M, N, K of C[M][N] = A[M][K] . B[N][K]^T */
#define SNIP_OP_LINEAR_FWD        2  /* M = T, N = out, K = in                    */
#define SNIP_OP_LINEAR_BWD        3  /* M = T, N = out, K = in                    */
#define SNIP_OP_QUANTIZE_DUAL     4  /* M = rows, N = cols                       */
#define SNIP_OP_LINEAR_FWD_SAVE   5  /* M = T, N = out, K = in                    */
#define SNIP_OP_LINEAR_BWD_SAVED  6  /* M = T, N = out, K = in                    */
#define SNIP_OP_QGEMM_QOUT        7  /* M, N, K as SNIP_OP_QGEMM                 */
size_t snip_workspace_size(int op, int64_t M, int64_t N, int64_t K, int format);

/* Bytes of one part of a quantized operand: part 0 = codes, 1 = scales.
 * Returns -1 on invalid arguments. */
int64_t snip_qtensor_bytes(int format, int64_t rows, int64_t k, int part);

/* ---- launch timing (measurement support) -------------------------------- */

/* Kinds of kernel launch that the library makes. */
#define SNIP_LAUNCH_AMAX      0  /* tensor-max pre-pass                         */
#define SNIP_LAUNCH_QUANTIZE  1  /* quantize (or bf16 copy / transpose) pass    */
#define SNIP_LAUNCH_GEMM      2  /* block-scaled GEMM main kernel               */
#define SNIP_LAUNCH_SPLITK    3  /* split-K partial-sum reduction               */
#define SNIP_LAUNCH_FINALIZE  4  /* statistics finalisation                     */

/* One timed launch. `work` is the launch's algorithmic work: GEMM 2*M*N*K
 * flop; quantize and amax: source elements read (all tensors of the
 * launch); split-K: output elements; finalize: tensors (the layer calls
 * finalise their statistics inside their last GEMM launch, as extra
 * workgroups, and make no finalize launch). `ms` is the time
 * between HIP events recorded on the launch's stream right before and
 * right after it. */
typedef struct snip_launch_record {
  int32_t kind;       /* SNIP_LAUNCH_*                                      */
  int32_t format;     /* SNIP_BF16.. for quantize / GEMM / split-K, else -1 */
  int32_t layout;     /* quantize: SNIP_ROWWISE / SNIP_COLWISE, or
                         SNIP_BOTHWISE for a dual pass; else -1            */
  int32_t rounding;   /* quantize: SNIP_RNE / SNIP_SR, else -1              */
  double work;
  double ms;
} snip_launch_record;   /* 32 bytes */

/* Start timing: creates `capacity` (1 .. 1<<20) event pairs on the current
 * device and, until snip_timing_read, brackets every kernel launch of the
 * library with an event pair (launches beyond `capacity` are counted, not
 * timed; launches on a stream under graph capture are not timed). Adds a
 * few microseconds per launch: for measurement runs, not for production.
 * Process-global: do not time from several threads at once.
 * Errors: SHAPE (capacity), HIP. */
int snip_timing_start(int capacity);

/* Stop timing, wait for the recorded events, copy up to `max` records
 * (host array, in launch order) and release the events. Returns the number
 * of records written (>= 0); *n_untimed (host, may be NULL) receives the
 * number of launches that exceeded the capacity. Errors: HIP, FORMAT
 * (timing was not started). */
int snip_timing_read(snip_launch_record* out, int max, int64_t* n_untimed);

/* Thread-local message for the last failed call ("" if none). */
const char* snip_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int snip_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SNIP_H */
