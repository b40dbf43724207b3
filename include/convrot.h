/*
 * convrot.h -- C ABI of the ConvRot W8A8 / W4A8 quantized linear for AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed (sources: web pages on ConvRot int8/int4 checkpoints):
 *  - "MOSS-Image Qwen3.5-9B text encoder, INT8 (W8A8, ConvRot)", file table:
 *    row "Quantized" -- every weight row is rotated per contiguous 256-column
 *    group by a Hadamard matrix and stored int8 with one fp32 scale per output
 *    row; row "Matmul" -- at run time the activations get the group-wise
 *    rotation too, one int8 scale per token, and the product runs in int8.
 *  - "qwen3.5_4b_int8_convrot", "Quantization Recipe": row-wise scaling with
 *    plain rounding (--scaling_mode row --simple), group size 256.
 *  - "craftingmod/Qwen3-VL-8B-Heretic-INT8", "Quantization metadata":
 *    convrot, convrot_groupsize 256, per_row, orig_dtype bfloat16.
 *  - "MossInt4", "Format": signed 4-bit weight codes two per byte with one
 *    F32 scale per row chosen by a clip search; 8-bit activations.
 * Around that path the library also has: the RMSNorm that precedes the
 * linears fused into the activation pass, several linears sharing one
 * quantized input, the weight-only (dequant) path with a bf16 matmul, and
 * small group sizes (16 for the vision widths, 1 for plain row-wise).
 *
 * Definitions used by every call (H is the Sylvester Hadamard matrix of
 * order g in natural order, H[i][j] = (-1)^popcount(i&j) / sqrt(g); a row is
 * rotated by multiplying each contiguous group of g columns by H):
 *    scale      = absmax(rotated row) / 127                  (fp32)
 *    code       = round_half_away_from_zero(rotated / scale)  (int8, |code| <= 127)
 *    acc[m][n]  = sum_k xq[m][k] * wq[n][k]                    (exact int32)
 *    y[m][n]    = bf16_rne(((float)acc[m][n] * x_scale[m]) * w_scale[n])
 * An all-zero row gets scale 0 and all codes 0.  The definition takes the
 * rotation and the quotient exactly, with only the scale rounded (to fp32).
 * The kernels rotate with an fp32 fast Walsh-Hadamard transform and divide in
 * fp32, so a code can land one step away where the exact quotient sits at a
 * rounding boundary (a few codes in a million on Gaussian activations).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers, row-major and contiguous; bf16
 *    values are passed as their raw 16-bit patterns (uint16_t).
 *  - The caller owns every buffer and the stream.  The library never
 *    allocates or frees device memory and keeps no pointer after returning;
 *    its only global state is a lock-guarded memo of how many workgroups of
 *    each kernel a device holds at once.  Calls from several host threads
 *    and on different streams may run concurrently.
 *  - Work is enqueued on `stream` (0 = the null stream) without any host
 *    synchronisation; results are valid once the stream has reached them.
 *  - Arguments are validated on the host before anything is enqueued; on a
 *    non-zero status nothing has been written.  M == 0 is a successful no-op
 *    for every call that has an M.  N == 0 is a successful no-op for the
 *    calls over weight rows alone (convrot_quantize_weight,
 *    convrot_quantize_weight_i4_clip, convrot_dequantize_weight); the calls
 *    that multiply (the linears and the GEMMs) return CONVROT_ERR_SHAPE for
 *    N <= 0.
 *  - Tensor pointers must be 16-byte aligned; scale pointers 4-byte aligned.
 *  - Shapes: K % 16 == 0, K % group == 0, K <= CONVROT_MAX_K; int4 weights
 *    additionally need K % 32 == 0.  The calls that multiply (the linears
 *    and the GEMMs) accept M, N <= 2^30 with ceil(M/128) * ceil(N/128) < 2^31
 *    (summed over the outputs of a multi-output call).  group must be a power of two in
 *    [1, 256]; group 1 means no rotation (plain row-wise int8).  Unlike the
 *    converter described on "qwen3vl_8b_int8_convrot" ("Layer and group
 *    selection"), the library never silently falls back to group 1 when K is
 *    not a multiple of the group: it returns CONVROT_ERR_SHAPE.
 */
#ifndef CONVROT_H_
#define CONVROT_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CONVROT_MAX_K 32768

/* Status codes returned by every entry point. */
enum convrot_status {
  CONVROT_OK = 0,
  CONVROT_ERR_NULL = 1,      /* a required pointer is NULL */
  CONVROT_ERR_SHAPE = 2,     /* M < 0, N <= 0, K <= 0, K % 16, K % group, K % 32 for int4, K or M/N too large */
  CONVROT_ERR_GROUP = 3,     /* group is not a power of two in [1, 256] */
  CONVROT_ERR_ALIGN = 4,     /* a tensor pointer is not 16-byte aligned (scales: 4-byte) */
  CONVROT_ERR_WORKSPACE = 5, /* workspace smaller than the call's workspace-size function gives */
  CONVROT_ERR_DEVICE = 6,    /* the HIP runtime reported an error while enqueueing */
  CONVROT_ERR_DTYPE = 7,     /* unsupported w_dtype or bits value */
  CONVROT_ERR_ARG = 8,       /* a scalar argument is out of range (eps negative, NaN or infinite;
                                n_outs outside [1, CONVROT_MAX_OUTS]) */
  CONVROT_ERR_SCRATCH = 9    /* the input needs more than the allocation-free call's scratch area */
};

/* Weight dtypes accepted by convrot_quantize_weight. */
enum convrot_wdtype { CONVROT_W_F32 = 0, CONVROT_W_BF16 = 1 };

/*
 * convrot_quantize_weight -- offline weight preparation.
 * Rotates every row of w [N, K] per group and quantizes it per output row
 * ("MOSS-Image ... INT8" page, file table, row "Quantized"; "MossInt4",
 * "Format" for bits == 4).
 *   w        : [N, K] weights, fp32 (w_dtype 0) or bf16 bits (w_dtype 1).
 *   bits == 8: wq is int8 [N, K]; codes = round_half_away(rotated/scale),
 *              scale = absmax/127 (round-to-nearest; "Quantization Recipe":
 *              --simple).
 *   bits == 4: wq is uint8 [N, K/2]; byte j of a row holds column 2j in its
 *              low nibble and column 2j+1 in its high nibble, each a signed
 *              4-bit code in [-7, 7]; the row scale is c*absmax/7 for the c in
 *              {1.00, 0.99, ..., 0.50} (evaluated as absmax*(100-i)/700 in
 *              fp64, rounded to fp32) that minimises the row's sum of squared
 *              reconstruction error (fp64), ties to the larger c.
 *   w_scale  : fp32 [N], written.
 * Returns a convrot_status.
 */
int convrot_quantize_weight(const void *w, int w_dtype, int64_t N, int64_t K, int group, int bits,
                            void *wq, float *w_scale, hipStream_t stream);

/*
 * convrot_rotate_quant -- run-time activation rotation + per-token int8
 * quantization ("MOSS-Image ... INT8" page, file table, row "Matmul").
 *   x       : bf16 bits [M, K]  (read)
 *   xq      : int8 [M, K]       (written)
 *   x_scale : fp32 [M]          (written)
 */
int convrot_rotate_quant(const uint16_t *x, int64_t M, int64_t K, int group, int8_t *xq, float *x_scale,
                         hipStream_t stream);

/*
 * convrot_rmsnorm_rotate_quant -- the RMSNorm that feeds a linear, fused with
 * its rotation + per-token int8 quantization in one pass over x.  The
 * norm-then-quantize chain is the one the "MOSS-Image ... INT8" page
 * describes: its file table, row "Changed", lists the RMSNorm weights that the
 * SmoothQuant folding rewrote, and "How it was made" says those (1 + w)
 * weights absorbed the activation smoothing, so the norm's output is exactly
 * what the rotated linear quantizes.  Per row of x (fp32 arithmetic unless
 * stated):
 *    ms     = (float)(sum_k x[k]^2 / K)          (sum and quotient in fp64)
 *    r      = 1 / sqrtf(ms + eps)                (IEEE divide and square root)
 *    y[k]   = bf16_rne((x[k] * r) * (1 + norm_w[k]))
 *    (xq, x_scale) = rotate_quant(y)             (as convrot_rotate_quant)
 *   x       : bf16 bits [M, K]  (read)
 *   norm_w  : fp32 [K]          (read; the stored weight w, applied as 1 + w;
 *                                16-byte aligned like the tensors)
 *   eps     : finite, >= 0; with eps == 0 an all-zero row has no defined
 *             output (its y is NaN and its codes and scale are unspecified)
 *   xq      : int8 [M, K]       (written)
 *   x_scale : fp32 [M]          (written)
 *   y_norm  : bf16 bits [M, K]  (written if not NULL: the normalised rows,
 *             for a residual stream or a second consumer)
 * The fp64 sum may be formed in any order; the codes and scale equal
 * convrot_rotate_quant applied to y.
 */
int convrot_rmsnorm_rotate_quant(const uint16_t *x, const float *norm_w, float eps, int64_t M, int64_t K,
                                 int group, int8_t *xq, float *x_scale, uint16_t *y_norm, hipStream_t stream);

/*
 * convrot_workspace_size -- bytes of device workspace convrot_w8a8_linear and
 * convrot_w4a8_linear need for an [M, K] input: the int8 codes and the fp32
 * token scales, each rounded up to 256 bytes.  Returns 0 for M <= 0 or K <= 0.
 */
size_t convrot_workspace_size(int64_t M, int64_t K);

/*
 * convrot_w8a8_linear -- the ConvRot W8A8 linear ("MOSS-Image ... INT8" page,
 * file table, row "Matmul"): y = bf16(((xq . wq^T) * x_scale) * w_scale)
 * where (xq, x_scale) = rotate_quant(x).
 *   x        : bf16 bits [M, K]            (read)
 *   wq       : int8 [N, K], rotated codes  (read; from convrot_quantize_weight, bits 8)
 *   w_scale  : fp32 [N]                    (read)
 *   y        : bf16 bits [M, N]            (written)
 *   workspace: device buffer of at least convrot_workspace_size(M, K) bytes,
 *              16-byte aligned; its contents are scratch.
 */
int convrot_w8a8_linear(const uint16_t *x, int64_t M, int64_t K, const int8_t *wq, const float *w_scale,
                        int64_t N, int group, uint16_t *y, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * convrot_w4a8_linear -- the int4-weight / int8-activation variant ("MossInt4",
 * "Format": computation runs with 8-bit activations).  Identical to
 * convrot_w8a8_linear except that wq4 is uint8 [N, K/2] holding two signed
 * 4-bit codes per byte (low nibble = even column); a nibble is read as a
 * two's-complement value in [-8, 7].  Requires K % 32 == 0.
 */
int convrot_w4a8_linear(const uint16_t *x, int64_t M, int64_t K, const uint8_t *wq4, const float *w_scale,
                        int64_t N, int group, uint16_t *y, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * convrot_gemm_i8 -- the integer product and rescale on already-quantized
 * operands (the GEMM half of the linear, exposed so a caller can share one
 * quantized input across several weights and check the int32 accumulators).
 *   xq       : int8 [M, K]                     (read)
 *   x_scale  : fp32 [M]                        (read; may be NULL if y is NULL)
 *   wq       : int8 [N, K] (wbits 8) or uint8 [N, K/2] (wbits 4)   (read)
 *   w_scale  : fp32 [N]                        (read; may be NULL if y is NULL)
 *   acc_out  : int32 [M, N] accumulators       (written if not NULL)
 *   y        : bf16 bits [M, N]                (written if not NULL)
 * At least one of acc_out and y must be non-NULL.
 */
int convrot_gemm_i8(const int8_t *xq, const float *x_scale, const void *wq, int wbits, const float *w_scale,
                    int64_t M, int64_t N, int64_t K, int32_t *acc_out, uint16_t *y, hipStream_t stream);

/*
 * convrot_quantize_weight_i4_clip -- convrot_quantize_weight(bits = 4) that
 * also writes, per row, the index i of the winning clip candidate
 * (c = 1 - i/100) into clip_index (int32 [N], device).  Same arguments and
 * errors otherwise; exposed so the clip search can be checked row by row.
 */
int convrot_quantize_weight_i4_clip(const void *w, int w_dtype, int64_t N, int64_t K, int group, uint8_t *wq4,
                                    float *w_scale, int32_t *clip_index, hipStream_t stream);

/*
 * Weight-only (dequant) path ("MOSS-Image ... INT8" page, file table row
 * "Matmul": a weight-only mode that expands the codes back into a bf16
 * weight and multiplies in bf16;
 * "qwen3.5_4b_int8_convrot" loads the checkpoints through that path).  The
 * activations are not quantized.
 */

/*
 * convrot_dequantize_weight -- undo the rotation of stored codes:
 *   W^[n][k] = bf16(fp32(sum_j code[n][j] * w_scale[n] * H[j][k]))  per group,
 * the inverse of convrot_quantize_weight up to its rounding (H is its own
 * inverse).  The codes' transform is exact; for even log2(group) the value
 * is rounded once to fp32 (then to bf16), for odd log2(group) the 1/sqrt(g)
 * adds one fp32 rounding.
 *   wq      : int8 [N, K] (wbits 8) or uint8 [N, K/2] (wbits 4, K % 32 == 0)
 *   w_scale : fp32 [N]
 *   w_out   : bf16 bits [N, K]   (written)
 */
int convrot_dequantize_weight(const void *wq, int wbits, const float *w_scale, int64_t N, int64_t K, int group,
                              uint16_t *w_out, hipStream_t stream);

/*
 * convrot_gemm_bf16 -- y = bf16_rne(x . w^T) with fp32 accumulation on the
 * matrix cores (v_mfma_f32_32x32x16_bf16); the summation order is the
 * hardware's, so y differs from the exactly rounded product by the fp32
 * accumulation error (at most about K * 2^-24 * sum|x*w| per output).
 *   x : bf16 bits [M, K], w : bf16 bits [N, K], y : bf16 bits [M, N]
 */
int convrot_gemm_bf16(const uint16_t *x, const uint16_t *w, int64_t M, int64_t N, int64_t K, uint16_t *y,
                      hipStream_t stream);

/* Workspace bytes convrot_dequant_linear needs: the bf16 weight, rounded up
 * to 256 bytes.  0 for N <= 0 or K <= 0. */
size_t convrot_dequant_workspace_size(int64_t N, int64_t K);

/*
 * convrot_dequant_linear -- the weight-only linear: dequantize wq into the
 * workspace (convrot_dequantize_weight), then y = convrot_gemm_bf16(x, W^).
 * Arguments as convrot_w8a8_linear / convrot_w4a8_linear (wbits 8 or 4);
 * workspace: at least convrot_dequant_workspace_size(N, K) bytes, 16-byte
 * aligned.  A caller that keeps W^ resident calls convrot_gemm_bf16 alone.
 */
int convrot_dequant_linear(const uint16_t *x, int64_t M, int64_t K, const void *wq, int wbits,
                           const float *w_scale, int64_t N, int group, uint16_t *y, void *workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * Several linears that read the same input: the q, k and v projections of an
 * attention block, or the gate and up projections of an MLP (the per-layer
 * projection list of "craftingmod/Qwen3-VL-8B-Heretic-INT8", "Quantization
 * metadata", names them; each is its own ConvRot int8 matrix as in
 * "MOSS-Image ... INT8", file table row "Quantized").  The input is rotated
 * and quantized once, and one GEMM launch computes every output: the column
 * tiles of all weight matrices form one grid, so small projections (k, v)
 * no longer leave compute units idle.  Each output is exactly what the
 * single-output call gives for the same weight.
 */
#define CONVROT_MAX_OUTS 8

/* One weight matrix of a multi-output call and where its results go. */
typedef struct convrot_linear_out {
  const void *wq;        /* int8 [N, K] (wbits 8) or uint8 [N, K/2] (wbits 4), 16-byte aligned */
  const float *w_scale;  /* fp32 [N]; may be NULL when y is NULL */
  int64_t N;             /* rows of wq, in (0, 2^30] */
  int32_t *acc_out;      /* int32 [M, N] accumulators, or NULL */
  uint16_t *y;           /* bf16 bits [M, N], or NULL */
} convrot_linear_out;

/*
 * convrot_gemm_i8_multi -- convrot_gemm_i8 for n_outs (1..CONVROT_MAX_OUTS)
 * weight matrices sharing xq [M, K] and x_scale [M], all of bit width wbits.
 * Every output must ask for the same results: y in all of them or in none,
 * likewise acc_out (CONVROT_ERR_NULL otherwise), and at least one of the
 * two.  outs is a HOST array, read before the call returns.
 */
int convrot_gemm_i8_multi(const int8_t *xq, const float *x_scale, int wbits, int64_t M, int64_t K,
                          const convrot_linear_out *outs, int n_outs, hipStream_t stream);

/*
 * convrot_linear_multi -- rotate + quantize x [M, K] once (as
 * convrot_rotate_quant) into the workspace, then convrot_gemm_i8_multi with
 * the bf16 epilogue: y_o = bf16(((xq . wq_o^T) * x_scale) * w_scale_o) for
 * every output o.  wbits 8 (W8A8) or 4 (W4A8, K % 32 == 0).  Every output
 * needs y and w_scale; acc_out must be NULL in all of them or set in all.
 * workspace: at least convrot_workspace_size(M, K) bytes, 16-byte aligned.
 */
int convrot_linear_multi(const uint16_t *x, int64_t M, int64_t K, int group, int wbits,
                         const convrot_linear_out *outs, int n_outs, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * convrot_w8a8_linear_noalloc -- convrot_w8a8_linear for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops that
 * forbid allocation, harnesses that own every allocation.  It takes no
 * workspace: the int8 codes and fp32 token scales of x go to a scratch area
 * the library holds in device memory, CONVROT_NOALLOC_SCRATCH_BYTES per GPU
 * (a file-scope device array, present on every GPU the library runs on until
 * the process ends).  The call itself allocates nothing and calls no
 * allocating routine; its first call on a GPU looks up that GPU's scratch
 * address once.  Arguments, results and errors as convrot_w8a8_linear, and
 * bit for bit the same output; an input whose convrot_workspace_size(M, K)
 * exceeds CONVROT_NOALLOC_SCRATCH_BYTES returns CONVROT_ERR_SCRATCH before
 * anything is enqueued.  Every call on one GPU shares that GPU's scratch
 * area, so calls that overlap on one GPU (several streams or host threads)
 * race: the caller serialises them.  Nothing in the area needs clearing
 * between calls (each call writes every byte it reads).
 */
#define CONVROT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int convrot_w8a8_linear_noalloc(const uint16_t *x, int64_t M, int64_t K, const int8_t *wq, const float *w_scale,
                                int64_t N, int group, uint16_t *y, hipStream_t stream);

/* Static, human-readable text for a status code (never NULL). */
const char *convrot_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int convrot_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_H_ */
