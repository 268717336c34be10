/*
 * qmm.h — C ABI of the MI355X (gfx950) GGUF block-quantized matrix product.
 *
 * The library computes the product that the page "The GGML ecosystem, and
 * where synapse fits" describes in §5 "Quantization", subsection "Products:
 * weights against quantized activations": the activation rows are quantized
 * once to the weight type's vec_dot_type (Q8_0 for Q4_0 and Q8_0 weights,
 * Q8_K for the K-quants), and each weight block is dotted with the matching
 * activation block in integer arithmetic, with only the block scales in
 * float.  Block formats are the rows of that section's format table.
 *
 * Orientation (page "ggml", examples/simple: ggml_mul_mat(A, B^T) = C^T):
 *   W  : M rows x K inputs, each row K/B consecutive blocks (a GGUF weight
 *        tensor with ne = [K, M]; page "The GGML ecosystem...", §2 "GGUF:
 *        the file format", tensor info: rows are contiguous);
 *   xq : N rows x K, each row K/Bx blocks of the activation type;
 *   y  : N x M fp32, y[n*M + m] = sum_k w[m][k] * x[n][k].
 *
 * Conventions for every call below:
 *   - Pointers named as device pointers must point to device memory (HIP);
 *     the caller owns every buffer.  The library never allocates, frees,
 *     copies to the host or synchronizes inside these calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it and runs asynchronously.
 *   - Inputs are validated before anything is enqueued; on any error no work
 *     is enqueued and no output byte is written.  Nothing throws.
 *   - Base pointers must be 16-byte aligned (QMM_ERR_ALIGN otherwise).
 *   - Sizes must be positive and K a multiple of the block size of every
 *     format involved (QMM_ERR_SHAPE otherwise): rows whose length is not a
 *     multiple of a format's block size cannot use that format (page "The
 *     GGML ecosystem...", §3, llama-quantize's fallback rule).
 *   - Activations must be finite; block bytes may hold any pattern (a NaN
 *     or Inf fp16 scale propagates per IEEE arithmetic).
 *   - Calls are stateless and may be made from several host threads.
 *   - Codec results (quantize, dequantize) are bit-exact and deterministic.
 *     qmm_mul_mat results are deterministic for a given library build and
 *     shape; they differ from an exact sum only by float summation order
 *     (page "The GGML ecosystem...", §5: products match "apart from float
 *     summation order").
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Block formats (this library's own codes; the pages print no type codes).
 * Values per block / bytes per block, from the format table:
 *   Q4_0  32 / 18   fp16 d; 32 four-bit quants; w = d (q - 8)
 *   Q8_0  32 / 34   fp16 d; 32 int8 quants;     w = d q
 *   Q4_K 256 / 144  fp16 d, dmin; 8 sub-blocks of 32 with 6-bit scale and
 *                   min; w = d sc q - dmin m
 *   Q6_K 256 / 210  fp16 d; 16 sub-blocks of 16 with int8 scales; 6-bit
 *                   quants in a 4-bit and a 2-bit plane; w = d sc (q - 32)
 *                   (the offset 32 is this library's reading: the table
 *                   gives no Q6_K formula)
 *   Q8_K 256 / 292  fp32 d; 256 int8 quants; 16 int16 sums of 16 quants;
 *                   activations only
 *   Q5_0  32 / 22   fp16 d; a 32-bit word of fifth bits; 32 four-bit low
 *                   parts; w = d (q - 16).  The type for rows whose length
 *                   is not a multiple of 256 (§3, fallback rule).
 * Bit arrangement inside a block: GGUF's on-disk arrangement (the pages give
 * field lists only): Q4_0 [d][qs:16] with element e<16 in the low nibble of
 * qs[e] and e>=16 in the high nibble of qs[e-16]; Q8_0 [d][qs:32];
 * Q4_K [d][dmin][scales:12][qs:128]; Q6_K [ql:128][qh:64][scales:16][d];
 * Q8_K [d:f32][qs:256][bsums:16 x int16]; Q5_0 [d][qh:4][qs:16] with the
 * low four bits arranged as Q4_0's nibbles and the fifth bit of element e in
 * bit e of the little-endian qh (this library's reading). */
typedef enum {
    QMM_Q4_0 = 1,
    QMM_Q8_0 = 2,
    QMM_Q4_K = 3,
    QMM_Q6_K = 4,
    QMM_Q8_K = 5,
    QMM_Q5_0 = 6
} qmm_type;

/* Status codes. */
enum {
    QMM_OK = 0,
    QMM_ERR_TYPE = -1,        /* unknown type code                              */
    QMM_ERR_SHAPE = -2,       /* size <= 0, K % block != 0, or size overflow    */
    QMM_ERR_NULL = -3,        /* a required pointer is NULL                     */
    QMM_ERR_ALIGN = -4,       /* a base pointer is not 16-byte aligned          */
    QMM_ERR_UNSUPPORTED = -5, /* valid type, but not for this operation         */
    QMM_ERR_HIP = -6          /* the HIP runtime reported an error on launch    */
};

/* Values per block (32 or 256); 0 for an unknown type. */
int qmm_block_size(int type);
/* Bytes per block (18, 34, 144, 210, 292, 22); 0 for an unknown type. */
size_t qmm_block_bytes(int type);
/* Bytes of one row of K values; 0 if the type is unknown, K <= 0 or K is not
 * a multiple of the block size. */
size_t qmm_row_bytes(int type, int64_t K);
/* The activation type a weight type is dotted with (page "The GGML
 * ecosystem...", §5, vec_dot_type): Q4_0, Q5_0, Q8_0 -> Q8_0; Q4_K, Q6_K -> Q8_K.
 * Returns QMM_ERR_TYPE or QMM_ERR_UNSUPPORTED (Q8_K is never a weight). */
int qmm_vec_dot_type(int wtype);

/* Round-to-nearest quantization of activations (§5, from_float: activations
 * are converted to the vec_dot_type once per row, before the product).
 *   dst : QMM_Q8_0 or QMM_Q8_K (else QMM_ERR_UNSUPPORTED)
 *   x   : device, N x K fp32, row-major
 *   xq  : device, N x qmm_row_bytes(dst, K) bytes, written
 * Per block of B values: d = amax/127 in fp32, id = 1/d (0 when d = 0),
 * q = roundf(x*id) (ties away from zero; the rounding rule and the use of 1/d
 * are this library's readings, the pages do not state them); Q8_0 stores
 * fp16(d) (round to nearest even), Q8_K stores d as fp32 and the 16 sums of
 * each run of 16 quants. */
int qmm_quantize_act(int dst, const float* x, void* xq, int64_t N, int64_t K, void* stream);

/* Round-to-nearest quantization of fp32 rows into any format this library
 * can encode: QMM_Q8_0 and QMM_Q8_K as in qmm_quantize_act, and QMM_Q4_0 for
 * weights (per 32 values, m = the value of largest magnitude, the first on
 * ties; d = m / -8; q = clamp(roundf(x*(1/d)), -8, 7) + 8; fp16(d) stored).
 * The Q4_0 rule is this library's reading: the pages print Q4_0's decode
 * formula w = d (q - 8) but no encoder.  K-quant weights are not encoded
 * (QMM_ERR_UNSUPPORTED).  Layout and errors as qmm_quantize_act. */
int qmm_quantize(int dst, const float* x, void* out, int64_t rows, int64_t K, void* stream);

/* Expand blocks to fp32 (§5: each format's dequantizer, used for embedding
 * lookups and norm weights).  All five types.
 *   blocks : device, rows x qmm_row_bytes(type, K) bytes
 *   out    : device, rows x K fp32, written
 * Element values, computed in fp32 in this order: Q4_0 d*(q-8); Q5_0 d*(q-16); Q8_0 d*q;
 * Q4_K (d*sc)*q - (dmin*m); Q6_K (d*sc)*(q-32); Q8_K d*q.  Every product is
 * exact in fp32 except Q8_K's, so results are the exact value rounded once. */
int qmm_dequantize(int type, const void* blocks, float* out, int64_t rows, int64_t K, void* stream);

/* y = W x^T over quantized weights and pre-quantized activations.
 *   wtype : QMM_Q4_0, QMM_Q5_0, QMM_Q8_0, QMM_Q4_K or QMM_Q6_K
 *   W     : device, M x qmm_row_bytes(wtype, K) bytes of raw blocks
 *   xq    : device, N x qmm_row_bytes(qmm_vec_dot_type(wtype), K) bytes
 *   y     : device, N x M fp32, written (y[n*M + m])
 * Per block: an exact integer dot product of the quants, then the block's
 * float scales; Q4_K and Q6_K take their min and offset terms from the Q8_K
 * block's 16-wide sums.  Accumulation is fp32.  Small N runs the
 * bandwidth-bound GEMV kernels (in groups of up to 8 activation rows), larger
 * N the int8-MFMA GEMM kernels; the switch is at the crossover measured on
 * MI355X: for Q6_K N > 4 when M > 24576, N > 6 when 8192 < M <= 24576,
 * N > 54 when M < 2048, else N > 30; for Q4_K N > 4 when
 * M > 8192 and K < 4096, else N > 2 (Q4_K with N <= 32
 * takes narrow MFMA kernels, on 32- or 16-row tiles, that split K over the
 * waves of a workgroup); for Q4_0 / Q5_0 / Q8_0, N > 8 / 8 / 7 when
 * M > 24576, N > 12 / 12 / 10 when 8192 < M <= 24576, else, when K < 2048, N > 21 / 23 / 26 for M <= 1024,
 * N > 14 / 16 / 15 for M < 4096 and N > 7 / 8 / 7 above; N > 17 / 19 / 17
 * when K = 2048; N > 28 / 32 / 26 when K <= 4096 and M >= 4096,
 * N > 23 / 26 / 26 when K <= 4096 and M < 4096; for wider rows
 * N > 30 / 33 / 31 when M < 2048 and N > 47 / 51 / 45 above. */
int qmm_mul_mat(int wtype, const void* W, const void* xq, float* y,
                int64_t M, int64_t N, int64_t K, void* stream);

/* qmm_mul_mat with the kernel family chosen by the caller:
 *   algo 0 = automatic (as qmm_mul_mat), 1 = GEMV kernels (any N, run in
 *   column groups of at most 8), 2 = int8-MFMA GEMM kernels (any N, every
 *   weight type).
 * Results of the two families agree to float summation order.  Any other
 * algo value returns QMM_ERR_UNSUPPORTED. */
int qmm_mul_mat_algo(int wtype, const void* W, const void* xq, float* y,
                     int64_t M, int64_t N, int64_t K, int algo, void* stream);

/* The kernel family the automatic choice of qmm_mul_mat takes for these
 * sizes: 1 = GEMV kernels, 2 = int8-MFMA GEMM kernels (for Q4_K with
 * N <= 32 the narrow ones); 0 for a type or shape qmm_mul_mat would reject.
 * Host logic only: no GPU work, no pointers. */
int qmm_mul_mat_choice(int wtype, int64_t M, int64_t N, int64_t K);

/* Several weight matrices that share K and the activation rows, in one
 * launch: e.g. the q, k and v projections of a layer, or its gate and up
 * projections, which all read the same normalized activations.  Each
 * matrix i computes y[i] = W[i] x^T exactly as qmm_mul_mat would (the same
 * values, bit for bit), with M[i] rows.
 *   count      : 1..4 matrices (QMM_ERR_SHAPE otherwise)
 *   W, y, M    : host arrays of count device pointers / row counts
 *   x          : device; with x_is_f32 == 0, N rows of quantized activations
 *                (as for qmm_mul_mat); with x_is_f32 != 0, N rows of K fp32
 *                values, which the launch quantizes itself to the
 *                vec_dot_type with exactly the rule and results of
 *                qmm_quantize_act (the quantized rows are not written out)
 * The fp32 form needs N <= 8 and K a multiple of 256; otherwise it returns
 * QMM_ERR_UNSUPPORTED.  Other errors as qmm_mul_mat. */
int qmm_mul_mat_multi(int wtype, int count, const void* const* W, float* const* y, const int64_t* M,
                      const void* x, int x_is_f32, int64_t N, int64_t K, void* stream);

/* Static text for a status code. */
const char* qmm_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* QMM_H */
