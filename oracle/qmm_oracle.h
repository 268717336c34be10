/*
 * qmm_oracle.h — plain, slow CPU oracle for the GGUF block-quantized matrix
 * product.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg may call it; the product path never does.
 *
 * Sources (all on the page "The GGML ecosystem, and where synapse fits"):
 *   - §5 "Quantization", the format table: block sizes, byte counts and the
 *     element formulas of Q4_0, Q8_0, Q4_K, Q6_K and Q8_K.
 *   - §5, "Products: weights against quantized activations": activations are
 *     quantized once per row to the weight type's vec_dot_type (Q8_0 for
 *     Q4_0/Q8_0, Q8_K for the K-quants) and dotted block by block in integer
 *     arithmetic, with only the block scales in float.
 *   - §2 "GGUF: the file format": a weight matrix with ne = [cols, rows] stores
 *     each row contiguously, as consecutive blocks.
 * Orientation of the product follows the page "ggml", examples/simple
 * ("ggml_mul_mat(A, B^T) = C^T"): y[n][m] = sum_k W[m][k] * x[n][k].
 *
 * Every function here is independent of the GPU library: no shared headers,
 * tables or helpers.  Floating point runs in fp64 unless a step is defined in
 * fp32 (the activation quantizers and the fp32 dequantizer), and the library
 * is built with -ffp-contract=off.
 *
 * Block layouts: the pages list the fields and byte counts only; the bit
 * arrangement inside a block is the GGUF on-disk reading described next to
 * each decoder in qmm_oracle.c.  Parity with a GGUF producer's bytes is
 * unpinned (no GGUF producer is available to compare with).
 */
#ifndef QMM_ORACLE_H
#define QMM_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Oracle type codes (its own; numerically equal to the library's by choice
 * of both, not by a shared header). */
enum { ORC_Q4_0 = 1, ORC_Q8_0 = 2, ORC_Q4_K = 3, ORC_Q6_K = 4, ORC_Q8_K = 5, ORC_Q5_0 = 6 };

int    orc_block_size(int type);   /* values per block; 0 if unknown */
size_t orc_block_bytes(int type);  /* bytes per block; 0 if unknown  */

/* IEEE 754 binary16 <-> binary32, written from the format definition.
 * Decode is exact (subnormals, signed zero, Inf; NaN stays NaN).
 * Encode rounds to nearest, ties to even, with subnormals; overflow -> Inf. */
float    orc_fp16_to_f32(uint16_t h);
uint16_t orc_f32_to_fp16(float f);
void     orc_fp16_to_f32_n(const uint16_t* h, float* out, int64_t n);
void     orc_f32_to_fp16_n(const float* f, uint16_t* out, int64_t n);

/* Round-to-nearest activation quantizers (rows x K fp32, K contiguous).
 * Q8_0: per 32 values, d = amax/127 (fp32), id = 1/d (0 if d = 0),
 *       q = roundf(x*id) (ties away from zero), stored as fp16(d) + 32 int8.
 * Q8_K: per 256 values, same steps, d stored as fp32, plus 16 int16 sums of
 *       each run of 16 quants.
 * Returns 0, or -1 if K is not a multiple of the block size. */
int orc_quantize_q8_0(const float* x, void* out, int64_t rows, int64_t K);
int orc_quantize_q8_k(const float* x, void* out, int64_t rows, int64_t K);

/* Q4_0 weight encoder (used to build Q4_0 test matrices from fp32 weights):
 * per 32 values, m = the value of largest magnitude (first one on ties),
 * d = m / -8, id = 1/d (0 if d = 0), q = clamp(roundf(x*id), -8, 7) + 8,
 * stored as fp16(d) + 16 bytes of nibbles. */
int orc_quantize_q4_0(const float* x, void* out, int64_t rows, int64_t K);

/* Dequantize rows x K values of `type` blocks into fp32, every element
 * computed in fp32 in the fixed order given next to each decoder. */
int orc_dequantize_f32(int type, const void* blocks, float* out, int64_t rows, int64_t K);
/* The exact real value of every element, in fp64. */
int orc_dequantize_f64(int type, const void* blocks, double* out, int64_t rows, int64_t K);

/* Plain definition of the product: y[n][m] = sum_k w[m][k] * x[n][k] with w
 * and x the exact values the blocks encode, accumulated in fp64.
 * wtype in {Q4_0, Q8_0, Q4_K, Q6_K}; xq holds N rows of its vec_dot_type.
 * T (may be NULL) receives the per-output magnitude sum used for the
 * tolerance: sum_k |w_k||x_k|, and for Q4_K sum_k |x_k|(|d sc q_k| + |dmin m|)
 * because that format's product sums its scale part and min part apart.
 * y and T are N x M, M contiguous.  Parallel over output rows (OpenMP). */
int orc_mul_mat(int wtype, const void* W, const void* xq, double* y, double* T,
                int64_t M, int64_t N, int64_t K);

/* The same product computed the way the method does: an exact integer dot
 * per block (int64), then the block's float scales (in fp64), then the sum
 * over blocks.  Q4_K and Q6_K use the activation block's stored 16-wide sums. */
int orc_mul_mat_blockwise(int wtype, const void* W, const void* xq, double* y,
                          int64_t M, int64_t N, int64_t K);

/* Q4_K sub-block scale/min and Q6_K element decoding, exposed for the
 * exhaustive bit-layout tests. */
void orc_q4k_scale_min(const uint8_t scales12[12], int j, int* sc, int* m);
int  orc_q6k_quant(const uint8_t* block210, int e); /* unsigned 6-bit q of element e */
/* Vector forms: n arrays of 12 scale bytes -> n x 8 scales and mins;
 * n Q6_K blocks -> n x 256 unsigned quants. */
void orc_q4k_scale_min_n(const uint8_t* scales12, int64_t n, int32_t* sc, int32_t* m);
void orc_q6k_quant_n(const uint8_t* blocks, int64_t n, uint8_t* q);
/* n Q5_0 blocks -> n x 32 unsigned 5-bit quants. */
void orc_q5_0_quant_n(const uint8_t* blocks, int64_t n, uint8_t* q);

/* Threads the OpenMP runtime will use (for the CPU baseline report). */
int orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
