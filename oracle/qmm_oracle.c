/*
 * qmm_oracle.c — plain CPU oracle for the GGUF block-quantized matrix
 * product (Q4_0, Q5_0, Q8_0, Q4_K, Q6_K weights; Q8_0 and Q8_K activations).
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  It shares no code with the GPU path.
 *
 * What it follows (page "The GGML ecosystem, and where synapse fits", §5
 * "Quantization"):
 *   - the format table: Q4_0 = fp16 d + 32 four-bit quants, w = d(q-8), 18 B;
 *     Q5_0 = fp16 d + a 32-bit word of fifth bits + 32 four-bit low parts,
 *     w = d(q-16), 22 B;
 *     Q8_0 = fp16 d + 32 int8, w = d q, 34 B; Q4_K = fp16 d, dmin, eight
 *     32-wide sub-blocks with a 6-bit scale and a 6-bit min each,
 *     w = d sc q - dmin m, 144 B; Q6_K = fp16 d, sixteen 16-wide sub-blocks
 *     with int8 scales, 6-bit quants split into a 4-bit and a 2-bit plane,
 *     210 B; Q8_K = fp32 d, 256 int8, sixteen int16 sums of 16, 292 B,
 *     activations only;
 *   - "Products: weights against quantized activations": the activation row
 *     is quantized once to the weight's vec_dot_type, then each weight block
 *     is dotted with the matching activation block in integers, and only the
 *     block scales are float.
 * Open points and the reading taken for each:
 *   - bit arrangement inside blocks: the pages give field lists only; the
 *     arrangement used is GGUF's on-disk one, stated at each decoder below.
 *     Parity with a GGUF producer's bytes is unpinned.
 *   - Q6_K element formula (not printed): w = d * sc * (q - 32), q the
 *     unsigned 6-bit quant, continuing the "q - 8" of the 4-bit Q4_0 and the
 *     "q - 16" of the 5-bit Q5_0 rows of the same table.
 *   - activation rounding ("round to nearest", rule unstated): d = amax/127
 *     in fp32, id = 1/d once per block (0 when d = 0), q = roundf(x * id),
 *     i.e. ties away from zero; the fp32 d (not its fp16 copy) is used.
 *   - Q8_K scale: the same rule as Q8_0, stored as fp32.
 */
#include "qmm_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ sizes */

int orc_block_size(int type) {
    switch (type) {
    case ORC_Q4_0: case ORC_Q5_0: case ORC_Q8_0: return 32;
    case ORC_Q4_K: case ORC_Q6_K: case ORC_Q8_K: return 256;
    default: return 0;
    }
}

size_t orc_block_bytes(int type) {
    switch (type) {
    case ORC_Q4_0: return 18;   /* 2 (d) + 16 (32 nibbles)                   */
    case ORC_Q5_0: return 22;   /* 2 (d) + 4 (32 fifth bits) + 16 (nibbles)  */
    case ORC_Q8_0: return 34;   /* 2 (d) + 32 (int8)                         */
    case ORC_Q4_K: return 144;  /* 2 (d) + 2 (dmin) + 12 (scales) + 128 (qs) */
    case ORC_Q6_K: return 210;  /* 128 (ql) + 64 (qh) + 16 (scales) + 2 (d)  */
    case ORC_Q8_K: return 292;  /* 4 (d) + 256 (qs) + 32 (16 x int16 sums)   */
    default: return 0;
    }
}

/* ------------------------------------------------------------------- fp16 */
/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Exponent field 0 holds zero and the subnormals (m * 2^-24); field 31
 * holds Inf (fraction 0) and NaN. */

float orc_fp16_to_f32(uint16_t h) {
    int sign = h >> 15;
    int ef = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (ef == 0)
        v = ldexp((double)m, -24);
    else if (ef == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), ef - 25);
    return (float)(sign ? -v : v);
}

uint16_t orc_f32_to_fp16(float f) {
    uint32_t bits;
    memcpy(&bits, &f, 4);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    if (isnan(f)) return (uint16_t)(sign | 0x7E00u | ((bits >> 13) & 0x3FFu));
    if (isinf(f)) return (uint16_t)(sign | 0x7C00u);
    double a = fabs((double)f);
    if (a == 0.0) return sign;
    /* binade: a in [2^E, 2^(E+1)); the subnormal range shares the quantum of
     * the smallest normal binade (E = -14). */
    int e2;
    (void)frexp(a, &e2);
    int E = e2 - 1;
    if (E < -14) E = -14;
    double quantum = ldexp(1.0, E - 10);
    double n = a / quantum;             /* exact: scaling by a power of two */
    double fl = floor(n);
    double frac = n - fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    if (fl >= 2048.0) { fl = 1024.0; E += 1; }
    if (E > 15) return (uint16_t)(sign | 0x7C00u);        /* overflow */
    if (fl < 1024.0) return (uint16_t)(sign | (uint16_t)fl); /* subnormal */
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(fl - 1024.0));
}

void orc_fp16_to_f32_n(const uint16_t* h, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp16_to_f32(h[i]);
}

void orc_f32_to_fp16_n(const float* f, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_fp16(f[i]);
}

static float rd_fp16(const uint8_t* p) { return orc_fp16_to_f32((uint16_t)(p[0] | (p[1] << 8))); }
static void wr_fp16(uint8_t* p, float v) {
    uint16_t h = orc_f32_to_fp16(v);
    p[0] = (uint8_t)(h & 0xFF);
    p[1] = (uint8_t)(h >> 8);
}
static float rd_f32(const uint8_t* p) { float v; memcpy(&v, p, 4); return v; }
static int16_t rd_i16(const uint8_t* p) { return (int16_t)(uint16_t)(p[0] | (p[1] << 8)); }

/* ------------------------------------------------ activation quantization */

/* One round-to-nearest block of n values: d = amax/127, id = 1/d,
 * q = roundf(x*id).  A NaN product (0 * Inf, reachable only when d is so
 * small that 1/d overflows) gives q = 0; the clamp keeps q in [-127, 127]. */
static float rtn_block(const float* x, int n, int8_t* q) {
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    float d = amax / 127.0f;
    float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    for (int i = 0; i < n; ++i) {
        float t = x[i] * id;
        float r = roundf(t);
        int v;
        if (r != r) v = 0;
        else if (r > 127.0f) v = 127;
        else if (r < -127.0f) v = -127;
        else v = (int)r;
        q[i] = (int8_t)v;
    }
    return d;
}

int orc_quantize_q8_0(const float* x, void* out, int64_t rows, int64_t K) {
    if (K % 32) return -1;
    uint8_t* o = (uint8_t*)out;
    int64_t nb = K / 32;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            uint8_t* blk = o + (r * nb + b) * 34;
            int8_t q[32];
            float d = rtn_block(x + r * K + b * 32, 32, q);
            wr_fp16(blk, d);
            memcpy(blk + 2, q, 32);
        }
    return 0;
}

int orc_quantize_q8_k(const float* x, void* out, int64_t rows, int64_t K) {
    if (K % 256) return -1;
    uint8_t* o = (uint8_t*)out;
    int64_t nb = K / 256;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            uint8_t* blk = o + (r * nb + b) * 292;
            int8_t q[256];
            float d = rtn_block(x + r * K + b * 256, 256, q);
            memcpy(blk, &d, 4);
            memcpy(blk + 4, q, 256);
            for (int j = 0; j < 16; ++j) {
                int s = 0;
                for (int i = 0; i < 16; ++i) s += q[16 * j + i];
                int16_t s16 = (int16_t)s;
                memcpy(blk + 260 + 2 * j, &s16, 2);
            }
        }
    return 0;
}

/* Q4_0 weight encoder: the extreme value m (sign kept) maps to level -8, so
 * d = m / -8; q = clamp(roundf(x * (1/d)), -8, 7) + 8. */
int orc_quantize_q4_0(const float* x, void* out, int64_t rows, int64_t K) {
    if (K % 32) return -1;
    uint8_t* o = (uint8_t*)out;
    int64_t nb = K / 32;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const float* xb = x + r * K + b * 32;
            uint8_t* blk = o + (r * nb + b) * 18;
            float amax = 0.0f, m = 0.0f;
            for (int i = 0; i < 32; ++i)
                if (fabsf(xb[i]) > amax) { amax = fabsf(xb[i]); m = xb[i]; }
            float d = m / -8.0f;
            float id = (d != 0.0f) ? 1.0f / d : 0.0f;
            int q[32];
            for (int i = 0; i < 32; ++i) {
                float rr = roundf(xb[i] * id);
                if (rr != rr) rr = 0.0f;
                if (rr < -8.0f) rr = -8.0f;
                if (rr > 7.0f) rr = 7.0f;
                q[i] = (int)rr + 8;
            }
            wr_fp16(blk, d);
            for (int j = 0; j < 16; ++j) blk[2 + j] = (uint8_t)(q[j] | (q[j + 16] << 4));
        }
    return 0;
}

/* --------------------------------------------------------- block decoders */
/* GGUF arrangements (the reading taken; little-endian multi-byte fields):
 *  Q4_0 [d:2][qs:16]        element e<16 = low nibble of qs[e],
 *                           e>=16 = high nibble of qs[e-16]
 *  Q5_0 [d:2][qh:4][qs:16]  low four bits as Q4_0's nibbles (in qs),
 *                           fifth bit of element e = bit e of the
 *                           little-endian 32-bit qh
 *  Q8_0 [d:2][qs:32 int8]
 *  Q4_K [d:2][dmin:2][scales:12][qs:128]  sub-block j = e/32 uses the
 *        32 bytes qs[32(j/2) ...], low nibbles for even j, high for odd j
 *  Q6_K [ql:128][qh:64][scales:16 int8][d:2]
 *  Q8_K [d:4 fp32][qs:256 int8][bsums:16 int16]                             */

static int q4_0_quant(const uint8_t* blk, int e) {
    const uint8_t* qs = blk + 2;
    return e < 16 ? (qs[e] & 0xF) : (qs[e - 16] >> 4);
}

static int q5_0_quant(const uint8_t* blk, int e) {
    const uint8_t* qs = blk + 6;
    uint32_t qh = (uint32_t)blk[2] | ((uint32_t)blk[3] << 8) | ((uint32_t)blk[4] << 16) | ((uint32_t)blk[5] << 24);
    int lo = e < 16 ? (qs[e] & 0xF) : (qs[e - 16] >> 4);
    return lo | (int)(((qh >> e) & 1u) << 4);
}

void orc_q5_0_quant_n(const uint8_t* blocks, int64_t n, uint8_t* q) {
    for (int64_t i = 0; i < n; ++i)
        for (int e = 0; e < 32; ++e) q[32 * i + e] = (uint8_t)q5_0_quant(blocks + 22 * i, e);
}

/* The 12 scale bytes hold eight 6-bit scales and eight 6-bit mins.  Bytes
 * 0-3 carry sc0-3 in their low six bits, bytes 4-7 carry m0-3 likewise;
 * bytes 8-11 carry the low four bits of sc4-7 (low nibble) and of m4-7 (high
 * nibble); the top two bits of bytes 0-3 are bits 4-5 of sc4-7 and the top
 * two bits of bytes 4-7 are bits 4-5 of m4-7. */
void orc_q4k_scale_min(const uint8_t s[12], int j, int* sc, int* m) {
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 0xF) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

void orc_q4k_scale_min_n(const uint8_t* s, int64_t n, int32_t* sc, int32_t* m) {
    for (int64_t i = 0; i < n; ++i)
        for (int j = 0; j < 8; ++j) {
            int a, b;
            orc_q4k_scale_min(s + 12 * i, j, &a, &b);
            sc[8 * i + j] = a;
            m[8 * i + j] = b;
        }
}

static int q4_k_quant(const uint8_t* blk, int e) {
    const uint8_t* qs = blk + 16;
    int j = e / 32, l = e % 32;
    uint8_t b = qs[32 * (j / 2) + l];
    return (j & 1) ? (b >> 4) : (b & 0xF);
}

/* Q6_K: each half h of 128 elements uses ql[64h .. 64h+64) and
 * qh[32h .. 32h+32).  Within a half, quarter c = (e%128)/32 and lane
 * l = e%32: the low four bits are the low nibble of ql[64h + l + 32(c&1)]
 * for c < 2 and its high nibble for c >= 2; the high two bits are bits
 * 2c, 2c+1 of qh[32h + l]. */
int orc_q6k_quant(const uint8_t* blk, int e) {
    const uint8_t* ql = blk;
    const uint8_t* qh = blk + 128;
    int h = e / 128, r = e % 128, c = r / 32, l = r % 32;
    uint8_t lb = ql[64 * h + l + 32 * (c & 1)];
    int lo = (c < 2) ? (lb & 0xF) : (lb >> 4);
    int hi = (qh[32 * h + l] >> (2 * c)) & 3;
    return lo | (hi << 4);
}

void orc_q6k_quant_n(const uint8_t* blocks, int64_t n, uint8_t* q) {
    for (int64_t i = 0; i < n; ++i)
        for (int e = 0; e < 256; ++e) q[256 * i + e] = (uint8_t)orc_q6k_quant(blocks + 210 * i, e);
}

/* fp32 dequantizer.  Order of operations per element (all fp32):
 *   Q4_0: d * (float)(q - 8)          Q8_0: d * (float)q
 *   Q5_0: d * (float)(q - 16)
 *   Q4_K: (d * sc) * q - (dmin * m)   Q6_K: (d * sc) * (float)(q - 32)
 *   Q8_K: d * (float)q
 * Every product above is exact in fp32 except Q8_K's, so the only roundings
 * are Q4_K's subtraction and Q8_K's product. */
int orc_dequantize_f32(int type, const void* blocks, float* out, int64_t rows, int64_t K) {
    int B = orc_block_size(type);
    size_t S = orc_block_bytes(type);
    if (!B || K % B) return -1;
    const uint8_t* base = (const uint8_t*)blocks;
    int64_t nblk = rows * (K / B);
    for (int64_t ib = 0; ib < nblk; ++ib) {
        const uint8_t* blk = base + ib * S;
        float* o = out + ib * B;
        switch (type) {
        case ORC_Q4_0: {
            float d = rd_fp16(blk);
            for (int e = 0; e < 32; ++e) o[e] = d * (float)(q4_0_quant(blk, e) - 8);
        } break;
        case ORC_Q5_0: {
            float d = rd_fp16(blk);
            for (int e = 0; e < 32; ++e) o[e] = d * (float)(q5_0_quant(blk, e) - 16);
        } break;
        case ORC_Q8_0: {
            float d = rd_fp16(blk);
            for (int e = 0; e < 32; ++e) o[e] = d * (float)(int8_t)blk[2 + e];
        } break;
        case ORC_Q4_K: {
            float d = rd_fp16(blk), dmin = rd_fp16(blk + 2);
            for (int e = 0; e < 256; ++e) {
                int sc, m;
                orc_q4k_scale_min(blk + 4, e / 32, &sc, &m);
                float a = d * (float)sc;
                float b = a * (float)q4_k_quant(blk, e);
                float c = dmin * (float)m;
                o[e] = b - c;
            }
        } break;
        case ORC_Q6_K: {
            float d = rd_fp16(blk + 208);
            for (int e = 0; e < 256; ++e) {
                int sc = (int8_t)blk[192 + e / 16];
                float a = d * (float)sc;
                o[e] = a * (float)(orc_q6k_quant(blk, e) - 32);
            }
        } break;
        case ORC_Q8_K: {
            float d = rd_f32(blk);
            for (int e = 0; e < 256; ++e) o[e] = d * (float)(int8_t)blk[4 + e];
        } break;
        default: return -1;
        }
    }
    return 0;
}

/* Exact element values in fp64 (the real numbers the blocks encode). */
static void deq_block_f64(int type, const uint8_t* blk, double* o) {
    switch (type) {
    case ORC_Q4_0: {
        double d = rd_fp16(blk);
        for (int e = 0; e < 32; ++e) o[e] = d * (q4_0_quant(blk, e) - 8);
    } break;
    case ORC_Q5_0: {
        double d = rd_fp16(blk);
        for (int e = 0; e < 32; ++e) o[e] = d * (q5_0_quant(blk, e) - 16);
    } break;
    case ORC_Q8_0: {
        double d = rd_fp16(blk);
        for (int e = 0; e < 32; ++e) o[e] = d * (int8_t)blk[2 + e];
    } break;
    case ORC_Q4_K: {
        double d = rd_fp16(blk), dmin = rd_fp16(blk + 2);
        for (int e = 0; e < 256; ++e) {
            int sc, m;
            orc_q4k_scale_min(blk + 4, e / 32, &sc, &m);
            o[e] = d * sc * q4_k_quant(blk, e) - dmin * m;
        }
    } break;
    case ORC_Q6_K: {
        double d = rd_fp16(blk + 208);
        for (int e = 0; e < 256; ++e)
            o[e] = d * (int8_t)blk[192 + e / 16] * (orc_q6k_quant(blk, e) - 32);
    } break;
    case ORC_Q8_K: {
        double d = rd_f32(blk);
        for (int e = 0; e < 256; ++e) o[e] = d * (int8_t)blk[4 + e];
    } break;
    }
}

int orc_dequantize_f64(int type, const void* blocks, double* out, int64_t rows, int64_t K) {
    int B = orc_block_size(type);
    size_t S = orc_block_bytes(type);
    if (!B || K % B) return -1;
    int64_t nblk = rows * (K / B);
    for (int64_t ib = 0; ib < nblk; ++ib)
        deq_block_f64(type, (const uint8_t*)blocks + ib * S, out + ib * B);
    return 0;
}

/* ----------------------------------------------------------------- product */

static int vec_dot_type(int wtype) {
    switch (wtype) {
    case ORC_Q4_0: case ORC_Q5_0: case ORC_Q8_0: return ORC_Q8_0;
    case ORC_Q4_K: case ORC_Q6_K: return ORC_Q8_K;
    default: return 0;
    }
}

int orc_mul_mat(int wtype, const void* W, const void* xq, double* y, double* T,
                int64_t M, int64_t N, int64_t K) {
    int xt = vec_dot_type(wtype);
    if (!xt) return -1;
    int B = orc_block_size(wtype), BX = orc_block_size(xt);
    if (K % B || K % BX) return -1;
    size_t wrow = (size_t)(K / B) * orc_block_bytes(wtype);
    double* xd = (double*)malloc(sizeof(double) * (size_t)(N * K));
    if (!xd) return -2;
    orc_dequantize_f64(xt, xq, xd, N, K);
    int fail = 0;
#pragma omp parallel
    {
        double* wd = (double*)malloc(sizeof(double) * (size_t)K);
        double* wa = (double*)malloc(sizeof(double) * (size_t)K); /* |w| for T */
        if (!wd || !wa) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t m = 0; m < M; ++m) {
                const uint8_t* row = (const uint8_t*)W + (size_t)m * wrow;
                for (int64_t b = 0; b < K / B; ++b)
                    deq_block_f64(wtype, row + b * orc_block_bytes(wtype), wd + b * B);
                if (T) {
                    if (wtype == ORC_Q4_K) {
                        /* |d sc q| + |dmin m| per element */
                        for (int64_t b = 0; b < K / 256; ++b) {
                            const uint8_t* blk = row + b * 144;
                            double d = rd_fp16(blk), dmin = rd_fp16(blk + 2);
                            for (int e = 0; e < 256; ++e) {
                                int sc, mm;
                                orc_q4k_scale_min(blk + 4, e / 32, &sc, &mm);
                                wa[b * 256 + e] = fabs(d * sc * q4_k_quant(blk, e)) + fabs(dmin * mm);
                            }
                        }
                    } else {
                        for (int64_t k = 0; k < K; ++k) wa[k] = fabs(wd[k]);
                    }
                }
                for (int64_t n = 0; n < N; ++n) {
                    const double* xr = xd + n * K;
                    double acc = 0.0, tacc = 0.0;
                    for (int64_t k = 0; k < K; ++k) acc += wd[k] * xr[k];
                    if (T)
                        for (int64_t k = 0; k < K; ++k) tacc += wa[k] * fabs(xr[k]);
                    y[n * M + m] = acc;
                    if (T) T[n * M + m] = tacc;
                }
            }
        }
        free(wd);
        free(wa);
    }
    free(xd);
    return fail ? -2 : 0;
}

int orc_mul_mat_blockwise(int wtype, const void* W, const void* xq, double* y,
                          int64_t M, int64_t N, int64_t K) {
    int xt = vec_dot_type(wtype);
    if (!xt) return -1;
    int B = orc_block_size(wtype);
    if (K % B || K % orc_block_size(xt)) return -1;
    size_t SW = orc_block_bytes(wtype), SX = orc_block_bytes(xt);
    int64_t nbw = K / B, nbx = K / orc_block_size(xt);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint8_t* wrow = (const uint8_t*)W + (size_t)m * nbw * SW;
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t* xrow = (const uint8_t*)xq + (size_t)n * nbx * SX;
            double acc = 0.0;
            for (int64_t b = 0; b < nbw; ++b) {
                const uint8_t* wb = wrow + b * SW;
                const uint8_t* xb = xrow + b * SX; /* same block size on both sides */
                if (wtype == ORC_Q8_0 || wtype == ORC_Q4_0 || wtype == ORC_Q5_0) {
                    int64_t isum = 0;
                    for (int e = 0; e < 32; ++e) {
                        int qw = (wtype == ORC_Q8_0) ? (int8_t)wb[2 + e]
                               : (wtype == ORC_Q4_0) ? q4_0_quant(wb, e) - 8 : q5_0_quant(wb, e) - 16;
                        isum += (int64_t)qw * (int8_t)xb[2 + e];
                    }
                    acc += (double)rd_fp16(wb) * (double)rd_fp16(xb) * (double)isum;
                } else if (wtype == ORC_Q4_K) {
                    int64_t sumi = 0, summ = 0;
                    for (int j = 0; j < 8; ++j) {
                        int sc, mm;
                        orc_q4k_scale_min(wb + 4, j, &sc, &mm);
                        int64_t s = 0;
                        for (int i = 0; i < 32; ++i)
                            s += (int64_t)q4_k_quant(wb, 32 * j + i) * (int8_t)xb[4 + 32 * j + i];
                        sumi += sc * s;
                        summ += (int64_t)mm * (rd_i16(xb + 260 + 4 * j) + rd_i16(xb + 262 + 4 * j));
                    }
                    double d = rd_fp16(wb), dmin = rd_fp16(wb + 2), dx = rd_f32(xb);
                    acc += dx * (d * (double)sumi - dmin * (double)summ);
                } else { /* Q6_K */
                    int64_t s = 0;
                    for (int j = 0; j < 16; ++j) {
                        int64_t p = 0;
                        for (int i = 0; i < 16; ++i)
                            p += (int64_t)orc_q6k_quant(wb, 16 * j + i) * (int8_t)xb[4 + 16 * j + i];
                        p -= 32 * (int64_t)rd_i16(xb + 260 + 2 * j);
                        s += (int64_t)(int8_t)wb[192 + j] * p;
                    }
                    acc += (double)rd_f32(xb) * (double)rd_fp16(wb + 208) * (double)s;
                }
            }
            y[n * M + m] = acc;
        }
    }
    return 0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads used by the parallel loops from now on (n >= 1); a timing control,
 * no effect on any result. */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
