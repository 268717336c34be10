/* Runs every function of the CPU oracle (oracle/qmm_oracle.h) on small
 * inputs, edge values included (zero blocks, NaN, Inf, huge and subnormal
 * values; raw blocks of random bytes, so fp16 scales may be NaN, Inf or
 * subnormal), under AddressSanitizer and UndefinedBehaviorSanitizer.  Any
 * sanitizer report, or a failed consistency check between the oracle's two
 * product forms, makes the program exit non-zero. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/qmm_oracle.h"

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void) {  /* xorshift64* */
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (uint32_t)((rng * 0x2545F4914F6CDD1Dull) >> 32);
}
static float uniform(void) { return (float)next32() / 4294967296.0f * 2.0f - 1.0f; }

static int failures = 0;
#define CHECK(c)                                                  \
    do {                                                          \
        if (!(c)) {                                               \
            fprintf(stderr, "line %d: check failed: %s\n", __LINE__, #c); \
            ++failures;                                           \
        }                                                         \
    } while (0)

static void fill_x(float* x, int64_t n, int kind) {
    for (int64_t i = 0; i < n; ++i) {
        float v = uniform() * 3.0f;
        switch (kind) {
        case 1: v = 0.0f; break;                                  /* zero blocks */
        case 2: v = (i % 7 == 0) ? NAN : v; break;                /* NaN mixed in */
        case 3: v = (i % 11 == 0) ? INFINITY : -v; break;         /* Inf mixed in */
        case 4: v *= 1e-42f; break;                               /* subnormal amax */
        case 5: v *= 3e38f; break;                                /* near FLT_MAX */
        default: break;
        }
        x[i] = v;
    }
}

int main(void) {
    /* fp16 both ways over all patterns */
    for (uint32_t h = 0; h < 65536; ++h) {
        float f = orc_fp16_to_f32((uint16_t)h);
        uint16_t back = orc_f32_to_fp16(f);
        if (f == f) CHECK(back == (uint16_t)h);
    }
    {
        float f[6] = {65520.0f, -1e9f, 1e-8f, 5.96e-8f, 2.98e-8f, 0.0f};
        uint16_t h[6];
        orc_f32_to_fp16_n(f, h, 6);
        float g[6];
        orc_fp16_to_f32_n(h, g, 6);
        CHECK(isinf(g[0]) && isinf(g[1]));
    }

    const int types[6] = {ORC_Q4_0, ORC_Q8_0, ORC_Q4_K, ORC_Q6_K, ORC_Q8_K, ORC_Q5_0};
    const int64_t M = 5, N = 3, K = 512;
    float* x = malloc(sizeof(float) * N * K);
    float* wf = malloc(sizeof(float) * M * K);
    uint8_t* xq = malloc(N * (K / 32) * 34 + N * (K / 256) * 292);
    uint8_t* wq = malloc(M * (K / 32) * 34 + 64);
    uint8_t* raw = malloc(M * (K / 32) * 34 + M * (K / 256) * 292);
    float* deq = malloc(sizeof(float) * M * K);
    double* deq64 = malloc(sizeof(double) * M * K);
    double *y = malloc(sizeof(double) * M * N), *T = malloc(sizeof(double) * M * N), *yb = malloc(sizeof(double) * M * N);

    /* quantizers on every input kind */
    for (int kind = 0; kind <= 5; ++kind) {
        fill_x(x, N * K, kind);
        CHECK(orc_quantize_q8_0(x, xq, N, K) == 0);
        CHECK(orc_quantize_q8_k(x, xq, N, K) == 0);
        CHECK(orc_quantize_q4_0(x, xq, N, K) == 0);
    }
    CHECK(orc_quantize_q8_0(x, xq, 1, 33) != 0);
    CHECK(orc_quantize_q8_k(x, xq, 1, 32) != 0);

    /* decoders and dequantizers on random bytes (any bit pattern) */
    for (int it = 0; it < 20; ++it) {
        for (size_t i = 0; i < (size_t)(M * (K / 32) * 34 + M * (K / 256) * 292); ++i) raw[i] = (uint8_t)next32();
        for (int t = 0; t < 6; ++t) {
            CHECK(orc_dequantize_f32(types[t], raw, deq, M, K) == 0);
            CHECK(orc_dequantize_f64(types[t], raw, deq64, M, K) == 0);
        }
        int32_t sc[16], mn[16];
        orc_q4k_scale_min_n(raw, 2, sc, mn);
        for (int j = 0; j < 16; ++j) CHECK(sc[j] >= 0 && sc[j] < 64 && mn[j] >= 0 && mn[j] < 64);
        uint8_t q[512];
        orc_q6k_quant_n(raw, 2, q);
        for (int e = 0; e < 512; ++e) CHECK(q[e] < 64);
        orc_q5_0_quant_n(raw, 16, q);
        for (int e = 0; e < 512; ++e) CHECK(q[e] < 32);
    }
    CHECK(orc_dequantize_f32(99, raw, deq, 1, 256) != 0);
    CHECK(orc_dequantize_f32(ORC_Q4_K, raw, deq, 1, 100) != 0);

    /* products: weights from the encoders and from random bytes */
    const int wts[5] = {ORC_Q4_0, ORC_Q8_0, ORC_Q4_K, ORC_Q6_K, ORC_Q5_0};
    for (int it = 0; it < 6; ++it) {
        fill_x(x, N * K, 0);
        fill_x(wf, M * K, 0);
        for (int t = 0; t < 5; ++t) {
            const int wt = wts[t];
            const int xt = (wt == ORC_Q4_K || wt == ORC_Q6_K) ? ORC_Q8_K : ORC_Q8_0;
            if (xt == ORC_Q8_0) CHECK(orc_quantize_q8_0(x, xq, N, K) == 0);
            else CHECK(orc_quantize_q8_k(x, xq, N, K) == 0);
            if (wt == ORC_Q4_0 && it % 2 == 0) CHECK(orc_quantize_q4_0(wf, wq, M, K) == 0);
            else if (wt == ORC_Q8_0 && it % 2 == 0) CHECK(orc_quantize_q8_0(wf, wq, M, K) == 0);
            else {
                const size_t nb = (size_t)M * (K / orc_block_size(wt)) * orc_block_bytes(wt);
                for (size_t i = 0; i < nb; ++i) wq[i] = (uint8_t)next32();
                /* keep the scales finite so the two forms can be compared */
                for (size_t b = 0; b < nb / orc_block_bytes(wt); ++b) {
                    uint8_t* blk = wq + b * orc_block_bytes(wt);
                    uint8_t* d = (wt == ORC_Q6_K) ? blk + 208 : blk;
                    d[1] &= 0x3F;
                    if (wt == ORC_Q4_K) blk[3] &= 0x3F;
                }
            }
            CHECK(orc_mul_mat(wt, wq, xq, y, T, M, N, K) == 0);
            CHECK(orc_mul_mat(wt, wq, xq, y, NULL, M, N, K) == 0);
            CHECK(orc_mul_mat_blockwise(wt, wq, xq, yb, M, N, K) == 0);
            for (int64_t i = 0; i < M * N; ++i) CHECK(fabs(y[i] - yb[i]) <= 1e-12 * T[i] + 1e-300);
        }
    }
    CHECK(orc_mul_mat(ORC_Q8_K, wq, xq, y, T, M, N, K) != 0);
    CHECK(orc_mul_mat(ORC_Q4_K, wq, xq, y, T, M, N, 100) != 0);
    CHECK(orc_num_threads() >= 1);

    free(x); free(wf); free(xq); free(wq); free(raw); free(deq); free(deq64); free(y); free(T); free(yb);
    if (failures) fprintf(stderr, "%d failures\n", failures);
    else printf("oracle ok\n");
    return failures ? 1 : 0;
}
