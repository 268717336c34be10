// Drives every entry point of include/qmm.h through its validation paths
// (valid calls, and each class of invalid argument) with the launchers
// replaced by counting stand-ins.  Built with -fsanitize=address,undefined;
// any sanitizer report, a wrong status, or a launch on an invalid call makes
// the program exit non-zero.  Pointers are host buffers that are never
// dereferenced by the validation code.
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "../../include/qmm.h"
#include "../../include/qmm_probe.h"

extern int g_launches;

static int failures = 0;

#define EXPECT(call, want, launched)                                                                \
    do {                                                                                            \
        const int before = g_launches;                                                              \
        const int got = (call);                                                                     \
        const int did = g_launches - before;                                                        \
        if (got != (want) || did != (launched)) {                                                   \
            fprintf(stderr, "line %d: %s -> %d (want %d), launches %d (want %d)\n", __LINE__, #call, got, \
                    (int)(want), did, (int)(launched));                                             \
            ++failures;                                                                             \
        }                                                                                           \
    } while (0)

alignas(16) static unsigned char buf_a[4096], buf_b[4096], buf_c[4096];

int main() {
    void* A = buf_a;
    void* X = buf_b;
    float* Y = reinterpret_cast<float*>(buf_c);
    void* mis = buf_a + 4;  // 4-byte aligned only
    const int types[] = {QMM_Q4_0, QMM_Q8_0, QMM_Q4_K, QMM_Q6_K, QMM_Q8_K, QMM_Q5_0};
    const int blk[] = {32, 32, 256, 256, 256, 32};
    const size_t bytes[] = {18, 34, 144, 210, 292, 22};

    // ---- sizes
    for (int i = 0; i < 6; ++i) {
        const int t = types[i];
        if (qmm_block_size(t) != blk[i] || qmm_block_bytes(t) != bytes[i]) ++failures;
        if (qmm_row_bytes(t, 4 * blk[i]) != 4 * bytes[i]) ++failures;
        if (qmm_row_bytes(t, blk[i] + 1) != 0 || qmm_row_bytes(t, 0) != 0 || qmm_row_bytes(t, -blk[i]) != 0) ++failures;
        if (qmm_row_bytes(t, INT64_MAX - (INT64_MAX % blk[i])) != 0) ++failures;
    }
    for (int t : {0, 7, -1, INT_MAX, INT_MIN}) {
        if (qmm_block_size(t) != 0 || qmm_block_bytes(t) != 0 || qmm_row_bytes(t, 256) != 0) ++failures;
        if (qmm_vec_dot_type(t) != QMM_ERR_TYPE) ++failures;
    }
    if (qmm_vec_dot_type(QMM_Q4_0) != QMM_Q8_0 || qmm_vec_dot_type(QMM_Q5_0) != QMM_Q8_0 ||
        qmm_vec_dot_type(QMM_Q8_0) != QMM_Q8_0 || qmm_vec_dot_type(QMM_Q4_K) != QMM_Q8_K ||
        qmm_vec_dot_type(QMM_Q6_K) != QMM_Q8_K || qmm_vec_dot_type(QMM_Q8_K) != QMM_ERR_UNSUPPORTED)
        ++failures;

    // ---- activation quantization
    const float* xf = reinterpret_cast<const float*>(buf_a);
    EXPECT(qmm_quantize_act(QMM_Q8_0, xf, X, 3, 64, nullptr), QMM_OK, 1);
    EXPECT(qmm_quantize_act(QMM_Q8_K, xf, X, 1, 256, nullptr), QMM_OK, 1);
    EXPECT(qmm_quantize_act(QMM_Q4_K, xf, X, 1, 256, nullptr), QMM_ERR_UNSUPPORTED, 0);
    EXPECT(qmm_quantize_act(QMM_Q4_0, xf, X, 1, 32, nullptr), QMM_ERR_UNSUPPORTED, 0);
    EXPECT(qmm_quantize_act(0, xf, X, 1, 32, nullptr), QMM_ERR_TYPE, 0);
    EXPECT(qmm_quantize_act(QMM_Q8_0, nullptr, X, 1, 32, nullptr), QMM_ERR_NULL, 0);
    EXPECT(qmm_quantize_act(QMM_Q8_0, xf, nullptr, 1, 32, nullptr), QMM_ERR_NULL, 0);
    EXPECT(qmm_quantize_act(QMM_Q8_0, reinterpret_cast<const float*>(mis), X, 1, 32, nullptr), QMM_ERR_ALIGN, 0);
    EXPECT(qmm_quantize_act(QMM_Q8_0, xf, mis, 1, 32, nullptr), QMM_ERR_ALIGN, 0);
    EXPECT(qmm_quantize_act(QMM_Q8_0, xf, X, 0, 32, nullptr), QMM_ERR_SHAPE, 0);
    EXPECT(qmm_quantize_act(QMM_Q8_0, xf, X, -5, 32, nullptr), QMM_ERR_SHAPE, 0);
    EXPECT(qmm_quantize_act(QMM_Q8_0, xf, X, 1, 33, nullptr), QMM_ERR_SHAPE, 0);
    EXPECT(qmm_quantize_act(QMM_Q8_K, xf, X, 1, 32, nullptr), QMM_ERR_SHAPE, 0);
    EXPECT(qmm_quantize_act(QMM_Q8_0, xf, X, INT64_MAX / 64, 64, nullptr), QMM_ERR_SHAPE, 0);
    EXPECT(qmm_quantize_act(QMM_Q8_0, xf, X, 2, INT64_MAX - 31, nullptr), QMM_ERR_SHAPE, 0);
    EXPECT(qmm_quantize(QMM_Q4_0, xf, X, 2, 64, nullptr), QMM_OK, 1);
    EXPECT(qmm_quantize(QMM_Q6_K, xf, X, 1, 256, nullptr), QMM_ERR_UNSUPPORTED, 0);

    // ---- dequantization (every type)
    for (int i = 0; i < 6; ++i) {
        EXPECT(qmm_dequantize(types[i], A, Y, 2, blk[i], nullptr), QMM_OK, 1);
        EXPECT(qmm_dequantize(types[i], A, Y, 2, blk[i] + 16, nullptr), QMM_ERR_SHAPE, 0);
        EXPECT(qmm_dequantize(types[i], nullptr, Y, 2, blk[i], nullptr), QMM_ERR_NULL, 0);
        EXPECT(qmm_dequantize(types[i], A, reinterpret_cast<float*>(mis), 2, blk[i], nullptr), QMM_ERR_ALIGN, 0);
    }
    EXPECT(qmm_dequantize(9, A, Y, 1, 256, nullptr), QMM_ERR_TYPE, 0);

    // ---- products
    const int wts[] = {QMM_Q4_0, QMM_Q8_0, QMM_Q4_K, QMM_Q6_K, QMM_Q5_0};
    for (int wt : wts) {
        for (int algo = 0; algo <= 2; ++algo) EXPECT(qmm_mul_mat_algo(wt, A, X, Y, 64, 3, 512, algo, nullptr), QMM_OK, 1);
        EXPECT(qmm_mul_mat_algo(wt, A, X, Y, 64, 3, 512, 3, nullptr), QMM_ERR_UNSUPPORTED, 0);
        EXPECT(qmm_mul_mat_algo(wt, A, X, Y, 64, 3, 512, -1, nullptr), QMM_ERR_UNSUPPORTED, 0);
        EXPECT(qmm_mul_mat(wt, A, X, Y, 64, 512, 512, nullptr), QMM_OK, 1);
        EXPECT(qmm_mul_mat(wt, nullptr, X, Y, 64, 1, 512, nullptr), QMM_ERR_NULL, 0);
        EXPECT(qmm_mul_mat(wt, A, nullptr, Y, 64, 1, 512, nullptr), QMM_ERR_NULL, 0);
        EXPECT(qmm_mul_mat(wt, A, X, nullptr, 64, 1, 512, nullptr), QMM_ERR_NULL, 0);
        EXPECT(qmm_mul_mat(wt, mis, X, Y, 64, 1, 512, nullptr), QMM_ERR_ALIGN, 0);
        EXPECT(qmm_mul_mat(wt, A, X, Y, 0, 1, 512, nullptr), QMM_ERR_SHAPE, 0);
        EXPECT(qmm_mul_mat(wt, A, X, Y, 64, 0, 512, nullptr), QMM_ERR_SHAPE, 0);
        EXPECT(qmm_mul_mat(wt, A, X, Y, 64, 1, 0, nullptr), QMM_ERR_SHAPE, 0);
        EXPECT(qmm_mul_mat(wt, A, X, Y, 64, 1, 512 + 16, nullptr), QMM_ERR_SHAPE, 0);
        EXPECT(qmm_mul_mat(wt, A, X, Y, (int64_t)INT_MAX + 1, 1, 256, nullptr), QMM_ERR_SHAPE, 0);
        EXPECT(qmm_mul_mat(wt, A, X, Y, 1, (int64_t)INT_MAX + 1, 256, nullptr), QMM_ERR_SHAPE, 0);
        EXPECT(qmm_mul_mat(wt, A, X, Y, 64, 1, 65536 + 256, nullptr), QMM_ERR_UNSUPPORTED, 0);
        EXPECT(qmm_mul_mat(wt, A, X, Y, INT64_MAX / 2, 1, 256, nullptr), QMM_ERR_SHAPE, 0);
    }
    // Q4_0 / Q8_0 / Q5_0 rows of 32-value blocks need the activation's block
    // size too: K = 96 is fine for them (Q8_0 activations)
    EXPECT(qmm_mul_mat(QMM_Q4_0, A, X, Y, 8, 1, 96, nullptr), QMM_OK, 1);
    EXPECT(qmm_mul_mat(QMM_Q4_K, A, X, Y, 8, 1, 96, nullptr), QMM_ERR_SHAPE, 0);
    EXPECT(qmm_mul_mat(QMM_Q8_K, A, X, Y, 8, 1, 256, nullptr), QMM_ERR_UNSUPPORTED, 0);
    EXPECT(qmm_mul_mat(42, A, X, Y, 8, 1, 256, nullptr), QMM_ERR_TYPE, 0);

    // ---- several matrices per launch
    const void* Ws[4] = {A, A, A, A};
    float* Ys[4] = {Y, Y, Y, Y};
    const int64_t Ms[4] = {64, 32, 32, 128};
    EXPECT(qmm_mul_mat_multi(QMM_Q4_0, 3, Ws, Ys, Ms, X, 0, 2, 512, nullptr), QMM_OK, 1);
    EXPECT(qmm_mul_mat_multi(QMM_Q4_0, 4, Ws, Ys, Ms, xf, 1, 8, 512, nullptr), QMM_OK, 1);
    EXPECT(qmm_mul_mat_multi(QMM_Q4_0, 4, Ws, Ys, Ms, xf, 1, 9, 512, nullptr), QMM_ERR_UNSUPPORTED, 0);
    EXPECT(qmm_mul_mat_multi(QMM_Q4_0, 1, Ws, Ys, Ms, xf, 1, 1, 96, nullptr), QMM_ERR_UNSUPPORTED, 0);
    EXPECT(qmm_mul_mat_multi(QMM_Q4_0, 1, Ws, Ys, Ms, X, 0, 1, 96, nullptr), QMM_OK, 1);
    EXPECT(qmm_mul_mat_multi(QMM_Q4_K, 0, Ws, Ys, Ms, X, 0, 1, 512, nullptr), QMM_ERR_SHAPE, 0);
    EXPECT(qmm_mul_mat_multi(QMM_Q4_K, 5, Ws, Ys, Ms, X, 0, 1, 512, nullptr), QMM_ERR_SHAPE, 0);
    EXPECT(qmm_mul_mat_multi(QMM_Q4_K, 2, nullptr, Ys, Ms, X, 0, 1, 512, nullptr), QMM_ERR_NULL, 0);
    EXPECT(qmm_mul_mat_multi(QMM_Q4_K, 2, Ws, nullptr, Ms, X, 0, 1, 512, nullptr), QMM_ERR_NULL, 0);
    EXPECT(qmm_mul_mat_multi(QMM_Q4_K, 2, Ws, Ys, nullptr, X, 0, 1, 512, nullptr), QMM_ERR_NULL, 0);
    const void* Wbad[2] = {A, mis};
    EXPECT(qmm_mul_mat_multi(QMM_Q4_K, 2, Wbad, Ys, Ms, X, 0, 1, 512, nullptr), QMM_ERR_ALIGN, 0);
    const int64_t Mbad[2] = {64, 0};
    EXPECT(qmm_mul_mat_multi(QMM_Q4_K, 2, Ws, Ys, Mbad, X, 0, 1, 512, nullptr), QMM_ERR_SHAPE, 0);
    EXPECT(qmm_mul_mat_multi(QMM_Q8_K, 1, Ws, Ys, Ms, X, 0, 1, 512, nullptr), QMM_ERR_UNSUPPORTED, 0);

    // ---- measurement aids
    uint32_t* sink = reinterpret_cast<uint32_t*>(Y);
    EXPECT(qmm_probe_read(A, 4096, sink, 0, nullptr), QMM_OK, 1);
    EXPECT(qmm_probe_read(A, 64, sink, 3, nullptr), QMM_OK, 1);
    EXPECT(qmm_probe_read(nullptr, 64, sink, 0, nullptr), QMM_ERR_NULL, 0);
    EXPECT(qmm_probe_read(A, 64, nullptr, 0, nullptr), QMM_ERR_NULL, 0);
    EXPECT(qmm_probe_read(mis, 64, sink, 0, nullptr), QMM_ERR_ALIGN, 0);
    EXPECT(qmm_probe_read(A, 0, sink, 0, nullptr), QMM_ERR_SHAPE, 0);
    EXPECT(qmm_probe_read(A, 40, sink, 0, nullptr), QMM_ERR_SHAPE, 0);
    EXPECT(qmm_probe_read(A, 64, sink, -1, nullptr), QMM_ERR_SHAPE, 0);
    EXPECT(qmm_probe_read(A, 64, sink, 65537, nullptr), QMM_ERR_SHAPE, 0);
    EXPECT(qmm_probe_mfma(512, 100, sink, nullptr), QMM_OK, 1);
    EXPECT(qmm_probe_mfma(512, 100, nullptr, nullptr), QMM_ERR_NULL, 0);
    EXPECT(qmm_probe_mfma(0, 100, sink, nullptr), QMM_ERR_SHAPE, 0);
    EXPECT(qmm_probe_mfma(512, 0, sink, nullptr), QMM_ERR_SHAPE, 0);
    EXPECT(qmm_probe_mfma(512, (int64_t(1) << 30) + 1, sink, nullptr), QMM_ERR_SHAPE, 0);
    if (qmm_probe_mfma_ops(2, 3) != 2LL * 16 * 3 * 65536 || qmm_probe_mfma_ops(65537, 1) != 0) ++failures;
    EXPECT(qmm_probe_mfma16(512, 100, sink, nullptr), QMM_OK, 1);
    EXPECT(qmm_probe_mfma16(512, 100, nullptr, nullptr), QMM_ERR_NULL, 0);
    EXPECT(qmm_probe_mfma16(0, 100, sink, nullptr), QMM_ERR_SHAPE, 0);
    EXPECT(qmm_probe_mfma16(512, 0, sink, nullptr), QMM_ERR_SHAPE, 0);
    if (qmm_probe_mfma16_ops(2, 3) != 2LL * 32 * 3 * 32768 || qmm_probe_mfma16_ops(65537, 1) != 0) ++failures;

    // ---- the automatic kernel choice (host logic)
    if (qmm_mul_mat_choice(QMM_Q4_K, 14336, 2, 4096) != 1 || qmm_mul_mat_choice(QMM_Q4_K, 14336, 3, 4096) != 2 ||
        qmm_mul_mat_choice(QMM_Q8_K, 64, 1, 256) != 0 || qmm_mul_mat_choice(QMM_Q4_0, 64, 1, 48) != 0 ||
        qmm_mul_mat_choice(QMM_Q4_0, int64_t(1) << 40, 1, 32) != 0)
        ++failures;

    // ---- status text
    for (int c = -8; c <= 1; ++c)
        if (!qmm_strerror(c) || !qmm_strerror(c)[0]) ++failures;

    if (failures) fprintf(stderr, "%d failures\n", failures);
    else printf("abi validation ok\n");
    return failures ? 1 : 0;
}
