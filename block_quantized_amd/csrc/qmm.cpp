// qmm.cpp — the C ABI: argument validation, then dispatch to the kernels.
// Every check runs before anything is enqueued, so an error return leaves
// every output untouched.  Nothing here allocates, copies or synchronizes.
#include <limits.h>
#include <stdint.h>

#include "qmm_internal.h"

using namespace qmm;

namespace {

constexpr int64_t kMaxK = 65536;  // activation rows must fit the GEMV's LDS staging

bool is_type(int t) { return t >= QMM_Q4_0 && t <= QMM_Q5_0; }
bool is_weight(int t) {
    return t == QMM_Q4_0 || t == QMM_Q5_0 || t == QMM_Q8_0 || t == QMM_Q4_K || t == QMM_Q6_K;
}

int check_ptr(const void* p) {
    if (!p) return QMM_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(p) & 15u) return QMM_ERR_ALIGN;
    return QMM_OK;
}

// rows x K values of type t: positive sizes, whole blocks, and byte counts
// (blocks and fp32) that fit comfortably in int64.
int check_dims(int t, int64_t rows, int64_t K) {
    if (rows <= 0 || K <= 0) return QMM_ERR_SHAPE;
    const int B = block_size(t);
    if (K % B) return QMM_ERR_SHAPE;
    const int64_t lim = INT64_MAX / 8;
    if (K > lim / 4 || rows > lim / (K * 4)) return QMM_ERR_SHAPE;  // rows*K*4 fp32 bytes
    return QMM_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? QMM_OK : QMM_ERR_HIP; }

// Largest N for which the automatic choice keeps the GEMV kernels: the
// crossovers measured on MI355X.  The GEMV decodes the weights once per
// activation row (in groups of 8 rows); the MFMA kernels once per 32 or 64
// rows, with a fixed cost per super-block or block that the Q4_0, Q5_0 and
// Q8_0 kernels' per-block scaling makes large.
int64_t gemm_min_rows(int wtype, int64_t M, int64_t K) {
    switch (wtype) {
    // the Q6_K GEMM has one 128-row workgroup per row block, and its time is
    // flat in N up to 32.  With about one row block per CU or more (32000x4096,
    // the 128256x4096 and 151936x1536 heads) it wins from N = 5 at the latest;
    // with 70-112 row blocks (8960x1536, 11008x2048, 14336x4096) once the GEMV
    // needs a second group of 6 rows; below 8192 rows near N = 30 (4096x14336:
    // 118 us at N <= 32 against 88 / 118 / 132 us at N = 20 / 30 / 32; 4096^2:
    // about 25), and below 2048 rows (1536x8960: 12 workgroups, 72 us at
    // N <= 32 and 104-106 us for N = 33-64) near N = 54
    case QMM_Q6_K: return M > 24576 ? 4 : M > 8192 ? 6 : M < 2048 ? 54 : 30;
    // the narrow MFMA kernels (weights staged through LDS) win from N = 3
    // (measured from 256 to 14336 rows with K = 4096, at 4096x14336, 1536x1536,
    // 1536x8960 and 256x1536; at N = 2 the two tie or the GEMV wins).  Above
    // 8192 rows with K < 4096 (8960x1536, 11008x2048, 16384x1536) the 32-row
    // kernel has only a few super-blocks per wave and the GEMV wins up to N = 4
    case QMM_Q4_K: return M > 8192 && K < 4096 ? 4 : 2;
    // Q4_0 / Q5_0 / Q8_0: while the grid has at most 256 tiles (M <= 8192 and
    // N <= 64, or larger M and N up to 256 * 128 * 64 / M), the GEMM's time is
    // its chain of 4-block chunks per wave, proportional to K and nearly
    // independent of M and N (4096x4096: 33-34 / 39-40 / 39 us, 2048x8192:
    // 61-66 / 72-77 / 71-78 us); the GEMV's grows by a step per group of activation rows,
    // a longer one for small matrices (which leave SIMDs idle) and for large
    // ones.  Measured switches: M > 24576 (32000x4096, 65536x2048: the GEMM
    // has a row block per CU or more); M > 8192 (14336x4096, 8960x1536,
    // 11008x2048); K < 2048
    // by rows (896x896; 1536x1536 and 2048x1024; 4864x896); K = 2048
    // (2048x2048, 8192x2048); K <= 4096 with M >= 4096 (4096x4096) and below
    // (1024x4096); wider rows, with M < 2048 (896x4864, 1536x8960) and above
    // (2048x8192).
    case QMM_Q4_0:
        return M > 24576  ? 8
               : M > 8192 ? 12
               : K < 2048 ? (M <= 1024 ? 21 : M < 4096 ? 14 : 7)
               : K == 2048 ? 17
               : K <= 4096 ? (M >= 4096 ? 28 : 23)
                           : (M < 2048 ? 30 : 47);
    case QMM_Q5_0:
        return M > 24576  ? 8
               : M > 8192 ? 12
               : K < 2048 ? (M <= 1024 ? 23 : M < 4096 ? 16 : 8)
               : K == 2048 ? 19
               : K <= 4096 ? (M >= 4096 ? 32 : 26)
                           : (M < 2048 ? 33 : 51);
    default:  // Q8_0
        return M > 24576  ? 7
               : M > 8192 ? 10
               : K < 2048 ? (M <= 1024 ? 26 : M < 4096 ? 15 : 7)
               : K == 2048 ? 17
               : K <= 4096 ? 26
                           : (M < 2048 ? 31 : 45);
    }
}

}  // namespace

extern "C" {

int qmm_block_size(int type) { return is_type(type) ? block_size(type) : 0; }

size_t qmm_block_bytes(int type) { return is_type(type) ? (size_t)block_bytes(type) : 0; }

size_t qmm_row_bytes(int type, int64_t K) {
    if (!is_type(type) || K <= 0 || K % block_size(type)) return 0;
    if (K > INT64_MAX / 8 / 4) return 0;
    return (size_t)(K / block_size(type)) * (size_t)block_bytes(type);
}

int qmm_vec_dot_type(int wtype) {
    if (!is_type(wtype)) return QMM_ERR_TYPE;
    if (wtype == QMM_Q4_0 || wtype == QMM_Q5_0 || wtype == QMM_Q8_0) return QMM_Q8_0;
    if (wtype == QMM_Q4_K || wtype == QMM_Q6_K) return QMM_Q8_K;
    return QMM_ERR_UNSUPPORTED;
}

int qmm_quantize(int dst, const float* x, void* out, int64_t rows, int64_t K, void* stream) {
    if (!is_type(dst)) return QMM_ERR_TYPE;
    if (dst != QMM_Q8_0 && dst != QMM_Q8_K && dst != QMM_Q4_0) return QMM_ERR_UNSUPPORTED;
    int rc;
    if ((rc = check_ptr(x)) || (rc = check_ptr(out))) return rc;
    if ((rc = check_dims(dst, rows, K))) return rc;
    return hip_status(launch_quantize(dst, x, out, rows, K, static_cast<hipStream_t>(stream)));
}

int qmm_quantize_act(int dst, const float* x, void* xq, int64_t N, int64_t K, void* stream) {
    if (!is_type(dst)) return QMM_ERR_TYPE;
    if (dst != QMM_Q8_0 && dst != QMM_Q8_K) return QMM_ERR_UNSUPPORTED;
    return qmm_quantize(dst, x, xq, N, K, stream);
}

int qmm_dequantize(int type, const void* blocks, float* out, int64_t rows, int64_t K, void* stream) {
    if (!is_type(type)) return QMM_ERR_TYPE;
    int rc;
    if ((rc = check_ptr(blocks)) || (rc = check_ptr(out))) return rc;
    if ((rc = check_dims(type, rows, K))) return rc;
    return hip_status(launch_dequantize(type, blocks, out, rows, K, static_cast<hipStream_t>(stream)));
}

int qmm_mul_mat_algo(int wtype, const void* W, const void* xq, float* y, int64_t M, int64_t N, int64_t K,
                     int algo, void* stream) {
    if (!is_type(wtype)) return QMM_ERR_TYPE;
    if (!is_weight(wtype)) return QMM_ERR_UNSUPPORTED;
    if (algo < 0 || algo > 2) return QMM_ERR_UNSUPPORTED;
    int rc;
    if ((rc = check_ptr(W)) || (rc = check_ptr(xq)) || (rc = check_ptr(y))) return rc;
    const int xt = qmm_vec_dot_type(wtype);
    if ((rc = check_dims(wtype, M, K)) || (rc = check_dims(xt, N, K))) return rc;
    if (M > INT_MAX || N > INT_MAX) return QMM_ERR_SHAPE;
    if (K > kMaxK) return QMM_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool has_gemm = gemm_supported(wtype);
    if (algo == 2 && !has_gemm) return QMM_ERR_UNSUPPORTED;
    const bool gemm = algo == 2 || (algo == 0 && has_gemm && N > gemm_min_rows(wtype, M, K));
    return hip_status(gemm ? launch_gemm(wtype, W, xq, y, M, N, K, s) : launch_gemv(wtype, W, xq, y, M, N, K, s));
}

int qmm_mul_mat_choice(int wtype, int64_t M, int64_t N, int64_t K) {
    if (!is_type(wtype) || !is_weight(wtype)) return 0;
    const int xt = qmm_vec_dot_type(wtype);
    if (check_dims(wtype, M, K) || check_dims(xt, N, K) || M > INT_MAX || N > INT_MAX || K > kMaxK) return 0;
    return gemm_supported(wtype) && N > gemm_min_rows(wtype, M, K) ? 2 : 1;
}

int qmm_mul_mat(int wtype, const void* W, const void* xq, float* y, int64_t M, int64_t N, int64_t K,
                void* stream) {
    return qmm_mul_mat_algo(wtype, W, xq, y, M, N, K, 0, stream);
}

int qmm_mul_mat_multi(int wtype, int count, const void* const* W, float* const* y, const int64_t* M,
                      const void* x, int x_is_f32, int64_t N, int64_t K, void* stream) {
    if (!is_type(wtype)) return QMM_ERR_TYPE;
    if (!is_weight(wtype)) return QMM_ERR_UNSUPPORTED;
    if (count < 1 || count > kMaxMulti) return QMM_ERR_SHAPE;
    if (!W || !y || !M) return QMM_ERR_NULL;
    int rc;
    for (int i = 0; i < count; ++i) {
        if ((rc = check_ptr(W[i])) || (rc = check_ptr(y[i]))) return rc;
        if ((rc = check_dims(wtype, M[i], K))) return rc;
        if (M[i] > INT_MAX) return QMM_ERR_SHAPE;
    }
    if ((rc = check_ptr(x))) return rc;
    const int xt = qmm_vec_dot_type(wtype);
    if ((rc = check_dims(xt, N, K))) return rc;
    if (N > INT_MAX) return QMM_ERR_SHAPE;
    if (K > kMaxK) return QMM_ERR_UNSUPPORTED;
    if (x_is_f32 && (N > 8 || !gemv_fused_supported(wtype, K))) return QMM_ERR_UNSUPPORTED;
    return hip_status(launch_gemv_multi(wtype, count, W, y, M, x, x_is_f32 != 0, N, K,
                                        static_cast<hipStream_t>(stream)));
}

int qmm_probe_read(const void* src, int64_t bytes, uint32_t* sink, int workgroups, void* stream) {
    if (!src || !sink) return QMM_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(src) & 15u) return QMM_ERR_ALIGN;
    if (bytes <= 0 || bytes % 16 || workgroups < 0 || workgroups > QMM_PROBE_SINK_WORDS) return QMM_ERR_SHAPE;
    const int64_t groups = workgroups ? workgroups : probe_read_groups(bytes);
    return hip_status(launch_probe_read(src, bytes, sink, groups, static_cast<hipStream_t>(stream)));
}

int64_t qmm_probe_mfma_ops(int workgroups, int64_t iters) {
    if (workgroups < 1 || workgroups > QMM_PROBE_SINK_WORDS || iters < 1 || iters > (int64_t(1) << 30)) return 0;
    return probe_mfma_ops(workgroups, iters);
}

int qmm_probe_mfma(int workgroups, int64_t iters, uint32_t* sink, void* stream) {
    if (!sink) return QMM_ERR_NULL;
    if (qmm_probe_mfma_ops(workgroups, iters) == 0) return QMM_ERR_SHAPE;
    return hip_status(launch_probe_mfma(workgroups, iters, sink, static_cast<hipStream_t>(stream)));
}

int64_t qmm_probe_mfma16_ops(int workgroups, int64_t iters) {
    if (workgroups < 1 || workgroups > QMM_PROBE_SINK_WORDS || iters < 1 || iters > (int64_t(1) << 30)) return 0;
    return probe_mfma16_ops(workgroups, iters);
}

int qmm_probe_mfma16(int workgroups, int64_t iters, uint32_t* sink, void* stream) {
    if (!sink) return QMM_ERR_NULL;
    if (qmm_probe_mfma16_ops(workgroups, iters) == 0) return QMM_ERR_SHAPE;
    return hip_status(launch_probe_mfma16(workgroups, iters, sink, static_cast<hipStream_t>(stream)));
}

const char* qmm_strerror(int code) {
    switch (code) {
    case QMM_OK: return "ok";
    case QMM_ERR_TYPE: return "unknown block type";
    case QMM_ERR_SHAPE: return "invalid shape (size <= 0, K not a multiple of the block size, or too large)";
    case QMM_ERR_NULL: return "null pointer";
    case QMM_ERR_ALIGN: return "pointer not 16-byte aligned";
    case QMM_ERR_UNSUPPORTED: return "operation not supported for this type or argument";
    case QMM_ERR_HIP: return "HIP launch error";
    default: return "unknown status code";
    }
}

}  // extern "C"
