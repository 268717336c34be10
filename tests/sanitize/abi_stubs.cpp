// Host-only stand-ins for the library's kernel launchers, so that the C ABI's
// argument validation (qmm.cpp) can be built with g++ under AddressSanitizer
// and UndefinedBehaviorSanitizer and driven on a machine without a GPU.  Each
// stand-in counts its calls and enqueues nothing.
#include "../../block_quantized_amd/csrc/qmm_internal.h"

int g_launches = 0;

namespace qmm {

hipError_t launch_quantize(int, const float*, void*, int64_t, int64_t, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_dequantize(int, const void*, float*, int64_t, int64_t, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_gemv(int, const void*, const void*, float*, int64_t, int64_t, int64_t, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_gemv_multi(int, int, const void* const*, float* const*, const int64_t*, const void*, bool, int64_t,
                             int64_t, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
// same rules as the real library: the fused fp32 form needs whole 256-value
// groups (Q6_K rows always are)
bool gemv_fused_supported(int wtype, int64_t K) { return wtype == QMM_Q6_K || K % 256 == 0; }
hipError_t launch_gemm(int, const void*, const void*, float*, int64_t, int64_t, int64_t, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
bool gemm_supported(int wtype) {
    return wtype == QMM_Q4_K || wtype == QMM_Q6_K || wtype == QMM_Q4_0 || wtype == QMM_Q5_0 || wtype == QMM_Q8_0;
}

int64_t probe_read_groups(int64_t bytes) { return bytes / 4096 > 0 ? (bytes / 4096 < 2048 ? bytes / 4096 : 2048) : 1; }
hipError_t launch_probe_read(const void*, int64_t, uint32_t*, int64_t, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_probe_mfma(int64_t, int64_t, uint32_t*, hipStream_t) { ++g_launches; return hipSuccess; }
int64_t probe_mfma_ops(int64_t groups, int64_t iters) { return groups * 16 * iters * 65536; }
hipError_t launch_probe_mfma16(int64_t, int64_t, uint32_t*, hipStream_t) { ++g_launches; return hipSuccess; }
int64_t probe_mfma16_ops(int64_t groups, int64_t iters) { return groups * 32 * iters * 32768; }

}  // namespace qmm
