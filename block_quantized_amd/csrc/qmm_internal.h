// qmm_internal.h — declarations shared by the library's translation units.
// Host-side launch functions (one per kernel family) and small device helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>

#include "../../include/qmm.h"
#include "../../include/qmm_probe.h"

namespace qmm {

// Block geometry of the format table (page "The GGML ecosystem, and where
// synapse fits", §5 "Quantization").
constexpr int kQ4_0Bytes = 18, kQ8_0Bytes = 34, kQ4_KBytes = 144, kQ6_KBytes = 210, kQ8_KBytes = 292,
              kQ5_0Bytes = 22;

__host__ __device__ constexpr int block_size(int t) {
    return (t == QMM_Q4_0 || t == QMM_Q8_0 || t == QMM_Q5_0) ? 32
         : (t == QMM_Q4_K || t == QMM_Q6_K || t == QMM_Q8_K) ? 256 : 0;
}
__host__ __device__ constexpr int block_bytes(int t) {
    return t == QMM_Q4_0 ? kQ4_0Bytes : t == QMM_Q5_0 ? kQ5_0Bytes : t == QMM_Q8_0 ? kQ8_0Bytes : t == QMM_Q4_K ? kQ4_KBytes
         : t == QMM_Q6_K ? kQ6_KBytes : t == QMM_Q8_K ? kQ8_KBytes : 0;
}

#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)
// IEEE binary16 bits -> fp32 (v_cvt_f32_f16: exact, subnormals kept).
__device__ __forceinline__ float h2f(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(bits16 & 0xFFFFu));
}
// fp32 -> binary16 bits, round to nearest even (v_cvt_f16_f32).
__device__ __forceinline__ uint32_t f2h(float f) {
    return (uint32_t)__builtin_bit_cast(unsigned short, (_Float16)f);
}
// Round-to-nearest activation code: roundf(t) (half away from zero); NaN
// (0 * Inf when 1/d overflowed) -> 0; clamp to [-127, 127].  Used by the
// stand-alone quantizers and by the product's fused quantization alike.
// Branch-free: v_med3 clamps (+-Inf -> +-127) and a select maps NaN to 0.
__device__ __forceinline__ int rtn_code(float t) {
    const float r = __builtin_amdgcn_fmed3f(roundf(t), -127.0f, 127.0f);
    return (t == t) ? (int)r : 0;
}
// Word 3 of a raw buffer resource on gfx9-family chips (gfx950 included):
// 32-bit data format, no swizzle.  With stride 0, an access at or past
// num_records bytes is out of range: loads return 0 and stores are dropped.
constexpr int kBufferWord3 = 0x00020000;
// The block scale and its reciprocal: d = amax / 127 (correctly rounded),
// id = 1/d, or 0 when d == 0.
__device__ __forceinline__ void rtn_scale(float amax, float& d, float& id) {
    d = amax / 127.0f;
    id = (d != 0.0f) ? 1.0f / d : 0.0f;
}
#endif

// Launches kernel k and returns the status of this launch alone.  Unlike
// hipGetLastError() after a triple-chevron launch, an error left by an
// earlier, unrelated HIP call in the same thread is neither reported nor
// cleared.  The arguments are converted to the kernel's parameter types.
template <typename... P, typename... A>
hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s, A... a) {
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    std::tuple<std::decay_t<P>...> args{static_cast<std::decay_t<P>>(a)...};
    void* ptrs[sizeof...(P) > 0 ? sizeof...(P) : 1] = {};
    std::apply([&ptrs](auto&... e) {
        int i = 0;
        ((ptrs[i++] = static_cast<void*>(&e)), ...);
    }, args);
    return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, ptrs, lds, s);
}

// ---- launchers (return hipError_t of the launch) ----
hipError_t launch_quantize(int dst, const float* x, void* out, int64_t rows, int64_t K, hipStream_t s);
hipError_t launch_dequantize(int t, const void* blocks, float* out, int64_t rows, int64_t K, hipStream_t s);
hipError_t launch_gemv(int wtype, const void* W, const void* xq, float* y, int64_t M, int64_t N, int64_t K,
                       hipStream_t s);
// Several matrices sharing K and x in one launch (count <= kMaxMulti).  x is
// either quantized activation blocks (x_f32 == false) or fp32 rows that the
// kernel quantizes itself, bit-identically to launch_quantize (N <= 8 then).
constexpr int kMaxMulti = 4;
hipError_t launch_gemv_multi(int wtype, int count, const void* const* W, float* const* y, const int64_t* M,
                             const void* x, bool x_f32, int64_t N, int64_t K, hipStream_t s);
bool gemv_fused_supported(int wtype, int64_t K);
// int8-MFMA product for many activation rows (weight types gemm_supported()).
hipError_t launch_gemm(int wtype, const void* W, const void* xq, float* y, int64_t M, int64_t N, int64_t K,
                       hipStream_t s);
bool gemm_supported(int wtype);
// Measurement kernels (qmm_probe.h).
int64_t probe_read_groups(int64_t bytes);
hipError_t launch_probe_read(const void* src, int64_t bytes, uint32_t* sink, int64_t groups, hipStream_t s);
hipError_t launch_probe_mfma(int64_t groups, int64_t iters, uint32_t* sink, hipStream_t s);
int64_t probe_mfma_ops(int64_t groups, int64_t iters);
hipError_t launch_probe_mfma16(int64_t groups, int64_t iters, uint32_t* sink, hipStream_t s);
int64_t probe_mfma16_ops(int64_t groups, int64_t iters);

}  // namespace qmm
