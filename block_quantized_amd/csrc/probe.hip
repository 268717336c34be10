// probe.hip — two measurement kernels that compute nothing of the product: a
// streaming read of a device buffer and a sustained int8-MFMA loop.  The
// product's rates are reported beside the vendor peaks and beside what these
// reach on the same chip, a measured ceiling next to a theoretical one in the
// manner of the worked table on the page "llama.cpp and GGUF" ("CPU and Edge
// Inference: When It Wins").
#include "qmm_internal.h"

namespace qmm {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;
constexpr int kReadMaxGroups = 2048;  // 8 workgroups of 4 waves per compute unit
constexpr int kMfmaThreads = 256;
constexpr int kMfmaChains = 4;        // independent accumulators per wave
constexpr int kMfma16Chains = 8;      // the same for the 16x16x64 form (shorter latency per instruction)

__device__ __forceinline__ uint32_t wave_xor(uint32_t x) {
    for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
    return x;
}

// Workgroup g stores the XOR of its threads' values to sink[g] (a plain
// store: one same-address atomic per wave would serialise thousands of
// waves at the end of a short launch).  256 threads.
__device__ __forceinline__ void store_group_xor(uint32_t x, uint32_t* sink) {
    __shared__ uint32_t part[4];
    x = wave_xor(x);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// Each 16-byte piece is loaded once: consecutive lanes take consecutive
// pieces, and a thread strides over the buffer by the grid's width, kReadUnroll
// pieces in flight per step.  Non-temporal loads: measured on MI355X over
// 2 GiB they stream at about 7.1 TB/s against 6.3 TB/s for ordinary loads.  The XOR of the 32-bit words a workgroup read
// goes to sink[workgroup], so no load can be dropped.
__global__ __launch_bounds__(kReadThreads) void read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                            uint32_t* sink) {
    const int64_t stride = (int64_t)gridDim.x * kReadThreads;
    int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int j = 0; j < kReadUnroll; ++j) v[j] = __builtin_nontemporal_load(src + i + j * stride);
#pragma unroll
        for (int j = 0; j < kReadUnroll; ++j) acc ^= v[j];
    }
    for (; i < n16; i += stride) acc ^= src[i];
    store_group_xor(acc.x ^ acc.y ^ acc.z ^ acc.w, sink);
}

// The same for v_mfma_i32_16x16x64_i8 (16x16 tiles over K = 64: the form
// the 16-row narrow kernels use), kMfma16Chains accumulators per wave.
__global__ __launch_bounds__(kMfmaThreads) void mfma16_kernel(int64_t iters, uint32_t* sink) {
    const int l = (int)threadIdx.x;
    const v4i a = {l * 0x01030507, l ^ 0x0f0e0d0c, l * 0x11, l + 0x7f7f7f7f};
    const v4i b = {l * 0x02040608, l ^ 0x70605040, l * 0x13, l - 0x01010101};
    v4i acc[kMfma16Chains];
#pragma unroll
    for (int c = 0; c < kMfma16Chains; ++c) acc[c] = (v4i){};
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kMfma16Chains; ++c) acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[c], 0, 0, 0);
    }
    uint32_t x = 0;
#pragma unroll
    for (int c = 0; c < kMfma16Chains; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) x ^= (uint32_t)acc[c][e] * (uint32_t)(2 * (c * 4 + e) + 1);
    store_group_xor(x, sink);
}

// kMfmaChains independent v_mfma_i32_32x32x32_i8 accumulations per wave,
// `iters` steps each, on operands that depend on the lane (so nothing folds);
// a digest of the accumulators goes to sink[workgroup].
__global__ __launch_bounds__(kMfmaThreads) void mfma_kernel(int64_t iters, uint32_t* sink) {
    const int l = (int)threadIdx.x;
    const v4i a = {l * 0x01030507, l ^ 0x0f0e0d0c, l * 0x11, l + 0x7f7f7f7f};
    const v4i b = {l * 0x02040608, l ^ 0x70605040, l * 0x13, l - 0x01010101};
    v16i acc[kMfmaChains];
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = (v16i){};
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kMfmaChains; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
    }
    uint32_t x = 0;
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) x ^= (uint32_t)acc[c][e] * (uint32_t)(2 * (c * 16 + e) + 1);
    store_group_xor(x, sink);
}

}  // namespace

int64_t probe_read_groups(int64_t bytes) {
    const int64_t n16 = bytes / 16;
    const int64_t g = (n16 + kReadThreads - 1) / kReadThreads;
    return g < 1 ? 1 : (g > kReadMaxGroups ? kReadMaxGroups : g);
}

hipError_t launch_probe_read(const void* src, int64_t bytes, uint32_t* sink, int64_t groups, hipStream_t s) {
    return launch(read_kernel, dim3((unsigned)groups), dim3(kReadThreads), 0, s,
                  static_cast<const u32x4*>(src), bytes / 16, sink);
}

hipError_t launch_probe_mfma(int64_t groups, int64_t iters, uint32_t* sink, hipStream_t s) {
    return launch(mfma_kernel, dim3((unsigned)groups), dim3(kMfmaThreads), 0, s, iters, sink);
}

int64_t probe_mfma_ops(int64_t groups, int64_t iters) {
    return groups * (kMfmaThreads / 64) * kMfmaChains * iters * (int64_t)(2 * 32 * 32 * 32);
}

hipError_t launch_probe_mfma16(int64_t groups, int64_t iters, uint32_t* sink, hipStream_t s) {
    return launch(mfma16_kernel, dim3((unsigned)groups), dim3(kMfmaThreads), 0, s, iters, sink);
}

int64_t probe_mfma16_ops(int64_t groups, int64_t iters) {
    return groups * (kMfmaThreads / 64) * kMfma16Chains * iters * (int64_t)(2 * 16 * 16 * 64);
}

}  // namespace qmm
