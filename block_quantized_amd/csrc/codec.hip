// codec.hip — round-to-nearest quantizers and dequantizers for gfx950.
//
// Formats: the format table of page "The GGML ecosystem, and where synapse
// fits", §5 "Quantization".  Activation quantization to the vec_dot_type
// happens once per activation row before the product (§5, "Products: weights
// against quantized activations").
//
// Bit-exactness: every result here is defined to the bit.  This translation
// unit is built with -ffp-contract=off and without fast-math, so fp32
// division is the correctly rounded v_div_scale/fmas/fixup sequence, roundf
// rounds half away from zero, fp32->fp16 rounds to nearest even with
// subnormals, and no multiply is fused into an add.
//
// Work mapping: one lane owns four consecutive fp32 values (one 16-byte
// load or store), so a 32-value block is 8 lanes and a 256-value block is a
// whole wavefront; block-wide maxima and sums are cross-lane butterflies.
#include "qmm_internal.h"

namespace qmm {
namespace {

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
           ((uint32_t)(d & 0xFF) << 24);
}

__device__ __forceinline__ void st_u16x2(uint8_t* p, uint32_t v) {  // p is 2-byte aligned
    reinterpret_cast<uint16_t*>(p)[0] = (uint16_t)(v & 0xFFFF);
    reinterpret_cast<uint16_t*>(p)[1] = (uint16_t)(v >> 16);
}

__device__ __forceinline__ uint32_t ld_u16x2(const uint8_t* p) {  // p is 2-byte aligned
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
    return (uint32_t)q[0] | ((uint32_t)q[1] << 16);
}

__device__ __forceinline__ float amax4(float4 v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// ---------------------------------------------------------------- Q8_0
// 8 lanes per 32-value block; fp16 d then 32 int8 codes (34 bytes).
__global__ __launch_bounds__(256) void quantize_q8_0_kernel(const float* __restrict__ x, uint8_t* __restrict__ out,
                                                            int64_t nblocks) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t b = t >> 3;
    const int sub = threadIdx.x & 7;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (b < nblocks) v = reinterpret_cast<const float4*>(x)[t];
    float a = amax4(v);
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    a = fmaxf(a, __shfl_xor(a, 4));
    if (b >= nblocks) return;
    float d, id;
    rtn_scale(a, d, id);
    const uint32_t q = pack4(rtn_code(v.x * id), rtn_code(v.y * id), rtn_code(v.z * id), rtn_code(v.w * id));
    uint8_t* blk = out + b * kQ8_0Bytes;
    st_u16x2(blk + 2 + 4 * sub, q);
    if (sub == 0) reinterpret_cast<uint16_t*>(blk)[0] = (uint16_t)f2h(d);
}

// ---------------------------------------------------------------- Q8_K
// One wavefront per 256-value block: fp32 d, 256 int8 codes, and the 16
// int16 sums of each run of 16 codes (292 bytes).
__global__ __launch_bounds__(256) void quantize_q8_k_kernel(const float* __restrict__ x, uint8_t* __restrict__ out,
                                                            int64_t nblocks) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t b = t >> 6;
    const int lane = threadIdx.x & 63;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (b < nblocks) v = reinterpret_cast<const float4*>(x)[t];
    float a = amax4(v);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) a = fmaxf(a, __shfl_xor(a, m));
    float d, id;
    rtn_scale(a, d, id);
    const int q0 = rtn_code(v.x * id), q1 = rtn_code(v.y * id), q2 = rtn_code(v.z * id), q3 = rtn_code(v.w * id);
    int s = q0 + q1 + q2 + q3;
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (b >= nblocks) return;
    uint8_t* blk = out + b * kQ8_KBytes;
    reinterpret_cast<uint32_t*>(blk + 4)[lane] = pack4(q0, q1, q2, q3);
    if ((lane & 3) == 0) reinterpret_cast<int16_t*>(blk + 260)[lane >> 2] = (int16_t)s;
    if (lane == 0) reinterpret_cast<float*>(blk)[0] = d;
}

// ---------------------------------------------------------------- Q4_0
// Weight encoder, 8 lanes per 32-value block.  m = first value of largest
// magnitude (+0 when the block is all zeros), d = m / -8, code =
// clamp(roundf(x * (1/d)), -8, 7) + 8; element e < 16 in the low nibble of
// byte e, e >= 16 in the high nibble of byte e - 16.
__global__ __launch_bounds__(256) void quantize_q4_0_kernel(const float* __restrict__ x, uint8_t* __restrict__ out,
                                                            int64_t nblocks) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t b = t >> 3;
    const int sub = threadIdx.x & 7;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (b < nblocks) v = reinterpret_cast<const float4*>(x)[t];
    // first maximum of |x| within the lane, then across the 8 lanes; every
    // element, the first included, must beat the running maximum (from 0)
    // with a strict >, so NaN never wins and an all-zero block keeps m = 0
    float ba = 0.0f, bm = 0.0f;
    int bi = 0;
    if (fabsf(v.x) > ba) { ba = fabsf(v.x); bm = v.x; }
    if (fabsf(v.y) > ba) { ba = fabsf(v.y); bm = v.y; bi = 1; }
    if (fabsf(v.z) > ba) { ba = fabsf(v.z); bm = v.z; bi = 2; }
    if (fabsf(v.w) > ba) { ba = fabsf(v.w); bm = v.w; bi = 3; }
    bi += 4 * sub;
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
        const float oa = __shfl_xor(ba, m), om = __shfl_xor(bm, m);
        const int oi = __shfl_xor(bi, m);
        if (oa > ba || (oa == ba && oi < bi)) { ba = oa; bm = om; bi = oi; }
    }
    const float mval = (ba > 0.0f) ? bm : 0.0f;
    const float d = mval / -8.0f;
    const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    auto code = [id](float xv) {
        float r = roundf(xv * id);
        if (r != r) r = 0.0f;
        if (r < -8.0f) r = -8.0f;
        if (r > 7.0f) r = 7.0f;
        return (int)r + 8;
    };
    const uint32_t q = pack4(code(v.x), code(v.y), code(v.z), code(v.w));
    const uint32_t qhi = __shfl_xor(q, 4);  // lanes 0-3 take elements 16.. from lanes 4-7
    if (b >= nblocks || sub >= 4) return;
    uint8_t* blk = out + b * kQ4_0Bytes;
    st_u16x2(blk + 2 + 4 * sub, q | (qhi << 4));
    if (sub == 0) reinterpret_cast<uint16_t*>(blk)[0] = (uint16_t)f2h(d);
}

// ------------------------------------------------------------ dequantize
// One lane writes four consecutive fp32 outputs (a 16-byte store).

__global__ __launch_bounds__(256) void dequant_q4_0_kernel(const uint8_t* __restrict__ w, float* __restrict__ out,
                                                           int64_t nquads) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= nquads) return;
    const int64_t b = t >> 3;
    const int sub = (int)(t & 7);
    const uint8_t* blk = w + b * kQ4_0Bytes;
    const float d = h2f(reinterpret_cast<const uint16_t*>(blk)[0]);
    uint32_t qs = ld_u16x2(blk + 2 + 4 * (sub & 3));
    if (sub >= 4) qs >>= 4;
    float4 r;
    r.x = d * (float)((int)(qs & 15) - 8);
    r.y = d * (float)((int)((qs >> 8) & 15) - 8);
    r.z = d * (float)((int)((qs >> 16) & 15) - 8);
    r.w = d * (float)((int)((qs >> 24) & 15) - 8);
    reinterpret_cast<float4*>(out)[t] = r;
}

// Q5_0: as Q4_0's nibbles, plus the fifth bit of element e from bit e of
// the little-endian 32-bit qh; w = d (q - 16), exact in fp32.
__global__ __launch_bounds__(256) void dequant_q5_0_kernel(const uint8_t* __restrict__ w, float* __restrict__ out,
                                                           int64_t nquads) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= nquads) return;
    const int64_t b = t >> 3;
    const int sub = (int)(t & 7);
    const uint8_t* blk = w + b * kQ5_0Bytes;
    const float d = h2f(reinterpret_cast<const uint16_t*>(blk)[0]);
    const uint32_t qh = ld_u16x2(blk + 2) >> (4 * sub);  // bits of elements 4 sub .. 4 sub + 3
    uint32_t qs = ld_u16x2(blk + 6 + 4 * (sub & 3));
    if (sub >= 4) qs >>= 4;
    float4 r;
    r.x = d * (float)((int)((qs & 15) | ((qh & 1) << 4)) - 16);
    r.y = d * (float)((int)(((qs >> 8) & 15) | (((qh >> 1) & 1) << 4)) - 16);
    r.z = d * (float)((int)(((qs >> 16) & 15) | (((qh >> 2) & 1) << 4)) - 16);
    r.w = d * (float)((int)(((qs >> 24) & 15) | (((qh >> 3) & 1) << 4)) - 16);
    reinterpret_cast<float4*>(out)[t] = r;
}

__global__ __launch_bounds__(256) void dequant_q8_0_kernel(const uint8_t* __restrict__ w, float* __restrict__ out,
                                                           int64_t nquads) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= nquads) return;
    const int64_t b = t >> 3;
    const int sub = (int)(t & 7);
    const uint8_t* blk = w + b * kQ8_0Bytes;
    const float d = h2f(reinterpret_cast<const uint16_t*>(blk)[0]);
    const uint32_t qs = ld_u16x2(blk + 2 + 4 * sub);
    float4 r;
    r.x = d * (float)(int8_t)(qs & 0xFF);
    r.y = d * (float)(int8_t)((qs >> 8) & 0xFF);
    r.z = d * (float)(int8_t)((qs >> 16) & 0xFF);
    r.w = d * (float)(int8_t)(qs >> 24);
    reinterpret_cast<float4*>(out)[t] = r;
}

// Q4_K: 64 lanes per super-block; lane owns elements 4l..4l+3 of sub-block
// j = l/8.  The 12 scale bytes hold sc0-3 / m0-3 in the low six bits of
// bytes 0-3 / 4-7, the low nibbles of sc4-7 / m4-7 in the low / high nibbles
// of bytes 8-11, and bits 4-5 of sc4-7 / m4-7 in the top two bits of bytes
// 0-3 / 4-7.
// (The 16-byte header d, dmin, scales is read as one 16-byte load, which
// every lane of a super-block shares, and both forms are computed and one
// selected: with byte loads behind a branch on j, half the lanes waited for
// a second memory round trip.)
__device__ __forceinline__ void q4k_scale_min(const uint4& hdr, int j, int& sc, int& m) {
    const int sh = 8 * (j & 3);
    const uint32_t s0 = (hdr.y >> sh) & 0xFF, s1 = (hdr.z >> sh) & 0xFF, s2 = (hdr.w >> sh) & 0xFF;
    const bool lo = j < 4;
    sc = (int)(lo ? (s0 & 63) : ((s2 & 15) | ((s0 >> 6) << 4)));
    m = (int)(lo ? (s1 & 63) : ((s2 >> 4) | ((s1 >> 6) << 4)));
}

__global__ __launch_bounds__(256) void dequant_q4_k_kernel(const uint8_t* __restrict__ w, float* __restrict__ out,
                                                           int64_t nquads) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= nquads) return;
    const int64_t b = t >> 6;
    const int l = (int)(t & 63);
    const uint8_t* blk = w + b * kQ4_KBytes;
    const int j = l >> 3;
    uint32_t qs = reinterpret_cast<const uint32_t*>(blk + 16 + 32 * (j >> 1))[l & 7];
    const uint4 hdr = reinterpret_cast<const uint4*>(blk)[0];
    const float d = h2f(hdr.x), dmin = h2f(hdr.x >> 16);
    int sc, m;
    q4k_scale_min(hdr, j, sc, m);
    if (j & 1) qs >>= 4;
    const float a = d * (float)sc;
    const float c = dmin * (float)m;
    float4 r;
    r.x = a * (float)(qs & 15) - c;
    r.y = a * (float)((qs >> 8) & 15) - c;
    r.z = a * (float)((qs >> 16) & 15) - c;
    r.w = a * (float)((qs >> 24) & 15) - c;
    reinterpret_cast<float4*>(out)[t] = r;
}

// Q6_K: 64 lanes per super-block; lane owns elements e = 4l..4l+3.  Half
// h = e/128, quarter c = (e%128)/32, position p = e%32: low four bits from
// ql[64h + p + 32(c&1)] (low nibble for c < 2, high for c >= 2), high two
// bits from bits 2c..2c+1 of qh[32h + p]; w = (d * sc[e/16]) * (q - 32).
__global__ __launch_bounds__(256) void dequant_q6_k_kernel(const uint8_t* __restrict__ w, float* __restrict__ out,
                                                           int64_t nquads) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= nquads) return;
    const int64_t b = t >> 6;
    const int l = (int)(t & 63);
    const uint8_t* blk = w + b * kQ6_KBytes;
    const int e = 4 * l, h = e >> 7, c = (e & 127) >> 5, p = e & 31;
    uint32_t lo = ld_u16x2(blk + 64 * h + p + 32 * (c & 1));
    if (c >= 2) lo >>= 4;
    const uint32_t hi = ld_u16x2(blk + 128 + 32 * h + p) >> (2 * c);
    const int sc = (int8_t)blk[192 + (e >> 4)];
    const float a = h2f(reinterpret_cast<const uint16_t*>(blk + 208)[0]) * (float)sc;
    float4 r;
    r.x = a * (float)((int)((lo & 15) | ((hi & 3) << 4)) - 32);
    r.y = a * (float)((int)(((lo >> 8) & 15) | (((hi >> 8) & 3) << 4)) - 32);
    r.z = a * (float)((int)(((lo >> 16) & 15) | (((hi >> 16) & 3) << 4)) - 32);
    r.w = a * (float)((int)(((lo >> 24) & 15) | (((hi >> 24) & 3) << 4)) - 32);
    reinterpret_cast<float4*>(out)[t] = r;
}

__global__ __launch_bounds__(256) void dequant_q8_k_kernel(const uint8_t* __restrict__ w, float* __restrict__ out,
                                                           int64_t nquads) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= nquads) return;
    const int64_t b = t >> 6;
    const int l = (int)(t & 63);
    const uint8_t* blk = w + b * kQ8_KBytes;
    const float d = reinterpret_cast<const float*>(blk)[0];
    const uint32_t qs = reinterpret_cast<const uint32_t*>(blk + 4)[l];
    float4 r;
    r.x = d * (float)(int8_t)(qs & 0xFF);
    r.y = d * (float)(int8_t)((qs >> 8) & 0xFF);
    r.z = d * (float)(int8_t)((qs >> 16) & 0xFF);
    r.w = d * (float)(int8_t)(qs >> 24);
    reinterpret_cast<float4*>(out)[t] = r;
}

inline unsigned grid_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

}  // namespace

hipError_t launch_quantize(int dst, const float* x, void* out, int64_t rows, int64_t K, hipStream_t s) {
    const int64_t nb = rows * (K / block_size(dst));
    uint8_t* o = static_cast<uint8_t*>(out);
    switch (dst) {
    case QMM_Q8_0: return launch(quantize_q8_0_kernel, dim3(grid_for(nb * 8)), dim3(256), 0, s, x, o, nb);
    case QMM_Q8_K: return launch(quantize_q8_k_kernel, dim3(grid_for(nb * 64)), dim3(256), 0, s, x, o, nb);
    case QMM_Q4_0: return launch(quantize_q4_0_kernel, dim3(grid_for(nb * 8)), dim3(256), 0, s, x, o, nb);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dequantize(int t, const void* blocks, float* out, int64_t rows, int64_t K, hipStream_t s) {
    const int64_t nq = rows * K / 4;
    const uint8_t* w = static_cast<const uint8_t*>(blocks);
    const dim3 g(grid_for(nq)), blk(256);
    switch (t) {
    case QMM_Q4_0: return launch(dequant_q4_0_kernel, g, blk, 0, s, w, out, nq);
    case QMM_Q8_0: return launch(dequant_q8_0_kernel, g, blk, 0, s, w, out, nq);
    case QMM_Q5_0: return launch(dequant_q5_0_kernel, g, blk, 0, s, w, out, nq);
    case QMM_Q4_K: return launch(dequant_q4_k_kernel, g, blk, 0, s, w, out, nq);
    case QMM_Q6_K: return launch(dequant_q6_k_kernel, g, blk, 0, s, w, out, nq);
    case QMM_Q8_K: return launch(dequant_q8_k_kernel, g, blk, 0, s, w, out, nq);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
