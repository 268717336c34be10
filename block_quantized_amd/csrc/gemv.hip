// gemv.hip — decode-path product y = W x^T for N <= 8 activation rows, on
// raw GGUF blocks, for gfx950.
//
// Method (page "The GGML ecosystem, and where synapse fits", §5, "Products:
// weights against quantized activations"): each weight block is dotted with
// the matching activation block in integer arithmetic (v_dot4_i32_i8 over
// packed int8 lanes) and only the block scales are float.  Per 256 weights:
//   Q4_0 x Q8_0: sum_i (dw*dx)_i * (sum q_w q_x - 8 sum q_x)       (8 blocks)
//   Q8_0 x Q8_0: sum_i (dw*dx)_i * sum q_w q_x                       (8 blocks)
//   Q4_K x Q8_K: dx * (d sum_j sc_j sum q_w q_x - dmin sum_j m_j S_j) (S_j: the
//                two 16-wide sums of sub-block j)
//   Q6_K x Q8_K: dx * d * sum_j sc_j (sum q_w q_x - 32 S_j)          (S_j: 16-wide sum)
// (the Q6_K offset 32 is this library's reading of the format table).
// Decode speed is bound by streaming the weights from memory (page "llama.cpp
// and GGUF", "The ggml Tensor Library and Backends": decode speed tracks memory
// bandwidth), so the kernel is organised around moving W at full HBM rate:
//
//  * The unit of work of one lane is 256 consecutive weights of one row
//    ("unit": 144 B of Q4_0 or Q4_K, 272 B of Q8_0, 210 B of Q6_K).  A row of
//    K weights is G = K/256 units.  P = next power of two >= min(G, 64)
//    lanes share a row; a wavefront covers RW = 64/P whole rows per "chunk",
//    or, when G > 64, a row in ceil(G/64) chunks of 64 units.  A chunk is one
//    contiguous byte range of W.
//  * Chunks are read with coalesced 16-byte loads (lane l reads bytes
//    16(l + 64j)), one chunk ahead of the compute, into VGPRs; the chunk is
//    then written to the wavefront's private LDS slot, where each lane reads
//    its own unit back.  No workgroup barrier is needed in the main loop.
//  * The activations (N rows of Q8_0 or Q8_K blocks) are repacked once per
//    workgroup into LDS records of 336 bytes per (row, 256-value group):
//    256 int8 codes, then the fp32 scales and precomputed integer sums.  The
//    record stride (84 dwords) keeps 16-byte LDS reads of consecutive groups
//    on distinct banks.
//  * Workgroups are persistent: each wavefront walks chunks with a grid
//    stride; lanes of a row are reduced with a fixed butterfly, so results
//    are bit-identical run to run.
#include "qmm_internal.h"

namespace qmm {
namespace {

template <int WT> struct GFmt;
template <> struct GFmt<QMM_Q4_0> { static constexpr int UB = 144, NJ = 9; };
template <> struct GFmt<QMM_Q8_0> { static constexpr int UB = 272, NJ = 17; };
template <> struct GFmt<QMM_Q4_K> { static constexpr int UB = 144, NJ = 9; };
template <> struct GFmt<QMM_Q6_K> { static constexpr int UB = 210, NJ = 14; };  // 13440 B + up to 14 B skew

constexpr int XREC = 336;  // LDS bytes per (activation row, 256-value group)

struct GemvArgs {
    const uint8_t* W;
    const uint8_t* xq;
    float* y;
    int64_t M;        // rows of W (and columns of y)
    int64_t rowB;     // bytes per W row
    int64_t total;    // bytes of W
    int64_t nwork;    // work items (row sets)
    int64_t ldy;      // row stride of y (= M of the full problem)
    int G;            // 256-weight units per row
    int logP;         // log2(lanes per row)
    int RW;           // rows per chunk
    int nkc;          // chunks per work item
};

__device__ __forceinline__ uint32_t ld_u16x2_g(const uint8_t* p) {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
    return (uint32_t)q[0] | ((uint32_t)q[1] << 16);
}

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// ---------------------------------------------------- activation staging

template <int WT, int NC>
__device__ void stage_x(const GemvArgs& a, uint8_t* xl) {
    const int G = a.G;
    if constexpr (WT == QMM_Q4_0 || WT == QMM_Q8_0) {
        // Q8_0 activations: group g of row n = blocks 8g..8g+7 (34 B each).
        const int64_t xrow = (int64_t)G * 8 * kQ8_0Bytes;
        for (int i = threadIdx.x; i < NC * G * 64; i += blockDim.x) {
            const int n = i / (G * 64), r = i - n * G * 64, g = r >> 6, qd = r & 63;
            const uint8_t* blk = a.xq + n * xrow + (int64_t)(8 * g + (qd >> 3)) * kQ8_0Bytes;
            reinterpret_cast<uint32_t*>(xl + (n * G + g) * XREC)[qd] = ld_u16x2_g(blk + 2 + 4 * (qd & 7));
        }
        for (int i = threadIdx.x; i < NC * G * 8; i += blockDim.x) {
            const int n = i / (G * 8), r = i - n * G * 8, g = r >> 3, bi = r & 7;
            const uint8_t* blk = a.xq + n * xrow + (int64_t)(8 * g + bi) * kQ8_0Bytes;
            uint32_t* rec = reinterpret_cast<uint32_t*>(xl + (n * G + g) * XREC);
            reinterpret_cast<float*>(rec)[64 + bi] = h2f(reinterpret_cast<const uint16_t*>(blk)[0]);
            int s = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) s = dot4(ld_u16x2_g(blk + 2 + 4 * k), 0x01010101u, s);
            reinterpret_cast<int*>(rec)[72 + bi] = 8 * s;  // Q4_0's offset term: 8 * sum q_x
        }
    } else {
        // Q8_K activations: group g of row n = block g (292 B).
        const int64_t xrow = (int64_t)G * kQ8_KBytes;
        for (int i = threadIdx.x; i < NC * G * 64; i += blockDim.x) {
            const int n = i / (G * 64), r = i - n * G * 64, g = r >> 6, qd = r & 63;
            const uint8_t* blk = a.xq + n * xrow + (int64_t)g * kQ8_KBytes;
            reinterpret_cast<uint32_t*>(xl + (n * G + g) * XREC)[qd] =
                reinterpret_cast<const uint32_t*>(blk + 4)[qd];
        }
        constexpr int NM = (WT == QMM_Q4_K) ? 8 : 16;
        for (int i = threadIdx.x; i < NC * G * (NM + 1); i += blockDim.x) {
            const int n = i / (G * (NM + 1)), r = i - n * G * (NM + 1), g = r / (NM + 1), j = r % (NM + 1);
            const uint8_t* blk = a.xq + n * xrow + (int64_t)g * kQ8_KBytes;
            uint32_t* rec = reinterpret_cast<uint32_t*>(xl + (n * G + g) * XREC);
            const int16_t* bs = reinterpret_cast<const int16_t*>(blk + 260);
            if (j == NM) {
                rec[64] = reinterpret_cast<const uint32_t*>(blk)[0];  // fp32 d
            } else if (WT == QMM_Q4_K) {
                reinterpret_cast<int*>(rec)[65 + j] = (int)bs[2 * j] + (int)bs[2 * j + 1];
            } else {
                reinterpret_cast<int*>(rec)[65 + j] = 32 * (int)bs[j];
            }
        }
    }
}

// ------------------------------------------------------- unit compute

template <int NC>
__device__ __forceinline__ void unit_q4_0(const uint32_t* __restrict__ u, const uint8_t* xr0, int xstride,
                                          float (&acc)[NC]) {
    uint32_t w[36];
#pragma unroll
    for (int i = 0; i < 9; ++i) reinterpret_cast<uint4*>(w)[i] = reinterpret_cast<const uint4*>(u)[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t db, q[4];
        if ((i & 1) == 0) {
            const int b = 9 * i / 2;
            db = w[b];
#pragma unroll
            for (int k = 0; k < 4; ++k) q[k] = __builtin_amdgcn_alignbyte(w[b + k + 1], w[b + k], 2);
        } else {
            const int b = 9 * (i - 1) / 2 + 4;
            db = w[b] >> 16;
#pragma unroll
            for (int k = 0; k < 4; ++k) q[k] = w[b + 1 + k];
        }
        const float dw = h2f(db);
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            lo[k] = q[k] & 0x0F0F0F0Fu;
            hi[k] = (q[k] >> 4) & 0x0F0F0F0Fu;
        }
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            const uint32_t* xr = reinterpret_cast<const uint32_t*>(xr0 + n * xstride);
            int dot = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                dot = dot4(lo[k], xr[8 * i + k], dot);
                dot = dot4(hi[k], xr[8 * i + 4 + k], dot);
            }
            const int isum = dot - reinterpret_cast<const int*>(xr)[72 + i];
            const float dx = reinterpret_cast<const float*>(xr)[64 + i];
            acc[n] += (float)isum * (dw * dx);
        }
    }
}

template <int NC>
__device__ __forceinline__ void unit_q8_0(const uint32_t* __restrict__ u, const uint8_t* xr0, int xstride,
                                          float (&acc)[NC]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t db, q[8];
        if ((i & 1) == 0) {
            const int b = 17 * i / 2;
            uint32_t w[9];
#pragma unroll
            for (int k = 0; k < 9; ++k) w[k] = u[b + k];
            db = w[0];
#pragma unroll
            for (int k = 0; k < 8; ++k) q[k] = __builtin_amdgcn_alignbyte(w[k + 1], w[k], 2);
        } else {
            const int b = (17 * i - 1) / 2;
            db = u[b] >> 16;
#pragma unroll
            for (int k = 0; k < 8; ++k) q[k] = u[b + 1 + k];
        }
        const float dw = h2f(db);
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            const uint32_t* xr = reinterpret_cast<const uint32_t*>(xr0 + n * xstride);
            int dot = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) dot = dot4(q[k], xr[8 * i + k], dot);
            const float dx = reinterpret_cast<const float*>(xr)[64 + i];
            acc[n] += (float)dot * (dw * dx);
        }
    }
}

template <int NC>
__device__ __forceinline__ void unit_q4_k(const uint32_t* __restrict__ u, const uint8_t* xr0, int xstride,
                                          float (&acc)[NC]) {
    const uint4 h = reinterpret_cast<const uint4*>(u)[0];
    const float d = h2f(h.x), dmin = h2f(h.x >> 16);
    // eight 6-bit scales and mins, one per byte
    const uint32_t sc03 = h.y & 0x3F3F3F3Fu, m03 = h.z & 0x3F3F3F3Fu;
    const uint32_t sc47 = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
    const uint32_t m47 = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
    int sumi[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) sumi[n] = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        uint32_t q[8];
        reinterpret_cast<uint4*>(q)[0] = reinterpret_cast<const uint4*>(u)[1 + 2 * g];
        reinterpret_cast<uint4*>(q)[1] = reinterpret_cast<const uint4*>(u)[2 + 2 * g];
        const uint32_t scw = (g < 2) ? sc03 : sc47;
        const int sc_lo = (scw >> (16 * (g & 1))) & 0xFF, sc_hi = (scw >> (16 * (g & 1) + 8)) & 0xFF;
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            const uint32_t* xr = reinterpret_cast<const uint32_t*>(xr0 + n * xstride);
            int dl = 0, dh = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                dl = dot4(q[k] & 0x0F0F0F0Fu, xr[16 * g + k], dl);
                dh = dot4((q[k] >> 4) & 0x0F0F0F0Fu, xr[16 * g + 8 + k], dh);
            }
            sumi[n] += sc_lo * dl + sc_hi * dh;
        }
    }
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const uint32_t* xr = reinterpret_cast<const uint32_t*>(xr0 + n * xstride);
        const int* bs = reinterpret_cast<const int*>(xr) + 65;
        int summ = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            summ += (int)((m03 >> (8 * j)) & 0xFF) * bs[j];
            summ += (int)((m47 >> (8 * j)) & 0xFF) * bs[4 + j];
        }
        const float dx = reinterpret_cast<const float*>(xr)[64];
        acc[n] += dx * (d * (float)sumi[n] - dmin * (float)summ);
    }
}

template <int NC>
__device__ __forceinline__ void unit_q6_k(const uint32_t* __restrict__ ubase, int uoff, const uint8_t* xr0,
                                          int xstride, float (&acc)[NC]) {
    // The super-block starts at an even byte offset; read whole dwords and
    // shift by 0 or 16 bits.
    const uint32_t* u = ubase + (uoff >> 2);
    const uint32_t sh = (uint32_t)(uoff & 2) * 8;
    auto W = [&](int i) { return __builtin_amdgcn_alignbit(u[i + 1], u[i], sh); };
    const float dw = h2f(W(52));
    int isum[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) isum[n] = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int h = j >> 3, c = (j >> 1) & 3, kk = j & 1;
        const int sc = __builtin_amdgcn_sbfe((int)W(48 + (j >> 2)), 8 * (j & 3), 8);
        uint32_t q[4];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            const int k = 4 * kk + k4;
            const uint32_t qlw = W(16 * h + 8 * (c & 1) + k);
            const uint32_t lo = (c < 2) ? (qlw & 0x0F0F0F0Fu) : ((qlw >> 4) & 0x0F0F0F0Fu);
            const uint32_t hi = (W(32 + 8 * h + k) >> (2 * c)) & 0x03030303u;
            q[k4] = lo | (hi << 4);
        }
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            const uint32_t* xr = reinterpret_cast<const uint32_t*>(xr0 + n * xstride);
            int t = 0;
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) t = dot4(q[k4], xr[4 * j + k4], t);
            t -= reinterpret_cast<const int*>(xr)[65 + j];  // 32 * (16-wide sum of x codes)
            isum[n] += sc * t;
        }
    }
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const float dx = reinterpret_cast<const float*>(xr0 + n * xstride)[64];
        acc[n] += (dw * dx) * (float)isum[n];
    }
}

// ------------------------------------------------------------- kernel

template <int WT, int NC, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemv_kernel(GemvArgs a) {
    using F = GFmt<WT>;
    constexpr int UB = F::UB, NJ = F::NJ, SLOT = NJ * 1024;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t* xl = smem + WAVES * SLOT;

    stage_x<WT, NC>(a, xl);
    __syncthreads();

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * WAVES + wave, TW = (int64_t)gridDim.x * WAVES;
    if (gw >= a.nwork) return;  // no barrier follows
    uint8_t* slot = smem + wave * SLOT;
    const int64_t nch = ((a.nwork - 1 - gw) / TW + 1) * a.nkc;
    const int P = 1 << a.logP;

    // byte range [s, e) of chunk c of this wavefront
    auto chunk_range = [&](int64_t c, int64_t& s, int64_t& e, int64_t& wi, int& kc) {
        wi = gw + (c / a.nkc) * TW;
        kc = (int)(c % a.nkc);
        if (a.nkc == 1) {
            s = wi * a.RW * a.rowB;
            const int64_t rend = (wi + 1) * a.RW < a.M ? (wi + 1) * a.RW : a.M;
            e = rend * a.rowB;
        } else {
            s = wi * a.rowB + (int64_t)kc * 64 * UB;
            const int64_t lim = (wi + 1) * a.rowB;
            e = s + 64 * UB < lim ? s + 64 * UB : lim;
        }
    };

    uint4 pre[NJ];
    auto load_chunk = [&](int64_t s, int64_t e) {
        const int64_t s0 = s & ~(int64_t)15;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int64_t off = s0 + 16 * (int64_t)(lane + 64 * j);
            uint4 v = make_uint4(0, 0, 0, 0);
            if (off < e) {
                if (off + 16 <= a.total) {
                    v = *reinterpret_cast<const uint4*>(a.W + off);
                } else {  // the last piece of W ends inside this 16-byte load
                    uint32_t t[4] = {0, 0, 0, 0};
                    for (int b = 0; b < 8 && off + 2 * b < a.total; ++b)
                        t[b >> 1] |= (uint32_t)reinterpret_cast<const uint16_t*>(a.W + off)[b] << (16 * (b & 1));
                    v = make_uint4(t[0], t[1], t[2], t[3]);
                }
            }
            pre[j] = v;
        }
    };

    int64_t s, e, wi;
    int kc;
    chunk_range(0, s, e, wi, kc);
    load_chunk(s, e);

    float acc[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) acc[n] = 0.f;

    for (int64_t c = 0; c < nch; ++c) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) reinterpret_cast<uint4*>(slot)[lane + 64 * j] = pre[j];
        const int delta = (int)(s & 15);
        const int64_t cw = wi;
        const int ckc = kc;
        if (c + 1 < nch) {
            chunk_range(c + 1, s, e, wi, kc);
            load_chunk(s, e);
        }
        // this lane's unit inside the chunk
        int r, g, uoff;
        bool valid;
        if (a.nkc == 1) {
            r = lane >> a.logP;
            g = lane & (P - 1);
            valid = g < a.G && cw * a.RW + r < a.M && r < a.RW;
            uoff = delta + (r * a.G + g) * UB;
        } else {
            r = 0;
            g = ckc * 64 + lane;
            valid = g < a.G;
            uoff = delta + lane * UB;
        }
        if (valid) {
            const uint8_t* xr0 = xl + g * XREC;
            const int xstride = a.G * XREC;
            const uint32_t* u = reinterpret_cast<const uint32_t*>(slot + uoff);
            if constexpr (WT == QMM_Q4_0) unit_q4_0<NC>(u, xr0, xstride, acc);
            else if constexpr (WT == QMM_Q8_0) unit_q8_0<NC>(u, xr0, xstride, acc);
            else if constexpr (WT == QMM_Q4_K) unit_q4_k<NC>(u, xr0, xstride, acc);
            else unit_q6_k<NC>(reinterpret_cast<const uint32_t*>(slot), uoff, xr0, xstride, acc);
        }
        if (ckc == a.nkc - 1) {
            // butterfly over the P lanes of each row, then one lane stores
#pragma unroll
            for (int n = 0; n < NC; ++n) {
                float v = acc[n];
                for (int o = P >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o);
                acc[n] = v;
            }
            const int64_t row = cw * a.RW + r;
            if ((lane & (P - 1)) == 0 && r < a.RW && row < a.M) {
#pragma unroll
                for (int n = 0; n < NC; ++n) a.y[n * a.ldy + row] = acc[n];
            }
#pragma unroll
            for (int n = 0; n < NC; ++n) acc[n] = 0.f;
        }
    }
}

// ------------------------------------------- rows not a multiple of 256

// Q4_0 / Q8_0 rows whose K is a multiple of 32 but not of 256: one wavefront
// per row, lanes over the 32-value blocks, plain 2-byte loads.  Correct for
// any such shape; the streaming kernel above handles the K % 256 == 0 case.
template <int WT>
__global__ __launch_bounds__(256) void gemv_rowwave_kernel(const uint8_t* __restrict__ W,
                                                           const uint8_t* __restrict__ xq, float* __restrict__ y,
                                                           int64_t M, int N, int64_t K) {
    constexpr int WB = (WT == QMM_Q4_0) ? kQ4_0Bytes : kQ8_0Bytes;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= M) return;
    const int64_t nb = K / 32;
    for (int n = 0; n < N; ++n) {
        float acc = 0.f;
        for (int64_t b = lane; b < nb; b += 64) {
            const uint8_t* wb = W + (row * nb + b) * WB;
            const uint8_t* xb = xq + ((int64_t)n * nb + b) * kQ8_0Bytes;
            const float dw = h2f(reinterpret_cast<const uint16_t*>(wb)[0]);
            const float dx = h2f(reinterpret_cast<const uint16_t*>(xb)[0]);
            int dot = 0;
            if constexpr (WT == QMM_Q4_0) {
                int sx = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t q = ld_u16x2_g(wb + 2 + 4 * k);
                    const uint32_t x0 = ld_u16x2_g(xb + 2 + 4 * k), x1 = ld_u16x2_g(xb + 18 + 4 * k);
                    dot = dot4(q & 0x0F0F0F0Fu, x0, dot);
                    dot = dot4((q >> 4) & 0x0F0F0F0Fu, x1, dot);
                    sx = dot4(x0, 0x01010101u, sx);
                    sx = dot4(x1, 0x01010101u, sx);
                }
                dot -= 8 * sx;
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) dot = dot4(ld_u16x2_g(wb + 2 + 4 * k), ld_u16x2_g(xb + 2 + 4 * k), dot);
            }
            acc += (float)dot * (dw * dx);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
        if (lane == 0) y[(int64_t)n * M + row] = acc;
    }
}

// ------------------------------------------------------------- host side

struct DevInfo {
    int cus = 0;
    size_t lds = 0;
};

DevInfo& dev_info() {
    static thread_local DevInfo cache[16];
    int dev = 0;
    (void)hipGetDevice(&dev);
    DevInfo& d = cache[dev & 15];
    if (d.cus == 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) == hipSuccess) {
            d.cus = p.multiProcessorCount;
            d.lds = p.sharedMemPerBlock;
        }
        if (d.cus <= 0) d.cus = 256;
        if (d.lds < 65536) d.lds = 65536;
    }
    return d;
}

template <int WT, int NC, int WAVES>
hipError_t launch_one(const GemvArgs& a, size_t lds, int grid, hipStream_t s) {
    static bool attr_set = false;  // raising the LDS limit is idempotent
    if (!attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_kernel<WT, NC, WAVES>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        attr_set = true;
    }
    hipLaunchKernelGGL((gemv_kernel<WT, NC, WAVES>), dim3(grid), dim3(WAVES * 64), lds, s, a);
    return hipGetLastError();
}

template <int WT, int WAVES>
hipError_t dispatch_nc(int nc, const GemvArgs& a, size_t lds, int grid, hipStream_t s) {
    switch (nc) {
    case 1: return launch_one<WT, 1, WAVES>(a, lds, grid, s);
    case 2: return launch_one<WT, 2, WAVES>(a, lds, grid, s);
    case 3: return launch_one<WT, 3, WAVES>(a, lds, grid, s);
    case 4: return launch_one<WT, 4, WAVES>(a, lds, grid, s);
    case 5: return launch_one<WT, 5, WAVES>(a, lds, grid, s);
    case 6: return launch_one<WT, 6, WAVES>(a, lds, grid, s);
    case 7: return launch_one<WT, 7, WAVES>(a, lds, grid, s);
    case 8: return launch_one<WT, 8, WAVES>(a, lds, grid, s);
    default: return hipErrorInvalidValue;
    }
}

template <int WT>
hipError_t gemv_typed(const void* W, const void* xq, float* y, int64_t M, int64_t N, int64_t K, hipStream_t s) {
    using F = GFmt<WT>;
    const DevInfo& di = dev_info();
    const size_t lds_cap = di.lds < 160 * 1024 ? di.lds : 160 * 1024;
    const int G = (int)(K / 256);
    const int64_t xrowB = (int64_t)G * (WT == QMM_Q4_0 || WT == QMM_Q8_0 ? 8 * kQ8_0Bytes : kQ8_KBytes);
    GemvArgs a;
    a.W = static_cast<const uint8_t*>(W);
    a.M = M;
    a.rowB = (int64_t)G * F::UB;
    a.total = M * a.rowB;
    a.ldy = M;
    a.G = G;
    const int Pl = G >= 64 ? 64 : G;
    int logP = 0;
    while ((1 << logP) < Pl) ++logP;
    a.logP = logP;
    a.RW = G >= 64 ? 1 : 64 >> logP;
    a.nkc = (G + 63) / 64;
    a.nwork = (M + a.RW - 1) / a.RW;
    const size_t slot = (size_t)F::NJ * 1024;
    for (int64_t n0 = 0; n0 < N;) {
        // columns per launch: as many (<= 8) as leave room for >= 2 wavefronts' slots
        int nc = (int)(N - n0 < 8 ? N - n0 : 8);
        while (nc > 1 && (size_t)nc * G * XREC + 2 * slot > lds_cap) --nc;
        const size_t xbytes = (size_t)nc * G * XREC;
        if (xbytes + 2 * slot > lds_cap) return hipErrorInvalidValue;
        int waves = 8;
        while (waves > 2 && xbytes + waves * slot > lds_cap) waves >>= 1;
        const size_t lds = xbytes + waves * slot;
        const int per_cu = (int)(lds_cap / lds) > 0 ? (int)(lds_cap / lds) : 1;
        const int64_t need = (a.nwork + waves - 1) / waves;
        const int64_t cap = (int64_t)di.cus * (per_cu < 2 ? per_cu : 2);
        const int grid = (int)(need < cap ? need : cap);
        a.xq = static_cast<const uint8_t*>(xq) + n0 * xrowB;
        a.y = y + n0 * M;
        hipError_t err;
        if (waves == 8) err = dispatch_nc<WT, 8>(nc, a, lds, grid, s);
        else if (waves == 4) err = dispatch_nc<WT, 4>(nc, a, lds, grid, s);
        else err = dispatch_nc<WT, 2>(nc, a, lds, grid, s);
        if (err != hipSuccess) return err;
        n0 += nc;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_gemv(int wtype, const void* W, const void* xq, float* y, int64_t M, int64_t N, int64_t K,
                       hipStream_t s) {
    if (K % 256 != 0) {
        const dim3 g((unsigned)((M + 3) / 4)), b(256);
        const uint8_t* w = static_cast<const uint8_t*>(W);
        const uint8_t* x = static_cast<const uint8_t*>(xq);
        if (wtype == QMM_Q4_0) hipLaunchKernelGGL(gemv_rowwave_kernel<QMM_Q4_0>, g, b, 0, s, w, x, y, M, (int)N, K);
        else if (wtype == QMM_Q8_0) hipLaunchKernelGGL(gemv_rowwave_kernel<QMM_Q8_0>, g, b, 0, s, w, x, y, M, (int)N, K);
        else return hipErrorInvalidValue;
        return hipGetLastError();
    }
    switch (wtype) {
    case QMM_Q4_0: return gemv_typed<QMM_Q4_0>(W, xq, y, M, N, K, s);
    case QMM_Q8_0: return gemv_typed<QMM_Q8_0>(W, xq, y, M, N, K, s);
    case QMM_Q4_K: return gemv_typed<QMM_Q4_K>(W, xq, y, M, N, K, s);
    case QMM_Q6_K: return gemv_typed<QMM_Q6_K>(W, xq, y, M, N, K, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
