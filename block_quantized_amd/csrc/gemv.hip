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
// Decode speed is bound by streaming W from memory (page "llama.cpp and
// GGUF", "The ggml Tensor Library and Backends": decode speed tracks memory
// bandwidth), so the kernel is organised around moving W at full HBM rate:
//
//  * A lane's unit of work is 256 consecutive weights of one row, loaded by
//    that lane alone with 16-byte loads straight into registers: 8 blocks
//    (144 B) for Q4_0, 8 blocks (272 B) for Q8_0, one 144 B super-block for
//    Q4_K, one 210 B super-block for Q6_K.  Consecutive lanes take
//    consecutive units, so a wavefront reads one contiguous run of memory.
//    Q6_K super-blocks are only 2-byte aligned: a lane reads 224 bytes from
//    the 4-byte boundary at or below its super-block (14 loads of 16 bytes;
//    the work item holding a matrix's last unit reads each unit's own last
//    16 bytes instead of the 14th piece, so nothing past the matrix is
//    read), and shifts by the 0 or 2 byte skew.
//    (Measured on MI355X: per-lane 144 B units stream as fast as fully
//    coalesced reads, ~6.3 TB/s, and so do the 210 B Q6_K units read this
//    way; 8-super-block Q6_K units per lane, read in 224 B windows 1680 B
//    apart, streamed at 2.4 TB/s in the same probe.  Staging through LDS
//    halved the rate.)
//  * Loads run one step ahead (two register buffers), and the first step's
//    loads are issued before the activations are staged.
//  * A row of K weights is G = K/256 units; P = next power of two >= min(G, 64)
//    lanes share a row, a wavefront covers RW = 64/P rows per chunk, or a
//    row in ceil(G/64) chunks when G > 64.  Lanes of a row are reduced with
//    a fixed butterfly, so results are bit-identical run to run.
//  * Several matrices sharing K and x (e.g. q|k|v, gate|up) can form one
//    launch: their chunks are concatenated ("segments").
//  * The activations (N rows of Q8_0 or Q8_K blocks) are repacked once per
//    workgroup into LDS records of 336 bytes per (row, 256-value group): 256
//    int8 codes, then the fp32 scales and precomputed integer sums.
#include "qmm_internal.h"

#include <atomic>

namespace qmm {
namespace {

// 16 bytes at a 4- or 2-byte-aligned address (Q6_K super-blocks are 2-byte aligned)
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));

template <int WT> struct U;
template <> struct U<QMM_Q4_0> { static constexpr int UB = 144, NV = 9; };
template <> struct U<QMM_Q8_0> { static constexpr int UB = 272, NV = 17; };
template <> struct U<QMM_Q5_0> { static constexpr int UB = 176, NV = 11; };
template <> struct U<QMM_Q4_K> { static constexpr int UB = 144, NV = 9; };
template <> struct U<QMM_Q6_K> { static constexpr int UB = kQ6_KBytes, NV = 14; };

template <int B> struct Buf { static constexpr int b = B; };  // register buffer B (compile-time)

constexpr int XREC = 336;  // LDS bytes per (activation row, 256-value group)
constexpr int kMaxSeg = 4;

struct Seg {
    const uint8_t* W;
    float* y;
    int64_t M;
    int64_t work0;  // first work item of this segment in the launch
};
// y of a segment is N x M (row stride M)

struct GemvArgs {
    Seg seg[kMaxSeg];
    int nseg;
    const uint8_t* xq;
    int64_t rowB;      // bytes per W row
    int64_t nwork;     // work items over all segments
    int G;             // 256-value groups per row (K / 256): activation records and lane units
    int logP;          // log2(lanes per row)
    int RW;            // rows per chunk
    int nkc;           // chunks per work item
};

__device__ __forceinline__ uint32_t ld_u16x2_g(const uint8_t* p) {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
    return (uint32_t)q[0] | ((uint32_t)q[1] << 16);
}

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// ---------------------------------------------------- activation staging
// Each thread owns whole staging items: one 34 B Q8_0 block, or a quarter of
// a 292 B Q8_K block.  All of a round's global loads are issued before any
// LDS store, so a round costs one memory round trip; `after_loads` runs once,
// right after the first round's loads (the W prefetch goes there, so waiting
// for x - loads retire in order - does not wait for W).  The activation rows
// are contiguous, so item i's bytes follow item i-1's.

template <bool First, int Lanes>
struct RoundTag {
    static constexpr bool first = First;
    static constexpr int lanes = Lanes;
};

template <int WT, int NC, bool XF, class Hook>
__device__ __forceinline__ void stage_x(const uint8_t* xq, int G, uint8_t* xl, Hook&& after_loads) {
    constexpr bool kQ80 = (WT == QMM_Q4_0 || WT == QMM_Q5_0 || WT == QMM_Q8_0);
    // One item per thread per round.  With four (the pre-quantized x once
    // took 76 registers per thread for it) the compiler reused load
    // destinations and waited for x loads inside the issue sequence: batch 1,
    // Q4_K 14336x4096 9.8 -> 9.2 us, 4096x14336 10.0 -> 9.2 us, Q8_0 2048x2048
    // 3.72 -> 3.64 us (measured on MI355X).  More rounds, when needed, run
    // before the W prefetch (below).
    constexpr int KB = 1;
    const int nitems = kQ80 ? NC * G * 8 : NC * G * 4;
    const int step = KB * blockDim.x;
    // A wave issues its loads when any of its lanes has an item (a lane past
    // the last item re-reads the last item and stores nothing); a wave with no
    // item skips them as a whole.  No lane-level branch guards a load, so the
    // waits retire exactly the loads they need - in particular, waiting for x
    // does not wait for the W prefetch issued after it.
    const int wave0 = __builtin_amdgcn_readfirstlane((int)threadIdx.x) & ~63;  // first thread of this wave
    auto round = [&](const int base, auto first) {
        constexpr bool kFirst = decltype(first)::first;
        if constexpr (XF && kQ80) {
            // fp32 rows quantized here to Q8_0 by S adjacent lanes per
            // 32-value block (each lane 32/S values; the block maximum and
            // the code sum are combined through shuffles), exactly as the
            // stand-alone quantizer does.  S is chosen by stage_x below.
            constexpr int S = decltype(first)::lanes;
            constexpr int NF = 8 / S;  // float4 per lane
            const int slot = (int)threadIdx.x / S, si = (int)threadIdx.x % S;
            const int i = base + slot;
            const int ic = i < nitems ? i : nitems - 1;
            float4 v[NF];
            if (base + wave0 / S < nitems) {
#pragma unroll
                for (int h = 0; h < NF; ++h) v[h] = reinterpret_cast<const float4*>(xq)[8 * ic + NF * si + h];
            }
            if constexpr (kFirst) {
                // Every wave of the workgroup issues its x loads before any
                // wave issues W loads: the memory pipeline serves a compute
                // unit's requests in order, and x (needed first, by every
                // wave) would otherwise queue behind other waves' W traffic.
                // The barrier waits for no data.
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                after_loads();
                // The W loads are issued here: left to itself the scheduler
                // sank some of them into the quantization below, into the
                // registers x had just freed, so that they waited for x (the
                // fused decode sweep: 0.331 -> 0.322 ms per step, measured on
                // MI355X).
                __builtin_amdgcn_sched_barrier(0);
            }
            float amax = 0.0f;
#pragma unroll
            for (int h = 0; h < NF; ++h)
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[h].x), fabsf(v[h].y)), fmaxf(fabsf(v[h].z), fabsf(v[h].w))));
#pragma unroll
            for (int o = 1; o < S; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
            float d, id;
            rtn_scale(amax, d, id);
            uint32_t q[NF];
            int sx = 0;
#pragma unroll
            for (int h = 0; h < NF; ++h) {
                q[h] = (uint32_t)(rtn_code(v[h].x * id) & 0xFF) | ((uint32_t)(rtn_code(v[h].y * id) & 0xFF) << 8) |
                       ((uint32_t)(rtn_code(v[h].z * id) & 0xFF) << 16) |
                       ((uint32_t)(rtn_code(v[h].w * id) & 0xFF) << 24);
                sx = dot4(q[h], 0x01010101u, sx);
            }
#pragma unroll
            for (int o = 1; o < S; o <<= 1) sx += __shfl_xor(sx, o);
            if (i < nitems) {
                uint8_t* rec = xl + (i >> 3) * XREC;
                const int bi = i & 7;
                uint32_t* dst = reinterpret_cast<uint32_t*>(rec + 32 * bi) + NF * si;
#pragma unroll
                for (int h = 0; h < NF; ++h) dst[h] = q[h];
                if (si == 0) {
                    reinterpret_cast<float*>(rec)[64 + bi] = h2f(f2h(d));  // the block stores fp16(d)
                    reinterpret_cast<int*>(rec)[72 + bi] = 8 * sx;
                }
            }
        } else if constexpr (XF) {
            // fp32 rows quantized here to Q8_K: item i = quarter i&3 of block
            // i>>2 (values 64i .. 64i+63); the four quarters of a block are
            // adjacent lanes and share the block maximum through shuffles.
            const int i = base + threadIdx.x;
            const int ic = i < nitems ? i : nitems - 1;
            float4 v[16];
            float amax = 0.0f;
            if (base + wave0 < nitems) {
#pragma unroll
                for (int h = 0; h < 16; ++h) v[h] = reinterpret_cast<const float4*>(xq)[16 * ic + h];
            }
            if constexpr (kFirst) {
                // Every wave of the workgroup issues its x loads before any
                // wave issues W loads: the memory pipeline serves a compute
                // unit's requests in order, and x (needed first, by every
                // wave) would otherwise queue behind other waves' W traffic.
                // The barrier waits for no data.
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                after_loads();
                __builtin_amdgcn_sched_barrier(0);  // W loads issued here, not sunk into the work below
            }
            if (i < nitems) {
#pragma unroll
                for (int h = 0; h < 16; ++h)
                    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[h].x), fabsf(v[h].y)), fmaxf(fabsf(v[h].z), fabsf(v[h].w))));
            }
            amax = fmaxf(amax, __shfl_xor(amax, 1));
            amax = fmaxf(amax, __shfl_xor(amax, 2));
            if (i < nitems) {
                float d, id;
                rtn_scale(amax, d, id);
                uint8_t* rec = xl + (i >> 2) * XREC;
                const int qq = i & 3;
                int bs[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    uint32_t q[4];
                    int sum = 0;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float4 f = v[4 * t + u];
                        q[u] = (uint32_t)(rtn_code(f.x * id) & 0xFF) | ((uint32_t)(rtn_code(f.y * id) & 0xFF) << 8) |
                               ((uint32_t)(rtn_code(f.z * id) & 0xFF) << 16) |
                               ((uint32_t)(rtn_code(f.w * id) & 0xFF) << 24);
                        sum = dot4(q[u], 0x01010101u, sum);
                    }
                    bs[t] = sum;  // exact sum of codes 64qq+16t .. +15
                    reinterpret_cast<uint4*>(rec + 64 * qq)[t] = make_uint4(q[0], q[1], q[2], q[3]);
                }
                int* meta = reinterpret_cast<int*>(rec) + 65;
                if constexpr (WT == QMM_Q4_K) {
                    meta[2 * qq] = bs[0] + bs[1];
                    meta[2 * qq + 1] = bs[2] + bs[3];
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t) meta[4 * qq + t] = 32 * bs[t];
                }
                if (qq == 0) reinterpret_cast<float*>(rec)[64] = d;
            }
        } else if constexpr (kQ80) {
            uint32_t v[KB][17];
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const int i = base + k * blockDim.x + threadIdx.x;
                const int ic = i < nitems ? i : nitems - 1;
                const uint16_t* p = reinterpret_cast<const uint16_t*>(xq + (int64_t)ic * kQ8_0Bytes);
                if (base + k * (int)blockDim.x + wave0 < nitems) {
#pragma unroll
                    for (int h = 0; h < 17; ++h) v[k][h] = p[h];
                }
            }
            if constexpr (kFirst) {
                // Every wave of the workgroup issues its x loads before any
                // wave issues W loads: the memory pipeline serves a compute
                // unit's requests in order, and x (needed first, by every
                // wave) would otherwise queue behind other waves' W traffic.
                // The barrier waits for no data.
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                after_loads();
                __builtin_amdgcn_sched_barrier(0);  // W loads issued here, not sunk into the work below
            }
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const int i = base + k * blockDim.x + threadIdx.x;
                if (i < nitems) {
                    uint8_t* rec = xl + (i >> 3) * XREC;
                    const int bi = i & 7;
                    uint32_t q[8];
                    int sx = 0;
#pragma unroll
                    for (int d = 0; d < 8; ++d) {
                        q[d] = v[k][1 + 2 * d] | (v[k][2 + 2 * d] << 16);
                        sx = dot4(q[d], 0x01010101u, sx);
                    }
                    reinterpret_cast<uint4*>(rec + 32 * bi)[0] = make_uint4(q[0], q[1], q[2], q[3]);
                    reinterpret_cast<uint4*>(rec + 32 * bi)[1] = make_uint4(q[4], q[5], q[6], q[7]);
                    reinterpret_cast<float*>(rec)[64 + bi] = h2f(v[k][0]);
                    reinterpret_cast<int*>(rec)[72 + bi] = 8 * sx;  // Q4_0's offset term: 8 * sum q_x
                }
            }
        } else {
            uint32_t v[KB][19];
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const int i = base + k * blockDim.x + threadIdx.x;
                const int ic = i < nitems ? i : nitems - 1;
                const uint32_t* p = reinterpret_cast<const uint32_t*>(xq + (int64_t)(ic >> 2) * kQ8_KBytes);
                const int qq = ic & 3;
                if (base + k * (int)blockDim.x + wave0 < nitems) {
#pragma unroll
                    for (int d = 0; d < 16; ++d) v[k][d] = p[1 + 16 * qq + d];
                    v[k][16] = p[65 + 2 * qq];  // bsums 4qq .. 4qq+3
                    v[k][17] = p[66 + 2 * qq];
                    v[k][18] = p[0];            // fp32 d
                }
            }
            if constexpr (kFirst) {
                // Every wave of the workgroup issues its x loads before any
                // wave issues W loads: the memory pipeline serves a compute
                // unit's requests in order, and x (needed first, by every
                // wave) would otherwise queue behind other waves' W traffic.
                // The barrier waits for no data.
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                after_loads();
                __builtin_amdgcn_sched_barrier(0);  // W loads issued here, not sunk into the work below
            }
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const int i = base + k * blockDim.x + threadIdx.x;
                if (i < nitems) {
                    uint8_t* rec = xl + (i >> 2) * XREC;
                    const int qq = i & 3;
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        reinterpret_cast<uint4*>(rec + 64 * qq)[d] =
                            make_uint4(v[k][4 * d], v[k][4 * d + 1], v[k][4 * d + 2], v[k][4 * d + 3]);
                    const int b0 = (int16_t)(v[k][16] & 0xFFFF), b1 = (int16_t)(v[k][16] >> 16);
                    const int b2 = (int16_t)(v[k][17] & 0xFFFF), b3 = (int16_t)(v[k][17] >> 16);
                    int* meta = reinterpret_cast<int*>(rec) + 65;
                    if constexpr (WT == QMM_Q4_K) {  // sums over the 32-wide sub-blocks 2qq, 2qq+1
                        meta[2 * qq] = b0 + b1;
                        meta[2 * qq + 1] = b2 + b3;
                    } else {                         // 32 * (16-wide sums) 4qq .. 4qq+3
                        meta[4 * qq] = 32 * b0;
                        meta[4 * qq + 1] = 32 * b1;
                        meta[4 * qq + 2] = 32 * b2;
                        meta[4 * qq + 3] = 32 * b3;
                    }
                    if (qq == 0) reinterpret_cast<uint32_t*>(rec)[64] = v[k][18];
                }
            }
        }
    };
    // When pre-quantized x takes more than one round, the earlier rounds run
    // first and the W prefetch goes with the last one, so that no round's
    // loads retire after W's (waiting for them would wait for W).  The fused
    // path keeps the first-round-first order (it takes a second round only
    // beyond K = 8192 at 256 threads; with this order and the LDS-only
    // barrier below, its decode sweep measured 1.7% slower).
    if constexpr (XF && kQ80) {
        // lanes per block: as many as the workgroup has to spare, up to 8
        const int spare = (int)blockDim.x / nitems;
        if (spare >= 8) round(0, RoundTag<true, 8>{});
        else if (spare >= 4) round(0, RoundTag<true, 4>{});
        else if (spare >= 2) round(0, RoundTag<true, 2>{});
        else round(0, RoundTag<true, 1>{});
        for (int base = step; base < nitems; base += step) round(base, RoundTag<false, 1>{});
    } else {
        const int last = nitems > step ? (nitems - 1) / step * step : 0;
        for (int base = 0; base < last; base += step) round(base, RoundTag<false, 1>{});
        round(last, RoundTag<true, 1>{});
    }
}

// ------------------------------------------------------- unit compute
// w: the unit's bytes as dwords (registers); xr0: LDS record of activation
// row 0 for this unit's first 256-value group; xstride: LDS bytes between
// activation rows.

template <int NC>
__device__ __forceinline__ void unit_q4_0(const uint32_t* w, const uint8_t* xr0, int xstride, float (&acc)[NC]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t db, q[4];
        if ((i & 1) == 0) {  // block at byte 18i = 4b: d in the low half of w[b]
            const int b = 9 * i / 2;
            db = w[b];
#pragma unroll
            for (int k = 0; k < 4; ++k) q[k] = __builtin_amdgcn_alignbyte(w[b + k + 1], w[b + k], 2);
        } else {             // block at byte 4b + 2: d in the high half of w[b]
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

// Fifth bits b3..b0 (of four consecutive elements) to bit 4 of four bytes:
// v * 0x00204081 places bit k at bit 8k (the four shifted copies do not
// overlap, so there are no carries).
__device__ __forceinline__ uint32_t fifth_bits(uint32_t v4) {
    return ((v4 * 0x00204081u) & 0x01010101u) << 4;
}

// Q5_0: eight 22-byte blocks per 176-byte unit; block i starts at byte 22i,
// i.e. dword 11i/2 for even i and two bytes into dword (22i-2)/4 for odd i.
template <int NC>
__device__ __forceinline__ void unit_q5_0(const uint32_t* w, const uint8_t* xr0, int xstride, float (&acc)[NC]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t db, qh, q[4];
        if ((i & 1) == 0) {
            const int b = 11 * i / 2;
            db = w[b];
            qh = __builtin_amdgcn_alignbyte(w[b + 1], w[b], 2);
#pragma unroll
            for (int k = 0; k < 4; ++k) q[k] = __builtin_amdgcn_alignbyte(w[b + 2 + k], w[b + 1 + k], 2);
        } else {
            const int b = (22 * i - 2) / 4;
            db = w[b] >> 16;
            qh = w[b + 1];
#pragma unroll
            for (int k = 0; k < 4; ++k) q[k] = w[b + 2 + k];
        }
        const float dw = h2f(db);
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            lo[k] = (q[k] & 0x0F0F0F0Fu) | fifth_bits((qh >> (4 * k)) & 15u);
            hi[k] = ((q[k] >> 4) & 0x0F0F0F0Fu) | fifth_bits((qh >> (16 + 4 * k)) & 15u);
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
            // the record holds 8 * sum q_x (Q4_0's offset); Q5_0's is 16 * sum q_x
            const int isum = dot - 2 * reinterpret_cast<const int*>(xr)[72 + i];
            const float dx = reinterpret_cast<const float*>(xr)[64 + i];
            acc[n] += (float)isum * (dw * dx);
        }
    }
}

template <int NC>
__device__ __forceinline__ void unit_q8_0(const uint32_t* w, const uint8_t* xr0, int xstride, float (&acc)[NC]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t db, q[8];
        if ((i & 1) == 0) {  // block at byte 34i = 4b
            const int b = 17 * i / 2;
            db = w[b];
#pragma unroll
            for (int k = 0; k < 8; ++k) q[k] = __builtin_amdgcn_alignbyte(w[b + k + 1], w[b + k], 2);
        } else {             // block at byte 4b + 2
            const int b = (17 * i - 1) / 2;
            db = w[b] >> 16;
#pragma unroll
            for (int k = 0; k < 8; ++k) q[k] = w[b + 1 + k];
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
__device__ __forceinline__ void unit_q4_k(const uint32_t* w, const uint8_t* xr0, int xstride, float (&acc)[NC]) {
    const float d = h2f(w[0]), dmin = h2f(w[0] >> 16);
    // eight 6-bit scales and mins, one per byte
    const uint32_t sc03 = w[1] & 0x3F3F3F3Fu, m03 = w[2] & 0x3F3F3F3Fu;
    const uint32_t sc47 = (w[3] & 0x0F0F0F0Fu) | ((w[1] >> 2) & 0x30303030u);
    const uint32_t m47 = ((w[3] >> 4) & 0x0F0F0F0Fu) | ((w[2] >> 2) & 0x30303030u);
    int sumi[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) sumi[n] = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {  // sub-blocks 2g (low nibbles) and 2g+1 (high nibbles)
        const uint32_t scw = (g < 2) ? sc03 : sc47;
        const int sc_lo = (scw >> (16 * (g & 1))) & 0xFF, sc_hi = (scw >> (16 * (g & 1) + 8)) & 0xFF;
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            const uint32_t* xr = reinterpret_cast<const uint32_t*>(xr0 + n * xstride);
            int dl = 0, dh = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t q = w[4 + 8 * g + k];
                dl = dot4(q & 0x0F0F0F0Fu, xr[16 * g + k], dl);
                dh = dot4((q >> 4) & 0x0F0F0F0Fu, xr[16 * g + 8 + k], dh);
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

// One Q6_K super-block.  r[0..51] are the 208 bytes from the 4-byte boundary
// at or below its first byte, which is byte `skew` (0 or 2) of r; when the
// skew is 2, r[52] is its bytes 206-209 (unused when 0); r[53] holds d (its
// bytes 208-209) in the low half.  Dword i < 52 of the super-block is bytes
// skew + 4i .. of r.
template <int NC>
__device__ __forceinline__ void unit_q6_k(const uint32_t* r, uint32_t skew, const uint8_t* xr0, int xstride,
                                          float (&acc)[NC]) {
    auto W = [&](int i) -> uint32_t { return __builtin_amdgcn_alignbyte(r[i + 1], r[i], skew); };
    const float dw = h2f(r[53]);
    int isum[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) isum[n] = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {  // 16-wide sub-blocks
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

template <int WT, int NC, bool XF>
__global__ __launch_bounds__(512) void gemv_kernel(GemvArgs a) {
    using F = U<WT>;
    constexpr int NV = F::NV;
    extern __shared__ __attribute__((aligned(16))) uint8_t xl[];

    // Every argument is read once, up front, so the kernel-argument loads form
    // one batch (no dependent scalar round trips before the first W load).
    const int nseg = a.nseg, logP = a.logP, RW = a.RW, NKC = a.nkc;
    const int64_t rowB = a.rowB, nwork = a.nwork;
    const uint8_t* xq = a.xq;
    const int G = a.G;
    const uint8_t* sW[kMaxSeg];
    float* sY[kMaxSeg];
    int64_t sM[kMaxSeg], sW0[kMaxSeg];
#pragma unroll
    for (int k = 0; k < kMaxSeg; ++k) {
        sW[k] = a.seg[k].W;
        sY[k] = a.seg[k].y;
        sM[k] = a.seg[k].M;
        sW0[k] = a.seg[k].work0;
    }

    const int lane = threadIdx.x & 63;
    const int wpg = blockDim.x >> 6;
    // wave-uniform bookkeeping lives in scalar registers
    const int gw = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * wpg + (threadIdx.x >> 6)));
    const int TW = gridDim.x * wpg;
    const int P = 1 << logP;
    // lane's place inside a chunk
    const int lr = lane >> logP;
    const int lg = lane & (P - 1);
    const bool lwriter = (lane & (P - 1)) == 0 && lr < RW;

    // Where this lane's unit lies.
    // Loads and stores are never skipped by a branch: a lane without a unit
    // reads a unit that exists (the first of segment 0) and discards it, and
    // outputs go through a buffer store whose offset is out of range for
    // lanes that must not write, which the hardware drops.  So the count of
    // memory operations in flight is the same on every path, and the
    // compiler's waits retire only the loads actually needed next.
    constexpr int kNoStore = 1 << 30;
    struct Loc {
        const uint8_t* p;  // first byte of the unit; if !valid, the work item's first unit
        float* yb;         // output of the chunk's first row (wave-uniform)
        int64_t ldy;       // stride between output columns (the segment's M)
        int nrec;          // bytes of output rows of this chunk that exist (wave-uniform)
        int yoff;          // this lane's byte offset from yb, or kNoStore
        int g;             // first 256-value activation group of the unit
        bool last;         // last chunk of its work item
        bool valid;
        bool tail;         // the work item holds the last unit of its matrix (wave-uniform)
    };
    auto locate = [&](int64_t wi, int kc) {  // work item wi (uniform), chunk kc of it
        Loc L;
        const uint8_t* W = sW[0];
        float* Y = sY[0];
        int64_t M = sM[0], w0 = sW0[0];
#pragma unroll
        for (int k = 1; k < kMaxSeg; ++k) {
            const bool in = k < nseg && wi >= sW0[k];
            W = in ? sW[k] : W;
            Y = in ? sY[k] : Y;
            M = in ? sM[k] : M;
            w0 = in ? sW0[k] : w0;
        }
        const int64_t row0 = (wi - w0) * RW;  // uniform
        const int gu = kc * P + lg;  // kc is 0 when a row fits one chunk
        const int64_t row = row0 + lr;
        const bool valid = gu < G && lr < RW && row < M;
        L.valid = valid;
        L.p = W + (valid ? row * rowB + (int64_t)gu * F::UB : row0 * rowB + (int64_t)kc * P * F::UB);
        L.yb = Y + row0;
        L.ldy = M;
        const int64_t left = M - row0;  // >= 1
        L.nrec = 4 * (int)(left < RW ? left : RW);
        L.yoff = lwriter ? 4 * lr : kNoStore;
        L.g = gu;
        L.last = kc == NKC - 1;
        L.tail = row0 + RW >= M && kc == NKC - 1;
        return L;
    };
    // A unit's bytes: NV 16-byte pieces.  Q6_K: the 14 pieces from the 4-byte
    // boundary at or below the unit, which end up to 14 bytes past it, in the
    // next unit.  The work item that holds the last unit of a matrix (a
    // wave-uniform choice, so no load sits behind a lane-level branch) takes
    // the unit's own last 16 bytes as the 14th piece instead, so no byte past
    // the matrix is read.  Either way dword 52 becomes the unit's bytes
    // 206-209 when the skew is 2, and dword 53 holds d (bytes 208-209) in its
    // low half.
    auto load = [&](const Loc& L, uint4 (&v)[NV]) {
        if constexpr (WT == QMM_Q6_K) {
            // (pointer arithmetic, not an integer round trip: the compiler
            // then still knows the address is global memory and emits
            // global loads, not flat ones, which would also count against
            // the LDS wait counter)
            const u32x4_a4* q = reinterpret_cast<const u32x4_a4*>(L.p - (reinterpret_cast<uintptr_t>(L.p) & 3u));
#pragma unroll
            for (int i = 0; i < NV - 1; ++i) {
                const u32x4_a4 t = q[i];
                v[i] = make_uint4(t.x, t.y, t.z, t.w);
            }
            // (This form makes the compiler wait for the prefetch before the
            // unit is computed, so a wave does not overlap its own loads with
            // its compute.  Measured on the 128256x4096 head, it is 5-8%
            // faster than the forms whose waits let the loads run under the
            // compute: 83-85 us against 87-92 us.)
            if (L.tail) {
                const u32x4_a2 t = *reinterpret_cast<const u32x4_a2*>(L.p + (kQ6_KBytes - 16));
                v[NV - 1] = make_uint4(t.w, t.w >> 16, 0u, 0u);
            } else {
                const u32x4_a4 t = q[NV - 1];
                const uint32_t sk = (uint32_t)reinterpret_cast<uintptr_t>(L.p) & 3u;
                v[NV - 1] = make_uint4(t.x, t.x >> (8 * sk), 0u, 0u);
            }
        } else {
            const uint4* q = reinterpret_cast<const uint4*>(L.p);
#pragma unroll
            for (int i = 0; i < NV; ++i) v[i] = q[i];
        }
    };

    uint4 buf[2][NV];
    Loc cur, nxt;
    int64_t nwi = gw;  // position of `nxt`: work item and chunk
    int pkc = 0;
    nxt = locate(gw < nwork ? gw : nwork - 1, 0);
    stage_x<WT, NC, XF>(xq, G, xl, [&]() { load(nxt, buf[0]); });
    // The activation records are complete in LDS for every wave.  The first
    // W unit's loads stay in flight across this barrier.  For pre-quantized x
    // the fences cover LDS only, so the barrier waits for the LDS stores and
    // nothing else whatever the compiler makes of the staging rounds (when a
    // later round followed the W loads, it waited for all of them here:
    // batch 1, Q4_K 14336x4096 10.4 -> 9.9 us, 4096x4096 5.1 -> 4.7 us,
    // measured on MI355X).  The fused path keeps __syncthreads.
    if constexpr (XF) {
        __syncthreads();
    } else {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    }
    if (gw >= nwork) return;  // no barrier follows

    float acc[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) acc[n] = 0.f;
    const int xstride = G * XREC;

    // One step: prefetch the next unit into the other buffer (unless this is
    // the wave's last), then compute `cur` from buffer B.
    auto step = [&](auto tag, auto more) {
        constexpr int B = decltype(tag)::b;
        if constexpr (decltype(more)::value) load(nxt, buf[B ^ 1]);
        if (cur.valid) {
            const uint32_t* w = reinterpret_cast<const uint32_t*>(buf[B]);
            const uint8_t* xr0 = xl + cur.g * XREC;
            if constexpr (WT == QMM_Q4_0) unit_q4_0<NC>(w, xr0, xstride, acc);
            else if constexpr (WT == QMM_Q5_0) unit_q5_0<NC>(w, xr0, xstride, acc);
            else if constexpr (WT == QMM_Q8_0) unit_q8_0<NC>(w, xr0, xstride, acc);
            else if constexpr (WT == QMM_Q4_K) unit_q4_k<NC>(w, xr0, xstride, acc);
            else unit_q6_k<NC>(w, (uint32_t)reinterpret_cast<uintptr_t>(cur.p) & 3u, xr0, xstride, acc);
        }
    };
    // After the last chunk of a work item: butterfly over the P lanes of
    // each row, then one lane stores.
    auto finish = [&]() {
        const int off = cur.last ? cur.yoff : kNoStore;
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            float v = acc[n];
            for (int o = P >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o);
            const __amdgpu_buffer_rsrc_t r =
                __builtin_amdgcn_make_buffer_rsrc(cur.yb + n * cur.ldy, (short)0, cur.nrec, kBufferWord3);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
            acc[n] = cur.last ? 0.f : acc[n];
        }
    };
    auto advance = [&]() {  // make `nxt` current and locate the unit after it
        cur = nxt;
        if (++pkc == NKC) {
            pkc = 0;
            nwi += TW;
        }
        const bool more = nwi < nwork;
        if (more) nxt = locate(nwi, pkc);
        return more;
    };

    // The last unit of a wave is computed by its own copy of the step, which
    // issues no further load (a uniform branch, taken once per wave).
    for (;;) {
        if (!advance()) {
            step(Buf<0>{}, std::false_type{});
            finish();
            break;
        }
        step(Buf<0>{}, std::true_type{});
        finish();
        if (!advance()) {
            step(Buf<1>{}, std::false_type{});
            finish();
            break;
        }
        step(Buf<1>{}, std::true_type{});
        finish();
    }
}

// ------------------------------------------------ shapes the kernel above skips
// Q4_0 / Q5_0 / Q8_0 rows whose K is a multiple of 32 but not of 256: one
// wavefront per row, lanes over the blocks, plain 2-byte loads.  Correct for
// any such shape.
template <int WT>
__global__ __launch_bounds__(256) void gemv_rowwave_kernel(const uint8_t* __restrict__ W,
                                                           const uint8_t* __restrict__ xq, float* __restrict__ y,
                                                           int64_t M, int N, int64_t K) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    static_assert(WT == QMM_Q4_0 || WT == QMM_Q5_0 || WT == QMM_Q8_0, "32-value block types only");
    if (row >= M) return;
    {
        constexpr int WB = (WT == QMM_Q4_0) ? kQ4_0Bytes : (WT == QMM_Q5_0) ? kQ5_0Bytes : kQ8_0Bytes;
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
                } else if constexpr (WT == QMM_Q5_0) {
                    const uint32_t qh = ld_u16x2_g(wb + 2);
                    int sx = 0;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t q = ld_u16x2_g(wb + 6 + 4 * k);
                        const uint32_t x0 = ld_u16x2_g(xb + 2 + 4 * k), x1 = ld_u16x2_g(xb + 18 + 4 * k);
                        dot = dot4((q & 0x0F0F0F0Fu) | fifth_bits((qh >> (4 * k)) & 15u), x0, dot);
                        dot = dot4(((q >> 4) & 0x0F0F0F0Fu) | fifth_bits((qh >> (16 + 4 * k)) & 15u), x1, dot);
                        sx = dot4(x0, 0x01010101u, sx);
                        sx = dot4(x1, 0x01010101u, sx);
                    }
                    dot -= 16 * sx;
                } else {
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        dot = dot4(ld_u16x2_g(wb + 2 + 4 * k), ld_u16x2_g(xb + 2 + 4 * k), dot);
                }
                acc += (float)dot * (dw * dx);
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
            if (lane == 0) y[(int64_t)n * M + row] = acc;
        }
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
        if (d.lds > 160 * 1024) d.lds = 160 * 1024;
    }
    return d;
}

template <int WT, int NC, bool XF>
hipError_t launch_one(const GemvArgs& a, size_t lds, int wpg, hipStream_t s) {
    // Workgroups per CU as registers and waves allow, by waves per workgroup
    // (LDS, which depends on K and the column count, is applied below).
    // Written once per entry; concurrent first calls store the same value.
    static std::atomic<int> occ[9];
    int occw = occ[wpg].load(std::memory_order_relaxed);
    if (!occw) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_kernel<WT, NC, XF>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemv_kernel<WT, NC, XF>, wpg * 64, 0) != hipSuccess ||
            n <= 0)
            n = 1;
        occw = n;
        occ[wpg].store(n, std::memory_order_relaxed);
    }
    const DevInfo& di = dev_info();
    const int by_lds = (int)(di.lds / (lds ? lds : 1));
    const int per_cu = by_lds < occw ? by_lds : occw;
    const int64_t need = (a.nwork + wpg - 1) / wpg;
    const int64_t cap = (int64_t)di.cus * (per_cu > 0 ? per_cu : 1);
    const int grid = (int)(need < cap ? need : cap);
    return launch(gemv_kernel<WT, NC, XF>, dim3(grid), dim3(wpg * 64), lds, s, a);
}

template <int WT, bool XF>
hipError_t dispatch_nc(int nc, const GemvArgs& a, size_t lds, int wpg, hipStream_t s) {
    switch (nc) {
    case 1: return launch_one<WT, 1, XF>(a, lds, wpg, s);
    case 2: return launch_one<WT, 2, XF>(a, lds, wpg, s);
    case 3: return launch_one<WT, 3, XF>(a, lds, wpg, s);
    case 4: return launch_one<WT, 4, XF>(a, lds, wpg, s);
    case 5: return launch_one<WT, 5, XF>(a, lds, wpg, s);
    case 6: return launch_one<WT, 6, XF>(a, lds, wpg, s);
    case 7: return launch_one<WT, 7, XF>(a, lds, wpg, s);
    case 8: return launch_one<WT, 8, XF>(a, lds, wpg, s);
    default: return hipErrorInvalidValue;
    }
}

template <int WT>
hipError_t gemv_typed(int nseg, const void* const* Ws, float* const* ys, const int64_t* Ms, const void* xq,
                      bool xf32, int64_t N, int64_t K, hipStream_t s) {
    using F = U<WT>;
    const DevInfo& di = dev_info();
    GemvArgs a;
    a.nseg = nseg;
    a.G = (int)(K / 256);
    a.rowB = (int64_t)a.G * F::UB;
    const int Pl = a.G >= 64 ? 64 : a.G;
    int logP = 0;
    while ((1 << logP) < Pl) ++logP;
    a.logP = logP;
    a.RW = 64 >> logP;
    a.nkc = (a.G + (1 << logP) - 1) >> logP;
    int64_t work = 0;
    for (int i = 0; i < nseg; ++i) {
        a.seg[i].W = static_cast<const uint8_t*>(Ws[i]);
        a.seg[i].M = Ms[i];
        a.seg[i].work0 = work;
        work += (Ms[i] + a.RW - 1) / a.RW;
    }
    for (int i = nseg; i < kMaxSeg; ++i) a.seg[i] = a.seg[0];
    a.nwork = work;
    const int64_t xrowB =
        xf32 ? K * 4 : (int64_t)a.G * (WT == QMM_Q4_0 || WT == QMM_Q5_0 || WT == QMM_Q8_0 ? 8 * kQ8_0Bytes : kQ8_KBytes);
    // waves per workgroup: spread small problems over all CUs.  A launch that
    // quantizes x itself uses 2 to 4 waves: enough lanes to share each
    // block's quantization, few enough that one compute unit's W requests do
    // not hold up the x loads of its later waves (measured on the 1B-Llama
    // decode shapes).
    const int64_t per_cu = (work + di.cus - 1) / di.cus;
    const int wpg = xf32 ? (per_cu >= 4 ? 4 : 2) : per_cu >= 8 ? 8 : per_cu >= 4 ? 4 : per_cu >= 2 ? 2 : 1;
    for (int64_t n0 = 0; n0 < N;) {
        // Q6_K in groups of at most 6 rows: its 7- and 8-row instances spill
        // (4096x14336 at N = 12 / 16 / 24: 48 / 67 / 94 us against 65 / 87 /
        // 128 us in groups of 8); the other types are fastest in groups of 8
        constexpr int kMaxNC = WT == QMM_Q6_K ? 6 : 8;
        int nc = (int)(N - n0 < kMaxNC ? N - n0 : kMaxNC);
        while (nc > 1 && (size_t)nc * a.G * XREC > di.lds) --nc;
        const size_t lds = (size_t)nc * a.G * XREC;
        if (lds > di.lds) return hipErrorInvalidValue;
        a.xq = static_cast<const uint8_t*>(xq) + n0 * xrowB;
        for (int i = 0; i < nseg; ++i) a.seg[i].y = ys[i] + n0 * Ms[i];
        for (int i = nseg; i < kMaxSeg; ++i) a.seg[i].y = a.seg[0].y;
        hipError_t err = xf32 ? dispatch_nc<WT, true>(nc, a, lds, wpg, s) : dispatch_nc<WT, false>(nc, a, lds, wpg, s);
        if (err != hipSuccess) return err;
        n0 += nc;
    }
    return hipSuccess;
}

hipError_t rowwave(int wtype, const void* W, const void* xq, float* y, int64_t M, int64_t N, int64_t K,
                   hipStream_t s) {
    const dim3 g((unsigned)((M + 3) / 4)), b(256);
    const uint8_t* w = static_cast<const uint8_t*>(W);
    const uint8_t* x = static_cast<const uint8_t*>(xq);
    if (wtype == QMM_Q4_0) return launch(gemv_rowwave_kernel<QMM_Q4_0>, g, b, 0, s, w, x, y, M, (int)N, K);
    if (wtype == QMM_Q8_0) return launch(gemv_rowwave_kernel<QMM_Q8_0>, g, b, 0, s, w, x, y, M, (int)N, K);
    if (wtype == QMM_Q5_0) return launch(gemv_rowwave_kernel<QMM_Q5_0>, g, b, 0, s, w, x, y, M, (int)N, K);
    return hipErrorInvalidValue;
}

bool needs_rowwave(int wtype, int64_t K) {
    return wtype != QMM_Q6_K && K % 256 != 0;  // (Q6_K rows are whole 256-value super-blocks)
}

}  // namespace

bool gemv_fused_supported(int wtype, int64_t K) { return !needs_rowwave(wtype, K); }

hipError_t launch_gemv_multi(int wtype, int count, const void* const* W, float* const* y, const int64_t* M,
                             const void* x, bool x_f32, int64_t N, int64_t K, hipStream_t s) {
    if (count < 1 || count > kMaxSeg) return hipErrorInvalidValue;
    if (needs_rowwave(wtype, K)) {
        if (x_f32) return hipErrorInvalidValue;
        for (int i = 0; i < count; ++i) {
            const hipError_t e = rowwave(wtype, W[i], x, y[i], M[i], N, K, s);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    switch (wtype) {
    case QMM_Q4_0: return gemv_typed<QMM_Q4_0>(count, W, y, M, x, x_f32, N, K, s);
    case QMM_Q8_0: return gemv_typed<QMM_Q8_0>(count, W, y, M, x, x_f32, N, K, s);
    case QMM_Q5_0: return gemv_typed<QMM_Q5_0>(count, W, y, M, x, x_f32, N, K, s);
    case QMM_Q4_K: return gemv_typed<QMM_Q4_K>(count, W, y, M, x, x_f32, N, K, s);
    case QMM_Q6_K: return gemv_typed<QMM_Q6_K>(count, W, y, M, x, x_f32, N, K, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv(int wtype, const void* W, const void* xq, float* y, int64_t M, int64_t N, int64_t K,
                       hipStream_t s) {
    const void* Ws[1] = {W};
    float* ys[1] = {y};
    const int64_t Ms[1] = {M};
    return launch_gemv_multi(wtype, 1, Ws, ys, Ms, xq, false, N, K, s);
}

}  // namespace qmm
