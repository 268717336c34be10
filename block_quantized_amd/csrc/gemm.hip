// gemm.hip — prefill-path product y = W x^T for many activation rows, on raw
// GGUF Q4_K blocks, with int8 matrix cores (gfx950 MFMA).
//
// Method (page "The GGML ecosystem, and where synapse fits", §5, "Products:
// weights against quantized activations"): weights stay in their blocks, the
// activations are Q8_K (int8 codes, fp32 scale per 256, 16-wide integer
// sums), and each super-block contributes
//     dx * ( d * sum_j sc_j * P_j  -  dmin * sum_j m_j * S_j )
// with P_j = sum over sub-block j of q_w * q_x (exact integers) and S_j the
// activation codes' sum over sub-block j.  Prefill is compute-bound (page
// "llama.cpp and GGUF": prefill costs about 2 P n FLOPs and is compute-bound),
// so the contraction runs on v_mfma_i32_32x32x32_i8:
//
//  * Exact int8 operands.  sc_j * q (6-bit scale times 4-bit quant, up to 945)
//    does not fit int8, so the weights enter as two int8 planes,
//    (sc_j >> 3) * q and (sc_j & 7) * q (each <= 105), and
//    sum_j sc_j P_j = 8 * P_hi + P_lo, both exact int32 sums over the super-block.
//  * The min term sum_i m_(i/2) * bsums_i (16 terms) runs on
//    v_mfma_f32_32x32x16_f16: mins (<= 63) and 16-wide sums (|s| <= 2032) are
//    exact in fp16 and the fp32 accumulation of 16 products is exact.
//  * Float scales are applied once per 256-value super-block (epilogue).
//  * Orientation: the MFMA computes C^T tiles (rows = activation rows n,
//    columns = weight rows m), so a lane's weight-row scales d, dmin are
//    per-lane values and its 16 outputs share them.
//  * A workgroup is 4 wavefronts; each owns 32 weight rows and NT x 32
//    activation rows.  The activation tile of each super-block is staged once
//    per workgroup in LDS (double-buffered, one barrier per super-block);
//    weights are loaded by each lane straight into registers one super-block
//    ahead (lane l: row l%32, 16 of the 32 bytes of each nibble pair of a
//    sub-block pair, per the MFMA operand layout: lane l feeds row/column
//    l%32 and K half l/32; result register r of lane l is row
//    8(r/4) + 4(l/32) + r%4, column l%32 — checked on the hardware).
//
// Q6_K weights (w = d * sc_j * (q - 32), 16-value sub-blocks with int8
// scales; the offset 32 is this library's reading of the format table) take
// v_mfma_i32_32x32x16_i8, one per sub-block: the weights enter as the int8
// values q - 32 (in [-32, 31]), so no activation sums are needed, and since
// sc_j * (q - 32) does not fit int8 the per-sub-block scale is applied to the
// int32 tile by VALU (acc += sc_j * P_j, exact).  Up to 32 activation rows
// (the output head) the product is bound by streaming W, and the weights go
// through LDS so that they can be read in row-contiguous 16-byte pieces.
#include "qmm_internal.h"

namespace qmm {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
// 4, 8 and 16 bytes at a 2-byte-aligned address (Q6_K super-blocks are 210
// bytes, Q5_0 and Q8_0 blocks 22 and 34)
typedef uint32_t u32_a2 __attribute__((aligned(2)));
typedef uint32_t u32x2_a2 __attribute__((ext_vector_type(2), aligned(2)));
typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
// 8 and 16 bytes at a 4-byte-aligned address (Q8_K blocks are 292 bytes)
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Makes `v` depend on `acc`, so that the matrix instruction consuming `v` is
// issued after the VALU work that produced `acc` (device code only; an empty
// asm statement emits no instruction).
template <class T>
__device__ __forceinline__ void order_after(long& v, const T& acc) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(v) : "v"(acc));
#endif
}

// XCD-aware tile order.  Workgroups are handed to the 8 XCDs round-robin
// (workgroup i runs on XCD i % 8) and each XCD has its own L2.  Tile t is
// (row block t / nb, column block t % nb); XCD k takes the contiguous run of
// tiles [k * per, (k + 1) * per), so the column blocks that share a row
// block's weights run on one XCD and read those weights into one L2, once.
// Returns false for the workgroups past the last tile.
__device__ __forceinline__ bool xcd_tile(int nb, int total, int& rb, int& cb) {
    const int per = (total + 7) >> 3;
    const int t = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (t >= total || (int)(blockIdx.x >> 3) >= per) return false;
    rb = t / nb;
    cb = t - rb * nb;
    return true;
}

constexpr int kCodeStride = 272;  // LDS bytes per activation row's 256 codes (+16: bank spread)

// bytes b of v (4 quants <= 15) times s (<= 7): each product <= 105 stays in its byte
__device__ __forceinline__ uint32_t mul_bytes(uint32_t v, uint32_t s) {
    u16x2 a = __builtin_bit_cast(u16x2, v);
    u16x2 r = a * (u16x2){(unsigned short)s, (unsigned short)s};
    return __builtin_bit_cast(uint32_t, r);
}

// ---------------------------------------------------------------- Q4_K
// A wave computes 32 weight rows x 32*TN activation rows (TN result tiles of
// v_mfma_i32_32x32x32_i8).  The weight planes of a sub-block are built once
// per wave and feed all TN tiles, so the VALU work of building them is
// spread over TN matrix instructions.  To keep one int32 accumulator per
// tile, the two planes run one after the other within each super-block: the
// (sc >> 3) plane of all eight sub-blocks, then the accumulator times 8
// (a shift), then the (sc & 7) plane on top of it, which leaves
// sum_j sc_j P_j exact in the accumulator.
//
// A workgroup is KS groups of W waves.  The W waves of a group take
// consecutive 32-row blocks of W and share one activation tile in LDS; the
// KS groups take consecutive ranges of super-blocks (K split), and their
// partial sums are added through LDS in a fixed order at the end.  All
// operands go through LDS, read one super-block ahead.
//
// Per super-block a wave issues about as much VALU work (the planes, and the
// fp32 epilogue, whose scales change every super-block) as matrix work, and
// on gfx950 the two overlap only in part, within a wave or across the waves
// of a SIMD: this, not the matrix cores, bounds the kernel.

// One super-block of operands in LDS for a K part: the 32*TN activation
// rows' codes (row n's 256 codes as 16 chunks of 16 bytes, chunk q at
// position q ^ (n & 15), so that the operand reads of 16 consecutive rows at
// one chunk cover all 64 LDS banks), and each wave's 32 weight rows (144
// bytes each, as in memory).  Double-buffered.
// (A wave's weights arrive as 5 reads of 64 x 16 bytes, so its region is
// 5120 bytes: the last 512 receive a repeat of the first 32 chunks.)
constexpr int kQ4KWaveW = 5 * 64 * 16;
template <int TN, int W, int KS, bool WLDS>
struct Q4KStage {
    uint8_t codes[KS][32 * TN][256];
    uint8_t w[KS][W][WLDS ? kQ4KWaveW : 16];
};
// The activation rows' 16 sums and scale for one super-block, double-buffered.
template <int TN, int KS>
struct Q4KSums {
    int16_t sums[KS][32 * TN][16];
    float dx[KS][32 * TN];
};

// The compiler must assume v changed here (emits no instruction).
__device__ __forceinline__ void opaque(uint4& v) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
#endif
}

// No instruction is moved across this point by the compiler's scheduler.
__device__ __forceinline__ void sched_fence() {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_sched_barrier(0);
#endif
}

// byte k of w in both 16-bit halves: (w.k, 0, w.k, 0)
__device__ __forceinline__ uint32_t byte_u16x2(uint32_t w, int k) {
    return __builtin_amdgcn_perm(0u, w, (0x0Cu << 24) | ((uint32_t)k << 16) | (0x0Cu << 8) | (uint32_t)k);
}
// four bytes (each <= 15) times the 16-bit pair s2 = (s, 0, s, 0), s <= 7:
// every product (<= 105) stays in its byte
__device__ __forceinline__ int mul_bytes2(uint32_t v, uint32_t s2) {
    return (int)__builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, v) * __builtin_bit_cast(u16x2, s2));
}

template <int TN, int W, int KS, int WPE>
__global__ __launch_bounds__(64 * W * KS) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void gemm_q4k_kernel(const uint8_t* __restrict__ Wt, const uint8_t* __restrict__ X, float* __restrict__ Y,
                     int M, int N, int SB, int mblk, int nblk) {
    constexpr int BN = 32 * TN;  // activation rows per workgroup
    static_assert(W == 1 || W == 2 || W == 4 || W == 8, "waves per K part");
    static_assert(TN == 2 || TN == 4, "tiles per wave");
    // Weights through LDS (coalesced reads of whole rows) for four tiles per
    // wave; with two, each lane reads its own row's header and nibble pairs
    // straight into registers (fewer LDS operations, registers to spare).
    constexpr bool kWLDS = TN == 4;
    __shared__ __attribute__((aligned(16))) Q4KStage<TN, W, KS, kWLDS> st[2];
    __shared__ __attribute__((aligned(16))) Q4KSums<TN, KS> sd[2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in a scalar register
    const int wave = wave_all % W, kp = wave_all / W;
    const int c = lane & 31, h = lane >> 5;
    int rb, cb;
    if (!xcd_tile(nblk, mblk * nblk, rb, cb)) return;  // whole workgroup: no barrier is skipped
    const int m0 = rb * (32 * W) + 32 * wave;
    const int n0 = cb * BN;
    const int nsb = SB / KS, sb0 = kp * nsb;  // this K part's super-blocks (SB % KS == 0)

    // ---- operand reads.  One buffer descriptor for the workgroup's activation
    // rows that exist and one for the wave's weight rows that exist; every
    // read's whole offset (row, super-block, bytes within the record) is in
    // the lane offset, which the descriptor's range check covers (the scalar
    // offset is 0), so rows at or past N (or M) read as zeros and no read
    // goes past them.  Adding the super-block in the lane offset also keeps
    // the per-read offsets from being hoisted out of the loop into registers
    // of their own.
    const int rowsB = SB * kQ8_KBytes, wrowB = SB * kQ4_KBytes;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(X) + (int64_t)n0 * rowsB, (short)0, min(BN, N - n0) * rowsB, kBufferWord3);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(Wt) + (int64_t)min(m0, M - 1) * wrowB, (short)0,
        __builtin_amdgcn_readfirstlane(max(0, min(32, M - m0))) * wrowB, kBufferWord3);
    // codes: 16-byte read i (of 8 TN per tile) holds tile rows 4i .. 4i+3
    // (lane l: row 4i + l/16, position l%16 of the LDS row, which holds chunk
    // (l%16) ^ (row & 15)); wave w takes reads w, w + W, ...  (read i's
    // offset is that of read i%4 plus i/4 16-row groups, a scalar: with
    // W >= 4 one vector register serves all of a wave's reads)
    constexpr int CPW = 8 * TN / W;  // code reads per wave
    static_assert(CPW * W == 8 * TN, "the code reads divide evenly among the waves");
    auto vo_code = [&](const int i) {
        const int row = 4 * (i & 3) + (lane >> 4);
        return (unsigned)(row * rowsB + 4 + 16 * ((lane & 15) ^ row)) + (unsigned)((i >> 2) * 16 * rowsB);
    };
    // weights: the wave's 32 rows of 144 bytes are 288 chunks of 16 bytes;
    // read k holds chunks 64k .. 64k+63, stored to bytes 1024k + 16 lane of
    // the wave's region (the last one's upper half repeats chunks 0-31 into
    // the region's last 512 bytes, which nothing reads)
    auto vo_w = [&](const int k) {
        const int ch = (64 * k + lane) % 288;
        return (unsigned)((ch / 9) * wrowB + 16 * (ch % 9));
    };
    // (weights into registers: read 0 is row c's header, read 1 + g its
    // 16-byte half h of nibble-pair chunk g)
    auto vo_wd = [&](const int k) { return (unsigned)(c * wrowB + (k ? 16 + 32 * (k - 1) + 16 * h : 0)); };
    // sums: one read covers 32 rows (lane l: row l/2, half l%2); dx: one
    // read covers 64 rows (4 bytes per lane).  Every wave issues the same
    // number of reads (waves beyond the count repeat another wave's: the
    // same bytes to the same place).
    constexpr int SUMS_PW = TN >= W ? TN / W : 1, DX_PW = TN / 2 >= W ? TN / 2 / W : 1;
    const unsigned vo_sums = (unsigned)((lane >> 1) * rowsB + 260 + 16 * (lane & 1));
    const unsigned vo_dx = (unsigned)(lane * rowsB);
    // The next super-block's operands are read into registers at the start
    // of a step and stored to LDS at its end, so their latency is covered by
    // the step's work (direct global-to-LDS copies would leave the compiler
    // to order every LDS read after every copy still in flight).
    u32x4 rc[CPW], rw[5], rs[SUMS_PW];
    uint32_t rd[DX_PW];
    auto fetch = [&](int sb) {
        const unsigned so = (unsigned)(sb * kQ8_KBytes), wo = (unsigned)(sb * kQ4_KBytes);
#pragma unroll
        for (int k = 0; k < CPW; ++k) rc[k] = __builtin_amdgcn_raw_buffer_load_b128(xr, vo_code(wave + W * k) + so, 0, 0);
#pragma unroll
        for (int k = 0; k < 5; ++k)
            rw[k] = __builtin_amdgcn_raw_buffer_load_b128(wr, (kWLDS ? vo_w(k) : vo_wd(k)) + wo, 0, 0);
#pragma unroll
        for (int k = 0; k < SUMS_PW; ++k) {
            const int g2 = (wave + W * k) % TN;  // 32-row group
            rs[k] = __builtin_amdgcn_raw_buffer_load_b128(xr, vo_sums + (unsigned)(32 * g2 * rowsB) + so, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < DX_PW; ++k) {
            const int g4 = (wave + W * k) % (TN / 2);  // 64-row group
            rd[k] = __builtin_amdgcn_raw_buffer_load_b32(xr, vo_dx + (unsigned)(64 * g4 * rowsB) + so, 0, 0);
        }
    };
    auto store = [&](Q4KStage<TN, W, KS, kWLDS>& S, Q4KSums<TN, KS>& D) {
#pragma unroll
        for (int k = 0; k < CPW; ++k) reinterpret_cast<u32x4*>(&S.codes[kp][4 * (wave + W * k)][0])[lane] = rc[k];
#pragma unroll
        for (int k = 0; k < (kWLDS ? 5 : 0); ++k) reinterpret_cast<u32x4*>(&S.w[kp][wave][64 * 16 * k])[lane] = rw[k];
#pragma unroll
        for (int k = 0; k < SUMS_PW; ++k) {
            const int g2 = (wave + W * k) % TN;
            reinterpret_cast<u32x4*>(&D.sums[kp][32 * g2][0])[lane] = rs[k];
        }
#pragma unroll
        for (int k = 0; k < DX_PW; ++k) {
            const int g4 = (wave + W * k) % (TN / 2);
            D.dx[kp][64 * g4 + lane] = __uint_as_float(rd[k]);
        }
    };

    float yacc[TN][16];
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) yacc[t][r] = 0.f;
    // With two tiles per wave there are registers for an accumulator per
    // plane (kDual), which halves the activation operand reads from LDS.
    constexpr bool kDual = TN == 2;
    v16i acc[TN], acc_lo[kDual ? TN : 1];
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[t] = (v16i){};

    // y[n][m] += dx_n * (d * sum_j sc_j P_j - dmin * sum_j m_j S_j) for the
    // super-block with header hdr and sums and scales D
    auto epilogue = [&](const uint4 hdr, const Q4KSums<TN, KS>& D) {
        const float d = h2f(hdr.x), dmin = h2f(hdr.x >> 16);
        const uint32_t m03 = hdr.z & 0x3F3F3F3Fu;
        const uint32_t m47 = ((hdr.w >> 4) & 0x0F0F0F0Fu) | ((hdr.z >> 2) & 0x30303030u);
        // min term: A = the activation rows' 16-wide sums 8h .. 8h+7 (exact
        // in fp16: |s| <= 2032), B = this lane's weight row's mins 4h .. 4h+3,
        // each twice; products and their sum (< 2^24) are exact in fp32
        const uint32_t mw = h ? m47 : m03;
        v8h mins;
#pragma unroll
        for (int e = 0; e < 8; ++e) mins[e] = (_Float16)(float)((mw >> (8 * (e >> 1))) & 0xFF);
#pragma unroll
        for (int t = 0; t < TN; ++t) {
            const v8s bi = *reinterpret_cast<const v8s*>(&D.sums[kp][32 * t + c][8 * h]);
            v8h bs;
#pragma unroll
            for (int e = 0; e < 8; ++e) bs[e] = (_Float16)bi[e];
            const v16f amin = __builtin_amdgcn_mfma_f32_32x32x16_f16(bs, mins, (v16f){}, 0, 0, 0);
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const float4 dx = *reinterpret_cast<const float4*>(&D.dx[kp][32 * t + 8 * qd + 4 * h]);
                const float dxa[4] = {dx.x, dx.y, dx.z, dx.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * qd + e;
                    const float v = __builtin_fmaf((float)acc[t][r], d, -(dmin * amin[r]));
                    yacc[t][r] = __builtin_fmaf(v, dxa[e], yacc[t][r]);
                }
            }
            sched_fence();  // one tile's min-term result (16 registers) live at a time
        }
    };

    const int hsw = c & 15;  // swizzle key of row 32t + c

    fetch(sb0);
    store(st[0], sd[0]);
    __syncthreads();
    for (int i = 0; i < nsb; ++i) {
        // super-block sb0 + i: its operands are in st[i % 2] and sd[i % 2];
        // the next one's go to the other buffers
        const int sb = sb0 + i, b2 = i & 1;
        const Q4KStage<TN, W, KS, kWLDS>& S = st[b2];
        // this lane's header and nibble-pair halves (row c, values 16h ..)
        const uint8_t* wl = &S.w[kp][wave][kQ4_KBytes * c];
        const uint4 hdr = kWLDS ? *reinterpret_cast<const uint4*>(wl) : __builtin_bit_cast(uint4, rw[0]);
        uint4 q[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
            q[g] = kWLDS ? *reinterpret_cast<const uint4*>(wl + 16 + 32 * g + 16 * h) : __builtin_bit_cast(uint4, rw[1 + g]);
        const uint32_t sc03 = hdr.y & 0x3F3F3F3Fu;
        const uint32_t sc47 = (hdr.w & 0x0F0F0F0Fu) | ((hdr.y >> 2) & 0x30303030u);
        auto operand = [&](const int j, const uint32_t s2) {
            const uint4 qq = q[j >> 1];
            const int sh = (j & 1) * 4;
            return (v4i){mul_bytes2((qq.x >> sh) & 0x0F0F0F0Fu, s2), mul_bytes2((qq.y >> sh) & 0x0F0F0F0Fu, s2),
                         mul_bytes2((qq.z >> sh) & 0x0F0F0F0Fu, s2), mul_bytes2((qq.w >> sh) & 0x0F0F0F0Fu, s2)};
        };
        auto act = [&](const int t, const int j) {
            return *reinterpret_cast<const v4i*>(&S.codes[kp][32 * t + c][16 * ((2 * j + h) ^ hsw)]);
        };
        // One plane pass: per sub-block j, the weight operand (VALU), then TN
        // matrix instructions, each followed by the LDS read of its
        // activation operand for j + 1 into the register it has just read.
        // A scheduling barrier after each sub-block keeps the compiler from
        // hoisting every read (which would hold 32 TN registers), so the
        // matrix core works through sub-block j while the wave builds the
        // operand of j + 1 and the reads of j + 1 are in flight.
        auto pass = [&](const uint32_t w03, const uint32_t w47, const bool first) {
            v4i a[TN];
#pragma unroll
            for (int t = 0; t < TN; ++t) a[t] = act(t, 0);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                // (the empty asm keeps the nibble extraction of a sub-block
                // pair here instead of hoisted to the top of the step, where
                // it would hold 32 registers)
                if (!(j & 1)) opaque(q[j >> 1]);
                const v4i b = operand(j, byte_u16x2(j < 4 ? w03 : w47, j & 3));
#pragma unroll
                for (int t = 0; t < TN; ++t) {
                    acc[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[t], b, (first && j == 0) ? (v16i){} : acc[t],
                                                                   0, 0, 0);
                    if (j < 7) a[t] = act(t, j + 1);
                }
                sched_fence();
            }
        };
        if constexpr (kDual) {
            // both planes per sub-block, each activation operand read once
            // for two matrix instructions: (sc >> 3) into acc, (sc & 7) into
            // acc_lo; the epilogue forms 8 acc + acc_lo
            fetch(min(sb + 1, sb0 + nsb - 1));
            const uint32_t h03 = (sc03 >> 3) & 0x07070707u, h47 = (sc47 >> 3) & 0x07070707u;
            const uint32_t l03 = sc03 & 0x07070707u, l47 = sc47 & 0x07070707u;
            v4i a[TN];
#pragma unroll
            for (int t = 0; t < TN; ++t) a[t] = act(t, 0);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (!(j & 1)) opaque(q[j >> 1]);
                const v4i bh = operand(j, byte_u16x2(j < 4 ? h03 : h47, j & 3));
                const v4i bl = operand(j, byte_u16x2(j < 4 ? l03 : l47, j & 3));
#pragma unroll
                for (int t = 0; t < TN; ++t) {
                    acc[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[t], bh, j ? acc[t] : (v16i){}, 0, 0, 0);
                    acc_lo[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[t], bl, j ? acc_lo[t] : (v16i){}, 0, 0, 0);
                    if (j < 7) a[t] = act(t, j + 1);
                }
                sched_fence();
            }
#pragma unroll
            for (int t = 0; t < TN; ++t) acc[t] = (acc[t] << 3) + acc_lo[t];
        } else {
            pass((sc03 >> 3) & 0x07070707u, (sc47 >> 3) & 0x07070707u, true);   // (sc >> 3) plane
            // the next super-block's operands, into registers (stored to the
            // free buffers at the end of the step; the last step repeats its
            // own).  Issued here rather than at the top, so that the registers
            // they occupy are not live during the first pass.
            fetch(min(sb + 1, sb0 + nsb - 1));
#pragma unroll
            for (int t = 0; t < TN; ++t) acc[t] = acc[t] << 3;
            pass(sc03 & 0x07070707u, sc47 & 0x07070707u, false);                 // (sc & 7) plane
        }

        epilogue(hdr, sd[b2]);
        store(st[b2 ^ 1], sd[b2 ^ 1]);
        __syncthreads();  // the next operands are in place, and this step's buffers are free
    }
    if constexpr (KS > 1) {
        // the K parts' partial sums, added in a fixed order through LDS (the
        // stage buffers are free: the last step ended with a barrier that
        // waited for its copy)
        constexpr int kPart = W * TN * 16 * 64;  // floats of one K part
        static_assert(sizeof(st[0]) >= (KS - 1) * kPart * sizeof(float), "partials fit a stage buffer");
        float* red = reinterpret_cast<float*>(&st[0]);
        if (kp > 0) {
            float* dst = red + (kp - 1) * kPart;
#pragma unroll
            for (int t = 0; t < TN; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) dst[((wave * TN + t) * 16 + r) * 64 + lane] = yacc[t][r];
        }
        __syncthreads();
        if (kp > 0) return;
#pragma unroll
        for (int p = 1; p < KS; ++p)
#pragma unroll
            for (int t = 0; t < TN; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) yacc[t][r] += red[(p - 1) * kPart + ((wave * TN + t) * 16 + r) * 64 + lane];
    }

    const int m = m0 + c;
    if (m < M) {
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int n = n0 + 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
                if (n < N) Y[(int64_t)n * M + m] = yacc[t][r];
            }
    }
}

// ------------------------------------------------------------------ Q6_K
// One v_mfma_i32_32x32x16_i8 per 16-value sub-block.  Lane l = (c = l%32,
// h = l/32) feeds weight row m0 + c and, for sub-block j (values 16j .. 16j+15
// of the super-block), the 8 values 16j + 8h .. +7; their low 4 bits are 8
// consecutive nibbles of ql and their high 2 bits a 2-bit field of 8
// consecutive qh bytes, so each lane's operand is an 8-byte ql chunk and an
// 8-byte qh chunk.  The activation operand holds the same 8 codes of the same
// sub-block (any consistent assignment of k to lanes gives the same sum).
//
// The weights are staged per wave through LDS.  Lane-per-row 8-byte chunk
// loads straight from memory touch 32 rows per instruction and streamed the
// 431 MB output head at about 4 TB/s (measured on MI355X).  Here a wave reads
// its tile of one super-block (32 rows x the 192 bytes of ql and qh) with
// 16-byte loads that consecutive lanes issue for consecutive pieces of a row
// (12 per row; about 5 TB/s for the same head in a read-only probe), writes
// the tile to its own LDS region after the current step's operands have been
// read from it, and each lane then reads its operand chunks from there.
// Scales and d are read per lane.  The 16 sub-blocks run in four groups that
// share a qh chunk, so a lane holds 6 operand registers at a time.  NT
// activation tiles of 32 rows per wave, WV waves per workgroup and K part, WPE
// waves per SIMD (which bounds the registers), KS K parts whose partial sums
// are added through LDS in a fixed order.
constexpr int kQ6WRow = 208;  // LDS bytes per weight row: ql|qh (192) + 16 (bank spread, 16-byte aligned)
template <int NT, int WV, int WPE, int KS = 1>
__global__ __launch_bounds__(64 * WV * KS) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void gemm_q6k_lds_kernel(
    const uint8_t* __restrict__ W, const uint8_t* __restrict__ X, float* __restrict__ Y, int M, int N, int SB,
    int mblk, int nblk) {
    constexpr int BN = NT * 32;
    constexpr int NTH = 64 * WV;  // threads of one K part
    __shared__ __attribute__((aligned(16))) uint8_t s_codes_all[KS][2][BN][kCodeStride];
    __shared__ __attribute__((aligned(16))) float s_dx_all[KS][2][BN];
    __shared__ __attribute__((aligned(16))) uint8_t s_w_all[KS][WV][32 * kQ6WRow];

    const int tid = threadIdx.x % NTH, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: bases in scalar registers
    // K part: KS groups of WV waves take consecutive ranges of SB / KS
    // super-blocks, each with its own LDS buffers
    const int kp = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / NTH));
    auto& s_codes = s_codes_all[kp];
    auto& s_dx = s_dx_all[kp];
    auto& s_w = s_w_all[kp];
    const int SBK = SB / KS, sbb = kp * SBK;
    const int c = lane & 31, h = lane >> 5;
    int rb, cb;
    if (!xcd_tile(nblk, mblk * nblk, rb, cb)) return;  // whole workgroup: no barrier is skipped
    const int m0 = rb * (32 * WV) + wave * 32;
    const int n0 = cb * BN;
    const int64_t rowB = (int64_t)SB * kQ6_KBytes;
    const int last = M - 1 - m0;  // rows past M are computed on a copy of row M-1 and not stored
    const uint8_t* wbase = W + (int64_t)min(m0, M - 1) * rowB;
    // this lane's 6 pieces: piece g = 64 i + lane is row g / 12, bytes 16 (g % 12) .. +15
    // (offsets recomputed where used: fewer registers held across the loop)
    const int lastc = max(last, 0);
    auto poff = [&](int i) {
        const int g = 64 * i + lane, r = g / 12, pc = g - 12 * r;
        return (uint32_t)(min(r, lastc) * (uint32_t)rowB + 16 * pc);
    };
    auto soff = [&](int i) {
        const int g = 64 * i + lane, r = g / 12, pc = g - 12 * r;
        return (uint32_t)(r * kQ6WRow + 16 * pc);
    };
    const uint32_t coff = (uint32_t)(min(c, max(last, 0)) * rowB);
    uint8_t* const sw = s_w[wave];

    // ---- activation staging: (row, piece) items of 16 codes; piece 0 also carries d
    constexpr int ITEMS = BN * 16;
    constexpr int IPT = (ITEMS + NTH - 1) / NTH;
    u32x4_a4 xc[IPT];
    uint32_t xd[IPT];
    auto x_load = [&](int sb) {
#pragma unroll
        for (int k = 0; k < IPT; ++k) {
            const int it = (tid + NTH * k) % ITEMS;
            const int rn = it >> 4, pc = it & 15;
            const int n = min(n0 + rn, N - 1);
            const uint8_t* p = X + ((int64_t)n * SB + sb) * kQ8_KBytes;
            xc[k] = *reinterpret_cast<const u32x4_a4*>(p + 4 + 16 * pc);
            xd[k] = *reinterpret_cast<const uint32_t*>(p);
        }
    };
    auto x_store = [&](int buf) {
#pragma unroll
        for (int k = 0; k < IPT; ++k) {
            const int it = tid + NTH * k;
            if (it < ITEMS) {
                const int rn = it >> 4, pc = it & 15;
                *reinterpret_cast<uint4*>(&s_codes[buf][rn][16 * pc]) = make_uint4(xc[k].x, xc[k].y, xc[k].z, xc[k].w);
                if (pc == 0) s_dx[buf][rn] = __uint_as_float(xd[k]);
            }
        }
    };
    u32x4_a2 wp[6];
    u32x4_a2 scn;
    uint32_t dn;
    auto w_load = [&](int sb) {
        const uint8_t* b = wbase + (int64_t)sb * kQ6_KBytes;
#pragma unroll
        for (int i = 0; i < 6; ++i) wp[i] = *reinterpret_cast<const u32x4_a2*>(b + poff(i));
        scn = *reinterpret_cast<const u32x4_a2*>(b + coff + 192);
        dn = *reinterpret_cast<const uint16_t*>(b + coff + 208);
    };
    auto w_store = [&]() {
#pragma unroll
        for (int i = 0; i < 6; ++i)
            *reinterpret_cast<uint4*>(sw + soff(i)) = make_uint4(wp[i].x, wp[i].y, wp[i].z, wp[i].w);
    };

    float yacc[NT][16];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) yacc[t][r] = 0.f;

    x_load(sbb);
    w_load(sbb);
    x_store(0);
    w_store();
    __syncthreads();

    const uint8_t* const wrow_l = sw + c * kQ6WRow + 8 * h;
    for (int sbi = 0; sbi < SBK; ++sbi) {
        const int sb = sbb + sbi, buf = sbi & 1;
        const u32x4_a2 sc4 = scn;
        const uint32_t dcur = dn;
        if (sbi + 1 < SBK) {
            x_load(sb + 1);
            w_load(sb + 1);
        }
        v16i acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = (v16i){};
        auto product = [&](const int j, const int t, const long bq) {
            const long a = *reinterpret_cast<const long*>(&s_codes[buf][32 * t + c][16 * j + 8 * h]);
            return __builtin_amdgcn_mfma_i32_32x32x16_i8(a, bq, (v16i){}, 0, 0, 0);
        };
        // sub-blocks in groups that share a qh chunk: group (h2, p) holds
        // j = 8 h2 + 2 cc + p for cc = 0..3; ql chunks (h2, cc & 1, p)
        v16i tl[2][NT];
        int prev_sc = 0, have = 0;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int h2 = gq >> 1, p = gq & 1;
            const u32x2 hq = *reinterpret_cast<const u32x2*>(wrow_l + 128 + 16 * (2 * h2 + p));
            const u32x2 lq0 = *reinterpret_cast<const u32x2*>(wrow_l + 16 * (4 * h2 + p));
            const u32x2 lq1 = *reinterpret_cast<const u32x2*>(wrow_l + 16 * (4 * h2 + 2 + p));
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                const int j = 8 * h2 + 2 * cc + p;
                const u32x2 lq = (cc & 1) ? lq1 : lq0;
                const int ls = (cc >> 1) * 4;
                uint32_t b[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const uint32_t lo = (lq[e] >> ls) & 0x0F0F0F0Fu;
                    const uint32_t hi = (hq[e] >> (2 * cc)) & 0x03030303u;
                    b[e] = lo | __builtin_amdgcn_perm(0u, 0x1000F0E0u, hi);
                }
                long bq = (long)(((uint64_t)b[1] << 32) | b[0]);
                if (have) {
#pragma unroll
                    for (int t = 0; t < NT; ++t) order_after(bq, acc[t]);
                }
                const int cur = have & 1;
#pragma unroll
                for (int t = 0; t < NT; ++t) tl[cur][t] = product(j, t, bq);
                if (have) {
#pragma unroll
                    for (int t = 0; t < NT; ++t)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[t][r] = __mul24(prev_sc, tl[cur ^ 1][t][r]) + acc[t][r];
                }
                prev_sc = (int)(int8_t)(sc4[j >> 2] >> (8 * (j & 3)));
                ++have;
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[t][r] = __mul24(prev_sc, tl[(have - 1) & 1][t][r]) + acc[t][r];
        const float dw = h2f(dcur);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const float4 dx = *reinterpret_cast<const float4*>(&s_dx[buf][32 * t + 8 * qd + 4 * h]);
                const float dxa[4] = {dx.x, dx.y, dx.z, dx.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * qd + e;
                    yacc[t][r] += (dw * dxa[e]) * (float)acc[t][r];
                }
            }
        }
        if (sbi + 1 < SBK) {
            x_store(buf ^ 1);
            w_store();
        }
        __syncthreads();
    }
    if constexpr (KS > 1) {
        // the K parts' partial sums, added in a fixed order through LDS (the
        // code tiles are free: the last step ended with a barrier)
        constexpr int kPart = WV * NT * 16 * 64;  // floats of one K part
        static_assert(sizeof(s_codes_all) >= (KS - 1) * kPart * sizeof(float), "partials fit the code tiles");
        float* red = reinterpret_cast<float*>(&s_codes_all[0][0][0][0]);
        if (kp > 0) {
            float* dst = red + (kp - 1) * kPart;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) dst[((wave * NT + t) * 16 + r) * 64 + lane] = yacc[t][r];
        }
        __syncthreads();
        if (kp > 0) return;
#pragma unroll
        for (int p = 1; p < KS; ++p)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) yacc[t][r] += red[(p - 1) * kPart + ((wave * NT + t) * 16 + r) * 64 + lane];
    }

    const int m = m0 + c;
    if (m < M) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int n = n0 + 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
                if (n < N) Y[(int64_t)n * M + m] = yacc[t][r];
            }
    }
}

// ------------------------------------------------- Q4_0, Q5_0, Q8_0 weights
// 32-value blocks with one fp16 scale each, against Q8_0 activations.  The
// weight codes enter the MFMA as int8 (q - 8, q - 16 or q itself), one
// v_mfma_i32_32x32x32_i8 per block and activation tile, and each block's
// integer tile is scaled by d_w * d_x in fp32.  The scales change every 32
// values, so this epilogue, not the matrix core, bounds the kernel: the tile
// of products d_x[n] * d_w[m] comes from the matrix core too (one fp16 MFMA
// on one-hot operands, exact), which leaves two VALU operations per output
// and block (convert, fused multiply-add).
// K runs in chunks of 4 blocks; the activation chunk of 64 rows is staged in
// LDS (codes at row stride 144, scales as [block][row] fp16 bits).
template <int WT>
struct Q32W;  // per-lane weight operand of one block: row c, values 16h .. 16h+15
template <>
struct Q32W<QMM_Q8_0> {
    static constexpr int kBytes = kQ8_0Bytes;
    uint32_t d;
    u32x4_a2 q;
    __device__ void load(const uint8_t* b, int h) {
        d = *reinterpret_cast<const uint16_t*>(b);
        q = *reinterpret_cast<const u32x4_a2*>(b + 2 + 16 * h);
    }
    __device__ v4i operand(int) const { return (v4i){(int)q.x, (int)q.y, (int)q.z, (int)q.w}; }
};
// 4-bit codes (0..15) minus 8 as int8, four per word: q + 0x78 stays below
// 0x100 (no carry into the next byte), and flipping bit 7 of it leaves
// q - 8 for q >= 8 and 0x100 + q - 8 for q < 8.  (Two full-rate operations;
// a 32-bit multiply is a quarter-rate one.)
__device__ __forceinline__ uint32_t nibbles_minus_8(uint32_t t) {
    return (t + 0x78787878u) ^ 0x80808080u;
}
template <>
struct Q32W<QMM_Q4_0> {
    static constexpr int kBytes = kQ4_0Bytes;
    uint32_t d;
    u32x4_a2 q;
    __device__ void load(const uint8_t* b, int) {
        d = *reinterpret_cast<const uint16_t*>(b);
        q = *reinterpret_cast<const u32x4_a2*>(b + 2);
    }
    __device__ v4i operand(int h) const {  // values 0-15: low nibbles, 16-31: high
        const int sh = 4 * h;
        return (v4i){(int)nibbles_minus_8((q.x >> sh) & 0x0F0F0F0Fu), (int)nibbles_minus_8((q.y >> sh) & 0x0F0F0F0Fu),
                     (int)nibbles_minus_8((q.z >> sh) & 0x0F0F0F0Fu), (int)nibbles_minus_8((q.w >> sh) & 0x0F0F0F0Fu)};
    }
};
// 5-bit codes minus 16: bits 0-3 from the nibble, bit 4 from qh (bit k of
// the 4 bits times 0x00204081 lands at bit 8k; a 24-bit multiply, full rate,
// which the compiler does not pick by itself here); then as for Q4_0 with
// q + 0x70, which stays below 0x100.
__device__ __forceinline__ uint32_t q5_minus_16(uint32_t nib, uint32_t bits4) {
    uint32_t sp;
    asm("v_mul_u32_u24_e32 %0, 0x204081, %1" : "=v"(sp) : "v"(bits4));
    const uint32_t t = nib | ((sp & 0x01010101u) << 4);
    return (t + 0x70707070u) ^ 0x80808080u;
}
template <>
struct Q32W<QMM_Q5_0> {
    static constexpr int kBytes = kQ5_0Bytes;
    uint32_t d, qh;
    u32x4_a2 q;
    __device__ void load(const uint8_t* b, int) {
        d = *reinterpret_cast<const uint16_t*>(b);
        qh = *reinterpret_cast<const u32_a2*>(b + 2);
        q = *reinterpret_cast<const u32x4_a2*>(b + 6);
    }
    __device__ v4i operand(int h) const {
        const int sh = 4 * h;
        const uint32_t hb = qh >> (16 * h);
        return (v4i){(int)q5_minus_16((q.x >> sh) & 0x0F0F0F0Fu, hb & 15u),
                     (int)q5_minus_16((q.y >> sh) & 0x0F0F0F0Fu, (hb >> 4) & 15u),
                     (int)q5_minus_16((q.z >> sh) & 0x0F0F0F0Fu, (hb >> 8) & 15u),
                     (int)q5_minus_16((q.w >> sh) & 0x0F0F0F0Fu, (hb >> 12) & 15u)};
    }
};

// One-hot fp16 operand of v_mfma_f32_32x32x8_f16: the fp16 in the low half of
// `bits` at the lane's first K slot, zeros in the other three.  With the A
// lane of row n holding d_x[n] and the B lane of column m holding d_w[m] (and
// the lanes of the other K half all zero), the product tile is d_x[n] d_w[m],
// exact in fp32 (two 11-bit significands).
__device__ __forceinline__ v4h onehot_f16(uint32_t bits) {
    return __builtin_bit_cast(v4h, ((v2i){(int)bits, 0}));
}

// K parts of the kernel on small grids: 4, four waves per SIMD (within the
// 128 VGPRs that allows; Q8_0, with 17 registers of next-chunk weights per
// lane, spills one).
constexpr int kSplitQ32 = 4;

// KS = 2 or 4 splits the chunks between KS groups of 4 waves, as in the Q4_K
// kernel (the launcher takes KS > 1 only when the chunks are full and there
// are at least KS of them).  The partial sums are added through LDS in a fixed
// tree, (p0 + p2) + (p1 + p3) for four parts, so results are deterministic.
template <int WT, int KS, bool WC>
__global__ __launch_bounds__(256 * KS, KS == 4 ? 1 : 2) void gemm_q32_kernel(const uint8_t* __restrict__ W,
                                                                 const uint8_t* __restrict__ X,
                                                                 float* __restrict__ Y, int M, int N, int NB,
                                                                 int mblk, int nblk) {
    constexpr int BN = 64, CB = 4;          // activation rows per workgroup, blocks per chunk
    constexpr int CS = 32 * CB + 16;        // LDS row stride of a chunk's codes
    static_assert(KS == 1 || KS == 2 || KS == 4, "K is split in 1, 2 or 4 parts");
    __shared__ __attribute__((aligned(16))) uint8_t s_codes_all[KS][2][BN][CS];
    // fp16 bits of the activation scales; entries BN .. 2 BN - 1 stay zero (the
    // scale operand of the lanes in the second K half)
    __shared__ __attribute__((aligned(16))) uint16_t s_dx_all[KS][2][CB][2 * BN];

    const int tid = threadIdx.x & 255, lane = tid & 63, wave = tid >> 6;
    const int kh = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);  // K part
    const int c = lane & 31, h = lane >> 5;
    auto& s_codes = s_codes_all[kh];
    auto& s_dx = s_dx_all[kh];
    int rb, cb;
    if (!xcd_tile(nblk, mblk * nblk, rb, cb)) return;  // whole workgroup: no barrier is skipped
    const int m0 = rb * 128 + wave * 32;
    const int n0 = cb * BN;
    const int mrow = min(m0 + c, M - 1);  // rows past M are computed on a copy and not stored
    const uint8_t* wrow = W + (int64_t)mrow * NB * Q32W<WT>::kBytes;
    const int nch = NB / CB, tail = NB % CB;  // full chunks; blocks in the last, partial one

    // activation staging: thread = (row rn, block jb) of the chunk, read
    // through a buffer descriptor over the workgroup's activation rows that
    // exist (rows past N read row N - 1), so the lane offset is 32-bit and no
    // 64-bit addresses are held in registers
    const int rn = tid >> 2, jb = tid & 3;
    const int xrowB = NB * kQ8_0Bytes;
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(X) + (int64_t)n0 * xrowB, (short)0, min(BN, N - n0) * xrowB, kBufferWord3);
    const unsigned xvo = (unsigned)(min(rn, N - 1 - n0) * xrowB);
    u32x4 xq0, xq1;
    uint32_t xdb;
    auto x_load = [&](int ch) {
        const int blk = min(ch * CB + jb, NB - 1);  // a partial chunk repeats its last block
        const unsigned o = xvo + (unsigned)(blk * kQ8_0Bytes);
        xdb = __builtin_amdgcn_raw_buffer_load_b16(xrs, o, 0, 0);
        xq0 = __builtin_amdgcn_raw_buffer_load_b128(xrs, o + 2, 0, 0);
        xq1 = __builtin_amdgcn_raw_buffer_load_b128(xrs, o + 18, 0, 0);
    };
    auto x_store = [&](int buf) {
        uint4* dst = reinterpret_cast<uint4*>(&s_codes[buf][rn][32 * jb]);
        dst[0] = make_uint4(xq0.x, xq0.y, xq0.z, xq0.w);
        dst[1] = make_uint4(xq1.x, xq1.y, xq1.z, xq1.w);
        s_dx[buf][jb][rn] = (uint16_t)xdb;
    };
    // Weights, WC (whole chunks, NB % CB == 0): the wave's 32 rows x CB blocks
    // as row-contiguous 8-byte pieces (consecutive lanes, consecutive pieces of
    // a row) into registers a chunk ahead, written to the wave's own LDS region
    // at the top of the chunk they belong to, where each lane then reads its
    // row's blocks.  Lane-per-row block loads touch 32 rows per instruction and
    // cost the texture path more (4096x4096, N = 512: Q4_0 70.9 -> 52.9 us,
    // Q5_0 86.5 -> 60.8 us, Q8_0 76.3 -> 54.4 us, measured on MI355X).  Without
    // WC each lane loads its own row's blocks.
    constexpr int RBc = CB * Q32W<WT>::kBytes, PR = RBc / 8, PW = (32 * PR + 63) / 64;
    static_assert(RBc % 8 == 0, "whole 8-byte pieces");
    __shared__ __attribute__((aligned(16))) uint8_t s_wc_all[KS][4][WC ? 32 * RBc : 8];
    uint8_t* const swc = s_wc_all[kh][wave];
    const int64_t rowWB = (int64_t)NB * Q32W<WT>::kBytes;
    u32x2 wpc[WC ? PW : 1];
    // the wave's first row that exists (uniform), a buffer descriptor over
    // its rows that exist, and each piece's 32-bit offset from that row (rows
    // past M read row M - 1; with K <= 65536 the offsets stay below 2^22)
    const int wr0 = __builtin_amdgcn_readfirstlane(min(m0, M - 1));
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(W) + (int64_t)wr0 * rowWB, (short)0,
        __builtin_amdgcn_readfirstlane(min(32, M - wr0)) * (int)rowWB, kBufferWord3);
    uint32_t woff[WC ? PW : 1];
    if constexpr (WC) {
#pragma unroll
        for (int i = 0; i < PW; ++i) {
            const int g = min(64 * i + lane, 32 * PR - 1), r = g / PR, pc = g - PR * r;
            woff[i] = (uint32_t)(min(m0 + r, M - 1) - wr0) * (uint32_t)rowWB + 8 * pc;
        }
    }
    Q32W<WT> wn[WC ? 1 : CB];
    auto w_load = [&](int ch) {
        if constexpr (WC) {
            const int so = min(ch, NB / CB - 1) * RBc;  // the chunk, in the scalar offset
#pragma unroll
            for (int i = 0; i < PW; ++i) {
                const v2i v = __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(wrs, woff[i], so, 0));
                wpc[i] = (u32x2){(uint32_t)v.x, (uint32_t)v.y};
            }
        } else {
#pragma unroll
            for (int j = 0; j < CB; ++j) wn[j].load(wrow + (int64_t)min(ch * CB + j, NB - 1) * Q32W<WT>::kBytes, h);
        }
    };
    auto w_put = [&]() {
#pragma unroll
        for (int i = 0; i < PW; ++i) {
            const int g = 64 * i + lane;
            if (g < 32 * PR) *reinterpret_cast<u32x2*>(swc + 8 * g) = wpc[i];
        }
    };

    float yacc[2][16];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) yacc[t][r] = 0.f;
    // the scale operands: d_x from LDS (lanes of the second K half read the
    // zero entries), d_w masked to zero in those lanes
    const int dxl = c + (h ? BN : 0);
    const uint32_t hmask = h ? 0u : 0xFFFFu;
#pragma unroll
    for (int i = tid; i < 2 * CB * BN; i += 256) s_dx[i / (CB * BN)][(i / BN) % CB][BN + i % BN] = 0;

    // this K part's chunks: part kh takes chunks [kh TC / KS, (kh + 1) TC / KS)
    // of the TC, so the parts differ by at most one chunk.  Every part runs
    // the longest part's count of iterations, so that the workgroup's barriers
    // pair up, and computes nothing in those past its own chunks (their loads
    // are clamped to chunks that exist).
    const int TC = nch + (tail ? 1 : 0);
    const int ch0 = kh * TC / KS, nper = (kh + 1) * TC / KS - ch0, nit = (TC + KS - 1) / KS;
    // Q5_0 issues the next chunk's loads and LDS store unconditionally
    // (after the last chunk they re-read blocks that exist and fill a buffer
    // nobody reads).  With a branch around them the compiler's load waits must
    // fit both paths, and the chunk's first block then also waits for most of
    // the next chunk's loads, of which Q5_0 has 12.  Measured at 4096x4096,
    // N = 512: Q5_0 86.8 us against 104.8; Q4_0 and Q8_0 2-3% slower, so they
    // keep the branch.
    constexpr bool kAlwaysNext = WT == QMM_Q5_0;
    x_load(ch0);
    w_load(ch0);
    x_store(0);
    __syncthreads();
    for (int i = 0; i < nit; ++i) {
        const int ch = ch0 + i, buf = i & 1;
        Q32W<WT> wc_[WC ? 1 : CB];  // without WC: this chunk's blocks, loaded a chunk ahead
        if constexpr (WC) {
            w_put();  // this chunk's weights (the previous chunk's reads of the region are done)
        } else {
#pragma unroll
            for (int j = 0; j < CB; ++j) wc_[j] = wn[j];
        }
        if (kAlwaysNext || i + 1 < nit) {
            x_load(ch + 1);
            w_load(ch + 1);
        }
        const int nb = i >= nper ? 0 : (ch < nch) ? CB : tail;  // blocks in this chunk
        // Per block: the weight block, both tiles' activation codes and scales
        // from LDS, then each tile's two matrix instructions and its epilogue
        // in turn (one tile's results live at a time, so that four waves per
        // SIMD fit their registers; the other waves hide the latencies).
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            Q32W<WT> wj;
            if constexpr (WC) wj.load(swc + c * RBc + j * Q32W<WT>::kBytes, h);
            else wj = wc_[j];
            v4i ar[2];
            uint32_t dxb[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                ar[t] = *reinterpret_cast<const v4i*>(&s_codes[buf][32 * t + c][32 * j + 16 * h]);
                dxb[t] = s_dx[buf][j][32 * t + dxl];
            }
            __builtin_amdgcn_sched_barrier(0);
            if (j < nb) {
                const v4i bq = wj.operand(h);
                const v4h dwo = onehot_f16(wj.d & hmask);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(ar[t], bq, (v16i){}, 0, 0, 0);
                    const v16f sc = __builtin_amdgcn_mfma_f32_32x32x8f16(onehot_f16(dxb[t]), dwo, (v16f){}, 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int r = 0; r < 16; ++r) yacc[t][r] = __builtin_fmaf(sc[r], (float)p[r], yacc[t][r]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        if (kAlwaysNext || i + 1 < nit) x_store(buf ^ 1);
        __syncthreads();
    }

    if constexpr (KS > 1) {
        // the tiles are free: the last chunk ended with a barrier.  Level s:
        // parts s .. 2s-1 hand their sums to parts 0 .. s-1.  Every wave
        // takes every barrier; only part 0 goes on to the stores.
        constexpr int kPart = 4 * 2 * 16 * 64;  // floats of one part's sums
        static_assert(sizeof(s_codes_all) >= KS / 2 * kPart * sizeof(float), "partials fit the code tiles");
        float* red = reinterpret_cast<float*>(&s_codes_all[0][0][0][0]);
#pragma unroll
        for (int lv = KS / 2; lv >= 1; lv /= 2) {
            if (kh >= lv && kh < 2 * lv) {
                float* dst = red + (kh - lv) * kPart;
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) dst[((wave * 2 + t) * 16 + r) * 64 + lane] = yacc[t][r];
            }
            __syncthreads();
            if (kh < lv) {
                const float* src = red + kh * kPart;
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) yacc[t][r] += src[((wave * 2 + t) * 16 + r) * 64 + lane];
            }
            __syncthreads();
        }
        if (kh != 0) return;
    }

    const int m = m0 + c;
    if (m < M) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int n = n0 + 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
                if (n < N) Y[(int64_t)n * M + m] = yacc[t][r];
            }
    }
}

// ------------------------------------------------------------ narrow batches
// N <= 32 activation rows (decode batches): one 32-wide MFMA column tile.
// The weights are streamed once and the kernel aims at HBM bandwidth: a
// workgroup of NW waves owns 32 weight rows, wave w takes super-blocks w,
// w + NW, ..., and the NW partial tiles are summed in LDS in a fixed order.
// Compared with the VALU GEMV, the weight decode (scale planes) is shared by
// all N columns instead of repeated per column.
//
// Orientation: the MFMA computes W-row x activation-row tiles (A = weight
// planes, B = activation codes), so a lane's result column is activation row
// c, with its scale dx per lane, and its 16 result registers are weight rows
// 8(r/4) + 4h + r%4, whose d and dmin come from the lanes that loaded those
// rows, through LDS.  Operands and registers follow the layout used above.
// Loads for the next super-block of a wave are issued before the current
// one is computed (two register stages, named statically).  Past the end a
// wave re-loads its last super-block, which it then skips.
template <int kNarrowWaves>
__global__ __launch_bounds__(64 * kNarrowWaves) void gemm_narrow_q4k_kernel(const uint8_t* __restrict__ W,
                                                                       const uint8_t* __restrict__ X,
                                                                       float* __restrict__ Y, int M, int N,
                                                                       int SB) {
    __shared__ __attribute__((aligned(16))) float s_d[kNarrowWaves][2][32];         // d, dmin of the 32 rows
    __shared__ __attribute__((aligned(16))) float s_part[kNarrowWaves][32][33];     // partial y[n][m]

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 31, h = lane >> 5;
    const int m0 = blockIdx.x * 32;  // rows past M are computed on a copy of row M-1 and not stored
    const int rowsB = SB * kQ8_KBytes;
    // activation rows past N read as zeros (their outputs are not stored)
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(X), (short)0,
                                                                         N * rowsB, kBufferWord3);
    const int vo_code = c * rowsB + 4 + 16 * h;  // chunk 2j + h of row c at + 32 j
    const int vo_sum = c * rowsB + 260 + 16 * h;  // sums 8h .. 8h+7 of row c
    const int vo_dx = c * rowsB;

    // The wave's 32 rows x 144 bytes of a super-block are read as 288
    // row-contiguous 16-byte pieces (consecutive lanes, consecutive pieces of a
    // row) and written to the wave's own LDS region, piece g = 9 r + p at byte
    // 16 g, where each lane then reads its row's header and nibble pairs.
    // Lane-per-row 16-byte loads touch 32 rows per instruction and cost the
    // texture path more: 13.7-14.3 us against 12.5-12.8 us at 14336x4096,
    // N = 4 and 8 (measured on MI355X).
    __shared__ __attribute__((aligned(16))) uint8_t s_wt[kNarrowWaves][5 * 64 * 16];
    uint8_t* const swt = s_wt[wave];
    const int64_t rowW = (int64_t)SB * kQ4_KBytes;
    struct Stage {
        u32x4 wp[5];
        u32x4 xa[8], bsum;
        uint32_t dx;
    };
    auto load = [&](Stage& st, int sb) {
        sb = min(sb, SB - 1);
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int g = min(64 * i + lane, 287), r = g / 9, pc = g - 9 * r;
            st.wp[i] = *reinterpret_cast<const u32x4*>(W + (int64_t)min(m0 + r, M - 1) * rowW +
                                                        (int64_t)sb * kQ4_KBytes + 16 * pc);
        }
        const int so = sb * kQ8_KBytes;
#pragma unroll
        for (int j = 0; j < 8; ++j) st.xa[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, vo_code + 32 * j, so, 0);
        st.bsum = __builtin_amdgcn_raw_buffer_load_b128(xr, vo_sum, so, 0);
        st.dx = __builtin_amdgcn_raw_buffer_load_b32(xr, vo_dx, so, 0);
    };

    float yacc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) yacc[r] = 0.f;

    auto compute = [&](const Stage& st) {
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int g = 64 * i + lane;
            if (g < 288) *reinterpret_cast<u32x4*>(swt + 16 * g) = st.wp[i];
        }
        const uint4 hdr = *reinterpret_cast<const uint4*>(swt + c * kQ4_KBytes);
        uint4 wqv[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) wqv[g] = *reinterpret_cast<const uint4*>(swt + c * kQ4_KBytes + 16 + 32 * g + 16 * h);
        const uint32_t sc03 = hdr.y & 0x3F3F3F3Fu, m03 = hdr.z & 0x3F3F3F3Fu;
        const uint32_t sc47 = (hdr.w & 0x0F0F0F0Fu) | ((hdr.y >> 2) & 0x30303030u);
        const uint32_t m47 = ((hdr.w >> 4) & 0x0F0F0F0Fu) | ((hdr.z >> 2) & 0x30303030u);
        if (h == 0) {  // this lane's row's scales, for the lanes whose registers hold that row
            s_d[wave][0][c] = h2f(hdr.x);
            s_d[wave][1][c] = h2f(hdr.x >> 16);
        }
        v16i ahi = {}, alo = {};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint4 qq = wqv[j >> 1];
            const int shift = (j & 1) * 4;
            const uint32_t scw = (j < 4) ? sc03 : sc47;
            const uint32_t sc = (scw >> (8 * (j & 3))) & 0xFF;
            const uint32_t sh = sc >> 3, sl = sc & 7;
            const uint32_t q0 = (qq.x >> shift) & 0x0F0F0F0Fu, q1 = (qq.y >> shift) & 0x0F0F0F0Fu;
            const uint32_t q2 = (qq.z >> shift) & 0x0F0F0F0Fu, q3 = (qq.w >> shift) & 0x0F0F0F0Fu;
            const v4i bh = {(int)mul_bytes(q0, sh), (int)mul_bytes(q1, sh), (int)mul_bytes(q2, sh), (int)mul_bytes(q3, sh)};
            const v4i bl = {(int)mul_bytes(q0, sl), (int)mul_bytes(q1, sl), (int)mul_bytes(q2, sl), (int)mul_bytes(q3, sl)};
            const v4i a = __builtin_bit_cast(v4i, st.xa[j]);
            ahi = __builtin_amdgcn_mfma_i32_32x32x32_i8(bh, a, ahi, 0, 0, 0);
            alo = __builtin_amdgcn_mfma_i32_32x32x32_i8(bl, a, alo, 0, 0, 0);
        }
        // min term: A = mins of the weight rows (K half h: mins 4h..4h+3 twice
        // each), B = the activation rows' 16-wide sums 8h..8h+7
        const uint32_t mw = h ? m47 : m03;
        v8h mins, bs;
        const v8s bi = __builtin_bit_cast(v8s, st.bsum);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            mins[e] = (_Float16)(float)((mw >> (8 * (e >> 1))) & 0xFF);
            bs[e] = (_Float16)bi[e];  // exact: |s| <= 2032
        }
        const v16f amin = __builtin_amdgcn_mfma_f32_32x32x16_f16(mins, bs, (v16f){}, 0, 0, 0);
        const float dx = __uint_as_float(st.dx);
        // y[n][m] += dx_n * (d_m * (8 P_hi + P_lo) - dmin_m * Smin), m = 8(r/4) + 4h + r%4
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const float4 dd = *reinterpret_cast<const float4*>(&s_d[wave][0][8 * qd + 4 * h]);
            const float4 dm = *reinterpret_cast<const float4*>(&s_d[wave][1][8 * qd + 4 * h]);
            const float da[4] = {dd.x, dd.y, dd.z, dd.w}, ma[4] = {dm.x, dm.y, dm.z, dm.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * qd + e;
                const float u = (float)(ahi[r] * 8 + alo[r]);
                const float v = __builtin_fmaf(u, da[e], -(ma[e] * amin[r]));
                yacc[r] = __builtin_fmaf(v, dx, yacc[r]);
            }
        }
    };

    Stage s0, s1;
    int sb = wave;
    load(s0, sb);
    load(s1, sb + kNarrowWaves);
    for (; sb < SB; sb += 2 * kNarrowWaves) {
        compute(s0);
        load(s0, sb + 2 * kNarrowWaves);
        if (sb + kNarrowWaves < SB) compute(s1);
        load(s1, sb + 3 * kNarrowWaves);
    }

    // sum the waves' partial tiles in a fixed order
#pragma unroll
    for (int r = 0; r < 16; ++r) s_part[wave][c][8 * (r >> 2) + 4 * h + (r & 3)] = yacc[r];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 1024 / (64 * kNarrowWaves); ++k) {
        const int idx = tid + 64 * kNarrowWaves * k;
        const int n = idx >> 5, mm = idx & 31;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < kNarrowWaves; ++w) acc += s_part[w][n][mm];
        if (n < N && m0 + mm < M) Y[(int64_t)n * M + m0 + mm] = acc;
    }
}

// N <= 16 with few weight rows (M <= 8192): the same kernel on 16-row tiles,
// twice as many workgroups.  v_mfma_i32_16x16x64_i8 (checked on the
// hardware): lane l gives row l%16 of A and column l%16 of B, k = 16(l/16)
// .. +15 of each 64-value group, and receives column l%16, rows 4(l/16)+i of
// the result; v_mfma_f32_16x16x16_f16 is the same with k = 4(l/16) .. +3.
// With the sub-block scales inside the planes, the four K quarters of a
// 64-value group may come from two sub-blocks.  Lane (r, q) = (l%16, l/16)
// takes, of 64-value group g, the 16 values 64g + 16q ..: the low (q < 2) or
// high (q >= 2) nibbles of qs[32g + 16(q&1) ..], of sub-block 2g + q/2.
template <int kNarrowWaves>
__global__ __launch_bounds__(64 * kNarrowWaves) void gemm_narrow16_q4k_kernel(const uint8_t* __restrict__ W,
                                                                         const uint8_t* __restrict__ X,
                                                                         float* __restrict__ Y, int M, int N,
                                                                         int SB) {
    __shared__ __attribute__((aligned(16))) float s_d[kNarrowWaves][2][16];      // d, dmin of the 16 rows
    __shared__ __attribute__((aligned(16))) float s_part[kNarrowWaves][16][17];  // partial y[n][m]

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, q = lane >> 4;
    const int m0 = blockIdx.x * 16;  // rows past M are computed on a copy of row M-1 and not stored
    const int rowsB = SB * kQ8_KBytes;
    // activation rows past N read as zeros (their outputs are not stored)
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(X), (short)0,
                                                                         N * rowsB, kBufferWord3);
    const int vo_code = r * rowsB + 4 + 16 * q;  // values 64g + 16q .. of row r at + 64 g
    const int vo_sum = r * rowsB + 260 + 8 * q;  // 16-wide sums 4q .. 4q+3 of row r
    const int vo_dx = r * rowsB;
    const int qsoff = 16 + 16 * (q & 1);         // this lane's 16 qs bytes of group g at + 32 g
    const int nsh = (q >> 1) * 4;                // low or high nibbles

    // the wave's 16 rows x 144 bytes of a super-block, staged as in the
    // 32-row kernel (144 pieces; 7.8 -> 5.9 us at 4096x4096, N = 8)
    __shared__ __attribute__((aligned(16))) uint8_t s_wt[kNarrowWaves][3 * 64 * 16];
    uint8_t* const swt = s_wt[wave];
    const int64_t rowW = (int64_t)SB * kQ4_KBytes;
    struct Stage {
        u32x4 wp[3];
        u32x4 xa[4];
        uint32_t bsum[2], dx;
    };
    auto load = [&](Stage& st, int sb) {
        sb = min(sb, SB - 1);
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int g = min(64 * i + lane, 143), rr = g / 9, pc = g - 9 * rr;
            st.wp[i] = *reinterpret_cast<const u32x4*>(W + (int64_t)min(m0 + rr, M - 1) * rowW +
                                                        (int64_t)sb * kQ4_KBytes + 16 * pc);
        }
        const int so = sb * kQ8_KBytes;
#pragma unroll
        for (int g = 0; g < 4; ++g) st.xa[g] = __builtin_amdgcn_raw_buffer_load_b128(xr, vo_code + 64 * g, so, 0);
        const u32x2 bs = __builtin_amdgcn_raw_buffer_load_b64(xr, vo_sum, so, 0);
        st.bsum[0] = bs.x;
        st.bsum[1] = bs.y;
        st.dx = __builtin_amdgcn_raw_buffer_load_b32(xr, vo_dx, so, 0);
    };

    float yacc[4] = {0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const Stage& st) {
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int g = 64 * i + lane;
            if (g < 144) *reinterpret_cast<u32x4*>(swt + 16 * g) = st.wp[i];
        }
        const uint4 hdr = *reinterpret_cast<const uint4*>(swt + r * kQ4_KBytes);
        uint4 wqv[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) wqv[g] = *reinterpret_cast<const uint4*>(swt + r * kQ4_KBytes + qsoff + 32 * g);
        const uint32_t sc03 = hdr.y & 0x3F3F3F3Fu, m03 = hdr.z & 0x3F3F3F3Fu;
        const uint32_t sc47 = (hdr.w & 0x0F0F0F0Fu) | ((hdr.y >> 2) & 0x30303030u);
        const uint32_t m47 = ((hdr.w >> 4) & 0x0F0F0F0Fu) | ((hdr.z >> 2) & 0x30303030u);
        if (q == 0) {  // this lane's row's scales, for the lanes whose registers hold that row
            s_d[wave][0][r] = h2f(hdr.x);
            s_d[wave][1][r] = h2f(hdr.x >> 16);
        }
        v4i ahi = {}, alo = {};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint4 qq = wqv[g];
            const int j = 2 * g + (q >> 1);  // sub-block of this lane's 16 values
            const uint32_t scw = (g < 2) ? sc03 : sc47;
            const uint32_t sc = (scw >> (8 * (j & 3))) & 0xFF;
            const uint32_t sh = sc >> 3, sl = sc & 7;
            const uint32_t q0 = (qq.x >> nsh) & 0x0F0F0F0Fu, q1 = (qq.y >> nsh) & 0x0F0F0F0Fu;
            const uint32_t q2 = (qq.z >> nsh) & 0x0F0F0F0Fu, q3 = (qq.w >> nsh) & 0x0F0F0F0Fu;
            const v4i bh = {(int)mul_bytes(q0, sh), (int)mul_bytes(q1, sh), (int)mul_bytes(q2, sh), (int)mul_bytes(q3, sh)};
            const v4i bl = {(int)mul_bytes(q0, sl), (int)mul_bytes(q1, sl), (int)mul_bytes(q2, sl), (int)mul_bytes(q3, sl)};
            const v4i a = __builtin_bit_cast(v4i, st.xa[g]);
            ahi = __builtin_amdgcn_mfma_i32_16x16x64_i8(bh, a, ahi, 0, 0, 0);
            alo = __builtin_amdgcn_mfma_i32_16x16x64_i8(bl, a, alo, 0, 0, 0);
        }
        // min term: A = mins of the weight rows (slots 4q .. 4q+3 are
        // sub-blocks 2q, 2q, 2q+1, 2q+1), B = the activation rows' sums
        const uint32_t mw = (q < 2) ? m03 : m47;
        const int mi = 2 * (q & 1);  // first of this lane's two mins within mw
        v4h mins, bs;
        mins[0] = mins[1] = (_Float16)(float)((mw >> (8 * mi)) & 0xFF);
        mins[2] = mins[3] = (_Float16)(float)((mw >> (8 * mi + 8)) & 0xFF);
        bs[0] = (_Float16)(float)(int16_t)(st.bsum[0] & 0xFFFF);  // exact: |s| <= 2032
        bs[1] = (_Float16)(float)(int16_t)(st.bsum[0] >> 16);
        bs[2] = (_Float16)(float)(int16_t)(st.bsum[1] & 0xFFFF);
        bs[3] = (_Float16)(float)(int16_t)(st.bsum[1] >> 16);
        const v4f amin = __builtin_amdgcn_mfma_f32_16x16x16f16(mins, bs, (v4f){}, 0, 0, 0);
        const float dx = __uint_as_float(st.dx);
        // y[n][m] += dx_n * (d_m * (8 P_hi + P_lo) - dmin_m * Smin), m = 4q + i
        const float4 dd = *reinterpret_cast<const float4*>(&s_d[wave][0][4 * q]);
        const float4 dm = *reinterpret_cast<const float4*>(&s_d[wave][1][4 * q]);
        const float da[4] = {dd.x, dd.y, dd.z, dd.w}, ma[4] = {dm.x, dm.y, dm.z, dm.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float u = (float)(ahi[i] * 8 + alo[i]);
            const float v = __builtin_fmaf(u, da[i], -(ma[i] * amin[i]));
            yacc[i] = __builtin_fmaf(v, dx, yacc[i]);
        }
    };

    Stage s0, s1;
    int sb = wave;
    load(s0, sb);
    load(s1, sb + kNarrowWaves);
    for (; sb < SB; sb += 2 * kNarrowWaves) {
        compute(s0);
        load(s0, sb + 2 * kNarrowWaves);
        if (sb + kNarrowWaves < SB) compute(s1);
        load(s1, sb + 3 * kNarrowWaves);
    }

    // sum the waves' partial tiles in a fixed order
#pragma unroll
    for (int i = 0; i < 4; ++i) s_part[wave][r][4 * q + i] = yacc[i];
    __syncthreads();
    if (tid < 256) {
        const int n = tid >> 4, mm = tid & 15;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < kNarrowWaves; ++w) acc += s_part[w][n][mm];
        if (n < N && m0 + mm < M) Y[(int64_t)n * M + m0 + mm] = acc;
    }
}

}  // namespace

bool gemm_supported(int wtype) {
    return wtype == QMM_Q4_K || wtype == QMM_Q6_K || wtype == QMM_Q4_0 || wtype == QMM_Q5_0 || wtype == QMM_Q8_0;
}

// Grids up to this many Q4_K tiles (one per CU) split K in two
constexpr int64_t kSplitKMaxTiles = 256;

// Q4_K kernel with TN tiles per wave, W waves per K part, KS K parts (SB %
// KS == 0), WPE waves per SIMD.
template <int TN, int W, int KS, int WPE>
hipError_t launch_q4k(const uint8_t* w, const uint8_t* x, float* y, int64_t M, int64_t N, int SB, hipStream_t s) {
    const int64_t mb = (M + 32 * W - 1) / (32 * W), nb = (N + 32 * TN - 1) / (32 * TN);
    const int64_t groups = (mb * nb + 7) / 8;  // workgroups are dealt to the 8 XCDs in turn
    if (groups * 8 * 64 * W * KS > (int64_t)UINT32_MAX) return hipErrorInvalidConfiguration;
    return launch(gemm_q4k_kernel<TN, W, KS, WPE>, dim3((unsigned)(8 * groups)), dim3(64 * W * KS), 0, s, w, x, y,
                  (int)M, (int)N, SB, (int)mb, (int)nb);
}

hipError_t launch_gemm(int wtype, const void* W, const void* xq, float* y, int64_t M, int64_t N, int64_t K,
                       hipStream_t s) {
    if (!gemm_supported(wtype)) return hipErrorNotSupported;
    const int SB = (int)(K / 256);
    const uint8_t* w = static_cast<const uint8_t*>(W);
    const uint8_t* x = static_cast<const uint8_t*>(xq);
    const int64_t mblocks = (M + 127) / 128;
    // one workgroup of 256 threads per tile; the whole grid must stay within
    // 2^32 work-items
    const int64_t tiles_max = (int64_t)mblocks * ((N + 63) / 64);
    if (8 * ((tiles_max + 7) / 8) * 256 > (int64_t)UINT32_MAX) return hipErrorInvalidConfiguration;
    auto grid = [](int64_t tiles) { return dim3((unsigned)(8 * ((tiles + 7) / 8))); };
    if (wtype == QMM_Q4_0 || wtype == QMM_Q5_0 || wtype == QMM_Q8_0) {
        const int64_t nb = (N + 63) / 64;
        const int NB = (int)(K / 32);
        const dim3 g = grid(mblocks * nb);
        // K split in KS parts (4 KS waves per workgroup) for small grids whose
        // 4-block chunks are full and at least KS in number, so that a SIMD
        // holds four waves: KS = 4 up to 256 tiles, 2 up to 512 (8192x4096,
        // N = 512: Q4_0 68.3 -> 63.9 us); whole chunks otherwise take the
        // row-contiguous weight staging (WC)
        auto run = [&](auto wtc) {
            constexpr int WT = decltype(wtc)::value, KS = kSplitQ32;
            if (mblocks * nb <= kSplitKMaxTiles && NB % 4 == 0 && NB >= 4 * KS)
                return launch(gemm_q32_kernel<WT, KS, true>, g, dim3(256 * KS), 0, s, w, x, y, (int)M, (int)N, NB,
                              (int)mblocks, (int)nb);
            if (mblocks * nb <= 2 * kSplitKMaxTiles && NB % 4 == 0 && NB >= 8)
                return launch(gemm_q32_kernel<WT, 2, true>, g, dim3(512), 0, s, w, x, y, (int)M, (int)N, NB,
                              (int)mblocks, (int)nb);
            if (NB % 4 == 0)
                return launch(gemm_q32_kernel<WT, 1, true>, g, dim3(256), 0, s, w, x, y, (int)M, (int)N, NB,
                              (int)mblocks, (int)nb);
            return launch(gemm_q32_kernel<WT, 1, false>, g, dim3(256), 0, s, w, x, y, (int)M, (int)N, NB,
                          (int)mblocks, (int)nb);
        };
        if (wtype == QMM_Q4_0) return run(std::integral_constant<int, QMM_Q4_0>{});
        if (wtype == QMM_Q5_0) return run(std::integral_constant<int, QMM_Q5_0>{});
        return run(std::integral_constant<int, QMM_Q8_0>{});
    }
    if (wtype == QMM_Q6_K) {
        // weights staged through LDS; up to N = 32 (W read once, bound by
        // streaming W) 32-row activation tiles and 3 waves per SIMD, wider
        // batches 64-row tiles (the registers of one wave per SIMD)
        if (N <= 32) {
            return launch(gemm_q6k_lds_kernel<1, 4, 3>, grid(mblocks), dim3(256), 0, s, w, x, y, (int)M, (int)N, SB,
                          (int)mblocks, 1);
        } else {
            const int64_t nb = (N + 63) / 64;
            // K in two parts: two waves per SIMD instead of one (N = 512:
            // 4096x14336 146 against 167 us, 8192x14336 291 against 340 us;
            // 128256x4096 at N = 64: 206 against 225 us)
            if (SB % 2 == 0)
                return launch(gemm_q6k_lds_kernel<2, 4, 2, 2>, grid(mblocks * nb), dim3(512), 0, s, w, x, y, (int)M,
                              (int)N, SB, (int)mblocks, (int)nb);
            return launch(gemm_q6k_lds_kernel<2, 4, 1>, grid(mblocks * nb), dim3(256), 0, s, w, x, y, (int)M, (int)N,
                          SB, (int)mblocks, (int)nb);
        }
    }
    if (N <= 16 && M <= 8192) {  // 16-row tiles: enough workgroups for every CU
        const int64_t tiles = (M + 15) / 16;
        if (tiles <= 256)
            return launch(gemm_narrow16_q4k_kernel<8>, dim3((unsigned)tiles), dim3(512), 0, s, w, x, y, (int)M,
                               (int)N, SB);
        else
            return launch(gemm_narrow16_q4k_kernel<4>, dim3((unsigned)tiles), dim3(256), 0, s, w, x, y, (int)M,
                               (int)N, SB);
    }
    if (N <= 32) {
        // 8 waves per workgroup (one workgroup per CU) while the row tiles fit
        // in one pass over the CUs; past that, 4 (two workgroups per CU)
        const int64_t tiles = (M + 31) / 32;
        if (tiles <= 256)
            return launch(gemm_narrow_q4k_kernel<8>, dim3((unsigned)tiles), dim3(512), 0, s, w, x, y, (int)M,
                               (int)N, SB);
        else
            return launch(gemm_narrow_q4k_kernel<4>, dim3((unsigned)tiles), dim3(256), 0, s, w, x, y, (int)M,
                               (int)N, SB);
    }
    // Grids of at least 192 workgroups of 256 weight rows x 128 activation
    // rows: 8 waves of 4 tiles each, one workgroup per CU (LDS).  Smaller
    // grids: 128 x 64 tiles with K split between two groups of 4 waves, or,
    // with an odd count of super-blocks, 4-wave workgroups, two per CU.
    const int64_t tiles_wide = ((M + 255) / 256) * ((N + 127) / 128);
    if (tiles_wide >= 192) return launch_q4k<4, 8, 1, 2>(w, x, y, M, N, SB, s);
    if (SB % 2 == 0) return launch_q4k<2, 4, 2, 2>(w, x, y, M, N, SB, s);
    return launch_q4k<2, 4, 1, 2>(w, x, y, M, N, SB, s);
}

}  // namespace qmm
