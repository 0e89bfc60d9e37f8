// Matrix-core schedule of the fused product, for any decode batch M <= 32.
//
// BiLoCo README, section "Kernel": y = FP4(x) FP4(R)^T + sum_i alpha_i (x.v_i) u_i
// for decode batches up to 32.  z = alpha (.) (V x) is computed from V's
// packed signs, and z is expanded through U's packed signs into the fp32
// accumulators before the bf16 store.  The pages run the FP4 GEMM on tensor
// cores with the batch padded to 128 rows.  Here, on gfx950 matrix cores, the
// batch is padded to 16 rows (M <= 16) or 32 rows.  The work is one to four
// launches on one stream:
//
// 1. mfma_z_kernel (r > 0) computes z/g = (alpha/g) (.) (x . V+-) with
//    v_mfma_f32_16x16x32_bf16.  The bf16 activation x is exact as an operand;
//    the +-1 operand is built in registers from V's sign words.  Workgroups
//    own (one 32-bit word of V, one K-slice).  With fewer than 8 K-slices the
//    last workgroup to arrive for a word (a counter, never a wait) sums the
//    slices and stores bf16 high + low parts in the register layout of the
//    correction MFMA; from 8 slices on, mfma_zreduce_kernel does that in a
//    launch of its own.
//
// 2. mfma_product_kernel: one workgroup of 8 waves per CU.  Each workgroup
//    owns one K-slice and a range of 16-row blocks of R.
//    - Each wave owns up to three 128-k chunks of the slice.  Its activation
//      tile for them is loaded once and dequantised into registers as exact
//      f16.
//    - Every wave requests its loads of R (raw buffer loads, zeros for
//      out-of-range slots) one or two row blocks ahead of the row block it
//      computes.  Its block scales go through a wave-private LDS window.
//    - Codes are dequantised in registers into the B operand of
//      v_mfma_f32_16x16x32_f16.  One v_cvt_scalef32_pk_f16_fp4 per byte
//      applies the power of two of the E4M3 block scale, and a packed f16
//      multiply applies its mantissa.  Both steps are exact.
//    - Each wave's share of the correction, (z/g) . U+- over rank words
//      w = slice, slice + S, ..., initialises its accumulators.
//    - The waves' sums meet in per-wave LDS slots.  With one K-slice the
//      workgroup stores y; otherwise it stores its slice's partial sums.
//
// 3. mfma_epilogue_kernel (K split in S > 1 slices) sums the slices,
//    multiplies by g and stores bf16 (a launch of its own: summing them in
//    the product by the last slice to arrive measured slower).
//
// MFMA operand layout of the 16x16x32 forms (checked on the device):
//   A[i][k] sits in lane i + 16 (k / 8), element k % 8.
//   B[k][j] sits in lane j + 16 (k / 8), element k % 8.
//   D[i][j] sits in lane j + 16 (i / 4), element i % 4.
// The reduction index k may be any permutation shared by A and B.
//
// K order inside a 128-k chunk: lane group q = lane / 16 holds the 32 k from
// 32 q to 32 q + 31.  These are one 16-byte code load and one 2-byte scale
// load per row.  K-step d of the chunk takes k = 32 q + 8 d + e, e < 8.
#include <mutex>

#include "biloco_device.h"
#include "biloco_internal.h"

namespace biloco {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kZThreads = 512;          // z kernel: 8 waves
constexpr int kZWaves = kZThreads / 64;
constexpr int kZStepsPerWave = 4;       // K-steps (32 k) per wave in the z kernel
constexpr int kPThreads = 512;          // product kernel: 8 waves
constexpr int kPWaves = kPThreads / 64;
constexpr int kChunkK = 128;
constexpr int kGridTarget = 256;        // one workgroup per CU
constexpr size_t kLdsLimit = 160 * 1024 - 1024;

constexpr int kSumBatch = 8;            // K-slice partials of y loaded at once by the epilogue
constexpr int kZSplitMinSlices = 8;     // z slices from which the exchange gets a launch of its own

// Per batch-tile-height tuning (MB m-blocks of 16 rows):
//   kCpw       128-k chunks per wave: the activation tile takes 16 kCpw MB
//              VGPRs, a workgroup covers 8 kCpw chunks of K
//   kRbw*      row blocks per workgroup: every wave holds kRbw x kCpw 16-byte
//              code loads in flight at once
//   kCpwWide, kRbwWide   the whole-K variant for M <= 16 (no K split while
//              8 kCpwWide chunks cover K): fewer row blocks, more chunks
//   kPipe      row blocks whose code loads are in flight ahead of the one
//              being computed
// A wave's scale bytes in a row (CPW x 8) fit a 16-byte-aligned window of
// scale_pieces(CPW) 16-byte pieces.
template <int MB> struct MfmaShape {
    static constexpr int kCpw = 3;
    static constexpr int kRbwSmall = 3;                 // row blocks per workgroup, small variant
    static constexpr int kRbwLarge = MB == 1 ? 8 : 7;   // row blocks per workgroup, large variant
    static constexpr int kCpwWide = 5;
    static constexpr int kRbwWide = 4;
    // row blocks of code loads requested ahead of the arithmetic (measured
    // best: 1 for one m-block, 2 for two; all at once was slower for both)
    static constexpr int kPipe = MB == 1 ? 1 : 2;
};
__host__ __device__ constexpr int scale_pieces(int cpw) { return (cpw * 8 + 14 + 15) / 16; }

struct MfmaParams {
    const uint8_t *a_codes;
    const uint8_t *a_scales;
    const uint16_t *x;
    const uint8_t *w_codes;
    const uint8_t *w_scales;
    const uint32_t *v;
    const uint32_t *u;
    const uint16_t *alpha;
    uint16_t *y;
    float *yf;              // if set: fp32 results here instead of y
    float g;
    int M, N, K, r, W;          // W = ceil(r / 32)
    // z kernel
    int zs, zsteps;             // K-slices and K-steps per slice
    float *zpart;               // [zs][W][MB][64 lanes][8] (correction A-operand order)
    uint32_t *zcnt;             // [W]
    uint32_t *zA;               // [W][MB][2 hi/lo][64 lanes][4] bf16 pairs of z / g
    float *zf;                  // if set: plain fp32 z [M][rpad] as well (separate-launch use)
    uint8_t *qa_codes;          // if set: the z kernel also quantises x (codes, scales)
    uint8_t *qa_scales;
    int rpad;
    int zsplit;                 // 1: the z launch stores its slice partials only, a reduce launch finishes
    // product kernel
    int S, cps, chunks, RB, Gs;
    float *ypart;               // [S][RB][MB][64 lanes][4] (D layout)
};

// One output element: bf16 into y, or fp32 into yf when the caller asked for it.
__device__ __forceinline__ void store_y(const MfmaParams &p, int64_t idx, float v) {
    if (p.yf) p.yf[idx] = v;
    else p.y[idx] = f32_to_bf16_rne(v);
}

__device__ __forceinline__ float4_t mfma_f16(const u32x4_t &a, const u32x4_t &b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ float4_t mfma_bf16(const u32x4_t &a, const u32x4_t &b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ half2_t mantissa_pair(float s) {
    const _Float16 m = (_Float16)__uint_as_float((__float_as_uint(s) & 0x007FFFFFu) | 0x3F800000u);
    return half2_t{m, m};
}
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_scaled(uint32_t w, float s, half2_t m2) {
    const half2_t h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, SEL);
    return __builtin_bit_cast(uint32_t, h * m2);
}
// eight E2M1 codes (element e in nibble e of `codes`) times an E4M3 scale s
// -> eight exact f16 values, element e in half e
__device__ __forceinline__ u32x4_t dequant8(uint32_t codes, float s, half2_t m2) {
    return u32x4_t{fp4x2_scaled<0>(codes, s, m2), fp4x2_scaled<1>(codes, s, m2),
                   fp4x2_scaled<2>(codes, s, m2), fp4x2_scaled<3>(codes, s, m2)};
}
// bits p and p + 16 of t -> bf16 pair (+-1, +-1); bit set means -1
__device__ __forceinline__ uint32_t sign_pair_bf16(uint32_t t, int p) {
    return ((t << (15 - p)) & 0x80008000u) | 0x3F803F80u;
}
// Cross-workgroup hand-off without cache-wide fences.  An agent-scope
// release or acquire fence on gfx950 writes back or invalidates a whole L2
// (buffer_wbl2 / buffer_inv), which costs tens of microseconds when every
// workgroup does it.  Instead, data that another workgroup reads in the same
// launch is written and read with relaxed agent-scope atomics, which are
// coherent per access (sc1).  A producer waits for its own stores to complete
// (s_waitcnt 0) before the workgroup barrier that precedes the counter
// increment.  The counter is a relaxed agent-scope fetch-add.
__device__ __forceinline__ void put(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stores_done() { __builtin_amdgcn_s_waitcnt(0); }
__device__ __forceinline__ uint32_t arrive(uint32_t *cnt) {
    return __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The slices' sum for word w times alpha_i / g as bf16 high + low parts into
// the correction operand (and plain fp32 z into zf when asked).  Thread
// (mb, l, j) sums one value; lanes j and j + 4 of a group of 8 threads form
// the (index, index + 16) pair of dword j & 3.  COHERENT: the partials were
// written in the same launch (relaxed agent-scope loads); else after a launch
// boundary (plain loads).
constexpr int kZSumBatch = 16;          // slice partials loaded at once
template <int MB, bool COHERENT>
__device__ __forceinline__ void z_finish(const MfmaParams &p, int w, int first = 0, int step = kZThreads) {
    const float ginv = 1.0f / p.g;
    for (int idx = first + (int)threadIdx.x; idx < MB * 64 * 8; idx += step) {
        const int j = idx & 7, l = (idx >> 3) & 63, mb = idx >> 9;
        const int m = 16 * mb + (l & 15), q = l >> 4;
        float sum = 0.0f;
        for (int t0 = 0; t0 < p.zs; t0 += kZSumBatch) {
            float part_v[kZSumBatch];
#pragma unroll
            for (int tt = 0; tt < kZSumBatch; ++tt) {
                const int t = min(t0 + tt, p.zs - 1);
                const float *src = p.zpart + ((int64_t)t * p.W + w) * MB * 64 * 8 + idx;
                part_v[tt] = COHERENT ? get(src) : *src;
            }
#pragma unroll
            for (int tt = 0; tt < kZSumBatch; ++tt)
                if (t0 + tt < p.zs) sum += part_v[tt];
        }
        const int i = 32 * w + 4 * q + (j & 3) + 16 * (j >> 2);
        const float al = bf16_to_f32(p.alpha[i < p.r ? i : p.r - 1]);
        const float zz = (i < p.r && m < p.M) ? sum * al * ginv : 0.0f;
        if (p.zf && i < p.r && m < p.M) p.zf[(int64_t)m * p.rpad + i] = sum * al;
        const uint32_t zh = f32_to_bf16_rne(zz);
        const uint32_t zl = f32_to_bf16_rne(zz - bf16_to_f32(zh));
        // pair with the partner thread (j ^ 4) of the same 8-thread group
        const uint32_t oh = __shfl_xor(zh, 4, 64), ol = __shfl_xor(zl, 4, 64);
        if (j < 4) {
            uint16_t *dst = reinterpret_cast<uint16_t *>(p.zA + ((((int64_t)w * MB + mb) * 2) * 64 + l) * 4 + j);
            reinterpret_cast<uint32_t *>(dst)[0] = zh | (oh << 16);
            reinterpret_cast<uint32_t *>(dst)[64 * 4] = zl | (ol << 16);
        }
    }
}

// =====================================================================
// launch 1: z / g
// =====================================================================
// Workgroup (w, s): the 32 indices of word w of V over K-slice s (at most
// 8 kZStepsPerWave K-steps), every row m.  Wave q takes the slice's K-steps
// q, q + 8, ...; it loads all of them first, then runs MB x 2 bf16 MFMAs per
// K-step.  The waves' sums meet in LDS, where the tile is also transposed to
// the A-operand layout of the correction MFMA: lane l of m-block mb holds,
// for m = 16 mb + l % 16 and q = l / 16, the eight values
// z[m][4q + j] (j < 4) and z[m][4q + j - 4 + 16] (j >= 4).  The slice's
// partial goes to the workspace in that layout; the last workgroup to arrive
// for the word (a counter, never a wait) sums the slices, scales by
// alpha_i / g and stores bf16 high and low parts.
template <int MB>
__global__ void __launch_bounds__(kZThreads) mfma_z_kernel(MfmaParams p) {
    __shared__ float4_t s_acc[kZWaves][MB * 2][64];
    __shared__ float s_t[MB * 16][33];
    __shared__ uint32_t s_last;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int w = blockIdx.x % p.W, s = blockIdx.x / p.W;
    // the activation's FP4 quantisation rides along (read by the product)
    if (p.qa_codes) {
        const int64_t nb = (int64_t)p.M * (p.K >> 4);
        for (int64_t blk = (int64_t)blockIdx.x * kZThreads + threadIdx.x; blk < nb;
             blk += (int64_t)gridDim.x * kZThreads)
            quant_act_block(p.x, blk, p.qa_codes, p.qa_scales);
    }
    const int col = lane & 15, grp = lane >> 4;
    const int steps = p.K >> 5;
    const int step0 = s * p.zsteps;
    const int nsteps = min(p.zsteps, steps - step0);
    const uint32_t *vrow = p.v + (int64_t)w * p.K;

    u32x4_t xa[kZStepsPerWave][MB];
    u32x4_t vv[kZStepsPerWave][2];
#pragma unroll
    for (int t = 0; t < kZStepsPerWave; ++t) {
        int st = wave + kZWaves * t;
        st = st < nsteps ? st : nsteps - 1;
        const int k0 = (step0 + st) * 32 + 8 * grp;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int m = 16 * mb + col;
            const int mc = m < p.M ? m : m % p.M;
            xa[t][mb] = *reinterpret_cast<const u32x4_t *>(p.x + (int64_t)mc * p.K + k0);
        }
        vv[t][0] = *reinterpret_cast<const u32x4_t *>(vrow + k0);
        vv[t][1] = *reinterpret_cast<const u32x4_t *>(vrow + k0 + 4);
    }
    float4_t acc[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb][0] = acc[mb][1] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kZStepsPerWave; ++t) {
        if (wave + kZWaves * t < nsteps) {
            const uint32_t vw[8] = {vv[t][0].x, vv[t][0].y, vv[t][0].z, vv[t][0].w,
                                    vv[t][1].x, vv[t][1].y, vv[t][1].z, vv[t][1].w};
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const int b = 16 * ib + col;      // rank index inside word w
                u32x4_t bv;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    bv[e] = (((vw[2 * e] >> b) & 1u) << 15) | (((vw[2 * e + 1] >> b) & 1u) << 31) |
                            0x3F803F80u;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    u32x4_t a = xa[t][mb];
                    if (16 * mb + col >= p.M) a = u32x4_t{0u, 0u, 0u, 0u};
                    acc[mb][ib] = mfma_bf16(a, bv, acc[mb][ib]);
                }
            }
        }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) s_acc[wave][mb * 2 + ib][lane] = acc[mb][ib];
    __syncthreads();
    // waves' sum, D layout (m = 16 mb + 4 (l / 16) + e, i = 16 ib + l % 16) -> s_t[m][i]
    for (int idx = threadIdx.x; idx < MB * 2 * 64; idx += kZThreads) {
        const int l = idx & 63, blk = idx >> 6;
        float4_t v = s_acc[0][blk][l];
#pragma unroll
        for (int q = 1; q < kZWaves; ++q) v += s_acc[q][blk][l];
        const int mb = blk >> 1, ib = blk & 1;
#pragma unroll
        for (int e = 0; e < 4; ++e) s_t[16 * mb + 4 * (l >> 4) + e][16 * ib + (l & 15)] = v[e];
    }
    __syncthreads();
    // this slice's partial in the operand layout: thread (mb, l, j); with a
    // reduce launch to follow, plain stores and nothing more
    float *part = p.zpart + ((int64_t)s * p.W + w) * MB * 64 * 8;
    if (p.zsplit) {
        for (int idx = threadIdx.x; idx < MB * 64 * 8; idx += kZThreads) {
            const int j = idx & 7, l = (idx >> 3) & 63, mb = idx >> 9;
            const int m = 16 * mb + (l & 15), q = l >> 4;
            part[idx] = s_t[m][4 * q + (j & 3) + 16 * (j >> 2)];
        }
        return;
    }
    for (int idx = threadIdx.x; idx < MB * 64 * 8; idx += kZThreads) {
        const int j = idx & 7, l = (idx >> 3) & 63, mb = idx >> 9;
        const int m = 16 * mb + (l & 15), q = l >> 4;
        put(part + idx, s_t[m][4 * q + (j & 3) + 16 * (j >> 2)]);
    }
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) s_last = arrive(p.zcnt + w) == (uint32_t)(p.zs - 1);
    __syncthreads();
    if (!s_last) return;
    z_finish<MB, true>(p, w);
    if (threadIdx.x == 0) p.zcnt[w] = 0u;   // ready for the next call on this workspace
}

// The reduce launch: workgroup (w, part) finishes the kZrThreads values
// [part kZrThreads, (part + 1) kZrThreads) of word w's operand from the
// slice partials, one value per thread.
constexpr int kZrThreads = 256;
template <int MB>
__global__ void __launch_bounds__(kZrThreads) mfma_zreduce_kernel(MfmaParams p) {
    constexpr int parts = MB * 64 * 8 / kZrThreads;
    z_finish<MB, false>(p, blockIdx.x / parts, (blockIdx.x % parts) * kZrThreads, MB * 64 * 8);
}

// =====================================================================
// launch 2: the product
// =====================================================================
// Workgroup (slice s, row-block range).  Wave q owns the chunks
// [q ncs / 8, (q + 1) ncs / 8) of the slice for every row block of the range:
// its activation tile (those chunks, every K-step, every m-block) lives in
// registers for the whole launch, so the stream of R meets no LDS read.
// The range is at most RBW row blocks.  The wave requests its activation
// (codes and scales) first, then the code loads and the block-scale window of
// R kPipe row blocks ahead of the row block it computes (CPW + 1 16-byte
// loads per row block).  A slot with no work
// (row block past the range, chunk past the wave's share) loads zeros
// through an out-of-range buffer offset, so every path issues the same loads
// and the hardware wait counts stay exact.
template <int MB, int RBW, int CPW>
__global__ void __launch_bounds__(kPThreads) mfma_product_kernel(MfmaParams p) {
    constexpr int PPR = scale_pieces(CPW);              // 16-byte scale pieces per row
    constexpr int kPipe = MfmaShape<MB>::kPipe;
    // LDS: the waves' partial sums [wave][row block][mb][64 lanes], then each
    // wave's block scales of R [wave][row][PPR 16-byte pieces]
    extern __shared__ float4_t s_part[];
    u32x4_t *s_sc = reinterpret_cast<u32x4_t *>(s_part + (size_t)kPWaves * RBW * MB * 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int KH = p.K >> 1, KB = p.K >> 4;
    const int s = blockIdx.x % p.S, wgi = blockIdx.x / p.S;
    const int rb_begin = (int)((int64_t)wgi * p.RB / p.Gs);      // Gs row groups of <= RBW blocks
    const int rb_end = (int)((int64_t)(wgi + 1) * p.RB / p.Gs);
    const int c0 = s * p.cps;
    const int ncs = min(p.cps, p.chunks - c0);
    const int wc0 = c0 + wave * ncs / kPWaves;                 // this wave's chunks
    const int cpw = c0 + (wave + 1) * ncs / kPWaves - wc0;     // 0 .. CPW
    const __amdgpu_buffer_rsrc_t r_wc = buffer_of(p.w_codes, (int64_t)p.N * KH);
    // the staged scale windows are 16-byte loads: the last one may cover up to
    // 14 bytes past the array, inside the 16-byte block (and page) that holds
    // its last byte; those bytes are never used
    const __amdgpu_buffer_rsrc_t r_ws = buffer_of(p.w_scales, ((int64_t)p.N * KB + 15) & ~(int64_t)15);
    const __amdgpu_buffer_rsrc_t r_ac = buffer_of(p.a_codes, (int64_t)p.M * KH);
    // (16-byte scale windows, as for R's scales: up to 15 bytes past the
    // array, inside the 16-byte block that holds its last byte)
    const __amdgpu_buffer_rsrc_t r_as = buffer_of(p.a_scales, ((int64_t)p.M * KB + 15) & ~(int64_t)15);

    // ---- activation tile loads (rows >= M, chunks past the wave's share and
    // the K tail read zeros)
    u32x4_t act_c[CPW][MB];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int m = 16 * mb + col, gc = wc0 + c;
            const bool ok = m < p.M && c < cpw && gc * kChunkK + grp * 32 < p.K;
            act_c[c][mb] = load16(r_ac, opaque(ok ? m * KH + gc * 64 + grp * 16 : kOob));
        }
    // its block scales: per m-block one 16-byte load per lane, lane
    // PPR rl + piece taking piece `piece` of row rl's 16-byte-aligned window
    // that holds the wave's CPW x 8 scale bytes (2-byte loads per lane
    // touched 16 rows per instruction for 128 bytes)
    static_assert(16 * PPR <= 64, "one load per lane covers an m-block's scale windows");
    u32x4_t act_sw[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int rl = lane / PPR, piece = lane - rl * PPR, m = 16 * mb + rl;
        const bool ok = rl < 16 && m < p.M && cpw > 0;
        act_sw[mb] = load16(r_as, opaque(ok ? ((m * KB + wc0 * 8) & ~15) + 16 * piece : kOob));
    }

    const int pb = rb_begin, nrb = rb_end - rb_begin;     // 1 .. RBW row blocks

    // correction words of this wave: w = s + S (wave + 8 j)
    const int nws = p.W > s ? (p.W - s + p.S - 1) / p.S : 0;

    // ---- correction operands for the first word of this wave
    u32x4_t zz[MB][2];
    uint32_t uw[RBW];
    auto corr_load = [&](int wi) {
        const int w = s + p.S * wi;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                zz[mb][h] = reinterpret_cast<const u32x4_t *>(p.zA)[(((int64_t)w * MB + mb) * 2 + h) * 64 + lane];
#pragma unroll
        for (int rbl = 0; rbl < RBW; ++rbl) {
            const int n = min((pb + min(rbl, nrb - 1)) * 16 + col, p.N - 1);
            uw[rbl] = p.u[(int64_t)w * p.N + n];
        }
    };
    const bool has_corr = wave < nws;
    if (has_corr) corr_load(wave);

    // ---- code loads of R: the first kPipe row blocks now, each further one
    // once the row block kPipe before it is done.  Issued all at once, the
    // last of them went out only after several microseconds (the memory
    // system takes new requests as old ones return) and no arithmetic could
    // start before; this way the wave computes while its later row blocks
    // are still being requested.  Every index is a constant, so each wait
    // counts exactly the loads issued after the ones it needs.
    u32x4_t cw[RBW][CPW];
    // block scales of R, requested with the row block's codes: per row the
    // 16-byte-aligned window of PPR pieces that holds the wave's (at most
    // CPW x 8) scale bytes, lane PPR row + piece
    u32x4_t scv[RBW];
    auto load_rb = [&](int rbl) {
        {
            const int rl = lane / PPR, piece = lane - rl * PPR, nr = (pb + rbl) * 16 + rl;
            const bool ok = rl < 16 && rbl < nrb && nr < p.N && cpw > 0;
            scv[rbl] = load16(r_ws, opaque(ok ? ((nr * KB + wc0 * 8) & ~15) + 16 * piece : kOob));
        }
        const int n = (pb + rbl) * 16 + col;
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const int gc = wc0 + c;
            const bool ok = rbl < nrb && n < p.N && c < cpw && gc * kChunkK + grp * 32 < p.K;
            cw[rbl][c] = load16(r_wc, opaque(ok ? n * KH + gc * 64 + grp * 16 : kOob));
        }
    };
#pragma unroll
    for (int rbl = 0; rbl < RBW; ++rbl)
        if (rbl < kPipe) load_rb(rbl);
    __builtin_amdgcn_sched_barrier(0);

    // this wave's scale windows go to its own LDS region, row block by row
    // block (no barrier: only this wave reads them)
    u32x4_t *my_sc = s_sc + (size_t)wave * RBW * 16 * PPR;
    // scale pair of chunk c of row block rbl for this lane: bytes 2 grp and
    // 2 grp + 1 of the chunk's 8, shifted by the row's window alignment
    auto scale_pair = [&](int rbl, int c) -> uint32_t {
        const int n = (pb + rbl) * 16 + col;
        const int delta = (n * KB + wc0 * 8) & 15;
        const int byte = (rbl * 16 + col) * (16 * PPR) + delta + c * 8 + grp * 2;
        return *reinterpret_cast<const uint16_t *>(reinterpret_cast<const uint8_t *>(my_sc) + byte);
    };

    // ---- the activation's scale windows, staged in this wave's partial-sum
    // slots (first written after its first row block)
    uint8_t *my_as = reinterpret_cast<uint8_t *>(s_part + (size_t)wave * RBW * MB * 64);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        if (lane < 16 * PPR) reinterpret_cast<u32x4_t *>(my_as)[mb * 64 + lane] = act_sw[mb];

    // ---- dequantise the activation tile (its loads are the oldest in flight)
    u32x4_t act[CPW][4][MB];           // exact f16 A operands, K-step d of chunk c
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            // scale bytes 2 grp and 2 grp + 1 of chunk c of row m; zero where
            // the codes read nothing (the window may hold any byte there)
            const int m = 16 * mb + col, gc = wc0 + c;
            const bool ok = m < p.M && c < cpw && gc * kChunkK + grp * 32 < p.K;
            const int byte = (mb * 64 + col * PPR) * 16 + ((m * KB + wc0 * 8) & 15) + c * 8 + grp * 2;
            const uint32_t sp = ok ? *reinterpret_cast<const uint16_t *>(my_as + byte) : 0u;
            const float s_lo = __builtin_amdgcn_cvt_f32_fp8(sp, 0);
            const float s_hi = __builtin_amdgcn_cvt_f32_fp8(sp, 1);
            const half2_t m_lo = mantissa_pair(s_lo), m_hi = mantissa_pair(s_hi);
#pragma unroll
            for (int d = 0; d < 4; ++d)
                act[c][d][mb] = d < 2 ? dequant8(act_c[c][mb][d], s_lo, m_lo)
                                      : dequant8(act_c[c][mb][d], s_hi, m_hi);
        }

    // ---- per row block: the correction of this wave's first word, then the
    // wave's chunks of the product, into the wave's own LDS slot
    float4_t *mine = s_part + (size_t)wave * RBW * MB * 64 + lane;
#pragma unroll
    for (int rbl = 0; rbl < RBW; ++rbl) {
        if (lane < 16 * PPR) my_sc[rbl * 16 * PPR + lane] = scv[rbl];
        if (rbl < nrb) {
            float4_t acc[MB][2];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb][0] = acc[mb][1] = float4_t{0.f, 0.f, 0.f, 0.f};
            if (has_corr) {
                const uint32_t t = uw[rbl];
                const u32x4_t bv = {sign_pair_bf16(t, 4 * grp + 0), sign_pair_bf16(t, 4 * grp + 1),
                                    sign_pair_bf16(t, 4 * grp + 2), sign_pair_bf16(t, 4 * grp + 3)};
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    acc[mb][0] = mfma_bf16(zz[mb][0], bv, acc[mb][0]);
                    acc[mb][1] = mfma_bf16(zz[mb][1], bv, acc[mb][1]);
                }
            }
#pragma unroll
            for (int c = 0; c < CPW; ++c) {
                if (c < cpw) {
                    const uint32_t sp = scale_pair(rbl, c);
                    const float s_lo = __builtin_amdgcn_cvt_f32_fp8(sp, 0);
                    const float s_hi = __builtin_amdgcn_cvt_f32_fp8(sp, 1);
                    const half2_t m_lo = mantissa_pair(s_lo), m_hi = mantissa_pair(s_hi);
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const u32x4_t bv = d < 2 ? dequant8(cw[rbl][c][d], s_lo, m_lo)
                                                 : dequant8(cw[rbl][c][d], s_hi, m_hi);
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
                            acc[mb][d & 1] = mfma_f16(act[c][d][mb], bv, acc[mb][d & 1]);
                    }
                }
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) mine[(rbl * MB + mb) * 64] = acc[mb][0] + acc[mb][1];
        }
        // keep each row block's dequantisation next to its MFMAs
        __builtin_amdgcn_sched_barrier(0);
        if (rbl + kPipe < RBW) load_rb(rbl + kPipe);
        __builtin_amdgcn_sched_barrier(0);
    }
    // further correction words of this wave (more than 8 per slice)
    for (int wi = wave + kPWaves; wi < nws; wi += kPWaves) {
        corr_load(wi);
#pragma unroll
        for (int rbl = 0; rbl < RBW; ++rbl) {
            if (rbl < nrb) {
                const uint32_t t = uw[rbl];
                const u32x4_t bv = {sign_pair_bf16(t, 4 * grp + 0), sign_pair_bf16(t, 4 * grp + 1),
                                    sign_pair_bf16(t, 4 * grp + 2), sign_pair_bf16(t, 4 * grp + 3)};
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    float4_t cacc = mfma_bf16(zz[mb][0], bv, float4_t{0.f, 0.f, 0.f, 0.f});
                    cacc = mfma_bf16(zz[mb][1], bv, cacc);
                    mine[(rbl * MB + mb) * 64] += cacc;
                }
            }
        }
    }
    __syncthreads();

    // ---- the waves' sums per row block (thread idx: row block, m-block, lane)
    auto wave_sum = [&](int idx) {
        float4_t v = s_part[idx];
#pragma unroll
        for (int q = 1; q < kPWaves; ++q) v += s_part[(size_t)q * RBW * MB * 64 + idx];
        return v;
    };

    // ---- output: direct (one slice), or this slice's partial sums for the
    // epilogue launch (plain stores; the launch boundary makes them visible)
    if (p.S == 1) {
        for (int idx = threadIdx.x; idx < nrb * MB * 64; idx += kPThreads) {
            const int l = idx & 63, mb = (idx >> 6) % MB, rbl = idx / (64 * MB);
            const int n = (pb + rbl) * 16 + (l & 15), m0 = 16 * mb + 4 * (l >> 4);
            const float4_t v = wave_sum(idx);
            if (n < p.N) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (m0 + e < p.M) store_y(p, (int64_t)(m0 + e) * p.N + n, p.g * v[e]);
            }
        }
    } else {
        float4_t *ypart = reinterpret_cast<float4_t *>(p.ypart);
        for (int idx = threadIdx.x; idx < nrb * MB * 64; idx += kPThreads) {
            const int l = idx & 63, mb = (idx >> 6) % MB, rbl = idx / (64 * MB);
            if (16 * mb + 4 * (l >> 4) < p.M)
                ypart[(((int64_t)s * p.RB + pb + rbl) * MB + mb) * 64 + l] = wave_sum(idx);
        }
    }
}

// =====================================================================
// launch 3 (K split in S > 1 slices): sum the slices, times g, bf16
// =====================================================================
// Thread (row block, m-block, lane) holds the D-layout element quadruple
// (m = 16 mb + 4 (lane / 16) + e, n = 16 rb + lane % 16).
template <int MB>
__global__ void __launch_bounds__(256) mfma_epilogue_kernel(MfmaParams p) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= p.RB * MB * 64) return;
    const int l = idx & 63, mb = (idx >> 6) % MB, rb = idx / (64 * MB);
    const int n = rb * 16 + (l & 15), m0 = 16 * mb + 4 * (l >> 4);
    if (m0 >= p.M || n >= p.N) return;
    const float4_t *ypart = reinterpret_cast<const float4_t *>(p.ypart);
    float4_t v = float4_t{0.f, 0.f, 0.f, 0.f};
    for (int t0 = 0; t0 < p.S; t0 += kSumBatch) {
        float4_t part[kSumBatch];
#pragma unroll
        for (int tt = 0; tt < kSumBatch; ++tt)
            part[tt] = ypart[((int64_t)min(t0 + tt, p.S - 1) * p.RB + rb) * MB * 64 + (int64_t)mb * 64 + l];
#pragma unroll
        for (int tt = 0; tt < kSumBatch; ++tt)
            if (t0 + tt < p.S) v += part[tt];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (m0 + e < p.M) store_y(p, (int64_t)(m0 + e) * p.N + n, p.g * v[e]);
}

// =====================================================================
// host side
// =====================================================================
namespace {
struct MfmaPlan {
    int mb, W, zs, zsteps, chunks, S, cps, RB, Gs, grid, rbw, cpw;
    size_t lds;
    // workspace offsets inside the matrix-core area
    size_t off_zpart, off_zcnt, off_za, off_ypart, bytes;
};

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

MfmaPlan mfma_plan(int M, int N, int K, int r) {
    MfmaPlan q{};
    q.mb = M <= 16 ? 1 : 2;
    q.W = (r + 31) / 32;
    // z: K-slices of at most kZWaves x kZStepsPerWave K-steps per word
    const int steps = K / 32;
    if (q.W > 0) {
        const int per = kZWaves * kZStepsPerWave;
        q.zs = (steps + per - 1) / per;
        q.zsteps = (steps + q.zs - 1) / q.zs;
        q.zs = (steps + q.zsteps - 1) / q.zsteps;
    }
    // product: the fewest K-slices whose chunks the 8 waves' activation
    // tiles cover; for one m-block, the whole-K variant when its wider tiles
    // take K in one slice and the narrow ones would not
    q.chunks = (K + kChunkK - 1) / kChunkK;
    q.cpw = q.mb == 1 ? MfmaShape<1>::kCpw : MfmaShape<2>::kCpw;
    const bool wide = q.mb == 1 && q.chunks > kPWaves * q.cpw && q.chunks <= kPWaves * MfmaShape<1>::kCpwWide;
    if (wide) q.cpw = MfmaShape<1>::kCpwWide;
    const int cps_max = kPWaves * q.cpw;
    q.S = (q.chunks + cps_max - 1) / cps_max;
    q.cps = (q.chunks + q.S - 1) / q.S;
    q.S = (q.chunks + q.cps - 1) / q.cps;
    q.RB = (N + 15) / 16;
    // row groups per slice: one workgroup per CU when the range of each fits
    // the large variant, more workgroups (several rounds) otherwise
    const int small = wide ? MfmaShape<1>::kRbwWide : q.mb == 1 ? MfmaShape<1>::kRbwSmall : MfmaShape<2>::kRbwSmall;
    const int large = wide ? MfmaShape<1>::kRbwWide : q.mb == 1 ? MfmaShape<1>::kRbwLarge : MfmaShape<2>::kRbwLarge;
    q.Gs = kGridTarget / q.S;
    if (q.Gs < 1) q.Gs = 1;
    if (q.Gs < (q.RB + large - 1) / large) q.Gs = (q.RB + large - 1) / large;
    if (q.Gs > q.RB) q.Gs = q.RB;
    q.grid = q.Gs * q.S;
    const int rb_wg = (q.RB + q.Gs - 1) / q.Gs;
    q.rbw = rb_wg <= small ? small : large;
    q.lds = (size_t)kPWaves * q.rbw * q.mb * 64 * 16 + (size_t)kPWaves * q.rbw * 16 * 16 * scale_pieces(q.cpw);
    // workspace
    size_t off = 0;
    q.off_zpart = off;
    off += (size_t)q.zs * q.W * q.mb * 64 * 8 * 4;
    q.off_zcnt = off;
    off = align256(off + (size_t)q.W * 4);
    q.off_za = off;
    off += (size_t)q.W * q.mb * 2 * 64 * 16;
    q.off_ypart = off;
    if (q.S > 1) off += (size_t)q.S * q.RB * q.mb * 64 * 16;
    q.bytes = off > 0 ? align256(off) : 0;
    return q;
}

// Dynamic LDS above 64 KiB must be allowed once per kernel.
template <int MB, int RBW, int CPW>
hipError_t allow_lds() {
    static std::once_flag once;
    static hipError_t err = hipSuccess;
    std::call_once(once, [] {
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(&mfma_product_kernel<MB, RBW, CPW>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsLimit);
    });
    return err;
}
}  // namespace

bool mfma_supported(int M, int N, int K, int r) {
    if (M < 1 || M > 32 || N < 1 || K < 32 || K % 32 != 0 || r < 0) return false;
    return mfma_plan(M, N, K, r).lds <= kLdsLimit;
}

size_t mfma_ws_bytes(int M, int N, int K, int r) {
    return mfma_supported(M, N, K, r) ? mfma_plan(M, N, K, r).bytes : 0;
}

namespace {
// Parameters and workspace areas of one call (shared by the launchers below).
MfmaParams mfma_params(const GemmArgs &a, MfmaPlan &q_out) {
    const MfmaPlan q = mfma_plan(a.M, a.N, a.K, a.r);
    q_out = q;
    MfmaParams p{};
    p.a_codes = a.a_codes;
    p.a_scales = a.a_scales;
    p.x = a.x;
    p.w_codes = a.w_codes;
    p.w_scales = a.w_scales;
    p.v = a.v;
    p.u = a.u;
    p.alpha = a.alpha;
    p.y = a.y;
    p.yf = a.yf;
    p.qa_codes = a.qa_codes;
    p.qa_scales = a.qa_scales;
    p.g = a.g;
    p.M = a.M;
    p.N = a.N;
    p.K = a.K;
    p.r = a.r;
    p.W = q.W;
    p.zs = q.zs;
    p.zsteps = q.zsteps;
    p.S = q.S;
    p.cps = q.cps;
    p.chunks = q.chunks;
    p.RB = q.RB;
    p.Gs = q.Gs;
    if (q.bytes > 0) {
        char *ws = static_cast<char *>(a.ws) + ws_mfma_offset(a.M, a.r);
        p.zpart = reinterpret_cast<float *>(ws + q.off_zpart);
        p.zcnt = reinterpret_cast<uint32_t *>(ws + q.off_zcnt);
        p.zA = reinterpret_cast<uint32_t *>(ws + q.off_za);
        p.ypart = reinterpret_cast<float *>(ws + q.off_ypart);
    }
    p.rpad = rpad32(a.r);
    return p;
}
}  // namespace

// The z kernel alone, also storing plain fp32 z at zf (separate-launch use).
hipError_t launch_z_mfma(const GemmArgs &a, float *zf, hipStream_t stream) {
    if (a.r < 1 || !mfma_supported(a.M, a.N, a.K, a.r)) return hipErrorNotSupported;
    MfmaPlan q;
    MfmaParams p = mfma_params(a, q);
    p.zf = zf;
    if (q.mb == 1)
        hipLaunchKernelGGL(mfma_z_kernel<1>, dim3(q.W * q.zs), dim3(kZThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(mfma_z_kernel<2>, dim3(q.W * q.zs), dim3(kZThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_gemm_mfma(const GemmArgs &a, hipStream_t stream) {
    if (!mfma_supported(a.M, a.N, a.K, a.r)) return hipErrorNotSupported;
    MfmaPlan q;
    MfmaParams p = mfma_params(a, q);
    hipError_t e = hipSuccess;
    if (a.r > 0) {
        // With many K-slices, the z slices store partials only and a reduce
        // launch finishes each word: there a launch boundary costs less than
        // the exchange of partials through a counter inside one launch
        // (measured: 8 and 14 slices gain, 5 loses).
        p.zsplit = q.zs >= kZSplitMinSlices ? 1 : 0;
        if (q.mb == 1) {
            hipLaunchKernelGGL(mfma_z_kernel<1>, dim3(q.W * q.zs), dim3(kZThreads), 0, stream, p);
            if (p.zsplit) hipLaunchKernelGGL(mfma_zreduce_kernel<1>, dim3(q.W * 2), dim3(kZrThreads), 0, stream, p);
        } else {
            hipLaunchKernelGGL(mfma_z_kernel<2>, dim3(q.W * q.zs), dim3(kZThreads), 0, stream, p);
            if (p.zsplit) hipLaunchKernelGGL(mfma_zreduce_kernel<2>, dim3(q.W * 4), dim3(kZrThreads), 0, stream, p);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        p.zsplit = 0;
    }
    const dim3 grid(q.grid), block(kPThreads);
    constexpr int c1 = MfmaShape<1>::kCpw, c2 = MfmaShape<2>::kCpw;
    constexpr int s1 = MfmaShape<1>::kRbwSmall, l1 = MfmaShape<1>::kRbwLarge;
    constexpr int s2 = MfmaShape<2>::kRbwSmall, l2 = MfmaShape<2>::kRbwLarge;
    constexpr int cw = MfmaShape<1>::kCpwWide, rw = MfmaShape<1>::kRbwWide;
    if (q.mb == 1 && q.cpw == cw) {
        e = allow_lds<1, rw, cw>();
        if (e == hipSuccess) hipLaunchKernelGGL((mfma_product_kernel<1, rw, cw>), grid, block, q.lds, stream, p);
    } else if (q.mb == 1 && q.rbw == s1) {
        e = allow_lds<1, s1, c1>();
        if (e == hipSuccess) hipLaunchKernelGGL((mfma_product_kernel<1, s1, c1>), grid, block, q.lds, stream, p);
    } else if (q.mb == 1) {
        e = allow_lds<1, l1, c1>();
        if (e == hipSuccess) hipLaunchKernelGGL((mfma_product_kernel<1, l1, c1>), grid, block, q.lds, stream, p);
    } else if (q.rbw == s2) {
        e = allow_lds<2, s2, c2>();
        if (e == hipSuccess) hipLaunchKernelGGL((mfma_product_kernel<2, s2, c2>), grid, block, q.lds, stream, p);
    } else {
        e = allow_lds<2, l2, c2>();
        if (e == hipSuccess) hipLaunchKernelGGL((mfma_product_kernel<2, l2, c2>), grid, block, q.lds, stream, p);
    }
    if (e != hipSuccess) return e;
    e = hipGetLastError();
    if (e != hipSuccess || q.S == 1) return e;
    const int items = q.RB * q.mb * 64;
    if (q.mb == 1)
        hipLaunchKernelGGL(mfma_epilogue_kernel<1>, dim3((items + 255) / 256), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(mfma_epilogue_kernel<2>, dim3((items + 255) / 256), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace biloco
