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
// 1. mfma_z_kernel (r > 0) computes z = alpha (.) (x . V+-) with
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
//    - Each wave's share of the correction, z . U+- over rank words
//      w = slice, slice + S, ..., goes to accumulators of its own; the
//      product's accumulators are scaled by g before the two meet (g P + C,
//      so that y is right for every finite g, g = 0 included).
//    - The waves' sums meet in per-wave LDS slots.  With one K-slice the
//      workgroup stores y; otherwise it stores its slice's partial sums.
//
// 3. mfma_epilogue_kernel (K split in S > 1 slices) sums the slices and
//    stores bf16 (a launch of its own: summing them in the product by the
//    last slice to arrive measured slower).
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
#include <algorithm>
#include <mutex>

#include "biloco_device.h"
#include "biloco_internal.h"

namespace biloco {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// measurement build only: per-wave stamps of the product kernel (slots:
// 0 start, 1 loads issued, 2 z tile counted in, 3 activation decoded, 4 row
// block 0 done, 5 finisher known, 6 finisher done, 7 last row-block slot
// reached, 8 row blocks done, 9 first correction word ready, 10 correction
// done, 11 stored; values: 12 finisher flag, 13 z computed locally)
#ifdef BILOCO_TIMELINE
__device__ uint64_t g_tl_mfma[kTlMaxWorkgroups * 8 * kTlSlots];
#define TLM(pt) BILOCO_TL_AT(g_tl_mfma, pt, __builtin_amdgcn_s_memrealtime())
#define TLMV(pt, v) BILOCO_TL_AT(g_tl_mfma, pt, (uint64_t)(v))
#else
#define TLM(pt) do { } while (0)
#define TLMV(pt, v) do { } while (0)
#endif

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
    uint32_t *zA;               // [W][MB][2 hi/lo][64 lanes][4] bf16 pairs of z
    float *zf;                  // if set: plain fp32 z [M][rpad] as well (separate-launch use)
    uint8_t *qa_codes;          // if set: the z kernel also quantises x (codes, scales)
    uint8_t *qa_scales;
    int rpad;
    int zsplit;                 // 1: the z launch stores its slice partials only, a reduce launch finishes
    // product kernel
    int S, cps, chunks, RB, Gs;
    float *ypart;               // [S][RB][MB][64 lanes][4] (D layout)
    // one launch (z computed by every workgroup at entry)
    uint32_t *epoch;            // workspace header word 0
    uint32_t *seen;             // workspace header flags, one per workgroup
    float *zpt;                 // tile partials of z [ntiles][MB 2][64 lanes][4] (D layout)
    uint64_t *zat;              // z operands as tagged words [W][MB][2 hi/lo][64 lanes][4]
    int P, psteps;              // K-parts per word and K-steps per part
    int ntiles;                 // W P tiles, tile t = part W + word
    int g8;                     // workgroups per XCD that hold a tile (0: tile = workgroup index)
    uint32_t spin_limit;        // bound of a wait on z, in 100 MHz ticks; 0 = compute z locally
    // side-workgroup schedule: the first n_side workgroups compute whole words
    // of z over all of K and stream no rows
    int n_side;
    int side_split;             // 1: a side workgroup per word; 2: per half of K of a word
    uint64_t *zhp;              // first halves' partial z, tagged, [W][MB 16][32] (split 2)
    // z-in-epilogue schedule: the first kZeParts workgroups compute z's
    // K-part partials (zs K-steps each, ze_sub of them staged in LDS at a
    // time), then finish its words; the K-slice epilogue applies them
    int ze_sub;
    int ze_wg;                  // word groups: side workgroup p takes K-part p % (n_side / ze_wg)
                                // of the words of group p / (n_side / ze_wg)
    float4_t *zep;              // partials [kZeParts][W][2 rank halves][MB][64 lanes] (D layout)
    uint32_t *zecnt;            // the side workgroups' arrival counter (zero between calls)
};

// One output element: bf16 into y, or fp32 into yf when the caller asked for it.
__device__ __forceinline__ void store_y(const MfmaParams &p, int64_t idx, float v) {
    if (p.yf) p.yf[idx] = v;
    else p.y[idx] = f32_to_bf16_rne(v);
}

// Workgroup b runs on XCD b mod 8.  This numbering gives XCD x the
// consecutive work indices [x G8, (x + 1) G8) (G8 = grid / 8, rounded down;
// the last grid mod 8 workgroups keep their index), so work that shares an
// input (a K-slice's x or activation) shares one XCD's L2.
__device__ __forceinline__ int xcd_major_index(int b, int grid) {
    const int g8 = grid >> 3;
    return b < 8 * g8 ? (b & 7) * g8 + (b >> 3) : b;
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

// The slices' sum for word w times alpha_i as bf16 high + low parts into
// the correction operand (and plain fp32 z into zf when asked).  Thread
// (mb, l, j) sums one value; lanes j and j + 4 of a group of 8 threads form
// the (index, index + 16) pair of dword j & 3.  COHERENT: the partials were
// written in the same launch (relaxed agent-scope loads); else after a launch
// boundary (plain loads).
constexpr int kZSumBatch = 16;          // slice partials loaded at once
template <int MB, bool COHERENT>
__device__ __forceinline__ void z_finish(const MfmaParams &p, int w, int first = 0, int step = kZThreads) {
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
        const float zz = (i < p.r && m < p.M) ? sum * al : 0.0f;
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
// launch 1: z
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
// alpha_i and stores bf16 high and low parts.
template <int MB>
__global__ void __launch_bounds__(kZThreads) mfma_z_kernel(MfmaParams p) {
    __shared__ float4_t s_acc[kZWaves][MB * 2][64];
    __shared__ float s_t[MB * 16][33];
    __shared__ uint32_t s_last;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = xcd_major_index((int)blockIdx.x, (int)gridDim.x);
    const int w = t % p.W, s = t / p.W;
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
// one launch: z of one word computed by one wave alone (the fallback after
// a bounded wait for the finisher's words ran out; slow, plain loads)
// =====================================================================
constexpr int kZsw = 4;          // z-tile K-steps per wave loaded at once
constexpr int kMaxZParts = 16;   // K-parts per word (the finisher loads them all at once)

// Lane (col = lane % 16, q = lane / 16) builds, per m-block, the correction
// operand words of z[m][32 w + 4 q + j] and z[m][32 w + 4 q + j + 16]
// (m = 16 mb + col), bf16 high and low parts, as the finisher does.
template <int MB>
__device__ __forceinline__ void z_word_local(const MfmaParams &p, int w, int lane, u32x4_t (&zz)[MB][2]) {
    const int col = lane & 15, q = lane >> 4;
    for (int mb = 0; mb < MB; ++mb) {
        const int m = 16 * mb + col;
        float acc[8];
        for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
        if (m < p.M) {
            for (int k = 0; k < p.K; ++k) {
                const float xv = bf16_to_f32(p.x[(int64_t)m * p.K + k]);
                const uint32_t vw = p.v[(int64_t)w * p.K + k];
                for (int j = 0; j < 8; ++j) {
                    const int ii = 4 * q + (j & 3) + 16 * (j >> 2);
                    acc[j] += ((vw >> ii) & 1u) ? -xv : xv;
                }
            }
        }
        for (int j = 0; j < 4; ++j) {
            uint32_t hi[2], lo[2];
            for (int t = 0; t < 2; ++t) {
                const int i = 32 * w + 4 * q + j + 16 * t;
                const float z = (i < p.r && m < p.M) ? acc[j + 4 * t] * bf16_to_f32(p.alpha[i]) : 0.0f;
                hi[t] = f32_to_bf16_rne(z);
                lo[t] = f32_to_bf16_rne(z - bf16_to_f32(hi[t]));
            }
            zz[mb][0][j] = hi[0] | (hi[1] << 16);
            zz[mb][1][j] = lo[0] | (lo[1] << 16);
        }
    }
}

// =====================================================================
// side-workgroup schedule: z by workgroups that stream no rows
// =====================================================================
// Side workgroup b computes the words b, b + n_side, ... of z over all of K
// (x . V+- with bf16 MFMAs, every m), scales them by alpha, splits them
// into bf16 high and low parts in the correction operand's order and
// publishes them as tagged words (value | the call's epoch + 1 << 32).  Its
// waves take the K-steps wave, wave + 8, ..., kSideSteps at a time, and
// meet in LDS.  Side workgroup 0 is also the bookkeeper: it advances the
// epoch once every workgroup of the launch has set its flag.  No side
// workgroup waits for anything but that.
constexpr int kSideSteps = 8;     // K-steps per wave per round of loads
template <int MB>
__device__ __forceinline__ void side_z_workgroup(const MfmaParams &p, float4_t *lds) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const uint32_t ep = ld_u32(p.epoch);
    if (threadIdx.x == 0) st_u32(p.seen + blockIdx.x, ep + 1u);
    const uint32_t tag = ep + 1u;
    const int steps = p.K >> 5;
    const __amdgpu_buffer_rsrc_t r_x = buffer_of(p.x, (int64_t)p.M * p.K * 2);
    float *s_zt = reinterpret_cast<float *>(lds + (size_t)kPWaves * MB * 2 * 64);   // [MB 16][32]
    const int split = p.side_split;
    for (int item = blockIdx.x; item < p.W * split; item += p.n_side) {
        // word w over the K-steps [hs0, hs1): all of K, or half h of it
        const int w = item % p.W, h = item / p.W;
        const int hs0 = h * steps / split, hs1 = (h + 1) * steps / split;
        const __amdgpu_buffer_rsrc_t r_v = buffer_of(p.v + (int64_t)w * p.K, (int64_t)p.K * 4);
        float4_t acc[MB][2];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb][0] = acc[mb][1] = float4_t{0.f, 0.f, 0.f, 0.f};
        for (int st0 = hs0; st0 < hs1; st0 += kPWaves * kSideSteps) {
            u32x4_t xs[kSideSteps][MB], vs[kSideSteps][2];
#pragma unroll
            for (int u = 0; u < kSideSteps; ++u) {
                const int st = st0 + wave + kPWaves * u;
                const bool ok = st < hs1;
                const int k0 = st * 32 + 8 * grp;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const int m = 16 * mb + col;
                    xs[u][mb] = load16(r_x, opaque(ok && m < p.M ? (m * p.K + k0) * 2 : kOob));
                }
                vs[u][0] = load16(r_v, opaque(ok ? k0 * 4 : kOob));
                vs[u][1] = load16(r_v, opaque(ok ? k0 * 4 + 16 : kOob));
            }
            if (st0 == hs0 && item == (int)blockIdx.x) TLM(3);
#pragma unroll
            for (int u = 0; u < kSideSteps; ++u) {
                if (st0 + wave + kPWaves * u < hs1) {
                    const uint32_t vw[8] = {vs[u][0].x, vs[u][0].y, vs[u][0].z, vs[u][0].w,
                                            vs[u][1].x, vs[u][1].y, vs[u][1].z, vs[u][1].w};
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) {
                        const int bit = 16 * ib + col;
                        u32x4_t bv;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            bv[e] = (((vw[2 * e] >> bit) & 1u) << 15) |
                                    (((vw[2 * e + 1] >> bit) & 1u) << 31) | 0x3F803F80u;
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb) acc[mb][ib] = mfma_bf16(xs[u][mb], bv, acc[mb][ib]);
                    }
                }
            }
            if (item == (int)blockIdx.x) {
                if (st0 == hs0) TLM(4);
                else if (st0 == hs0 + kPWaves * kSideSteps) TLM(5);
            }
        }
        // the waves' sums (D layout: m = 16 mb + 4 (l / 16) + e, rank 16 ib + l % 16)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) lds[((size_t)wave * MB * 2 + mb * 2 + ib) * 64 + lane] = acc[mb][ib];
        __syncthreads();
        if (item == (int)blockIdx.x) TLM(6);
        if ((int)threadIdx.x < MB * 128) {
            const int l = threadIdx.x & 63, blk = threadIdx.x >> 6, mb = blk >> 1, ib = blk & 1;
            float4_t v = lds[(size_t)blk * 64 + l];
#pragma unroll
            for (int q = 1; q < kPWaves; ++q) v += lds[((size_t)q * MB * 2 + blk) * 64 + l];
#pragma unroll
            for (int e = 0; e < 4; ++e) s_zt[(16 * mb + 4 * (l >> 4) + e) * 32 + 16 * ib + (l & 15)] = v[e];
        }
        __syncthreads();
        if (split == 2) {
            uint64_t *hp = p.zhp + (size_t)w * MB * 512;
            if (h == 0) {
                // the first half's sums, tagged, for the word's second-half workgroup
                for (int idx = threadIdx.x; idx < MB * 512; idx += kPThreads) st_tagged(hp + idx, s_zt[idx], tag);
                __syncthreads();     // the LDS serves the next item
                continue;
            }
            // second half: add the first half's sums (a bounded wait; past it,
            // each value is summed here over the first half's K-steps)
            const __amdgpu_buffer_rsrc_t r_hp = buffer_of(hp, (int64_t)MB * 512 * 8);
            for (int idx = threadIdx.x; idx < MB * 512; idx += kPThreads) {
                uint64_t a = ld_tagged(r_hp, opaque(idx * 8));
                if ((uint32_t)(a >> 32) != tag && p.spin_limit) {
                    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
                    do {
                        __builtin_amdgcn_s_sleep(1);
                        a = ld_tagged(r_hp, opaque(idx * 8));
                    } while ((uint32_t)(a >> 32) != tag &&
                             __builtin_amdgcn_s_memrealtime() - t0 < (uint64_t)p.spin_limit);
                }
                float first;
                if ((uint32_t)(a >> 32) == tag && p.spin_limit) {
                    first = __uint_as_float((uint32_t)a);
                } else {
                    const int m = idx >> 5, ii = idx & 31;
                    first = 0.0f;
                    if (m < p.M)
                        for (int k = 0; k < hs0 * 32; ++k) {
                            const float xv = bf16_to_f32(p.x[(int64_t)m * p.K + k]);
                            first += ((p.v[(int64_t)w * p.K + k] >> ii) & 1u) ? -xv : xv;
                        }
                }
                s_zt[idx] += first;
            }
            __syncthreads();
        }
#pragma unroll
        for (int idx0 = 0; idx0 < MB * 512; idx0 += kPThreads) {
            const int idx = idx0 + threadIdx.x;
            const int j = idx & 7, l = (idx >> 3) & 63, mb = idx >> 9;
            const int m = 16 * mb + (l & 15), q = l >> 4;
            const int ii = 4 * q + (j & 3) + 16 * (j >> 2);
            const int i = 32 * w + ii;
            const float al = bf16_to_f32(p.alpha[i < p.r ? i : p.r - 1]);
            const float zz = (i < p.r && m < p.M) ? s_zt[m * 32 + ii] * al : 0.0f;
            const uint32_t zh = f32_to_bf16_rne(zz);
            const uint32_t zl = f32_to_bf16_rne(zz - bf16_to_f32(zh));
            const uint32_t oh = __shfl_xor(zh, 4, 64), ol = __shfl_xor(zl, 4, 64);
            if (j < 4) {
                uint64_t *dst = p.zat + ((((size_t)w * MB + mb) * 2) * 64 + l) * 4 + j;
                st_tagged_u32(dst, zh | (oh << 16), tag);
                st_tagged_u32(dst + 64 * 4, zl | (ol << 16), tag);
            }
        }
        __syncthreads();     // the LDS serves the next word
        TLM(2);
    }
    if (blockIdx.x == 0) {
        for (int j = 1 + (int)threadIdx.x; j < (int)gridDim.x; j += kPThreads)
            while (ld_u32(p.seen + j) != ep + 1u) __builtin_amdgcn_s_sleep(2);
        __syncthreads();
        if (threadIdx.x == 0) st_u32(p.epoch, ep + 1u);
    }
}

// =====================================================================
// z-in-epilogue schedule: z by K-part in side workgroups, its correction
// in the K-slice epilogue
// =====================================================================
// Side workgroup p of P (n_side) takes K-steps [p zs, (p + 1) zs) of every
// word: it stages that part of x (A-operand order) and of V's words in LDS,
// ze_sub K-steps at a time, and wave q computes words q, q + 8, ... with
// bf16 MFMAs of x against V's +-1 signs.  The staging pairs the sign bits of
// k and k + 1 of 16 ranks into one dword by a byte permute, once per dword;
// the MFMA loop reads one such dword per lane and word for two K-steps and
// hands it to the lane's 16-lane row by DPP broadcast.  It stores its
// partials (D layout) with 16-byte stores through to the coherence point
// (sc1), counts itself in, and waits (bounded) until all P have; then it
// sums the parts of words p, p + P, ..., scales them by alpha and stores z's
// bf16 high and low parts in the correction operand's order (zA), read by
// the epilogue launch after this one.  A word whose parts did not all arrive
// in time is computed from x and V by the workgroup's wave 0 alone
// (z_word_local: slow, never expected).  The wait polls the arrival counter
// itself, which starts every call at zero: the epilogue launch clears it,
// after the launch boundary, when no side workgroup reads it any more.
// B operand of +-1 signs from four pair dwords held by lanes L0 .. L0 + 3 of
// this lane's 16-lane row (DPP row broadcast): this lane's rank is bit col
// of each half
template <int L0>
__device__ __forceinline__ u32x4_t signs_from_row(uint32_t pv, uint32_t mcol, int col) {
    const uint32_t p0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)pv, 0x150 + L0, 0xF, 0xF, false);
    const uint32_t p1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)pv, 0x151 + L0, 0xF, 0xF, false);
    const uint32_t p2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)pv, 0x152 + L0, 0xF, 0xF, false);
    const uint32_t p3 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)pv, 0x153 + L0, 0xF, 0xF, false);
    const int sh = 15 - col;
    return u32x4_t{((p0 & mcol) << sh) | 0x3F803F80u, ((p1 & mcol) << sh) | 0x3F803F80u,
                   ((p2 & mcol) << sh) | 0x3F803F80u, ((p3 & mcol) << sh) | 0x3F803F80u};
}
constexpr int kZeParts = 32;      // side workgroups (K-parts) at most; a multiple of 8 per shape
constexpr int kZeWordsPerWave = 4;    // r <= 1024: 32 words over 8 waves
constexpr int kZeLoads = 8;           // 16-byte pieces of x, and of V, per thread per staged round
template <int MB>
__device__ void ze_side_workgroup(const MfmaParams &p, float4_t *lds) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int P = p.n_side, Pk = P / p.ze_wg;
    const int part = (int)blockIdx.x % Pk, wgrp = (int)blockIdx.x / Pk;
    const int Wg = (p.W + p.ze_wg - 1) / p.ze_wg, w0 = wgrp * Wg;
    const int nw = max(0, min(Wg, p.W - w0));                  // words of this group
    TLM(0);
    TLMV(14, 1);
    const int steps = p.K >> 5;
    const int st0 = part * p.zsteps;
    const int nst = max(0, min(p.zsteps, steps - st0));
    u32x4_t *s_x = reinterpret_cast<u32x4_t *>(lds);                     // [sub][MB][64]
    // V's bits of a word and K-step, as the B operand's lanes want them:
    // [grp][ib][e] holds ranks 16 ib .. 16 ib + 15 at k = 8 grp + 2 e (low
    // half) and + 1 (high half)
    uint32_t *s_p = reinterpret_cast<uint32_t *>(s_x + (size_t)p.ze_sub * MB * 64);   // [W][sub][32]
    float4_t acc[kZeWordsPerWave][2][MB];
#pragma unroll
    for (int jw = 0; jw < kZeWordsPerWave; ++jw)
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[jw][ib][mb] = float4_t{0.f, 0.f, 0.f, 0.f};
    const __amdgpu_buffer_rsrc_t r_x = buffer_of(p.x, (int64_t)p.M * p.K * 2);
    const __amdgpu_buffer_rsrc_t r_v = buffer_of(p.v, (int64_t)p.W * p.K * 4);
    // this lane's two sign bits of every pair dword (rank col, rank 16 + col)
    const uint32_t mcol = 0x00010001u << col;
    const int nwords = (nw - wave + kPWaves - 1) / kPWaves;     // words of this wave (group-local
                                                                // wave + 8 jw)
    for (int sub0 = 0; sub0 < nst; sub0 += p.ze_sub) {
        const int ns = min(p.ze_sub, nst - sub0);
        const int k00 = (st0 + sub0) * 32;
        if (sub0 > 0) __syncthreads();              // the previous round is consumed
        // every load of the round first (at most kZeLoads 16-byte pieces of x
        // and of V per thread: ze_sub is sized for that), then the LDS stores
        u32x4_t lx[kZeLoads], lv[kZeLoads];
#pragma unroll
        for (int j = 0; j < kZeLoads; ++j) {
            const int idx = (int)threadIdx.x + kPThreads * j;
            const int l = idx & 63, mb = (idx >> 6) % MB, t = idx / (64 * MB);
            const int m = 16 * mb + (l & 15), k0 = k00 + t * 32 + 8 * (l >> 4);
            lx[j] = load16(r_x, opaque(t < ns && m < p.M ? (m * p.K + k0) * 2 : kOob));
            const int w = idx / (ns * 8), j4 = idx - w * (ns * 8);
            lv[j] = load16(r_v, opaque(w < nw ? ((w0 + w) * p.K + k00 + 4 * j4) * 4 : kOob));
        }
#pragma unroll
        for (int j = 0; j < kZeLoads; ++j) {
            const int idx = (int)threadIdx.x + kPThreads * j;
            if (idx < ns * MB * 64) s_x[idx] = lx[j];
            const int w = idx / (ns * 8), j4 = idx - w * (ns * 8);
            if (w < nw) {
                // k = 4 q .. 4 q + 3 of step t: pairs e = 2 h and 2 h + 1 of
                // group q / 2
                const int t = j4 >> 3, q = j4 & 7, gq = q >> 1, h = q & 1;
                uint32_t *dst = s_p + ((size_t)w * p.ze_sub + t) * 32 + gq * 8 + 2 * h;
                *reinterpret_cast<uint2 *>(dst) =
                    uint2{__builtin_amdgcn_perm(lv[j].y, lv[j].x, 0x05040100u),
                          __builtin_amdgcn_perm(lv[j].w, lv[j].z, 0x05040100u)};
                *reinterpret_cast<uint2 *>(dst + 4) =
                    uint2{__builtin_amdgcn_perm(lv[j].y, lv[j].x, 0x07060302u),
                          __builtin_amdgcn_perm(lv[j].w, lv[j].z, 0x07060302u)};
            }
        }
        __syncthreads();
        TLM(1);
        // two K-steps per round of LDS reads: x's A operands of both, and one
        // pair dword per lane and word (lanes col < 8 hold step t's eight,
        // the others step t + 1's), which the row's lanes share by DPP
        // broadcast; read one round ahead of their MFMAs (two register sets)
        struct ZeOps { u32x4_t a[2][MB]; uint32_t pv[kZeWordsPerWave]; };
        auto ld_ops = [&](int t, ZeOps &o) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int ts = min(t + s2, ns - 1);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) o.a[s2][mb] = s_x[(ts * MB + mb) * 64 + lane];
            }
            const int tp = min(t + (col >> 3), ns - 1);
#pragma unroll
            for (int jw = 0; jw < kZeWordsPerWave; ++jw)
                if (jw < nwords)
                    o.pv[jw] = s_p[((size_t)(wave + kPWaves * jw) * p.ze_sub + tp) * 32 + grp * 8 + (col & 7)];
        };
        auto step2 = [&](const ZeOps &o, int t) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                if (s2 == 1 && t + 1 >= ns) break;
#pragma unroll
                for (int jw = 0; jw < kZeWordsPerWave; ++jw) {
                    if (jw < nwords) {
#pragma unroll
                        for (int ib = 0; ib < 2; ++ib) {
                            const u32x4_t bv = s2 == 0 ? (ib == 0 ? signs_from_row<0>(o.pv[jw], mcol, col)
                                                                  : signs_from_row<4>(o.pv[jw], mcol, col))
                                                       : (ib == 0 ? signs_from_row<8>(o.pv[jw], mcol, col)
                                                                  : signs_from_row<12>(o.pv[jw], mcol, col));
#pragma unroll
                            for (int mb = 0; mb < MB; ++mb)
                                acc[jw][ib][mb] = mfma_bf16(o.a[s2][mb], bv, acc[jw][ib][mb]);
                        }
                    }
                }
            }
        };
        ZeOps oa, ob;
        ld_ops(0, oa);
        for (int t = 0; t < ns; t += 4) {
            if (t + 2 < ns) ld_ops(t + 2, ob);
            step2(oa, t);
            if (t + 4 < ns) ld_ops(t + 4, oa);
            if (t + 2 < ns) step2(ob, t + 2);
        }
    }
    TLM(2);
    // this part's partials (16-byte stores through to the coherence point,
    // sc1), then the count
    const __amdgpu_buffer_rsrc_t r_zep = buffer_of(p.zep, (int64_t)kZeParts * p.W * 2 * MB * 64 * 16);
#pragma unroll
    for (int jw = 0; jw < kZeWordsPerWave; ++jw) {
        const int wl = wave + kPWaves * jw, w = w0 + wl;
        if (wl < nw) {
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(u32x4_t, acc[jw][ib][mb]), r_zep,
                        (((((part * p.W + w) * 2 + ib) * MB + mb) * 64) + lane) * 16, 0, kPolicySc1);
        }
    }
    stores_done();
    TLM(3);
    __syncthreads();
    __shared__ uint32_t s_ok;
    if (threadIdx.x == 0) {
        // the counter starts the call at zero (the K-slice sum launch of the
        // previous call cleared it) and only grows during the launch
        bool ok = true;
        if (arrive(p.zecnt) != (uint32_t)(P - 1)) {
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            while (ld_u32(p.zecnt) < (uint32_t)P) {
                if (!p.spin_limit || __builtin_amdgcn_s_memrealtime() - t0 >= (uint64_t)p.spin_limit) {
                    ok = false;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        s_ok = ok ? 1u : 0u;
    }
    __syncthreads();
    TLM(4);
    const bool all_in = s_ok != 0u;
    for (int w = (int)blockIdx.x; w < p.W; w += P) {
        if (!all_in) {
            // fallback: wave 0 computes the word from x and V alone
            if (wave == 0) {
                u32x4_t zz[MB][2];
                z_word_local<MB>(p, w, lane, zz);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        reinterpret_cast<u32x4_t *>(p.zA)[(((size_t)w * MB + mb) * 2 + h) * 64 + lane] = zz[mb][h];
            }
            continue;
        }
        // the parts' sum in D layout: thread t loads float4 t % F (F = 2 MB 64
        // per word) of the parts t / F, t / F + 2, ... (16-byte coherent
        // loads, all requested first), the two halves meet in LDS
        constexpr int F = 2 * MB * 64, NH = kPThreads / F, PPH = kZeParts / NH;
        // (the parts of word w: the K-parts of its group, Pk of them)
        const int f = threadIdx.x % F, h = threadIdx.x / F;
        float4_t pv[PPH];
#pragma unroll
        for (int j = 0; j < PPH; ++j) {
            const int pp = h + NH * j;
            pv[j] = __builtin_bit_cast(float4_t,
                load16_sc1(r_zep, opaque(pp < Pk ? ((pp * p.W + w) * F + f) * 16 : kOob)));
        }
        float4_t sum4 = pv[0];
#pragma unroll
        for (int j = 1; j < PPH; ++j) sum4 += pv[j];
        float4_t *s_red = reinterpret_cast<float4_t *>(lds);      // [NH][F], then the sums [F]
        __syncthreads();                        // (the staging area is free)
        s_red[h * F + f] = sum4;
        __syncthreads();
        if ((int)threadIdx.x < F) {
            float4_t v = s_red[threadIdx.x];
#pragma unroll
            for (int hh = 1; hh < NH; ++hh) v += s_red[hh * F + threadIdx.x];
            s_red[NH * F + threadIdx.x] = v;
        }
        __syncthreads();
        const float *s_dz = reinterpret_cast<const float *>(s_red + NH * F);
        // value (mb, l, j): z[m][ii], m = 16 mb + l % 16, ii = 4 (l / 16) +
        // (j & 3) + 16 (j >> 2); its sum sits at D position (rank half
        // ii / 16, lane ii % 16 + 16 ((m % 16) / 4), element m % 4)
#pragma unroll
        for (int v = 0; v < MB; ++v) {
            const int idx = (int)threadIdx.x + kPThreads * v;
            const int j = idx & 7, l = (idx >> 3) & 63, mb = idx >> 9;
            const int mm = l & 15, m = 16 * mb + mm, q = l >> 4;
            const int ii = 4 * q + (j & 3) + 16 * (j >> 2);
            const int ib = ii >> 4, dl = (ii & 15) + 16 * (mm >> 2), de = mm & 3;
            const float sum = s_dz[((ib * MB + mb) * 64 + dl) * 4 + de];
            const int i = 32 * w + ii;
            const float al = bf16_to_f32(p.alpha[i < p.r ? i : p.r - 1]);
            const float zz = (i < p.r && m < p.M) ? sum * al : 0.0f;
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
    TLM(5);
}

// The K-slice sum with z's correction (z-in-epilogue schedule).  Workgroup
// b takes m-block b % MB of the kEpWaves kEpRbw row blocks from
// kEpWaves kEpRbw (b / MB), kEpRbw per wave: z's operands of that m-block
// (every word's bf16 high and low parts) go to LDS once, then each wave
// sums the slices' partials of its tiles (g times the product, D layout),
// adds z . U+- by bf16 MFMAs of z against U's signs over every word, and
// stores.
constexpr int kEpWaves = 4, kEpRbw = 1;
template <int MB>
__global__ void __launch_bounds__(64 * kEpWaves) mfma_epilogue_zc_kernel(MfmaParams p) {
    extern __shared__ u32x4_t s_za[];             // [W][2 hi/lo][64 lanes]
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, grp = lane >> 4;
    // the side workgroups' counter, for the next call (none of them reads it
    // after the launch boundary)
    if (blockIdx.x == 0 && threadIdx.x == 0) st_u32(p.zecnt, 0u);
    const int mb = blockIdx.x % MB, rb0 = ((blockIdx.x / MB) * kEpWaves + wave) * kEpRbw;
    const int m0 = 16 * mb + 4 * grp;
    // z's operands (at most 32 words: 8 16-byte pieces per thread), U's
    // words of this lane's rows, the slices' partials: all requested first
    constexpr int kZaPieces = 32 * 2 * 64 / (64 * kEpWaves);
    u32x4_t za[kZaPieces];
    const __amdgpu_buffer_rsrc_t r_za = buffer_of(p.zA, (int64_t)p.W * MB * 2 * 64 * 16);
#pragma unroll
    for (int j = 0; j < kZaPieces; ++j) {
        const int idx = (int)threadIdx.x + 64 * kEpWaves * j;
        const int l = idx & 63, h = (idx >> 6) & 1, w = idx >> 7;
        za[j] = load16(r_za, opaque(w < p.W ? ((((w * MB + mb) * 2 + h) * 64) + l) * 16 : kOob));
    }
    const float4_t *ypart = reinterpret_cast<const float4_t *>(p.ypart);
    float4_t v[kEpRbw];
#pragma unroll
    for (int rr = 0; rr < kEpRbw; ++rr) {
        const int rbc = min(rb0 + rr, p.RB - 1);
        v[rr] = float4_t{0.f, 0.f, 0.f, 0.f};
        for (int t0 = 0; t0 < p.S; t0 += kSumBatch) {
            float4_t part[kSumBatch];
#pragma unroll
            for (int tt = 0; tt < kSumBatch; ++tt)
                part[tt] = ypart[((int64_t)min(t0 + tt, p.S - 1) * p.RB + rbc) * MB * 64 + (int64_t)mb * 64 + lane];
#pragma unroll
            for (int tt = 0; tt < kSumBatch; ++tt)
                if (t0 + tt < p.S) v[rr] += part[tt];
        }
    }
    const __amdgpu_buffer_rsrc_t r_u = buffer_of(p.u, (int64_t)p.W * p.N * 4);
    uint32_t uw[kEpRbw][32];
#pragma unroll
    for (int rr = 0; rr < kEpRbw; ++rr) {
        const int nc = min((rb0 + rr) * 16 + col, p.N - 1);
#pragma unroll
        for (int j = 0; j < 32; ++j)
            uw[rr][j] = __builtin_amdgcn_raw_buffer_load_b32(r_u, opaque(j < p.W ? (j * p.N + nc) * 4 : kOob), 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kZaPieces; ++j) {
        const int idx = (int)threadIdx.x + 64 * kEpWaves * j;
        if (idx < p.W * 2 * 64) s_za[idx] = za[j];
    }
    __syncthreads();
    // every word: the MFMAs of z (from LDS) against U's signs
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        if (j < p.W) {
            const u32x4_t zh = s_za[(j * 2 + 0) * 64 + lane], zl = s_za[(j * 2 + 1) * 64 + lane];
#pragma unroll
            for (int rr = 0; rr < kEpRbw; ++rr) {
                const uint32_t t = uw[rr][j];
                const u32x4_t bv = {sign_pair_bf16(t, 4 * grp + 0), sign_pair_bf16(t, 4 * grp + 1),
                                    sign_pair_bf16(t, 4 * grp + 2), sign_pair_bf16(t, 4 * grp + 3)};
                v[rr] = mfma_bf16(zh, bv, v[rr]);
                v[rr] = mfma_bf16(zl, bv, v[rr]);
            }
        }
    }
#pragma unroll
    for (int rr = 0; rr < kEpRbw; ++rr) {
        const int n = (rb0 + rr) * 16 + col;
        if (rb0 + rr < p.RB && n < p.N) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (m0 + e < p.M) store_y(p, (int64_t)(m0 + e) * p.N + n, v[rr][e]);
        }
    }
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
// ZM: 0 = z from the z launch (operands complete at the start); 1 = every
// workgroup computes a tile of z at entry (all-workgroup schedule); 2 = the
// first n_side workgroups compute z (side-workgroup schedule); 3 = the first
// kZeParts workgroups compute z for the epilogue, and the product applies
// no correction (z-in-epilogue schedule).  With 1 and 2 the product applies
// tagged z words after its row blocks.
template <int MB, int RBW, int CPW, int ZM>
__global__ void __launch_bounds__(kPThreads) mfma_product_kernel(MfmaParams p) {
    constexpr bool ONE = ZM == 1 || ZM == 2, TILE = ZM == 1, SIDE = ZM == 2, EPI = ZM == 3;
    constexpr int PPR = scale_pieces(CPW);              // 16-byte scale pieces per row
    constexpr int kPipe = MfmaShape<MB>::kPipe;
    static_assert(!TILE || RBW >= 3, "the z tile's wave sums use the last two row-block slots");
    // LDS: the waves' partial sums [wave][row block][mb][64 lanes], then each
    // wave's block scales of R [wave][row][PPR 16-byte pieces].  One launch:
    // the finisher's sums [512] and its transpose of z [MB 16][32] use the
    // waves' slots of the last row block (free until that row block ends) for
    // two m-blocks, a region of their own after the scales for one.
    extern __shared__ float4_t s_part[];
    u32x4_t *s_sc = reinterpret_cast<u32x4_t *>(s_part + (size_t)kPWaves * RBW * MB * 64);
    float4_t *s_tail = reinterpret_cast<float4_t *>(s_sc + (size_t)kPWaves * RBW * 16 * PPR);
    auto fin_at = [&](int t) -> float4_t & {
        if constexpr (MB == 2) return s_part[((size_t)(t >> 6) * RBW + RBW - 1) * MB * 64 + (t & 63)];
        else return s_tail[t];
    };
    auto zt_at = [&](int m, int i) -> float & {
        if constexpr (MB == 2)
            return reinterpret_cast<float *>(s_part + ((size_t)(m >> 3) * RBW + RBW - 1) * MB * 64 + 64)[(m & 7) * 32 + i];
        else return reinterpret_cast<float *>(s_tail + kPThreads)[m * 32 + i];
    };
    __shared__ uint32_t s_flag;
    // the wave index as a scalar, so that what derives from it (its chunks,
    // its correction words) is known to be the same on every lane and its
    // branches need no lane masks (measured 1-3% faster, except for one
    // m-block in the multi-launch schedule, which took up to 5% longer)
    const int lane = threadIdx.x & 63;
    const int wave = MB == 2 || ZM != 0 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int KH = p.K >> 1, KB = p.K >> 4;
    TLM(0);

    // ---- one launch: the call's epoch, and this workgroup's z tile (word
    // zw, K-part zkp), whose inputs are requested before anything else
    if constexpr (SIDE) {
        if ((int)blockIdx.x < p.n_side) {
            side_z_workgroup<MB>(p, s_part);
            return;
        }
    }
    if constexpr (EPI) {
        if ((int)blockIdx.x < p.n_side) {
            ze_side_workgroup<MB>(p, s_part);
            return;
        }
    }
    uint32_t ep = 0;
    if constexpr (ONE) ep = ld_u32(p.epoch);
    int zt = p.ntiles;
    if constexpr (TILE) {
        const int xq = blockIdx.x & 7, jq = blockIdx.x >> 3;
        zt = p.g8 > 0 ? (jq < p.g8 ? xq * p.g8 + jq : p.ntiles) : (int)blockIdx.x;
    }
    const bool has_tile = TILE && zt < p.ntiles;
    const int zw = has_tile ? zt % p.W : 0, zkp = has_tile ? zt / p.W : 0;
    const int zst0 = zkp * p.psteps;
    const int znst = has_tile ? min(p.psteps, (p.K >> 5) - zst0) : 0;
    constexpr int ZU = TILE ? kZsw : 1;
    u32x4_t zx[ZU][MB], zv[ZU][2];
    const __amdgpu_buffer_rsrc_t r_x = buffer_of(p.x, TILE ? (int64_t)p.M * p.K * 2 : 0);
    const __amdgpu_buffer_rsrc_t r_v = buffer_of(p.v + (TILE ? (int64_t)zw * p.K : 0), TILE ? (int64_t)p.K * 4 : 0);
    // K-steps round * 8 kZsw + wave + 8 u of the part (rows past M and steps
    // past the part read zeros)
    auto z_load = [&](int round) {
#pragma unroll
        for (int u = 0; u < ZU; ++u) {
            const int st = round * kPWaves * ZU + wave + kPWaves * u;
            const bool ok = st < znst;
            const int k0 = (zst0 + st) * 32 + 8 * grp;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int m = 16 * mb + col;
                zx[u][mb] = load16(r_x, opaque(ok && m < p.M ? (m * p.K + k0) * 2 : kOob));
            }
            zv[u][0] = load16(r_v, opaque(ok ? k0 * 4 : kOob));
            zv[u][1] = load16(r_v, opaque(ok ? k0 * 4 + 16 : kOob));
        }
    };
    if (has_tile) z_load(0);
    // slice-major work index: the workgroups of one K-slice share an XCD
    const int wt = SIDE || EPI ? xcd_major_index((int)blockIdx.x - p.n_side, (int)gridDim.x - p.n_side)
                        : xcd_major_index((int)blockIdx.x, (int)gridDim.x);
    const int s = wt / p.Gs, wgi = wt % p.Gs;
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
    const int nws = !EPI && p.W > s ? (p.W - s + p.S - 1) / p.S : 0;

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
    auto u_load = [&](int wi) {
        const int w = s + p.S * wi;
#pragma unroll
        for (int rbl = 0; rbl < RBW; ++rbl) {
            const int n = min((pb + min(rbl, nrb - 1)) * 16 + col, p.N - 1);
            uw[rbl] = p.u[(int64_t)w * p.N + n];
        }
    };
    if (has_corr) {
        if constexpr (ONE) u_load(wave);
        else corr_load(wave);
    }

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
    // CPW x 8) scale bytes, lane PPR row + piece.  (Exact 8-byte loads of each
    // chunk's scales, where K allows them, changed neither the HBM traffic
    // measurably nor the time.)
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

    TLM(1);
    // ---- one launch: the epoch has been read (the bookkeeper may advance it
    // once every workgroup says so); the z tile: x . V+- over the part, every
    // m, the 32 ranks of word zw, by all 8 waves, summed in LDS by wave 0,
    // which stores the tile's partial, waits for the store, and counts the
    // tile in (the last of the P tiles of a word finishes it further down)
    uint32_t zold = 0;
    if constexpr (ONE) {
        if (threadIdx.x == 0) st_u32(p.seen + blockIdx.x, ep + 1u);
        if (has_tile) {
            float4_t zacc[MB][2];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) zacc[mb][0] = zacc[mb][1] = float4_t{0.f, 0.f, 0.f, 0.f};
            auto z_mfma = [&](int round) {
#pragma unroll
                for (int u = 0; u < ZU; ++u) {
                    if (round * kPWaves * ZU + wave + kPWaves * u < znst) {
                        const uint32_t vw[8] = {zv[u][0].x, zv[u][0].y, zv[u][0].z, zv[u][0].w,
                                                zv[u][1].x, zv[u][1].y, zv[u][1].z, zv[u][1].w};
#pragma unroll
                        for (int ib = 0; ib < 2; ++ib) {
                            const int bit = 16 * ib + col;
                            u32x4_t bv;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                bv[e] = (((vw[2 * e] >> bit) & 1u) << 15) |
                                        (((vw[2 * e + 1] >> bit) & 1u) << 31) | 0x3F803F80u;
#pragma unroll
                            for (int mb = 0; mb < MB; ++mb) zacc[mb][ib] = mfma_bf16(zx[u][mb], bv, zacc[mb][ib]);
                        }
                    }
                }
            };
            z_mfma(0);
            for (int round = 1; round * kPWaves * ZU < znst; ++round) {
                z_load(round);
                z_mfma(round);
            }
            float4_t *zslot = s_part + ((size_t)wave * RBW + RBW - 2) * MB * 64 + lane;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) zslot[(mb * 2 + ib) * 64] = zacc[mb][ib];
            __syncthreads();
            if (wave == 0) {
#pragma unroll
                for (int q = 1; q < kPWaves; ++q)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int ib = 0; ib < 2; ++ib)
                            zacc[mb][ib] += s_part[((size_t)q * RBW + RBW - 2) * MB * 64 + (mb * 2 + ib) * 64 + lane];
            }
            __syncthreads();
            if (wave == 0) {
                uint64_t *dst = reinterpret_cast<uint64_t *>(p.zpt) + ((size_t)zt * MB * 2 * 64 + lane) * 2;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) {
                        const float4_t v = zacc[mb][ib];
                        uint64_t *d = dst + (size_t)(mb * 2 + ib) * 64 * 2;
                        __hip_atomic_store(d, ((uint64_t)__float_as_uint(v[1]) << 32) | __float_as_uint(v[0]),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        __hip_atomic_store(d + 1, ((uint64_t)__float_as_uint(v[3]) << 32) | __float_as_uint(v[2]),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                stores_done();
                if (lane == 0) zold = arrive(p.zcnt + zw);
            }
            TLM(2);
        }
    }

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

    // ---- one launch: the finisher of a word (the workgroup whose tile came
    // in last) sums the word's P tile partials, scales by alpha, splits into
    // bf16 high and low parts in the correction operand's layout and
    // publishes them as tagged words.  It learns that it is the last after
    // its first row blocks (the count's reply has come back by then), loads
    // the partials ahead of the next row block's codes and finishes two row
    // blocks later, when they have arrived.
    constexpr int NF4 = MB * 128;                      // float4 per tile partial
    constexpr int FJ = kMaxZParts * NF4 / kPThreads;   // partial float4 per thread
    const int f_idx = threadIdx.x % NF4, f_p0 = threadIdx.x / NF4, f_step = kPThreads / NF4;
    float4_t fin[FJ];
    const __amdgpu_buffer_rsrc_t r_zp =
        buffer_of(p.zpt, TILE ? (int64_t)p.ntiles * NF4 * 16 : 0);
    auto fin_load = [&]() {
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            const int kp = f_p0 + f_step * j;
            const bool ok = kp < p.P;
            fin[j] = __builtin_bit_cast(float4_t,
                load16_sc1(r_zp, opaque(ok ? ((kp * p.W + zw) * NF4 + f_idx) * 16 : kOob)));
        }
    };
    auto finish = [&]() {
        float4_t sum = fin[0];
#pragma unroll
        for (int j = 1; j < FJ; ++j) sum += fin[j];
        fin_at(threadIdx.x) = sum;
        __syncthreads();
        if ((int)threadIdx.x < NF4) {
            float4_t v = fin_at(threadIdx.x);
            for (int gq = 1; gq < f_step; ++gq) v += fin_at(gq * NF4 + threadIdx.x);
            const int l = threadIdx.x & 63, blk = threadIdx.x >> 6, mb = blk >> 1, ib = blk & 1;
#pragma unroll
            for (int e = 0; e < 4; ++e) zt_at(16 * mb + 4 * (l >> 4) + e, 16 * ib + (l & 15)) = v[e];
        }
        __syncthreads();
        const uint32_t tag = ep + 1u;
#pragma unroll
        for (int idx0 = 0; idx0 < MB * 512; idx0 += kPThreads) {
            const int idx = idx0 + threadIdx.x;
            const int j = idx & 7, l = (idx >> 3) & 63, mb = idx >> 9;
            const int m = 16 * mb + (l & 15), q = l >> 4;
            const int ii = 4 * q + (j & 3) + 16 * (j >> 2);
            const int i = 32 * zw + ii;
            const float al = bf16_to_f32(p.alpha[i < p.r ? i : p.r - 1]);
            const float zz = (i < p.r && m < p.M) ? zt_at(m, ii) * al : 0.0f;
            const uint32_t zh = f32_to_bf16_rne(zz);
            const uint32_t zl = f32_to_bf16_rne(zz - bf16_to_f32(zh));
            const uint32_t oh = __shfl_xor(zh, 4, 64), ol = __shfl_xor(zl, 4, 64);
            if (j < 4) {
                uint64_t *dst = p.zat + ((((size_t)zw * MB + mb) * 2) * 64 + l) * 4 + j;
                st_tagged_u32(dst, zh | (oh << 16), tag);
                st_tagged_u32(dst + 64 * 4, zl | (ol << 16), tag);
            }
        }
        // every tile of the word has been counted: ready for the next call
        if (threadIdx.x == 0) st_u32(p.zcnt + zw, 0u);
        // the LDS it used holds row-block sums again from here on
        __syncthreads();
    };
    // (kA <= 1 and kB <= RBW - 2 keep the partials' registers and the
    // prefetched z words, taken at row block RBW - 1, from ever being live
    // at once)
    const int kA = min(1, nrb - 1), kB = min(min(kA + 2, nrb - 1), RBW - 2);
    bool last = false;

    // ---- one launch: this wave's first correction word, as tagged words,
    // requested at the start of the last row-block slot (the last row block
    // of a workgroup with a full range; with side workgroups, requesting them
    // one slot earlier found them not yet published and measured slower)
    constexpr int kZaSlot = RBW - 1;
    u32x4_t za[MB][2][2];
    const __amdgpu_buffer_rsrc_t r_za = buffer_of(p.zat, ONE ? (int64_t)p.W * MB * 2 * 64 * 4 * 8 : 0);
    auto za_load = [&](int wi) {
        const int w = s + p.S * wi;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                    za[mb][h][hf] = load16_sc1(r_za, opaque(((((w * MB + mb) * 2 + h) * 64 + lane) * 4 + 2 * hf) * 8));
    };

    TLM(3);
    // ---- per row block: the correction of this wave's first word, then the
    // wave's chunks of the product, into the wave's own LDS slot
    float4_t *mine = s_part + (size_t)wave * RBW * MB * 64 + lane;
#pragma unroll
    for (int rbl = 0; rbl < RBW; ++rbl) {
        if (lane < 16 * PPR) my_sc[rbl * 16 * PPR + lane] = scv[rbl];
        if constexpr (ONE)
            if (rbl == kZaSlot && has_corr) za_load(wave);
        if (rbl == RBW - 1) TLM(7);
        if (rbl < nrb) {
            float4_t acc[MB][2], cacc[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[mb][0] = acc[mb][1] = cacc[mb] = float4_t{0.f, 0.f, 0.f, 0.f};
            if (!ONE && has_corr) {
                const uint32_t t = uw[rbl];
                const u32x4_t bv = {sign_pair_bf16(t, 4 * grp + 0), sign_pair_bf16(t, 4 * grp + 1),
                                    sign_pair_bf16(t, 4 * grp + 2), sign_pair_bf16(t, 4 * grp + 3)};
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    cacc[mb] = mfma_bf16(zz[mb][0], bv, cacc[mb]);
                    cacc[mb] = mfma_bf16(zz[mb][1], bv, cacc[mb]);
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
            for (int mb = 0; mb < MB; ++mb)
                mine[(rbl * MB + mb) * 64] = p.g * (acc[mb][0] + acc[mb][1]) + cacc[mb];
            if (rbl == 0) TLM(4);
            if constexpr (TILE) {
                if (rbl == kA) {
                    if (threadIdx.x == 0) s_flag = (has_tile && zold == (uint32_t)(p.P - 1)) ? 1u : 0u;
                    __syncthreads();
                    last = s_flag != 0u;
                    TLM(5);
                    TLMV(12, last ? 1 : 0);
                    if (last) fin_load();
                }
                if (rbl == kB && last) {
                    finish();
                    TLM(6);
                }
            }
        }
        // keep each row block's dequantisation next to its MFMAs
        __builtin_amdgcn_sched_barrier(0);
        if (rbl + kPipe < RBW) load_rb(rbl + kPipe);
        __builtin_amdgcn_sched_barrier(0);
    }
    TLM(8);
    // ---- one launch: every correction word of this wave, from the tagged
    // operands (a word not yet published is read again within a bounded
    // time, then computed by the wave itself)
    if constexpr (ONE) {
        const uint32_t tag = ep + 1u;
        for (int wi = wave; wi < nws; wi += kPWaves) {
            const int w = s + p.S * wi;
            if (wi != wave) {
                u_load(wi);
                za_load(wi);
            }
            bool local = p.spin_limit == 0u;
            if (!local) {
                const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
                while (true) {
                    bool ok = true;
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int h = 0; h < 2; ++h)
#pragma unroll
                            for (int hf = 0; hf < 2; ++hf)
                                ok = ok && za[mb][h][hf].y == tag && za[mb][h][hf].w == tag;
                    if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
                    if (__builtin_amdgcn_s_memrealtime() - t0 >= (uint64_t)p.spin_limit) {
                        local = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                    za_load(wi);
                }
            }
            if (wi == wave) {
                TLM(9);
                TLMV(13, local ? 1 : 0);
            }
            u32x4_t zz1[MB][2];
            if (!local) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        zz1[mb][h] = u32x4_t{za[mb][h][0].x, za[mb][h][0].z, za[mb][h][1].x, za[mb][h][1].z};
            } else {
                z_word_local<MB>(p, w, lane, zz1);
            }
#pragma unroll
            for (int rbl = 0; rbl < RBW; ++rbl) {
                if (rbl < nrb) {
                    const uint32_t t = uw[rbl];
                    const u32x4_t bv = {sign_pair_bf16(t, 4 * grp + 0), sign_pair_bf16(t, 4 * grp + 1),
                                        sign_pair_bf16(t, 4 * grp + 2), sign_pair_bf16(t, 4 * grp + 3)};
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        float4_t cacc = mfma_bf16(zz1[mb][0], bv, float4_t{0.f, 0.f, 0.f, 0.f});
                        cacc = mfma_bf16(zz1[mb][1], bv, cacc);
                        mine[(rbl * MB + mb) * 64] += cacc;
                    }
                }
            }
        }
    }
    TLM(10);
    // further correction words of this wave (more than 8 per slice)
    for (int wi = wave + kPWaves; !ONE && wi < nws; wi += kPWaves) {
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
                    if (m0 + e < p.M) store_y(p, (int64_t)(m0 + e) * p.N + n, v[e]);
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
    TLM(11);
    // one launch: workgroup 0 advances the epoch once every workgroup has read
    // it (its flag shows epoch + 1), so no workgroup of this call can see the
    // next value.  Every workgroup sets its flag near its start and none waits
    // for this one, so the wait ends once all have started.
    if constexpr (TILE) {
        if (blockIdx.x == 0) {
            for (int j = 1 + (int)threadIdx.x; j < (int)gridDim.x; j += kPThreads)
                while (ld_u32(p.seen + j) != ep + 1u) __builtin_amdgcn_s_sleep(2);
            __syncthreads();
            if (threadIdx.x == 0) st_u32(p.epoch, ep + 1u);
        }
    }
}

// =====================================================================
// launch 3 (K split in S > 1 slices): sum the slices, bf16
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
        if (m0 + e < p.M) store_y(p, (int64_t)(m0 + e) * p.N + n, v[e]);
}

// =====================================================================
// host side
// =====================================================================
namespace {
struct MfmaPlan {
    int mb, W, zs, zsteps, chunks, S, cps, RB, Gs, grid, rbw, cpw;
    size_t lds;
    // one launch: z tiles (P K-parts of psteps K-steps per word), their
    // placement, whether the shape takes that schedule, and its LDS
    int P, psteps, ntiles, g8;
    bool one_ok;
    size_t lds_one;
    // side-workgroup schedule: side workgroups ahead of the product's, and
    // whether each word's K is split over two of them
    int n_side, side_split;
    // z-in-epilogue schedule: K-steps per side workgroup's part, and per
    // round staged in LDS
    int ze_steps, ze_sub, ze_wg;
    // workspace offsets inside the matrix-core area
    size_t off_zpart, off_za, off_ypart, off_zpt, off_zat, off_zhp, off_zep, bytes;
};

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// Side workgroups of the side-workgroup schedule (a multiple of 8, so that
// the product's XCD-major numbering keeps its XCDs): two per word, each over
// half of K, while 2 W <= 32; else 16, a word each.  The shape qualifies when
// x is small enough for a workgroup to read it once per word and the product
// still fits the remaining CUs.
constexpr int kSideMaxXBytes = 96 * 1024;
int side_split_of(int W) { return 2 * W <= 32 ? 2 : 1; }
int side_count(int W) { return side_split_of(W) == 2 ? (2 * W + 7) / 8 * 8 : 16; }

MfmaPlan mfma_plan(int M, int N, int K, int r, int grid_target = kGridTarget) {
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
    q.Gs = grid_target / q.S;
    if (q.Gs < 1) q.Gs = 1;
    if (q.Gs < (q.RB + large - 1) / large) q.Gs = (q.RB + large - 1) / large;
    if (q.Gs > q.RB) q.Gs = q.RB;
    q.grid = q.Gs * q.S;
    const int rb_wg = (q.RB + q.Gs - 1) / q.Gs;
    q.rbw = rb_wg <= small ? small : large;
    q.lds = (size_t)kPWaves * q.rbw * q.mb * 64 * 16 + (size_t)kPWaves * q.rbw * 16 * 16 * scale_pieces(q.cpw);
    // (two m-blocks: the finisher's LDS lives in the row-block slots)
    q.lds_one = q.lds + (q.mb == 2 ? 0 : (size_t)kPThreads * 16 + (size_t)q.mb * 16 * 32 * 4);
    // one launch: as many K-parts per word as the workgroups hold tiles (at
    // most kMaxZParts); tiles of one part sit on one XCD (workgroup b runs on
    // XCD b % 8), so x's part is fetched once per XCD
    if (q.W > 0) {
        q.g8 = q.grid >= 8 ? q.grid / 8 : 0;
        const int tmax = q.g8 > 0 ? 8 * q.g8 : q.grid;
        int P = tmax / q.W;
        P = P < kMaxZParts ? P : kMaxZParts;
        P = P < steps ? P : steps;
        if (P >= 1) {
            q.psteps = (steps + P - 1) / P;
            q.P = (steps + q.psteps - 1) / q.psteps;
            q.ntiles = q.W * q.P;
        }
        q.one_ok = P >= 1 && q.rbw >= 3 && (int64_t)M * K * 2 <= (int64_t)INT32_MAX - 16 &&
                   q.lds_one <= kLdsLimit;
    }
    // workspace
    size_t off = 0;
    q.off_zpart = off;
    off = align256(off + (size_t)q.zs * q.W * q.mb * 64 * 8 * 4);
    q.off_za = off;
    off += (size_t)q.W * q.mb * 2 * 64 * 16;
    q.off_ypart = off;
    if (q.S > 1) off += (size_t)q.S * q.RB * q.mb * 64 * 16;
    if (q.W > 0) {
        // tagged z operand words (all-workgroup and side-workgroup schedules),
        // then the side workgroups' tagged first-half sums
        off = align256(off);
        q.off_zat = off;
        off += (size_t)q.W * q.mb * 2 * 64 * 4 * 8;
        q.off_zhp = off;
        off += (size_t)q.W * q.mb * 512 * 8;
    }
    if (q.one_ok) {
        off = align256(off);
        q.off_zpt = off;
        off += (size_t)q.ntiles * q.mb * 128 * 16;
    }
    // z-in-epilogue schedule (K split): the side workgroups' z partials
    if (q.W > 0 && q.S > 1) {
        q.ze_steps = (steps + kZeParts - 1) / kZeParts;
        // a staged round: its LDS fits the product's, and its loads kZeLoads
        // 16-byte pieces of x and of V per thread
        const size_t per_step = (size_t)q.mb * 64 * 16 + (size_t)q.W * 32 * 4;
        q.ze_sub = (int)(q.lds / per_step);
        q.ze_sub = std::min(q.ze_sub, q.ze_steps);
        q.ze_sub = std::min(q.ze_sub, kZeLoads * kPThreads / (64 * q.mb));
        q.ze_sub = std::min(q.ze_sub, kZeLoads * kPThreads / (8 * q.W));
        off = align256(off);
        q.off_zep = off;
        off += (size_t)kZeParts * q.W * 2 * q.mb * 64 * 16;
    }
    q.bytes = off > 0 ? align256(off) : 0;
    return q;
}

// Dynamic LDS above 64 KiB must be allowed once per kernel.
template <int MB, int RBW, int CPW, int ZM>
hipError_t allow_lds() {
    static std::once_flag once;
    static hipError_t err = hipSuccess;
    std::call_once(once, [] {
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(&mfma_product_kernel<MB, RBW, CPW, ZM>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsLimit);
    });
    return err;
}
}  // namespace

bool mfma_supported(int M, int N, int K, int r) {
    if (M < 1 || M > 32 || N < 1 || K < 32 || K % 32 != 0 || r < 0) return false;
    return mfma_plan(M, N, K, r).lds <= kLdsLimit;
}

bool mfma_one_supported(int M, int N, int K, int r) {
    if (r < 1 || !mfma_supported(M, N, K, r)) return false;
    return mfma_plan(M, N, K, r).one_ok;
}

namespace {
// the product's plan with room for the side workgroups (grid = q.grid + n_side)
MfmaPlan side_plan(int M, int N, int K, int r) {
    const int W = (r + 31) / 32;
    const int n_side = side_count(W);
    MfmaPlan q = mfma_plan(M, N, K, r, kGridTarget - n_side);
    q.n_side = n_side;
    q.side_split = side_split_of(W);
    return q;
}
}  // namespace

bool mfma_side_supported(int M, int N, int K, int r) {
    if (r < 1 || !mfma_supported(M, N, K, r)) return false;
    if ((int64_t)M * K * 2 > kSideMaxXBytes) return false;
    const MfmaPlan q = side_plan(M, N, K, r);
    // every workgroup resident at once: the product's fit the CUs the side
    // workgroups leave, and the side path's LDS fits the product's
    return q.grid + q.n_side <= kGridTarget && q.lds <= kLdsLimit &&
           (size_t)kPWaves * q.mb * 2 * 64 * 16 + (size_t)q.mb * 16 * 32 * 4 <= q.lds;
}

namespace {
// the product's plan with room for the z-in-epilogue side workgroups
// (kZeParts side workgroups; fewer, in multiples of 8, where the product's
// workgroups would not fit the CUs left)
MfmaPlan ze_plan(int M, int N, int K, int r) {
    MfmaPlan q = mfma_plan(M, N, K, r, kGridTarget - kZeParts);
    q.n_side = kZeParts;
    if (q.grid + q.n_side > kGridTarget && kGridTarget - q.grid >= 8) q.n_side = (kGridTarget - q.grid) / 8 * 8;
    // K-steps per part and per staged round for ze_wg word groups; two
    // groups (each side workgroup a K-part twice as long, of half the words:
    // half the partials to store and to sum) where every wave still has a
    // word and the part still fits one staged round, one round trip under
    // the stream.  Measured: M = 32, K = N = 8192, r = 1024: 21.6-21.9 us
    // per call against 22.3-22.5 us with one group; M = 32, K = 13824,
    // N = 5120, r = 512 would take two rounds: 24.2-24.4 us against
    // 21.4-21.7 us.
    auto steps_for = [&](int wg) {
        const int Pk = q.n_side / wg, Wg = (q.W + wg - 1) / wg;
        q.ze_wg = wg;
        q.ze_steps = (K / 32 + Pk - 1) / Pk;
        const size_t per_step = (size_t)q.mb * 64 * 16 + (size_t)Wg * 32 * 4;
        q.ze_sub = (int)std::min<size_t>(q.lds / per_step, (size_t)q.ze_steps);
        q.ze_sub = std::min(q.ze_sub, kZeLoads * kPThreads / (64 * q.mb));
        q.ze_sub = std::min(q.ze_sub, kZeLoads * kPThreads / (8 * Wg));
    };
    if (q.W >= 2 * kPWaves && q.n_side % 2 == 0) {
        steps_for(2);
        if (q.ze_sub >= q.ze_steps) return q;
    }
    steps_for(1);
    return q;
}
}  // namespace

bool mfma_ze_supported(int M, int N, int K, int r) {
    if (r < 1 || r > 32 * kZeWordsPerWave * kPWaves || !mfma_supported(M, N, K, r)) return false;
    const MfmaPlan q = ze_plan(M, N, K, r);
    // K split (the epilogue launch applies z) and a round of the side
    // workgroups' staging fits the product's LDS.  (No product workgroup
    // waits for anything, so a grid past one workgroup per CU only costs a
    // second round of them; the side workgroups, dispatched first, wait only
    // for one another, within a bound.)
    return q.S > 1 && q.ze_sub >= 1;
}

size_t mfma_ws_bytes(int M, int N, int K, int r) {
    return mfma_supported(M, N, K, r) ? mfma_plan(M, N, K, r).bytes : 0;
}

namespace {
// Parameters and workspace areas of one call (shared by the launchers below).
MfmaParams mfma_params(const GemmArgs &a, const MfmaPlan &q) {
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
        char *ws = static_cast<char *>(a.ws) + (a.ws_is_mfma_area ? 0 : ws_mfma_offset(a.M, a.r));
        p.zpart = reinterpret_cast<float *>(ws + q.off_zpart);
        p.zA = reinterpret_cast<uint32_t *>(ws + q.off_za);
        p.ypart = reinterpret_cast<float *>(ws + q.off_ypart);
    }
    // the z launch's per-word counters sit at a fixed place of the header
    // (r > 0 calls always get a whole workspace)
    if (a.r > 0) p.zcnt = reinterpret_cast<uint32_t *>(static_cast<char *>(a.ws) + kWsZcntOffset);
    p.rpad = rpad32(a.r);
    if (q.W > 0 && q.bytes > 0) {
        char *ws = static_cast<char *>(a.ws) + (a.ws_is_mfma_area ? 0 : ws_mfma_offset(a.M, a.r));
        p.zat = reinterpret_cast<uint64_t *>(ws + q.off_zat);
        p.zhp = reinterpret_cast<uint64_t *>(ws + q.off_zhp);
        p.epoch = reinterpret_cast<uint32_t *>(static_cast<char *>(a.ws) + ws_epoch_offset());
        p.seen = reinterpret_cast<uint32_t *>(static_cast<char *>(a.ws) + ws_seen_offset());
        if (q.one_ok) {
            p.zpt = reinterpret_cast<float *>(ws + q.off_zpt);
            p.P = q.P;
            p.psteps = q.psteps;
            p.ntiles = q.ntiles;
            p.g8 = q.g8;
        }
    }
    if (q.W > 0 && q.S > 1 && q.bytes > 0) {
        char *ws = static_cast<char *>(a.ws) + (a.ws_is_mfma_area ? 0 : ws_mfma_offset(a.M, a.r));
        p.zep = reinterpret_cast<float4_t *>(ws + q.off_zep);
        p.zecnt = reinterpret_cast<uint32_t *>(static_cast<char *>(a.ws) + kWsZeCntOffset);
    }
    static const uint32_t spin = spin_limit_default();
    p.spin_limit = spin;
    return p;
}

// The product launch (and, with K split, the epilogue launch).
template <int ZM>
hipError_t launch_product(const MfmaPlan &q, const MfmaParams &p, hipStream_t stream) {
    const dim3 grid(q.grid + (ZM == 2 || ZM == 3 ? q.n_side : 0)), block(kPThreads);
    const size_t lds = ZM == 1 ? q.lds_one : q.lds;
    constexpr int c1 = MfmaShape<1>::kCpw, c2 = MfmaShape<2>::kCpw;
    constexpr int s1 = MfmaShape<1>::kRbwSmall, l1 = MfmaShape<1>::kRbwLarge;
    constexpr int s2 = MfmaShape<2>::kRbwSmall, l2 = MfmaShape<2>::kRbwLarge;
    constexpr int cw = MfmaShape<1>::kCpwWide, rw = MfmaShape<1>::kRbwWide;
    hipError_t e;
    if (q.mb == 1 && q.cpw == cw) {
        e = allow_lds<1, rw, cw, ZM>();
        if (e == hipSuccess) hipLaunchKernelGGL((mfma_product_kernel<1, rw, cw, ZM>), grid, block, lds, stream, p);
    } else if (q.mb == 1 && q.rbw == s1) {
        e = allow_lds<1, s1, c1, ZM>();
        if (e == hipSuccess) hipLaunchKernelGGL((mfma_product_kernel<1, s1, c1, ZM>), grid, block, lds, stream, p);
    } else if (q.mb == 1) {
        e = allow_lds<1, l1, c1, ZM>();
        if (e == hipSuccess) hipLaunchKernelGGL((mfma_product_kernel<1, l1, c1, ZM>), grid, block, lds, stream, p);
    } else if (q.rbw == s2) {
        e = allow_lds<2, s2, c2, ZM>();
        if (e == hipSuccess) hipLaunchKernelGGL((mfma_product_kernel<2, s2, c2, ZM>), grid, block, lds, stream, p);
    } else {
        e = allow_lds<2, l2, c2, ZM>();
        if (e == hipSuccess) hipLaunchKernelGGL((mfma_product_kernel<2, l2, c2, ZM>), grid, block, lds, stream, p);
    }
    if (e != hipSuccess) return e;
    e = hipGetLastError();
    if (e != hipSuccess || q.S == 1) return e;
    const int items = q.RB * q.mb * 64;
    if (ZM == 3) {
        // the K-slice sum with z's correction: kEpWaves row blocks of one
        // m-block per workgroup, z's operands of that m-block in LDS
        const dim3 eg(q.mb * ((q.RB + kEpWaves * kEpRbw - 1) / (kEpWaves * kEpRbw))), eb(64 * kEpWaves);
        const size_t elds = (size_t)q.W * 2 * 64 * 16;
        if (q.mb == 1)
            hipLaunchKernelGGL(mfma_epilogue_zc_kernel<1>, eg, eb, elds, stream, p);
        else
            hipLaunchKernelGGL(mfma_epilogue_zc_kernel<2>, eg, eb, elds, stream, p);
    } else if (q.mb == 1)
        hipLaunchKernelGGL(mfma_epilogue_kernel<1>, dim3((items + 255) / 256), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(mfma_epilogue_kernel<2>, dim3((items + 255) / 256), dim3(256), 0, stream, p);
    return hipGetLastError();
}
}  // namespace

// The z kernel alone, also storing plain fp32 z at zf (separate-launch use).
hipError_t launch_z_mfma(const GemmArgs &a, float *zf, hipStream_t stream) {
    if (a.r < 1 || !mfma_supported(a.M, a.N, a.K, a.r)) return hipErrorNotSupported;
    const MfmaPlan q = mfma_plan(a.M, a.N, a.K, a.r);
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
    const MfmaPlan q = mfma_plan(a.M, a.N, a.K, a.r);
    MfmaParams p = mfma_params(a, q);
    hipError_t e = hipSuccess;
    if (a.r > 0) {
        // With many K-slices, the z slices store partials only and a reduce
        // launch finishes each word: there a launch boundary costs less than
        // the exchange of partials through a counter inside one launch
        // (measured: 8 and 14 slices gain, 5 loses).
        p.zsplit = (q.zs >= kZSplitMinSlices || q.W > kWsZcntMax) ? 1 : 0;
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
    return launch_product<0>(q, p, stream);
}

// One launch: every workgroup computes one tile of z at entry, the last
// tile of each word finishes it, and the product's workgroups apply the
// finished words after their row blocks (plus the split-K epilogue when K
// is split).
hipError_t launch_gemm_mfma_one(const GemmArgs &a, hipStream_t stream) {
    if (!mfma_one_supported(a.M, a.N, a.K, a.r)) return hipErrorNotSupported;
    const MfmaPlan q = mfma_plan(a.M, a.N, a.K, a.r);
    MfmaParams p = mfma_params(a, q);
    return launch_product<1>(q, p, stream);
}

// Side workgroups: the first side_count(W) workgroups compute z word by word
// while the others stream R; the product applies the tagged words after its
// row blocks (plus the K-slice sum launch when K is split).
hipError_t launch_gemm_mfma_side(const GemmArgs &a, hipStream_t stream) {
    if (!mfma_side_supported(a.M, a.N, a.K, a.r)) return hipErrorNotSupported;
    const MfmaPlan q = side_plan(a.M, a.N, a.K, a.r);
    MfmaParams p = mfma_params(a, q);
    p.n_side = q.n_side;
    p.side_split = q.side_split;
    return launch_product<2>(q, p, stream);
}

// z in side workgroups of the product launch, by K-part; its correction in
// the K-slice epilogue launch (K split only).
hipError_t launch_gemm_mfma_ze(const GemmArgs &a, hipStream_t stream) {
    if (!mfma_ze_supported(a.M, a.N, a.K, a.r)) return hipErrorNotSupported;
    const MfmaPlan q = ze_plan(a.M, a.N, a.K, a.r);
    MfmaParams p = mfma_params(a, q);
    p.n_side = q.n_side;
    p.zsteps = q.ze_steps;
    p.ze_sub = q.ze_sub;
    p.ze_wg = q.ze_wg;
    return launch_product<3>(q, p, stream);
}

#ifdef BILOCO_TIMELINE
extern "C" int biloco_tl_mfma_zero() {
    static uint64_t z[kTlMaxWorkgroups * 8 * kTlSlots];
    return (int)hipMemcpyToSymbol(HIP_SYMBOL(g_tl_mfma), z, sizeof(z), 0, hipMemcpyHostToDevice);
}
extern "C" int biloco_tl_mfma_read(uint64_t *host, int n) {
    if (n < 0 || n > kTlMaxWorkgroups * 8 * kTlSlots) return -1;
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_tl_mfma), (size_t)n * 8, 0, hipMemcpyDeviceToHost);
}
#endif
}  // namespace biloco
