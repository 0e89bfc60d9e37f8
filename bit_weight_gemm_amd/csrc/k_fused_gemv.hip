// Vector product for decode batches M <= 2 (schedules
// BILOCO_SCHED_UNFUSED, the default, and BILOCO_SCHED_FUSED_GEMV).
//
// BiLoCo README, section "Kernel": y = FP4(x) FP4(R)^T + sum_i alpha_i (x.v_i) u_i;
// z = alpha (.) (V x) comes from the packed signs of V, and the epilogue
// expands z through U's packed signs before the bf16 store.  Designed here
// for gfx950, where at M <= 2 the product is a matrix-vector stream bound
// by HBM:
//
//  * about one workgroup per CU streams R, 8 waves (two per SIMD), every
//    wave owning up to 4 whole rows (full K), so no partial sum crosses a
//    workgroup; lanes stride over the 16-element NVFP4 blocks of a row;
//  * R is dequantised in registers: one v_cvt_scalef32_pk_f16_fp4 per code
//    byte applies the block scale's power of two, the scale's mantissa
//    (1 + m/8) multiplies the block's fp32 partial sum; the products with
//    the exact f16 activation are v_dot2 (f16 x f16 -> fp32);
//  * the FP4 activation is requested first; at small K M every lane loads
//    and decodes its own blocks once its rows of R are requested (no LDS,
//    no barrier before the stream), otherwise the workgroup decodes it into
//    LDS behind one barrier;
//  * z: v_dot2 (bf16) of x against bf16 pairs of +-1 built from V's words,
//    exact products, one workgroup per two indices i over all of K;
//  * the correction multiplies U's signs (bf16 pairs) with z split into bf16
//    high and low parts (about 16 bits of z) and joins the row sum before
//    the one reduction per row and m.
//
// Two forms of the z hand-off:
//  * two launches (the default): z_kernel writes z, already split into its
//    high/low parts in the lane order of the correction, and (in the
//    quantising call) quantises x in workgroups of its own; the product then
//    loads those operands straight into registers;
//  * one launch: the first workgroups also produce z while every workgroup
//    streams R.  Each z value is published as one 64-bit word (fp32 value |
//    epoch << 32) with a relaxed device-scope store and read back with
//    device-scope loads, so data and tag travel together and no fence is
//    needed.  The call's epoch is a plain load at start; every workgroup
//    then writes a "seen" flag, and workgroup 0 advances the epoch at its
//    end once every flag is in.  A consumer's wait for z is bounded: when it
//    runs out the consumer computes the z values itself, so the kernel ends
//    whatever else runs.
#include <type_traits>

#include "biloco_device.h"
#include "biloco_internal.h"

#include <stdlib.h>

namespace biloco {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kGemvThreads = 512;   // 8 waves per workgroup

struct GemvParams {
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
    uint8_t *qa_codes;      // if set: z_kernel also quantises x (codes, scales)
    uint8_t *qa_scales;
    uint32_t *epoch;        // workspace header word 0
    uint32_t *seen;         // workspace header flags, one per workgroup
    uint64_t *zt;           // z as (value | tag << 32), [M][rpad]  (one launch)
    const float *zf;        // z as plain fp32 [M][rpad] from the z kernel (two launches)
    float *zf_out;          // the same area, written by the z kernel
    // z / correction operands per lane, [M][ceil(rpad / 512)][64][4][hi, lo]
    // bf16 pairs (two launches): written by the z kernel when set
    uint32_t *zop_out;
    const uint32_t *zop;
    float g;
    int N, K, r, rpad;
    int rows_per_wg;
    int z_items;            // ceil(r / kZI)
    uint32_t spin_limit;    // bound of a wait on z; 0 = compute z locally at once
};

__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b),
                                  c, false);
}
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}
// Two FP4 codes (byte SEL of w) -> two f16 values times 2^exponent(scale).
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_f16x2(uint32_t w, float scale) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, SEL));
}
// Sign bits at positions p and p+16 of t -> bf16 pair (+-1, +-1): bit set = -1.
__device__ __forceinline__ uint32_t signs_bf16x2(uint32_t t, int p) {
    return ((t << (15 - p)) & 0x80008000u) | 0x3F803F80u;
}
// Mantissa factor (1 + m/8) of a scale's fp32 form: scale = 2^e * factor.
__device__ __forceinline__ float scale_mant(float s) {
    return __uint_as_float((__float_as_uint(s) & 0x007FFFFFu) | 0x3F800000u);
}

__device__ __forceinline__ uint64_t ld_tagged(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_tagged(uint64_t *p, float v, uint32_t tag) {
    const uint64_t w = ((uint64_t)tag << 32) | __float_as_uint(v);
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_u32(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u32(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum of one value over the 8 waves of the workgroup (red: 8 floats).
__device__ __forceinline__ float block_sum8(float v, float *red) {
    const float s = wave_sum_dpp(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    const float t =
        ((red[0] + red[1]) + (red[2] + red[3])) + ((red[4] + red[5]) + (red[6] + red[7]));
    __syncthreads();
    return t;
}

// z for the kZI indices i0.. (bits of one V word) and all MM rows m,
// computed by the whole workgroup over all of K and published with the tag
// (the call's epoch + 1).  The inputs of the first round (V words, x pairs,
// the coefficients) are requested by z_prefetch, early; z_item consumes
// them and runs any further rounds.
constexpr int kZU = 8;   // pairs (k, k+1) per thread per round
constexpr int kZI = 2;   // indices i per z item (two sign bits of one V word)

template <int MM>
struct ZInputs {
    uint2 vv[kZU];
    uint32_t xp[kZU][MM];
    uint32_t al[kZI];
};

template <int MM>
__device__ __forceinline__ void z_load_round(const GemvParams &p, int item, int kp0,
                                             ZInputs<MM> &in) {
    const int w = (item * kZI) >> 5;
    const uint32_t *vrow = p.v + (int64_t)w * p.K;
    const int KP = p.K / 2;
#pragma unroll
    for (int u = 0; u < kZU; ++u) {
        const int kp = kp0 + threadIdx.x + kGemvThreads * u, kc = kp < KP ? kp : KP - 1;
        in.vv[u] = *reinterpret_cast<const uint2 *>(vrow + 2 * kc);
#pragma unroll
        for (int m = 0; m < MM; ++m)
            in.xp[u][m] = *reinterpret_cast<const uint32_t *>(p.x + (int64_t)m * p.K + 2 * kc);
    }
}

template <int MM>
__device__ __forceinline__ void z_prefetch(const GemvParams &p, int item, ZInputs<MM> &in) {
    const int i0 = item * kZI;
#pragma unroll
    for (int i = 0; i < kZI; ++i) {
        const int ii = i0 + i < p.r ? i0 + i : p.r - 1;
        in.al[i] = p.alpha[ii];
    }
    z_load_round<MM>(p, item, 0, in);
}

// The sign-by-x products of one z item, summed per thread.
template <int MM>
__device__ __forceinline__ void z_accumulate(const GemvParams &p, int item, ZInputs<MM> &in, float (&acc)[kZI][MM]) {
    const int i0 = item * kZI, o = i0 & 31;
    const int s = o & 15;                 // bit offset inside the 16-bit half
    const bool high = o >= 16;
#pragma unroll
    for (int i = 0; i < kZI; ++i)
#pragma unroll
        for (int m = 0; m < MM; ++m) acc[i][m] = 0.0f;
    const int KP = p.K / 2;
    for (int kp0 = 0; kp0 < KP; kp0 += kGemvThreads * kZU) {
        if (kp0 > 0) z_load_round<MM>(p, item, kp0, in);
#pragma unroll
        for (int u = 0; u < kZU; ++u) {
            const bool valid = kp0 + (int)threadIdx.x + kGemvThreads * u < KP;
            // t: the 16 sign bits of k in the low half, those of k+1 in the high half
            const uint32_t t = high ? __builtin_amdgcn_perm(in.vv[u].y, in.vv[u].x, 0x07060302u)
                                    : __builtin_amdgcn_perm(in.vv[u].y, in.vv[u].x, 0x05040100u);
#pragma unroll
            for (int i = 0; i < kZI; ++i) {
                const uint32_t sg = signs_bf16x2(t, s + i);
#pragma unroll
                for (int m = 0; m < MM; ++m)
                    acc[i][m] = dot2_bf16(sg, valid ? in.xp[u][m] : 0u, acc[i][m]);
            }
        }
    }
}

// The workgroup sums of a z item, times alpha_i, published with the call's
// epoch + 1: all sums first, then the kZI * MM stores from as many threads,
// with no wait behind them (a store would otherwise hold up the next wait).
template <int MM>
__device__ __forceinline__ void z_publish(const GemvParams &p, int item, const ZInputs<MM> &in,
                          float (&acc)[kZI][MM], uint32_t epoch, float *red) {
    const int i0 = item * kZI;
    float zs[kZI][MM];
#pragma unroll
    for (int i = 0; i < kZI; ++i)
#pragma unroll
        for (int m = 0; m < MM; ++m) zs[i][m] = block_sum8(acc[i][m], red);
    const uint32_t tag = epoch + 1u;
#pragma unroll
    for (int i = 0; i < kZI; ++i)
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            const int ii = i0 + i;
            if ((int)threadIdx.x == 64 * i + m && ii < p.r)
                st_tagged(p.zt + (int64_t)m * p.rpad + ii, zs[i][m] * bf16_to_f32(in.al[i]), tag);
        }
}

// The same item with no barrier (one launch, inside a wave's row section):
// only the first round of inputs (K <= 2 kGemvThreads kZU), each wave's sums
// go to its LDS slot, then a workgroup-scope counter; the wave that arrives
// last adds the slots in wave order (so the result does not depend on the
// order of arrival), publishes, and resets the counter.
template <int MM>
__device__ __forceinline__ void z_item_waves(const GemvParams &p, int item, const ZInputs<MM> &in, uint32_t epoch,
                             float (*slots)[kZI * MM], uint32_t *cnt) {
    const int i0 = item * kZI, o = i0 & 31;
    const int s = o & 15;
    const bool high = o >= 16;
    float acc[kZI][MM];
#pragma unroll
    for (int i = 0; i < kZI; ++i)
#pragma unroll
        for (int m = 0; m < MM; ++m) acc[i][m] = 0.0f;
    const int KP = p.K / 2;
#pragma unroll
    for (int u = 0; u < kZU; ++u) {
        const bool valid = (int)threadIdx.x + kGemvThreads * u < KP;
        const uint32_t t = high ? __builtin_amdgcn_perm(in.vv[u].y, in.vv[u].x, 0x07060302u)
                                : __builtin_amdgcn_perm(in.vv[u].y, in.vv[u].x, 0x05040100u);
#pragma unroll
        for (int i = 0; i < kZI; ++i) {
            const uint32_t sg = signs_bf16x2(t, s + i);
#pragma unroll
            for (int m = 0; m < MM; ++m) acc[i][m] = dot2_bf16(sg, valid ? in.xp[u][m] : 0u, acc[i][m]);
        }
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float v[kZI * MM];
#pragma unroll
    for (int i = 0; i < kZI; ++i)
#pragma unroll
        for (int m = 0; m < MM; ++m) v[i * MM + m] = wave_sum_dpp(acc[i][m]);
    uint32_t old = 0;
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < kZI * MM; ++j) slots[wave][j] = v[j];
        old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != (uint32_t)(kGemvThreads / 64 - 1)) return;
    if (lane < kZI * MM) {
        float sum = 0.0f;
#pragma unroll
        for (int q = 0; q < kGemvThreads / 64; ++q) sum += slots[q][lane];
        const int i = lane / MM, m = lane - i * MM, ii = i0 + i;
        // alpha of index i, selected with constant indices (a register array
        // indexed by a lane-dependent value would go to scratch memory)
        uint32_t al = in.al[0];
#pragma unroll
        for (int c = 1; c < kZI; ++c) al = i == c ? in.al[c] : al;
        if (ii < p.r) st_tagged(p.zt + (int64_t)m * p.rpad + ii, sum * bf16_to_f32(al), epoch + 1u);
    }
    if (lane == 0) *cnt = 0u;
}

// Fallback: z[m][i] for one index, computed by one thread alone (slow; used
// only after a bounded wait ran out).
__device__ float z_local(const GemvParams &p, int m, int i) {
    const uint32_t *vrow = p.v + (int64_t)(i >> 5) * p.K;
    const int b = i & 31;
    float acc = 0.0f;
    for (int k = 0; k < p.K; ++k) {
        const float xv = bf16_to_f32(p.x[(int64_t)m * p.K + k]);
        acc += ((vrow[k] >> b) & 1u) ? -xv : xv;
    }
    return acc * bf16_to_f32(p.alpha[i]);
}

// Rows per wave of the R stream for KBL blocks per lane and MM rows of x:
// a register budget of about 200 VGPRs for the row buffers (3 KBL each), the
// activation (8 KBL MM) and U's words (4 per row).
__host__ __device__ constexpr int gemv_rows_per_wave(int kbl, int mm) {
    return (200 - 8 * kbl * mm) / (3 * kbl + 4) >= 4 ? 4
         : ((200 - 8 * kbl * mm) / (3 * kbl + 4) <= 1 ? 1 : (200 - 8 * kbl * mm) / (3 * kbl + 4));
}

// z in LDS: value (m, i) at m (rpad + rpad / 16) + i + 2 (i / 32).  The two
// spare floats per 32 put the values one read of the correction takes (16
// words apart by 32 indices, 4 lane groups apart by 1) on distinct banks.
__device__ __forceinline__ int zslot(const GemvParams &p, int m, int i) {
    return m * (p.rpad + (p.rpad >> 4)) + i + 2 * (i >> 5);
}

// Correction of the wave's first NR rows: bit pairs (pb, pb + 16),
// pb = lane / 16 + 4 j, of the lane's U words (lane % 16) + 16 q, against z
// (LDS) split into bf16 high + bf16 low parts; added to the per-lane row sums.
template <int MM, int NR, int R, int QMAX>
__device__ __forceinline__ void add_correction(const GemvParams &p, const float *s_z,
                                               const uint32_t (&ul)[QMAX],
                                               float (&part)[R][MM]) {
    const int lane = threadIdx.x & 63;
    const int W = p.rpad >> 5;
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
        if (16 * q >= W) break;
        const int w = (lane & 15) + 16 * q;
        const bool wok = w < W;
        // word w of row rr, from lane 16 rr + w % 16 (which loaded it)
        uint32_t uw[NR];
#pragma unroll
        for (int rr = 0; rr < NR; ++rr) uw[rr] = __shfl(ul[q], 16 * rr + (lane & 15), 64);
        uint32_t zhi[4][MM], zlo[4][MM];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pb = (lane >> 4) + 4 * j;
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                const int i0 = 32 * w + pb, i1 = i0 + 16;
                const float z0 = (wok && i0 < p.r) ? s_z[zslot(p, m, i0)] : 0.0f;
                const float z1 = (wok && i1 < p.r) ? s_z[zslot(p, m, i1)] : 0.0f;
                const uint32_t h0 = __float_as_uint(z0) & 0xFFFF0000u;
                const uint32_t h1 = __float_as_uint(z1) & 0xFFFF0000u;
                const uint32_t l0 = __float_as_uint(z0 - __uint_as_float(h0));
                const uint32_t l1 = __float_as_uint(z1 - __uint_as_float(h1));
                zhi[j][m] = (h0 >> 16) | h1;
                zlo[j][m] = (l0 >> 16) | (l1 & 0xFFFF0000u);
            }
        }
#pragma unroll
        for (int rr = 0; rr < NR; ++rr) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t sg = signs_bf16x2(uw[rr], (lane >> 4) + 4 * j);
#pragma unroll
                for (int m = 0; m < MM; ++m) {
                    part[rr][m] = dot2_bf16(sg, zhi[j][m], part[rr][m]);
                    part[rr][m] = dot2_bf16(sg, zlo[j][m], part[rr][m]);
                }
            }
        }
    }
}

// The same correction with the operands in registers (two launches): zo[q][m]
// holds, for j = 0 .. 3, the high and low bf16 pairs of z at the lane's
// indices (i, i + 16), i = 32 w + lane / 16 + 4 j.
template <int MM, int NR, int R, int QMAX>
__device__ __forceinline__ void add_correction_ops(const GemvParams &p, const uint32_t (&ul)[QMAX],
                                                   const u32x4_t (&zo)[QMAX][MM][2],
                                                   float (&part)[R][MM]) {
    const int lane = threadIdx.x & 63;
    const int W = p.rpad >> 5;
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
        if (16 * q >= W) break;
        uint32_t uw[NR];
#pragma unroll
        for (int rr = 0; rr < NR; ++rr) uw[rr] = __shfl(ul[q], 16 * rr + (lane & 15), 64);
#pragma unroll
        for (int rr = 0; rr < NR; ++rr) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t sg = signs_bf16x2(uw[rr], (lane >> 4) + 4 * j);
#pragma unroll
                for (int m = 0; m < MM; ++m) {
                    const u32x4_t &v = zo[q][m][j >> 1];
                    part[rr][m] = dot2_bf16(sg, v[2 * (j & 1)], part[rr][m]);
                    part[rr][m] = dot2_bf16(sg, v[2 * (j & 1) + 1], part[rr][m]);
                }
            }
        }
    }
}

// ZMODE 0: no correction (r == 0); 1: z produced in this launch by the first
// workgroups and polled through epoch tags; 2: z complete in the workspace
// (written by z_kernel earlier on the same stream).
template <int MM, int KBL, int ZMODE>
__global__ void __launch_bounds__(kGemvThreads) fused_gemv_kernel(GemvParams p) {
    constexpr int R = gemv_rows_per_wave(KBL, MM);
    static_assert(R >= 1 && R <= 4, "the row-count switch covers 1 .. 4 rows per wave");
    constexpr bool has_z = ZMODE != 0;
    constexpr int QMAX = 2;                    // r <= 1024: two rounds of 16 words
    constexpr int ZP = 2 * MM;                 // z values per thread (MM * r <= MM * 1024)
    constexpr int AMAX = (MM * KBL * 64 + kGemvThreads - 1) / kGemvThreads;  // blocks per thread
    __shared__ float s_red[8];
    __shared__ uint32_t s_bcast;
    __shared__ float s_zslots[kGemvThreads / 64][kZI * MM];   // one launch: per-wave z item sums
    __shared__ uint32_t s_zcnt;
    extern __shared__ uint32_t s_dyn[];   // activation f16 pairs [MM][KB][8], then z [MM][rpad]

    // the wave index as a scalar, so that the row count below is one too
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int KB = p.K >> 4, KH = p.K >> 1;
    uint32_t *s_act = s_dyn;
    float *s_z = reinterpret_cast<float *>(s_dyn + (size_t)MM * KB * 8);

    // the call's epoch (one launch): a device-scope load by every thread,
    // requested with the correction inputs (first, it would hold up the
    // activation: the word was last written on another XCD)
    uint32_t ep = 0u;
    if constexpr (ZMODE == 1) {
        // the z item's arrival counter, zeroed before any wave can use it
        if (threadIdx.x == 0) s_zcnt = 0u;
        __syncthreads();
    }

    // rows of this workgroup, spread over its 8 waves (the first get one more)
    const int wg_row0 = blockIdx.x * p.rows_per_wg;
    int wg_rows = p.N - wg_row0;
    wg_rows = wg_rows < 0 ? 0 : (wg_rows > p.rows_per_wg ? p.rows_per_wg : wg_rows);
    const int base = wg_rows >> 3, extra = wg_rows & 7;
    const int nrows = base + (wave < extra ? 1 : 0);
    const int row0 = wg_row0 + wave * base + (wave < extra ? wave : extra);

    // ---- small inputs first.  Requested behind the stream of R, scattered
    // reads come back only once the stream has drained; requested first, they
    // are in hand before any row of R is asked for.
    // 1. the FP4 activation.  lane_act: each lane loads the codes and scales
    // of its own blocks (lane + 64 t) and decodes them in registers once the
    // rows of R are requested, so no barrier and no LDS stand between the
    // start and the stream.  Otherwise the blocks this thread decodes into
    // LDS for the workgroup (clamped addresses).
    // (beyond these sizes: too many registers; one launch also holds its z
    // item's inputs)
    constexpr bool lane_act = KBL * MM <= (ZMODE == 1 ? 6 : 8);
    const int nact = MM * KB;
    uint2 ac[AMAX];
    uint32_t asb[AMAX];
    uint2 lac[lane_act ? KBL : 1][MM];
    uint32_t las[lane_act ? KBL : 1][MM];
    if constexpr (lane_act) {
        // scales as the aligned 4-byte word holding the lane's byte (a byte
        // load's widening would be placed, and waited for, right here); the
        // last word may cover up to 3 bytes past the array, inside the
        // 16-byte block that holds its last byte, and those bytes are unused
        const __amdgpu_buffer_rsrc_t r_as = buffer_of(p.a_scales, ((int64_t)MM * KB + 3) & ~(int64_t)3);
#pragma unroll
        for (int t = 0; t < KBL; ++t) {
            const int b = lane + 64 * t, bc = b < KB ? b : KB - 1;
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                lac[t][m] = *reinterpret_cast<const uint2 *>(p.a_codes + (int64_t)m * KH + bc * 8);
                las[t][m] = __builtin_amdgcn_raw_buffer_load_b32(r_as, (m * KB + bc) & ~3, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int a = 0; a < AMAX; ++a) {
            const int ai = threadIdx.x + kGemvThreads * a, aic = ai < nact ? ai : nact - 1;
            const int m = aic / KB, b = aic - m * KB;
            ac[a] = *reinterpret_cast<const uint2 *>(p.a_codes + (int64_t)m * KH + b * 8);
            asb[a] = p.a_scales[(int64_t)m * KB + b];
        }
    }
    // 2. a z item's inputs (one launch) or the finished z (two launches)
    const bool z_wg = ZMODE == 1 && (int)blockIdx.x < p.z_items;
    // the z item published early (inside the row section, no barrier) when
    // its inputs fit beside the rows' registers: KBL MM <= 8, which also
    // bounds K by 8192, one round of inputs; otherwise after the rows
    constexpr bool z_early = KBL * MM <= 8;
    static_assert(!z_early || 64 * KBL * 16 <= 2 * kGemvThreads * kZU, "one round of z inputs");
    ZInputs<MM> zin;
    const int nz = MM * p.r;
    // Correction inputs, requested once the activation is decoded, just ahead
    // of the rows of R (they are needed only at the end; requested with the
    // activation, they would hold it up).
    // Two launches: this lane's correction operands (z split into bf16 high
    // and low parts, two dwords per j) for each round of 16 words; a round
    // past the last reads zeros through the offset kOob (no memory access,
    // exact wait counts); no wait until the correction
    u32x4_t zo[QMAX][MM][2];
    uint32_t ul[QMAX];
    auto request_correction_inputs = [&]() {
    // one launch: the epoch and this workgroup's z item's inputs
    // (unconditionally, the index clamped, so the waits for the rows stay
    // exact)
    if constexpr (ZMODE == 1) {
        ep = ld_u32(p.epoch);
        if constexpr (z_early) z_prefetch<MM>(p, min((int)blockIdx.x, p.z_items - 1), zin);
    }
    if constexpr (ZMODE == 2) {
        const int QW = zop_rounds(p.r);
        const __amdgpu_buffer_rsrc_t r_zo = buffer_of(p.zop, (int64_t)MM * QW * 2048);
#pragma unroll
        for (int q = 0; q < QMAX; ++q)
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                const int off = ((m * QW + q) * 64 + lane) * 32;
                zo[q][m][0] = load16(r_zo, opaque(q < QW ? off : kOob));
                zo[q][m][1] = load16(r_zo, opaque(q < QW ? off + 16 : kOob));
            }
    }
    // U's words for these rows, one load per round of 16 words: lane
    // 16 rr + c fetches word c + 16 q of row rr (clamped to a row and word
    // that exist; such values are never used; a round past the last reads
    // zeros through kOob).  No branch, so the waits for the rows count these
    // loads exactly; the correction shuffles the words to their lanes.
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
        ul[q] = 0u;
        if constexpr (has_z) {
            const int W = p.rpad >> 5;
            const __amdgpu_buffer_rsrc_t r_u = buffer_of(p.u, (int64_t)W * p.N * 4);
            const int w = min((lane & 15) + 16 * q, W - 1);
            const int n = min(row0 + min(lane >> 4, max(nrows - 1, 0)), p.N - 1);
            ul[q] = __builtin_amdgcn_raw_buffer_load_b32(r_u, opaque(16 * q < W ? (w * p.N + n) * 4 : kOob), 0, 0);
        }
    }
    };

    // 4. decode the activation into LDS: [m][block][8 f16 pairs], exact values;
    // z (two launches) into its own LDS area
    // exact f16 values of one block's 16 codes (8 pairs) under scale byte sb
    auto decode_block = [&](uint2 c, uint32_t sb, uint32_t (&o)[8]) {
        const float sa = __builtin_amdgcn_cvt_f32_fp8(sb, 0);
        const _Float16 mh = (_Float16)scale_mant(sa);
        const half2_t mm2 = {mh, mh};
        const uint32_t raw[8] = {
            fp4x2_to_f16x2<0>(c.x, sa), fp4x2_to_f16x2<1>(c.x, sa),
            fp4x2_to_f16x2<2>(c.x, sa), fp4x2_to_f16x2<3>(c.x, sa),
            fp4x2_to_f16x2<0>(c.y, sa), fp4x2_to_f16x2<1>(c.y, sa),
            fp4x2_to_f16x2<2>(c.y, sa), fp4x2_to_f16x2<3>(c.y, sa)};
#pragma unroll
        for (int d = 0; d < 8; ++d)
            o[d] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, raw[d]) * mm2);
    };
    uint32_t act[KBL][MM][8];
    if constexpr (!lane_act) {
#pragma unroll
    for (int a = 0; a < AMAX; ++a) {
        const int ai = threadIdx.x + kGemvThreads * a;
        if (ai < nact) {
            const float sa = __builtin_amdgcn_cvt_f32_fp8(asb[a], 0);
            const _Float16 mh = (_Float16)scale_mant(sa);
            const half2_t mm2 = {mh, mh};
            const uint32_t raw[8] = {
                fp4x2_to_f16x2<0>(ac[a].x, sa), fp4x2_to_f16x2<1>(ac[a].x, sa),
                fp4x2_to_f16x2<2>(ac[a].x, sa), fp4x2_to_f16x2<3>(ac[a].x, sa),
                fp4x2_to_f16x2<0>(ac[a].y, sa), fp4x2_to_f16x2<1>(ac[a].y, sa),
                fp4x2_to_f16x2<2>(ac[a].y, sa), fp4x2_to_f16x2<3>(ac[a].y, sa)};
            uint32_t o[8];
#pragma unroll
            for (int d = 0; d < 8; ++d)
                o[d] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, raw[d]) * mm2);
            uint4 *dst = reinterpret_cast<uint4 *>(s_act + (size_t)ai * 8);
            dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
            dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < KBL; ++t) {
        const int b = lane + 64 * t, bc = b < KB ? b : KB - 1;
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            const uint4 *src = reinterpret_cast<const uint4 *>(s_act + ((size_t)m * KB + bc) * 8);
            const uint4 lo = src[0], hi = src[1];
            act[t][m][0] = lo.x; act[t][m][1] = lo.y; act[t][m][2] = lo.z; act[t][m][3] = lo.w;
            act[t][m][4] = hi.x; act[t][m][5] = hi.y; act[t][m][6] = hi.z; act[t][m][7] = hi.w;
        }
    }
    }

    // 6-8. the rows of R, the FP4 product of every row, times g, onto the
    // per-lane sums, then the correction (two launches).
    // The body is specialised on the wave's row count (a scalar), so every
    // load it issues is one it needs and the wait before each row's
    // arithmetic counts exactly the loads issued after that row: no row
    // waits for a later one.  No barrier inside.
    float part[R][MM];
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int m = 0; m < MM; ++m) part[rr][m] = 0.0f;
    auto rows = [&](auto nr_c) {
        constexpr int NR = decltype(nr_c)::value;
        u32x2_t codes[NR][KBL];
        uint32_t sc[NR][KBL];
#pragma unroll
        for (int rr = 0; rr < NR; ++rr) {
            const int n = row0 + rr;
#pragma unroll
            for (int t = 0; t < KBL; ++t) {
                // blocks past the row end load a valid block; they are zeroed at use
                const int b = lane + 64 * t, bc = b < KB ? b : KB - 1;
                codes[rr][t] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x2_t *>(p.w_codes + (int64_t)n * KH + bc * 8));
                sc[rr][t] = __builtin_nontemporal_load(p.w_scales + (int64_t)n * KB + bc);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // the lane's activation, decoded while the rows stream in (its words
        // pass an empty asm here, so that neither the decode nor its wait is
        // hoisted out of this row-count case to before the rows' loads)
        if constexpr (lane_act) {
#pragma unroll
            for (int t = 0; t < KBL; ++t)
#pragma unroll
                for (int m = 0; m < MM; ++m) {
                    const uint2 c = make_uint2((uint32_t)opaque((int)lac[t][m].x),
                                               (uint32_t)opaque((int)lac[t][m].y));
                    const int b = lane + 64 * t, bc = b < KB ? b : KB - 1;
                    const uint32_t sb = ((uint32_t)opaque((int)las[t][m]) >> (8 * ((m * KB + bc) & 3))) & 0xFFu;
                    decode_block(c, sb, act[t][m]);
                }
        }
        // one launch: the z item, published while the rows stream in
        if constexpr (ZMODE == 1 && z_early) {
            if (z_wg) z_item_waves<MM>(p, blockIdx.x, zin, ep, s_zslots, &s_zcnt);
        }
#pragma unroll
        for (int rr = 0; rr < NR; ++rr) {
            float gacc[MM];
#pragma unroll
            for (int m = 0; m < MM; ++m) gacc[m] = 0.0f;
#pragma unroll
            for (int t = 0; t < KBL; ++t) {
                const bool valid = lane + 64 * t < KB;
                const float sw = __builtin_amdgcn_cvt_f32_fp8(sc[rr][t], 0);
                const float mant = scale_mant(sw);
                const uint32_t c0 = valid ? codes[rr][t].x : 0u;
                const uint32_t c1 = valid ? codes[rr][t].y : 0u;
                const uint32_t wv[8] = {
                    fp4x2_to_f16x2<0>(c0, sw), fp4x2_to_f16x2<1>(c0, sw),
                    fp4x2_to_f16x2<2>(c0, sw), fp4x2_to_f16x2<3>(c0, sw),
                    fp4x2_to_f16x2<0>(c1, sw), fp4x2_to_f16x2<1>(c1, sw),
                    fp4x2_to_f16x2<2>(c1, sw), fp4x2_to_f16x2<3>(c1, sw)};
#pragma unroll
                for (int m = 0; m < MM; ++m) {
                    float bl = 0.0f;
#pragma unroll
                    for (int d = 0; d < 8; ++d) bl = dot2_f16(wv[d], act[t][m][d], bl);
                    gacc[m] = __builtin_fmaf(bl, mant, gacc[m]);
                }
            }
#pragma unroll
            for (int m = 0; m < MM; ++m) part[rr][m] = __builtin_fmaf(p.g, gacc[m], part[rr][m]);
            // keep each row's decoding next to its products (hoisted, it
            // would wait for every row's loads)
            __builtin_amdgcn_sched_barrier(0);
        }
        // the correction last: U's scattered words come back while the rows
        // are consumed, so no row waits for them
        if constexpr (ZMODE == 2) add_correction_ops<MM, NR, R, QMAX>(p, ul, zo, part);
    };
    request_correction_inputs();
    __builtin_amdgcn_sched_barrier(0);
    switch (nrows) {
        case 1: rows(std::integral_constant<int, 1>{}); break;
        case 2: if constexpr (R >= 2) rows(std::integral_constant<int, 2>{}); break;
        case 3: if constexpr (R >= 3) rows(std::integral_constant<int, 3>{}); break;
        case 4: if constexpr (R >= 4) rows(std::integral_constant<int, 4>{}); break;
        default:   // no rows: nothing is stored
            if constexpr (ZMODE == 1 && z_early) {
                if (z_wg) z_item_waves<MM>(p, blockIdx.x, zin, ep, s_zslots, &s_zcnt);
            }
            break;
    }

    // one launch: the z item, computed and published once the rows are done
    // (its inputs came in ahead of them); computed before the rows, it held
    // up every workgroup's stream.  Every other workgroup then records that
    // it has read the epoch.
    if (ZMODE == 1) {
        if (z_wg) {
            float zacc[kZI][MM];
            if constexpr (!z_early) {
                z_prefetch<MM>(p, blockIdx.x, zin);
                z_accumulate<MM>(p, blockIdx.x, zin, zacc);
                z_publish<MM>(p, blockIdx.x, zin, zacc, ep, s_red);
            }
            for (int it = blockIdx.x + gridDim.x; it < p.z_items; it += gridDim.x) {
                z_prefetch<MM>(p, it, zin);
                z_accumulate<MM>(p, it, zin, zacc);
                z_publish<MM>(p, it, zin, zacc, ep, s_red);
            }
        }
        if (threadIdx.x == 0 && blockIdx.x > 0) st_u32(p.seen + blockIdx.x, ep + 1u);
    }

    // 9. one launch: z of this call into LDS (every thread requests its z
    // words at once, then re-reads the ones not yet published, bounded), then
    // the correction
    if (ZMODE == 1) {
        if (threadIdx.x == 0) s_bcast = ep;
        __syncthreads();
        const uint32_t tag = s_bcast + 1u;
        uint64_t zv[ZP];
#pragma unroll
        for (int j = 0; j < ZP; ++j) {
            const int idx = threadIdx.x + kGemvThreads * j;
            const int ic = idx < nz ? idx : nz - 1;
            const int m = ic / p.r, i = ic - m * p.r;
            zv[j] = ld_tagged(p.zt + (int64_t)m * p.rpad + i);
        }
#pragma unroll
        for (int j = 0; j < ZP; ++j) {
            const int idx = threadIdx.x + kGemvThreads * j;
            if (idx < nz) {
                const int m = idx / p.r, i = idx - m * p.r;
                const uint64_t *src = p.zt + (int64_t)m * p.rpad + i;
                uint64_t a = zv[j];
                uint32_t spins = 0;
                while ((uint32_t)(a >> 32) != tag && spins < p.spin_limit) {
                    __builtin_amdgcn_s_sleep(1);
                    a = ld_tagged(src);
                    ++spins;
                }
                s_z[zslot(p, m, i)] = (uint32_t)(a >> 32) == tag ? __uint_as_float((uint32_t)a)
                                                                 : z_local(p, m, i);
            }
        }
        __syncthreads();
        add_correction<MM, R, R, QMAX>(p, s_z, ul, part);
    }

    // 10. one reduction per row and m, then the bf16 (or fp32) store
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            const float sum = wave_sum_dpp(part[rr][m]);
            if (lane == 0 && rr < nrows) {
                if (p.yf) p.yf[(int64_t)m * p.N + row0 + rr] = sum;
                else p.y[(int64_t)m * p.N + row0 + rr] = f32_to_bf16_rne(sum);
            }
        }

    // 11. one launch: workgroup 0 advances the epoch once every other
    // workgroup has read it (its flag shows epoch + 1); the next call then
    // starts from epoch + 1
    if (ZMODE == 1 && blockIdx.x == 0) {
        for (int j = 1 + threadIdx.x; j < (int)gridDim.x; j += kGemvThreads)
            while (ld_u32(p.seen + j) != ep + 1u) __builtin_amdgcn_s_sleep(2);
        __syncthreads();
        if (threadIdx.x == 0) st_u32(p.epoch, ep + 1u);
    }
}

// z[m][i] into its correction operand slot: index i = 32 w + 16 h + 4 j + g
// (w = 16 q + c) is half h of the high and low dwords j of lane c + 16 g in
// round q.  High part: the top 16 bits of z; low part: the top 16 bits of
// the remainder (z minus the high part), as the correction has always split z.
__device__ __forceinline__ void put_zop(const GemvParams &p, int m, int i, float z) {
    const uint32_t hi = __float_as_uint(z) & 0xFFFF0000u;
    const uint32_t lo = __float_as_uint(z - __uint_as_float(hi));
    const int w = i >> 5, h = (i >> 4) & 1, j = (i >> 2) & 3, g = i & 3;
    const int lane = (w & 15) + 16 * g;
    const int64_t dw = (((int64_t)m * zop_rounds(p.r) + (w >> 4)) * 64 + lane) * 8 + 2 * j;
    uint16_t *half = reinterpret_cast<uint16_t *>(p.zop_out + dw) + h;
    half[0] = (uint16_t)(hi >> 16);
    half[2] = (uint16_t)(lo >> 16);
}

// z of the two-launch schedule: one workgroup per z item (kZI indices i over
// all of K), plain fp32 stores (and the product's operand halves); the
// product kernel that follows on the same stream reads z complete.
template <int MM>
__global__ void __launch_bounds__(kGemvThreads) z_kernel(GemvParams p) {
    __shared__ float s_red[8];
    // The activation's FP4 quantisation rides along (read by the product) in
    // the first zq workgroups, one block per thread, dispatched first, so no
    // z item waits for it.
    const int zq = (int)gridDim.x - p.z_items;
    if ((int)blockIdx.x < zq) {
        const int64_t nb = (int64_t)MM * (p.K >> 4);
        for (int64_t blk = (int64_t)blockIdx.x * kGemvThreads + threadIdx.x; blk < nb;
             blk += (int64_t)zq * kGemvThreads)
            quant_act_block(p.x, blk, p.qa_codes, p.qa_scales);
        return;
    }
    // Workgroups are dispatched to the 8 XCDs in turn.  The items of one V
    // word (32 / kZI consecutive items) are mapped to workgroups whose index
    // b (counted after the quantisation workgroups) agrees mod 8, that is to
    // one XCD, so that word's column of V is fetched into one L2 only.  The
    // map is a permutation of [0, z_items) whatever the dispatch does.
    const int b = blockIdx.x - zq, G = p.z_items, x = b & 7, q = G >> 3, rem = G & 7;
    const int item = x * q + (x < rem ? x : rem) + (b >> 3);
    ZInputs<MM> zin;
    z_prefetch<MM>(p, item, zin);
    float acc[kZI][MM];
    z_accumulate<MM>(p, item, zin, acc);
    const int i0 = item * kZI;
    float zs[kZI][MM];
#pragma unroll
    for (int i = 0; i < kZI; ++i)
#pragma unroll
        for (int m = 0; m < MM; ++m) zs[i][m] = block_sum8(acc[i][m], s_red);
#pragma unroll
    for (int i = 0; i < kZI; ++i)
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            const int ii = i0 + i;
            if ((int)threadIdx.x == 64 * i + m && ii < p.r) {
                const float zv = zs[i][m] * bf16_to_f32(zin.al[i]);
                p.zf_out[(int64_t)m * p.rpad + ii] = zv;
                if (p.zop_out) put_zop(p, m, ii, zv);
            }
        }
    // the operand slots of the padding indices r .. 512 ceil(rpad / 512) hold 0
    if (p.zop_out && b == 0) {
        const int span = zop_rounds(p.r) * 512 - p.r;
        for (int t = threadIdx.x; t < MM * span; t += kGemvThreads)
            put_zop(p, t / span, p.r + t % span, 0.0f);
    }
}

namespace {
size_t gemv_lds_bytes(int M, int K, int rpad) {
    return (size_t)M * (size_t)(K / 16) * 32 + (size_t)M * (size_t)(rpad + rpad / 16) * 4;
}

template <int MM, int KBL, int ZMODE>
hipError_t launch_t(const GemvParams &p, int grid, size_t lds, hipStream_t stream) {
    hipLaunchKernelGGL((fused_gemv_kernel<MM, KBL, ZMODE>), dim3(grid), dim3(kGemvThreads), lds,
                       stream, p);
    return hipGetLastError();
}

template <int MM, int ZMODE>
hipError_t launch_mz(const GemvParams &p, int kbl, int grid, size_t lds, hipStream_t stream) {
    switch (kbl) {
        case 1: return launch_t<MM, 1, ZMODE>(p, grid, lds, stream);
        case 2: return launch_t<MM, 2, ZMODE>(p, grid, lds, stream);
        case 3: return launch_t<MM, 3, ZMODE>(p, grid, lds, stream);
        case 4: return launch_t<MM, 4, ZMODE>(p, grid, lds, stream);
        case 5: return launch_t<MM, 5, ZMODE>(p, grid, lds, stream);
        case 6: return launch_t<MM, 6, ZMODE>(p, grid, lds, stream);
        case 7:
        case 8: return launch_t<MM, 8, ZMODE>(p, grid, lds, stream);
        case 9:
        case 10:
        case 11:
        case 12: if (MM == 1) return launch_t<1, 12, ZMODE>(p, grid, lds, stream); break;
        case 13:
        case 14:
        case 15:
        case 16: if (MM == 1) return launch_t<1, 16, ZMODE>(p, grid, lds, stream); break;
        default: break;
    }
    return hipErrorNotSupported;
}

template <int MM>
hipError_t launch_m(const GemvParams &p, int kbl, int grid, size_t lds, int zmode,
                    hipStream_t stream) {
    switch (zmode) {
        case 0: return launch_mz<MM, 0>(p, kbl, grid, lds, stream);
        case 1: return launch_mz<MM, 1>(p, kbl, grid, lds, stream);
        default: return launch_mz<MM, 2>(p, kbl, grid, lds, stream);
    }
}

uint32_t spin_limit_default() {
    // debug override (BILOCO_DEBUG_SPIN_LIMIT): shortens the bounded wait on z
    // so that tests can force the self-computing fallback
    const char *s = getenv("BILOCO_DEBUG_SPIN_LIMIT");
    return s ? (uint32_t)strtoul(s, nullptr, 10) : (uint32_t)(1u << 20);
}

int kbl_of(int K) { return (K / 16 + 63) / 64; }
// the instantiated KBL a K runs with (see launch_m)
int kbl_launch(int kbl) {
    return kbl <= 6 ? kbl : (kbl <= 8 ? 8 : (kbl <= 12 ? 12 : 16));
}

// Stream workgroups and rows per workgroup: about one workgroup per CU while
// its rows fit the waves' register budget, more workgroups beyond that.
void gemv_grid(int N, int kbl, int mm, int *wgs, int *rows_per_wg) {
    const int cap = 8 * gemv_rows_per_wave(kbl, mm);
    int rpg = (N + 255) / 256;
    if (rpg > cap) rpg = cap;
    *rows_per_wg = rpg;
    *wgs = (N + rpg - 1) / rpg;
}
}  // namespace

bool gemv_supported(int M, int N, int K, int r) {
    const int kbl = kbl_of(K);
    if (M < 1 || M > 2 || r < 0 || r > 1024 || N < 1) return false;
    if (M * (K / 16) > 4 * kGemvThreads) return false;
    if (gemv_lds_bytes(M, K, rpad32(r)) > 64 * 1024) return false;
    int wgs, rpg;
    gemv_grid(N, kbl_launch(kbl), M, &wgs, &rpg);
    if (wgs > kGemvMaxWorkgroups) return false;
    return M == 1 ? kbl <= 16 : kbl <= 8;
}

namespace {
hipError_t launch_gemv(const GemmArgs &a, bool two_launch, hipStream_t stream) {
    if (!gemv_supported(a.M, a.N, a.K, a.r)) return hipErrorNotSupported;
    GemvParams p{};
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
    p.N = a.N;
    p.K = a.K;
    p.r = a.r;
    p.rpad = rpad32(a.r);
    const int kbl = kbl_of(a.K);
    int swgs = 0;
    gemv_grid(a.N, kbl_launch(kbl), a.M, &swgs, &p.rows_per_wg);
    p.z_items = (a.r + kZI - 1) / kZI;
    int zmode = 0;
    if (a.r > 0) {
        char *ws = static_cast<char *>(a.ws);
        p.epoch = reinterpret_cast<uint32_t *>(ws + ws_epoch_offset());
        p.seen = reinterpret_cast<uint32_t *>(ws + ws_seen_offset());
        p.zt = reinterpret_cast<uint64_t *>(ws + ws_zt_offset());
        p.zf_out = reinterpret_cast<float *>(ws + ws_zf_offset(a.M, a.r));
        p.zf = p.zf_out;
        if (two_launch) {
            p.zop_out = reinterpret_cast<uint32_t *>(ws + ws_zop_offset(a.M, a.r));
            p.zop = p.zop_out;
        }
        zmode = two_launch ? 2 : 1;
    } else {
        // no correction: the kernel still reads one epoch word and one U word
        // per lane (results unused); point both at the first bytes of R
        p.epoch = reinterpret_cast<uint32_t *>(const_cast<uint8_t *>(a.w_codes));
        p.u = reinterpret_cast<const uint32_t *>(a.w_codes);
    }
    static const uint32_t spin = spin_limit_default();
    p.spin_limit = spin;
    if (zmode == 2) {
        // the quantisation workgroups (if any), then the z items
        const int zq = a.qa_codes ? (a.M * (a.K / 16) + kGemvThreads - 1) / kGemvThreads : 0;
        if (a.M == 1)
            hipLaunchKernelGGL(z_kernel<1>, dim3(p.z_items + zq), dim3(kGemvThreads), 0, stream, p);
        else
            hipLaunchKernelGGL(z_kernel<2>, dim3(p.z_items + zq), dim3(kGemvThreads), 0, stream, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const size_t lds = gemv_lds_bytes(a.M, a.K, p.rpad);
    switch (a.M) {
        case 1: return launch_m<1>(p, kbl, swgs, lds, zmode, stream);
        case 2: return launch_m<2>(p, kbl, swgs, lds, zmode, stream);
        default: return hipErrorNotSupported;
    }
}
}  // namespace

// The z kernel alone (plain fp32 z at z), for compositions of separate launches.
hipError_t launch_z_gemv(const GemmArgs &a, float *z, hipStream_t stream) {
    if (a.M < 1 || a.M > 2 || a.r < 1) return hipErrorNotSupported;
    GemvParams p{};
    p.x = a.x;
    p.v = a.v;
    p.alpha = a.alpha;
    p.N = a.N;
    p.K = a.K;
    p.r = a.r;
    p.rpad = rpad32(a.r);
    p.z_items = (a.r + kZI - 1) / kZI;
    p.zf_out = z;
    if (a.M == 1)
        hipLaunchKernelGGL(z_kernel<1>, dim3(p.z_items), dim3(kGemvThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(z_kernel<2>, dim3(p.z_items), dim3(kGemvThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_gemm_fused_gemv(const GemmArgs &a, hipStream_t stream) {
    return launch_gemv(a, false, stream);
}

hipError_t launch_gemm_gemv_two_launch(const GemmArgs &a, hipStream_t stream) {
    return launch_gemv(a, true, stream);
}

}  // namespace biloco
