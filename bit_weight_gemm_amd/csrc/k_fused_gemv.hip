// One-launch product for small decode batches (schedule BILOCO_SCHED_FUSED_GEMV).
//
// BiLoCo README, section "Kernel": y = FP4(x) FP4(R)^T + sum_i alpha_i (x.v_i) u_i
// in one launch; side work computes z = alpha (.) (V x) from the packed signs of
// V while the FP4 product streams R; z values are published with an epoch tag
// that the output tiles poll; the epilogue expands z through U's packed signs
// and adds it before the bf16 store.  Designed here for gfx950 and M <= 4,
// where the product is a matrix-vector stream bound by HBM:
//
//  * every wave owns whole output rows (full K), so no partial sums cross
//    workgroups; lanes stride over the 16-element NVFP4 blocks of a row;
//  * R is dequantised in registers: one v_cvt_scalef32_pk_f16_fp4 per code
//    byte applies the block scale's power of two, the scale's mantissa
//    (1 + m/8) multiplies the block's fp32 partial sum; the FP4 activation is
//    pre-scaled once per wave into f16 registers (exact); products are
//    v_dot2 (f16 x f16 -> fp32);
//  * z is split over the first workgroups, 8 values of i per workgroup over
//    all of K; the +-1 signs of two consecutive k come out of one pair of V
//    words as a bf16 pair, so x (bf16) and the signs meet in v_dot2 (bf16)
//    with exact products;
//  * each z value is published as one 64-bit word (fp32 value, 32-bit epoch
//    tag) with a relaxed device-scope store, read back with device-scope
//    loads: no fences; a call's epoch is read at start and advanced by the
//    last workgroup to arrive, so repeated calls never reset anything;
//  * the correction multiplies U's signs (again as bf16 pairs) with z split
//    into a bf16 high part and a bf16 low part (about 16 bits of z);
//  * every wait is bounded: a consumer that has waited too long computes the
//    z values it needs by itself, so the kernel finishes whatever else runs
//    on the device.
#include "biloco_device.h"
#include "biloco_internal.h"

#include <stdlib.h>

namespace biloco {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

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
    uint64_t *hdr;          // workspace header: epoch << 32 | arrival counter
    uint64_t *zt;           // workspace z: (value | tag << 32) [M][rpad]
    float g;
    int N, K, r, rpad;
    int rows_per_wave;
    int z_items;            // ceil(r / 8)
    int z_wgs;              // workgroups that produce z (placed first)
    uint32_t spin_limit;    // bounded wait on z; 0 = compute z locally at once
};

__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b),
                                  c, false);
}
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}
// Two FP4 codes (byte `sel` of w) -> two f16 values times 2^exponent(scale).
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_f16x2(uint32_t w, float scale) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, SEL));
}
// Sign bits at positions p and p+16 of t -> bf16 pair (+-1, +-1): bit set = -1.
__device__ __forceinline__ uint32_t signs_bf16x2(uint32_t t, int p) {
    return ((t << (15 - p)) & 0x80008000u) | 0x3F803F80u;
}

__device__ __forceinline__ uint64_t ld_tagged(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_tagged(uint64_t *p, float v, uint32_t tag) {
    const uint64_t w = ((uint64_t)tag << 32) | __float_as_uint(v);
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// z for the 8 indices i0..i0+7 (same 32-bit word of V) and all MM rows,
// computed by one whole workgroup over all of K and published with `tag`.
template <int MM>
__device__ void z_item(const GemvParams &p, int item, const uint32_t *s_tag, float *red) {
    const int i0 = item * 8, w = i0 >> 5, o = i0 & 31;
    const int s = o & 15;                 // bit offset inside the 16-bit half
    const bool high = o >= 16;
    const uint32_t *vrow = p.v + (int64_t)w * p.K;
    float acc[8][MM];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int m = 0; m < MM; ++m) acc[i][m] = 0.0f;
    // ZU pairs (k, k+1) per thread per round, all loads issued before use
    constexpr int ZU = 16;
    const int KP = p.K / 2;
    for (int kp0 = 0; kp0 < KP; kp0 += 256 * ZU) {
        uint2 vv[ZU];
        uint32_t xp[ZU][MM];
#pragma unroll
        for (int u = 0; u < ZU; ++u) {
            const int kp = kp0 + threadIdx.x + 256 * u, kc = kp < KP ? kp : KP - 1;
            vv[u] = *reinterpret_cast<const uint2 *>(vrow + 2 * kc);
#pragma unroll
            for (int m = 0; m < MM; ++m)
                xp[u][m] = *reinterpret_cast<const uint32_t *>(p.x + (int64_t)m * p.K + 2 * kc);
        }
#pragma unroll
        for (int u = 0; u < ZU; ++u) {
            const bool valid = kp0 + (int)threadIdx.x + 256 * u < KP;
            // t: the 16 sign bits of k in the low half, those of k+1 in the high half
            const uint32_t t = high ? __builtin_amdgcn_perm(vv[u].y, vv[u].x, 0x07060302u)
                                    : __builtin_amdgcn_perm(vv[u].y, vv[u].x, 0x05040100u);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t sg = signs_bf16x2(t, s + i);
#pragma unroll
                for (int m = 0; m < MM; ++m)
                    acc[i][m] = dot2_bf16(sg, valid ? xp[u][m] : 0u, acc[i][m]);
            }
        }
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            const float v = wave_sum_dpp(acc[i][m]);
            if (lane == 0) red[(wave * 8 + i) * MM + m] = v;
        }
    __syncthreads();
    if (threadIdx.x < 8 * MM) {
        const int i = threadIdx.x / MM, m = threadIdx.x % MM, ii = i0 + i;
        if (ii < p.r) {
            const float sum = (red[(0 * 8 + i) * MM + m] + red[(1 * 8 + i) * MM + m]) +
                              (red[(2 * 8 + i) * MM + m] + red[(3 * 8 + i) * MM + m]);
            st_tagged(p.zt + (int64_t)m * p.rpad + ii, sum * bf16_to_f32(p.alpha[ii]), *s_tag);
        }
    }
    __syncthreads();
}

// Fallback: z[m][i] for one index, computed by one thread alone (slow; only
// used after a bounded wait ran out).
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

// Workgroups [0, z_wgs) compute z items; workgroups [z_wgs, grid) stream R.
template <int MM, int KBL>
__global__ void __launch_bounds__(256) fused_gemv_kernel(GemvParams p) {
    __shared__ uint32_t s_tag;
    __shared__ uint32_t s_last;
    __shared__ float s_red[4 * 8 * MM];
    __shared__ float s_G[4][64][MM];
    extern __shared__ float s_z[];        // [MM][rpad] z values of this call

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int KB = p.K >> 4, KH = p.K >> 1;

    // one 64-bit fetch-add returns (epoch << 32 | arrivals so far); its value
    // is first needed after the stream has been issued
    uint64_t hv = 0;
    if (threadIdx.x == 0 && p.hdr)
        hv = __hip_atomic_fetch_add(p.hdr, (uint64_t)1, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);

    if ((int)blockIdx.x < p.z_wgs) {
        // ------------------------------------------------ z producer
        if (threadIdx.x == 0) {
            s_tag = (uint32_t)(hv >> 32) + 1u;
            s_last = (uint32_t)hv == gridDim.x - 1;
        }
        __syncthreads();
        for (int it = blockIdx.x; it < p.z_items; it += p.z_wgs) z_item<MM>(p, it, &s_tag, s_red);
    } else {
        // ------------------------------------------------ R stream
        const int gwave = (blockIdx.x - p.z_wgs) * 4 + wave;
        const int row0 = gwave * p.rows_per_wave;
        int nrows = p.N - row0;
        nrows = nrows < 0 ? 0 : (nrows > p.rows_per_wave ? p.rows_per_wave : nrows);

        // activation loads first (they are waited on first), pre-scaled to
        // f16 pairs: act[t][m][d] holds elements 2d, 2d+1 of block lane + 64t
        uint2 ac[KBL][MM];
        uint32_t asb[KBL][MM];
#pragma unroll
        for (int t = 0; t < KBL; ++t) {
            const int b = lane + 64 * t, bc = b < KB ? b : KB - 1;
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                ac[t][m] = *reinterpret_cast<const uint2 *>(p.a_codes + (int64_t)m * KH + bc * 8);
                asb[t][m] = p.a_scales[(int64_t)m * KB + bc];
            }
        }
        // R rows stream through a ring of PD row buffers
        constexpr int PD = (40 / KBL) < 2 ? 2 : ((40 / KBL) > 8 ? 8 : (40 / KBL));
        u32x2_t codes[PD][KBL];
        uint32_t sc[PD][KBL];
#pragma unroll
        for (int sl = 0; sl < PD; ++sl) {
            if (sl < nrows) {
                const int64_t n = row0 + sl;
#pragma unroll
                for (int t = 0; t < KBL; ++t) {
                    const int b = lane + 64 * t, bc = b < KB ? b : KB - 1;
                    codes[sl][t] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x2_t *>(p.w_codes + n * KH + bc * 8));
                    sc[sl][t] = __builtin_nontemporal_load(p.w_scales + n * KB + bc);
                }
            }
        }
        uint32_t act[KBL][MM][8];
#pragma unroll
        for (int t = 0; t < KBL; ++t) {
            const bool valid = lane + 64 * t < KB;
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                const uint32_t cx = valid ? ac[t][m].x : 0u, cy = valid ? ac[t][m].y : 0u;
                const float sa = __builtin_amdgcn_cvt_f32_fp8(asb[t][m], 0);
                const uint32_t mant = (__float_as_uint(sa) & 0x007FFFFFu) | 0x3F800000u;
                const _Float16 mh = (_Float16)__uint_as_float(mant);
                const half2_t mm2 = {mh, mh};
                const uint32_t raw[8] = {fp4x2_to_f16x2<0>(cx, sa), fp4x2_to_f16x2<1>(cx, sa),
                                         fp4x2_to_f16x2<2>(cx, sa), fp4x2_to_f16x2<3>(cx, sa),
                                         fp4x2_to_f16x2<0>(cy, sa), fp4x2_to_f16x2<1>(cy, sa),
                                         fp4x2_to_f16x2<2>(cy, sa), fp4x2_to_f16x2<3>(cy, sa)};
#pragma unroll
                for (int d = 0; d < 8; ++d)
                    act[t][m][d] =
                        __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, raw[d]) * mm2);
            }
        }

        for (int base = 0; base < nrows; base += PD) {
            float part[PD][MM];
#pragma unroll
            for (int sl = 0; sl < PD; ++sl) {
                const int rr = base + sl;
#pragma unroll
                for (int m = 0; m < MM; ++m) part[sl][m] = 0.0f;
                if (rr < nrows) {
#pragma unroll
                    for (int t = 0; t < KBL; ++t) {
                        const bool valid = lane + 64 * t < KB;
                        const float sw = __builtin_amdgcn_cvt_f32_fp8(sc[sl][t], 0);
                        const float mant = __uint_as_float(
                            (__float_as_uint(sw) & 0x007FFFFFu) | 0x3F800000u);
                        const uint32_t c0 = valid ? codes[sl][t].x : 0u;
                        const uint32_t c1 = valid ? codes[sl][t].y : 0u;
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
                            part[sl][m] = __builtin_fmaf(bl, mant, part[sl][m]);
                        }
                    }
                    // refill this slot with the row PD ahead
                    if (rr + PD < nrows) {
                        const int64_t n = row0 + rr + PD;
#pragma unroll
                        for (int t = 0; t < KBL; ++t) {
                            const int b = lane + 64 * t, bc = b < KB ? b : KB - 1;
                            codes[sl][t] = __builtin_nontemporal_load(
                                reinterpret_cast<const u32x2_t *>(p.w_codes + n * KH + bc * 8));
                            sc[sl][t] = __builtin_nontemporal_load(p.w_scales + n * KB + bc);
                        }
                    }
                }
            }
            // the PD row sums of this ring cycle, reduced together
#pragma unroll
            for (int sl = 0; sl < PD; ++sl)
#pragma unroll
                for (int m = 0; m < MM; ++m) {
                    const float sum = wave_sum_dpp(part[sl][m]);
                    if (lane == 0 && base + sl < nrows) s_G[wave][base + sl][m] = p.g * sum;
                }
        }

        // ------------------------------------------------ z acquire
        if (threadIdx.x == 0) {
            s_tag = (uint32_t)(hv >> 32) + 1u;
            s_last = (uint32_t)hv == gridDim.x - 1;
        }
        __syncthreads();
        const uint32_t tag = s_tag;
        for (int idx = threadIdx.x; idx < MM * p.r; idx += 256) {
            const int m = idx / p.r, i = idx - m * p.r;
            const uint64_t *src = p.zt + (int64_t)m * p.rpad + i;
            uint64_t a = ld_tagged(src);
            uint32_t spins = 0;
            while ((uint32_t)(a >> 32) != tag && spins < p.spin_limit) {
                __builtin_amdgcn_s_sleep(1);
                a = ld_tagged(src);
                ++spins;
            }
            s_z[m * p.rpad + i] = (uint32_t)(a >> 32) == tag ? __uint_as_float((uint32_t)a)
                                                             : z_local(p, m, i);
        }
        __syncthreads();

        // ------------------------------------------------ correction + store
        // lane covers word (lane % 16) + 16 q and bit pairs (pb, pb + 16),
        // pb = lane / 16 + 4 j, j = 0..3; z as bf16 high + bf16 low parts
        const int W = p.rpad >> 5;
        for (int q = 0; q * 16 < W; ++q) {
            const int w = (lane & 15) + 16 * q;
            const bool wok = w < W;
            uint32_t zhi[4][MM], zlo[4][MM];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int pb = (lane >> 4) + 4 * j;
#pragma unroll
                for (int m = 0; m < MM; ++m) {
                    const int i0 = 32 * w + pb, i1 = i0 + 16;
                    const float z0 = (wok && i0 < p.r) ? s_z[m * p.rpad + i0] : 0.0f;
                    const float z1 = (wok && i1 < p.r) ? s_z[m * p.rpad + i1] : 0.0f;
                    const uint32_t h0 = __float_as_uint(z0) & 0xFFFF0000u;
                    const uint32_t h1 = __float_as_uint(z1) & 0xFFFF0000u;
                    const uint32_t l0 = __float_as_uint(z0 - __uint_as_float(h0));
                    const uint32_t l1 = __float_as_uint(z1 - __uint_as_float(h1));
                    zhi[j][m] = (h0 >> 16) | h1;
                    zlo[j][m] = (l0 >> 16) | (l1 & 0xFFFF0000u);
                }
            }
            for (int base = 0; base < nrows; base += 8) {
                uint32_t uw[8];
#pragma unroll
                for (int sl = 0; sl < 8; ++sl) {
                    const int rr = base + sl < nrows ? base + sl : nrows - 1;
                    uw[sl] = wok ? p.u[(int64_t)w * p.N + row0 + rr] : 0u;
                }
                float c[8][MM];
#pragma unroll
                for (int sl = 0; sl < 8; ++sl)
#pragma unroll
                    for (int m = 0; m < MM; ++m) c[sl][m] = 0.0f;
#pragma unroll
                for (int sl = 0; sl < 8; ++sl)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t sg = signs_bf16x2(uw[sl], (lane >> 4) + 4 * j);
#pragma unroll
                        for (int m = 0; m < MM; ++m) {
                            c[sl][m] = dot2_bf16(sg, zhi[j][m], c[sl][m]);
                            c[sl][m] = dot2_bf16(sg, zlo[j][m], c[sl][m]);
                        }
                    }
#pragma unroll
                for (int sl = 0; sl < 8; ++sl)
#pragma unroll
                    for (int m = 0; m < MM; ++m) {
                        const float cs = wave_sum_dpp(c[sl][m]);
                        if (lane == 0 && base + sl < nrows) s_G[wave][base + sl][m] += cs;
                    }
            }
        }
        if (lane == 0) {
            for (int rr = 0; rr < nrows; ++rr)
#pragma unroll
                for (int m = 0; m < MM; ++m)
                    p.y[(int64_t)m * p.N + row0 + rr] = f32_to_bf16_rne(s_G[wave][rr][m]);
        }
    }

    // last workgroup to arrive: every workgroup has taken this call's epoch,
    // so the next call may start from epoch + 1 with the counter at zero
    if (threadIdx.x == 0 && p.hdr && (uint32_t)hv == gridDim.x - 1) {
        const uint64_t next = ((hv >> 32) + 1u) << 32;
        __hip_atomic_store(p.hdr, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

namespace {
template <int MM, int KBL>
hipError_t launch_t(const GemvParams &p, int grid, hipStream_t stream) {
    const size_t lds = (size_t)MM * (size_t)(p.rpad > 0 ? p.rpad : 1) * sizeof(float);
    hipLaunchKernelGGL((fused_gemv_kernel<MM, KBL>), dim3(grid), dim3(256), lds, stream, p);
    return hipGetLastError();
}

template <int MM>
hipError_t launch_m(const GemvParams &p, int kbl, int grid, hipStream_t stream) {
    switch (kbl) {
        case 1: return launch_t<MM, 1>(p, grid, stream);
        case 2: return launch_t<MM, 2>(p, grid, stream);
        case 3: return launch_t<MM, 3>(p, grid, stream);
        case 4: return launch_t<MM, 4>(p, grid, stream);
        case 5: if (MM <= 3) return launch_t<MM <= 3 ? MM : 1, 5>(p, grid, stream); break;
        case 6: if (MM <= 2) return launch_t<MM <= 2 ? MM : 1, 6>(p, grid, stream); break;
        case 7:
        case 8: if (MM <= 2) return launch_t<MM <= 2 ? MM : 1, 8>(p, grid, stream); break;
        case 9:
        case 10:
        case 11:
        case 12: if (MM == 1) return launch_t<1, 12>(p, grid, stream); break;
        case 13:
        case 14:
        case 15:
        case 16: if (MM == 1) return launch_t<1, 16>(p, grid, stream); break;
        default: break;
    }
    return hipErrorNotSupported;
}

uint32_t spin_limit_default() {
    // a debug override (BILOCO_DEBUG_SPIN_LIMIT) shortens the bounded wait on
    // z so that tests can force the self-computing fallback
    const char *s = getenv("BILOCO_DEBUG_SPIN_LIMIT");
    return s ? (uint32_t)strtoul(s, nullptr, 10) : (uint32_t)(1u << 20);
}
}  // namespace

int gemv_rows_per_wave(int N) { return (N + 1023) / 1024; }

bool gemv_supported(int M, int N, int K, int r) {
    const int kbl = (K / 16 + 63) / 64;
    if (M < 1 || M > 4 || r > 2048 || gemv_rows_per_wave(N) > 64) return false;
    if (M == 1) return kbl <= 16;
    if (M == 2) return kbl <= 8;
    if (M == 3) return kbl <= 5;
    return kbl <= 4;
}

hipError_t launch_gemm_fused_gemv(const GemmArgs &a, hipStream_t stream) {
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
    p.g = a.g;
    p.N = a.N;
    p.K = a.K;
    p.r = a.r;
    p.rpad = rpad32(a.r);
    // rows per wave: aim at ~1024 streaming waves (one per SIMD)
    p.rows_per_wave = gemv_rows_per_wave(a.N);
    const int waves = (a.N + p.rows_per_wave - 1) / p.rows_per_wave;
    const int gemm_wgs = (waves + 3) / 4;
    p.z_items = (a.r + 7) / 8;
    p.z_wgs = p.z_items;
    p.hdr = a.r > 0 ? reinterpret_cast<uint64_t *>(a.ws) : nullptr;
    p.zt = a.r > 0 ? reinterpret_cast<uint64_t *>(static_cast<char *>(a.ws) + ws_zt_offset())
                   : nullptr;
    static const uint32_t spin = spin_limit_default();
    p.spin_limit = spin;
    const int grid = p.z_wgs + gemm_wgs;
    const int kbl = (a.K / 16 + 63) / 64;
    switch (a.M) {
        case 1: return launch_m<1>(p, kbl, grid, stream);
        case 2: return launch_m<2>(p, kbl, grid, stream);
        case 3: return launch_m<3>(p, kbl, grid, stream);
        case 4: return launch_m<4>(p, kbl, grid, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace biloco
