// Device-side helpers of the HIP path: element formats and wave reductions.
// Formats follow the NVFP4 layout that the BiLoCo README's section "Kernel"
// names for R and for the activation: E2M1 element codes (two per byte, even
// element in the low nibble) and E4M3 block scales (one per 16 elements).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace biloco {

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint32_t h16) {
    return __uint_as_float(h16 << 16);
}

// fp32 -> bf16 with round-to-nearest-even; NaN kept quiet.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------- E4M3 (OCP FN)
// Byte -> fp32.  Exponent field 0 is subnormal (m * 2^-9).  The NaN pattern
// never occurs in scales this library writes or accepts as meaningful.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    uint32_t e = (b >> 3) & 15u, m = b & 7u;
    float mag = (e == 0u) ? (float)m * 0.001953125f                       // m * 2^-9
                          : __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (b & 0x80u) ? -mag : mag;
}

// Non-negative finite fp32 -> E4M3 byte, round to nearest, ties to an even
// mantissa; saturates to 448 (0x7E).
__device__ __forceinline__ uint32_t f32_to_e4m3_rne(float q) {
    if (q >= 448.0f) return 0x7Eu;
    if (q < 0.015625f) {                       // below 2^-6: subnormal grid of 2^-9
        // q * 512 is exact; rint rounds half to even.  A result of 8 is the
        // smallest normal 2^-6, whose byte is also 8.
        return (uint32_t)__builtin_rintf(q * 512.0f);
    }
    uint32_t u = __float_as_uint(q);
    uint32_t rnd = u + 0x7FFFFu + ((u >> 20) & 1u);   // round mantissa to 3 bits
    uint32_t e = (rnd >> 23) - 120u;                  // rebias 127 -> 7
    return (e << 3) | ((rnd >> 20) & 7u);
}

// ---------------------------------------------------------------- E2M1
// Code (0..15) -> fp32.
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
    uint32_t e = (c >> 1) & 3u, m = c & 1u;
    float mag = (e == 0u) ? 0.5f * (float)m : __uint_as_float(((e + 126u) << 23) | (m << 22));
    return (c & 8u) ? -mag : mag;
}

// Nearest-even E2M1 magnitude code of a = |x| for a scale s > 0.  Each
// product s * t below is exact in fp32 (s has at most 4 significant bits and
// every t at most 3), so the comparisons decide the rounding exactly.
__device__ __forceinline__ uint32_t e2m1_mag_code(float a, float s) {
    return (uint32_t)(a > 0.25f * s) + (uint32_t)(a >= 0.75f * s) + (uint32_t)(a > 1.25f * s) +
           (uint32_t)(a >= 1.75f * s) + (uint32_t)(a > 2.5f * s) + (uint32_t)(a >= 3.5f * s) +
           (uint32_t)(a > 5.0f * s);
}

// ---------------------------------------------------------------- activation FP4
// One block of 16 activations (blocks are numbered row-major over [M][K/16]):
// two 16-byte loads, amax by integer max over the magnitude bits (bf16
// magnitudes order like integers), scale = E4M3(amax / 6) with a correctly
// rounded fp32 division, codes by exact comparisons with the E2M1 midpoints
// times the scale; one 8-byte store of the codes and one byte of scale.
// The arithmetic of one block: its 16 bf16 values (two per dword, element
// 2j in the low half of w[j]) -> the two dwords of E2M1 codes (element e in
// nibble e) and the E4M3 scale byte.
__device__ __forceinline__ uint32_t quant16(const uint32_t (&w)[8], uint32_t &lo, uint32_t &hi) {
    uint32_t amax_bits = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        amax_bits = max(amax_bits, w[j] & 0x7FFFu);
        amax_bits = max(amax_bits, (w[j] >> 16) & 0x7FFFu);
    }
    const float amax = bf16_to_f32(amax_bits);
    const uint32_t sb = f32_to_e4m3_rne(amax / 6.0f);
    const float s = e4m3_to_f32(sb);
    lo = 0;
    hi = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const uint32_t h = (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu);
        const float a = bf16_to_f32(h & 0x7FFFu);
        const uint32_t mag = (sb == 0u) ? 0u : e2m1_mag_code(a, s);
        const uint32_t code = mag | ((h >> 12) & 8u);
        if (j < 8) lo |= code << (4 * j);
        else hi |= code << (4 * (j - 8));
    }
    return sb;
}

// The same block without a comparison per midpoint: each |x| / s is
// Markstein's corrected quotient (q0 = |x| r, e = fma(-q0, s, |x|),
// q = fma(e, r, q0), r = fp32(1 / s)) and the hardware FP4 conversion with
// unit scale rounds it (nearest, ties to the even code, saturating at 6; the
// sign of x is put back on q, so that -0 and negatives rounding to 0 keep
// it).  The codes equal quant16's for every positive bf16 value and every
// E4M3 scale a block can have (checked exhaustively on the CPU,
// tests/csrc/act_code_check.c; the conversion's rounding was checked on
// gfx950 at every E2M1 midpoint and its neighbours).  A zero scale (the
// block is all zeros, or its amax / 6 rounds to 0) gives signed zeros.
// elements 2j, 2j + 1 (the halves of wj) -> byte SEL of c
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t c, uint32_t wj, float s, float r) {
    const uint32_t b[2] = {wj << 16, wj & 0xFFFF0000u};
    float y[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const float a = __uint_as_float(b[h] & 0x7FFFFFFFu);
        const float q0 = a * r;
        const float e = __builtin_fmaf(-q0, s, a);
        const float q = __builtin_fmaf(e, r, q0);
        y[h] = __uint_as_float(__float_as_uint(q) | (b[h] & 0x80000000u));
    }
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, y[0], y[1], 1.0f, SEL);
}
__device__ __forceinline__ uint32_t quant16_fast(const uint32_t (&w)[8], uint32_t &lo, uint32_t &hi) {
    uint32_t amax_bits = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        amax_bits = max(amax_bits, w[j] & 0x7FFFu);
        amax_bits = max(amax_bits, (w[j] >> 16) & 0x7FFFu);
    }
    const uint32_t sb = f32_to_e4m3_rne(bf16_to_f32(amax_bits) / 6.0f);
    const float s = sb ? e4m3_to_f32(sb) : 1.0f;
    const float r = sb ? 1.0f / s : 0.0f;
    lo = fp4_pair<0>(0u, w[0], s, r);
    lo = fp4_pair<1>(lo, w[1], s, r);
    lo = fp4_pair<2>(lo, w[2], s, r);
    lo = fp4_pair<3>(lo, w[3], s, r);
    hi = fp4_pair<0>(0u, w[4], s, r);
    hi = fp4_pair<1>(hi, w[5], s, r);
    hi = fp4_pair<2>(hi, w[6], s, r);
    hi = fp4_pair<3>(hi, w[7], s, r);
    return sb;
}

__device__ __forceinline__ void quant_act_block(const uint16_t *__restrict__ x, int64_t blk,
                                                uint8_t *__restrict__ codes,
                                                uint8_t *__restrict__ scales) {
    const uint4 *src = reinterpret_cast<const uint4 *>(x + blk * 16);
    const uint4 v0 = src[0], v1 = src[1];
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t lo, hi;
    const uint32_t sb = quant16(w, lo, hi);
    *reinterpret_cast<uint2 *>(codes + blk * 8) = make_uint2(lo, hi);
    scales[blk] = (uint8_t)sb;
}

// ---------------------------------------------------------------- buffer loads
// Raw buffer resources over the arrays a kernel streams.  A buffer load whose
// offset is past the resource's size returns zeros without a memory access;
// loads with nothing to fetch (rows past N, blocks past a row, the K tail)
// use the offset kOob, so every lane and every path issues the same loads
// and the hardware wait counts stay exact.
constexpr int kOob = 0x7FFFFFF0;
constexpr int kRsrcWord3 = 0x00020000;    // raw 32-bit buffer, gfx9 family
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcWord3);
}
// The offset goes through an empty asm so that it is one VGPR value: left
// as a select between a computed offset and the constant kOob, the compiler
// splits the load into two exec-masked loads of the same registers and waits
// for the first before issuing the second, which serialises the stream.
__device__ __forceinline__ int opaque(int v) {
    __asm__ volatile("" : "+v"(v));
    return v;
}
__device__ __forceinline__ u32x4_t load16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x2_t load8(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t load2(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t load1(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
// Streaming variants with the non-temporal cache policy (bit 1 of the
// cache-policy operand on gfx950), for data read once.
constexpr int kPolicyNt = 2;
// Loads that bypass the CU's L1 and are served by the XCD's L2 (sc0): how a
// workgroup reads values another workgroup of the same XCD stored in the
// same launch.
constexpr int kPolicySc0 = 1;
__device__ __forceinline__ u32x2_t load8_nt(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kPolicyNt));
}
__device__ __forceinline__ uint32_t load1_nt(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, kPolicyNt);
}

// ---------------------------------------------------------------- timelines
// Per-wave stamps of the 100 MHz real-time counter at named points of a
// kernel, for the measurement build only (compiled with BILOCO_TIMELINE: a
// library of its own; in the product library the macros are empty).  Slot
// pt of wave w of workgroup b: tl[(b * 8 + w) * kTlSlots + pt], workgroups
// below kTlMaxWorkgroups; written by lane 0 with an ordinary vector store.
constexpr int kTlSlots = 16, kTlMaxWorkgroups = 4096;
#ifdef BILOCO_TIMELINE
#define BILOCO_TL_AT(buf, pt, v)                                                              \
    do {                                                                                       \
        if ((threadIdx.x & 63) == 0 && blockIdx.x < (unsigned)kTlMaxWorkgroups)               \
            (buf)[((int)blockIdx.x * 8 + (int)(threadIdx.x >> 6)) * kTlSlots + (pt)] = (v);   \
    } while (0)
#else
#define BILOCO_TL_AT(buf, pt, v) do { } while (0)
#endif

// ---------------------------------------------------------------- hand-offs
// Values one workgroup publishes for others of the same launch.  Relaxed
// agent-scope atomics are coherent per access across the XCDs' L2 caches
// (sc1), with no cache-wide fence.  A tagged word carries the fp32 (or
// 32-bit) value with the call's tag in its high half, so data and tag travel
// together and a reader can tell a value of this call from a stale one.
__device__ __forceinline__ uint32_t ld_u32(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u32(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_tagged_u32(uint64_t *p, uint32_t v, uint32_t tag) {
    __hip_atomic_store(p, ((uint64_t)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_tagged(uint64_t *p, float v, uint32_t tag) {
    st_tagged_u32(p, __float_as_uint(v), tag);
}
// agent-scope loads (sc1) through a buffer resource: ordinary vector loads
// for the wait counters
constexpr int kPolicySc1 = 16;
__device__ __forceinline__ uint64_t ld_tagged(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kPolicySc1));
}
__device__ __forceinline__ u32x4_t load16_sc1(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kPolicySc1));
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Sum over the 64 lanes, returned (uniform) to every lane: DPP sums inside
// each row of 16 lanes (quad pairs, quads, half-row mirror, row mirror),
// then the four row sums are read into scalars.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += dpp_mov<0xB1>(v);     // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);     // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);    // row_half_mirror
    v += dpp_mov<0x140>(v);    // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

}  // namespace biloco
