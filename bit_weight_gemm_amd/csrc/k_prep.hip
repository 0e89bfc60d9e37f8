// Operand preparation kernels: sign packing, activation FP4 quantisation and
// NVFP4 quantisation of the weight residual.
// BiLoCo README, section "Kernel": the launcher receives pack_signs(V.T) and
// pack_signs(U.T), and the product consumes FP4(x) as NVFP4 codes + scales.
#include "biloco_device.h"
#include "biloco_internal.h"

namespace biloco {

// One thread per output word (w, c): bit b <- signs[32w+b][c] < 0.  Adjacent
// threads read adjacent columns, so every byte load of a wave is contiguous.
__global__ void __launch_bounds__(256)
pack_signs_kernel(const int8_t *__restrict__ signs, int64_t rows, int64_t cols,
                  int64_t col_blocks, uint32_t *__restrict__ packed) {
    const int64_t w = blockIdx.x / col_blocks;
    const int64_t c = (blockIdx.x % col_blocks) * 256 + threadIdx.x;
    if (c >= cols) return;
    const int64_t r0 = w * 32;
    const int nb = (int)((rows - r0) < 32 ? (rows - r0) : 32);
    const int8_t *src = signs + r0 * cols + c;
    uint32_t word = 0;
    for (int b = 0; b < nb; ++b) word |= (uint32_t)(src[(int64_t)b * cols] < 0) << b;
    packed[w * cols + c] = word;
}

hipError_t launch_pack_signs(const int8_t *signs, int64_t rows, int64_t cols, uint32_t *packed,
                             hipStream_t stream) {
    const int64_t W = (rows + 31) / 32;
    const int64_t cb = (cols + 255) / 256;
    if (W * cb > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pack_signs_kernel, dim3((unsigned)(W * cb)), dim3(256), 0, stream, signs,
                       rows, cols, cb, packed);
    return hipGetLastError();
}

// One thread per block of 16 activations (row m, block b); the arithmetic is
// quant_act_block (biloco_device.h).
__global__ void __launch_bounds__(256)
quant_act_kernel(const uint16_t *__restrict__ x, int64_t nblocks, uint8_t *__restrict__ codes,
                 uint8_t *__restrict__ scales) {
    const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (blk >= nblocks) return;
    quant_act_block(x, blk, codes, scales);
}

hipError_t launch_quant_act(const uint16_t *x, int M, int K, uint8_t *codes, uint8_t *scales,
                            hipStream_t stream) {
    const int64_t nblocks = (int64_t)M * (K / 16);
    const int64_t grid = (nblocks + 255) / 256;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)grid), dim3(256), 0, stream, x, nblocks,
                       codes, scales);
    return hipGetLastError();
}

}  // namespace biloco

namespace biloco {

// ---------------------------------------------------------------- NVFP4 weights
// Quantisation of an fp32 weight matrix (the residual R of the BiLoCo README's
// intro and section "Decomposition", which it stores in NVFP4; section
// "Kernel" gives the stored form: codes, E4M3 block scales, fp32 global
// scale).  g = max|w| / (6 * 448) puts the largest block scale on the largest
// E4M3 value.  The matrix is one flat run of N*K floats (K % 16 == 0, so no
// block straddles a row): lane l of a wave owns one float4, a quad of lanes
// owns one block of 16, and the block maximum is two DPP steps inside the
// quad.  Two launches: the global maximum needs every element before the
// first scale can be rounded.
constexpr int kWqThreads = 256;
constexpr int kWqAmaxUnroll = 8;       // float4 loads in flight per thread, pass 1
constexpr int kWqQuantUnroll = 4;      // pass 2
constexpr int kWqAmaxGrid = 512;       // most pass-1 partials (the workspace holds them)
constexpr int kWqQuantGrid = 2048;

__device__ __forceinline__ uint32_t abs_max4(float4 v) {
    const uint32_t m = 0x7FFFFFFFu;
    return max(max(__float_as_uint(v.x) & m, __float_as_uint(v.y) & m),
               max(__float_as_uint(v.z) & m, __float_as_uint(v.w) & m));
}

// Unsigned maximum over the 64 lanes (finite non-negative floats order like
// their bit patterns).
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}

__device__ __forceinline__ uint32_t block_umax(uint32_t v, uint32_t *lds) {
    v = wave_umax(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds[wave] = v;
    __syncthreads();
    v = lds[0];
#pragma unroll
    for (int i = 1; i < kWqThreads / 64; ++i) v = max(v, lds[i]);
    return v;
}

// Pass 1: one max |w| per workgroup over a grid-stride share of tiles of
// kWqThreads * kWqAmaxUnroll float4.  Full tiles load without checks; the one
// ragged tile (if any) is taken by the workgroup its index falls on.
__global__ void __launch_bounds__(kWqThreads)
wq_amax_kernel(const float4 *__restrict__ w, int64_t n4, uint32_t *__restrict__ part) {
    __shared__ uint32_t lds[kWqThreads / 64];
    constexpr int64_t kTile = (int64_t)kWqThreads * kWqAmaxUnroll;
    const int64_t full = n4 / kTile;
    uint32_t m = 0;
    for (int64_t t = blockIdx.x; t < full; t += gridDim.x) {
        const float4 *src = w + t * kTile + threadIdx.x;
        float4 v[kWqAmaxUnroll];
#pragma unroll
        for (int j = 0; j < kWqAmaxUnroll; ++j) v[j] = src[j * kWqThreads];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kWqAmaxUnroll; ++j) m = max(m, abs_max4(v[j]));
    }
    if (full * kTile < n4 && (int64_t)blockIdx.x == full % gridDim.x) {
        for (int64_t i = full * kTile + threadIdx.x; i < n4; i += kWqThreads) m = max(m, abs_max4(w[i]));
    }
    m = block_umax(m, lds);
    if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// The block maximum of the quad that holds lane l's float4 (all four lanes
// of the quad must be active).
__device__ __forceinline__ float quad_amax(float4 v) {
    uint32_t am = abs_max4(v);
    am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
    am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
    return __uint_as_float(am);
}

// Correctly rounded quotient n / b from the correctly rounded reciprocal
// rb = fp32(1 / b): one product, its exact residual by a fused multiply-add,
// and one corrective fused multiply-add (P. Markstein, "Computation of
// elementary functions on the IBM RISC System/6000 processor", 1990).  The
// three roundings give fp32(n / b) exactly wherever this file relies on it,
// which was checked exhaustively on the CPU: for n / 6 over every float
// n >= 2^-124; for t / g near every E4M3 rounding midpoint and |w| / d near
// every E2M1 midpoint, over every 24-bit divisor significand at divisor
// exponents from -99 to 100 (normal operands and quotients).  Away from those
// midpoints a quotient within a few units in the last place rounds to the
// same code.
__device__ __forceinline__ float quotient(float n, float b, float rb) {
    const float q0 = n * rb;
    const float r = __builtin_fmaf(-b, q0, n);
    return __builtin_fmaf(r, rb, q0);
}

// Fast path of a quad's block (global scale g >= 2^-90, so every nonzero
// block scale gives d >= 2^-99 and the quotients above stay in their checked
// range).  tab[s] = (d, fp32(1 / d)) with d = fp32(e4m3(s) * g), and (1, 0)
// for s = 0, which turns every quotient into a signed zero.  The E4M3 byte is
// the hardware conversion of q <= 448 (round to nearest even; its only
// difference from saturation is above 464) and the E2M1 nibbles are the
// hardware conversion with unit scale (round to nearest even, saturating at
// 6, sign kept on zero): both checked against the format definitions on
// gfx950 over every rounding midpoint and its neighbours.
__device__ __forceinline__ uint32_t wq_quant4_fast(float4 v, float g, float rg, const float2 *tab,
                                                   uint32_t *sb_out) {
    constexpr float kRcp6 = 1.0f / 6.0f;     // fp32(1/6)
    const float t = quotient(quad_amax(v), 6.0f, kRcp6);
    const float q = fminf(quotient(t, g, rg), 448.0f);
    const uint32_t sb = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q, q, 0, false) & 0xFFu;
    const float2 dy = tab[sb];
    const float e[4] = {v.x, v.y, v.z, v.w};
    float y[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t bits = __float_as_uint(e[k]);
        const float a = quotient(__uint_as_float(bits & 0x7FFFFFFFu), dy.x, dy.y);
        y[k] = __uint_as_float(__float_as_uint(a) | (bits & 0x80000000u));
    }
    uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[0], y[1], 1.0f, 0);
    c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, y[2], y[3], 1.0f, 1);
    *sb_out = sb;
    return c & 0xFFFFu;
}

// Exact path (any g, used when g < 2^-90): correctly rounded divisions and
// comparisons with the E2M1 midpoints, as the definition reads.
__device__ __forceinline__ uint32_t wq_quant4_exact(float4 v, float g, uint32_t *sb_out) {
    const float t = quad_amax(v) / 6.0f;
    float q = t / g;
    q = (q == q) ? q : 0.0f;                 // 0/0 only when g underflowed and the block is 0
    const uint32_t sb = f32_to_e4m3_rne(q);
    const float d = e4m3_to_f32(sb) * g;
    const float e[4] = {v.x, v.y, v.z, v.w};
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t bits = __float_as_uint(e[k]);
        const uint32_t mag = d == 0.0f ? 0u : e2m1_mag_code(__uint_as_float(bits & 0x7FFFFFFFu) / d, 1.0f);
        c |= (mag | ((bits >> 28) & 8u)) << (4 * k);
    }
    *sb_out = sb;
    return c;
}

template <bool FAST>
__device__ __forceinline__ uint32_t wq_quant4(float4 v, float g, float rg, const float2 *tab,
                                              uint32_t *sb) {
    if constexpr (FAST) return wq_quant4_fast(v, g, rg, tab, sb);
    else return wq_quant4_exact(v, g, sb);
}

// The tiles of one workgroup: full tiles of kWqThreads * kWqQuantUnroll
// float4 without checks, then the ragged tile if this workgroup owns it.
// n4 is a multiple of 4, so every quad is wholly in or out; lanes past the
// end compute on zeros (all lanes stay active for the DPP steps) and store
// nothing.  One 2-byte code store per lane, one scale byte per quad.
template <bool FAST>
__device__ __forceinline__ void wq_tiles(const float4 *__restrict__ w, int64_t n4, float g,
                                         float rg, const float2 *tab, uint16_t *__restrict__ codes,
                                         uint8_t *__restrict__ scales) {
    constexpr int64_t kTile = (int64_t)kWqThreads * kWqQuantUnroll;
    const int64_t full = n4 / kTile;
    const bool lead = (threadIdx.x & 3) == 0;
    for (int64_t t = blockIdx.x; t < full; t += gridDim.x) {
        const int64_t i0 = t * kTile + threadIdx.x;
        float4 v[kWqQuantUnroll];
#pragma unroll
        for (int j = 0; j < kWqQuantUnroll; ++j) v[j] = w[i0 + j * kWqThreads];
        // all loads of the tile issue before any arithmetic (left alone, the
        // scheduler pulls the first block's work up and waits for its load
        // before issuing the others)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kWqQuantUnroll; ++j) {
            const int64_t i = i0 + j * kWqThreads;
            uint32_t sb;
            codes[i] = (uint16_t)wq_quant4<FAST>(v[j], g, rg, tab, &sb);
            if (lead) scales[i >> 2] = (uint8_t)sb;
        }
    }
    if (full * kTile < n4 && (int64_t)blockIdx.x == full % gridDim.x) {
        for (int64_t base = full * kTile; base < n4; base += kWqThreads) {
            const int64_t i = base + threadIdx.x;
            const bool in = i < n4;
            const float4 v = in ? w[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            uint32_t sb;
            const uint32_t c = wq_quant4<FAST>(v, g, rg, tab, &sb);
            if (in) {
                codes[i] = (uint16_t)c;
                if (lead) scales[i >> 2] = (uint8_t)sb;
            }
        }
    }
}

// Pass 2: every workgroup reduces the pass-1 partials to max|w| and g
// (workgroup 0 stores g), builds its (d, 1/d) table, then quantises a
// grid-stride share of the tiles.
__global__ void __launch_bounds__(kWqThreads)
wq_quant_kernel(const float4 *__restrict__ w, int64_t n4, const uint32_t *__restrict__ part,
                int nparts, uint16_t *__restrict__ codes, uint8_t *__restrict__ scales,
                float *__restrict__ g_out) {
    __shared__ uint32_t lds[kWqThreads / 64];
    __shared__ float2 tab[128];
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nparts; i += kWqThreads) m = max(m, part[i]);
    const float amax = __uint_as_float(block_umax(m, lds));
    const float g = amax > 0.0f ? amax / 2688.0f : 1.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) *g_out = g;
    if (g >= 0x1p-90f) {                     // uniform over the grid
        if (threadIdx.x < 128) {
            const float d = e4m3_to_f32(threadIdx.x) * g;
            tab[threadIdx.x] = threadIdx.x == 0 ? make_float2(1.0f, 0.0f) : make_float2(d, 1.0f / d);
        }
        __syncthreads();
        wq_tiles<true>(w, n4, g, 1.0f / g, tab, codes, scales);
    } else {
        wq_tiles<false>(w, n4, g, 0.0f, tab, codes, scales);
    }
}

size_t quant_weight_ws_bytes() { return (size_t)4 * kWqAmaxGrid; }

hipError_t launch_quant_weight(const float *w, int64_t N, int64_t K, uint8_t *codes,
                               uint8_t *scales, float *g_out, void *ws, hipStream_t stream) {
    const int64_t n4 = N * K / 4;
    const int64_t t1 = (n4 + (int64_t)kWqThreads * kWqAmaxUnroll - 1) / ((int64_t)kWqThreads * kWqAmaxUnroll);
    const int64_t t2 = (n4 + (int64_t)kWqThreads * kWqQuantUnroll - 1) / ((int64_t)kWqThreads * kWqQuantUnroll);
    const int g1 = (int)(t1 < kWqAmaxGrid ? t1 : kWqAmaxGrid);
    const int g2 = (int)(t2 < kWqQuantGrid ? t2 : kWqQuantGrid);
    uint32_t *part = static_cast<uint32_t *>(ws);
    hipLaunchKernelGGL(wq_amax_kernel, dim3(g1), dim3(kWqThreads), 0, stream,
                       reinterpret_cast<const float4 *>(w), n4, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(wq_quant_kernel, dim3(g2), dim3(kWqThreads), 0, stream,
                       reinterpret_cast<const float4 *>(w), n4, part, g1,
                       reinterpret_cast<uint16_t *>(codes), scales, g_out);
    return hipGetLastError();
}

}  // namespace biloco
