// Schedule BILOCO_SCHED_COMPOSED: the product as a composition of separate
// launches, the unfused form the BiLoCo README's layout keeps next to its
// fused kernel (section "Layout": an unfused reference in the launcher and in
// the extension) and that the fused kernel is timed against:
//   1. G = g * Q4(x) . deq(R)^T            the plain FP4 product (r = 0 path), fp32
//   2. z = alpha (.) (x . V)                fp32, workspace
//   3. y = bf16(G + z . U^T)                the correction
// Each launch is this library's kernel for that part; only the hand-off
// differs from the fused schedules (G makes an fp32 round trip through HBM
// and z is complete before the correction starts).
//
// Two routes for the correction, the two ways of multiplying by +-1 signs
// that the pages weigh (schedule BILOCO_SCHED_COMPOSED and
// BILOCO_SCHED_COMPOSED_MFMA):
//  * lookup tables: 4 sign-adds become one table lookup (the sub-vector
//    lookup tables of FluxBin, prior art the BiLoCo README cites for binary
//    products): for a row m and four consecutive indices 4q..4q+3, the 16
//    sums sum_j (+-1) z[m][4q+j] over every sign pattern are built once in
//    LDS, and each output then adds one entry per 4-bit nibble of its U word;
//  * matrix cores: bf16 MFMAs of z (high + low parts) against U's signs.
#include "biloco_device.h"
#include "biloco_internal.h"

namespace biloco {

constexpr int kLutThreads = 256;     // outputs n per workgroup
constexpr int kLutRows = 2;          // batch rows m per workgroup

// LDS: lut[row][q][16], q < rpad / 4.  Entry (row, q, nib) = sum over j < 4
// of (bit j of nib ? -1 : +1) * z[m][4q + j], with z taken as 0 for indices
// >= r (their sign bits are 0 in U).  y = bf16(yf + correction).
__global__ void __launch_bounds__(kLutThreads)
lut_correction_kernel(const float *__restrict__ z, int rpad, const uint32_t *__restrict__ u,
                      const float *__restrict__ yf, int M, int N, int r,
                      uint16_t *__restrict__ y) {
    extern __shared__ float lut[];
    const int Q = rpad / 4, W = rpad / 32;
    const int m0 = blockIdx.y * kLutRows;
    const int rows = M - m0 < kLutRows ? M - m0 : kLutRows;
    for (int task = threadIdx.x; task < rows * Q; task += kLutThreads) {
        const int row = task / Q, q = task - row * Q, i0 = 4 * q;
        const float *zr = z + (int64_t)(m0 + row) * rpad + i0;
        float zz[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) zz[j] = i0 + j < r ? zr[j] : 0.0f;
        float *dst = lut + (int64_t)task * 16;
#pragma unroll
        for (int nib = 0; nib < 16; ++nib) {
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) s += ((nib >> j) & 1) ? -zz[j] : zz[j];
            dst[nib] = s;
        }
    }
    __syncthreads();
    const int n = blockIdx.x * kLutThreads + threadIdx.x;
    if (n >= N) return;
    float acc[kLutRows] = {};
    for (int w = 0; w < W; ++w) {
        const uint32_t word = u[(int64_t)w * N + n];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int off = (8 * w + k) * 16 + ((word >> (4 * k)) & 15u);
#pragma unroll
            for (int row = 0; row < kLutRows; ++row)
                if (row < rows) acc[row] += lut[row * Q * 16 + off];
        }
    }
#pragma unroll
    for (int row = 0; row < kLutRows; ++row)
        if (row < rows) {
            const int64_t idx = (int64_t)(m0 + row) * N + n;
            y[idx] = f32_to_bf16_rne(yf[idx] + acc[row]);
        }
}

// ---------------------------------------------------------------------------
// The same correction on the matrix cores (the +-1 route): y = bf16(yf + Z U^T)
// with Z = z split into bf16 high + low parts (A operand) and U's signs as
// bf16 +-1 (B operand) of v_mfma_f32_16x16x32_bf16; the 32 ranks of one U
// word are one MFMA's K.  Workgroup = 16 outputs n and every batch row; its 4
// waves take every fourth U word and meet in LDS at the end.
typedef __bf16 bf16x8c_t __attribute__((ext_vector_type(8)));
typedef float float4c_t __attribute__((ext_vector_type(4)));
constexpr int kMcRound = 4;            // U words of a wave whose loads issue together

__device__ __forceinline__ float4c_t mfma_bf16c(const u32x4_t &a, const u32x4_t &b, float4c_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8c_t, a),
                                                   __builtin_bit_cast(bf16x8c_t, b), c, 0, 0, 0);
}

// B operand of lane (n, grp): ranks 8 grp + e, e = 0..7, from word t; bf16
// pair d holds ranks 8 grp + 2d (low half) and 8 grp + 2d + 1 (high half).
__device__ __forceinline__ u32x4_t signs_b(uint32_t t, int grp) {
    const uint32_t s = t >> (8 * grp);
    u32x4_t b;
#pragma unroll
    for (int d = 0; d < 4; ++d)
        b[d] = ((s << (15 - 2 * d)) & 0x8000u) | ((s << (30 - 2 * d)) & 0x80000000u) | 0x3F803F80u;
    return b;
}

template <int MB>
__global__ void __launch_bounds__(256)
mfma_correction_kernel(const float *__restrict__ z, int rpad, const uint32_t *__restrict__ u,
                       const float *__restrict__ yf, int M, int N, int r, uint16_t *__restrict__ y) {
    __shared__ float4c_t red[4][MB][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
    const int n = blockIdx.x * 16 + col;
    const int W = rpad / 32;
    float4c_t acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = float4c_t{0.f, 0.f, 0.f, 0.f};
    // this wave's words w = wave + 4 j, in rounds of kMcRound words: every
    // load of a round is issued before its MFMAs
    for (int w0 = wave; w0 < W; w0 += 4 * kMcRound) {
        uint32_t t[kMcRound];
        float4 zq[kMcRound][MB][2];
#pragma unroll
        for (int j = 0; j < kMcRound; ++j) {
            const int w = w0 + 4 * j;
            t[j] = (n < N && w < W) ? u[(int64_t)w * N + n] : 0u;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int m = 16 * mb + col;
                const float *zr = z + (int64_t)(m < M ? m : 0) * rpad + 32 * (w < W ? w : 0) + 8 * grp;
                zq[j][mb][0] = *reinterpret_cast<const float4 *>(zr);
                zq[j][mb][1] = *reinterpret_cast<const float4 *>(zr + 4);
            }
        }
#pragma unroll
        for (int j = 0; j < kMcRound; ++j) {
            const int w = w0 + 4 * j;
            if (w >= W) break;
            const u32x4_t b = signs_b(t[j], grp);
            const int i0 = 32 * w + 8 * grp;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                // A operand: row m = 16 mb + lane % 16, ranks i0 .. i0 + 7
                const bool live = 16 * mb + col < M;
                const float v8[8] = {zq[j][mb][0].x, zq[j][mb][0].y, zq[j][mb][0].z, zq[j][mb][0].w,
                                     zq[j][mb][1].x, zq[j][mb][1].y, zq[j][mb][1].z, zq[j][mb][1].w};
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = (live && i0 + e < r) ? v8[e] : 0.0f;
                u32x4_t ah, al;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t h0 = f32_to_bf16_rne(v[2 * d]), h1 = f32_to_bf16_rne(v[2 * d + 1]);
                    ah[d] = h0 | (h1 << 16);
                    al[d] = f32_to_bf16_rne(v[2 * d] - bf16_to_f32(h0)) |
                            (f32_to_bf16_rne(v[2 * d + 1] - bf16_to_f32(h1)) << 16);
                }
                acc[mb] = mfma_bf16c(ah, b, acc[mb]);
                acc[mb] = mfma_bf16c(al, b, acc[mb]);
            }
        }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[wave][mb][lane] = acc[mb];
    __syncthreads();
    if (wave != 0 || n >= N) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const float4c_t s = (red[0][mb][lane] + red[1][mb][lane]) + (red[2][mb][lane] + red[3][mb][lane]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 16 * mb + 4 * grp + e;
            if (m < M) {
                const int64_t idx = (int64_t)m * N + n;
                y[idx] = f32_to_bf16_rne(yf[idx] + s[e]);
            }
        }
    }
}

bool composed_supported(int M, int N, int K, int r) {
    (void)N;
    (void)K;
    return M >= 1 && M <= 32 && r >= 0 && r <= kComposedMaxRank;
}

hipError_t launch_gemm_composed(const GemmArgs &a, bool mfma_correction, hipStream_t stream) {
    if (!composed_supported(a.M, a.N, a.K, a.r)) return hipErrorNotSupported;
    // 1. the plain product, through the fastest r = 0 schedule of the shape;
    // its split-K partials (if any) have their own workspace area, apart
    // from the z kernel's counters
    GemmArgs g0 = a;
    g0.r = 0;
    if (a.r > 0) g0.yf = reinterpret_cast<float *>(static_cast<char *>(a.ws) +
                                                   ws_yf_offset(a.M, a.N, a.K, a.r));
    g0.x = nullptr;
    g0.v = g0.u = nullptr;
    g0.alpha = nullptr;
    if (a.r > 0) {
        g0.ws = static_cast<char *>(a.ws) + ws_g0_offset(a.M, a.N, a.K, a.r);
        g0.ws_bytes = a.ws_bytes - ws_g0_offset(a.M, a.N, a.K, a.r);
        g0.ws_is_mfma_area = true;
    }
    hipError_t e;
    if (a.M >= 3 && mfma_supported(a.M, a.N, a.K, 0)) {
        if (mfma_ws_bytes(a.M, a.N, a.K, 0) > g0.ws_bytes) return hipErrorInvalidValue;
        e = launch_gemm_mfma(g0, stream);
    } else {
        e = launch_gemm_unfused(g0, stream);
    }
    if (e != hipSuccess || a.r == 0) return e;
    // 2. z, plain fp32
    float *z = reinterpret_cast<float *>(static_cast<char *>(a.ws) + ws_zf_offset(a.M, a.r));
    e = launch_z_fp32(a, z, stream);
    if (e != hipSuccess) return e;
    // 3. the correction
    const int rpad = rpad32(a.r);
    if (mfma_correction) {
        const dim3 grid((unsigned)((a.N + 15) / 16));
        if (a.M <= 16)
            hipLaunchKernelGGL(mfma_correction_kernel<1>, grid, dim3(256), 0, stream, z, rpad, a.u,
                               g0.yf, a.M, a.N, a.r, a.y);
        else
            hipLaunchKernelGGL(mfma_correction_kernel<2>, grid, dim3(256), 0, stream, z, rpad, a.u,
                               g0.yf, a.M, a.N, a.r, a.y);
        return hipGetLastError();
    }
    const size_t lds = (size_t)kLutRows * (size_t)(rpad / 4) * 16 * sizeof(float);
    const dim3 grid((unsigned)((a.N + kLutThreads - 1) / kLutThreads),
                    (unsigned)((a.M + kLutRows - 1) / kLutRows));
    hipLaunchKernelGGL(lut_correction_kernel, grid, dim3(kLutThreads), lds, stream, z, rpad, a.u,
                       g0.yf, a.M, a.N, a.r, a.y);
    return hipGetLastError();
}

}  // namespace biloco
