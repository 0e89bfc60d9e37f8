// Two-launch composition of the product (schedule BILOCO_SCHED_UNFUSED):
//   launch 1: z[m][i] = alpha_i * sum_k x[m][k] V[k][i]       (fp32, workspace)
//   launch 2: y[m][n] = bf16(g * sum_k A[m][k] B[n][k] + sum_i z[m][i] U[n][i])
// BiLoCo README, section "Kernel" (the fused product; the side work that
// produces z; the epilogue expansion of z through U), and its layout list,
// which keeps an unfused reference next to the fused kernel.  This is the
// plain composition: every output is finished by one wave, and z is complete
// before launch 2 starts because both launches are ordered on one stream.
#include "biloco_device.h"
#include "biloco_internal.h"

namespace biloco {

// One workgroup per (32-wide group of i, row m).  Threads stride over k; each
// keeps 32 partial sums, one per sign bit of the word V[w][k] (the sign of
// x[m][k] is flipped where the bit is 1), then the block sums them.
__global__ void __launch_bounds__(256)
z_unfused_kernel(const uint16_t *__restrict__ x, const uint32_t *__restrict__ v,
                 const uint16_t *__restrict__ alpha, int K, int r, int rpad,
                 float *__restrict__ z) {
    const int w = blockIdx.x, m = blockIdx.y;
    float acc[32];
#pragma unroll
    for (int b = 0; b < 32; ++b) acc[b] = 0.0f;
    const uint32_t *vrow = v + (int64_t)w * K;
    const uint16_t *xrow = x + (int64_t)m * K;
    for (int k = threadIdx.x; k < K; k += 256) {
        const uint32_t word = vrow[k];
        const uint32_t xb = __float_as_uint(bf16_to_f32(xrow[k]));
#pragma unroll
        for (int b = 0; b < 32; ++b)
            acc[b] += __uint_as_float(xb ^ ((word << (31 - b)) & 0x80000000u));
    }
    __shared__ float red[4][32];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int b = 0; b < 32; ++b) {
        const float s = wave_sum(acc[b]);
        if (lane == 0) red[wave][b] = s;
    }
    __syncthreads();
    if (threadIdx.x < 32) {
        const int b = threadIdx.x, i = w * 32 + b;
        if (i < r) {
            const float s = (red[0][b] + red[1][b]) + (red[2][b] + red[3][b]);
            z[(int64_t)m * rpad + i] = s * bf16_to_f32(alpha[i]);
        }
    }
}

// One wave per output row n (grid-stride).  Lanes stride over the 16-element
// blocks of K: each lane dequantises its block of R and of the activation,
// sums the 16 exact products, scales by both block scales, and the wave sums
// the lanes.  The correction reads z and U's packed words for the same n.
__global__ void __launch_bounds__(256)
gemv_unfused_kernel(const uint8_t *__restrict__ a_codes, const uint8_t *__restrict__ a_scales,
                    const uint8_t *__restrict__ w_codes, const uint8_t *__restrict__ w_scales,
                    float g, const uint32_t *__restrict__ u, const float *__restrict__ z, int M,
                    int N, int K, int r, int rpad, uint16_t *__restrict__ y,
                    float *__restrict__ yf) {
    const int lane = threadIdx.x & 63;
    const int64_t gw = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
    const int64_t nw = (int64_t)gridDim.x * 4;
    const int KB = K / 16;
    for (int64_t n = gw; n < N; n += nw) {
        const uint8_t *wc_row = w_codes + n * (K / 2);
        const uint8_t *ws_row = w_scales + n * KB;
        for (int m = 0; m < M; ++m) {
            const uint8_t *ac_row = a_codes + (int64_t)m * (K / 2);
            const uint8_t *as_row = a_scales + (int64_t)m * KB;
            float acc = 0.0f;
            for (int b = lane; b < KB; b += 64) {
                const uint2 wc = *reinterpret_cast<const uint2 *>(wc_row + b * 8);
                const uint2 ac = *reinterpret_cast<const uint2 *>(ac_row + b * 8);
                float p = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    p += e2m1_to_f32((wc.x >> (4 * j)) & 15u) * e2m1_to_f32((ac.x >> (4 * j)) & 15u);
                    p += e2m1_to_f32((wc.y >> (4 * j)) & 15u) * e2m1_to_f32((ac.y >> (4 * j)) & 15u);
                }
                acc += p * (e4m3_to_f32(ws_row[b]) * e4m3_to_f32(as_row[b]));
            }
            float cacc = 0.0f;
            for (int i = lane; i < r; i += 64) {
                const uint32_t word = u[(int64_t)(i >> 5) * N + n];
                const float zz = z[(int64_t)m * rpad + i];
                cacc += ((word >> (i & 31)) & 1u) ? -zz : zz;
            }
            const float gs = wave_sum(acc), cs = wave_sum(cacc);
            if (lane == 0) {
                if (yf) yf[(int64_t)m * N + n] = g * gs + cs;
                else y[(int64_t)m * N + n] = f32_to_bf16_rne(g * gs + cs);
            }
        }
    }
}

hipError_t launch_z_fp32(const GemmArgs &a, float *z, hipStream_t stream) {
    if (a.M <= 2 && gemv_supported(a.M, a.N, a.K, a.r)) return launch_z_gemv(a, z, stream);
    if (mfma_supported(a.M, a.N, a.K, a.r)) return launch_z_mfma(a, z, stream);
    hipLaunchKernelGGL(z_unfused_kernel, dim3(rpad32(a.r) / 32, a.M), dim3(256), 0, stream, a.x,
                       a.v, a.alpha, a.K, a.r, rpad32(a.r), z);
    return hipGetLastError();
}

hipError_t launch_gemm_unfused(const GemmArgs &a, hipStream_t stream) {
    // small batches: the z kernel and the streaming product kernel of the
    // vector-ALU path
    if (gemv_supported(a.M, a.N, a.K, a.r)) return launch_gemm_gemv_two_launch(a, stream);
    const int rpad = rpad32(a.r);
    float *z = a.r > 0 ? reinterpret_cast<float *>(static_cast<char *>(a.ws) + ws_zf_offset(a.M, a.r))
                       : nullptr;
    if (a.r > 0) {
        hipLaunchKernelGGL(z_unfused_kernel, dim3(rpad / 32, a.M), dim3(256), 0, stream, a.x, a.v,
                           a.alpha, a.K, a.r, rpad, z);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t blocks = ((int64_t)a.N + 3) / 4;
    const unsigned grid = (unsigned)(blocks < 4096 ? blocks : 4096);
    hipLaunchKernelGGL(gemv_unfused_kernel, dim3(grid), dim3(256), 0, stream, a.a_codes,
                       a.a_scales, a.w_codes, a.w_scales, a.g, a.u, z, a.M, a.N, a.K, a.r, rpad,
                       a.y, a.yf);
    return hipGetLastError();
}

}  // namespace biloco
