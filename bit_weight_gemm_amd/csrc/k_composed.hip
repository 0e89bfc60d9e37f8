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
// The correction replaces 4 sign-adds by one table lookup (the sub-vector
// lookup tables of FluxBin, prior art the BiLoCo README cites for binary
// products): for a row m and four consecutive indices 4q..4q+3, the 16 sums
// sum_j (+-1) z[m][4q+j] over every sign pattern are built once in LDS, and
// each output then adds one entry per 4-bit nibble of its U word.
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

bool composed_supported(int M, int N, int K, int r) {
    (void)N;
    (void)K;
    return M >= 1 && M <= 32 && r >= 0 && r <= kComposedMaxRank;
}

hipError_t launch_gemm_composed(const GemmArgs &a, hipStream_t stream) {
    if (!composed_supported(a.M, a.N, a.K, a.r)) return hipErrorNotSupported;
    // 1. the plain product, through the fastest r = 0 schedule of the shape;
    // its workspace (split-K partials, if any) sits in the matrix-core area
    // of this call's workspace, which is at least as large
    GemmArgs g0 = a;
    g0.r = 0;
    if (a.r > 0) g0.yf = reinterpret_cast<float *>(static_cast<char *>(a.ws) +
                                                   ws_yf_offset(a.M, a.N, a.K, a.r));
    g0.x = nullptr;
    g0.v = g0.u = nullptr;
    g0.alpha = nullptr;
    if (a.r > 0) {
        g0.ws = static_cast<char *>(a.ws) + ws_mfma_offset(a.M, a.r);
        g0.ws_bytes = a.ws_bytes - ws_mfma_offset(a.M, a.r);
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
    const size_t lds = (size_t)kLutRows * (size_t)(rpad / 4) * 16 * sizeof(float);
    const dim3 grid((unsigned)((a.N + kLutThreads - 1) / kLutThreads),
                    (unsigned)((a.M + kLutRows - 1) / kLutRows));
    hipLaunchKernelGGL(lut_correction_kernel, grid, dim3(kLutThreads), lds, stream, z, rpad, a.u,
                       g0.yf, a.M, a.N, a.r, a.y);
    return hipGetLastError();
}

}  // namespace biloco
