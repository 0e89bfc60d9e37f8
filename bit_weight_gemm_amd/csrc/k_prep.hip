// Operand preparation kernels: sign packing and activation FP4 quantisation.
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

// One thread per block of 16 activations (row m, block b): two 16-byte loads,
// amax by integer max over the magnitude bits (bf16 magnitudes order like
// integers), scale = E4M3(amax / 6) with a correctly rounded fp32 division,
// codes by exact comparisons with the E2M1 midpoints times the scale; one
// 8-byte store of the codes and one byte of scale.
__global__ void __launch_bounds__(256)
quant_act_kernel(const uint16_t *__restrict__ x, int64_t nblocks, uint8_t *__restrict__ codes,
                 uint8_t *__restrict__ scales) {
    const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (blk >= nblocks) return;
    const uint4 *src = reinterpret_cast<const uint4 *>(x + blk * 16);
    const uint4 v0 = src[0], v1 = src[1];
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t amax_bits = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        amax_bits = max(amax_bits, w[j] & 0x7FFFu);
        amax_bits = max(amax_bits, (w[j] >> 16) & 0x7FFFu);
    }
    const float amax = bf16_to_f32(amax_bits);
    const uint32_t sb = f32_to_e4m3_rne(amax / 6.0f);
    const float s = e4m3_to_f32(sb);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const uint32_t h = (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu);
        const float a = bf16_to_f32(h & 0x7FFFu);
        const uint32_t mag = (sb == 0u) ? 0u : e2m1_mag_code(a, s);
        const uint32_t code = mag | ((h >> 12) & 8u);
        if (j < 8) lo |= code << (4 * j);
        else hi |= code << (4 * (j - 8));
    }
    *reinterpret_cast<uint2 *>(codes + blk * 8) = make_uint2(lo, hi);
    scales[blk] = (uint8_t)sb;
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
