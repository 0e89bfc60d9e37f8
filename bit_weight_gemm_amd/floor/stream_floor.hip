// Measurement only (bench.py's stream-floor leg; not part of libbiloco_hip):
// the time a launch takes to read a given number of bytes with nothing else
// to do, and the time of an empty launch.  These are the floors a product
// call of the same byte count is compared with: one launch, one pass over
// the bytes from HBM.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 512;
constexpr int kRsrcWord3 = 0x00020000;

// Workgroup b reads 16-byte units [b 512 J, (b + 1) 512 J): every thread
// requests its J units at once (non-temporal, as the product streams R),
// then folds them; units past the end read zeros (buffer bounds).  The fold
// goes to memory only if it equals a value no input here produces, which
// the compiler cannot know: the loads are not removed.
template <int J>
__global__ void __launch_bounds__(kThreads) floor_read_kernel(const void *p, int64_t bytes,
                                                              uint32_t *out) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(p), (short)0, (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF), kRsrcWord3);
    const int64_t base = (int64_t)blockIdx.x * kThreads * J + threadIdx.x;
    uint32_t v[J][4];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int64_t u = base + (int64_t)kThreads * j;
        const auto q = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(u * 16 < 0x7FFFFFF0 ? u * 16 : 0x7FFFFFF0), 0, 2);
        v[j][0] = q[0]; v[j][1] = q[1]; v[j][2] = q[2]; v[j][3] = q[3];
    }
    uint32_t acc = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    if (acc == 0x9E3779B9u) out[blockIdx.x] = acc;
}

__global__ void floor_empty_kernel() {}

}  // namespace

extern "C" int biloco_floor_read(const void *p, int64_t bytes, uint32_t *out, int32_t target_grid,
                                 hipStream_t stream) {
    if (!p || !out || bytes <= 0 || bytes > 0x7FFFFFF0 || target_grid < 1) return 1;
    const int64_t units = (bytes + 15) / 16;
    // the fewest units per thread (of 4, 8, 16, 32) that keep the grid at
    // or below the target (about one workgroup per CU)
    int J = 4;
    while (J < 32 && (units + (int64_t)kThreads * J - 1) / ((int64_t)kThreads * J) > target_grid) J *= 2;
    const unsigned grid = (unsigned)((units + (int64_t)kThreads * J - 1) / ((int64_t)kThreads * J));
    switch (J) {
        case 4: hipLaunchKernelGGL(floor_read_kernel<4>, dim3(grid), dim3(kThreads), 0, stream, p, bytes, out); break;
        case 8: hipLaunchKernelGGL(floor_read_kernel<8>, dim3(grid), dim3(kThreads), 0, stream, p, bytes, out); break;
        case 16: hipLaunchKernelGGL(floor_read_kernel<16>, dim3(grid), dim3(kThreads), 0, stream, p, bytes, out); break;
        default: hipLaunchKernelGGL(floor_read_kernel<32>, dim3(grid), dim3(kThreads), 0, stream, p, bytes, out); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

extern "C" int biloco_floor_empty(hipStream_t stream) {
    hipLaunchKernelGGL(floor_empty_kernel, dim3(1), dim3(64), 0, stream);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}
