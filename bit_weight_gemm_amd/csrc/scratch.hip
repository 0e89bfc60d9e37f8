// The quantise-and-multiply call without a workspace argument, for callers
// that cannot allocate (code under graph capture, tight serving loops,
// harnesses that forbid allocation): its workspace is a file-scope device
// array of fixed size, one copy per GPU, held until the process ends.
#include <mutex>

#include "../../include/biloco.h"
#include "biloco_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;   // BILOCO_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == BILOCO_NOALLOC_SCRATCH_BYTES, "header and source agree");

// Zero-initialised at load, as every device variable without an initializer:
// the state the library needs at a workspace's first use.  In host code this
// name is a stand-in, not a device address; only its per-device address,
// taken once below, is ever used.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_addr[kMaxDevices];

// The current device's copy of the array (its address is taken on the first
// call on that device and kept).
hipError_t scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_addr[dev] = p;
    }
    *out = g_addr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" biloco_status biloco_gemm_lowrank_quant_noalloc(
    const uint16_t *x_bf16, uint8_t *a_codes, uint8_t *a_scales, const uint8_t *w_codes,
    const uint8_t *w_scales, float w_global_scale, const uint32_t *v_packed,
    const uint32_t *u_packed, const uint16_t *alpha_bf16, int32_t M, int32_t N, int32_t K, int32_t r,
    uint16_t *y_bf16, int32_t schedule, hipStream_t stream) {
    size_t need = 0;
    const biloco_status st = biloco_gemm_workspace_bytes(M, N, K, r, &need);
    if (st != BILOCO_OK) return st;
    if (need > kScratchBytes) return BILOCO_ERR_UNSUPPORTED;   // the shape needs more than the array
    void *ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return BILOCO_ERR_HIP;
    return biloco_gemm_lowrank_quant(x_bf16, a_codes, a_scales, w_codes, w_scales, w_global_scale,
                                     v_packed, u_packed, alpha_bf16, M, N, K, r, y_bf16, ws,
                                     kScratchBytes, schedule, stream);
}
