// One-launch matrix-core schedule (BILOCO_SCHED_FUSED_MFMA): not built yet.
#include "biloco_internal.h"

namespace biloco {

hipError_t launch_gemm_fused_mfma(const GemmArgs &a, hipStream_t stream) {
    (void)a; (void)stream;
    return hipErrorNotSupported;
}

}  // namespace biloco
