// Internal interface between the C ABI layer (biloco_api.cpp) and the HIP
// launch code.  Not installed; not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace biloco {

struct GemmArgs {
    const uint8_t *a_codes;
    const uint8_t *a_scales;
    const uint16_t *x;
    const uint8_t *w_codes;
    const uint8_t *w_scales;
    float g;
    const uint32_t *v;
    const uint32_t *u;
    const uint16_t *alpha;
    int M, N, K, r;
    uint16_t *y;
    void *ws;
    size_t ws_bytes;
    float *yf = nullptr;    // if set: fp32 results here instead of bf16 y (r = 0 products only)
    // if set: the z launch also quantises x into these (they are a_codes and
    // a_scales of the same call); only for schedules whose z has a launch
    uint8_t *qa_codes = nullptr;
    uint8_t *qa_scales = nullptr;
    // if set: ws is the matrix-core area itself (a sub-call of the
    // separate-launch schedule), not a whole workspace
    bool ws_is_mfma_area = false;
};

// Workspace layout (byte offsets).  The first 80 KiB are fixed for every
// shape, so that no call of one shape can write over the counters, flags or
// tagged values another shape relies on (one workspace may serve calls of
// different shapes, one after the other):
//   [0, 4)                 epoch of the one-launch schedules (uint32)
//   [256, 256 + 4 G)       one "seen" flag per workgroup of a one-launch call
//                          (G <= kGemvMaxWorkgroups + 1)
//   [kWsZcntOffset, kWsZeCntOffset) per-word arrival counters of the
//                          matrix-core z launch and of the all-workgroup
//                          schedule's z tiles (at most kWsZcntMax words), zero
//                          between calls
//   [kWsZeCntOffset, 64 KiB) the arrival counter of the z-in-epilogue
//                          schedule's side workgroups, zero between calls
//                          (that schedule's K-slice sum launch clears it)
//   [64 KiB, 80 KiB)       z as (fp32 value | 32-bit epoch tag << 32) words of
//                          the one-launch vector schedule, [MM <= 2][rpad <= 1024]
//   [80 KiB, ...)          the areas of the shape, in this order:
//     r > 0: z as plain fp32 [M][Rpad] (two-launch schedule)
//     r > 0, M <= 2: the vector product's correction operands: z split into
//            bf16 high and low parts, laid out per lane
//            [M][ceil(Rpad / 512)][64 lanes][4][high, low] (bf16 pairs)
//     (256-aligned) the matrix-core schedules' area: z slice partials, z
//            operands, K-slice partials of y, and (r > 0) the all-workgroup
//            schedule's z tile partials and tagged z operand words (sized by
//            mfma_ws_bytes)
//     (256-aligned, r > 0) the separate-launch schedule's fp32 product [M][N]
//            and its r = 0 product's split-K partials
constexpr int kGemvMaxWorkgroups = 8192;
constexpr size_t kWsHeaderBytes = 64 * 1024;
constexpr size_t kWsZcntOffset = 34 * 1024;
constexpr size_t kWsZeCntOffset = kWsHeaderBytes - 256;
constexpr int kWsZcntMax = (int)((kWsZeCntOffset - kWsZcntOffset) / 4);
constexpr int kZtMaxRows = 2, kZtMaxRank = 1024;
constexpr size_t kWsZtOffset = kWsHeaderBytes;
constexpr size_t kWsZtBytes = (size_t)8 * kZtMaxRows * kZtMaxRank;
constexpr size_t kWsAreaOffset = kWsZtOffset + kWsZtBytes;    // 80 KiB
static_assert(256 + 4 * (kGemvMaxWorkgroups + 1) <= kWsZcntOffset, "seen flags fit the header");
__host__ __device__ inline int rpad32(int r) { return (r + 31) / 32 * 32; }
inline size_t ws_epoch_offset() { return 0; }
inline size_t ws_seen_offset() { return 256; }
inline size_t ws_zt_offset() { return kWsZtOffset; }
inline size_t ws_zf_offset(int, int) { return kWsAreaOffset; }
inline size_t ws_zf_bytes(int M, int r) { return (size_t)4 * (size_t)M * (size_t)rpad32(r); }
inline size_t ws_zop_offset(int M, int r) { return ws_zf_offset(M, r) + ws_zf_bytes(M, r); }
__host__ __device__ inline int zop_rounds(int r) { return (rpad32(r) + 511) / 512; }
inline size_t ws_zop_bytes(int M, int r) {
    return M <= 2 ? (size_t)M * (size_t)zop_rounds(r) * 2048 : 0;
}
inline size_t ws_mfma_offset(int M, int r) {
    return r > 0 ? (ws_zop_offset(M, r) + ws_zop_bytes(M, r) + 255) / 256 * 256 : kWsAreaOffset;
}
bool mfma_supported(int M, int N, int K, int r);     // shapes the matrix-core schedule handles
size_t mfma_ws_bytes(int M, int N, int K, int r);    // its workspace area (0 if none is needed)
// The separate-launch schedule's fp32 product [M][N] (r > 0 only) follows,
// then that schedule's own area for the r = 0 product's K-slice partials.
inline size_t ws_yf_offset(int M, int N, int K, int r) {
    return (ws_mfma_offset(M, r) + mfma_ws_bytes(M, N, K, r) + 255) / 256 * 256;
}
inline size_t ws_g0_offset(int M, int N, int K, int r) {
    return (ws_yf_offset(M, N, K, r) + (size_t)4 * (size_t)M * (size_t)N + 255) / 256 * 256;
}
// Workspace for every schedule of the shape: nothing for r = 0 unless the
// matrix-core schedule splits K (then the fixed part as well, so that the
// partials never touch another shape's counters).
inline size_t ws_total_bytes(int M, int N, int K, int r) {
    if (r > 0) return ws_g0_offset(M, N, K, r) + mfma_ws_bytes(M, N, K, 0);
    const size_t b = mfma_ws_bytes(M, N, K, 0);
    return b > 0 ? ws_mfma_offset(M, 0) + b : 0;
}

hipError_t launch_pack_signs(const int8_t *signs, int64_t rows, int64_t cols, uint32_t *packed,
                             hipStream_t stream);
hipError_t launch_quant_act(const uint16_t *x, int M, int K, uint8_t *codes, uint8_t *scales,
                            hipStream_t stream);
size_t quant_weight_ws_bytes();   // pass-1 partials of the weight quantiser
hipError_t launch_quant_weight(const float *w, int64_t N, int64_t K, uint8_t *codes,
                               uint8_t *scales, float *g_out, void *ws, hipStream_t stream);
size_t peel_ws_bytes(int64_t m, int64_t n, int r);
hipError_t launch_peel(const float *W, int64_t m, int64_t n, int r, int T, const uint32_t *v_init,
                       uint32_t *u_packed, uint32_t *v_packed, float *alpha, float *alpha_greedy,
                       float *R, void *ws, hipStream_t stream);
hipError_t launch_gemm_unfused(const GemmArgs &a, hipStream_t stream);
hipError_t launch_gemm_fused_gemv(const GemmArgs &a, hipStream_t stream);
hipError_t launch_gemm_gemv_two_launch(const GemmArgs &a, hipStream_t stream);
hipError_t launch_z_gemv(const GemmArgs &a, float *z, hipStream_t stream);   // M <= 2
bool gemv_supported(int M, int N, int K, int r);   // shapes the one-launch vector-ALU schedule handles
// bound of a one-launch consumer's wait for z, in ticks of the 100 MHz
// real-time counter; 0 makes consumers compute z themselves
uint32_t spin_limit_default();
hipError_t launch_gemm_mfma(const GemmArgs &a, hipStream_t stream);
bool mfma_one_supported(int M, int N, int K, int r);   // shapes the one-launch matrix-core schedule handles
hipError_t launch_gemm_mfma_one(const GemmArgs &a, hipStream_t stream);
bool mfma_side_supported(int M, int N, int K, int r);  // shapes the side-workgroup matrix-core schedule handles
hipError_t launch_gemm_mfma_side(const GemmArgs &a, hipStream_t stream);
bool mfma_ze_supported(int M, int N, int K, int r);    // shapes the z-in-epilogue matrix-core schedule handles
hipError_t launch_gemm_mfma_ze(const GemmArgs &a, hipStream_t stream);
hipError_t launch_z_mfma(const GemmArgs &a, float *zf, hipStream_t stream);   // M >= 1, r >= 1
// z = alpha (.) (x . V) as plain fp32 [M][rpad32(r)] at z (r > 0)
hipError_t launch_z_fp32(const GemmArgs &a, float *z, hipStream_t stream);
constexpr int kComposedMaxRank = 1024;   // the correction's lookup tables fit 32 KiB of LDS
bool composed_supported(int M, int N, int K, int r);
hipError_t launch_gemm_composed(const GemmArgs &a, bool mfma_correction, hipStream_t stream);

}  // namespace biloco
