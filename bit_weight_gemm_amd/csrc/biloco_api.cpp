// C ABI layer of libbiloco_hip: argument checks (no HIP call), workspace
// sizing, schedule choice, dispatch to the launchers.
#include "../../include/biloco.h"
#include "biloco_internal.h"

#include <stdint.h>

using namespace biloco;

namespace {

// Largest weight matrix (elements) the quantiser takes: 2^38 fp32 values (1 TiB).
constexpr int64_t kMaxWeightElems = (int64_t)1 << 38;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}


bool schedule_allowed(int s, int M, int N, int K, int r) {
    switch (s) {
        case BILOCO_SCHED_UNFUSED: return true;
        case BILOCO_SCHED_FUSED_GEMV: return gemv_supported(M, N, K, r);
        case BILOCO_SCHED_FUSED_MFMA: return mfma_supported(M, N, K, r);
        case BILOCO_SCHED_COMPOSED:
        case BILOCO_SCHED_COMPOSED_MFMA: return composed_supported(M, N, K, r);
        case BILOCO_SCHED_MFMA_ALLWG: return mfma_one_supported(M, N, K, r);
        case BILOCO_SCHED_MFMA_SIDE: return mfma_side_supported(M, N, K, r);
        case BILOCO_SCHED_MFMA_ZEPI: return mfma_ze_supported(M, N, K, r);
        default: return false;
    }
}

biloco_status check_shape(int32_t M, int32_t N, int32_t K, int32_t r) {
    if (M < 1 || N < 1 || K < 1 || r < 0) return BILOCO_ERR_INVALID_VALUE;
    if (K % 16 != 0) return BILOCO_ERR_INVALID_VALUE;   // NVFP4 blocks of 16
    if (M > 32) return BILOCO_ERR_UNSUPPORTED;          // decode batches up to 32
    if (K % 32 != 0 || K < 32) return BILOCO_ERR_UNSUPPORTED;
    // the kernels address R's codes (N x K/2 bytes) and the sign words of U
    // and V (ceil(r/32) x N or K words) with 32-bit byte offsets
    if ((int64_t)N * (K / 2) > (int64_t)INT32_MAX) return BILOCO_ERR_UNSUPPORTED;
    const int64_t W = ((int64_t)r + 31) / 32;
    if (W * 4 * (N > K ? N : K) > (int64_t)INT32_MAX) return BILOCO_ERR_UNSUPPORTED;
    return BILOCO_OK;
}

// Measured on MI355X (M = 1, K = N = 5120, r = 512, graph replay): the
// one-launch vector-ALU schedule (side workgroups compute z while the
// others stream R) takes 7.0-7.2 us per call and 7.7-7.9 us per quantising
// call, against 8.8 and 9.5 us for two launches (z, then the product).  r = 0
// has one launch either way.  From M = 3 on, the matrix-core schedules: with
// side workgroups where x is small enough for one workgroup to read it per
// word (M = 8, K = 5120, N = 13824, r = 512: 16.4-16.9 us per call against
// 20.9-21.1 us with z in launches of its own), else with z in launches of
// its own.  Where K is split over workgroups and x is larger (M = 32,
// K = 13824, N = 5120, r = 512 and M = 32, K = 8192, N = 8192, r = 1024),
// z computed by K-part in side workgroups and applied in the K-slice sum
// launch: 20.5-22.5 us against 26.4-27.4 us with z in launches of its own.
int resolve_schedule(int M, int N, int K, int r) {
    if (M >= 3 && mfma_side_supported(M, N, K, r)) return BILOCO_SCHED_MFMA_SIDE;
    if (M >= 3 && mfma_ze_supported(M, N, K, r)) return BILOCO_SCHED_MFMA_ZEPI;
    if (M >= 3 && mfma_supported(M, N, K, r)) return BILOCO_SCHED_FUSED_MFMA;
    if (r > 0 && gemv_supported(M, N, K, r)) return BILOCO_SCHED_FUSED_GEMV;
    return BILOCO_SCHED_UNFUSED;
}

}  // namespace

extern "C" {

const char *biloco_status_string(biloco_status s) {
    switch (s) {
        case BILOCO_OK: return "BILOCO_OK";
        case BILOCO_ERR_INVALID_VALUE: return "BILOCO_ERR_INVALID_VALUE";
        case BILOCO_ERR_UNSUPPORTED: return "BILOCO_ERR_UNSUPPORTED";
        case BILOCO_ERR_HIP: return "BILOCO_ERR_HIP";
        case BILOCO_ERR_WORKSPACE_TOO_SMALL: return "BILOCO_ERR_WORKSPACE_TOO_SMALL";
        default: return "BILOCO_ERR_UNKNOWN";
    }
}

biloco_status biloco_pack_signs(const int8_t *signs, int64_t rows, int64_t cols, uint32_t *packed,
                                hipStream_t stream) {
    if (!signs || !packed || rows < 1 || cols < 1) return BILOCO_ERR_INVALID_VALUE;
    if (!aligned16(signs) || !aligned16(packed)) return BILOCO_ERR_INVALID_VALUE;
    if (rows > ((int64_t)1 << 40) / cols) return BILOCO_ERR_UNSUPPORTED;
    if (overlaps(signs, (size_t)(rows * cols), packed, (size_t)(((rows + 31) / 32) * cols * 4)))
        return BILOCO_ERR_INVALID_VALUE;
    return launch_pack_signs(signs, rows, cols, packed, stream) == hipSuccess ? BILOCO_OK
                                                                             : BILOCO_ERR_HIP;
}

biloco_status biloco_quant_act_fp4(const uint16_t *x_bf16, int32_t M, int32_t K, uint8_t *a_codes,
                                   uint8_t *a_scales, hipStream_t stream) {
    if (!x_bf16 || !a_codes || !a_scales || M < 1 || K < 1) return BILOCO_ERR_INVALID_VALUE;
    if (K % 16 != 0) return BILOCO_ERR_INVALID_VALUE;
    if (K % 32 != 0) return BILOCO_ERR_UNSUPPORTED;
    if (!aligned16(x_bf16) || !aligned16(a_codes) || !aligned16(a_scales))
        return BILOCO_ERR_INVALID_VALUE;
    size_t nx = (size_t)M * K * 2, nc = (size_t)M * K / 2, ns = (size_t)M * K / 16;
    if (overlaps(x_bf16, nx, a_codes, nc) || overlaps(x_bf16, nx, a_scales, ns) ||
        overlaps(a_codes, nc, a_scales, ns))
        return BILOCO_ERR_INVALID_VALUE;
    return launch_quant_act(x_bf16, M, K, a_codes, a_scales, stream) == hipSuccess
               ? BILOCO_OK
               : BILOCO_ERR_HIP;
}

biloco_status biloco_quant_weight_workspace_bytes(int64_t N, int64_t K, size_t *bytes) {
    if (!bytes || N < 1 || K < 16 || K % 16 != 0) return BILOCO_ERR_INVALID_VALUE;
    if (N > kMaxWeightElems / K) return BILOCO_ERR_UNSUPPORTED;
    *bytes = quant_weight_ws_bytes();
    return BILOCO_OK;
}

biloco_status biloco_quant_weight_nvfp4(const float *w, int64_t N, int64_t K, uint8_t *codes,
                                        uint8_t *scales, float *g_out, void *workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
    size_t need = 0;
    biloco_status st = biloco_quant_weight_workspace_bytes(N, K, &need);
    if (st != BILOCO_OK) return st;
    if (!w || !codes || !scales || !g_out || !workspace) return BILOCO_ERR_INVALID_VALUE;
    if (!aligned16(w) || !aligned16(codes) || !aligned16(scales) || !aligned16(g_out) ||
        !aligned16(workspace))
        return BILOCO_ERR_INVALID_VALUE;
    if (workspace_bytes < need) return BILOCO_ERR_WORKSPACE_TOO_SMALL;
    const size_t n = (size_t)N * (size_t)K;
    struct { const void *p; size_t n; } arr[] = {
        {w, 4 * n}, {codes, n / 2}, {scales, n / 16}, {g_out, 4}, {workspace, need}};
    for (int i = 0; i < 5; ++i)
        for (int j = i + 1; j < 5; ++j)
            if (overlaps(arr[i].p, arr[i].n, arr[j].p, arr[j].n)) return BILOCO_ERR_INVALID_VALUE;
    return launch_quant_weight(w, N, K, codes, scales, g_out, workspace, stream) == hipSuccess
               ? BILOCO_OK
               : BILOCO_ERR_HIP;
}

// Limits of the sign-peeling decomposition: coordinates per side (one
// packed sign row in 32 KiB of LDS) and rank (a one-workgroup solve).
constexpr int64_t kPeelMaxDim = (int64_t)1 << 18;
constexpr int32_t kPeelMaxRank = 1024;

biloco_status biloco_peel_workspace_bytes(int64_t m, int64_t n, int32_t r, size_t *bytes) {
    if (!bytes || m < 1 || n < 4 || n % 4 != 0 || r < 1) return BILOCO_ERR_INVALID_VALUE;
    if (m > kPeelMaxDim || n > kPeelMaxDim || r > kPeelMaxRank) return BILOCO_ERR_UNSUPPORTED;
    *bytes = peel_ws_bytes(m, n, r);
    return BILOCO_OK;
}

biloco_status biloco_peel_decompose(const float *W, int64_t m, int64_t n, int32_t r, int32_t T,
                                    const uint32_t *v_init, uint32_t *u_packed, uint32_t *v_packed,
                                    float *alpha, float *alpha_greedy, float *R, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    size_t need = 0;
    biloco_status st = biloco_peel_workspace_bytes(m, n, r, &need);
    if (st != BILOCO_OK) return st;
    if (T < 1) return BILOCO_ERR_INVALID_VALUE;
    if (!W || !v_init || !u_packed || !v_packed || !alpha || !workspace)
        return BILOCO_ERR_INVALID_VALUE;
    const void *ptrs[] = {W, v_init, u_packed, v_packed, alpha, alpha_greedy, R, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return BILOCO_ERR_INVALID_VALUE;
    if (workspace_bytes < need) return BILOCO_ERR_WORKSPACE_TOO_SMALL;
    const size_t RW = (size_t)(r + 31) / 32, mn = (size_t)m * (size_t)n;
    struct { const void *p; size_t n; } arr[] = {
        {W, 4 * mn},           {v_init, (size_t)r * ((n + 31) / 32) * 4},
        {u_packed, RW * m * 4}, {v_packed, RW * n * 4}, {alpha, (size_t)r * 4},
        {alpha_greedy, (size_t)r * 4}, {R, 4 * mn},  {workspace, need}};
    for (int i = 0; i < 8; ++i)
        for (int j = i + 1; j < 8; ++j)
            if (overlaps(arr[i].p, arr[i].n, arr[j].p, arr[j].n)) return BILOCO_ERR_INVALID_VALUE;
    return launch_peel(W, m, n, r, T, v_init, u_packed, v_packed, alpha, alpha_greedy, R, workspace,
                       stream) == hipSuccess
               ? BILOCO_OK
               : BILOCO_ERR_HIP;
}

biloco_status biloco_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t r,
                                          size_t *bytes) {
    if (!bytes) return BILOCO_ERR_INVALID_VALUE;
    biloco_status st = check_shape(M, N, K, r);
    if (st != BILOCO_OK) return st;
    *bytes = ws_total_bytes(M, N, K, r);
    return BILOCO_OK;
}

biloco_status biloco_gemm_check(const void *a_codes, const void *a_scales, const void *x_bf16,
                                const void *w_codes, const void *w_scales, const void *v_packed,
                                const void *u_packed, const void *alpha_bf16, int32_t M, int32_t N,
                                int32_t K, int32_t r, const void *y_bf16, const void *workspace,
                                size_t workspace_bytes, int32_t schedule) {
    biloco_status st = check_shape(M, N, K, r);
    if (st != BILOCO_OK) return st;
    if (!a_codes || !a_scales || !w_codes || !w_scales || !y_bf16) return BILOCO_ERR_INVALID_VALUE;
    if (r > 0 && (!x_bf16 || !v_packed || !u_packed || !alpha_bf16))
        return BILOCO_ERR_INVALID_VALUE;
    const void *ptrs[] = {a_codes, a_scales, x_bf16, w_codes, w_scales,
                          v_packed, u_packed, alpha_bf16, y_bf16, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return BILOCO_ERR_INVALID_VALUE;
    size_t need = ws_total_bytes(M, N, K, r);
    if (need > 0 && !workspace) return BILOCO_ERR_INVALID_VALUE;
    if (workspace_bytes < need) return BILOCO_ERR_WORKSPACE_TOO_SMALL;
    // the output must not overlap any operand
    size_t W = (size_t)(r + 31) / 32;
    size_t ny = (size_t)M * N * 2;
    struct { const void *p; size_t n; } ins[] = {
        {a_codes, (size_t)M * K / 2},  {a_scales, (size_t)M * K / 16},
        {x_bf16, r > 0 ? (size_t)M * K * 2 : 0},
        {w_codes, (size_t)N * K / 2},  {w_scales, (size_t)N * K / 16},
        {v_packed, W * (size_t)K * 4}, {u_packed, W * (size_t)N * 4},
        {alpha_bf16, (size_t)r * 2},   {workspace, need}};
    for (auto &in : ins)
        if (overlaps(y_bf16, ny, in.p, in.n)) return BILOCO_ERR_INVALID_VALUE;
    if (schedule < BILOCO_SCHED_AUTO || schedule > BILOCO_SCHED_MFMA_ZEPI)
        return BILOCO_ERR_INVALID_VALUE;
    if (schedule != BILOCO_SCHED_AUTO && !schedule_allowed(schedule, M, N, K, r))
        return BILOCO_ERR_UNSUPPORTED;
    return BILOCO_OK;
}

int32_t biloco_default_schedule(int32_t M, int32_t N, int32_t K, int32_t r) {
    if (check_shape(M, N, K, r) != BILOCO_OK) return 0;
    return resolve_schedule(M, N, K, r);
}

int32_t biloco_schedules_for(int32_t M, int32_t N, int32_t K, int32_t r, int32_t *out,
                             int32_t cap) {
    if (check_shape(M, N, K, r) != BILOCO_OK) return 0;
    int32_t n = 0;
    for (int s = BILOCO_SCHED_UNFUSED; s <= BILOCO_SCHED_MFMA_ZEPI; ++s)
        if (schedule_allowed(s, M, N, K, r)) {
            if (out && n < cap) out[n] = s;
            ++n;
        }
    return n;
}

biloco_status biloco_gemm_lowrank_sched(const uint8_t *a_codes, const uint8_t *a_scales,
                                        const uint16_t *x_bf16, const uint8_t *w_codes,
                                        const uint8_t *w_scales, float w_global_scale,
                                        const uint32_t *v_packed, const uint32_t *u_packed,
                                        const uint16_t *alpha_bf16, int32_t M, int32_t N,
                                        int32_t K, int32_t r, uint16_t *y_bf16, void *workspace,
                                        size_t workspace_bytes, int32_t schedule,
                                        hipStream_t stream) {
    biloco_status st = biloco_gemm_check(a_codes, a_scales, x_bf16, w_codes, w_scales, v_packed,
                                         u_packed, alpha_bf16, M, N, K, r, y_bf16, workspace,
                                         workspace_bytes, schedule);
    if (st != BILOCO_OK) return st;
    GemmArgs a{a_codes, a_scales, x_bf16, w_codes, w_scales, w_global_scale, v_packed,
               u_packed, alpha_bf16, M,       N,        K,     r,      y_bf16,
               workspace, workspace_bytes};
    int s = schedule == BILOCO_SCHED_AUTO ? resolve_schedule(M, N, K, r) : schedule;
    hipError_t e;
    switch (s) {
        case BILOCO_SCHED_FUSED_GEMV: e = launch_gemm_fused_gemv(a, stream); break;
        case BILOCO_SCHED_FUSED_MFMA: e = launch_gemm_mfma(a, stream); break;
        case BILOCO_SCHED_COMPOSED: e = launch_gemm_composed(a, false, stream); break;
        case BILOCO_SCHED_COMPOSED_MFMA: e = launch_gemm_composed(a, true, stream); break;
        case BILOCO_SCHED_MFMA_ALLWG: e = launch_gemm_mfma_one(a, stream); break;
        case BILOCO_SCHED_MFMA_SIDE: e = launch_gemm_mfma_side(a, stream); break;
        case BILOCO_SCHED_MFMA_ZEPI: e = launch_gemm_mfma_ze(a, stream); break;
        default: e = launch_gemm_unfused(a, stream); break;
    }
    return e == hipSuccess ? BILOCO_OK : BILOCO_ERR_HIP;
}

biloco_status biloco_gemm_lowrank_quant(const uint16_t *x_bf16, uint8_t *a_codes, uint8_t *a_scales,
                                        const uint8_t *w_codes, const uint8_t *w_scales,
                                        float w_global_scale, const uint32_t *v_packed,
                                        const uint32_t *u_packed, const uint16_t *alpha_bf16,
                                        int32_t M, int32_t N, int32_t K, int32_t r, uint16_t *y_bf16,
                                        void *workspace, size_t workspace_bytes, int32_t schedule,
                                        hipStream_t stream) {
    if (!x_bf16) return BILOCO_ERR_INVALID_VALUE;
    biloco_status st = biloco_gemm_check(a_codes, a_scales, x_bf16, w_codes, w_scales, v_packed,
                                         u_packed, alpha_bf16, M, N, K, r, y_bf16, workspace,
                                         workspace_bytes, schedule);
    if (st != BILOCO_OK) return st;
    // the activation outputs must not overlap any other array of the call
    const size_t nc = (size_t)M * K / 2, ns = (size_t)M * K / 16;
    const size_t W = (size_t)(r + 31) / 32;
    struct { const void *p; size_t n; } others[] = {
        {x_bf16, (size_t)M * K * 2},   {w_codes, (size_t)N * K / 2}, {w_scales, (size_t)N * K / 16},
        {v_packed, W * (size_t)K * 4}, {u_packed, W * (size_t)N * 4}, {alpha_bf16, (size_t)r * 2},
        {workspace, ws_total_bytes(M, N, K, r)}, {a_scales, ns}};
    for (auto &o : others) {
        if (overlaps(a_codes, nc, o.p, o.n)) return BILOCO_ERR_INVALID_VALUE;
        if (o.p != a_scales && overlaps(a_scales, ns, o.p, o.n)) return BILOCO_ERR_INVALID_VALUE;
    }
    GemmArgs a{a_codes, a_scales, x_bf16, w_codes, w_scales, w_global_scale, v_packed,
               u_packed, alpha_bf16, M,       N,        K,     r,      y_bf16,
               workspace, workspace_bytes};
    const int s = schedule == BILOCO_SCHED_AUTO ? resolve_schedule(M, N, K, r) : schedule;
    // the vector-ALU schedules quantise x in the product launch (or, in the
    // two-launch form, in the z launch); the matrix-core schedule in its z
    // launch when r > 0; otherwise a launch of its own comes first
    const bool gemv = (s == BILOCO_SCHED_UNFUSED && gemv_supported(M, N, K, r)) ||
                      s == BILOCO_SCHED_FUSED_GEMV;
    const bool in_z = gemv || (r > 0 && s == BILOCO_SCHED_FUSED_MFMA);
    hipError_t e = hipSuccess;
    if (in_z) {
        a.qa_codes = a_codes;
        a.qa_scales = a_scales;
    } else {
        e = launch_quant_act(x_bf16, M, K, a_codes, a_scales, stream);
        if (e != hipSuccess) return BILOCO_ERR_HIP;
    }
    switch (s) {
        case BILOCO_SCHED_FUSED_GEMV: e = launch_gemm_fused_gemv(a, stream); break;
        case BILOCO_SCHED_FUSED_MFMA: e = launch_gemm_mfma(a, stream); break;
        case BILOCO_SCHED_COMPOSED: e = launch_gemm_composed(a, false, stream); break;
        case BILOCO_SCHED_COMPOSED_MFMA: e = launch_gemm_composed(a, true, stream); break;
        case BILOCO_SCHED_MFMA_ALLWG: e = launch_gemm_mfma_one(a, stream); break;
        case BILOCO_SCHED_MFMA_SIDE: e = launch_gemm_mfma_side(a, stream); break;
        case BILOCO_SCHED_MFMA_ZEPI: e = launch_gemm_mfma_ze(a, stream); break;
        default: e = launch_gemm_unfused(a, stream); break;
    }
    return e == hipSuccess ? BILOCO_OK : BILOCO_ERR_HIP;
}

biloco_status biloco_gemm_lowrank(const uint8_t *a_codes, const uint8_t *a_scales,
                                  const uint16_t *x_bf16, const uint8_t *w_codes,
                                  const uint8_t *w_scales, float w_global_scale,
                                  const uint32_t *v_packed, const uint32_t *u_packed,
                                  const uint16_t *alpha_bf16, int32_t M, int32_t N, int32_t K,
                                  int32_t r, uint16_t *y_bf16, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    return biloco_gemm_lowrank_sched(a_codes, a_scales, x_bf16, w_codes, w_scales, w_global_scale,
                                     v_packed, u_packed, alpha_bf16, M, N, K, r, y_bf16, workspace,
                                     workspace_bytes, BILOCO_SCHED_AUTO, stream);
}

}  // extern "C"
