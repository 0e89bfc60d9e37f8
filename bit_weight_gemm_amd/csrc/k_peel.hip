// Greedy sign peeling and the joint least-squares refit of the coefficients,
// on the GPU: W ~ U diag(alpha) V^T + R with U in {+-1}^{m x r},
// V in {+-1}^{n x r} (BiLoCo README, intro and section "Decomposition": each
// rank-one term starts from random signs and alternates u = sign(R v),
// v = sign(R^T u) for T steps, takes the Frobenius-optimal coefficient
// u^T R v / (m n) and deflates R; after all r terms the coefficients are refit
// together by least squares for the fixed signs).
//
// The residual is never stored during the peel.  With the terms found so far
// (j < i), R v = W v - sum_j alpha_j (v_j . v) u_j and
// R^T u = W^T u - sum_j alpha_j (u_j . u) v_j; the sign dot products are
// exact integers from XOR and popcount of packed sign words.  Every step is
// then one pass over the read-only fp32 W (row products for R v, column
// products for R^T u) plus small kernels, and W stays the only large array.
//
// Per step of term i: coef (beta_j = alpha_j (v_j . v)), row (R v and
// u = sign(R v) by atomic or), coef (gamma_j = alpha_j (u_j . u)), col
// (K-slice partials of W^T u), colfin (t = R^T u, v = sign(t)); the two coef
// launches only when i > 0; after the T steps one term-finishing launch.  At the end: the Gram matrix of the sign terms, a
// blocked Cholesky solve of the normal equations, and R = W - U diag(alpha)
// V^T with 4-bit lookup tables of the coefficients.
//
// Sign words: bit set = -1.  Term-major rows (bits of term j over the m or n
// coordinates, for the popcounts) live in the workspace; the outputs are the
// row-major packed forms [ceil(r/32)][m] and [ceil(r/32)][n] that
// biloco_gemm_lowrank takes as pack_signs(U^T) and pack_signs(V^T).
#include "biloco_device.h"
#include "biloco_internal.h"

namespace biloco {

namespace {

constexpr int kPeelThreads = 256;
constexpr int kColTarget = 512;        // workgroups of the column pass (K-slices x column tiles)
constexpr int kColUnroll = 8;          // rows in flight per thread in the column pass

struct PeelLayout {
    int64_t m, n;
    int r, Wm, Wn, RW, S, rows_per_slice, NBf;
    size_t ubits, vbits, ucur, vcur, coef, ag, tpart, red, bvec, gram, sol, bad, total;
};

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

PeelLayout peel_layout(int64_t m, int64_t n, int r) {
    PeelLayout L{};
    L.m = m;
    L.n = n;
    L.r = r;
    L.Wm = (int)((m + 31) / 32);
    L.Wn = (int)((n + 31) / 32);
    L.RW = (r + 31) / 32;
    const int64_t tiles = (n / 4 + kPeelThreads - 1) / kPeelThreads;
    int64_t S = (kColTarget + tiles - 1) / tiles;
    if (S > m) S = m;
    L.rows_per_slice = (int)((m + S - 1) / S);
    L.S = (int)((m + L.rows_per_slice - 1) / L.rows_per_slice);
    L.NBf = L.Wn;                         // colfin workgroups: one per word of v
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = al256(o + bytes); return at; };
    L.ubits = take((size_t)r * L.Wm * 4);
    L.vbits = take((size_t)r * L.Wn * 4);
    L.ucur = take((size_t)L.Wm * 4);
    L.vcur = take((size_t)L.Wn * 4);
    L.coef = take((size_t)r * 4);
    L.ag = take((size_t)r * 4);
    L.tpart = take((size_t)L.S * (size_t)n * 4);
    L.red = take((size_t)2 * L.NBf * 4);
    L.bvec = take((size_t)r * 8);
    L.gram = take((size_t)r * r * 8);
    L.sol = take((size_t)r * 8);
    L.bad = take((size_t)r * 4);      // one "dropped" flag per coefficient
    L.total = o;
    return L;
}

struct PeelPtrs {
    uint32_t *ubits, *vbits, *ucur, *vcur;
    float *coef, *ag, *tpart, *red;
    double *bvec, *gram, *sol;
    int *bad;
};

PeelPtrs peel_ptrs(const PeelLayout &L, void *ws) {
    char *b = static_cast<char *>(ws);
    return PeelPtrs{reinterpret_cast<uint32_t *>(b + L.ubits), reinterpret_cast<uint32_t *>(b + L.vbits),
                    reinterpret_cast<uint32_t *>(b + L.ucur),  reinterpret_cast<uint32_t *>(b + L.vcur),
                    reinterpret_cast<float *>(b + L.coef),
                    reinterpret_cast<float *>(b + L.ag),       reinterpret_cast<float *>(b + L.tpart),
                    reinterpret_cast<float *>(b + L.red),      reinterpret_cast<double *>(b + L.bvec),
                    reinterpret_cast<double *>(b + L.gram),    reinterpret_cast<double *>(b + L.sol),
                    reinterpret_cast<int *>(b + L.bad)};
}

// mask of the valid bits of word w of a length-len sign row
__device__ __forceinline__ uint32_t valid_mask(int w, int64_t len) {
    const int64_t rem = len - (int64_t)w * 32;
    return rem >= 32 ? 0xFFFFFFFFu : ((1u << rem) - 1u);
}

__device__ __forceinline__ int wave_isum(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

}  // namespace

// ---------------------------------------------------------------------------
// coef: one wave per earlier term j < i:
//   coef[j] = alpha_j * (len - 2 popcount(rows[j] ^ cur))       (= alpha_j (x_j . x))
// cur (the current u or v words, bits past len cleared) is staged in LDS.
__global__ void __launch_bounds__(kPeelThreads)
peel_coef_kernel(const uint32_t *__restrict__ rows, const uint32_t *__restrict__ cur_in, int words,
                 int64_t len, int i, const float *__restrict__ ag, float *__restrict__ coef) {
    extern __shared__ uint32_t cur[];
    for (int w = threadIdx.x; w < words; w += kPeelThreads) cur[w] = cur_in[w] & valid_mask(w, len);
    __syncthreads();
    const int j = blockIdx.x * (kPeelThreads / 64) + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (j >= i) return;
    int pc = 0;
    for (int w = lane; w < words; w += 64) pc += __popc(rows[(int64_t)j * words + w] ^ cur[w]);
    pc = wave_isum(pc);
    if (lane == 0) coef[j] = ag[j] * (float)(len - 2 * (int64_t)pc);
}

// ---------------------------------------------------------------------------
// row: one wave per row a (4 rows per workgroup):
//   s_a = sum_k W[a][k] v_k  -  sum_{j<i} coef[j] u_j[a],  u_a = sign(s_a)
// v from its packed bits (LDS); u_j[a] from the row-major packed U words;
// u's bit goes into ucur by an atomic or (ucur cleared before the launch).
__global__ void __launch_bounds__(kPeelThreads)
peel_row_kernel(const float4 *__restrict__ W, int64_t m, int64_t n4, const uint32_t *__restrict__ vbits,
                int Wn, const uint32_t *__restrict__ up, int i, const float *__restrict__ coef,
                uint32_t *__restrict__ ucur) {
    extern __shared__ uint32_t vb[];
    for (int w = threadIdx.x; w < Wn; w += kPeelThreads) vb[w] = vbits[w];
    __syncthreads();
    const int64_t a = (int64_t)blockIdx.x * (kPeelThreads / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (a >= m) return;
    const float4 *row = W + a * n4;
    float acc0 = 0.0f, acc1 = 0.0f;
    int64_t q = lane;
    for (; q + 64 < n4; q += 128) {
        const float4 x0 = row[q], x1 = row[q + 64];
        const uint32_t b0 = vb[q >> 3] >> (4 * (q & 7)), b1 = vb[(q + 64) >> 3] >> (4 * ((q + 64) & 7));
        acc0 += __uint_as_float(__float_as_uint(x0.x) ^ ((b0 << 31) & 0x80000000u));
        acc0 += __uint_as_float(__float_as_uint(x0.y) ^ ((b0 << 30) & 0x80000000u));
        acc0 += __uint_as_float(__float_as_uint(x0.z) ^ ((b0 << 29) & 0x80000000u));
        acc0 += __uint_as_float(__float_as_uint(x0.w) ^ ((b0 << 28) & 0x80000000u));
        acc1 += __uint_as_float(__float_as_uint(x1.x) ^ ((b1 << 31) & 0x80000000u));
        acc1 += __uint_as_float(__float_as_uint(x1.y) ^ ((b1 << 30) & 0x80000000u));
        acc1 += __uint_as_float(__float_as_uint(x1.z) ^ ((b1 << 29) & 0x80000000u));
        acc1 += __uint_as_float(__float_as_uint(x1.w) ^ ((b1 << 28) & 0x80000000u));
    }
    if (q < n4) {
        const float4 x0 = row[q];
        const uint32_t b0 = vb[q >> 3] >> (4 * (q & 7));
        acc0 += __uint_as_float(__float_as_uint(x0.x) ^ ((b0 << 31) & 0x80000000u));
        acc0 += __uint_as_float(__float_as_uint(x0.y) ^ ((b0 << 30) & 0x80000000u));
        acc0 += __uint_as_float(__float_as_uint(x0.z) ^ ((b0 << 29) & 0x80000000u));
        acc0 += __uint_as_float(__float_as_uint(x0.w) ^ ((b0 << 28) & 0x80000000u));
    }
    float corr = 0.0f;
    for (int j = lane; j < i; j += 64) {
        const uint32_t bit = (up[(int64_t)(j >> 5) * m + a] >> (j & 31)) & 1u;
        corr += bit ? -coef[j] : coef[j];
    }
    const float tot = wave_sum(acc0 + acc1) - wave_sum(corr);
    // u = sign(R v): set the row's bit (the word was cleared before this launch)
    if (lane == 0 && tot < 0.0f)
        __hip_atomic_fetch_or(ucur + (a >> 5), 1u << (a & 31), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// col: K-slice partials of W^T u.  Thread = one float4 of columns; workgroup
// (column tile, slice of rows):  tpart[slice][4q..4q+3] = sum_a u_a W[a][4q..]
__global__ void __launch_bounds__(kPeelThreads)
peel_col_kernel(const float4 *__restrict__ W, int64_t m, int64_t n4, const uint32_t *__restrict__ ucur,
                int rows_per_slice, float4 *__restrict__ tpart) {
    const int64_t q = (int64_t)blockIdx.x * kPeelThreads + threadIdx.x;
    const int slice = blockIdx.y;
    const int64_t a0 = (int64_t)slice * rows_per_slice;
    int64_t a1 = a0 + rows_per_slice;
    if (a1 > m) a1 = m;
    if (q >= n4) return;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    int64_t a = a0;
    for (; a + kColUnroll <= a1; a += kColUnroll) {
        float4 x[kColUnroll];
#pragma unroll
        for (int e = 0; e < kColUnroll; ++e) x[e] = W[(a + e) * n4 + q];
#pragma unroll
        for (int e = 0; e < kColUnroll; ++e) {
            const uint32_t sg = ((ucur[(a + e) >> 5] >> ((a + e) & 31)) & 1u) << 31;
            acc.x += __uint_as_float(__float_as_uint(x[e].x) ^ sg);
            acc.y += __uint_as_float(__float_as_uint(x[e].y) ^ sg);
            acc.z += __uint_as_float(__float_as_uint(x[e].z) ^ sg);
            acc.w += __uint_as_float(__float_as_uint(x[e].w) ^ sg);
        }
    }
    for (; a < a1; ++a) {
        const float4 x = W[a * n4 + q];
        const uint32_t sg = ((ucur[a >> 5] >> (a & 31)) & 1u) << 31;
        acc.x += __uint_as_float(__float_as_uint(x.x) ^ sg);
        acc.y += __uint_as_float(__float_as_uint(x.y) ^ sg);
        acc.z += __uint_as_float(__float_as_uint(x.z) ^ sg);
        acc.w += __uint_as_float(__float_as_uint(x.w) ^ sg);
    }
    tpart[(int64_t)slice * n4 + q] = acc;
}

// ---------------------------------------------------------------------------
// colfin: workgroup = 32 columns (one word of v); its 8 groups of 32 threads
// split the slices and the earlier terms, and the first 32 lanes finish:
//   tw_k = sum_slices tpart,  t_k = tw_k - sum_{j<i} coef[j] v_j[k],
//   v bits = (t_k < 0) by ballot.
// On the last step of a term it also leaves per-workgroup partial sums of
// |t_k| (for alpha_i) and of tw_k v_k (for the refit's b_i) in red.
__global__ void __launch_bounds__(kPeelThreads)
peel_colfin_kernel(const float *__restrict__ tpart, int S, int64_t n, const uint32_t *__restrict__ vp,
                   int i, const float *__restrict__ coef, uint32_t *__restrict__ vcur, int last,
                   float *__restrict__ red, uint32_t *__restrict__ ucur, int Wm) {
    // u of this step has been read (coef, col); clear it for the next step's
    // row launch, except after a term's last step (the term launch reads it)
    if (!last)
        for (int w = blockIdx.x * kPeelThreads + threadIdx.x; w < Wm; w += gridDim.x * kPeelThreads)
            ucur[w] = 0u;
    __shared__ float part[8][32], corr[8][32];
    const int grp = threadIdx.x >> 5, c = threadIdx.x & 31;
    const int64_t k = (int64_t)blockIdx.x * 32 + c;
    float tw = 0.0f, cs = 0.0f;
    if (k < n) {
        for (int sl = grp; sl < S; sl += 8) tw += tpart[(int64_t)sl * n + k];
        for (int w = grp; w < (i + 31) / 32; w += 8) {
            const uint32_t word = vp[(int64_t)w * n + k];
            const int jn = i - 32 * w < 32 ? i - 32 * w : 32;
            for (int b = 0; b < jn; ++b) {
                const float cf = coef[32 * w + b];
                cs += ((word >> b) & 1u) ? -cf : cf;
            }
        }
    }
    part[grp][c] = tw;
    corr[grp][c] = cs;
    __syncthreads();
    if (threadIdx.x >= 64) return;
    const int lane = threadIdx.x;          // wave 0; lanes 32..63 repeat columns 0..31
    float twk = 0.0f, ck = 0.0f;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        twk += part[g][c];
        ck += corr[g][c];
    }
    const bool mine = lane < 32 && k < n;
    const float t = twk - ck;
    const bool neg = mine && t < 0.0f;
    const uint64_t bal = __ballot(neg);
    if (lane == 0) vcur[blockIdx.x] = (uint32_t)bal;
    if (last) {
        const float at = wave_sum(mine ? fabsf(t) : 0.0f);
        const float bt = wave_sum(mine ? (neg ? -twk : twk) : 0.0f);
        if (lane == 0) {
            red[2 * blockIdx.x] = at;
            red[2 * blockIdx.x + 1] = bt;
        }
    }
}

// ---------------------------------------------------------------------------
// term: one workgroup.  alpha_i = sum|t| / (m n), b_i = sum tw v; the term's
// sign rows are copied to the term-major arrays and its bit i is set in the
// row-major packed outputs (cleared before the first term).
__global__ void __launch_bounds__(1024)
peel_term_kernel(int i, int64_t m, int64_t n, int NBf, const float *__restrict__ red,
                 uint32_t *__restrict__ ucur, const uint32_t *__restrict__ vcur, int Wm, int Wn,
                 float *__restrict__ ag, double *__restrict__ bvec, uint32_t *__restrict__ ubits,
                 uint32_t *__restrict__ vbits, uint32_t *__restrict__ up, uint32_t *__restrict__ vp) {
    __shared__ double sa[16], sb[16];
    double a = 0.0, b = 0.0;
    for (int x = threadIdx.x; x < NBf; x += 1024) {
        a += (double)red[2 * x];
        b += (double)red[2 * x + 1];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        a += __shfl_xor(a, o, 64);
        b += __shfl_xor(b, o, 64);
    }
    if ((threadIdx.x & 63) == 0) {
        sa[threadIdx.x >> 6] = a;
        sb[threadIdx.x >> 6] = b;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double ta = 0.0, tb = 0.0;
        for (int w = 0; w < 16; ++w) {
            ta += sa[w];
            tb += sb[w];
        }
        ag[i] = (float)(ta / ((double)m * (double)n));
        bvec[i] = tb;
    }
    for (int w = threadIdx.x; w < Wm; w += 1024) ubits[(int64_t)i * Wm + w] = ucur[w];
    for (int w = threadIdx.x; w < Wn; w += 1024) vbits[(int64_t)i * Wn + w] = vcur[w];
    const int wr = i >> 5, sh = i & 31;
    for (int64_t x = threadIdx.x; x < m; x += 1024)
        up[(int64_t)wr * m + x] |= ((ucur[x >> 5] >> (x & 31)) & 1u) << sh;
    for (int64_t x = threadIdx.x; x < n; x += 1024)
        vp[(int64_t)wr * n + x] |= ((vcur[x >> 5] >> (x & 31)) & 1u) << sh;
    __syncthreads();
    for (int w = threadIdx.x; w < Wm; w += 1024) ucur[w] = 0u;   // for the next term's first row launch
}

// zero-fill (no memset node: callers may capture the call in a graph)
__global__ void __launch_bounds__(kPeelThreads) peel_zero_kernel(uint32_t *p, int64_t words) {
    for (int64_t x = (int64_t)blockIdx.x * kPeelThreads + threadIdx.x; x < words;
         x += (int64_t)gridDim.x * kPeelThreads)
        p[x] = 0u;
}

// ---------------------------------------------------------------------------
// gram: G[i][j] = (m - 2 popcount(U_i ^ U_j)) (n - 2 popcount(V_i ^ V_j)),
// exact integers in fp64.  Workgroup = a 16 x 16 tile of (i, j); its 32 sign
// rows are staged through LDS a chunk of words at a time.
constexpr int kGramChunk = 64;
__global__ void __launch_bounds__(256)
peel_gram_kernel(const uint32_t *__restrict__ ubits, const uint32_t *__restrict__ vbits, int Wm,
                 int Wn, int r, int64_t m, int64_t n, double *__restrict__ gram) {
    __shared__ uint32_t ri[16][kGramChunk + 1], rj[16][kGramChunk + 1];
    const int ti = threadIdx.x >> 4, tj = threadIdx.x & 15;
    const int i = blockIdx.y * 16 + ti, j = blockIdx.x * 16 + tj;
    int pc[2] = {0, 0};
    for (int side = 0; side < 2; ++side) {
        const uint32_t *rows = side ? vbits : ubits;
        const int words = side ? Wn : Wm;
        for (int w0 = 0; w0 < words; w0 += kGramChunk) {
            __syncthreads();
            for (int x = threadIdx.x; x < 16 * kGramChunk; x += 256) {
                const int rr = x / kGramChunk, w = w0 + x % kGramChunk;
                const int gi = blockIdx.y * 16 + rr, gj = blockIdx.x * 16 + rr;
                ri[rr][x % kGramChunk] = (gi < r && w < words) ? rows[(int64_t)gi * words + w] : 0u;
                rj[rr][x % kGramChunk] = (gj < r && w < words) ? rows[(int64_t)gj * words + w] : 0u;
            }
            __syncthreads();
            for (int w = 0; w < kGramChunk; ++w) pc[side] += __popc(ri[ti][w] ^ rj[tj][w]);
        }
    }
    if (i < r && j < r)
        gram[(int64_t)i * r + j] = (double)(m - 2 * (int64_t)pc[0]) * (double)(n - 2 * (int64_t)pc[1]);
}

// ---------------------------------------------------------------------------
// solve: blocked right-looking Cholesky G = L L^T in place (lower triangle,
// fp64), panels of kChol columns.  Per panel, one workgroup factors the
// diagonal block in LDS and solves the rows below it (L21 = A21 L11^-T, one
// thread per row), then a tiled update A22 -= L21 L21^T runs over many
// workgroups.  A last workgroup solves L y = b, L^T x = y.  A pivot below
// 1e-6 m n (every diagonal entry of G is m n) means that term's sign outer
// product lies in the span of the earlier kept ones (e.g. a term found
// twice): the term is dropped from the solve (its column of L is zero, its
// coefficient 0), which leaves the span of the design matrix, and so the
// least-squares minimum, unchanged -- the refit is still a least-squares
// minimiser, the one with the dropped coefficients at zero.
constexpr int kChol = 32;

__global__ void __launch_bounds__(1024)
peel_chol_panel_kernel(double *__restrict__ G, int r, int k0, double G_diag, int *__restrict__ dropped) {
    __shared__ double L[kChol][kChol + 1];
    __shared__ int s_drop[kChol];
    const int kb = r - k0 < kChol ? r - k0 : kChol;
    for (int e = threadIdx.x; e < kb * kb; e += 1024) {
        const int a = e / kb, c = e % kb;
        L[a][c] = G[(int64_t)(k0 + a) * r + k0 + c];
    }
    __syncthreads();
    for (int c = 0; c < kb; ++c) {
        if (threadIdx.x == 0) {
            const double d = L[c][c];
            const bool ok = d > 1e-6 * G_diag;
            s_drop[c] = ok ? 0 : 1;
            dropped[k0 + c] = ok ? 0 : 1;
            L[c][c] = ok ? sqrt(d) : 1.0;
        }
        __syncthreads();
        // a dropped column is zero below the diagonal, so no later column
        // subtracts anything for it
        for (int a = c + 1 + (int)threadIdx.x; a < kb; a += 1024) L[a][c] = s_drop[c] ? 0.0 : L[a][c] / L[c][c];
        __syncthreads();
        const int rem = kb - c - 1;
        for (int e = threadIdx.x; e < rem * rem; e += 1024) {
            const int a = c + 1 + e / rem, cc = c + 1 + e % rem;
            if (cc <= a) L[a][cc] -= L[a][c] * L[cc][c];
        }
        __syncthreads();
    }
    for (int e = threadIdx.x; e < kb * kb; e += 1024) {
        const int a = e / kb, c = e % kb;
        if (c <= a) G[(int64_t)(k0 + a) * r + k0 + c] = L[a][c];
    }
    // rows below the block: L21[i][:] = A21[i][:] L11^-T (forward substitution)
    for (int i = k0 + kb + (int)threadIdx.x; i < r; i += 1024) {
        double x[kChol];
        double *row = G + (int64_t)i * r + k0;
#pragma unroll
        for (int c = 0; c < kChol; ++c) x[c] = c < kb ? row[c] : 0.0;
#pragma unroll
        for (int c = 0; c < kChol; ++c) {
            if (c < kb) {
                double v = x[c];
#pragma unroll
                for (int cc = 0; cc < c; ++cc) v -= x[cc] * L[c][cc];
                x[c] = s_drop[c] ? 0.0 : v / L[c][c];
            }
        }
#pragma unroll
        for (int c = 0; c < kChol; ++c)
            if (c < kb) row[c] = x[c];
    }
}

// A22 -= L21 L21^T on the lower triangle of the trailing matrix: workgroup =
// one 32 x 32 tile (ti >= tj), thread = 4 entries; both panels via LDS.
__global__ void __launch_bounds__(256)
peel_chol_update_kernel(double *__restrict__ G, int r, int k0) {
    __shared__ double Pi[kChol][kChol + 1], Pj[kChol][kChol + 1];
    const int kb = r - k0 < kChol ? r - k0 : kChol;
    const int base = k0 + kb;
    // blockIdx.x -> (ti, tj), tj <= ti
    int ti = (int)((sqrt(8.0 * (double)blockIdx.x + 1.0) - 1.0) * 0.5);
    while ((ti + 1) * (ti + 2) / 2 <= (int)blockIdx.x) ++ti;
    while (ti * (ti + 1) / 2 > (int)blockIdx.x) --ti;
    const int tj = (int)blockIdx.x - ti * (ti + 1) / 2;
    const int i0 = base + 32 * ti, j0 = base + 32 * tj;
    for (int e = threadIdx.x; e < 32 * kChol; e += 256) {
        const int a = e / kChol, c = e % kChol;
        Pi[a][c] = (i0 + a < r && c < kb) ? G[(int64_t)(i0 + a) * r + k0 + c] : 0.0;
        Pj[a][c] = (j0 + a < r && c < kb) ? G[(int64_t)(j0 + a) * r + k0 + c] : 0.0;
    }
    __syncthreads();
    const int a = threadIdx.x >> 3, c0 = (threadIdx.x & 7) * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int gi = i0 + a, gj = j0 + c0 + q;
        if (gi < r && gj < r && gj <= gi) {
            double v = 0.0;
#pragma unroll
            for (int c = 0; c < kChol; ++c) v += Pi[a][c] * Pj[c0 + q][c];
            G[(int64_t)gi * r + gj] -= v;
        }
    }
}

// L y = b and L^T x = y (one workgroup), then the outputs.
__global__ void __launch_bounds__(1024)
peel_trisolve_kernel(const double *__restrict__ G, const double *__restrict__ b, double *__restrict__ x,
                     int r, const int *__restrict__ dropped, const float *__restrict__ ag,
                     float *__restrict__ alpha, float *__restrict__ alpha_greedy) {
    for (int t = threadIdx.x; t < r; t += 1024) x[t] = b[t];
    __syncthreads();
    // a dropped term's unknown is 0 in both passes (its column of L is zero,
    // so it never reaches the other unknowns of the forward pass)
    for (int i = 0; i < r; ++i) {
        if (threadIdx.x == 0) x[i] = dropped[i] ? 0.0 : x[i] / G[(int64_t)i * r + i];
        __syncthreads();
        for (int t = i + 1 + threadIdx.x; t < r; t += 1024) x[t] -= G[(int64_t)t * r + i] * x[i];
        __syncthreads();
    }
    for (int i = r - 1; i >= 0; --i) {
        if (threadIdx.x == 0) x[i] = dropped[i] ? 0.0 : x[i] / G[(int64_t)i * r + i];
        __syncthreads();
        for (int t = threadIdx.x; t < i; t += 1024) x[t] -= G[(int64_t)i * r + t] * x[i];
        __syncthreads();
    }
    for (int i = threadIdx.x; i < r; i += 1024) {
        alpha[i] = (float)x[i];
        if (alpha_greedy) alpha_greedy[i] = ag[i];
    }
}

// ---------------------------------------------------------------------------
// resid: R = W - sum_j alpha_j u_j[a] v_j[k].  The sign of term j's product
// is bit j of (U word ^ V word); lut[q][nib] = sum over the 4 terms 4q..4q+3
// of (bit set ? -alpha : +alpha), so each 4-bit nibble of the XOR is one
// lookup.  Thread = one float4 of a row; workgroup = 256 float4 of one row
// (workgroup b: row b / tiles, tile b % tiles).
__global__ void __launch_bounds__(kPeelThreads)
peel_resid_kernel(const float4 *__restrict__ W, int64_t m, int64_t n4, const uint32_t *__restrict__ up,
                  const uint32_t *__restrict__ vp, const float *__restrict__ alpha, int r, int RW,
                  float4 *__restrict__ R) {
    extern __shared__ float lut[];
    const int Q = RW * 8;
    for (int e = threadIdx.x; e < Q * 16; e += kPeelThreads) {
        const int q = e >> 4, nib = e & 15;
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = 4 * q + j;
            const float a = t < r ? alpha[t] : 0.0f;
            s += ((nib >> j) & 1) ? -a : a;
        }
        lut[e] = s;
    }
    __syncthreads();
    const int64_t tiles = (n4 + kPeelThreads - 1) / kPeelThreads;
    const int64_t a = (int64_t)blockIdx.x / tiles;
    const int64_t q = ((int64_t)blockIdx.x % tiles) * kPeelThreads + threadIdx.x;
    if (q >= n4) return;
    const int64_t n = n4 * 4;
    float c[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int w = 0; w < RW; ++w) {
        const uint32_t uw = up[(int64_t)w * m + a];
        const uint4 vw = *reinterpret_cast<const uint4 *>(vp + (int64_t)w * n + 4 * q);
        const uint32_t x[4] = {uw ^ vw.x, uw ^ vw.y, uw ^ vw.z, uw ^ vw.w};
#pragma unroll
        for (int h = 0; h < 8; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) c[e] += lut[(8 * w + h) * 16 + ((x[e] >> (4 * h)) & 15u)];
    }
    const float4 wv = W[a * n4 + q];
    R[a * n4 + q] = make_float4(wv.x - c[0], wv.y - c[1], wv.z - c[2], wv.w - c[3]);
}

// ---------------------------------------------------------------------------
size_t peel_ws_bytes(int64_t m, int64_t n, int r) { return peel_layout(m, n, r).total; }

hipError_t launch_peel(const float *W, int64_t m, int64_t n, int r, int T, const uint32_t *v_init,
                       uint32_t *u_packed, uint32_t *v_packed, float *alpha, float *alpha_greedy,
                       float *R, void *ws, hipStream_t stream) {
    const PeelLayout L = peel_layout(m, n, r);
    const PeelPtrs P = peel_ptrs(L, ws);
    const int64_t n4 = n / 4;
    const float4 *W4 = reinterpret_cast<const float4 *>(W);
#define PEEL_CHECK()                                  \
    do {                                              \
        const hipError_t e_ = hipGetLastError();      \
        if (e_ != hipSuccess) return e_;              \
    } while (0)
    {
        const int64_t words = (int64_t)L.RW * (m + n);
        const int64_t grid = (words + kPeelThreads - 1) / kPeelThreads;
        hipLaunchKernelGGL(peel_zero_kernel, dim3((unsigned)(grid < 4096 ? grid : 4096)),
                           dim3(kPeelThreads), 0, stream, u_packed, (int64_t)L.RW * m);
        PEEL_CHECK();
        hipLaunchKernelGGL(peel_zero_kernel, dim3((unsigned)(grid < 4096 ? grid : 4096)),
                           dim3(kPeelThreads), 0, stream, v_packed, (int64_t)L.RW * n);
        PEEL_CHECK();
        hipLaunchKernelGGL(peel_zero_kernel, dim3(1), dim3(kPeelThreads), 0, stream, P.ucur,
                           (int64_t)L.Wm);
        PEEL_CHECK();
    }
    const unsigned row_grid = (unsigned)((m + 3) / 4);
    const dim3 col_grid((unsigned)((n4 + kPeelThreads - 1) / kPeelThreads), (unsigned)L.S);
    const unsigned fin_grid = (unsigned)L.NBf;
    for (int i = 0; i < r; ++i) {
        for (int t = 0; t < T; ++t) {
            const uint32_t *vsrc = t == 0 ? v_init + (int64_t)i * L.Wn : P.vcur;
            // beta_j = alpha_j (v_j . v)
            if (i > 0) {
                hipLaunchKernelGGL(peel_coef_kernel, dim3((unsigned)((i + 3) / 4)), dim3(kPeelThreads),
                                   (size_t)L.Wn * 4, stream, P.vbits, vsrc, L.Wn, n, i, P.ag, P.coef);
                PEEL_CHECK();
            }
            // s = R v
            hipLaunchKernelGGL(peel_row_kernel, dim3(row_grid), dim3(kPeelThreads), (size_t)L.Wn * 4,
                               stream, W4, m, n4, vsrc, L.Wn, u_packed, i, P.coef, P.ucur);
            PEEL_CHECK();
            // gamma_j = alpha_j (u_j . u)
            if (i > 0) {
                hipLaunchKernelGGL(peel_coef_kernel, dim3((unsigned)((i + 3) / 4)), dim3(kPeelThreads),
                                   (size_t)L.Wm * 4, stream, P.ubits, P.ucur, L.Wm, m, i, P.ag, P.coef);
                PEEL_CHECK();
            }
            // W^T u in K-slices, then t = R^T u and v = sign(t)
            hipLaunchKernelGGL(peel_col_kernel, col_grid, dim3(kPeelThreads), 0, stream, W4, m, n4,
                               P.ucur, L.rows_per_slice, reinterpret_cast<float4 *>(P.tpart));
            PEEL_CHECK();
            hipLaunchKernelGGL(peel_colfin_kernel, dim3(fin_grid), dim3(kPeelThreads), 0, stream,
                               P.tpart, L.S, n, v_packed, i, P.coef, P.vcur, t == T - 1 ? 1 : 0,
                               P.red, P.ucur, L.Wm);
            PEEL_CHECK();
        }
        hipLaunchKernelGGL(peel_term_kernel, dim3(1), dim3(1024), 0, stream, i, m, n, L.NBf, P.red,
                           P.ucur, P.vcur, L.Wm, L.Wn, P.ag, P.bvec, P.ubits, P.vbits, u_packed,
                           v_packed);
        PEEL_CHECK();
    }
    const unsigned gt = (unsigned)((r + 15) / 16);
    hipLaunchKernelGGL(peel_gram_kernel, dim3(gt, gt), dim3(256), 0, stream, P.ubits, P.vbits, L.Wm,
                       L.Wn, r, m, n, P.gram);
    PEEL_CHECK();
    for (int k0 = 0; k0 < r; k0 += kChol) {
        hipLaunchKernelGGL(peel_chol_panel_kernel, dim3(1), dim3(1024), 0, stream, P.gram, r, k0,
                           (double)m * (double)n, P.bad);
        PEEL_CHECK();
        const int rest = r - k0 - kChol;
        if (rest > 0) {
            const int T = (rest + 31) / 32;
            hipLaunchKernelGGL(peel_chol_update_kernel, dim3((unsigned)(T * (T + 1) / 2)), dim3(256), 0,
                               stream, P.gram, r, k0);
            PEEL_CHECK();
        }
    }
    hipLaunchKernelGGL(peel_trisolve_kernel, dim3(1), dim3(1024), 0, stream, P.gram, P.bvec, P.sol, r,
                       P.bad, P.ag, alpha, alpha_greedy);
    PEEL_CHECK();
    if (R) {
        const int64_t g = ((n4 + kPeelThreads - 1) / kPeelThreads) * m;
        hipLaunchKernelGGL(peel_resid_kernel, dim3((unsigned)g), dim3(kPeelThreads), (size_t)L.RW * 8 * 16 * 4, stream,
                           W4, m, n4, u_packed, v_packed, alpha, r, L.RW, reinterpret_cast<float4 *>(R));
        PEEL_CHECK();
    }
#undef PEEL_CHECK
    return hipSuccess;
}

}  // namespace biloco
