// Stages 2 and 3: damping with dead-channel skip, and the upper factor U of
// H^-1 (aicassindra.com "tm_gptq_math", "The Cholesky trick for the inverse
// Hessian"; math4ai "GPTQ Hessian", column-sweep paragraph, H^-1 = U^T U;
// mbrenndoerfer "GPTQ > Mathematical Details of the Update", Cholesky
// paragraph).
//
// Route: with J the index reversal, J H J = L L^T (ordinary lower Cholesky)
// gives H = R R^T with R = J L J upper, and U = R^-1 = J L^-1 J is the upper
// Cholesky factor of H^-1 by uniqueness.  L^-1 is formed together with L in
// one right-looking blocked sweep over G = J H J (float64, in place): step k
// factors the diagonal block and inverts it (one workgroup), forms the panel
// P_i = G_ik L_kk^-T and the inverse row M_kj = L_kk^-1 G_kj (MFMA f64), and
// updates every block below it,
//     G_ij -= P_i M_kj   (j <= k, the inverse being built)
//     G_ij -= P_i P_j^T  (k < j <= i, the trailing matrix),
// which is forward substitution L M = I carried alongside the factorization.
// After the last step the lower triangle of G holds M = L^-1 and U is read
// off it reversed and rounded to float32.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace gptq {

namespace {

constexpr int NB = kCholNB;  // 64
constexpr int kGemmThreads = 256;
constexpr int kKc = 32;        // k per LDS stage of the tile GEMM
constexpr int kLdsLd = NB + 8;   // padded LDS row (doubles)

struct HinvWs {
    double* G;      // [n_pad, n_pad]
    double* P;      // [n_pad / NB][NB][NB]
    double* scal;   // [0] = lambda
    int* fail;      // device flag: set once a pivot fails
};

__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

HinvWs carve(void* ws, int64_t n) {
    const int64_t np = round_up(n, NB);
    char* p = static_cast<char*>(ws);
    HinvWs w;
    w.G = reinterpret_cast<double*>(p);
    p += round_up(np * np * 8, 256);
    w.P = reinterpret_cast<double*>(p);
    p += round_up(np * NB * 8, 256);
    w.scal = reinterpret_cast<double*>(p);
    p += 256;
    w.fail = reinterpret_cast<int*>(p);
    return w;
}

__device__ __forceinline__ void tri_index(int64_t b, int64_t& I, int64_t& J) {
    int64_t i = (int64_t)((sqrt(8.0 * (double)b + 1.0) - 1.0) * 0.5);
    while ((i + 1) * (i + 2) / 2 <= b) ++i;
    while (i * (i + 1) / 2 > b) --i;
    I = i;
    J = b - i * (i + 1) / 2;
}

// ---------------------------------------------------------------------------
// S2: lambda = damp * mean(diag H), dead flags, status words cleared
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void diag_stats_kernel(const float* __restrict__ H, int64_t n, double damp,
                                                          uint8_t* __restrict__ dead, double* __restrict__ scal,
                                                          double* __restrict__ lambda_out, int32_t* __restrict__ info,
                                                          int* __restrict__ fail) {
    __shared__ double part[16];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
        float h = H[i * n + i];
        s += (double)h;
        if (dead) dead[i] = (h == 0.0f) ? 1 : 0;
    }
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += part[w];
        double lam = damp * (t / (double)n);
        scal[0] = lam;
        if (lambda_out) *lambda_out = lam;
        *info = 0;
        *fail = 0;
    }
}

// ---------------------------------------------------------------------------
// G = J (H + damping) J in float64, lower triangle, padded with identity.
// G[i][j] = H[n-1-j][n-1-i] (a lower-triangle element of H for i >= j).
// One 64x64 lower tile of G per workgroup, transposed through LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void load_reversed_kernel(const float* __restrict__ H, int64_t n, int64_t np,
                                                            const double* __restrict__ scal,
                                                            double* __restrict__ G) {
    __shared__ float T[64][65];
    int64_t TI, TJ;
    tri_index(blockIdx.x, TI, TJ);
    const double lam = scal[0];
    const int tid = threadIdx.x;
    // stage: T[jj][ii] = H[n-1-(64TJ+jj)][n-1-(64TI+ii)], reading H rows contiguously
    for (int e = tid; e < 64 * 64; e += 256) {
        int jj = e >> 6, ii = e & 63;
        int64_t i = TI * 64 + ii, j = TJ * 64 + jj;
        float v = 0.0f;
        if (i < n && j < n && i >= j) v = H[(n - 1 - j) * n + (n - 1 - i)];
        T[jj][ii] = v;
    }
    __syncthreads();
    for (int e = tid; e < 64 * 64; e += 256) {
        int ii = e >> 6, jj = e & 63;
        int64_t i = TI * 64 + ii, j = TJ * 64 + jj;
        double g;
        if (i >= n || j >= n) {
            g = (i == j) ? 1.0 : 0.0;
        } else if (i == j) {
            double h = (double)T[jj][ii];
            g = (h == 0.0 ? 1.0 : h) + lam;
        } else if (i > j) {
            g = (double)T[jj][ii];
        } else {
            g = 0.0;
        }
        G[i * np + j] = g;
    }
}

// ---------------------------------------------------------------------------
// Diagonal block k: Cholesky factor L_kk and its inverse M = L_kk^-1 in one
// workgroup, as Gauss-Jordan elimination of [A | I] with symmetric pivots.
// Pivot c with p = A_cc uses the raw vectors
//     a_i = A_ic for i > c, 0 otherwise          (column c of A)
//     b_j = B_cj for j <= c, 0 otherwise         (row c of B)
// and every thread updates its own entries with no case split:
//     A_ij -= (a_i / p) a_j        B_ij -= (a_i / p) b_j
// (the zeros leave finished rows and unreached columns untouched); then the
// owners of column c store L_ic = a_i / sqrt(p), L_cc = sqrt(p), and the
// owners of row c store M_cj = b_j / sqrt(p).  The owners of column c+1 and
// row c+1 publish the next raw vectors and pivot into the other LDS buffer
// right after their update, so one barrier per pivot suffices.
// 512 threads; thread t owns rows 2(t/16)..+1, columns 4(t%16)..+3 of both
// A and B in registers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double rsqrt_f64(double x) {
    double y = __builtin_amdgcn_rsq(x);
    const double h = 0.5 * x * y;
    y = fma(y, fma(-h, y, 0.5), y);
    return y;
}

struct DiagVec {
    double a[2][NB];
    double b[2][NB];
    double piv[2];
};

// publish the raw vectors of pivot c (into buffer c & 1) from registers
template <int CC>
__device__ __forceinline__ void diag_publish(int c, int a, int b, const double (&g)[2][4], const double (&m)[2][4],
                                             DiagVec& v) {
    constexpr int CR = CC & 1;
    const int buf = c & 1;
    if (b == (c >> 2)) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int i = 2 * a + r;
            v.a[buf][i] = (i > c) ? g[r][CC] : 0.0;
            if (i == c) v.piv[buf] = g[r][CC];
        }
    }
    if (a == (c >> 1)) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int j = 4 * b + q;
            v.b[buf][j] = (j <= c) ? m[CR][q] : 0.0;
        }
    }
}

template <int CC>
__device__ __forceinline__ bool diag_pivot(int c, int a, int b, double (&g)[2][4], double (&m)[2][4], DiagVec& v) {
    constexpr int CR = CC & 1;
    const int buf = c & 1;
    const double pv = v.piv[buf];
    if (!(pv > 0.0)) return false;  // uniform: every thread reads the same value
    const double rs = rsqrt_f64(pv);
    const double inv = rs * rs;
    double ti[2], aj[4], bj[4];
#pragma unroll
    for (int r = 0; r < 2; ++r) ti[r] = v.a[buf][2 * a + r] * inv;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        aj[q] = v.a[buf][4 * b + q];
        bj[q] = v.b[buf][4 * b + q];
    }
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            g[r][q] = fma(-ti[r], aj[q], g[r][q]);
            m[r][q] = fma(-ti[r], bj[q], m[r][q]);
        }
    if (b == (c >> 2)) {  // column c of L
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int i = 2 * a + r;
            g[r][CC] = (i > c) ? g[r][CC] * rs : ((i == c) ? pv * rs : g[r][CC]);
        }
    }
    if (a == (c >> 1)) {  // row c of M
#pragma unroll
        for (int q = 0; q < 4; ++q) m[CR][q] *= rs;
    }
    if (c + 1 < NB) diag_publish<(CC + 1) & 3>(c + 1, a, b, g, m, v);
    __syncthreads();
    return true;
}

__global__ __launch_bounds__(512) void chol_diag_kernel(double* __restrict__ G, int64_t np, int k,
                                                        int32_t* __restrict__ info, int* __restrict__ fail) {
    __shared__ __align__(16) DiagVec v;
    if (*fail) return;
    const int tid = threadIdx.x;
    const int a = tid >> 4, b = tid & 15;  // rows 2a, 2a+1; columns 4b .. 4b+3
    double* blk = G + (int64_t)k * NB * np + (int64_t)k * NB;
    double g[2][4], m[2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            g[r][c] = blk[(int64_t)(2 * a + r) * np + 4 * b + c];
            m[r][c] = (2 * a + r == 4 * b + c) ? 1.0 : 0.0;
        }
    diag_publish<0>(0, a, b, g, m, v);
    __syncthreads();

    int failed_at = -1;
    for (int c0 = 0; c0 < NB; c0 += 4) {
        if (!diag_pivot<0>(c0 + 0, a, b, g, m, v)) { failed_at = c0 + 0; break; }
        if (!diag_pivot<1>(c0 + 1, a, b, g, m, v)) { failed_at = c0 + 1; break; }
        if (!diag_pivot<2>(c0 + 2, a, b, g, m, v)) { failed_at = c0 + 2; break; }
        if (!diag_pivot<3>(c0 + 3, a, b, g, m, v)) { failed_at = c0 + 3; break; }
    }
    if (failed_at >= 0) {
        if (tid == 0) {
            *info = k * NB + failed_at + 1;
            *fail = 1;
        }
        return;
    }
    // write back M = L^-1 (exactly zero above the diagonal)
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) blk[(int64_t)(2 * a + r) * np + 4 * b + q] = m[r][q];
}

// ---------------------------------------------------------------------------
// 64x64x64 float64 tile product on MFMA 16x16x4 f64:  acc += A B.
// A is given row-major [64 rows][64 k] (lda); B is row-major [64 k][64 cols]
// (ldb) or, with kBT, its transpose given row-major [64 cols][64 k].
// Four waves in a 2x2 grid, each 32x32 as 2x2 MFMA tiles.  K runs in two
// chunks of 32: chunk 1 is fetched into registers while the MFMAs consume
// chunk 0 (two LDS buffers, one barrier per chunk).
// ---------------------------------------------------------------------------
struct GemmLds {
    double A[2][kKc][kLdsLd];
    double B[2][kKc][kLdsLd];
};

template <bool kBT>
struct GemmRegs {
    double a[8];
    double b[8];
};

// thread -> A^T: row tid&63, k run (tid>>6)*8 ; B direct: k row tid>>3, cols (tid&7)*8 ;
// B^T: col tid&63, k run (tid>>6)*8
template <bool kBT>
__device__ __forceinline__ void gemm_fetch(GemmRegs<kBT>& r, const double* __restrict__ A, int64_t lda,
                                           const double* __restrict__ B, int64_t ldb, int k0, int tid) {
    const double* sa = A + (int64_t)(tid & 63) * lda + k0 + (tid >> 6) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) r.a[e] = sa[e];
    if (kBT) {
        const double* sb = B + (int64_t)(tid & 63) * ldb + k0 + (tid >> 6) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) r.b[e] = sb[e];
    } else {
        const double* sb = B + (int64_t)(k0 + (tid >> 3)) * ldb + (tid & 7) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) r.b[e] = sb[e];
    }
}

template <bool kBT>
__device__ __forceinline__ void gemm_stash(const GemmRegs<kBT>& r, GemmLds& s, int buf, int tid) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s.A[buf][(tid >> 6) * 8 + e][tid & 63] = r.a[e];
    if (kBT) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s.B[buf][(tid >> 6) * 8 + e][tid & 63] = r.b[e];
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) s.B[buf][tid >> 3][(tid & 7) * 8 + e] = r.b[e];
    }
}

template <bool kBT>
__device__ __forceinline__ void tile_gemm_f64(const double* __restrict__ A, int64_t lda,
                                              const double* __restrict__ B, int64_t ldb, GemmLds& s,
                                              double4v (&acc)[2][2]) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wi = w >> 1, wj = w & 1;
    GemmRegs<kBT> regs;
    gemm_fetch<kBT>(regs, A, lda, B, ldb, 0, tid);
    constexpr int nch = NB / kKc;
#pragma unroll
    for (int c = 0; c < nch; ++c) {
        const int buf = c & 1;
        gemm_stash<kBT>(regs, s, buf, tid);
        __syncthreads();
        if (c + 1 < nch) gemm_fetch<kBT>(regs, A, lda, B, ldb, (c + 1) * kKc, tid);
#pragma unroll
        for (int ks = 0; ks < kKc; ks += 4) {
            double av[2], bv[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) av[m] = s.A[buf][ks + (lane >> 4)][wi * 32 + 16 * m + (lane & 15)];
#pragma unroll
            for (int q = 0; q < 2; ++q) bv[q] = s.B[buf][ks + (lane >> 4)][wj * 32 + 16 * q + (lane & 15)];
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int q = 0; q < 2; ++q) acc[m][q] = mfma16x16x4_f64(av[m], bv[q], acc[m][q]);
        }
    }
}

// mode 0: C = acc ; mode 1: C -= acc ; mode 2: C = -acc
template <int kMode>
__device__ __forceinline__ void tile_store_f64(double* __restrict__ C, int64_t ldc, const double4v (&acc)[2][2]) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wi = w >> 1, wj = w & 1;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = wi * 32 + 16 * m + 4 * v + (lane >> 4);
                const int col = wj * 32 + 16 * q + (lane & 15);
                double* p = C + (int64_t)row * ldc + col;
                if (kMode == 0) *p = acc[m][q][v];
                else if (kMode == 1) *p = *p - acc[m][q][v];
                else *p = -acc[m][q][v];
            }
}

__device__ __forceinline__ void zero_acc(double4v (&acc)[2][2]) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[m][q] = (double4v){};
}

// Panel of step k: blocks t < k form M_kt = Linv_kk G_kt (in place); blocks
// t >= k form P_i = G_ik Linv_kk^T with i = t + 1.
__global__ __launch_bounds__(kGemmThreads) void chol_panel_kernel(double* __restrict__ G, int64_t np,
                                                                  double* __restrict__ P, int k,
                                                                  const int* __restrict__ fail) {
    __shared__ GemmLds s;
    if (*fail) return;
    const int t = blockIdx.x;
    const double* Lkk = G + (int64_t)k * NB * np + (int64_t)k * NB;
    double4v acc[2][2];
    zero_acc(acc);
    if (t < k) {
        double* Gkt = G + (int64_t)k * NB * np + (int64_t)t * NB;
        tile_gemm_f64<false>(Lkk, np, Gkt, np, s, acc);
        tile_store_f64<0>(Gkt, np, acc);
    } else {
        const int i = t + 1;
        const double* Gik = G + (int64_t)i * NB * np + (int64_t)k * NB;
        tile_gemm_f64<true>(Gik, np, Lkk, np, s, acc);
        tile_store_f64<0>(P + (int64_t)i * NB * NB, NB, acc);
    }
}

// Update of step k over blocks (i, j), k < i, j <= i.
__global__ __launch_bounds__(kGemmThreads) void chol_trail_kernel(double* __restrict__ G, int64_t np,
                                                                  const double* __restrict__ P, int k,
                                                                  const int* __restrict__ fail) {
    __shared__ GemmLds s;
    if (*fail) return;
    const int64_t base = (int64_t)(k + 1) * (k + 2) / 2;
    int64_t i, j;
    tri_index(base + blockIdx.x, i, j);
    const double* Pi = P + i * NB * NB;
    double* Gij = G + i * NB * np + j * NB;
    double4v acc[2][2];
    zero_acc(acc);
    if (j < k) {
        tile_gemm_f64<false>(Pi, NB, G + (int64_t)k * NB * np + j * NB, np, s, acc);
        tile_store_f64<1>(Gij, np, acc);
    } else if (j == k) {
        tile_gemm_f64<false>(Pi, NB, G + (int64_t)k * NB * np + (int64_t)k * NB, np, s, acc);
        tile_store_f64<2>(Gij, np, acc);
    } else {
        tile_gemm_f64<true>(Pi, NB, P + j * NB * NB, NB, s, acc);
        tile_store_f64<1>(Gij, np, acc);
    }
}

// U[i][j] = M[n-1-i][n-1-j] for j >= i, 0 below the diagonal; one row per block.
__global__ __launch_bounds__(256) void store_u_kernel(const double* __restrict__ G, int64_t np, int64_t n,
                                                      float* __restrict__ U, const int* __restrict__ fail) {
    if (*fail) return;
    const int64_t i = blockIdx.x;
    const double* grow = G + (n - 1 - i) * np;
    float* urow = U + i * n;
    for (int64_t j = threadIdx.x; j < n; j += blockDim.x) urow[j] = (j >= i) ? (float)grow[n - 1 - j] : 0.0f;
}

}  // namespace

size_t hinv_workspace_bytes(int64_t n) {
    const int64_t np = round_up(n, NB);
    return (size_t)(round_up(np * np * 8, 256) + round_up(np * NB * 8, 256) + 256 + 256);
}

hipError_t launch_prepare_hinv(const float* H, int64_t n, double damp_frac, float* U, uint8_t* dead,
                               int32_t* info, double* lambda_out, void* ws, hipStream_t s) {
    if (n == 0) return hipSuccess;
    HinvWs w = carve(ws, n);
    const int64_t np = round_up(n, NB);
    const int T = (int)(np / NB);
    {
        TimedLaunch t(K_HINV_DIAGSUM, s);
        hipLaunchKernelGGL(diag_stats_kernel, dim3(1), dim3(1024), 0, s, H, n, damp_frac, dead, w.scal, lambda_out,
                           info, w.fail);
    }
    {
        TimedLaunch t(K_HINV_LOAD, s);
        hipLaunchKernelGGL(load_reversed_kernel, dim3((unsigned)((int64_t)T * (T + 1) / 2)), dim3(256), 0, s, H, n,
                           np, (const double*)w.scal, w.G);
    }
    for (int k = 0; k < T; ++k) {
        {
            TimedLaunch t(K_CHOL_DIAG, s);
            hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(512), 0, s, w.G, np, k, info, w.fail);
        }
        if (T > 1) {
            TimedLaunch t(K_CHOL_PANEL, s);
            hipLaunchKernelGGL(chol_panel_kernel, dim3(T - 1), dim3(kGemmThreads), 0, s, w.G, np, w.P, k,
                               (const int*)w.fail);
        }
        const int64_t tiles = (int64_t)T * (T + 1) / 2 - (int64_t)(k + 1) * (k + 2) / 2;
        if (tiles > 0) {
            TimedLaunch t(K_CHOL_TRAIL, s);
            hipLaunchKernelGGL(chol_trail_kernel, dim3((unsigned)tiles), dim3(kGemmThreads), 0, s, w.G, np,
                               (const double*)w.P, k, (const int*)w.fail);
        }
    }
    {
        TimedLaunch t(K_HINV_STORE, s);
        hipLaunchKernelGGL(store_u_kernel, dim3((unsigned)n), dim3(256), 0, s, (const double*)w.G, np, n, U,
                           (const int*)w.fail);
    }
    return hipGetLastError();
}

}  // namespace gptq
