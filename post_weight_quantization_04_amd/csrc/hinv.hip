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
constexpr int kLdsLd = NB + 16;  // padded LDS row (doubles)

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
// Diagonal block k: in-place Cholesky with simultaneous inversion.
// Pivot c: d = sqrt(G_cc); row c becomes the scaled inverse row, column c
// below the pivot becomes l = G_ic / d, and every later row is updated:
//   j < c: G_ij -= l_i M_cj ; j == c: G_ic = -l_i / d ; j > c: G_ij -= l_i l_j.
// Thread t owns the 4x4 sub-block (t/16, t%16) in registers.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void chol_diag_kernel(double* __restrict__ G, int64_t np, int k,
                                                        int32_t* __restrict__ info, int* __restrict__ fail) {
    __shared__ double s_piv;
    __shared__ double prow[2][NB];
    __shared__ double lcol[2][NB];
    if (*fail) return;
    const int tid = threadIdx.x;
    const int a = tid >> 4, b = tid & 15;
    const bool active = (b <= a);
    double* blk = G + (int64_t)k * NB * np + (int64_t)k * NB;
    double g[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) g[r][c] = active ? blk[(int64_t)(4 * a + r) * np + 4 * b + c] : 0.0;

    for (int c = 0; c < NB; ++c) {
        const int buf = c & 1, ca = c >> 2, cr = c & 3;
        if (a == ca && b == ca) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (r == cr) s_piv = g[r][r];
        }
        __syncthreads();
        const double pv = s_piv;
        if (!(pv > 0.0)) {  // uniform: every thread reads the same value
            if (tid == 0) {
                *info = k * NB + c + 1;
                *fail = 1;
            }
            return;
        }
        const double rd = 1.0 / sqrt(pv);
        if (active && a == ca) {
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                int j = 4 * b + cc;
                if (j < c) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (r == cr) prow[buf][j] = g[r][cc] * rd;
                }
            }
        }
        if (active && b == ca) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                int i = 4 * a + rr;
                if (i > c) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (q == cr) lcol[buf][i] = g[rr][q] * rd;
                }
            }
        }
        __syncthreads();
        if (active && 4 * a + 3 >= c) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int i = 4 * a + rr;
                if (i < c) continue;
                const double li = (i > c) ? lcol[buf][i] : 0.0;
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    const int j = 4 * b + cc;
                    if (j > i) continue;
                    if (i == c) {
                        g[rr][cc] = (j < c) ? g[rr][cc] * rd : rd;
                    } else if (j < c) {
                        g[rr][cc] -= li * prow[buf][j];
                    } else if (j == c) {
                        g[rr][cc] = -li * rd;
                    } else {
                        g[rr][cc] -= li * lcol[buf][j];
                    }
                }
            }
        }
    }
    // write back L^-1 of the block with an explicit zero upper triangle
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            int i = 4 * a + r, j = 4 * b + c;
            blk[(int64_t)i * np + j] = (j <= i) ? g[r][c] : 0.0;
        }
}

// ---------------------------------------------------------------------------
// 64x64x64 float64 tile product on MFMA 16x16x4 f64:  acc += A B.
// A is given row-major [64 rows][64 k] (lda); B is row-major [64 k][64 cols]
// (ldb) or, with kBT, its transpose given row-major [64 cols][64 k].
// Four waves in a 2x2 grid, each 32x32 as 2x2 MFMA tiles.
// ---------------------------------------------------------------------------
struct GemmLds {
    double A[kKc][kLdsLd];
    double B[kKc][kLdsLd];
};

template <bool kBT>
__device__ __forceinline__ void tile_gemm_f64(const double* __restrict__ A, int64_t lda,
                                              const double* __restrict__ B, int64_t ldb, GemmLds& s,
                                              double4v (&acc)[2][2]) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wi = w >> 1, wj = w & 1;
    for (int k0 = 0; k0 < NB; k0 += kKc) {
        {  // A^T into LDS: thread -> (row = tid & 63, k run of 8)
            const int row = tid & 63, kc = (tid >> 6) * 8;
            const double* src = A + (int64_t)row * lda + k0 + kc;
#pragma unroll
            for (int e = 0; e < 8; ++e) s.A[kc + e][row] = src[e];
        }
        if (kBT) {
            const int col = tid & 63, kc = (tid >> 6) * 8;
            const double* src = B + (int64_t)col * ldb + k0 + kc;
#pragma unroll
            for (int e = 0; e < 8; ++e) s.B[kc + e][col] = src[e];
        } else {
            const int kk = tid >> 3, cc = (tid & 7) * 8;
            const double* src = B + (int64_t)(k0 + kk) * ldb + cc;
#pragma unroll
            for (int e = 0; e < 8; ++e) s.B[kk][cc + e] = src[e];
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kKc; ks += 4) {
            double av[2], bv[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) av[m] = s.A[ks + (lane >> 4)][wi * 32 + 16 * m + (lane & 15)];
#pragma unroll
            for (int q = 0; q < 2; ++q) bv[q] = s.B[ks + (lane >> 4)][wj * 32 + 16 * q + (lane & 15)];
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int q = 0; q < 2; ++q) acc[m][q] = mfma16x16x4_f64(av[m], bv[q], acc[m][q]);
        }
        __syncthreads();
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
            hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(256), 0, s, w.G, np, k, info, w.fail);
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
