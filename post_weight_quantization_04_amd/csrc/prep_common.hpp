// Stage 2 plumbing shared by both factorization precisions (float64 and
// float32 tiles): the damping statistics, the reversed load of H into the
// tiled working matrix G = J (H + damping) J, and the read-off of U from
// G = L^-1 (aicassindra.com "tm_gptq_math", "The Cholesky trick for the
// inverse Hessian"; mbrenndoerfer "GPTQ > Mathematical Details of the
// Update", Cholesky paragraph).  Included by one translation unit per
// precision; everything here has internal linkage.
#pragma once

#include <math.h>
#include <stdint.h>

#include "common.hpp"
#include "kernels.hpp"

namespace gptq {
namespace {

constexpr int kPrepNB = kCholNB;  // 64: tile side of G

__host__ __device__ constexpr int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// G is stored by 64x64 tiles: tile (I, J) of the np x np matrix is 64*64
// contiguous elements, row-major inside (row stride 64), so that every tile
// the factorization reads or writes is one contiguous block.
__host__ __device__ inline int64_t gt(int64_t np, int64_t I, int64_t J) {
    return (I * (np / kPrepNB) + J) * kPrepNB * kPrepNB;
}

// Lower tile b of a row-major enumeration of the lower triangle: (I, J).
__device__ __forceinline__ void tri_index(int64_t b, int64_t& I, int64_t& J) {
    int64_t i = (int64_t)((sqrt(8.0 * (double)b + 1.0) - 1.0) * 0.5);
    while ((i + 1) * (i + 2) / 2 <= b) ++i;
    while (i * (i + 1) / 2 > b) --i;
    I = i;
    J = b - i * (i + 1) / 2;
}

// The statistics inside the reversed load: every workgroup of a diagonal
// tile sums the whole diagonal of H itself, in float64 and in one fixed
// order (so every copy of lambda is the same number), and marks the dead
// channels of its own tile; workgroup 0 (tile (0, 0)) publishes lambda and
// clears the status words.  This replaces diag_stats_kernel and its launch.
__device__ __forceinline__ double diag_lambda(const float* __restrict__ H, int64_t n, double damp, double* red) {
    double s = 0.0;
    constexpr int kB = 8;
    for (int64_t i0 = threadIdx.x; i0 < n; i0 += (int64_t)kB * blockDim.x) {
        float h[kB];
#pragma unroll
        for (int b = 0; b < kB; ++b) {
            const int64_t i = i0 + (int64_t)b * blockDim.x;
            h[b] = (i < n) ? H[i * n + i] : 0.0f;
        }
#pragma unroll
        for (int b = 0; b < kB; ++b) s += (double)h[b];
    }
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    double t = 0.0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
    return damp * (t / (double)n);
}

// G = J (H + damping) J, lower triangle, padded with identity, in the tile
// element type E.  G[i][j] = H[n-1-j][n-1-i] (a lower-triangle element of H
// for i >= j); a dead channel's zero diagonal becomes 1 before the damping
// is added, which decouples it (its row and column are zero).  The damped
// diagonal is formed in float64 and rounded once to E.  One 64x64 lower tile
// of G per workgroup, transposed through LDS.
template <typename E>
__global__ __launch_bounds__(256) void load_reversed_kernel(const float* __restrict__ H, int64_t n, int64_t np,
                                                            double damp, uint8_t* __restrict__ dead,
                                                            double* __restrict__ lambda_out,
                                                            int32_t* __restrict__ info, int* __restrict__ fail,
                                                            E* __restrict__ G) {
    __shared__ float T[64][65];
    __shared__ double red[4];
    int64_t TI, TJ;
    tri_index(blockIdx.x, TI, TJ);
    const int tid = threadIdx.x;
    double lam = 0.0;
    if (TI == TJ) {  // block-uniform
        lam = diag_lambda(H, n, damp, red);
        // dead flags of this tile's channels: G index i is channel n-1-i
        if (dead && tid < 64) {
            const int64_t i = TI * 64 + tid;
            if (i < n) dead[n - 1 - i] = (H[(n - 1 - i) * n + (n - 1 - i)] == 0.0f) ? 1 : 0;
        }
        if (blockIdx.x == 0 && tid == 0) {
            if (lambda_out) *lambda_out = lam;
            *info = 0;
            *fail = 0;
        }
    }
    // stage: T[jj][ii] = H[n-1-(64TJ+jj)][n-1-(64TI+ii)], reading H rows
    // contiguously; a thread's 16 loads are issued before any is used
    // (entries outside the triangle load H[0] and are replaced by zero)
    float v[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int e = tid + 256 * m;
        const int jj = e >> 6, ii = e & 63;
        const int64_t i = TI * 64 + ii, j = TJ * 64 + jj;
        const bool ok = i < n && j < n && i >= j;
        v[m] = H[ok ? (n - 1 - j) * n + (n - 1 - i) : 0];
        if (!ok) v[m] = 0.0f;
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int e = tid + 256 * m;
        T[e >> 6][e & 63] = v[m];
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
        G[gt(np, TI, TJ) + e] = (E)g;
    }
}

// U[i][j] = M[n-1-i][n-1-j] for j >= i, 0 below the diagonal, with M = L^-1
// in the lower triangle of G; one row per workgroup.
template <typename E>
__global__ __launch_bounds__(256) void store_u_kernel(const E* __restrict__ G, int64_t np, int64_t n,
                                                      float* __restrict__ U, const int* __restrict__ fail) {
    if (*fail) return;
    const int64_t i = blockIdx.x;
    const int64_t r = n - 1 - i;
    const E* grow = G + gt(np, r / kPrepNB, 0) + (r % kPrepNB) * kPrepNB;  // row r of tile column 0
    float* urow = U + i * n;
    // eight loads per thread in flight before any store (entries below the
    // diagonal load grow[0] and are written as zero)
    constexpr int kB = 8;
    for (int64_t j0 = threadIdx.x; j0 < n; j0 += (int64_t)kB * blockDim.x) {
        E g[kB];
#pragma unroll
        for (int b = 0; b < kB; ++b) {
            const int64_t j = j0 + (int64_t)b * blockDim.x;
            const int64_t c = n - 1 - j;
            const bool ok = j < n && j >= i;
            g[b] = grow[ok ? (c / kPrepNB) * kPrepNB * kPrepNB + (c % kPrepNB) : 0];
        }
#pragma unroll
        for (int b = 0; b < kB; ++b) {
            const int64_t j = j0 + (int64_t)b * blockDim.x;
            if (j < n) urow[j] = (j >= i) ? (float)g[b] : 0.0f;
        }
    }
}

}  // namespace
}  // namespace gptq
