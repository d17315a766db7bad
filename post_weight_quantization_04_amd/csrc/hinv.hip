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
#include <stdlib.h>

#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "prep_common.hpp"
#include "sched.hpp"

namespace gptq {

namespace {

constexpr int NB = kCholNB;  // 64
constexpr int kMaxDevices = 64;
constexpr int kGemmThreads = 256;
// Steps are paired (every other update of the rest deferred, then applied
// with the next step's as one 128-deep product) from sched::kPairMinTiles
// 64-wide tiles on.  Measured on MI355X: at d_in = 11008 (172 tiles) the
// factorization takes 25.5 ms paired against 29.0 ms unpaired (its
// trailing-matrix traffic dominates); at 4096 (64 tiles) 2.46 against
// 2.21 ms (the odd steps' longer critical part dominates).
constexpr int kLdsLd = NB + 8;   // padded LDS row (doubles)

struct HinvWs {
    double* G;      // n_pad x n_pad by 64x64 tiles (see gt)
    double* P;      // 3 x [n_pad / NB][NB][NB] (step s uses buffer s % 3)
    int* fail;      // device flag: set once a pivot fails
};

// Bytes of the factorization workspace for order n (layout in carve()).
constexpr size_t ws_bytes(int64_t n) {
    return (size_t)(round_up(round_up(n, NB) * round_up(n, NB) * 8, 256) + 3 * round_up(round_up(n, NB) * NB * 8, 256) +
                    256);
}

// Fixed device scratch of gptq_prepare_hinv_noalloc, for callers that cannot
// allocate: the workspace of the largest order it takes.  In host code the
// name is only a stand-in; the device address comes from
// hinv_noalloc_scratch() below.
static __device__ __align__(256) unsigned char scratch[ws_bytes(kNoAllocMaxDin)];

HinvWs carve(void* ws, int64_t n) {
    const int64_t np = round_up(n, NB);
    char* p = static_cast<char*>(ws);
    HinvWs w;
    w.G = reinterpret_cast<double*>(p);
    p += round_up(np * np * 8, 256);
    w.P = reinterpret_cast<double*>(p);  // three panel buffers
    p += 3 * round_up(np * NB * 8, 256);
    w.fail = reinterpret_cast<int*>(p);
    return w;
}

// ---------------------------------------------------------------------------
// Diagonal block k: M = L_kk^-1 where A = L_kk L_kk^T is the 64x64 block,
// by the same blocked route one level down, on 16x16 sub-blocks in LDS.
// Sub-step s (columns 16s .. 16s+15):
//   1. one wave inverts the Cholesky factor of the sub-block A_ss by
//      Gauss-Jordan elimination in registers (gj16 below): Ls = L_ss^-1;
//   2. P_i = A_is Ls^T for sub-blocks i > s, and M_sj = Ls A_sj in place for
//      j < s (one 16x16x16 MFMA product per wave);
//   3. A_ij -= P_i P_j^T (s < j <= i), A_is = -P_i Ls, A_ij -= P_i M_sj
//      (j < s), for every i > s.
// Only lower-triangle entries are read; the block returned holds exact
// zeros above the diagonal.
// ---------------------------------------------------------------------------
// 1/sqrt(x) to float64 accuracy: v_rsq_f64 refined by the second-order
// step y0 (1 + e/2 + 3e^2/8), e = 1 - x y0^2.
__device__ __forceinline__ double rsqrt_f64(double x) {
    const double y = __builtin_amdgcn_rsq(x);
    const double e = fma(-(x * y), y, 1.0);
    return fma(fma(0.375, e, 0.5) * e, y, y);
}

constexpr int kSb = 16;           // sub-block width
constexpr int kDLd = NB + 1;      // padded LDS row (doubles)

struct DiagLds {
    double g[NB][kDLd];           // the block: Schur complement, then the inverse
    double p[3][kSb][kSb + 1];    // P_i of the current sub-step
    int status;
};

// Lane-crossing moves of a double within one wave (no LDS):
//   bcast_in_row<N>: lane N of each 16-lane row, to the whole row (DPP
//     row_newbcast);
//   bcast_row<R>: row R (lanes 16R .. 16R+15), to all four rows, lane
//     position kept (permlane16 then permlane32 swap);
//   read_lane: one lane's value, uniform.
__device__ __forceinline__ uint32_t lo32(double x) { return (uint32_t)__builtin_bit_cast(uint64_t, x); }
__device__ __forceinline__ uint32_t hi32(double x) { return (uint32_t)(__builtin_bit_cast(uint64_t, x) >> 32); }
__device__ __forceinline__ double join64(uint32_t lo, uint32_t hi) {
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
template <int N>
__device__ __forceinline__ double bcast_in_row(double x) {
    const uint32_t lo = __builtin_amdgcn_mov_dpp((int)lo32(x), 0x150 + N, 0xF, 0xF, false);
    const uint32_t hi = __builtin_amdgcn_mov_dpp((int)hi32(x), 0x150 + N, 0xF, 0xF, false);
    return join64(lo, hi);
}
template <int R>
__device__ __forceinline__ uint32_t bcast_row32(uint32_t v) {
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // {rows 0,0,2,2}, {rows 1,1,3,3}
    const uint32_t y = (R & 1) ? a[1] : a[0];
    const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);  // {low half twice}, {high half twice}
    return (R & 2) ? b[1] : b[0];
}
template <int R>
__device__ __forceinline__ double bcast_row(double x) {
    return join64(bcast_row32<R>(lo32(x)), bcast_row32<R>(hi32(x)));
}
__device__ __forceinline__ double read_lane(double x, int l) {
    return join64((uint32_t)__builtin_amdgcn_readlane((int)lo32(x), l), (uint32_t)__builtin_amdgcn_readlane((int)hi32(x), l));
}

// 1/x to float64 accuracy: v_rcp_f64 refined by the cubic step
// y0 (1 + e + e^2), e = 1 - x y0 (three dependent FMAs).
__device__ __forceinline__ double rcp_f64(double x) {
    const double y = __builtin_amdgcn_rcp(x);
    const double e = fma(-x, y, 1.0);
    return fma(fma(e, e, e), y, y);
}

// Pivot C of the symmetric elimination of a 16x16 block A = L D L^T, kept
// in one array per lane.  With u_r = A_rC / p (p the pivot), every row r
// below C takes A_rj -= u_r A_Cj; column C of row r then keeps A_rC, which
// is -p times the entry (r, C) of L_unit^-1 (row operations applied to the
// identity).  That scaling is the same in every row, so the later pivots
// update those entries in place like the rest.  The pivot row is cleared
// from column C on after it has been broadcast (the broadcast copy carries
// a zero at C, which leaves column C as it is), so that no later pivot
// touches a row above it.  Lane (g = lane/16, j = lane%16) holds rows
// 4g .. 4g+3 of column j; pj collects the pivot of column j.  `first`
// records 1 + the first pivot that is not positive.
template <int C>
__device__ __forceinline__ void gj_step(int g, int j, double (&x)[4], double& pj, int& first) {
    constexpr int R = C >> 2, S = C & 3;
    const double p = read_lane(x[S], kSb * R + C);
    if (!(p > 0.0) && first == 0) first = C + 1;
    const double inv = rcp_f64(p);
    const double yrow = bcast_row<R>((j == C) ? 0.0 : x[S]);  // A[C][j], zero at j = C
    if (g == R && j >= C) x[S] = 0.0;
    if (j == C) pj = p;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const double u = bcast_in_row<C>(x[e]) * inv;  // A[4g+e][C] / p, zero for rows <= C
        x[e] = fma(-u, yrow, x[e]);
    }
}

// Sub-block s of L.g (one wave): Ls = inverse of its Cholesky factor,
// written in place (exact zeros above the diagonal).  After the pivots,
// entry (r, j < r) is -p_j (L_unit^-1)_rj and Ls = D^-1/2 L_unit^-1.
// Returns 0, or 1 + the local column of the first pivot that is not
// positive (wave-uniform).
__device__ __forceinline__ int gj16(DiagLds& L, int s, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int o = kSb * s;
    double x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        x[e] = (r >= j) ? L.g[o + r][o + j] : L.g[o + j][o + r];  // symmetric from the lower triangle
    }
    double pj = 1.0;
    int first = 0;
    gj_step<0>(g, j, x, pj, first);
    gj_step<1>(g, j, x, pj, first);
    gj_step<2>(g, j, x, pj, first);
    gj_step<3>(g, j, x, pj, first);
    gj_step<4>(g, j, x, pj, first);
    gj_step<5>(g, j, x, pj, first);
    gj_step<6>(g, j, x, pj, first);
    gj_step<7>(g, j, x, pj, first);
    gj_step<8>(g, j, x, pj, first);
    gj_step<9>(g, j, x, pj, first);
    gj_step<10>(g, j, x, pj, first);
    gj_step<11>(g, j, x, pj, first);
    gj_step<12>(g, j, x, pj, first);
    gj_step<13>(g, j, x, pj, first);
    gj_step<14>(g, j, x, pj, first);
    gj_step<15>(g, j, x, pj, first);
    const double nrj = -rcp_f64(pj);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        // the pivot of row r sits in lane 16 g + r (column r of the same row group)
        const int src = 4 * (kSb * g + r);
        const double pr = join64((uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)lo32(pj)),
                                 (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)hi32(pj)));
        const double rs = rsqrt_f64(pr);
        L.g[o + r][o + j] = (r < j) ? 0.0 : (r == j) ? rs : rs * (x[e] * nrj);
    }
    return first;
}

// 16x16x16 product on MFMA 16x16x4 f64: acc = X Y with X[i][k] = fx(i, k),
// Y[k][j] = fy(k, j); lane l gets C[4v + l/16][l%16] in acc[v].
template <typename FX, typename FY>
__device__ __forceinline__ double4v mm16(FX fx, FY fy, int lane) {
    double4v acc = {};
#pragma unroll
    for (int kk = 0; kk < kSb; kk += 4) {
        const int k = kk + (lane >> 4);
        acc = mfma16x16x4_f64(fx(lane & 15, k), fy(k, lane & 15), acc);
    }
    return acc;
}

// The lanes of one wave exchange data through LDS: the wave's LDS
// operations execute in order, so ordering the compiler is enough.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Factor and invert the block held in L.g (256 threads).  Returns 0 or
// 1 + the local column of the first pivot that is not positive
// (block-uniform).  One sub-step of lookahead: while wave 0 forms P_{s+1},
// updates the diagonal sub-block s+1 with it and runs that sub-block's
// pivots, waves 1..3 do every other panel and update tile of sub-step s.
// Two barriers per sub-step order the roles:
//   phase 1  wave 0: P_{s+1} = A_{s+1,s} Ls^T;  waves 1..3: P_i (i > s+1)
//            and M_sj = Ls A_sj (j < s), in place;
//   phase 2  wave 0: A_{s+1,s+1} -= P_{s+1} P_{s+1}^T, pivots of s+1;
//            waves 1..3: the other tiles (i, j), i > s, j <= i.
__device__ __forceinline__ int diag64(DiagLds& L) {
    const int lane = threadIdx.x & 63, w = wave_id();
    constexpr int S = NB / kSb;
    if (w == 0) {
        const int st = gj16(L, 0, lane);
        if (lane == 0) L.status = st;
    }
    __syncthreads();
    if (L.status) return L.status;
    for (int s = 0; s < S; ++s) {
        const int o = kSb * s;
        auto panel_p = [&](int i, int slot) {  // P_i = A_is Ls^T
            const double4v acc = mm16([&](int a, int k) { return L.g[kSb * i + a][o + k]; },
                                      [&](int k, int b) { return L.g[o + b][o + k]; }, lane);
#pragma unroll
            for (int v = 0; v < 4; ++v) L.p[slot][4 * v + (lane >> 4)][lane & 15] = acc[v];
        };
        // phase 1
        if (w == 0) {
            if (s + 1 < S) panel_p(s + 1, 0);
        } else {
            const int nP = S - 2 - s > 0 ? S - 2 - s : 0;  // P_i, i = s+2 .. S-1
            for (int q = w - 1; q < nP + s; q += 3) {
                if (q < nP) {
                    panel_p(s + 2 + q, q + 1);
                } else {
                    const int j = q - nP;
                    const double4v acc = mm16([&](int a, int k) { return L.g[o + a][o + k]; },
                                              [&](int k, int b) { return L.g[o + k][kSb * j + b]; }, lane);
#pragma unroll
                    for (int v = 0; v < 4; ++v) L.g[o + 4 * v + (lane >> 4)][kSb * j + (lane & 15)] = acc[v];
                }
            }
        }
        __syncthreads();
        // phase 2
        if (w == 0) {
            if (s + 1 < S) {
                const int o1 = o + kSb;
                const double4v acc = mm16([&](int a, int k) { return L.p[0][a][k]; },
                                          [&](int k, int b) { return L.p[0][b][k]; }, lane);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    double& d = L.g[o1 + 4 * v + (lane >> 4)][o1 + (lane & 15)];
                    d = d - acc[v];
                }
                wave_lds_sync();
                const int st = gj16(L, s + 1, lane);
                if (lane == 0) L.status = st;
            }
        } else {
            int t = 0;
            for (int i = s + 1; i < S; ++i) {
                for (int j = 0; j <= i; ++j) {
                    if (i == s + 1 && j == s + 1) continue;  // wave 0's
                    if (t++ % 3 != w - 1) continue;
                    const int pi = i - s - 1;
                    double4v acc;
                    if (j > s) {
                        const int pj = j - s - 1;
                        acc = mm16([&](int a, int k) { return L.p[pi][a][k]; },
                                   [&](int k, int b) { return L.p[pj][b][k]; }, lane);
                    } else {
                        acc = mm16([&](int a, int k) { return L.p[pi][a][k]; },
                                   [&](int k, int b) { return L.g[o + k][kSb * j + b]; }, lane);
                    }
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        double& d = L.g[kSb * i + 4 * v + (lane >> 4)][kSb * j + (lane & 15)];
                        d = (j == s) ? -acc[v] : d - acc[v];
                    }
                }
            }
        }
        __syncthreads();
        if (s + 1 < S && L.status) return kSb * (s + 1) + L.status;
    }
    return 0;
}

// ---------------------------------------------------------------------------
// 64x64x64 float64 tile product on MFMA 16x16x4 f64:  acc += A B.
// A is given row-major [64 rows][64 k] (lda); B is row-major [64 k][64 cols]
// (ldb) or, with kBT, its transpose given row-major [64 cols][64 k].
// Every operand tile is fetched in 16-byte pieces that run along its rows
// (thread t holds row 8e + t/32, columns 2(t%32) and 2(t%32)+1, in
// registers 2e and 2e+1, e = 0..7), so each wave's load covers two whole
// 512-byte rows; all of K is in registers at once (16 doubles of A and of B
// per thread, every load in flight together).  K is staged in LDS in two
// halves of 32 through one buffer (33.8 KB): A and a transposed B row-major
// with an odd row stride (33 doubles), so that the MFMA reads of 16 rows at
// one k fall on distinct banks; a direct B as [k][col] rows.  The four waves
// (2x2 grid, 32x32 each as 2x2 MFMA tiles) run 8 k-steps per half.
// ---------------------------------------------------------------------------
constexpr int kHalf = NB / 2;
constexpr int kRs = kHalf + 1;  // row stride of a row-major half stage (doubles)

struct GemmLds {
    double A[NB * kRs];  // A[row][k - 32h] at row * kRs
    double B[NB * kRs];  // B^T[col][k - 32h] at col * kRs, or B[k - 32h][col] at (k - 32h) * NB
};

struct GemmRegs {
    double a[16];
    double b[16];
};

typedef double double2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void tile_fetch(double (&r)[16], const double* __restrict__ src, int64_t ld, int tid) {
    const double* p = src + (int64_t)(tid >> 5) * ld + 2 * (tid & 31);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const double2v v = *reinterpret_cast<const double2v*>(p + (int64_t)(8 * e) * ld);
        r[2 * e] = v[0];
        r[2 * e + 1] = v[1];
    }
}
__device__ __forceinline__ void gemm_fetch_a(double (&a)[16], const double* __restrict__ A, int64_t lda, int tid) {
    tile_fetch(a, A, lda, tid);
}
template <bool kBT>
__device__ __forceinline__ void gemm_fetch_b(double (&b)[16], const double* __restrict__ B, int64_t ldb, int tid) {
    tile_fetch(b, B, ldb, tid);
}
template <bool kBT>
__device__ __forceinline__ void gemm_fetch(GemmRegs& r, const double* __restrict__ A, int64_t lda,
                                           const double* __restrict__ B, int64_t ldb, int tid) {
    tile_fetch(r.a, A, lda, tid);
    tile_fetch(r.b, B, ldb, tid);
}

// stage half h of a fetched tile kept row-major by k (A, or B given
// transposed): the threads whose two columns lie in that half write them
__device__ __forceinline__ void stash_rows(const double (&r)[16], double* __restrict__ S, int tid, int h) {
    const int col = 2 * (tid & 31);
    if ((col >> 5) != h) return;
    const int c = col - kHalf * h;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int row = 8 * e + (tid >> 5);
        S[row * kRs + c] = r[2 * e];
        S[row * kRs + c + 1] = r[2 * e + 1];
    }
}
// stage half h of a direct B (rows are k): registers 2e, e in 4h .. 4h+3
__device__ __forceinline__ void stash_direct(const double (&r)[16], double* __restrict__ S, int tid, int h) {
    const int col = 2 * (tid & 31);
#pragma unroll
    for (int e = 4 * h; e < 4 * h + 4; ++e) {
        const int k = 8 * e + (tid >> 5) - kHalf * h;
        *reinterpret_cast<double2v*>(&S[k * NB + col]) = (double2v){r[2 * e], r[2 * e + 1]};
    }
}
__device__ __forceinline__ void gemm_stash_a(const double (&a)[16], GemmLds& s, int tid, int h) {
    stash_rows(a, s.A, tid, h);
}
template <bool kBT>
__device__ __forceinline__ void gemm_stash_b(const double (&b)[16], GemmLds& s, int tid, int h) {
    if (kBT) stash_rows(b, s.B, tid, h);
    else stash_direct(b, s.B, tid, h);
}

template <bool kBT>
__device__ __forceinline__ void gemm_compute_half(const GemmLds& s, double4v (&acc)[2][2]) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wi = w >> 1, wj = w & 1;
#pragma unroll
    for (int ks = 0; ks < kHalf; ks += 4) {
        const int k = ks + (lane >> 4);
        double av[2], bv[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) av[m] = s.A[(wi * 32 + 16 * m + (lane & 15)) * kRs + k];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int col = wj * 32 + 16 * q + (lane & 15);
            bv[q] = kBT ? s.B[col * kRs + k] : s.B[k * NB + col];
        }
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int q = 0; q < 2; ++q) acc[m][q] = mfma16x16x4_f64(av[m], bv[q], acc[m][q]);
    }
}

// both halves from fetched registers
template <bool kBT>
__device__ __forceinline__ void gemm_stage_compute(const GemmRegs& r, GemmLds& s, double4v (&acc)[2][2]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (h) __syncthreads();  // every wave is done with half 0
        gemm_stash_a(r.a, s, tid, h);
        gemm_stash_b<kBT>(r.b, s, tid, h);
        __syncthreads();
        gemm_compute_half<kBT>(s, acc);
    }
}

// both halves from fetched registers, when the LDS stage may still be read
// by a previous product
template <bool kBT>
__device__ __forceinline__ void gemm_stage_compute_after(const GemmRegs& r, GemmLds& s, double4v (&acc)[2][2]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        __syncthreads();
        gemm_stash_a(r.a, s, tid, h);
        gemm_stash_b<kBT>(r.b, s, tid, h);
        __syncthreads();
        gemm_compute_half<kBT>(s, acc);
    }
}

template <bool kBT>
__device__ __forceinline__ void tile_gemm_f64(const double* __restrict__ A, int64_t lda,
                                              const double* __restrict__ B, int64_t ldb, GemmLds& s,
                                              double4v (&acc)[2][2]) {
    GemmRegs regs;
    gemm_fetch<kBT>(regs, A, lda, B, ldb, threadIdx.x);
    gemm_stage_compute<kBT>(regs, s, acc);
}

// C[row][col] of the accumulator element (m, q, v) of this thread
__device__ __forceinline__ int acc_row(int m, int v) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    return (w >> 1) * 32 + 16 * m + 4 * v + (lane >> 4);
}
__device__ __forceinline__ int acc_col(int q) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    return (w & 1) * 32 + 16 * q + (lane & 15);
}

// C -= A B with C's old values loaded behind the operand loads, so that
// their latency overlaps the staging and the products
template <bool kBT>
__device__ __forceinline__ void tile_gemm_sub_f64(const double* __restrict__ A, int64_t lda,
                                                  const double* __restrict__ B, int64_t ldb, double* __restrict__ C,
                                                  int64_t ldc, GemmLds& s) {
    GemmRegs regs;
    gemm_fetch<kBT>(regs, A, lda, B, ldb, threadIdx.x);
    double c[2][2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) c[m][q][v] = C[(int64_t)acc_row(m, v) * ldc + acc_col(q)];
    double4v acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[m][q] = (double4v){};
    gemm_stage_compute<kBT>(regs, s, acc);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) C[(int64_t)acc_row(m, v) * ldc + acc_col(q)] = c[m][q][v] - acc[m][q][v];
}

// C -= A1 B1 + A2 B2 (kSub) or C = -(A1 B1 + A2 B2): one 128-deep product
// with one read and one write of C.  The second pair's operands are fetched
// into the same registers once the first pair is staged, so their latency
// overlaps the first pair's second half; C's old values are loaded behind
// the first pair's operands.
template <bool kBT, bool kSub>
__device__ __forceinline__ void tile_gemm2_f64(const double* __restrict__ A1, const double* __restrict__ B1,
                                               const double* __restrict__ A2, const double* __restrict__ B2,
                                               double* __restrict__ C, GemmLds& s) {
    const int tid = threadIdx.x;
    GemmRegs r;
    gemm_fetch<kBT>(r, A1, NB, B1, NB, tid);
    double c[2][2][4];
    if (kSub) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int v = 0; v < 4; ++v) c[m][q][v] = C[acc_row(m, v) * NB + acc_col(q)];
    }
    double4v acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[m][q] = (double4v){};
    gemm_stash_a(r.a, s, tid, 0);
    gemm_stash_b<kBT>(r.b, s, tid, 0);
    __syncthreads();
    gemm_compute_half<kBT>(s, acc);
    __syncthreads();
    gemm_stash_a(r.a, s, tid, 1);
    gemm_stash_b<kBT>(r.b, s, tid, 1);
    __syncthreads();
    gemm_fetch<kBT>(r, A2, NB, B2, NB, tid);
    gemm_compute_half<kBT>(s, acc);
    gemm_stage_compute_after<kBT>(r, s, acc);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                C[acc_row(m, v) * NB + acc_col(q)] = kSub ? c[m][q][v] - acc[m][q][v] : -acc[m][q][v];
}

// mode 0: C = acc ; mode 2: C = -acc
template <int kMode>
__device__ __forceinline__ void tile_store_f64(double* __restrict__ C, int64_t ldc, const double4v (&acc)[2][2]) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                double* p = C + (int64_t)acc_row(m, v) * ldc + acc_col(q);
                *p = (kMode == 0) ? acc[m][q][v] : -acc[m][q][v];
            }
}

__device__ __forceinline__ void zero_acc(double4v (&acc)[2][2]) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[m][q] = (double4v){};
}

// Diagonal block and panel of step k in one launch.  Every workgroup factors
// and inverts the diagonal block itself (the work is latency-bound, so the
// copies cost no time) with its own panel operand already in flight, then
// forms its panel tile: t < k: M_kt = M_kk G_kt (in place); t >= k:
// P_i = G_ik M_kk^T with i = t + 1, into the panel buffer.  Workgroup 0 also
// writes M_kk (exact zeros above the diagonal) to tile 0 of the panel buffer,
// which the update of step k reads; G_kk itself is rewritten only later (by
// the early update), because other workgroups may still be reading it.
union DiagPanelLds {
    DiagLds diag;  // the factorization, then
    GemmLds gemm;  // the panel product (M_kk passes through registers)
};

__device__ __forceinline__ void diag_panel_body(DiagPanelLds& u, double* __restrict__ G, int64_t np, double* __restrict__ P, int k,
                                int T, int t, int32_t* __restrict__ info, int* __restrict__ fail) {
    const int tid = threadIdx.x;
    const bool has_tile = t < T - 1;
    const bool inv_row = t < k;  // M_kt rather than P_{t+1}
    double opnd[16];
    if (has_tile) {
        if (inv_row) gemm_fetch_b<false>(opnd, G + gt(np, k, t), NB, tid);
        else gemm_fetch_a(opnd, G + gt(np, t + 1, k), NB, tid);
    }
    DiagLds& L = u.diag;
    const double* blk = G + gt(np, k, k);
#pragma unroll
    for (int m = 0; m < NB * NB / kGemmThreads; ++m) {
        const int idx = tid + kGemmThreads * m;
        L.g[idx >> 6][idx & 63] = blk[idx];
    }
    __syncthreads();
    const int st = diag64(L);
    if (st) {
        if (t == 0 && tid == 0) {
            *info = k * NB + st;
            *fail = 1;
        }
        return;
    }
    if (t == 0) {
#pragma unroll
        for (int m = 0; m < NB * NB / kGemmThreads; ++m) {
            const int idx = tid + kGemmThreads * m;
            const int r = idx >> 6, c = idx & 63;
            P[idx] = (c <= r) ? L.g[r][c] : 0.0;
        }
    }
    if (!has_tile) return;
    // element e = (kk, x): M[x][kk] is A[x][kk] (M_kk as A) or B^T[x][kk]
    // (M_kk^T as B), both staged row-major by k; read out before the LDS is
    // restaged
    double mv[NB * NB / kGemmThreads];
#pragma unroll
    for (int m = 0; m < NB * NB / kGemmThreads; ++m) {
        const int e = tid + kGemmThreads * m;
        const int kk = e >> 6, x = e & 63;
        mv[m] = (kk <= x) ? L.g[x][kk] : 0.0;
    }
    __syncthreads();
    GemmLds& s = u.gemm;
    double4v acc[2][2];
    zero_acc(acc);
    // m = 0..7 fall in k-half 0 (kk = 4m + tid/64 < 32), m = 8..15 in half 1
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (h) __syncthreads();
        if (inv_row) {
#pragma unroll
            for (int m = 8 * h; m < 8 * h + 8; ++m) {
                const int e = tid + kGemmThreads * m;
                s.A[(e & 63) * kRs + (e >> 6) - kHalf * h] = mv[m];
            }
            gemm_stash_b<false>(opnd, s, tid, h);
        } else {
            gemm_stash_a(opnd, s, tid, h);
#pragma unroll
            for (int m = 8 * h; m < 8 * h + 8; ++m) {
                const int e = tid + kGemmThreads * m;
                s.B[(e & 63) * kRs + (e >> 6) - kHalf * h] = mv[m];
            }
        }
        __syncthreads();
        if (inv_row) gemm_compute_half<false>(s, acc);
        else gemm_compute_half<true>(s, acc);
    }
    if (inv_row) tile_store_f64<0>(G + gt(np, k, t), NB, acc);
    else tile_store_f64<0>(P + (int64_t)(t + 1) * NB * NB, NB, acc);
}

// A 64x64 tile held in accumulator layout (element (m, q, v) of each
// thread at acc_row(m, v), acc_col(q)).
__device__ __forceinline__ void tile_load_acc(double (&c)[2][2][4], const double* __restrict__ C, int64_t ldc) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) c[m][q][v] = C[(int64_t)acc_row(m, v) * ldc + acc_col(q)];
}

// Stage half h (k = 32h .. 32h+31) of an accumulator-layout tile X as the
// operand A = X (row-major by k); the columns of half h sit in waves
// w & 1 == h.
__device__ __forceinline__ void stash_acc_as_a(const double (&x)[2][2][4], GemmLds& s, int h) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if ((w & 1) != h) return;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) s.A[acc_row(m, v) * kRs + 16 * q + (lane & 15)] = x[m][q][v];
}

// ... as the direct operand B = X ([k][col] rows); the rows of half h sit
// in waves w >> 1 == h.
__device__ __forceinline__ void stash_acc_as_b(const double (&x)[2][2][4], GemmLds& s, int h) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if ((w >> 1) != h) return;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int kl = 16 * m + 4 * v + (lane >> 4);
                s.B[kl * NB + acc_col(q)] = x[m][q][v];
            }
}

// Diagonal block and panel of step k1 = k+1, with the update of step k of
// the blocks they read applied in the same workgroup (in registers, none of
// it written back): every workgroup forms D = G_k1k1 - P_k1 P_k1^T (the
// diagonal block after step k) and its own operand after step k,
//   t >= k1:  G_{t+1,k1} - P_{t+1} P_k1^T   (column block k1),
//   t == k:   -P_k1 M_kk                    (row block k1, G_{k1,k} = -P_k1 M_kk),
//   t <  k:   G_{k1,t} - P_k1 M_kt          (row block k1, M_kt in place in G_kt),
// with P_i and M_kk from the panel buffer of step k (Pk).  D is factored and
// inverted as in diag_panel_body and the panel tile formed from the
// updated operand: t < k1: M_k1t = M_k1k1 G_k1t (in place); t >= k1:
// P_{t+1} = G_{t+1,k1} M_k1k1^T into the panel buffer of step k1 (Pk1).
// The column-block blocks G_{t+1,k1} keep their old values: step k1
// overwrites them from P_{t+1} alone.
// The diagonal block and the product staging in separate storage (71 KB),
// so that D goes to LDS as soon as it is formed.
struct DiagPanelNextLds {
    DiagLds diag;
    GemmLds gemm;
};

template <bool kPair>
__device__ __forceinline__ void diag_panel_next_body(DiagPanelNextLds& u, double* __restrict__ G, int64_t np,
                                                     double* __restrict__ Pk1, const double* __restrict__ Pk,
                                                     const double* __restrict__ Pkm, int k, int T, int t,
                                                     int32_t* __restrict__ info, int* __restrict__ fail) {
    const int tid = threadIdx.x;
    const int k1 = k + 1;
    const bool has_tile = t < T - 1;
    const bool inv_row = t < k1;
    GemmLds& s = u.gemm;
    DiagLds& L = u.diag;
    const double* Pd = Pk + (int64_t)k1 * NB * NB;  // P_k1 of step k
    // operands of both products in flight at once: P_k1 serves as A and as
    // B^T of the first product and as one operand of the second
    double pd[16];
    gemm_fetch_a(pd, Pd, NB, tid);
    double xo[16];
    double c2[2][2][4];
    // with kPair, step k-1's update is still owed too, and G_{k1,k-1} holds
    // nothing yet (its step k-1 value -P_k1 M_{k-1,k-1} was never stored)
    const bool neg = inv_row && (t == k || (kPair && t == k - 1));
    if (has_tile) {
        if (!inv_row) {
            gemm_fetch_a(xo, Pk + (int64_t)(t + 1) * NB * NB, NB, tid);
            tile_load_acc(c2, G + gt(np, t + 1, k1), NB);
        } else if (t == k) {
            gemm_fetch_b<false>(xo, Pk, NB, tid);  // M_kk (zeros above the diagonal)
        } else {
            gemm_fetch_b<false>(xo, G + gt(np, k, t), NB, tid);
            if (!neg) tile_load_acc(c2, G + gt(np, k1, t), NB);
        }
    }
    {
        const double* blk = G + gt(np, k1, k1);
#pragma unroll
        for (int m = 0; m < NB * NB / kGemmThreads; ++m) {
            const int idx = tid + kGemmThreads * m;
            L.g[idx >> 6][idx & 63] = blk[idx];
        }
    }
    double4v acc[2][2];
    zero_acc(acc);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (h) __syncthreads();
        gemm_stash_a(pd, s, tid, h);
        gemm_stash_b<true>(pd, s, tid, h);
        __syncthreads();
        gemm_compute_half<true>(s, acc);
    }
    // D = G_k1k1 - P_k1 P_k1^T in place (every element is this thread's own)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) L.g[acc_row(m, v)][acc_col(q)] -= acc[m][q][v];
    if (has_tile) {
        zero_acc(acc);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            __syncthreads();
            if (!inv_row) {
                gemm_stash_a(xo, s, tid, h);
                gemm_stash_b<true>(pd, s, tid, h);
            } else {
                gemm_stash_a(pd, s, tid, h);
                gemm_stash_b<false>(xo, s, tid, h);
            }
            __syncthreads();
            if (!inv_row) gemm_compute_half<true>(s, acc);
            else gemm_compute_half<false>(s, acc);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int v = 0; v < 4; ++v) c2[m][q][v] = neg ? -acc[m][q][v] : c2[m][q][v] - acc[m][q][v];
    }
    if (kPair) {
        // step k-1's part: D -= P'_k1 P'_k1^T and the operand's own term,
        //   t >= k1:    - P'_{t+1} P'_k1^T
        //   t == k-1:   - P'_k1 M_{k-1,k-1}
        //   t <  k-1:   - P'_k1 M_{k-1,t}
        // with P' and M_{k-1,k-1} from the panel buffer of step k-1 (Pkm)
        double pm[16], xm[16];
        gemm_fetch_a(pm, Pkm + (int64_t)k1 * NB * NB, NB, tid);
        const bool xterm = has_tile && t != k;
        if (xterm) {
            if (!inv_row) gemm_fetch_a(xm, Pkm + (int64_t)(t + 1) * NB * NB, NB, tid);
            else if (t == k - 1) gemm_fetch_b<false>(xm, Pkm, NB, tid);
            else gemm_fetch_b<false>(xm, G + gt(np, k - 1, t), NB, tid);
        }
        zero_acc(acc);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            __syncthreads();
            gemm_stash_a(pm, s, tid, h);
            gemm_stash_b<true>(pm, s, tid, h);
            __syncthreads();
            gemm_compute_half<true>(s, acc);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int v = 0; v < 4; ++v) L.g[acc_row(m, v)][acc_col(q)] -= acc[m][q][v];
        if (xterm) {
            zero_acc(acc);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                __syncthreads();
                if (!inv_row) {
                    gemm_stash_a(xm, s, tid, h);
                    gemm_stash_b<true>(pm, s, tid, h);
                } else {
                    gemm_stash_a(pm, s, tid, h);
                    gemm_stash_b<false>(xm, s, tid, h);
                }
                __syncthreads();
                if (!inv_row) gemm_compute_half<true>(s, acc);
                else gemm_compute_half<false>(s, acc);
            }
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int v = 0; v < 4; ++v) c2[m][q][v] -= acc[m][q][v];
        }
    }
    __syncthreads();
    const int st = diag64(L);
    if (st) {
        if (t == 0 && tid == 0) {
            *info = k1 * NB + st;
            *fail = 1;
        }
        return;
    }
    if (t == 0) {
#pragma unroll
        for (int m = 0; m < NB * NB / kGemmThreads; ++m) {
            const int idx = tid + kGemmThreads * m;
            const int r = idx >> 6, c = idx & 63;
            Pk1[idx] = (c <= r) ? L.g[r][c] : 0.0;
        }
    }
    if (!has_tile) return;
    double mv[NB * NB / kGemmThreads];
#pragma unroll
    for (int m = 0; m < NB * NB / kGemmThreads; ++m) {
        const int e = tid + kGemmThreads * m;
        const int kk = e >> 6, x = e & 63;
        mv[m] = (kk <= x) ? L.g[x][kk] : 0.0;
    }
    __syncthreads();
    zero_acc(acc);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (h) __syncthreads();
        if (inv_row) {
#pragma unroll
            for (int m = 8 * h; m < 8 * h + 8; ++m) {
                const int e = tid + kGemmThreads * m;
                s.A[(e & 63) * kRs + (e >> 6) - kHalf * h] = mv[m];
            }
            stash_acc_as_b(c2, s, h);
        } else {
            stash_acc_as_a(c2, s, h);
#pragma unroll
            for (int m = 8 * h; m < 8 * h + 8; ++m) {
                const int e = tid + kGemmThreads * m;
                s.B[(e & 63) * kRs + (e >> 6) - kHalf * h] = mv[m];
            }
        }
        __syncthreads();
        if (inv_row) gemm_compute_half<false>(s, acc);
        else gemm_compute_half<true>(s, acc);
    }
    if (inv_row) tile_store_f64<0>(G + gt(np, k1, t), NB, acc);
    else tile_store_f64<0>(Pk1 + (int64_t)(t + 1) * NB * NB, NB, acc);
}

// The rest of the update of step k: the blocks (i, j), j <= i, with
// i > k+1 and j != k+1 (column and row block k+1 are updated inside the
// diagonal-block workgroups of step k+1), enumerated by sched::rest_tile.

// Diagonal block and panel of step 0 (later steps run inside chol_step_kernel).
__global__ __launch_bounds__(kGemmThreads, 2) void chol_diag_panel_kernel(double* __restrict__ G, int64_t np,
                                                                       double* __restrict__ P, int T,
                                                                       int32_t* __restrict__ info,
                                                                       int* __restrict__ fail) {
    __shared__ __align__(16) DiagPanelLds u;
    if (*fail) return;
    diag_panel_body(u, G, np, P, 0, T, blockIdx.x, info, fail);
}

// Update of block (i, j) by step k.  M_kk is read from tile 0 of the panel
// buffer P.
__device__ __forceinline__ void trail_body(GemmLds& s, double* __restrict__ G, int64_t np, const double* __restrict__ P, int k,
                           int64_t i, int64_t j) {
    const double* Pi = P + i * NB * NB;
    double* Gij = G + gt(np, i, j);
    if (j < k) {
        tile_gemm_sub_f64<false>(Pi, NB, G + gt(np, k, j), NB, Gij, NB, s);
    } else if (j == k) {
        double4v acc[2][2];
        zero_acc(acc);
        tile_gemm_f64<false>(Pi, NB, P, NB, s, acc);
        tile_store_f64<2>(Gij, NB, acc);
    } else {
        tile_gemm_sub_f64<true>(Pi, NB, P + j * NB * NB, NB, Gij, NB, s);
    }
}

// Update of block (i, j) by steps k-1 and k together (the update of step
// k-1 was deferred): one 128-deep product per block.  P' and M_{k-1,k-1}
// come from the panel buffer of step k-1 (Pm), P and M_kk from that of
// step k (P); rows k-1 and k of the inverse (M_{k-1,j}, M_kj) are in place
// in G.
__device__ __forceinline__ void trail_body2(GemmLds& s, double* __restrict__ G, int64_t np,
                                            const double* __restrict__ P, const double* __restrict__ Pm, int k,
                                            int64_t i, int64_t j) {
    const double* Pi = P + i * NB * NB;
    const double* Pmi = Pm + i * NB * NB;
    double* Gij = G + gt(np, i, j);
    if (j < k - 1) {
        tile_gemm2_f64<false, true>(Pmi, G + gt(np, k - 1, j), Pi, G + gt(np, k, j), Gij, s);
    } else if (j == k - 1) {
        tile_gemm2_f64<false, false>(Pmi, Pm, Pi, G + gt(np, k, j), Gij, s);
    } else if (j == k) {
        double4v acc[2][2];
        zero_acc(acc);
        tile_gemm_f64<false>(Pi, NB, P, NB, s, acc);
        tile_store_f64<2>(Gij, NB, acc);
    } else {
        tile_gemm2_f64<true, true>(Pmi, Pm + j * NB * NB, Pi, P + j * NB * NB, Gij, s);
    }
}

// One launch per step k: the diagonal block and panel of step k1 = k+1
// together with the update of step k of the blocks they read (workgroups
// 0 .. npan-1, dispatched first), one workgroup that copies M_kk into G_kk
// (nothing reads G_kk after the launch that factored it), and the rest of
// the update of step k (the others).  The parts touch disjoint blocks (the
// rest excludes column and row block k1) and different panel buffers, so
// nothing but the launch order separates the steps.
template <bool kPair>
__global__ __launch_bounds__(kGemmThreads, 2) void chol_step_kernel(double* __restrict__ G, int64_t np,
                                                                 double* __restrict__ Pk1,
                                                                 const double* __restrict__ Pk,
                                                                 const double* __restrict__ Pkm, int k, int T,
                                                                 int npan, int32_t* __restrict__ info,
                                                                 int* __restrict__ fail) {
    __shared__ __align__(16) DiagPanelNextLds u;
    if (*fail) return;
    const int b = (int)blockIdx.x;
    if (b < npan) {
        diag_panel_next_body<kPair>(u, G, np, Pk1, Pk, Pkm, k, T, b, info, fail);
    } else if (b == npan) {
        double* Gkk = G + gt(np, k, k);
#pragma unroll
        for (int m = 0; m < NB * NB / kGemmThreads; ++m) {
            const int idx = threadIdx.x + kGemmThreads * m;
            Gkk[idx] = Pk[idx];
        }
    } else {
        int64_t i, j;
        sched::rest_tile(k, (int64_t)(b - npan - 1), i, j);
        if (kPair) trail_body2(u.gemm, G, np, Pk, Pkm, k, i, j);
        else trail_body(u.gemm, G, np, Pk, k, i, j);
    }
}

}  // namespace

size_t hinv_workspace_bytes(int64_t n) { return ws_bytes(n); }

size_t hinv_noalloc_scratch_bytes() { return sizeof(scratch); }

// Device address of `scratch` on the current device, looked up once per
// device (each device holds its own copy of the array at its own address).
hipError_t hinv_noalloc_scratch(void** out) {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}


// Schedule with one step of lookahead, on the caller's stream only: the
// diagonal block and panel of step 0, then per step k one launch that holds
// the diagonal block and panel of step k+1 (with the part of step k's update
// they read) and the rest of step k's update.  The panel buffer alternates
// between steps; its tile 0 holds M_kk.
hipError_t launch_prepare_hinv(const float* H, int64_t n, double damp_frac, float* U, uint8_t* dead,
                               int32_t* info, double* lambda_out, void* ws, hipStream_t s) {
    if (n == 0) return hipSuccess;
    HinvWs w = carve(ws, n);
    const int64_t np = round_up(n, NB);
    const int T = (int)(np / NB);
    const int64_t pstride = round_up(np * NB * 8, 256) / 8;
    double* Pbuf[3] = {w.P, w.P + pstride, w.P + 2 * pstride};  // step s: buffer s % 3
    hipError_t e = hipSuccess;
    {
        // lambda, the dead flags and the status words come with the reversed
        // load (its diagonal-tile workgroups)
        TimedLaunch t(K_HINV_LOAD, s);
        GPTQ_LAUNCH(t, load_reversed_kernel<double>, dim3((unsigned)((int64_t)T * (T + 1) / 2)), dim3(256), 0, s,
                           H, n, np, damp_frac, dead, lambda_out, info, w.fail, w.G);
    }
    const int npan = std::max(T - 1, 1);  // workgroups of the diagonal-block + panel launch of step 0
    {
        TimedLaunch t(K_CHOL_STEP, s);
        GPTQ_LAUNCH(t, chol_diag_panel_kernel, dim3((unsigned)npan), dim3(kGemmThreads), 0, s, w.G, np, Pbuf[0], T,
                           info, w.fail);
    }
    // wide layers pair the steps: an even step's update of the rest is
    // deferred and applied with the next step's as one 128-deep product
    // (GPTQ_SCHED_PAIR=1 pairs them at any width: a test override, never
    // needed for correctness)
    bool paired = sched::chol_paired(T);
    if (const char* e = getenv("GPTQ_SCHED_PAIR")) paired = paired || atoi(e) == 1;
    for (int k = 0; k < T; ++k) {
        const sched::CholLaunch g = sched::chol_launch(k, T, paired);
        const int np1 = g.nchain;
        const bool odd = (k & 1) != 0;
        const dim3 grid((unsigned)g.grid);
        double* pk1 = Pbuf[(k + 1) % 3];
        const double* pk = Pbuf[k % 3];
        const double* pkm = Pbuf[(k + 2) % 3];  // step k-1
        TimedLaunch t(K_CHOL_STEP, s);
        if (paired && odd)
            GPTQ_LAUNCH(t, chol_step_kernel<true>, grid, dim3(kGemmThreads), 0, s, w.G, np, pk1, pk, pkm, k, T,
                               np1, info, w.fail);
        else
            GPTQ_LAUNCH(t, chol_step_kernel<false>, grid, dim3(kGemmThreads), 0, s, w.G, np, pk1, pk, pkm, k, T,
                               np1, info, w.fail);
    }
    {
        TimedLaunch t(K_HINV_STORE, s);
        GPTQ_LAUNCH(t, store_u_kernel<double>, dim3((unsigned)n), dim3(256), 0, s, (const double*)w.G, np, n, U,
                           (const int*)w.fail);
    }
    return hipGetLastError();
}

}  // namespace gptq
