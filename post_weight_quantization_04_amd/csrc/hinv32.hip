// Stages 2 and 3 with float32 tiles: the upper factor U of H^-1 by the same
// route as the float64 factorization (aicassindra.com "tm_gptq_math", "The
// Cholesky trick for the inverse Hessian"; math4ai "GPTQ Hessian",
// column-sweep paragraph, H^-1 = U^T U; mbrenndoerfer "GPTQ > Mathematical
// Details of the Update", Cholesky paragraph), with every product on MFMA
// f32 16x16x4 accumulating in float32 and the 16x16 pivot chains in
// float32.
//
// Route: with J the index reversal, J H J = L L^T gives U = J L^-1 J.  L^-1
// is formed together with L in one right-looking blocked sweep over
// G = J H J (in place, 64x64 tiles): step k factors and inverts the
// diagonal block, forms the panel P_i = G_ik L_kk^-T and the inverse row
// M_kj = L_kk^-1 G_kj, and updates every block below it,
//     G_ij -= P_i M_kj   (j <= k, the inverse being built)
//     G_ij -= P_i P_j^T  (k < j <= i, the trailing matrix).
// The launch schedule (which workgroup does what, steps paired on wide
// layers) is the float64 factorization's, from sched.hpp.
//
// Float32 rounding: every product of the sweep is a float32 MFMA sum, so
// the computed L L^T equals G up to a perturbation of order n * 2^-24 of
// |L| |L^T|, and U's relative error grows with the condition of the damped
// H.  The damping (at least 1% of the mean diagonal here) bounds that
// condition; float64 remains the path for inputs where it does not.
#include <math.h>
#include <stdlib.h>

#include "common.hpp"
#include "kernels.hpp"
#include "prep_common.hpp"
#include "sched.hpp"

namespace gptq {

namespace {

constexpr int NB = kCholNB;  // 64
constexpr int kThreads = 256;

struct Ws32 {
    float* G;      // n_pad x n_pad by 64x64 tiles (see gt)
    float* P;      // 3 x [n_pad / NB][NB][NB] (step s uses buffer s % 3)
    int* fail;     // device flag: set once a pivot fails
};

constexpr size_t ws32_bytes(int64_t n) {
    return (size_t)(round_up(round_up(n, NB) * round_up(n, NB) * 4, 256) + 3 * round_up(round_up(n, NB) * NB * 4, 256) +
                    256);
}

Ws32 carve32(void* ws, int64_t n) {
    const int64_t np = round_up(n, NB);
    char* p = static_cast<char*>(ws);
    Ws32 w;
    w.G = reinterpret_cast<float*>(p);
    p += round_up(np * np * 4, 256);
    w.P = reinterpret_cast<float*>(p);
    p += 3 * round_up(np * NB * 4, 256);
    w.fail = reinterpret_cast<int*>(p);
    return w;
}

// ---------------------------------------------------------------------------
// Diagonal block: M = L_kk^-1 where A = L_kk L_kk^T is the 64x64 block,
// blocked on 16x16 sub-blocks in LDS.  Sub-step s (columns 16s .. 16s+15):
//   1. one wave inverts the Cholesky factor of the sub-block A_ss by
//      symmetric Gauss-Jordan elimination in registers: Ls = L_ss^-1;
//   2. P_i = A_is Ls^T for sub-blocks i > s, and M_sj = Ls A_sj in place for
//      j < s (one 16x16x16 MFMA product per wave);
//   3. A_ij -= P_i P_j^T (s < j <= i), A_is = -P_i Ls, A_ij -= P_i M_sj
//      (j < s), for every i > s.
// Only lower-triangle entries are read; the block returned holds exact
// zeros above the diagonal.
// ---------------------------------------------------------------------------
constexpr int kSb = 16;       // sub-block width
constexpr int kDLd = NB + 1;  // padded LDS row (floats)

struct Diag32 {
    float g[NB][kDLd];         // the block: Schur complement, then the inverse
    float p[3][kSb][kSb + 1];  // P_i of the current sub-step
    int status;
};

// 1/x and 1/sqrt(x): the hardware estimate refined by one Newton step.
__device__ __forceinline__ float rcp32(float x) {
    const float y = __builtin_amdgcn_rcpf(x);
    const float e = fmaf(-x, y, 1.0f);
    return fmaf(e, y, y);
}
__device__ __forceinline__ float rsqrt32(float x) {
    const float y = __builtin_amdgcn_rsqf(x);
    const float e = fmaf(-(x * y), y, 1.0f);
    return fmaf(0.5f * e, y, y);
}

__device__ __forceinline__ int fbits(float x) { return __builtin_bit_cast(int, x); }
__device__ __forceinline__ float bitsf(int x) { return __builtin_bit_cast(float, x); }

// Lane-crossing moves within one wave (no LDS):
//   bcast_in_row<N>: lane N of each 16-lane row, to the whole row (DPP
//     row_newbcast);
//   bcast_row<R>: row R (lanes 16R .. 16R+15), to all four rows, lane
//     position kept (permlane16 then permlane32 swap).
template <int N>
__device__ __forceinline__ float bcast_in_row(float x) {
    return bitsf(__builtin_amdgcn_mov_dpp(fbits(x), 0x150 + N, 0xF, 0xF, false));
}
template <int R>
__device__ __forceinline__ float bcast_row(float x) {
    const uint32_t v = (uint32_t)fbits(x);
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // {rows 0,0,2,2}, {rows 1,1,3,3}
    const uint32_t y = (R & 1) ? a[1] : a[0];
    const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);  // {low half twice}, {high half twice}
    return bitsf((int)((R & 2) ? b[1] : b[0]));
}

// Pivot C of the symmetric elimination of a 16x16 block A = L D L^T, kept
// in one array per lane.  With y_j = A_Cj / p (p the pivot), every row r
// below C takes A_rj -= A_rC y_j; column C of row r then keeps A_rC, which
// is -p times the entry (r, C) of L_unit^-1 (row operations applied to the
// identity).  That scaling is the same in every row, so the later pivots
// update those entries in place like the rest.  The pivot row is cleared
// from column C on after it has been broadcast (y carries a zero at C,
// which leaves column C as it is), so that no later pivot touches a row
// above it.  Lane (g = lane/16, j = lane%16) holds rows 4g .. 4g+3 of
// column j; pj collects the pivot of column j.
// One pivot is a single wave's in-order instruction stream, so it is kept
// short: the pivot comes from the broadcast row by a DPP read (no
// round trip through a scalar register), the reciprocal is the hardware's
// (within 1 ulp; the sums of the blocked products round far more), and the
// row is scaled once so that each row update is one fused multiply-add
// whose broadcast operand the compiler reads through DPP.
template <int C>
__device__ __forceinline__ void gj_step(int g, int j, float (&x)[4], float& pj) {
    constexpr int R = C >> 2, S = C & 3;
    const float row = bcast_row<R>(x[S]);  // A[C][j] in every row group
    const float p = bcast_in_row<C>(row);  // A[C][C] in every lane
    const float ny = (j == C) ? 0.0f : -(row * __builtin_amdgcn_rcpf(p));
    if (g == R && j >= C) x[S] = 0.0f;
    if (j == C) pj = p;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = fmaf(bcast_in_row<C>(x[e]), ny, x[e]);  // A[4g+e][C] y_j, zero for rows <= C
}

// Sub-block s of L.g (one wave): Ls = inverse of its Cholesky factor,
// written in place (exact zeros above the diagonal).  After the pivots,
// entry (r, j < r) is -p_j (L_unit^-1)_rj and Ls = D^-1/2 L_unit^-1.
// Returns 0, or 1 + the local column of the first pivot that is not
// positive (wave-uniform; the pivots after it are then meaningless).
__device__ __forceinline__ int gj16(Diag32& L, int s, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int o = kSb * s;
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        x[e] = (r >= j) ? L.g[o + r][o + j] : L.g[o + j][o + r];  // symmetric from the lower triangle
    }
    float pj = 1.0f;
    gj_step<0>(g, j, x, pj);
    gj_step<1>(g, j, x, pj);
    gj_step<2>(g, j, x, pj);
    gj_step<3>(g, j, x, pj);
    gj_step<4>(g, j, x, pj);
    gj_step<5>(g, j, x, pj);
    gj_step<6>(g, j, x, pj);
    gj_step<7>(g, j, x, pj);
    gj_step<8>(g, j, x, pj);
    gj_step<9>(g, j, x, pj);
    gj_step<10>(g, j, x, pj);
    gj_step<11>(g, j, x, pj);
    gj_step<12>(g, j, x, pj);
    gj_step<13>(g, j, x, pj);
    gj_step<14>(g, j, x, pj);
    gj_step<15>(g, j, x, pj);
    // lanes 0..15 hold the pivots of columns 0..15
    const uint64_t bad = __ballot(!(pj > 0.0f)) & 0xFFFFull;
    const int first = bad ? __builtin_ctzll(bad) + 1 : 0;
    const float nrj = -rcp32(pj);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        // the pivot of row r sits in lane 16 g + r (column r of the same row group)
        const float pr = bitsf(__builtin_amdgcn_ds_bpermute(4 * (kSb * g + r), fbits(pj)));
        const float rs = rsqrt32(pr);
        L.g[o + r][o + j] = (r < j) ? 0.0f : (r == j) ? rs : rs * (x[e] * nrj);
    }
    return first;
}

// 16x16x16 product on MFMA 16x16x4 f32: acc = X Y with X[i][k] = fx(i, k),
// Y[k][j] = fy(k, j); lane l gets C[4 (l/16) + v][l%16] in acc[v].
template <typename FX, typename FY>
__device__ __forceinline__ float4v mm16(FX fx, FY fy, int lane) {
    float4v acc = {};
#pragma unroll
    for (int kk = 0; kk < kSb; kk += 4) {
        const int k = kk + (lane >> 4);
        acc = mfma16x16x4_f32(fx(lane & 15, k), fy(k, lane & 15), acc);
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

// Workgroup barrier that orders LDS accesses only (the diagonal block and
// the chain's product stages exchange data through LDS alone), so that
// global loads still in flight are not waited for, as __syncthreads would.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Factor and invert the block held in L.g (256 threads).  Returns 0 or
// 1 + the local column of the first pivot that is not positive
// (block-uniform).  One sub-step of lookahead: while wave 0 forms P_{s+1},
// updates the diagonal sub-block s+1 with it and runs that sub-block's
// pivots, waves 1..3 do every other panel and update tile of sub-step s.
//   phase 1  wave 0: P_{s+1} = A_{s+1,s} Ls^T;  waves 1..3: P_i (i > s+1)
//            and M_sj = Ls A_sj (j < s), in place;
//   phase 2  wave 0: A_{s+1,s+1} -= P_{s+1} P_{s+1}^T, pivots of s+1;
//            waves 1..3: the other tiles (i, j), i > s, j <= i.
// hook(0) runs on waves 1..3 while wave 0 pivots the first sub-block, hook(1)
// on the same waves right after that (before their first update work), and
// hook(2) on them after their update tiles of sub-step 2 (where wave 0's
// pivots of sub-block 3 leave them idle).
template <typename Hook>
__device__ __forceinline__ int diag64(Diag32& L, Hook&& hook) {
    const int lane = threadIdx.x & 63, w = wave_id();
    const int crow = 4 * (lane >> 4);  // first result row of this lane
    constexpr int S = NB / kSb;
    if (w == 0) {
        const int st = gj16(L, 0, lane);
        if (lane == 0) L.status = st;
    } else {
        hook(0);
    }
    lds_barrier();
    if (L.status) return L.status;
    if (w != 0) hook(1);
    for (int s = 0; s < S; ++s) {
        const int o = kSb * s;
        auto panel_p = [&](int i, int slot) {  // P_i = A_is Ls^T
            const float4v acc = mm16([&](int a, int k) { return L.g[kSb * i + a][o + k]; },
                                     [&](int k, int b) { return L.g[o + b][o + k]; }, lane);
#pragma unroll
            for (int v = 0; v < 4; ++v) L.p[slot][crow + v][lane & 15] = acc[v];
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
                    const float4v acc = mm16([&](int a, int k) { return L.g[o + a][o + k]; },
                                             [&](int k, int b) { return L.g[o + k][kSb * j + b]; }, lane);
#pragma unroll
                    for (int v = 0; v < 4; ++v) L.g[o + crow + v][kSb * j + (lane & 15)] = acc[v];
                }
            }
        }
        lds_barrier();
        // phase 2
        if (w == 0) {
            if (s + 1 < S) {
                const int o1 = o + kSb;
                const float4v acc = mm16([&](int a, int k) { return L.p[0][a][k]; },
                                         [&](int k, int b) { return L.p[0][b][k]; }, lane);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    float& d = L.g[o1 + crow + v][o1 + (lane & 15)];
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
                    float4v acc;
                    if (j > s) {
                        const int pjx = j - s - 1;
                        acc = mm16([&](int a, int k) { return L.p[pi][a][k]; },
                                   [&](int k, int b) { return L.p[pjx][b][k]; }, lane);
                    } else {
                        acc = mm16([&](int a, int k) { return L.p[pi][a][k]; },
                                   [&](int k, int b) { return L.g[o + k][kSb * j + b]; }, lane);
                    }
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        float& d = L.g[kSb * i + crow + v][kSb * j + (lane & 15)];
                        d = (j == s) ? -acc[v] : d - acc[v];
                    }
                }
            }
            if (s == 2) hook(2);
        }
        lds_barrier();
        if (s + 1 < S && L.status) return kSb * (s + 1) + L.status;
    }
    return 0;
}

__device__ __forceinline__ int diag64(Diag32& L) {
    return diag64(L, [](int) {});
}

// ---------------------------------------------------------------------------
// 64x64x64 float32 tile product on MFMA 16x16x4 f32: acc += A B, all of K
// staged in LDS at once.  A is row-major [64 rows][64 k]; B is row-major
// [64 k][64 cols] or, with kBT, its transpose given row-major [64 cols]
// [64 k].  Every operand tile is fetched in 16-byte pieces along its rows
// (thread t holds row 16e + t/16, columns 4(t%16) .. 4(t%16)+3, in
// registers 4e .. 4e+3, e = 0..3), each wave covering four whole 256-byte
// rows.  A and a transposed B are staged [x][k] with a row stride of 68
// floats, a direct B as [k][col] rows with a stride of 80, so that the 64
// lanes of one MFMA operand read (16 rows or columns at four consecutive k)
// fall on distinct banks.  The four waves (2x2 grid, 32x32 each as 2x2
// MFMA tiles) run 16 k-steps.
// ---------------------------------------------------------------------------
constexpr int kAs = NB + 4;   // [x][k] stage row stride (floats)
constexpr int kBd = NB + 16;  // direct [k][col] stage row stride (floats)

struct alignas(16) Gemm32 {
    float A[NB * kAs];
    float B[NB * kBd];  // B^T as [col][k] (stride kAs) or B as [k][col] (stride kBd)
};

// Diagonal block in LDS next to the product staging, so that the block can
// be loaded while a product still reads the stage.
struct Chain32Lds {
    Diag32 diag;
    Gemm32 gemm;
};

__device__ __forceinline__ void tile_fetch(float (&r)[16], const float* __restrict__ src, int tid) {
    const float* p = src + (tid >> 4) * NB + 4 * (tid & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float4v v = *reinterpret_cast<const float4v*>(p + 16 * e * NB);
#pragma unroll
        for (int c = 0; c < 4; ++c) r[4 * e + c] = v[c];
    }
}

// stage a fetched tile with row stride ld: rows [x][k] (A, B^T) use kAs,
// a direct B ([k][col]) kBd
template <int kLd>
__device__ __forceinline__ void stash(const float (&r)[16], float* __restrict__ S, int tid) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
        *reinterpret_cast<float4v*>(&S[(16 * e + (tid >> 4)) * kLd + 4 * (tid & 15)]) =
            (float4v){r[4 * e], r[4 * e + 1], r[4 * e + 2], r[4 * e + 3]};
}
__device__ __forceinline__ void stash_a(const float (&r)[16], Gemm32& s, int tid) { stash<kAs>(r, s.A, tid); }
template <bool kBT>
__device__ __forceinline__ void stash_b(const float (&r)[16], Gemm32& s, int tid) {
    if (kBT) stash<kAs>(r, s.B, tid);
    else stash<kBd>(r, s.B, tid);
}

template <bool kBT>
__device__ __forceinline__ void gemm_compute(const Gemm32& s, float4v (&acc)[2][2]) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wi = w >> 1, wj = w & 1;
#pragma unroll
    for (int ks = 0; ks < NB; ks += 4) {
        const int k = ks + (lane >> 4);
        float av[2], bv[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) av[m] = s.A[(wi * 32 + 16 * m + (lane & 15)) * kAs + k];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int col = wj * 32 + 16 * q + (lane & 15);
            bv[q] = kBT ? s.B[col * kAs + k] : s.B[k * kBd + col];
        }
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int q = 0; q < 2; ++q) acc[m][q] = mfma16x16x4_f32(av[m], bv[q], acc[m][q]);
    }
}

// C[row][col] of the accumulator element (m, q, v) of this thread
__device__ __forceinline__ int acc_row(int m, int v) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    return (w >> 1) * 32 + 16 * m + 4 * (lane >> 4) + v;
}
__device__ __forceinline__ int acc_col(int q) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    return (w & 1) * 32 + 16 * q + (lane & 15);
}

__device__ __forceinline__ void zero_acc(float4v (&acc)[2][2]) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[m][q] = (float4v){};
}

// A 64x64 tile (row stride NB) in accumulator layout.
__device__ __forceinline__ void tile_load_acc(float (&c)[2][2][4], const float* __restrict__ C) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) c[m][q][v] = C[acc_row(m, v) * NB + acc_col(q)];
}

// mode 0: C = acc ; mode 1: C = c - acc ; mode 2: C = -acc
template <int kMode>
__device__ __forceinline__ void tile_store(float* __restrict__ C, const float4v (&acc)[2][2],
                                           const float (&c)[2][2][4]) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float a = acc[m][q][v];
                C[acc_row(m, v) * NB + acc_col(q)] = (kMode == 0) ? a : (kMode == 1) ? c[m][q][v] - a : -a;
            }
}

// Stage an accumulator-layout tile X as the operand A = X ([row][k]) or as
// a direct B = X ([k][col]).
__device__ __forceinline__ void stash_acc_as_a(const float (&x)[2][2][4], Gemm32& s) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) s.A[acc_row(m, v) * kAs + acc_col(q)] = x[m][q][v];
}
__device__ __forceinline__ void stash_acc_as_b(const float (&x)[2][2][4], Gemm32& s) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) s.B[acc_row(m, v) * kBd + acc_col(q)] = x[m][q][v];
}

// Stage M = the inverted diagonal block in L.g (zeros above the diagonal)
// as A = M ([row][k], into s.A) or as B = M^T (given transposed, [col][k] =
// M[col][k], into s.B): both are M row-major with stride kAs.
__device__ __forceinline__ void stash_m(const Diag32& L, float* __restrict__ S) {
#pragma unroll
    for (int m = 0; m < NB * NB / kThreads; ++m) {
        const int e = threadIdx.x + kThreads * m;
        const int x = e >> 6, kk = e & 63;
        S[x * kAs + kk] = (kk <= x) ? L.g[x][kk] : 0.0f;
    }
}

// Load the diagonal block at blk into L.g.
__device__ __forceinline__ void load_block(Diag32& L, const float* __restrict__ blk) {
#pragma unroll
    for (int m = 0; m < NB * NB / kThreads; ++m) {
        const int idx = threadIdx.x + kThreads * m;
        L.g[idx >> 6][idx & 63] = blk[idx];
    }
}

// Write M (zeros above the diagonal) to a 64x64 tile.
__device__ __forceinline__ void store_m(const Diag32& L, float* __restrict__ dst) {
#pragma unroll
    for (int m = 0; m < NB * NB / kThreads; ++m) {
        const int idx = threadIdx.x + kThreads * m;
        const int r = idx >> 6, c = idx & 63;
        dst[idx] = (c <= r) ? L.g[r][c] : 0.0f;
    }
}

// Panel tile t of the step whose inverted diagonal block is in L.g, from
// the operand X (accumulator layout): t < kd: M_kd,t = M X (X = G_kd,t
// after its update), written in place; t >= kd: P_{t+1} = X M^T, into the
// panel buffer.  The LDS stage must be free.
__device__ __forceinline__ void panel_product(Chain32Lds& u, const float (&x)[2][2][4], bool inv_row,
                                              float* __restrict__ dst) {
    Gemm32& s = u.gemm;
    if (inv_row) {
        stash_m(u.diag, s.A);
        stash_acc_as_b(x, s);
    } else {
        stash_acc_as_a(x, s);
        stash_m(u.diag, s.B);
    }
    __syncthreads();
    float4v acc[2][2];
    zero_acc(acc);
    if (inv_row) gemm_compute<false>(s, acc);
    else gemm_compute<true>(s, acc);
    const float none[2][2][4] = {};
    tile_store<0>(dst, acc, none);
}

// ---------------------------------------------------------------------------
// Diagonal block and panel of step 0 (later steps run inside the step
// kernel).  Every workgroup factors and inverts the diagonal block itself
// (the work is latency-bound, so the copies cost no time) with its own
// panel operand already in flight, then forms its panel tile t:
// P_{t+1} = G_{t+1,0} M_00^T into the panel buffer.  Workgroup 0 also
// writes M_00 to tile 0 of the panel buffer.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads, 2) void chol32_diag_panel_kernel(float* __restrict__ G, int64_t np,
                                                                      float* __restrict__ P, int T,
                                                                      int32_t* __restrict__ info,
                                                                      int* __restrict__ fail) {
    __shared__ __align__(16) Chain32Lds u;
    if (*fail) return;
    const int t = (int)blockIdx.x, tid = threadIdx.x;
    const bool has_tile = t < T - 1;
    float x[2][2][4];
    if (has_tile) tile_load_acc(x, G + gt(np, t + 1, 0));
    load_block(u.diag, G + gt(np, 0, 0));
    __syncthreads();
    const int st = diag64(u.diag);
    if (st) {
        if (t == 0 && tid == 0) {
            *info = st;
            *fail = 1;
        }
        return;
    }
    if (t == 0) store_m(u.diag, P);
    if (!has_tile) return;
    panel_product(u, x, false, P + (int64_t)(t + 1) * NB * NB);
}

// ---------------------------------------------------------------------------
// Diagonal block and panel of step k1 = k+1, with the update of step k of
// the blocks they read applied in the same workgroup (in registers, none of
// it written back): every workgroup forms D = G_k1k1 - P_k1 P_k1^T (the
// diagonal block after step k) and its own operand after step k,
//   t >= k1:  G_{t+1,k1} - P_{t+1} P_k1^T   (column block k1),
//   t == k:   -P_k1 M_kk                    (row block k1, G_{k1,k} = -P_k1 M_kk),
//   t <  k:   G_{k1,t} - P_k1 M_kt          (row block k1, M_kt in place in G_kt),
// with P_i and M_kk from the panel buffer of step k (Pk).  D is factored and
// inverted and the panel tile formed from the updated operand: t < k1:
// M_k1t = M_k1k1 G_k1t (in place); t >= k1: P_{t+1} = G_{t+1,k1} M_k1k1^T
// into the panel buffer of step k1 (Pk1).  With kPair, step k-1's update of
// the same blocks is still owed too and is applied here as well (P' and
// M_{k-1,k-1} from the panel buffer of step k-1, Pkm).
// ---------------------------------------------------------------------------
template <bool kPair>
__device__ __forceinline__ void diag_panel_next_body(Chain32Lds& u, float* __restrict__ G, int64_t np,
                                                     float* __restrict__ Pk1, const float* __restrict__ Pk,
                                                     const float* __restrict__ Pkm, int k, int T, int t,
                                                     int32_t* __restrict__ info, int* __restrict__ fail) {
    const int tid = threadIdx.x;
    const int k1 = k + 1;
    const bool has_tile = t < T - 1;
    const bool inv_row = t < k1;
    Gemm32& s = u.gemm;
    Diag32& L = u.diag;
    // operands of both products in flight at once: P_k1 serves as A and as
    // B^T of the first product and as one operand of the second
    float pd[16];
    tile_fetch(pd, Pk + (int64_t)k1 * NB * NB, tid);
    float xo[16];
    float c2[2][2][4] = {};
    // G_{k1,k} (and with kPair G_{k1,k-1}) holds nothing yet: its value is
    // minus the product alone
    const bool neg = inv_row && (t == k || (kPair && t == k - 1));
    if (has_tile) {
        if (!inv_row) {
            tile_fetch(xo, Pk + (int64_t)(t + 1) * NB * NB, tid);
            tile_load_acc(c2, G + gt(np, t + 1, k1));
        } else if (t == k) {
            tile_fetch(xo, Pk, tid);  // M_kk (zeros above the diagonal)
        } else {
            tile_fetch(xo, G + gt(np, k, t), tid);
            if (!neg) tile_load_acc(c2, G + gt(np, k1, t));
        }
    }
    load_block(L, G + gt(np, k1, k1));
    float4v acc[2][2];
    zero_acc(acc);
    stash_a(pd, s, tid);
    stash_b<true>(pd, s, tid);
    __syncthreads();
    gemm_compute<true>(s, acc);
    // D = G_k1k1 - P_k1 P_k1^T in place (every element is this thread's own)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) L.g[acc_row(m, v)][acc_col(q)] -= acc[m][q][v];
    if (has_tile) {
        zero_acc(acc);
        __syncthreads();
        if (!inv_row) {
            stash_a(xo, s, tid);
            stash_b<true>(pd, s, tid);
        } else {
            stash_a(pd, s, tid);
            stash_b<false>(xo, s, tid);
        }
        __syncthreads();
        if (!inv_row) gemm_compute<true>(s, acc);
        else gemm_compute<false>(s, acc);
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
        float pm[16], xm[16];
        tile_fetch(pm, Pkm + (int64_t)k1 * NB * NB, tid);
        const bool xterm = has_tile && t != k;
        if (xterm) {
            if (!inv_row) tile_fetch(xm, Pkm + (int64_t)(t + 1) * NB * NB, tid);
            else if (t == k - 1) tile_fetch(xm, Pkm, tid);
            else tile_fetch(xm, G + gt(np, k - 1, t), tid);
        }
        zero_acc(acc);
        __syncthreads();
        stash_a(pm, s, tid);
        stash_b<true>(pm, s, tid);
        __syncthreads();
        gemm_compute<true>(s, acc);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int v = 0; v < 4; ++v) L.g[acc_row(m, v)][acc_col(q)] -= acc[m][q][v];
        if (xterm) {
            zero_acc(acc);
            __syncthreads();
            if (!inv_row) {
                stash_a(xm, s, tid);
                stash_b<true>(pm, s, tid);
            } else {
                stash_a(pm, s, tid);
                stash_b<false>(xm, s, tid);
            }
            __syncthreads();
            if (!inv_row) gemm_compute<true>(s, acc);
            else gemm_compute<false>(s, acc);
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
    if (t == 0) store_m(L, Pk1);
    if (!has_tile) return;
    panel_product(u, c2, inv_row, inv_row ? G + gt(np, k1, t) : Pk1 + (int64_t)(t + 1) * NB * NB);
}

// ---------------------------------------------------------------------------
// The same step without pairing, with the panel operand's update taken off
// the critical chain: its operands are staged right after the D product and
// waves 1..3 form it as 16x16 tiles in the diagonal block's idle time (four
// tiles while wave 0 pivots the first sub-block, the rest after their update
// tiles of sub-step 2); after the diagonal block they write it into the
// stage as the panel product's operand: A = X for t >= k1, a direct B = X
// for t < k1.  Wave w takes row band w-1 (four tiles) and on row band 3 the
// tiles (3,0), (3,1) (w = 1), (3,2) (w = 2) or (3,3) (w = 3).
// ---------------------------------------------------------------------------
constexpr int kOpMax = 6;  // op tiles of one wave

__device__ __forceinline__ bool op_tile_of(int w, int j, int& mt, int& nt) {
    if (j < 4) {
        mt = w - 1;
        nt = j;
        return true;
    }
    mt = 3;
    if (w == 1) {
        nt = j - 4;
        return j < 6;
    }
    nt = (w == 2) ? 2 : 3;
    return j == 4;
}

// 16x16 tile (mt, nt) of A B from the stage; lane l gets C[16 mt + 4 (l/16) + v][16 nt + l%16].
template <bool kBT>
__device__ __forceinline__ float4v op_tile(const Gemm32& s, int mt, int nt, int lane) {
    const int i = lane & 15, g = lane >> 4;
    float4v acc = {};
#pragma unroll
    for (int ks = 0; ks < NB; ks += 4) {
        const int k = ks + g;
        const float a = s.A[(16 * mt + i) * kAs + k];
        const float b = kBT ? s.B[(16 * nt + i) * kAs + k] : s.B[k * kBd + 16 * nt + i];
        acc = mfma16x16x4_f32(a, b, acc);
    }
    return acc;
}

// Panel tile from an operand already in the stage (A for t >= kd, direct B
// for t < kd) and M from L.g.
__device__ __forceinline__ void panel_product_staged(Chain32Lds& u, bool inv_row, float* __restrict__ dst) {
    Gemm32& s = u.gemm;
    if (inv_row) stash_m(u.diag, s.A);
    else stash_m(u.diag, s.B);
    lds_barrier();
    float4v acc[2][2];
    zero_acc(acc);
    if (inv_row) gemm_compute<false>(s, acc);
    else gemm_compute<true>(s, acc);
    const float none[2][2][4] = {};
    tile_store<0>(dst, acc, none);
}

__device__ __forceinline__ void diag_panel_next_overlap(Chain32Lds& u, float* __restrict__ G, int64_t np,
                                                        float* __restrict__ Pk1, const float* __restrict__ Pk, int k,
                                                        int T, int t, int32_t* __restrict__ info,
                                                        int* __restrict__ fail) {
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int k1 = k + 1;
    const bool has_tile = t < T - 1;
    const bool inv_row = t < k1;
    const bool neg = inv_row && t == k;  // G_{k1,k} holds nothing yet: X = -P_k1 M_kk
    Gemm32& s = u.gemm;
    Diag32& L = u.diag;
    float pd[16];
    tile_fetch(pd, Pk + (int64_t)k1 * NB * NB, tid);
    float xo[16];
    float cold[kOpMax][4];  // old values of the operand, op-tile layout (waves 1..3)
    if (has_tile) {
        if (!inv_row) tile_fetch(xo, Pk + (int64_t)(t + 1) * NB * NB, tid);
        else if (t == k) tile_fetch(xo, Pk, tid);  // M_kk (zeros above the diagonal)
        else tile_fetch(xo, G + gt(np, k, t), tid);
    }
    load_block(L, G + gt(np, k1, k1));
    // D = G_k1k1 - P_k1 P_k1^T
    float4v acc[2][2];
    zero_acc(acc);
    stash_a(pd, s, tid);
    stash_b<true>(pd, s, tid);
    __syncthreads();
    gemm_compute<true>(s, acc);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) L.g[acc_row(m, v)][acc_col(q)] -= acc[m][q][v];
    // the old values are needed only after the op tiles: loaded now, they
    // do not delay the D product's operands
    if (has_tile && w != 0 && !neg) {
        const float* ct = !inv_row ? G + gt(np, t + 1, k1) : G + gt(np, k1, t);
#pragma unroll
        for (int j = 0; j < kOpMax; ++j) {
            int mt, nt;
            if (op_tile_of(w, j, mt, nt)) {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    cold[j][v] = ct[(16 * mt + 4 * (lane >> 4) + v) * NB + 16 * nt + (lane & 15)];
            }
        }
    }
    if (has_tile) {
        lds_barrier();  // every wave is done with the D product's stage
        if (!inv_row) {
            stash_a(xo, s, tid);
            stash_b<true>(pd, s, tid);
        } else {
            stash_a(pd, s, tid);
            stash_b<false>(xo, s, tid);
        }
    }
    lds_barrier();
    float4v oacc[kOpMax];
    // stage 0: the four tiles of the wave's row band; stage 2: its tiles on
    // row band 3.  The tiles stay in registers until the diagonal block is
    // done (other waves read the operands until then).
    auto hook = [&](int stage) {
        if (!has_tile || stage == 1) return;
#pragma unroll
        for (int j = 0; j < kOpMax; ++j) {
            int mt, nt;
            if ((j < 4) != (stage == 0) || !op_tile_of(w, j, mt, nt)) continue;
            oacc[j] = inv_row ? op_tile<false>(s, mt, nt, lane) : op_tile<true>(s, mt, nt, lane);
        }
    };
    const int st = diag64(L, hook);
    if (st) {
        if (t == 0 && tid == 0) {
            *info = k1 * NB + st;
            *fail = 1;
        }
        return;
    }
    if (t == 0) store_m(L, Pk1);
    if (!has_tile) return;
    // X into the stage as the panel product's operand (every wave is past
    // the diagonal block's last barrier, so the op operands are dead)
    if (w != 0) {
#pragma unroll
        for (int j = 0; j < kOpMax; ++j) {
            int mt, nt;
            if (!op_tile_of(w, j, mt, nt)) continue;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = 16 * mt + 4 * (lane >> 4) + v, col = 16 * nt + (lane & 15);
                const float x = neg ? -oacc[j][v] : cold[j][v] - oacc[j][v];
                if (inv_row) s.B[row * kBd + col] = x;
                else s.A[row * kAs + col] = x;
            }
        }
    }
    panel_product_staged(u, inv_row, inv_row ? G + gt(np, k1, t) : Pk1 + (int64_t)(t + 1) * NB * NB);
}

// ---------------------------------------------------------------------------
// The rest of the update of step k: the blocks (i, j), j <= i, with
// i > k+1 and j != k+1 (column and row block k+1 are updated inside the
// diagonal-block workgroups of step k+1), enumerated by sched::rest_tile.
// ---------------------------------------------------------------------------
// C -= A B (kSub) with C's old values loaded behind the operands, or
// C = -A B.
template <bool kBT, bool kSub>
__device__ __forceinline__ void tile_update(const float* __restrict__ A, const float* __restrict__ B,
                                            float* __restrict__ C, Gemm32& s) {
    const int tid = threadIdx.x;
    float a[16], b[16];
    tile_fetch(a, A, tid);
    tile_fetch(b, B, tid);
    float c[2][2][4] = {};
    if (kSub) tile_load_acc(c, C);
    stash_a(a, s, tid);
    stash_b<kBT>(b, s, tid);
    __syncthreads();
    float4v acc[2][2];
    zero_acc(acc);
    gemm_compute<kBT>(s, acc);
    if (kSub) tile_store<1>(C, acc, c);
    else tile_store<2>(C, acc, c);
}

// C -= A1 B1 + A2 B2 (kSub) or C = -(A1 B1 + A2 B2): one 128-deep product
// with one read and one write of C.  The second pair's operands are fetched
// into the same registers once the first pair is staged, so their latency
// overlaps the first pair's products.
template <bool kBT, bool kSub>
__device__ __forceinline__ void tile_update2(const float* __restrict__ A1, const float* __restrict__ B1,
                                             const float* __restrict__ A2, const float* __restrict__ B2,
                                             float* __restrict__ C, Gemm32& s) {
    const int tid = threadIdx.x;
    float a[16], b[16];
    tile_fetch(a, A1, tid);
    tile_fetch(b, B1, tid);
    float c[2][2][4] = {};
    if (kSub) tile_load_acc(c, C);
    stash_a(a, s, tid);
    stash_b<kBT>(b, s, tid);
    __syncthreads();
    tile_fetch(a, A2, tid);
    tile_fetch(b, B2, tid);
    float4v acc[2][2];
    zero_acc(acc);
    gemm_compute<kBT>(s, acc);
    __syncthreads();
    stash_a(a, s, tid);
    stash_b<kBT>(b, s, tid);
    __syncthreads();
    gemm_compute<kBT>(s, acc);
    if (kSub) tile_store<1>(C, acc, c);
    else tile_store<2>(C, acc, c);
}

// Update of block (i, j) by step k.  M_kk is read from tile 0 of the panel
// buffer P; the inverse row M_kj (j < k) is in place in G_kj.
__device__ __forceinline__ void trail_body(Gemm32& s, float* __restrict__ G, int64_t np, const float* __restrict__ P,
                                           int k, int64_t i, int64_t j) {
    const float* Pi = P + i * NB * NB;
    float* Gij = G + gt(np, i, j);
    if (j < k) tile_update<false, true>(Pi, G + gt(np, k, j), Gij, s);
    else if (j == k) tile_update<false, false>(Pi, P, Gij, s);
    else tile_update<true, true>(Pi, P + j * NB * NB, Gij, s);
}

// Update of block (i, j) by steps k-1 and k together (the update of step
// k-1 was deferred): one 128-deep product per block.  P' and M_{k-1,k-1}
// come from the panel buffer of step k-1 (Pm), P and M_kk from that of
// step k (P); rows k-1 and k of the inverse are in place in G.
__device__ __forceinline__ void trail_body2(Gemm32& s, float* __restrict__ G, int64_t np, const float* __restrict__ P,
                                            const float* __restrict__ Pm, int k, int64_t i, int64_t j) {
    const float* Pi = P + i * NB * NB;
    const float* Pmi = Pm + i * NB * NB;
    float* Gij = G + gt(np, i, j);
    if (j < k - 1) tile_update2<false, true>(Pmi, G + gt(np, k - 1, j), Pi, G + gt(np, k, j), Gij, s);
    else if (j == k - 1) tile_update2<false, false>(Pmi, Pm, Pi, G + gt(np, k, j), Gij, s);
    else if (j == k) tile_update<false, false>(Pi, P, Gij, s);
    else tile_update2<true, true>(Pmi, Pm + j * NB * NB, Pi, P + j * NB * NB, Gij, s);
}

// One launch per step k: the diagonal block and panel of step k+1 together
// with the update of step k of the blocks they read (workgroups 0 .. npan-1,
// dispatched first), one workgroup that copies M_kk into G_kk, and the rest
// of the update of step k (the others).  The parts touch disjoint blocks
// and different panel buffers, so nothing but the launch order separates
// the steps.
template <bool kPair>
__global__ __launch_bounds__(kThreads, 2) void chol32_step_kernel(float* __restrict__ G, int64_t np,
                                                                float* __restrict__ Pk1, const float* __restrict__ Pk,
                                                                const float* __restrict__ Pkm, int k, int T, int npan,
                                                                int32_t* __restrict__ info, int* __restrict__ fail) {
    __shared__ __align__(16) Chain32Lds u;
    if (*fail) return;
    const int b = (int)blockIdx.x;
    if (b < npan) {
        if (kPair) diag_panel_next_body<true>(u, G, np, Pk1, Pk, Pkm, k, T, b, info, fail);
        else diag_panel_next_overlap(u, G, np, Pk1, Pk, k, T, b, info, fail);
    } else if (b == npan) {
        float* Gkk = G + gt(np, k, k);
#pragma unroll
        for (int m = 0; m < NB * NB / kThreads; ++m) {
            const int idx = threadIdx.x + kThreads * m;
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

size_t hinv32_workspace_bytes(int64_t n) { return ws32_bytes(n); }

// Same schedule as the float64 factorization: statistics, reversed load,
// the diagonal block and panel of step 0, one launch per step k (diagonal
// block and panel of step k+1 with the part of step k's update they read,
// plus the rest of step k's update), and the read-off of U.
hipError_t launch_prepare_hinv32(const float* H, int64_t n, double damp_frac, float* U, uint8_t* dead,
                                 int32_t* info, double* lambda_out, void* ws, hipStream_t s) {
    if (n == 0) return hipSuccess;
    Ws32 w = carve32(ws, n);
    const int64_t np = round_up(n, NB);
    const int T = (int)(np / NB);
    const int64_t pstride = round_up(np * NB * 4, 256) / 4;
    float* Pbuf[3] = {w.P, w.P + pstride, w.P + 2 * pstride};  // step s: buffer s % 3
    {
        // lambda, the dead flags and the status words come with the reversed
        // load (its diagonal-tile workgroups)
        TimedLaunch t(K_HINV32_LOAD, s);
        GPTQ_LAUNCH(t, load_reversed_kernel<float>, dim3((unsigned)((int64_t)T * (T + 1) / 2)), dim3(256), 0, s,
                           H, n, np, damp_frac, dead, lambda_out, info, w.fail, w.G);
    }
    const int npan = T - 1 > 1 ? T - 1 : 1;  // workgroups of the step-0 launch
    {
        TimedLaunch t(K_CHOL32_STEP, s);
        GPTQ_LAUNCH(t, chol32_diag_panel_kernel, dim3((unsigned)npan), dim3(kThreads), 0, s, w.G, np, Pbuf[0], T,
                           info, w.fail);
    }
    bool paired = sched::chol_paired(T);
    if (const char* e = getenv("GPTQ_SCHED_PAIR")) paired = paired || atoi(e) == 1;
    for (int k = 0; k < T; ++k) {
        const sched::CholLaunch g = sched::chol_launch(k, T, paired);
        const bool odd = (k & 1) != 0;
        const dim3 grid((unsigned)g.grid);
        float* pk1 = Pbuf[(k + 1) % 3];
        const float* pk = Pbuf[k % 3];
        const float* pkm = Pbuf[(k + 2) % 3];  // step k-1
        TimedLaunch t(K_CHOL32_STEP, s);
        if (paired && odd)
            GPTQ_LAUNCH(t, chol32_step_kernel<true>, grid, dim3(kThreads), 0, s, w.G, np, pk1, pk, pkm, k, T,
                               g.nchain, info, w.fail);
        else
            GPTQ_LAUNCH(t, chol32_step_kernel<false>, grid, dim3(kThreads), 0, s, w.G, np, pk1, pk, pkm, k, T,
                               g.nchain, info, w.fail);
    }
    {
        TimedLaunch t(K_HINV32_STORE, s);
        GPTQ_LAUNCH(t, store_u_kernel<float>, dim3((unsigned)n), dim3(256), 0, s, (const float*)w.G, np, n, U,
                           (const int*)w.fail);
    }
    return hipGetLastError();
}

}  // namespace gptq
