// Greedy-order quantization of small layers (OBQ), the variant that the
// fixed column order replaces (aicassindra.com "tm_gptq_math", "Greedy
// quantization with error compensation" and "GPTQ's speedups: fixed order
// and lazy batches"; the downdate of the inverse by the Schur complement
// from mbrenndoerfer.com "GPTQ", "Mathematical Details of the Update").
//
// Per row, with Hf^-1 the inverse Hessian restricted to the free weights
// (initially the inverse of the damped H): round every free weight to the
// row's grid, pick the one with the smallest e_q^2 / [Hf^-1]_qq (the lowest
// index among equal scores), move the free weights by
// -(e_q / [Hf^-1]_qq) Hf^-1[:, q] and fix w_q at its grid value, then remove
// q from the inverse: Hf^-1 -= Hf^-1[:, q] Hf^-1[q, :] / [Hf^-1]_qq.
//
// Every row has its own order and its own copy of the inverse, so nothing is
// shared between rows: one workgroup per row, the d_in x d_in inverse
// (d_in <= 128) held in registers, 8 x 8 fp64 values per thread; the cost is
// d_in^3 fp64 multiply-adds per row (the pages' reason to drop the greedy
// order on large layers).
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace gptq {

namespace {

constexpr int kObqMax = 128;  // largest d_in: 16 x 16 threads, 8 x 8 values each

// H^-1 = U^T U in fp64 (U fp32 upper triangular): entry (i, j) sums
// U[k][i] U[k][j] over k <= min(i, j); the products are exact in fp64.
__global__ __launch_bounds__(256) void obq_hinv_kernel(const float* __restrict__ U, int n, double* __restrict__ Hinv) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)n * n) return;
    const int i = (int)(idx / n), j = (int)(idx % n);
    const int m = min(i, j);
    double acc = 0.0;
    for (int k = 0; k <= m; ++k) acc += (double)U[(int64_t)k * n + i] * (double)U[(int64_t)k * n + j];
    Hinv[idx] = acc;
}

// (score, index) minimum with the lower index winning a tie
__device__ __forceinline__ void argmin_pair(double& s, int& i, double s2, int i2) {
    if (s2 < s || (s2 == s && i2 < i)) {
        s = s2;
        i = i2;
    }
}

struct ObqLds {
    double diag[kObqMax];   // [Hf^-1]_ii of the current step
    double col[kObqMax];    // Hf^-1[:, q] of the current step
    double wmin[2];         // per-wave minimum score
    int wimin[2];
    double e, wq;           // the pick's error and grid value
    float red[8];           // grid reductions
};

template <typename T>
__global__ __launch_bounds__(256) void obq_row_kernel(const T* __restrict__ W, int d_in, const double* __restrict__ Hinv,
                                                      const uint8_t* __restrict__ dead, int bits,
                                                      uint8_t* __restrict__ codes, float* __restrict__ scales,
                                                      int32_t* __restrict__ zeros, int32_t* __restrict__ order,
                                                      double* __restrict__ loss) {
    __shared__ ObqLds L;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int ty = tid >> 4, tx = tid & 15;
    const int64_t r = blockIdx.x;
    const float maxq = (float)((1 << bits) - 1);

    // this thread's 8 x 8 block of the inverse: rows 8ty.., columns 8tx..
    double h[8][8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int i = 8 * ty + a, j = 8 * tx + b;
            h[a][b] = (i < d_in && j < d_in) ? Hinv[(int64_t)i * d_in + j] : 0.0;
        }

    // the row's weight (threads 0 .. d_in-1 own one each) and its grid from
    // the input row: [min(0, min w), max(0, max w)], an all-zero range
    // becoming [-1, 1]; s = fl32(fl32(mx - mn) / maxq), z = clamp(rint(fl32(-mn / s)))
    const bool own = tid < d_in;
    float w32 = own ? (float)W[r * d_in + tid] : 0.0f;
    float mn = own ? w32 : 0.0f, mx = own ? w32 : 0.0f;
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
        L.red[wv] = mn;
        L.red[4 + wv] = mx;
    }
    __syncthreads();
    mn = fminf(fminf(L.red[0], L.red[1]), fminf(L.red[2], L.red[3]));
    mx = fmaxf(fmaxf(L.red[4], L.red[5]), fmaxf(L.red[6], L.red[7]));
    mn = fminf(mn, 0.0f);
    mx = fmaxf(mx, 0.0f);
    if (mn == 0.0f && mx == 0.0f) {
        mn = -1.0f;
        mx = 1.0f;
    }
    const float s = __fdiv_rn(mx - mn, maxq);
    const float z = fminf(fmaxf(rintf(__fdiv_rn(-mn, s)), 0.0f), maxq);
    if (tid == 0) {
        scales[r] = s;
        zeros[r] = (int32_t)z;
    }
    // dead columns are zeroed after the grid
    double w = (own && !(dead && dead[tid])) ? (double)w32 : 0.0;
    bool free_ = own;
    double lsum = 0.0;

    for (int t = 0; t < d_in; ++t) {
        // 1. the current diagonal of the inverse
        if (tx == ty) {
#pragma unroll
            for (int a = 0; a < 8; ++a) L.diag[8 * ty + a] = h[a][a];
        }
        __syncthreads();
        // 2. every free weight rounded to the grid (decision in fp32), its
        //    score e^2 / [Hf^-1]_ii, and the minimum over the row
        float code = 0.0f;
        double e = 0.0, wq = 0.0, score = INFINITY;
        if (free_) {
            const float v = __fadd_rn(__fdiv_rn((float)w, s), z);
            code = fminf(fmaxf(rintf(v), 0.0f), maxq);
            wq = (double)s * ((double)code - (double)z);
            e = w - wq;
            score = e * e / L.diag[tid];
            if (!(score <= INFINITY)) score = INFINITY;  // a NaN score ranks last (ties at +inf go to the lowest index)
        }
        double bs = score;
        int bi = free_ ? tid : 0x7fffffff;
        if (wv < 2) {
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const double s2 = __shfl_xor(bs, o, kWave);
                const int i2 = __shfl_xor(bi, o, kWave);
                argmin_pair(bs, bi, s2, i2);
            }
            if (lane == 0) {
                L.wmin[wv] = bs;
                L.wimin[wv] = bi;
            }
        }
        __syncthreads();
        double ms = L.wmin[0];
        int q = L.wimin[0];
        argmin_pair(ms, q, L.wmin[1], L.wimin[1]);
        // a free weight always exists (one is fixed per step), and free
        // weights hold finite or +inf scores with valid indices; the clamp
        // only keeps every index below in range
        q = min(q, d_in - 1);
        // 3. column q of the inverse, and the pick's error and grid value
        if (tx == (q >> 3)) {
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                double c = h[a][0];
#pragma unroll
                for (int b = 1; b < 8; ++b)
                    if ((q & 7) == b) c = h[a][b];
                L.col[8 * ty + a] = c;
            }
        }
        if (tid == q) {
            L.e = e;
            L.wq = wq;
            codes[r * d_in + q] = (uint8_t)code;
            if (order) order[r * d_in + t] = q;
        }
        __syncthreads();
        // 4. compensation of the free weights, the pick fixed, and the
        //    Schur downdate of the inverse
        const double d = L.col[q];
        const double eq = L.e;
        const double f = eq / d;
        lsum += eq * f;
        if (tid == q) {
            w = L.wq;
            free_ = false;
        } else if (free_) {
            w -= f * L.col[tid];
        }
        const double rd = 1.0 / d;
        double cr[8], cc[8];
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            cr[a] = L.col[8 * ty + a];
            cc[a] = L.col[8 * tx + a] * rd;
        }
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int b = 0; b < 8; ++b) h[a][b] = fma(-cr[a], cc[b], h[a][b]);
    }
    if (tid == 0 && loss) loss[r] = lsum;
}

}  // namespace

size_t obq_workspace_bytes(int64_t d_in) { return (size_t)(d_in * d_in * 8); }

hipError_t launch_obq(const void* W, int w_is_f16, int64_t d_out, int64_t d_in, const float* U, const uint8_t* dead,
                      int bits, uint8_t* codes, float* scales, int32_t* zeros, int32_t* order, double* loss,
                      void* ws, hipStream_t s) {
    double* Hinv = static_cast<double*>(ws);
    {
        TimedLaunch t(K_OBQ_HINV, s);
        const int64_t n2 = d_in * d_in;
        GPTQ_LAUNCH(t, obq_hinv_kernel, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, s, U, (int)d_in, Hinv);
    }
    TimedLaunch t(K_OBQ_ROWS, s);
    if (w_is_f16)
        GPTQ_LAUNCH(t, obq_row_kernel<half_t>, dim3((unsigned)d_out), dim3(256), 0, s,
                           static_cast<const half_t*>(W), (int)d_in, (const double*)Hinv, dead, bits, codes, scales,
                           zeros, order, loss);
    else
        GPTQ_LAUNCH(t, obq_row_kernel<float>, dim3((unsigned)d_out), dim3(256), 0, s,
                           static_cast<const float*>(W), (int)d_in, (const double*)Hinv, dead, bits, codes, scales,
                           zeros, order, loss);
    return hipGetLastError();
}

}  // namespace gptq
