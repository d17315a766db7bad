// Propagation to the next layer of a chain quantized one layer at a time:
// Y = act(What X) (math4ai "GPTQ Hessian", opening paragraph: a network is
// quantized one linear layer at a time; aicassindra.com "tm_gptq_math",
// "Post-training quantization and the per-layer objective": a layer is fitted
// to its own input activations X).  The next layer's X is the already
// quantized layer's output; act is the identity or max(0, .).
//
// One workgroup per 128 x 128 tile of Y (rows of What x tokens), four waves
// in 2 x 2, each a 64 x 64 quarter as 2 x 2 MFMA 32x32x16 f16 accumulators
// (exact f16 products, fp32 accumulation), rounded once to f16 at the end.
// K runs in slabs of 32 through two LDS buffers, the next slab fetched into
// registers while the MFMAs consume the current one.  Both operands are
// staged k-contiguous (What rows as they are, X transposed on the way in:
// X is token-contiguous, so each thread gathers one token's 16 k values, a
// 64-byte run across 32 lanes per k), so that every MFMA operand is one
// 16-byte LDS read.
#include "common.hpp"
#include "kernels.hpp"

namespace gptq {

namespace {

constexpr int kPT = 128;          // tile edge
constexpr int kPK = 32;           // K per slab
constexpr int kPLd = kPK + 8;     // padded LDS row (halves): 16-byte reads of 16 rows hit distinct banks
constexpr int kPThreads = 256;

// Thread t stages row (or token) t/2 of a slab, k run (t % 2) * 16 .. +16.
// Every load is issued unconditionally at a clamped address (rows, tokens
// and k past the ends read a valid element) and replaced by zero after, so
// that a thread's loads are in flight together.
struct PropRegs {
    half8 a[2];
    half_t b[16];
};

template <bool kVecA>
__device__ __forceinline__ void prop_fetch(PropRegs& r, const half_t* __restrict__ W, int64_t M, int64_t K,
                                           const half_t* __restrict__ X, int64_t N, int64_t ldx, int64_t m0,
                                           int64_t n0, int64_t k0, int tid) {
    const int sr = tid >> 1, kh = (tid & 1) * 16;
    const int64_t k = k0 + kh;
    {
        const int64_t row = m0 + sr;
        const int64_t rc = min(row, M - 1);
        if (kVecA && k + 16 <= K) {
            r.a[0] = *reinterpret_cast<const half8*>(W + rc * K + k);
            r.a[1] = *reinterpret_cast<const half8*>(W + rc * K + k + 8);
            if (row >= M) r.a[0] = r.a[1] = (half8){};
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t kk = min(k + e, K - 1);
                const half_t v = W[rc * K + kk];
                r.a[e >> 3][e & 7] = (row < M && k + e < K) ? v : (half_t)0;
            }
        }
    }
    {
        const int64_t tok = n0 + sr;
        const int64_t tc = min(tok, N - 1);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t kk = min(k + e, K - 1);
            const half_t v = X[kk * ldx + tc];
            r.b[e] = (tok < N && k + e < K) ? v : (half_t)0;
        }
    }
}

__device__ __forceinline__ void prop_stash(const PropRegs& r, half_t* __restrict__ As, half_t* __restrict__ Bt,
                                           int tid) {
    const int sr = tid >> 1, kh = (tid & 1) * 16;
    *reinterpret_cast<half8*>(&As[sr * kPLd + kh]) = r.a[0];
    *reinterpret_cast<half8*>(&As[sr * kPLd + kh + 8]) = r.a[1];
    half8 b0, b1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        b0[e] = r.b[e];
        b1[e] = r.b[e + 8];
    }
    *reinterpret_cast<half8*>(&Bt[sr * kPLd + kh]) = b0;
    *reinterpret_cast<half8*>(&Bt[sr * kPLd + kh + 8]) = b1;
}

template <bool kVecA, bool kRelu>
__global__ __launch_bounds__(kPThreads, 2) void propagate_kernel(const half_t* __restrict__ W, int64_t M, int64_t K,
                                                               const half_t* __restrict__ X, int64_t N,
                                                               int64_t ldx, half_t* __restrict__ Y, int64_t ldy) {
    __shared__ half_t As[2][kPT * kPLd];
    __shared__ half_t Bt[2][kPT * kPLd];
    const int64_t n0 = (int64_t)blockIdx.x * kPT, m0 = (int64_t)blockIdx.y * kPT;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wi = w >> 1, wj = w & 1;

    float16v acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[m][q] = (float16v){};

    const int64_t nslab = (K + kPK - 1) / kPK;
    PropRegs r;
    if (nslab > 0) prop_fetch<kVecA>(r, W, M, K, X, N, ldx, m0, n0, 0, tid);  // K = 0 gives Y = act(0)
    for (int64_t sl = 0; sl < nslab; ++sl) {
        const int buf = (int)(sl & 1);
        // buffer buf was last read by slab sl-2, finished before the previous barrier
        prop_stash(r, As[buf], Bt[buf], tid);
        __syncthreads();
        if (sl + 1 < nslab) prop_fetch<kVecA>(r, W, M, K, X, N, ldx, m0, n0, (sl + 1) * kPK, tid);
        const half_t* Ap = As[buf];
        const half_t* Bp = Bt[buf];
#pragma unroll
        for (int ks = 0; ks < kPK; ks += 16) {
            half8 a[2], b[2];
#pragma unroll
            for (int m = 0; m < 2; ++m)
                a[m] = *reinterpret_cast<const half8*>(&Ap[(wi * 64 + 32 * m + (lane & 31)) * kPLd + ks + 8 * (lane >> 5)]);
#pragma unroll
            for (int q = 0; q < 2; ++q)
                b[q] = *reinterpret_cast<const half8*>(&Bp[(wj * 64 + 32 * q + (lane & 31)) * kPLd + ks + 8 * (lane >> 5)]);
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int q = 0; q < 2; ++q) acc[m][q] = mfma32x32x16_f16(a[m], b[q], acc[m][q]);
        }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + wi * 64 + 32 * m + acc32_row(v, lane);
                const int64_t col = n0 + wj * 64 + 32 * q + (lane & 31);
                float y = acc[m][q][v];
                if (kRelu) y = fmaxf(y, 0.0f);
                if (row < M && col < N) Y[row * ldy + col] = (half_t)y;
            }
}

}  // namespace

hipError_t launch_propagate(const void* W, int64_t d_out, int64_t d_in, const void* X, int64_t ntok, int64_t ldx,
                            void* Y, int64_t ldy, int relu, hipStream_t s) {
    if (d_out == 0 || ntok == 0) return hipSuccess;
    const dim3 grid((unsigned)((ntok + kPT - 1) / kPT), (unsigned)((d_out + kPT - 1) / kPT));
    const bool vec = (reinterpret_cast<uintptr_t>(W) % 16 == 0) && (d_in % 8 == 0);
    const half_t* w = static_cast<const half_t*>(W);
    const half_t* x = static_cast<const half_t*>(X);
    half_t* y = static_cast<half_t*>(Y);
    TimedLaunch t(K_PROPAGATE, s);
#define PROP_LAUNCH(V, R) \
    hipLaunchKernelGGL((propagate_kernel<V, R>), grid, dim3(kPThreads), 0, s, w, d_out, d_in, x, ntok, ldx, y, ldy)
    if (vec) {
        if (relu) PROP_LAUNCH(true, true);
        else PROP_LAUNCH(true, false);
    } else {
        if (relu) PROP_LAUNCH(false, true);
        else PROP_LAUNCH(false, false);
    }
#undef PROP_LAUNCH
    return hipGetLastError();
}

}  // namespace gptq
