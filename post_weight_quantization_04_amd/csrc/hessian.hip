// Stage 1: H += 2 X X^T on the lower triangle (aicassindra.com
// "tm_gptq_math", "Why it is second-order: the Hessian").
//
// One workgroup per 128x128 lower-triangle tile (I >= J) of H; four waves,
// each owning a 64x64 quarter as 2x2 MFMA 32x32 accumulators.  Token slabs
// of X rows I and J are staged through LDS; products run on MFMA with fp32
// accumulation (f16 inputs: 32x32x16 f16, exact products; f32 inputs:
// 32x32x2 f32).  Each call adds its token range into H once at the end.
#include "common.hpp"
#include "kernels.hpp"

namespace gptq {

namespace {

constexpr int kTile = 128;
constexpr int kThreads = 256;

__device__ __forceinline__ void tile_of(int b, int& I, int& J) {
    int i = (int)((sqrtf(8.0f * (float)b + 1.0f) - 1.0f) * 0.5f);
    while ((i + 1) * (i + 2) / 2 <= b) ++i;
    while (i * (i + 1) / 2 > b) --i;
    I = i;
    J = b - i * (i + 1) / 2;
}

// Adds 2*acc into the lower triangle of H for one wave's 64x64 quarter.
__device__ __forceinline__ void store_quarter(float* __restrict__ H, int64_t n, int r0, int c0,
                                              const float16v (&acc)[2][2], int lane) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                int row = r0 + 32 * m + acc32_row(v, lane);
                int col = c0 + 32 * q + (lane & 31);
                if (row < n && col <= row) {
                    float* p = H + (int64_t)row * n + col;
                    *p = *p + 2.0f * acc[m][q][v];
                }
            }
}

// ---------------------------------------------------------------------------
// float16 inputs
// ---------------------------------------------------------------------------
constexpr int kK16 = 64;       // tokens per LDS stage
constexpr int kLd16 = kK16 + 8;  // padded LDS row (halves)

// Each thread moves 4 rows x 8 halves of a 128 x 64 slab: row (tid>>3) + 32 i,
// halves (tid&7)*8 .. +8.
template <bool kVec>
__device__ __forceinline__ void fetch_slab_f16(half8 (&v)[4], const half_t* __restrict__ X, int64_t n, int64_t ldx,
                                               int64_t ntok, int r0, int64_t k0, int tid) {
    const int kk = (tid & 7) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t row = r0 + (tid >> 3) + 32 * i;
        const int64_t k = k0 + kk;
        if (kVec && row < n && k + 8 <= ntok) {
            v[i] = *reinterpret_cast<const half8*>(X + row * ldx + k);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[i][e] = (row < n && k + e < ntok) ? X[row * ldx + k + e] : (half_t)0;
        }
    }
}

__device__ __forceinline__ void stash_slab_f16(const half8 (&v)[4], half_t (*S)[kLd16], int tid) {
    const int kk = (tid & 7) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<half8*>(&S[(tid >> 3) + 32 * i][kk]) = v[i];
}

// Token slab k+1 is fetched into registers while the MFMAs consume slab k
// from one of two LDS buffers (one barrier per slab).
template <bool kVec>
__global__ __launch_bounds__(kThreads) void hessian_f16_kernel(float* __restrict__ H, int64_t n,
                                                              const half_t* __restrict__ X, int64_t ldx,
                                                              int64_t ntok) {
    __shared__ half_t As[2][kTile][kLd16];
    __shared__ half_t Bs[2][kTile][kLd16];
    int I, J;
    tile_of(blockIdx.x, I, J);
    const bool diag = (I == J);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wi = w >> 1, wj = w & 1;
    const bool active = !(diag && wi < wj);  // upper quarter of a diagonal tile

    float16v acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[m][q] = (float16v){};

    half8 ra[4], rb[4];
    fetch_slab_f16<kVec>(ra, X, n, ldx, ntok, I * kTile, 0, tid);
    if (!diag) fetch_slab_f16<kVec>(rb, X, n, ldx, ntok, J * kTile, 0, tid);
    const int64_t nslab = (ntok + kK16 - 1) / kK16;
    for (int64_t sl = 0; sl < nslab; ++sl) {
        const int buf = (int)(sl & 1);
        stash_slab_f16(ra, As[buf], tid);
        if (!diag) stash_slab_f16(rb, Bs[buf], tid);
        __syncthreads();
        if (sl + 1 < nslab) {
            fetch_slab_f16<kVec>(ra, X, n, ldx, ntok, I * kTile, (sl + 1) * kK16, tid);
            if (!diag) fetch_slab_f16<kVec>(rb, X, n, ldx, ntok, J * kTile, (sl + 1) * kK16, tid);
        }
        half_t(*Ap)[kLd16] = As[buf];
        half_t(*Bp)[kLd16] = diag ? As[buf] : Bs[buf];
        if (active) {
#pragma unroll
            for (int ks = 0; ks < kK16; ks += 16) {
                half8 a[2], b[2];
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    a[m] = *reinterpret_cast<const half8*>(&Ap[wi * 64 + 32 * m + (lane & 31)][ks + 8 * (lane >> 5)]);
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    b[q] = *reinterpret_cast<const half8*>(&Bp[wj * 64 + 32 * q + (lane & 31)][ks + 8 * (lane >> 5)]);
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int q = 0; q < 2; ++q) acc[m][q] = mfma32x32x16_f16(a[m], b[q], acc[m][q]);
            }
        }
    }
    if (active) store_quarter(H, n, I * kTile + wi * 64, J * kTile + wj * 64, acc, lane);
}

// ---------------------------------------------------------------------------
// float32 inputs
// ---------------------------------------------------------------------------
constexpr int kK32 = 32;
constexpr int kLd32 = kK32 + 4;

template <bool kVec>
__device__ __forceinline__ void load_slab_f32(float (*S)[kLd32], const float* __restrict__ X, int64_t n,
                                              int64_t ldx, int64_t ntok, int r0, int64_t k0, int tid) {
    const int kk = (tid & 7) * 4;
#pragma unroll
    for (int rr = 0; rr < kTile; rr += kThreads / 8) {
        int r = rr + (tid >> 3);
        int64_t row = r0 + r;
        int64_t k = k0 + kk;
        float4v v;
        if (kVec && row < n && k + 4 <= ntok) {
            v = *reinterpret_cast<const float4v*>(X + row * ldx + k);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (row < n && k + e < ntok) ? X[row * ldx + k + e] : 0.0f;
        }
        *reinterpret_cast<float4v*>(&S[r][kk]) = v;
    }
}

template <bool kVec>
__global__ __launch_bounds__(kThreads) void hessian_f32_kernel(float* __restrict__ H, int64_t n,
                                                              const float* __restrict__ X, int64_t ldx,
                                                              int64_t ntok) {
    __shared__ float As[kTile][kLd32];
    __shared__ float Bs[kTile][kLd32];
    int I, J;
    tile_of(blockIdx.x, I, J);
    const bool diag = (I == J);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wi = w >> 1, wj = w & 1;
    const bool active = !(diag && wi < wj);
    float(*Bp)[kLd32] = diag ? As : Bs;

    float16v acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[m][q] = (float16v){};

    for (int64_t k0 = 0; k0 < ntok; k0 += kK32) {
        load_slab_f32<kVec>(As, X, n, ldx, ntok, I * kTile, k0, tid);
        if (!diag) load_slab_f32<kVec>(Bs, X, n, ldx, ntok, J * kTile, k0, tid);
        __syncthreads();
        if (active) {
#pragma unroll
            for (int ks = 0; ks < kK32; ks += 2) {
                float a[2], b[2];
#pragma unroll
                for (int m = 0; m < 2; ++m) a[m] = As[wi * 64 + 32 * m + (lane & 31)][ks + (lane >> 5)];
#pragma unroll
                for (int q = 0; q < 2; ++q) b[q] = Bp[wj * 64 + 32 * q + (lane & 31)][ks + (lane >> 5)];
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int q = 0; q < 2; ++q) acc[m][q] = mfma32x32x2_f32(a[m], b[q], acc[m][q]);
            }
        }
        __syncthreads();
    }
    if (active) store_quarter(H, n, I * kTile + wi * 64, J * kTile + wj * 64, acc, lane);
}

}  // namespace

hipError_t launch_hessian(float* H, int64_t n, const void* X, int x_is_f16, int64_t ntok, int64_t ldx,
                          hipStream_t s) {
    const int64_t T = (n + kTile - 1) / kTile;
    const int64_t tiles = T * (T + 1) / 2;
    if (tiles == 0 || ntok == 0) return hipSuccess;
    const uintptr_t addr = reinterpret_cast<uintptr_t>(X);
    if (x_is_f16) {
        TimedLaunch t(K_HESS_F16, s);
        const bool vec = (addr % 16 == 0) && (ldx % 8 == 0);
        if (vec)
            hipLaunchKernelGGL(hessian_f16_kernel<true>, dim3((unsigned)tiles), dim3(kThreads), 0, s, H, n,
                               static_cast<const half_t*>(X), ldx, ntok);
        else
            hipLaunchKernelGGL(hessian_f16_kernel<false>, dim3((unsigned)tiles), dim3(kThreads), 0, s, H, n,
                               static_cast<const half_t*>(X), ldx, ntok);
    } else {
        TimedLaunch t(K_HESS_F32, s);
        const bool vec = (addr % 16 == 0) && (ldx % 4 == 0);
        if (vec)
            hipLaunchKernelGGL(hessian_f32_kernel<true>, dim3((unsigned)tiles), dim3(kThreads), 0, s, H, n,
                               static_cast<const float*>(X), ldx, ntok);
        else
            hipLaunchKernelGGL(hessian_f32_kernel<false>, dim3((unsigned)tiles), dim3(kThreads), 0, s, H, n,
                               static_cast<const float*>(X), ldx, ntok);
    }
    return hipGetLastError();
}

}  // namespace gptq
