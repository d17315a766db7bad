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
// K runs in slabs of 64 through two LDS buffers, the next slab fetched into
// registers while the MFMAs consume the current one.  Both operands are
// staged k-contiguous, so that every MFMA operand is one 16-byte LDS read:
// What rows as they are; X (token-contiguous) transposed on the way in, each
// thread loading four k rows of eight tokens with 16-byte loads and writing
// each token's four k values with one 8-byte LDS store.
//
// Every load is a buffer load issued unconditionally: a lane whose element
// lies outside the operand gets an offset past the end of the buffer, for
// which the hardware returns zero.  No load is under a condition, so the
// loads of a slab are in flight together.
#include "common.hpp"
#include "kernels.hpp"

namespace gptq {

namespace {

constexpr int kPT = 128;          // tile edge
constexpr int kPK = 64;           // K per slab
constexpr int kPLd = kPK + 8;     // LDS row (halves): 36 dwords, so 16-byte reads of 8 rows and
                                  // 8-byte transposing stores of 16 lanes hit distinct banks
constexpr int kPThreads = 256;
constexpr uint32_t kPOut = 0x80000000u;  // an offset past every buffer: the load returns zero

typedef _Float16 half4 __attribute__((ext_vector_type(4)));

// buffer descriptor of a raw (unstrided) byte range; word 3 as for every gfx9 part
__device__ __forceinline__ __amdgpu_buffer_rsrc_t prop_rsrc(const half_t* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<half_t*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ half8 prop_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ half_t prop_load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(half_t, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}

// What: thread t holds rows t/8 + 32 i (i < 4) of the tile, k run 8 (t % 8) .. +8
// of the slab.  rw covers the tile's valid rows, rows x K halves from its first.
template <bool kVec>
__device__ __forceinline__ void prop_fetch_w(half8 (&a)[4], __amdgpu_buffer_rsrc_t rw, int64_t rows, int64_t K,
                                             int64_t k0, int tid) {
    const int64_t k = k0 + 8 * (tid % 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t r = tid / 8 + 32 * i;
        if (kVec) {
            // K % 8 == 0: a run is wholly inside or wholly past the row
            const bool ok = r < rows && k < K;
            a[i] = prop_load8(rw, ok ? (uint32_t)((r * K + k) * 2) : kPOut);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool ok = r < rows && k + e < K;
                a[i][e] = prop_load1(rw, ok ? (uint32_t)((r * K + k + e) * 2) : kPOut);
            }
        }
    }
}

// X: thread t holds k rows 4 (t % 16) + i (i < 4) of the slab, tokens
// 8 (t / 16) .. +8 of the tile.  rx covers the slab from (k0, n0): krows rows
// of ldx halves, the last ncols long.
template <bool kVec>
__device__ __forceinline__ void prop_fetch_x(half8 (&b)[4], __amdgpu_buffer_rsrc_t rx, int64_t krows, int64_t ncols,
                                             int64_t ldx, int tid) {
    const int64_t t = 8 * (tid / 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t kr = 4 * (tid % 16) + i;
        if (kVec) {
            // ncols % 8 == 0: a run of eight tokens is wholly valid or wholly past the end
            const bool ok = kr < krows && t < ncols;
            b[i] = prop_load8(rx, ok ? (uint32_t)((kr * ldx + t) * 2) : kPOut);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool ok = kr < krows && t + e < ncols;
                b[i][e] = prop_load1(rx, ok ? (uint32_t)((kr * ldx + t + e) * 2) : kPOut);
            }
        }
    }
}

__device__ __forceinline__ void prop_stash(const half8 (&a)[4], const half8 (&b)[4], half_t* __restrict__ As,
                                           half_t* __restrict__ Bt, int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<half8*>(&As[(tid / 8 + 32 * i) * kPLd + 8 * (tid % 8)]) = a[i];
    // token 8 (t/16) + e takes k values 4 (t%16) .. +4
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const half4 v = {b[0][e], b[1][e], b[2][e], b[3][e]};
        *reinterpret_cast<half4*>(&Bt[(8 * (tid / 16) + e) * kPLd + 4 * (tid % 16)]) = v;
    }
}

// Tiles are numbered token-fastest; workgroups are dealt to the eight XCDs in
// turn, so workgroup id is given tile (id % 8) * (tiles / 8) + id / 8: each XCD
// works on a band of What rows against every token and keeps that band in
// its own L2.
template <bool kVecA, bool kVecB, bool kRelu>
__global__ __launch_bounds__(kPThreads, 2) void propagate_kernel(const half_t* __restrict__ W, int64_t M, int64_t K,
                                                               const half_t* __restrict__ X, int64_t N,
                                                               int64_t ldx, half_t* __restrict__ Y, int64_t ldy,
                                                               int64_t ntn) {
    __shared__ half_t As[2][kPT * kPLd];
    __shared__ half_t Bt[2][kPT * kPLd];
    const int64_t tiles = (int64_t)gridDim.x;
    int64_t id = blockIdx.x;
    if (tiles % 8 == 0) id = (id % 8) * (tiles / 8) + id / 8;
    const int64_t n0 = (id % ntn) * kPT, m0 = (id / ntn) * kPT;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wi = w >> 1, wj = w & 1;
    const int64_t rows = min(M - m0, (int64_t)kPT), ncols = min(N - n0, (int64_t)kPT);
    const __amdgpu_buffer_rsrc_t rw = prop_rsrc(W + m0 * K, (uint32_t)(rows * K * 2));

    float16v acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[m][q] = (float16v){};

    // Slab k0 into registers.  A slab past the end (k0 >= K) is fetched with
    // every offset out of range and a zero-length X descriptor: zeros, no
    // memory read, so that every iteration issues the same loads.
    auto fetch = [&](half8 (&a)[4], half8 (&b)[4], int64_t k0) {
        const int64_t krows = max((int64_t)0, min(K - k0, (int64_t)kPK));
        prop_fetch_w<kVecA>(a, rw, rows, K, k0, tid);
        const bool live = krows > 0;
        const __amdgpu_buffer_rsrc_t rx = prop_rsrc(X + (live ? k0 * ldx + n0 : 0),
                                                    live ? (uint32_t)(((krows - 1) * ldx + ncols) * 2) : 0u);
        prop_fetch_x<kVecB>(b, rx, krows, ncols, ldx, tid);
    };
    // MFMA operands of step ks of a slab: one 16-byte LDS read each
    auto operands = [&](half8 (&a)[2], half8 (&b)[2], int buf, int ks) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
            a[m] = *reinterpret_cast<const half8*>(&As[buf][(wi * 64 + 32 * m + (lane & 31)) * kPLd + ks + 8 * (lane >> 5)]);
#pragma unroll
        for (int q = 0; q < 2; ++q)
            b[q] = *reinterpret_cast<const half8*>(&Bt[buf][(wj * 64 + 32 * q + (lane & 31)) * kPLd + ks + 8 * (lane >> 5)]);
    };
    auto mfmas = [&](const half8 (&a)[2], const half8 (&b)[2]) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int q = 0; q < 2; ++q) acc[m][q] = mfma32x32x16_f16(a[m], b[q], acc[m][q]);
    };

    // One slab in flight in registers, two LDS buffers; within a slab the
    // operands of the next 16-deep step are read while the MFMAs of the
    // current one run.
    const int64_t nslab = (K + kPK - 1) / kPK;
    half8 ra[4], rb[4];
    if (nslab > 0) fetch(ra, rb, 0);  // K = 0 gives Y = act(0)
    for (int64_t sl = 0; sl < nslab; ++sl) {
        const int buf = (int)(sl & 1);
        // buffer buf was last read by slab sl-2, finished before the previous barrier
        prop_stash(ra, rb, As[buf], Bt[buf], tid);
        __syncthreads();
        fetch(ra, rb, (sl + 1) * kPK);  // past the end on the last slab: zeros, never stashed
        half8 a0[2], b0[2], a1[2], b1[2];
        operands(a0, b0, buf, 0);
#pragma unroll
        for (int ks = 0; ks < kPK; ks += 32) {
            operands(a1, b1, buf, ks + 16);
            mfmas(a0, b0);
            if (ks + 32 < kPK) operands(a0, b0, buf, ks + 32);
            mfmas(a1, b1);
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

// Offsets inside one tile's rows of What and one slab of X stay below 2^31
// bytes for d_in <= 2^22 and ldx <= 2^23, which the entry point enforces.
hipError_t launch_propagate(const void* W, int64_t d_out, int64_t d_in, const void* X, int64_t ntok, int64_t ldx,
                            void* Y, int64_t ldy, int relu, hipStream_t s) {
    if (d_out == 0 || ntok == 0) return hipSuccess;
    const int64_t ntn = (ntok + kPT - 1) / kPT, ntm = (d_out + kPT - 1) / kPT;
    const dim3 grid((unsigned)(ntn * ntm));
    const bool va = (reinterpret_cast<uintptr_t>(W) % 16 == 0) && (d_in % 8 == 0);
    const bool vb = (reinterpret_cast<uintptr_t>(X) % 16 == 0) && (ldx % 8 == 0) && (ntok % 8 == 0);
    const half_t* w = static_cast<const half_t*>(W);
    const half_t* x = static_cast<const half_t*>(X);
    half_t* y = static_cast<half_t*>(Y);
    TimedLaunch t(K_PROPAGATE, s);
#define PROP_LAUNCH(A, B, R) \
    GPTQ_LAUNCH(t, (propagate_kernel<A, B, R>), grid, dim3(kPThreads), 0, s, w, d_out, d_in, x, ntok, ldx, y, ldy, ntn)
#define PROP_RELU(A, B) \
    do {                \
        if (relu) PROP_LAUNCH(A, B, true); \
        else PROP_LAUNCH(A, B, false);     \
    } while (0)
    if (va && vb) PROP_RELU(true, true);
    else if (va) PROP_RELU(true, false);
    else if (vb) PROP_RELU(false, true);
    else PROP_RELU(false, false);
#undef PROP_RELU
#undef PROP_LAUNCH
    return hipGetLastError();
}

}  // namespace gptq
