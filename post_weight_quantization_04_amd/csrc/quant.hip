// Stage 4: the fixed-order, block-lazy quantize-and-compensate sweep
// (aicassindra.com "tm_gptq_math", "Greedy quantization with error
// compensation" and "GPTQ's speedups: fixed order and lazy batches"; math4ai
// "GPTQ Hessian", column-sweep paragraph).
//
// One launch of step_kernel per lazy block [b0, b1), on the caller's stream:
//   sweep part     workgroups 0 .. ceil(d_out/64)-1, 64 rows each (lane =
//                  row), 512 threads; wave q owns the 16 block columns
//                  b0+16q.. in registers.  The previous block's scaled errors
//                  first reach these columns in registers (MFMA 16x16x4 f32
//                  against that block's rows of U), then in phase p wave p
//                  rounds its columns one by one and compensates the rest of
//                  its 16 at once; its scaled errors go to LDS and the waves
//                  owning later columns fold them in on MFMA 16x16x4 f32 (the
//                  same OBS updates, grouped by sub-block).  The block's rows
//                  of U are staged in LDS as packed 16x16 upper sub-blocks.
//   far part       the previous block's update of every column from b1 on,
//                  W[:, b1:] -= E_prev U[prev block, b1:], cut into 128-row x
//                  64-column units dealt to every CU as contiguous ranges
//                  (sched::far_split); the sweeping workgroups take a smaller
//                  share after their sweep.  Products on MFMA 32x32x2 f32
//                  with fp32 accumulation, or (split path) as six products
//                  of bf16 pieces on MFMA 32x32x16 bf16.
// On the split path the near update also runs on bf16 pieces, and the first
// block's launch, which has no far part, forms the bf16 pieces of U for all
// later launches on its non-sweeping workgroups.
// trail_kernel runs only at the start of a group wider than the block: the
// previous block's update of every column from the group on, so that the
// group's grid sees the updated weights.
#include <math.h>

#include <algorithm>

#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "sched.hpp"

namespace gptq {

namespace {

constexpr int kSub = 16;      // columns per wave in the sweep
constexpr int kRowsPerWg = 64;
constexpr int kMaxBlock = 128;
constexpr int kEld = 65;      // padded LDS row of the scaled-error exchange

__host__ __device__ inline int64_t rup(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

struct QuantWs {
    float* Wk;     // [d_out, d_in] working weights
    float* E[2];   // scaled errors of a block at eoff, alternating between blocks
    float* rdiag;  // [d_in] 1 / U_jj
    __bf16* U3;    // split path: bf16 pieces of U by lazy block, [nb][3][ldk/16][d_in][16]
};

// k extent of one block's U pieces (whole 16-deep chunks)
__host__ __device__ inline int64_t split_ldk(int64_t block) { return (block + 15) / 16 * 16; }
// Offset of the scaled error of row r, block column k: runs of 16 columns,
// each holding every row's 16 values together, so that a sub-block's errors
// are written, and a K chunk's are read, as consecutive memory.
__host__ __device__ inline int64_t eoff(int64_t d_out, int64_t r, int k) {
    return ((int64_t)(k >> 4) * d_out + r) * 16 + (k & 15);
}
// Offset of piece p of U[k][c] inside one block's pieces: runs of 16 k, each
// holding every column's 16 values together, so that the 16-byte operand
// reads of one k run over consecutive columns are consecutive in memory.
__host__ __device__ inline int64_t u3_offset(int64_t d_in, int64_t ldk, int p, int64_t k, int64_t c) {
    return ((p * (ldk / 16) + k / 16) * d_in + c) * 16 + (k & 15);
}
__host__ __device__ inline int64_t split_u_elems(int64_t d_in, int64_t block) {
    return ((d_in + block - 1) / block) * 3 * d_in * split_ldk(block);
}

QuantWs carve(void* ws, int64_t d_out, int64_t d_in, int64_t block) {
    char* p = static_cast<char*>(ws);
    QuantWs w;
    w.Wk = reinterpret_cast<float*>(p);
    p += rup(d_out * d_in * 4, 256);
    for (int i = 0; i < 2; ++i) {
        w.E[i] = reinterpret_cast<float*>(p);
        p += rup(d_out * split_ldk(block) * 4, 256);
    }
    w.rdiag = reinterpret_cast<float*>(p);
    p += rup(d_in * 4, 256);
    w.U3 = reinterpret_cast<__bf16*>(p);
    return w;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __bf16 bf16_rne(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return __builtin_bit_cast(__bf16, (uint16_t)(u >> 16));
}
__device__ __forceinline__ float bf16_f(__bf16 h) {
    return __builtin_bit_cast(float, (uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}
// x = p0 + p1 + p2 to within 2^-27 |x|: p0 the nearest bf16 to x, p1 that of
// x - p0, p2 that of x - p0 - p1 (both differences exact in fp32)
__device__ __forceinline__ void split3(float x, __bf16& p0, __bf16& p1, __bf16& p2) {
    p0 = bf16_rne(x);
    const float r1 = x - bf16_f(p0);
    p1 = bf16_rne(r1);
    p2 = bf16_rne(r1 - bf16_f(p1));
}

// The bf16 pieces of U for the split trailing update, written once per
// layer: piece p of U[b*block + kk][c] at U3 + b*3*d_in*ldk + u3_offset(p,
// kk, c) (kk < ldk, zero past the block), so that a block's rows of U reach
// the MFMA B operand as 16-byte reads along k.  Block b's rows are read by
// the launch of block b+1 (near update, columns of block b+1) and by the
// updates of the later columns, so only the columns from (b+1)*block on are
// written (the rest of U3 is never read).  The work comes in items of 64
// columns x one block, each read along rows and transposed through LDS
// (T: 128 x 65 floats) by the kThreads threads of a workgroup; the items are
// split by the workgroups of the first block's launch that do not sweep.
constexpr int kSplitCols = 64;

__host__ __device__ inline int64_t split_items(int64_t d_in, int64_t block) {
    return ((d_in + kSplitCols - 1) / kSplitCols) * ((d_in + block - 1) / block - 1);
}

template <int kThreads>
__device__ __forceinline__ void split_u_item(float (*T)[kSplitCols + 1], const float* __restrict__ U, int64_t d_in,
                                             int64_t block, int64_t ldk, __bf16* __restrict__ U3, int64_t item) {
    const int64_t nslab = (d_in + kSplitCols - 1) / kSplitCols;
    const int64_t b = item / nslab;
    const int64_t c0 = (item - b * nslab) * kSplitCols;
    if (c0 + kSplitCols <= (b + 1) * block) return;  // columns this block's pieces are never read for
    const int64_t k0 = b * block;
    const int kb = (int)min(block, d_in - k0);
    const int tid = threadIdx.x;
    if (c0 + kSplitCols <= d_in && (d_in & 3) == 0 && (reinterpret_cast<uintptr_t>(U) & 15) == 0) {
        // every load of the slab in flight before the first LDS store:
        // thread t reads 16 bytes of rows t/16 + (kThreads/16) i, columns
        // 4 (t%16) ..
        constexpr int kPer = kMaxBlock * 16 / kThreads;
        float4v v[kPer];
        const int cc = 4 * (tid & 15);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int kk = (tid >> 4) + (kThreads / 16) * i;
            v[i] = (kk < kb) ? *reinterpret_cast<const float4v*>(U + (k0 + kk) * d_in + c0 + cc) : (float4v){};
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int kk = (tid >> 4) + (kThreads / 16) * i;
#pragma unroll
            for (int x = 0; x < 4; ++x) T[kk][cc + x] = v[i][x];
        }
    } else {
        for (int e = tid; e < kMaxBlock * kSplitCols; e += kThreads) {
            const int kk = e / kSplitCols, cc = e % kSplitCols;
            const int64_t c = c0 + cc;
            T[kk][cc] = (kk < kb && c < d_in) ? U[(k0 + kk) * d_in + c] : 0.0f;
        }
    }
    __syncthreads();
    __bf16* out = U3 + b * 3 * d_in * ldk;
    const int groups = (int)(ldk / 8);
    // consecutive threads: the two halves of one column's 16-k run, then the
    // next column, so that the stores of a run are consecutive
    for (int e = tid; e < kSplitCols * groups; e += kThreads) {
        const int run = e / (2 * kSplitCols), cc = (e % (2 * kSplitCols)) >> 1, g = 2 * run + (e & 1);
        const int64_t c = c0 + cc;
        if (c >= d_in) continue;
        bf16x8 p[3];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
            __bf16 h0, h1, h2;
            split3(T[8 * g + x][cc], h0, h1, h2);
            p[0][x] = h0;
            p[1][x] = h1;
            p[2][x] = h2;
        }
#pragma unroll
        for (int q = 0; q < 3; ++q)
            *reinterpret_cast<bf16x8*>(&out[u3_offset(d_in, ldk, q, 8 * g, c)]) = p[q];
    }
    __syncthreads();  // T is free for the next item
}

template <typename T>
__device__ __forceinline__ float to_f32(T v) {
    return (float)v;
}

// Group grid from the current working weights W[:, c0 : c0+g) (g > block).
__global__ __launch_bounds__(256) void group_grid_kernel(const float* __restrict__ Wk, int64_t d_out, int64_t d_in,
                                                         int64_t c0, int64_t g, int64_t gi, int64_t ng, float maxq,
                                                         float* __restrict__ scales, int32_t* __restrict__ zeros,
                                                         float* __restrict__ minmax) {
    const int64_t R = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (R >= d_out) return;
    float lo = INFINITY, hi = -INFINITY;
    const float* row = Wk + R * d_in + c0;
    for (int64_t c = lane; c < g; c += 64) {
        float x = row[c];
        lo = fminf(lo, x);
        hi = fmaxf(hi, x);
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) {
        lo = fminf(lo, 0.0f);
        hi = fmaxf(hi, 0.0f);
        Grid gr = make_grid(lo, hi, maxq);
        scales[R * ng + gi] = gr.s;
        zeros[R * ng + gi] = (int32_t)gr.z;
        if (minmax) {
            minmax[2 * (R * ng + gi)] = lo;
            minmax[2 * (R * ng + gi) + 1] = hi;
        }
    }
}

// One pass over the input W, one wave per row: the fp32 working copy with
// dead columns zeroed (exact for f16 inputs, subnormals included) and, with
// kGrid, the row's grid from the input values (min/max by butterfly
// shuffles).  kVec: rows of 16-byte aligned 8-element pieces (d_in % 8 == 0),
// taken in batches of kBatch pieces per lane whose loads (and dead flags,
// 8 at a time, with kDead) are all issued before any is used: pieces past
// the row end load the lane's first piece again (harmless to the min/max)
// and are not stored.  The same launch writes 1/U_jj (grid-stride over
// all threads) and clears the per-row error sums.
template <typename T, bool kVec, bool kGrid, bool kDead>
__global__ __launch_bounds__(256) void grid_convert_kernel(const T* __restrict__ W, float* __restrict__ Wk,
                                                           int64_t d_out, int64_t d_in,
                                                           const uint8_t* __restrict__ dead, float maxq,
                                                           float* __restrict__ scales, int32_t* __restrict__ zeros,
                                                           float* __restrict__ minmax, const float* __restrict__ U,
                                                           float* __restrict__ rdiag, float* __restrict__ err_row) {
    constexpr int kBatch = 8;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < d_in; j += (int64_t)gridDim.x * blockDim.x)
        rdiag[j] = 1.0f / U[j * d_in + j];
    const int64_t R = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (R >= d_out) return;
    if (err_row && lane == 0) err_row[R] = 0.0f;
    const T* row = W + R * d_in;
    float* out = Wk + R * d_in;
    float lo = INFINITY, hi = -INFINITY;
    if (kVec) {
        for (int64_t base = 8 * lane; base < d_in; base += 8 * kWave * kBatch) {
            float x[kBatch][8];
            uint2 dd[kBatch];
            int64_t cs[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
                const int64_t c = base + (int64_t)8 * kWave * i;
                cs[i] = c < d_in ? c : base;
                if constexpr (sizeof(T) == 2) {
                    const half8 h = *reinterpret_cast<const half8*>(row + cs[i]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[i][e] = (float)h[e];
                } else {
                    const float4v a = *reinterpret_cast<const float4v*>(row + cs[i]);
                    const float4v b = *reinterpret_cast<const float4v*>(row + cs[i] + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[i][e] = a[e];
                        x[i][e + 4] = b[e];
                    }
                }
                if (kDead) dd[i] = *reinterpret_cast<const uint2*>(dead + cs[i]);
            }
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    lo = fminf(lo, x[i][e]);
                    hi = fmaxf(hi, x[i][e]);
                    if (kDead && ((((e < 4) ? dd[i].x : dd[i].y) >> (8 * (e & 3))) & 0xffu)) x[i][e] = 0.0f;
                }
                if (base + (int64_t)8 * kWave * i < d_in) {
                    *reinterpret_cast<float4v*>(out + cs[i]) = (float4v){x[i][0], x[i][1], x[i][2], x[i][3]};
                    *reinterpret_cast<float4v*>(out + cs[i] + 4) = (float4v){x[i][4], x[i][5], x[i][6], x[i][7]};
                }
            }
        }
    } else {
        for (int64_t c = lane; c < d_in; c += kWave) {
            float x = to_f32(row[c]);
            lo = fminf(lo, x);
            hi = fmaxf(hi, x);
            if (kDead && dead[c]) x = 0.0f;
            out[c] = x;
        }
    }
    if (kGrid) {
        lo = wave_min(lo);
        hi = wave_max(hi);
        if (lane == 0) {
            lo = fminf(lo, 0.0f);
            hi = fmaxf(hi, 0.0f);
            Grid g = make_grid(lo, hi, maxq);
            scales[R] = g.s;
            zeros[R] = (int32_t)g.z;
            if (minmax) {
                minmax[2 * R] = lo;
                minmax[2 * R + 1] = hi;
            }
        }
    }
}


// ---------------------------------------------------------------------------
// In-block sweep.  Dynamic LDS: Up, the upper block triangle of the U block
// as nw(nw+1)/2 packed 16x16 sub-blocks (a, b), a <= b, row stride 16 (the
// strictly lower sub-blocks are never read); rdg [bw] f32 (1 / U_jj);
// Ebuf [2][16][kEld] f32 (scaled errors of the current and previous
// sub-block; only the previous one is folded in); red [nw][64][2] f32;
// errs [nw][64] f32.  Codes and scaled errors go from registers to global
// memory.  About 51 KB at bw = 128, so a sweep workgroup fits on a CU next
// to a trailing-update workgroup.
// ---------------------------------------------------------------------------
constexpr int kUld = kSub;  // row stride inside a packed U sub-block

__host__ __device__ inline int ublk_index(int a, int b, int nw) { return a * nw - a * (a - 1) / 2 + (b - a); }

__host__ __device__ inline size_t sweep_lds_bytes(int bw) {
    const int nw = (bw + kSub - 1) / kSub;
    return (size_t)nw * (nw + 1) / 2 * kSub * kSub * 4 + (size_t)bw * 4 + (size_t)2 * kSub * kEld * 4 +
           (size_t)nw * 64 * 2 * 4 + (size_t)nw * 64 * 4;
}

// Folds the 16 scaled errors of an earlier sub-block into this wave's
// columns: w_c -= sum_t e_t U[t][c].  kFull: all 16 columns present (no
// guards, so every LDS read can be issued ahead of the FMAs).
template <bool kFull, bool kVecU>
__device__ __forceinline__ void fold_in(float (&wv)[kSub], const float* __restrict__ ebp,
                                        const float* __restrict__ ublk, int uld, int lane, int cq) {
    float e[kSub];
#pragma unroll
    for (int t = 0; t < kSub; ++t) e[t] = ebp[t * kEld + lane];
#pragma unroll
    for (int t = 0; t < kSub; ++t) {
        float u[kSub];
        if (kVecU) {  // packed sub-block rows are 64 bytes apart
#pragma unroll
            for (int c = 0; c < kSub; c += 4) *reinterpret_cast<float4v*>(&u[c]) = *reinterpret_cast<const float4v*>(ublk + t * uld + c);
        } else {
#pragma unroll
            for (int c = 0; c < kSub; ++c) u[c] = ublk[t * uld + c];
        }
#pragma unroll
        for (int c = 0; c < kSub; ++c)
            if (kFull || c < cq) wv[c] -= e[t] * u[c];
    }
}

// 4x4 transpose across the four 16-lane rows of a wave: on entry register m
// of lane row g holds X[g][m]; on exit register j of lane row m holds X[j][m]
// (permlane32 swaps exchange row pairs {0,1} <-> {2,3}, permlane16 swaps odd
// and even rows).  The swaps are written as inline asm with both registers
// read-write: the compiler's two-result builtins lost the second result in
// this pattern.  Each swap is preceded by the two wait states a permlane
// read needs after a VALU write of its operands.
__device__ __forceinline__ void swap32(float& x, float& y) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void swap16(float& x, float& y) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void xpose_rows4(float& r0, float& r1, float& r2, float& r3) {
    swap32(r0, r2);  // r0 = rows {X[0][0], X[1][0], X[0][2], X[1][2]}, r2 = {X[2][0], X[3][0], X[2][2], X[3][2]}
    swap32(r1, r3);
    swap16(r0, r1);  // r0 = {X[0][0..3]} by row, r1 = {X[1][0..3]}
    swap16(r2, r3);
}

// Tile m of acc holds D[16m + l%16][4(l/16) + v] in lane l, register v
// (D[row][c], 64 rows x 16 columns); the row transpose gives lane r the 16
// entries of its own row, which are subtracted from wv.
__device__ __forceinline__ void sub_row_deltas(float (&wv)[kSub], const float4v (&acc)[4]) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        // plain VALU copies: the asm reads registers the MFMA hazard rules
        // no longer apply to
        float r0 = acc[0][v] + 0.0f, r1 = acc[1][v] + 0.0f, r2 = acc[2][v] + 0.0f, r3 = acc[3][v] + 0.0f;
        xpose_rows4(r0, r1, r2, r3);
        wv[v] -= r0;
        wv[4 + v] -= r1;
        wv[8 + v] -= r2;
        wv[12 + v] -= r3;
    }
}

// The same fold-in on MFMA, for a wave whose 16 columns are all present:
// D^T = U_blk^T E^T (16 columns x 64 rows, four 16x16 tiles, K = 16), so that
// every lane reads its own operand words instead of a broadcast U row.
// Tile m leaves D[16m + l%16][4(l/16) + v] in lane l, register v; the row
// transpose then gives lane r the 16 deltas of its own row.
__device__ __forceinline__ void fold_in_mfma(float (&wv)[kSub], const float* __restrict__ ebp,
                                             const float* __restrict__ ublk, int uld, int lane) {
    const int i = lane & 15, g = lane >> 4;
    float4v acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = (float4v){};
#pragma unroll
    for (int kk = 0; kk < kSub; kk += 4) {
        const float a = ublk[(kk + g) * uld + i];  // U_blk^T[i][kk+g]
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m] = mfma16x16x4_f32(a, ebp[(kk + g) * kEld + 16 * m + i], acc[m]);
    }
    sub_row_deltas(wv, acc);
}

// Near update of this wave's columns by the scaled errors of the previous
// block, before the sweep: wv[c] -= sum_k E_prev[row][k] U[bp0 + k][c0q + c]
// over the kp columns of that block (the part of the lazy trailing update
// that lands on this block), on MFMA 16x16x4 f32 as in fold_in_mfma.
// E_prev^T is staged in LDS (et[k][row], zero rows up to a multiple of 4)
// and the U operand comes prefetched in registers, ua[j] =
// U[bp0 + 4j + l/16][c0q + l%16].
constexpr int kEtl = kRowsPerWg + 1;  // padded LDS row of the staged E_prev^T

__device__ __forceinline__ void near_update(float (&wv)[kSub], const float (&ua)[kMaxBlock / 4],
                                            const float* __restrict__ et, int kp, int lane) {
    const int i = lane & 15, g = lane >> 4;
    float4v acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = (float4v){};
#pragma unroll
    for (int j = 0; j < kMaxBlock / 4; ++j) {
        if (4 * j < kp) {
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[m] = mfma16x16x4_f32(ua[j], et[(4 * j + g) * kEtl + 16 * m + i], acc[m]);
        }
    }
    sub_row_deltas(wv, acc);
}

// The same near update with split-precision products (the split path): the
// scaled errors E_prev and U are each the sum of three bf16 pieces, and the
// update is formed from the six piece products with i + j <= 2 on MFMA
// 16x16x32 bf16 (each product exact in fp32, fp32 accumulation), as in the
// far update.  The U operand U_blk^T (16 columns x kp) is read as 16-byte
// runs along k from the pieces split once per layer (U3p: the previous
// block's, at u3_offset; zero past the block); the E
// operand from its pieces staged in LDS by row (ets[p][row][k], zero past kp).
// The result has the layout of near_update's, so the same row transpose
// applies it.
constexpr int kEtsLd = kMaxBlock + 8;                 // LDS row of a staged E piece (bf16)
constexpr int kEtsPiece = kRowsPerWg * kEtsLd;       // one E piece (bf16)

__device__ __forceinline__ float4v mfma16x16x32_bf16(bf16x8 a, bf16x8 b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The U operands of the near update (lane: column c0q + lane%16, k run
// 32 c + 8 (lane/16) .. +8 of chunk c), loaded at the start of the sweep so
// that their latency overlaps the staging; addresses are clamped to valid
// ones and the values past the block's columns or k range set to zero.
__device__ __forceinline__ void near_split_fetch(bf16x8 (&na)[kMaxBlock / 32][3], const __bf16* __restrict__ U3p,
                                                 int64_t d_in, int64_t ldk, int64_t c0q, int cq, int kp, int lane) {
    const int i = lane & 15, g = lane >> 4;
    const int64_t col = c0q + (i < cq ? i : cq - 1);
#pragma unroll
    for (int c = 0; c < kMaxBlock / 32; ++c) {
        if (32 * c < kp && cq > 0) {  // wave-uniform
            const int k0 = 32 * c + 8 * g;
            const int kk = k0 < ldk ? k0 : (int)ldk - 8;
#pragma unroll
            for (int q = 0; q < 3; ++q) na[c][q] = *reinterpret_cast<const bf16x8*>(U3p + u3_offset(d_in, ldk, q, kk, col));
        }
    }
}

__device__ __forceinline__ void near_update_split(float (&wv)[kSub], const bf16x8 (&na)[kMaxBlock / 32][3],
                                                  int64_t ldk, int cq, const __bf16* __restrict__ ets, int kp,
                                                  int lane) {
    const int i = lane & 15, g = lane >> 4;
    float4v acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = (float4v){};
#pragma unroll
    for (int c = 0; c < kMaxBlock / 32; ++c) {
        if (32 * c < kp) {
            const int k0 = 32 * c + 8 * g;
            bf16x8 a[3];
#pragma unroll
            for (int q = 0; q < 3; ++q) a[q] = (i < cq && k0 < ldk) ? na[c][q] : (bf16x8){};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                bf16x8 b[3];
#pragma unroll
                for (int q = 0; q < 3; ++q)
                    b[q] = *reinterpret_cast<const bf16x8*>(&ets[q * kEtsPiece + (16 * m + i) * kEtsLd + k0]);
                // the smaller piece products first
                acc[m] = mfma16x16x32_bf16(a[2], b[0], acc[m]);
                acc[m] = mfma16x16x32_bf16(a[1], b[1], acc[m]);
                acc[m] = mfma16x16x32_bf16(a[0], b[2], acc[m]);
                acc[m] = mfma16x16x32_bf16(a[1], b[0], acc[m]);
                acc[m] = mfma16x16x32_bf16(a[0], b[1], acc[m]);
                acc[m] = mfma16x16x32_bf16(a[0], b[0], acc[m]);
            }
        }
    }
    sub_row_deltas(wv, acc);
}

// LDS of the staged E_prev: transposed fp32 (near_update) or three bf16
// pieces by row (near_update_split), after the sweep's own regions; 16 bytes
// of slack let the pieces start 16-byte aligned.
__host__ __device__ inline size_t near_lds_bytes(int kp, bool split) {
    if (kp <= 0) return 0;
    return split ? (size_t)3 * kEtsPiece * 2 + 16 : (size_t)((kp + 3) & ~3) * kEtl * 4;
}

// Rounds this wave's columns in order, compensating the later columns of
// the sub-block at once.  U rows of the sub-block and 1/U_jj are read into
// registers before the dependent chain starts.
// The rounding decision needs x = fl32(w / s) exactly.  With y = fl32(1/s)
// computed once per grid, q0 = fl32(w y), r = fma(-q0, s, w) (exact) and
// fl32(q0 + r y) is the correctly rounded quotient (Markstein's theorem for
// round-to-nearest; no overflow or underflow at these magnitudes), which
// replaces the full IEEE division sequence in the dependent chain.
__device__ __forceinline__ float div_rn(float w, float s, float y) {
    const float q0 = w * y;
    const float r = __builtin_fmaf(-q0, s, w);
    return __builtin_fmaf(r, y, q0);
}

template <bool kFull, bool kVecU>
__device__ __forceinline__ void sweep_sub(float (&wv)[kSub], float s, float sinv, float zf, float maxq,
                                          const float* __restrict__ ublk, int uld, const float* __restrict__ rd,
                                          float* __restrict__ ebq, uint32_t (&cw)[kSub / 4], float (&ev)[kSub],
                                          int lane, int cq, float& errsq) {
#pragma unroll
    for (int i = 0; i < kSub / 4; ++i) cw[i] = 0;
    float r[kSub];
#pragma unroll
    for (int t = 0; t < kSub; ++t) r[t] = rd[t];
    // kVecU: U rows in two register sets, row t+1 loaded at the start of
    // column t, so that the loads are in flight through a whole column's
    // dependent chain.  Only the entries used (columns after t) are loaded:
    // 16-byte loads for whole quads, single ones before the first whole quad
    // (a vector load with unused lanes lets the chain reuse its registers,
    // which then waits for the load)
    float ub[2][kSub];
    auto load_row = [&](float (&u)[kSub], int t) {
        const int q0 = 4 * ((t + 4) / 4);  // first whole quad after column t
#pragma unroll
        for (int c = t + 1; c < q0 && c < kSub; ++c) u[c] = ublk[t * uld + c];
#pragma unroll
        for (int c = q0; c < kSub; c += 4) *reinterpret_cast<float4v*>(&u[c]) = *reinterpret_cast<const float4v*>(ublk + t * uld + c);
    };
    if (kVecU) load_row(ub[0], 0);
#pragma unroll
    for (int t = 0; t < kSub; ++t) {
        if (kFull || t < cq) {
            float u[kSub];
            if (kVecU) {
                if (t + 1 < kSub) load_row(ub[(t + 1) & 1], t + 1);
#pragma unroll
                for (int c = t + 1; c < kSub; ++c) u[c] = ub[t & 1][c];
            } else {
#pragma unroll
                for (int t2 = t + 1; t2 < kSub; ++t2) u[t2] = ublk[t * uld + t2];
            }
            const float w = wv[t];
            const float x = div_rn(w, s, sinv);
            const float v = x + zf;
            float qf = __builtin_rintf(v);
            qf = fminf(fmaxf(qf, 0.0f), maxq);
            const float what = (qf - zf) * s;
            const float e = (w - what) * r[t];
            cw[t >> 2] |= (uint32_t)qf << (8 * (t & 3));
            ev[t] = e;
            ebq[t * kEld + lane] = e;
            errsq += e * e;
#pragma unroll
            for (int t2 = t + 1; t2 < kSub; ++t2)
                if (kFull || t2 < cq) wv[t2] -= e * u[t2];
        }
    }
}

// Sweep of rows 64 rt .. 64 rt + 63 (512 threads).  kAllFull: the block
// width is a multiple of 16, so every wave owns 16 columns and the unguarded
// code paths are the only ones compiled.  With kp > 0 the scaled errors Ep
// of the previous block [bp0, bp0 + kp) are applied to this block's columns
// first (near_update, or near_update_split with kSplit); the LDS then holds
// E_prev^T (or its bf16 pieces) after the sweep's own regions.
template <bool kAllFull, bool kSplit>
__device__ __forceinline__ void sweep_body(unsigned char* smem, int rt, const float* __restrict__ Wk, int64_t d_out,
                                           int64_t d_in, const float* __restrict__ U,
                                           const float* __restrict__ rdiag, int64_t b0, int64_t b1, int bits,
                                           int64_t group, int64_t ng, float* __restrict__ scales,
                                           int32_t* __restrict__ zeros, float* __restrict__ minmax,
                                           uint8_t* __restrict__ codes, float* __restrict__ E,
                                           float* __restrict__ err_row, const float* __restrict__ Ep, int64_t bp0,
                                           int kp, const __bf16* __restrict__ U3p, int64_t ldk) {
    const int bw = (int)(b1 - b0);
    const int nw = (bw + kSub - 1) / kSub;
    const int uld = kUld;
    float* Up = reinterpret_cast<float*>(smem);                         // nw(nw+1)/2 * 256
    float* rdg = Up + nw * (nw + 1) / 2 * kSub * kSub;                    // bw
    float* Ebuf = rdg + bw;                                               // 2*16*kEld
    float* red = Ebuf + 2 * kSub * kEld;                                  // nw*64*2
    float* errs = red + nw * 64 * 2;                                      // nw*64
    float* et = errs + nw * 64;                                           // [kp rounded up to 4][kEtl]
    // split path: [3][kRowsPerWg][kEtsLd] bf16 pieces, 16-byte aligned
    __bf16* ets = reinterpret_cast<__bf16*>(smem + ((reinterpret_cast<uintptr_t>(et) - reinterpret_cast<uintptr_t>(smem) + 15) & ~(uintptr_t)15));

    const int lane = threadIdx.x & 63;
    const int q = wave_id();
    const int64_t R = (int64_t)rt * kRowsPerWg + lane;
    const bool rowok = R < d_out;
    // waves past the block (q >= nw: a narrow block in a 512-thread launch)
    // hold no columns and only take part in the barriers
    const int cq = (q >= nw) ? 0 : kAllFull ? kSub : min(kSub, bw - kSub * q);
    const int64_t c0q = b0 + kSub * q;
    const float maxq = (float)((1 << bits) - 1);

    // this wave's columns of the working weights and the row grid: loads
    // issued first so that their latency overlaps the staging below
    float wv[kSub];
    const bool vec_row = rowok && cq == kSub && ((d_in | c0q) & 3) == 0;  // 16-byte aligned full row slice
    if (vec_row) {
#pragma unroll
        for (int t = 0; t < kSub; t += 4) *reinterpret_cast<float4v*>(&wv[t]) = *reinterpret_cast<const float4v*>(Wk + R * d_in + c0q + t);
    } else {
#pragma unroll
        for (int t = 0; t < kSub; ++t) wv[t] = (rowok && t < cq) ? Wk[R * d_in + c0q + t] : 0.0f;
    }

    bf16x8 na[kMaxBlock / 32][3];
    if (kSplit && kp > 0) near_split_fetch(na, U3p, d_in, ldk, c0q, cq, kp, lane);

    float s = 1.0f, zf = 0.0f;
    if (group == 0) {
        if (rowok) {
            s = scales[R];
            zf = (float)zeros[R];
        }
    } else if (group > bw) {
        // group wider than the block (a multiple of it): grid prepared at the
        // group start by group_grid_kernel
        const int64_t gi = b0 / group;
        if (rowok) {
            s = scales[R * ng + gi];
            zf = (float)zeros[R * ng + gi];
        }
    }

    // near update operands: U rows of the previous block for this wave's
    // columns, and 16 entries of E_prev per thread (row tid%64, the k run
    // 16 (tid/64): a wave reads one run of 64 rows, 4 KB in a row)
    float ua[kMaxBlock / 4];
    float ep[16];
    const int er = threadIdx.x & 63, ek = (threadIdx.x >> 6) * 16;
    if (kp > 0) {
        const int i = lane & 15, g = lane >> 4;
        if (!kSplit) {
#pragma unroll
            for (int j = 0; j < kMaxBlock / 4; ++j) {
                const int k = 4 * j + g;
                ua[j] = (k < kp && i < cq) ? U[(bp0 + k) * d_in + c0q + i] : 0.0f;
            }
        }
        const int64_t Re = (int64_t)rt * kRowsPerWg + er;
        const float* src = Ep + eoff(d_out, Re, ek);
        if (Re < d_out && ek + 16 <= kp && (reinterpret_cast<uintptr_t>(Ep) & 15) == 0) {
#pragma unroll
            for (int e = 0; e < 16; e += 4) *reinterpret_cast<float4v*>(&ep[e]) = *reinterpret_cast<const float4v*>(src + e);
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) ep[e] = (Re < d_out && ek + e < kp) ? src[e] : 0.0f;
        }
    }

    // stage the U block (upper part; the rest is never read) and 1/U_jj,
    // with every thread's loads in flight before its LDS stores
    const int nth = blockDim.x;
    if (bw == kMaxBlock && nth == 512 && ((b0 | d_in) & 3) == 0 &&
        (reinterpret_cast<uintptr_t>(U) & 15) == 0) {
        // full block: 16-byte loads, 8 per thread
        float4v t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = threadIdx.x + i * 512;
            const int r = e >> 5, c = (e & 31) * 4;
            t[i] = ((r >> 4) <= (c >> 4)) ? *reinterpret_cast<const float4v*>(U + (b0 + r) * d_in + b0 + c) : (float4v){};
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = threadIdx.x + i * 512;
            const int r = e >> 5, c = (e & 31) * 4;
            if ((r >> 4) <= (c >> 4))
                *reinterpret_cast<float4v*>(Up + ublk_index(r >> 4, c >> 4, nw) * (kSub * kSub) + (r & 15) * kUld + (c & 15)) = t[i];
        }
    } else {
        constexpr int kPer = (kMaxBlock * kMaxBlock + 511) / 512;  // elements per thread at 512 threads
        float t[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = threadIdx.x + i * nth;
            const int r = e / bw, c = e % bw;
            t[i] = (e < bw * bw && c >= r) ? U[(b0 + r) * d_in + b0 + c] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = threadIdx.x + i * nth;
            const int r = e / bw, c = e % bw;
            if (e < bw * bw && (r >> 4) <= (c >> 4))
                Up[ublk_index(r >> 4, c >> 4, nw) * (kSub * kSub) + (r & 15) * kUld + (c & 15)] = t[i];
        }
    }
    for (int e = threadIdx.x; e < bw; e += nth) rdg[e] = rdiag[b0 + e];
    if (kp > 0) {
        if (kSplit) {
            // the three bf16 pieces of E_prev row er, k = ek .. ek + 15 (zero
            // past kp: ep holds zeros there)
            bf16x8 p[3][2];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                __bf16 h0, h1, h2;
                split3(ep[e], h0, h1, h2);
                p[0][e >> 3][e & 7] = h0;
                p[1][e >> 3][e & 7] = h1;
                p[2][e >> 3][e & 7] = h2;
            }
#pragma unroll
            for (int q = 0; q < 3; ++q)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    *reinterpret_cast<bf16x8*>(&ets[q * kEtsPiece + er * kEtsLd + ek + 8 * h]) = p[q][h];
        } else {
            const int kp4 = (kp + 3) & ~3;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (ek + e < kp4) et[(ek + e) * kEtl + er] = ep[e];
        }
    }

    float sinv = 1.0f / s;
    float errsq = 0.0f;
    __syncthreads();
    if (kp > 0) {
        if (kSplit) near_update_split(wv, na, ldk, cq, ets, kp, lane);
        else near_update(wv, ua, et, kp, lane);
    }

    for (int p = 0; p < nw; ++p) {
        // wave p carries the dependent chain of this phase: it gets issue
        // priority over the waves that only fold errors in for later phases
        if (q == p) __builtin_amdgcn_s_setprio(2);
        if (p > 0 && q >= p && q < nw) {
            // fold in the scaled errors of sub-block p-1 (16 full columns)
            const float* ebp = Ebuf + ((p - 1) & 1) * kSub * kEld;
            const float* ublk = Up + ublk_index(p - 1, q, nw) * (kSub * kSub);
            if (kAllFull)
                fold_in_mfma(wv, ebp, ublk, uld, lane);
            else if (cq == kSub)
                fold_in<true, false>(wv, ebp, ublk, uld, lane, cq);
            else
                fold_in<false, false>(wv, ebp, ublk, uld, lane, cq);
        }
        if (group > 0 && group <= bw && ((int64_t)kSub * p) % group == 0) {
            // group start at column b0 + 16p: grid from the current weights
            const int gwaves = (int)(group / kSub);
            if (q >= p && q < p + gwaves) {
                float lo = INFINITY, hi = -INFINITY;
#pragma unroll
                for (int c = 0; c < kSub; ++c)
                    if (c < cq) {
                        lo = fminf(lo, wv[c]);
                        hi = fmaxf(hi, wv[c]);
                    }
                red[(q * 64 + lane) * 2] = lo;
                red[(q * 64 + lane) * 2 + 1] = hi;
            }
            __syncthreads();
            float lo = INFINITY, hi = -INFINITY;
            for (int qq = p; qq < p + gwaves; ++qq) {
                lo = fminf(lo, red[(qq * 64 + lane) * 2]);
                hi = fmaxf(hi, red[(qq * 64 + lane) * 2 + 1]);
            }
            lo = fminf(lo, 0.0f);
            hi = fmaxf(hi, 0.0f);
            Grid g = make_grid(lo, hi, maxq);
            s = g.s;
            sinv = 1.0f / s;
            zf = g.z;
            if (q == p && rowok) {
                const int64_t gi = (b0 + kSub * p) / group;
                scales[R * ng + gi] = g.s;
                zeros[R * ng + gi] = (int32_t)g.z;
                if (minmax) {
                    minmax[2 * (R * ng + gi)] = lo;
                    minmax[2 * (R * ng + gi) + 1] = hi;
                }
            }
        }
        if (q == p) {
            float* ebq = Ebuf + (p & 1) * kSub * kEld;
            const float* ublk = Up + ublk_index(p, p, nw) * (kSub * kSub);
            const float* rd = rdg + kSub * p;
            uint32_t cw[kSub / 4];
            float ev[kSub];
            if (kAllFull || cq == kSub)
                sweep_sub<true, kAllFull>(wv, s, sinv, zf, maxq, ublk, uld, rd, ebq, cw, ev, lane, cq, errsq);
            else
                sweep_sub<false, false>(wv, s, sinv, zf, maxq, ublk, uld, rd, ebq, cw, ev, lane, cq, errsq);
            __builtin_amdgcn_s_setprio(0);
            // this sub-block's codes and scaled errors are final: store them
            // now so that the stores drain while the later sub-blocks run
            const int64_t ce = kSub * (int64_t)p;  // column of the block
            const bool vec_out = vec_row && (d_in & 15) == 0 && ((b0 + ce) & 15) == 0 &&
                                 ((reinterpret_cast<uintptr_t>(codes) | reinterpret_cast<uintptr_t>(E)) & 15) == 0;
            if (vec_out) {
                *reinterpret_cast<uint4*>(codes + R * d_in + b0 + ce) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
#pragma unroll
                for (int t = 0; t < kSub; t += 4) *reinterpret_cast<float4v*>(E + eoff(d_out, R, (int)ce + t)) = *reinterpret_cast<const float4v*>(&ev[t]);
            } else if (rowok) {
#pragma unroll
                for (int t = 0; t < kSub; ++t)
                    if (t < cq) {
                        codes[R * d_in + b0 + ce + t] = (uint8_t)(cw[t >> 2] >> (8 * (t & 3)));
                        E[eoff(d_out, R, (int)ce + t)] = ev[t];
                    }
            }
        }
        __syncthreads();
    }
    if (q < nw) errs[q * 64 + lane] = errsq;
    __syncthreads();

    if (err_row && q == 0 && rowok) {
        float acc = err_row[R];
        for (int qq = 0; qq < nw; ++qq) acc += errs[qq * 64 + lane];
        err_row[R] = acc;
    }
}

// ---------------------------------------------------------------------------
// Lazy trailing update W[:, b1:] -= E[:, :K] U[b0:b1, b1:], K = b1 - b0.
// kRT x 128 tile per workgroup (kRT = 64 in use); 4 waves in 2x2, each
// kRT/2 x 64 as (kRT/64) x 2 MFMA 32x32x2 f32 tiles.  K runs in chunks of
// 32: chunk c+1 is fetched into registers while the MFMAs consume chunk c
// from one of two LDS buffers (one barrier per chunk).
// E is staged row-major with an odd row stride, so the A-operand reads
// (32 rows, one k) hit distinct banks.
// ---------------------------------------------------------------------------
constexpr int kTT = 128;         // columns per trailing-update tile
constexpr int kTrailRows = 64;   // rows per trailing-update tile
constexpr int kTK = 32;
constexpr int kEs = kTK + 1;   // E stage row stride (odd)
constexpr int kUs = kTT + 4;   // U stage row stride

struct TrailLds {
    float E[2][kTrailRows * kEs];  // sized for the 64-row tiles in use (50.7 KB in all: three workgroups per CU)
    float U[2][kTK * kUs];
};

// Per-thread staging registers for a tile of kRT rows: E holds kRT/8 floats
// (row tid / (256/kRT), k run of kRT/8), U 16 floats (k row tid/8, 16 columns).
template <int kRT>
struct TrailRegs {
    static constexpr int kE = kRT / 8;
    float e[kE];
    float u[16];
};

template <bool kVec, int kRT>
__device__ __forceinline__ void trail_fetch(TrailRegs<kRT>& r, const float* __restrict__ E,
                                            const float* __restrict__ U, int64_t d_out, int64_t d_in, int64_t r0,
                                            int64_t c0, int64_t b0, int K, int kc, int tid, int64_t c_end) {
    constexpr int kE = TrailRegs<kRT>::kE;
    constexpr int kPerRow = kTK / kE;  // threads per E row
    {
        const int64_t R = r0 + tid / kPerRow;
        const int k = kc + (tid % kPerRow) * kE;  // kE-aligned: its kE entries lie in one run
        const float* src = E + eoff(d_out, R, k);
        if (kVec && R < d_out && k + kE <= K) {
#pragma unroll
            for (int e = 0; e < kE; e += 4) *reinterpret_cast<float4v*>(&r.e[e]) = *reinterpret_cast<const float4v*>(src + e);
        } else {
#pragma unroll
            for (int e = 0; e < kE; ++e) r.e[e] = (R < d_out && k + e < K) ? src[e] : 0.0f;
        }
    }
    {
        const int k = kc + (tid >> 3);
        const int64_t col = c0 + (tid & 7) * 16;
        const float* src = U + (b0 + k) * d_in + col;
        if (kVec && k < K && col + 16 <= c_end) {
#pragma unroll
            for (int e = 0; e < 16; e += 4) *reinterpret_cast<float4v*>(&r.u[e]) = *reinterpret_cast<const float4v*>(src + e);
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) r.u[e] = (k < K && col + e < c_end) ? src[e] : 0.0f;
        }
    }
}

template <int kRT>
__device__ __forceinline__ void trail_stash(const TrailRegs<kRT>& r, TrailLds& s, int buf, int tid) {
    constexpr int kE = TrailRegs<kRT>::kE;
    constexpr int kPerRow = kTK / kE;
    float* Es = s.E[buf] + (tid / kPerRow) * kEs + (tid % kPerRow) * kE;
#pragma unroll
    for (int e = 0; e < kE; ++e) Es[e] = r.e[e];
    float* Us = s.U[buf] + (tid >> 3) * kUs + (tid & 7) * 16;
#pragma unroll
    for (int e = 0; e < 16; e += 4) *reinterpret_cast<float4v*>(&Us[e]) = *reinterpret_cast<const float4v*>(&r.u[e]);
}

// W[r0 .. r0+kRT, c0 .. c0+128] -= E[rows, 0..K) U[b0 .. b1, cols] for the
// tile (blockIdx.y, blockIdx.x) of columns [c_begin, c_end).  Four waves in
// a 2x2 grid, each kRT/2 x 64 as (kRT/64) x 2 MFMA 32x32x2 f32 tiles; K in
// chunks of 32 through two LDS buffers with a register prefetch.
template <bool kVec, int kRT>
__global__ __launch_bounds__(256) void trail_kernel(float* __restrict__ Wk, int64_t d_out, int64_t d_in,
                                                    const float* __restrict__ E,
                                                    const float* __restrict__ U, int64_t b0, int64_t b1,
                                                    int64_t c_begin, int64_t c_end) {
    static_assert(kRT <= kTrailRows, "the E stage is sized for kTrailRows rows");
    constexpr int kM = kRT / 64;  // MFMA row tiles per wave
    __shared__ TrailLds s;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wi = w >> 1, wj = w & 1;
    const int64_t r0 = (int64_t)blockIdx.y * kRT;
    const int64_t c0 = c_begin + (int64_t)blockIdx.x * kTT;
    const int K = (int)(b1 - b0);
    const int nchunks = (K + kTK - 1) / kTK;

    float16v acc[kM][2];
#pragma unroll
    for (int m = 0; m < kM; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[m][q] = (float16v){};

    TrailRegs<kRT> regs;
    trail_fetch<kVec, kRT>(regs, E, U, d_out, d_in, r0, c0, b0, K, 0, tid, c_end);
    // the 64-row tile reads its W tile early (a 128-row tile would need 64
    // more registers for it and lose occupancy)
    constexpr bool kPre = kRT == 64;
    float wold[kM][2][16];
    if (kPre) {
#pragma unroll
        for (int m = 0; m < kM; ++m)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t row = r0 + wi * (kRT / 2) + 32 * m + acc32_row(v, lane);
                    const int64_t col = c0 + wj * 64 + 32 * q + (lane & 31);
                    wold[m][q][v] = (row < d_out && col < c_end) ? Wk[row * d_in + col] : 0.0f;
                }
    }
    for (int c = 0; c < nchunks; ++c) {
        const int buf = c & 1;
        trail_stash<kRT>(regs, s, buf, tid);
        __syncthreads();
        if (c + 1 < nchunks) trail_fetch<kVec, kRT>(regs, E, U, d_out, d_in, r0, c0, b0, K, (c + 1) * kTK, tid, c_end);
        const float* Es = s.E[buf];
        const float* Us = s.U[buf];
#pragma unroll
        for (int ks = 0; ks < kTK; ks += 2) {
            float a[kM], b[2];
#pragma unroll
            for (int m = 0; m < kM; ++m) a[m] = Es[(wi * (kRT / 2) + 32 * m + (lane & 31)) * kEs + ks + (lane >> 5)];
#pragma unroll
            for (int q = 0; q < 2; ++q) b[q] = Us[(ks + (lane >> 5)) * kUs + wj * 64 + 32 * q + (lane & 31)];
#pragma unroll
            for (int m = 0; m < kM; ++m)
#pragma unroll
                for (int q = 0; q < 2; ++q) acc[m][q] = mfma32x32x2_f32(a[m], b[q], acc[m][q]);
        }
    }
#pragma unroll
    for (int m = 0; m < kM; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = r0 + wi * (kRT / 2) + 32 * m + acc32_row(v, lane);
                const int64_t col = c0 + wj * 64 + 32 * q + (lane & 31);
                if (row < d_out && col < c_end) {
                    float* p = Wk + row * d_in + col;
                    *p = (kPre ? wold[m][q][v] : *p) - acc[m][q][v];
                }
            }
}

// ---------------------------------------------------------------------------
// The far part of the lazy trailing update inside the per-block launch:
// W[r0 .. r0+128, c0 .. c_end) -= E_prev[rows, :kp] U[bp0 .. bp0+kp, cols]
// for one sub-tile of at most 256 columns.  512 threads: eight waves in a
// 4x2 grid, each 32 rows x 128 columns as four MFMA 32x32x2 f32 tiles (the
// products of 32-column pieces past c_end are skipped); K in chunks of 32
// through two LDS buffers with a register prefetch, and the W tile read
// ahead of the products.  The launch is one workgroup per CU (its LDS), so
// the per-wave work is large and the registers plentiful.
// ---------------------------------------------------------------------------
constexpr int kRestRows = sched::kFarRows;
constexpr int kRestCols = sched::kFarCols;
constexpr int kStrip = sched::kFarStrip;  // unit of the far-update partition: 128 rows x 64 columns
constexpr int kRUs = kRestCols + 4;  // U stage row stride

__host__ __device__ inline size_t rest_lds_bytes() {
    return (size_t)(2 * kRestRows * kEs + 2 * kTK * kRUs) * 4;
}

__device__ __forceinline__ void rest_fetch(float (&e)[8], float (&u)[16], const float* __restrict__ E,
                                           const float* __restrict__ U, int64_t d_out, int64_t d_in, int64_t r0,
                                           int64_t c0, int64_t c_end, int64_t bp0, int kp, int kc, int tid, bool vec) {
    {
        const int64_t R = r0 + (tid >> 2);
        const int k = kc + (tid & 3) * 8;  // 8-aligned: its 8 entries lie in one run
        const float* src = E + eoff(d_out, R, k);
        if (vec && R < d_out && k + 8 <= kp) {
#pragma unroll
            for (int x = 0; x < 8; x += 4) *reinterpret_cast<float4v*>(&e[x]) = *reinterpret_cast<const float4v*>(src + x);
        } else {
#pragma unroll
            for (int x = 0; x < 8; ++x) e[x] = (R < d_out && k + x < kp) ? src[x] : 0.0f;
        }
    }
    {
        const int k = kc + (tid >> 4);
        const int64_t col = c0 + (tid & 15) * 16;
        const float* src = U + (bp0 + k) * d_in + col;
        if (vec && k < kp && col + 16 <= c_end) {
#pragma unroll
            for (int x = 0; x < 16; x += 4) *reinterpret_cast<float4v*>(&u[x]) = *reinterpret_cast<const float4v*>(src + x);
        } else {
#pragma unroll
            for (int x = 0; x < 16; ++x) u[x] = (k < kp && col + x < c_end) ? src[x] : 0.0f;
        }
    }
}

// products of one K chunk for a wave's NQ 32-column pieces
template <int NQ>
__device__ __forceinline__ void rest_chunk(const float* Eb, const float* Ub, int wi, int colw, int lane,
                                           float16v (&acc)[4]) {
#pragma unroll
    for (int ks = 0; ks < kTK; ks += 2) {
        const float a = Eb[(wi * 32 + (lane & 31)) * kEs + ks + (lane >> 5)];
        float b[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) b[q] = Ub[(ks + (lane >> 5)) * kRUs + colw + 32 * q + (lane & 31)];
#pragma unroll
        for (int q = 0; q < NQ; ++q) acc[q] = mfma32x32x2_f32(a, b[q], acc[q]);
    }
}

__device__ __forceinline__ void rest_body(unsigned char* smem, int64_t r0, int64_t c0, int64_t c_end,
                                          float* __restrict__ Wk, int64_t d_out, int64_t d_in,
                                          const float* __restrict__ E, const float* __restrict__ U,
                                          int64_t bp0, int kp, bool vec) {
    float* Es = reinterpret_cast<float*>(smem);  // [2][kRestRows * kEs]
    float* Us = Es + 2 * kRestRows * kEs;        // [2][kTK * kRUs]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wi = w >> 1, wj = w & 1;
    const int nchunks = (kp + kTK - 1) / kTK;
    // the sub-tile's 64-column strips split between the two column halves of
    // the wave grid: each wave takes ns 32-column pieces (fewer at c_end)
    const int ns = (int)((c_end - c0 + kStrip - 1) / kStrip);
    const int colw = wj * ns * 32;
    const int64_t cw = c0 + colw;
    const int nq = (int)std::min<int64_t>(ns, std::max<int64_t>(0, (c_end - cw + 31) / 32));
    const bool inner = (r0 + kRestRows <= d_out) && (cw + 32 * nq <= c_end);

    float16v acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = (float16v){};
    float e[8], u[16];
    rest_fetch(e, u, E, U, d_out, d_in, r0, c0, c_end, bp0, kp, 0, tid, vec);
    float wold[4][16];
    for (int c = 0; c < nchunks; ++c) {
        const int buf = c & 1;
        {
            float* ed = Es + buf * kRestRows * kEs + (tid >> 2) * kEs + (tid & 3) * 8;
#pragma unroll
            for (int x = 0; x < 8; ++x) ed[x] = e[x];
            float* ud = Us + buf * kTK * kRUs + (tid >> 4) * kRUs + (tid & 15) * 16;
#pragma unroll
            for (int x = 0; x < 16; x += 4) *reinterpret_cast<float4v*>(&ud[x]) = *reinterpret_cast<const float4v*>(&u[x]);
        }
        __syncthreads();
        if (c + 1 < nchunks)
            rest_fetch(e, u, E, U, d_out, d_in, r0, c0, c_end, bp0, kp, (c + 1) * kTK, tid, vec);
        if (c == 0) {
            // the old W tile, behind the next chunk's operands (so that their
            // wait does not include it); addresses outside the sub-tile are
            // clamped to its first element, so that every load is issued
            // without a branch (those values are never stored)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (q < nq) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int64_t row = r0 + wi * 32 + acc32_row(v, lane);
                        const int64_t col = cw + 32 * q + (lane & 31);
                        const bool ok = row < d_out && col < c_end;
                        wold[q][v] = Wk[ok ? row * d_in + col : r0 * d_in + c0];
                    }
                }
        }
        const float* Eb = Es + buf * kRestRows * kEs;
        const float* Ub = Us + buf * kTK * kRUs;
        switch (nq) {
            case 4: rest_chunk<4>(Eb, Ub, wi, colw, lane, acc); break;
            case 3: rest_chunk<3>(Eb, Ub, wi, colw, lane, acc); break;
            case 2: rest_chunk<2>(Eb, Ub, wi, colw, lane, acc); break;
            case 1: rest_chunk<1>(Eb, Ub, wi, colw, lane, acc); break;
            default: break;
        }
    }
    if (nchunks == 0) return;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (q < nq) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = r0 + wi * 32 + acc32_row(v, lane);
                const int64_t col = cw + 32 * q + (lane & 31);
                if (inner || (row < d_out && col < c_end)) Wk[row * d_in + col] = wold[q][v] - acc[q][v];
            }
        }
}

// ---------------------------------------------------------------------------
// The same far update with split-precision products: each fp32 operand is
// the sum of three bf16 pieces, x = x0 + x1 + x2 (x0 = bf16(x) to nearest
// even, x1 = bf16(x - x0), x2 = bf16(x - x0 - x1); both differences are
// exact in fp32), and E U is formed from the six piece products with
// i + j <= 2 on MFMA 32x32x16 bf16 (each product exact in fp32, fp32
// accumulation).  The three dropped products are below 2^-26 of |e u|; the
// piece products take 6 bf16 MFMAs (192 cycles) where fp32 MFMA 32x32x2
// takes 8 (512 cycles) per 16-deep step.  K in chunks of 16 through two LDS
// buffers: E pieces row-major by k, U pieces transposed (column-major by k)
// so that both MFMA operands are 16-byte reads along k.
// ---------------------------------------------------------------------------
constexpr int kSK = 16;           // K per chunk
constexpr int kSLd = kSK + 8;     // padded LDS row of a piece stage (bf16)
constexpr int kSEPiece = kRestRows * kSLd;  // one E piece of one buffer (bf16)
constexpr int kSUPiece = kRestCols * kSLd;  // one U piece of one buffer (bf16)
constexpr int kSBuf = 3 * (kSEPiece + kSUPiece);

__host__ __device__ inline size_t rest_split_lds_bytes() { return (size_t)2 * kSBuf * 2; }


// chunk operands: E rows r0 + tid/4, k kc + 4(tid%4) .. +4 (split here);
// the U pieces of column c0 + tid/2, k kc + 8(tid%2) .. +8, already
// split (U3b: the previous block's pieces at u3_offset, so that a wave's
// reads of one piece are 1 KB in a row).  Columns past
// c_end load column c0 (their products are never stored).
__device__ __forceinline__ void rest_split_fetch(float (&e)[4], bf16x8 (&u)[3], const float* __restrict__ E,
                                                 const __bf16* __restrict__ U3b, int64_t ldk,
                                                 int64_t d_out, int64_t d_in, int64_t r0, int64_t c0, int64_t c_end,
                                                 int kp, int kc, int tid, bool vec) {
    // addresses formed anew at each fetch from an opaque copy of the thread
    // index: the run offsets of successive fetches are too far apart for an
    // instruction offset, and addresses kept from one fetch to the next would
    // cost registers
    int t = tid;
    asm volatile("" : "+v"(t));
    {
        const int64_t R = r0 + (t >> 2);
        const int k = kc + (t & 3) * 4;
        // eoff(R, k), its run part (kc / 16) uniform
        const float* src = E + ((int64_t)(kc >> 4) * d_out + R) * 16 + (t & 3) * 4;
        if (vec && R < d_out && k + 4 <= kp) {
            *reinterpret_cast<float4v*>(&e[0]) = *reinterpret_cast<const float4v*>(src);
        } else {
#pragma unroll
            for (int x = 0; x < 4; ++x) e[x] = (R < d_out && k + x < kp) ? src[x] : 0.0f;
        }
    }
    {
        int64_t col = c0 + (t >> 1);
        if (col >= c_end) col = c0;
        // u3_offset(0, kc + 8 (t%2), col), its run part (kc / 16) uniform
        const __bf16* src = U3b + (int64_t)(kc >> 4) * d_in * 16 + col * 16 + (t & 1) * 8;
#pragma unroll
        for (int q = 0; q < 3; ++q) u[q] = *reinterpret_cast<const bf16x8*>(src + q * d_in * ldk);
    }
}

__device__ __forceinline__ void rest_split_stash(const float (&e)[4], const bf16x8 (&u)[3], __bf16* __restrict__ S,
                                                 int tid) {
    {
        bf16x4 p[3];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            __bf16 h0, h1, h2;
            split3(e[x], h0, h1, h2);
            p[0][x] = h0;
            p[1][x] = h1;
            p[2][x] = h2;
        }
        const int off = (tid >> 2) * kSLd + (tid & 3) * 4;
#pragma unroll
        for (int q = 0; q < 3; ++q) *reinterpret_cast<bf16x4*>(&S[q * kSEPiece + off]) = p[q];
    }
    {
        const int off = 3 * kSEPiece + (tid >> 1) * kSLd + (tid & 1) * 8;
#pragma unroll
        for (int q = 0; q < 3; ++q) *reinterpret_cast<bf16x8*>(&S[off + q * kSUPiece]) = u[q];
    }
}

__device__ __forceinline__ float16v mfma32x32x16_bf16(bf16x8 a, bf16x8 b, float16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int NQ>
__device__ __forceinline__ void rest_split_chunk(const __bf16* S, int wi, int colw, int lane, float16v (&acc)[4]) {
    const int kk = 8 * (lane >> 5);
    bf16x8 a[3], b[3][NQ];
#pragma unroll
    for (int p = 0; p < 3; ++p)
        a[p] = *reinterpret_cast<const bf16x8*>(&S[p * kSEPiece + (wi * 32 + (lane & 31)) * kSLd + kk]);
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            b[p][q] = *reinterpret_cast<const bf16x8*>(
                &S[3 * kSEPiece + p * kSUPiece + (colw + 32 * q + (lane & 31)) * kSLd + kk]);
    // the smaller piece products first
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q] = mfma32x32x16_bf16(a[2], b[0][q], acc[q]);
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q] = mfma32x32x16_bf16(a[1], b[1][q], acc[q]);
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q] = mfma32x32x16_bf16(a[0], b[2][q], acc[q]);
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q] = mfma32x32x16_bf16(a[1], b[0][q], acc[q]);
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q] = mfma32x32x16_bf16(a[0], b[1][q], acc[q]);
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q] = mfma32x32x16_bf16(a[0], b[0][q], acc[q]);
}

// A full sub-tile (128 x 256 inside W, K = 128: eight chunks, four 32-column
// pieces per wave): the chunk loop unrolled, the operands of chunk c+2
// fetched while chunk c is multiplied (two register sets), and the old W
// tile read during the last two chunks, behind every operand fetch.  Loads
// complete in issue order, so no operand wait includes the W tile.
__device__ __forceinline__ void rest_split_body_full(unsigned char* smem, int64_t r0, int64_t c0,
                                                     float* __restrict__ Wk, int64_t d_out, int64_t d_in,
                                                     const float* __restrict__ E,
                                                     const __bf16* __restrict__ U3b, int64_t ldk, bool vec) {
    constexpr int kChunks = kMaxBlock / kSK;
    __bf16* S0 = reinterpret_cast<__bf16*>(smem);  // [2][kSBuf]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wi = w >> 1, wj = w & 1;
    const int colw = wj * 4 * 32;
    const int64_t cw = c0 + colw;
    const int64_t c_end = c0 + kRestCols;
    // wave-uniform base and 32-bit element offsets (at most 31 d_in + 127)
    float* __restrict__ wbase = Wk + (r0 + wi * 32) * d_in + cw;
    const int di = (int)d_in;
    // offsets formed at each use from an opaque copy of the lane index, so
    // that the 64 addresses are not kept live from the loads to the stores
    auto woff = [&](int q, int v) {
        int l = lane;
        asm volatile("" : "+v"(l));
        return (unsigned)(acc32_row(v, l) * di + 32 * q + (l & 31));
    };

    float16v acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = (float16v){};
    float e[2][4];
    bf16x8 u[2][3];
    rest_split_fetch(e[0], u[0], E, U3b, ldk, d_out, d_in, r0, c0, c_end, kMaxBlock, 0, tid, vec);
    __builtin_amdgcn_sched_barrier(0);
    rest_split_fetch(e[1], u[1], E, U3b, ldk, d_out, d_in, r0, c0, c_end, kMaxBlock, kSK, tid, vec);
    float wold[4][16];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        __bf16* S = S0 + (c & 1) * kSBuf;
        rest_split_stash(e[c & 1], u[c & 1], S, tid);
        __syncthreads();
        if (c + 2 < kChunks)
            rest_split_fetch(e[c & 1], u[c & 1], E, U3b, ldk, d_out, d_in, r0, c0, c_end, kMaxBlock,
                             (c + 2) * kSK, tid, vec);
        if (c >= kChunks - 2) {
            // half of the old W tile: pieces 2 (c - 6) and 2 (c - 6) + 1
#pragma unroll
            for (int q = 2 * (c - (kChunks - 2)); q < 2 * (c - (kChunks - 2)) + 2; ++q)
#pragma unroll
                for (int v = 0; v < 16; ++v) wold[q][v] = wbase[woff(q, v)];
        }
        rest_split_chunk<4>(S, wi, colw, lane, acc);
        __builtin_amdgcn_sched_barrier(0);  // keep each chunk's work inside its own iteration
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int v = 0; v < 16; ++v) wbase[woff(q, v)] = wold[q][v] - acc[q][v];
}

__device__ __forceinline__ void rest_split_body(unsigned char* smem, int64_t r0, int64_t c0, int64_t c_end,
                                                float* __restrict__ Wk, int64_t d_out, int64_t d_in,
                                                const float* __restrict__ E,
                                                const __bf16* __restrict__ U3b, int64_t ldk, int kp, bool vec) {
    __bf16* S0 = reinterpret_cast<__bf16*>(smem);  // [2][kSBuf]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wi = w >> 1, wj = w & 1;
    const int nchunks = (kp + kSK - 1) / kSK;
    const int ns = (int)((c_end - c0 + kStrip - 1) / kStrip);
    const int colw = wj * ns * 32;
    const int64_t cw = c0 + colw;
    const int nq = (int)std::min<int64_t>(ns, std::max<int64_t>(0, (c_end - cw + 31) / 32));
    const bool inner = (r0 + kRestRows <= d_out) && (cw + 32 * nq <= c_end);
    if (kp == kMaxBlock && nq == 4 && inner && c_end - c0 == kRestCols) {
        rest_split_body_full(smem, r0, c0, Wk, d_out, d_in, E, U3b, ldk, vec);
        return;
    }

    float16v acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = (float16v){};
    float e[4];
    bf16x8 u[3];
    rest_split_fetch(e, u, E, U3b, ldk, d_out, d_in, r0, c0, c_end, kp, 0, tid, vec);
    float wold[4][16];
    for (int c = 0; c < nchunks; ++c) {
        __bf16* S = S0 + (c & 1) * kSBuf;
        rest_split_stash(e, u, S, tid);
        __syncthreads();
        if (c + 1 < nchunks)
            rest_split_fetch(e, u, E, U3b, ldk, d_out, d_in, r0, c0, c_end, kp, (c + 1) * kSK, tid, vec);
        if (c == 0) {
            // the old W tile, behind the next chunk's operands; addresses
            // outside the sub-tile are clamped to its first element (never
            // stored)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (q < nq) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int64_t row = r0 + wi * 32 + acc32_row(v, lane);
                        const int64_t col = cw + 32 * q + (lane & 31);
                        const bool ok = row < d_out && col < c_end;
                        wold[q][v] = Wk[ok ? row * d_in + col : r0 * d_in + c0];
                    }
                }
        }
        switch (nq) {
            case 4: rest_split_chunk<4>(S, wi, colw, lane, acc); break;
            case 3: rest_split_chunk<3>(S, wi, colw, lane, acc); break;
            case 2: rest_split_chunk<2>(S, wi, colw, lane, acc); break;
            case 1: rest_split_chunk<1>(S, wi, colw, lane, acc); break;
            default: break;
        }
    }
    if (nchunks == 0) return;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (q < nq) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = r0 + wi * 32 + acc32_row(v, lane);
                const int64_t col = cw + 32 * q + (lane & 31);
                if (inner || (row < d_out && col < c_end)) Wk[row * d_in + col] = wold[q][v] - acc[q][v];
            }
        }
}

// The far update of one launch is split into units of 128 rows x 64
// columns (unit u: row tile u / nstrip, strip u % nstrip of the columns
// [c_begin, d_in)), dealt out as contiguous ranges: the sweeping workgroups
// take `per_sweep` units each after their sweep, the far-only workgroups
// share the rest evenly.  With one workgroup per CU every range starts at
// once, so the launch ends when the longest range does.
using sched::FarSplit;

template <bool kSplit>
__device__ __forceinline__ void far_range(unsigned char* smem, int64_t u0, int64_t u1, const FarSplit& fs,
                                          float* __restrict__ Wk, int64_t d_out, int64_t d_in,
                                          const float* __restrict__ E, const float* __restrict__ U,
                                          const __bf16* __restrict__ U3b, int64_t ldk, int64_t bp0, int kp,
                                          bool vec) {
    for (int64_t u = u0; u < u1;) {
        const sched::FarSub t = sched::far_sub(fs, u, u1, d_in);
        __syncthreads();  // the LDS stages of the previous sub-tile (or the sweep) are free again
        if (kSplit)
            rest_split_body(smem, t.rt * kRestRows, t.c0, t.c_end, Wk, d_out, d_in, E, U3b, ldk, kp, vec);
        else
            rest_body(smem, t.rt * kRestRows, t.c0, t.c_end, Wk, d_out, d_in, E, U, bp0, kp, vec);
        u += t.ns;
    }
}

// One launch per lazy block [b0, b1): workgroups 0 .. row_tiles-1 sweep the
// block (after the near update by the previous block's errors when kp > 0),
// then take their share of the previous block's update of the columns from
// b1 on; the other workgroups do only that update.  The two parts touch
// disjoint columns of W and different error buffers, so nothing but the
// launch order separates the blocks.  In the first block's launch of the
// split path (split_wgs > 0), which has no update, split_wgs workgroups
// after the sweeping ones form the bf16 pieces of U (U3w) instead; they are
// first read by the next launch.
template <bool kAllFull, bool kSplit>
__global__ __launch_bounds__(512) void step_kernel(float* __restrict__ Wk, int64_t d_out, int64_t d_in,
                                                   const float* __restrict__ U, const float* __restrict__ rdiag,
                                                   int64_t b0, int64_t b1, int bits, int64_t group, int64_t ng,
                                                   float* __restrict__ scales, int32_t* __restrict__ zeros,
                                                   float* __restrict__ minmax, uint8_t* __restrict__ codes,
                                                   float* __restrict__ E, float* __restrict__ err_row,
                                                   const float* __restrict__ Ep, int64_t bp0, int kp, int row_tiles,
                                                   FarSplit fs, int vec_rest, const __bf16* __restrict__ U3b,
                                                   int64_t ldk, __bf16* __restrict__ U3w, int split_wgs) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int b = (int)blockIdx.x;
    if (kSplit && split_wgs > 0 && b >= row_tiles) {
        float(*T)[kSplitCols + 1] = reinterpret_cast<float(*)[kSplitCols + 1]>(smem);
        const int64_t n = split_items(d_in, b1 - b0);
        for (int64_t i = b - row_tiles; i < n; i += split_wgs) split_u_item<512>(T, U, d_in, b1 - b0, ldk, U3w, i);
        return;
    }
    if (b < row_tiles)
        sweep_body<kAllFull, kSplit>(smem, b, Wk, d_out, d_in, U, rdiag, b0, b1, bits, group, ng, scales, zeros,
                                     minmax, codes, E, err_row, Ep, bp0, kp, U3b, ldk);
    int64_t u0, u1;
    sched::far_units(fs, b, row_tiles, u0, u1);
    if (u1 > u0) far_range<kSplit>(smem, u0, u1, fs, Wk, d_out, d_in, Ep, U, U3b, ldk, bp0, kp, vec_rest != 0);
}

}  // namespace

namespace {
// The step kernel's dynamic LDS limit, raised once per device to the largest
// size asked for so far (the attribute is per device).
hipError_t allow_step_lds(size_t bytes) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static size_t allowed[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (allowed[dev] >= bytes) return hipSuccess;
    const void* fns[4] = {reinterpret_cast<const void*>(&step_kernel<true, false>),
                          reinterpret_cast<const void*>(&step_kernel<false, false>),
                          reinterpret_cast<const void*>(&step_kernel<true, true>),
                          reinterpret_cast<const void*>(&step_kernel<false, true>)};
    for (const void* f : fns) {
        e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
        if (e != hipSuccess) return e;
    }
    allowed[dev] = bytes;
    return e;
}
}  // namespace

size_t quant_workspace_bytes(int64_t d_out, int64_t d_in, int64_t block, int split) {
    return (size_t)(rup(d_out * d_in * 4, 256) + 2 * rup(d_out * split_ldk(block) * 4, 256) + rup(d_in * 4, 256) +
                    (split ? rup(split_u_elems(d_in, block) * 2, 256) : 0));
}

hipError_t launch_quantize(const void* W, int w_is_f16, int64_t d_out, int64_t d_in, const float* U,
                           const uint8_t* dead, int bits, int64_t group, int64_t block, uint8_t* codes,
                           float* scales, int32_t* zeros, float* err_row, float* minmax, void* ws, int split,
                           hipStream_t s) {
    if (d_out == 0 || d_in == 0) return hipSuccess;
    QuantWs w = carve(ws, d_out, d_in, block);
    const int64_t ng = group ? d_in / group : 1;
    const float maxq = (float)((1 << bits) - 1);
    const unsigned rows4 = (unsigned)((d_out + 3) / 4);
    {
        // the working copy, and for per-row grids the grid, in one pass over W
        // (with 1/U_jj and the cleared error sums)
        TimedLaunch t(K_Q_CONVERT, s);
        const uintptr_t wa = reinterpret_cast<uintptr_t>(W), da = reinterpret_cast<uintptr_t>(dead);
        const bool vec = (d_in % 8 == 0) && (wa % 16 == 0) && (da % 8 == 0);
        const dim3 grid(rows4), blk(256);
#define GC_LAUNCH(T, V, G)                                                                                    \
    do {                                                                                                      \
        if (dead)                                                                                             \
            GPTQ_LAUNCH(t, (grid_convert_kernel<T, V, G, true>), grid, blk, 0, s, static_cast<const T*>(W), \
                               w.Wk, d_out, d_in, dead, maxq, scales, zeros, minmax, U, w.rdiag, err_row);      \
        else                                                                                                  \
            GPTQ_LAUNCH(t, (grid_convert_kernel<T, V, G, false>), grid, blk, 0, s, static_cast<const T*>(W), \
                               w.Wk, d_out, d_in, dead, maxq, scales, zeros, minmax, U, w.rdiag, err_row);      \
    } while (0)
        if (w_is_f16) {
            if (group == 0) {
                if (vec) GC_LAUNCH(half_t, true, true);
                else GC_LAUNCH(half_t, false, true);
            } else {
                if (vec) GC_LAUNCH(half_t, true, false);
                else GC_LAUNCH(half_t, false, false);
            }
        } else {
            if (group == 0) {
                if (vec) GC_LAUNCH(float, true, true);
                else GC_LAUNCH(float, false, true);
            } else {
                if (vec) GC_LAUNCH(float, true, false);
                else GC_LAUNCH(float, false, false);
            }
        }
#undef GC_LAUNCH
    }
    const bool vec = (reinterpret_cast<uintptr_t>(U) % 16 == 0) && (d_in % 4 == 0) && (block % 4 == 0);  // E rows are 16-byte aligned when block % 4 == 0
    const int64_t ldk = split_ldk(block);
    const int bmax = (int)std::min(block, d_in);
    const size_t near_bytes = near_lds_bytes(bmax, split);
    const size_t rest_bytes = split ? rest_split_lds_bytes() : rest_lds_bytes();
    const size_t ldsmax = std::max(sweep_lds_bytes(bmax) + near_bytes, rest_bytes);
    if (ldsmax > 64 * 1024) {
        hipError_t e = allow_step_lds(ldsmax);
        if (e != hipSuccess) return e;
    }
    const int row_tiles = (int)((d_out + kRowsPerWg - 1) / kRowsPerWg);
    const int rest_rows = (int)((d_out + kRestRows - 1) / kRestRows);
    const int n_cu = device_cu_count();
    if (n_cu <= 0) return hipErrorInvalidDevice;
    hipError_t err = hipSuccess;
    // One launch per lazy block on the caller's stream: the sweep of block b
    // (its columns first receive block b-1's update, in registers) and, in
    // the same launch, block b-1's update of every column from b1 on.  A
    // group wider than the block needs its columns fully updated before its
    // grid is formed: at such a group start the previous block's update of
    // the columns from b0 on runs as its own launch first.
    int bi = 0;
    for (int64_t b0 = 0; b0 < d_in; b0 += block, ++bi) {
        const int64_t b1 = std::min(b0 + block, d_in);
        const int bw = (int)(b1 - b0);
        const int nw = (bw + kSub - 1) / kSub;
        float* Eb = w.E[bi & 1];
        const float* Ep = bi > 0 ? w.E[(bi - 1) & 1] : nullptr;
        const int64_t bp0 = b0 - block;
        int kp = bi > 0 ? (int)block : 0;
        // the previous block's U pieces (split path only)
        const __bf16* U3b = (split && bi > 0) ? w.U3 + (int64_t)(bi - 1) * 3 * d_in * ldk : nullptr;
        if (group > block && b0 % group == 0) {
            if (kp > 0) {
                TimedLaunch t(K_Q_TRAIL, s);
                dim3 grid((unsigned)((d_in - b0 + kTT - 1) / kTT), (unsigned)((d_out + kTrailRows - 1) / kTrailRows));
                if (vec)
                    GPTQ_LAUNCH(t, (trail_kernel<true, kTrailRows>), grid, dim3(256), 0, s, w.Wk, d_out, d_in, Ep,
                                       U, bp0, b0, b0, d_in);
                else
                    GPTQ_LAUNCH(t, (trail_kernel<false, kTrailRows>), grid, dim3(256), 0, s, w.Wk, d_out, d_in, Ep,
                                       U, bp0, b0, b0, d_in);
                kp = 0;
            }
            TimedLaunch t(K_Q_GROUPGRID, s);
            GPTQ_LAUNCH(t, group_grid_kernel, dim3(rows4), dim3(256), 0, s, (const float*)w.Wk, d_out, d_in, b0,
                               group, b0 / group, ng, maxq, scales, zeros, minmax);
        }
        FarSplit fs;
        fs.c_begin = b1;
        fs.nstrip = (int)((d_in - b1 + kStrip - 1) / kStrip);
        const int64_t n_units = (kp > 0 && b1 < d_in) ? (int64_t)rest_rows * fs.nstrip : 0;
        const int n_far =
            sched::far_split(n_units, row_tiles, n_cu, fs, split ? sched::kSweepUnits : sched::kSweepUnitsF32);
        size_t lds = sweep_lds_bytes(bw) + near_lds_bytes(kp, split);
        if (n_units > 0) lds = std::max(lds, rest_bytes);
        // the bf16 pieces of every block's rows of U (split path), once per
        // layer, by the CUs the first block's sweep leaves free
        const int split_wgs = (split && bi == 0 && d_in > block) ? std::max(n_cu - row_tiles, 32) : 0;
        if (split_wgs > 0) lds = std::max(lds, (size_t)kMaxBlock * (kSplitCols + 1) * 4);
        TimedLaunch t(K_Q_STEP, s);
        const dim3 grid((unsigned)(row_tiles + n_far + split_wgs));
#define STEP_LAUNCH(FULL, SPLIT)                                                                             \
    GPTQ_LAUNCH(t, (step_kernel<FULL, SPLIT>), grid, dim3(512), lds, s, w.Wk, d_out, d_in, U,              \
                       (const float*)w.rdiag, b0, b1, bits, group, ng, scales, zeros, minmax, codes, Eb, \
                       err_row, Ep, bp0, kp, row_tiles, fs, (int)vec, U3b, ldk, w.U3, split_wgs)
        if (bw % kSub == 0) {
            if (split) STEP_LAUNCH(true, true);
            else STEP_LAUNCH(true, false);
        } else {
            if (split) STEP_LAUNCH(false, true);
            else STEP_LAUNCH(false, false);
        }
#undef STEP_LAUNCH
    }
    (void)err;
    return hipGetLastError();
}

}  // namespace gptq
