// Shared device helpers for the gfx950 (CDNA4) kernels: vector types, MFMA
// wrappers, wave reductions and launch bookkeeping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gptq {

typedef _Float16 half_t;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef double double4v __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// MFMA wrappers.  Operand layouts (wave64, lane l):
//   32x32xK (f16 K=16, f32 K=2): A[i][k] from lane i + 32*kg, B[k][j] from
//     lane j + 32*kg, with kg = l / 32 selecting the k group; result lane l
//     holds C[8*(v/4) + 4*(l/32) + (v%4)][l % 32] for v = 0..15.
//   16x16x4 f64: A[i][k] from lane i + 16*k, B[k][j] from lane j + 16*k;
//     result lane l holds C[4*v + l/16][l % 16] for v = 0..3 (measured on
//     gfx950; rows interleave across the four lane groups).
//   16x16x4 f32: same operand map; result lane l holds C[4*(l/16) + v][l % 16]
//     (measured on gfx950: the f32 and f64 variants differ).
// The k order inside a group is the hardware's; a product A B^T of two
// operands loaded with the same lane->k map is independent of it.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float16v mfma32x32x16_f16(half8 a, half8 b, float16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float16v mfma32x32x2_f32(float a, float b, float16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4v mfma16x16x4_f32(float a, float b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ double4v mfma16x16x4_f64(double a, double b, double4v c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// row index of accumulator element v of a 32x32 MFMA result in lane l
__device__ __forceinline__ int acc32_row(int v, int lane) {
    return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

// ---------------------------------------------------------------------------
// Wave-wide reductions over 64 lanes (butterfly with __shfl_xor)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// wave index as a scalar (uniform) value
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// ---------------------------------------------------------------------------
// Asymmetric min-max grid, IEEE float32 op sequence (only subtraction,
// division and rint: nothing a compiler could contract).
//   mn = min(0, lo), mx = max(0, hi); an all-zero range becomes [-1, 1];
//   s = fl32(fl32(mx - mn) / maxq); z = clamp(rint(fl32(-mn / s)), 0, maxq)
// ---------------------------------------------------------------------------
struct Grid {
    float s;
    float z;
};

__device__ __forceinline__ Grid make_grid(float lo, float hi, float maxq) {
    float mn = fminf(lo, 0.0f);
    float mx = fmaxf(hi, 0.0f);
    if (mn == 0.0f && mx == 0.0f) {
        mn = -1.0f;
        mx = 1.0f;
    }
    float range = mx - mn;
    Grid g;
    g.s = range / maxq;
    float zz = __builtin_rintf((-mn) / g.s);
    g.z = fminf(fmaxf(zz, 0.0f), maxq);
    return g;
}

}  // namespace gptq
