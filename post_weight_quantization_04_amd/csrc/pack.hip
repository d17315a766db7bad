// Few-bit storage of the codes, dequantization, and the per-row output error
// from the loss identity (aicassindra.com "tm_gptq_math", "Post-training
// quantization in one paragraph": weights kept as few-bit integers; "The
// reconstruction objective, written out" with the damped Hessian of "The
// Cholesky trick for the inverse Hessian").
//
// Storage: each row's codes form one little-endian bit stream, code j in
// bits [j bits, (j+1) bits), least significant bit first, cut into 32-bit
// words (nw = ceil(d_in bits / 32) per row, the last zero-padded).  A code
// may straddle two words when bits does not divide 32.
//
// All three kernels stream memory once (HBM-bound): one thread per output
// word (packing), per output weight (dequantization), one workgroup per row
// (output error).
#include "common.hpp"
#include "kernels.hpp"

namespace gptq {

namespace {

// code j of a packed row
__device__ __forceinline__ uint32_t code_at(const uint32_t* __restrict__ row, int64_t j, int bits) {
    const int64_t t = j * bits;
    const int64_t w = t >> 5;
    const int sh = (int)(t & 31);
    uint32_t v = row[w] >> sh;
    if (sh + bits > 32) v |= row[w + 1] << (32 - sh);
    return v & ((1u << bits) - 1u);
}

__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* __restrict__ codes, int64_t d_out,
                                                         int64_t d_in, int bits, int64_t nw,
                                                         uint32_t* __restrict__ packed) {
    const uint32_t mask = (1u << bits) - 1u;
    const int64_t total = d_out * nw;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = idx / nw, w = idx - r * nw;
        const int64_t b0 = 32 * w;                  // first bit of the word
        const int64_t j0 = b0 / bits;               // first code touching it
        const int64_t j1 = min((b0 + 31) / bits, d_in - 1);
        const uint8_t* crow = codes + r * d_in;
        uint32_t word = 0;
        for (int64_t j = j0; j <= j1; ++j) {
            const uint32_t c = crow[j] & mask;
            const int64_t sh = j * bits - b0;       // negative: the code began in the word before
            word |= (sh >= 0) ? (c << sh) : (c >> (-sh));
        }
        packed[idx] = word;
    }
}

template <typename T>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ packed, int bits, int64_t nw,
                                                      int64_t d_out, int64_t d_in,
                                                      const float* __restrict__ scales,
                                                      const int32_t* __restrict__ zeros, int64_t group,
                                                      int64_t ng, T* __restrict__ out) {
    const int64_t total = d_out * d_in;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = idx / d_in, j = idx - r * d_in;
        const uint32_t q = code_at(packed + r * nw, j, bits);
        const int64_t g = group ? j / group : 0;
        const float s = scales[r * ng + g];
        const int32_t z = zeros[r * ng + g];
        // one rounding of the exact product to T: q - z is exact in fp32, and
        // for an fp16 T the multiply and the narrowing fuse into one
        // mixed-precision multiply (v_fma_mix) with a single rounding
        const float v = s * (float)((int32_t)q - z);
        out[idx] = (T)v;
    }
}

// out[r] = (err_row[r] - lambda ||dw_r||^2) / 2 with dw = W0 - What, W0 the
// weights with dead columns zeroed; the squares are summed in fp64.
template <typename T>
__global__ __launch_bounds__(256) void output_error_kernel(const T* __restrict__ W, const uint8_t* __restrict__ dead,
                                                           const uint32_t* __restrict__ packed, int bits,
                                                           int64_t nw, int64_t d_in,
                                                           const float* __restrict__ scales,
                                                           const int32_t* __restrict__ zeros, int64_t group,
                                                           int64_t ng, const float* __restrict__ err_row,
                                                           const double* __restrict__ lambda,
                                                           float* __restrict__ out) {
    __shared__ double part[4];
    const int64_t r = blockIdx.x;
    const T* wrow = W + r * d_in;
    const uint32_t* prow = packed + r * nw;
    double acc = 0.0;
    for (int64_t j = threadIdx.x; j < d_in; j += blockDim.x) {
        const float w = (dead && dead[j]) ? 0.0f : (float)wrow[j];
        const int64_t g = group ? j / group : 0;
        const float s = scales[r * ng + g];
        const int32_t z = zeros[r * ng + g];
        const float wh = s * (float)((int32_t)code_at(prow, j, bits) - z);
        const double d = (double)w - (double)wh;
        acc += d * d;
    }
    acc = wave_sum(acc);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        const double dw2 = part[0] + part[1] + part[2] + part[3];
        out[r] = (float)(((double)err_row[r] - lambda[0] * dw2) * 0.5);
    }
}

unsigned grid_for(int64_t total) {
    return (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
}

}  // namespace

int64_t packed_words(int64_t d_in, int bits) { return (d_in * bits + 31) / 32; }

hipError_t launch_pack(const uint8_t* codes, int64_t d_out, int64_t d_in, int bits, uint32_t* packed, hipStream_t s) {
    const int64_t nw = packed_words(d_in, bits);
    TimedLaunch t(K_PACK, s);
    hipLaunchKernelGGL(pack_codes_kernel, dim3(grid_for(d_out * nw)), dim3(256), 0, s, codes, d_out, d_in, bits, nw,
                       packed);
    return hipGetLastError();
}

hipError_t launch_dequant(const uint32_t* packed, int bits, int64_t d_out, int64_t d_in, const float* scales,
                          const int32_t* zeros, int64_t group, void* out, int out_is_f16, hipStream_t s) {
    const int64_t nw = packed_words(d_in, bits);
    const int64_t ng = group ? d_in / group : 1;
    TimedLaunch t(K_DEQUANT, s);
    if (out_is_f16)
        hipLaunchKernelGGL(dequant_kernel<half_t>, dim3(grid_for(d_out * d_in)), dim3(256), 0, s, packed, bits, nw,
                           d_out, d_in, scales, zeros, group, ng, static_cast<half_t*>(out));
    else
        hipLaunchKernelGGL(dequant_kernel<float>, dim3(grid_for(d_out * d_in)), dim3(256), 0, s, packed, bits, nw,
                           d_out, d_in, scales, zeros, group, ng, static_cast<float*>(out));
    return hipGetLastError();
}

hipError_t launch_output_error(const void* W, int w_is_f16, const uint8_t* dead, const uint32_t* packed, int bits,
                               const float* scales, const int32_t* zeros, int64_t group, int64_t d_out,
                               int64_t d_in, const float* err_row, const double* lambda, float* out,
                               hipStream_t s) {
    const int64_t nw = packed_words(d_in, bits);
    const int64_t ng = group ? d_in / group : 1;
    TimedLaunch t(K_OUTERR, s);
    if (w_is_f16)
        hipLaunchKernelGGL(output_error_kernel<half_t>, dim3((unsigned)d_out), dim3(256), 0, s,
                           static_cast<const half_t*>(W), dead, packed, bits, nw, d_in, scales, zeros, group, ng,
                           err_row, lambda, out);
    else
        hipLaunchKernelGGL(output_error_kernel<float>, dim3((unsigned)d_out), dim3(256), 0, s,
                           static_cast<const float*>(W), dead, packed, bits, nw, d_in, scales, zeros, group, ng,
                           err_row, lambda, out);
    return hipGetLastError();
}

}  // namespace gptq
