// Few-bit storage of the codes, dequantization, and the per-row output error
// from the loss identity (aicassindra.com "tm_gptq_math", "Post-training
// quantization and the per-layer objective": weights lowered to low-bit
// integers, 4-bit the example given; "The
// reconstruction objective, written out" with the damped Hessian of "The
// Cholesky trick for the inverse Hessian").
//
// Storage: each row's codes form one little-endian bit stream, code j in
// bits [j bits, (j+1) bits), least significant bit first, cut into 32-bit
// words (nw = ceil(d_in bits / 32) per row, the last zero-padded).  A code
// may straddle two words when bits does not divide 32.
//
// All three kernels stream memory once (HBM-bound): one thread per output
// word (packing), per eight output weights (dequantization), one workgroup
// per row (output error); rows run along the grid's y dimension.
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

// codes j0 .. j0+7 of a packed row (j0 a multiple of 8): the bits
// [j0 bits, (j0+8) bits) of the stream, read as up to three words (codes
// past the row's end come out as garbage and are not used)
__device__ __forceinline__ void codes8(const uint32_t* __restrict__ prow, int nw, int j0, int bits, uint32_t (&q)[8]) {
    const int t0 = j0 * bits;
    const int w = t0 >> 5, sh = t0 & 31;
    const uint32_t w0 = prow[w];
    const uint32_t w1 = (w + 1 < nw) ? prow[w + 1] : 0u;
    const uint32_t w2 = (w + 2 < nw) ? prow[w + 2] : 0u;
    const uint64_t lo = (uint64_t)w0 | ((uint64_t)w1 << 32);
    const uint64_t hi = (uint64_t)w1 | ((uint64_t)w2 << 32);
    const uint32_t mask = (1u << bits) - 1u;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int bit = sh + c * bits;
        q[c] = (uint32_t)((bit < 32 ? lo >> bit : hi >> (bit - 32))) & mask;
    }
}

// one thread per output word, blockIdx.y = row (no 64-bit division)
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* __restrict__ codes, int d_in, int bits,
                                                         int nw, uint32_t* __restrict__ packed) {
    const int w = blockIdx.x * blockDim.x + threadIdx.x;
    if (w >= nw) return;
    const int64_t r = blockIdx.y;
    const uint32_t mask = (1u << bits) - 1u;
    const int b0 = 32 * w;                  // first bit of the word
    const int j0 = b0 / bits;               // first code touching it
    const int j1 = min((b0 + 31) / bits, d_in - 1);
    const uint8_t* crow = codes + r * d_in;
    uint32_t word = 0;
    for (int j = j0; j <= j1; ++j) {
        const uint32_t c = crow[j] & mask;
        const int sh = j * bits - b0;       // negative: the code began in the word before
        word |= (sh >= 0) ? (c << sh) : (c >> (-sh));
    }
    packed[r * nw + w] = word;
}

// Eight consecutive outputs per thread (blockIdx.y = row): their codes are
// the bits [8 j0 bits, 8 (j0+8) bits) of the row stream, read as up to
// three words; stored as one 16-byte (fp16) or two 16-byte (fp32) pieces
// when the row is aligned for it.
template <typename T>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ packed, int bits, int nw, int d_in,
                                                      const float* __restrict__ scales,
                                                      const int32_t* __restrict__ zeros, int group, int ng,
                                                      T* __restrict__ out) {
    const int j0 = 8 * (blockIdx.x * blockDim.x + threadIdx.x);
    if (j0 >= d_in) return;
    const int64_t r = blockIdx.y;
    uint32_t q8[8];
    codes8(packed + r * nw, nw, j0, bits, q8);
    T v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t q = q8[c];
        const int j = min(j0 + c, d_in - 1);
        const int g = group ? j / group : 0;
        const float s = scales[r * ng + g];
        const int32_t z = zeros[r * ng + g];
        // one rounding of the exact product to T: q - z is exact in fp32, and
        // for an fp16 T the multiply and the narrowing fuse into one
        // mixed-precision multiply (v_fma_mix) with a single rounding
        v[c] = (T)(s * (float)((int32_t)q - z));
    }
    T* orow = out + r * d_in;
    if (j0 + 8 <= d_in && (d_in % 8) == 0) {
        uint32_t u[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            if constexpr (sizeof(T) == 2) u[c] = (uint32_t)__builtin_bit_cast(uint16_t, v[c]);
            else u[c] = __builtin_bit_cast(uint32_t, v[c]);
        }
        uint4* dst = reinterpret_cast<uint4*>(orow + j0);
        if constexpr (sizeof(T) == 2) {
            dst[0] = make_uint4(u[0] | (u[1] << 16), u[2] | (u[3] << 16), u[4] | (u[5] << 16), u[6] | (u[7] << 16));
        } else {
            dst[0] = make_uint4(u[0], u[1], u[2], u[3]);
            dst[1] = make_uint4(u[4], u[5], u[6], u[7]);
        }
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c)
            if (j0 + c < d_in) orow[j0 + c] = v[c];
    }
}

// out[r] = (err_row[r] - lambda ||dw_r||^2) / 2 with dw = W0 - What, W0 the
// weights with dead columns zeroed; the squares are summed in fp64.  One
// workgroup per row, eight consecutive columns per thread and step.
template <typename T>
__global__ __launch_bounds__(256) void output_error_kernel(const T* __restrict__ W, const uint8_t* __restrict__ dead,
                                                           const uint32_t* __restrict__ packed, int bits, int nw,
                                                           int d_in, const float* __restrict__ scales,
                                                           const int32_t* __restrict__ zeros, int group, int ng,
                                                           const float* __restrict__ err_row,
                                                           const double* __restrict__ lambda,
                                                           float* __restrict__ out) {
    __shared__ double part[4];
    const int64_t r = blockIdx.x;
    const T* wrow = W + r * d_in;
    const uint32_t* prow = packed + r * nw;
    const bool aligned = (d_in % 8) == 0;
    double acc = 0.0;
    for (int j0 = 8 * threadIdx.x; j0 < d_in; j0 += 8 * blockDim.x) {
        uint32_t q8[8];
        codes8(prow, nw, j0, bits, q8);
        float w8[8];
        if (aligned) {  // the row's eight weights as one (fp16) or two (fp32) 16-byte loads
            const uint4* src = reinterpret_cast<const uint4*>(wrow + j0);
            if constexpr (sizeof(T) == 2) {
                const uint4 a = src[0];
                const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    w8[2 * c] = (float)__builtin_bit_cast(T, (uint16_t)(u[c] & 0xffffu));
                    w8[2 * c + 1] = (float)__builtin_bit_cast(T, (uint16_t)(u[c] >> 16));
                }
            } else {
                const uint4 a = src[0], b = src[1];
                const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                for (int c = 0; c < 8; ++c) w8[c] = __builtin_bit_cast(float, u[c]);
            }
        } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) w8[c] = (j0 + c < d_in) ? (float)wrow[j0 + c] : 0.0f;
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int j = j0 + c;
            if (j < d_in) {
                const float w = (dead && dead[j]) ? 0.0f : w8[c];
                const int g = group ? j / group : 0;
                const float wh = scales[r * ng + g] * (float)((int32_t)q8[c] - zeros[r * ng + g]);
                const double d = (double)w - (double)wh;
                acc += d * d;
            }
        }
    }
    acc = wave_sum(acc);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        const double dw2 = part[0] + part[1] + part[2] + part[3];
        out[r] = (float)(((double)err_row[r] - lambda[0] * dw2) * 0.5);
    }
}

}  // namespace

int64_t packed_words(int64_t d_in, int bits) { return (d_in * bits + 31) / 32; }

hipError_t launch_pack(const uint8_t* codes, int64_t d_out, int64_t d_in, int bits, uint32_t* packed, hipStream_t s) {
    const int64_t nw = packed_words(d_in, bits);
    TimedLaunch t(K_PACK, s);
    for (int64_t r0 = 0; r0 < d_out; r0 += 65535) {  // grid y is at most 65535 rows per launch
        const unsigned rows = (unsigned)std::min<int64_t>(65535, d_out - r0);
        GPTQ_LAUNCH(t, pack_codes_kernel, dim3((unsigned)((nw + 255) / 256), rows), dim3(256), 0, s,
                           codes + r0 * d_in, (int)d_in, bits, (int)nw, packed + r0 * nw);
    }
    return hipGetLastError();
}

hipError_t launch_dequant(const uint32_t* packed, int bits, int64_t d_out, int64_t d_in, const float* scales,
                          const int32_t* zeros, int64_t group, void* out, int out_is_f16, hipStream_t s) {
    const int64_t nw = packed_words(d_in, bits);
    const int64_t ng = group ? d_in / group : 1;
    TimedLaunch t(K_DEQUANT, s);
    const unsigned gx = (unsigned)((d_in + 8 * 256 - 1) / (8 * 256));
    for (int64_t r0 = 0; r0 < d_out; r0 += 65535) {
        const unsigned rows = (unsigned)std::min<int64_t>(65535, d_out - r0);
        if (out_is_f16)
            GPTQ_LAUNCH(t, dequant_kernel<half_t>, dim3(gx, rows), dim3(256), 0, s, packed + r0 * nw, bits,
                               (int)nw, (int)d_in, scales + r0 * ng, zeros + r0 * ng, (int)group, (int)ng,
                               static_cast<half_t*>(out) + r0 * d_in);
        else
            GPTQ_LAUNCH(t, dequant_kernel<float>, dim3(gx, rows), dim3(256), 0, s, packed + r0 * nw, bits,
                               (int)nw, (int)d_in, scales + r0 * ng, zeros + r0 * ng, (int)group, (int)ng,
                               static_cast<float*>(out) + r0 * d_in);
    }
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
        GPTQ_LAUNCH(t, output_error_kernel<half_t>, dim3((unsigned)d_out), dim3(256), 0, s,
                           static_cast<const half_t*>(W), dead, packed, bits, (int)nw, (int)d_in, scales, zeros,
                           (int)group, (int)ng, err_row, lambda, out);
    else
        GPTQ_LAUNCH(t, output_error_kernel<float>, dim3((unsigned)d_out), dim3(256), 0, s,
                           static_cast<const float*>(W), dead, packed, bits, (int)nw, (int)d_in, scales, zeros,
                           (int)group, (int)ng, err_row, lambda, out);
    return hipGetLastError();
}

}  // namespace gptq
