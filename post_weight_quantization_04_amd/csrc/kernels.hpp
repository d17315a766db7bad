// Host-side launchers of the gfx950 kernels (one translation unit per stage)
// and the kernel-timing hook shared by them.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace gptq {

enum KernelId {
    K_HESS_F16 = 0,
    K_HESS_F32,
    K_HINV_LOAD,
    K_CHOL_STEP,
    K_HINV_STORE,
    K_Q_CONVERT,
    K_Q_GROUPGRID,
    K_Q_STEP,
    K_Q_TRAIL,
    K_PACK,
    K_DEQUANT,
    K_OUTERR,
    K_OBQ_HINV,
    K_OBQ_ROWS,
    K_PROPAGATE,
    K_HINV32_LOAD,
    K_CHOL32_STEP,
    K_HINV32_STORE,
    K_COUNT
};

// Kernel id of the launches in its scope, for the timing hook (see
// gptq_timing_enable).  Every launch goes through GPTQ_LAUNCH, which, while
// timing is enabled for that id, has the dispatch itself stamp a fresh HIP
// event pair with the kernel's start and end (no marker packets between the
// launches, so timed launches keep their spacing); a plain launch otherwise.
struct TimedLaunch {
    TimedLaunch(int kernel_id, hipStream_t) : id(kernel_id) {}
    int id;
};
struct LaunchEvents {
    explicit LaunchEvents(int id);
    hipEvent_t a = nullptr, b = nullptr;
};
#define GPTQ_LAUNCH(t, kernel, grid, block, shmem, stream, ...)                                        \
    do {                                                                                             \
        const ::gptq::LaunchEvents gptq_ev_((t).id);                                                 \
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, gptq_ev_.a, gptq_ev_.b, 0u, __VA_ARGS__); \
    } while (0)

// While alive, launches record no events on this thread (the timing hook
// creates HIP events, which entry points that must not allocate avoid).
struct TimingOff {
    TimingOff();
    ~TimingOff();
    bool prev;
};

// Compute units of the current device, queried once per device (0 on error).
int device_cu_count();

// ---- stage 1 ---------------------------------------------------------------
// nchunks token chunks Xs[0..nchunks) of ntok tokens each, one row stride;
// set: the first chunk writes H instead of adding into it.
hipError_t launch_hessian(float* H, int64_t n, const void* const* Xs, int64_t nchunks, int x_is_f16, int64_t ntok,
                          int64_t ldx, int set, hipStream_t s);

// ---- stages 2 + 3 ----------------------------------------------------------
constexpr int kCholNB = 64;  // panel width of the blocked factorization
size_t hinv_workspace_bytes(int64_t n);
hipError_t launch_prepare_hinv(const float* H, int64_t n, double damp_frac, float* U, uint8_t* dead,
                               int32_t* info, double* lambda_out, void* ws, hipStream_t s);
// Largest order the no-allocation entry point takes, its fixed scratch size,
// and the scratch's device address on the current device.
constexpr int64_t kNoAllocMaxDin = 4096;
size_t hinv_noalloc_scratch_bytes();
hipError_t hinv_noalloc_scratch(void** out);

// The same stages with float32 tiles and MFMA f32 products.
size_t hinv32_workspace_bytes(int64_t n);
hipError_t launch_prepare_hinv32(const float* H, int64_t n, double damp_frac, float* U, uint8_t* dead,
                                 int32_t* info, double* lambda_out, void* ws, hipStream_t s);

// ---- stage 4 ---------------------------------------------------------------
size_t quant_workspace_bytes(int64_t d_out, int64_t d_in, int64_t block, int split);
hipError_t launch_quantize(const void* W, int w_is_f16, int64_t d_out, int64_t d_in, const float* U,
                           const uint8_t* dead, int bits, int64_t group, int64_t block,
                           uint8_t* codes, float* scales, int32_t* zeros, float* err_row,
                           float* minmax, void* ws, int split, hipStream_t s);

// ---- few-bit storage, dequantization, output error ---------------------------
int64_t packed_words(int64_t d_in, int bits);
hipError_t launch_pack(const uint8_t* codes, int64_t d_out, int64_t d_in, int bits, uint32_t* packed,
                       hipStream_t s);
hipError_t launch_dequant(const uint32_t* packed, int bits, int64_t d_out, int64_t d_in, const float* scales,
                          const int32_t* zeros, int64_t group, void* out, int out_is_f16, hipStream_t s);
hipError_t launch_output_error(const void* W, int w_is_f16, const uint8_t* dead, const uint32_t* packed, int bits,
                               const float* scales, const int32_t* zeros, int64_t group, int64_t d_out,
                               int64_t d_in, const float* err_row, const double* lambda, float* out,
                               hipStream_t s);

// ---- greedy-order variant (small layers) -------------------------------------
size_t obq_workspace_bytes(int64_t d_in);
hipError_t launch_obq(const void* W, int w_is_f16, int64_t d_out, int64_t d_in, const float* U, const uint8_t* dead,
                      int bits, uint8_t* codes, float* scales, int32_t* zeros, int32_t* order, double* loss,
                      void* ws, hipStream_t s);

// ---- propagation to the next layer ------------------------------------------
hipError_t launch_propagate(const void* W, int64_t d_out, int64_t d_in, const void* X, int64_t ntok, int64_t ldx,
                            void* Y, int64_t ldy, int relu, hipStream_t s);

}  // namespace gptq
