// C ABI entry points: argument validation (before any HIP call), workspace
// checks, launch sequencing on the caller's stream, and kernel timing.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/gptq.h"
#include "kernels.hpp"

namespace gptq {

// ---------------------------------------------------------------------------
// Kernel timing: host-side list of event pairs for the selected kernel id,
// one pair per launch, stamped by the dispatch (GPTQ_LAUNCH).
// ---------------------------------------------------------------------------
namespace {
const char* const kNames[K_COUNT] = {
    "hessian_f16", "hessian_f32", "hinv_load_reversed", "chol_step", "hinv_store_u",
    "q_grid_convert",         "q_group_grid",       "q_step",    "q_trail",
    "pack_codes",  "dequantize",  "output_error", "obq_hinv", "obq_rows", "propagate",
    "hinv32_load_reversed", "chol32_step", "hinv32_store_u",
};
// The timing state is process-wide; the mutex makes concurrent entry-point
// calls from several host threads safe, though the events then interleave.
std::mutex g_mu;
int g_timed = -1;
struct EventPair {
    hipEvent_t a, b;
};
std::vector<EventPair> g_pending;
std::vector<EventPair> g_free;
thread_local bool t_timing_off = false;
}  // namespace

TimingOff::TimingOff() : prev(t_timing_off) { t_timing_off = true; }
TimingOff::~TimingOff() { t_timing_off = prev; }

LaunchEvents::LaunchEvents(int id) {
    if (t_timing_off) return;
    std::lock_guard<std::mutex> lock(g_mu);
    if (id != g_timed) return;
    EventPair ep;
    if (!g_free.empty()) {
        ep = g_free.back();
        g_free.pop_back();
    } else {
        if (hipEventCreate(&ep.a) != hipSuccess) return;
        if (hipEventCreate(&ep.b) != hipSuccess) {
            (void)hipEventDestroy(ep.a);
            return;
        }
    }
    g_pending.push_back(ep);
    a = ep.a;
    b = ep.b;
}

int device_cu_count() {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static int count[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (count[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        count[dev] = n;
    }
    return count[dev];
}

}  // namespace gptq

using namespace gptq;

namespace {
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline int hip_status(hipError_t e) { return e == hipSuccess ? GPTQ_OK : GPTQ_EHIP; }
}  // namespace

extern "C" {

const char* gptq_status_string(int status) {
    switch (status) {
        case GPTQ_OK: return "GPTQ_OK";
        case GPTQ_EINVAL: return "GPTQ_EINVAL: invalid argument";
        case GPTQ_EUNSUPPORTED: return "GPTQ_EUNSUPPORTED: valid request not handled by these kernels";
        case GPTQ_EHIP: return "GPTQ_EHIP: HIP runtime or launch failure";
        case GPTQ_EWORKSPACE: return "GPTQ_EWORKSPACE: workspace missing or too small";
        case GPTQ_ESCRATCH:
            return "GPTQ_ESCRATCH: problem larger than the fixed scratch of the no-allocation entry point "
                   "(d_in above gptq_prepare_hinv_noalloc_max_din())";
        default: return "GPTQ: unknown status";
    }
}

int gptq_kernel_count(void) { return K_COUNT; }

const char* gptq_kernel_name(int id) { return (id >= 0 && id < K_COUNT) ? kNames[id] : nullptr; }

int gptq_timing_enable(int id) {
    if (id >= K_COUNT) return GPTQ_EINVAL;
    std::lock_guard<std::mutex> lock(g_mu);
    g_timed = id < 0 ? -1 : id;
    return GPTQ_OK;
}

int gptq_timing_read(double* total_ms, int64_t* launches) {
    if (!total_ms || !launches) return GPTQ_EINVAL;
    std::lock_guard<std::mutex> lock(g_mu);
    double tot = 0.0;
    int64_t cnt = 0;
    int rc = GPTQ_OK;
    for (auto& ep : g_pending) {
        if (hipEventSynchronize(ep.b) != hipSuccess) {
            rc = GPTQ_EHIP;
            continue;
        }
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, ep.a, ep.b) != hipSuccess) {
            rc = GPTQ_EHIP;
            continue;
        }
        tot += ms;
        ++cnt;
    }
    for (auto& ep : g_pending) g_free.push_back(ep);
    g_pending.clear();
    *total_ms = tot;
    *launches = cnt;
    return rc;
}

int gptq_hessian_accumulate(float* H, int64_t d_in, const void* X, int x_dtype, int64_t n_tokens, int64_t ldx,
                            void* stream) {
    if (d_in < 0 || n_tokens < 0 || ldx < n_tokens) return GPTQ_EINVAL;
    if (x_dtype != GPTQ_F16 && x_dtype != GPTQ_F32) return GPTQ_EINVAL;
    if (d_in == 0 || n_tokens == 0) return GPTQ_OK;
    if (!H || !X) return GPTQ_EINVAL;
    if (d_in > (int64_t)1 << 20) return GPTQ_EUNSUPPORTED;
    return hip_status(launch_hessian(H, d_in, &X, 1, x_dtype == GPTQ_F16, n_tokens, ldx, 0, as_stream(stream)));
}

int gptq_hessian_set(float* H, int64_t d_in, const void* X, int x_dtype, int64_t n_tokens, int64_t ldx,
                     void* stream) {
    if (d_in < 0 || n_tokens < 0 || ldx < n_tokens) return GPTQ_EINVAL;
    if (x_dtype != GPTQ_F16 && x_dtype != GPTQ_F32) return GPTQ_EINVAL;
    if (d_in == 0) return GPTQ_OK;
    if (!H || (n_tokens > 0 && !X)) return GPTQ_EINVAL;
    if (d_in > (int64_t)1 << 20) return GPTQ_EUNSUPPORTED;
    return hip_status(launch_hessian(H, d_in, &X, 1, x_dtype == GPTQ_F16, n_tokens, ldx, 1, as_stream(stream)));
}

int gptq_hessian_accumulate_chunks(float* H, int64_t d_in, const void* const* X_chunks, int64_t n_chunks,
                                   int x_dtype, int64_t n_tokens, int64_t ldx, int set, void* stream) {
    if (d_in < 0 || n_chunks < 0 || n_tokens < 0 || ldx < n_tokens) return GPTQ_EINVAL;
    if (x_dtype != GPTQ_F16 && x_dtype != GPTQ_F32) return GPTQ_EINVAL;
    if (set != 0 && set != 1) return GPTQ_EINVAL;
    if (d_in == 0) return GPTQ_OK;
    if (n_chunks > 0 && n_tokens > 0) {
        if (!X_chunks) return GPTQ_EINVAL;
        for (int64_t c = 0; c < n_chunks; ++c)
            if (!X_chunks[c]) return GPTQ_EINVAL;
    }
    if (n_chunks == 0 || n_tokens == 0) {
        if (!set) return GPTQ_OK;
        if (!H) return GPTQ_EINVAL;
        if (d_in > (int64_t)1 << 20) return GPTQ_EUNSUPPORTED;
        // an empty sum: the lower triangle becomes zero
        const void* none = nullptr;
        return hip_status(launch_hessian(H, d_in, &none, 1, x_dtype == GPTQ_F16, 0, ldx, 1, as_stream(stream)));
    }
    if (!H) return GPTQ_EINVAL;
    if (d_in > (int64_t)1 << 20) return GPTQ_EUNSUPPORTED;
    return hip_status(launch_hessian(H, d_in, X_chunks, n_chunks, x_dtype == GPTQ_F16, n_tokens, ldx, set,
                                     as_stream(stream)));
}

size_t gptq_prepare_hinv_workspace(int64_t d_in) { return d_in > 0 ? hinv_workspace_bytes(d_in) : 0; }

int gptq_prepare_hinv(const float* H, int64_t d_in, double damp_frac, float* U, uint8_t* dead, int32_t* info,
                      double* lambda_out, void* workspace, size_t workspace_bytes, void* stream) {
    if (d_in < 0 || !(damp_frac >= 0.0) || !isfinite(damp_frac)) return GPTQ_EINVAL;
    if (d_in == 0) return GPTQ_OK;
    if (!H || !U || !info) return GPTQ_EINVAL;
    if (d_in > (int64_t)1 << 17) return GPTQ_EUNSUPPORTED;
    if (!workspace || workspace_bytes < hinv_workspace_bytes(d_in) ||
        reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return GPTQ_EWORKSPACE;
    return hip_status(
        launch_prepare_hinv(H, d_in, damp_frac, U, dead, info, lambda_out, workspace, as_stream(stream)));
}

size_t gptq_prepare_hinv_fp32_workspace(int64_t d_in) { return d_in > 0 ? hinv32_workspace_bytes(d_in) : 0; }

int gptq_prepare_hinv_fp32(const float* H, int64_t d_in, double damp_frac, float* U, uint8_t* dead, int32_t* info,
                           double* lambda_out, void* workspace, size_t workspace_bytes, void* stream) {
    if (d_in < 0 || !(damp_frac >= 0.0) || !isfinite(damp_frac)) return GPTQ_EINVAL;
    if (d_in == 0) return GPTQ_OK;
    if (!H || !U || !info) return GPTQ_EINVAL;
    if (d_in > (int64_t)1 << 17) return GPTQ_EUNSUPPORTED;
    if (!workspace || workspace_bytes < hinv32_workspace_bytes(d_in) ||
        reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return GPTQ_EWORKSPACE;
    return hip_status(
        launch_prepare_hinv32(H, d_in, damp_frac, U, dead, info, lambda_out, workspace, as_stream(stream)));
}

int gptq_prepare_hinv_noalloc(const float* H, int64_t d_in, double damp_frac, float* U, uint8_t* dead,
                              int32_t* info, double* lambda_out, void* stream) {
    if (d_in < 0 || !(damp_frac >= 0.0) || !isfinite(damp_frac)) return GPTQ_EINVAL;
    if (d_in == 0) return GPTQ_OK;
    if (!H || !U || !info) return GPTQ_EINVAL;
    if (d_in > kNoAllocMaxDin) return GPTQ_ESCRATCH;
    void* ws = nullptr;
    const hipError_t e = hinv_noalloc_scratch(&ws);
    if (e != hipSuccess) return GPTQ_EHIP;
    if (hinv_noalloc_scratch_bytes() < hinv_workspace_bytes(d_in)) return GPTQ_ESCRATCH;
    TimingOff no_events;
    return hip_status(launch_prepare_hinv(H, d_in, damp_frac, U, dead, info, lambda_out, ws, as_stream(stream)));
}

int64_t gptq_prepare_hinv_noalloc_max_din(void) { return kNoAllocMaxDin; }

size_t gptq_quantize_layer_workspace(int64_t d_out, int64_t d_in, int64_t block_size) {
    if (d_out <= 0 || d_in <= 0 || block_size <= 0) return 0;
    return quant_workspace_bytes(d_out, d_in, block_size, 0);
}

size_t gptq_quantize_layer_split_workspace(int64_t d_out, int64_t d_in, int64_t block_size) {
    if (d_out <= 0 || d_in <= 0 || block_size <= 0) return 0;
    return quant_workspace_bytes(d_out, d_in, block_size, 1);
}

namespace {
int quantize_layer(const void* W, int w_dtype, int64_t d_out, int64_t d_in, const float* U, const uint8_t* dead,
                   int bits, int64_t group_size, int64_t block_size, uint8_t* codes, float* scales, int32_t* zeros,
                   float* err_row, float* minmax, void* workspace, size_t workspace_bytes, int split, void* stream) {
    if (d_out < 0 || d_in < 0) return GPTQ_EINVAL;
    if (w_dtype != GPTQ_F16 && w_dtype != GPTQ_F32) return GPTQ_EINVAL;
    if (bits < 2 || bits > 8) return GPTQ_EINVAL;
    if (block_size < 1 || block_size > 128) return GPTQ_EINVAL;
    if (group_size < 0) return GPTQ_EINVAL;
    if (group_size > 0 && d_in > 0 && d_in % group_size != 0) return GPTQ_EINVAL;
    if (group_size > 0) {
        if (group_size % 16 != 0) return GPTQ_EUNSUPPORTED;
        if (block_size % group_size != 0 && group_size % block_size != 0) return GPTQ_EUNSUPPORTED;
    }
    if (d_out == 0 || d_in == 0) return GPTQ_OK;
    if (!W || !U || !codes || !scales || !zeros) return GPTQ_EINVAL;
    if (d_out > ((int64_t)1 << 24) || d_in > ((int64_t)1 << 20)) return GPTQ_EUNSUPPORTED;
    if (!workspace || workspace_bytes < quant_workspace_bytes(d_out, d_in, block_size, split) ||
        reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return GPTQ_EWORKSPACE;
    return hip_status(launch_quantize(W, w_dtype == GPTQ_F16, d_out, d_in, U, dead, bits, group_size, block_size,
                                      codes, scales, zeros, err_row, minmax, workspace, split,
                                      reinterpret_cast<hipStream_t>(stream)));
}
}  // namespace

int gptq_quantize_layer(const void* W, int w_dtype, int64_t d_out, int64_t d_in, const float* U,
                        const uint8_t* dead, int bits, int64_t group_size, int64_t block_size, uint8_t* codes,
                        float* scales, int32_t* zeros, float* err_row, float* minmax, void* workspace,
                        size_t workspace_bytes, void* stream) {
    return quantize_layer(W, w_dtype, d_out, d_in, U, dead, bits, group_size, block_size, codes, scales, zeros,
                          err_row, minmax, workspace, workspace_bytes, 0, stream);
}

int gptq_quantize_layer_split(const void* W, int w_dtype, int64_t d_out, int64_t d_in, const float* U,
                              const uint8_t* dead, int bits, int64_t group_size, int64_t block_size, uint8_t* codes,
                              float* scales, int32_t* zeros, float* err_row, float* minmax, void* workspace,
                              size_t workspace_bytes, void* stream) {
    return quantize_layer(W, w_dtype, d_out, d_in, U, dead, bits, group_size, block_size, codes, scales, zeros,
                          err_row, minmax, workspace, workspace_bytes, 1, stream);
}

size_t gptq_obq_workspace(int64_t d_in) {
    if (d_in <= 0 || d_in > 128) return 0;
    return obq_workspace_bytes(d_in);
}

int gptq_obq_quantize(const void* W, int w_dtype, int64_t d_out, int64_t d_in, const float* U, const uint8_t* dead,
                      int bits, uint8_t* codes, float* scales, int32_t* zeros, int32_t* order, double* loss,
                      void* workspace, size_t workspace_bytes, void* stream) {
    if (d_out < 0 || d_in < 0) return GPTQ_EINVAL;
    if (w_dtype != GPTQ_F16 && w_dtype != GPTQ_F32) return GPTQ_EINVAL;
    if (bits < 2 || bits > 8) return GPTQ_EINVAL;
    if (d_out == 0 || d_in == 0) return GPTQ_OK;
    if (!W || !U || !codes || !scales || !zeros) return GPTQ_EINVAL;
    if (d_in > 128 || d_out > ((int64_t)1 << 24)) return GPTQ_EUNSUPPORTED;
    if (!workspace || workspace_bytes < obq_workspace_bytes(d_in) || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return GPTQ_EWORKSPACE;
    return hip_status(launch_obq(W, w_dtype == GPTQ_F16, d_out, d_in, U, dead, bits, codes, scales, zeros, order, loss,
                                 workspace, as_stream(stream)));
}

int64_t gptq_packed_words(int64_t d_in, int bits) {
    if (d_in < 0 || bits < 2 || bits > 8) return -1;
    return packed_words(d_in, bits);
}

int gptq_pack_codes(const uint8_t* codes, int64_t d_out, int64_t d_in, int bits, uint32_t* packed, void* stream) {
    if (d_out < 0 || d_in < 0 || bits < 2 || bits > 8) return GPTQ_EINVAL;
    if (d_out == 0 || d_in == 0) return GPTQ_OK;
    if (!codes || !packed) return GPTQ_EINVAL;
    if (d_in > ((int64_t)1 << 24) || d_out > ((int64_t)1 << 24)) return GPTQ_EUNSUPPORTED;
    return hip_status(launch_pack(codes, d_out, d_in, bits, packed, as_stream(stream)));
}

int gptq_dequantize(const uint32_t* packed, int bits, int64_t d_out, int64_t d_in, const float* scales,
                    const int32_t* zeros, int64_t group_size, void* out, int out_dtype, void* stream) {
    if (d_out < 0 || d_in < 0 || bits < 2 || bits > 8 || group_size < 0) return GPTQ_EINVAL;
    if (out_dtype != GPTQ_F16 && out_dtype != GPTQ_F32) return GPTQ_EINVAL;
    if (group_size > 0 && d_in > 0 && d_in % group_size != 0) return GPTQ_EINVAL;
    if (d_out == 0 || d_in == 0) return GPTQ_OK;
    if (!packed || !scales || !zeros || !out) return GPTQ_EINVAL;
    if (d_in > ((int64_t)1 << 24) || d_out > ((int64_t)1 << 24)) return GPTQ_EUNSUPPORTED;
    return hip_status(
        launch_dequant(packed, bits, d_out, d_in, scales, zeros, group_size, out, out_dtype == GPTQ_F16, as_stream(stream)));
}

int gptq_output_error(const void* W, int w_dtype, const uint8_t* dead, const uint32_t* packed, int bits,
                      const float* scales, const int32_t* zeros, int64_t group_size, int64_t d_out, int64_t d_in,
                      const float* err_row, const double* lambda, float* out_row, void* stream) {
    if (d_out < 0 || d_in < 0 || bits < 2 || bits > 8 || group_size < 0) return GPTQ_EINVAL;
    if (w_dtype != GPTQ_F16 && w_dtype != GPTQ_F32) return GPTQ_EINVAL;
    if (group_size > 0 && d_in > 0 && d_in % group_size != 0) return GPTQ_EINVAL;
    if (d_out == 0 || d_in == 0) return GPTQ_OK;
    if (!W || !packed || !scales || !zeros || !err_row || !lambda || !out_row) return GPTQ_EINVAL;
    if (d_in > ((int64_t)1 << 24) || d_out > ((int64_t)1 << 24)) return GPTQ_EUNSUPPORTED;
    return hip_status(launch_output_error(W, w_dtype == GPTQ_F16, dead, packed, bits, scales, zeros, group_size,
                                          d_out, d_in, err_row, lambda, out_row, as_stream(stream)));
}

int gptq_propagate(const void* W_hat, int w_dtype, int64_t d_out, int64_t d_in, const void* X, int x_dtype,
                   int64_t n_tokens, int64_t ldx, void* Y, int64_t ldy, int activation, void* stream) {
    if (d_out < 0 || d_in < 0 || n_tokens < 0) return GPTQ_EINVAL;
    if (activation != 0 && activation != 1) return GPTQ_EINVAL;
    if ((w_dtype != GPTQ_F16 && w_dtype != GPTQ_F32) || (x_dtype != GPTQ_F16 && x_dtype != GPTQ_F32))
        return GPTQ_EINVAL;
    if (d_out == 0 || n_tokens == 0) return GPTQ_OK;
    if (ldx < n_tokens || ldy < n_tokens) return GPTQ_EINVAL;
    if (!Y || (d_in > 0 && (!W_hat || !X))) return GPTQ_EINVAL;
    if (w_dtype != GPTQ_F16 || x_dtype != GPTQ_F16) return GPTQ_EUNSUPPORTED;
    if (d_out > ((int64_t)1 << 24) || d_in > ((int64_t)1 << 22) || ldx > ((int64_t)1 << 23)) return GPTQ_EUNSUPPORTED;
    if (((d_out + 127) / 128) * ((n_tokens + 127) / 128) > (int64_t)INT32_MAX) return GPTQ_EUNSUPPORTED;
    return hip_status(launch_propagate(W_hat, d_out, d_in, X, n_tokens, ldx, Y, ldy, activation, as_stream(stream)));
}

}  // extern "C"
