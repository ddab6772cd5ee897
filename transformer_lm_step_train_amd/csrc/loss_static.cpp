// The loss step of the model's forward (fused softmax + cross-entropy over
// the vocabulary, then the mean over positions) on caller-owned device
// buffers, allocating nothing: the per-row losses go to a fixed device array
// of this file instead of the model's arena.  For callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// Every call on a device shares that device's array, which keeps the last
// call's contents; each call overwrites the rows it uses before reading
// them, so nothing needs clearing.  Calls that overlap on one device race on
// the array.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/gpt2.h"
#include "dtype.h"
#include "kernels.h"

int gpt2_set_error(int code, const char* msg);  // host.cpp

namespace {

// Rows one call may hold (the library's largest batch of positions).
constexpr int kMaxRows = 32768;

__device__ __align__(256) float scratch[kMaxRows];

// Device address of `scratch` on each device, taken once per device with
// that device current.  (In host code `scratch` names a host-side stand-in,
// not device memory.)
constexpr int kMaxDevices = 64;
float* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

int scratch_ptr(float** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return gpt2_set_error(GPT2_EDEVICE, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return gpt2_set_error(GPT2_EDEVICE, "device index outside the supported 0..63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return gpt2_set_error(GPT2_EDEVICE, e != hipSuccess ? hipGetErrorString(e)
                                                                : "scratch address is NULL");
        g_scratch[dev] = static_cast<float*>(p);
    }
    *out = g_scratch[dev];
    return GPT2_OK;
}

int launch_error(hipError_t e) {
    return e == hipSuccess ? GPT2_OK : gpt2_set_error(GPT2_EDEVICE, hipGetErrorString(e));
}

}  // namespace

extern "C" int gpt2_cross_entropy_static(const void* logits, int64_t ldv,
                                         const int32_t* targets, int N, int V, int precision,
                                         float grad_scale, float* mean_loss, int32_t* flag,
                                         void* hip_stream) {
    if (!logits || !targets || !mean_loss || !flag)
        return gpt2_set_error(GPT2_EINVAL, "NULL argument");
    if (reinterpret_cast<uintptr_t>(logits) % 16 != 0)
        return gpt2_set_error(GPT2_EINVAL, "logits must be 16-byte aligned");
    if (N < 1 || N > kMaxRows)
        return gpt2_set_error(GPT2_EINVAL,
                              "N outside 1..32768 (the rows the static scratch holds)");
    if (V < 1 || ldv < V || ldv % 4 != 0 || ldv > 65536)
        return gpt2_set_error(GPT2_EINVAL, "need 1 <= V <= ldv <= 65536 with ldv % 4 == 0");
    const int dt = precision == GPT2_FP32         ? DT_F32
                   : precision == GPT2_BF16_MIXED ? DT_BF16
                   : precision == GPT2_F16_MIXED  ? DT_F16
                                                  : -1;
    if (dt < 0) return gpt2_set_error(GPT2_EINVAL, "unknown precision");
    float* rows = nullptr;
    const int rc = scratch_ptr(&rows);
    if (rc != GPT2_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    int r = launch_error(gk::fill_zero(s, reinterpret_cast<float*>(flag), 1));
    if (r == GPT2_OK)
        r = launch_error(gk::softmax_ce(s, const_cast<void*>(logits), rows, targets, N, V,
                                        (int)ldv, grad_scale, nullptr, flag, dt));
    if (r == GPT2_OK) r = launch_error(gk::mean_reduce(s, mean_loss, rows, N));
    return r;
}
