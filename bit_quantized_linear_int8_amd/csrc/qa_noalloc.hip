// qa_noalloc.hip -- the LLM.int8() mixed linear with no workspace argument,
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The call runs exactly the kernels of qa_qlinear_int8_mixed; its scratch
// (outlier flag words, outlier list and count, per-token scales, int8 codes,
// compact outlier rows) lives in one file-scope device array per GPU.  Host
// code never passes the array's name to a kernel: on the host that name is a
// stand-in, not a device address.  The device address of each GPU's copy is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and kept; every launch takes that address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qa.h"
#include "qa_launch.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)40 << 20;   // QA_NOALLOC_SCRATCH_BYTES in qa.h
static_assert(kScratchBytes == QA_NOALLOC_SCRATCH_BYTES, "qa.h states the scratch size");

// Nothing in it needs to start at zero: every slot a call reads was written
// earlier in the same call.  Every call on a GPU uses this same memory.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_lookup[kMaxDevices];

// Device address of `scratch` on device dev (looked up once, with dev current,
// then the caller's current device is restored).
hipError_t scratch_address(int dev, void** p) {
    std::call_once(g_once[dev], [dev] {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        void* a = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (cur >= 0 && cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        g_scratch[dev] = e == hipSuccess ? a : nullptr;
        g_lookup[dev] = e;
    });
    *p = g_scratch[dev];
    return g_lookup[dev];
}

}  // namespace

extern "C" qa_status qa_qlinear_int8_mixed_noalloc(const void* X_f16, int64_t M, int64_t K, const int8_t* Wq,
                                                   const float* s_w, const void* W_f16_or_null, int64_t N,
                                                   float threshold, void* out, qa_dtype out_dtype, void* stream) {
    static const char* fn = "qa_qlinear_int8_mixed_noalloc";
    bool empty = false;
    const qa_status v = qa::mixed_validate(fn, X_f16, M, K, Wq, s_w, W_f16_or_null, N, threshold, out, out_dtype,
                                           false, nullptr, 0, &empty);
    if (v != QA_OK || empty) return v;
    const size_t need = qa_qlinear_int8_mixed_workspace(M, K);
    if (need > kScratchBytes)
        return qa::record_error(QA_ERR_WORKSPACE,
                                "%s: M = %lld, K = %lld need %zu bytes of scratch; the static scratch holds %zu "
                                "(use qa_qlinear_int8_mixed with a workspace)",
                                fn, (long long)M, (long long)K, need, kScratchBytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = -1;
    hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return qa::record_error(QA_ERR_DEVICE, "%s: device of the stream: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return qa::record_error(QA_ERR_DEVICE, "%s: device %d out of range", fn, dev);
    void* ws = nullptr;
    e = scratch_address(dev, &ws);
    if (e != hipSuccess || !ws)
        return qa::record_error(QA_ERR_DEVICE, "%s: scratch address on device %d: %s", fn, dev, hipGetErrorString(e));
    return qa::mixed_run(fn, X_f16, M, K, Wq, s_w, W_f16_or_null, N, threshold, out, out_dtype, ws, stream);
}
