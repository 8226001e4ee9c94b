// qlin_linear without caller staging buffers: the quantized activations live
// in a fixed device array of this library (one per GPU, for the process's
// lifetime), for callers that cannot allocate device memory.  The kernels are
// those of qlin_linear; only the staging memory differs.
#include <mutex>

#include <hip/hip_runtime.h>

#include "qlin_internal.h"

namespace {

constexpr size_t kCodeBytes = QLIN_NOALLOC_MAX_CODE_BYTES;
constexpr size_t kScaleBytes = (size_t)4 * QLIN_NOALLOC_MAX_SCALES;

// The staging: codes first, then the f32 scales.  In host code `scratch`
// names a host-side stand-in, not device memory: kernels get the device
// address from hipGetSymbolAddress, looked up per device below.
static __device__ __align__(256) uint8_t scratch[kCodeBytes + kScaleBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device (null until looked up)

qlin_status scratch_address(int device, uint8_t** out) {
    if (device < 0 || device >= kMaxDevices) return QLIN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch[device] == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) return QLIN_ERR_HIP;
        g_scratch[device] = p;
    }
    *out = static_cast<uint8_t*>(g_scratch[device]);
    return QLIN_OK;
}

}  // namespace

extern "C" qlin_status qlin_linear_noalloc(qlin_scheme scheme, const uint16_t* x, int64_t M, int64_t K,
                                           const qlin_segment* segments, int32_t nseg, qlin_out out,
                                           hipStream_t stream) {
    // size first: a call the scratch cannot stage is refused before anything else
    if (M > 0 && K > 0) {
        const bool block = scheme == QLIN_SCHEME_FP8_BLOCK;
        const int64_t scales = block ? M * (K / 128) : M;
        if (M > (int64_t)kCodeBytes / K || scales > (int64_t)QLIN_NOALLOC_MAX_SCALES) return QLIN_ERR_TOO_LARGE;
    }
    bool noop = false;
    const qlin_status v = qlin::linear_validate(scheme, x, M, K, segments, nseg, out, &noop);
    if (v != QLIN_OK || noop) return v;
    if (qlin::linear_is_one_launch(scheme, M, K, segments, nseg))   // no staging needed
        return qlin::linear_call(scheme, x, M, K, segments, nseg, out, nullptr, nullptr, stream);
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return QLIN_ERR_HIP;
    if (stream != nullptr) {
        int sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return QLIN_ERR_HIP;
        if (sdev != device) return QLIN_ERR_UNSUPPORTED;
    }
    uint8_t* base = nullptr;
    const qlin_status st = scratch_address(device, &base);   // validation passed: now the device
    if (st != QLIN_OK) return st;
    return qlin::linear_call(scheme, x, M, K, segments, nseg, out, base, reinterpret_cast<float*>(base + kCodeBytes),
                             stream);
}
