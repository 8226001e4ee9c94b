// Host-only stand-ins for the kernel launchers, linked with the C-ABI layer
// (qlin_api.hip) into a sanitizer build that runs on a CPU: every launcher
// records that it was reached and returns success without touching memory.
// Test infrastructure: never part of libqlin.so.
#include <atomic>

#include "../../quantized_linear_layers_token_amd/csrc/qlin_internal.h"

namespace {
std::atomic<int> g_launches{0};
hipError_t reached() {
    ++g_launches;
    return hipSuccess;
}
}  // namespace

extern "C" int qlin_hostcheck_launches(void) { return g_launches.load(); }
extern "C" void qlin_hostcheck_reset(void) { g_launches = 0; }

namespace qlin {
hipError_t launch_quant_int8(const uint16_t*, int64_t, int64_t, int8_t*, float*, hipStream_t) { return reached(); }
hipError_t launch_quant_fp8(const uint16_t*, int64_t, int64_t, int, uint8_t*, float*, hipStream_t) { return reached(); }
hipError_t launch_gemv(int, const uint8_t*, const float*, const uint8_t*, const uint16_t*, void*, int64_t, int64_t, int,
                       hipStream_t) {
    return reached();
}
hipError_t launch_gemm_small(int, const uint8_t*, const float*, const SegmentArgs&, int64_t, int64_t, int,
                             hipStream_t) {
    return reached();
}
hipError_t launch_gemm_large_cfg(int, int, const uint8_t*, const float*, const SegmentArgs&, int64_t, int64_t, int,
                                 hipStream_t) {
    return reached();
}
hipError_t launch_gemm_large(int, const uint8_t*, const float*, const SegmentArgs&, int64_t, int64_t, int,
                             hipStream_t) {
    return reached();
}
hipError_t launch_linear_decode(int, const uint16_t*, int64_t, const SegmentArgs&, int, uint8_t*, float*,
                                hipStream_t) {
    return reached();
}
hipError_t launch_linear_tokens(int, const uint16_t*, int64_t, int64_t, const SegmentArgs&, int, uint8_t*, float*,
                                hipStream_t) {
    return reached();
}
hipError_t launch_gemm_small_fused(int, const uint16_t*, int64_t, int64_t, const SegmentArgs&, int, uint8_t*, float*,
                                   hipStream_t) {
    return reached();
}
hipError_t launch_gemm_packed(int, const uint8_t*, const float*, const SegmentArgs&, int64_t, int64_t, int,
                              hipStream_t) {
    return reached();
}
hipError_t launch_pack_weights(int, const uint8_t*, int64_t, int64_t, uint8_t*, hipStream_t) { return reached(); }
hipError_t launch_weight_only(int, const uint16_t*, int64_t, int64_t, const SegmentArgs&, int, hipStream_t) {
    return reached();
}
}  // namespace qlin
