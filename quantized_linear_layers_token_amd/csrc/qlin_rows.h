// Device helpers of the row-streaming kernels (fused one-launch products):
// rounding a bf16 row to int8 / OCP E4M3 codes the way the standalone
// quantizers do, and one weight row's products with rounded activations.
#pragma once

#include "qlin_device.h"

namespace qlin {

// absmax over 8 bf16 magnitudes (bit patterns with the sign cleared: for
// non-negative finite floats the bit order is the value order)
__device__ __forceinline__ uint32_t chunk_absmax(const v4u& v) {
    uint32_t a = v.x & 0x7FFF7FFFu, b = v.y & 0x7FFF7FFFu;
    uint32_t c = v.z & 0x7FFF7FFFu, d = v.w & 0x7FFF7FFFu;
    uint32_t m0 = max(a & 0xFFFFu, a >> 16), m1 = max(b & 0xFFFFu, b >> 16);
    uint32_t m2 = max(c & 0xFFFFu, c >> 16), m3 = max(d & 0xFFFFu, d >> 16);
    return max(max(m0, m1), max(m2, m3));
}

template <bool FP8>
__device__ __forceinline__ void scales_from_absmax(uint32_t amax_bits, float& s, RoundFactor& rf) {
    const float q = FP8 ? 448.0f : 127.0f;
    s = __uint_as_float(amax_bits << 16) / q;
    rf = round_factor(amax_bits, q);
}

__device__ __forceinline__ uint32_t q4_int8(uint32_t w0, uint32_t w1, RoundFactor rf) {
    auto q = [rf](float v) {
        float t = __builtin_rintf((v * rf.pre) * rf.inv);
        t = fminf(fmaxf(t, -127.0f), 127.0f);
        return (uint32_t)(uint8_t)(int8_t)(int)t;
    };
    return q(bf16_lo(w0)) | (q(bf16_hi(w0)) << 8) | (q(bf16_lo(w1)) << 16) | (q(bf16_hi(w1)) << 24);
}

__device__ __forceinline__ uint32_t q4_fp8(uint32_t w0, uint32_t w1, RoundFactor rf) {
    auto c = [rf](float v) { return fminf(fmaxf((v * rf.pre) * rf.inv, -448.0f), 448.0f); };
    const uint32_t lo = e4m3_pack_lo(c(bf16_lo(w0)), c(bf16_hi(w0)));
    return e4m3_pack_hi(lo, c(bf16_lo(w1)), c(bf16_hi(w1)));
}

template <bool FP8>
__device__ __forceinline__ v2u quant8(const v4u& v, RoundFactor rf) {
    if constexpr (FP8) return v2u{q4_fp8(v.x, v.y, rf), q4_fp8(v.z, v.w, rf)};
    else return v2u{q4_int8(v.x, v.y, rf), q4_int8(v.z, v.w, rf)};
}

__device__ __forceinline__ int dot16_i8(const v4u& w, const v4u& x, int acc) {
    acc = __builtin_amdgcn_sdot4((int)w.x, (int)x.x, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.y, (int)x.y, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.z, (int)x.z, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.w, (int)x.w, acc, false);
    return acc;
}

// E4M3 products on the matrix cores, one weight row at a time.  A 16x16x128
// MFMA whose A operand is this lane's 32 weight bytes and whose B operand is
// the activation bytes at the same positions returns, on its diagonal,
// C[i][i] = the sum over the four lanes l with l % 16 == i of their bytewise
// products (both operands map register bytes to K slots the same way).  The
// diagonal sits in lanes with (l % 16) / 4 == l / 16, register l % 4.
__device__ __forceinline__ v4f mfma_e4m3(const v4u& w0, const v4u& w1, const v4u& x0, const v4u& x1, v4f c) {
    const v8i a = v8i{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
    const v8i b = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ float mfma16_diag(const v4f& c, int lane) {
    const int e = lane & 3;
    const float v = e == 0 ? c.x : (e == 1 ? c.y : (e == 2 ? c.z : c.w));
    return ((lane & 15) >> 2) == (lane >> 4) ? v : 0.0f;
}

}  // namespace qlin
