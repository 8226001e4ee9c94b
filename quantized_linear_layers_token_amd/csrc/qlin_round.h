// The dynamic activation rounding, in one place: every kernel that rounds bf16
// inputs to int8 or OCP E4M3 codes (the standalone quantizers and the fused
// products that round the tokens themselves) uses these functions, so all of
// them produce the same codes and scales.
//
// Per token (or 128-input group) with absmax a and range Q (127 for int8: W8A8
// model card, intro; 448, the largest finite E4M3 value, for FP8: FP8-dynamic
// README, "Creation" recipe, and Qwen3 8B FP8 card, "Loading"):
//   s = fl32(a / Q),  inv = fl32(Q / a),  code = sat_Q(round_half_even(fl32(x * inv)))
// (E4M3: nearest code of the saturated value, ties to even).
#pragma once

#include "qlin_device.h"

namespace qlin {

// Factors of the activation rounding t = fl32(fl32(x * pre) * inv) for a token
// (or group) with absmax a (bf16 bits, sign cleared) and range Q: pre = 1,
// inv = fl32(Q / a); for a < 2^-64, where Q / a can exceed the f32 range,
// pre = 2^64 and inv = fl32(Q / (a * 2^64)).  Scaling by 2^64 is exact, so
// wherever Q / a is finite both forms give the same t (the dynamic scale of
// the W8A8 and FP8 model cards, "Loading": code = x / (a / Q), rounded).
struct RoundFactor {
    float pre, inv;
};
__device__ __forceinline__ RoundFactor round_factor(uint32_t amax_bits, float q) {
    const float pre = amax_bits < 0x1F80u ? 0x1p64f : 1.0f;       // 0x1F80: bf16 bits of 2^-64
    const float a = __uint_as_float(amax_bits << 16) * pre;
    return RoundFactor{pre, amax_bits == 0 ? 0.0f : q / a};
}
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

}  // namespace qlin
