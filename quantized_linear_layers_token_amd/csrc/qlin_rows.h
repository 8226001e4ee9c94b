// Device helpers of the row-streaming kernels: one weight row's products with
// rounded activations (int8 dot products, E4M3 on the vector ALUs or the
// matrix cores).
#pragma once

#include "qlin_round.h"

namespace qlin {

__device__ __forceinline__ int dot16_i8(const v4u& w, const v4u& x, int acc) {
    acc = __builtin_amdgcn_sdot4((int)w.x, (int)x.x, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.y, (int)x.y, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.z, (int)x.z, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.w, (int)x.w, acc, false);
    return acc;
}

// E4M3 products on the vector ALUs: byte pairs decoded to f32
// (v_cvt_pk_f32_fp8; every product of two E4M3 values is exact in f32) and
// summed with FMAs, two chains per 16 bytes.
__device__ __forceinline__ float dot4_e4m3(uint32_t w, uint32_t x, float acc) {
    const v2f w01 = e4m3_unpack2<false>(w), w23 = e4m3_unpack2<true>(w);
    const v2f x01 = e4m3_unpack2<false>(x), x23 = e4m3_unpack2<true>(x);
    acc = __builtin_fmaf(w01.x, x01.x, acc);
    acc = __builtin_fmaf(w01.y, x01.y, acc);
    acc = __builtin_fmaf(w23.x, x23.x, acc);
    acc = __builtin_fmaf(w23.y, x23.y, acc);
    return acc;
}

__device__ __forceinline__ float dot16_e4m3(const v4u& w, const v4u& x) {
    float a = dot4_e4m3(w.x, x.x, 0.0f);
    float b = dot4_e4m3(w.y, x.y, 0.0f);
    a = dot4_e4m3(w.z, x.z, a);
    b = dot4_e4m3(w.w, x.w, b);
    return a + b;
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
