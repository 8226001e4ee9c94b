// Device-side helpers shared by the gfx950 kernels: bf16 / E4M3 conversions,
// wavefront reductions over DPP, MFMA operand types and the scale epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlin_internal.h"

namespace qlin {

typedef int   v4i  __attribute__((ext_vector_type(4)));
typedef int   v8i  __attribute__((ext_vector_type(8)));
typedef int   v16i __attribute__((ext_vector_type(16)));
typedef float v4f  __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// A raw buffer descriptor over [base, base + bytes): loads at offsets at or
// past `bytes` return zero.  Arguments must be wave-uniform; they are moved to
// scalar registers explicitly, since a descriptor that the compiler cannot
// prove uniform gets a readfirstlane loop around every load that uses it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, 0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

constexpr int kWave = 64;

// Entry i (< kMaxSegments) of a kernel-argument array, picked by selects over
// entries loaded at static offsets: the compiler then loads the whole array
// with the other kernel arguments instead of computing an address and loading
// once more, a dependent scalar load at the start of every workgroup (the empty
// asm keeps it from turning the selects back into that load).  pick_global
// returns a global-memory pointer, so that loads through it stay global loads.
__device__ __forceinline__ int pick_int(const int* a, int i) {
    int v = 0;
#pragma unroll
    for (int t = 0; t < kMaxSegments; ++t) {
        int e = a[t];
        asm volatile("" : "+s"(e));
        v = (i == t) ? e : v;
    }
    return v;
}
template <class T>
__device__ __forceinline__ T* pick_ptr(T* const* a, int i) {
    uint64_t v = 0;
#pragma unroll
    for (int t = 0; t < kMaxSegments; ++t) {
        uint64_t e = reinterpret_cast<uint64_t>(a[t]);
        asm volatile("" : "+s"(e));
        v = (i == t) ? e : v;
    }
    return reinterpret_cast<T*>(v);
}
template <class T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* pick_global(const T* const* a, int i) {
    uint64_t v = 0;
#pragma unroll
    for (int t = 0; t < kMaxSegments; ++t) {
        uint64_t e = reinterpret_cast<uint64_t>(a[t]);
        asm volatile("" : "+s"(e));
        v = (i == t) ? e : v;
    }
    return reinterpret_cast<const __attribute__((address_space(1))) T*>(v);
}

// Idle issue slots after the last matrix-core (XDL) instruction of a sequence,
// before anything else touches its destination registers.  The hardware does
// not interlock a vector-ALU, LDS or memory access against an XDL result: on
// CDNA3 the software must leave NumPasses + 3 independent slots, and gfx950
// needs one more for ops of 4 or more passes (NumPasses + 4: 20 for the
// 16-pass 32x32x64 E4M3 op, 12 for 32x32x32 int8 and 16x16x128 E4M3, 8 for
// 16x16x64 int8 and 16x16x32 bf16).  This compiler pads some accumulator
// reads that follow a loop's last MFMAs with only NumPasses + 3 slots (19
// after a 32x32x64 E4M3 op in the tiled GEMM's exit path), which let the
// epilogue read the last registers of the last MFMA before they were written.
// Three s_nop 7 give 24 slots, enough for every op used here whatever the
// compiler adds; called once per tile, after the K loop.
__device__ __forceinline__ void mfma_drain() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------

// Exact widening of a bf16 bit pattern (low 16 bits of b) to f32.
__device__ __forceinline__ float bf16_lo(uint32_t b) { return __uint_as_float(b << 16); }

// Widening of the high bf16 of a packed pair.
__device__ __forceinline__ float bf16_hi(uint32_t b) { return __uint_as_float(b & 0xFFFF0000u); }

// f32 -> bf16 with round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

// ---------------------------------------------------------------------------
// OCP E4M3 encode: the caller saturates to [-448, 448] first; the hardware
// conversion rounds to nearest even.  Packs (a, b) into bytes 0/1 or 2/3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_pack_lo(float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
}
__device__ __forceinline__ uint32_t e4m3_pack_hi(uint32_t old, float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, true);
}

// ---------------------------------------------------------------------------
// DPP reductions.  Row = 16 lanes.  After row_* every lane of the row holds
// the row result; wave_* returns the wave-uniform result.
// Controls: quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
    v = max(v, (uint32_t)dpp_i<0xB1>((int)v));
    v = max(v, (uint32_t)dpp_i<0x4E>((int)v));
    v = max(v, (uint32_t)dpp_i<0x141>((int)v));
    v = max(v, (uint32_t)dpp_i<0x140>((int)v));
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = row_max_u32(v);
    uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, d));
}

__device__ __forceinline__ int row_sum_i32(int v) {
    v += dpp_i<0xB1>(v);
    v += dpp_i<0x4E>(v);
    v += dpp_i<0x141>(v);
    v += dpp_i<0x140>(v);
    return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
    v = row_sum_i32(v);
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
           __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

__device__ __forceinline__ float row_sum_f32(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
    v = row_sum_f32(v);
    float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (a + b) + (c + d);
}

// ---------------------------------------------------------------------------
// Scale epilogue: y = fl32(acc) * fl32(s_x * s_w), written as bf16 (RNE),
// f32, or (int8 schemes) the raw int32 accumulator.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_rowwise_i32acc(void* y, int64_t idx, int acc, float sx,
                                                     uint32_t sw_bits, int mode) {
    if (mode == OUT_I32) {
        static_cast<int*>(y)[idx] = acc;
        return;
    }
    const float sc = sx * bf16_lo(sw_bits);
    const float v = (float)acc * sc;
    if (mode == OUT_F32) static_cast<float*>(y)[idx] = v;
    else static_cast<uint16_t*>(y)[idx] = f32_to_bf16(v);
}

__device__ __forceinline__ void store_f32(void* y, int64_t idx, float v, int mode) {
    if (mode == OUT_F32) static_cast<float*>(y)[idx] = v;
    else static_cast<uint16_t*>(y)[idx] = f32_to_bf16(v);
}

// Four consecutive outputs y[idx .. idx+3] of one row (idx % 4 == 0 and the row
// length a multiple of 4, so the store is 8- or 16-byte aligned).  Same
// arithmetic as the scalar stores above: fl32(acc) * fl32(s_x * s_w), RNE.
__device__ __forceinline__ void store4_rowwise_i32acc(void* y, int64_t idx, const int (&acc)[4], float sx,
                                                      const float (&sw)[4], int mode) {
    if (mode == OUT_I32) {
        *reinterpret_cast<v4i*>(static_cast<int*>(y) + idx) = v4i{acc[0], acc[1], acc[2], acc[3]};
        return;
    }
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = (float)acc[k] * (sx * sw[k]);
    if (mode == OUT_F32) {
        *reinterpret_cast<v4f*>(static_cast<float*>(y) + idx) = v4f{v[0], v[1], v[2], v[3]};
    } else {
        const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        *reinterpret_cast<v2u*>(static_cast<uint16_t*>(y) + idx) = v2u{lo, hi};
    }
}

__device__ __forceinline__ void store4_f32(void* y, int64_t idx, const float (&v)[4], int mode) {
    if (mode == OUT_F32) {
        *reinterpret_cast<v4f*>(static_cast<float*>(y) + idx) = v4f{v[0], v[1], v[2], v[3]};
    } else {
        const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        *reinterpret_cast<v2u*>(static_cast<uint16_t*>(y) + idx) = v2u{lo, hi};
    }
}

// SwiGLU of one gate/up output pair.  Each projection output is first rounded
// to bf16, as the projection alone would write it; silu(t) = t / (1 + e^-t) is
// evaluated in f32 on that value and rounded to bf16, and the product with the
// bf16 up value is rounded to bf16.  (For t below about -88, e^-t is +inf in
// f32 and the quotient is -0; the true value is then below 1e-36.)
__device__ __forceinline__ uint16_t swiglu_bf16(float g, float u) {
    const float gb = bf16_lo(f32_to_bf16(g));
    const float ub = bf16_lo(f32_to_bf16(u));
    const float s = bf16_lo(f32_to_bf16(gb / (1.0f + __expf(-gb))));
    return f32_to_bf16(s * ub);
}

// E4M3 pair decode (bytes 0/1 when HI == false, bytes 2/3 when HI == true).
typedef float v2f __attribute__((ext_vector_type(2)));
template <bool HI>
__device__ __forceinline__ v2f e4m3_unpack2(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}

}  // namespace qlin
