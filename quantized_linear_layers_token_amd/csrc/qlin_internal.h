// Launchers shared between the kernel files and the C-ABI layer.  All
// arguments are validated by the caller (qlin_api.hip) before a launch.
// Host declarations only (the C-ABI layer also builds as plain host C++).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/qlin.h"

namespace qlin {

enum Variant : int { VAR_INT8 = 0, VAR_FP8_ROW = 1, VAR_FP8_BLOCK = 2 };

enum OutMode : int { OUT_BF16 = 0, OUT_I32 = 1, OUT_F32 = 2,
                     // gate/up pair: segments 0 and 1 are the gate and up weights (equal
                     // widths), y[0] receives bf16 silu(gate) * up (swiglu_bf16)
                     OUT_SWIGLU = 3 };

// Weight segments that read the same activation row (e.g. q, k, v): rows of
// segment i are global rows [start[i], start[i+1]).  Passed by value.
constexpr int kMaxSegments = 4;
struct SegmentArgs {
    const uint8_t* w[kMaxSegments];
    const uint16_t* sw[kMaxSegments];
    void* y[kMaxSegments];
    int start[kMaxSegments + 1];
    int nseg;
};

hipError_t launch_quant_int8(const uint16_t* x, int64_t M, int64_t K, int8_t* q, float* s, hipStream_t st);
hipError_t launch_quant_fp8(const uint16_t* x, int64_t M, int64_t K, int group, uint8_t* q, float* s,
                            hipStream_t st);

hipError_t launch_gemv(int variant, const uint8_t* qx, const float* sx, const uint8_t* qw, const uint16_t* sw,
                       void* y, int64_t N, int64_t K, int mode, hipStream_t st);
// Small-M product over every segment of sa in one launch (16-row tiles never
// straddle two segments).
hipError_t launch_gemm_small(int variant, const uint8_t* qx, const float* sx, const SegmentArgs& sa, int64_t M,
                             int64_t K, int mode, hipStream_t st);
// A single product as a one-segment SegmentArgs.
inline SegmentArgs one_segment(const uint8_t* w, const uint16_t* sw, void* y, int64_t n) {
    SegmentArgs sa{};
    sa.w[0] = w;
    sa.sw[0] = sw;
    sa.y[0] = y;
    sa.start[0] = 0;
    for (int i = 1; i <= kMaxSegments; ++i) sa.start[i] = (int)n;
    sa.nseg = 1;
    return sa;
}

// Output tiles of the tiled GEMM (weight rows x tokens), in the order of the
// fixed-tile paths of the C ABI.
enum LargeTile : int {
    kTile256x128 = 0, kTile128x128 = 1, kTile128x64 = 2, kTile128x256 = 3, kTile128x128K2 = 4, kTile128x64K2 = 5,
    kTile256x256W8 = 6,  // rowwise schemes only
    kTile256x256 = 7     // rowwise schemes only
};
// The tiled GEMM over every segment of sa (one launch; a weight panel never
// straddles two segments).  cfg: LargeTile.
hipError_t launch_gemm_large_cfg(int cfg, int variant, const uint8_t* qx, const float* sx, const SegmentArgs& sa,
                                 int64_t M, int64_t K, int mode, hipStream_t st);
int large_tile_config(int variant, int64_t M, const SegmentArgs& sa);
hipError_t launch_gemm_large(int variant, const uint8_t* qx, const float* sx, const SegmentArgs& sa, int64_t M,
                             int64_t K, int mode, hipStream_t st);

// The tiled product on weights in the matrix-core operand order (every scheme;
// every segment's width a multiple of 128, K % 128 == 0): one launch over every
// segment, or with mode OUT_SWIGLU over the gate (segment 0) / up (segment 1)
// pair into h.  launch_pack_weights writes that order from row-major codes
// ([N, K], N % 128 == 0, K % 128 == 0; block FP8 codes as E4M3, VAR_FP8_ROW).
hipError_t launch_gemm_packed(int variant, const uint8_t* qx, const float* sx, const SegmentArgs& sa, int64_t M,
                              int64_t K, int mode, hipStream_t st);
hipError_t launch_pack_weights(int variant, const uint8_t* w, int64_t N, int64_t K, uint8_t* p, hipStream_t st);

hipError_t launch_linear_decode(int variant, const uint16_t* x, int64_t K, const SegmentArgs& sa, int mode,
                                uint8_t* qx, float* sx, hipStream_t st);
constexpr int64_t kDecodeMaxK = 16384;   // fused one-row path keeps the quantized row in LDS/registers

// Fused product for a few tokens streaming the weights row by row (every
// segment of sa in one launch); fits when the tokens' codes fit in LDS.  The
// kernel supports up to 8 tokens; the dispatch uses it where it was measured
// faster than quantizer + matrix-core kernel: 2 tokens.
constexpr int64_t kLinearTokensMaxM = 2;
// Block FP8 rows longer than 8 KiB measured slower here than on the staged
// path (Qwen3-8B layer at two tokens with down on this kernel: 0.261-0.265
// against 0.249-0.250 ms per 4 layers), and so did calls streaming more than
// 64 MB of weights (the gate/up pair), where the quantizer launch is amortized
// and the matrix-core kernel streams faster.
inline bool linear_tokens_fits(int variant, int64_t M, int64_t K, int64_t rows) {
    const int64_t kc = (K + 1023) / 1024;
    if (variant == VAR_FP8_BLOCK && kc > 8) return false;
    if (rows * K > (int64_t(64) << 20)) return false;
    return M >= 2 && M <= kLinearTokensMaxM && kc <= 16 && kLinearTokensMaxM * kc <= 64;
}
hipError_t launch_linear_tokens(int variant, const uint16_t* x, int64_t M, int64_t K, const SegmentArgs& sa, int mode,
                                uint8_t* qx, float* sx, hipStream_t st);

// Fused product for up to kSmallFusedMaxM tokens of up to kSmallFusedMaxK
// inputs on the small-M matrix-core kernel: every workgroup rounds the tokens
// into its LDS (dynamic: kSmallFusedScaleBytes of scales, then per token K
// rounded up to a 128-byte step + 64 bytes of codes), so no quantizer launch
// precedes it.
constexpr int64_t kSmallFusedMaxM = 4;
constexpr int64_t kSmallFusedMaxK = 4096;
constexpr int kSmallFusedChunks = (int)(kSmallFusedMaxK / 8 / 64);   // bf16 chunks per lane and token
constexpr int kSmallFusedGroups = (int)(kSmallFusedMaxK / 128);     // 128-input groups per token
constexpr int kSmallFusedScaleBytes = (int)kSmallFusedMaxM * kSmallFusedGroups * 4;
inline size_t small_fused_lds_bytes(int64_t M, int64_t K) {
    return (size_t)kSmallFusedScaleBytes + (size_t)M * (size_t)(((K + 127) & ~int64_t(127)) + 64);
}
// Longer rows (the down projections) measured slower rounded inside every
// workgroup than with the quantizer launch before the kernel.
inline bool small_fused_fits(int64_t M, int64_t K) {
    return M >= 1 && M <= kSmallFusedMaxM && K <= kSmallFusedMaxK;
}
hipError_t launch_gemm_small_fused(int variant, const uint16_t* x, int64_t M, int64_t K, const SegmentArgs& sa,
                                   int mode, uint8_t* qx_out, float* sx_out, hipStream_t st);

// Weight-only ("equivalent") numerics: bf16 activations times dequantized
// weights, every segment of sa in one launch.  M <= 32.
constexpr int64_t kWeightOnlyRowMaxK = 16384;   // one-token kernel keeps the bf16 row in LDS
hipError_t launch_weight_only(int variant, const uint16_t* x, int64_t M, int64_t K, const SegmentArgs& sa, int mode,
                              hipStream_t st);

int gemv_rows_per_wave(int64_t N, int64_t K);

// qlin_linear with its arguments: validation, then the launch form the call
// takes (defined with the C ABI).  linear_is_one_launch: the call runs as one
// launch and needs no staging buffers.
bool linear_is_one_launch(qlin_scheme scheme, int64_t M, int64_t K, const qlin_segment* segments, int32_t nseg);
// Every check of qlin_linear except those of the staging buffers; *noop when
// the call has nothing to do.
qlin_status linear_validate(qlin_scheme scheme, const uint16_t* x, int64_t M, int64_t K, const qlin_segment* segments,
                            int32_t nseg, qlin_out out, bool* noop);
qlin_status linear_call(qlin_scheme scheme, const uint16_t* x, int64_t M, int64_t K, const qlin_segment* segments,
                        int32_t nseg, qlin_out out, void* q_x, float* s_x, hipStream_t stream);
int small_waves_per_tile(int64_t N, int64_t K);

}  // namespace qlin
