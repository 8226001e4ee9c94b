// One-token products (M = 1): each weight byte is read from HBM exactly once.
//
// W8A8 model card, "Loading" (and the Qwen3 8B FP8 card's "Loading" for the
// FP8 weights): a single input row is served by a kernel that touches every
// weight byte exactly once.
//
// Layout of the work: a wavefront owns R consecutive weight rows.  Lane l of
// the wave reads bytes [1024 j + 16 l, 1024 j + 16 l + 16) of each row for
// j = 0 .. KC-1 with 16-byte (dwordx4) loads, so each wave load instruction
// covers 1 KiB of one row, fully coalesced.  The matching 16-byte slices of
// the activation row are loaded once per wave into registers and reused for
// all R rows.  int8: v_dot4_i32_i8 (four int8 products summed into int32 per
// instruction); E4M3: pairs decoded to f32 with v_cvt_pk_f32_fp8 and summed
// with FMAs.  The per-lane partial sums are reduced across the wave with DPP.
#include "qlin_device.h"
#include "qlin_internal.h"
#include "qlin_rows.h"

namespace qlin {

namespace {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;

// V: VAR_INT8 / VAR_FP8_ROW / VAR_FP8_BLOCK.  KC: 1 KiB chunks per row held in
// registers (K <= 1024 KC).  R: rows per wave.
template <int V, int KC, int R>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint8_t* __restrict__ qw, const uint16_t* __restrict__ sw,
    void* __restrict__ y, int N, int K, int mode) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform row bookkeeping
    const int64_t n0 = ((int64_t)blockIdx.x * kGemvWaves + wave) * R;
    if (n0 >= N) return;                       // the whole wave leaves together

    const int k16 = K >> 4;                    // 16-byte slices per row
    // Weights first, branch-free: slices past K re-read the row's last slice
    // and meet zero activation slices; tail rows re-read the last row (not stored).
    v4u wr[R][KC];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t n = min(n0 + r, (int64_t)N - 1);
        const v4u* wrow = reinterpret_cast<const v4u*>(qw + n * K);
#pragma unroll
        for (int j = 0; j < KC; ++j) wr[r][j] = __builtin_nontemporal_load(wrow + min(j * kWave + lane, k16 - 1));
    }
    const v4u* xv = reinterpret_cast<const v4u*>(qx);
    v4u xr[KC];
#pragma unroll
    for (int j = 0; j < KC; ++j) {
        const int o = j * kWave + lane;
        const v4u v = xv[min(o, k16 - 1)];
        xr[j] = (o < k16) ? v : v4u{0, 0, 0, 0};
    }

    if constexpr (V == VAR_INT8) {
        int acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int a = 0;
#pragma unroll
            for (int j = 0; j < KC; ++j) a = dot16_i8(wr[r][j], xr[j], a);
            acc[r] = wave_sum_i32(a);
        }
        if (lane < R && n0 + lane < N) {
            int a = acc[0];
#pragma unroll
            for (int r = 1; r < R; ++r) a = (lane == r) ? acc[r] : a;
            const int64_t n = n0 + lane;
            store_rowwise_i32acc(y, n, a, sx[0], sw[n], mode);
        }
    } else {
        float acc[R];
        const int kbs = K >> 7;                // 128-wide K blocks per row
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float a = 0.0f;
            if constexpr (V == VAR_FP8_BLOCK) {
                const int64_t n = min(n0 + r, (int64_t)N - 1);
                const uint16_t* swr = sw + (n >> 7) * kbs;
#pragma unroll
                for (int j = 0; j < KC; ++j) {
                    const int kb = min(j * kWave + lane, k16 - 1) >> 3;  // 8 slices of 16 bytes per block
                    const float f = sx[kb] * bf16_lo(swr[kb]);
                    a = __builtin_fmaf(dot16_e4m3(wr[r][j], xr[j]), f, a);
                }
            } else {
#pragma unroll
                for (int j = 0; j < KC; ++j) a += dot16_e4m3(wr[r][j], xr[j]);
            }
            acc[r] = wave_sum_f32(a);
        }
        if (lane < R && n0 + lane < N) {
            float a = acc[0];
#pragma unroll
            for (int r = 1; r < R; ++r) a = (lane == r) ? acc[r] : a;
            const int64_t n = n0 + lane;
            if constexpr (V == VAR_FP8_BLOCK) {
                store_f32(y, n, a, mode);
            } else {
                const float sc = sx[0] * bf16_lo(sw[n]);
                store_f32(y, n, a * sc, mode);
            }
        }
    }
}

// Rows longer than 16 KiB: the row is walked in 16 KiB segments; the
// activation slices are reloaded per segment (from L1/L2).
template <int V, int R>
__global__ __launch_bounds__(kGemvThreads) void gemv_loop_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint8_t* __restrict__ qw, const uint16_t* __restrict__ sw,
    void* __restrict__ y, int N, int K, int mode) {
    constexpr int KC = 16;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n0 = ((int64_t)blockIdx.x * kGemvWaves + wave) * R;
    if (n0 >= N) return;
    const int k16 = K >> 4;
    const int kbs = K >> 7;
    const v4u* xv = reinterpret_cast<const v4u*>(qx);
    int iacc[R];
    float facc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) { iacc[r] = 0; facc[r] = 0.0f; }
    for (int seg = 0; seg < k16; seg += KC * kWave) {
        v4u xr[KC];
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            const int o = seg + j * kWave + lane;
            xr[j] = (o < k16) ? xv[o] : v4u{0, 0, 0, 0};
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t n = min(n0 + r, (int64_t)N - 1);
            const v4u* wrow = reinterpret_cast<const v4u*>(qw + n * K);
            v4u wr[KC];
#pragma unroll
            for (int j = 0; j < KC; ++j) {
                const int o = seg + j * kWave + lane;
                wr[j] = (o < k16) ? __builtin_nontemporal_load(wrow + o) : v4u{0, 0, 0, 0};
            }
#pragma unroll
            for (int j = 0; j < KC; ++j) {
                const int o = seg + j * kWave + lane;
                if constexpr (V == VAR_INT8) {
                    iacc[r] = dot16_i8(wr[j], xr[j], iacc[r]);
                } else if constexpr (V == VAR_FP8_BLOCK) {
                    if (o < k16) {
                        const int kb = o >> 3;
                        const float f = sx[kb] * bf16_lo(sw[(n >> 7) * kbs + kb]);
                        facc[r] = __builtin_fmaf(dot16_e4m3(wr[j], xr[j]), f, facc[r]);
                    }
                } else {
                    facc[r] += dot16_e4m3(wr[j], xr[j]);
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if constexpr (V == VAR_INT8) iacc[r] = wave_sum_i32(iacc[r]);
        else facc[r] = wave_sum_f32(facc[r]);
    }
    if (lane < R && n0 + lane < N) {
        const int64_t n = n0 + lane;
        int ia = iacc[0];
        float fa = facc[0];
#pragma unroll
        for (int r = 1; r < R; ++r) {
            ia = (lane == r) ? iacc[r] : ia;
            fa = (lane == r) ? facc[r] : fa;
        }
        if constexpr (V == VAR_INT8) store_rowwise_i32acc(y, n, ia, sx[0], sw[n], mode);
        else if constexpr (V == VAR_FP8_BLOCK) store_f32(y, n, fa, mode);
        else store_f32(y, n, fa * (sx[0] * bf16_lo(sw[n])), mode);
    }
}

template <int V, int KC>
void launch_kc(int R, dim3 grid, hipStream_t st, const uint8_t* qx, const float* sx, const uint8_t* qw,
               const uint16_t* sw, void* y, int N, int K, int mode) {
    dim3 block(kGemvThreads);
    if (R >= 4) hipLaunchKernelGGL((gemv_kernel<V, KC, 4>), grid, block, 0, st, qx, sx, qw, sw, y, N, K, mode);
    else if (R == 2) hipLaunchKernelGGL((gemv_kernel<V, KC, 2>), grid, block, 0, st, qx, sx, qw, sw, y, N, K, mode);
    else hipLaunchKernelGGL((gemv_kernel<V, KC, 1>), grid, block, 0, st, qx, sx, qw, sw, y, N, K, mode);
}

}  // namespace

// Rows per wave: as many as keep >= 2048 waves in flight (8 per CU) while the
// weight registers (R * KC * 4 VGPRs) stay within 64.
int gemv_rows_per_wave(int64_t N, int64_t K) {
    const int64_t kc = (K + 1023) / 1024;
    for (int R = 4; R > 1; R /= 2)
        if (N / R >= 2048 && R * kc <= 16) return R;
    return 1;
}

hipError_t launch_gemv(int variant, const uint8_t* qx, const float* sx, const uint8_t* qw, const uint16_t* sw,
                       void* y, int64_t N, int64_t K, int mode, hipStream_t st) {
    const int64_t kc = (K + 1023) / 1024;
    int R = gemv_rows_per_wave(N, K);
    if (kc > 16) R = 1;
    const int64_t waves = (N + R - 1) / R;
    dim3 grid((unsigned)((waves + kGemvWaves - 1) / kGemvWaves));
    const int n = (int)N, k = (int)K;
#define QLIN_GEMV_KC(VV)                                                                  \
    do {                                                                                  \
        if (kc <= 1) launch_kc<VV, 1>(R, grid, st, qx, sx, qw, sw, y, n, k, mode);        \
        else if (kc <= 2) launch_kc<VV, 2>(R, grid, st, qx, sx, qw, sw, y, n, k, mode);   \
        else if (kc <= 4) launch_kc<VV, 4>(R, grid, st, qx, sx, qw, sw, y, n, k, mode);   \
        else if (kc <= 8) launch_kc<VV, 8>(R, grid, st, qx, sx, qw, sw, y, n, k, mode);   \
        else if (kc <= 12) launch_kc<VV, 12>(R, grid, st, qx, sx, qw, sw, y, n, k, mode); \
        else if (kc <= 14) launch_kc<VV, 14>(R, grid, st, qx, sx, qw, sw, y, n, k, mode); \
        else if (kc <= 16) launch_kc<VV, 16>(R, grid, st, qx, sx, qw, sw, y, n, k, mode); \
        else hipLaunchKernelGGL((gemv_loop_kernel<VV, 1>), grid, dim3(kGemvThreads), 0, st, qx, sx, qw, sw, y, n, k, mode); \
    } while (0)
    if (variant == VAR_INT8) QLIN_GEMV_KC(VAR_INT8);
    else if (variant == VAR_FP8_ROW) QLIN_GEMV_KC(VAR_FP8_ROW);
    else QLIN_GEMV_KC(VAR_FP8_BLOCK);
#undef QLIN_GEMV_KC
    return hipGetLastError();
}

}  // namespace qlin
