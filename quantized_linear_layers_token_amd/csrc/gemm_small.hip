// Products for up to 32 tokens on the matrix cores (W8A8 model card and Qwen3
// 8B FP8 card, "Loading": inputs of at most 32 rows go to the matrix units).
//
// The weights dominate the traffic (arithmetic intensity <= 2M ops/byte), so
// the kernel is a weight stream: every weight byte is loaded from HBM once,
// straight into MFMA operand registers (no LDS staging).
//
//   workgroup = one tile of 16 weight rows (output channels) x the full K,
//               split over NW wavefronts along K (each owns a contiguous run
//               of 128-byte K steps);
//   MFMA      = A: 16 weight rows x 128 bytes of K, B: 128 bytes of K x 16
//               tokens, C[n][m] (4 rows of one token column per lane).
//               int8: two v_mfma_i32_16x16x64_i8 per step; E4M3: one
//               v_mfma_f32_16x16x128_f8f6f4 per step.  Lane l supplies the 32
//               contiguous bytes [32 (l/16), 32 (l/16) + 32) of the step for
//               row (or token) l % 16 of both operands; since both operands
//               use the same byte-to-slot assignment the contraction is
//               unchanged by it.
//   block FP8 = a step is exactly one 128-wide K block: the step's MFMA
//               result is scaled by s_x[m, kb] * s_w[n/128, kb] (one factor
//               per lane, as a lane's four rows share one 128-row block) and
//               added to the f32 accumulator (Qwen3 8B FP8 card: per-block
//               weight scales, per-128-input activation scales).
//   split-K   = the NW partial tiles are summed through LDS, then the scale
//               epilogue writes y.
#include "qlin_device.h"
#include "qlin_internal.h"

namespace qlin {

namespace {

constexpr int kSmallUnroll = 4;     // K steps whose loads are issued together

template <int V> struct SmallAcc { typedef v4i T; };
template <> struct SmallAcc<VAR_FP8_ROW> { typedef v4f T; };
template <> struct SmallAcc<VAR_FP8_BLOCK> { typedef v4f T; };

template <int V, int MT, int NW>
__global__ __launch_bounds__(NW * 64) void gemm_small_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint8_t* __restrict__ qw, const uint16_t* __restrict__ sw,
    void* __restrict__ y, int M, int N, int K, int mode) {
    typedef typename SmallAcc<V>::T Acc;
    __shared__ Acc red[NW][MT][kWave];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int r16 = lane & 15;           // weight row / token column within the tile
    const int grp = lane >> 4;           // which 32-byte quarter of a K step
    const int n0 = blockIdx.x * 16;

    const int nsteps = (K + 127) >> 7;
    const int per = (nsteps + NW - 1) / NW;
    const int s_begin = wave * per;
    const int s_end = min(nsteps, s_begin + per);

    // Rows past N or tokens past M re-read a valid row; their outputs are
    // never stored, and A rows / B columns do not mix in the MFMA.
    const int nrow = min(n0 + r16, N - 1);
    const uint8_t* wbase = qw + (int64_t)nrow * K + grp * 32;
    const uint8_t* xbase[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) xbase[t] = qx + (int64_t)min(t * 16 + r16, M - 1) * K + grp * 32;

    const int kbs = K >> 7;
    const uint16_t* swblk = sw + (int64_t)(n0 >> 7) * kbs;  // block FP8: this tile's row block

    Acc acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = Acc{0, 0, 0, 0};

    for (int s0 = s_begin; s0 < s_end; s0 += kSmallUnroll) {
        v4u wa[kSmallUnroll][2], xa[kSmallUnroll][MT][2];
        float fx[kSmallUnroll][MT], fw[kSmallUnroll];
#pragma unroll
        for (int u = 0; u < kSmallUnroll; ++u) {
            const int s = s0 + u;
            const int k = s * 128 + grp * 32;
            const bool ok0 = (s < s_end) && (k < K);
            const bool ok1 = (s < s_end) && (k + 16 < K);
            const v4u* wp = reinterpret_cast<const v4u*>(wbase + (int64_t)s * 128);
            wa[u][0] = ok0 ? __builtin_nontemporal_load(wp) : v4u{0, 0, 0, 0};
            wa[u][1] = ok1 ? __builtin_nontemporal_load(wp + 1) : v4u{0, 0, 0, 0};
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const v4u* xp = reinterpret_cast<const v4u*>(xbase[t] + (int64_t)s * 128);
                xa[u][t][0] = ok0 ? xp[0] : v4u{0, 0, 0, 0};
                xa[u][t][1] = ok1 ? xp[1] : v4u{0, 0, 0, 0};
            }
            if constexpr (V == VAR_FP8_BLOCK) {
                const int sb = min(s, s_end - 1);
                fw[u] = bf16_lo(swblk[sb]);
#pragma unroll
                for (int t = 0; t < MT; ++t) fx[u][t] = sx[(int64_t)min(t * 16 + r16, M - 1) * kbs + sb];
            }
        }
#pragma unroll
        for (int u = 0; u < kSmallUnroll; ++u) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if constexpr (V == VAR_INT8) {
                    acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                        __builtin_bit_cast(v4i, wa[u][0]), __builtin_bit_cast(v4i, xa[u][t][0]), acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                        __builtin_bit_cast(v4i, wa[u][1]), __builtin_bit_cast(v4i, xa[u][t][1]), acc[t], 0, 0, 0);
                } else {
                    const v8i a = v8i{(int)wa[u][0].x, (int)wa[u][0].y, (int)wa[u][0].z, (int)wa[u][0].w,
                                      (int)wa[u][1].x, (int)wa[u][1].y, (int)wa[u][1].z, (int)wa[u][1].w};
                    const v8i b = v8i{(int)xa[u][t][0].x, (int)xa[u][t][0].y, (int)xa[u][t][0].z, (int)xa[u][t][0].w,
                                      (int)xa[u][t][1].x, (int)xa[u][t][1].y, (int)xa[u][t][1].z, (int)xa[u][t][1].w};
                    if constexpr (V == VAR_FP8_ROW) {
                        acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[t], 0, 0, 0, 0, 0, 0);
                    } else {
                        const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            a, b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                        if (s0 + u < s_end) {
                            const float f = fx[u][t] * fw[u];
                            acc[t].x = __builtin_fmaf(p.x, f, acc[t].x);
                            acc[t].y = __builtin_fmaf(p.y, f, acc[t].y);
                            acc[t].z = __builtin_fmaf(p.z, f, acc[t].z);
                            acc[t].w = __builtin_fmaf(p.w, f, acc[t].w);
                        }
                    }
                }
            }
        }
    }

#pragma unroll
    for (int t = 0; t < MT; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();

    // Sum the NW partial tiles; thread (t, lane) finishes token column t*16 + lane%16.
    if (threadIdx.x < MT * kWave) {
        const int t = threadIdx.x >> 6;
        Acc sum = red[0][t][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) sum += red[w][t][lane];
        const int m = t * 16 + r16;
        if (m < M) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int n = n0 + grp * 4 + r;
                if (n < N) {
                    const int64_t idx = (int64_t)m * N + n;
                    if constexpr (V == VAR_INT8) store_rowwise_i32acc(y, idx, sum[r], sx[m], sw[n], mode);
                    else if constexpr (V == VAR_FP8_ROW) store_f32(y, idx, sum[r] * (sx[m] * bf16_lo(sw[n])), mode);
                    else store_f32(y, idx, sum[r], mode);
                }
            }
        }
    }
}

template <int V, int MT>
void launch_mt(int nw, dim3 grid, hipStream_t st, const uint8_t* qx, const float* sx, const uint8_t* qw,
               const uint16_t* sw, void* y, int M, int N, int K, int mode) {
    if (nw >= 16)
        hipLaunchKernelGGL((gemm_small_kernel<V, MT, 16>), grid, dim3(16 * 64), 0, st, qx, sx, qw, sw, y, M, N, K, mode);
    else if (nw >= 8)
        hipLaunchKernelGGL((gemm_small_kernel<V, MT, 8>), grid, dim3(8 * 64), 0, st, qx, sx, qw, sw, y, M, N, K, mode);
    else
        hipLaunchKernelGGL((gemm_small_kernel<V, MT, 4>), grid, dim3(4 * 64), 0, st, qx, sx, qw, sw, y, M, N, K, mode);
}

}  // namespace

// K-split depth: enough waves for >= 2048 in flight, bounded by the K steps.
int small_waves_per_tile(int64_t N, int64_t K) {
    const int64_t tiles = (N + 15) / 16;
    const int64_t steps = (K + 127) / 128;
    int nw = 4;
    while (nw < 16 && tiles * nw < 2048 && steps >= 2 * nw * kSmallUnroll) nw *= 2;
    return nw;
}

hipError_t launch_gemm_small(int variant, const uint8_t* qx, const float* sx, const uint8_t* qw,
                             const uint16_t* sw, void* y, int64_t M, int64_t N, int64_t K, int mode,
                             hipStream_t st) {
    dim3 grid((unsigned)((N + 15) / 16));
    const int nw = small_waves_per_tile(N, K);
    const int m = (int)M, n = (int)N, k = (int)K;
    const bool two = M > 16;
#define QLIN_SMALL(VV)                                                          \
    do {                                                                        \
        if (two) launch_mt<VV, 2>(nw, grid, st, qx, sx, qw, sw, y, m, n, k, mode); \
        else launch_mt<VV, 1>(nw, grid, st, qx, sx, qw, sw, y, m, n, k, mode);     \
    } while (0)
    if (variant == VAR_INT8) QLIN_SMALL(VAR_INT8);
    else if (variant == VAR_FP8_ROW) QLIN_SMALL(VAR_FP8_ROW);
    else QLIN_SMALL(VAR_FP8_BLOCK);
#undef QLIN_SMALL
    return hipGetLastError();
}

}  // namespace qlin
