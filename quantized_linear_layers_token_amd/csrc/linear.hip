// Fused projection: bf16 activations in, quantized product out, in one launch
// at M = 1; several weight segments that read the same input (q/k/v, or
// gate/up) are served by the same launch and the same activation rounding.
//
// The activation row is quantized cooperatively by every workgroup (W8A8 model
// card, intro: activations quantized to int8 per token; FP8-dynamic README,
// "Creation": per-token dynamic E4M3; Qwen3 8B FP8 card, "Loading": E4M3 per
// 128 inputs): 256 threads load the bf16 row once, reduce the absmax (DPP
// inside a wavefront, LDS across the four), round into an LDS copy of the
// quantized row, and each wavefront then holds its 16-byte slices of that row
// in registers.  The arithmetic of the rounding is the standalone quantizers'
// (same divides, same rounding), so every workgroup produces the same codes.
//
// Weight rows are then streamed exactly as in the one-row product: the
// concatenated rows of all segments are split evenly over the wavefronts of the
// grid; each wavefront reads R rows at a time with 16-byte non-temporal loads
// (one wave instruction = 1 KiB of one row) and reduces with DPP.
//
// SwiGLU mode (SG): segments 0 and 1 are the gate and up weights of one MLP;
// the work items are the intermediate indices j, a wavefront reads gate row j
// and up row j together and writes h[j] = swiglu_bf16(gate_j, up_j), the bf16
// input of the down projection.
#include "qlin_device.h"
#include "qlin_internal.h"

namespace qlin {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t chunk_absmax(const v4u& v) {
    uint32_t a = v.x & 0x7FFF7FFFu, b = v.y & 0x7FFF7FFFu;
    uint32_t c = v.z & 0x7FFF7FFFu, d = v.w & 0x7FFF7FFFu;
    uint32_t m0 = max(a & 0xFFFFu, a >> 16), m1 = max(b & 0xFFFFu, b >> 16);
    uint32_t m2 = max(c & 0xFFFFu, c >> 16), m3 = max(d & 0xFFFFu, d >> 16);
    return max(max(m0, m1), max(m2, m3));
}

template <bool FP8>
__device__ __forceinline__ void scales_from_absmax(uint32_t amax_bits, float& s, float& inv) {
    const float q = FP8 ? 448.0f : 127.0f;
    const float a = __uint_as_float(amax_bits << 16);
    s = a / q;
    inv = (amax_bits == 0) ? 0.0f : q / a;
}

__device__ __forceinline__ uint32_t q4_int8(uint32_t w0, uint32_t w1, float inv) {
    auto q = [inv](float v) {
        float t = __builtin_rintf(v * inv);
        t = fminf(fmaxf(t, -127.0f), 127.0f);
        return (uint32_t)(uint8_t)(int8_t)(int)t;
    };
    return q(bf16_lo(w0)) | (q(bf16_hi(w0)) << 8) | (q(bf16_lo(w1)) << 16) | (q(bf16_hi(w1)) << 24);
}

__device__ __forceinline__ uint32_t q4_fp8(uint32_t w0, uint32_t w1, float inv) {
    auto c = [inv](float v) { return fminf(fmaxf(v * inv, -448.0f), 448.0f); };
    const uint32_t lo = e4m3_pack_lo(c(bf16_lo(w0)), c(bf16_hi(w0)));
    return e4m3_pack_hi(lo, c(bf16_lo(w1)), c(bf16_hi(w1)));
}

template <bool FP8>
__device__ __forceinline__ v2u quant8(const v4u& v, float inv) {
    if constexpr (FP8) return v2u{q4_fp8(v.x, v.y, inv), q4_fp8(v.z, v.w, inv)};
    else return v2u{q4_int8(v.x, v.y, inv), q4_int8(v.z, v.w, inv)};
}

__device__ __forceinline__ int dot16_i8(const v4u& w, const v4u& x, int acc) {
    acc = __builtin_amdgcn_sdot4((int)w.x, (int)x.x, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.y, (int)x.y, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.z, (int)x.z, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.w, (int)x.w, acc, false);
    return acc;
}

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

// V: scheme; KC: 1 KiB slices per row in registers (K <= 1024 KC); R: rows
// (SG: gate/up row pairs) per wave per iteration; SG: SwiGLU mode.  CPT = bf16
// chunks of 8 per thread for the rounding.
template <int V, int KC, int R, bool SG>
__global__ __launch_bounds__(kThreads) void linear_decode_kernel(
    const uint16_t* __restrict__ x, int K, SegmentArgs sa, int mode,
    uint8_t* __restrict__ qx_out, float* __restrict__ sx_out) {
    constexpr bool FP8 = V != VAR_INT8;
    constexpr int CPT = (KC + 1) / 2;
    constexpr int RL = SG ? 2 * R : R;   // weight rows loaded per iteration
    __shared__ uint32_t red[kThreads / kWave];
    __shared__ __attribute__((aligned(16))) uint8_t xq[KC * 1024];
    __shared__ float gsc[KC * 8];   // block scheme: one scale per 128-input group

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: row bookkeeping stays scalar
    const int nchunks = K >> 3;
    const int k16 = K >> 4;

    // ---- load the bf16 row (chunk c = tid + 256 j), then the first weight rows.
    // Loads past the end of a row re-read its last chunk instead of branching
    // (branch-free loads keep the wait counts exact): a re-read bf16 chunk does
    // not change the absmax and is never stored; a re-read weight slice meets a
    // zero activation slice, so it adds nothing.
    v4u xb[CPT];
    const v4u* xv = reinterpret_cast<const v4u*>(x);
#pragma unroll
    for (int j = 0; j < CPT; ++j) xb[j] = xv[min(tid + j * kThreads, nchunks - 1)];

    const int ntot = SG ? sa.start[1] : sa.start[sa.nseg];   // work items: rows, or gate/up pairs
    const int W = gridDim.x * (kThreads / kWave);
    const int w = blockIdx.x * (kThreads / kWave) + wave;
    const int rb = (int)((int64_t)ntot * w / W);
    const int re = (int)((int64_t)ntot * (w + 1) / W);

    auto seg_of = [&](int r) {
        int i = 0;
#pragma unroll
        for (int t = 1; t < kMaxSegments; ++t) i += (t < sa.nseg && r >= sa.start[t]) ? 1 : 0;
        return i;
    };
    // loaded row r of the group at work item n0: its segment and row within it
    // (items past the wave's range re-read a valid row)
    auto row_of = [&](int r, int n0, int& i, int& local) {
        if constexpr (SG) {
            local = max(min(n0 + r / 2, re - 1), 0);
            i = r & 1;
        } else {
            const int n = max(min(n0 + r, re - 1), 0);
            i = seg_of(n);
            local = n - sa.start[i];
        }
    };
    auto load_rows = [&](v4u (&dst)[RL][KC], int n0) {
#pragma unroll
        for (int r = 0; r < RL; ++r) {
            int i, local;
            row_of(r, n0, i, local);
            const v4u* wrow = reinterpret_cast<const v4u*>(sa.w[i] + (int64_t)local * K);
#pragma unroll
            for (int j = 0; j < KC; ++j) dst[r][j] = __builtin_nontemporal_load(wrow + min(j * kWave + lane, k16 - 1));
        }
    };
    v4u cur[RL][KC];
    load_rows(cur, rb);     // unconditional: the rounding below only waits for the bf16 row

    // ---- activation rounding into LDS
    if constexpr (V == VAR_FP8_BLOCK) {
        // chunk c belongs to group c / 16: sixteen consecutive threads of one DPP row
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = tid + j * kThreads;
            const uint32_t amax = row_max_u32(chunk_absmax(xb[j]));
            float sg, inv;
            scales_from_absmax<true>(amax, sg, inv);
            if (c < nchunks) {
                *reinterpret_cast<v2u*>(xq + c * 8) = quant8<true>(xb[j], inv);
                if ((tid & 15) == 0) gsc[c >> 4] = sg;
            }
        }
    } else {
        uint32_t amax = 0;
#pragma unroll
        for (int j = 0; j < CPT; ++j) amax = max(amax, chunk_absmax(xb[j]));
        amax = wave_max_u32(amax);
        if (lane == 0) red[wave] = amax;
        __syncthreads();
        amax = max(max(red[0], red[1]), max(red[2], red[3]));
        float s, inv;
        scales_from_absmax<FP8>(amax, s, inv);
        if (tid == 0) gsc[0] = s;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = tid + j * kThreads;
            if (c < nchunks) *reinterpret_cast<v2u*>(xq + c * 8) = quant8<FP8>(xb[j], inv);
        }
    }
    __syncthreads();

    if (qx_out != nullptr && blockIdx.x == 0) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = tid + j * kThreads;
            if (c < nchunks) *reinterpret_cast<v2u*>(qx_out + c * 8) = *reinterpret_cast<const v2u*>(xq + c * 8);
        }
        if constexpr (V == VAR_FP8_BLOCK) {
            if (tid < (K >> 7)) sx_out[tid] = gsc[tid];
            for (int g = tid + kThreads; g < (K >> 7); g += kThreads) sx_out[g] = gsc[g];
        } else {
            if (tid == 0) sx_out[0] = gsc[0];
        }
    }

    v4u xr[KC];
#pragma unroll
    for (int j = 0; j < KC; ++j) {
        const int o = j * kWave + lane;
        xr[j] = (o < k16) ? *reinterpret_cast<const v4u*>(xq + o * 16) : v4u{0, 0, 0, 0};
    }
    const float s_tok = gsc[0];
    const int kbs = K >> 7;

    // ---- stream the weight rows: the first group was loaded before the rounding
    auto process = [&](const v4u (&wr)[RL][KC], int n0) {
        float facc[RL];
        int iacc[RL];
#pragma unroll
        for (int r = 0; r < RL; ++r) {
            if constexpr (V == VAR_INT8) {
                int a = 0;
#pragma unroll
                for (int j = 0; j < KC; ++j) a = dot16_i8(wr[r][j], xr[j], a);
                iacc[r] = wave_sum_i32(a);
            } else if constexpr (V == VAR_FP8_ROW) {
                float a = 0.0f;
#pragma unroll
                for (int j = 0; j < KC; ++j) a += dot16_e4m3(wr[r][j], xr[j]);
                facc[r] = wave_sum_f32(a);
            } else {
                int i, local;
                row_of(r, n0, i, local);
                const uint16_t* swr = sa.sw[i] + (int64_t)(local >> 7) * kbs;
                float a = 0.0f;
#pragma unroll
                for (int j = 0; j < KC; ++j) {
                    const int kb = min(j * kWave + lane, k16 - 1) >> 3;   // slices past K: zero activations
                    a = __builtin_fmaf(dot16_e4m3(wr[r][j], xr[j]), gsc[kb] * bf16_lo(swr[kb]), a);
                }
                facc[r] = wave_sum_f32(a);
            }
        }
        if constexpr (SG) {
            if (lane < R && n0 + lane < re) {
                const int j = n0 + lane;
                float g = 0.0f, u = 0.0f;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (lane != r) continue;
                    if constexpr (V == VAR_INT8) {
                        g = (float)iacc[2 * r] * (s_tok * bf16_lo(sa.sw[0][j]));
                        u = (float)iacc[2 * r + 1] * (s_tok * bf16_lo(sa.sw[1][j]));
                    } else if constexpr (V == VAR_FP8_ROW) {
                        g = facc[2 * r] * (s_tok * bf16_lo(sa.sw[0][j]));
                        u = facc[2 * r + 1] * (s_tok * bf16_lo(sa.sw[1][j]));
                    } else {
                        g = facc[2 * r];
                        u = facc[2 * r + 1];
                    }
                }
                static_cast<uint16_t*>(sa.y[0])[j] = swiglu_bf16(g, u);
            }
            return;
        }
        if (lane < R && n0 + lane < re) {
            const int n = n0 + lane;
            const int i = seg_of(n);
            const int64_t local = n - sa.start[i];
            if constexpr (V == VAR_INT8) {
                int a = iacc[0];
#pragma unroll
                for (int r = 1; r < R; ++r) a = (lane == r) ? iacc[r] : a;
                store_rowwise_i32acc(sa.y[i], local, a, s_tok, sa.sw[i][local], mode);
            } else {
                float a = facc[0];
#pragma unroll
                for (int r = 1; r < R; ++r) a = (lane == r) ? facc[r] : a;
                if constexpr (V == VAR_FP8_ROW) store_f32(sa.y[i], local, a * (s_tok * bf16_lo(sa.sw[i][local])), mode);
                else store_f32(sa.y[i], local, a, mode);
            }
        }
    };
    if (rb < re) process(cur, rb);
    for (int n0 = rb + R; n0 < re; n0 += R) {
        load_rows(cur, n0);
        process(cur, n0);
    }
}

template <int V, int KC>
void launch_kc(int R, int grid, hipStream_t st, const uint16_t* x, int K, const SegmentArgs& sa, int mode,
               uint8_t* qx, float* sx) {
    if (mode == OUT_SWIGLU)
        hipLaunchKernelGGL((linear_decode_kernel<V, KC, 1, true>), dim3(grid), dim3(kThreads), 0, st, x, K, sa, mode,
                           qx, sx);
    else if constexpr (KC > 4 && KC <= 8) {   // the only row lengths read two rows at a time
        if (R >= 2)
            hipLaunchKernelGGL((linear_decode_kernel<V, KC, 2, false>), dim3(grid), dim3(kThreads), 0, st, x, K, sa,
                               mode, qx, sx);
        else
            hipLaunchKernelGGL((linear_decode_kernel<V, KC, 1, false>), dim3(grid), dim3(kThreads), 0, st, x, K, sa,
                               mode, qx, sx);
    } else
        hipLaunchKernelGGL((linear_decode_kernel<V, KC, 1, false>), dim3(grid), dim3(kThreads), 0, st, x, K, sa, mode,
                           qx, sx);
}

}  // namespace

// Launch shape (compared on one MI355X over the Llama-3.1-8B decode step):
// rows of up to 4 KiB: one row per wavefront (the most workgroups, every load
// issued at once); up to 8 KiB: two rows per wavefront read together; longer
// rows: two rows per wavefront read one after the other (R = 1).
// SwiGLU mode: a wavefront reads one gate/up row pair at a time (two rows in
// flight), one pair per wavefront for rows up to 4 KiB, else two in turn.
void decode_launch_shape(int64_t ntot, int64_t K, int* R, int* grid) {
    const int64_t kc = (K + 1023) / 1024;
    *R = (kc > 4 && kc <= 8) ? 2 : 1;
    const int64_t rows = 4 * (kc <= 4 ? 1 : 2);         // rows per workgroup of four wavefronts
    const int64_t g = (ntot + rows - 1) / rows;
    *grid = (int)(g < 1 ? 1 : g);
}

hipError_t launch_linear_decode(int variant, const uint16_t* x, int64_t K, const SegmentArgs& sa, int mode,
                                uint8_t* qx, float* sx, hipStream_t st) {
    const int64_t ntot = mode == OUT_SWIGLU ? sa.start[1] : sa.start[sa.nseg];
    int R, grid;
    decode_launch_shape(ntot, K, &R, &grid);
    const int64_t kc = (K + 1023) / 1024;
    const int k = (int)K;
#define QLIN_DEC(VV)                                                              \
    do {                                                                          \
        if (kc <= 1) launch_kc<VV, 1>(R, grid, st, x, k, sa, mode, qx, sx);       \
        else if (kc <= 2) launch_kc<VV, 2>(R, grid, st, x, k, sa, mode, qx, sx);  \
        else if (kc <= 4) launch_kc<VV, 4>(R, grid, st, x, k, sa, mode, qx, sx);  \
        else if (kc <= 8) launch_kc<VV, 8>(R, grid, st, x, k, sa, mode, qx, sx);  \
        else if (kc <= 12) launch_kc<VV, 12>(R, grid, st, x, k, sa, mode, qx, sx); \
        else if (kc <= 14) launch_kc<VV, 14>(R, grid, st, x, k, sa, mode, qx, sx); \
        else launch_kc<VV, 16>(R, grid, st, x, k, sa, mode, qx, sx);              \
    } while (0)
    if (variant == VAR_INT8) QLIN_DEC(VAR_INT8);
    else if (variant == VAR_FP8_ROW) QLIN_DEC(VAR_FP8_ROW);
    else QLIN_DEC(VAR_FP8_BLOCK);
#undef QLIN_DEC
    return hipGetLastError();
}

}  // namespace qlin
