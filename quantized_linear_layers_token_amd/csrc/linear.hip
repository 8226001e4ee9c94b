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
#include "qlin_rows.h"

namespace qlin {

namespace {

constexpr int kThreads = 256;

// V: scheme; KC: 1 KiB slices per row in registers (K <= 1024 KC); R: rows
// (SG: gate/up row pairs) per wave per iteration; SG: SwiGLU mode.  CPT = bf16
// chunks of 8 per thread for the rounding.
template <int V, int KC, int R, bool SG>
__global__ __launch_bounds__(kThreads) void linear_decode_kernel(
    const uint16_t* __restrict__ x, int K, SegmentArgs sa, int mode,
    uint8_t* __restrict__ qx_out, float* __restrict__ sx_out) {
    constexpr bool FP8 = V != VAR_INT8;
    constexpr int CPT = (128 * KC + kThreads - 1) / kThreads;
    constexpr int RL = SG ? 2 * R : R;   // weight rows loaded per iteration
    constexpr int SL = KC;   // 16-byte slots per lane and row
    __shared__ uint32_t red[kThreads / kWave];
    __shared__ __attribute__((aligned(16))) uint8_t xq[SL * 1024];
    __shared__ float gsc[KC * 8];   // block scheme: one scale per 128-input group
    // block scheme, rows of an even number of KiB: each wavefront's 2 KiB chunk of
    // a row, 128-byte groups with their 16-byte pieces rotated by the group index
    constexpr bool BPAIR = V == VAR_FP8_BLOCK && KC % 2 == 0;
    __shared__ __attribute__((aligned(16))) uint8_t wst[BPAIR ? kThreads / kWave : 1][BPAIR ? 2048 : 16];

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

    const int ntot = SG ? sa.start[1] : pick_int(sa.start + 1, sa.nseg - 1);   // work items: rows, or gate/up pairs
    // wave w takes items [rb, re): q or q + 1 of them (the first ntot % W waves
    // one more), in 32-bit arithmetic
    const unsigned W = gridDim.x * (kThreads / kWave);
    const unsigned w = blockIdx.x * (kThreads / kWave) + wave;
    const unsigned q = (unsigned)ntot / W, qr = (unsigned)ntot - q * W;
    const int rb = (int)(w * q + min(w, qr));
    const int re = rb + (int)q + (w < qr ? 1 : 0);

    auto seg_of = [&](int r) {
        int i = 0;
#pragma unroll
        for (int t = 1; t < kMaxSegments; ++t) i += (t < sa.nseg && r >= sa.start[t]) ? 1 : 0;
        return i;
    };
    // 16-byte slot j of a row held by this lane, in units of 16 bytes: one wave
    // load covers the j-th KiB of the row, lane l its bytes at 16 l.
    auto slot = [&](int j) { return j * kWave + lane; };
    // loaded row r of the group at work item n0: its segment and row within it
    // (items past the wave's range re-read a valid row)
    auto row_of = [&](int r, int n0, int& i, int& local) {
        if constexpr (SG) {
            local = max(min(n0 + r / 2, re - 1), 0);
            i = r & 1;
        } else {
            const int n = max(min(n0 + r, re - 1), 0);
            i = seg_of(n);
            local = n - pick_int(sa.start, i);
        }
    };
    // block FP8: with its weights, the row's weight-block scales, lane l holding
    // group l (and 64 + l): at most 128 groups (K <= 16384)
    constexpr int NF = V == VAR_FP8_BLOCK ? (KC > 8 ? 2 : 1) : 1;
    const int kbs = K >> 7;
    auto load_rows = [&](v4u (&dst)[RL][SL], uint32_t (&fsw)[RL][NF], int n0) {
#pragma unroll
        for (int r = 0; r < RL; ++r) {
            int i, local;
            row_of(r, n0, i, local);
            const __attribute__((address_space(1))) v4u* wrow =
                reinterpret_cast<const __attribute__((address_space(1))) v4u*>(pick_global(sa.w, i) + (int64_t)local * K);
#pragma unroll
            for (int j = 0; j < SL; ++j) dst[r][j] = __builtin_nontemporal_load(wrow + min(slot(j), k16 - 1));
            if constexpr (V == VAR_FP8_BLOCK) {
                const __attribute__((address_space(1))) uint16_t* swr = pick_global(sa.sw, i) + (int64_t)(local >> 7) * kbs;
#pragma unroll
                for (int q = 0; q < NF; ++q) fsw[r][q] = swr[min(64 * q + lane, kbs - 1)];
            }
        }
    };
    v4u cur[RL][SL];
    uint32_t fsw[RL][NF];
    load_rows(cur, fsw, rb);     // unconditional: the rounding below only waits for the bf16 row

    // ---- activation rounding into LDS
    if constexpr (V == VAR_FP8_BLOCK) {
        // chunk c belongs to group c / 16: sixteen consecutive threads of one DPP row
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = tid + j * kThreads;
            const uint32_t amax = row_max_u32(chunk_absmax(xb[j]));
            float sg;
            RoundFactor rf;
            scales_from_absmax<true>(amax, sg, rf);
            if (c < nchunks) {
                *reinterpret_cast<v2u*>(xq + c * 8) = quant8<true>(xb[j], rf);
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
        amax = red[0];
#pragma unroll
        for (int i = 1; i < kThreads / kWave; ++i) amax = max(amax, red[i]);
        float s;
        RoundFactor rf;
        scales_from_absmax<FP8>(amax, s, rf);
        if (tid == 0) gsc[0] = s;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = tid + j * kThreads;
            if (c < nchunks) *reinterpret_cast<v2u*>(xq + c * 8) = quant8<FP8>(xb[j], rf);
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

    // The lane's slices of the rounded token stay in registers (int8, FP8
    // rowwise), except for FP8 rowwise rows longer than 8 KiB (XL): there each
    // slice is read from the LDS copy where it is used and a wavefront takes
    // one row, which keeps the kernel at or below 128 registers (four
    // wavefronts per SIMD, every row of the launch in flight).  Measured over
    // the Llama-3.1-8B decode step: FP8 rowwise 1.392 -> 1.376 ms; the same form
    // made int8 slower (1.372 -> 1.387 ms).  Block FP8 reads its (permuted)
    // slices from LDS at every row length (TL), takes the XL form for rows up
    // to 4 KiB (one row per wavefront: 42 registers, eight wavefronts per SIMD
    // instead of six) and keeps two rows per wavefront in turn beyond 8 KiB;
    // its partial products are consumed two at a time.  Qwen3-8B block decode
    // 1.541-1.556 -> 1.502-1.507 ms per token (alternated on one box, outputs
    // bit-identical).
    constexpr bool XL = (KC > 8 && V == VAR_FP8_ROW) || (KC <= 4 && V == VAR_FP8_BLOCK);
    constexpr bool TL = XL || V == VAR_FP8_BLOCK;
    v4u xr[TL ? 1 : SL];
    if constexpr (!TL) {
#pragma unroll
        for (int j = 0; j < SL; ++j) {
            const int o = slot(j);
            xr[j] = (o < k16) ? *reinterpret_cast<const v4u*>(xq + o * 16) : v4u{0, 0, 0, 0};
        }
    }
    const float s_tok = gsc[0];

    // Block FP8 on the matrix cores needs the four lanes of MFMA row i (lanes
    // i, i + 16, i + 32, i + 48) to hold one 128-input group.  Rows of an even
    // number of KiB (BPAIR) pass each 2 KiB chunk through the wavefront's LDS
    // buffer, so row i holds all of group i of the chunk and one MFMA covers
    // 2 KiB; measured against the per-KiB form below, Qwen3-8B block decode
    // 1.513-1.521 -> 1.448-1.457 ms per token (alternated on one box).  Rows of
    // an odd number of KiB: lane l takes (ds_bpermute) the 16 bytes loaded by
    // lane 4 (l % 16) + l / 16, so row i holds bytes [64 i, 64 i + 64) of each
    // KiB, half of group i / 2, one MFMA per KiB with half its K slots zero.
    const int paddr = 4 * (4 * (lane & 15) + (lane >> 4));
    auto bperm = [&](const v4u& v) {
        return v4u{(unsigned)__builtin_amdgcn_ds_bpermute(paddr, (int)v.x),
                   (unsigned)__builtin_amdgcn_ds_bpermute(paddr, (int)v.y),
                   (unsigned)__builtin_amdgcn_ds_bpermute(paddr, (int)v.z),
                   (unsigned)__builtin_amdgcn_ds_bpermute(paddr, (int)v.w)};
    };
    float gx[NF];                  // block FP8: s_x of group l (and 64 + l)
    if constexpr (V == VAR_FP8_BLOCK) {
        if constexpr (!TL) {
#pragma unroll
            for (int j = 0; j < SL; ++j) xr[j] = bperm(xr[j]);
        }
#pragma unroll
        for (int q = 0; q < NF; ++q) gx[q] = gsc[min(64 * q + lane, kbs - 1)];
    }

    // the lane's token slice j (block FP8: the slice lane 4 (l % 16) + l / 16 loaded)
    const int tlane = V == VAR_FP8_BLOCK ? 4 * (lane & 15) + (lane >> 4) : lane;
    auto tok = [&](int j) -> v4u {
        if constexpr (TL) {
            const int o = j * kWave + tlane;
            return (o < k16) ? *reinterpret_cast<const v4u*>(xq + o * 16) : v4u{0, 0, 0, 0};
        } else {
            return xr[j];
        }
    };

    // ---- stream the weight rows: the first group was loaded before the rounding
    auto process = [&](const v4u (&wr)[RL][SL], const uint32_t (&fw)[RL][NF], int n0) {
        float facc[RL];
        int iacc[RL];
#pragma unroll
        for (int r = 0; r < RL; ++r) {
            if constexpr (V == VAR_INT8) {
                int a = 0;
#pragma unroll
                for (int j = 0; j < KC; ++j) a = dot16_i8(wr[r][j], tok(j), a);
                iacc[r] = wave_sum_i32(a);
            } else if constexpr (V == VAR_FP8_ROW) {
                v4f c = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < (SL + 1) / 2; ++q)
                    c = mfma_e4m3(wr[r][2 * q], 2 * q + 1 < SL ? wr[r][2 * q + 1] : v4u{0, 0, 0, 0}, tok(2 * q),
                                  2 * q + 1 < SL ? tok(2 * q + 1) : v4u{0, 0, 0, 0}, c);
                facc[r] = wave_sum_f32(mfma16_diag(c, lane));
            } else if constexpr (BPAIR) {
                // one MFMA per 2 KiB: the chunk goes through this wavefront's LDS
                // buffer so that MFMA row i (lanes i, i + 16, i + 32, i + 48) holds
                // the whole group i of the chunk (lane i + 16 p its bytes 32 p ..
                // 32 p + 31); diagonal element i is then group 16 c + i of the row,
                // scaled by its s_x * s_w (groups past K meet zero activations)
                float f[NF];
#pragma unroll
                for (int h = 0; h < NF; ++h) f[h] = gx[h] * bf16_lo(fw[r][h]);
                uint8_t* const wb = wst[wave];
                const int gi = lane & 15, gp = lane >> 4;
                float a = 0.0f;
#pragma unroll
                for (int c = 0; c < SL / 2; ++c) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int g = 8 * h + (lane >> 3);
                        *reinterpret_cast<v4u*>(wb + 128 * g + 16 * (((lane & 7) + g) & 7)) = wr[r][2 * c + h];
                    }
                    const v4u w0 = *reinterpret_cast<const v4u*>(wb + 128 * gi + 16 * ((2 * gp + gi) & 7));
                    const v4u w1 = *reinterpret_cast<const v4u*>(wb + 128 * gi + 16 * ((2 * gp + 1 + gi) & 7));
                    const int o = 2048 * c + 128 * gi + 32 * gp;     // byte offset of the lane's 32 bytes in the row
                    const v4u x0 = (o >> 4) < k16 ? *reinterpret_cast<const v4u*>(xq + o) : v4u{0, 0, 0, 0};
                    const v4u x1 = (o >> 4) + 1 < k16 ? *reinterpret_cast<const v4u*>(xq + o + 16) : v4u{0, 0, 0, 0};
                    const v4f pp = mfma_e4m3(w0, w1, x0, x1, v4f{0.f, 0.f, 0.f, 0.f});
                    const int g = 16 * c + gi;                        // this lane's diagonal group
                    const float fg = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (g & 63), __float_as_int(f[(16 * c) / 64])));
                    a = __builtin_fmaf(mfma16_diag(pp, lane), fg, a);
                    if (c % 2 == 1) __builtin_amdgcn_sched_barrier(0);
                }
                facc[r] = wave_sum_f32(a);
            } else {
                // one MFMA per KiB (half of its K slots zero): diagonal element i
                // is half of group 8 q + i / 2, scaled by s_x[group] * s_w[row
                // block, group] before it is added (groups past K meet zero
                // activations; their factors are clamped copies)
                float f[NF];
#pragma unroll
                for (int h = 0; h < NF; ++h) f[h] = gx[h] * bf16_lo(fw[r][h]);
                float a = 0.0f;
#pragma unroll
                for (int q = 0; q < SL; ++q) {
                    const v4f p = mfma_e4m3(bperm(wr[r][q]), v4u{0, 0, 0, 0}, tok(q), v4u{0, 0, 0, 0},
                                            v4f{0.f, 0.f, 0.f, 0.f});
                    const int g = (8 * q + ((lane & 15) >> 1)) & 63;   // group 8 q + i / 2, in register q / 8
                    const float fg = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * g, __float_as_int(f[q / 8])));
                    a = __builtin_fmaf(mfma16_diag(p, lane), fg, a);
                    // at most two partial products in flight: nothing is
                    // scheduled across this point
                    if (q % 2 == 1) __builtin_amdgcn_sched_barrier(0);
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
    if (rb < re) process(cur, fsw, rb);
    // XL launches give every wavefront at most one row (or gate/up pair):
    // without a second row in the loop the compiler keeps one row of weights
    if constexpr (!XL) {
        for (int n0 = rb + R; n0 < re; n0 += R) {
            load_rows(cur, fsw, n0);
            process(cur, fsw, n0);
        }
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
// rows: two rows per wavefront read one after the other (R = 1), except FP8
// rowwise: one row per wavefront, the token's slices read from LDS as they
// are used (the kernel's long-row form).
// SwiGLU mode: a wavefront reads one gate/up row pair at a time (two rows in
// flight), one pair per wavefront for rows up to 4 KiB or past 8 KiB, else two
// in turn.
void decode_launch_shape(int variant, int64_t ntot, int64_t K, int* R, int* grid) {
    const int64_t kc = (K + 1023) / 1024;
    *R = (kc > 4 && kc <= 8) ? 2 : 1;
    // one row per wavefront up to 4 KiB and, for FP8 rowwise, past 8 KiB (the
    // kernel's XL form -- FP8 rowwise past 8 KiB, block FP8 up to 4 KiB --
    // handles exactly one), else two per wavefront
    const bool one = kc <= 4 || (kc > 8 && variant == VAR_FP8_ROW);
    const int64_t rows = (kThreads / kWave) * (one ? 1 : 2);   // rows per workgroup
    const int64_t g = (ntot + rows - 1) / rows;
    *grid = (int)(g < 1 ? 1 : g);
}

hipError_t launch_linear_decode(int variant, const uint16_t* x, int64_t K, const SegmentArgs& sa, int mode,
                                uint8_t* qx, float* sx, hipStream_t st) {
    const int64_t ntot = mode == OUT_SWIGLU ? sa.start[1] : sa.start[sa.nseg];
    int R, grid;
    decode_launch_shape(variant, ntot, K, &R, &grid);
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
