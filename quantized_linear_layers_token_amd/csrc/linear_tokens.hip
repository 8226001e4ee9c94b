// Fused projection for a few tokens (2 <= M <= MT): bf16 activations in,
// quantized product out, in one launch, every weight byte streamed once in
// 1 KiB-contiguous wave loads (the one-token kernel's access pattern) rather
// than in matrix-core tiles.
//
// Workgroups are persistent: each rounds the M tokens into LDS once (the
// standalone quantizers' arithmetic: W8A8 model card, intro; FP8-dynamic
// README, "Creation"; Qwen3 8B FP8 card, "Loading"), then its four wavefronts
// walk the concatenated weight rows of all segments with a stride of every
// wavefront of the grid, one row at a time with the next row's loads in
// flight.  Per row and token: int8 with `v_dot4` against the token's codes
// read from LDS; E4M3 on the matrix cores with the one-token kernel's
// diagonal trick (one MFMA per 2 KiB of the row and token); block E4M3 with
// the lane permutation that puts one 128-input group in each MFMA row, the
// token's codes stored in LDS already permuted.
#include "qlin_device.h"
#include "qlin_internal.h"
#include "qlin_rows.h"

namespace qlin {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kAuxStream = 2;   // buffer-load cache policy: streaming

// V: scheme; KC: KiB slices per row (K <= 1024 KC); MT: token capacity.
template <int V, int KC, int MT>
__global__ __launch_bounds__(kThreads) void linear_tokens_kernel(
    const uint16_t* __restrict__ x, int M, int K, SegmentArgs sa, int mode,
    uint8_t* __restrict__ qx_out, float* __restrict__ sx_out) {
    constexpr bool FP8 = V != VAR_INT8;
    constexpr bool BLOCK = V == VAR_FP8_BLOCK;
    constexpr int CPT = (128 * KC + kThreads - 1) / kThreads;   // bf16 chunks of 8 per thread and token
    constexpr int NF = BLOCK ? (KC > 8 ? 2 : 1) : 1;             // block scales per lane and row
    __shared__ uint32_t red[MT][kWaves];
    __shared__ __attribute__((aligned(16))) uint8_t xq[MT][KC * 1024];
    __shared__ float gsc[MT][KC * 8];   // per token: its scale (rowwise) or one per 128-input group
    // block FP8, rows of an even number of KiB: each wavefront's 2 KiB chunk of
    // the row, 128-byte groups with their 16-byte pieces rotated by the group
    // index (the tokens' codes then stay in row order)
    constexpr bool BPAIR = BLOCK && KC % 2 == 0;
    __shared__ __attribute__((aligned(16))) uint8_t wst[BPAIR ? kWaves : 1][BPAIR ? 2048 : 16];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nchunks = K >> 3;
    const int k16 = K >> 4;
    const int kbs = K >> 7;
    const int ntot = sa.start[sa.nseg];
    const int W = gridDim.x * kWaves;
    const int w0 = blockIdx.x * kWaves + wave;

    auto seg_of = [&](int r) {
        int i = 0;
#pragma unroll
        for (int t = 1; t < kMaxSegments; ++t) i += (t < sa.nseg && r >= sa.start[t]) ? 1 : 0;
        return i;
    };
    // Row n of the concatenated segments through a buffer descriptor that is
    // empty for n >= ntot: such loads return zero and touch no memory, so the
    // prefetch past a wave's last row costs nothing.
    auto load_row = [&](v4u (&dst)[KC], uint32_t (&fsw)[NF], int n) {
        const int nc = min(n, ntot - 1);
        const int i = seg_of(nc);
        const int local = nc - sa.start[i];
        const __amdgpu_buffer_rsrc_t d = uniform_rsrc(sa.w[i] + (int64_t)local * K, n < ntot ? K : 0);
#pragma unroll
        for (int j = 0; j < KC; ++j)
            dst[j] = __builtin_amdgcn_raw_buffer_load_b128(d, min(j * kWave + lane, k16 - 1) * 16, 0, kAuxStream);
        if constexpr (BLOCK) {
            const uint16_t* swr = sa.sw[i] + (int64_t)(local >> 7) * kbs;
#pragma unroll
            for (int q = 0; q < NF; ++q) fsw[q] = swr[min(64 * q + lane, kbs - 1)];
        }
    };
    v4u cur[KC];
    uint32_t fcur[NF];
    load_row(cur, fcur, w0);   // the first row is in flight while the tokens are rounded

    // ---- the M tokens' bf16 rows, all loads issued before any reduction
    const v4u* xv = reinterpret_cast<const v4u*>(x);
    v4u xb[MT][CPT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < CPT; ++j)
            xb[t][j] = xv[(int64_t)min(t, M - 1) * nchunks + min(tid + j * kThreads, nchunks - 1)];

    // LDS byte offset of the codes of bf16 chunk c (8 codes).  Block FP8 rows of
    // an odd number of KiB store 16-byte piece m of each KiB at position
    // 16 (m % 4) + m / 4, so a lane l reading piece l gets the piece of lane
    // 4 (l % 16) + l / 16 (the MFMA row permutation of the weights); rows of an
    // even number of KiB keep row order (the weights go through LDS instead:
    // Qwen3-8B layer at two tokens 0.2502-0.2549 -> 0.2477-0.2510 ms per 4
    // layers, alternated on one box).
    auto code_off = [&](int c) {
        if constexpr (BLOCK && !BPAIR) {
            const int p = c >> 1, m = p & 63;
            return ((p & ~63) + 16 * (m & 3) + (m >> 2)) * 16 + (c & 1) * 8;
        } else {
            return c * 8;
        }
    };
    if constexpr (BLOCK) {
        // chunk c belongs to group c / 16: sixteen consecutive threads of one DPP row
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t >= M) break;
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                const int c = tid + j * kThreads;
                const uint32_t amax = row_max_u32(chunk_absmax(xb[t][j]));
                float sg;
                RoundFactor rf;
                scales_from_absmax<true>(amax, sg, rf);
                if (c < nchunks) {
                    *reinterpret_cast<v2u*>(&xq[t][code_off(c)]) = quant8<true>(xb[t][j], rf);
                    if ((tid & 15) == 0) gsc[t][c >> 4] = sg;
                }
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            uint32_t amax = 0;
#pragma unroll
            for (int j = 0; j < CPT; ++j) amax = max(amax, chunk_absmax(xb[t][j]));
            amax = wave_max_u32(amax);
            if (lane == 0) red[t][wave] = amax;
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t >= M) break;
            uint32_t amax = red[t][0];
#pragma unroll
            for (int i = 1; i < kWaves; ++i) amax = max(amax, red[t][i]);
            float s;
            RoundFactor rf;
            scales_from_absmax<FP8>(amax, s, rf);
            if (tid == 0) gsc[t][0] = s;
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                const int c = tid + j * kThreads;
                if (c < nchunks) *reinterpret_cast<v2u*>(&xq[t][code_off(c)]) = quant8<FP8>(xb[t][j], rf);
            }
        }
    }
    __syncthreads();

    if (qx_out != nullptr && blockIdx.x == 0) {
        for (int t = 0; t < M; ++t) {
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                const int c = tid + j * kThreads;
                if (c < nchunks)
                    *reinterpret_cast<v2u*>(qx_out + (int64_t)t * K + c * 8) =
                        *reinterpret_cast<const v2u*>(&xq[t][code_off(c)]);
            }
            if constexpr (BLOCK) {
                for (int g = tid; g < kbs; g += kThreads) sx_out[(int64_t)t * kbs + g] = gsc[t][g];
            } else {
                if (tid == 0) sx_out[t] = gsc[t][0];
            }
        }
    }

    // Block FP8: lane l takes the weight bytes loaded by lane 4 (l % 16) + l / 16
    const int paddr = 4 * (4 * (lane & 15) + (lane >> 4));
    auto bperm = [&](const v4u& v) {
        return v4u{(unsigned)__builtin_amdgcn_ds_bpermute(paddr, (int)v.x),
                   (unsigned)__builtin_amdgcn_ds_bpermute(paddr, (int)v.y),
                   (unsigned)__builtin_amdgcn_ds_bpermute(paddr, (int)v.z),
                   (unsigned)__builtin_amdgcn_ds_bpermute(paddr, (int)v.w)};
    };
    // the 16 codes of the token matching this lane's weight slice j (block FP8:
    // the permuted piece), zero past K
    const int src = BLOCK ? 4 * (lane & 15) + (lane >> 4) : lane;
    auto xslice = [&](int t, int j) {
        return j * kWave + src < k16 ? *reinterpret_cast<const v4u*>(&xq[t][(j * kWave + lane) * 16])
                                     : v4u{0, 0, 0, 0};
    };

    auto process = [&](const v4u (&wr)[KC], const uint32_t (&fw)[NF], int n) {
        const int i = seg_of(n);
        const int local = n - sa.start[i];
        const int N = sa.start[i + 1] - sa.start[i];
        float res[MT];
        int ires[MT];
        if constexpr (V == VAR_INT8) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t >= M) break;
                int a = 0;
#pragma unroll
                for (int j = 0; j < KC; ++j) a = dot16_i8(wr[j], xslice(t, j), a);
                ires[t] = wave_sum_i32(a);
            }
        } else if constexpr (V == VAR_FP8_ROW) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t >= M) break;
                v4f c = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < (KC + 1) / 2; ++q)
                    c = mfma_e4m3(wr[2 * q], 2 * q + 1 < KC ? wr[2 * q + 1] : v4u{0, 0, 0, 0}, xslice(t, 2 * q),
                                  2 * q + 1 < KC ? xslice(t, 2 * q + 1) : v4u{0, 0, 0, 0}, c);
                res[t] = wave_sum_f32(mfma16_diag(c, lane));
            }
        } else if constexpr (BPAIR) {
            // one MFMA per 2 KiB and token: the chunk goes through this
            // wavefront's LDS buffer so that MFMA row i (lanes i, i + 16, i + 32,
            // i + 48) holds the whole group i of the chunk (lane i + 16 p its
            // bytes 32 p .. 32 p + 31), shared by the tokens; diagonal element i
            // is group 16 c + i, scaled by s_x[t][group] * s_w[row block, group]
            uint8_t* const wb = wst[wave];
            const int gi = lane & 15, gp = lane >> 4;
            float a[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) a[t] = 0.0f;
#pragma unroll
            for (int c = 0; c < KC / 2; ++c) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int g = 8 * h + (lane >> 3);
                    *reinterpret_cast<v4u*>(wb + 128 * g + 16 * (((lane & 7) + g) & 7)) = wr[2 * c + h];
                }
                const v4u w0 = *reinterpret_cast<const v4u*>(wb + 128 * gi + 16 * ((2 * gp + gi) & 7));
                const v4u w1 = *reinterpret_cast<const v4u*>(wb + 128 * gi + 16 * ((2 * gp + 1 + gi) & 7));
                const int g = 16 * c + gi;                       // this lane's diagonal group
                const float fwg = bf16_lo((uint32_t)__builtin_amdgcn_ds_bpermute(4 * (g & 63), (int)fw[(16 * c) / 64]));
                const int o = 2048 * c + 128 * gi + 32 * gp;    // byte offset of the lane's 32 bytes in the row
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    if (t >= M) break;
                    const v4u x0 = (o >> 4) < k16 ? *reinterpret_cast<const v4u*>(&xq[t][o]) : v4u{0, 0, 0, 0};
                    const v4u x1 = (o >> 4) + 1 < k16 ? *reinterpret_cast<const v4u*>(&xq[t][o + 16]) : v4u{0, 0, 0, 0};
                    const v4f p = mfma_e4m3(w0, w1, x0, x1, v4f{0.f, 0.f, 0.f, 0.f});
                    a[t] = __builtin_fmaf(mfma16_diag(p, lane), gsc[t][min(g, kbs - 1)] * fwg, a[t]);
                }
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t >= M) break;
                res[t] = wave_sum_f32(a[t]);
            }
        } else {
            // the row's weights permuted once, shared by every token; group 8 q + i / 2
            // of diagonal element i: its weight-block scale moved from lane (group % 64)
            v4u wp[KC];
            float fwg[KC];
#pragma unroll
            for (int q = 0; q < KC; ++q) {
                wp[q] = bperm(wr[q]);
                const int g = (8 * q + ((lane & 15) >> 1)) & 63;
                fwg[q] = bf16_lo((uint32_t)__builtin_amdgcn_ds_bpermute(4 * g, (int)fw[q / 8]));
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t >= M) break;
                float a = 0.0f;
#pragma unroll
                for (int q = 0; q < KC; ++q) {
                    const v4f p = mfma_e4m3(wp[q], v4u{0, 0, 0, 0}, xslice(t, q), v4u{0, 0, 0, 0},
                                            v4f{0.f, 0.f, 0.f, 0.f});
                    const int g = min(8 * q + ((lane & 15) >> 1), kbs - 1);
                    a = __builtin_fmaf(mfma16_diag(p, lane), gsc[t][g] * fwg[q], a);
                }
                res[t] = wave_sum_f32(a);
            }
        }
        // lane t writes token t's output
        if (lane < M) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t != lane) continue;
                const int64_t idx = (int64_t)t * N + local;
                if constexpr (V == VAR_INT8) store_rowwise_i32acc(sa.y[i], idx, ires[t], gsc[t][0], sa.sw[i][local], mode);
                else if constexpr (V == VAR_FP8_ROW)
                    store_f32(sa.y[i], idx, res[t] * (gsc[t][0] * bf16_lo(sa.sw[i][local])), mode);
                else store_f32(sa.y[i], idx, res[t], mode);
            }
        }
    };

    for (int n = w0; n < ntot; n += W) {
        v4u nxt[KC];
        uint32_t fnxt[NF];
        load_row(nxt, fnxt, n + W);
        process(cur, fcur, n);
#pragma unroll
        for (int j = 0; j < KC; ++j) cur[j] = nxt[j];
#pragma unroll
        for (int q = 0; q < NF; ++q) fcur[q] = fnxt[q];
    }
}

// Instantiated for two tokens, the only count the dispatch sends here (at four
// and eight tokens the per-row token work made it slower than quantizer +
// matrix-core kernel on the Llama shapes).
template <int V, int KC>
hipError_t launch_mt(int M, int grid, hipStream_t st, const uint16_t* x, int K, const SegmentArgs& sa, int mode,
                     uint8_t* qx, float* sx) {
    static_assert(kLinearTokensMaxM == 2, "instantiate the token capacities the dispatch uses");
    hipLaunchKernelGGL((linear_tokens_kernel<V, KC, 2>), dim3(grid), dim3(kThreads), 0, st, x, M, K, sa, mode, qx, sx);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_tokens(int variant, const uint16_t* x, int64_t M, int64_t K, const SegmentArgs& sa, int mode,
                                uint8_t* qx, float* sx, hipStream_t st) {
    const int64_t ntot = sa.start[sa.nseg];
    if (!linear_tokens_fits(variant, M, K, ntot)) return hipErrorInvalidValue;
    // persistent: two workgroups per CU at most, never more than one row per wavefront
    const int64_t g = (ntot + kWaves - 1) / kWaves;
    const int grid = (int)(g < 512 ? (g < 1 ? 1 : g) : 512);
    const int64_t kc = (K + 1023) / 1024;
    const int m = (int)M, k = (int)K;
#define QLIN_TOK(VV)                                                                      \
    do {                                                                                  \
        if (kc <= 1) return launch_mt<VV, 1>(m, grid, st, x, k, sa, mode, qx, sx);        \
        if (kc <= 2) return launch_mt<VV, 2>(m, grid, st, x, k, sa, mode, qx, sx);        \
        if (kc <= 4) return launch_mt<VV, 4>(m, grid, st, x, k, sa, mode, qx, sx);        \
        if (kc <= 8) return launch_mt<VV, 8>(m, grid, st, x, k, sa, mode, qx, sx);        \
        if (kc <= 12) return launch_mt<VV, 12>(m, grid, st, x, k, sa, mode, qx, sx);      \
        if (kc <= 14) return launch_mt<VV, 14>(m, grid, st, x, k, sa, mode, qx, sx);      \
        return launch_mt<VV, 16>(m, grid, st, x, k, sa, mode, qx, sx);                    \
    } while (0)
    if (variant == VAR_INT8) QLIN_TOK(VAR_INT8);
    if (variant == VAR_FP8_ROW) QLIN_TOK(VAR_FP8_ROW);
    QLIN_TOK(VAR_FP8_BLOCK);
#undef QLIN_TOK
}

}  // namespace qlin
