// Products for up to 32 tokens on the matrix cores (W8A8 model card and Qwen3
// 8B FP8 card, "Loading": inputs of at most 32 rows go to the matrix units).
//
// The weights dominate the traffic (arithmetic intensity <= 2M ops/byte), so
// the kernel is a weight stream: every weight byte is loaded from HBM once.
// Loads cover whole 128-byte lines (8 rows per instruction) and each K step
// goes through a per-wave LDS buffer into the MFMA register layout: loading
// that layout directly (16 rows x 64 bytes per instruction) left the kernel
// bound by the L1 address path.
//
//   workgroup = one tile of 16 weight rows (output channels) x the full K,
//               split over NW wavefronts along K (each owns a contiguous run
//               of 128-byte K steps);
//   MFMA      = A: 16 weight rows x 128 bytes of K, B: 128 bytes of K x 16
//               tokens, C[n][m] (4 rows of one token column per lane).
//               int8: two v_mfma_i32_16x16x64_i8 per step; E4M3: one
//               v_mfma_f32_16x16x128_f8f6f4 per step.  Lane l supplies bytes
//               [16 (l/16), +16) and [64 + 16 (l/16), +16) of the step for
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
//   fused     = (FU, at most 4 tokens of at most 4096 inputs; with or without
//               SwiGLU) the kernel takes
//               the bf16 activations: each of the first M wavefronts rounds
//               one token (the standalone quantizers' arithmetic) into the
//               workgroup's LDS while the first weight batch is in flight,
//               and the token operand is read from there; no quantizer
//               launch precedes the product.
//   SwiGLU    = (SG) the first RT/2 MFMA row tiles are gate rows j0.., the
//               other RT/2 the up rows with the same indices: after the
//               reduction a lane holds gate and up of the same (j, m) and
//               writes h = swiglu_bf16(gate, up).
#include <type_traits>

#include "qlin_device.h"
#include "qlin_internal.h"
#include "qlin_rows.h"

namespace qlin {

namespace {

template <int U> using IC = std::integral_constant<int, U>;
constexpr int kSmallBatch = 2;      // K steps per load batch for 64-row tiles (two batches in flight)
constexpr int kOOB = 0x40000000;    // an offset past every descriptor's range: reads zero
constexpr int kAuxStream = 2;       // buffer-load cache policy: streaming (slc)

template <int V> struct SmallAcc { typedef v4i T; };
template <> struct SmallAcc<VAR_FP8_ROW> { typedef v4f T; };
template <> struct SmallAcc<VAR_FP8_BLOCK> { typedef v4f T; };

// FU (fused): the kernel takes the bf16 input and rounds its M <= kSmallFusedMaxM
// tokens itself: waves 0 .. M - 1 each round one token into this workgroup's
// LDS (per token, or per 128-input group for block FP8; the standalone
// quantizers' arithmetic), while the first weight batch is in flight; the
// MFMA token operand is then read from there.  Workgroup 0 also fills the
// optional staging buffers qx_out / sx_out.
template <int V, int MT, int NW, int RT, bool SG, bool FU = false>
__global__ __launch_bounds__(NW * 64) void gemm_small_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx, SegmentArgs sa, int M, int K, int mode,
    const uint16_t* __restrict__ xbf, uint8_t* __restrict__ qx_out, float* __restrict__ sx_out) {
    typedef typename SmallAcc<V>::T Acc;
    static_assert(!FU || MT == 1, "fused rounding: one token tile");
    // per-wave transpose buffer for one K step (RT weight tiles + MT token
    // tiles, 16 rows x 128 bytes each), reused for the split-K reduction
    constexpr int TPB = (RT + (FU ? 0 : MT)) * 2048;
    constexpr int SMEM = NW * TPB > (int)(NW * RT * MT * kWave * sizeof(Acc)) ? NW * TPB
                                                                              : (int)(NW * RT * MT * kWave * sizeof(Acc));
    __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
    auto red = reinterpret_cast<Acc(*)[RT * MT][kWave]>(smem);
    // FU: per token its scale (or one per 128-input group) and its codes,
    // rows of XS bytes (K rounded up to a 128-byte step, zero past K, + 64 so
    // that the four rows fall on distinct LDS bank groups)
    extern __shared__ __attribute__((aligned(16))) uint8_t fdyn[];
    float* const fsc = reinterpret_cast<float*>(fdyn);
    uint8_t* const xq = fdyn + kSmallFusedScaleBytes;
    const int XS = ((K + 127) & ~127) + 64;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15;           // weight row / token column within a 16 x 16 MFMA tile
    const int grp = lane >> 4;           // which 16-byte piece of each 64-byte half of a K step

    // tiles of 16 RT weight rows (RT MFMA tiles sharing the token loads) are numbered across the segments (q, k, v or gate, up
    // sharing one input); a tile never straddles two segments
    // (SG: a tile is 8 RT gate rows and the same 8 RT up rows)
    static_assert(!SG || RT % 2 == 0, "SwiGLU tiles pair gate and up row tiles");
    constexpr int TR = SG ? 8 * RT : 16 * RT;          // rows of one segment per tile
    constexpr int RH = SG ? RT / 2 : RT;               // row tiles per segment
    int tile = blockIdx.x, seg = 0;
    if constexpr (!SG) {
#pragma unroll
        for (int i = 0; i + 1 < kMaxSegments; ++i) {
            const int nt = (sa.start[i + 1] - sa.start[i] + TR - 1) / TR;
            if (seg == i && i + 1 < sa.nseg && tile >= nt) {
                tile -= nt;
                seg = i + 1;
            }
        }
    }
    const uint8_t* __restrict__ qw = pick_ptr(sa.w, seg);
    const uint16_t* __restrict__ sw = pick_ptr(sa.sw, seg);
    void* __restrict__ y = pick_ptr(sa.y, seg);
    const int N = pick_int(sa.start + 1, seg) - pick_int(sa.start, seg);
    const int n0 = __builtin_amdgcn_readfirstlane(tile * TR);

    const int nsteps = (K + 127) >> 7;
    const int per = (nsteps + NW - 1) / NW;
    const int s_begin = wave * per;
    const int s_end = min(nsteps, s_begin + per);

    // Buffer descriptors over the tile's weight rows and over the M token
    // rows: rows past N or M, K past the end and steps past the wave's range
    // read as zero (an out-of-range offset), with no select after the load.
    const __amdgpu_buffer_rsrc_t dw = uniform_rsrc(qw + (int64_t)n0 * K, min(TR, N - n0) * K);
    // SG: the up rows with the same indices (segment 1, equal width)
    const __amdgpu_buffer_rsrc_t du = uniform_rsrc(sa.w[SG ? 1 : 0] + (int64_t)n0 * K, SG ? min(TR, N - n0) * K : 0);
    const __amdgpu_buffer_rsrc_t dx = uniform_rsrc(qx, M * K);
    // Loads cover whole 128-byte lines: lane l reads 16 bytes 16 (l % 8) of row
    // l / 8 (and of row 8 + l / 8) of a tile; the K step is then transposed
    // through this wave's LDS buffer into the MFMA layout, lane l holding
    // bytes [16 g, +16) and [64 + 16 g, +16) of row l % 16, g = l / 16 (both
    // operands the same way, so the contraction is unchanged).  The RT weight
    // tiles of a wavefront share its token fragments.
    const int lr = lane >> 3, lp = lane & 7;
    const int woff = lr * K + lp * 16;
    int xoff[MT][2];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int m = t * 16 + 8 * h + lr;
            xoff[t][h] = m < M ? m * K + lp * 16 : kOOB;
        }
    auto swz = [](int r) { return (r & 7) ^ ((r >> 3) & 1); };
    uint8_t* tpw = smem + wave * TPB;
    const int wr_off0 = lr * 128 + ((lp ^ swz(lr)) << 4);             // LDS position of this lane's piece, row lr
    const int wr_off1 = (lr + 8) * 128 + ((lp ^ swz(lr + 8)) << 4);    // ... row lr + 8
    const int rd_off0 = r16 * 128 + ((grp ^ swz(r16)) << 4);          // MFMA layout: piece g of row l % 16
    const int rd_off1 = r16 * 128 + (((4 + grp) ^ swz(r16)) << 4);    // ... piece 4 + g

    const int kbs = K >> 7;
    // block FP8: the tile's 128-row block of weight scales, read in the K loop.
    // One token tile: through global-memory pointers, so the loop waits for one
    // load batch at a time (through a generic pointer they are flat loads, and
    // with a flat load in flight the compiler waits for every load, the batch
    // just issued included): Qwen3-8B block layer at 4 tokens 0.256 -> 0.243 ms
    // per 4 layers, at 16 unchanged.  Two token tiles (17..32 tokens) measured
    // slower with the batch-wise waits (0.351 -> 0.363 ms at 32 tokens) and
    // keep the generic pointer.
    typedef typename std::conditional<MT == 1, const __attribute__((address_space(1))) uint16_t*,
                                      const uint16_t*>::type SwPtr;
    SwPtr swblk, swblk_u;
    if constexpr (MT == 1) {
        swblk = pick_global(sa.sw, seg) + (int64_t)(n0 >> 7) * kbs;
        swblk_u = pick_global(sa.sw, SG ? 1 : 0) + (int64_t)(n0 >> 7) * kbs;
    } else {
        swblk = sw + (int64_t)(n0 >> 7) * kbs;
        swblk_u = sa.sw[SG ? 1 : 0] + (int64_t)(n0 >> 7) * kbs;
    }

    Acc acc[RT][MT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = Acc{0, 0, 0, 0};

    // Batches of kSmallBatch K steps, double-buffered: batch b + 1 is loaded
    // while batch b is multiplied, so a wavefront keeps two batches of loads
    // in flight.  Loads past the wavefront's steps read zero.
    constexpr int U = RT == 1 ? 2 * kSmallBatch : kSmallBatch;   // same register budget either way
    v4u wa[2][U][RT][2], xa[2][U][MT][2];
    float fx[2][U][MT], fw[2][U][SG ? 2 : 1];
    auto issue = [&](auto bufc, int s0) {
        constexpr int bi = decltype(bufc)::value;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + u;
            const int k = s * 128 + lp * 16;
            const bool ok = (s < s_end) && (k < K);
            // weights stream once: non-temporal
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const bool up = SG && r >= RH;
                const int o = woff + (up ? r - RH : r) * 16 * K + s * 128;
                wa[bi][u][r][0] = __builtin_amdgcn_raw_buffer_load_b128(up ? du : dw, ok ? o : kOOB, 0, kAuxStream);
                wa[bi][u][r][1] = __builtin_amdgcn_raw_buffer_load_b128(up ? du : dw, ok ? o + 8 * K : kOOB, 0, kAuxStream);
            }
            if constexpr (!FU) {
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    xa[bi][u][t][0] = __builtin_amdgcn_raw_buffer_load_b128(dx, ok && xoff[t][0] != kOOB ? xoff[t][0] + s * 128 : kOOB, 0, 0);
                    xa[bi][u][t][1] = __builtin_amdgcn_raw_buffer_load_b128(dx, ok && xoff[t][1] != kOOB ? xoff[t][1] + s * 128 : kOOB, 0, 0);
                }
            }
            if constexpr (V == VAR_FP8_BLOCK) {
                const int sb = min(s, s_end - 1);
                fw[bi][u][0] = bf16_lo(swblk[sb]);
                if constexpr (SG) fw[bi][u][1] = bf16_lo(swblk_u[sb]);
                if constexpr (!FU) {
#pragma unroll
                    for (int t = 0; t < MT; ++t) fx[bi][u][t] = sx[(int64_t)min(t * 16 + r16, M - 1) * kbs + sb];
                }
            }
        }
    };
    auto compute = [&](auto bufc, int s0) {
        constexpr int bi = decltype(bufc)::value;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // transpose this step through the wave's LDS buffer
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                *reinterpret_cast<v4u*>(tpw + r * 2048 + wr_off0) = wa[bi][u][r][0];
                *reinterpret_cast<v4u*>(tpw + r * 2048 + wr_off1) = wa[bi][u][r][1];
            }
            if constexpr (!FU) {
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    *reinterpret_cast<v4u*>(tpw + (RT + t) * 2048 + wr_off0) = xa[bi][u][t][0];
                    *reinterpret_cast<v4u*>(tpw + (RT + t) * 2048 + wr_off1) = xa[bi][u][t][1];
                }
            }
            v4u ta[RT][2], tx[MT][2];
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                ta[r][0] = *reinterpret_cast<const v4u*>(tpw + r * 2048 + rd_off0);
                ta[r][1] = *reinterpret_cast<const v4u*>(tpw + r * 2048 + rd_off1);
            }
            if constexpr (FU) {
                // token r16's bytes [16 g, +16) and [64 + 16 g, +16) of this step
                const int s = s0 + u;
                const bool tok = r16 < M && s < nsteps;
                const uint8_t* p = xq + r16 * XS + s * 128 + 16 * grp;
                tx[0][0] = tok ? *reinterpret_cast<const v4u*>(p) : v4u{0, 0, 0, 0};
                tx[0][1] = tok ? *reinterpret_cast<const v4u*>(p + 64) : v4u{0, 0, 0, 0};
            } else {
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    tx[t][0] = *reinterpret_cast<const v4u*>(tpw + (RT + t) * 2048 + rd_off0);
                    tx[t][1] = *reinterpret_cast<const v4u*>(tpw + (RT + t) * 2048 + rd_off1);
                }
            }
            if constexpr (V == VAR_FP8_BLOCK) {
                // every tile's partial product of this step first, then the
                // scaling: the MFMAs issue back to back instead of each waiting
                // for the previous one's result to be read (steps past the
                // wavefront's range multiplied zeros: factor 0, branch-free, so
                // every path from an MFMA to its first read is the padded one)
                v4f pp[RT][MT];
#pragma unroll
                for (int r = 0; r < RT; ++r)
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        const v4u w0 = ta[r][0], w1 = ta[r][1], x0 = tx[t][0], x1 = tx[t][1];
                        const v8i a = v8i{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
                        const v8i b = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
                        pp[r][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                                                   0, 0, 0);
                    }
#pragma unroll
                for (int r = 0; r < RT; ++r)
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        const float fxv = FU ? fsc[min(r16, M - 1) * kSmallFusedGroups + min(s0 + u, s_end - 1)]
                                             : fx[bi][u][t];
                        const float f = s0 + u < s_end ? fxv * fw[bi][u][(SG && r >= RH) ? 1 : 0] : 0.0f;
                        acc[r][t].x = __builtin_fmaf(pp[r][t].x, f, acc[r][t].x);
                        acc[r][t].y = __builtin_fmaf(pp[r][t].y, f, acc[r][t].y);
                        acc[r][t].z = __builtin_fmaf(pp[r][t].z, f, acc[r][t].z);
                        acc[r][t].w = __builtin_fmaf(pp[r][t].w, f, acc[r][t].w);
                    }
            } else
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const v4u w0 = ta[r][0], w1 = ta[r][1], x0 = tx[t][0], x1 = tx[t][1];
                    if constexpr (V == VAR_INT8) {
                        acc[r][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, w0),
                                                                          __builtin_bit_cast(v4i, x0), acc[r][t], 0, 0, 0);
                        acc[r][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, w1),
                                                                          __builtin_bit_cast(v4i, x1), acc[r][t], 0, 0, 0);
                    } else {
                        const v8i a = v8i{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
                        const v8i b = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
                        if constexpr (V == VAR_FP8_ROW) {
                            acc[r][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[r][t], 0, 0, 0, 0, 0, 0);
                        } else {
                            const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                a, b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                            // steps past the wavefront's range multiplied zeros: factor 0
                            // (branch-free, so every path from the MFMA to its first read
                            // is the padded one)
                            const float fxv = FU ? fsc[min(r16, M - 1) * kSmallFusedGroups + min(s0 + u, s_end - 1)]
                                                 : fx[bi][u][t];
                            const float f = s0 + u < s_end ? fxv * fw[bi][u][(SG && r >= RH) ? 1 : 0] : 0.0f;
                            acc[r][t].x = __builtin_fmaf(p.x, f, acc[r][t].x);
                            acc[r][t].y = __builtin_fmaf(p.y, f, acc[r][t].y);
                            acc[r][t].z = __builtin_fmaf(p.z, f, acc[r][t].z);
                            acc[r][t].w = __builtin_fmaf(p.w, f, acc[r][t].w);
                        }
                    }
                }
        }
    };

    issue(IC<0>{}, s_begin);
    if constexpr (FU) {
        // round the tokens while the first weight batch is in flight; a lane
        // holds chunks lane + 64 j of its token (K <= 4096: at most 8)
        const int nch = K >> 3;                            // 16-byte chunks of 8 bf16
        if (wave < M) {
            const int t = wave;
            const v4u* xr = reinterpret_cast<const v4u*>(xbf + (int64_t)t * K);
            uint8_t* row = xq + t * XS;
            const bool stage = qx_out != nullptr && blockIdx.x == 0;
            v4u v[kSmallFusedChunks];
#pragma unroll
            for (int j = 0; j < kSmallFusedChunks; ++j) {
                const int c = lane + kWave * j;
                v[j] = c < nch ? xr[c] : v4u{0, 0, 0, 0};
            }
            if constexpr (V == VAR_FP8_BLOCK) {
                // chunks 64 j + 16 r .. + 15 are one 128-input group: one DPP row
#pragma unroll
                for (int j = 0; j < kSmallFusedChunks; ++j) {
                    const int c = lane + kWave * j;
                    float sg;
                    RoundFactor rf;
                    scales_from_absmax<true>(row_max_u32(chunk_absmax(v[j])), sg, rf);
                    if (c < nch) {
                        const v2u q = quant8<true>(v[j], rf);
                        *reinterpret_cast<v2u*>(row + 8 * c) = q;
                        if (stage) *reinterpret_cast<v2u*>(qx_out + (int64_t)t * K + 8 * c) = q;
                        if ((lane & 15) == 0) {
                            fsc[t * kSmallFusedGroups + (c >> 4)] = sg;
                            if (stage) sx_out[(int64_t)t * kbs + (c >> 4)] = sg;
                        }
                    }
                }
            } else {
                uint32_t amax = 0;
#pragma unroll
                for (int j = 0; j < kSmallFusedChunks; ++j) amax = max(amax, chunk_absmax(v[j]));
                float sc;
                RoundFactor rf;
                scales_from_absmax<V != VAR_INT8>(wave_max_u32(amax), sc, rf);
#pragma unroll
                for (int j = 0; j < kSmallFusedChunks; ++j) {
                    const int c = lane + kWave * j;
                    if (c < nch) {
                        const v2u q = quant8<V != VAR_INT8>(v[j], rf);
                        *reinterpret_cast<v2u*>(row + 8 * c) = q;
                        if (stage) *reinterpret_cast<v2u*>(qx_out + (int64_t)t * K + 8 * c) = q;
                    }
                }
                if (lane == 0) {
                    fsc[t] = sc;
                    if (stage) sx_out[t] = sc;
                }
            }
            // zeros from K to the end of the last 128-byte step
            for (int b = K + 16 * lane; b < ((K + 127) & ~127); b += 16 * kWave)
                *reinterpret_cast<v4u*>(row + b) = v4u{0, 0, 0, 0};
        }
        __syncthreads();
    }
    int s0 = s_begin;
    for (; s0 + U < s_end; s0 += 2 * U) {                 // at least two batches left
        issue(IC<1>{}, s0 + U);
        __builtin_amdgcn_sched_barrier(0);                 // both batches in flight before the first wait
        compute(IC<0>{}, s0);
        issue(IC<0>{}, s0 + 2 * U);                        // possibly all past the end: zeros, never used
        __builtin_amdgcn_sched_barrier(0);
        compute(IC<1>{}, s0 + U);
    }
    if (s0 < s_end) compute(IC<0>{}, s0);
    mfma_drain();      // the accumulators are stored to LDS next
    __syncthreads();   // every wave is done with its transpose buffer before the reduction reuses it

#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) red[wave][r * MT + t][lane] = acc[r][t];
    __syncthreads();

    // Sum the NW partial tiles.  Item (r, t, l): weight rows n0 + 16 r + 4 (l / 16)
    // .. + 3 of token m = 16 t + l % 16.
    if constexpr (SG) {
        for (int it = tid; it < RH * MT * kWave; it += NW * kWave) {
            const int rt = it / kWave, l = it % kWave;
            const int r = rt / MT, t = rt % MT;
            const int ru = (r + RH) * MT + t;
            Acc g = red[0][rt][l], u = red[0][ru][l];
#pragma unroll
            for (int w = 1; w < NW; ++w) {
                g += red[w][rt][l];
                u += red[w][ru][l];
            }
            const int m = t * 16 + (l & 15);
            if (m < M) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int n = n0 + 16 * r + (l >> 4) * 4 + e;
                    if (n < N) {
                        float gv, uv;
                        const float sxm = FU ? fsc[m] : sx[m];
                        if constexpr (V == VAR_INT8) {
                            gv = (float)g[e] * (sxm * bf16_lo(sw[n]));
                            uv = (float)u[e] * (sxm * bf16_lo(sa.sw[1][n]));
                        } else if constexpr (V == VAR_FP8_ROW) {
                            gv = g[e] * (sxm * bf16_lo(sw[n]));
                            uv = u[e] * (sxm * bf16_lo(sa.sw[1][n]));
                        } else {
                            gv = g[e];
                            uv = u[e];
                        }
                        static_cast<uint16_t*>(y)[(int64_t)m * N + n] = swiglu_bf16(gv, uv);
                    }
                }
            }
        }
        return;
    }
    for (int it = tid; it < RT * MT * kWave; it += NW * kWave) {
        const int rt = it / kWave, l = it % kWave;
        const int r = rt / MT, t = rt % MT;
        Acc sum = red[0][rt][l];
#pragma unroll
        for (int w = 1; w < NW; ++w) sum += red[w][rt][l];
        const int m = t * 16 + (l & 15);
        if (m < M) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = n0 + 16 * r + (l >> 4) * 4 + e;
                if (n < N) {
                    const int64_t idx = (int64_t)m * N + n;
                    const float sxm = FU ? fsc[m] : sx[m];
                    if constexpr (V == VAR_INT8) store_rowwise_i32acc(y, idx, sum[e], sxm, sw[n], mode);
                    else if constexpr (V == VAR_FP8_ROW) store_f32(y, idx, sum[e] * (sxm * bf16_lo(sw[n])), mode);
                    else store_f32(y, idx, sum[e], mode);
                }
            }
        }
    }
}

template <int V, int MT, int RT, bool SG = false, bool FU = false>
void launch_mt(int nw, dim3 grid, hipStream_t st, const uint8_t* qx, const float* sx, const SegmentArgs& sa,
               int M, int K, int mode, const uint16_t* xbf = nullptr, uint8_t* qx_out = nullptr,
               float* sx_out = nullptr) {
    const size_t dyn = FU ? small_fused_lds_bytes(M, K) : 0;
    if (nw >= 8)
        hipLaunchKernelGGL((gemm_small_kernel<V, MT, 8, RT, SG, FU>), grid, dim3(8 * 64), dyn, st, qx, sx, sa, M, K,
                           mode, xbf, qx_out, sx_out);
    else
        hipLaunchKernelGGL((gemm_small_kernel<V, MT, 4, RT, SG, FU>), grid, dim3(4 * 64), dyn, st, qx, sx, sa, M, K,
                           mode, xbf, qx_out, sx_out);
}

int64_t small_tiles(const SegmentArgs& sa, int rows) {
    int64_t tiles = 0;
    for (int i = 0; i < sa.nseg; ++i) tiles += (sa.start[i + 1] - sa.start[i] + rows - 1) / rows;
    return tiles;
}

}  // namespace

// K-split depth: 4 wavefronts for K up to 4 Ki (each keeps its eight steps in
// flight as four batches), else 8.
int small_waves_per_tile(int64_t N, int64_t K) {
    (void)N;
    return K <= 4096 ? 4 : 8;
}

hipError_t launch_gemm_small(int variant, const uint8_t* qx, const float* sx, const SegmentArgs& sa, int64_t M,
                             int64_t K, int mode, hipStream_t st) {
    if (mode == OUT_SWIGLU) {
        // tiles of 32 gate + 32 up rows with a workgroup per CU or more, else 16 + 16
        const int64_t I = sa.start[1];
        const bool wide = (I + 31) / 32 >= 256;
        const int64_t tiles = (I + (wide ? 31 : 15)) / (wide ? 32 : 16);
        dim3 grid((unsigned)tiles);
        const int nw = small_waves_per_tile(tiles, K);
        const int m = (int)M, k = (int)K;
        const bool two = M > 16;
#define QLIN_SMALL_SG(VV)                                                                   \
        do {                                                                                \
            if (wide) {                                                                     \
                if (two) launch_mt<VV, 2, 4, true>(nw, grid, st, qx, sx, sa, m, k, mode);   \
                else launch_mt<VV, 1, 4, true>(nw, grid, st, qx, sx, sa, m, k, mode);       \
            } else {                                                                        \
                if (two) launch_mt<VV, 2, 2, true>(nw, grid, st, qx, sx, sa, m, k, mode);   \
                else launch_mt<VV, 1, 2, true>(nw, grid, st, qx, sx, sa, m, k, mode);       \
            }                                                                               \
        } while (0)
        if (variant == VAR_INT8) QLIN_SMALL_SG(VAR_INT8);
        else if (variant == VAR_FP8_ROW) QLIN_SMALL_SG(VAR_FP8_ROW);
        else QLIN_SMALL_SG(VAR_FP8_BLOCK);
#undef QLIN_SMALL_SG
        return hipGetLastError();
    }
    // 64-row tiles share each token load four ways, but only pay off with at
    // least a workgroup per CU for every 64 rows (the wide gate/up launch).
    // 32-row tiles, with at least 192 of them and K <= 4096: q/k/v (6144 rows)
    // at 8 / 16 / 32 tokens took 8.9 / 10.0 / 12.2 -> 7.7 / 8.8 / 9.5 us; with
    // 128 tiles (4096 rows) they lost (6.4 -> 7.0 us at 8 tokens).
    const bool wide = small_tiles(sa, 64) >= 256;
    const bool mid = !wide && K <= 4096 && small_tiles(sa, 32) >= 192;
    const int64_t tiles = small_tiles(sa, wide ? 64 : (mid ? 32 : 16));
    dim3 grid((unsigned)tiles);
    const int nw = small_waves_per_tile(tiles, K);
    const int m = (int)M, k = (int)K;
    const bool two = M > 16;
#define QLIN_SMALL(VV)                                                                \
    do {                                                                              \
        if (wide) {                                                                   \
            if (two) launch_mt<VV, 2, 4>(nw, grid, st, qx, sx, sa, m, k, mode);       \
            else launch_mt<VV, 1, 4>(nw, grid, st, qx, sx, sa, m, k, mode);           \
        } else if (mid) {                                                             \
            if (two) launch_mt<VV, 2, 2>(nw, grid, st, qx, sx, sa, m, k, mode);       \
            else launch_mt<VV, 1, 2>(nw, grid, st, qx, sx, sa, m, k, mode);           \
        } else {                                                                      \
            if (two) launch_mt<VV, 2, 1>(nw, grid, st, qx, sx, sa, m, k, mode);       \
            else launch_mt<VV, 1, 1>(nw, grid, st, qx, sx, sa, m, k, mode);           \
        }                                                                             \
    } while (0)
    if (variant == VAR_INT8) QLIN_SMALL(VAR_INT8);
    else if (variant == VAR_FP8_ROW) QLIN_SMALL(VAR_FP8_ROW);
    else QLIN_SMALL(VAR_FP8_BLOCK);
#undef QLIN_SMALL
    return hipGetLastError();
}

hipError_t launch_gemm_small_fused(int variant, const uint16_t* x, int64_t M, int64_t K, const SegmentArgs& sa,
                                   int mode, uint8_t* qx_out, float* sx_out, hipStream_t st) {
    if (!small_fused_fits(M, K)) return hipErrorInvalidValue;
    const int m = (int)M, k = (int)K;
    if (mode == OUT_SWIGLU) {
        // the same tiles as the staged SwiGLU launch
        const int64_t I = sa.start[1];
        const bool wide = (I + 31) / 32 >= 256;
        dim3 grid((unsigned)((I + (wide ? 31 : 15)) / (wide ? 32 : 16)));
        const int nw = small_waves_per_tile(grid.x, K);
#define QLIN_SMALL_FU_SG(VV)                                                                                      \
        do {                                                                                                      \
            if (wide) launch_mt<VV, 1, 4, true, true>(nw, grid, st, nullptr, nullptr, sa, m, k, mode, x, qx_out, sx_out); \
            else launch_mt<VV, 1, 2, true, true>(nw, grid, st, nullptr, nullptr, sa, m, k, mode, x, qx_out, sx_out);      \
        } while (0)
        if (variant == VAR_INT8) QLIN_SMALL_FU_SG(VAR_INT8);
        else if (variant == VAR_FP8_ROW) QLIN_SMALL_FU_SG(VAR_FP8_ROW);
        else QLIN_SMALL_FU_SG(VAR_FP8_BLOCK);
#undef QLIN_SMALL_FU_SG
        return hipGetLastError();
    }
    // the same tiles as the staged small-M launch
    const bool wide = small_tiles(sa, 64) >= 256;
    const int64_t tiles = small_tiles(sa, wide ? 64 : 16);
    dim3 grid((unsigned)tiles);
    const int nw = small_waves_per_tile(tiles, K);
#define QLIN_SMALL_FU(VV)                                                                                      \
    do {                                                                                                       \
        if (wide) launch_mt<VV, 1, 4, false, true>(nw, grid, st, nullptr, nullptr, sa, m, k, mode, x, qx_out, sx_out); \
        else launch_mt<VV, 1, 1, false, true>(nw, grid, st, nullptr, nullptr, sa, m, k, mode, x, qx_out, sx_out);      \
    } while (0)
    if (variant == VAR_INT8) QLIN_SMALL_FU(VAR_INT8);
    else if (variant == VAR_FP8_ROW) QLIN_SMALL_FU(VAR_FP8_ROW);
    else QLIN_SMALL_FU(VAR_FP8_BLOCK);
#undef QLIN_SMALL_FU
    return hipGetLastError();
}

}  // namespace qlin
