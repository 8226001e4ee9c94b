// Weight-only ("equivalent") numerics: the bf16 input is never rounded and is
// multiplied by the dequantized weights (W8A8 model card and Qwen3 8B FP8
// card, "Against bf16": the "equivalent" mode keeps the input unrounded;
// "Loading": the numerics option).
//
//   y[m, n] = s_w[n] * sum_k x[m, k] * q_w[n, k]                 (rowwise)
//   y[m, n] = sum_kb s_w[n/128, kb] * sum_{k in kb} x[m, k] * q_w[n, k]   (block)
//
// Every product of a bf16 input and an int8 or E4M3 code is exact in f32; the
// sums are f32.
//
// One token (M = 1, K <= 16384): wo_gemv_kernel streams each weight byte once
// like the quantized one-row product; the workgroup stages the bf16 row in
// LDS and every wavefront keeps the 32-byte input slices matching its 16-byte
// weight slices in registers.  The codes widen exactly to bf16 and meet the
// inputs on the matrix cores (the diagonal of a 16x16x32 bf16 MFMA per 8
// codes), so the vector ALUs only widen.
//
// 2..32 tokens (or longer K): wo_small_kernel, the small-M weight stream with
// the codes widened exactly to bf16 in registers and multiplied on the matrix
// cores (v_mfma_f32_16x16x32_bf16) against the bf16 input.
#include <type_traits>

#include "qlin_device.h"
#include "qlin_internal.h"

namespace qlin {

namespace {

constexpr int kThreads = 256;
constexpr int kOOB = 0x40000000;    // an offset past every descriptor's range: reads zero
constexpr int kAuxStream = 2;       // buffer-load cache policy: streaming
template <int U> using IC = std::integral_constant<int, U>;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// code b of a packed dword, widened exactly
__device__ __forceinline__ float i8_at(uint32_t w, int b) { return (float)((int)(w << (24 - 8 * b)) >> 24); }

// 8 codes (two dwords) widened exactly to bf16
template <int V>
__device__ __forceinline__ v8bf codes_to_bf16(uint32_t w0, uint32_t w1) {
    float f[8];
    if constexpr (V == VAR_INT8) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            f[b] = i8_at(w0, b);
            f[4 + b] = i8_at(w1, b);
        }
    } else {
        const v2f a = e4m3_unpack2<false>(w0), b = e4m3_unpack2<true>(w0);
        const v2f c = e4m3_unpack2<false>(w1), d = e4m3_unpack2<true>(w1);
        f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y;
        f[4] = c.x; f[5] = c.y; f[6] = d.x; f[7] = d.y;
    }
    // every such value has at most 8 significant bits: the high half of its
    // f32 pattern is its bf16 pattern
    v4u p;
    p.x = __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
    p.y = __builtin_amdgcn_perm(__float_as_uint(f[3]), __float_as_uint(f[2]), 0x07060302u);
    p.z = __builtin_amdgcn_perm(__float_as_uint(f[5]), __float_as_uint(f[4]), 0x07060302u);
    p.w = __builtin_amdgcn_perm(__float_as_uint(f[7]), __float_as_uint(f[6]), 0x07060302u);
    return __builtin_bit_cast(v8bf, p);
}

// ---------------------------------------------------------------------------
// M = 1
// ---------------------------------------------------------------------------

// V: weight format; KC: 1 KiB weight slices per row in registers (K <= 1024 KC);
// R: rows per wavefront per iteration.
template <int V, int KC, int R>
__global__ __launch_bounds__(kThreads) void wo_gemv_kernel(const uint16_t* __restrict__ x, int K, SegmentArgs sa,
                                                           int mode) {
    constexpr int CPT = (KC * 128 + kThreads - 1) / kThreads;   // 16-byte input chunks per thread
    __shared__ __attribute__((aligned(16))) uint8_t xs[KC * 2048];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nchunks = K >> 3;                    // 8 bf16 per chunk
    const int k16 = K >> 4;                        // 16-byte weight slices per row

    const int ntot = sa.start[sa.nseg];
    const int W = gridDim.x * (kThreads / kWave);
    const int w = blockIdx.x * (kThreads / kWave) + wave;
    const int rb = (int)((int64_t)ntot * w / W);
    const int re = (int)((int64_t)ntot * (w + 1) / W);

    // input chunks first (the barrier below waits for them only), then the
    // first weight rows; loads past the end re-read a valid address
    v4u xb[CPT];
    const v4u* xv = reinterpret_cast<const v4u*>(x);
#pragma unroll
    for (int j = 0; j < CPT; ++j) xb[j] = xv[min(tid + j * kThreads, nchunks - 1)];

    auto seg_of = [&](int r) {
        int i = 0;
#pragma unroll
        for (int t = 1; t < kMaxSegments; ++t) i += (t < sa.nseg && r >= sa.start[t]) ? 1 : 0;
        return i;
    };
    auto load_rows = [&](v4u (&dst)[R][KC], int n0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = max(min(n0 + r, re - 1), 0);
            const int i = seg_of(n);
            const v4u* wrow = reinterpret_cast<const v4u*>(sa.w[i] + (int64_t)(n - sa.start[i]) * K);
#pragma unroll
            for (int j = 0; j < KC; ++j) dst[r][j] = __builtin_nontemporal_load(wrow + min(j * kWave + lane, k16 - 1));
        }
    };
    v4u cur[R][KC];
    load_rows(cur, rb);

#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + j * kThreads;
        if (c < nchunks) *reinterpret_cast<v4u*>(xs + c * 16) = xb[j];
    }
    __syncthreads();
    // The products run on the matrix cores: one 16x16x32 bf16 MFMA per 8 codes,
    // A = this lane's codes widened to bf16, B = the inputs at the same
    // positions, so the diagonal C[i][i] sums the products of the four lanes
    // with l % 16 == i.  Block FP8: lane l takes the codes loaded by lane
    // 4 (l % 16) + l / 16 (and reads the matching inputs), so diagonal
    // element i holds half of one 128-input group.
    const int src = V == VAR_FP8_BLOCK ? 4 * (lane & 15) + (lane >> 4) : lane;
    const int paddr = 4 * src;
    // slice o = j*64 + src: inputs 16 o .. 16 o + 15; slices past K are zero
    v4u xa[KC], xc[KC];
#pragma unroll
    for (int j = 0; j < KC; ++j) {
        const int o = j * kWave + src;
        const bool ok = o < k16;
        xa[j] = ok ? *reinterpret_cast<const v4u*>(xs + o * 32) : v4u{0, 0, 0, 0};
        xc[j] = ok ? *reinterpret_cast<const v4u*>(xs + o * 32 + 16) : v4u{0, 0, 0, 0};
    }
    const int kbs = K >> 7;
    auto slice_mfma = [&](const v4u& w, int j, v4f c) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16<V>(w.x, w.y), __builtin_bit_cast(v8bf, xa[j]), c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16<V>(w.z, w.w), __builtin_bit_cast(v8bf, xc[j]), c, 0, 0,
                                                       0);
    };
    auto diag = [&](const v4f& c) {
        const int e = lane & 3;
        const float v = e == 0 ? c.x : (e == 1 ? c.y : (e == 2 ? c.z : c.w));
        return ((lane & 15) >> 2) == (lane >> 4) ? v : 0.0f;
    };

    auto process = [&](const v4u (&wr)[R][KC], int n0) {
        float facc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float a = 0.0f;
            if constexpr (V == VAR_FP8_BLOCK) {
                const int n = max(min(n0 + r, re - 1), 0);
                const int i = seg_of(n);
                const uint16_t* swr = sa.sw[i] + (int64_t)((n - sa.start[i]) >> 7) * kbs;
#pragma unroll
                for (int j = 0; j < KC; ++j) {
                    const v4u w = {(unsigned)__builtin_amdgcn_ds_bpermute(paddr, (int)wr[r][j].x),
                                   (unsigned)__builtin_amdgcn_ds_bpermute(paddr, (int)wr[r][j].y),
                                   (unsigned)__builtin_amdgcn_ds_bpermute(paddr, (int)wr[r][j].z),
                                   (unsigned)__builtin_amdgcn_ds_bpermute(paddr, (int)wr[r][j].w)};
                    const v4f p = slice_mfma(w, j, v4f{0.f, 0.f, 0.f, 0.f});
                    const int g = min(8 * j + ((lane & 15) >> 1), kbs - 1);   // the diagonal element's group
                    a = __builtin_fmaf(diag(p), bf16_lo(swr[g]), a);
                }
            } else {
                v4f c = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < KC; ++j) c = slice_mfma(wr[r][j], j, c);
                a = diag(c);
            }
            facc[r] = wave_sum_f32(a);
        }
        if (lane < R && n0 + lane < re) {
            const int n = n0 + lane;
            const int i = seg_of(n);
            const int64_t local = n - sa.start[i];
            float a = facc[0];
#pragma unroll
            for (int r = 1; r < R; ++r) a = (lane == r) ? facc[r] : a;
            if constexpr (V == VAR_FP8_BLOCK) store_f32(sa.y[i], local, a, mode);
            else store_f32(sa.y[i], local, a * bf16_lo(sa.sw[i][local]), mode);
        }
    };
    if (rb < re) process(cur, rb);
    for (int n0 = rb + R; n0 < re; n0 += R) {
        load_rows(cur, n0);
        process(cur, n0);
    }
}

// ---------------------------------------------------------------------------
// 2..32 tokens
// ---------------------------------------------------------------------------

constexpr int kWoBatch = 2;         // K steps per load batch (two batches in flight)

template <int V, int MT, int NW>
__global__ __launch_bounds__(NW * 64) void wo_small_kernel(const uint16_t* __restrict__ x, SegmentArgs sa, int M,
                                                           int K, int mode) {
    // per-wave transpose buffer for one K step: 16 weight rows x 128 bytes,
    // then MT token tiles of 16 tokens x 256 bytes (bf16); reused for the
    // split-K reduction
    constexpr int TPB = 2048 + MT * 4096;
    constexpr int SMEM = NW * TPB > (int)(NW * MT * kWave * sizeof(v4f)) ? NW * TPB : (int)(NW * MT * kWave * sizeof(v4f));
    __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
    auto red = reinterpret_cast<v4f(*)[MT][kWave]>(smem);

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15;
    const int grp = lane >> 4;

    // 16-row tiles numbered across the segments; a tile never straddles two
    int tile = blockIdx.x, seg = 0;
#pragma unroll
    for (int i = 0; i + 1 < kMaxSegments; ++i) {
        const int nt = (sa.start[i + 1] - sa.start[i] + 15) >> 4;
        if (seg == i && i + 1 < sa.nseg && tile >= nt) {
            tile -= nt;
            seg = i + 1;
        }
    }
    const uint8_t* __restrict__ qw = sa.w[seg];
    const uint16_t* __restrict__ sw = sa.sw[seg];
    void* __restrict__ y = sa.y[seg];
    const int N = sa.start[seg + 1] - sa.start[seg];
    const int n0 = __builtin_amdgcn_readfirstlane(tile * 16);

    const int nsteps = (K + 127) >> 7;
    const int per = (nsteps + NW - 1) / NW;
    const int s_begin = wave * per;
    const int s_end = min(nsteps, s_begin + per);

    // Lane (r16, grp) takes K positions [16 grp, +16) and [64 + 16 grp, +16)
    // of each 128-wide step, for its weight row and for its tokens (both
    // operands use the same positions, so the contraction is unchanged).
    // Rows past N or M, K past the end and steps past the wave's range read
    // zero through the descriptors.
    const __amdgpu_buffer_rsrc_t dw = uniform_rsrc(qw + (int64_t)n0 * K, min(16, N - n0) * K);
    const __amdgpu_buffer_rsrc_t dx = uniform_rsrc(x, M * K * 2);
    // Loads cover whole 128-byte lines and go through this wave's LDS buffer
    // into the MFMA layout above: weights 8 rows x 128 bytes per instruction
    // (lane l: row l / 8, bytes 16 (l % 8)), inputs 4 tokens x 256 bytes per
    // instruction (lane l: token l / 16, bytes 16 (l % 16)).
    const int lr = lane >> 3, lp = lane & 7;
    const int woff = lr * K + lp * 16;
    int xoff[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = t * 16 + 4 * q + (lane >> 4);
            xoff[t][q] = m < M ? (m * K) * 2 + (lane & 15) * 16 : kOOB;
        }
    auto swz = [](int r) { return (r & 7) ^ ((r >> 3) & 1); };
    uint8_t* tpw = smem + wave * TPB;
    const int ww0 = lr * 128 + ((lp ^ swz(lr)) << 4), ww1 = (lr + 8) * 128 + ((lp ^ swz(lr + 8)) << 4);
    const int wr0 = r16 * 128 + ((grp ^ swz(r16)) << 4), wr1 = r16 * 128 + (((4 + grp) ^ swz(r16)) << 4);
    // token rows of 256 bytes, 16-byte chunk c of token m at chunk c ^ (m % 16)
    int xw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int m = 4 * q + (lane >> 4);
        xw[q] = m * 256 + (((lane & 15) ^ m) << 4);
    }
    const int xr[4] = {r16 * 256 + (((2 * grp) ^ r16) << 4), r16 * 256 + (((2 * grp + 1) ^ r16) << 4),
                       r16 * 256 + (((8 + 2 * grp) ^ r16) << 4), r16 * 256 + (((9 + 2 * grp) ^ r16) << 4)};
    const int kbs = K >> 7;
    const uint16_t* swblk = sw + (int64_t)(n0 >> 7) * kbs;  // block: the tile's 128-row block

    v4f acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

    constexpr int U = kWoBatch;
    v4u wa[2][U][2], xa[2][U][MT][4];
    float fw[2][U];
    auto issue = [&](auto bufc, int s0) {
        constexpr int bi = decltype(bufc)::value;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + u;
            const bool okw = (s < s_end) && (s * 128 + lp * 16 < K);
            const bool okx = (s < s_end) && (s * 128 + (lane & 15) * 8 < K);
            wa[bi][u][0] = __builtin_amdgcn_raw_buffer_load_b128(dw, okw ? woff + s * 128 : kOOB, 0, kAuxStream);
            wa[bi][u][1] = __builtin_amdgcn_raw_buffer_load_b128(dw, okw ? woff + 8 * K + s * 128 : kOOB, 0, kAuxStream);
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    xa[bi][u][t][q] = __builtin_amdgcn_raw_buffer_load_b128(
                        dx, okx && xoff[t][q] != kOOB ? xoff[t][q] + s * 256 : kOOB, 0, 0);
            if constexpr (V == VAR_FP8_BLOCK) fw[bi][u] = bf16_lo(swblk[min(s, s_end - 1)]);
        }
    };
    auto compute = [&](auto bufc, int s0) {
        constexpr int bi = decltype(bufc)::value;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // transpose this step through the wave's LDS buffer
            *reinterpret_cast<v4u*>(tpw + ww0) = wa[bi][u][0];
            *reinterpret_cast<v4u*>(tpw + ww1) = wa[bi][u][1];
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q) *reinterpret_cast<v4u*>(tpw + 2048 + t * 4096 + xw[q]) = xa[bi][u][t][q];
            const v4u w0 = *reinterpret_cast<const v4u*>(tpw + wr0), w1 = *reinterpret_cast<const v4u*>(tpw + wr1);
            v4u tx[MT][4];
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) tx[t][i] = *reinterpret_cast<const v4u*>(tpw + 2048 + t * 4096 + xr[i]);
            const v8bf a[4] = {codes_to_bf16<V>(w0.x, w0.y), codes_to_bf16<V>(w0.z, w0.w),
                               codes_to_bf16<V>(w1.x, w1.y), codes_to_bf16<V>(w1.z, w1.w)};
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                v4f p = V == VAR_FP8_BLOCK ? v4f{0.f, 0.f, 0.f, 0.f} : acc[t];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], __builtin_bit_cast(v8bf, tx[t][i]), p, 0, 0, 0);
                if constexpr (V == VAR_FP8_BLOCK) {
                    if (s0 + u < s_end) {
                        const float f = fw[bi][u];
                        acc[t].x = __builtin_fmaf(p.x, f, acc[t].x);
                        acc[t].y = __builtin_fmaf(p.y, f, acc[t].y);
                        acc[t].z = __builtin_fmaf(p.z, f, acc[t].z);
                        acc[t].w = __builtin_fmaf(p.w, f, acc[t].w);
                    }
                } else {
                    acc[t] = p;
                }
            }
        }
    };

    issue(IC<0>{}, s_begin);
    int s0 = s_begin;
    for (; s0 + U < s_end; s0 += 2 * U) {
        issue(IC<1>{}, s0 + U);
        __builtin_amdgcn_sched_barrier(0);
        compute(IC<0>{}, s0);
        issue(IC<0>{}, s0 + 2 * U);
        __builtin_amdgcn_sched_barrier(0);
        compute(IC<1>{}, s0 + U);
    }
    if (s0 < s_end) compute(IC<0>{}, s0);
    mfma_drain();      // the accumulators are stored to LDS next
    __syncthreads();   // every wave is done with its transpose buffer before the reduction reuses it

#pragma unroll
    for (int t = 0; t < MT; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();

    // sum the NW partial tiles; item (t, l): rows n0 + 4 (l / 16) .. + 3 of token 16 t + l % 16
    for (int it = tid; it < MT * kWave; it += NW * kWave) {
        const int t = it / kWave, l = it % kWave;
        v4f sum = red[0][t][l];
#pragma unroll
        for (int w2 = 1; w2 < NW; ++w2) sum += red[w2][t][l];
        const int m = t * 16 + (l & 15);
        if (m < M) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = n0 + (l >> 4) * 4 + e;
                if (n < N) {
                    const int64_t idx = (int64_t)m * N + n;
                    if constexpr (V == VAR_FP8_BLOCK) store_f32(y, idx, sum[e], mode);
                    else store_f32(y, idx, sum[e] * bf16_lo(sw[n]), mode);
                }
            }
        }
    }
}

template <int V, int KC>
void launch_wo_gemv_kc(int R, int grid, hipStream_t st, const uint16_t* x, int K, const SegmentArgs& sa, int mode) {
    if (R >= 2)
        hipLaunchKernelGGL((wo_gemv_kernel<V, KC, 2>), dim3(grid), dim3(kThreads), 0, st, x, K, sa, mode);
    else
        hipLaunchKernelGGL((wo_gemv_kernel<V, KC, 1>), dim3(grid), dim3(kThreads), 0, st, x, K, sa, mode);
}

template <int V>
void launch_wo_gemv_v(const uint16_t* x, int64_t K, const SegmentArgs& sa, int mode, hipStream_t st) {
    const int64_t ntot = sa.start[sa.nseg];
    const int64_t kc = (K + 1023) / 1024;
    // as the quantized one-row launch: one row per wavefront for rows up to
    // 4 KiB, two read together up to 8 KiB, two in turn beyond
    const int R = (kc > 4 && kc <= 8) ? 2 : 1;
    const int64_t rows = kc <= 4 ? 4 : 8;          // rows per workgroup of four wavefronts
    const int grid = (int)std::max<int64_t>(1, (ntot + rows - 1) / rows);
    const int k = (int)K;
    if (kc <= 1) launch_wo_gemv_kc<V, 1>(R, grid, st, x, k, sa, mode);
    else if (kc <= 2) launch_wo_gemv_kc<V, 2>(R, grid, st, x, k, sa, mode);
    else if (kc <= 4) launch_wo_gemv_kc<V, 4>(R, grid, st, x, k, sa, mode);
    else if (kc <= 8) launch_wo_gemv_kc<V, 8>(R, grid, st, x, k, sa, mode);
    else if (kc <= 12) launch_wo_gemv_kc<V, 12>(R, grid, st, x, k, sa, mode);
    else if (kc <= 14) launch_wo_gemv_kc<V, 14>(R, grid, st, x, k, sa, mode);
    else launch_wo_gemv_kc<V, 16>(R, grid, st, x, k, sa, mode);
}

template <int V>
void launch_wo_small_v(const uint16_t* x, int64_t M, int64_t K, const SegmentArgs& sa, int mode, hipStream_t st) {
    int64_t tiles = 0;
    for (int i = 0; i < sa.nseg; ++i) tiles += (sa.start[i + 1] - sa.start[i] + 15) / 16;
    const dim3 grid((unsigned)tiles);
    const int m = (int)M, k = (int)K;
    const bool wide_k = K > 4096;                  // 8 wavefronts split longer K
    if (M > 16) {
        if (wide_k) hipLaunchKernelGGL((wo_small_kernel<V, 2, 8>), grid, dim3(512), 0, st, x, sa, m, k, mode);
        else hipLaunchKernelGGL((wo_small_kernel<V, 2, 4>), grid, dim3(256), 0, st, x, sa, m, k, mode);
    } else {
        if (wide_k) hipLaunchKernelGGL((wo_small_kernel<V, 1, 8>), grid, dim3(512), 0, st, x, sa, m, k, mode);
        else hipLaunchKernelGGL((wo_small_kernel<V, 1, 4>), grid, dim3(256), 0, st, x, sa, m, k, mode);
    }
}

}  // namespace

hipError_t launch_weight_only(int variant, const uint16_t* x, int64_t M, int64_t K, const SegmentArgs& sa, int mode,
                              hipStream_t st) {
    const bool one = (M == 1) && (K <= kWeightOnlyRowMaxK);
    if (variant == VAR_INT8) {
        if (one) launch_wo_gemv_v<VAR_INT8>(x, K, sa, mode, st);
        else launch_wo_small_v<VAR_INT8>(x, M, K, sa, mode, st);
    } else if (variant == VAR_FP8_ROW) {
        if (one) launch_wo_gemv_v<VAR_FP8_ROW>(x, K, sa, mode, st);
        else launch_wo_small_v<VAR_FP8_ROW>(x, M, K, sa, mode, st);
    } else {
        if (one) launch_wo_gemv_v<VAR_FP8_BLOCK>(x, K, sa, mode, st);
        else launch_wo_small_v<VAR_FP8_BLOCK>(x, M, K, sa, mode, st);
    }
    return hipGetLastError();
}

}  // namespace qlin
