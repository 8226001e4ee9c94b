// Long-input products with the weights stored in the matrix-core operand
// order (W8A8 model card, "Loading": inputs of more than 32 rows are rounded
// per row and multiplied in int8 with int32 sums; the FP8 rowwise scheme the
// same way on E4M3 codes; Qwen3 8B FP8 card, "Loading": block-scaled E4M3
// with per-128-input activation scales).
//
// Packed layout ("operand order").  q_w [N, K] is cut into blocks of 32 rows
// and K-slices of S bytes (S = 32 for int8, 64 for E4M3: one MFMA's K); each
// slice of a block is stored as H = S / 32 units of 1 KB, unit h holding, for
// lane l = 0..63 of a wavefront, the 16 bytes that lane passes to the MFMA:
//   packed[((rb * (K / S) + s) * H + h) * 1024 + 16 l + b]
//     = q_w[32 rb + l % 32][S s + (S / 2) (l / 32) + 16 h + b],   b < 16.
// (v_mfma_i32_32x32x32_i8 takes row l % 32, bytes 16 (l / 32) .. + 16 of a
// 32-byte slice from lane l; v_mfma_f32_32x32x64_f8f6f4 bytes 32 (l / 32) ..
// + 32 of a 64-byte slice.)  In both code types a 128-byte K stage of one
// block is 4 KB of consecutive units.
//
// Why: a 128 x 64 output tile per CU (the o and down projections at 512
// tokens, whose outputs leave no larger tile for 256 CUs) moves 72 KB through
// LDS per 256 MFMA cycles when both operands are staged there -- 288 B/clk,
// above the LDS rate.  With the weights in operand order each wavefront loads
// its own 32 weight rows straight into registers, 1 KB contiguous per load,
// and only the tokens go through LDS (40 KB per 256 cycles).  The loop is then
// bound by its load instructions rather than by LDS or the matrix cores.
//
// Tile: 128 weight rows x BM tokens (BM = 64 or 128); KG = 1 or 2 K groups of
// four wavefronts (group g multiplies stages g, g + KG, ...), wavefront w of a
// group owns weight rows [32 w, 32 w + 32) and all BM tokens.  Tokens: a ring
// of four LDS buffers per group filled by direct copies (buffer_load ... lds)
// three steps ahead, 16-byte chunks XOR-swizzled by row; weights: a ring of
// four register sets loaded three steps ahead.  One barrier per step.  Group
// 1 adds its sums into group 0's through LDS; the epilogue is the rowwise one
// of the row-major tiled product (same f32 order, bf16 staged through LDS).
// Block FP8: a 128-row tile lies in one 128-row scale block, so a stage (one
// 128-input block) has one weight scale; each token tile's partial product is
// scaled by s_x[m][s] * s_w[n0 / 128][s] into the f32 accumulator.  SwiGLU
// (SG): the tile's rows are 64 gate rows and the up rows with the same
// indices, and the gate outputs reach the up wavefronts through LDS.
#include <type_traits>

#include "qlin_device.h"
#include "qlin_internal.h"

namespace qlin {

namespace {

template <int U> using PIC = std::integral_constant<int, U>;

constexpr int kPBN = 128;            // weight rows per tile
constexpr int kPGT = 256;            // threads per K group
constexpr int kPOOB = 0x40000000;    // an offset past every descriptor: reads zero

__device__ __forceinline__ int pswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ void pdma16(__amdgpu_buffer_rsrc_t r, uint8_t* dst, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, 0);
}

template <int V> struct PackedAcc { typedef v16f T; };
template <> struct PackedAcc<VAR_INT8> { typedef v16i T; };

__device__ __forceinline__ void pdma4(__amdgpu_buffer_rsrc_t r, void* dst, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 4, voff, 0, 0, 0);
}

template <int V, int BM, int KG, bool SG>
__global__ __launch_bounds__(kPGT * KG) void gemm_packed_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx, SegmentArgs sa, int M, int K, int mode,
    int tiles_m, int tiles_n) {
    typedef typename PackedAcc<V>::T Acc;
    constexpr bool BLK = V == VAR_FP8_BLOCK;
    constexpr int TM = BM / 32;                  // 32 x 32 MFMA tiles per wavefront (one weight row block)
    constexpr int BST = BM * 128;                // token bytes of one group stage
    constexpr int BW = BM / 32;                  // 1 KB token copies per wavefront and stage
    constexpr int PITCH = kPBN * 2 + 16;         // bf16 epilogue tile: BM rows of 128 outputs + 16 bytes
    static_assert(KG == 1 || KG == 2, "one or two K groups");
    static_assert((BM / 4) * PITCH <= KG * BST, "a quarter of the bf16 tile fits one ring array");
    static_assert(2 * TM * 16 * 64 * 4 <= KG * BST || KG == 1, "two wavefronts' partial sums fit one ring array");
    // four distinct arrays: the compiler then knows which buffer a copy writes
    __shared__ __attribute__((aligned(1024))) uint8_t L0[KG * BST], L1[KG * BST], L2[KG * BST], L3[KG * BST];
    // the epilogue's scales, copied straight into LDS (raw bf16 row scales, f32
    // token scales); not used by block FP8
    // (SwiGLU: the gate rows' scales in [0, 64), the up rows' in [128, 192))
    __shared__ __attribute__((aligned(16))) uint16_t s_w_raw[BLK ? 2 : SG ? 2 * kPBN : kPBN];
    __shared__ __attribute__((aligned(16))) float s_x_t[BLK ? 1 : BM];
    // block FP8: each stage's token scales s_x[m][s] ride a ring of four more
    // distinct arrays beside the token copies; wavefronts with no tokens to
    // copy write zeros to a spare slot so every wavefront issues the same count
    constexpr int XN = BLK ? KG * BM : 1;
    __shared__ __attribute__((aligned(16))) float X0[XN], X1[XN], X2[XN], X3[XN], XS[BLK ? 64 : 1];

    const int tid = threadIdx.x;
    const int grp = KG == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid / kPGT);
    const int gtid = tid & (kPGT - 1);
    const int wave = __builtin_amdgcn_readfirstlane(gtid >> 6);
    const int lane = tid & 63;
    const int half = lane >> 5;

    // XCD-aware tile order (workgroup b runs on XCD b % 8): the token tiles of
    // one weight panel run consecutively on one XCD
    const int ntiles = tiles_m * tiles_n;
    const int b = blockIdx.x;
    const int t = (ntiles & 7) ? b : ((b & 7) * (ntiles >> 3) + (b >> 3));
    int panel = __builtin_amdgcn_readfirstlane(t / tiles_m), seg = 0;
    if constexpr (!SG) {
#pragma unroll
        for (int i = 0; i + 1 < kMaxSegments; ++i) {
            const int np = (sa.start[i + 1] - sa.start[i]) / kPBN;   // segment widths are multiples of 128
            if (seg == i && i + 1 < sa.nseg && panel >= np) {
                panel -= np;
                seg = i + 1;
            }
        }
    }
    // SwiGLU (segment 0 = gate, 1 = up, both [I, K], y = h [M, I]): a tile's
    // 128 rows are 64 gate rows (wavefronts 0, 1) and the up rows with the same
    // indices (wavefronts 2, 3)
    const bool upw = SG && wave >= 2;
    // (selects over the statically loaded argument entries: no dependent scalar load)
    const uint8_t* __restrict__ wp = SG ? (upw ? sa.w[1] : sa.w[0]) : pick_ptr(sa.w, seg);
    const uint16_t* __restrict__ sw = SG ? (upw ? sa.sw[1] : sa.sw[0]) : pick_ptr(sa.sw, seg);
    void* __restrict__ y = SG ? sa.y[0] : pick_ptr(sa.y, seg);
    const int N = SG ? sa.start[1] : pick_int(sa.start + 1, seg) - pick_int(sa.start, seg);
    const int n0 = panel * (SG ? kPBN / 2 : kPBN);
    const int m0 = __builtin_amdgcn_readfirstlane((t % tiles_m) * BM);

    // this wavefront's 32-row weight block: 32 K bytes, 4 KB per stage
    const int rb = (n0 >> 5) + (SG ? (wave & 1) : wave);
    const __amdgpu_buffer_rsrc_t da = uniform_rsrc(wp + (int64_t)rb * 32 * K, 32 * K);
    const __amdgpu_buffer_rsrc_t db = uniform_rsrc(qx + (int64_t)m0 * K, min(BM, M - m0) * K);
    const int nk = K >> 7;
    // block FP8: the tokens' scales s_x[m][*] and the tile's block scales s_w[n0 / 128][*]
    const __amdgpu_buffer_rsrc_t dsx = uniform_rsrc(sx + (BLK ? (int64_t)m0 * nk : 0), BLK ? min(BM, M - m0) * nk * 4 : 0);
    const __amdgpu_buffer_rsrc_t dsw = uniform_rsrc(sw + (BLK ? (int64_t)(n0 >> 7) * nk : 0), BLK ? nk * 2 : 0);
    const int nko = (nk + KG - 1) / KG;
    const int nsteps = (nko + 3) & ~3;           // whole unrolled iterations; steps past the end multiply zeros
    auto gs = [&](int i) { return KG * i + grp; };

    auto buf = [&](auto bi) -> uint8_t* {
        constexpr int v = decltype(bi)::value;
        return (v == 0 ? L0 : v == 1 ? L1 : v == 2 ? L2 : L3) + grp * BST;
    };
    auto xbuf = [&](auto bi) -> float* {
        constexpr int v = decltype(bi)::value;
        return (v == 0 ? X0 : v == 1 ? X1 : v == 2 ? X2 : X3) + grp * BM;
    };
    v4u a0[4], a1[4], a2[4], a3[4];
    uint32_t wsc[4];                             // block FP8: each stage's s_w, beside its weights
    auto aset = [&](auto bi) -> v4u(&)[4] {
        constexpr int v = decltype(bi)::value;
        if constexpr (v == 0) return a0;
        else if constexpr (v == 1) return a1;
        else if constexpr (v == 2) return a2;
        else return a3;
    };
    // stage s: the wavefront's 4 weight units into register set bi, its share
    // of the token rows into LDS buffer bi (1 KB = 8 rows per copy, lane l in
    // row l / 8 loading logical chunk (l % 8) ^ swz(row) to keep the swizzle)
    auto issue = [&](auto bi, int s) {
        v4u(&ar)[4] = aset(bi);
        const bool in = s < nk;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            ar[u] = __builtin_amdgcn_raw_buffer_load_b128(da, in ? s * 4096 + u * 1024 + 16 * lane : kPOOB, 0, 0);
        uint8_t* dst = buf(bi);
#pragma unroll
        for (int j = 0; j < BW; ++j) {
            const int blk = wave * BW + j;
            const int r = blk * 8 + (lane >> 3);
            const int k = s * 128 + (((lane & 7) ^ pswz(r)) << 4);
            pdma16(db, dst + blk * 1024, k < K ? r * K + k : kPOOB);
        }
        if constexpr (BLK) {
            // the stage's weight block scale (2 bytes, every lane) into register set bi
            wsc[decltype(bi)::value] = __builtin_amdgcn_raw_buffer_load_b16(dsw, in ? 2 * s : kPOOB, 0, 0);
            // wavefront w < BM / 64 copies the scales of tokens 64 w .. 64 w + 63
            const bool real = wave < BM / 64;
            const int tok = 64 * wave + lane;
            pdma4(dsx, real ? (void*)(xbuf(bi) + 64 * wave) : (void*)XS, real && in ? (tok * nk + s) * 4 : kPOOB);
        }
    };


    Acc acc[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) acc[i] = Acc{};

    // Token fragments: sub-step u of a stage is one MFMA K slice (int8: 4 of
    // 32 bytes, E4M3: 2 of 64 bytes); a wavefront reads the TM fragments of
    // sub-step u + 1 from LDS while it multiplies those of u (two sets; the
    // scheduling barriers keep the compiler from sinking the reads next to
    // their MFMAs, which would expose the LDS latency at every pair).
    constexpr int NSUB = V == VAR_INT8 ? 4 : 2;
    typedef typename std::conditional<V == VAR_INT8, v4i, v8i>::type BFrag;
    BFrag bq[2][TM];
    auto rdsub = [&](auto bi, int p, int sub) {
        const uint8_t* base = buf(bi);
        auto rdq = [&](int r, int c) { return *reinterpret_cast<const v4i*>(base + r * 128 + ((c ^ pswz(r)) << 4)); };
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = i * 32 + (lane & 31);
            if constexpr (V == VAR_INT8) {
                bq[p][i] = rdq(r, 2 * sub + half);
            } else {
                const v4i lo = rdq(r, 4 * sub + 2 * half), hi = rdq(r, 4 * sub + 2 * half + 1);
                bq[p][i] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            }
        }
    };
    auto mfsub = [&](auto bi, int p, int sub) {
        const v4u(&ar)[4] = aset(bi);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if constexpr (V == VAR_INT8) {
                acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(v4i, ar[sub]), bq[p][i], acc[i], 0, 0, 0);
            } else {
                const v4u lo = ar[2 * sub], hi = ar[2 * sub + 1];
                const v8i a = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bq[p][i], acc[i], 0, 0, 0, 0, 0, 0);
            }
        }
    };
    // sub-step 0's reads were issued before the stage's loads (see step)
    auto compute = [&](auto bi) {
#pragma unroll
        for (int sub = 0; sub < NSUB; ++sub) {
            if (sub + 1 < NSUB) rdsub(bi, (sub + 1) & 1, sub + 1);
            __builtin_amdgcn_sched_barrier(0);
            mfsub(bi, sub & 1, sub);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Block FP8, tile-major: token tile i's two MFMAs (the stage's two K
    // slices, one 128-input block) start from zero, and the partial is scaled
    // by s_x[m][s] * s_w[n0 / 128][s] into the accumulator while the next
    // tile's MFMAs run (two partials live); tile i + 1's fragments are read
    // while tile i is multiplied.
    v8i bt[2][2];
    v16f pt[2];
    auto rdtile = [&](auto bi, int p, int i) {
        const uint8_t* base = buf(bi);
        auto rdq = [&](int r, int c) { return *reinterpret_cast<const v4i*>(base + r * 128 + ((c ^ pswz(r)) << 4)); };
        const int r = i * 32 + (lane & 31);
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const v4i lo = rdq(r, 4 * sub + 2 * half), hi = rdq(r, 4 * sub + 2 * half + 1);
            bt[p][sub] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        }
    };
    auto compute_blk = [&](auto bi) {
        const v4u(&ar)[4] = aset(bi);
        const v8i a0v = v8i{(int)ar[0].x, (int)ar[0].y, (int)ar[0].z, (int)ar[0].w,
                            (int)ar[1].x, (int)ar[1].y, (int)ar[1].z, (int)ar[1].w};
        const v8i a1v = v8i{(int)ar[2].x, (int)ar[2].y, (int)ar[2].z, (int)ar[2].w,
                            (int)ar[3].x, (int)ar[3].y, (int)ar[3].z, (int)ar[3].w};
        // (stages past the end carry zero codes and zero scales)
        const float fw = bf16_lo(wsc[decltype(bi)::value]);
        float fx[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) fx[i] = xbuf(bi)[i * 32 + (lane & 31)] * fw;
#pragma unroll
        for (int t = 0; t <= TM; ++t) {
            if (t + 1 < TM) rdtile(bi, (t + 1) & 1, t + 1);
            __builtin_amdgcn_sched_barrier(0);
            if (t < TM) {
                pt[t & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0v, bt[t & 1][0], v16f{}, 0, 0, 0, 0, 0, 0);
                pt[t & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1v, bt[t & 1][1], pt[t & 1], 0, 0, 0, 0, 0, 0);
            }
            if (t > 0) {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    acc[t - 1][e] = __builtin_fmaf(pt[(t - 1) & 1][e], fx[t - 1], acc[t - 1][e]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Step kt multiplies stage gs(kt) from register set / buffer kt % 4 once
    // this wavefront's loads of it are complete (the loads of the two later
    // stages may stay in flight: vmcnt <= twice one stage's count, 4 + BW, and
    // two more for block FP8's scales) and every wavefront has
    // passed the barrier (so their copies of it are in LDS and nobody still
    // reads buffer (kt + 3) % 4), then issues stage gs(kt + 3) into set and
    // buffer (kt + 3) % 4.  The explicit s_barrier (no fence) leaves those
    // later copies in flight; the memory clobber keeps LDS reads after it.
    constexpr int VMC = 2 * (4 + BW + (BLK ? 2 : 0));
    constexpr int WIMM = (VMC & 15) | ((VMC >> 4) << 14) | 0x0F70;   // vmcnt(VMC), expcnt and lgkmcnt not waited
    // scales first (older than every stage load, so the first step's wait
    // covers them; no register waits for them): wavefront 0 of group 0 copies
    // the 128 row scales (256 bytes), wavefront 1 the BM token scales (tokens
    // past M read as zero and are never stored); block FP8 loads its scales
    // with each stage instead
    if (!BLK && grp == 0 && (wave == 0 || (SG && wave == 2))) {
        // SwiGLU: 64 gate scales (wavefront 0) and 64 up scales (wavefront 2);
        // the other half of each copy reads zeros
        const __amdgpu_buffer_rsrc_t ds = uniform_rsrc(sw + n0, SG ? kPBN : kPBN * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ds, (__attribute__((address_space(3))) void*)(s_w_raw + (upw ? kPBN : 0)), 4,
                                                 4 * lane, 0, 0, 0);
    } else if (!BLK && grp == 0 && wave == 1) {
        const __amdgpu_buffer_rsrc_t ds = uniform_rsrc(sx + m0, min(BM, M - m0) * 4);
#pragma unroll
        for (int j = 0; j < BM / 64; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ds, (__attribute__((address_space(3))) void*)(s_x_t + 64 * j), 4,
                                                     4 * (64 * j + lane), 0, 0, 0);
    }
    // the first three stages in issue order (stage 0's weights and tokens are
    // the oldest loads: the first step's vmcnt bound relies on it)
    __builtin_amdgcn_sched_barrier(0);
    issue(PIC<0>{}, gs(0));
    __builtin_amdgcn_sched_barrier(0);
    issue(PIC<1>{}, gs(1));
    __builtin_amdgcn_sched_barrier(0);
    issue(PIC<2>{}, gs(2));
    int kt = 0;
    auto step = [&](auto bi) {
        constexpr int v = decltype(bi)::value;
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(WIMM);
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (BLK) rdtile(bi, 0, 0);    // in flight while the next stage's loads issue
        else rdsub(bi, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        issue(PIC<(v + 3) & 3>{}, gs(kt + 3));
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (BLK) compute_blk(bi);
        else compute(bi);
    };
    // one loop exit (with an exit after every step the compiler drains every
    // load in flight at the top of the loop)
    for (; kt < nsteps; kt += 4) {
        step(PIC<0>{});
        ++kt;
        step(PIC<1>{});
        ++kt;
        step(PIC<2>{});
        ++kt;
        step(PIC<3>{});
        kt -= 3;
    }
    mfma_drain();
    __builtin_amdgcn_s_waitcnt(0x0F70);          // the copies of the stages past the end have landed
    __syncthreads();

    // group 1 hands its sums to group 0 (wavefronts 0, 1 through L0, 2, 3 through L1)
    uint32_t* part = reinterpret_cast<uint32_t*>(wave < 2 ? L0 : L1) + ((wave & 1) * TM * 16) * 64 + lane;
    if (KG == 2 && grp == 1) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                if constexpr (V == VAR_INT8) part[(i * 16 + e) * 64] = (uint32_t)acc[i][e];
                else part[(i * 16 + e) * 64] = __float_as_uint(acc[i][e]);
            }
    }
    if (KG == 2) __syncthreads();
    if (KG == 2 && grp == 0) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t v = part[(i * 16 + e) * 64];
                if constexpr (V == VAR_INT8) acc[i][e] += (int)v;
                else acc[i][e] += __uint_as_float(v);
            }
    }

    // Epilogue.  Lane l, element e of token tile i: weight row
    // n0 + 32 w + 8 (e / 4) + 4 (l / 32) + e % 4, token m0 + 32 i + l % 32
    // (SwiGLU: gate / up row n0 + 32 (w % 2) + ...).  The scaled f32 output:
    auto outv = [&](int i, int e) -> float {
        if constexpr (BLK) {
            return acc[i][e];                    // scaled per block in the loop
        } else {
            const int nl = wave * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
            const float f = s_x_t[BLK ? 0 : i * 32 + (lane & 31)] * bf16_lo(s_w_raw[SG && nl >= 64 ? nl + 64 : nl]);
            if constexpr (V == VAR_INT8) return (float)acc[i][e] * f;
            else return acc[i][e] * f;
        }
    };
    if constexpr (SG) {
        // the gate wavefronts' outputs go to LDS (wavefront 0 to L2, 1 to L3,
        // free after the partial sums went through L0 / L1); the up wavefront
        // with the same rows (2, 3) forms h = swiglu(g, u) for them, staged in
        // L0 / L1 as BM rows of 64 bf16, then written as 16-byte row pieces
        if (KG == 2) __syncthreads();            // group 0 has read the partial sums
        float* gx = reinterpret_cast<float*>((wave & 1) ? L3 : L2) + lane;
        if (grp == 0 && wave < 2) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) gx[(i * 16 + e) * 64] = outv(i, e);
        }
        __syncthreads();
        constexpr int HP = kPBN + 16;           // 64 bf16 + 16 bytes per staged row
        auto hrow = [&](int r) { return r < BM / 2 ? L0 + r * HP : L1 + (r - BM / 2) * HP; };
        if (grp == 0 && wave >= 2) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int ml = i * 32 + (lane & 31);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    uint16_t hv[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) hv[k] = swiglu_bf16(gx[(i * 16 + 4 * g + k) * 64], outv(i, 4 * g + k));
                    const int jl = (wave - 2) * 32 + 8 * g + 4 * half;
                    *reinterpret_cast<v2u*>(hrow(ml) + jl * 2) =
                        v2u{(uint32_t)hv[0] | ((uint32_t)hv[1] << 16), (uint32_t)hv[2] | ((uint32_t)hv[3] << 16)};
                }
            }
        }
        __syncthreads();
        for (int id = tid; id < BM * 8; id += kPGT * KG) {
            const int row = id >> 3, c = id & 7;
            const int m = m0 + row;
            if (m < M)
                *reinterpret_cast<v4u*>(static_cast<uint16_t*>(y) + (int64_t)m * N + n0 + 8 * c) =
                    *reinterpret_cast<const v4u*>(hrow(row) + 16 * c);
        }
        return;
    }
    if (mode == OUT_BF16) {
        // a quarter of the tile's token rows in each ring array (free: the
        // partial sums went through L0 / L1 before the barrier below them)
        constexpr int RQ = BM / 4;
        auto erow = [&](int r) {
            const int q = r / RQ;
            return (q == 0 ? L0 : q == 1 ? L1 : q == 2 ? L2 : L3) + (r % RQ) * PITCH;
        };
        if (KG == 2) __syncthreads();          // group 0 has read the partial sums
        if (grp == 0) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int ml = i * 32 + (lane & 31);
                const float sxm = BLK ? 0.f : s_x_t[BLK ? 0 : ml];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int nl = wave * 32 + 8 * g + 4 * half;
                    float v[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        if constexpr (V == VAR_INT8) v[k] = (float)acc[i][4 * g + k] * (sxm * bf16_lo(s_w_raw[nl + k]));
                        else if constexpr (BLK) v[k] = acc[i][4 * g + k];     // scaled per block in the loop
                        else v[k] = acc[i][4 * g + k] * (sxm * bf16_lo(s_w_raw[nl + k]));
                    }
                    const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
                    const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
                    *reinterpret_cast<v2u*>(erow(ml) + nl * 2) = v2u{lo, hi};
                }
            }
        }
        __syncthreads();
        constexpr int CPR = kPBN * 2 / 16;       // 16-byte pieces per tile row
        for (int id = tid; id < BM * CPR; id += kPGT * KG) {
            const int row = id / CPR, c = id % CPR;
            const int m = m0 + row;
            if (m < M)
                *reinterpret_cast<v4u*>(static_cast<uint16_t*>(y) + (int64_t)m * N + n0 + 8 * c) =
                    *reinterpret_cast<const v4u*>(erow(row) + 16 * c);
        }
        return;
    }
    if (grp != 0) return;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int ml = i * 32 + (lane & 31);
        const int m = m0 + ml;
        if (m >= M) continue;
        const float sxm = BLK ? 0.f : s_x_t[BLK ? 0 : ml];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int nl = wave * 32 + 8 * g + 4 * half;
            const int64_t idx = (int64_t)m * N + n0 + nl;
            if constexpr (V == VAR_INT8) {
                const int a[4] = {acc[i][4 * g], acc[i][4 * g + 1], acc[i][4 * g + 2], acc[i][4 * g + 3]};
                const float w4[4] = {bf16_lo(s_w_raw[nl]), bf16_lo(s_w_raw[nl + 1]), bf16_lo(s_w_raw[nl + 2]), bf16_lo(s_w_raw[nl + 3])};
                store4_rowwise_i32acc(y, idx, a, sxm, w4, mode);
            } else if constexpr (BLK) {
                const float v4[4] = {acc[i][4 * g], acc[i][4 * g + 1], acc[i][4 * g + 2], acc[i][4 * g + 3]};
                store4_f32(y, idx, v4, mode);
            } else {
                const float v4[4] = {acc[i][4 * g] * (sxm * bf16_lo(s_w_raw[nl])), acc[i][4 * g + 1] * (sxm * bf16_lo(s_w_raw[nl + 1])),
                                     acc[i][4 * g + 2] * (sxm * bf16_lo(s_w_raw[nl + 2])), acc[i][4 * g + 3] * (sxm * bf16_lo(s_w_raw[nl + 3]))};
                store4_f32(y, idx, v4, mode);
            }
        }
    }
}

// One thread per 16-byte unit of the packed layout (see the top of this file).
template <int S>
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint8_t* __restrict__ w, uint8_t* __restrict__ p,
                                                           int64_t units, int K) {
    constexpr int H = S / 32;
    const int64_t per_block = (int64_t)K / S * H * 64;     // units per 32-row block
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < units; g += (int64_t)gridDim.x * 256) {
        const int64_t rb = g / per_block;
        const int64_t q = g - rb * per_block;
        const int l = (int)(q & 63);
        const int64_t sh = q >> 6;                          // s * H + h
        const int64_t s = sh / H;
        const int h = (int)(sh - s * H);
        const int64_t row = 32 * rb + (l & 31);
        const int64_t col = S * s + (S / 2) * (l >> 5) + 16 * h;
        *reinterpret_cast<v4u*>(p + g * 16) = *reinterpret_cast<const v4u*>(w + row * K + col);
    }
}

// weight panels of a call: 128 rows of the segments, or (SwiGLU) 64 gate rows
// with the matching up rows
int64_t packed_panels(const SegmentArgs& sa, int mode) {
    if (mode == OUT_SWIGLU) return sa.start[1] / (kPBN / 2);
    int64_t tn = 0;
    for (int i = 0; i < sa.nseg; ++i) tn += (sa.start[i + 1] - sa.start[i]) / kPBN;
    return tn;
}

template <int V, int BM, int KG>
hipError_t launch_packed_tile(const uint8_t* qx, const float* sx, const SegmentArgs& sa, int64_t M, int64_t K,
                              int mode, hipStream_t st) {
    const int64_t tm = (M + BM - 1) / BM;
    const int64_t tn = packed_panels(sa, mode);
    if (tm * tn > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (mode == OUT_SWIGLU)
        hipLaunchKernelGGL((gemm_packed_kernel<V, BM, KG, true>), dim3((unsigned)(tm * tn)), dim3(kPGT * KG), 0, st,
                           qx, sx, sa, (int)M, (int)K, mode, (int)tm, (int)tn);
    else
        hipLaunchKernelGGL((gemm_packed_kernel<V, BM, KG, false>), dim3((unsigned)(tm * tn)), dim3(kPGT * KG), 0, st,
                           qx, sx, sa, (int)M, (int)K, mode, (int)tm, (int)tn);
    return hipGetLastError();
}

template <int V>
hipError_t launch_packed_shape(int shape, const uint8_t* qx, const float* sx, const SegmentArgs& sa, int64_t M,
                               int64_t K, int mode, hipStream_t st) {
    return shape == 2   ? launch_packed_tile<V, 128, 1>(qx, sx, sa, M, K, mode, st)
           : shape == 1 ? launch_packed_tile<V, 128, 2>(qx, sx, sa, M, K, mode, st)
                        : launch_packed_tile<V, 64, 2>(qx, sx, sa, M, K, mode, st);
}

}  // namespace

// Tile choice.  One 8-wavefront workgroup (two K groups) per CU: 128 x 128
// tiles when there are 192 to 256 of them (q/k/v at 512 tokens, o and down at
// 1024), else 128 x 64 below that (o and down at 512 tokens).  Past 256 tiles
// of 128 x 128 (q/k/v at 1024 tokens: 384) a second round of 8-wavefront
// workgroups would leave half the CUs idle; 4-wavefront workgroups (one K
// group, 64 KB of LDS) run two per CU instead.
hipError_t launch_gemm_packed(int variant, const uint8_t* qx, const float* sx, const SegmentArgs& sa, int64_t M,
                              int64_t K, int mode, hipStream_t st) {
    const int64_t t128 = ((M + 127) / 128) * packed_panels(sa, mode);
    const int shape = t128 > 256 ? 2 : t128 >= 192 ? 1 : 0;
    if (variant == VAR_INT8) return launch_packed_shape<VAR_INT8>(shape, qx, sx, sa, M, K, mode, st);
    if (variant == VAR_FP8_ROW) return launch_packed_shape<VAR_FP8_ROW>(shape, qx, sx, sa, M, K, mode, st);
    if (variant == VAR_FP8_BLOCK) return launch_packed_shape<VAR_FP8_BLOCK>(shape, qx, sx, sa, M, K, mode, st);
    return hipErrorInvalidValue;
}

hipError_t launch_pack_weights(int variant, const uint8_t* w, int64_t N, int64_t K, uint8_t* p, hipStream_t st) {
    const int64_t units = N * K / 16;
    const int64_t blocks = (units + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
    if (variant == VAR_INT8) hipLaunchKernelGGL((pack_weights_kernel<32>), dim3(grid), dim3(256), 0, st, w, p, units, (int)K);
    else if (variant == VAR_FP8_ROW || variant == VAR_FP8_BLOCK)
        hipLaunchKernelGGL((pack_weights_kernel<64>), dim3(grid), dim3(256), 0, st, w, p, units, (int)K);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace qlin
