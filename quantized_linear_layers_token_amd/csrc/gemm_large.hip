// Long-input products on the matrix cores (W8A8 model card, "Loading": inputs
// of more than 32 rows are quantized per row and multiplied in int8 with int32
// accumulation; Qwen3 8B FP8 card, "Loading": block-scaled FP8 product).
//
// Tiled GEMM, both operands K-contiguous.  Output tile = BN weight rows x BM
// tokens, 4 wavefronts (8 for two K groups or the 8-wave 256 x 256 tile) in a
// WN x WM grid; a wave owns a (BN/WN) x (BM/WM) sub-tile of 32 x 32 MFMA tiles:
//   int8: v_mfma_i32_32x32x32_i8      (4 per 128-byte K stage, 32 cycles each)
//   E4M3: v_mfma_f32_32x32x64_f8f6f4  (2 per 128-byte K stage, 64 cycles each)
// (32 x 32 tiles need half the LDS operand bytes per MAC of 16 x 16 ones.)
// Unit rates measured on one CU: LDS reads ~240 B/clk, LDS writes (ds_write
// or direct loads) ~75 B/clk, global loads ~60 B/clk, so a tile's LDS writes
// and global loads per MFMA cycle are what bigger tiles save.
//
// K advances in 128-byte stages, one barrier per stage.  Register staging
// (every tile but one): stage s is loaded from global memory into one of two
// register sets at iteration s - 2, written to one of two LDS buffers at
// iteration s - 1, and multiplied at iteration s; register loads give the
// compiler exact per-register wait counts, so two stages of loads stay in
// flight.  Direct staging (the 4-wavefront 256 x 256 tile): stage s + 1 goes
// from global memory straight into the other LDS buffer while stage s is
// multiplied, and the step ends by waiting for it; the two buffers are
// distinct LDS arrays, so the compiler does not drain those loads before the
// reads of the current buffer.  LDS rows are 128 bytes with the
// 16-byte chunk index XOR-swizzled by swz(row) = (row & 7) ^ ((row >> 3) & 1):
// an MFMA operand read (one logical chunk of 16 consecutive rows per 16-lane
// phase) hits 16 distinct 16-byte bank groups.
//
// A operand = weight rows (n), B operand = tokens (m): a lane's 16 accumulator
// values are 16 rows n of one token column m inside one 32-row slab.  For block
// FP8 a stage is exactly one 128-wide K block: the stage's partial product is
// scaled by s_x[m, kb] * s_w[n/128, kb] (one factor per lane and MFMA tile)
// and added to the f32 accumulator; the factors ride with the stage's loads.
//
// Tile order is XCD-aware: workgroup b runs on XCD b % 8; tile ids are
// assigned so that tiles sharing a weight panel are consecutive on one XCD.
//
// 256 x 256 tiles (rowwise schemes), one workgroup per CU; per MAC they fetch
// and write to LDS half the bytes of a 128 x 128 tile.  With 4 wavefronts of
// 128 x 128 (one per SIMD, 256 accumulators each) the operands of K sub-step
// s + 1 are read while the MFMAs of s run.  With 8 wavefronts of 128 x 64 (two
// per SIMD, 128 accumulators and two staging sets each) there is no room for
// that read-ahead: operands are read right before their MFMAs and the other
// wavefront on the SIMD covers the latency.
//
// K groups (KG = 2): 512 threads in two groups of four wavefronts; group g
// multiplies stages g, g + 2, ... of the same tile from its own pair of LDS
// buffers, and group 1 adds its partial sums into group 0's through LDS before
// the epilogue (int32 sums stay exact).  With too few tiles for two
// workgroups per CU, a tile then still keeps two wavefronts per SIMD.
//
// SwiGLU mode (SG): the BN weight rows of a tile are BN/2 gate rows j0.. and
// the up rows with the same indices; the bf16 epilogue tile in LDS then holds
// gate and up of each (j, m), and the store pass writes
// h = swiglu_bf16(gate, up), BN/2 columns per tile.
#include <type_traits>

#include "qlin_device.h"
#include "qlin_internal.h"

namespace qlin {

namespace {

constexpr int kBK = 128;

template <int V> struct LargeAcc { typedef v16i T; };
template <> struct LargeAcc<VAR_FP8_ROW> { typedef v16f T; };
template <> struct LargeAcc<VAR_FP8_BLOCK> { typedef v16f T; };

template <int U> using IC = std::integral_constant<int, U>;

// 16 bytes per lane from a buffer into LDS: lane l's bytes land at dst + 16 l
// (dst is the same for the whole wave).  A plain device function: inside the
// kernel's lambdas the builtin would also be seen by the host pass.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* dst, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int V, int BN, int BM, int WN, int WM, bool SG, int KG, bool DM>
__global__ __launch_bounds__(64 * WN * WM * KG) void gemm_large_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx, SegmentArgs sa,
    int M, int K, int mode, int tiles_m, int tiles_n) {
    typedef typename LargeAcc<V>::T Acc;
    static_assert(WN * WM == 4 || WN * WM == 8, "four or eight wavefronts per K group");
    constexpr int GT = 64 * WN * WM;                     // threads per K group
    static_assert(KG == 1 || KG == 2, "one or two K groups");
    constexpr int NTH = GT * KG;
    constexpr int SN = BN / WN, SM = BM / WM;              // wave sub-tile
    constexpr int TN = SN / 32, TM = SM / 32;              // 32x32 MFMA tiles per wave
    constexpr int ROWS = BN + BM;                          // LDS rows per stage (weights first)
    constexpr int STAGE = ROWS * kBK;
    constexpr int CH = ROWS * 8 / GT;                      // 16-byte chunks per thread per stage
    static_assert(ROWS * 8 % GT == 0 && TN >= 1 && TM >= 1 && SN % 32 == 0 && SM % 32 == 0, "tile");
    // MFMA groups per stage at which loads are issued (see compute)
    constexpr int HOOKS = V == VAR_INT8 ? 4 * TN : (V == VAR_FP8_ROW ? 2 * TN : TN * TM);
    constexpr bool LOWREG = BN == 256 && BM == 256;        // 8 wavefronts of 128 x 64
    // Two LDS arrays: stage buffer 0 of every K group in ldsA, buffer 1 in
    // ldsB (distinct arrays, so the compiler knows that the direct loads into
    // one buffer leave reads of the other alone).  The bf16 epilogue tile (BM
    // rows of BN bf16 + 16 bytes) reuses them: its first BM/2 rows in ldsA,
    // the rest in ldsB.
    constexpr int PITCH = BN * 2 + 16;
    constexpr int LDSH = KG * STAGE > (BM / 2) * PITCH ? KG * STAGE : (BM / 2) * PITCH;
    __shared__ __attribute__((aligned(1024))) uint8_t ldsA[LDSH];
    __shared__ __attribute__((aligned(1024))) uint8_t ldsB[LDSH];
    auto erow = [&](int r) { return r < BM / 2 ? ldsA + r * PITCH : ldsB + (r - BM / 2) * PITCH; };
    __shared__ float s_w_t[BN], s_x_t[BM];                // rowwise schemes: this tile's scales

    const int tid = threadIdx.x;
    const int gtid = tid & (GT - 1);                       // thread index inside its K group
    const int grp = __builtin_amdgcn_readfirstlane(tid / GT);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(gtid >> 6);
    const int wn = wave / WM, wm = wave % WM;

    const int ntiles = tiles_m * tiles_n;
    const int b = blockIdx.x;
    const int t = (ntiles & 7) ? b : ((b & 7) * (ntiles >> 3) + (b >> 3));
    // weight panels are numbered across the segments (q, k, v or gate, up
    // sharing one input); a panel never straddles two segments.  The integer
    // division runs on the vector ALU: readfirstlane returns the (uniform)
    // results to scalar registers, so the buffer descriptors built from them
    // are scalar (a descriptor the compiler takes as divergent costs a
    // readfirstlane loop around every load).
    // (SG: a panel is BN/2 gate rows and the same BN/2 up rows)
    constexpr int PR = SG ? BN / 2 : BN;                   // rows of one segment per panel
    int panel = __builtin_amdgcn_readfirstlane(t / tiles_m), seg = 0;
    if constexpr (!SG) {
#pragma unroll
        for (int i = 0; i + 1 < kMaxSegments; ++i) {
            const int np = (sa.start[i + 1] - sa.start[i] + BN - 1) / BN;
            if (seg == i && i + 1 < sa.nseg && panel >= np) {
                panel -= np;
                seg = i + 1;
            }
        }
    }
    const uint8_t* __restrict__ qw = sa.w[seg];
    const uint16_t* __restrict__ sw = sa.sw[seg];
    const uint16_t* __restrict__ sw_u = sa.sw[SG ? 1 : 0];
    void* __restrict__ y = sa.y[seg];
    const int N = sa.start[seg + 1] - sa.start[seg];
    const int n0 = panel * PR;
    const int m0 = __builtin_amdgcn_readfirstlane((t % tiles_m) * BM);

    // ---- global -> register -> LDS assignment.  Thread tid carries logical
    // 16-byte chunk tid % 8 of rows tid / 8 + RP j (RP = GT / 8 rows per pass).  Loads go through buffer
    // descriptors spanning this tile's weight rows and token rows: rows past N
    // or M lie outside the descriptor's range and read as zero.
    constexpr int RP = GT / 8;
    constexpr int JW = BN / RP, JX = BM / RP, JR = JW > JX ? JW : JX;
    static_assert(JW + JX == CH, "chunk split");
    const int cthr = gtid & 7;
    const __amdgpu_buffer_rsrc_t dw = uniform_rsrc(qw + (int64_t)n0 * K, min(PR, N - n0) * K);
    const __amdgpu_buffer_rsrc_t du = uniform_rsrc(sa.w[SG ? 1 : 0] + (int64_t)n0 * K, SG ? min(PR, N - n0) * K : 0);
    const __amdgpu_buffer_rsrc_t dx = uniform_rsrc(qx + (int64_t)m0 * K, min(BM, M - m0) * K);
    int roff[JR];                                          // byte offset of each carried row
#pragma unroll
    for (int j = 0; j < JR; ++j) roff[j] = ((gtid >> 3) + RP * j) * K;
    // LDS byte offset of carried row j: row r = tid / 8 + RP j keeps swz(r)
    const int loff0 = (gtid >> 3) * kBK + ((cthr ^ swz(gtid >> 3)) << 4);
    const int nk = (K + kBK - 1) / kBK;
    // K group g multiplies stages g, g + KG, g + 2 KG, ... from its own pair of
    // LDS buffers; both groups run the same number of steps (barriers are
    // shared), a step past the last stage multiplies a zero stage.
    const int nko = (nk + KG - 1) / KG;
    // LDS stage buffer b of this thread's K group
    auto sbuf = [&](auto b) { return (decltype(b)::value ? ldsB : ldsA) + grp * STAGE; };
    auto gs = [&](int i) { return KG * i + grp; };
    const int kbs = K >> 7;

    // Register staging: stage s is loaded into register set s % 2 while stage
    // s - 2 is multiplied, and written to LDS buffer s % 2 after stage s - 1
    // is multiplied.  The loads are spread between the MFMAs (hook points in
    // compute) so that the address unit is never handed a burst that stalls
    // MFMA issue.  Block FP8: a stage's factors load with the set and move to
    // the buffer's copy when the set is written.
    v4u rx[CH], ry[CH];
    float fxx[TM], fwx[TN], fxy[TM], fwy[TN];             // factors of the register sets
    float fx0[TM], fw0[TN], fx1[TM], fw1[TN];             // factors of the LDS buffers
    auto issue_one = [&](auto set, int s, int j) {
        v4u(&r)[CH] = decltype(set)::value ? ry : rx;
        // chunks past K re-read the row's last chunk (zeroed when written to LDS),
        // so every in-range offset stays inside its row
        const int k = min(s * kBK + cthr * 16, K - 16);
        if (SG && j >= JW / 2 && j < JW) r[j] = __builtin_amdgcn_raw_buffer_load_b128(du, roff[j - JW / 2] + k, 0, 0);
        else if (j < JW) r[j] = __builtin_amdgcn_raw_buffer_load_b128(dw, roff[j] + k, 0, 0);
        else r[j] = __builtin_amdgcn_raw_buffer_load_b128(dx, roff[j - JW] + k, 0, 0);
    };
    auto issue_fac = [&](auto set, int s) {
        if constexpr (V == VAR_FP8_BLOCK) {
            float(&fx)[TM] = decltype(set)::value ? fxy : fxx;
            float(&fw)[TN] = decltype(set)::value ? fwy : fwx;
            const int kb = min(s, kbs - 1);                    // a stage past the end reloads the last block's factors
#pragma unroll
            for (int jj = 0; jj < TM; ++jj)
                fx[jj] = sx[(int64_t)min(m0 + wm * SM + jj * 32 + (lane & 31), M - 1) * kbs + kb];
#pragma unroll
            for (int ii = 0; ii < TN; ++ii) {
                const int rr = wn * SN + ii * 32;              // tile row (SG: >= BN/2 are up rows)
                if (SG && rr >= PR) fw[ii] = bf16_lo(sw_u[(int64_t)(min(n0 + rr - PR, N - 1) >> 7) * kbs + kb]);
                else fw[ii] = bf16_lo(sw[(int64_t)(min(n0 + rr, N - 1) >> 7) * kbs + kb]);
            }
        }
    };
    auto issue_all = [&](auto set, int s) {
#pragma unroll
        for (int j = 0; j < CH; ++j) issue_one(set, s, j);
        issue_fac(set, s);
    };
    // hook point h of HOOKS in one stage's MFMA sequence: its share of the loads
    auto hook = [&](auto set, int s, int h) {
        __builtin_amdgcn_sched_barrier(0);
        if (h == 0) issue_fac(set, s);
#pragma unroll
        for (int j = h * CH / HOOKS; j < (h + 1) * CH / HOOKS; ++j) issue_one(set, s, j);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto write = [&](auto set, auto buf, int s) {
        const v4u(&r)[CH] = decltype(set)::value ? ry : rx;
        uint8_t* base = sbuf(buf);
        if (KG > 1 && s >= nk) {
            // a K group's step past the last stage: zeros
#pragma unroll
            for (int j = 0; j < CH; ++j) *reinterpret_cast<v4u*>(base + loff0 + j * RP * kBK) = v4u{0, 0, 0, 0};
        } else if ((K & (kBK - 1)) == 0) {
            // whole stages only: a stage past the end is written but never multiplied
#pragma unroll
            for (int j = 0; j < CH; ++j) *reinterpret_cast<v4u*>(base + loff0 + j * RP * kBK) = r[j];
        } else {
            const bool ok = s * kBK + cthr * 16 < K;       // false in the ragged last stage and past the end
#pragma unroll
            for (int j = 0; j < CH; ++j)
                *reinterpret_cast<v4u*>(base + loff0 + j * RP * kBK) = ok ? r[j] : v4u{0, 0, 0, 0};
        }
        if constexpr (V == VAR_FP8_BLOCK) {
            const float(&fxs)[TM] = decltype(set)::value ? fxy : fxx;
            const float(&fws)[TN] = decltype(set)::value ? fwy : fwx;
            float(&fxb)[TM] = decltype(buf)::value ? fx1 : fx0;
            float(&fwb)[TN] = decltype(buf)::value ? fw1 : fw0;
#pragma unroll
            for (int jj = 0; jj < TM; ++jj) fxb[jj] = fxs[jj];
#pragma unroll
            for (int ii = 0; ii < TN; ++ii) fwb[ii] = fws[ii];
        }
    };

    // Direct staging (DM): the stage goes from global memory straight into
    // LDS (buffer_load_dwordx4 ... lds).  One instruction of a wave fills 1 KB
    // of LDS in lane order, i.e. 8 rows of 128 bytes: lane l lands in row
    // (its carried row), slot l % 8, so it loads logical chunk
    // (l % 8) ^ swz(row) to keep the swizzled layout.  Chunks at or past K
    // (the ragged last stage, a K group's step past the end) take an offset
    // outside the descriptor and land as zeros.
    constexpr int kOOB = 0x40000000;
    const int cdma = cthr ^ swz(gtid >> 3);
    auto dma_one = [&](auto buf, int s, int j) {
        const int k = s * kBK + (cdma << 4);
        const bool in = k < K;
        uint8_t* dst = sbuf(buf) + j * RP * kBK + wave * 1024;
        if (SG && j >= JW / 2 && j < JW) dma16(du, dst, in ? roff[j - JW / 2] + k : kOOB);
        else if (j < JW) dma16(dw, dst, in ? roff[j] + k : kOOB);
        else dma16(dx, dst, in ? roff[j - JW] + k : kOOB);
    };
    // block FP8: the stage's factors load straight into the buffer's registers
    auto dma_fac = [&](auto buf, int s) {
        if constexpr (V == VAR_FP8_BLOCK) {
            float(&fx)[TM] = decltype(buf)::value ? fx1 : fx0;
            float(&fw)[TN] = decltype(buf)::value ? fw1 : fw0;
            const int kb = min(s, kbs - 1);
#pragma unroll
            for (int jj = 0; jj < TM; ++jj)
                fx[jj] = sx[(int64_t)min(m0 + wm * SM + jj * 32 + (lane & 31), M - 1) * kbs + kb];
#pragma unroll
            for (int ii = 0; ii < TN; ++ii) {
                const int rr = wn * SN + ii * 32;
                if (SG && rr >= PR) fw[ii] = bf16_lo(sw_u[(int64_t)(min(n0 + rr - PR, N - 1) >> 7) * kbs + kb]);
                else fw[ii] = bf16_lo(sw[(int64_t)(min(n0 + rr, N - 1) >> 7) * kbs + kb]);
            }
        }
    };
    // the next stage's loads go out in the first half of this stage's MFMAs,
    // so they have the second half to land before the closing barrier
    constexpr int DH = HOOKS / 2 > 0 ? HOOKS / 2 : 1;
    auto dma_hook = [&](auto buf, int s, int h) {
        if (h >= DH) return;
        __builtin_amdgcn_sched_barrier(0);
        if (h == 0) dma_fac(buf, s);
#pragma unroll
        for (int j = h * CH / DH; j < (h + 1) * CH / DH; ++j) dma_one(buf, s, j);
        __builtin_amdgcn_sched_barrier(0);
    };
    // every direct load of the stage has written LDS (vmcnt 0), before the barrier
    auto dma_wait = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };

    // With 512 threads a wave may hold 256 registers.  Unless AGPRs are known
    // to be in use, the compiler then takes all 256 as VGPRs, selects the
    // VGPR form of the MFMAs and spills; naming one AGPR keeps the
    // accumulators in AGPRs (128 + 128).
    if constexpr (GT * KG > 256) asm volatile("" ::: "a0");
    Acc acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = Acc{};

    const int arow0 = wn * SN + (lane & 31);
    const int brow0 = BN + wm * SM + (lane & 31);
    const int half = lane >> 5;

    // the epilogue's scales, staged once; their loads go out after the first
    // stage's, so that both wait for memory together
    auto stage_scales = [&]() {
        if constexpr (V != VAR_FP8_BLOCK) {
            for (int i = tid; i < BN; i += NTH)
                s_w_t[i] = (SG && i >= PR) ? bf16_lo(sw_u[min(n0 + i - PR, N - 1)]) : bf16_lo(sw[min(n0 + i, N - 1)]);
            for (int i = tid; i < BM; i += NTH) s_x_t[i] = sx[min(m0 + i, M - 1)];
        }
    };

    // prologue: stage 0 in LDS buffer 0 (register staging: stage 1 in flight)
    if constexpr (DM) {
#pragma unroll
        for (int j = 0; j < CH; ++j) dma_one(IC<0>{}, gs(0), j);
        dma_fac(IC<0>{}, gs(0));
        stage_scales();
        dma_wait();
    } else {
        issue_all(IC<0>{}, gs(0));
        stage_scales();
        write(IC<0>{}, IC<0>{}, gs(0));
        issue_all(IC<1>{}, gs(1));
    }
    __syncthreads();

    // A wave issues its stage's MFMAs at raised priority (back to normal for the
    // LDS writes and the barrier), so a SIMD shared by two workgroups keeps
    // feeding the matrix core while the other wave is in its write phase.
    auto compute = [&](auto buf, const float (&fx)[TM], const float (&fw)[TN], auto&& hk) {
        __builtin_amdgcn_s_setprio(1);
        const uint8_t* base = sbuf(buf);
        auto rdq = [&](int r, int c) { return *reinterpret_cast<const v4i*>(base + r * kBK + ((c ^ swz(r)) << 4)); };
        if constexpr (LOWREG && WN * WM == 4) {
            // 256 x 256 tiles with one wavefront per SIMD: the operands of K
            // sub-step s + 1 are read while the MFMAs of s run
            static_assert(V != VAR_FP8_BLOCK, "rowwise schemes only");
            constexpr int SUB = V == VAR_INT8 ? 4 : 2;
            typedef typename std::conditional<V == VAR_INT8, v4i, v8i>::type Op;
            Op aq[2][TN], bq[2][TM];
            auto rop = [&](int r, int sub) {
                if constexpr (V == VAR_INT8) {
                    return rdq(r, 2 * sub + half);
                } else {
                    const int c0 = 4 * sub + 2 * half;
                    const v4i lo = rdq(r, c0), hi = rdq(r, c0 + 1);
                    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                }
            };
            auto rd = [&](int p, int sub) {
#pragma unroll
                for (int j = 0; j < TM; ++j) bq[p][j] = rop(brow0 + j * 32, sub);
#pragma unroll
                for (int i = 0; i < TN; ++i) aq[p][i] = rop(arow0 + i * 32, sub);
            };
            // (FP8: a sub-step's 16 reads go out after the first MFMAs of the
            // previous one, so that at most 16 reads wait in the LDS queue)
            rd(0, 0);
#pragma unroll
            for (int sub = 0; sub < SUB; ++sub) {
                if (V == VAR_INT8 && sub + 1 < SUB) rd((sub + 1) & 1, sub + 1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < TN; ++i) {
#pragma unroll
                    for (int j = 0; j < TM; ++j) {
                        if constexpr (V == VAR_INT8)
                            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aq[sub & 1][i], bq[sub & 1][j], acc[i][j], 0, 0, 0);
                        else
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aq[sub & 1][i], bq[sub & 1][j], acc[i][j],
                                                                                       0, 0, 0, 0, 0, 0);
                    }
                    if (V != VAR_INT8 && i == 0 && sub + 1 < SUB) {
                        __builtin_amdgcn_sched_barrier(0);
                        rd((sub + 1) & 1, sub + 1);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    hk(sub * TN + i);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else if constexpr (LOWREG) {
            // 256 x 256 tiles: 128 accumulators and two staging sets leave no
            // room for a read-ahead, so per K sub-step the token tiles are
            // read once and each weight tile right before its MFMAs (the
            // other wavefront on the SIMD covers the LDS latency)
            static_assert(V != VAR_FP8_BLOCK, "rowwise schemes only");
            constexpr int SUB = V == VAR_INT8 ? 4 : 2;      // 32- or 64-byte sub-steps
#pragma unroll
            for (int sub = 0; sub < SUB; ++sub) {
                if constexpr (V == VAR_INT8) {
                    const int c = 2 * sub + half;
                    v4i bq[TM];
#pragma unroll
                    for (int j = 0; j < TM; ++j) bq[j] = rdq(brow0 + j * 32, c);
#pragma unroll
                    for (int i = 0; i < TN; ++i) {
                        const v4i aq = rdq(arow0 + i * 32, c);
#pragma unroll
                        for (int j = 0; j < TM; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aq, bq[j], acc[i][j], 0, 0, 0);
                        hk(sub * TN + i);
                    }
                } else {
                    const int c0 = 4 * sub + 2 * half;
                    v8i bq[TM];
#pragma unroll
                    for (int j = 0; j < TM; ++j) {
                        const v4i lo = rdq(brow0 + j * 32, c0), hi = rdq(brow0 + j * 32, c0 + 1);
                        bq[j] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                    }
#pragma unroll
                    for (int i = 0; i < TN; ++i) {
                        const v4i lo = rdq(arow0 + i * 32, c0), hi = rdq(arow0 + i * 32, c0 + 1);
                        const v8i aq = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
                        for (int j = 0; j < TM; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aq, bq[j], acc[i][j], 0, 0, 0, 0, 0, 0);
                        hk(sub * TN + i);
                    }
                }
            }
        } else if constexpr (V == VAR_INT8) {
            constexpr int SUB = 4;                    // 32-byte K sub-steps per stage
            v4i a[SUB][TN], bb[SUB][TM];
            auto rd = [&](int sub) {
                const int c = 2 * sub + half;
#pragma unroll
                for (int i = 0; i < TN; ++i) {
                    const int r = arow0 + i * 32;
                    a[sub][i] = *reinterpret_cast<const v4i*>(base + r * kBK + ((c ^ swz(r)) << 4));
                }
#pragma unroll
                for (int j = 0; j < TM; ++j) {
                    const int r = brow0 + j * 32;
                    bb[sub][j] = *reinterpret_cast<const v4i*>(base + r * kBK + ((c ^ swz(r)) << 4));
                }
            };
            auto mm = [&](int sub) {
#pragma unroll
                for (int i = 0; i < TN; ++i) {
#pragma unroll
                    for (int j = 0; j < TM; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[sub][i], bb[sub][j], acc[i][j], 0, 0, 0);
                    hk(sub * TN + i);
                }
            };
            // the reads of sub-step s + 1 are in flight while the MFMAs of s run
            rd(0);
            rd(1);
            __builtin_amdgcn_sched_barrier(0);
            mm(0);
            __builtin_amdgcn_sched_barrier(0);
            rd(2);
            __builtin_amdgcn_sched_barrier(0);
            mm(1);
            __builtin_amdgcn_sched_barrier(0);
            rd(3);
            __builtin_amdgcn_sched_barrier(0);
            mm(2);
            __builtin_amdgcn_sched_barrier(0);
            mm(3);
        } else {
            v8i a[2][TN], bb[2][TM];
            auto rd = [&](int sub) {
                const int c0 = 4 * sub + 2 * half;
#pragma unroll
                for (int i = 0; i < TN; ++i) {
                    const int r = arow0 + i * 32;
                    const v4i lo = *reinterpret_cast<const v4i*>(base + r * kBK + ((c0 ^ swz(r)) << 4));
                    const v4i hi = *reinterpret_cast<const v4i*>(base + r * kBK + (((c0 + 1) ^ swz(r)) << 4));
                    a[sub][i] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                }
#pragma unroll
                for (int j = 0; j < TM; ++j) {
                    const int r = brow0 + j * 32;
                    const v4i lo = *reinterpret_cast<const v4i*>(base + r * kBK + ((c0 ^ swz(r)) << 4));
                    const v4i hi = *reinterpret_cast<const v4i*>(base + r * kBK + (((c0 + 1) ^ swz(r)) << 4));
                    bb[sub][j] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                }
            };
            rd(0);
            __builtin_amdgcn_sched_barrier(0);
            rd(1);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (V == VAR_FP8_ROW) {
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                    for (int i = 0; i < TN; ++i) {
#pragma unroll
                        for (int j = 0; j < TM; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[sub][i], bb[sub][j], acc[i][j], 0, 0, 0, 0, 0, 0);
                        hk(sub * TN + i);
                    }
            } else {
                // one MFMA tile at a time: the block's partial product of tile t is
                // scaled into the accumulator while the MFMAs of tile t + 1 run,
                // so only two partial tiles are live
                constexpr int NT = TN * TM;
                v16f part[2];
#pragma unroll
                for (int t = 0; t <= NT; ++t) {
                    if (t < NT) {
                        const int i = t / TM, j = t % TM;
                        part[t & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[0][i], bb[0][j], v16f{}, 0, 0, 0, 0, 0, 0);
                        part[t & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[1][i], bb[1][j], part[t & 1], 0, 0, 0, 0, 0, 0);
                    }
                    if (t > 0) {
                        const int i = (t - 1) / TM, j = (t - 1) % TM;
                        const float f = fx[j] * fw[i];
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            acc[i][j][e] = __builtin_fmaf(part[(t - 1) & 1][e], f, acc[i][j][e]);
                    }
                    if (t < NT) hk(t);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };

    // Step kt multiplies LDS buffer kt % 2 while the loads of a later stage
    // run between its MFMAs, writes the next stage into the other buffer and
    // meets the barrier.  Unrolled by two so that buffers and register sets
    // are compile-time choices; a single loop exit keeps the accumulators in
    // place (an odd last stage runs after the loop).  Loads and writes run
    // unconditionally: a stage past the end re-reads in-range bytes and
    // writes zeros to a buffer that is not multiplied again (a conditional
    // load makes the compiler assume the shallower pipeline everywhere).
    //
    // Direct staging: step kt multiplies buffer kt % 2 while the next stage
    // loads into the other buffer (free since the previous barrier); the
    // step ends by waiting for those loads and meeting the barrier.
    int kt = 0;
    if constexpr (DM) {
        for (; kt + 1 < nko; kt += 2) {
            compute(IC<0>{}, fx0, fw0, [&](int h) { dma_hook(IC<1>{}, gs(kt + 1), h); });
            __builtin_amdgcn_s_setprio(0);
            dma_wait();
            __syncthreads();
            compute(IC<1>{}, fx1, fw1, [&](int h) { dma_hook(IC<0>{}, gs(kt + 2), h); });
            __builtin_amdgcn_s_setprio(0);
            dma_wait();
            __syncthreads();
        }
    } else {
        for (; kt + 1 < nko; kt += 2) {
            compute(IC<0>{}, fx0, fw0, [&](int h) { hook(IC<0>{}, gs(kt + 2), h); });
            __builtin_amdgcn_s_setprio(0);
            write(IC<1>{}, IC<1>{}, gs(kt + 1));
            __syncthreads();
            compute(IC<1>{}, fx1, fw1, [&](int h) { hook(IC<1>{}, gs(kt + 3), h); });
            __builtin_amdgcn_s_setprio(0);
            write(IC<0>{}, IC<0>{}, gs(kt + 2));
            __syncthreads();
        }
    }
    // The K-group hand-off and the epilogue read the accumulators next.  The
    // padding sits inside each exit path: the compiler places its accumulator
    // copies where the two paths join.
    mfma_drain();
    if (kt < nko) {
        compute(IC<0>{}, fx0, fw0, [&](int) {});
        mfma_drain();
    }
    __builtin_amdgcn_s_setprio(0);

    if constexpr (KG == 2) {
        // group 1 hands its partial sums to group 0 through LDS (one dword per
        // lane and accumulator element, lane-contiguous), group 0 adds them
        constexpr int NACC = TN * TM * 16;
        static_assert(WN * WM * NACC * 64 * 4 <= (int)sizeof(ldsA), "partials fit the stage buffers");
        uint32_t* part = reinterpret_cast<uint32_t*>(ldsA) + wave * NACC * 64 + lane;
        __syncthreads();                                   // both groups are done with their stages
        if (grp == 1) {
#pragma unroll
            for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int j = 0; j < TM; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        // (a bit cast of the vector element itself reads element 0)
                        if constexpr (V == VAR_INT8) part[((i * TM + j) * 16 + e) * 64] = (uint32_t)acc[i][j][e];
                        else part[((i * TM + j) * 16 + e) * 64] = __float_as_uint(acc[i][j][e]);
                    }
        }
        __syncthreads();
        if (grp == 0) {
#pragma unroll
            for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int j = 0; j < TM; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const uint32_t v = part[((i * TM + j) * 16 + e) * 64];
                        if constexpr (V == VAR_INT8) acc[i][j][e] += (int)v;
                        else acc[i][j][e] += __uint_as_float(v);
                    }
        }
    }

    // Epilogue.  Lane l, accumulator element e of MFMA tile (i, j):
    //   n = n0 + wn*SN + i*32 + 8*(e/4) + 4*(l/32) + e%4,   m = m0 + wm*SM + j*32 + l%32,
    // so elements 4g .. 4g+3 are four consecutive outputs of one row.
    //
    // bf16 output with 16-byte aligned rows goes through LDS: the waves write
    // their converted sub-tiles into a row-major [BM][BN] tile (row pitch
    // padded by 16 bytes so the 32 rows of one column group fall on distinct
    // banks), then every thread streams whole 16-byte pieces of output rows,
    // a wave covering 1 KB of contiguous rows per store instead of 32 rows x
    // 16 bytes.
    if (SG || (mode == OUT_BF16 && (N & 7) == 0)) {
        static_assert((BM / 2) * PITCH <= (int)sizeof(ldsA), "bf16 staging tile fits the stage buffers");
        __syncthreads();                                   // every wave is done with the last stage
        if (grp == 0) {
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int ml = wm * SM + j * 32 + (lane & 31);
            const float sxm = (V == VAR_FP8_BLOCK) ? 0.0f : s_x_t[ml];
#pragma unroll
            for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int nl = wn * SN + i * 32 + 8 * g + 4 * half;
                    float v[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        if constexpr (V == VAR_INT8) v[k] = (float)acc[i][j][4 * g + k] * (sxm * s_w_t[nl + k]);
                        else if constexpr (V == VAR_FP8_ROW) v[k] = acc[i][j][4 * g + k] * (sxm * s_w_t[nl + k]);
                        else v[k] = acc[i][j][4 * g + k];
                    }
                    const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
                    const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
                    *reinterpret_cast<v2u*>(erow(ml) + nl * 2) = v2u{lo, hi};
                }
        }
        }
        __syncthreads();
        if constexpr (SG) {
            // gate of (row, j) at column j - n0, up at column PR + j - n0
            constexpr int CPH = PR * 2 / 16;               // 16-byte pieces per h row
            for (int id = tid; id < BM * CPH; id += NTH) {
                const int row = id / CPH, c = id % CPH;
                const int m = m0 + row, j = n0 + 8 * c;
                if (m >= M || j >= N) continue;
                const v4u g = *reinterpret_cast<const v4u*>(erow(row) + 16 * c);
                const v4u u = *reinterpret_cast<const v4u*>(erow(row) + PR * 2 + 16 * c);
                const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, uw[4] = {u.x, u.y, u.z, u.w};
                uint32_t hw[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    hw[q] = (uint32_t)swiglu_bf16(bf16_lo(gw[q]), bf16_lo(uw[q])) |
                            ((uint32_t)swiglu_bf16(bf16_hi(gw[q]), bf16_hi(uw[q])) << 16);
                uint16_t* hp = static_cast<uint16_t*>(y) + (int64_t)m * N + j;
                if ((N & 7) == 0) {
                    *reinterpret_cast<v4u*>(hp) = v4u{hw[0], hw[1], hw[2], hw[3]};
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (j + e < N) hp[e] = (uint16_t)(hw[e >> 1] >> (16 * (e & 1)));
                }
            }
            return;
        }
        constexpr int CPR = BN * 2 / 16;                   // 16-byte pieces per tile row
#pragma unroll 4
        for (int id = tid; id < BM * CPR; id += NTH) {
            const int row = id / CPR, c = id % CPR;
            const int m = m0 + row, n = n0 + 8 * c;
            if (m < M && n < N)
                *reinterpret_cast<v4u*>(static_cast<uint16_t*>(y) + (int64_t)m * N + n) =
                    *reinterpret_cast<const v4u*>(erow(row) + 16 * c);
        }
        return;
    }
    // Other outputs: straight from the accumulators, one 8-byte (bf16) or
    // 16-byte (f32 / i32) store per four outputs when the row length allows it.
    if (grp != 0) return;
    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        const int ml = wm * SM + j * 32 + (lane & 31);
        const int m = m0 + ml;
        if (m >= M) continue;
        const float sxm = (V == VAR_FP8_BLOCK) ? 0.0f : s_x_t[ml];
#pragma unroll
        for (int i = 0; i < TN; ++i) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int nl = wn * SN + i * 32 + 8 * g + 4 * half;
                const int n = n0 + nl;
                const int64_t idx = (int64_t)m * N + n;
                if (vec && n + 3 < N) {
                    if constexpr (V == VAR_INT8) {
                        const int a[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                        const float w4[4] = {s_w_t[nl], s_w_t[nl + 1], s_w_t[nl + 2], s_w_t[nl + 3]};
                        store4_rowwise_i32acc(y, idx, a, sxm, w4, mode);
                    } else if constexpr (V == VAR_FP8_ROW) {
                        const float v4[4] = {acc[i][j][4 * g] * (sxm * s_w_t[nl]), acc[i][j][4 * g + 1] * (sxm * s_w_t[nl + 1]),
                                             acc[i][j][4 * g + 2] * (sxm * s_w_t[nl + 2]), acc[i][j][4 * g + 3] * (sxm * s_w_t[nl + 3])};
                        store4_f32(y, idx, v4, mode);
                    } else {
                        const float v4[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                        store4_f32(y, idx, v4, mode);
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        if (n + k >= N) break;
                        const int e = 4 * g + k;
                        if constexpr (V == VAR_INT8) store_rowwise_i32acc(y, idx + k, acc[i][j][e], sxm, sw[n + k], mode);
                        else if constexpr (V == VAR_FP8_ROW) store_f32(y, idx + k, acc[i][j][e] * (sxm * s_w_t[nl + k]), mode);
                        else store_f32(y, idx + k, acc[i][j][e], mode);
                    }
                }
            }
        }
    }
}

template <int V, int BN, int BM, int WN, int WM, int KG = 1, bool DM = false>
hipError_t launch_tile(const uint8_t* qx, const float* sx, const SegmentArgs& sa, int64_t M, int64_t K, int mode,
                       hipStream_t st) {
    const int tm = (int)((M + BM - 1) / BM);
    dim3 block(64 * WN * WM * KG);
    if (mode == OUT_SWIGLU) {
        const int tn = (sa.start[1] + BN / 2 - 1) / (BN / 2);
        hipLaunchKernelGGL((gemm_large_kernel<V, BN, BM, WN, WM, true, KG, DM>), dim3((unsigned)(tm * tn)),
                           block, 0, st, qx, sx, sa, (int)M, (int)K, mode, tm, tn);
        return hipGetLastError();
    }
    int tn = 0;
    for (int i = 0; i < sa.nseg; ++i) tn += (sa.start[i + 1] - sa.start[i] + BN - 1) / BN;
    hipLaunchKernelGGL((gemm_large_kernel<V, BN, BM, WN, WM, false, KG, DM>), dim3((unsigned)(tm * tn)), block,
                       0, st, qx, sx, sa, (int)M, (int)K, mode, tm, tn);
    return hipGetLastError();
}

template <int V>
hipError_t launch_variant(int cfg, const uint8_t* qx, const float* sx, const SegmentArgs& sa, int64_t M, int64_t K,
                          int mode, hipStream_t st) {
    constexpr bool BD = V == VAR_FP8_BLOCK;
    switch (cfg) {
        // block FP8 stages straight into LDS on the one-group tiles: its
        // per-stage rescale needs the registers that register staging would
        // take (the two-group tiles keep register staging: direct staging made
        // Qwen3 o and down at 512 tokens slower, 22.7 -> 27.7 and 63.3 -> 77.6 us)
        case kTile256x128: return launch_tile<V, 256, 128, 2, 2, 1, BD>(qx, sx, sa, M, K, mode, st);
        case kTile128x128: return launch_tile<V, 128, 128, 2, 2, 1, BD>(qx, sx, sa, M, K, mode, st);
        case kTile128x64: return launch_tile<V, 128, 64, 2, 2, 1, BD>(qx, sx, sa, M, K, mode, st);
        case kTile128x256: return launch_tile<V, 128, 256, 2, 2, 1, BD>(qx, sx, sa, M, K, mode, st);
        case kTile128x128K2: return launch_tile<V, 128, 128, 2, 2, 2>(qx, sx, sa, M, K, mode, st);
        case kTile128x64K2: return launch_tile<V, 128, 64, 2, 2, 2>(qx, sx, sa, M, K, mode, st);
        case kTile256x256W8:
            // block FP8 rescales partial products per stage: no registers left at this tile.
            // Two wavefronts per SIMD leave no room for a whole stage of operands, which
            // direct staging needs: register staging.
            if constexpr (V == VAR_FP8_BLOCK) return hipErrorInvalidValue;
            else return launch_tile<V, 256, 256, 2, 4>(qx, sx, sa, M, K, mode, st);
        case kTile256x256:
            if constexpr (V == VAR_FP8_BLOCK) return hipErrorInvalidValue;
            else return launch_tile<V, 256, 256, 2, 2, 1, true>(qx, sx, sa, M, K, mode, st);

        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Tile choice, from timings of every tile on the Llama-8B projections at 256,
// 512, 1024 and 2048 tokens (t = number of 128 x 128 tiles, t256 = number of
// 256 x 256 tiles, 256 CUs):
//   int8 with t256 >= 224 (7 of 8 CUs busy): 256 x 256 with 4 wavefronts and
//     direct staging (gate/up at 512 tokens: 80.5 -> 77.1 us, at 1024:
//     147.9 -> 134.5 us against the 8-wavefront tile);
//   FP8 rowwise with t256 >= 512: the same tile (8192^2 x 8192: 476 -> 462 us);
//   FP8 rowwise with 224 <= t256 < 512: 256 x 256 with 8 wavefronts (gate/up
//     at 512 tokens: 67.8 us against 72.3 for the 4-wavefront tile);
//   t >= 384: 128 x 128, two workgroups share a CU;
//   192 <= t < 384: 128 x 128 with two K groups (8 wavefronts, one tile per
//     CU, two wavefronts per SIMD);
//   t < 192: 128 x 64 with two K groups.
// Direct staging lost on every 128-row tile of the rowwise schemes (e.g. int8
// down at 512 tokens, 128 x 64 with two K groups: 46 -> 53 us), so those stage
// through registers.  Block FP8 scales every stage's partial products on the
// vector ALUs: with register staging its 128 x 128 tiles spill; with direct
// staging it runs 128 x 128 for t >= 1024 (Qwen3 gate/up at 1024 tokens:
// 196.8 us for 128 x 64 with register staging -> 158.7 us), else 128 x 64
// (direct staging took Qwen3 q/k/v at 1024 tokens from 51.5 to 43.9 us), with
// two K groups and register staging below 192 tiles.
// The 256 x 128 tiles (4 or 8 wavefronts) lost on the Llama shapes at 512 and
// 1024 tokens.
int large_tile_config(int variant, int64_t M, const SegmentArgs& sa) {
    int64_t panels = 0, panels256 = 0;
    for (int i = 0; i < sa.nseg; ++i) {
        panels += (sa.start[i + 1] - sa.start[i] + 127) / 128;
        panels256 += (sa.start[i + 1] - sa.start[i] + 255) / 256;
    }
    const int64_t t = ((M + 127) / 128) * panels;
    if (variant == VAR_FP8_BLOCK) return t >= 1024 ? kTile128x128 : (t < 192 ? kTile128x64K2 : kTile128x64);
    const int64_t t256 = ((M + 255) / 256) * panels256;
    if (variant == VAR_INT8 && t256 >= 224) return kTile256x256;
    if (variant == VAR_FP8_ROW && t256 >= 512) return kTile256x256;
    if (variant == VAR_FP8_ROW && t256 >= 224) return kTile256x256W8;
    if (t >= 384) return kTile128x128;
    return t >= 192 ? kTile128x128K2 : kTile128x64K2;
}

hipError_t launch_gemm_large_cfg(int cfg, int variant, const uint8_t* qx, const float* sx, const SegmentArgs& sa,
                                 int64_t M, int64_t K, int mode, hipStream_t st) {
    if (variant == VAR_INT8) return launch_variant<VAR_INT8>(cfg, qx, sx, sa, M, K, mode, st);
    if (variant == VAR_FP8_ROW) return launch_variant<VAR_FP8_ROW>(cfg, qx, sx, sa, M, K, mode, st);
    return launch_variant<VAR_FP8_BLOCK>(cfg, qx, sx, sa, M, K, mode, st);
}

hipError_t launch_gemm_large(int variant, const uint8_t* qx, const float* sx, const SegmentArgs& sa, int64_t M,
                             int64_t K, int mode, hipStream_t st) {
    return launch_gemm_large_cfg(large_tile_config(variant, M, sa), variant, qx, sx, sa, M, K, mode, st);
}

}  // namespace qlin
