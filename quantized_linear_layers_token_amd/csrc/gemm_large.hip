// Long-input products on the matrix cores (W8A8 model card, "Loading": longer
// inputs rounded a row at a time and multiplied in int8, summing in int32;
// Qwen3 8B FP8 card, "Loading": block-scaled FP8 product).
//
// Tiled GEMM, both operands K-contiguous ("NT"): the output tile is BN
// weight rows x BM tokens; 256 threads = 4 wavefronts in a 2 x 2 grid, each
// owning a (BN/2) x (BM/2) sub-tile made of 32 x 32 MFMA tiles:
//   int8: v_mfma_i32_32x32x32_i8  (4 per 128-byte K stage)
//   E4M3: v_mfma_f32_32x32x64_f8f6f4 (2 per 128-byte K stage)
// K advances in stages of 128 bytes through a double-buffered LDS tile: the
// next stage's global loads are in flight while the current stage is
// multiplied, then land in the other buffer; one barrier per stage.  LDS rows
// are 128 bytes with the 16-byte chunk index XOR-swizzled by (row & 7) so that
// the MFMA operand reads (eight rows, same chunk) hit distinct banks.
//
// A operand = weight rows (n), B operand = tokens (m): a lane's 16 accumulator
// values are 16 rows n of one token column m, all inside one 32-row slab.  For
// block FP8 each stage is exactly one 128-wide K block, so one factor
// s_x[m, kb] * s_w[n/128, kb] per lane and MFMA tile scales the stage's partial
// product before it is added to the f32 accumulator.
//
// Tile order is XCD-aware: workgroup b runs on XCD b % 8; tile ids are
// assigned so that the tiles sharing one weight panel (same n tile) are
// consecutive on one XCD and share its L2.
#include "qlin_device.h"
#include "qlin_internal.h"

namespace qlin {

namespace {

constexpr int kLargeThreads = 256;
constexpr int kBK = 128;

template <int V> struct LargeAcc { typedef v16i T; };
template <> struct LargeAcc<VAR_FP8_ROW> { typedef v16f T; };
template <> struct LargeAcc<VAR_FP8_BLOCK> { typedef v16f T; };

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 4); }

template <int V, int BN, int BM>
__global__ __launch_bounds__(kLargeThreads) void gemm_large_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint8_t* __restrict__ qw, const uint16_t* __restrict__ sw,
    void* __restrict__ y, int M, int N, int K, int mode, int tiles_m, int tiles_n) {
    typedef typename LargeAcc<V>::T Acc;
    constexpr int WN = BN / 2, WM = BM / 2;
    constexpr int TN = WN / 32, TM = WM / 32;
    constexpr int CA = BN * 8 / kLargeThreads;   // 16-byte chunks per thread per stage (weights)
    constexpr int CB = BM * 8 / kLargeThreads;   // (tokens)
    static_assert(CA >= 1 && CB >= 1, "tile too small for 256 threads");
    constexpr int TILE_BYTES = (BN + BM) * kBK;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * TILE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave >> 1, wm = wave & 1;

    // XCD-aware tile order (identity when the tile count is not a multiple of 8).
    const int ntiles = tiles_m * tiles_n;
    const int b = blockIdx.x;
    const int t = (ntiles & 7) ? b : ((b & 7) * (ntiles >> 3) + (b >> 3));
    const int n0 = (t / tiles_m) * BN;
    const int m0 = (t % tiles_m) * BM;

    // Global -> register staging assignment: chunk i = tid + 256 j -> (row i/8, chunk i%8).
    const uint8_t* ga[CA];
    const uint8_t* gb[CB];
    int la[CA], lb[CB];
#pragma unroll
    for (int j = 0; j < CA; ++j) {
        const int i = tid + j * kLargeThreads, row = i >> 3, c = i & 7;
        ga[j] = qw + (int64_t)min(n0 + row, N - 1) * K + c * 16;
        la[j] = swz(row, c);
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
        const int i = tid + j * kLargeThreads, row = i >> 3, c = i & 7;
        gb[j] = qx + (int64_t)min(m0 + row, M - 1) * K + c * 16;
        lb[j] = BN * kBK + swz(row, c);
    }
    const int cthr = (tid & 7) * 16;   // this thread's chunk offset inside a stage (same for all j)

    v4u ra[CA], rb[CB];
    auto load_stage = [&](int kt) {
        const int k = kt * kBK + cthr;
        const bool ok = k < K;
#pragma unroll
        for (int j = 0; j < CA; ++j)
            ra[j] = ok ? *reinterpret_cast<const v4u*>(ga[j] + (int64_t)kt * kBK) : v4u{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < CB; ++j)
            rb[j] = ok ? *reinterpret_cast<const v4u*>(gb[j] + (int64_t)kt * kBK) : v4u{0, 0, 0, 0};
    };
    auto store_stage = [&](int buf) {
        uint8_t* base = lds + buf * TILE_BYTES;
#pragma unroll
        for (int j = 0; j < CA; ++j) *reinterpret_cast<v4u*>(base + la[j]) = ra[j];
#pragma unroll
        for (int j = 0; j < CB; ++j) *reinterpret_cast<v4u*>(base + lb[j]) = rb[j];
    };

    Acc acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = Acc{};

    // Operand rows inside the LDS tile for this lane.
    const int arow0 = wn * WN + (lane & 31);
    const int brow0 = BN + wm * WM + (lane & 31);   // B rows follow the BN weight rows
    const int half = lane >> 5;

    const int nk = (K + kBK - 1) / kBK;
    const int kbs = K >> 7;

    load_stage(0);
    store_stage(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_stage(kt + 1);
        const uint8_t* base = lds + buf * TILE_BYTES;

        float fx[TM], fw[TN];
        if constexpr (V == VAR_FP8_BLOCK) {
#pragma unroll
            for (int j = 0; j < TM; ++j)
                fx[j] = sx[(int64_t)min(m0 + wm * WM + j * 32 + (lane & 31), M - 1) * kbs + kt];
#pragma unroll
            for (int i = 0; i < TN; ++i)
                fw[i] = bf16_lo(sw[(int64_t)(min(n0 + wn * WN + i * 32, N - 1) >> 7) * kbs + kt]);
        }

        if constexpr (V == VAR_INT8) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int c = 2 * s + half;
                v4i a[TN], bb[TM];
#pragma unroll
                for (int i = 0; i < TN; ++i)
                    a[i] = *reinterpret_cast<const v4i*>(base + ((arow0 + i * 32) * kBK + ((c ^ ((arow0 + i * 32) & 7)) << 4)));
#pragma unroll
                for (int j = 0; j < TM; ++j)
                    bb[j] = *reinterpret_cast<const v4i*>(base + ((brow0 + j * 32) * kBK + ((c ^ ((brow0 + j * 32) & 7)) << 4)));
#pragma unroll
                for (int i = 0; i < TN; ++i)
#pragma unroll
                    for (int j = 0; j < TM; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], bb[j], acc[i][j], 0, 0, 0);
            }
        } else {
            v16f part[TN][TM];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int c0 = 4 * s + 2 * half;
                v8i a[TN], bb[TM];
#pragma unroll
                for (int i = 0; i < TN; ++i) {
                    const int r = arow0 + i * 32;
                    const v4i lo = *reinterpret_cast<const v4i*>(base + r * kBK + ((c0 ^ (r & 7)) << 4));
                    const v4i hi = *reinterpret_cast<const v4i*>(base + r * kBK + (((c0 + 1) ^ (r & 7)) << 4));
                    a[i] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                }
#pragma unroll
                for (int j = 0; j < TM; ++j) {
                    const int r = brow0 + j * 32;
                    const v4i lo = *reinterpret_cast<const v4i*>(base + r * kBK + ((c0 ^ (r & 7)) << 4));
                    const v4i hi = *reinterpret_cast<const v4i*>(base + r * kBK + (((c0 + 1) ^ (r & 7)) << 4));
                    bb[j] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                }
#pragma unroll
                for (int i = 0; i < TN; ++i)
#pragma unroll
                    for (int j = 0; j < TM; ++j) {
                        if constexpr (V == VAR_FP8_ROW) {
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], bb[j], acc[i][j], 0, 0, 0, 0, 0, 0);
                        } else {
                            part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                a[i], bb[j], s == 0 ? v16f{} : part[i][j], 0, 0, 0, 0, 0, 0);
                        }
                    }
            }
            if constexpr (V == VAR_FP8_BLOCK) {
#pragma unroll
                for (int i = 0; i < TN; ++i)
#pragma unroll
                    for (int j = 0; j < TM; ++j) {
                        const float f = fx[j] * fw[i];
#pragma unroll
                        for (int e = 0; e < 16; ++e) acc[i][j][e] = __builtin_fmaf(part[i][j][e], f, acc[i][j][e]);
                    }
            }
        }

        if (kt + 1 < nk) store_stage(buf ^ 1);
        __syncthreads();
    }

    // Epilogue.  Lane l, accumulator element e of MFMA tile (i, j):
    //   n = n0 + wn*WN + i*32 + 8*(e/4) + 4*(l/32) + e%4,   m = m0 + wm*WM + j*32 + l%32.
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        const int m = m0 + wm * WM + j * 32 + (lane & 31);
        if (m >= M) continue;
        const float sxm = (V == VAR_FP8_BLOCK) ? 0.0f : sx[m];
#pragma unroll
        for (int i = 0; i < TN; ++i) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int n = n0 + wn * WN + i * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
                if (n >= N) continue;
                const int64_t idx = (int64_t)m * N + n;
                if constexpr (V == VAR_INT8) store_rowwise_i32acc(y, idx, acc[i][j][e], sxm, sw[n], mode);
                else if constexpr (V == VAR_FP8_ROW) store_f32(y, idx, acc[i][j][e] * (sxm * bf16_lo(sw[n])), mode);
                else store_f32(y, idx, acc[i][j][e], mode);
            }
        }
    }
}

template <int V, int BN, int BM>
hipError_t launch_tile(const uint8_t* qx, const float* sx, const uint8_t* qw, const uint16_t* sw, void* y,
                       int64_t M, int64_t N, int64_t K, int mode, hipStream_t st) {
    const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
    dim3 grid((unsigned)(tm * tn)), block(kLargeThreads);
    hipLaunchKernelGGL((gemm_large_kernel<V, BN, BM>), grid, block, 0, st, qx, sx, qw, sw, y, (int)M, (int)N,
                       (int)K, mode, tm, tn);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_large(int variant, const uint8_t* qx, const float* sx, const uint8_t* qw,
                             const uint16_t* sw, void* y, int64_t M, int64_t N, int64_t K, int mode,
                             hipStream_t st) {
    if (variant == VAR_INT8) return launch_tile<VAR_INT8, 128, 128>(qx, sx, qw, sw, y, M, N, K, mode, st);
    if (variant == VAR_FP8_ROW) return launch_tile<VAR_FP8_ROW, 128, 128>(qx, sx, qw, sw, y, M, N, K, mode, st);
    return launch_tile<VAR_FP8_BLOCK, 128, 128>(qx, sx, qw, sw, y, M, N, K, mode, st);
}

}  // namespace qlin
