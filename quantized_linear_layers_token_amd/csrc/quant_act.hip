// Dynamic activation quantizers (bf16 -> int8 or OCP E4M3) for gfx950.
//
// Per token (W8A8 model card, intro and "Loading"; FP8-dynamic README,
// "Creation" recipe): one workgroup per row; each thread holds its 16-byte
// chunks of the row in registers, so the row is read from HBM once.  The
// absmax is an integer max over the bf16 bit patterns with the sign bit
// cleared (for non-negative finite floats the bit order is the value order),
// reduced across the wavefront with DPP and across the four waves via LDS.
//
// Per 128-input group (Qwen3 8B FP8 model card, "Loading"): a group is 16
// lanes x 8 values, i.e. exactly one 16-lane DPP row, so the group absmax is a
// DPP row reduction with no LDS at all.
#include "qlin_internal.h"
#include "qlin_round.h"

namespace qlin {

namespace {

constexpr int kQuantThreads = 256;
constexpr int kQuantWaves = kQuantThreads / kWave;

// One workgroup per token row.  CPT = 16-byte chunks held per thread; the
// row has K/8 chunks, chunk c is handled by thread c % 256.
template <int CPT, bool FP8>
__global__ __launch_bounds__(kQuantThreads) void quant_token_kernel(
    const uint16_t* __restrict__ x, int64_t K, uint8_t* __restrict__ q, float* __restrict__ s) {
    __shared__ uint32_t red[kQuantWaves];
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    const int nchunks = (int)(K >> 3);
    const v4u* xr = reinterpret_cast<const v4u*>(x + m * K);

    v4u v[CPT];
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + j * kQuantThreads;
        v[j] = (c < nchunks) ? __builtin_nontemporal_load(xr + c) : v4u{0, 0, 0, 0};
        amax = max(amax, chunk_absmax(v[j]));
    }
    amax = wave_max_u32(amax);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = amax;
    __syncthreads();
    amax = max(max(red[0], red[1]), max(red[2], red[3]));

    float sc;
    RoundFactor rf;
    scales_from_absmax<FP8>(amax, sc, rf);
    if (tid == 0) s[m] = sc;

    v2u* qr = reinterpret_cast<v2u*>(q + m * K);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + j * kQuantThreads;
        if (c < nchunks) qr[c] = quant8<FP8>(v[j], rf);
    }
}

// Rows longer than 256 * 8 * 16 values: two passes over the row (the second
// pass re-reads x, normally from L2).
template <bool FP8>
__global__ __launch_bounds__(kQuantThreads) void quant_token_loop_kernel(
    const uint16_t* __restrict__ x, int64_t K, uint8_t* __restrict__ q, float* __restrict__ s) {
    __shared__ uint32_t red[kQuantWaves];
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t nchunks = K >> 3;
    const v4u* xr = reinterpret_cast<const v4u*>(x + m * K);
    uint32_t amax = 0;
    for (int64_t c = tid; c < nchunks; c += kQuantThreads) amax = max(amax, chunk_absmax(xr[c]));
    amax = wave_max_u32(amax);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = amax;
    __syncthreads();
    amax = max(max(red[0], red[1]), max(red[2], red[3]));
    float sc;
    RoundFactor rf;
    scales_from_absmax<FP8>(amax, sc, rf);
    if (tid == 0) s[m] = sc;
    v2u* qr = reinterpret_cast<v2u*>(q + m * K);
    for (int64_t c = tid; c < nchunks; c += kQuantThreads) qr[c] = quant8<FP8>(xr[c], rf);
}

// 128-input groups: group g of the flattened [M*K] array is x[128 g, 128 g + 128)
// (K % 128 == 0 keeps groups inside rows, and s[M][K/128] flattened is s[g]).
// Each 16-lane DPP row handles one group; 16 groups per workgroup.
__global__ __launch_bounds__(kQuantThreads) void quant_group128_fp8_kernel(
    const uint16_t* __restrict__ x, int64_t ngroups, uint8_t* __restrict__ q, float* __restrict__ s) {
    const int tid = threadIdx.x;
    const int64_t g = (int64_t)blockIdx.x * (kQuantThreads / 16) + (tid >> 4);
    if (g >= ngroups) return;                 // whole 16-lane rows leave together
    const int64_t c = g * 16 + (tid & 15);    // chunk index in the flattened array
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(x) + c);
    const uint32_t amax = row_max_u32(chunk_absmax(v));
    float sc;
    RoundFactor rf;
    scales_from_absmax<true>(amax, sc, rf);
    if ((tid & 15) == 0) s[g] = sc;
    reinterpret_cast<v2u*>(q)[c] = quant8<true>(v, rf);
}

template <bool FP8>
hipError_t launch_token(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s, hipStream_t st) {
    const int64_t chunks = K / 8;
    const int64_t cpt = (chunks + kQuantThreads - 1) / kQuantThreads;
    dim3 grid((unsigned)M), block(kQuantThreads);
    if (cpt <= 1) hipLaunchKernelGGL((quant_token_kernel<1, FP8>), grid, block, 0, st, x, K, q, s);
    else if (cpt <= 2) hipLaunchKernelGGL((quant_token_kernel<2, FP8>), grid, block, 0, st, x, K, q, s);
    else if (cpt <= 4) hipLaunchKernelGGL((quant_token_kernel<4, FP8>), grid, block, 0, st, x, K, q, s);
    else if (cpt <= 8) hipLaunchKernelGGL((quant_token_kernel<8, FP8>), grid, block, 0, st, x, K, q, s);
    else if (cpt <= 16) hipLaunchKernelGGL((quant_token_kernel<16, FP8>), grid, block, 0, st, x, K, q, s);
    else hipLaunchKernelGGL((quant_token_loop_kernel<FP8>), grid, block, 0, st, x, K, q, s);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_int8(const uint16_t* x, int64_t M, int64_t K, int8_t* q, float* s, hipStream_t st) {
    return launch_token<false>(x, M, K, reinterpret_cast<uint8_t*>(q), s, st);
}

hipError_t launch_quant_fp8(const uint16_t* x, int64_t M, int64_t K, int group, uint8_t* q, float* s,
                            hipStream_t st) {
    if (group == 0) return launch_token<true>(x, M, K, q, s, st);
    const int64_t ngroups = M * (K / 128);
    const int64_t per_block = kQuantThreads / 16;
    dim3 grid((unsigned)((ngroups + per_block - 1) / per_block)), block(kQuantThreads);
    hipLaunchKernelGGL(quant_group128_fp8_kernel, grid, block, 0, st, x, ngroups, q, s);
    return hipGetLastError();
}

}  // namespace qlin
