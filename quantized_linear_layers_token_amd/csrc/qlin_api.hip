// C ABI: argument validation and regime dispatch.  No allocation, no
// synchronization; every check runs before the first launch.
#include <stdint.h>

#include "../../include/qlin.h"
#include "qlin_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
    uintptr_t lo, hi;
};
Range rng(const void* p, int64_t bytes) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(p);
    return Range{b, b + (uintptr_t)bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

qlin_status hip_status(hipError_t e) {
    if (e == hipSuccess) return QLIN_OK;
    g_last_hip_error = (int)e;
    return QLIN_ERR_HIP;
}

bool valid_k(int64_t K) { return K > 0 && (K % 16) == 0 && K <= QLIN_MAX_K; }
bool valid_mn(int64_t v) { return v >= 0 && v <= QLIN_MAX_MN; }

int out_bytes(qlin_out o) { return o == QLIN_OUT_BF16 ? 2 : 4; }

// Shared checks of the product calls.  variant: qlin::Variant.
qlin_status check_product(int variant, const void* q_x, const float* s_x, const void* q_w, const uint16_t* s_w,
                          const void* y, int64_t M, int64_t N, int64_t K, qlin_out out, qlin_path path,
                          bool* noop) {
    *noop = false;
    if (!valid_mn(M) || !valid_mn(N) || !valid_k(K)) return QLIN_ERR_SHAPE;
    if (variant == qlin::VAR_FP8_BLOCK && ((N % 128) != 0 || (K % 128) != 0)) return QLIN_ERR_SHAPE;
    if (out != QLIN_OUT_BF16 && out != QLIN_OUT_F32 && out != QLIN_OUT_I32) return QLIN_ERR_UNSUPPORTED;
    if (out == QLIN_OUT_I32 && variant != qlin::VAR_INT8) return QLIN_ERR_UNSUPPORTED;
    if (path < QLIN_PATH_AUTO || path > QLIN_PATH_LARGE_256X256) return QLIN_ERR_UNSUPPORTED;
    if ((path == QLIN_PATH_LARGE_256X256_W8 || path == QLIN_PATH_LARGE_256X256) && variant == qlin::VAR_FP8_BLOCK)
        return QLIN_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) {
        *noop = true;
        return QLIN_OK;
    }
    if (path == QLIN_PATH_GEMV && M != 1) return QLIN_ERR_UNSUPPORTED;
    if (path == QLIN_PATH_SMALL && M > 32) return QLIN_ERR_UNSUPPORTED;
    if (!q_x || !s_x || !q_w || !s_w || !y) return QLIN_ERR_NULL;
    if (!aligned(q_x, 16) || !aligned(q_w, 16) || !aligned(y, 16) || !aligned(s_x, 4) || !aligned(s_w, 2))
        return QLIN_ERR_ALIGN;
    const int64_t kb = K / 128;
    const int64_t sx_n = variant == qlin::VAR_FP8_BLOCK ? M * kb : M;
    const int64_t sw_n = variant == qlin::VAR_FP8_BLOCK ? (N / 128) * kb : N;
    const Range ry = rng(y, M * N * out_bytes(out));
    if (overlap(ry, rng(q_x, M * K)) || overlap(ry, rng(q_w, N * K)) || overlap(ry, rng(s_x, sx_n * 4)) ||
        overlap(ry, rng(s_w, sw_n * 2)))
        return QLIN_ERR_ALIAS;
    return QLIN_OK;
}

qlin_status run_product(int variant, const void* q_x, const float* s_x, const void* q_w, const uint16_t* s_w,
                        void* y, int64_t M, int64_t N, int64_t K, qlin_out out, qlin_path path,
                        hipStream_t stream) {
    bool noop = false;
    const qlin_status st = check_product(variant, q_x, s_x, q_w, s_w, y, M, N, K, out, path, &noop);
    if (st != QLIN_OK || noop) return st;
    const uint8_t* qx = static_cast<const uint8_t*>(q_x);
    const uint8_t* qw = static_cast<const uint8_t*>(q_w);
    qlin_path p = path;
    if (p == QLIN_PATH_AUTO) p = (M == 1) ? QLIN_PATH_GEMV : (M <= 32 ? QLIN_PATH_SMALL : QLIN_PATH_LARGE);
    hipError_t e;
    if (p == QLIN_PATH_GEMV) e = qlin::launch_gemv(variant, qx, s_x, qw, s_w, y, N, K, (int)out, stream);
    else if (p == QLIN_PATH_SMALL)
        e = qlin::launch_gemm_small(variant, qx, s_x, qlin::one_segment(qw, s_w, y, N), M, K, (int)out, stream);
    else if (p == QLIN_PATH_LARGE)
        e = qlin::launch_gemm_large(variant, qx, s_x, qlin::one_segment(qw, s_w, y, N), M, K, (int)out, stream);
    else
        e = qlin::launch_gemm_large_cfg((int)p - (int)QLIN_PATH_LARGE_256X128, variant, qx, s_x,
                                        qlin::one_segment(qw, s_w, y, N), M, K, (int)out, stream);
    return hip_status(e);
}

qlin_status check_quant(const uint16_t* x, int64_t M, int64_t K, const void* q, const float* s, int64_t s_count,
                        bool* noop) {
    *noop = false;
    if (!valid_mn(M) || !valid_k(K)) return QLIN_ERR_SHAPE;
    if (M == 0) {
        *noop = true;
        return QLIN_OK;
    }
    if (!x || !q || !s) return QLIN_ERR_NULL;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4)) return QLIN_ERR_ALIGN;
    const Range rx = rng(x, M * K * 2), rq = rng(q, M * K), rs = rng(s, s_count * 4);
    if (overlap(rq, rx) || overlap(rs, rx) || overlap(rq, rs)) return QLIN_ERR_ALIAS;
    return QLIN_OK;
}

qlin_status check_linear(qlin_scheme scheme, const uint16_t* x, int64_t M, int64_t K, const qlin_segment* segs,
                         int32_t nseg, qlin_out out, const void* q_x, const float* s_x, bool fused, bool* noop) {
    *noop = false;
    if (scheme != QLIN_SCHEME_W8A8 && scheme != QLIN_SCHEME_FP8_ROWWISE && scheme != QLIN_SCHEME_FP8_BLOCK)
        return QLIN_ERR_UNSUPPORTED;
    if (!segs) return QLIN_ERR_NULL;
    if (nseg < 1 || nseg > QLIN_MAX_SEGMENTS) return QLIN_ERR_SHAPE;
    if (!valid_mn(M) || !valid_k(K)) return QLIN_ERR_SHAPE;
    const bool block = scheme == QLIN_SCHEME_FP8_BLOCK;
    if (block && (K % 128) != 0) return QLIN_ERR_SHAPE;
    if (out != QLIN_OUT_BF16 && out != QLIN_OUT_F32 && out != QLIN_OUT_I32) return QLIN_ERR_UNSUPPORTED;
    if (out == QLIN_OUT_I32 && scheme != QLIN_SCHEME_W8A8) return QLIN_ERR_UNSUPPORTED;
    int64_t ntot = 0;
    for (int i = 0; i < nseg; ++i) {
        if (!valid_mn(segs[i].n)) return QLIN_ERR_SHAPE;
        if (block && (segs[i].n % 128) != 0) return QLIN_ERR_SHAPE;
        ntot += segs[i].n;
    }
    if (ntot > QLIN_MAX_MN) return QLIN_ERR_SHAPE;
    if (M == 0 || ntot == 0) {
        *noop = true;
        return QLIN_OK;
    }
    if (!x) return QLIN_ERR_NULL;
    if (!fused && (!q_x || !s_x)) return QLIN_ERR_NULL;
    if ((q_x == nullptr) != (s_x == nullptr)) return QLIN_ERR_NULL;
    if (!aligned(x, 16) || (q_x && !aligned(q_x, 16)) || (s_x && !aligned(s_x, 4))) return QLIN_ERR_ALIGN;
    const int64_t sx_n = block ? M * (K / 128) : M;
    const Range rx = rng(x, M * K * 2);
    Range rq = rng(q_x, q_x ? M * K : 0), rs = rng(s_x, s_x ? sx_n * 4 : 0);
    if (q_x && (overlap(rq, rx) || overlap(rs, rx) || overlap(rq, rs))) return QLIN_ERR_ALIAS;
    for (int i = 0; i < nseg; ++i) {
        if (segs[i].n == 0) continue;
        if (!segs[i].q_w || !segs[i].s_w || !segs[i].y) return QLIN_ERR_NULL;
        if (!aligned(segs[i].q_w, 16) || !aligned(segs[i].y, 16) || !aligned(segs[i].s_w, 2)) return QLIN_ERR_ALIGN;
        // the staging buffers are written while the weights are read
        const int64_t swi = block ? (segs[i].n / 128) * (K / 128) : segs[i].n;
        const Range rw = rng(segs[i].q_w, segs[i].n * K), rsw = rng(segs[i].s_w, swi * 2);
        if (q_x && (overlap(rq, rw) || overlap(rq, rsw) || overlap(rs, rw) || overlap(rs, rsw))) return QLIN_ERR_ALIAS;
        const Range ry = rng(segs[i].y, M * segs[i].n * out_bytes(out));
        if (overlap(ry, rx) || (q_x && (overlap(ry, rq) || overlap(ry, rs)))) return QLIN_ERR_ALIAS;
        for (int j = 0; j < nseg; ++j) {
            if (segs[j].n == 0) continue;
            const int64_t swn = block ? (segs[j].n / 128) * (K / 128) : segs[j].n;
            if (overlap(ry, rng(segs[j].q_w, segs[j].n * K)) || overlap(ry, rng(segs[j].s_w, swn * 2)))
                return QLIN_ERR_ALIAS;
            if (j != i && overlap(ry, rng(segs[j].y, M * segs[j].n * out_bytes(out)))) return QLIN_ERR_ALIAS;
        }
    }
    return QLIN_OK;
}

}  // namespace

namespace qlin {

qlin_status linear_validate(qlin_scheme scheme, const uint16_t* x, int64_t M, int64_t K, const qlin_segment* segments,
                            int32_t nseg, qlin_out out, bool* noop) {
    return check_linear(scheme, x, M, K, segments, nseg, out, nullptr, nullptr, true, noop);
}

bool linear_is_one_launch(qlin_scheme scheme, int64_t M, int64_t K, const qlin_segment* segments, int32_t nseg) {
    const int variant = scheme == QLIN_SCHEME_W8A8 ? VAR_INT8 : scheme == QLIN_SCHEME_FP8_ROWWISE ? VAR_FP8_ROW
                                                                                                   : VAR_FP8_BLOCK;
    int64_t rows = 0;   // weight rows of the call (validated separately)
    if (segments != nullptr && nseg >= 1 && nseg <= QLIN_MAX_SEGMENTS)
        for (int i = 0; i < nseg; ++i) rows += segments[i].n > 0 ? segments[i].n : 0;
    return ((M == 1) && (K <= kDecodeMaxK)) || linear_tokens_fits(variant, M, K, rows) || small_fused_fits(M, K);
}

qlin_status linear_call(qlin_scheme scheme, const uint16_t* x, int64_t M, int64_t K, const qlin_segment* segments,
                        int32_t nseg, qlin_out out, void* q_x, float* s_x, hipStream_t stream) {
    const int variant = scheme == QLIN_SCHEME_W8A8 ? qlin::VAR_INT8
                        : scheme == QLIN_SCHEME_FP8_ROWWISE ? qlin::VAR_FP8_ROW : qlin::VAR_FP8_BLOCK;
    int64_t rows = 0;   // weight rows of the call (validated by check_linear below)
    if (segments != nullptr && nseg >= 1 && nseg <= QLIN_MAX_SEGMENTS)
        for (int i = 0; i < nseg; ++i) rows += segments[i].n > 0 ? segments[i].n : 0;
    const bool tokens = qlin::linear_tokens_fits(variant, M, K, rows);
    const bool fused = linear_is_one_launch(scheme, M, K, segments, nseg);
    bool noop = false;
    const qlin_status st = check_linear(scheme, x, M, K, segments, nseg, out, q_x, s_x, fused, &noop);
    if (st != QLIN_OK || noop) return st;
    // the non-empty segments, packed
    qlin::SegmentArgs sa{};
    int n = 0, k = 0;
    for (int i = 0; i < nseg; ++i) {
        if (segments[i].n == 0) continue;
        sa.w[k] = static_cast<const uint8_t*>(segments[i].q_w);
        sa.sw[k] = segments[i].s_w;
        sa.y[k] = segments[i].y;
        sa.start[k] = n;
        n += (int)segments[i].n;
        ++k;
    }
    sa.nseg = k;
    for (int i = k; i <= qlin::kMaxSegments; ++i) sa.start[i] = n;
    if (fused && M == 1)
        return hip_status(qlin::launch_linear_decode(variant, x, K, sa, (int)out, static_cast<uint8_t*>(q_x), s_x,
                                                     stream));
    if (tokens)
        return hip_status(qlin::launch_linear_tokens(variant, x, M, K, sa, (int)out, static_cast<uint8_t*>(q_x), s_x,
                                                     stream));
    if (fused)
        return hip_status(qlin::launch_gemm_small_fused(variant, x, M, K, sa, (int)out, static_cast<uint8_t*>(q_x),
                                                        s_x, stream));
    hipError_t e;
    if (variant == qlin::VAR_INT8) e = qlin::launch_quant_int8(x, M, K, static_cast<int8_t*>(q_x), s_x, stream);
    else e = qlin::launch_quant_fp8(x, M, K, variant == qlin::VAR_FP8_BLOCK ? 128 : 0, static_cast<uint8_t*>(q_x),
                                    s_x, stream);
    if (e != hipSuccess) return hip_status(e);
    if (M > 32)   // every segment in one tiled-GEMM launch
        return hip_status(qlin::launch_gemm_large(variant, static_cast<const uint8_t*>(q_x), s_x, sa, M, K, (int)out,
                                                  stream));
    if (M > 1)    // every segment in one small-M launch
        return hip_status(qlin::launch_gemm_small(variant, static_cast<const uint8_t*>(q_x), s_x, sa, M, K, (int)out,
                                                  stream));
    for (int i = 0; i < nseg; ++i) {
        if (segments[i].n == 0) continue;
        const qlin_status s = run_product(variant, q_x, s_x, segments[i].q_w, segments[i].s_w, segments[i].y, M,
                                          segments[i].n, K, out, QLIN_PATH_AUTO, stream);
        if (s != QLIN_OK) return s;
    }
    return QLIN_OK;
}

}  // namespace qlin

extern "C" {

qlin_status qlin_linear(qlin_scheme scheme, const uint16_t* x, int64_t M, int64_t K, const qlin_segment* segments,
                        int32_t nseg, qlin_out out, void* q_x, float* s_x, hipStream_t stream) {
    return qlin::linear_call(scheme, x, M, K, segments, nseg, out, q_x, s_x, stream);
}


qlin_status qlin_pack_weights(qlin_scheme scheme, const void* q_w, int64_t N, int64_t K, void* q_w_packed,
                              hipStream_t stream) {
    if (scheme != QLIN_SCHEME_W8A8 && scheme != QLIN_SCHEME_FP8_ROWWISE && scheme != QLIN_SCHEME_FP8_BLOCK)
        return QLIN_ERR_UNSUPPORTED;
    if (!valid_mn(N) || !valid_k(K) || (N % 128) != 0 || (K % 128) != 0) return QLIN_ERR_SHAPE;
    if (N == 0) return QLIN_OK;
    if (!q_w || !q_w_packed) return QLIN_ERR_NULL;
    if (!aligned(q_w, 16) || !aligned(q_w_packed, 16)) return QLIN_ERR_ALIGN;
    if (overlap(rng(q_w, N * K), rng(q_w_packed, N * K))) return QLIN_ERR_ALIAS;
    // the block scheme's codes are E4M3 like the rowwise one's: same layout
    const int variant = scheme == QLIN_SCHEME_W8A8 ? qlin::VAR_INT8 : qlin::VAR_FP8_ROW;
    return hip_status(qlin::launch_pack_weights(variant, static_cast<const uint8_t*>(q_w), N, K,
                                                static_cast<uint8_t*>(q_w_packed), stream));
}

qlin_status qlin_linear_packed(qlin_scheme scheme, const uint16_t* x, int64_t M, int64_t K,
                               const qlin_segment* segments, int32_t nseg, qlin_out out, void* q_x, float* s_x,
                               hipStream_t stream) {
    bool noop = false;
    // the staged form's checks (staging buffers required)
    const qlin_status st = check_linear(scheme, x, M, K, segments, nseg, out, q_x, s_x, false, &noop);
    if (st != QLIN_OK || noop) return st;
    if ((K % 128) != 0) return QLIN_ERR_SHAPE;
    for (int i = 0; i < nseg; ++i)
        if ((segments[i].n % 128) != 0) return QLIN_ERR_SHAPE;
    if (M < 33) return QLIN_ERR_UNSUPPORTED;
    const int variant = scheme == QLIN_SCHEME_W8A8 ? qlin::VAR_INT8
                        : scheme == QLIN_SCHEME_FP8_ROWWISE ? qlin::VAR_FP8_ROW : qlin::VAR_FP8_BLOCK;
    qlin::SegmentArgs sa{};
    int n = 0, k = 0;
    for (int i = 0; i < nseg; ++i) {
        if (segments[i].n == 0) continue;
        sa.w[k] = static_cast<const uint8_t*>(segments[i].q_w);
        sa.sw[k] = segments[i].s_w;
        sa.y[k] = segments[i].y;
        sa.start[k] = n;
        n += (int)segments[i].n;
        ++k;
    }
    sa.nseg = k;
    for (int i = k; i <= qlin::kMaxSegments; ++i) sa.start[i] = n;
    hipError_t e;
    if (variant == qlin::VAR_INT8) e = qlin::launch_quant_int8(x, M, K, static_cast<int8_t*>(q_x), s_x, stream);
    else e = qlin::launch_quant_fp8(x, M, K, variant == qlin::VAR_FP8_BLOCK ? 128 : 0, static_cast<uint8_t*>(q_x),
                                    s_x, stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(qlin::launch_gemm_packed(variant, static_cast<const uint8_t*>(q_x), s_x, sa, M, K, (int)out,
                                               stream));
}

qlin_status qlin_linear_weight_only(qlin_scheme scheme, const uint16_t* x, int64_t M, int64_t K,
                                    const qlin_segment* segments, int32_t nseg, qlin_out out, hipStream_t stream) {
    if (out == QLIN_OUT_I32) return QLIN_ERR_UNSUPPORTED;
    bool noop = false;
    const qlin_status st = check_linear(scheme, x, M, K, segments, nseg, out, nullptr, nullptr, true, &noop);
    if (st != QLIN_OK || noop) return st;
    if (M > 32) return QLIN_ERR_UNSUPPORTED;
    const int variant = scheme == QLIN_SCHEME_W8A8 ? qlin::VAR_INT8
                        : scheme == QLIN_SCHEME_FP8_ROWWISE ? qlin::VAR_FP8_ROW : qlin::VAR_FP8_BLOCK;
    qlin::SegmentArgs sa{};
    int n = 0, k = 0;
    for (int i = 0; i < nseg; ++i) {
        if (segments[i].n == 0) continue;
        sa.w[k] = static_cast<const uint8_t*>(segments[i].q_w);
        sa.sw[k] = segments[i].s_w;
        sa.y[k] = segments[i].y;
        sa.start[k] = n;
        n += (int)segments[i].n;
        ++k;
    }
    sa.nseg = k;
    for (int i = k; i <= qlin::kMaxSegments; ++i) sa.start[i] = n;
    return hip_status(qlin::launch_weight_only(variant, x, M, K, sa, (int)out, stream));
}

qlin_status qlin_linear_swiglu(qlin_scheme scheme, const uint16_t* x, int64_t M, int64_t K, const void* gate_q_w,
                               const uint16_t* gate_s_w, const void* up_q_w, const uint16_t* up_s_w, int64_t I,
                               uint16_t* h, void* q_x, float* s_x, hipStream_t stream) {
    const bool decode = (M == 1) && (K <= qlin::kDecodeMaxK);
    const bool fused = decode || qlin::small_fused_fits(M, K);
    // the gate and up projections each checked as a bf16 projection into h:
    // together this covers h against x, the staging buffers and both weights
    const qlin_segment gate{gate_q_w, gate_s_w, h, I}, up{up_q_w, up_s_w, h, I};
    bool noop = false;
    qlin_status st = check_linear(scheme, x, M, K, &gate, 1, QLIN_OUT_BF16, q_x, s_x, fused, &noop);
    if (st != QLIN_OK || noop) return st;
    st = check_linear(scheme, x, M, K, &up, 1, QLIN_OUT_BF16, q_x, s_x, fused, &noop);
    if (st != QLIN_OK || noop) return st;
    const int variant = scheme == QLIN_SCHEME_W8A8 ? qlin::VAR_INT8
                        : scheme == QLIN_SCHEME_FP8_ROWWISE ? qlin::VAR_FP8_ROW : qlin::VAR_FP8_BLOCK;
    qlin::SegmentArgs sa{};
    sa.w[0] = static_cast<const uint8_t*>(gate_q_w);
    sa.w[1] = static_cast<const uint8_t*>(up_q_w);
    sa.sw[0] = gate_s_w;
    sa.sw[1] = up_s_w;
    sa.y[0] = sa.y[1] = h;
    sa.start[0] = 0;
    sa.start[1] = (int)I;
    for (int i = 2; i <= qlin::kMaxSegments; ++i) sa.start[i] = (int)(2 * I);
    sa.nseg = 2;
    const int mode = qlin::OUT_SWIGLU;
    if (decode)
        return hip_status(qlin::launch_linear_decode(variant, x, K, sa, mode, static_cast<uint8_t*>(q_x), s_x, stream));
    if (fused)
        return hip_status(qlin::launch_gemm_small_fused(variant, x, M, K, sa, mode, static_cast<uint8_t*>(q_x), s_x,
                                                        stream));
    hipError_t e;
    if (variant == qlin::VAR_INT8) e = qlin::launch_quant_int8(x, M, K, static_cast<int8_t*>(q_x), s_x, stream);
    else e = qlin::launch_quant_fp8(x, M, K, variant == qlin::VAR_FP8_BLOCK ? 128 : 0, static_cast<uint8_t*>(q_x),
                                    s_x, stream);
    if (e != hipSuccess) return hip_status(e);
    if (M > 32)
        return hip_status(qlin::launch_gemm_large(variant, static_cast<const uint8_t*>(q_x), s_x, sa, M, K, mode,
                                                  stream));
    return hip_status(qlin::launch_gemm_small(variant, static_cast<const uint8_t*>(q_x), s_x, sa, M, K, mode,
                                              stream));
}

qlin_status qlin_linear_swiglu_packed(qlin_scheme scheme, const uint16_t* x, int64_t M, int64_t K,
                                      const void* gate_q_w_packed, const uint16_t* gate_s_w, const void* up_q_w_packed,
                                      const uint16_t* up_s_w, int64_t I, uint16_t* h, void* q_x, float* s_x,
                                      hipStream_t stream) {
    // checked as qlin_linear_swiglu's staged form (staging required)
    const qlin_segment gate{gate_q_w_packed, gate_s_w, h, I}, up{up_q_w_packed, up_s_w, h, I};
    bool noop = false;
    qlin_status st = check_linear(scheme, x, M, K, &gate, 1, QLIN_OUT_BF16, q_x, s_x, false, &noop);
    if (st != QLIN_OK || noop) return st;
    st = check_linear(scheme, x, M, K, &up, 1, QLIN_OUT_BF16, q_x, s_x, false, &noop);
    if (st != QLIN_OK || noop) return st;
    if ((K % 128) != 0 || (I % 128) != 0) return QLIN_ERR_SHAPE;
    if (M < 33) return QLIN_ERR_UNSUPPORTED;
    const int variant = scheme == QLIN_SCHEME_W8A8 ? qlin::VAR_INT8
                        : scheme == QLIN_SCHEME_FP8_ROWWISE ? qlin::VAR_FP8_ROW : qlin::VAR_FP8_BLOCK;
    qlin::SegmentArgs sa{};
    sa.w[0] = static_cast<const uint8_t*>(gate_q_w_packed);
    sa.w[1] = static_cast<const uint8_t*>(up_q_w_packed);
    sa.sw[0] = gate_s_w;
    sa.sw[1] = up_s_w;
    sa.y[0] = sa.y[1] = h;
    sa.start[0] = 0;
    sa.start[1] = (int)I;
    for (int i = 2; i <= qlin::kMaxSegments; ++i) sa.start[i] = (int)(2 * I);
    sa.nseg = 2;
    hipError_t e;
    if (variant == qlin::VAR_INT8) e = qlin::launch_quant_int8(x, M, K, static_cast<int8_t*>(q_x), s_x, stream);
    else e = qlin::launch_quant_fp8(x, M, K, variant == qlin::VAR_FP8_BLOCK ? 128 : 0, static_cast<uint8_t*>(q_x),
                                    s_x, stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(qlin::launch_gemm_packed(variant, static_cast<const uint8_t*>(q_x), s_x, sa, M, K,
                                               qlin::OUT_SWIGLU, stream));
}

qlin_status qlin_quant_act_int8(const uint16_t* x, int64_t M, int64_t K, int8_t* q, float* s, hipStream_t stream) {
    bool noop = false;
    const qlin_status st = check_quant(x, M, K, q, s, M, &noop);
    if (st != QLIN_OK || noop) return st;
    return hip_status(qlin::launch_quant_int8(x, M, K, q, s, stream));
}

qlin_status qlin_quant_act_fp8(const uint16_t* x, int64_t M, int64_t K, int32_t group, uint8_t* q, float* s,
                               hipStream_t stream) {
    if (group != 0 && group != 128) return QLIN_ERR_SHAPE;
    if (group == 128 && (K % 128) != 0) return QLIN_ERR_SHAPE;
    bool noop = false;
    const int64_t s_count = group ? M * (K / 128) : M;
    const qlin_status st = check_quant(x, M, K, q, s, s_count, &noop);
    if (st != QLIN_OK || noop) return st;
    return hip_status(qlin::launch_quant_fp8(x, M, K, group, q, s, stream));
}

qlin_status qlin_gemv_w8a8(const int8_t* q_x, const float* s_x, const int8_t* q_w, const uint16_t* s_w, void* y,
                           int64_t N, int64_t K, qlin_out out, hipStream_t stream) {
    return run_product(qlin::VAR_INT8, q_x, s_x, q_w, s_w, y, 1, N, K, out, QLIN_PATH_GEMV, stream);
}

qlin_status qlin_gemm_w8a8(const int8_t* q_x, const float* s_x, const int8_t* q_w, const uint16_t* s_w, void* y,
                           int64_t M, int64_t N, int64_t K, qlin_out out, hipStream_t stream) {
    return run_product(qlin::VAR_INT8, q_x, s_x, q_w, s_w, y, M, N, K, out, QLIN_PATH_AUTO, stream);
}

qlin_status qlin_gemm_w8a8_ex(const int8_t* q_x, const float* s_x, const int8_t* q_w, const uint16_t* s_w, void* y,
                              int64_t M, int64_t N, int64_t K, qlin_out out, qlin_path path, hipStream_t stream) {
    return run_product(qlin::VAR_INT8, q_x, s_x, q_w, s_w, y, M, N, K, out, path, stream);
}

qlin_status qlin_gemm_fp8_rowwise(const uint8_t* q_x, const float* s_x, const uint8_t* q_w, const uint16_t* s_w,
                                  void* y, int64_t M, int64_t N, int64_t K, qlin_out out, hipStream_t stream) {
    return run_product(qlin::VAR_FP8_ROW, q_x, s_x, q_w, s_w, y, M, N, K, out, QLIN_PATH_AUTO, stream);
}

qlin_status qlin_gemm_fp8_rowwise_ex(const uint8_t* q_x, const float* s_x, const uint8_t* q_w,
                                     const uint16_t* s_w, void* y, int64_t M, int64_t N, int64_t K, qlin_out out,
                                     qlin_path path, hipStream_t stream) {
    return run_product(qlin::VAR_FP8_ROW, q_x, s_x, q_w, s_w, y, M, N, K, out, path, stream);
}

qlin_status qlin_gemm_fp8_block(const uint8_t* q_x, const float* s_x, const uint8_t* q_w, const uint16_t* s_w,
                                void* y, int64_t M, int64_t N, int64_t K, qlin_out out, hipStream_t stream) {
    return run_product(qlin::VAR_FP8_BLOCK, q_x, s_x, q_w, s_w, y, M, N, K, out, QLIN_PATH_AUTO, stream);
}

qlin_status qlin_gemm_fp8_block_ex(const uint8_t* q_x, const float* s_x, const uint8_t* q_w, const uint16_t* s_w,
                                   void* y, int64_t M, int64_t N, int64_t K, qlin_out out, qlin_path path,
                                   hipStream_t stream) {
    return run_product(qlin::VAR_FP8_BLOCK, q_x, s_x, q_w, s_w, y, M, N, K, out, path, stream);
}

const char* qlin_status_string(qlin_status status) {
    switch (status) {
        case QLIN_OK: return "QLIN_OK";
        case QLIN_ERR_NULL: return "QLIN_ERR_NULL: a required pointer is null";
        case QLIN_ERR_SHAPE: return "QLIN_ERR_SHAPE: invalid M, N, K or group";
        case QLIN_ERR_ALIGN: return "QLIN_ERR_ALIGN: a pointer misses its required alignment";
        case QLIN_ERR_UNSUPPORTED: return "QLIN_ERR_UNSUPPORTED: output mode or path not available";
        case QLIN_ERR_HIP: return "QLIN_ERR_HIP: the HIP runtime rejected the launch";
        case QLIN_ERR_ALIAS: return "QLIN_ERR_ALIAS: an output overlaps an input";
        case QLIN_ERR_TOO_LARGE:
            return "QLIN_ERR_TOO_LARGE: the call needs more staging than the allocation-free scratch holds";
    }
    return "QLIN_ERR_UNKNOWN";
}

int qlin_abi_version(void) { return QLIN_ABI_VERSION; }

int qlin_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
