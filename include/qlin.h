/*
 * qlin -- quantized decoder projections for AMD Instinct MI355X (gfx950).
 *
 * One operation in three schemes:
 *
 *     y[m, n] = (s_x[m] * s_w[n]) * sum_k q_x[m, k] * q_w[n, k]
 *
 *   W8A8 int8   -- "Llama 3.1 8B Instruct W8A8" model card, intro and section
 *                  "Loading": int8 weights with one bf16 scale per output row,
 *                  activations quantized to int8 per token, int8
 *                  products accumulated in int32.
 *   FP8 rowwise -- "Llama 3.1 8B Instruct FP8" page intro and the
 *                  "Meta-Llama-3.1-8B-Instruct-FP8-dynamic" README ("Model
 *                  Optimizations", "Creation"): E4M3 weights with one scale
 *                  per output channel, per-token dynamic E4M3 inputs.
 *   FP8 block   -- "Qwen3 8B FP8" model card, intro and "Loading": E4M3
 *                  weights with one bf16 scale per 128x128 block (a
 *                  multiplier), activations quantized to E4M3 in groups of 128; widths
 *                  are multiples of 128.  Per K block kb:
 *                  y[m, n] = sum_kb s_x[m, kb] * s_w[n/128, kb] * P_kb[m, n].
 *
 * Conventions shared by every entry point
 *  - Pointers are caller-owned DEVICE memory.  The library never allocates,
 *    frees or synchronizes; work is enqueued on `stream` (0 = the null
 *    stream) and the call returns at once.  Outputs must not overlap inputs.
 *  - Matrices are contiguous and row-major with K fastest: x / q_x are
 *    [M, K], q_w is [N, K] (one row per output channel), y is [M, N].
 *  - Matrix pointers (x, q, q_x, q_w, y) must be 16-byte aligned; f32 scale
 *    pointers 4-byte aligned; bf16 scale pointers 2-byte aligned.
 *  - K must be a positive multiple of 16 and at most QLIN_MAX_K; M and N are
 *    >= 0 and at most QLIN_MAX_MN.  M == 0 or N == 0 is a no-op returning
 *    QLIN_OK.
 *  - bf16 values are passed as their uint16 bit patterns; E4M3 values as
 *    uint8 codes (OCP E4M3: bias 7, max 448, 0x7F/0xFF NaN, no infinities).
 *  - Errors are returned, never thrown.  Arguments are validated before any
 *    work is enqueued: on an error return nothing was launched and no output
 *    was touched.  QLIN_ERR_HIP means the launch itself failed; the HIP error
 *    code is then available from qlin_last_hip_error() on the calling thread.
 *  - Calls are thread-safe; calls on different streams may run concurrently.
 */
#ifndef QLIN_H_
#define QLIN_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's own hipStream_t. */
typedef struct ihipStream_t* hipStream_t;

#define QLIN_ABI_VERSION 3
#define QLIN_MAX_K  131072          /* 127 * 128 * K stays below 2^31 */
#define QLIN_MAX_MN (1 << 24)

typedef enum qlin_status {
    QLIN_OK = 0,
    QLIN_ERR_NULL = 1,         /* a required pointer is null */
    QLIN_ERR_SHAPE = 2,        /* bad size: K <= 0, K % 16, > max, block sizes not multiples of 128, bad group */
    QLIN_ERR_ALIGN = 3,        /* a pointer misses its required alignment */
    QLIN_ERR_UNSUPPORTED = 4,  /* output mode or forced path not available for this call */
    QLIN_ERR_HIP = 5,          /* the HIP runtime rejected the launch */
    QLIN_ERR_ALIAS = 6,        /* an output range overlaps an input range */
    QLIN_ERR_TOO_LARGE = 7     /* the call needs more staging than qlin_linear_noalloc's fixed scratch */
} qlin_status;

/* Output element type written to y. */
typedef enum qlin_out {
    QLIN_OUT_BF16 = 0,  /* bf16, round to nearest even of the f32 result */
    QLIN_OUT_I32 = 1,   /* int8 schemes only: the raw int32 accumulator sum_k q_x*q_w */
    QLIN_OUT_F32 = 2    /* the f32 result before the bf16 rounding */
} qlin_out;

/* Kernel regime.  AUTO follows the pages' split ("Loading" sections of the
 * W8A8 and Qwen3 model cards): a single row -> a kernel touching every
 * weight byte exactly once; at most 32 rows -> matrix cores streaming the
 * weights; more rows -> a tiled matrix-core GEMM.  The other values force one kernel at
 * any M (for testing each kernel outside its default regime). */
typedef enum qlin_path {
    QLIN_PATH_AUTO = 0,
    QLIN_PATH_GEMV = 1,   /* M must be 1 */
    QLIN_PATH_SMALL = 2,  /* M must be <= 32 */
    QLIN_PATH_LARGE = 3,  /* any M; tile shape chosen from M and N */
    /* the tiled GEMM with one fixed output tile (weight rows x tokens), any M */
    QLIN_PATH_LARGE_256X128 = 4,
    QLIN_PATH_LARGE_128X128 = 5,
    QLIN_PATH_LARGE_128X64 = 6,
    QLIN_PATH_LARGE_128X256 = 7,
    /* the same tiles with 8 wavefronts: two groups of four split the K stages
     * of one tile and add their partial sums before the epilogue */
    QLIN_PATH_LARGE_128X128_K2 = 8,
    QLIN_PATH_LARGE_128X64_K2 = 9,
    /* 256 x 256 with 8 wavefronts of 128 x 64, one workgroup per CU; int8 and
     * FP8 rowwise only (QLIN_ERR_UNSUPPORTED for block FP8) */
    QLIN_PATH_LARGE_256X256_W8 = 10,
    /* 256 x 256 with 4 wavefronts of 128 x 128 (one per SIMD), one workgroup
     * per CU; int8 and FP8 rowwise only */
    QLIN_PATH_LARGE_256X256 = 11
} qlin_path;

/* ---------------------------------------------------------------------- */
/* Dynamic activation quantizers                                          */
/* ---------------------------------------------------------------------- */

/* Per-token int8 quantization (W8A8 model card, intro and "Loading": each
 * token of the input gets its own int8 scale).  For each row m of x (bf16 [M, K]):
 *   a = max_k |x[m,k]|;  s[m] = fl32(a / 127);  inv = fl32(127 / a) (0 if a == 0)
 *   q[m,k] = clamp(round_half_even(fl32(x[m,k] * inv)), -127, 127)
 * For a < 2^-64 (where 127/a can overflow f32) x and a are first scaled by
 * 2^64, exactly: q = ...(fl32(fl32(x * 2^64) * fl32(127 / (a * 2^64)))), which
 * equals the form above wherever 127/a is finite.
 * q: int8 [M, K] (written), s: f32 [M] (written).  Non-finite inputs are
 * outside the contract (no fault, values of that row unspecified). */
qlin_status qlin_quant_act_int8(const uint16_t* x, int64_t M, int64_t K,
                                int8_t* q, float* s, hipStream_t stream);

/* Dynamic FP8 (OCP E4M3) quantization.
 *   group == 0:   one scale per token (FP8-dynamic README, "Creation" recipe:
 *                 per-token, dynamic, symmetric); s is f32 [M].
 *   group == 128: one scale per 128 consecutive inputs, groups aligned at
 *                 k = 128 g (Qwen3 8B FP8 model card, "Loading"); K % 128 == 0;
 *                 s is f32 [M, K/128] row-major.
 * Per token or group: s = fl32(a / 448), inv = fl32(448 / a) (0 if a == 0),
 *   q = nearest E4M3 code of clamp(fl32(x * inv), -448, 448), ties to even,
 *   sign of zero kept; for a < 2^-64 with x and a scaled by 2^64 first, as
 *   for qlin_quant_act_int8.  Non-finite inputs: as for qlin_quant_act_int8. */
qlin_status qlin_quant_act_fp8(const uint16_t* x, int64_t M, int64_t K, int32_t group,
                               uint8_t* q, float* s, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Products                                                               */
/* ---------------------------------------------------------------------- */

/* One-token W8A8 product (M = 1; W8A8 model card, "Loading": a single row
 * is served by a kernel touching every weight byte exactly once).
 *   q_x int8 [K], s_x f32 [1], q_w int8 [N, K], s_w bf16 [N], y [N].
 *   acc[n] = sum_k q_x[k] q_w[n,k] (exact int32);
 *   BF16/F32: y[n] = fl32(acc) * fl32(s_x * s_w[n]), rounded to bf16 for BF16;
 *   I32: y[n] = acc. */
qlin_status qlin_gemv_w8a8(const int8_t* q_x, const float* s_x,
                           const int8_t* q_w, const uint16_t* s_w,
                           void* y, int64_t N, int64_t K, qlin_out out,
                           hipStream_t stream);

/* W8A8 product for any M ("Llama 3.1 8B Instruct W8A8" model card, intro:
 * int8 weights with one bf16 scale per output row times per-token int8
 * activations; "Loading": one row goes to a kernel reading each weight byte
 * once, up to 32 rows to the matrix units, longer inputs to a tiled product
 * summing the int8 products in int32).  Same formula per row m as
 * qlin_gemv_w8a8; s_x f32 [M], y [M, N].
 * Dispatch (AUTO): M == 1 -> the one-row kernel; 2..32 -> matrix-core
 * streaming kernel; larger -> tiled matrix-core GEMM.  A fused projection
 * (e.g. q/k/v or gate/up) is the same call on row-concatenated q_w / s_w.
 * Same validation and error behaviour as every entry point (see the top of
 * this file); _ex forces one kernel (qlin_path), QLIN_ERR_UNSUPPORTED where it
 * cannot run this call. */
qlin_status qlin_gemm_w8a8(const int8_t* q_x, const float* s_x,
                           const int8_t* q_w, const uint16_t* s_w,
                           void* y, int64_t M, int64_t N, int64_t K, qlin_out out,
                           hipStream_t stream);
qlin_status qlin_gemm_w8a8_ex(const int8_t* q_x, const float* s_x,
                              const int8_t* q_w, const uint16_t* s_w,
                              void* y, int64_t M, int64_t N, int64_t K, qlin_out out,
                              qlin_path path, hipStream_t stream);

/* FP8 E4M3 product with per-token activation scales s_x f32 [M] and
 * per-output-channel weight scales s_w bf16 [N] ("Llama 3.1 8B Instruct FP8"
 * intro; FP8-dynamic README "Model Optimizations").  q_x uint8 [M, K],
 * q_w uint8 [N, K].  acc = sum_k e4m3(q_x) e4m3(q_w) in f32 (any order);
 * y = acc * fl32(s_x[m] * s_w[n]).  Out modes: BF16, F32. */
qlin_status qlin_gemm_fp8_rowwise(const uint8_t* q_x, const float* s_x,
                                  const uint8_t* q_w, const uint16_t* s_w,
                                  void* y, int64_t M, int64_t N, int64_t K, qlin_out out,
                                  hipStream_t stream);
qlin_status qlin_gemm_fp8_rowwise_ex(const uint8_t* q_x, const float* s_x,
                                     const uint8_t* q_w, const uint16_t* s_w,
                                     void* y, int64_t M, int64_t N, int64_t K, qlin_out out,
                                     qlin_path path, hipStream_t stream);

/* FP8 E4M3 product with 128x128 weight-block scales and 1x128 activation
 * group scales (Qwen3 8B FP8 model card, intro and "Loading"; the weight
 * scale multiplies).  N % 128 == 0 and K % 128 == 0.
 *   s_x f32 [M, K/128], s_w bf16 [N/128, K/128] (row-major).
 *   y[m,n] = sum_kb (s_x[m,kb] * s_w[n/128,kb]) * P_kb[m,n], f32 accumulate,
 *   where P_kb is the E4M3 dot product over k in [128 kb, 128 kb + 128).
 * Out modes: BF16, F32. */
qlin_status qlin_gemm_fp8_block(const uint8_t* q_x, const float* s_x,
                                const uint8_t* q_w, const uint16_t* s_w,
                                void* y, int64_t M, int64_t N, int64_t K, qlin_out out,
                                hipStream_t stream);
qlin_status qlin_gemm_fp8_block_ex(const uint8_t* q_x, const float* s_x,
                                   const uint8_t* q_w, const uint16_t* s_w,
                                   void* y, int64_t M, int64_t N, int64_t K, qlin_out out,
                                   qlin_path path, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Fused projection: bf16 activations in                                  */
/* ---------------------------------------------------------------------- */

typedef enum qlin_scheme {
    QLIN_SCHEME_W8A8 = 0,         /* int8 per-token activations, int8 weights, bf16 row scales */
    QLIN_SCHEME_FP8_ROWWISE = 1,  /* E4M3 per-token activations, E4M3 weights, bf16 row scales */
    QLIN_SCHEME_FP8_BLOCK = 2     /* E4M3 1x128-group activations, E4M3 weights, bf16 128x128 block scales */
} qlin_scheme;

#define QLIN_MAX_SEGMENTS 4

/* One weight matrix reading the call's activations.  q_w [n, K] (int8 or E4M3
 * codes), s_w bf16 [n] (rowwise schemes) or [n/128, K/128] (block scheme; n % 128
 * == 0), y [M, n] in the call's output mode.  Host struct; pointers are device
 * memory. */
typedef struct qlin_segment {
    const void* q_w;
    const uint16_t* s_w;
    void* y;
    int64_t n;
} qlin_segment;

/* Quantize the bf16 activations x [M, K] with the scheme's dynamic rounding and
 * multiply them by each of the nseg (1..QLIN_MAX_SEGMENTS) weight segments:
 * segments[i].y = product of x with segments[i] (the definition of
 * qlin_gemm_w8a8 / qlin_gemm_fp8_rowwise / qlin_gemm_fp8_block applied to the
 * codes and scales of qlin_quant_act_int8 / qlin_quant_act_fp8).  Projections
 * that read the same layer input (q/k/v, gate/up) share one rounding of it
 * (W8A8 model card, intro and "Loading"; Qwen3 8B FP8 card, "Loading").
 *
 * M == 1 and K <= 16384: one launch -- every workgroup rounds the row into LDS
 * and streams its share of all segments' weight rows.  M == 2, K <= 16384
 * (FP8_BLOCK: K <= 8192) and at most 64 MiB of weights in the call: one launch
 * as well -- persistent workgroups round both tokens into LDS once and stream
 * the weight rows one at a time.  Otherwise 2 <= M <= 4 with K <= 4096: one
 * launch of the small-M matrix-core kernel, every workgroup rounding the
 * tokens into its LDS.  In these
 * one-launch cases q_x / s_x may be null, and when given receive the codes and
 * scale(s).  Otherwise q_x (M*K bytes) and s_x ([M] or [M, K/128] f32) are
 * required caller-owned staging buffers: one quantizer launch, then one product
 * launch covering every segment (regime by M).  The segments array is read
 * during the call only. */
qlin_status qlin_linear(qlin_scheme scheme, const uint16_t* x, int64_t M, int64_t K,
                        const qlin_segment* segments, int32_t nseg, qlin_out out,
                        void* q_x, float* s_x, hipStream_t stream);

/* Weight-only ("equivalent") numerics: the input is never rounded (W8A8 model
 * card and Qwen3 8B FP8 card, "Against bf16"; "Loading": the numerics option).
 * For each segment, with the codes and scales of the scheme's weights:
 *   W8A8, FP8_ROWWISE:  y[m, n] = s_w[n] * sum_k x[m, k] * q_w[n, k]
 *   FP8_BLOCK:          y[m, n] = sum_kb s_w[n/128, kb] * sum_{k in block kb} x[m, k] * q_w[n, k]
 * x bf16 [M, K] (16-byte aligned, K % 16 == 0; K % 128 == 0 for FP8_BLOCK),
 * 1 <= M <= 32 (larger M: QLIN_ERR_UNSUPPORTED), segments as for qlin_linear.
 * out: QLIN_OUT_BF16 (round to nearest even) or QLIN_OUT_F32; QLIN_OUT_I32 is
 * QLIN_ERR_UNSUPPORTED.  Products of the bf16 inputs and the codes are exact;
 * the sums are f32.  One launch for all segments: M == 1 with K <= 16384 streams
 * each weight byte once on the vector ALUs; otherwise the codes are widened to
 * bf16 in registers for the matrix cores.  Same validation, ownership and error
 * behaviour as qlin_linear. */
qlin_status qlin_linear_weight_only(qlin_scheme scheme, const uint16_t* x, int64_t M, int64_t K,
                                    const qlin_segment* segments, int32_t nseg, qlin_out out,
                                    hipStream_t stream);

/* Gate/up pair of a gated MLP with SwiGLU applied on the way out.  The pages
 * stop at the projections; this is the plain definition of the MLP of the
 * models their "Command line" sections run (Llama 3.1 8B, Qwen3 8B):
 *   g = x W_gate^T,  u = x W_up^T   -- each exactly as qlin_linear computes it
 *                                      (one shared rounding of x) and rounded
 *                                      to bf16 as qlin_linear would write it,
 *   h[m, j] = bf16( bf16(silu(g[m, j])) * u[m, j] ),  silu(t) = t / (1 + e^-t),
 * silu evaluated in f32 on the bf16 g.  h is the down projection's input
 * (qlin_linear rounds it for down in the down projection's own launch).
 *   gate_q_w, up_q_w: [I, K] codes of the scheme; gate_s_w, up_s_w: bf16 [I]
 *   (rowwise schemes) or [I/128, K/128] (block scheme; I % 128 == 0);
 *   h: bf16 [M, I], 16-byte aligned, written.
 * Same validation, q_x / s_x staging and dispatch as qlin_linear with the two
 * weights as segments: M == 1 with K <= 16384 is one launch in which each
 * wavefront streams a gate row and the up row with the same index; 2 <= M <= 4
 * with K <= 4096 is one launch of the small-M kernel rounding the tokens in
 * every workgroup (in both cases q_x / s_x are optional); otherwise a
 * quantizer launch, then one product launch.  The product tiles hold gate rows
 * and the matching up rows.  Neither g nor u is written to memory.  h may not overlap
 * x, q_x, s_x or either weight or scale array (QLIN_ERR_ALIAS). */
qlin_status qlin_linear_swiglu(qlin_scheme scheme, const uint16_t* x, int64_t M, int64_t K,
                               const void* gate_q_w, const uint16_t* gate_s_w,
                               const void* up_q_w, const uint16_t* up_s_w, int64_t I,
                               uint16_t* h, void* q_x, float* s_x, hipStream_t stream);

/* Weights in the matrix-core operand order ("packed"), for long inputs.
 * The pages give the product only for row-major codes (W8A8 model card,
 * "Loading": longer inputs are rounded per row and multiplied in int8 with
 * int32 sums); this is the same product with the weight bytes reordered so
 * that each wavefront of the tiled kernel loads its weight rows straight into
 * the matrix-core operand registers, 1 KB contiguous per load, and only the
 * tokens pass through LDS.  q_w [N, K] is cut into blocks of 32 rows and
 * K-slices of S bytes (S = 32 for W8A8, 64 for the E4M3 schemes); with H = S / 32:
 *   packed[((rb * (K / S) + s) * H + h) * 1024 + 16 l + b]
 *     = q_w[32 rb + l % 32][S s + (S / 2) (l / 32) + 16 h + b],   l < 64, b < 16
 * (a permutation of the N * K bytes).
 *
 * qlin_pack_weights: q_w row-major [N, K] codes in, q_w_packed [N * K bytes]
 * out (caller-owned device memory, 16-byte aligned, not overlapping q_w).
 * Any scheme (the block scheme's E4M3 codes take the FP8_ROWWISE layout);
 * N % 128 == 0 and K % 128 == 0 (else QLIN_ERR_SHAPE); N == 0 is a no-op.
 * One launch on stream; the scales are not touched (s_w keeps its layout:
 * per row, or [N/128][K/128] blocks). */
qlin_status qlin_pack_weights(qlin_scheme scheme, const void* q_w, int64_t N, int64_t K, void* q_w_packed,
                              hipStream_t stream);

/* qlin_linear on packed weights: every segments[i].q_w is the qlin_pack_weights
 * output of that segment's codes (s_w and y as for qlin_linear).  Same results
 * as qlin_linear bit for bit for W8A8 (same int32 sums, same epilogue order);
 * the FP8 schemes within the tolerance of the FP8 paths (f32 sums, another
 * summation order; the block scheme scales each 128-input block's partial sum
 * by s_x[m][kb] * s_w[n/128][kb] into the f32 accumulator, as qlin_linear
 * does, Qwen3 8B FP8 model card, "Loading").  For long inputs only: M >= 33
 * (smaller M: QLIN_ERR_UNSUPPORTED, the one-row and small-M kernels read
 * row-major weights), every segment's n % 128 == 0 and K % 128 == 0
 * (QLIN_ERR_SHAPE); q_x / s_x are required staging buffers as in the staged
 * qlin_linear (s_x [M][K/128] for the block scheme): one quantizer launch,
 * then one tiled launch over every segment (128 weight rows x 64 or 128 tokens
 * per tile).  Validation, aliasing rules and error behaviour as qlin_linear.
 * Packing pays on projections whose outputs give each CU at most a 128 x 128
 * tile (q/k/v, o and down of an 8B model at 512-1024 tokens); for W8A8 and
 * FP8_ROWWISE the wide gate/up projection runs as fast row-major, on the
 * 256 x 256 tiles of qlin_linear / qlin_linear_swiglu.  FP8_BLOCK has no such
 * row-major tile and is faster packed on every projection. */
qlin_status qlin_linear_packed(qlin_scheme scheme, const uint16_t* x, int64_t M, int64_t K,
                               const qlin_segment* segments, int32_t nseg, qlin_out out,
                               void* q_x, float* s_x, hipStream_t stream);

/* qlin_linear_swiglu on packed weights: gate_q_w_packed and up_q_w_packed are
 * the qlin_pack_weights outputs of the gate and up codes ([I, K] each); scales,
 * h and the result as for qlin_linear_swiglu (h = bf16(bf16(silu(g)) * u) with
 * g, u the projections rounded to bf16; W8A8 bit for bit with
 * qlin_linear_swiglu).  Long inputs only: M >= 33 (else QLIN_ERR_UNSUPPORTED),
 * I % 128 == 0 and K % 128 == 0 (QLIN_ERR_SHAPE); q_x / s_x staging required.
 * One quantizer launch, then one tiled launch whose tiles hold 64 gate rows and
 * the up rows with the same indices.  Validation, aliasing rules and error
 * behaviour as qlin_linear_swiglu. */
qlin_status qlin_linear_swiglu_packed(qlin_scheme scheme, const uint16_t* x, int64_t M, int64_t K,
                                      const void* gate_q_w_packed, const uint16_t* gate_s_w,
                                      const void* up_q_w_packed, const uint16_t* up_s_w, int64_t I,
                                      uint16_t* h, void* q_x, float* s_x, hipStream_t stream);

/* Staging capacity of qlin_linear_noalloc: activation codes (M * K bytes) and
 * activation scales (M or M * K/128 floats). */
#define QLIN_NOALLOC_MAX_CODE_BYTES  (16 << 20)
#define QLIN_NOALLOC_MAX_SCALES      (1 << 20)

/* qlin_linear for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same call with the same results, bit for bit, but the quantized-activation
 * staging buffers come from a fixed scratch array inside the library instead
 * of q_x / s_x arguments.  The array is a static device variable of
 * QLIN_NOALLOC_MAX_CODE_BYTES + 4 * QLIN_NOALLOC_MAX_SCALES bytes (20 MiB),
 * held on every GPU the library runs on until the process ends; its address
 * is looked up once per device, on the first call there.  Nothing is
 * allocated or freed, here or later.
 *   Calls whose staging exceeds the scratch (M * K > QLIN_NOALLOC_MAX_CODE_BYTES,
 *   or more than QLIN_NOALLOC_MAX_SCALES activation scales) return
 *   QLIN_ERR_TOO_LARGE before any launch; otherwise validation and errors are
 *   those of qlin_linear.  The stream's device must be the current device
 *   (QLIN_ERR_UNSUPPORTED otherwise).
 *   Every call on one GPU uses that GPU's one scratch array: two calls that
 *   may run at the same time on one GPU (different streams, or host threads
 *   enqueuing concurrently) race on it and give wrong results.  Calls in one
 *   stream are ordered and safe.  The scratch keeps the last call's codes; no
 *   call relies on its previous contents. */
qlin_status qlin_linear_noalloc(qlin_scheme scheme, const uint16_t* x, int64_t M, int64_t K,
                                const qlin_segment* segments, int32_t nseg, qlin_out out,
                                hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Helpers                                                                */
/* ---------------------------------------------------------------------- */

/* Static string naming a status value (never null). */
const char* qlin_status_string(qlin_status status);
/* QLIN_ABI_VERSION of the built library. */
int qlin_abi_version(void);
/* HIP error code of the last QLIN_ERR_HIP returned on this thread (0 if none). */
int qlin_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QLIN_H_ */
