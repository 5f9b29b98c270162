/*
 * qcast.h -- C ABI of the MI355X (gfx950) quantization-cast library.
 *
 * The operations are the memory-bound quantization casts of DeepSeek's
 * TileKernels quant/ module as the pages describe them:
 *   [WALK]  "DeepSeek开源TileKernels：用Python写的GPU算子逼近硬件性能上限"
 *           (itsolotime.com): quick start (per_token_cast(x, fmt='e4m3',
 *           num_per_channels=128) -> (out, out_sf)), §3.1 (CastInputConfig /
 *           CastOutputConfig, clamp_min_value), §3.2 (per-token cast kernel),
 *           §3.3 (SwiGLU fused with the per-token cast).
 *   [SPLIT] "TileKernels 与 DeepGEMM 的分界线：DeepSeek 开源内核栈的分工"
 *           (chatdocs.ruinique.com): §二 operator table (per_token_cast,
 *           per_block_cast, per_channel_cast (+transpose),
 *           swiglu_forward_and_per_token_cast), §四 A (E4M3 / E2M1 formats),
 *           §六 (where the casts sit in a MoE layer).
 *   [NEWS]  "刚刚！DeepSeek开源高性能GPU算子库TileKernels" (info.datadowell.com):
 *           item 2 (the quant/ module; SwiGLU fused with cast and transpose).
 *
 * What every cast computes, per scale group of elements x_i:
 *     amax   = max_i |x_i|
 *     a      = max(amax, floor)                      fp32
 *     sf     = a / fmt_max                           fp32, IEEE division
 *     sf_inv = 1 / sf                                fp32, IEEE division
 *     code_i = encode(x_i * sf_inv)                  fp32 product, then
 *              round to nearest (ties to even mantissa), saturating, sign kept
 * fmt_max is 448 for E4M3, 57344 for E5M2 and 6 for E2M1. The default floor
 * ([WALK] §3.1) is 1e-4f for E4M3 and 6 * 2^-126 for E2M1; the page names no
 * floor for E5M2, which takes the E4M3 one, 1e-4f. A clamp_min > 0 replaces
 * the default; clamp_min <= 0 (-inf included) keeps it; a NaN or +inf
 * clamp_min is rejected with QCAST_ERR_VALUE. Formats: OCP E4M3 ("fn") and
 * E5M2, OCP MX E2M1; E5M2 is in the format list of [SPLIT] §四 A.
 *
 * Conventions shared by every entry point:
 *  - Every data pointer is a DEVICE pointer on the current HIP device, owned
 *    (allocated and freed) by the caller. The library never allocates,
 *    frees, synchronizes or keeps a pointer after returning (its only device
 *    memory is a static array of QCAST_NOALLOC_SCRATCH_BYTES per GPU).
 *  - Tensors are row-major and contiguous. bf16 inputs are passed as raw
 *    16-bit patterns. Inputs must not overlap outputs.
 *  - Alignment: inputs and code outputs 16 bytes, scale outputs 4 bytes,
 *    the optional row weight 4 bytes, a clamp counter 8 bytes, a count
 *    workspace 128 bytes.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *    the default stream) and the call returns at once.
 *  - The return value is a qcast_status. Arguments are checked before any
 *    HIP call; on an error nothing is launched and no output is touched.
 *    QCAST_ERR_LAUNCH reports a failed launch (hipGetLastError).
 *  - rows == 0 (or an empty row) is valid and launches nothing.
 *  - Shapes past the kernels' 32-bit indexing return QCAST_ERR_SHAPE before
 *    any HIP call: rows * cols / group < 2^31 scale groups for the per-token
 *    casts; for the others, the limits stated with each entry point.
 *  - Calls on one stream are ordered; concurrent calls on different streams
 *    are independent (a count workspace is the caller's, and concurrent
 *    calls need different ones). The one piece of mutable device state the
 *    library holds is the count array of qcast_swiglu_per_token_noalloc.
 *  - Entry points may be called from several host threads at once: the
 *    library's host-side state (cached CU counts, the CU override, the
 *    measurement events of qcast_bench_time_next) is atomic or per thread.
 */
#ifndef QCAST_H
#define QCAST_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QCAST_ABI_VERSION 5

/* Bytes of the optional clamp-count workspace (count_ws) of the SwiGLU casts. */
#define QCAST_COUNT_WS_BYTES 8192

/* Bytes of the library's own device array that qcast_swiglu_per_token_noalloc
 * counts through (one per GPU, held until the process ends). */
#define QCAST_NOALLOC_SCRATCH_BYTES 8192

#ifndef QCAST_API
#define QCAST_API __attribute__((visibility("default")))
#endif

typedef enum {
  QCAST_OK = 0,
  QCAST_ERR_NULL = 1,   /* a required pointer is NULL */
  QCAST_ERR_SHAPE = 2,  /* negative size, sizes not divisible as required, or past the
                           32-bit indexing limits */
  QCAST_ERR_ALIGN = 3,  /* a pointer is not aligned as required */
  QCAST_ERR_FORMAT = 4, /* format not supported by this entry point */
  QCAST_ERR_GROUP = 5,  /* group / block size not supported */
  QCAST_ERR_LAUNCH = 6, /* the kernel launch failed */
  QCAST_ERR_DEVICE = 7, /* no usable HIP device */
  QCAST_ERR_VALUE = 8   /* a scalar argument is out of range (a NaN SwiGLU clamp, a NaN or
                           +inf clamp_min) */
} qcast_status;

/*
 * QCAST_FMT_E5M6 ([SPLIT] §二 per_token_cast_to_e5m6 / cast_back_e5m6; [NEWS]
 * item 2, a format between FP8 and FP16 for attention gradients). The pages
 * give no bit layout; it is read as the IEEE-like 12-bit format with a 5-bit
 * exponent (bias 15) and 6 mantissa bits -- the top 12 bits of an fp16
 * pattern -- maximum 65024, floor 1e-4, codes saturating. A row of codes is
 * a little-endian bit stream, column j in bits 12j .. 12j+11: two codes per
 * three bytes, [rows, cols/2*3] bytes.
 */
typedef enum {
  QCAST_FMT_E4M3 = 1,
  QCAST_FMT_E2M1 = 2,
  QCAST_FMT_E5M2 = 3,
  QCAST_FMT_E5M6 = 4
} qcast_fmt;

/*
 * Scale-factor layout options of the *_sf entry points (the cast config of
 * [WALK] §3.1 round_sf, and the layouts [SPLIT] §四 C says the casts write
 * directly for the FP8 GEMMs that consume them). Let groups = cols / group
 * and rows_pad = ceil(rows / 4) * 4 (16 bytes of 4-byte entries).
 *   0                        fp32 sf[rows][groups] (the plain entry points)
 *   QCAST_SF_ROUND_POW2      sf rounded UP to a power of two (at least
 *                            2^-126) before the codes are formed, so no value
 *                            saturates; codes use its exact inverse.
 *   QCAST_SF_COL_MAJOR       fp32 sf[groups][rows_pad]; the padding entries
 *                            are not written.
 *   QCAST_SF_PACKED_UE8M0    implies ROUND_POW2; each scale stored as its
 *                            biased exponent byte (UE8M0), 4 per uint32 along
 *                            the groups of a row, group 4j+i in byte i of
 *                            word j: uint32 [rows][groups/4], or with
 *                            COL_MAJOR uint32 [groups/4][rows_pad]. Requires
 *                            groups % 4 == 0.
 */
typedef enum {
  QCAST_SF_ROUND_POW2 = 1,
  QCAST_SF_COL_MAJOR = 2,
  QCAST_SF_PACKED_UE8M0 = 4
} qcast_sf_flags;

/*
 * The other casts take the same options where their scales have a per-token
 * row structure ([SPLIT] §四 C: the casts write the consumer's layout while
 * they quantize or re-arrange):
 *   - the SwiGLU backward (qcast_swiglu_backward_per_token_sf): the layouts
 *     of its code rows [dg | du], rows = rows, groups = 2*cols/group;
 *     packed needs (cols/group) % 4 == 0, so no word spans the two halves;
 *   - the transposed per-channel casts (qcast_per_channel_T_sf,
 *     qcast_swiglu_per_channel_T_sf): the layouts of the per-token cast of
 *     x^T, whose rows are the cols channels and whose groups are the
 *     rows/group token groups: fp32 sf[cols][rows/group], COL_MAJOR
 *     sf[rows/group][ceil(cols/4)*4], packed uint32 [cols][rows/group/4]
 *     or [rows/group/4][ceil(cols/4)*4]; packed needs (rows/group) % 4 == 0;
 *   - the per-block and input-layout per-channel casts (qcast_per_block_sf,
 *     qcast_per_channel_sf): QCAST_SF_ROUND_POW2 only (any other bit returns
 *     QCAST_ERR_FORMAT); their fp32 scale arrays keep their shapes.
 */

/* Output type of qcast_cast_back. */
typedef enum { QCAST_OUT_BF16 = 1, QCAST_OUT_F32 = 2 } qcast_out_dtype;

/*
 * Per-token cast ([WALK] quick start and §3.2; [SPLIT] §二 per_token_cast).
 * One scale per run of `group` consecutive elements of a row (the page's
 * num_per_channels).
 *   x     [rows, cols] bf16.
 *   fmt   QCAST_FMT_E4M3, QCAST_FMT_E5M2, QCAST_FMT_E2M1 or QCAST_FMT_E5M6.
 *   q     E4M3 / E5M2: [rows, cols] bytes.  E2M1: [rows, cols/2] bytes,
 *         column 2k in the low nibble of byte k and column 2k+1 in its high
 *         nibble.  E5M6: [rows, cols/2*3] bytes (see QCAST_FMT_E5M6).
 *   sf    [rows, cols/group] fp32.
 *   group 32, 64 or 128; cols % group == 0.
 *   clamp_min  <= 0 selects the format's default floor; NaN or +inf returns
 *              QCAST_ERR_VALUE.
 */
QCAST_API int qcast_per_token(const void* x, int64_t rows, int64_t cols, int fmt, int group,
                    float clamp_min, void* q, float* sf, void* stream);

/* qcast_per_token with a scale-factor layout (qcast_sf_flags); sf points to
 * float or uint32 storage of the layout's shape (4-byte aligned). */
QCAST_API int qcast_per_token_sf(const void* x, int64_t rows, int64_t cols, int fmt, int group,
                                 float clamp_min, int sf_flags, void* q, void* sf, void* stream);

/*
 * Per-token cast to packed FP4 E2M1 ([SPLIT] §四 A format list; [WALK] §3.1
 * float4_e2m1fn floor). Same as qcast_per_token with fmt = QCAST_FMT_E2M1.
 *   q_packed [rows, cols/2] bytes; sf [rows, cols/group] fp32.
 */
QCAST_API int qcast_e2m1(const void* x, int64_t rows, int64_t cols, int group, float clamp_min,
               uint8_t* q_packed, float* sf, void* stream);

/*
 * SwiGLU forward fused with the per-token cast ([WALK] §3.3; [SPLIT] §二
 * swiglu_forward_and_per_token_cast, §六 step 6).
 *   h          [rows, 2*cols] bf16: columns [0, cols) are the gate (the SiLU
 *              input), columns [cols, 2*cols) the up projection.
 *   row_weight [rows] fp32 routing weight, or NULL for none.
 *   v[r][j] = (g / (1 + exp(-g))) * u * row_weight[r], fp32, never rounded
 *   to bf16; then the per-token cast of v with `group`.
 *   q    codes of [rows, cols] values stored as qcast_per_token stores them
 *        for `fmt`; sf [rows, cols/group] fp32.
 *   fmt  any of the four formats ([SPLIT] §四 A lists E4M3 / E5M2 / E2M1 /
 *        E5M6 for this cast). The exponential and the division
 *   use the hardware's fast forms, so the codes may differ from an exact
 *   evaluation by one step where v lies next to a rounding midpoint.
 */
QCAST_API int qcast_swiglu_per_token(const void* h, int64_t rows, int64_t cols,
                                     const float* row_weight, int fmt, int group,
                                     float clamp_min, void* q, float* sf, void* stream);

/* qcast_swiglu_per_token with a scale-factor layout (qcast_sf_flags). */
QCAST_API int qcast_swiglu_per_token_sf(const void* h, int64_t rows, int64_t cols,
                                        const float* row_weight, int fmt, int group,
                                        float clamp_min, int sf_flags, void* q, void* sf,
                                        void* stream);

/*
 * SwiGLU forward with the optional clamp of [WALK] §3.3, fused with the
 * per-token cast and a scale-factor layout.
 *   swiglu_clamp  c > 0 replaces the gate g by min(g, c) and the up value u
 *                 by min(max(u, -c), c) before the product; c <= 0 (or
 *                 +inf) clamps nothing. NaN is rejected (QCAST_ERR_VALUE).
 *   clamp_count   NULL, or a device uint64 (8-byte aligned) to which the
 *                 number of gate and up values the clamp changed is ADDED
 *                 (atomically; the caller zeroes it, or lets it accumulate
 *                 over calls). Untouched when c <= 0.
 *   count_ws      NULL, or QCAST_COUNT_WS_BYTES of device memory (128-byte
 *                 aligned) that is all zero before the call; the call leaves
 *                 it all zero again once its kernels end. With it the
 *                 counting kernel spreads its atomics over the workspace and
 *                 runs the full grid (measured 20% faster on 8192 x 2048
 *                 outputs); without it, a capped grid adds into clamp_count
 *                 directly. Calls that may run at the same time (on
 *                 different streams) need different workspaces; calls in
 *                 order on one stream may share one. Ignored unless
 *                 clamp_count is given and c > 0.
 *   Everything else as qcast_swiglu_per_token_sf.
 */
QCAST_API int qcast_swiglu_per_token_ex(const void* h, int64_t rows, int64_t cols,
                                        const float* row_weight, int fmt, int group,
                                        float clamp_min, int sf_flags, float swiglu_clamp,
                                        void* q, void* sf, uint64_t* clamp_count,
                                        void* count_ws, void* stream);

/*
 * qcast_swiglu_per_token_ex for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same cast, with no count_ws argument. When it counts
 * (clamp_count given, swiglu_clamp > 0) the count slots live in a device
 * array of the library, QCAST_NOALLOC_SCRATCH_BYTES per GPU, that the call
 * first clears with a small kernel on `stream`; the call itself allocates
 * nothing. Every shape qcast_swiglu_per_token_ex takes fits that array (the
 * slots are reused by every slab of rows, so no call needs more than
 * QCAST_COUNT_WS_BYTES); a call that would need more returns
 * QCAST_ERR_SHAPE. All calls on one GPU share the array: calls that may
 * overlap on one GPU (on different streams, or from several threads without
 * ordering) race on it and their counts are undefined; calls in order on
 * one stream are safe. Results (codes, scales, count) equal those of
 * qcast_swiglu_per_token_ex with a workspace. Errors as that entry point;
 * QCAST_ERR_DEVICE if the array's device address cannot be obtained.
 */
QCAST_API int qcast_swiglu_per_token_noalloc(const void* h, int64_t rows, int64_t cols,
                                             const float* row_weight, int fmt, int group,
                                             float clamp_min, int sf_flags, float swiglu_clamp,
                                             void* q, void* sf, uint64_t* clamp_count,
                                             void* stream);

/*
 * SwiGLU backward fused with the per-token cast of the input gradient
 * ([SPLIT] §二 swiglu_backward_and_per_token_cast; §六 step 13). The pages
 * name the operation; the derivative is that of the forward of [WALK] §3.3:
 * with g, u the (clamped) gate and up values of h and dv the gradient of v,
 *   s = 1 / (1 + exp(-g)), silu = g * s, dsilu = s + silu * (1 - s),
 *   dg = (dv * w) * u * dsilu,  du = (dv * w) * silu        (fp32)
 * and dg = 0 where g > c, du = 0 where |u| > c when swiglu_clamp c > 0.
 *   h   [rows, 2*cols] bf16 (gate | up); dv [rows, cols] bf16;
 *   row_weight [rows] fp32 or NULL.
 *   q   the codes of the row [dg | du], one code row of 2*cols columns per
 *       row, stored as qcast_per_token stores them for `fmt`.
 *   sf  [rows, 2*cols/group] fp32 (the dg groups, then the du groups).
 *   fmt any of the four formats ([SPLIT] §四 A pairs the SwiGLU cast's
 *       formats with a matching backward); group 32, 64 or 128;
 *   cols % group == 0. The exponential and reciprocal are the hardware's fast
 *   forms (codes may differ by one step next to a rounding midpoint).
 */
QCAST_API int qcast_swiglu_backward_per_token(const void* h, const void* dv, int64_t rows,
                                              int64_t cols, const float* row_weight, int fmt,
                                              int group, float clamp_min, float swiglu_clamp,
                                              void* q, float* sf, void* stream);

/* qcast_swiglu_backward_per_token with a scale-factor layout (qcast_sf_flags
 * over the rows [dg | du]: groups = 2*cols/group, packed needs
 * (cols/group) % 4 == 0); sf is float or uint32 storage accordingly. */
QCAST_API int qcast_swiglu_backward_per_token_sf(const void* h, const void* dv, int64_t rows,
                                                 int64_t cols, const float* row_weight, int fmt,
                                                 int group, float clamp_min, int sf_flags,
                                                 float swiglu_clamp, void* q, void* sf,
                                                 void* stream);

/*
 * SwiGLU forward fused with the per-channel cast and the transpose ([NEWS]
 * item 2; the SwiGLU of [WALK] §3.3, the transposed per-channel layout of
 * qcast_per_channel_T).
 *   h   [rows, 2*cols] bf16 (gate | up), rows = tokens; row_weight as above.
 *   v   = SwiGLU values [rows, cols] (clamped as in qcast_swiglu_per_token_ex)
 *   qT  one code row of `rows` codes per channel c, holding the codes of
 *       v[0..rows-1][c] stored as qcast_per_token stores a row for `fmt`
 *       ([cols, rows] bytes for E4M3 / E5M2, [cols, rows/2] E2M1 with the
 *       even token in the low nibble, [cols, rows/2*3] E5M6).
 *   sf  [cols, rows/group] fp32, groups of `group` tokens of one channel.
 *   group must be 128; rows % group == 0; cols % 8 == 0; any format;
 *   clamp_count and count_ws as above.
 *   Limits: 256 * cols < 2^31, 64 * rows < 2^31 (96 * rows for E5M6).
 */
QCAST_API int qcast_swiglu_per_channel_T(const void* h, int64_t rows, int64_t cols,
                                         const float* row_weight, int fmt, int group,
                                         float clamp_min, float swiglu_clamp, void* qT, float* sf,
                                         uint64_t* clamp_count, void* count_ws, void* stream);

/* qcast_swiglu_per_channel_T with a scale-factor layout: the per-token
 * layouts of v^T (rows = the cols channels, groups = the rows/group token
 * groups; packed needs (rows/group) % 4 == 0). */
QCAST_API int qcast_swiglu_per_channel_T_sf(const void* h, int64_t rows, int64_t cols,
                                            const float* row_weight, int fmt, int group,
                                            float clamp_min, int sf_flags, float swiglu_clamp,
                                            void* qT, void* sf, uint64_t* clamp_count,
                                            void* count_ws, void* stream);

/*
 * Per-block cast of a weight ([SPLIT] §二 per_block_cast; [NEWS]
 * "刚刚！DeepSeek开源高性能GPU算子库TileKernels", item 2, per-block granularity).
 * One scale per block x block tile.
 *   x  [rows, cols] bf16; rows % block == 0 and cols % block == 0.
 *   q  codes stored as qcast_per_token stores them for `fmt` (any of the
 *      four formats: the TileKernels overview of "DeepSeek 的 GPU 内核帝国"
 *      lists FP8 / FP4 / E5M6 at per-block granularity);
 *   sf [rows/block, cols/block] fp32. block must be 128.
 *   Limits: (rows/128) * (cols/128) < 2^31 and 128 * cols < 2^31.
 */
QCAST_API int qcast_per_block(const void* x, int64_t rows, int64_t cols, int fmt, int block,
                              float clamp_min, void* q, float* sf, void* stream);

/* qcast_per_block with round_sf ([WALK] §3.1): sf_flags 0 or
 * QCAST_SF_ROUND_POW2 (each tile's scale rounded up to a power of two, the
 * codes formed with its exact inverse); sf keeps its fp32 shape. */
QCAST_API int qcast_per_block_sf(const void* x, int64_t rows, int64_t cols, int fmt, int block,
                                 float clamp_min, int sf_flags, void* q, float* sf,
                                 void* stream);

/*
 * Per-channel cast written transposed ([SPLIT] §二 per_channel_cast
 * (+transpose); it feeds the weight-gradient GEMMs of §三 / §六 steps 12, 15,
 * which contract over tokens).
 *   x   [rows, cols] bf16, rows = tokens, cols = channels.
 *   The scale groups run along tokens: group g of channel c is
 *   x[g*group .. g*group + group - 1][c].
 *   qT  one code row of `rows` codes per channel c, holding the codes of
 *       x[0..rows-1][c] stored as qcast_per_token stores a row for `fmt`
 *       ([cols, rows] bytes for E4M3 / E5M2: qT[c][t] is the code of x[t][c];
 *       [cols, rows/2] E2M1, even token in the low nibble; [cols, rows/2*3]
 *       E5M6).
 *   sf  [cols, rows/group] fp32.
 *   group must be 128; rows % group == 0; cols % 8 == 0; any format.
 *   Limits: 128 * cols < 2^31, 64 * rows < 2^31 (96 * rows for E5M6).
 */
QCAST_API int qcast_per_channel_T(const void* x, int64_t rows, int64_t cols, int fmt, int group,
                                  float clamp_min, void* qT, float* sf, void* stream);

/* qcast_per_channel_T with a scale-factor layout: the per-token layouts of
 * x^T (rows = the cols channels, groups = the rows/group token groups):
 * fp32 sf[cols][rows/group] or, COL_MAJOR, sf[rows/group][ceil(cols/4)*4];
 * packed uint32 [cols][rows/group/4] or [rows/group/4][ceil(cols/4)*4],
 * which needs (rows/group) % 4 == 0. */
QCAST_API int qcast_per_channel_T_sf(const void* x, int64_t rows, int64_t cols, int fmt,
                                     int group, float clamp_min, int sf_flags, void* qT,
                                     void* sf, void* stream);

/*
 * Per-channel cast in the input layout ([SPLIT] §二 per_channel_cast without
 * the transpose).
 *   x   [rows, cols] bf16, rows = tokens, cols = channels.
 *   q   codes of x in its own layout, stored as qcast_per_token stores them
 *       for `fmt` (for E4M3 / E5M2 q[t][c] is the code of x[t][c]).
 *   sf  [rows/group, cols] fp32: sf[g][c] is the scale of tokens
 *       g*group .. g*group + group - 1 of channel c.
 *   group must be 128; rows % group == 0; cols % 8 == 0; any format.
 *   Limits: 128 * cols < 2^31.
 */
QCAST_API int qcast_per_channel(const void* x, int64_t rows, int64_t cols, int fmt, int group,
                                float clamp_min, void* q, float* sf, void* stream);

/* qcast_per_channel with round_sf: sf_flags 0 or QCAST_SF_ROUND_POW2. */
QCAST_API int qcast_per_channel_sf(const void* x, int64_t rows, int64_t cols, int fmt, int group,
                                   float clamp_min, int sf_flags, void* q, float* sf,
                                   void* stream);

/*
 * cast_back: dequantize per-token codes ([SPLIT] §二 cast_back).
 *   out[r][c] = decode(q[r][c]) * sf[r][c/group], one fp32 product, rounded
 *   to bf16 (nearest even) when out_dtype is QCAST_OUT_BF16.
 *   q    codes as qcast_per_token writes them for `fmt` and `group` (any of
 *        the four formats; E5M6 is cast_back_e5m6 of [SPLIT] §二).
 *   sf   [rows, cols/group] fp32.
 *   out  [rows, cols] bf16 (QCAST_OUT_BF16) or fp32 (QCAST_OUT_F32).
 *   group 32, 64 or 128; cols % group == 0.
 */
QCAST_API int qcast_cast_back(const void* q, const float* sf, int64_t rows, int64_t cols, int fmt,
                              int group, int out_dtype, void* out, void* stream);

/* Human-readable name of a status code (static string). */
QCAST_API const char* qcast_status_str(int status);

/* QCAST_ABI_VERSION of the built library. */
QCAST_API int qcast_abi_version(void);

/*
 * Override the compute-unit count used to size the persistent grids
 * (the pages' config.py get_num_sms() override, [WALK] §1.2). 0 restores the
 * device's own count. Affects later launches only; results never depend on it.
 * The only grids sized by it are the capped ones of the counting SwiGLU casts
 * run without a count workspace (qcast_swiglu_per_token_ex and
 * qcast_swiglu_per_channel_T with clamp_count given, swiglu_clamp > 0 and
 * count_ws NULL); every other launch takes one workgroup per unit of work and
 * ignores it.
 */
QCAST_API void qcast_set_num_cus(int n);

#ifdef __cplusplus
}
#endif

#endif /* QCAST_H */
