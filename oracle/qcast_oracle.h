/*
 * qcast_oracle.h -- the CPU oracle's own interface.
 *
 * TEST INFRASTRUCTURE. This header and qcast_oracle.cpp are a plain, slow,
 * single-threaded restatement of what the quantization casts compute. Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no source with the GPU library and must never be used as a
 * fallback for it.
 *
 * All pointers are HOST pointers, row-major and contiguous. Inputs are bf16
 * bit patterns (uint16_t). Codes are bytes (E4M3, E5M2), packed nibbles
 * (E2M1: byte k of a row holds column 2k in its low nibble, 2k+1 in its high
 * nibble) or a little-endian bit stream of 12-bit codes (E5M6: column j in
 * bits 12j..12j+11 of the row, three bytes per column pair). Scales are fp32.
 *
 * Every cast returns ORACLE_OK or an error code; on an error nothing is
 * written.
 */
#ifndef QCAST_ORACLE_H
#define QCAST_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ORACLE_OK = 0,
  ORACLE_ERR_NULL = 1,
  ORACLE_ERR_SHAPE = 2,
  ORACLE_ERR_FORMAT = 4,
  ORACLE_ERR_GROUP = 5,
  ORACLE_ERR_FPENV = 7 /* FTZ/DAZ set or rounding mode not nearest */
};

enum { ORACLE_FMT_E4M3 = 1, ORACLE_FMT_E2M1 = 2, ORACLE_FMT_E5M2 = 3, ORACLE_FMT_E5M6 = 4 };
enum { ORACLE_OUT_BF16 = 1, ORACLE_OUT_F32 = 2 };
/* Scale-factor layout flags (see oracle_per_token_sf). */
enum { ORACLE_SF_ROUND_POW2 = 1, ORACLE_SF_COL_MAJOR = 2, ORACLE_SF_PACKED_UE8M0 = 4 };

int oracle_version(void);

/* ---- format codecs (one element at a time, and array forms) ---- */
/* Byte codes (E4M3, E5M2, E2M1; E5M6 is refused: NaN / 0 / nothing written). */
float oracle_decode(int fmt, uint8_t code);     /* NaN for E4M3 0x7F/0xFF */
uint8_t oracle_encode(int fmt, float y);        /* RNE, saturating, signed zero */
void oracle_encode_array(int fmt, const float* y, int64_t n, uint8_t* codes);
void oracle_decode_array(int fmt, const uint8_t* codes, int64_t n, float* out);
/* 16-bit codes, every format (E5M6: sign bit 11, exponent bits 6-10). */
float oracle_decode16(int fmt, uint16_t code);
uint16_t oracle_encode16(int fmt, float y);
void oracle_encode_array16(int fmt, const float* y, int64_t n, uint16_t* codes);
void oracle_decode_array16(int fmt, const uint16_t* codes, int64_t n, float* out);
/* e^x rounded to the nearest fp32 value (the exponential of SiLU). */
void oracle_exp_array(const float* x, int64_t n, float* out);
float oracle_format_max(int fmt);
float oracle_default_floor(int fmt);

/* Scale of one group: a = max(amax, floor); sf = a / fmt_max; sf_inv = 1/sf.
 * clamp_min <= 0 selects the format's default floor. */
int oracle_scale(int fmt, float amax, float clamp_min, float* sf, float* sf_inv);

/* ---- casts ---- */
/* x [rows, cols] bf16 -> q [rows, cols] (E4M3) or [rows, cols/2] (E2M1),
 * sf [rows, cols/group]. */
int oracle_per_token(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int group,
                     float clamp_min, uint8_t* q, float* sf);

/* h [rows, 2*cols] bf16 = [gate | up]; w [rows] fp32 or NULL.
 * v = (g / (1 + exp(-g))) * u (* w[r]) in fp32, then the per-token cast of v. */
int oracle_swiglu_per_token(const uint16_t* h, int64_t rows, int64_t cols, const float* w,
                            int fmt, int group, float clamp_min, uint8_t* q, float* sf);

/* The fp32 SwiGLU values alone: v [rows, cols]. */
int oracle_swiglu_values(const uint16_t* h, int64_t rows, int64_t cols, const float* w,
                         float* v);

/* Per-token cast of fp32 input values (used to check the SwiGLU path and the
 * dequantize/requantize round trip). */
int oracle_per_token_f32(const float* x, int64_t rows, int64_t cols, int fmt, int group,
                         float clamp_min, uint8_t* q, float* sf);

/* x [rows, cols] bf16; one scale per block x block tile: sf [rows/block, cols/block];
 * q like per_token. */
int oracle_per_block(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int block,
                     float clamp_min, uint8_t* q, float* sf);

/* x [rows (tokens), cols (channels)] bf16; the scale groups run along tokens:
 * group g of channel c is x[g*G .. g*G+G-1][c]. Output transposed:
 * qT [cols, rows] (E4M3) or [cols, rows/2] (E2M1), sf [cols, rows/group]. */
int oracle_per_channel_T(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int group,
                         float clamp_min, uint8_t* qT, float* sf);

/* Dequantize per-token codes: out[r][c] = decode(q[r][c]) * sf[r][c/group] (fp32). */
int oracle_dequant_per_token(const uint8_t* q, const float* sf, int64_t rows, int64_t cols,
                             int fmt, int group, float* out);

/* cast_back of per-token codes: the fp32 product decode(q) * sf, written as
 * fp32 (out_dtype ORACLE_OUT_F32, out is float*) or rounded to bf16 with
 * round-to-nearest-even (ORACLE_OUT_BF16, out is uint16_t* bit patterns). */
int oracle_cast_back(const uint8_t* q, const float* sf, int64_t rows, int64_t cols, int fmt,
                     int group, int out_dtype, void* out);

/* Per-token cast (fp32 values already widened from bf16, or SwiGLU values)
 * with the scale-factor options of a cast config:
 *   ORACLE_SF_ROUND_POW2   sf rounded up to the smallest power of two that is
 *                          >= sf and >= 2^-126; codes use 1 / that power.
 *   ORACLE_SF_COL_MAJOR    scales stored [cols/group][rows_pad] with
 *                          rows_pad = ceil(rows / 4) * 4; padding untouched.
 *   ORACLE_SF_PACKED_UE8M0 (implies ROUND_POW2) each scale stored as its
 *                          biased exponent byte, 4 per uint32 along the
 *                          groups of a row (group 4j + i in byte i of word j);
 *                          requires (cols/group) % 4 == 0. Row-major
 *                          [rows][cols/group/4], or with COL_MAJOR
 *                          [cols/group/4][rows_pad].
 * sf points to float or uint32 storage accordingly. */
int oracle_per_token_sf(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int group,
                        float clamp_min, int sf_flags, uint8_t* q, void* sf);
int oracle_swiglu_per_token_sf(const uint16_t* h, int64_t rows, int64_t cols, const float* w,
                               int fmt, int group, float clamp_min, int sf_flags, uint8_t* q,
                               void* sf);

/* The other casts with scale-factor options (the same ORACLE_SF_* bits):
 *  - per-block and per-channel (input layout): ORACLE_SF_ROUND_POW2 only;
 *    the scales keep their fp32 [rows/block, cols/block] and
 *    [rows/group, cols] shapes.
 *  - per-channel + transpose (plain and SwiGLU): the per-token layouts of
 *    x^T, whose rows are the cols channels and whose groups are the
 *    rows/group token groups: fp32 [cols][rows/group], COL_MAJOR
 *    [rows/group][ceil(cols/4)*4], PACKED_UE8M0 [cols][rows/group/4] or
 *    [rows/group/4][ceil(cols/4)*4] (requires (rows/group) % 4 == 0).
 *  - SwiGLU backward: the per-token layouts of the rows [dg | du] of
 *    2*cols values: groups per row 2*cols/group. */
int oracle_per_block_sf(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int block,
                        float clamp_min, int sf_flags, uint8_t* q, float* sf);
int oracle_per_channel_sf(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int group,
                          float clamp_min, int sf_flags, uint8_t* q, float* sf);
int oracle_per_channel_T_sf(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int group,
                            float clamp_min, int sf_flags, uint8_t* qT, void* sf);
int oracle_swiglu_per_channel_T_sf(const uint16_t* h, int64_t rows, int64_t cols, const float* w,
                                   int fmt, int group, float clamp_min, int sf_flags,
                                   float swiglu_clamp, uint8_t* qT, void* sf);
int oracle_swiglu_backward_per_token_sf(const uint16_t* h, const uint16_t* dv, int64_t rows,
                                        int64_t cols, const float* w, int fmt, int group,
                                        float clamp_min, int sf_flags, float swiglu_clamp,
                                        uint8_t* q, void* sf);

/* ---- SwiGLU variants and per-channel without transpose ---- */

/* SwiGLU values with the optional clamp of the walk-through page §3.3:
 * g' = min(g, c), u' = min(max(u, -c), c) for swiglu_clamp = c > 0 (no
 * clamp for c <= 0); *count (if not NULL) is increased by the number of gate
 * and up values the clamp changed. v [rows, cols]. */
int oracle_swiglu_values_ex(const uint16_t* h, int64_t rows, int64_t cols, const float* w,
                            float swiglu_clamp, float* v, uint64_t* count);

/* Forward SwiGLU (with clamp) + per-token cast with a scale layout. */
int oracle_swiglu_per_token_ex(const uint16_t* h, int64_t rows, int64_t cols, const float* w,
                               int fmt, int group, float clamp_min, int sf_flags,
                               float swiglu_clamp, uint8_t* q, void* sf, uint64_t* count);

/* SwiGLU backward values: dv [rows, cols] bf16 is the gradient of v; out
 * [rows, 2*cols] fp32 = [dg | du] with
 *   e = exp(-g'), s = 1 / (1 + e), silu = g' * s, dsilu = s + silu * (1 - s),
 *   dvw = dv * w, dg = dvw * u' * dsilu, du = dvw * silu,
 * where g', u' are the clamped values, and dg = 0 where g > c, du = 0 where
 * |u| > c (the clamp's derivative). */
int oracle_swiglu_backward_values(const uint16_t* h, const uint16_t* dv, int64_t rows,
                                  int64_t cols, const float* w, float swiglu_clamp, float* out);

/* SwiGLU backward + per-token cast of [dg | du]: q holds one code row of
 * 2*cols columns per row (any format, stored as the per-token cast stores
 * it), sf [rows, 2*cols/group]. */
int oracle_swiglu_backward_per_token(const uint16_t* h, const uint16_t* dv, int64_t rows,
                                     int64_t cols, const float* w, int fmt, int group,
                                     float clamp_min, float swiglu_clamp, uint8_t* q, float* sf);

/* Forward SwiGLU + per-channel cast written transposed (token groups of
 * `group`): qT [cols, rows], sf [cols, rows/group]. */
int oracle_swiglu_per_channel_T(const uint16_t* h, int64_t rows, int64_t cols, const float* w,
                                int fmt, int group, float clamp_min, float swiglu_clamp,
                                uint8_t* qT, float* sf);

/* Per-channel cast in the input layout: groups of `group` tokens of one
 * channel; q [rows, cols], sf [rows/group, cols]. */
int oracle_per_channel(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int group,
                       float clamp_min, uint8_t* q, float* sf);

/* fp32 -> bf16 bit pattern, round to nearest even (NaN kept quiet). */
uint16_t oracle_f32_to_bf16(float f);

#ifdef __cplusplus
}
#endif

#endif /* QCAST_ORACLE_H */
