/*
 * qcast_oracle.cpp -- CPU oracle for the TileKernels-style quantization casts.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load this library. It shares no
 * source with the GPU library (no headers, tables or helpers); the two meet
 * only on byte buffers produced by the seeded input generators.
 *
 * Sources (web pages; cited by title and section):
 *  [WALK]  "DeepSeek开源TileKernels：用Python写的GPU算子逼近硬件性能上限"
 *          (itsolotime.com), §3.1 quantization config, §3.2 per-token cast
 *          kernel, §3.3 SwiGLU fused with the cast.
 *  [SPLIT] "TileKernels 与 DeepGEMM 的分界线：DeepSeek 开源内核栈的分工"
 *          (chatdocs.ruinique.com), §二 operator table (per_token_cast,
 *          per_block_cast, per_channel_cast (+transpose),
 *          swiglu_forward_and_per_token_cast), §四 A (formats E4M3/E2M1).
 *  [NEWS]  "刚刚！DeepSeek开源高性能GPU算子库TileKernels", item 2 (quant/:
 *          per-token, per-block and per-channel granularities).
 * The number formats are the ones [WALK] §3.1 names, float8_e4m3fn and
 * float4_e2m1fn, plus E5M2 from the format list of [SPLIT] §四 A; their bit
 * layouts follow the OCP 8-bit floating point specification (E4M3, "fn": no
 * infinities, one NaN pattern per sign; E5M2: IEEE-like with infinities and
 * NaNs) and the OCP Microscaling specification (E2M1: no infinities, no NaN).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - rounding is to nearest, ties to the code with an even mantissa;
 *  - a magnitude at or beyond the format maximum saturates to it;
 *  - the sign of zero is kept (-0 and tiny negatives give the negative zero);
 *  - the floor is applied to the group abs-max before the division;
 *  - sf_inv is the fp32 reciprocal of sf, and the codes come from x * sf_inv
 *    ([WALK] §3.2 multiplies by the inverse scale);
 *  - SwiGLU values stay fp32 and are never rounded to bf16;
 *  - NaN inputs are not defined by the pages; this oracle maps them to the
 *    E4M3 NaN code and, for E2M1, to the saturated maximum (not graded);
 *  - [WALK] §3.1 gives floors for E4M3 and E2M1 only; E5M2, the other 8-bit
 *    format, takes the E4M3 floor 1e-4;
 *  - cast_back is the fp32 product decode(code) * sf, rounded to bf16 to
 *    nearest even when bf16 output is asked for;
 *  - round_sf ([WALK] §3.1) rounds sf UP to a power of two, so that no value
 *    saturates ([SPLIT] §一 says the quant ops take exponents with bit
 *    operations); a scale below 2^-126 becomes 2^-126;
 *  - the SwiGLU clamp counter counts every gate value and every up value the
 *    clamp changes; the backward of SwiGLU (named in [SPLIT] §二 and §六 step
 *    13, not written out on the pages) is the derivative of the forward, with
 *    zero gradient where a value was clamped; the fused SwiGLU + cast +
 *    transpose ([NEWS] item 2) is the per-channel cast of the SwiGLU values
 *    written transposed; per_channel_cast without transpose keeps the input
 *    layout and stores sf[group][channel];
 *  - E5M6 ([SPLIT] §二 per_token_cast_to_e5m6 / cast_back_e5m6, §四 A;
 *    [NEWS] item 2: a custom format between FP8 and FP16 for attention
 *    gradients) is read as the IEEE-like 12-bit format with a 5-bit exponent
 *    (bias 15) and 6 mantissa bits, maximum 65024, floor 1e-4, and its codes
 *    are stored as a little-endian bit stream (two per three bytes);
 *  - the layouts of [SPLIT] §四 C: "TMA-aligned column-major" stores the
 *    scales group-major with the row count padded to a multiple of 4 (16
 *    bytes of fp32 or of packed words); "packed UE8M0" stores each (power of
 *    two) scale as its biased exponent byte, 4 per 32-bit word along the
 *    groups of a row, lowest group in the lowest byte. The transposed
 *    per-channel casts write the layouts of the per-token cast of x^T (its
 *    rows are the channels), the SwiGLU backward those of its rows
 *    [dg | du]; the per-block and input-layout per-channel casts take
 *    round_sf only (their scale arrays have no per-token row structure).
 *
 *  - the exponential in SiLU ([WALK] §3.3) is exp(-g) rounded once to the
 *    nearest fp32 value (exp_f32 below), so the SwiGLU forms are a fixed
 *    sequence of correctly rounded fp32 operations.
 *
 * Pins (tests/test_oracle_*.py) hold every function to sources other than
 * itself; exp_f32 is pinned to a correctly rounded decimal exponential. The
 * GPU's SwiGLU kernels use the hardware exponential, so they are held to a
 * tolerance against these values, not to bit equality.
 *
 * Arithmetic discipline: plain C++ on one thread, fp32 where the method is
 * fp32 (the scale, the inverse, the scaled value, SwiGLU) with no
 * contraction, no fast-math, and denormals kept (checked at every entry).
 * The encoder is deliberately unlike a bit-trick: it searches a sorted table
 * of every representable magnitude and compares against exact midpoints.
 */
#include "qcast_oracle.h"

#include <cfloat>
#include <cmath>
#include <cstring>
#include <vector>
#include <xmmintrin.h>

namespace {

float f32_from_bits(uint32_t u) {
  float f;
  std::memcpy(&f, &u, sizeof f);
  return f;
}

/* A bf16 is the upper 16 bits of an fp32, so widening is exact. */
float bf16_value(uint16_t h) { return f32_from_bits(static_cast<uint32_t>(h) << 16); }

/* ------------------------------------------------------------------------ */
/* Formats                                                                   */
/* ------------------------------------------------------------------------ */

/* The non-negative finite values of a format, in code order. For every format
 * the codes 0..n-1 are ordered by magnitude, so index == code. */
struct FormatTable {
  int n = 0;                 /* number of non-negative finite codes */
  std::vector<double> value; /* value[code] */
  uint16_t sign_bit = 0;     /* bit that makes a code negative */
  uint16_t nan_code = 0;     /* positive NaN code, or the max code if none */
  int inf_code = -1;         /* positive infinity code, -1 if none */
  float max = 0.0f;          /* largest finite magnitude */
  float default_floor = 0.0f;
};

/* E4M3 "fn" (OCP FP8): s eeee mmm, exponent bias 7. Exponent field 0 holds
 * the subnormals m * 2^-9; fields 1..15 hold (1 + m/8) * 2^(e-7), except that
 * 0x7F / 0xFF are NaN. There is no infinity. */
double e4m3_magnitude(int code7) {
  const int e = (code7 >> 3) & 0xF;
  const int m = code7 & 0x7;
  if (e == 0) return std::ldexp(static_cast<double>(m), -9);
  return std::ldexp(1.0 + m / 8.0, e - 7);
}

/* E2M1 (OCP MX FP4): s ee m, exponent bias 1. Exponent field 0 holds the
 * subnormal m * 0.5; fields 1..3 hold (1 + m/2) * 2^(e-1). No NaN, no inf. */
double e2m1_magnitude(int code3) {
  const int e = (code3 >> 1) & 0x3;
  const int m = code3 & 0x1;
  if (e == 0) return 0.5 * m;
  return std::ldexp(1.0 + m / 2.0, e - 1);
}

FormatTable make_e4m3() {
  FormatTable t;
  t.n = 127; /* 0x00 .. 0x7E; 0x7F is NaN */
  t.value.resize(t.n);
  for (int c = 0; c < t.n; ++c) t.value[c] = e4m3_magnitude(c);
  t.sign_bit = 0x80;
  t.nan_code = 0x7F;
  t.max = static_cast<float>(t.value[t.n - 1]); /* 448 */
  /* [WALK] §3.1: clamp_min_value is 1e-4 for float8_e4m3fn; as an fp32 that is
   * the float nearest to 1e-4. */
  t.default_floor = 1e-4f;
  return t;
}

/* E5M2 (OCP FP8): s eeeee mm, exponent bias 15. Exponent field 0 holds the
 * subnormals m * 2^-16; fields 1..30 hold (1 + m/4) * 2^(e-15); field 31 is
 * infinity (m = 0) or NaN. */
double e5m2_magnitude(int code7) {
  const int e = (code7 >> 2) & 0x1F;
  const int m = code7 & 0x3;
  if (e == 0) return std::ldexp(static_cast<double>(m), -16);
  return std::ldexp(1.0 + m / 4.0, e - 15);
}

FormatTable make_e5m2() {
  FormatTable t;
  t.n = 124; /* 0x00 .. 0x7B; 0x7C is infinity, 0x7D..0x7F NaN */
  t.value.resize(t.n);
  for (int c = 0; c < t.n; ++c) t.value[c] = e5m2_magnitude(c);
  t.sign_bit = 0x80;
  t.nan_code = 0x7F;
  t.inf_code = 0x7C;
  t.max = static_cast<float>(t.value[t.n - 1]); /* 57344 */
  t.default_floor = 1e-4f;
  return t;
}

/* E5M6: s eeeee mmmmmm (12 bits), exponent bias 15, the same exponent field
 * as E5M2 and fp16 with six mantissa bits. The pages name the format and its
 * purpose (between FP8 and FP16 in precision, for attention gradients) but not
 * its bit layout; this reading takes the IEEE-like layout of the other 5-bit
 * exponent formats: field 0 holds the subnormals m * 2^-20, fields 1..30 hold
 * (1 + m/64) * 2^(e-15), field 31 is infinity (m = 0) or NaN. */
double e5m6_magnitude(int code11) {
  const int e = (code11 >> 6) & 0x1F;
  const int m = code11 & 0x3F;
  if (e == 0) return std::ldexp(static_cast<double>(m), -20);
  return std::ldexp(1.0 + m / 64.0, e - 15);
}

FormatTable make_e5m6() {
  FormatTable t;
  t.n = 0x7C0; /* 0x000 .. 0x7BF; 0x7C0 is infinity, 0x7C1..0x7FF NaN */
  t.value.resize(t.n);
  for (int c = 0; c < t.n; ++c) t.value[c] = e5m6_magnitude(c);
  t.sign_bit = 0x800;
  t.nan_code = 0x7FF;
  t.inf_code = 0x7C0;
  t.max = static_cast<float>(t.value[t.n - 1]); /* 65024 */
  t.default_floor = 1e-4f;
  return t;
}

FormatTable make_e2m1() {
  FormatTable t;
  t.n = 8;
  t.value.resize(t.n);
  for (int c = 0; c < t.n; ++c) t.value[c] = e2m1_magnitude(c);
  t.sign_bit = 0x08;
  t.nan_code = 0x07;
  t.max = static_cast<float>(t.value[t.n - 1]); /* 6 */
  /* [WALK] §3.1: for float4_e2m1fn the floor is the format maximum times
   * 2^-126, which puts sf = floor / max at the fp32 normal boundary. */
  t.default_floor = static_cast<float>(std::ldexp(6.0, -126));
  return t;
}

const FormatTable* table_for(int fmt) {
  static const FormatTable e4m3 = make_e4m3();
  static const FormatTable e2m1 = make_e2m1();
  static const FormatTable e5m2 = make_e5m2();
  static const FormatTable e5m6 = make_e5m6();
  if (fmt == ORACLE_FMT_E5M6) return &e5m6;
  if (fmt == ORACLE_FMT_E4M3) return &e4m3;
  if (fmt == ORACLE_FMT_E2M1) return &e2m1;
  if (fmt == ORACLE_FMT_E5M2) return &e5m2;
  return nullptr;
}

/* Encode an fp32 value: nearest representable magnitude, ties to the even
 * code, saturating at the maximum, sign attached afterwards. Comparisons are
 * made in double, where every table value, every midpoint and every fp32 is
 * exact. */
uint16_t encode(const FormatTable& t, float y) {
  if (std::isnan(y)) return t.nan_code;
  const bool negative = std::signbit(y);
  const double a = std::fabs(static_cast<double>(y));
  int code;
  if (a >= t.value[t.n - 1]) {
    code = t.n - 1;
  } else {
    int lo = 0, hi = t.n - 1; /* invariant: value[lo] <= a < value[hi] */
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (t.value[mid] <= a) lo = mid; else hi = mid;
    }
    const double midpoint = 0.5 * (t.value[lo] + t.value[hi]);
    if (a < midpoint) code = lo;
    else if (a > midpoint) code = hi;
    else code = (lo % 2 == 0) ? lo : hi;
  }
  return static_cast<uint16_t>(code | (negative ? t.sign_bit : 0));
}

float decode(const FormatTable& t, uint16_t code) {
  const uint16_t magnitude_code = code & static_cast<uint16_t>(t.sign_bit - 1);
  const bool negative = (code & t.sign_bit) != 0;
  if (magnitude_code == t.inf_code) return negative ? -HUGE_VALF : HUGE_VALF;
  if (magnitude_code >= t.n) return std::nanf("");
  const float v = static_cast<float>(t.value[magnitude_code]);
  return negative ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Floating-point environment                                                */
/* ------------------------------------------------------------------------ */

/* The fp32 steps must run with denormals kept and round-to-nearest. MXCSR bit
 * 15 is flush-to-zero, bit 6 denormals-are-zero, bits 13-14 the rounding
 * control. */
bool fp_env_ok() {
  const unsigned csr = _mm_getcsr();
  return (csr & 0x8000u) == 0 && (csr & 0x0040u) == 0 && (csr & 0x6000u) == 0;
}

/* ------------------------------------------------------------------------ */
/* Exponential                                                               */
/* ------------------------------------------------------------------------ */

/* e^x rounded to the nearest fp32 value. The double exponential lies within
 * about one double ulp of e^x, so rounding it to fp32 picks the correctly
 * rounded value unless it sits next to a midpoint between two fp32 values.
 * There (within 2^-45 relative, which happens for 370 of the 2^32 inputs)
 * the 64-bit-mantissa expl decides; over every fp32 input, the closest any
 * double result comes to a midpoint is 2^-53 relative, about 2^11 expl ulps.
 * 2^128 stands for the value after FLT_MAX: a result rounded up to it
 * overflows to infinity. */
float exp_f32(float x) {
  const double d = std::exp(static_cast<double>(x));
  const float f = static_cast<float>(d);
  if (static_cast<double>(f) == d) return f; /* exact: x == 0, or +inf / 0 limits */
  double lo, hi; /* the two fp32 values (or 2^128) around d */
  if (static_cast<double>(f) < d) {
    lo = f;
    hi = (f == FLT_MAX) ? 0x1p128 : nextafterf(f, INFINITY);
  } else {
    hi = std::isinf(f) ? 0x1p128 : static_cast<double>(f);
    lo = std::isinf(f) ? FLT_MAX : nextafterf(f, 0.0f);
  }
  const double mid = 0.5 * (lo + hi); /* exact */
  if (std::fabs(d - mid) > 0x1p-45 * mid) return f;
  const long double e = expl(static_cast<long double>(x));
  const double pick = (e > static_cast<long double>(mid)) ? hi : lo;
  return pick == 0x1p128 ? INFINITY : static_cast<float>(pick);
}

/* ------------------------------------------------------------------------ */
/* Scale ([WALK] §3.1 clamp_min_value, §3.2 get_sf_and_inv)                  */
/* ------------------------------------------------------------------------ */

struct Scale {
  float sf;
  float sf_inv;
};

float floor_for(const FormatTable& t, float clamp_min) {
  /* [WALK] §3.1: a custom clamp value, when given, replaces the default. */
  return clamp_min > 0.0f ? clamp_min : t.default_floor;
}

Scale scale_from_amax(const FormatTable& t, float amax, float floor) {
  const float a = (amax < floor) ? floor : amax;
  Scale s;
  s.sf = a / t.max;
  s.sf_inv = 1.0f / s.sf;
  return s;
}

/* ------------------------------------------------------------------------ */
/* Code storage                                                              */
/* ------------------------------------------------------------------------ */

/* Formats whose codes are packed two columns at a time (whole bytes per
 * column pair), so rows need an even number of columns. */
bool pairs(int fmt) { return fmt == ORACLE_FMT_E2M1 || fmt == ORACLE_FMT_E5M6; }

/* Bytes of one row of codes with `cols` columns. */
int64_t code_row_bytes(int fmt, int64_t cols) {
  if (fmt == ORACLE_FMT_E2M1) return cols / 2;
  if (fmt == ORACLE_FMT_E5M6) return cols / 2 * 3;
  return cols;
}

/* Store a code at (row, col) of an output with `cols` logical columns. The
 * 8-bit formats take a byte per code; E2M1 packs column 2k into the low
 * nibble and 2k+1 into the high nibble of byte k of the row; E5M6 writes the
 * row as a little-endian bit stream of 12-bit codes (column j in bits
 * 12j .. 12j+11, lowest bit first: two codes per three bytes). */
void put_code(int fmt, uint8_t* q, int64_t cols, int64_t row, int64_t col, uint16_t code) {
  if (fmt == ORACLE_FMT_E5M6) {
    uint8_t* r = q + row * code_row_bytes(fmt, cols);
    for (int b = 0; b < 12; ++b) {
      const int64_t bit = 12 * col + b;
      const uint8_t mask = static_cast<uint8_t>(1u << (bit % 8));
      if ((code >> b) & 1u) r[bit / 8] |= mask;
      else r[bit / 8] &= static_cast<uint8_t>(~mask);
    }
  } else if (fmt != ORACLE_FMT_E2M1) {
    q[row * cols + col] = static_cast<uint8_t>(code);
  } else {
    uint8_t& b = q[row * (cols / 2) + col / 2];
    if (col % 2 == 0) b = static_cast<uint8_t>((b & 0xF0) | (code & 0x0F));
    else b = static_cast<uint8_t>((b & 0x0F) | ((code & 0x0F) << 4));
  }
}

uint16_t get_code(int fmt, const uint8_t* q, int64_t cols, int64_t row, int64_t col) {
  if (fmt == ORACLE_FMT_E5M6) {
    const uint8_t* r = q + row * code_row_bytes(fmt, cols);
    uint16_t code = 0;
    for (int b = 0; b < 12; ++b) {
      const int64_t bit = 12 * col + b;
      code = static_cast<uint16_t>(code | (((r[bit / 8] >> (bit % 8)) & 1u) << b));
    }
    return code;
  }
  if (fmt != ORACLE_FMT_E2M1) return q[row * cols + col];
  const uint8_t b = q[row * (cols / 2) + col / 2];
  return (col % 2 == 0) ? (b & 0x0F) : (b >> 4);
}

/* Common checks for a per-token style cast. */
int check_common(const void* a, const void* b, const void* c, int fmt, int group) {
  if (!a || !b || !c) return ORACLE_ERR_NULL;
  if (!table_for(fmt)) return ORACLE_ERR_FORMAT;
  if (group <= 0) return ORACLE_ERR_GROUP;
  if (!fp_env_ok()) return ORACLE_ERR_FPENV;
  return ORACLE_OK;
}

/* The smallest power of two that is >= sf and >= 2^-126 (round_sf). */
float round_up_pow2(float sf) {
  if (sf <= std::ldexp(1.0f, -126)) return std::ldexp(1.0f, -126);
  int e = 0;
  const float m = std::frexp(sf, &e); /* sf = m * 2^e, m in [0.5, 1) */
  return (m == 0.5f) ? sf : std::ldexp(1.0f, e);
}

/* Biased exponent of a normal power of two (its UE8M0 byte). */
uint8_t ue8m0_of(float pow2) {
  int e = 0;
  std::frexp(pow2, &e); /* pow2 = 0.5 * 2^e */
  return static_cast<uint8_t>(e - 1 + 127);
}

/* Per-token cast of rows of fp32 values ([WALK] §3.2): for each row and each
 * run of `group` columns, the abs-max, the scale, then every element times
 * the inverse scale, encoded. */
void per_token_rows(const float* x, int64_t rows, int64_t cols, int fmt, int group, float floor,
                    uint8_t* q, float* sf) {
  const FormatTable& t = *table_for(fmt);
  const int64_t groups = cols / group;
  for (int64_t r = 0; r < rows; ++r) {
    const float* xr = x + r * cols;
    for (int64_t k = 0; k < groups; ++k) {
      float amax = 0.0f;
      for (int64_t i = 0; i < group; ++i) {
        const float m = std::fabs(xr[k * group + i]);
        if (m > amax) amax = m;
      }
      const Scale s = scale_from_amax(t, amax, floor);
      for (int64_t i = 0; i < group; ++i) {
        const int64_t c = k * group + i;
        const float y = xr[c] * s.sf_inv;
        put_code(fmt, q, cols, r, c, encode(t, y));
      }
      sf[r * groups + k] = s.sf;
    }
  }
}

/* Per-token cast of one row of fp32 values with the scale-factor options;
 * stores the scales of row r into the chosen layout. */
void per_token_row_sf(const float* xr, int64_t r, int64_t rows, int64_t cols, int fmt, int group,
                      float floor, int flags, uint8_t* qr, void* sf) {
  const FormatTable& t = *table_for(fmt);
  const int64_t groups = cols / group;
  const int64_t rows_pad = (rows + 3) / 4 * 4;
  const bool round = (flags & (ORACLE_SF_ROUND_POW2 | ORACLE_SF_PACKED_UE8M0)) != 0;
  for (int64_t k = 0; k < groups; ++k) {
    float amax = 0.0f;
    for (int64_t i = 0; i < group; ++i) {
      const float m = std::fabs(xr[k * group + i]);
      if (m > amax) amax = m;
    }
    Scale s = scale_from_amax(t, amax, floor);
    if (round) {
      s.sf = round_up_pow2(s.sf);
      s.sf_inv = 1.0f / s.sf;
    }
    for (int64_t i = 0; i < group; ++i) {
      const int64_t c = k * group + i;
      put_code(fmt, qr, cols, 0, c, encode(t, xr[c] * s.sf_inv));
    }
    if (flags & ORACLE_SF_PACKED_UE8M0) {
      uint32_t* words = static_cast<uint32_t*>(sf);
      const int64_t word = (flags & ORACLE_SF_COL_MAJOR) ? (k / 4) * rows_pad + r
                                                         : r * (groups / 4) + k / 4;
      const int shift = 8 * static_cast<int>(k % 4);
      words[word] = (words[word] & ~(0xFFu << shift)) |
                    (static_cast<uint32_t>(ue8m0_of(s.sf)) << shift);
    } else {
      float* f = static_cast<float*>(sf);
      f[(flags & ORACLE_SF_COL_MAJOR) ? k * rows_pad + r : r * groups + k] = s.sf;
    }
  }
}

/* Per-channel cast of an fp32 matrix x [rows, cols]: groups of `group`
 * tokens of one channel. transposed: code of x[t][c] at q[c][t], scale at
 * sf[c][g]; otherwise at q[t][c] and sf[g][c]. round: sf rounded up to a
 * power of two (round_sf), codes from its inverse. */
void per_channel_f32(const float* x, int64_t rows, int64_t cols, int fmt, int group, float floor,
                     bool transposed, bool round, uint8_t* q, float* sf) {
  const FormatTable& t = *table_for(fmt);
  const int64_t groups = rows / group;
  for (int64_t c = 0; c < cols; ++c) {
    for (int64_t g = 0; g < groups; ++g) {
      float amax = 0.0f;
      for (int64_t tk = g * group; tk < (g + 1) * group; ++tk) {
        const float m = std::fabs(x[tk * cols + c]);
        if (m > amax) amax = m;
      }
      Scale s = scale_from_amax(t, amax, floor);
      if (round) {
        s.sf = round_up_pow2(s.sf);
        s.sf_inv = 1.0f / s.sf;
      }
      for (int64_t tk = g * group; tk < (g + 1) * group; ++tk) {
        const uint16_t code = encode(t, x[tk * cols + c] * s.sf_inv);
        if (transposed) put_code(fmt, q, rows, c, tk, code);
        else put_code(fmt, q, cols, tk, c, code);
      }
      if (transposed) sf[c * groups + g] = s.sf;
      else sf[g * cols + c] = s.sf;
    }
  }
}

/* SwiGLU of one row with the clamp of [WALK] §3.3. */
void swiglu_row(const uint16_t* hr, int64_t cols, float wr, bool weighted, float clamp,
                float* v, uint64_t* count) {
  for (int64_t j = 0; j < cols; ++j) {
    float g = bf16_value(hr[j]);
    float u = bf16_value(hr[cols + j]);
    if (clamp > 0.0f) {
      if (g > clamp) { g = clamp; if (count) ++*count; }
      if (u > clamp) { u = clamp; if (count) ++*count; }
      else if (u < -clamp) { u = -clamp; if (count) ++*count; }
    }
    const float silu = g / (1.0f + exp_f32(-g));
    float val = silu * u;
    if (weighted) val = val * wr;
    v[j] = val;
  }
}

int check_sf_flags(int flags, int64_t cols, int group) {
  if (flags & ~(ORACLE_SF_ROUND_POW2 | ORACLE_SF_COL_MAJOR | ORACLE_SF_PACKED_UE8M0))
    return ORACLE_ERR_FORMAT;
  if ((flags & ORACLE_SF_PACKED_UE8M0) && (cols / group) % 4 != 0) return ORACLE_ERR_SHAPE;
  return ORACLE_OK;
}

/* The transposed per-channel cast with a scale layout is the per-token cast
 * of x^T: channel c of the fp32 matrix x [rows, cols] is row c of x^T, a
 * row of `rows` tokens, and the layout's rows are the channels. */
void per_channel_T_sf_f32(const float* x, int64_t rows, int64_t cols, int fmt, int group,
                          float floor, int flags, uint8_t* qT, void* sf) {
  std::vector<float> col(static_cast<size_t>(rows));
  const int64_t code_bytes = code_row_bytes(fmt, rows);
  for (int64_t c = 0; c < cols; ++c) {
    for (int64_t tk = 0; tk < rows; ++tk) col[tk] = x[tk * cols + c];
    per_token_row_sf(col.data(), c, cols, rows, fmt, group, floor, flags, qT + c * code_bytes, sf);
  }
}

} /* namespace */

/* ======================================================================== */
/* Exported functions                                                        */
/* ======================================================================== */

extern "C" {

int oracle_version(void) { return 1; }

void oracle_exp_array(const float* x, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = exp_f32(x[i]);
}

/* The byte forms serve the formats whose codes fit a byte; E5M6 codes go
 * through the 16-bit forms. */
const FormatTable* byte_table_for(int fmt) {
  return fmt == ORACLE_FMT_E5M6 ? nullptr : table_for(fmt);
}

float oracle_decode(int fmt, uint8_t code) {
  const FormatTable* t = byte_table_for(fmt);
  return t ? decode(*t, code) : std::nanf("");
}

uint8_t oracle_encode(int fmt, float y) {
  const FormatTable* t = byte_table_for(fmt);
  return t ? static_cast<uint8_t>(encode(*t, y)) : 0;
}

void oracle_encode_array(int fmt, const float* y, int64_t n, uint8_t* codes) {
  const FormatTable* t = byte_table_for(fmt);
  if (!t) return;
  for (int64_t i = 0; i < n; ++i) codes[i] = static_cast<uint8_t>(encode(*t, y[i]));
}

void oracle_decode_array(int fmt, const uint8_t* codes, int64_t n, float* out) {
  const FormatTable* t = byte_table_for(fmt);
  if (!t) return;
  for (int64_t i = 0; i < n; ++i) out[i] = decode(*t, codes[i]);
}

float oracle_decode16(int fmt, uint16_t code) {
  const FormatTable* t = table_for(fmt);
  return t ? decode(*t, code) : std::nanf("");
}

uint16_t oracle_encode16(int fmt, float y) {
  const FormatTable* t = table_for(fmt);
  return t ? encode(*t, y) : 0;
}

void oracle_encode_array16(int fmt, const float* y, int64_t n, uint16_t* codes) {
  const FormatTable* t = table_for(fmt);
  if (!t) return;
  for (int64_t i = 0; i < n; ++i) codes[i] = encode(*t, y[i]);
}

void oracle_decode_array16(int fmt, const uint16_t* codes, int64_t n, float* out) {
  const FormatTable* t = table_for(fmt);
  if (!t) return;
  for (int64_t i = 0; i < n; ++i) out[i] = decode(*t, codes[i]);
}

float oracle_format_max(int fmt) {
  const FormatTable* t = table_for(fmt);
  return t ? t->max : 0.0f;
}

float oracle_default_floor(int fmt) {
  const FormatTable* t = table_for(fmt);
  return t ? t->default_floor : 0.0f;
}

int oracle_scale(int fmt, float amax, float clamp_min, float* sf, float* sf_inv) {
  const FormatTable* t = table_for(fmt);
  if (!t) return ORACLE_ERR_FORMAT;
  if (!sf || !sf_inv) return ORACLE_ERR_NULL;
  if (!fp_env_ok()) return ORACLE_ERR_FPENV;
  const Scale s = scale_from_amax(*t, amax, floor_for(*t, clamp_min));
  *sf = s.sf;
  *sf_inv = s.sf_inv;
  return ORACLE_OK;
}

int oracle_per_token_f32(const float* x, int64_t rows, int64_t cols, int fmt, int group,
                         float clamp_min, uint8_t* q, float* sf) {
  const int rc = check_common(x, q, sf, fmt, group);
  if (rc != ORACLE_OK) return rc;
  if (rows < 0 || cols < 0 || cols % group != 0) return ORACLE_ERR_SHAPE;
  if (pairs(fmt) && group % 2 != 0) return ORACLE_ERR_GROUP;
  per_token_rows(x, rows, cols, fmt, group, floor_for(*table_for(fmt), clamp_min), q, sf);
  return ORACLE_OK;
}

int oracle_per_token(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int group,
                     float clamp_min, uint8_t* q, float* sf) {
  const int rc = check_common(x, q, sf, fmt, group);
  if (rc != ORACLE_OK) return rc;
  if (rows < 0 || cols < 0 || cols % group != 0) return ORACLE_ERR_SHAPE;
  if (pairs(fmt) && group % 2 != 0) return ORACLE_ERR_GROUP;
  const float floor = floor_for(*table_for(fmt), clamp_min);
  std::vector<float> row(static_cast<size_t>(cols));
  const int64_t code_bytes = code_row_bytes(fmt, cols);
  const int64_t groups = cols / group;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) row[c] = bf16_value(x[r * cols + c]);
    per_token_rows(row.data(), 1, cols, fmt, group, floor, q + r * code_bytes, sf + r * groups);
  }
  return ORACLE_OK;
}

int oracle_swiglu_values(const uint16_t* h, int64_t rows, int64_t cols, const float* w,
                         float* v) {
  return oracle_swiglu_values_ex(h, rows, cols, w, 0.0f, v, nullptr);
}

int oracle_swiglu_values_ex(const uint16_t* h, int64_t rows, int64_t cols, const float* w,
                            float swiglu_clamp, float* v, uint64_t* count) {
  if (!h || !v) return ORACLE_ERR_NULL;
  if (rows < 0 || cols < 0) return ORACLE_ERR_SHAPE;
  if (!fp_env_ok()) return ORACLE_ERR_FPENV;
  /* [WALK] §3.3: the left half is the SiLU input, the right half multiplies
   * it; SiLU is written g / (1 + exp(-g)); the routing weight multiplies last.
   * All in fp32. */
  for (int64_t r = 0; r < rows; ++r)
    swiglu_row(h + r * 2 * cols, cols, w ? w[r] : 1.0f, w != nullptr, swiglu_clamp,
               v + r * cols, count);
  return ORACLE_OK;
}

int oracle_swiglu_per_token(const uint16_t* h, int64_t rows, int64_t cols, const float* w,
                            int fmt, int group, float clamp_min, uint8_t* q, float* sf) {
  const int rc = check_common(h, q, sf, fmt, group);
  if (rc != ORACLE_OK) return rc;
  if (rows < 0 || cols < 0 || cols % group != 0) return ORACLE_ERR_SHAPE;
  if (pairs(fmt) && group % 2 != 0) return ORACLE_ERR_GROUP;
  const float floor = floor_for(*table_for(fmt), clamp_min);
  std::vector<float> v(static_cast<size_t>(cols));
  const int64_t code_bytes = code_row_bytes(fmt, cols);
  const int64_t groups = cols / group;
  for (int64_t r = 0; r < rows; ++r) {
    oracle_swiglu_values(h + r * 2 * cols, 1, cols, w ? w + r : nullptr, v.data());
    per_token_rows(v.data(), 1, cols, fmt, group, floor, q + r * code_bytes, sf + r * groups);
  }
  return ORACLE_OK;
}

int oracle_per_block(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int block,
                     float clamp_min, uint8_t* q, float* sf) {
  return oracle_per_block_sf(x, rows, cols, fmt, block, clamp_min, 0, q, sf);
}

int oracle_per_block_sf(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int block,
                        float clamp_min, int sf_flags, uint8_t* q, float* sf) {
  const int rc = check_common(x, q, sf, fmt, block);
  if (rc != ORACLE_OK) return rc;
  if (sf_flags & ~ORACLE_SF_ROUND_POW2) return ORACLE_ERR_FORMAT;
  if (rows < 0 || cols < 0 || rows % block != 0 || cols % block != 0) return ORACLE_ERR_SHAPE;
  if (pairs(fmt) && block % 2 != 0) return ORACLE_ERR_GROUP;
  const FormatTable& t = *table_for(fmt);
  const float floor = floor_for(t, clamp_min);
  const int64_t brows = rows / block, bcols = cols / block;
  for (int64_t bi = 0; bi < brows; ++bi) {
    for (int64_t bj = 0; bj < bcols; ++bj) {
      float amax = 0.0f;
      for (int64_t r = bi * block; r < (bi + 1) * block; ++r)
        for (int64_t c = bj * block; c < (bj + 1) * block; ++c) {
          const float m = std::fabs(bf16_value(x[r * cols + c]));
          if (m > amax) amax = m;
        }
      Scale s = scale_from_amax(t, amax, floor);
      if (sf_flags & ORACLE_SF_ROUND_POW2) {
        s.sf = round_up_pow2(s.sf);
        s.sf_inv = 1.0f / s.sf;
      }
      for (int64_t r = bi * block; r < (bi + 1) * block; ++r)
        for (int64_t c = bj * block; c < (bj + 1) * block; ++c) {
          const float y = bf16_value(x[r * cols + c]) * s.sf_inv;
          put_code(fmt, q, cols, r, c, encode(t, y));
        }
      sf[bi * bcols + bj] = s.sf;
    }
  }
  return ORACLE_OK;
}

int oracle_per_channel_T(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int group,
                         float clamp_min, uint8_t* qT, float* sf) {
  const int rc = check_common(x, qT, sf, fmt, group);
  if (rc != ORACLE_OK) return rc;
  if (rows < 0 || cols < 0 || rows % group != 0) return ORACLE_ERR_SHAPE;
  if (pairs(fmt) && group % 2 != 0) return ORACLE_ERR_GROUP;
  std::vector<float> xf(static_cast<size_t>(rows * cols));
  for (int64_t i = 0; i < rows * cols; ++i) xf[i] = bf16_value(x[i]);
  per_channel_f32(xf.data(), rows, cols, fmt, group, floor_for(*table_for(fmt), clamp_min), true,
                  false, qT, sf);
  return ORACLE_OK;
}

int oracle_per_channel(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int group,
                       float clamp_min, uint8_t* q, float* sf) {
  const int rc = check_common(x, q, sf, fmt, group);
  if (rc != ORACLE_OK) return rc;
  if (rows < 0 || cols < 0 || rows % group != 0) return ORACLE_ERR_SHAPE;
  if (pairs(fmt) && cols % 2 != 0) return ORACLE_ERR_SHAPE;
  std::vector<float> xf(static_cast<size_t>(rows * cols));
  for (int64_t i = 0; i < rows * cols; ++i) xf[i] = bf16_value(x[i]);
  per_channel_f32(xf.data(), rows, cols, fmt, group, floor_for(*table_for(fmt), clamp_min), false,
                  false, q, sf);
  return ORACLE_OK;
}

int oracle_dequant_per_token(const uint8_t* q, const float* sf, int64_t rows, int64_t cols,
                             int fmt, int group, float* out) {
  const int rc = check_common(q, sf, out, fmt, group);
  if (rc != ORACLE_OK) return rc;
  if (rows < 0 || cols < 0 || cols % group != 0) return ORACLE_ERR_SHAPE;
  const FormatTable& t = *table_for(fmt);
  const int64_t groups = cols / group;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c)
      out[r * cols + c] = decode(t, get_code(fmt, q, cols, r, c)) * sf[r * groups + c / group];
  return ORACLE_OK;
}

int oracle_per_token_sf(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int group,
                        float clamp_min, int sf_flags, uint8_t* q, void* sf) {
  int rc = check_common(x, q, sf, fmt, group);
  if (rc != ORACLE_OK) return rc;
  if (rows < 0 || cols < 0 || cols % group != 0) return ORACLE_ERR_SHAPE;
  if (pairs(fmt) && group % 2 != 0) return ORACLE_ERR_GROUP;
  if ((rc = check_sf_flags(sf_flags, cols, group)) != ORACLE_OK) return rc;
  const float floor = floor_for(*table_for(fmt), clamp_min);
  const int64_t code_bytes = code_row_bytes(fmt, cols);
  std::vector<float> row(static_cast<size_t>(cols));
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) row[c] = bf16_value(x[r * cols + c]);
    per_token_row_sf(row.data(), r, rows, cols, fmt, group, floor, sf_flags, q + r * code_bytes,
                     sf);
  }
  return ORACLE_OK;
}

int oracle_swiglu_per_token_sf(const uint16_t* h, int64_t rows, int64_t cols, const float* w,
                               int fmt, int group, float clamp_min, int sf_flags, uint8_t* q,
                               void* sf) {
  int rc = check_common(h, q, sf, fmt, group);
  if (rc != ORACLE_OK) return rc;
  if (rows < 0 || cols < 0 || cols % group != 0) return ORACLE_ERR_SHAPE;
  if (pairs(fmt) && group % 2 != 0) return ORACLE_ERR_GROUP;
  if ((rc = check_sf_flags(sf_flags, cols, group)) != ORACLE_OK) return rc;
  const float floor = floor_for(*table_for(fmt), clamp_min);
  const int64_t code_bytes = code_row_bytes(fmt, cols);
  std::vector<float> v(static_cast<size_t>(cols));
  for (int64_t r = 0; r < rows; ++r) {
    oracle_swiglu_values(h + r * 2 * cols, 1, cols, w ? w + r : nullptr, v.data());
    per_token_row_sf(v.data(), r, rows, cols, fmt, group, floor, sf_flags, q + r * code_bytes, sf);
  }
  return ORACLE_OK;
}

int oracle_swiglu_per_token_ex(const uint16_t* h, int64_t rows, int64_t cols, const float* w,
                               int fmt, int group, float clamp_min, int sf_flags,
                               float swiglu_clamp, uint8_t* q, void* sf, uint64_t* count) {
  int rc = check_common(h, q, sf, fmt, group);
  if (rc != ORACLE_OK) return rc;
  if (rows < 0 || cols < 0 || cols % group != 0) return ORACLE_ERR_SHAPE;
  if (pairs(fmt) && group % 2 != 0) return ORACLE_ERR_GROUP;
  if ((rc = check_sf_flags(sf_flags, cols, group)) != ORACLE_OK) return rc;
  const float floor = floor_for(*table_for(fmt), clamp_min);
  const int64_t code_bytes = code_row_bytes(fmt, cols);
  std::vector<float> v(static_cast<size_t>(cols));
  for (int64_t r = 0; r < rows; ++r) {
    swiglu_row(h + r * 2 * cols, cols, w ? w[r] : 1.0f, w != nullptr, swiglu_clamp, v.data(),
               count);
    per_token_row_sf(v.data(), r, rows, cols, fmt, group, floor, sf_flags, q + r * code_bytes, sf);
  }
  return ORACLE_OK;
}

int oracle_swiglu_backward_values(const uint16_t* h, const uint16_t* dv, int64_t rows,
                                  int64_t cols, const float* w, float swiglu_clamp, float* out) {
  if (!h || !dv || !out) return ORACLE_ERR_NULL;
  if (rows < 0 || cols < 0) return ORACLE_ERR_SHAPE;
  if (!fp_env_ok()) return ORACLE_ERR_FPENV;
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t* hr = h + r * 2 * cols;
    float* o = out + r * 2 * cols;
    for (int64_t j = 0; j < cols; ++j) {
      float g = bf16_value(hr[j]);
      float u = bf16_value(hr[cols + j]);
      bool g_pass = true, u_pass = true;
      if (swiglu_clamp > 0.0f) {
        if (g > swiglu_clamp) { g = swiglu_clamp; g_pass = false; }
        if (u > swiglu_clamp) { u = swiglu_clamp; u_pass = false; }
        else if (u < -swiglu_clamp) { u = -swiglu_clamp; u_pass = false; }
      }
      const float e = exp_f32(-g);
      const float s = 1.0f / (1.0f + e);
      const float silu = g * s;
      const float dsilu = s + silu * (1.0f - s);
      float dvw = bf16_value(dv[r * cols + j]);
      if (w) dvw = dvw * w[r];
      o[j] = g_pass ? dvw * u * dsilu : 0.0f;
      o[cols + j] = u_pass ? dvw * silu : 0.0f;
    }
  }
  return ORACLE_OK;
}

int oracle_swiglu_backward_per_token(const uint16_t* h, const uint16_t* dv, int64_t rows,
                                     int64_t cols, const float* w, int fmt, int group,
                                     float clamp_min, float swiglu_clamp, uint8_t* q,
                                     float* sf) {
  const int rc = check_common(h, q, sf, fmt, group);
  if (rc != ORACLE_OK) return rc;
  if (!dv) return ORACLE_ERR_NULL;
  if (rows < 0 || cols < 0 || cols % group != 0) return ORACLE_ERR_SHAPE;
  /* Every format of the forward cast: [SPLIT] §四 A pairs the SwiGLU cast
   * (E4M3 / E5M2 / E2M1 / E5M6) with a matching backward. The row [dg | du]
   * is one row of 2 * cols codes. */
  if (pairs(fmt) && group % 2 != 0) return ORACLE_ERR_GROUP;
  std::vector<float> vals(static_cast<size_t>(rows * 2 * cols));
  oracle_swiglu_backward_values(h, dv, rows, cols, w, swiglu_clamp, vals.data());
  per_token_rows(vals.data(), rows, 2 * cols, fmt, group, floor_for(*table_for(fmt), clamp_min),
                 q, sf);
  return ORACLE_OK;
}

int oracle_swiglu_per_channel_T(const uint16_t* h, int64_t rows, int64_t cols, const float* w,
                                int fmt, int group, float clamp_min, float swiglu_clamp,
                                uint8_t* qT, float* sf) {
  const int rc = check_common(h, qT, sf, fmt, group);
  if (rc != ORACLE_OK) return rc;
  if (rows < 0 || cols < 0 || rows % group != 0) return ORACLE_ERR_SHAPE;
  if (pairs(fmt) && group % 2 != 0) return ORACLE_ERR_GROUP;
  std::vector<float> v(static_cast<size_t>(rows * cols));
  oracle_swiglu_values_ex(h, rows, cols, w, swiglu_clamp, v.data(), nullptr);
  per_channel_f32(v.data(), rows, cols, fmt, group, floor_for(*table_for(fmt), clamp_min), true,
                  false, qT, sf);
  return ORACLE_OK;
}

int oracle_per_channel_sf(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int group,
                          float clamp_min, int sf_flags, uint8_t* q, float* sf) {
  const int rc = check_common(x, q, sf, fmt, group);
  if (rc != ORACLE_OK) return rc;
  if (sf_flags & ~ORACLE_SF_ROUND_POW2) return ORACLE_ERR_FORMAT;
  if (rows < 0 || cols < 0 || rows % group != 0) return ORACLE_ERR_SHAPE;
  if (pairs(fmt) && cols % 2 != 0) return ORACLE_ERR_SHAPE;
  std::vector<float> xf(static_cast<size_t>(rows * cols));
  for (int64_t i = 0; i < rows * cols; ++i) xf[i] = bf16_value(x[i]);
  per_channel_f32(xf.data(), rows, cols, fmt, group, floor_for(*table_for(fmt), clamp_min), false,
                  (sf_flags & ORACLE_SF_ROUND_POW2) != 0, q, sf);
  return ORACLE_OK;
}

int oracle_per_channel_T_sf(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int group,
                            float clamp_min, int sf_flags, uint8_t* qT, void* sf) {
  int rc = check_common(x, qT, sf, fmt, group);
  if (rc != ORACLE_OK) return rc;
  if (rows < 0 || cols < 0 || rows % group != 0) return ORACLE_ERR_SHAPE;
  if (pairs(fmt) && group % 2 != 0) return ORACLE_ERR_GROUP;
  if ((rc = check_sf_flags(sf_flags, rows, group)) != ORACLE_OK) return rc;
  std::vector<float> xf(static_cast<size_t>(rows * cols));
  for (int64_t i = 0; i < rows * cols; ++i) xf[i] = bf16_value(x[i]);
  per_channel_T_sf_f32(xf.data(), rows, cols, fmt, group, floor_for(*table_for(fmt), clamp_min),
                       sf_flags, qT, sf);
  return ORACLE_OK;
}

int oracle_swiglu_per_channel_T_sf(const uint16_t* h, int64_t rows, int64_t cols, const float* w,
                                   int fmt, int group, float clamp_min, int sf_flags,
                                   float swiglu_clamp, uint8_t* qT, void* sf) {
  int rc = check_common(h, qT, sf, fmt, group);
  if (rc != ORACLE_OK) return rc;
  if (rows < 0 || cols < 0 || rows % group != 0) return ORACLE_ERR_SHAPE;
  if (pairs(fmt) && group % 2 != 0) return ORACLE_ERR_GROUP;
  if ((rc = check_sf_flags(sf_flags, rows, group)) != ORACLE_OK) return rc;
  std::vector<float> v(static_cast<size_t>(rows * cols));
  oracle_swiglu_values_ex(h, rows, cols, w, swiglu_clamp, v.data(), nullptr);
  per_channel_T_sf_f32(v.data(), rows, cols, fmt, group, floor_for(*table_for(fmt), clamp_min),
                       sf_flags, qT, sf);
  return ORACLE_OK;
}

int oracle_swiglu_backward_per_token_sf(const uint16_t* h, const uint16_t* dv, int64_t rows,
                                        int64_t cols, const float* w, int fmt, int group,
                                        float clamp_min, int sf_flags, float swiglu_clamp,
                                        uint8_t* q, void* sf) {
  int rc = check_common(h, q, sf, fmt, group);
  if (rc != ORACLE_OK) return rc;
  if (!dv) return ORACLE_ERR_NULL;
  if (rows < 0 || cols < 0 || cols % group != 0) return ORACLE_ERR_SHAPE;
  if (pairs(fmt) && group % 2 != 0) return ORACLE_ERR_GROUP;
  if ((rc = check_sf_flags(sf_flags, 2 * cols, group)) != ORACLE_OK) return rc;
  std::vector<float> vals(static_cast<size_t>(rows * 2 * cols));
  oracle_swiglu_backward_values(h, dv, rows, cols, w, swiglu_clamp, vals.data());
  const float floor = floor_for(*table_for(fmt), clamp_min);
  const int64_t code_bytes = code_row_bytes(fmt, 2 * cols);
  for (int64_t r = 0; r < rows; ++r)
    per_token_row_sf(vals.data() + r * 2 * cols, r, rows, 2 * cols, fmt, group, floor, sf_flags,
                     q + r * code_bytes, sf);
  return ORACLE_OK;
}

uint16_t oracle_f32_to_bf16(float f) {
  /* Round to nearest even on the 16 bits that are dropped: add 0x7FFF plus
   * the lowest kept bit, then truncate. NaNs are returned quiet. */
  uint32_t u;
  std::memcpy(&u, &f, sizeof u);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
  const uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return static_cast<uint16_t>(u >> 16);
}

int oracle_cast_back(const uint8_t* q, const float* sf, int64_t rows, int64_t cols, int fmt,
                     int group, int out_dtype, void* out) {
  const int rc = check_common(q, sf, out, fmt, group);
  if (rc != ORACLE_OK) return rc;
  if (rows < 0 || cols < 0 || cols % group != 0) return ORACLE_ERR_SHAPE;
  if (out_dtype != ORACLE_OUT_BF16 && out_dtype != ORACLE_OUT_F32) return ORACLE_ERR_FORMAT;
  const FormatTable& t = *table_for(fmt);
  const int64_t groups = cols / group;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      const float v = decode(t, get_code(fmt, q, cols, r, c)) * sf[r * groups + c / group];
      if (out_dtype == ORACLE_OUT_F32) static_cast<float*>(out)[r * cols + c] = v;
      else static_cast<uint16_t*>(out)[r * cols + c] = oracle_f32_to_bf16(v);
    }
  return ORACLE_OK;
}

} /* extern "C" */
