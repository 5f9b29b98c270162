// cast_back.hip -- dequantize per-token codes back to bf16 or fp32.
//
// Operation: cast_back of the operator table on the page "TileKernels 与
// DeepGEMM 的分界线：DeepSeek 开源内核栈的分工", §二: every code times the
// fp32 scale of its group, out[r][c] = decode(q[r][c]) * sf[r][c / group],
// one fp32 product, then rounded to bf16 (nearest even) when bf16 output is
// asked for. The codes and scales are laid out as the per-token cast writes
// them ("DeepSeek开源TileKernels：用Python写的GPU算子逼近硬件性能上限", §3.2).
//
// gfx950 design. The per-token stream walked backwards: one lane per 8 codes
// (8 bytes of E4M3 / E5M2, 4 bytes of E2M1, 12 bytes of E5M6), decoded
// exactly by the hardware (v_cvt_pk_f32_fp8 / v_cvt_pk_f32_bf8 /
// v_cvt_scalef32_pk_f32_fp4 with scale 1; v_cvt_f32_f16 of the E5M6 code
// shifted to the top of an fp16 pattern -- cast_back_e5m6 of the same
// table), multiplied by the group's scale (the lanes of a group read the
// same scale word), and written as 8 bf16 (one 16-byte store, converted with
// v_cvt_pk_bf16_f32) or 8 fp32 (two 16-byte stores). One workgroup per
// 256 * kUnroll chunks (kUnroll by format, below).
#include "qcast_device.h"
#include "qcast_kernels.h"

namespace qcast {
namespace {

// Chunks per lane. The 8-, 12-byte code loads of E4M3, E5M2 and E5M6 run
// best at 1 (about 8% faster than 2 or 4 on 4096 x 7168: the kernel writes
// twice what it reads, and more workgroups spread those writes better).
// E2M1's 4-byte code loads want more in flight: 14.6 us at 4 chunks per
// lane against 14.8 at 2 and 16.2 at 1 (interleaved, 100 rounds).
#ifndef QCAST_CB_UNROLL
#define QCAST_CB_UNROLL 1
#endif
#ifndef QCAST_CB_UNROLL_E2M1
#define QCAST_CB_UNROLL_E2M1 4
#endif
template <int kFmt>
constexpr int kUnroll = kFmt == kE2M1 ? QCAST_CB_UNROLL_E2M1 : QCAST_CB_UNROLL;
constexpr int kMinUnroll =
    QCAST_CB_UNROLL < QCAST_CB_UNROLL_E2M1 ? QCAST_CB_UNROLL : QCAST_CB_UNROLL_E2M1;

typedef float f32x2 __attribute__((ext_vector_type(2)));

// One E5M6 code (low 12 bits of c) -> fp32: it is the top of an fp16
// pattern, so v_cvt_f32_f16 of c << 4 is exact.
__device__ __forceinline__ float e5m6_value(uint32_t c) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)((c << 4) & 0xfff0u));
}

// Eight codes -> eight exact fp32 values (E5M6: 96 bits in codes.x, .y, .z).
template <int kFmt>
__device__ __forceinline__ void decode8(u32x4 codes, float v[8]) {
  if constexpr (kFmt == kE5M6) {
    const uint32_t w0 = codes.x, w1 = codes.y, w2 = codes.z;
    v[0] = e5m6_value(w0);
    v[1] = e5m6_value(w0 >> 12);
    v[2] = e5m6_value((w0 >> 24) | (w1 << 8));
    v[3] = e5m6_value(w1 >> 4);
    v[4] = e5m6_value(w1 >> 16);
    v[5] = e5m6_value((w1 >> 28) | (w2 << 4));
    v[6] = e5m6_value(w2 >> 8);
    v[7] = e5m6_value(w2 >> 20);
  } else if constexpr (kFmt == kE2M1) {
    const uint32_t w = codes.x;  // 8 nibbles; the byte selector is an immediate
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    v[0] = p0.x; v[1] = p0.y; v[2] = p1.x; v[3] = p1.y;
    v[4] = p2.x; v[5] = p2.y; v[6] = p3.x; v[7] = p3.y;
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w = h ? codes.y : codes.x;
      f32x2 lo, hi;
      if constexpr (kFmt == kE4M3) {
        lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
        hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
      } else {
        lo = __builtin_amdgcn_cvt_pk_f32_bf8(w, false);
        hi = __builtin_amdgcn_cvt_pk_f32_bf8(w, true);
      }
      v[4 * h + 0] = lo.x;
      v[4 * h + 1] = lo.y;
      v[4 * h + 2] = hi.x;
      v[4 * h + 3] = hi.y;
    }
  }
}

__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
  const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
  const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(b));
  return lo | (hi << 16);
}

template <int kLanes, int kFmt, bool kBf16>
__global__ __launch_bounds__(kThreads) void cast_back_kernel(const uint8_t* __restrict__ q,
                                                             const float* __restrict__ sf,
                                                             int64_t nchunks,
                                                             void* __restrict__ out) {
  constexpr int kU = kUnroll<kFmt>;
  const int64_t base = (int64_t)blockIdx.x * kThreads * kU + threadIdx.x;
  u32x4 codes[kU];
  float s[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t c = base + (int64_t)u * kThreads;
    if (c < nchunks) {
      codes[u] = u32x4{0u, 0u, 0u, 0u};
      if constexpr (kFmt == kE2M1) {
        codes[u].x = load_stream(reinterpret_cast<const uint32_t*>(q) + c);
      } else if constexpr (kFmt == kE5M6) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(q) + 3 * c;
        codes[u].x = load_stream(p);
        codes[u].y = load_stream(p + 1);
        codes[u].z = load_stream(p + 2);
      } else {
        const u32x2 w = load_stream(reinterpret_cast<const u32x2*>(q) + c);
        codes[u].x = w.x;
        codes[u].y = w.y;
      }
      s[u] = sf[c / kLanes];
    }
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t c = base + (int64_t)u * kThreads;
    if (c < nchunks) {
      float v[8];
      decode8<kFmt>(codes[u], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = v[i] * s[u];
      if constexpr (kBf16) {
        const u32x4 o = {bf16x2(v[0], v[1]), bf16x2(v[2], v[3]), bf16x2(v[4], v[5]),
                         bf16x2(v[6], v[7])};
        store_stream(reinterpret_cast<u32x4*>(out) + c, o);
      } else {
        const u32x4 o0 = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                          __float_as_uint(v[3])};
        const u32x4 o1 = {__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
                          __float_as_uint(v[7])};
        store_stream(reinterpret_cast<u32x4*>(out) + 2 * c, o0);
        store_stream(reinterpret_cast<u32x4*>(out) + 2 * c + 1, o1);
      }
    }
  }
}

template <int kLanes, int kFmt>
hipError_t launch(const void* q, const float* sf, int64_t nchunks, bool out_bf16, void* out,
                  hipStream_t stream) {
  const int64_t per_block = (int64_t)kThreads * kUnroll<kFmt>;
  const int64_t blocks = (nchunks + per_block - 1) / per_block;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  if (out_bf16)
    launch_kernel((cast_back_kernel<kLanes, kFmt, true>), dim3((unsigned)blocks),
                  dim3(kThreads), 0, stream, static_cast<const uint8_t*>(q), sf, nchunks, out);
  else
    launch_kernel((cast_back_kernel<kLanes, kFmt, false>), dim3((unsigned)blocks),
                  dim3(kThreads), 0, stream, static_cast<const uint8_t*>(q), sf, nchunks, out);
  return hipGetLastError();
}

template <int kFmt>
hipError_t launch_fmt(const void* q, const float* sf, int64_t nchunks, int group, bool out_bf16,
                      void* out, hipStream_t stream) {
  switch (group) {
    case 32: return launch<4, kFmt>(q, sf, nchunks, out_bf16, out, stream);
    case 64: return launch<8, kFmt>(q, sf, nchunks, out_bf16, out, stream);
    case 128: return launch<16, kFmt>(q, sf, nchunks, out_bf16, out, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool cast_back_fits(int64_t rows, int64_t cols) {
  const int64_t per_block = (int64_t)kThreads * kMinUnroll;  // the largest grid of any format
  return (rows * cols / 8 + per_block - 1) / per_block < (int64_t(1) << 31);
}

hipError_t launch_cast_back(const void* q, const float* sf, int64_t rows, int64_t cols, int fmt,
                            int group, bool out_bf16, void* out, hipStream_t stream,
                            const LaunchCaps& caps) {
  (void)caps;
  const int64_t nchunks = rows * cols / 8;
  if (nchunks == 0) return hipSuccess;
  switch (fmt) {
    case kE4M3: return launch_fmt<kE4M3>(q, sf, nchunks, group, out_bf16, out, stream);
    case kE5M2: return launch_fmt<kE5M2>(q, sf, nchunks, group, out_bf16, out, stream);
    case kE2M1: return launch_fmt<kE2M1>(q, sf, nchunks, group, out_bf16, out, stream);
    case kE5M6: return launch_fmt<kE5M6>(q, sf, nchunks, group, out_bf16, out, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace qcast
