// per_channel_t_wave.hip -- the transposed per-channel casts (plain, and
// fused with SwiGLU) with the transpose done in registers: every code format
// (E4M3, E5M2, packed E2M1, packed E5M6).
//
// Operation: per_channel_cast (+transpose) of the operator table on the page
// "TileKernels 与 DeepGEMM 的分界线：DeepSeek 开源内核栈的分工", §二, in the
// formats its §四 A lists (and the FP8 / FP4 / E5M6 of the TileKernels
// overview of "DeepSeek 的 GPU 内核帝国", quant/): groups of 128 tokens of one
// channel, codes written channel-major, qT[c] holding the codes of tokens
// 0 .. rows-1 of channel c as one code row (a byte per code, a nibble for
// E2M1 with the even token low, 12 bits for E5M6). The SwiGLU form casts
// v = silu(g) * u * w of the walk-through page "DeepSeek开源TileKernels：用
// Python写的GPU算子逼近硬件性能上限", §3.3 (the three-way fusion of "刚刚！
// DeepSeek开源高性能GPU算子库TileKernels", item 2).
//
// gfx950 design. One wave owns a tile of one 128-token group x 8 * kCC
// channels. Lane (tb, cc) loads the 16-byte chunk cc (8 channels) of kT
// consecutive tokens tb * kT .. tb * kT + kT - 1, all loads issued before any
// is used (kT = 16 for bf16 input: 256 bytes in flight per lane; kT = 8 for
// SwiGLU, which loads gate and up). The lane then holds, for each of its 8
// channels, kT consecutive tokens: exactly a run of the transposed output.
// So nothing crosses lanes but the column abs-maxima (packed 16-bit or fp32
// maxima over the lane's tokens, then DPP row rotations and two cross-row
// shuffles over the lanes that share the channel chunk), and there is no LDS
// and no barrier: every lane forms its 8 channels' scales, scales its values
// and stores, per channel, its run of kT codes (16 bytes of E4M3 per store;
// the kL lanes of a channel chunk cover the channel's 128 tokens
// contiguously). Each lane stores one scale. Workgroups hold four waves on
// four consecutive tiles of the same walk as the LDS-tile kernel
// (per_channel_t.hip): each XCD takes a contiguous range, in strips of
// channel tiles, token group outer.
#include "qcast_device.h"
#include "qcast_kernels.h"

namespace qcast {
namespace {

constexpr int kGroupTokens = 128;
constexpr int kXcds = 8;
constexpr int kWaves = kThreads / 64;

#ifndef QCAST_PCW_STRIP
#define QCAST_PCW_STRIP 2
#endif
constexpr uint32_t kStripW = QCAST_PCW_STRIP;

// Tile geometry for kT tokens per lane.
template <int kT>
struct Geo {
  static constexpr int kL = kGroupTokens / kT;  // lanes per channel chunk (8 or 16)
  static constexpr int kCC = 64 / kL;           // channel chunks per wave (8 or 4)
  static constexpr int kWc = 8 * kCC;           // channels per tile (64 or 32)
};

struct WaveTile {
  uint32_t c0, t0, gt;
  bool valid;
};

// Tile of wave w of workgroup b: workgroups remapped so that each XCD walks
// a contiguous range; inside it, strips of kStripW channel tiles, token group
// outer, channel tile inner.
__device__ __forceinline__ WaveTile wave_tile(uint32_t b, uint32_t per_xcd, uint32_t ntiles,
                                              uint32_t nct, uint32_t ntg, uint32_t wc) {
  const uint32_t wg = (b % kXcds) * per_xcd + b / kXcds;
  const uint32_t tau = wg * kWaves + (threadIdx.x >> 6);
  WaveTile t;
  t.valid = tau < ntiles;
  const uint32_t strip = tau / (kStripW * ntg);
  const uint32_t width = nct - strip * kStripW < kStripW ? nct - strip * kStripW : kStripW;
  const uint32_t rem = tau - strip * kStripW * ntg;
  t.gt = rem / width;
  const uint32_t ct = strip * kStripW + (rem - t.gt * width);
  t.c0 = ct * wc;
  t.t0 = t.gt * kGroupTokens;
  return t;
}

// Abs-maxima over the kL lanes that share a channel chunk (lanes kCC apart).
template <int kCC>
__device__ __forceinline__ uint32_t chunk_max_u32(uint32_t m) {
  if (kCC == 4) m = umax(m, dpp<0x124>(m));   // row_ror:4
  m = umax(m, dpp<kDppRor8>(m));
  m = umax(m, (uint32_t)__shfl_xor((int)m, 16));
  m = umax(m, (uint32_t)__shfl_xor((int)m, 32));
  return m;
}
template <int kCC>
__device__ __forceinline__ uint32_t chunk_max_pk16(uint32_t m) {
  if (kCC == 4) m = pk_umax16(m, dpp<0x124>(m));
  m = pk_umax16(m, dpp<kDppRor8>(m));
  m = pk_umax16(m, (uint32_t)__shfl_xor((int)m, 16));
  m = pk_umax16(m, (uint32_t)__shfl_xor((int)m, 32));
  return m;
}

// Codes of kT consecutive elements starting at element e of a code row
// (e a multiple of kT), stored non-temporally.
template <int kFmt, int kT>
__device__ __forceinline__ void store_run(uint8_t* row, uint32_t e, const float (&y)[kT]) {
  if constexpr (kT == 8) {
    store_chunk8<kFmt>(row, e / 8, y);
  } else {
    static_assert(kT == 16, "runs of 8 or 16 codes");
    if constexpr (kFmt == kE2M1) {
      u32x2 o;
      o.x = e2m1x8(&y[0]);
      o.y = e2m1x8(&y[8]);
      store_stream(reinterpret_cast<u32x2*>(row + e / 2), o);
    } else if constexpr (kFmt == kE5M6) {
      const E5M6x8 a = e5m6x8(&y[0]);
      const E5M6x8 b = e5m6x8(&y[8]);
      u32x2* o = reinterpret_cast<u32x2*>(row + e / 2 * 3);
      store_stream(o, u32x2{a.w0, a.w1});
      store_stream(o + 1, u32x2{a.w2, b.w0});
      store_stream(o + 2, u32x2{b.w1, b.w2});
    } else {
      u32x4 o;
      o.x = fp8x4<kFmt>(y[0], y[1], y[2], y[3]);
      o.y = fp8x4<kFmt>(y[4], y[5], y[6], y[7]);
      o.z = fp8x4<kFmt>(y[8], y[9], y[10], y[11]);
      o.w = fp8x4<kFmt>(y[12], y[13], y[14], y[15]);
      store_stream(reinterpret_cast<u32x4*>(row + e), o);
    }
  }
}

// Scales and codes of a tile whose column abs-maxima am[8] (of the lane's 8
// channels) are known; value(i, j) is the lane's value of token i, channel j.
template <int kFmt, int kT, class ValueFn>
__device__ __forceinline__ void finish_tile(const WaveTile& tl, const float (&am)[8],
                                            uint32_t rows, uint32_t cols, uint32_t ngroups,
                                            float floor, uint8_t* __restrict__ qT,
                                            float* __restrict__ sf, ValueFn value) {
  using G = Geo<kT>;
  const int lane = threadIdx.x & 63;
  const int cc = lane % G::kCC;
  const int tb = lane / G::kCC;
  const uint32_t c_lane = tl.c0 + 8 * cc;
  if (c_lane >= cols) return;
  float inv[8];
  float my_sf = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const Scale s = group_scale<kFmt>(am[j], floor);
    inv[j] = s.inv;
    my_sf = (tb == j) ? s.sf : my_sf;
  }
  // lane (tb, cc) with tb < 8 stores the scale of channel 8 * cc + tb
  if (tb < 8) sf[(uint64_t)(c_lane + tb) * ngroups + tl.gt] = my_sf;
  const uint32_t row_bytes = code_bytes<kFmt>(rows);
  uint8_t* base = qT + (uint64_t)c_lane * row_bytes + code_bytes<kFmt>(tl.t0);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float y[kT];
#pragma unroll
    for (int i = 0; i < kT; ++i) y[i] = value(i, j) * inv[j];
    store_run<kFmt, kT>(base + (uint32_t)j * row_bytes, (uint32_t)(kT * tb), y);
  }
}

// The plain cast: kT = 16 tokens of packed bf16 per lane.
template <int kFmt>
__global__ __launch_bounds__(kThreads) void per_channel_t_wave_kernel(
    const uint16_t* __restrict__ x, uint32_t rows, uint32_t cols, uint32_t ngroups,
    uint32_t nct, uint32_t ntiles, uint32_t per_xcd, float floor, uint8_t* __restrict__ qT,
    float* __restrict__ sf) {
  constexpr int kT = 16;
  using G = Geo<kT>;
  const WaveTile tl = wave_tile(blockIdx.x, per_xcd, ntiles, nct, ngroups, G::kWc);
  if (!tl.valid) return;   // no barrier in this kernel: a wave may leave alone
  const int lane = threadIdx.x & 63;
  const int cc = lane % G::kCC;
  const int tb = lane / G::kCC;
  const bool valid = tl.c0 + 8 * cc < cols;
  const uint16_t* src = x + (uint64_t)tl.t0 * cols + tl.c0 + 8 * cc;
  u32x4 raw[kT];
#pragma unroll
  for (int i = 0; i < kT; ++i) {
    const uint32_t off = (uint32_t)(kT * tb + i) * cols;
    raw[i] = valid ? load_stream(reinterpret_cast<const u32x4*>(src + off))
                   : u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t m[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < kT; ++i) {
    m[0] = pk_umax16(m[0], raw[i].x & 0x7fff7fffu);
    m[1] = pk_umax16(m[1], raw[i].y & 0x7fff7fffu);
    m[2] = pk_umax16(m[2], raw[i].z & 0x7fff7fffu);
    m[3] = pk_umax16(m[3], raw[i].w & 0x7fff7fffu);
  }
  float am[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    m[w] = chunk_max_pk16<G::kCC>(m[w]);
    am[2 * w] = bf16_lo(m[w]);
    am[2 * w + 1] = bf16_hi(m[w]);
  }
  finish_tile<kFmt, kT>(tl, am, rows, cols, ngroups, floor, qT, sf, [&](int i, int j) {
    const uint32_t word = raw[i][j >> 1];
    return (j & 1) ? bf16_hi(word) : bf16_lo(word);
  });
}

constexpr float kLog2e = 1.4426950408889634f;

// SwiGLU + the same cast: kT = 8 tokens per lane, gate and up loaded, v kept
// in fp32. Counting modes as in per_channel_t.hip: none; through the slots
// of a count workspace (every workgroup of the grid reports once); or one
// atomic per workgroup of a capped grid that walks the virtual workgroups
// [0, vgrid) with a stride of gridDim.x.
template <int kFmt, bool kWeighted, bool kClamp, int kCount>
__global__ __launch_bounds__(kThreads) void swiglu_per_channel_t_wave_kernel(
    const uint16_t* __restrict__ h, const float* __restrict__ w, uint32_t rows, uint32_t cols,
    uint32_t ngroups, uint32_t nct, uint32_t ntiles, uint32_t per_xcd, uint32_t vgrid,
    float floor, float clamp, unsigned long long* __restrict__ count,
    unsigned long long* __restrict__ slots, uint8_t* __restrict__ qT, float* __restrict__ sf) {
  constexpr int kT = 8;
  using G = Geo<kT>;
  const int lane = threadIdx.x & 63;
  const int cc = lane % G::kCC;
  const int tb = lane / G::kCC;
  uint32_t nclamp = 0;
  const uint32_t stride = kCount == kCountDirect ? gridDim.x : vgrid;
  for (uint32_t b = blockIdx.x; b < vgrid; b += stride) {
    const WaveTile tl = wave_tile(b, per_xcd, ntiles, nct, ngroups, G::kWc);
    if (!tl.valid) continue;   // the counting epilogue below is reached by every wave
    const bool valid = tl.c0 + 8 * cc < cols;
    const uint16_t* src = h + (uint64_t)tl.t0 * 2 * cols + tl.c0 + 8 * cc;
    u32x4 graw[kT], uraw[kT];
    float wr[kT];
#pragma unroll
    for (int i = 0; i < kT; ++i) {
      const uint32_t tok = (uint32_t)(kT * tb + i);
      const uint32_t off = tok * 2 * cols;
      const u32x4 z = {0u, 0u, 0u, 0u};
      graw[i] = valid ? load_stream(reinterpret_cast<const u32x4*>(src + off)) : z;
      uraw[i] = valid ? load_stream(reinterpret_cast<const u32x4*>(src + off + cols)) : z;
      wr[i] = (kWeighted && valid) ? w[tl.t0 + tok] : 1.0f;
    }
    float v[kT][8];
    uint32_t m[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kT; ++i) {
      float gv[8], uv[8];
      unpack8(graw[i], gv);
      unpack8(uraw[i], uv);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (kCount != kCountNone) nclamp += wave_clamp_count(gv[j], uv[j], clamp);
        if (kClamp) clamp_gate_up(gv[j], uv[j], clamp);
        const float e = __builtin_amdgcn_exp2f(-gv[j] * kLog2e);
        float val = gv[j] * __builtin_amdgcn_rcpf(1.0f + e) * uv[j];
        if (kWeighted) val = val * wr[i];
        v[i][j] = val;
        m[j] = umax(m[j], __float_as_uint(val) & 0x7fffffffu);
      }
    }
    float am[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) am[j] = __uint_as_float(chunk_max_u32<G::kCC>(m[j]));
    finish_tile<kFmt, kT>(tl, am, rows, cols, ngroups, floor, qT, sf,
                          [&](int i, int j) { return v[i][j]; });
    if (kCount == kCountNone) break;   // one tile per wave without counting
  }
  if constexpr (kCount == kCountDirect) add_wave_counts(nclamp, count);
  if constexpr (kCount == kCountSlotted) add_wave_counts_slotted(nclamp, slots, count);
}

struct GridW {
  uint32_t ngroups, nct, ntiles, per_xcd, grid;
};

template <int kT>
bool make_grid_w(int64_t rows, int64_t cols, int64_t row_stride, int64_t code_row_bytes,
                 GridW* g) {
  using G = Geo<kT>;
  const int64_t ngroups = rows / kGroupTokens;
  const int64_t nct = (cols + G::kWc - 1) / G::kWc;
  const int64_t ntiles = ngroups * nct;
  const int64_t lim = int64_t(1) << 31;
  const int64_t wgs = (ntiles + kWaves - 1) / kWaves;
  if (ntiles + kWaves * kXcds >= lim || (int64_t)kGroupTokens * row_stride >= lim ||
      (int64_t)G::kWc * code_row_bytes >= lim || rows >= lim || row_stride >= lim)
    return false;
  g->ngroups = (uint32_t)ngroups;
  g->nct = (uint32_t)nct;
  g->ntiles = (uint32_t)ntiles;
  g->per_xcd = (uint32_t)((wgs + kXcds - 1) / kXcds);
  g->grid = g->per_xcd * kXcds;
  return true;
}

#ifndef QCAST_PCW_COUNT_WG_PER_CU
#define QCAST_PCW_COUNT_WG_PER_CU 4
#endif

template <int kFmt, bool kWeighted, bool kClamp>
hipError_t launch_sw(const uint16_t* h, const float* w, int64_t rows, int64_t cols,
                     const GridW& g, float floor, float clamp, unsigned long long* count,
                     unsigned long long* slots, uint8_t* qT, float* sf, hipStream_t stream,
                     const LaunchCaps& caps) {
  if constexpr (kClamp) {
    if (count && slots && (int64_t)g.grid < (int64_t(kCountSlots) << (64 - kSlotArrivalShift))) {
      launch_kernel((swiglu_per_channel_t_wave_kernel<kFmt, kWeighted, true, kCountSlotted>),
                    dim3(g.grid), dim3(kThreads), 0, stream, h, w, (uint32_t)rows,
                    (uint32_t)cols, g.ngroups, g.nct, g.ntiles, g.per_xcd, g.grid, floor, clamp,
                    count, slots, qT, sf);
      return hipGetLastError();
    }
    if (count) {
      uint32_t grid = g.grid;
      const int64_t cap = (int64_t)caps.num_cus * QCAST_PCW_COUNT_WG_PER_CU;
      if (cap < grid) grid = (uint32_t)cap;
      launch_kernel((swiglu_per_channel_t_wave_kernel<kFmt, kWeighted, true, kCountDirect>),
                    dim3(grid), dim3(kThreads), 0, stream, h, w, (uint32_t)rows,
                    (uint32_t)cols, g.ngroups, g.nct, g.ntiles, g.per_xcd, g.grid, floor, clamp,
                    count, slots, qT, sf);
      return hipGetLastError();
    }
  }
  launch_kernel((swiglu_per_channel_t_wave_kernel<kFmt, kWeighted, kClamp, kCountNone>),
                dim3(g.grid), dim3(kThreads), 0, stream, h, w, (uint32_t)rows, (uint32_t)cols,
                g.ngroups, g.nct, g.ntiles, g.per_xcd, g.grid, floor, clamp, count, slots, qT,
                sf);
  return hipGetLastError();
}

template <int kFmt>
hipError_t launch_sw_fmt(const uint16_t* h, const float* w, int64_t rows, int64_t cols,
                         const GridW& g, float floor, float clamp, unsigned long long* count,
                         unsigned long long* slots, uint8_t* qT, float* sf, hipStream_t stream,
                         const LaunchCaps& caps) {
  if (w)
    return clamp > 0.0f ? launch_sw<kFmt, true, true>(h, w, rows, cols, g, floor, clamp, count,
                                                      slots, qT, sf, stream, caps)
                        : launch_sw<kFmt, true, false>(h, w, rows, cols, g, floor, clamp, count,
                                                       slots, qT, sf, stream, caps);
  return clamp > 0.0f ? launch_sw<kFmt, false, true>(h, w, rows, cols, g, floor, clamp, count,
                                                     slots, qT, sf, stream, caps)
                      : launch_sw<kFmt, false, false>(h, w, rows, cols, g, floor, clamp, count,
                                                      slots, qT, sf, stream, caps);
}

int64_t code_row_bytes_of(int fmt, int64_t n) {
  return fmt == kE2M1 ? n / 2 : fmt == kE5M6 ? n / 2 * 3 : n;
}

}  // namespace

bool per_channel_t_wave_fits(int64_t rows, int64_t cols, int64_t row_stride, int fmt,
                             bool swiglu) {
  GridW g;
  const int64_t rb = code_row_bytes_of(fmt, rows);
  return swiglu ? make_grid_w<8>(rows, cols, row_stride, rb, &g)
                : make_grid_w<16>(rows, cols, row_stride, rb, &g);
}

hipError_t launch_per_channel_T_wave(const void* x, int64_t rows, int64_t cols, int fmt,
                                     float floor, void* qT, float* sf, hipStream_t stream) {
  GridW g;
  if (!make_grid_w<16>(rows, cols, cols, code_row_bytes_of(fmt, rows), &g))
    return hipErrorInvalidValue;
  if (g.ntiles == 0) return hipSuccess;
  auto kernel = fmt == kE4M3   ? per_channel_t_wave_kernel<kE4M3>
                : fmt == kE5M2 ? per_channel_t_wave_kernel<kE5M2>
                : fmt == kE2M1 ? per_channel_t_wave_kernel<kE2M1>
                : fmt == kE5M6 ? per_channel_t_wave_kernel<kE5M6>
                               : nullptr;
  if (!kernel) return hipErrorInvalidValue;
  launch_kernel(kernel, dim3(g.grid), dim3(kThreads), 0, stream,
                static_cast<const uint16_t*>(x), (uint32_t)rows, (uint32_t)cols, g.ngroups,
                g.nct, g.ntiles, g.per_xcd, floor, static_cast<uint8_t*>(qT), sf);
  return hipGetLastError();
}

hipError_t launch_swiglu_per_channel_T_wave(const void* h, int64_t rows, int64_t cols,
                                            const float* w, int fmt, float floor,
                                            float swiglu_clamp, unsigned long long* clamp_count,
                                            unsigned long long* count_ws, void* qT, float* sf,
                                            hipStream_t stream, const LaunchCaps& caps) {
  GridW g;
  if (!make_grid_w<8>(rows, cols, 2 * cols, code_row_bytes_of(fmt, rows), &g))
    return hipErrorInvalidValue;
  if (g.ntiles == 0) return hipSuccess;
  const uint16_t* hp = static_cast<const uint16_t*>(h);
  uint8_t* qp = static_cast<uint8_t*>(qT);
  switch (fmt) {
    case kE4M3:
      return launch_sw_fmt<kE4M3>(hp, w, rows, cols, g, floor, swiglu_clamp, clamp_count,
                                  count_ws, qp, sf, stream, caps);
    case kE5M2:
      return launch_sw_fmt<kE5M2>(hp, w, rows, cols, g, floor, swiglu_clamp, clamp_count,
                                  count_ws, qp, sf, stream, caps);
    case kE2M1:
      return launch_sw_fmt<kE2M1>(hp, w, rows, cols, g, floor, swiglu_clamp, clamp_count,
                                  count_ws, qp, sf, stream, caps);
    case kE5M6:
      return launch_sw_fmt<kE5M6>(hp, w, rows, cols, g, floor, swiglu_clamp, clamp_count,
                                  count_ws, qp, sf, stream, caps);
  }
  return hipErrorInvalidValue;
}

}  // namespace qcast
