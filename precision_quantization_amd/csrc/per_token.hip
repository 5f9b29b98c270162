// per_token.hip -- per-token cast of bf16 rows to E4M3, E5M2, packed E2M1 or
// packed E5M6.
//
// Operation: the per-token cast of the walk-through page
// "DeepSeek开源TileKernels：用Python写的GPU算子逼近硬件性能上限", quick start and
// §3.2 (abs-max over each run of num_per_channels elements of a row, scale
// and inverse, codes of x * inverse); E2M1 output per §3.1 (float4_e2m1fn),
// E5M2 from the format list of "TileKernels 与 DeepGEMM 的分界线", §四 A, and
// E5M6 from per_token_cast_to_e5m6 of the operator table of the same page,
// §二 (12-bit codes, two per three bytes).
//
// gfx950 design. A contiguous [rows, cols] matrix with cols % G == 0 is one
// flat stream of groups: group k is elements [kG, kG + G) and owns scale
// sf[k], whatever the row length. The kernel walks that stream in 16-byte
// chunks (8 bf16 per lane, one global_load_dwordx4), so a group of G
// elements is G/8 consecutive lanes inside one DPP row; its abs-max is a
// 2-4 step DPP reduction in registers and no LDS is touched. Each lane then
// forms the scale, multiplies its 8 values and converts them with the
// hardware pack-converts: 8 E4M3 bytes (one dwordx2 store) or 8 E2M1 nibbles
// (one dword store); E5M6 codes are formed from the fp32 bits (no hardware
// converter) and stored as 12 bytes. The first lane of each group stores the scale.
// A workgroup keeps kUnroll chunks per lane in flight before using any.
#include "qcast_device.h"
#include "qcast_kernels.h"

namespace qcast {
namespace {

// Launch shape (compile-time; the defaults were chosen by measurement):
// chunks in flight per lane, and the cap on resident workgroups per CU for
// the persistent grid (0: one workgroup per kUnroll*256 chunks, no loop).
#ifndef QCAST_PT_UNROLL
#define QCAST_PT_UNROLL 2
#endif
#ifndef QCAST_PT_WG_PER_CU
#define QCAST_PT_WG_PER_CU 0
#endif
// Workgroup order of the one-shot grid. Natural order (consecutive
// workgroups go round-robin to the 8 XCDs) for row-major scales. With a
// column-major scale layout each XCD takes a contiguous range of the stream
// instead, so the scale words that neighbouring rows write into one line
// meet in one L2 and leave it as one write (measured 2.5% faster there and
// 3-6% slower for row-major scales, where the lines are never shared).
constexpr int kUnroll = QCAST_PT_UNROLL;
constexpr int kWgPerCu = QCAST_PT_WG_PER_CU;
constexpr int kXcds = 8;

template <int kLanes, int kFmt>
__global__ __launch_bounds__(kThreads) void per_token_kernel(
    const u32x4* __restrict__ x, int64_t nchunks, float floor, uint8_t* __restrict__ q,
    void* __restrict__ sf, SfLayout lay, uint32_t per_xcd) {
  uint32_t blk = blockIdx.x;
  if (per_xcd) blk = (blk % kXcds) * per_xcd + blk / kXcds;
  const int64_t step = (int64_t)gridDim.x * kThreads * kUnroll;
  for (int64_t base = (int64_t)blk * kThreads * kUnroll + threadIdx.x; base < nchunks;
       base += step) {
    u32x4 raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = base + (int64_t)u * kThreads;
      if (c < nchunks) raw[u] = load_stream(x + c);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = base + (int64_t)u * kThreads;
      // Whole groups are in or out together: nchunks is a multiple of kLanes
      // and c % 64 equals the lane index.
      if (c < nchunks) {
        float v[8];
        unpack8(raw[u], v);
        const float amax = lane_group_max<kLanes>(absmax8(v));
        Scale s = group_scale<kFmt>(amax, floor);
        if (lay.flags & kSfRound) s = round_scale_pow2(s);
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = v[i] * s.inv;
        if constexpr (kFmt == kE2M1) {
          store_stream(reinterpret_cast<uint32_t*>(q) + c, e2m1x8(y));
        } else if constexpr (kFmt == kE5M6) {
          const E5M6x8 p = e5m6x8(y);
          uint32_t* o = reinterpret_cast<uint32_t*>(q) + 3 * c;
          store_stream(o, p.w0);
          store_stream(o + 1, p.w1);
          store_stream(o + 2, p.w2);
        } else {
          u32x2 out;
          out.x = fp8x4<kFmt>(y[0], y[1], y[2], y[3]);
          out.y = fp8x4<kFmt>(y[4], y[5], y[6], y[7]);
          store_stream(reinterpret_cast<u32x2*>(q) + c, out);
        }
        store_group_scale<kLanes>(sf, (uint32_t)(c / kLanes), s, lay);
      }
    }
  }
}

// Column-major scales with 1 x 32 groups, fp32 or packed UE8M0:
// sf[group][row] puts a row's scales 4 * rows_pad bytes apart and a
// workgroup of the flat walk covers less than a row, so every scale (or
// packed word) would leave as a lone 4-byte store (fp32 scales: the cast 20%
// slower than with row-major scales). Here workgroup b casts a tile
// of kCmRows rows x kCmSpan chunks (two chunks per lane), parks the tile's
// scales in LDS and writes each group column's kCmRows consecutive rows as
// one 64-byte run (packed: each word column's, the word formed from the
// parked scales with no cross-lane gather). A tile 256 columns wide and 16
// rows tall ran 3% faster than one 128 wide and 32 tall; taller tiles, with
// longer scale runs, ran slower. Packed scales take 16.5 us here against
// 16.8 for the flat walk (4096 x 7168, interleaved, 150 rounds). Tiles walk
// the chunk columns fastest; the bottom and right tiles may be partial,
// always in whole groups (cols % 32 == 0).
constexpr int kCmSpan = 32;                          // chunks per tile row
constexpr int kCmRows = 2 * kThreads / kCmSpan;      // 16 rows

template <int kFmt, bool kPacked>
__global__ __launch_bounds__(kThreads) void per_token_cm32_kernel(
    const u32x4* __restrict__ x, uint32_t rows, uint32_t cpr, uint32_t col_tiles, float floor,
    uint8_t* __restrict__ q, float* __restrict__ sf, SfLayout lay) {
  constexpr int kLanes = 4;                          // lanes per 32-group
  constexpr int kGroupCols = kCmSpan / kLanes;
  static_assert(kGroupCols * kCmRows <= kThreads, "one scale store per lane at most");
  __shared__ float tile_sf[kGroupCols][kCmRows];
  const uint32_t rt = blockIdx.x / col_tiles;
  const uint32_t ct = blockIdx.x - rt * col_tiles;
  const uint32_t row0 = rt * kCmRows, c0 = ct * kCmSpan;
  const uint32_t nrows = rows - row0 < (uint32_t)kCmRows ? rows - row0 : (uint32_t)kCmRows;
  const uint32_t nspan = cpr - c0 < (uint32_t)kCmSpan ? cpr - c0 : (uint32_t)kCmSpan;
  u32x4 raw[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t l = threadIdx.x + u * kThreads;
    const uint32_t tr = l / kCmSpan, tc = l % kCmSpan;
    if (tr < nrows && tc < nspan) raw[u] = load_stream(x + ((int64_t)(row0 + tr) * cpr + c0 + tc));
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t l = threadIdx.x + u * kThreads;
    const uint32_t tr = l / kCmSpan, tc = l % kCmSpan;
    // a group's 4 lanes share tr and are all inside or all outside
    if (tr < nrows && tc < nspan) {
      float v[8];
      unpack8(raw[u], v);
      const float amax = lane_group_max<kLanes>(absmax8(v));
      Scale s = group_scale<kFmt>(amax, floor);
      if (lay.flags & kSfRound) s = round_scale_pow2(s);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = v[i] * s.inv;
      store_chunk8<kFmt>(q, (int64_t)(row0 + tr) * cpr + c0 + tc, v);
      if ((threadIdx.x & (kLanes - 1)) == 0) tile_sf[tc / kLanes][tr] = s.sf;
    }
  }
  __syncthreads();
  if constexpr (kPacked) {
    // word column wc of the tile: the exponent bytes of its groups 4wc..4wc+3
    // (power-of-two scales), for kCmRows consecutive rows from consecutive
    // lanes. Packed rows hold whole words (cols % 128 == 0), so a partial
    // tile holds whole words too.
    constexpr int kWordCols = kGroupCols / 4;
    const uint32_t wc = threadIdx.x / kCmRows, r = threadIdx.x % kCmRows;
    if (wc < (uint32_t)kWordCols && (wc + 1) * 4 * kLanes <= nspan && r < nrows) {
      uint32_t w = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) w |= (__float_as_uint(tile_sf[4 * wc + i][r]) >> 23) << (8 * i);
      reinterpret_cast<uint32_t*>(sf)[(size_t)(c0 / (4 * kLanes) + wc) * lay.rows_pad + row0 + r] =
          w;
    }
  } else {
    // group column gc of the tile: kCmRows consecutive rows from consecutive lanes
    const uint32_t gc = threadIdx.x / kCmRows, r = threadIdx.x % kCmRows;
    if (gc < (uint32_t)kGroupCols && gc * kLanes < nspan && r < nrows)
      sf[(size_t)(c0 / kLanes + gc) * lay.rows_pad + row0 + r] = tile_sf[gc][r];
  }
}

template <int kFmt>
hipError_t launch_cm32(const void* x, int64_t rows, int64_t cols, float floor, void* q, void* sf,
                       const SfLayout& lay, hipStream_t stream) {
  const int64_t cpr = cols / 8;
  const int64_t col_tiles = (cpr + kCmSpan - 1) / kCmSpan;
  const int64_t blocks = (rows + kCmRows - 1) / kCmRows * col_tiles;
  if (blocks >= (int64_t(1) << 31) || rows >= (int64_t(1) << 31) || cpr >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  auto kernel = (lay.flags & kSfPacked) ? per_token_cm32_kernel<kFmt, true>
                                        : per_token_cm32_kernel<kFmt, false>;
  launch_kernel(kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                static_cast<const u32x4*>(x), (uint32_t)rows, (uint32_t)cpr,
                (uint32_t)col_tiles, floor, static_cast<uint8_t*>(q), static_cast<float*>(sf),
                lay);
  return hipGetLastError();
}

template <int kLanes, int kFmt>
hipError_t launch(const void* x, int64_t nchunks, float floor, void* q, void* sf,
                  const SfLayout& lay, hipStream_t stream, const LaunchCaps& caps) {
  const int64_t per_block_iter = (int64_t)kThreads * kUnroll;
  const int64_t iters = (nchunks + per_block_iter - 1) / per_block_iter;
  // Persistent grid: at most kWgPerCu workgroups per CU, the same number of
  // iterations for every workgroup.
  const int64_t max_blocks = kWgPerCu > 0 ? (int64_t)caps.num_cus * kWgPerCu : iters;
  const int64_t iters_per_block = (iters + max_blocks - 1) / max_blocks;
  int64_t blocks = (iters + iters_per_block - 1) / iters_per_block;
  int64_t per_xcd = 0;
  if (kWgPerCu == 0 && (lay.flags & kSfColMajor)) {
    // Remapped workgroups past the end find base >= nchunks and do nothing.
    per_xcd = (blocks + kXcds - 1) / kXcds;
    blocks = per_xcd * kXcds;
  }
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  launch_kernel((per_token_kernel<kLanes, kFmt>), dim3((unsigned)blocks), dim3(kThreads), 0,
                stream, static_cast<const u32x4*>(x), nchunks, floor,
                static_cast<uint8_t*>(q), sf, lay, (uint32_t)per_xcd);
  return hipGetLastError();
}

template <int kFmt>
hipError_t launch_fmt(const void* x, int64_t nchunks, int group, float floor, void* q,
                      void* sf, const SfLayout& lay, hipStream_t stream,
                      const LaunchCaps& caps) {
  switch (group) {
    case 32: return launch<4, kFmt>(x, nchunks, floor, q, sf, lay, stream, caps);
    case 64: return launch<8, kFmt>(x, nchunks, floor, q, sf, lay, stream, caps);
    case 128: return launch<16, kFmt>(x, nchunks, floor, q, sf, lay, stream, caps);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_per_token(const void* x, int64_t rows, int64_t cols, int fmt, int group,
                            float floor, uint32_t sf_flags, void* q, void* sf,
                            hipStream_t stream, const LaunchCaps& caps) {
  const int64_t nchunks = rows * cols / 8;
  if (nchunks == 0) return hipSuccess;
  if (rows * cols / group >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const SfLayout lay = make_sf_layout(rows, cols, group, sf_flags);
  if (group == 32 && (lay.flags & kSfColMajor)) {
    switch (fmt) {
      case kE4M3: return launch_cm32<kE4M3>(x, rows, cols, floor, q, sf, lay, stream);
      case kE2M1: return launch_cm32<kE2M1>(x, rows, cols, floor, q, sf, lay, stream);
      case kE5M2: return launch_cm32<kE5M2>(x, rows, cols, floor, q, sf, lay, stream);
      case kE5M6: return launch_cm32<kE5M6>(x, rows, cols, floor, q, sf, lay, stream);
    }
    return hipErrorInvalidValue;
  }
  switch (fmt) {
    case kE4M3: return launch_fmt<kE4M3>(x, nchunks, group, floor, q, sf, lay, stream, caps);
    case kE2M1: return launch_fmt<kE2M1>(x, nchunks, group, floor, q, sf, lay, stream, caps);
    case kE5M2: return launch_fmt<kE5M2>(x, nchunks, group, floor, q, sf, lay, stream, caps);
    case kE5M6: return launch_fmt<kE5M6>(x, nchunks, group, floor, q, sf, lay, stream, caps);
  }
  return hipErrorInvalidValue;
}

}  // namespace qcast
