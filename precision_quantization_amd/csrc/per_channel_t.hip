// per_channel_t.hip -- per-channel cast of bf16 activations, written
// transposed, to E4M3 or E5M2.
//
// Operation: per_channel_cast (+transpose) of the operator table on the page
// "TileKernels 与 DeepGEMM 的分界线：DeepSeek 开源内核栈的分工", §二. The scale
// groups run along the token axis (128 tokens of one channel), the axis the
// weight-gradient GEMMs of §六 (steps 12 and 15, dW = X^T dY) contract over,
// and the codes are written channel-major so those tokens are contiguous.
// Scale rule and codes as in the per-token cast of "DeepSeek开源TileKernels：
// 用Python写的GPU算子逼近硬件性能上限", §3.1-§3.2.
//
// gfx950 design. A workgroup owns a tile of kTG token groups (128 tokens
// each) x 8*kCC channels. Lane (k, ch) loads the 16-byte chunk ch (8
// channels) of tokens 4k..4k+3 in each of kPasses passes, all loads issued
// before any is used; the data stays in registers as packed bf16.
// Column abs-maxima per token group: packed 16-bit maxima of the magnitude
// bits (v_pk_max_u16) over the lane's tokens, the same over the lanes that
// hold the same channel chunk (DPP / cross-lane), then a 4-wave LDS
// exchange; one lane per (group, channel) forms the scale. Each lane packs
// the codes of 4 tokens of one channel into a dword and writes it to an LDS
// tile [channel][token] whose dword index is XOR-swizzled by
// 4 * ((channel/8) mod 8): the eight channel chunks a half-wave writes land
// in distinct banks, and each 16-byte run of tokens stays contiguous and
// aligned, so the read-back is one ds_read_b128 per lane and the store is a
// full row of qT (128 * kTG bytes) per channel. (The pages' transpose pads
// its shared tile and rotates the column index for the same purpose; the
// XOR form keeps 16-byte reads aligned.) Workgroups are numbered so that
// each of the 8 XCDs walks a contiguous range of tiles, in strips of two
// channel tiles: token group outer, channel tile inner. Workgroups started
// together then read both 128-byte halves of the same 256-byte row segments
// and write neighbouring 128-byte pieces of the same qT rows and scale
// lines (measured about 3% faster than walking token groups of one channel
// tile, and much faster than walking channel tiles first).
#include "qcast_device.h"
#include "qcast_kernels.h"

namespace qcast {
namespace {

constexpr int kGroupTokens = 128;  // tokens per scale group
constexpr int kXcds = 8;

// Tile shape (compile-time; the default was chosen by measurement): token
// groups per tile and 8-channel chunks per tile.
#ifndef QCAST_PC_TG
#define QCAST_PC_TG 1
#endif
#ifndef QCAST_PC_CC
#define QCAST_PC_CC 8
#endif
// Order in which workgroups walk the tiles. Bit 0: 0 = token groups fastest,
// 1 = channel tiles fastest. Bit 1: 0 = each XCD takes a contiguous range,
// 1 = plain order. Bit 2: strips of QCAST_PC_STRIP channel tiles, token
// group outer and channel tile inner inside a strip (bit 0 ignored), so the
// tiles in flight cover a compact block of both the input and the output.
#ifndef QCAST_PC_ORDER
#define QCAST_PC_ORDER 4
#endif
#ifndef QCAST_PC_STRIP
#define QCAST_PC_STRIP 2
#endif
constexpr uint32_t kStrip = QCAST_PC_STRIP;
constexpr int kTG = QCAST_PC_TG;
constexpr int kCC = QCAST_PC_CC;
constexpr int kOrder = QCAST_PC_ORDER;
static_assert(kTG == 1 || kTG == 2, "1 or 2 token groups per tile");
static_assert(kCC == 8 || kCC == 16, "8 or 16 channel chunks per tile");

constexpr int kChannels = 8 * kCC;                  // channels per tile
constexpr int kTileTokens = kGroupTokens * kTG;     // tokens per tile
constexpr int kQuads = kThreads / kCC;              // token quads per pass
constexpr int kPassTokens = 4 * kQuads;             // tokens per pass
constexpr int kPasses = kTileTokens / kPassTokens;  // load passes per lane
constexpr int kPassesPerGroup = kPasses / kTG;
constexpr int kRowDw = kTileTokens / 4;             // dwords per LDS channel row
constexpr int kRowVec = kRowDw / 4;                 // 16-byte vectors per row
constexpr int kReadPasses = kChannels * kRowVec / kThreads;
static_assert(kPassesPerGroup >= 1 && kReadPasses >= 1, "tile shape");

// Dword index of token dword d of channel row c in the swizzled tile.
__device__ __forceinline__ int tile_index(int c, int d) {
  return c * kRowDw + (d ^ (4 * ((c >> 3) & 7)));
}

// Position of a tile: first channel, first token, valid channels and groups.
// Tile counts and in-tile offsets fit in 32 bits (checked by the launcher).
struct TileCoord {
  uint32_t c0, t0, gt;
  int nc, ng;
};

__device__ __forceinline__ TileCoord tile_coord(uint32_t tau, uint32_t ngroups, uint32_t cols,
                                                uint32_t nct, uint32_t ntg) {
  TileCoord tc;
  uint32_t ct;
  if (kOrder & 4) {
    const uint32_t strip = tau / (kStrip * ntg);
    const uint32_t width = nct - strip * kStrip < kStrip ? nct - strip * kStrip : kStrip;
    const uint32_t rem = tau - strip * kStrip * ntg;
    tc.gt = rem / width;
    ct = strip * kStrip + (rem - tc.gt * width);
  } else {
    ct = (kOrder & 1) ? tau % nct : tau / ntg;
    tc.gt = (kOrder & 1) ? tau / nct : tau - ct * ntg;
  }
  tc.c0 = ct * kChannels;
  tc.t0 = tc.gt * kTileTokens;
  tc.nc = (int)(cols - tc.c0 < (uint32_t)kChannels ? cols - tc.c0 : kChannels);
  tc.ng = (int)(ngroups - tc.gt * kTG < (uint32_t)kTG ? ngroups - tc.gt * kTG : kTG);
  return tc;
}

// Issue the lane's loads of a tile (zeros outside the tensor).
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ x, uint32_t cols,
                                          const TileCoord& tc, u32x4 (&raw)[kPasses][4]) {
  const int t = threadIdx.x;
  const int ch = t % kCC;
  const int k = t / kCC;
  const bool valid_ch = ch * 8 < tc.nc;
  // 64-bit tile base, 32-bit offsets inside the tile
  const uint16_t* base = x + (uint64_t)tc.t0 * cols + tc.c0;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const bool valid = valid_ch && (p / kPassesPerGroup) < tc.ng;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t off = (uint32_t)(p * kPassTokens + 4 * k + i) * cols + ch * 8;
      raw[p][i] = valid ? load_stream(reinterpret_cast<const u32x4*>(base + off))
                        : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

struct Smem {
  uint32_t tile[kChannels * kRowDw];
  float wave_amax[kTG][4][kChannels];
  float inv_s[kTG][kChannels];
};

// Scales, codes and stores of one tile whose values are in raw. Starts and
// ends with the workgroup converged; the LDS is free again on return.
template <int kFmt>
__device__ __forceinline__ void process_tile(const TileCoord& tc, const u32x4 (&raw)[kPasses][4],
                                             uint32_t rows, uint32_t ngroups, float floor,
                                             Smem& sm, uint8_t* __restrict__ qT,
                                             float* __restrict__ sf) {
  const int t = threadIdx.x;
  const int ch = t % kCC;
  const int k = t / kCC;
  const int wave = t >> 6;
  // Column abs-maxima per token group, as packed 16-bit magnitudes: word w
  // of a lane holds channels 8ch + 2w (low half) and 8ch + 2w + 1.
#pragma unroll
  for (int gi = 0; gi < kTG; ++gi) {
    uint32_t m[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int pp = 0; pp < kPassesPerGroup; ++pp) {
      const int p = gi * kPassesPerGroup + pp;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m[0] = pk_umax16(m[0], raw[p][i].x & 0x7fff7fffu);
        m[1] = pk_umax16(m[1], raw[p][i].y & 0x7fff7fffu);
        m[2] = pk_umax16(m[2], raw[p][i].z & 0x7fff7fffu);
        m[3] = pk_umax16(m[3], raw[p][i].w & 0x7fff7fffu);
      }
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (kCC == 8) m[w] = pk_umax16(m[w], dpp<kDppRor8>(m[w]));
      m[w] = pk_umax16(m[w], (uint32_t)__shfl_xor((int)m[w], 16));
      m[w] = pk_umax16(m[w], (uint32_t)__shfl_xor((int)m[w], 32));
    }
    if ((t & 63) < kCC) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        sm.wave_amax[gi][wave][ch * 8 + 2 * w] = bf16_lo(m[w]);
        sm.wave_amax[gi][wave][ch * 8 + 2 * w + 1] = bf16_hi(m[w]);
      }
    }
  }
  __syncthreads();
  if (t < kTG * kChannels) {
    const int gi = t / kChannels;
    const int c = t % kChannels;
    const float m = fmaxf(fmaxf(sm.wave_amax[gi][0][c], sm.wave_amax[gi][1][c]),
                          fmaxf(sm.wave_amax[gi][2][c], sm.wave_amax[gi][3][c]));
    const Scale s = group_scale<kFmt>(m, floor);
    sm.inv_s[gi][c] = s.inv;
    if (c < tc.nc && gi < tc.ng)
      sf[(uint64_t)tc.c0 * ngroups + (uint32_t)c * ngroups + tc.gt * kTG + gi] = s.sf;
  }
  __syncthreads();

  // Codes: for each pass and each of the lane's 8 channels, the 4 tokens
  // 4k..4k+3 of the pass as one dword of the channel's LDS row.
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int gi = p / kPassesPerGroup;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float inv = sm.inv_s[gi][ch * 8 + j];
      float y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t word = raw[p][i][j >> 1];
        y[i] = ((j & 1) ? bf16_hi(word) : bf16_lo(word)) * inv;
      }
      sm.tile[tile_index(ch * 8 + j, p * (kPassTokens / 4) + k)] =
          fp8x4<kFmt>(y[0], y[1], y[2], y[3]);
    }
  }
  __syncthreads();

  // Read back channel rows, 16 bytes per lane, and store them to qT.
  uint8_t* out = qT + (uint64_t)tc.c0 * rows + tc.t0;
#pragma unroll
  for (int r = 0; r < kReadPasses; ++r) {
    const int idx = t + r * kThreads;
    const int c = idx / kRowVec;
    const int mv = idx % kRowVec;
    if (c < tc.nc && mv * 16 < tc.ng * kGroupTokens) {
      const u32x4 val = *reinterpret_cast<const u32x4*>(&sm.tile[tile_index(c, 4 * mv)]);
      store_stream(reinterpret_cast<u32x4*>(out + (uint32_t)c * rows + mv * 16), val);
    }
  }
  __syncthreads();  // the LDS tile is reused by the next tile
}

// One workgroup per tile.
template <int kFmt>
__global__ __launch_bounds__(kThreads) void per_channel_t_kernel(
    const uint16_t* __restrict__ x, uint32_t rows, uint32_t cols, uint32_t ngroups,
    uint32_t nct, uint32_t ntiles, uint32_t per_xcd, float floor, uint8_t* __restrict__ qT,
    float* __restrict__ sf) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  const uint32_t b = blockIdx.x;
  const uint32_t tau = (kOrder & 2) ? b : (b % kXcds) * per_xcd + b / kXcds;
  if (tau >= ntiles) return;
  const TileCoord tc = tile_coord(tau, ngroups, cols, nct, ntiles / nct);
  u32x4 raw[kPasses][4];
  load_tile(x, cols, tc, raw);
  process_tile<kFmt>(tc, raw, rows, ngroups, floor, sm, qT, sf);
}

}  // namespace

hipError_t launch_per_channel_T(const void* x, int64_t rows, int64_t cols, int fmt, float floor,
                                void* qT, float* sf, hipStream_t stream,
                                const LaunchCaps& caps) {
  (void)caps;
  const int64_t ngroups = rows / kGroupTokens;
  const int64_t ntg = (ngroups + kTG - 1) / kTG;
  const int64_t nct = (cols + kChannels - 1) / kChannels;
  const int64_t ntiles = ntg * nct;
  if (ntiles == 0) return hipSuccess;
  // The kernels index tiles, and offsets inside a tile's rows, in 32 bits.
  const int64_t lim = int64_t(1) << 31;
  if (ntiles + 2 * kXcds >= lim || (int64_t)kTileTokens * cols >= lim ||
      (int64_t)kChannels * rows >= lim || rows >= lim || cols >= lim)
    return hipErrorInvalidValue;
  const int64_t per_xcd = (ntiles + kXcds - 1) / kXcds;
  const int64_t grid = (kOrder & 2) ? ntiles : per_xcd * kXcds;
  auto kernel = fmt == kE4M3 ? per_channel_t_kernel<kE4M3>
               : fmt == kE5M2 ? per_channel_t_kernel<kE5M2> : nullptr;
  if (!kernel) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(x), (uint32_t)rows, (uint32_t)cols,
                     (uint32_t)ngroups, (uint32_t)nct, (uint32_t)ntiles, (uint32_t)per_xcd, floor,
                     static_cast<uint8_t*>(qT), sf);
  return hipGetLastError();
}

}  // namespace qcast
