// per_channel_t.hip -- per-channel cast of bf16 activations, written
// transposed, to E4M3.
//
// Operation: per_channel_cast (+transpose) of the operator table on the page
// "TileKernels 与 DeepGEMM 的分界线：DeepSeek 开源内核栈的分工", §二. The scale
// groups run along the token axis (128 tokens of one channel), the axis the
// weight-gradient GEMMs of §六 (steps 12 and 15, dW = X^T dY) contract over,
// and the codes are written channel-major so those tokens are contiguous.
// Scale rule and codes as in the per-token cast of "DeepSeek开源TileKernels：
// 用Python写的GPU算子逼近硬件性能上限", §3.1-§3.2.
//
// gfx950 design. A workgroup owns a tile of 128 tokens x 64 channels: one
// token group for 64 channels. Lane (k, ch) loads the 16-byte chunk ch
// (8 channels) of tokens 4k..4k+3, so each wave load reads eight 128-byte row
// segments. Column abs-maxima: a register max over the lane's 4 tokens, a DPP
// and two cross-lane steps over the 8 token quads of the wave, then a
// 4 x 64 LDS exchange; 64 lanes form the 64 scales. Each lane packs the
// codes of its 4 tokens of one channel into a dword and writes it to an LDS
// tile [channel][token] whose dword index is XOR-swizzled by 4 * (channel/8):
// the eight channels groups a half-wave writes land in distinct banks, and a
// 16-byte run of tokens stays contiguous, so the read-back is one
// ds_read_b128 per lane, conflict-free, and the store is a full 128-byte row
// of qT per 8 lanes. (The pages' transpose pads its shared tile and rotates
// the column index for the same purpose; the XOR form keeps 16-byte reads
// aligned.) Workgroups are numbered so that each of the 8 XCDs walks a
// contiguous range of tiles with the token group fastest: neighbouring tiles
// on one XCD fill the same scale lines in its L2.
#include "qcast_device.h"
#include "qcast_kernels.h"

namespace qcast {
namespace {

constexpr int kTokens = 128;       // tokens per tile = scale group
constexpr int kChannels = 64;      // channels per tile
constexpr int kXcds = 8;

// Order in which workgroups walk the tiles (compile-time; default chosen by
// measurement). Bit 0: 0 = token group fastest, 1 = channel tile fastest.
// Bit 1: 0 = each XCD takes a contiguous range of tiles, 1 = plain order.
#ifndef QCAST_PC_ORDER
#define QCAST_PC_ORDER 0
#endif
constexpr int kOrder = QCAST_PC_ORDER;

__global__ __launch_bounds__(kThreads) void per_channel_t_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ngroups,
    int64_t ntiles, int64_t per_xcd, float floor, uint8_t* __restrict__ qT,
    float* __restrict__ sf) {
  __shared__ __attribute__((aligned(16))) uint32_t tile[kChannels * (kTokens / 4)];  // 8 KiB
  __shared__ __attribute__((aligned(16))) float wave_amax[4][kChannels];
  __shared__ float inv_s[kChannels];

  const int64_t b = blockIdx.x;
  const int64_t tau = (kOrder & 2) ? b : (b % kXcds) * per_xcd + b / kXcds;
  if (tau >= ntiles) return;
  const int64_t nct = ntiles / ngroups;
  const int64_t ct = (kOrder & 1) ? tau % nct : tau / ngroups;
  const int64_t g = (kOrder & 1) ? tau / nct : tau - ct * ngroups;
  const int64_t c0 = ct * kChannels;
  const int64_t t0 = g * kTokens;
  const int nc = (int)(cols - c0 < kChannels ? cols - c0 : kChannels);

  const int t = threadIdx.x;
  const int ch = t & 7;        // channel chunk: channels c0 + 8ch .. +7
  const int k = t >> 3;        // token quad: tokens t0 + 4k .. +3
  const bool valid = ch * 8 < nc;

  u32x4 raw[4];
  if (valid) {
    const uint16_t* src = x + (t0 + 4 * k) * cols + c0 + ch * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = load_stream(reinterpret_cast<const u32x4*>(src + i * cols));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = u32x4{0u, 0u, 0u, 0u};
  }
  float v[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) unpack8(raw[i], v[i]);

  // Column abs-max over the wave's 32 tokens: own 4 tokens, then the lanes
  // holding the same channel chunk (lane ^ 8, ^ 16, ^ 32).
  float pm[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float m = fmaxf(fmaxf(fabsf(v[0][j]), fabsf(v[1][j])), fmaxf(fabsf(v[2][j]), fabsf(v[3][j])));
    uint32_t b = __float_as_uint(m);
    b = umax(b, dpp<kDppRor8>(b));
    b = umax(b, (uint32_t)__shfl_xor((int)b, 16));
    b = umax(b, (uint32_t)__shfl_xor((int)b, 32));
    pm[j] = __uint_as_float(b);
  }
  const int wave = t >> 6;
  if ((t & 63) < 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) wave_amax[wave][ch * 8 + j] = pm[j];
  }
  __syncthreads();
  if (t < kChannels) {
    const float m = fmaxf(fmaxf(wave_amax[0][t], wave_amax[1][t]),
                          fmaxf(wave_amax[2][t], wave_amax[3][t]));
    const Scale s = group_scale<kE4M3>(m, floor);
    inv_s[t] = s.inv;
    if (t < nc) sf[(c0 + t) * ngroups + g] = s.sf;
  }
  __syncthreads();

  // Codes of tokens 4k..4k+3 for each of the lane's 8 channels, one dword
  // per channel, into the swizzled [channel][token dword] tile.
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float inv = inv_s[ch * 8 + j];
    const uint32_t word = e4m3x4(v[0][j] * inv, v[1][j] * inv, v[2][j] * inv, v[3][j] * inv);
    const int c = ch * 8 + j;
    tile[c * (kTokens / 4) + (k ^ (4 * ch))] = word;
  }
  __syncthreads();

  // Read back channel rows: 8 lanes x 16 bytes per 128-token row.
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int idx = t + p * kThreads;
    const int c = idx >> 3;
    const int m4 = (idx & 7) * 4;
    if (c < nc) {
      const u32x4 val =
          *reinterpret_cast<const u32x4*>(&tile[c * (kTokens / 4) + (m4 ^ (4 * (c >> 3)))]);
      store_stream(reinterpret_cast<u32x4*>(qT + (c0 + c) * rows + t0 + m4 * 4), val);
    }
  }
}

}  // namespace

hipError_t launch_per_channel_T(const void* x, int64_t rows, int64_t cols, float floor,
                                void* qT, float* sf, hipStream_t stream,
                                const LaunchCaps& caps) {
  (void)caps;
  const int64_t ngroups = rows / kTokens;
  const int64_t nctiles = (cols + kChannels - 1) / kChannels;
  const int64_t ntiles = ngroups * nctiles;
  if (ntiles == 0) return hipSuccess;
  const int64_t per_xcd = (ntiles + kXcds - 1) / kXcds;
  const int64_t grid = per_xcd * kXcds;
  if (grid >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(per_channel_t_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(x), rows, cols, ngroups, ntiles, per_xcd,
                     floor, static_cast<uint8_t*>(qT), sf);
  return hipGetLastError();
}

}  // namespace qcast
