// per_channel.hip -- per-channel cast of bf16 activations to E4M3, E5M2,
// packed E2M1 or packed E5M6, codes kept in the input layout.
//
// Operation: per_channel_cast (without the transpose) of the operator table
// on the page "TileKernels 与 DeepGEMM 的分界线：DeepSeek 开源内核栈的分工", §二:
// the scale groups run along the token axis (128 tokens of one channel), as
// for the transposed form, but code x[t][c] stays at q[t][c] and the scale
// of group g of channel c is stored at sf[g][c] (one scale line per token
// group, contiguous over channels). Scale rule and codes as in the per-token
// cast of "DeepSeek开源TileKernels：用Python写的GPU算子逼近硬件性能上限",
// §3.1-§3.2.
//
// gfx950 design. No data moves between lanes except the column maxima: a
// workgroup owns 128 tokens x 256 channels; lane (k, ch) loads the 16-byte
// chunk ch (8 channels) of the 16 tokens k, k + 8, ..., k + 120, so each
// wave reads two whole 512-byte row segments per load instruction and keeps
// 16 chunks in flight per lane. The column abs-maxima are packed 16-bit
// maxima of the magnitude bits over the lane's tokens, one cross-lane step
// inside the wave, then a 4-wave exchange in LDS; thread t forms the scale of
// channel t and writes the workgroup's 256 scales as one contiguous line.
// Each lane then converts its own values and writes 8 codes per token: each
// store instruction of a wave covers two 256-byte row segments of q (128-byte
// segments of E2M1 nibbles, 384-byte segments of E5M6 codes).
#include "qcast_device.h"
#include "qcast_kernels.h"

namespace qcast {
namespace {

constexpr int kGroupTokens = 128;             // tokens per scale group
constexpr int kChunks = 32;                   // 8-channel chunks per tile
constexpr int kTileChannels = 8 * kChunks;    // 256
constexpr int kSlices = kThreads / kChunks;   // 8 token slices
constexpr int kTokensPerLane = kGroupTokens / kSlices;  // 16
static_assert(kTileChannels == kThreads, "one scale per thread");

template <int kFmt>
__global__ __launch_bounds__(kThreads) void per_channel_kernel(
    const uint16_t* __restrict__ x, uint32_t cols, uint32_t nct, float floor, uint32_t round_sf,
    uint8_t* __restrict__ q, float* __restrict__ sf) {
  __shared__ float wave_amax[kThreads / 64][kTileChannels];
  __shared__ __attribute__((aligned(16))) float inv_s[kTileChannels];
  const int t = threadIdx.x;
  const int ch = t % kChunks;
  const int k = t / kChunks;
  const int wave = t >> 6;
  const uint32_t g = blockIdx.x / nct;
  const uint32_t c0 = (blockIdx.x - g * nct) * kTileChannels;
  const bool valid = c0 + 8 * ch < cols;
  // 64-bit tile base, 32-bit offsets inside the tile
  const uint64_t tile_base = (uint64_t)g * kGroupTokens * cols + c0;
  const uint16_t* xb = x + tile_base;

  u32x4 raw[kTokensPerLane];
#pragma unroll
  for (int j = 0; j < kTokensPerLane; ++j) {
    const uint32_t off = (uint32_t)(k + kSlices * j) * cols + 8 * ch;
    raw[j] = valid ? load_stream(reinterpret_cast<const u32x4*>(xb + off))
                   : u32x4{0u, 0u, 0u, 0u};
  }

  // Column abs-maxima: word w holds channels 8ch + 2w (low) and 8ch + 2w + 1.
  uint32_t m[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < kTokensPerLane; ++j) {
    m[0] = pk_umax16(m[0], raw[j].x & 0x7fff7fffu);
    m[1] = pk_umax16(m[1], raw[j].y & 0x7fff7fffu);
    m[2] = pk_umax16(m[2], raw[j].z & 0x7fff7fffu);
    m[3] = pk_umax16(m[3], raw[j].w & 0x7fff7fffu);
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) m[w] = pk_max_xor32(m[w]);
  if ((t & 63) < kChunks) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wave_amax[wave][8 * ch + 2 * w] = bf16_lo(m[w]);
      wave_amax[wave][8 * ch + 2 * w + 1] = bf16_hi(m[w]);
    }
  }
  __syncthreads();
  {
    float a = wave_amax[0][t];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) a = fmaxf(a, wave_amax[w][t]);
    Scale s = group_scale<kFmt>(a, floor);
    if (round_sf) s = round_scale_pow2(s);
    inv_s[t] = s.inv;
    if (c0 + t < cols) sf[(uint64_t)g * cols + c0 + t] = s.sf;
  }
  __syncthreads();

  if (!valid) return;
  float inv[8];
  *reinterpret_cast<float4*>(&inv[0]) = *reinterpret_cast<const float4*>(&inv_s[8 * ch]);
  *reinterpret_cast<float4*>(&inv[4]) = *reinterpret_cast<const float4*>(&inv_s[8 * ch + 4]);
  uint8_t* qb = q + code_bytes<kFmt>(tile_base);
#pragma unroll
  for (int j = 0; j < kTokensPerLane; ++j) {
    float v[8];
    unpack8(raw[j], v);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= inv[i];
    const uint32_t off = (uint32_t)(k + kSlices * j) * cols + 8 * ch;
    store_chunk8<kFmt>(qb, off / 8, v);
  }
}

}  // namespace

bool per_channel_fits(int64_t rows, int64_t cols) {
  const int64_t lim = int64_t(1) << 31;
  const int64_t nct = (cols + kTileChannels - 1) / kTileChannels;
  return (rows / kGroupTokens) * nct < lim && (int64_t)kGroupTokens * cols < lim;
}

hipError_t launch_per_channel(const void* x, int64_t rows, int64_t cols, int fmt, float floor,
                              uint32_t sf_flags, void* q, float* sf, hipStream_t stream,
                              const LaunchCaps& caps) {
  (void)caps;
  const int64_t ngroups = rows / kGroupTokens;
  const int64_t nct = (cols + kTileChannels - 1) / kTileChannels;
  const int64_t ntiles = ngroups * nct;
  if (ntiles == 0) return hipSuccess;
  // Tile counts and in-tile offsets are 32-bit.
  if (!per_channel_fits(rows, cols)) return hipErrorInvalidValue;
  auto kernel = fmt == kE4M3 ? per_channel_kernel<kE4M3>
               : fmt == kE5M2 ? per_channel_kernel<kE5M2>
               : fmt == kE2M1 ? per_channel_kernel<kE2M1>
               : fmt == kE5M6 ? per_channel_kernel<kE5M6> : nullptr;
  if (!kernel) return hipErrorInvalidValue;
  launch_kernel(kernel, dim3((unsigned)ntiles), dim3(kThreads), 0, stream,
                static_cast<const uint16_t*>(x), (uint32_t)cols, (uint32_t)nct, floor,
                (uint32_t)(sf_flags & kSfRound), static_cast<uint8_t*>(q), sf);
  return hipGetLastError();
}

}  // namespace qcast
