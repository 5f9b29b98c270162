// per_block.hip -- per-block (128 x 128) cast of a bf16 weight to E4M3 or E5M2.
//
// Operation: per_block_cast of the operator table on the page
// "TileKernels 与 DeepGEMM 的分界线：DeepSeek 开源内核栈的分工", §二 (one scale
// per 128 x 128 tile of the weight); the scale rule and the codes are those
// of the per-token cast on "DeepSeek开源TileKernels：用Python写的GPU算子逼近硬件
// 性能上限", §3.1-§3.2, with the tile as the group.
//
// gfx950 design. One 256-thread workgroup per tile. Lane (r0, cc) of the
// workgroup owns the 16-byte chunk cc (8 columns) of tile rows r0, r0 + 16,
// ..., r0 + 112: eight dwordx4 loads, all issued before any is used, so each
// wave load instruction reads four full 256-byte row segments. The values
// stay packed as bf16 in registers (32 VGPRs); the tile's abs-max is a
// packed 16-bit max of their magnitude bits (v_pk_max_u16), a DPP +
// cross-row reduction inside each wave, and a 4-entry LDS exchange between
// the waves. Every lane
// then forms the scale, converts its 64 values and stores 8 dwordx2; lane 0
// stores the tile's scale. Tiles are independent, so the grid is one
// workgroup per tile and the hardware balances them across the CUs. Tile
// indices and in-tile offsets are 32-bit; only the tile base is 64-bit.
#include "qcast_device.h"
#include "qcast_kernels.h"

namespace qcast {
namespace {

constexpr int kBlock = 128;
constexpr int kRowsPerPass = kThreads / (kBlock / 8);   // 16
constexpr int kPasses = kBlock / kRowsPerPass;          // 8

template <int kFmt>
__global__ __launch_bounds__(kThreads) void per_block_kernel(
    const uint16_t* __restrict__ x, uint32_t cols, uint32_t bcols, float floor,
    uint8_t* __restrict__ q, float* __restrict__ sf) {
  __shared__ float wave_amax[kThreads / 64];
  const int t = threadIdx.x;
  const int cc = t & 15;
  const int r0 = t >> 4;
  const uint32_t b = blockIdx.x;
  const uint32_t bi = b / bcols;
  const uint32_t bj = b - bi * bcols;
  // 64-bit tile base, 32-bit offsets inside the tile (checked by the launcher)
  const uint64_t tile = (uint64_t)bi * kBlock * cols + (uint64_t)bj * kBlock;
  const uint16_t* src = x + tile;
  uint8_t* dst = q + tile;
  u32x4 raw[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const uint32_t off = (uint32_t)(r0 + p * kRowsPerPass) * cols + cc * 8;
    raw[p] = load_stream(reinterpret_cast<const u32x4*>(src + off));
  }
  // Abs-max as packed 16-bit magnitudes of the bf16 values, then the larger
  // half; the values stay packed in registers until they are encoded.
  uint32_t m16 = 0u;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    m16 = pk_umax16(m16, raw[p].x & 0x7fff7fffu);
    m16 = pk_umax16(m16, raw[p].y & 0x7fff7fffu);
    m16 = pk_umax16(m16, raw[p].z & 0x7fff7fffu);
    m16 = pk_umax16(m16, raw[p].w & 0x7fff7fffu);
  }
  float m = fmaxf(bf16_lo(m16), bf16_hi(m16));
  m = wave_max(m);
  if ((t & 63) == 0) wave_amax[t >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wave_amax[0], wave_amax[1]), fmaxf(wave_amax[2], wave_amax[3]));
  const Scale s = group_scale<kFmt>(m, floor);
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    float v[8];
    unpack8(raw[p], v);
    u32x2 out;
    out.x = fp8x4<kFmt>(v[0] * s.inv, v[1] * s.inv, v[2] * s.inv, v[3] * s.inv);
    out.y = fp8x4<kFmt>(v[4] * s.inv, v[5] * s.inv, v[6] * s.inv, v[7] * s.inv);
    const uint32_t off = (uint32_t)(r0 + p * kRowsPerPass) * cols + cc * 8;
    store_stream(reinterpret_cast<u32x2*>(dst + off), out);
  }
  if (t == 0) sf[b] = s.sf;
}

}  // namespace

bool per_block_fits(int64_t rows, int64_t cols) {
  const int64_t lim = int64_t(1) << 31;
  return (rows / kBlock) * (cols / kBlock) < lim && (int64_t)kBlock * cols < lim;
}

hipError_t launch_per_block(const void* x, int64_t rows, int64_t cols, int fmt, float floor,
                            void* q, float* sf, hipStream_t stream, const LaunchCaps& caps) {
  (void)caps;
  const int64_t bcols = cols / kBlock;
  const int64_t nblocks = (rows / kBlock) * bcols;
  if (nblocks == 0) return hipSuccess;
  // One workgroup per tile; tile counts and in-tile offsets in 32 bits.
  if (!per_block_fits(rows, cols)) return hipErrorInvalidValue;
  if (fmt == kE4M3)
    launch_kernel(per_block_kernel<kE4M3>, dim3((unsigned)nblocks), dim3(kThreads), 0, stream,
                  static_cast<const uint16_t*>(x), (uint32_t)cols, (uint32_t)bcols, floor,
                  static_cast<uint8_t*>(q), sf);
  else if (fmt == kE5M2)
    launch_kernel(per_block_kernel<kE5M2>, dim3((unsigned)nblocks), dim3(kThreads), 0, stream,
                  static_cast<const uint16_t*>(x), (uint32_t)cols, (uint32_t)bcols, floor,
                  static_cast<uint8_t*>(q), sf);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace qcast
