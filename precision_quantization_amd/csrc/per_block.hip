// per_block.hip -- per-block (128 x 128) cast of a bf16 weight to E4M3.
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
// wave load instruction reads four full 256-byte row segments. The tile's
// abs-max is a register max over the 64 values, a DPP + cross-row reduction
// inside each wave, and a 4-entry LDS exchange between the waves. Every lane
// then forms the scale, converts its 64 values and stores 8 dwordx2; lane 0
// stores the tile's scale. Tiles are independent, so the grid is one
// workgroup per tile and the hardware balances them across the CUs.
#include "qcast_device.h"
#include "qcast_kernels.h"

namespace qcast {
namespace {

constexpr int kBlock = 128;
constexpr int kRowsPerPass = kThreads / (kBlock / 8);   // 16
constexpr int kPasses = kBlock / kRowsPerPass;          // 8

__global__ __launch_bounds__(kThreads) void per_block_kernel(
    const uint16_t* __restrict__ x, int64_t cols, int64_t bcols, int64_t nblocks, float floor,
    uint8_t* __restrict__ q, float* __restrict__ sf) {
  __shared__ float wave_amax[kThreads / 64];
  const int t = threadIdx.x;
  const int cc = t & 15;
  const int r0 = t >> 4;
  for (int64_t b = blockIdx.x; b < nblocks; b += gridDim.x) {
    const int64_t bi = b / bcols;
    const int64_t bj = b - bi * bcols;
    const int64_t first = (bi * kBlock + r0) * cols + bj * kBlock + cc * 8;
    u32x4 raw[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
      raw[p] = load_stream(reinterpret_cast<const u32x4*>(x + first + (int64_t)p * kRowsPerPass * cols));
    float v[kPasses][8];
    float m = 0.0f;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      unpack8(raw[p], v[p]);
      m = fmaxf(m, absmax8(v[p]));
    }
    m = wave_max(m);
    if ((t & 63) == 0) wave_amax[t >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(wave_amax[0], wave_amax[1]), fmaxf(wave_amax[2], wave_amax[3]));
    const Scale s = group_scale<kE4M3>(m, floor);
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      u32x2 out;
      out.x = e4m3x4(v[p][0] * s.inv, v[p][1] * s.inv, v[p][2] * s.inv, v[p][3] * s.inv);
      out.y = e4m3x4(v[p][4] * s.inv, v[p][5] * s.inv, v[p][6] * s.inv, v[p][7] * s.inv);
      store_stream(reinterpret_cast<u32x2*>(q + first + (int64_t)p * kRowsPerPass * cols), out);
    }
    if (t == 0) sf[b] = s.sf;
    __syncthreads();  // wave_amax is rewritten by the next tile
  }
}

}  // namespace

hipError_t launch_per_block(const void* x, int64_t rows, int64_t cols, float floor, void* q,
                            float* sf, hipStream_t stream, const LaunchCaps& caps) {
  const int64_t bcols = cols / kBlock;
  const int64_t nblocks = (rows / kBlock) * bcols;
  if (nblocks == 0) return hipSuccess;
  (void)caps;
  const int64_t grid = nblocks < (int64_t(1) << 30) ? nblocks : (int64_t(1) << 30);
  hipLaunchKernelGGL(per_block_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(x), cols, bcols, nblocks, floor,
                     static_cast<uint8_t*>(q), sf);
  return hipGetLastError();
}

}  // namespace qcast
