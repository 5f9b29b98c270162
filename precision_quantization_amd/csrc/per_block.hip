// per_block.hip -- per-block (128 x 128) cast of a bf16 weight to E4M3, E5M2,
// packed E2M1 or packed E5M6.
//
// Operation: per_block_cast of the operator table on the page
// "TileKernels 与 DeepGEMM 的分界线：DeepSeek 开源内核栈的分工", §二 (one scale
// per 128 x 128 tile of the weight); the scale rule and the codes are those
// of the per-token cast on "DeepSeek开源TileKernels：用Python写的GPU算子逼近硬件
// 性能上限", §3.1-§3.2, with the tile as the group.
//
// gfx950 design. One 256-thread workgroup per pair of horizontally
// adjacent tiles (one tile when the tile columns are odd in number). Lane
// (r0, cc) owns the 16-byte chunk cc (8 columns) of rows r0, r0 + 8, ...,
// r0 + 120 of the pair: sixteen dwordx4 loads, all issued before any is
// used, so each wave load instruction reads two full 512-byte row segments
// (measured 5% faster than one tile of 256-byte segments per workgroup).
// The values stay packed as bf16 in registers; each tile's abs-max is a
// packed 16-bit max of their magnitude bits (v_pk_max_u16), a DPP reduction
// inside each 16-lane row (one tile's columns of one row), one cross-row
// shuffle, and a 4-wave LDS exchange. Every lane then forms its tile's
// scale, converts its 128 values and stores 16 chunks of 8 codes (dwordx2
// for the 8-bit formats, a dword of E2M1 nibbles, 12 bytes of E5M6 codes; the
// formats of the TileKernels overview of "DeepSeek 的 GPU 内核帝国", quant/:
// FP8 / FP4 / E5M6 at per-block granularity); the first lane of
// each tile stores the tile's scale. Tiles are independent, so the grid is
// one workgroup per pair and the hardware balances them across the CUs.
// Tile indices and in-tile offsets are 32-bit; only the tile base is 64-bit.
#include "qcast_device.h"
#include "qcast_kernels.h"

namespace qcast {
namespace {

constexpr int kBlock = 128;

// kSpan tiles side by side per workgroup.
template <int kFmt, int kSpan>
__global__ __launch_bounds__(kThreads) void per_block_kernel(
    const uint16_t* __restrict__ x, uint32_t cols, uint32_t bcols, float floor,
    uint32_t round_sf, uint8_t* __restrict__ q, float* __restrict__ sf) {
  constexpr int kChunksPerRow = kSpan * kBlock / 8;       // lanes per row: 16 or 32
  constexpr int kRowsPerPass = kThreads / kChunksPerRow;  // 16 or 8
  constexpr int kPasses = kBlock / kRowsPerPass;          // 8 or 16
  static_assert(kSpan == 1 || kSpan == 2, "one or two tiles per workgroup");
  __shared__ float wave_amax[kThreads / 64][kSpan];
  const int t = threadIdx.x;
  const int cc = t % kChunksPerRow;
  const int r0 = t / kChunksPerRow;
  const int ti = cc >> 4;   // tile of the lane's chunk inside the span
  const uint32_t b = blockIdx.x;
  const uint32_t spans = bcols / kSpan;
  const uint32_t bi = b / spans;
  const uint32_t bj = kSpan * (b - bi * spans);
  // 64-bit tile base, 32-bit offsets inside the tiles (checked by the launcher)
  const uint64_t tile = (uint64_t)bi * kBlock * cols + (uint64_t)bj * kBlock;
  const uint16_t* src = x + tile;
  uint8_t* dst = q + code_bytes<kFmt>(tile);
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
  // A 16-lane DPP row holds one tile's 128 columns of one row; the rows of
  // a wave that hold the same tile are kChunksPerRow lanes apart.
  uint32_t mb = __float_as_uint(lane_group_max<16>(fmaxf(bf16_lo(m16), bf16_hi(m16))));
  if (kChunksPerRow == 16) mb = max_xor16(mb);
  mb = max_xor32(mb);
  if ((t & 63) < kChunksPerRow && (t & 15) == 0) wave_amax[t >> 6][ti] = __uint_as_float(mb);
  __syncthreads();
  const float m = fmaxf(fmaxf(wave_amax[0][ti], wave_amax[1][ti]),
                        fmaxf(wave_amax[2][ti], wave_amax[3][ti]));
  Scale s = group_scale<kFmt>(m, floor);
  if (round_sf) s = round_scale_pow2(s);
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    float v[8];
    unpack8(raw[p], v);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= s.inv;
    const uint32_t off = (uint32_t)(r0 + p * kRowsPerPass) * cols + cc * 8;
    store_chunk8<kFmt>(dst, off / 8, v);
  }
  if (t < kChunksPerRow && (t & 15) == 0) sf[(uint64_t)bi * bcols + bj + ti] = s.sf;
}

template <int kFmt>
hipError_t launch_fmt(const uint16_t* x, int64_t nblocks, int64_t cols, int64_t bcols,
                      float floor, uint32_t round_sf, uint8_t* q, float* sf,
                      hipStream_t stream) {
  if (bcols % 2 == 0)
    launch_kernel(per_block_kernel<kFmt, 2>, dim3((unsigned)(nblocks / 2)), dim3(kThreads), 0,
                  stream, x, (uint32_t)cols, (uint32_t)bcols, floor, round_sf, q, sf);
  else
    launch_kernel(per_block_kernel<kFmt, 1>, dim3((unsigned)nblocks), dim3(kThreads), 0,
                  stream, x, (uint32_t)cols, (uint32_t)bcols, floor, round_sf, q, sf);
  return hipGetLastError();
}

}  // namespace

bool per_block_fits(int64_t rows, int64_t cols) {
  const int64_t lim = int64_t(1) << 31;
  return (rows / kBlock) * (cols / kBlock) < lim && (int64_t)kBlock * cols < lim;
}

hipError_t launch_per_block(const void* x, int64_t rows, int64_t cols, int fmt, float floor,
                            uint32_t sf_flags, void* q, float* sf, hipStream_t stream,
                            const LaunchCaps& caps) {
  (void)caps;
  const int64_t bcols = cols / kBlock;
  const int64_t nblocks = (rows / kBlock) * bcols;
  if (nblocks == 0) return hipSuccess;
  // Tile counts and in-tile offsets in 32 bits.
  if (!per_block_fits(rows, cols)) return hipErrorInvalidValue;
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  uint8_t* qp = static_cast<uint8_t*>(q);
  const uint32_t r = sf_flags & kSfRound;
  switch (fmt) {
    case kE4M3: return launch_fmt<kE4M3>(xp, nblocks, cols, bcols, floor, r, qp, sf, stream);
    case kE5M2: return launch_fmt<kE5M2>(xp, nblocks, cols, bcols, floor, r, qp, sf, stream);
    case kE2M1: return launch_fmt<kE2M1>(xp, nblocks, cols, bcols, floor, r, qp, sf, stream);
    case kE5M6: return launch_fmt<kE5M6>(xp, nblocks, cols, bcols, floor, r, qp, sf, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace qcast
