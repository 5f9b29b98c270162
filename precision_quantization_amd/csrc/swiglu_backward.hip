// swiglu_backward.hip -- SwiGLU backward fused with the per-token cast (E4M3,
// E5M2, packed E2M1 or packed E5M6) of the two input gradients.
//
// Operation: swiglu_backward_and_per_token_cast of the operator table on the
// page "TileKernels 与 DeepGEMM 的分界线：DeepSeek 开源内核栈的分工", §二 (the
// backward of the SwiGLU of "DeepSeek开源TileKernels：用Python写的GPU算子逼近硬件
// 性能上限", §3.3, step 13 of the training step in §六 of the first page). For
// v = silu(g) * u * w with the gradient dv of v:
//   s = 1 / (1 + exp(-g)), silu = g * s, silu' = s + silu * (1 - s),
//   dg = (dv * w) * u * silu',  du = (dv * w) * silu,
// evaluated in fp32 on the clamped g, u when a clamp c > 0 is given, with a
// zero gradient where the clamp changed the value (g > c; |u| > c). The row
// [dg | du] (2 * cols values) is then cast per token like any other row:
// one code row of 2 * cols columns per row, scales [rows, 2 * cols / group]
// or, on request, in the per-token scale layouts of those rows (round_sf,
// TMA-aligned column-major, packed UE8M0: the cast config of the second
// page, §3.1, and the consumer layouts of the first page, §四 C). The same
// page, §四 A, pairs the SwiGLU cast's four formats with this backward.
//
// gfx950 design. A lane owns 8 consecutive columns j of one row: three
// 16-byte loads (gate, up, dv) and two stores of 8 codes, dg at column j and
// du at column cols + j. The G / 8 lanes of a column group hold both the dg
// group and the du group over the same columns, so both abs-maxima come from
// the same DPP reduction pattern and each lane group writes two scales.
// exp(-g) and 1 / (1 + exp(-g)) are the hardware base-2 exponential and
// reciprocal (a few ulps from the exact fp32 expressions).
#include "qcast_device.h"
#include "qcast_kernels.h"

namespace qcast {
namespace {

#ifndef QCAST_SB_UNROLL
#define QCAST_SB_UNROLL 1
#endif
constexpr int kUnroll = QCAST_SB_UNROLL;
constexpr float kLog2e = 1.4426950408889634f;
// Chunk-to-row division as in the forward SwiGLU kernel: (c * magic) >> 40
// is exact for c < 2^24 and chunks per row < 2^16.
constexpr int64_t kMaxChunksPerLaunch = int64_t(1) << 24;
constexpr int64_t kMaxChunksPerRow = int64_t(1) << 16;
constexpr int kXcds = 8;

// kLayout: scale options other than plain fp32 row-major.
template <int kLanes, bool kWeighted, int kFmt, bool kClamp, bool kLayout>
__global__ __launch_bounds__(kThreads) void swiglu_backward_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ dv,
    const float* __restrict__ w, int64_t nchunks, uint32_t chunks_per_row, uint64_t row_magic,
    int64_t cols, float floor, float clamp, uint32_t row0, SfLayout lay, uint32_t per_xcd,
    uint8_t* __restrict__ q, void* __restrict__ sf) {
  // With column-major scales each XCD takes a contiguous range of rows, so
  // the scale words of neighbouring rows meet in one L2 before they are
  // written back (workgroups remapped past the end find no chunk). E2M1
  // takes that order in every layout (20.1 against 20.8 us on the 8192 x
  // 2048 gradient, interleaved, 100 rounds; E4M3 22.8 against 22.5 and
  // E5M6 25.9 against 25.6 keep the natural order).
  uint32_t blk = blockIdx.x;
  if ((kLayout || kFmt == kE2M1) && per_xcd) blk = (blk % kXcds) * per_xcd + blk / kXcds;
  const int64_t base0 = (int64_t)blk * kThreads * kUnroll + threadIdx.x;
  const uint32_t groups_per_half = chunks_per_row / kLanes;
  u32x4 graw[kUnroll], uraw[kUnroll], draw[kUnroll];
  float wr[kUnroll];
#pragma unroll
  for (int k = 0; k < kUnroll; ++k) {
    const int64_t c = base0 + (int64_t)k * kThreads;
    if (c < nchunks) {
      const uint32_t row = (uint32_t)(((uint64_t)c * row_magic) >> 40);
      const uint32_t jc = (uint32_t)c - row * chunks_per_row;
      const u32x4* g = reinterpret_cast<const u32x4*>(h + (int64_t)row * 2 * cols) + jc;
      graw[k] = load_stream(g);
      uraw[k] = load_stream(g + chunks_per_row);
      draw[k] = load_stream(reinterpret_cast<const u32x4*>(dv) + c);
      wr[k] = kWeighted ? w[row] : 1.0f;
    }
  }
#pragma unroll
  for (int k = 0; k < kUnroll; ++k) {
    const int64_t c = base0 + (int64_t)k * kThreads;
    if (c < nchunks) {
      const uint32_t row = (uint32_t)(((uint64_t)c * row_magic) >> 40);
      const uint32_t jc = (uint32_t)c - row * chunks_per_row;
      float gv[8], uv[8], dvv[8], dg[8], du[8];
      unpack8(graw[k], gv);
      unpack8(uraw[k], uv);
      unpack8(draw[k], dvv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        bool g_pass = true, u_pass = true;
        if (kClamp) {
          g_pass = !(gv[i] > clamp);
          u_pass = !(uv[i] > clamp) && !(uv[i] < -clamp);
          gv[i] = g_pass ? gv[i] : clamp;
          uv[i] = uv[i] > clamp ? clamp : (uv[i] < -clamp ? -clamp : uv[i]);
        }
        const float e = __builtin_amdgcn_exp2f(-gv[i] * kLog2e);
        const float s = __builtin_amdgcn_rcpf(1.0f + e);
        const float silu = gv[i] * s;
        const float dsilu = s + silu * (1.0f - s);
        const float dvw = kWeighted ? dvv[i] * wr[k] : dvv[i];
        dg[i] = g_pass ? dvw * uv[i] * dsilu : 0.0f;
        du[i] = u_pass ? dvw * silu : 0.0f;
      }
      const float amax_g = lane_group_max<kLanes>(absmax8(dg));
      const float amax_u = lane_group_max<kLanes>(absmax8(du));
      Scale sg = group_scale<kFmt>(amax_g, floor);
      Scale su = group_scale<kFmt>(amax_u, floor);
      if (kLayout && (lay.flags & kSfRound)) {
        sg = round_scale_pow2(sg);
        su = round_scale_pow2(su);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        dg[i] = dg[i] * sg.inv;
        du[i] = du[i] * su.inv;
      }
      // the row [dg | du] is one code row of 2 * chunks_per_row chunks
      const uint32_t qc = row * 2 * chunks_per_row + jc;
      store_chunk8<kFmt>(q, qc, dg);
      store_chunk8<kFmt>(q, qc + chunks_per_row, du);
      // dg groups first, then the du groups, of row row0 + row (a packed
      // word's 4 groups sit in aligned lanes: groups_per_half % 4 == 0)
      if (kLayout) {
        store_row_group_scale<kLanes>(sf, row0 + row, jc / kLanes, sg, lay);
        store_row_group_scale<kLanes>(sf, row0 + row, groups_per_half + jc / kLanes, su, lay);
      } else if ((threadIdx.x & (kLanes - 1)) == 0) {
        float* srow = static_cast<float*>(sf) + (uint64_t)(row0 + row) * 2 * groups_per_half;
        srow[jc / kLanes] = sg.sf;
        srow[groups_per_half + jc / kLanes] = su.sf;
      }
    }
  }
}

template <int kLanes, bool kWeighted, int kFmt, bool kClamp, bool kLayout>
hipError_t launch(const uint16_t* h, const uint16_t* dv, const float* w, int64_t rows,
                  int64_t cols, float floor, float clamp, const SfLayout& lay, uint8_t* q,
                  void* sf, hipStream_t stream) {
  const int64_t cpr = cols / 8;
  const uint64_t magic = ((uint64_t(1) << 40) + (uint64_t)cpr - 1) / (uint64_t)cpr;
  const int64_t slab_rows = kMaxChunksPerLaunch / cpr;
  for (int64_t r0 = 0; r0 < rows; r0 += slab_rows) {
    const int64_t nr = rows - r0 < slab_rows ? rows - r0 : slab_rows;
    const int64_t nchunks = nr * cpr;
    const int64_t per_block = (int64_t)kThreads * kUnroll;
    int64_t blocks = (nchunks + per_block - 1) / per_block;
    int64_t per_xcd = 0;
    if (kFmt == kE2M1 || (kLayout && (lay.flags & kSfColMajor))) {
      per_xcd = (blocks + kXcds - 1) / kXcds;
      blocks = per_xcd * kXcds;
    }
    launch_kernel((swiglu_backward_kernel<kLanes, kWeighted, kFmt, kClamp, kLayout>),
                  dim3((unsigned)blocks), dim3(kThreads), 0, stream, h + r0 * 2 * cols,
                  dv + r0 * cols, kWeighted ? w + r0 : nullptr, nchunks, (uint32_t)cpr,
                  magic, cols, floor, clamp, (uint32_t)r0, lay, (uint32_t)per_xcd,
                  q + code_bytes<kFmt>(r0 * 2 * cols), sf);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

template <int kLanes, int kFmt, bool kClamp>
hipError_t launch_w(const uint16_t* h, const uint16_t* dv, const float* w, int64_t rows,
                    int64_t cols, float floor, float clamp, const SfLayout& lay, uint8_t* q,
                    void* sf, hipStream_t stream) {
  if (lay.flags) {
    return w ? launch<kLanes, true, kFmt, kClamp, true>(h, dv, w, rows, cols, floor, clamp, lay,
                                                        q, sf, stream)
             : launch<kLanes, false, kFmt, kClamp, true>(h, dv, w, rows, cols, floor, clamp, lay,
                                                         q, sf, stream);
  }
  return w ? launch<kLanes, true, kFmt, kClamp, false>(h, dv, w, rows, cols, floor, clamp, lay, q,
                                                       sf, stream)
           : launch<kLanes, false, kFmt, kClamp, false>(h, dv, w, rows, cols, floor, clamp, lay,
                                                        q, sf, stream);
}

template <int kFmt, bool kClamp>
hipError_t launch_g(const uint16_t* h, const uint16_t* dv, const float* w, int64_t rows,
                    int64_t cols, int group, float floor, float clamp, const SfLayout& lay,
                    uint8_t* q, void* sf, hipStream_t stream) {
  switch (group) {
    case 32:
      return launch_w<4, kFmt, kClamp>(h, dv, w, rows, cols, floor, clamp, lay, q, sf, stream);
    case 64:
      return launch_w<8, kFmt, kClamp>(h, dv, w, rows, cols, floor, clamp, lay, q, sf, stream);
    case 128:
      return launch_w<16, kFmt, kClamp>(h, dv, w, rows, cols, floor, clamp, lay, q, sf, stream);
  }
  return hipErrorInvalidValue;
}

template <int kFmt>
hipError_t launch_c(const uint16_t* h, const uint16_t* dv, const float* w, int64_t rows,
                    int64_t cols, int group, float floor, float clamp, const SfLayout& lay,
                    uint8_t* q, void* sf, hipStream_t stream) {
  return clamp > 0.0f
             ? launch_g<kFmt, true>(h, dv, w, rows, cols, group, floor, clamp, lay, q, sf, stream)
             : launch_g<kFmt, false>(h, dv, w, rows, cols, group, floor, clamp, lay, q, sf,
                                     stream);
}

}  // namespace

hipError_t launch_swiglu_backward(const void* h, const void* dv, int64_t rows, int64_t cols,
                                  const float* w, int fmt, int group, float floor,
                                  uint32_t sf_flags, float swiglu_clamp, void* q, void* sf,
                                  hipStream_t stream, const LaunchCaps& caps) {
  (void)caps;
  if (rows == 0 || cols == 0) return hipSuccess;
  if (cols / 8 >= kMaxChunksPerRow || rows >= (int64_t(1) << 32)) return hipErrorInvalidValue;
  // The scale layout of the rows [dg | du]; packed words of 4 groups must
  // not straddle the two halves.
  if ((sf_flags & kSfPacked) && (cols / group) % 4 != 0) return hipErrorInvalidValue;
  const SfLayout lay = make_sf_layout(rows, 2 * cols, group, sf_flags);
  const uint16_t* hp = static_cast<const uint16_t*>(h);
  const uint16_t* dp = static_cast<const uint16_t*>(dv);
  uint8_t* qp = static_cast<uint8_t*>(q);
  switch (fmt) {
    case kE4M3:
      return launch_c<kE4M3>(hp, dp, w, rows, cols, group, floor, swiglu_clamp, lay, qp, sf,
                             stream);
    case kE5M2:
      return launch_c<kE5M2>(hp, dp, w, rows, cols, group, floor, swiglu_clamp, lay, qp, sf,
                             stream);
    case kE2M1:
      return launch_c<kE2M1>(hp, dp, w, rows, cols, group, floor, swiglu_clamp, lay, qp, sf,
                             stream);
    case kE5M6:
      return launch_c<kE5M6>(hp, dp, w, rows, cols, group, floor, swiglu_clamp, lay, qp, sf,
                             stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace qcast
