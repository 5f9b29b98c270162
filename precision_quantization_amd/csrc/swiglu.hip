// swiglu.hip -- SwiGLU forward fused with the per-token cast (E4M3, E5M2,
// packed E2M1 or packed E5M6: the format list the page "TileKernels 与
// DeepGEMM 的分界线：DeepSeek 开源内核栈的分工", §四 A, gives for this cast).
//
// Operation: swiglu_forward_and_per_token_cast of the walk-through page
// "DeepSeek开源TileKernels：用Python写的GPU算子逼近硬件性能上限", §3.3: with the
// left half of each row as the gate g and the right half as the up value u,
// v = g / (1 + exp(-g)) * u * w[row] in fp32, then the per-token cast of v
// (§3.2). The page's point is that the unfused form costs three launches,
// each reading and writing the whole tensor; here v lives only in registers.
//
// gfx950 design. Output chunk c (8 consecutive outputs of one row) needs two
// 16-byte loads: 8 gate values and the 8 up values cols further on. The
// output stream is walked like the per-token cast (G/8 lanes per group, DPP
// abs-max), so the row of chunk c comes from a multiply-shift division by
// the chunks per row. exp(-g) is the hardware base-2 exponential of
// -g * log2(e), and the division by 1 + exp(-g) is a multiply by the
// hardware reciprocal: together a few ulps from the exact fp32 expression,
// which moves a code only where v lies next to a rounding midpoint. When
// exp(-g) overflows, the reciprocal is 0 and v is a zero of the right sign,
// as in the exact expression.
//
// The optional clamp of the same section bounds the gate from above and the
// up value to [-c, c] before the product; the number of values it changed
// is summed per workgroup and reaches a 64-bit counter either through the
// slots of a caller's count workspace (full grid) or with one atomic per
// workgroup of a capped grid (no workspace).
#include "qcast_device.h"
#include "qcast_kernels.h"

namespace qcast {
namespace {

// Launch shape (compile-time; defaults chosen by measurement): output
// chunks in flight per lane, and the cap on workgroups per CU (0: no cap).
// The E5M6 form, whose encode takes about three times the arithmetic per
// value, keeps 2 chunks per lane in flight (17.1 against 17.9 us at 1 and
// 18.2 at 4 on the 8192 x 2048 output, interleaved); the other formats are
// fastest at 1 (E4M3 15.0 against 15.3 at 2; E2M1 13.9 at 1 and 2).
#ifndef QCAST_SW_UNROLL
#define QCAST_SW_UNROLL 1
#endif
#ifndef QCAST_SW_UNROLL_E5M6
#define QCAST_SW_UNROLL_E5M6 2
#endif
#ifndef QCAST_SW_WG_PER_CU
#define QCAST_SW_WG_PER_CU 0
#endif
// Workgroup order of the launch without a counter. Each XCD takes a
// contiguous range of the chunk stream (the grid padded to a multiple of 8):
// 14.84 against 15.04 us for E4M3 and 13.52 against 14.00 for E2M1 on the
// 8192 x 2048 output (interleaved, 100 rounds). E5M6 keeps the natural
// round-robin order, which was faster for it (17.32 against 18.32).
template <int kFmt>
constexpr bool kXcdOrder = kFmt != kE5M6;
constexpr int kXcds = 8;
// With a clamp counter and no workspace, every workgroup ends in one atomic
// add on the same 64-bit word, and those adds are serialized where the word
// lives (about 12 ns each, measured), so the counting kernel runs a capped,
// grid-strided grid of this many workgroups per CU, each of kCountBlock
// threads (large workgroups keep the waves per CU up while the atomics stay
// few). With a workspace the adds are spread over its slots and the grid is
// uncapped, with kSlotUnroll chunks per lane (2 measured fastest of 1, 2, 4).
#ifndef QCAST_SW_COUNT_WG_PER_CU
#define QCAST_SW_COUNT_WG_PER_CU 1
#endif
#ifndef QCAST_SW_COUNT_BLOCK
#define QCAST_SW_COUNT_BLOCK 1024
#endif
#ifndef QCAST_SW_COUNT_UNROLL
#define QCAST_SW_COUNT_UNROLL 1
#endif
#ifndef QCAST_SW_SLOT_UNROLL
#define QCAST_SW_SLOT_UNROLL 2
#endif
constexpr int kSlotUnroll = QCAST_SW_SLOT_UNROLL;
constexpr int kCountBlock = QCAST_SW_COUNT_BLOCK;
constexpr int kCountUnroll = QCAST_SW_COUNT_UNROLL;
template <int kFmt>
constexpr int kStreamUnroll = kFmt == kE5M6 ? QCAST_SW_UNROLL_E5M6 : QCAST_SW_UNROLL;
constexpr int kWgPerCu = QCAST_SW_WG_PER_CU;
constexpr int kCountWgPerCu = QCAST_SW_COUNT_WG_PER_CU;
constexpr float kLog2e = 1.4426950408889634f;
// Chunk-to-row division: row = (c * magic) >> 40 is exact for c < 2^24 and
// chunks-per-row d < 2^16 when magic = ceil(2^40 / d).
constexpr int64_t kMaxChunksPerLaunch = int64_t(1) << 24;
constexpr int64_t kMaxChunksPerRow = int64_t(1) << 16;

__device__ __forceinline__ float silu_times(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * kLog2e);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

template <int kLanes, bool kWeighted, int kFmt, bool kClamp, int kCount, int kBlock,
          int kUnroll>
__global__ __launch_bounds__(kBlock) void swiglu_kernel(
    const uint16_t* __restrict__ h, const float* __restrict__ w, int64_t nchunks,
    uint32_t chunks_per_row, uint64_t row_magic, float floor,
    uint8_t* __restrict__ q, void* __restrict__ sf, SfLayout lay, uint32_t group0,
    float clamp, unsigned long long* __restrict__ count, unsigned long long* __restrict__ slots) {
  uint32_t nclamp = 0;
  // nchunks < 2^24 per launch: every chunk index and in-slab offset is 32-bit
  const uint32_t n32 = (uint32_t)nchunks;
  const u32x4* h4 = reinterpret_cast<const u32x4*>(h);
  const uint32_t row_chunks = 2 * chunks_per_row;
  if constexpr (kCount == kCountSlotted) {
    // The grid covers the stream in one pass. The values come first, then
    // the workgroup's count goes to its slot, and the slot atomic's round
    // trip overlaps the codes and stores that follow.
    const uint32_t base = blockIdx.x * kBlock * kUnroll + threadIdx.x;
    u32x4 graw[kUnroll], uraw[kUnroll];
    float wr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t c = base + u * kBlock;
      if (c < n32) {
        const uint32_t row = (uint32_t)(((uint64_t)c * row_magic) >> 40);
        const uint32_t gi = row * row_chunks + (c - row * chunks_per_row);
        graw[u] = load_stream(h4 + gi);
        uraw[u] = load_stream(h4 + (gi + chunks_per_row));
        wr[u] = kWeighted ? w[row] : 1.0f;
      }
    }
    float v[kUnroll][8];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (base + u * kBlock < n32) {
        float gv[8], uv[8];
        unpack8(graw[u], gv);
        unpack8(uraw[u], uv);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          nclamp += wave_clamp_count(gv[i], uv[i], clamp);
          clamp_gate_up(gv[i], uv[i], clamp);
          v[u][i] = silu_times(gv[i], uv[i]);
          if (kWeighted) v[u][i] = v[u][i] * wr[u];
        }
      }
    }
    SlotCount<kBlock> sc;
    sc.arrive(nclamp, slots);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t c = base + u * kBlock;
      if (c < n32) {
        const float amax = lane_group_max<kLanes>(absmax8(v[u]));
        Scale s = group_scale<kFmt>(amax, floor);
        if (lay.flags & kSfRound) s = round_scale_pow2(s);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[u][i] = v[u][i] * s.inv;
        store_chunk8<kFmt>(q, c, v[u]);
        store_group_scale<kLanes>(sf, group0 + c / kLanes, s, lay);
      }
    }
    sc.finish(slots, count);
    return;
  }
  const uint32_t step = gridDim.x * kBlock * kUnroll;
  uint32_t blk = blockIdx.x;
  if (kCount == kCountNone && kXcdOrder<kFmt>) {
    const uint32_t per_xcd = gridDim.x / kXcds;  // the grid is a multiple of kXcds
    blk = (blk % kXcds) * per_xcd + blk / kXcds;
  }
  for (uint32_t base = blk * kBlock * kUnroll + threadIdx.x; base < n32; base += step) {
    u32x4 graw[kUnroll], uraw[kUnroll];
    float wr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t c = base + u * kBlock;
      if (c < n32) {
        const uint32_t row = (uint32_t)(((uint64_t)c * row_magic) >> 40);
        const uint32_t jc = c - row * chunks_per_row;
        const uint32_t gi = row * row_chunks + jc;
        graw[u] = load_stream(h4 + gi);
        uraw[u] = load_stream(h4 + (gi + chunks_per_row));
        wr[u] = kWeighted ? w[row] : 1.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t c = base + u * kBlock;
      if (c < n32) {
        float gv[8], uv[8], v[8];
        unpack8(graw[u], gv);
        unpack8(uraw[u], uv);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (kCount) nclamp += wave_clamp_count(gv[i], uv[i], clamp);
          if (kClamp) clamp_gate_up(gv[i], uv[i], clamp);
          v[i] = silu_times(gv[i], uv[i]);
          if (kWeighted) v[i] = v[i] * wr[u];
        }
        const float amax = lane_group_max<kLanes>(absmax8(v));
        Scale s = group_scale<kFmt>(amax, floor);
        if (lay.flags & kSfRound) s = round_scale_pow2(s);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = v[i] * s.inv;
        store_chunk8<kFmt>(q, c, v);
        store_group_scale<kLanes>(sf, group0 + c / kLanes, s, lay);
      }
    }
  }
  if constexpr (kCount == kCountDirect) add_wave_counts<kBlock>(nclamp, count);
}

struct ClampArgs {
  float c;                    // > 0: clamp bound
  unsigned long long* count;  // device counter or null
  unsigned long long* slots;  // count workspace or null
};

// Pointers and first scale-group index of one slab of rows.
struct SlabArgs {
  const uint16_t* h;
  const float* w;
  uint8_t* q;
  uint32_t group0;
};

template <int kLanes, bool kWeighted, int kFmt, bool kClamp>
hipError_t launch(const uint16_t* h, const float* w, int64_t rows, int64_t cols, float floor,
                  uint8_t* q, void* sf, const SfLayout& lay, const ClampArgs& ca,
                  hipStream_t stream, const LaunchCaps& caps) {
  const int64_t cpr = cols / 8;
  const uint64_t magic = ((uint64_t(1) << 40) + (uint64_t)cpr - 1) / (uint64_t)cpr;
  const int64_t groups_per_row = cols / (kLanes * 8);
  // Slabs of whole rows, each under 2^24 chunks, keep the division exact.
  const int64_t slab_rows = kMaxChunksPerLaunch / cpr;
  for (int64_t r0 = 0; r0 < rows; r0 += slab_rows) {
    const int64_t nr = rows - r0 < slab_rows ? rows - r0 : slab_rows;
    const int64_t nchunks = nr * cpr;
    const bool counting = kClamp && ca.count;
    // Slotted: at most 2^24 / (kThreads * kSlotUnroll) workgroups and 2^28
    // clamped values per slab, within the slots' 24 and 40 bits.
    const bool slotted = counting && ca.slots;
    const int block = counting && !slotted ? kCountBlock : kThreads;
    const int unroll = slotted ? kSlotUnroll : counting ? kCountUnroll : kStreamUnroll<kFmt>;
    const int64_t per_block_iter = (int64_t)block * unroll;
    const int64_t iters = (nchunks + per_block_iter - 1) / per_block_iter;
    const int wg_per_cu = slotted ? 0 : counting ? kCountWgPerCu : kWgPerCu;
    const int64_t max_blocks = wg_per_cu > 0 ? (int64_t)caps.num_cus * wg_per_cu : iters;
    const int64_t iters_per_block = (iters + max_blocks - 1) / max_blocks;
    const int64_t blocks = (iters + iters_per_block - 1) / iters_per_block;
    const SlabArgs args{h + r0 * 2 * cols, kWeighted ? w + r0 : nullptr,
                        q + code_bytes<kFmt>(r0 * cols), (uint32_t)(r0 * groups_per_row)};
    auto plain = [&] {
      // workgroups of the padding find no chunk and return
      const int64_t grid = kXcdOrder<kFmt> ? (blocks + kXcds - 1) / kXcds * kXcds : blocks;
      launch_kernel((swiglu_kernel<kLanes, kWeighted, kFmt, kClamp, kCountNone, kThreads,
                                   kStreamUnroll<kFmt>>),
                    dim3((unsigned)grid), dim3(kThreads), 0, stream, args.h, args.w, nchunks,
                    (uint32_t)cpr, magic, floor, args.q, sf, lay, args.group0, ca.c,
                    ca.count, ca.slots);
    };
    if constexpr (kClamp) {
      if (slotted)
        launch_kernel((swiglu_kernel<kLanes, kWeighted, kFmt, true, kCountSlotted, kThreads,
                                     kSlotUnroll>),
                      dim3((unsigned)blocks), dim3(kThreads), 0, stream, args.h, args.w, nchunks,
                      (uint32_t)cpr, magic, floor, args.q, sf, lay, args.group0, ca.c,
                      ca.count, ca.slots);
      else if (counting)
        launch_kernel((swiglu_kernel<kLanes, kWeighted, kFmt, true, kCountDirect, kCountBlock,
                                     kCountUnroll>),
                      dim3((unsigned)blocks), dim3(kCountBlock), 0, stream, args.h, args.w,
                      nchunks, (uint32_t)cpr, magic, floor, args.q, sf, lay, args.group0,
                      ca.c, ca.count, ca.slots);
      else
        plain();
    } else {
      plain();
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

template <int kLanes, int kFmt, bool kClamp>
hipError_t launch_w(const uint16_t* h, const float* w, int64_t rows, int64_t cols, float floor,
                    uint8_t* q, void* sf, const SfLayout& lay, const ClampArgs& ca,
                    hipStream_t stream, const LaunchCaps& caps) {
  return w ? launch<kLanes, true, kFmt, kClamp>(h, w, rows, cols, floor, q, sf, lay, ca, stream,
                                                caps)
           : launch<kLanes, false, kFmt, kClamp>(h, w, rows, cols, floor, q, sf, lay, ca, stream,
                                                 caps);
}

template <int kFmt, bool kClamp>
hipError_t launch_g(const uint16_t* h, const float* w, int64_t rows, int64_t cols, int group,
                    float floor, uint8_t* q, void* sf, const SfLayout& lay, const ClampArgs& ca,
                    hipStream_t stream, const LaunchCaps& caps) {
  switch (group) {
    case 32:
      return launch_w<4, kFmt, kClamp>(h, w, rows, cols, floor, q, sf, lay, ca, stream, caps);
    case 64:
      return launch_w<8, kFmt, kClamp>(h, w, rows, cols, floor, q, sf, lay, ca, stream, caps);
    case 128:
      return launch_w<16, kFmt, kClamp>(h, w, rows, cols, floor, q, sf, lay, ca, stream, caps);
  }
  return hipErrorInvalidValue;
}

template <int kFmt>
hipError_t launch_c(const uint16_t* h, const float* w, int64_t rows, int64_t cols, int group,
                    float floor, uint8_t* q, void* sf, const SfLayout& lay, const ClampArgs& ca,
                    hipStream_t stream, const LaunchCaps& caps) {
  return ca.c > 0.0f
             ? launch_g<kFmt, true>(h, w, rows, cols, group, floor, q, sf, lay, ca, stream, caps)
             : launch_g<kFmt, false>(h, w, rows, cols, group, floor, q, sf, lay, ca, stream, caps);
}

}  // namespace

hipError_t launch_swiglu_per_token(const void* h, int64_t rows, int64_t cols, const float* w,
                                   int fmt, int group, float floor, uint32_t sf_flags,
                                   float swiglu_clamp, unsigned long long* clamp_count,
                                   unsigned long long* count_ws, void* q, void* sf,
                                   hipStream_t stream, const LaunchCaps& caps) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (cols / 8 >= kMaxChunksPerRow) return hipErrorInvalidValue;
  if (rows * cols / group >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const SfLayout lay = make_sf_layout(rows, cols, group, sf_flags);
  const ClampArgs ca{swiglu_clamp, clamp_count, count_ws};
  const uint16_t* hp = static_cast<const uint16_t*>(h);
  uint8_t* qp = static_cast<uint8_t*>(q);
  switch (fmt) {
    case kE4M3:
      return launch_c<kE4M3>(hp, w, rows, cols, group, floor, qp, sf, lay, ca, stream, caps);
    case kE5M2:
      return launch_c<kE5M2>(hp, w, rows, cols, group, floor, qp, sf, lay, ca, stream, caps);
    case kE2M1:
      return launch_c<kE2M1>(hp, w, rows, cols, group, floor, qp, sf, lay, ca, stream, caps);
    case kE5M6:
      return launch_c<kE5M6>(hp, w, rows, cols, group, floor, qp, sf, lay, ca, stream, caps);
  }
  return hipErrorInvalidValue;
}

}  // namespace qcast
