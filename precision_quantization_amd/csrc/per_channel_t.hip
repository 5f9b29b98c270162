// per_channel_t.hip -- per-channel cast of bf16 activations, written
// transposed, to E4M3, E5M2, packed E2M1 or packed E5M6.
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
// bits (v_pk_max_u16) over the lane's tokens, then a butterfly over the 8
// lanes that hold the same channel chunk (permlane swaps that each carry two
// channels, and a DPP step), after which every lane holds one channel's
// maximum of the wave; a 4-wave LDS exchange, and one lane per (group,
// channel) forms the scale. Each lane packs
// the codes of 4 tokens of one channel into a dword and writes it to an LDS
// tile [channel][token] whose dword index is XOR-swizzled by
// 4 * ((channel/8) mod 8): the eight channel chunks a half-wave writes land
// in distinct banks, and each 16-byte run of tokens stays contiguous and
// aligned, so the read-back is one ds_read_b128 per lane and the store is a
// full row of qT (128 * kTG bytes) per channel. The packed formats wait in
// LDS one code per byte (E2M1) or per 16-bit half (E5M6, rows twice as
// long), and the read-back lane packs them (nibbles; 12-bit codes) before it
// stores: 8 or 12 bytes per lane instead of 16. (A kernel that transposes in
// registers instead -- each lane holding 16 tokens of 8 channels, no LDS, no
// barrier -- was measured slower in every format: 66.0 against 63.3 us for
// E4M3 on the 16384 x 7168 activation, 62.3 against 57.2 for E2M1, 103.5
// against 82.5 for E5M6.) (The pages' transpose pads
// its shared tile and rotates the column index for the same purpose; the
// XOR form keeps 16-byte reads aligned.) Workgroups are numbered so that
// each of the 8 XCDs walks a contiguous range of tiles, in strips of two
// channel tiles: token group outer, channel tile inner. Workgroups started
// together then read both 128-byte halves of the same 256-byte row segments
// and write neighbouring 128-byte pieces of the same qT rows and scale
// lines (measured about 3% faster than walking token groups of one channel
// tile, and much faster than walking channel tiles first).
//
// The same tile machinery serves SwiGLU fused with the cast and the
// transpose (the three-way fusion of "刚刚！DeepSeek开源高性能GPU算子库
// TileKernels", item 2, applied to the SwiGLU of the walk-through page,
// §3.3): each lane loads the gate and up chunks of its tokens and the row
// weights, forms
// v = silu(g) * u * w in fp32 registers (clamped first when asked, counting
// the changed values), and the tile continues from fp32 values instead of
// packed bf16.
//
// Scales: fp32 sf[channel][token group] by default; on request the layouts
// of the per-token cast of the transposed input, whose rows are the
// channels (round_sf, TMA-aligned column-major sf[group][channels padded to
// 4], packed UE8M0 words: the cast config of the walk-through page, §3.1, and
// the consumer layouts the first page's §四 C says the casts write while
// they quantize or re-arrange). One lane forms each scale, so a packed word,
// whose four bytes belong to four token groups of other tiles, is written
// one byte at a time.
//
// A traffic-only twin of the cast (per_channel_t_traffic_kernel: the same
// walk, loads and qT stores, no arithmetic) serves measurement only.
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
// The SwiGLU form reads two 128-byte pieces per token row (gate and up,
// cols apart) and walks each channel tile's token groups in turn (strips of
// one): 16.4 us against 18.2 us with strips of two on the 8192 x 2048
// output, interleaved.
#ifndef QCAST_PC_SW_STRIP
#define QCAST_PC_SW_STRIP 1
#endif
constexpr uint32_t kStrip = QCAST_PC_STRIP;
constexpr uint32_t kSwStrip = QCAST_PC_SW_STRIP;
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

// Dword index of token dword d of channel row c in the swizzled tile of
// rows of kDw dwords (the XOR moves whole 16-byte groups and keeps d < kDw
// for kDw a multiple of 32).
template <int kDw = kRowDw>
__device__ __forceinline__ int tile_index(int c, int d) {
  static_assert(kDw % 32 == 0, "rows of whole 32-dword blocks");
  return c * kDw + (d ^ (4 * ((c >> 3) & 7)));
}

// The LDS tile of a format. Codes wait in LDS one per byte (E4M3, E5M2, and
// E2M1 with the code in the low nibble) or one per 16-bit half (E5M6), so a
// lane's 4 tokens of a channel are one dword (two for E5M6); the read-back
// lane packs E2M1 to nibbles and E5M6 to 12-bit codes before its store.
template <int kFmt>
struct TileGeo {
  static constexpr int kCodeBytes = kFmt == kE5M6 ? 2 : 1;   // LDS bytes per code
  static constexpr int kRowDw = kTileTokens * kCodeBytes / 4;
  static constexpr int kRowVec = kRowDw / 4;                 // 16-byte vectors per row
  static constexpr int kVecTokens = 16 / kCodeBytes;         // tokens per vector
  static constexpr int kReadPasses = kChannels * kRowVec / kThreads;
  static_assert(kReadPasses >= 1, "tile shape");
};

// Position of a tile: first channel, first token, valid channels and groups.
// Tile counts and in-tile offsets fit in 32 bits (checked by the launcher).
struct TileCoord {
  uint32_t c0, t0, gt;
  int nc, ng;
};

// The strip walk divides by kS * ntg with a host-computed multiply and shift
// (sdiv), and by the strip width with a shift (kS is a power of two; only a
// last, narrower strip divides), so a workgroup issues its loads a few
// instructions after it starts.
template <uint32_t kS = kStrip>
__device__ __forceinline__ TileCoord tile_coord(uint32_t tau, uint32_t ngroups, uint32_t cols,
                                                uint32_t nct, uint32_t ntg, FastDiv sdiv) {
  static_assert((kS & (kS - 1)) == 0, "strips of a power of two");
  TileCoord tc;
  uint32_t ct;
  if (kOrder & 4) {
    const uint32_t strip = fast_div(tau, sdiv);
    const uint32_t rem = tau - strip * kS * ntg;
    if (nct - strip * kS >= kS) {
      tc.gt = rem / kS;
      ct = strip * kS + (rem & (kS - 1));
    } else {
      const uint32_t width = nct - strip * kS;
      tc.gt = rem / width;
      ct = strip * kS + (rem - tc.gt * width);
    }
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

// Issue the lane's loads of a tile of a bf16 matrix whose rows are `stride`
// elements apart (zeros outside the tensor).
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ x, uint32_t stride,
                                          const TileCoord& tc, u32x4 (&raw)[kPasses][4]) {
  const int t = threadIdx.x;
  const int ch = t % kCC;
  const int k = t / kCC;
  const bool valid_ch = ch * 8 < tc.nc;
  // 64-bit tile base, 32-bit offsets inside the tile
  const uint16_t* base = x + (uint64_t)tc.t0 * stride + tc.c0;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const bool valid = valid_ch && (p / kPassesPerGroup) < tc.ng;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t off = (uint32_t)(p * kPassTokens + 4 * k + i) * stride + ch * 8;
      raw[p][i] = valid ? load_stream(reinterpret_cast<const u32x4*>(base + off))
                        : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// A tile's values as packed bf16 (the plain cast): word w of raw[p][i] holds
// channels 8ch + 2w (low half) and 8ch + 2w + 1 of the lane's token i of
// pass p.
struct Bf16Tile {
  u32x4 raw[kPasses][4];

  // Abs-maxima of the lane's 8 channels over token group gi, reduced over
  // the lanes holding the same channel chunk: packed 16-bit maxima of the
  // magnitude bits (v_pk_max_u16), unpacked at the end.
  __device__ __forceinline__ void group_amax(int gi, float out[8]) const {
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
      m[w] = pk_max_xor16(m[w]);
      m[w] = pk_max_xor32(m[w]);
      out[2 * w] = bf16_lo(m[w]);
      out[2 * w + 1] = bf16_hi(m[w]);
    }
  }

  // The same maxima, reduced as a butterfly over the 8 lanes (bits 3, 4, 5
  // of the lane index) that hold the chunk, each exchange carrying two
  // different channels: after it every lane holds one channel's maximum,
  // channel lane_channel() of its chunk. 3 swaps and 4 packed maxima
  // instead of 8 swaps and 12.
  __device__ __forceinline__ float group_amax_lane(int gi) const {
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
    // lanes i ^ 16: words 0, 1 stay with the even rows, words 2, 3 go to the odd
    uint32_t n[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const auto r = __builtin_amdgcn_permlane16_swap(m[w], m[w + 2], false, false);
      n[w] = pk_umax16((uint32_t)r[0], (uint32_t)r[1]);
    }
    // lanes i ^ 32: word n[0] stays with the lower half, n[1] goes to the upper
    const auto r = __builtin_amdgcn_permlane32_swap(n[0], n[1], false, false);
    uint32_t q = pk_umax16((uint32_t)r[0], (uint32_t)r[1]);
    // lanes i ^ 8 (both halves), then each lane takes its half
    q = pk_umax16(q, dpp<kDppRor8>(q));
    return (threadIdx.x & 8) ? bf16_hi(q) : bf16_lo(q);
  }

  __device__ __forceinline__ float value(int p, int i, int j) const {
    const uint32_t word = raw[p][i][j >> 1];
    return (j & 1) ? bf16_hi(word) : bf16_lo(word);
  }
};

// A tile's values as fp32 (the SwiGLU output).
struct F32Tile {
  float v[kPasses][4][8];

  // The lane's maximum is an fp32 max of magnitudes (one v_max_f32 with an
  // abs modifier per value); the cross-lane steps then compare the bit
  // patterns of those non-negative values, which order as the values do.
  __device__ __forceinline__ void group_amax(int gi, float out[8]) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float mf = 0.0f;
#pragma unroll
      for (int pp = 0; pp < kPassesPerGroup; ++pp) {
#pragma unroll
        for (int i = 0; i < 4; ++i) mf = fmaxf(mf, fabsf(v[gi * kPassesPerGroup + pp][i][j]));
      }
      uint32_t m = __float_as_uint(mf);
      if (kCC == 8) m = umax(m, dpp<kDppRor8>(m));
      m = max_xor16(m);
      m = max_xor32(m);
      out[j] = __uint_as_float(m);
    }
  }

  // As Bf16Tile::group_amax_lane, on fp32 values: 6 swaps and 7 maxima
  // instead of 16 swaps and 24.
  __device__ __forceinline__ float group_amax_lane(int gi) const {
    uint32_t m[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float mf = 0.0f;
#pragma unroll
      for (int pp = 0; pp < kPassesPerGroup; ++pp) {
#pragma unroll
        for (int i = 0; i < 4; ++i) mf = fmaxf(mf, fabsf(v[gi * kPassesPerGroup + pp][i][j]));
      }
      m[j] = __float_as_uint(mf);
    }
    uint32_t n[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto r = __builtin_amdgcn_permlane16_swap(m[j], m[j + 4], false, false);
      n[j] = umax((uint32_t)r[0], (uint32_t)r[1]);
    }
    uint32_t q[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const auto r = __builtin_amdgcn_permlane32_swap(n[j], n[j + 2], false, false);
      q[j] = umax((uint32_t)r[0], (uint32_t)r[1]);
    }
    const bool odd = (threadIdx.x & 8) != 0;
    const uint32_t keep = odd ? q[1] : q[0];
    const uint32_t send = odd ? q[0] : q[1];
    return __uint_as_float(umax(keep, dpp<kDppRor8>(send)));
  }

  __device__ __forceinline__ float value(int p, int i, int j) const { return v[p][i][j]; }
};

// The channel of its 8-channel chunk whose column maximum a lane holds after
// group_amax_lane: v_permlane16_swap exchanges the odd rows of its first
// operand with the even rows of its second, v_permlane32_swap the upper half
// of the first with the lower half of the second, so lane bit 4 picks the
// upper four channels, bit 5 the upper two of those, bit 3 the odd one.
__device__ __forceinline__ int lane_channel() {
  const int l = threadIdx.x & 63;
  return ((l >> 3) & 1) | (((l >> 5) & 1) << 1) | (((l >> 4) & 1) << 2);
}

constexpr float kLog2e = 1.4426950408889634f;

// Load a tile of the SwiGLU input h [rows, 2 * cols] and form
// v = silu(g) * u (* w[token]); with kCount, returns the number of values the
// clamp changed in the whole wave (the same in every lane). Tokens and
// channels outside the tensor give 0 and are never counted.
template <bool kWeighted, bool kClamp, bool kCount>
__device__ __forceinline__ uint32_t load_swiglu_tile(const uint16_t* __restrict__ h,
                                                     const float* __restrict__ w, uint32_t cols,
                                                     float clamp, const TileCoord& tc,
                                                     F32Tile& tile) {
  const int t = threadIdx.x;
  const int ch = t % kCC;
  const int k = t / kCC;
  const bool valid_ch = ch * 8 < tc.nc;
  u32x4 graw[kPasses][4], uraw[kPasses][4];
  float wr[kPasses][4];
  const uint16_t* base = h + (uint64_t)tc.t0 * 2 * cols + tc.c0;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const bool valid = valid_ch && (p / kPassesPerGroup) < tc.ng;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t tok = (uint32_t)(p * kPassTokens + 4 * k + i);
      const uint32_t off = tok * 2 * cols + ch * 8;
      const u32x4 z = {0u, 0u, 0u, 0u};
      graw[p][i] = valid ? load_stream(reinterpret_cast<const u32x4*>(base + off)) : z;
      uraw[p][i] = valid ? load_stream(reinterpret_cast<const u32x4*>(base + off + cols)) : z;
      wr[p][i] = (kWeighted && valid) ? w[tc.t0 + tok] : 1.0f;
    }
  }
  uint32_t nclamp = 0;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float gv[8], uv[8];
      unpack8(graw[p][i], gv);
      unpack8(uraw[p][i], uv);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (kCount) nclamp += wave_clamp_count(gv[j], uv[j], clamp);
        if (kClamp) clamp_gate_up(gv[j], uv[j], clamp);
        const float e = __builtin_amdgcn_exp2f(-gv[j] * kLog2e);
        float val = gv[j] * __builtin_amdgcn_rcpf(1.0f + e) * uv[j];
        if (kWeighted) val = val * wr[p][i];
        tile.v[p][i][j] = val;
      }
    }
  }
  return nclamp;
}

template <int kFmt>
struct Smem {
  uint32_t tile[kChannels * TileGeo<kFmt>::kRowDw];
  float wave_amax[kTG][4][kChannels];
  float inv_s[kTG][kChannels];
};

// Scales, codes and stores of one tile whose values are in raw. Starts with
// the workgroup converged; with kReuse (a workgroup that goes on to another
// tile) it also ends converged, with the LDS free again.
template <int kFmt, bool kReuse, bool kLayout, class Tile>
__device__ __forceinline__ void process_tile(const TileCoord& tc, const Tile& tile, uint32_t rows,
                                             float floor, const SfLayout& lay, Smem<kFmt>& sm,
                                             uint8_t* __restrict__ qT, void* __restrict__ sf) {
  using TG = TileGeo<kFmt>;
  const int t = threadIdx.x;
  const int ch = t % kCC;
  const int k = t / kCC;
  const int wave = t >> 6;
  // Column abs-maxima per token group within each wave, then across waves.
#pragma unroll
  for (int gi = 0; gi < kTG; ++gi) {
    if constexpr (kCC == 8) {
      // every lane writes one channel's maximum of the wave
      sm.wave_amax[gi][wave][ch * 8 + lane_channel()] = tile.group_amax_lane(gi);
    } else {
      float m[8];
      tile.group_amax(gi, m);
      if ((t & 63) < kCC) {
#pragma unroll
        for (int j = 0; j < 8; ++j) sm.wave_amax[gi][wave][ch * 8 + j] = m[j];
      }
    }
  }
  __syncthreads();
  if (t < kTG * kChannels) {
    const int gi = t / kChannels;
    const int c = t % kChannels;
    const float m = fmaxf(fmaxf(sm.wave_amax[gi][0][c], sm.wave_amax[gi][1][c]),
                          fmaxf(sm.wave_amax[gi][2][c], sm.wave_amax[gi][3][c]));
    Scale s = group_scale<kFmt>(m, floor);
    if (kLayout && (lay.flags & kSfRound)) s = round_scale_pow2(s);
    sm.inv_s[gi][c] = s.inv;
    if (c < tc.nc && gi < tc.ng) {
      if (kLayout)
        store_lone_scale(sf, tc.c0 + c, tc.gt * kTG + gi, s, lay);
      else
        static_cast<float*>(sf)[(uint64_t)(tc.c0 + c) * lay.gpr + tc.gt * kTG + gi] = s.sf;
    }
  }
  __syncthreads();

  // Codes: for each pass and each of the lane's 8 channels, the 4 tokens
  // 4k..4k+3 of the pass as one dword (two for E5M6) of the channel's LDS row.
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int gi = p / kPassesPerGroup;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float inv = sm.inv_s[gi][ch * 8 + j];
      float y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = tile.value(p, i, j) * inv;
      const int quad = p * (kPassTokens / 4) + k;
      if constexpr (kFmt == kE5M6) {
        u32x2 w;
        w.x = e5m6_pair(y[0], y[1]);
        w.y = e5m6_pair(y[2], y[3]);
        *reinterpret_cast<u32x2*>(&sm.tile[tile_index<TG::kRowDw>(ch * 8 + j, 2 * quad)]) = w;
      } else if constexpr (kFmt == kE2M1) {
        sm.tile[tile_index<TG::kRowDw>(ch * 8 + j, quad)] = e2m1_bytes4(y[0], y[1], y[2], y[3]);
      } else {
        sm.tile[tile_index<TG::kRowDw>(ch * 8 + j, quad)] = fp8x4<kFmt>(y[0], y[1], y[2], y[3]);
      }
    }
  }
  __syncthreads();

  // Read back channel rows, 16 bytes of LDS per lane (16 codes; 8 of E5M6),
  // and store them to qT: 16 bytes of 8-bit codes, 8 of E2M1 nibbles, 12 of
  // E5M6 codes.
  const uint32_t row_bytes = code_bytes<kFmt>(rows);
  uint8_t* out = qT + (uint64_t)tc.c0 * row_bytes + code_bytes<kFmt>(tc.t0);
#pragma unroll
  for (int r = 0; r < TG::kReadPasses; ++r) {
    const int idx = t + r * kThreads;
    const int c = idx / TG::kRowVec;
    const int mv = idx % TG::kRowVec;
    if (c < tc.nc && mv * TG::kVecTokens < tc.ng * kGroupTokens) {
      const u32x4 val =
          *reinterpret_cast<const u32x4*>(&sm.tile[tile_index<TG::kRowDw>(c, 4 * mv)]);
      uint8_t* dst = out + (uint32_t)c * row_bytes + code_bytes<kFmt>(mv * TG::kVecTokens);
      // A tile's run of packed codes per channel is 64 bytes (E2M1) or 192
      // (E5M6), part of a 128-byte line whose other part a neighbouring tile
      // writes: plain stores let the two meet in L2 and leave as whole lines
      // (E2M1 on 16384 x 7168: 54.9 us against 57.3 with streaming stores).
      if constexpr (kFmt == kE5M6) {
        const E5M6x8 e = e5m6_pack_pairs(val.x, val.y, val.z, val.w);
        uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);
        d32[0] = e.w0;
        d32[1] = e.w1;
        d32[2] = e.w2;
      } else if constexpr (kFmt == kE2M1) {
        u32x2 o;
        o.x = e2m1_pack_bytes(val.x) | (e2m1_pack_bytes(val.y) << 16);
        o.y = e2m1_pack_bytes(val.z) | (e2m1_pack_bytes(val.w) << 16);
        *reinterpret_cast<u32x2*>(dst) = o;
      } else {
        store_stream(reinterpret_cast<u32x4*>(dst), val);
      }
    }
  }
  if (kReuse) __syncthreads();  // the LDS tile is reused by the next tile
}

// One workgroup per tile; kLayout: scale options other than plain fp32.
template <int kFmt, bool kLayout>
__global__ __launch_bounds__(kThreads) void per_channel_t_kernel(
    const uint16_t* __restrict__ x, uint32_t rows, uint32_t cols, uint32_t ngroups,
    uint32_t nct, uint32_t ntg, uint32_t ntiles, uint32_t per_xcd, FastDiv sdiv, float floor,
    SfLayout lay, uint8_t* __restrict__ qT, void* __restrict__ sf) {
  __shared__ __attribute__((aligned(16))) Smem<kFmt> sm;
  const uint32_t b = blockIdx.x;
  const uint32_t tau = (kOrder & 2) ? b : (b % kXcds) * per_xcd + b / kXcds;
  if (tau >= ntiles) return;
  const TileCoord tc = tile_coord(tau, ngroups, cols, nct, ntg, sdiv);
  Bf16Tile tile;
  load_tile(x, cols, tc, tile.raw);
  process_tile<kFmt, false, kLayout>(tc, tile, rows, floor, lay, sm, qT, sf);
}

// The cast's memory traffic alone, for measurement: the same workgroup ->
// tile walk, the same loads, and the same qT stores (each stored 16 bytes
// the XOR of two loaded vectors of the lane, so every loaded vector reaches
// exactly one store), with no scale, code or LDS work.
__global__ __launch_bounds__(kThreads) void per_channel_t_traffic_kernel(
    const uint16_t* __restrict__ x, uint32_t rows, uint32_t cols, uint32_t ngroups,
    uint32_t nct, uint32_t ntg, uint32_t ntiles, uint32_t per_xcd, FastDiv sdiv,
    uint8_t* __restrict__ qT) {
  static_assert(kPasses * 4 == 2 * kReadPasses, "two loaded vectors per stored one");
  const uint32_t b = blockIdx.x;
  const uint32_t tau = (kOrder & 2) ? b : (b % kXcds) * per_xcd + b / kXcds;
  if (tau >= ntiles) return;
  const TileCoord tc = tile_coord(tau, ngroups, cols, nct, ntg, sdiv);
  u32x4 raw[kPasses][4];
  load_tile(x, cols, tc, raw);
  const int t = threadIdx.x;
  uint8_t* out = qT + (uint64_t)tc.c0 * rows + tc.t0;
#pragma unroll
  for (int r = 0; r < kReadPasses; ++r) {
    const int idx = t + r * kThreads;
    const int c = idx / kRowVec;
    const int mv = idx % kRowVec;
    if (c < tc.nc && mv * 16 < tc.ng * kGroupTokens) {
      const u32x4 val = raw[(2 * r) / 4][(2 * r) % 4] ^ raw[(2 * r + 1) / 4][(2 * r + 1) % 4];
      store_stream(reinterpret_cast<u32x4*>(out + (uint32_t)c * rows + mv * 16), val);
    }
  }
}

// SwiGLU + the same cast. Without a clamp counter (kCountNone): one
// workgroup per tile. With a counter and a count workspace (kCountSlotted):
// the same, every workgroup (also one past the last tile) ending in one
// atomic on a workspace slot. With a counter alone (kCountDirect): every
// workgroup ends in an atomic add on the same word, serialized where the
// word lives, so a capped grid walks the virtual workgroup indices
// [0, vgrid) with a stride of gridDim.x.
template <int kFmt, bool kWeighted, bool kClamp, int kCount, bool kLayout>
__global__ __launch_bounds__(kThreads) void swiglu_per_channel_t_kernel(
    const uint16_t* __restrict__ h, const float* __restrict__ w, uint32_t rows, uint32_t cols,
    uint32_t ngroups, uint32_t nct, uint32_t ntg, uint32_t ntiles, uint32_t per_xcd,
    FastDiv sdiv, uint32_t vgrid, float floor, float clamp, SfLayout lay,
    unsigned long long* __restrict__ count, unsigned long long* __restrict__ slots,
    uint8_t* __restrict__ qT, void* __restrict__ sf) {
  __shared__ __attribute__((aligned(16))) Smem<kFmt> sm;
  if constexpr (kCount == kCountDirect) {
    uint32_t n = 0;
    for (uint32_t b = blockIdx.x; b < vgrid; b += gridDim.x) {
      const uint32_t tau = (kOrder & 2) ? b : (b % kXcds) * per_xcd + b / kXcds;
      if (tau >= ntiles) continue;  // uniform over the workgroup
      const TileCoord tc = tile_coord<kSwStrip>(tau, ngroups, cols, nct, ntg, sdiv);
      F32Tile tile;
      n += load_swiglu_tile<kWeighted, kClamp, true>(h, w, cols, clamp, tc, tile);
      process_tile<kFmt, true, kLayout>(tc, tile, rows, floor, lay, sm, qT, sf);
    }
    add_wave_counts(n, count);
  } else {
    const uint32_t b = blockIdx.x;
    const uint32_t tau = (kOrder & 2) ? b : (b % kXcds) * per_xcd + b / kXcds;
    const bool has_tile = tau < ntiles;  // uniform over the workgroup
    uint32_t n = 0;
    TileCoord tc{};
    F32Tile tile;
    if (has_tile) {
      tc = tile_coord<kSwStrip>(tau, ngroups, cols, nct, ntg, sdiv);
      n = load_swiglu_tile<kWeighted, kClamp, kCount == kCountSlotted>(h, w, cols, clamp, tc,
                                                                        tile);
    }
    // With a workspace the count goes to its slot before the tile is
    // processed, so the slot atomic's round trip overlaps that work.
    SlotCount<> sc;
    if constexpr (kCount == kCountSlotted) sc.arrive(n, slots);
    if (has_tile) process_tile<kFmt, false, kLayout>(tc, tile, rows, floor, lay, sm, qT, sf);
    if constexpr (kCount == kCountSlotted) sc.finish(slots, count);
  }
}

struct Grid {
  uint32_t ngroups, nct, ntg, ntiles, per_xcd, grid;
  FastDiv strip_div, sw_strip_div;   // by kStrip * ntg, kSwStrip * ntg
};

// Tile counts of a [rows, cols] cast; false when the kernels' 32-bit tile
// and in-tile offsets would not hold (row_stride: elements between rows; a
// tile's qT rows are kChannels code rows of `rows` codes of fmt).
bool make_grid(int64_t rows, int64_t cols, int64_t row_stride, int fmt, Grid* g) {
  const int64_t ngroups = rows / kGroupTokens;
  const int64_t ntg = (ngroups + kTG - 1) / kTG;
  const int64_t nct = (cols + kChannels - 1) / kChannels;
  const int64_t ntiles = ntg * nct;
  const int64_t lim = int64_t(1) << 31;
  if (ntiles + 2 * kXcds >= lim || (int64_t)kTileTokens * row_stride >= lim ||
      (int64_t)kChannels * rows >= lim || rows >= lim || row_stride >= lim ||
      (fmt == kE5M6 && (int64_t)kChannels * (rows / 2 * 3) >= lim))
    return false;
  const int64_t per_xcd = (ntiles + kXcds - 1) / kXcds;
  g->ngroups = (uint32_t)ngroups;
  g->nct = (uint32_t)nct;
  g->ntg = (uint32_t)ntg;
  g->strip_div = make_fast_div((uint32_t)(kStrip * ntg > 0 ? kStrip * ntg : 1));
  g->sw_strip_div = make_fast_div((uint32_t)(kSwStrip * ntg > 0 ? kSwStrip * ntg : 1));
  g->ntiles = (uint32_t)ntiles;
  g->per_xcd = (uint32_t)per_xcd;
  g->grid = (uint32_t)((kOrder & 2) ? ntiles : per_xcd * kXcds);
  return true;
}

// Workgroups per CU of the capped grid that counts clamped values (4 was
// the fastest of 1, 2, 4 and 8 on the 8192 x 2048 SwiGLU output; one
// workgroup per tile, 2048 atomics, was 25% slower).
#ifndef QCAST_PC_COUNT_WG_PER_CU
#define QCAST_PC_COUNT_WG_PER_CU 4
#endif

struct CountArgs {
  unsigned long long* count;  // device counter or null
  unsigned long long* slots;  // count workspace or null
};

template <int kFmt, bool kWeighted, bool kClamp, bool kLayout>
hipError_t launch_swiglu_t(const uint16_t* h, const float* w, int64_t rows, int64_t cols,
                           const Grid& g, float floor, float clamp, const SfLayout& lay,
                           const CountArgs& ca, uint8_t* qT, void* sf, hipStream_t stream,
                           const LaunchCaps& caps) {
  if constexpr (kClamp) {
    // The slots count the workgroups that reach them in 24 bits (and the
    // clamped values in 40: at most 2 * rows * cols, under 2^37 for any h
    // that fits in memory).
    const bool slotted =
        ca.slots && (int64_t)g.grid < (int64_t(kCountSlots) << (64 - kSlotArrivalShift));
    if (ca.count && slotted) {
      launch_kernel((swiglu_per_channel_t_kernel<kFmt, kWeighted, true, kCountSlotted, kLayout>),
                    dim3(g.grid), dim3(kThreads), 0, stream, h, w, (uint32_t)rows,
                    (uint32_t)cols, g.ngroups, g.nct, g.ntg, g.ntiles, g.per_xcd,
                    g.sw_strip_div, g.grid, floor, clamp, lay, ca.count, ca.slots, qT, sf);
      return hipGetLastError();
    }
    if (ca.count) {
      uint32_t grid = g.grid;
      const int64_t cap = (int64_t)caps.num_cus * QCAST_PC_COUNT_WG_PER_CU;
      if (QCAST_PC_COUNT_WG_PER_CU > 0 && cap < grid) grid = (uint32_t)cap;
      launch_kernel((swiglu_per_channel_t_kernel<kFmt, kWeighted, true, kCountDirect, kLayout>),
                    dim3(grid), dim3(kThreads), 0, stream, h, w, (uint32_t)rows,
                    (uint32_t)cols, g.ngroups, g.nct, g.ntg, g.ntiles, g.per_xcd,
                    g.sw_strip_div, g.grid, floor, clamp, lay, ca.count, ca.slots, qT, sf);
      return hipGetLastError();
    }
  }
  launch_kernel((swiglu_per_channel_t_kernel<kFmt, kWeighted, kClamp, kCountNone, kLayout>),
                dim3(g.grid), dim3(kThreads), 0, stream, h, w, (uint32_t)rows, (uint32_t)cols,
                g.ngroups, g.nct, g.ntg, g.ntiles, g.per_xcd, g.sw_strip_div, g.grid, floor,
                clamp, lay, ca.count, ca.slots, qT, sf);
  return hipGetLastError();
}

template <int kFmt, bool kLayout>
hipError_t launch_swiglu_t_wc(const uint16_t* h, const float* w, int64_t rows, int64_t cols,
                              const Grid& g, float floor, float clamp, const SfLayout& lay,
                              const CountArgs& ca, uint8_t* qT, void* sf, hipStream_t stream,
                              const LaunchCaps& caps) {
  if (w) {
    return clamp > 0.0f
               ? launch_swiglu_t<kFmt, true, true, kLayout>(h, w, rows, cols, g, floor, clamp,
                                                            lay, ca, qT, sf, stream, caps)
               : launch_swiglu_t<kFmt, true, false, kLayout>(h, w, rows, cols, g, floor, clamp,
                                                             lay, ca, qT, sf, stream, caps);
  }
  return clamp > 0.0f
             ? launch_swiglu_t<kFmt, false, true, kLayout>(h, w, rows, cols, g, floor, clamp,
                                                           lay, ca, qT, sf, stream, caps)
             : launch_swiglu_t<kFmt, false, false, kLayout>(h, w, rows, cols, g, floor, clamp,
                                                            lay, ca, qT, sf, stream, caps);
}

template <int kFmt>
hipError_t launch_swiglu_t_fmt(const uint16_t* h, const float* w, int64_t rows, int64_t cols,
                               const Grid& g, float floor, float clamp, const SfLayout& lay,
                               const CountArgs& ca, uint8_t* qT, void* sf, hipStream_t stream,
                               const LaunchCaps& caps) {
  return lay.flags ? launch_swiglu_t_wc<kFmt, true>(h, w, rows, cols, g, floor, clamp, lay, ca,
                                                    qT, sf, stream, caps)
                   : launch_swiglu_t_wc<kFmt, false>(h, w, rows, cols, g, floor, clamp, lay, ca,
                                                     qT, sf, stream, caps);
}

// The transposed cast's kernel for fmt, with or without scale options.
template <int kFmt>
auto cast_kernel(bool layout) {
  return layout ? per_channel_t_kernel<kFmt, true> : per_channel_t_kernel<kFmt, false>;
}

}  // namespace

bool per_channel_t_fits(int64_t rows, int64_t cols, int64_t row_stride, int fmt) {
  Grid g;
  return make_grid(rows, cols, row_stride, fmt, &g);
}

hipError_t launch_per_channel_T(const void* x, int64_t rows, int64_t cols, int fmt, float floor,
                                uint32_t sf_flags, void* qT, void* sf, hipStream_t stream,
                                const LaunchCaps& caps) {
  (void)caps;
  Grid g;
  // The kernels index tiles, and offsets inside a tile's rows, in 32 bits.
  if (!make_grid(rows, cols, cols, fmt, &g)) return hipErrorInvalidValue;
  if (g.ntiles == 0) return hipSuccess;
  if ((sf_flags & kSfPacked) && g.ngroups % 4 != 0) return hipErrorInvalidValue;
  const bool any = sf_flags != 0;
  auto kernel = fmt == kE4M3   ? cast_kernel<kE4M3>(any)
                : fmt == kE5M2 ? cast_kernel<kE5M2>(any)
                : fmt == kE2M1 ? cast_kernel<kE2M1>(any)
                : fmt == kE5M6 ? cast_kernel<kE5M6>(any)
                               : nullptr;
  if (!kernel) return hipErrorInvalidValue;
  // the layout of x^T: rows are the channels, groups the token groups
  const SfLayout lay = make_sf_layout(cols, rows, kGroupTokens, sf_flags);
  launch_kernel(kernel, dim3(g.grid), dim3(kThreads), 0, stream,
                static_cast<const uint16_t*>(x), (uint32_t)rows, (uint32_t)cols, g.ngroups,
                g.nct, g.ntg, g.ntiles, g.per_xcd, g.strip_div, floor, lay,
                static_cast<uint8_t*>(qT), sf);
  return hipGetLastError();
}

hipError_t launch_per_channel_T_traffic(const void* x, int64_t rows, int64_t cols, void* qT,
                                        hipStream_t stream) {
  Grid g;
  if (!make_grid(rows, cols, cols, kE4M3, &g)) return hipErrorInvalidValue;
  if (g.ntiles == 0) return hipSuccess;
  launch_kernel(per_channel_t_traffic_kernel, dim3(g.grid), dim3(kThreads), 0, stream,
                static_cast<const uint16_t*>(x), (uint32_t)rows, (uint32_t)cols, g.ngroups,
                g.nct, g.ntg, g.ntiles, g.per_xcd, g.strip_div, static_cast<uint8_t*>(qT));
  return hipGetLastError();
}

hipError_t launch_swiglu_per_channel_T(const void* h, int64_t rows, int64_t cols, const float* w,
                                       int fmt, float floor, uint32_t sf_flags,
                                       float swiglu_clamp, unsigned long long* clamp_count,
                                       unsigned long long* count_ws, void* qT, void* sf,
                                       hipStream_t stream, const LaunchCaps& caps) {
  Grid g;
  if (!make_grid(rows, cols, 2 * cols, fmt, &g)) return hipErrorInvalidValue;
  if (g.ntiles == 0) return hipSuccess;
  if ((sf_flags & kSfPacked) && g.ngroups % 4 != 0) return hipErrorInvalidValue;
  const SfLayout lay = make_sf_layout(cols, rows, kGroupTokens, sf_flags);
  const uint16_t* hp = static_cast<const uint16_t*>(h);
  uint8_t* qp = static_cast<uint8_t*>(qT);
  const CountArgs ca{clamp_count, count_ws};
  switch (fmt) {
    case kE4M3:
      return launch_swiglu_t_fmt<kE4M3>(hp, w, rows, cols, g, floor, swiglu_clamp, lay, ca, qp,
                                        sf, stream, caps);
    case kE5M2:
      return launch_swiglu_t_fmt<kE5M2>(hp, w, rows, cols, g, floor, swiglu_clamp, lay, ca, qp,
                                        sf, stream, caps);
    case kE2M1:
      return launch_swiglu_t_fmt<kE2M1>(hp, w, rows, cols, g, floor, swiglu_clamp, lay, ca, qp,
                                        sf, stream, caps);
    case kE5M6:
      return launch_swiglu_t_fmt<kE5M6>(hp, w, rows, cols, g, floor, swiglu_clamp, lay, ca, qp,
                                        sf, stream, caps);
  }
  return hipErrorInvalidValue;
}

}  // namespace qcast
