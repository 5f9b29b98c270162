// qcast_kernels.h -- launchers of the gfx950 cast kernels (internal to the
// library; the C ABI in qcast_abi.hip validates arguments before calling).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qcast_device.h"

namespace qcast {

// Start and stop events for the next kernel launched by the calling thread
// (qcast_bench_time_next); both null when none were asked for. Taking them
// clears them.
struct LaunchTiming {
  hipEvent_t start;
  hipEvent_t stop;
};
LaunchTiming take_launch_timing();

// Every kernel of the library is launched through here: with timing events
// pending, hipExtLaunchKernel records them from the dispatch itself (the
// kernel's own start and end, with no marker packets around it).
template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem,
                          hipStream_t stream, Args... args) {
  const LaunchTiming t = take_launch_timing();
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, t.start, t.stop, 0u, args...);
}

// Whether a shape fits the kernels' 32-bit tile counts and in-tile offsets
// (checked by the C ABI before any HIP call; the launchers check again).
bool per_block_fits(int64_t rows, int64_t cols);
bool per_channel_t_fits(int64_t rows, int64_t cols, int64_t row_stride, int fmt);
bool per_channel_fits(int64_t rows, int64_t cols);
bool cast_back_fits(int64_t rows, int64_t cols);

// Launch shape knobs shared by the launchers.
struct LaunchCaps {
  int num_cus;          // compute units on the device (or the override)
};

// The scale-factor layout of a per-token cast of [rows, cols] with `group`.
inline SfLayout make_sf_layout(int64_t rows, int64_t cols, int group, uint32_t flags) {
  SfLayout lay;
  lay.flags = (flags & kSfPacked) ? (flags | kSfRound) : flags;
  lay.gpr = (uint32_t)(cols / group);
  lay.rows_pad = (uint32_t)((rows + 3) / 4 * 4);
  lay.inv_gpr = lay.gpr ? 1.0 / (double)lay.gpr : 0.0;
  return lay;
}

// x [rows, cols] bf16 -> per-token codes + scales in the layout sf_flags
// (kSf* bits); group in {32, 64, 128}; fmt kE4M3, kE5M2 or kE2M1. Requires
// cols % group == 0, and (cols / group) % 4 == 0 for kSfPacked.
hipError_t launch_per_token(const void* x, int64_t rows, int64_t cols, int fmt, int group,
                            float floor, uint32_t sf_flags, void* q, void* sf,
                            hipStream_t stream, const LaunchCaps& caps);

// h [rows, 2*cols] bf16 (gate | up), w [rows] fp32 or null -> 8-bit codes
// (kE4M3 / kE5M2) + scales of silu(gate) * up * w; group in {32, 64, 128};
// cols % group == 0. swiglu_clamp > 0 clamps gate and up first and adds the
// number of changed values to *clamp_count (when not null), through the
// zeroed count workspace count_ws (kCountSlots slots, left zeroed) when that
// is not null, else with one atomic per workgroup of a capped grid.
hipError_t launch_swiglu_per_token(const void* h, int64_t rows, int64_t cols, const float* w,
                                   int fmt, int group, float floor, uint32_t sf_flags,
                                   float swiglu_clamp, unsigned long long* clamp_count,
                                   unsigned long long* count_ws, void* q, void* sf,
                                   hipStream_t stream, const LaunchCaps& caps);

// SwiGLU backward: h [rows, 2*cols] bf16, dv [rows, cols] bf16, w or null
// -> codes of the rows [dgate | dup] (2*cols columns each) + scales in the
// per-token layout sf_flags of those rows; (cols / group) % 4 == 0 for
// kSfPacked.
hipError_t launch_swiglu_backward(const void* h, const void* dv, int64_t rows, int64_t cols,
                                  const float* w, int fmt, int group, float floor,
                                  uint32_t sf_flags, float swiglu_clamp, void* q, void* sf,
                                  hipStream_t stream, const LaunchCaps& caps);

// x [rows, cols] bf16 -> codes + one scale per 128 x 128 block (rounded up
// to a power of two when sf_flags has kSfRound; no other option).
hipError_t launch_per_block(const void* x, int64_t rows, int64_t cols, int fmt, float floor,
                            uint32_t sf_flags, void* q, float* sf, hipStream_t stream,
                            const LaunchCaps& caps);

// x [rows (tokens), cols (channels)] bf16 -> qT [cols, rows] codes + scales
// in the per-token layout sf_flags of x^T (rows = the cols channels, groups
// = the rows/128 token groups); rows % 128 == 0, cols % 8 == 0, and
// (rows / 128) % 4 == 0 for kSfPacked.
hipError_t launch_per_channel_T(const void* x, int64_t rows, int64_t cols, int fmt, float floor,
                                uint32_t sf_flags, void* qT, void* sf, hipStream_t stream,
                                const LaunchCaps& caps);

// The memory traffic of launch_per_channel_T alone (same grid, loads and
// qT stores; meaningless bytes, no scales), for measurement.
hipError_t launch_per_channel_T_traffic(const void* x, int64_t rows, int64_t cols, void* qT,
                                        hipStream_t stream);

// SwiGLU of h [rows, 2*cols] (clamped when swiglu_clamp > 0, changed values
// added to *clamp_count when not null, through count_ws as above), then the
// per-channel cast written transposed: qT [cols, rows], scales as
// launch_per_channel_T writes them.
hipError_t launch_swiglu_per_channel_T(const void* h, int64_t rows, int64_t cols, const float* w,
                                       int fmt, float floor, uint32_t sf_flags,
                                       float swiglu_clamp, unsigned long long* clamp_count,
                                       unsigned long long* count_ws, void* qT, void* sf,
                                       hipStream_t stream, const LaunchCaps& caps);

// x [rows (tokens), cols (channels)] bf16 -> q [rows, cols] 8-bit codes in the
// input layout + sf [rows/128, cols] (rounded up to powers of two with
// kSfRound, the one option); rows % 128 == 0, cols % 8 == 0.
hipError_t launch_per_channel(const void* x, int64_t rows, int64_t cols, int fmt, float floor,
                              uint32_t sf_flags, void* q, float* sf, hipStream_t stream,
                              const LaunchCaps& caps);

// q per-token codes [rows, cols] (or [rows, cols/2] E2M1) + sf [rows, cols/group]
// -> out [rows, cols] bf16 (out_bf16) or fp32: decode(q) * sf.
hipError_t launch_cast_back(const void* q, const float* sf, int64_t rows, int64_t cols, int fmt,
                            int group, bool out_bf16, void* out, hipStream_t stream,
                            const LaunchCaps& caps);

}  // namespace qcast
