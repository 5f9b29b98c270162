// qcast_kernels.h -- launchers of the gfx950 cast kernels (internal to the
// library; the C ABI in qcast_abi.hip validates arguments before calling).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qcast {

// Launch shape knobs shared by the launchers.
struct LaunchCaps {
  int num_cus;          // compute units on the device (or the override)
};

// x [rows, cols] bf16 -> per-token codes + scales; group in {32, 64, 128};
// fmt kE4M3 or kE2M1. Requires cols % group == 0.
hipError_t launch_per_token(const void* x, int64_t rows, int64_t cols, int fmt, int group,
                            float floor, void* q, float* sf, hipStream_t stream,
                            const LaunchCaps& caps);

// h [rows, 2*cols] bf16 (gate | up), w [rows] fp32 or null -> E4M3 codes +
// scales of silu(gate) * up * w; group in {32, 64, 128}; cols % group == 0.
hipError_t launch_swiglu_per_token(const void* h, int64_t rows, int64_t cols, const float* w,
                                   int group, float floor, void* q, float* sf,
                                   hipStream_t stream, const LaunchCaps& caps);

// x [rows, cols] bf16 -> E4M3 codes + one scale per 128 x 128 block.
hipError_t launch_per_block(const void* x, int64_t rows, int64_t cols, float floor, void* q,
                            float* sf, hipStream_t stream, const LaunchCaps& caps);

// x [rows (tokens), cols (channels)] bf16 -> qT [cols, rows] E4M3 codes +
// sf [cols, rows/128]; rows % 128 == 0, cols % 8 == 0.
hipError_t launch_per_channel_T(const void* x, int64_t rows, int64_t cols, float floor,
                                void* qT, float* sf, hipStream_t stream,
                                const LaunchCaps& caps);

}  // namespace qcast
