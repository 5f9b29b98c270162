// bench_helpers.hip -- the helpers declared in include/qcast_bench.h:
//  - start/stop events for the next kernel a thread launches, recorded by
//    the dispatch itself (hipExtLaunchKernel), for per-kernel durations;
//  - a streaming copy, the bandwidth ceiling and counter calibration for the
//    cast kernels (16-byte non-temporal loads and stores, as the casts);
//  - an exhaustive check of the kernels' scale routine against IEEE
//    division;
//  - the transposed per-channel cast's memory traffic without its
//    arithmetic (the kernel lives beside the cast, in per_channel_t.hip).
#include <atomic>

#include "qcast_bench.h"
#include "qcast_device.h"
#include "qcast_kernels.h"

namespace qcast {

namespace {
// Timing events for the next launch of the calling thread.
thread_local LaunchTiming t_timing = {nullptr, nullptr};
}  // namespace

LaunchTiming take_launch_timing() {
  const LaunchTiming t = t_timing;
  t_timing = LaunchTiming{nullptr, nullptr};
  return t;
}

namespace {

#ifndef QCAST_CP_UNROLL
#define QCAST_CP_UNROLL 4
#endif
#ifndef QCAST_CP_WG_PER_CU
#define QCAST_CP_WG_PER_CU 0
#endif
constexpr int kCopyUnroll = QCAST_CP_UNROLL;
constexpr int kCopyWgPerCu = QCAST_CP_WG_PER_CU;

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, int64_t n) {
  const int64_t step = (int64_t)gridDim.x * kThreads * kCopyUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kCopyUnroll + threadIdx.x; base < n;
       base += step) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kThreads;
      if (i < n) v[u] = load_stream(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kThreads;
      if (i < n) store_stream(dst + i, v[u]);
    }
  }
}

// Every positive pattern in [first, last] through group_scale<kFmt> (the
// routine the casts use) against the IEEE quotients; per-workgroup counts.
template <int kFmt>
__global__ __launch_bounds__(kThreads) void check_scale_kernel(uint32_t first, uint32_t last,
                                                               uint32_t* __restrict__ counts) {
  constexpr float kMax = fmt_max<kFmt>();
  __shared__ uint32_t red[2][kThreads];
  const uint64_t nthreads = (uint64_t)gridDim.x * kThreads;
  const uint64_t total = (uint64_t)last - first + 1;
  const uint64_t per = (total + nthreads - 1) / nthreads;
  const uint64_t t = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t bad_sf = 0, bad_inv = 0;
  for (uint64_t i = 0; i < per; ++i) {
    const uint64_t b = first + t * per + i;
    if (b > last) break;
    const float a = __uint_as_float((uint32_t)b);
    const Scale s = group_scale<kFmt>(a, 0.0f);
    const float sf_ref = a / kMax;
    const float inv_ref = 1.0f / sf_ref;
    bad_sf += __float_as_uint(s.sf) != __float_as_uint(sf_ref);
    bad_inv += __float_as_uint(s.inv) != __float_as_uint(inv_ref);
  }
  red[0][threadIdx.x] = bad_sf;
  red[1][threadIdx.x] = bad_inv;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      red[0][threadIdx.x] += red[0][threadIdx.x + w];
      red[1][threadIdx.x] += red[1][threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x < 2) counts[2 * blockIdx.x + threadIdx.x] = red[threadIdx.x][0];
}

}  // namespace
}  // namespace qcast

extern "C" int qcast_bench_check_scale(int fmt, uint32_t first, uint32_t last, uint32_t* counts,
                                       void* stream) {
  if (fmt != QCAST_FMT_E4M3 && fmt != QCAST_FMT_E2M1 && fmt != QCAST_FMT_E5M2 &&
      fmt != QCAST_FMT_E5M6)
    return QCAST_ERR_FORMAT;
  if (first > last || last > 0x7f7fffffu) return QCAST_ERR_SHAPE;
  if (!counts) return QCAST_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(counts) & 3) return QCAST_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fmt == QCAST_FMT_E4M3)
    qcast::launch_kernel(qcast::check_scale_kernel<qcast::kE4M3>, dim3(QCAST_CHECK_BLOCKS),
                         dim3(qcast::kThreads), 0, s, first, last, counts);
  else if (fmt == QCAST_FMT_E2M1)
    qcast::launch_kernel(qcast::check_scale_kernel<qcast::kE2M1>, dim3(QCAST_CHECK_BLOCKS),
                         dim3(qcast::kThreads), 0, s, first, last, counts);
  else if (fmt == QCAST_FMT_E5M2)
    qcast::launch_kernel(qcast::check_scale_kernel<qcast::kE5M2>, dim3(QCAST_CHECK_BLOCKS),
                         dim3(qcast::kThreads), 0, s, first, last, counts);
  else
    qcast::launch_kernel(qcast::check_scale_kernel<qcast::kE5M6>, dim3(QCAST_CHECK_BLOCKS),
                         dim3(qcast::kThreads), 0, s, first, last, counts);
  return hipGetLastError() == hipSuccess ? QCAST_OK : QCAST_ERR_LAUNCH;
}

extern "C" int qcast_bench_copy(const void* src, void* dst, int64_t nbytes, void* stream) {
  if (nbytes < 0 || nbytes % 16 != 0) return QCAST_ERR_SHAPE;
  if (nbytes == 0) return QCAST_OK;
  if (!src || !dst) return QCAST_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15)
    return QCAST_ERR_ALIGN;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return QCAST_ERR_DEVICE;
  const int64_t n = nbytes / 16;
  const int64_t per_iter = (int64_t)qcast::kThreads * qcast::kCopyUnroll;
  const int64_t iters = (n + per_iter - 1) / per_iter;
  const int64_t max_blocks = qcast::kCopyWgPerCu > 0 ? (int64_t)cus * qcast::kCopyWgPerCu : iters;
  const int64_t ipb = (iters + max_blocks - 1) / max_blocks;
  const int64_t blocks = (iters + ipb - 1) / ipb;
  qcast::launch_kernel(qcast::copy_kernel, dim3((unsigned)blocks), dim3(qcast::kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const qcast::u32x4*>(src),
                       static_cast<qcast::u32x4*>(dst), n);
  return hipGetLastError() == hipSuccess ? QCAST_OK : QCAST_ERR_LAUNCH;
}

extern "C" int qcast_bench_per_channel_T_traffic(const void* x, int64_t rows, int64_t cols,
                                                 void* qT, void* stream) {
  if (rows < 0 || cols < 0 || rows % 128 != 0 || cols % 8 != 0 ||
      !qcast::per_channel_t_fits(rows, cols, cols, QCAST_FMT_E4M3))
    return QCAST_ERR_SHAPE;
  if (rows == 0 || cols == 0) return QCAST_OK;
  if (!x || !qT) return QCAST_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(qT)) & 15)
    return QCAST_ERR_ALIGN;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QCAST_ERR_DEVICE;
  return qcast::launch_per_channel_T_traffic(x, rows, cols, qT,
                                             static_cast<hipStream_t>(stream)) == hipSuccess
             ? QCAST_OK
             : QCAST_ERR_LAUNCH;
}

extern "C" int qcast_bench_time_next(void* start_event, void* stop_event) {
  if (!start_event || !stop_event) return QCAST_ERR_NULL;
  qcast::t_timing = qcast::LaunchTiming{static_cast<hipEvent_t>(start_event),
                                        static_cast<hipEvent_t>(stop_event)};
  return QCAST_OK;
}
