// qcast_abi.hip -- the C ABI declared in include/qcast.h: argument checks,
// the format floors, the compute-unit count, and dispatch to the launchers.
//
// Floors ("DeepSeek开源TileKernels：用Python写的GPU算子逼近硬件性能上限", §3.1):
// 1e-4 for E4M3 and the E2M1 maximum times 2^-126 for E2M1, unless the caller
// passes its own clamp_min > 0; E5M2 and E5M6, for which the page names
// none, take the E4M3 floor.
#include <atomic>
#include <mutex>

#include "qcast.h"
#include "qcast_device.h"
#include "qcast_kernels.h"

// The clamp-count slots of qcast_swiglu_per_token_noalloc: a file-scope
// device array (one copy per GPU, held until the process ends), used in
// place of a caller's count workspace. Host code never passes its name to a
// kernel (on the host it is only a stand-in for the symbol); it uses the
// device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned long long scratch[QCAST_NOALLOC_SCRATCH_BYTES / 8];

namespace {

static_assert(qcast::kCountSlots * qcast::kSlotWords * sizeof(uint64_t) == QCAST_COUNT_WS_BYTES,
              "count workspace size");

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];   // 0 = not queried yet
std::atomic<int> g_cu_override{0};

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

float default_floor(int fmt) {
  if (fmt == QCAST_FMT_E2M1) return 6.0f * 0x1.0p-126f;   // E2M1 maximum times 2^-126
  return 1e-4f;   // E4M3; E5M2 and E5M6 take the same floor
}

bool any_fmt(int fmt) {
  return fmt == QCAST_FMT_E4M3 || fmt == QCAST_FMT_E2M1 || fmt == QCAST_FMT_E5M2 ||
         fmt == QCAST_FMT_E5M6;
}

float floor_for(int fmt, float clamp_min) {
  return clamp_min > 0.0f ? clamp_min : default_floor(fmt);
}

// A caller's floor must be a number below +inf: NaN would silently select the
// default, and +inf would make every scale infinite (and, rounded to a power
// of two, wrap its inverse's exponent).
bool clamp_min_ok(float c) { return c == c && c <= 3.4028235e38f; }

int caps_for_current_device(qcast::LaunchCaps* caps) {
  const int override_n = g_cu_override.load(std::memory_order_relaxed);
  if (override_n > 0) {
    caps->num_cus = override_n;
    return QCAST_OK;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return QCAST_ERR_DEVICE;
  if (dev < kMaxDevices) {
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
      if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
          n <= 0)
        return QCAST_ERR_DEVICE;
      g_cu_count[dev].store(n, std::memory_order_relaxed);
    }
    caps->num_cus = n;
    return QCAST_OK;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return QCAST_ERR_DEVICE;
  caps->num_cus = n;
  return QCAST_OK;
}

int finish(hipError_t err) { return err == hipSuccess ? QCAST_OK : QCAST_ERR_LAUNCH; }

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_for_current_device(unsigned long long** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QCAST_ERR_DEVICE;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
        return QCAST_ERR_DEVICE;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = static_cast<unsigned long long*>(p);
  return QCAST_OK;
}

// Zeroes n 64-bit words (a fill kernel, not a memset: a caller may capture
// the call in a graph).
__global__ __launch_bounds__(qcast::kThreads) void zero_words(unsigned long long* p, int n) {
  for (int i = threadIdx.x; i < n; i += qcast::kThreads) p[i] = 0ull;
}

// A clamp bound of +inf clamps nothing; so does any bound <= 0.
float clamp_value(float c) { return (c > 0.0f && c <= 3.4028235e38f) ? c : 0.0f; }

bool per_token_group_ok(int group) { return group == 32 || group == 64 || group == 128; }

bool sf_flags_ok(int flags) {
  return (flags & ~(QCAST_SF_ROUND_POW2 | QCAST_SF_COL_MAJOR | QCAST_SF_PACKED_UE8M0)) == 0;
}

// Group indices are 32-bit in the scale store; packed words need whole
// quadruples of groups in every row.
bool sf_shape_ok(int64_t rows, int64_t cols, int group, int flags) {
  if (cols > 0 && rows > ((int64_t(1) << 31) - 1) / (cols / group > 0 ? cols / group : 1))
    return false;
  if ((flags & QCAST_SF_PACKED_UE8M0) && (cols / group) % 4 != 0) return false;
  return true;
}

// Element counts beyond 2^62 would overflow the kernels' int64 offsets.
bool too_big(int64_t rows, int64_t cols) {
  return cols > 0 && rows > (int64_t(1) << 62) / cols;
}

// Argument checks of the per-token SwiGLU casts, before any HIP call;
// *empty when the call casts nothing (and launches nothing).
int check_swiglu_ex(const void* h, int64_t rows, int64_t cols, const float* row_weight, int fmt,
                    int group, float clamp_min, int sf_flags, float swiglu_clamp, const void* q,
                    const void* sf, const uint64_t* clamp_count, const void* count_ws,
                    bool* empty) {
  *empty = false;
  if (!any_fmt(fmt)) return QCAST_ERR_FORMAT;
  if (!sf_flags_ok(sf_flags)) return QCAST_ERR_FORMAT;
  if (!per_token_group_ok(group)) return QCAST_ERR_GROUP;
  if (rows < 0 || cols < 0 || cols % group != 0 || cols / 8 >= (int64_t(1) << 16) ||
      too_big(rows, 2 * cols) || !sf_shape_ok(rows, cols, group, sf_flags))
    return QCAST_ERR_SHAPE;
  if (swiglu_clamp != swiglu_clamp) return QCAST_ERR_VALUE;
  if (!clamp_min_ok(clamp_min)) return QCAST_ERR_VALUE;
  if (rows == 0 || cols == 0) {
    *empty = true;
    return QCAST_OK;
  }
  if (!h || !q || !sf) return QCAST_ERR_NULL;
  if (!aligned(h, 16) || !aligned(q, 16) || !aligned(sf, 4) ||
      (row_weight && !aligned(row_weight, 4)) || (clamp_count && !aligned(clamp_count, 8)) ||
      (count_ws && !aligned(count_ws, 128)))
    return QCAST_ERR_ALIGN;
  return QCAST_OK;
}

}  // namespace

extern "C" {

int qcast_abi_version(void) { return QCAST_ABI_VERSION; }

const char* qcast_status_str(int status) {
  switch (status) {
    case QCAST_OK: return "ok";
    case QCAST_ERR_NULL: return "a required pointer is NULL";
    case QCAST_ERR_SHAPE:
      return "unsupported shape (negative, not divisible as required, or past the 32-bit "
             "indexing limits)";
    case QCAST_ERR_ALIGN: return "pointer not aligned as required";
    case QCAST_ERR_FORMAT: return "format not supported by this entry point";
    case QCAST_ERR_GROUP: return "group or block size not supported";
    case QCAST_ERR_LAUNCH: return "kernel launch failed";
    case QCAST_ERR_DEVICE: return "no usable HIP device";
    case QCAST_ERR_VALUE: return "a scalar argument is out of range";
  }
  return "unknown status";
}

void qcast_set_num_cus(int n) { g_cu_override.store(n > 0 ? n : 0, std::memory_order_relaxed); }

int qcast_per_token_sf(const void* x, int64_t rows, int64_t cols, int fmt, int group,
                       float clamp_min, int sf_flags, void* q, void* sf, void* stream) {
  if (!any_fmt(fmt)) return QCAST_ERR_FORMAT;
  if (!sf_flags_ok(sf_flags)) return QCAST_ERR_FORMAT;
  if (!per_token_group_ok(group)) return QCAST_ERR_GROUP;
  if (rows < 0 || cols < 0 || cols % group != 0 || too_big(rows, cols) ||
      !sf_shape_ok(rows, cols, group, sf_flags))
    return QCAST_ERR_SHAPE;
  if (!clamp_min_ok(clamp_min)) return QCAST_ERR_VALUE;
  if (rows == 0 || cols == 0) return QCAST_OK;
  if (!x || !q || !sf) return QCAST_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(sf, 4)) return QCAST_ERR_ALIGN;
  qcast::LaunchCaps caps;
  const int rc = caps_for_current_device(&caps);
  if (rc != QCAST_OK) return rc;
  return finish(qcast::launch_per_token(x, rows, cols, fmt, group, floor_for(fmt, clamp_min),
                                        (uint32_t)sf_flags, q, sf,
                                        static_cast<hipStream_t>(stream), caps));
}

int qcast_per_token(const void* x, int64_t rows, int64_t cols, int fmt, int group,
                    float clamp_min, void* q, float* sf, void* stream) {
  return qcast_per_token_sf(x, rows, cols, fmt, group, clamp_min, 0, q, sf, stream);
}

int qcast_e2m1(const void* x, int64_t rows, int64_t cols, int group, float clamp_min,
               uint8_t* q_packed, float* sf, void* stream) {
  return qcast_per_token(x, rows, cols, QCAST_FMT_E2M1, group, clamp_min, q_packed, sf, stream);
}

int qcast_swiglu_per_token_ex(const void* h, int64_t rows, int64_t cols,
                              const float* row_weight, int fmt, int group, float clamp_min,
                              int sf_flags, float swiglu_clamp, void* q, void* sf,
                              uint64_t* clamp_count, void* count_ws, void* stream) {
  bool empty = false;
  int rc = check_swiglu_ex(h, rows, cols, row_weight, fmt, group, clamp_min, sf_flags,
                           swiglu_clamp, q, sf, clamp_count, count_ws, &empty);
  if (rc != QCAST_OK || empty) return rc;
  qcast::LaunchCaps caps;
  if ((rc = caps_for_current_device(&caps)) != QCAST_OK) return rc;
  return finish(qcast::launch_swiglu_per_token(
      h, rows, cols, row_weight, fmt, group, floor_for(fmt, clamp_min), (uint32_t)sf_flags,
      clamp_value(swiglu_clamp), reinterpret_cast<unsigned long long*>(clamp_count),
      static_cast<unsigned long long*>(count_ws), q, sf, static_cast<hipStream_t>(stream), caps));
}

int qcast_swiglu_per_token_noalloc(const void* h, int64_t rows, int64_t cols,
                                   const float* row_weight, int fmt, int group, float clamp_min,
                                   int sf_flags, float swiglu_clamp, void* q, void* sf,
                                   uint64_t* clamp_count, void* stream) {
  static_assert(sizeof(scratch) == QCAST_NOALLOC_SCRATCH_BYTES, "scratch size");
  bool empty = false;
  int rc = check_swiglu_ex(h, rows, cols, row_weight, fmt, group, clamp_min, sf_flags,
                           swiglu_clamp, q, sf, clamp_count, nullptr, &empty);
  if (rc != QCAST_OK || empty) return rc;
  // The count slots are reused by every slab of rows, so every shape needs
  // QCAST_COUNT_WS_BYTES of scratch, no more; a library built with a
  // smaller array refuses the counting call.
  const bool counting = clamp_count && clamp_value(swiglu_clamp) > 0.0f;
  if (counting && sizeof(scratch) < QCAST_COUNT_WS_BYTES) return QCAST_ERR_SHAPE;
  qcast::LaunchCaps caps;
  if ((rc = caps_for_current_device(&caps)) != QCAST_OK) return rc;
  unsigned long long* slots = nullptr;
  if (counting) {
    if ((rc = scratch_for_current_device(&slots)) != QCAST_OK) return rc;
    // The array keeps what the last call on this GPU left in it: clear the
    // slots on the stream, ahead of the cast.
    hipLaunchKernelGGL(zero_words, dim3(1), dim3(qcast::kThreads), 0,
                       static_cast<hipStream_t>(stream), slots,
                       (int)(QCAST_COUNT_WS_BYTES / sizeof(unsigned long long)));
    if (hipGetLastError() != hipSuccess) return QCAST_ERR_LAUNCH;
  }
  return finish(qcast::launch_swiglu_per_token(
      h, rows, cols, row_weight, fmt, group, floor_for(fmt, clamp_min), (uint32_t)sf_flags,
      clamp_value(swiglu_clamp), reinterpret_cast<unsigned long long*>(clamp_count), slots, q,
      sf, static_cast<hipStream_t>(stream), caps));
}

int qcast_swiglu_per_token_sf(const void* h, int64_t rows, int64_t cols,
                              const float* row_weight, int fmt, int group, float clamp_min,
                              int sf_flags, void* q, void* sf, void* stream) {
  return qcast_swiglu_per_token_ex(h, rows, cols, row_weight, fmt, group, clamp_min, sf_flags,
                                   0.0f, q, sf, nullptr, nullptr, stream);
}

int qcast_swiglu_backward_per_token_sf(const void* h, const void* dv, int64_t rows,
                                       int64_t cols, const float* row_weight, int fmt, int group,
                                       float clamp_min, int sf_flags, float swiglu_clamp, void* q,
                                       void* sf, void* stream) {
  if (!any_fmt(fmt)) return QCAST_ERR_FORMAT;
  if (!sf_flags_ok(sf_flags)) return QCAST_ERR_FORMAT;
  if (!per_token_group_ok(group)) return QCAST_ERR_GROUP;
  // The scales are those of rows of 2 * cols values; a packed word never
  // straddles the dg and du halves.
  if (rows < 0 || cols < 0 || cols % group != 0 || cols / 8 >= (int64_t(1) << 16) ||
      too_big(rows, 2 * cols) || !sf_shape_ok(rows, 2 * cols, group, sf_flags) ||
      ((sf_flags & QCAST_SF_PACKED_UE8M0) && (cols / group) % 4 != 0))
    return QCAST_ERR_SHAPE;
  if (swiglu_clamp != swiglu_clamp) return QCAST_ERR_VALUE;
  if (!clamp_min_ok(clamp_min)) return QCAST_ERR_VALUE;
  if (rows == 0 || cols == 0) return QCAST_OK;
  if (!h || !dv || !q || !sf) return QCAST_ERR_NULL;
  if (!aligned(h, 16) || !aligned(dv, 16) || !aligned(q, 16) || !aligned(sf, 4) ||
      (row_weight && !aligned(row_weight, 4)))
    return QCAST_ERR_ALIGN;
  qcast::LaunchCaps caps;
  const int rc = caps_for_current_device(&caps);
  if (rc != QCAST_OK) return rc;
  return finish(qcast::launch_swiglu_backward(
      h, dv, rows, cols, row_weight, fmt, group, floor_for(fmt, clamp_min), (uint32_t)sf_flags,
      clamp_value(swiglu_clamp), q, sf, static_cast<hipStream_t>(stream), caps));
}

int qcast_swiglu_backward_per_token(const void* h, const void* dv, int64_t rows, int64_t cols,
                                    const float* row_weight, int fmt, int group, float clamp_min,
                                    float swiglu_clamp, void* q, float* sf, void* stream) {
  return qcast_swiglu_backward_per_token_sf(h, dv, rows, cols, row_weight, fmt, group, clamp_min,
                                            0, swiglu_clamp, q, sf, stream);
}

int qcast_swiglu_per_channel_T_sf(const void* h, int64_t rows, int64_t cols,
                                  const float* row_weight, int fmt, int group, float clamp_min,
                                  int sf_flags, float swiglu_clamp, void* qT, void* sf,
                                  uint64_t* clamp_count, void* count_ws, void* stream) {
  if (!any_fmt(fmt)) return QCAST_ERR_FORMAT;
  if (!sf_flags_ok(sf_flags)) return QCAST_ERR_FORMAT;
  if (group != 128) return QCAST_ERR_GROUP;
  if (rows < 0 || cols < 0 || rows % group != 0 || cols % 8 != 0 || too_big(rows, 2 * cols) ||
      !qcast::per_channel_t_fits(rows, cols, 2 * cols, fmt) ||
      ((sf_flags & QCAST_SF_PACKED_UE8M0) && (rows / group) % 4 != 0))
    return QCAST_ERR_SHAPE;
  if (swiglu_clamp != swiglu_clamp) return QCAST_ERR_VALUE;
  if (!clamp_min_ok(clamp_min)) return QCAST_ERR_VALUE;
  if (rows == 0 || cols == 0) return QCAST_OK;
  if (!h || !qT || !sf) return QCAST_ERR_NULL;
  if (!aligned(h, 16) || !aligned(qT, 16) || !aligned(sf, 4) ||
      (row_weight && !aligned(row_weight, 4)) || (clamp_count && !aligned(clamp_count, 8)) ||
      (count_ws && !aligned(count_ws, 128)))
    return QCAST_ERR_ALIGN;
  qcast::LaunchCaps caps;
  const int rc = caps_for_current_device(&caps);
  if (rc != QCAST_OK) return rc;
  return finish(qcast::launch_swiglu_per_channel_T(
      h, rows, cols, row_weight, fmt, floor_for(fmt, clamp_min), (uint32_t)sf_flags,
      clamp_value(swiglu_clamp), reinterpret_cast<unsigned long long*>(clamp_count),
      static_cast<unsigned long long*>(count_ws), qT, sf, static_cast<hipStream_t>(stream),
      caps));
}

int qcast_swiglu_per_channel_T(const void* h, int64_t rows, int64_t cols, const float* row_weight,
                               int fmt, int group, float clamp_min, float swiglu_clamp, void* qT,
                               float* sf, uint64_t* clamp_count, void* count_ws,
                               void* stream) {
  return qcast_swiglu_per_channel_T_sf(h, rows, cols, row_weight, fmt, group, clamp_min, 0,
                                       swiglu_clamp, qT, sf, clamp_count, count_ws, stream);
}

int qcast_swiglu_per_token(const void* h, int64_t rows, int64_t cols, const float* row_weight,
                           int fmt, int group, float clamp_min, void* q, float* sf,
                           void* stream) {
  return qcast_swiglu_per_token_sf(h, rows, cols, row_weight, fmt, group, clamp_min, 0, q, sf,
                                   stream);
}

int qcast_per_block_sf(const void* x, int64_t rows, int64_t cols, int fmt, int block,
                       float clamp_min, int sf_flags, void* q, float* sf, void* stream) {
  if (!any_fmt(fmt)) return QCAST_ERR_FORMAT;
  if (sf_flags & ~QCAST_SF_ROUND_POW2) return QCAST_ERR_FORMAT;
  if (block != 128) return QCAST_ERR_GROUP;
  if (rows < 0 || cols < 0 || rows % block != 0 || cols % block != 0 || too_big(rows, cols) ||
      !qcast::per_block_fits(rows, cols))
    return QCAST_ERR_SHAPE;
  if (!clamp_min_ok(clamp_min)) return QCAST_ERR_VALUE;
  if (rows == 0 || cols == 0) return QCAST_OK;
  if (!x || !q || !sf) return QCAST_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(sf, 4)) return QCAST_ERR_ALIGN;
  qcast::LaunchCaps caps;
  const int rc = caps_for_current_device(&caps);
  if (rc != QCAST_OK) return rc;
  return finish(qcast::launch_per_block(x, rows, cols, fmt, floor_for(fmt, clamp_min),
                                        (uint32_t)sf_flags, q, sf,
                                        static_cast<hipStream_t>(stream), caps));
}

int qcast_per_block(const void* x, int64_t rows, int64_t cols, int fmt, int block,
                    float clamp_min, void* q, float* sf, void* stream) {
  return qcast_per_block_sf(x, rows, cols, fmt, block, clamp_min, 0, q, sf, stream);
}

int qcast_per_channel_T_sf(const void* x, int64_t rows, int64_t cols, int fmt, int group,
                           float clamp_min, int sf_flags, void* qT, void* sf, void* stream) {
  if (!any_fmt(fmt)) return QCAST_ERR_FORMAT;
  if (!sf_flags_ok(sf_flags)) return QCAST_ERR_FORMAT;
  if (group != 128) return QCAST_ERR_GROUP;
  if (rows < 0 || cols < 0 || rows % group != 0 || cols % 8 != 0 || too_big(rows, cols) ||
      !qcast::per_channel_t_fits(rows, cols, cols, fmt) ||
      ((sf_flags & QCAST_SF_PACKED_UE8M0) && (rows / group) % 4 != 0))
    return QCAST_ERR_SHAPE;
  if (!clamp_min_ok(clamp_min)) return QCAST_ERR_VALUE;
  if (rows == 0 || cols == 0) return QCAST_OK;
  if (!x || !qT || !sf) return QCAST_ERR_NULL;
  if (!aligned(x, 16) || !aligned(qT, 16) || !aligned(sf, 4)) return QCAST_ERR_ALIGN;
  qcast::LaunchCaps caps;
  const int rc = caps_for_current_device(&caps);
  if (rc != QCAST_OK) return rc;
  return finish(qcast::launch_per_channel_T(x, rows, cols, fmt, floor_for(fmt, clamp_min),
                                            (uint32_t)sf_flags, qT, sf,
                                            static_cast<hipStream_t>(stream), caps));
}

int qcast_per_channel_T(const void* x, int64_t rows, int64_t cols, int fmt, int group,
                        float clamp_min, void* qT, float* sf, void* stream) {
  return qcast_per_channel_T_sf(x, rows, cols, fmt, group, clamp_min, 0, qT, sf, stream);
}

int qcast_per_channel_sf(const void* x, int64_t rows, int64_t cols, int fmt, int group,
                         float clamp_min, int sf_flags, void* q, float* sf, void* stream) {
  if (!any_fmt(fmt)) return QCAST_ERR_FORMAT;
  if (sf_flags & ~QCAST_SF_ROUND_POW2) return QCAST_ERR_FORMAT;
  if (group != 128) return QCAST_ERR_GROUP;
  if (rows < 0 || cols < 0 || rows % group != 0 || cols % 8 != 0 || too_big(rows, cols) ||
      !qcast::per_channel_fits(rows, cols))
    return QCAST_ERR_SHAPE;
  if (!clamp_min_ok(clamp_min)) return QCAST_ERR_VALUE;
  if (rows == 0 || cols == 0) return QCAST_OK;
  if (!x || !q || !sf) return QCAST_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(sf, 4)) return QCAST_ERR_ALIGN;
  qcast::LaunchCaps caps;
  const int rc = caps_for_current_device(&caps);
  if (rc != QCAST_OK) return rc;
  return finish(qcast::launch_per_channel(x, rows, cols, fmt, floor_for(fmt, clamp_min),
                                          (uint32_t)sf_flags, q, sf,
                                          static_cast<hipStream_t>(stream), caps));
}

int qcast_per_channel(const void* x, int64_t rows, int64_t cols, int fmt, int group,
                      float clamp_min, void* q, float* sf, void* stream) {
  return qcast_per_channel_sf(x, rows, cols, fmt, group, clamp_min, 0, q, sf, stream);
}

int qcast_cast_back(const void* q, const float* sf, int64_t rows, int64_t cols, int fmt,
                    int group, int out_dtype, void* out, void* stream) {
  if (!any_fmt(fmt)) return QCAST_ERR_FORMAT;
  if (out_dtype != QCAST_OUT_BF16 && out_dtype != QCAST_OUT_F32) return QCAST_ERR_FORMAT;
  if (!per_token_group_ok(group)) return QCAST_ERR_GROUP;
  if (rows < 0 || cols < 0 || cols % group != 0 || too_big(rows, cols) ||
      !qcast::cast_back_fits(rows, cols))
    return QCAST_ERR_SHAPE;
  if (rows == 0 || cols == 0) return QCAST_OK;
  if (!q || !sf || !out) return QCAST_ERR_NULL;
  if (!aligned(q, 16) || !aligned(sf, 4) || !aligned(out, 16)) return QCAST_ERR_ALIGN;
  qcast::LaunchCaps caps;
  const int rc = caps_for_current_device(&caps);
  if (rc != QCAST_OK) return rc;
  return finish(qcast::launch_cast_back(q, sf, rows, cols, fmt, group, out_dtype == QCAST_OUT_BF16,
                                        out, static_cast<hipStream_t>(stream), caps));
}

}  // extern "C"
