/*
 * qcast_bench.h -- measurement and self-check helpers exported by
 * libqcast.so. None is part of the quantization method.
 *
 * qcast_bench_copy: a plain streaming copy with the casts' access pattern
 * (16-byte non-temporal loads and stores, 256-thread workgroups). bench.py
 * times it as the empirical bandwidth ceiling and reads its HBM byte
 * counters to calibrate those of the casts (a copy of n bytes must read n
 * and write n bytes).
 *
 * qcast_bench_time_next: hands a pair of HIP events to the next kernel the
 * calling thread launches through the library, which records them from the
 * dispatch itself (hipExtLaunchKernel): their elapsed time is that kernel's
 * own duration, with no marker packets around it.
 *
 * qcast_bench_per_channel_T_traffic: the memory traffic of qcast_per_channel_T
 * alone -- its workgroup-to-tile walk, its loads and its qT stores, with no
 * arithmetic -- so that bench.py can time the ceiling the transposed layout
 * sets for that cast, next to the copy's.
 *
 * qcast_bench_check_scale: runs the kernels' own scale routine on a range of
 * fp32 bit patterns and counts where it differs from the IEEE quotients
 * a / fmt_max and 1 / sf. The casts compute sf and sf_inv with short FMA
 * sequences in the common range and fall back to IEEE division elsewhere;
 * this entry point lets a test check that claim over every positive fp32.
 */
#ifndef QCAST_BENCH_H
#define QCAST_BENCH_H

#include <stdint.h>

#include "qcast.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Copy nbytes from src to dst (device pointers, 16-byte aligned, nbytes a
 * multiple of 16, not overlapping) on `stream`. Returns a qcast_status:
 * QCAST_ERR_NULL, QCAST_ERR_ALIGN or QCAST_ERR_SHAPE before any HIP call,
 * QCAST_ERR_LAUNCH if the launch fails. nbytes == 0 launches nothing. */
QCAST_API int qcast_bench_copy(const void* src, void* dst, int64_t nbytes, void* stream);

/* The next kernel launched by the calling thread through any entry point
 * records start_event when it begins and stop_event when it ends (both
 * hipEvent_t, created by the caller on the launch's device; the library
 * keeps no reference after that launch). An entry point that launches
 * several kernels (inputs split into slabs) times only its first; one that
 * returns an error before launching leaves the events pending for the next
 * launch. Returns QCAST_ERR_NULL if either event is null. */
QCAST_API int qcast_bench_time_next(void* start_event, void* stop_event);

/* Loads x [rows, cols] bf16 and stores qT [cols, rows] bytes exactly as
 * qcast_per_channel_T with group 128 does (same launch, same addresses);
 * every stored 16 bytes is the XOR of two 16-byte vectors the same lane
 * loaded. With cols a multiple of 64 (whole channel tiles) every loaded
 * vector goes into exactly one store, so the XOR of all of qT's 16-byte
 * vectors equals that of all of x's. No scales are written. Same
 * shape, limit and alignment rules as qcast_per_channel_T: QCAST_ERR_SHAPE,
 * QCAST_ERR_NULL or QCAST_ERR_ALIGN before any HIP call, QCAST_ERR_LAUNCH if
 * the launch fails; rows == 0 or cols == 0 launches nothing. */
QCAST_API int qcast_bench_per_channel_T_traffic(const void* x, int64_t rows, int64_t cols,
                                                void* qT, void* stream);

/* Number of workgroups of qcast_bench_check_scale: `counts` holds two
 * uint32 per workgroup. */
#define QCAST_CHECK_BLOCKS 2048

/* For every bit pattern b in [first, last] (as fp32 a = b, taken as the
 * group abs-max with a zero floor), compare the kernels' (sf, sf_inv) for
 * format `fmt` with (a / fmt_max, 1 / (a / fmt_max)) computed by IEEE
 * division. counts (device, uint32 [2 * QCAST_CHECK_BLOCKS], written, not
 * accumulated) receives per workgroup the number of sf mismatches and of
 * sf_inv mismatches. Requires first <= last <= 0x7f7fffff (positive finite
 * patterns). Returns QCAST_ERR_FORMAT, QCAST_ERR_SHAPE, QCAST_ERR_NULL or
 * QCAST_ERR_ALIGN before any HIP call, QCAST_ERR_LAUNCH if the launch fails. */
QCAST_API int qcast_bench_check_scale(int fmt, uint32_t first, uint32_t last, uint32_t* counts,
                                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QCAST_BENCH_H */
