/*
 * abi_smoke.c -- the C ABI used from plain C, with no Python or torch: read
 * bf16 bit patterns [rows, cols] from a file, run the five casts of the hot
 * path on the current HIP device -- per-token E4M3 (groups of 128), the
 * transposed per-channel cast, packed E2M1 (groups of 32), the 128x128
 * per-block cast, and SwiGLU + per-token E4M3 (groups of 64, no routing
 * weight) reading the same rows as [gate | up] halves of cols/2 each --
 * and the transposed cast again with round_sf column-major scales
 * (qcast_per_channel_T_sf), and write codes and scales to files for the
 * test to compare with the oracle.
 *
 *   abi_smoke IN ROWS COLS OUT_PREFIX
 * writes OUT_PREFIX.{q,sf,qT,sfT,q4,sf4,qb,sfb,qs,sfs,qTr,sfTr}; prints "ok" and
 * returns 0, or prints the failing call and its status text and returns 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "qcast.h"

static int fail(const char* what, int status) {
  fprintf(stderr, "%s: %s\n", what, qcast_status_str(status));
  return 1;
}

static int hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return 1;
  fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return 0;
}

static int save(const char* prefix, const char* ext, const void* dev, size_t n) {
  char path[4096];
  snprintf(path, sizeof path, "%s.%s", prefix, ext);
  void* host = malloc(n ? n : 1);
  if (!host || !hip_ok(hipMemcpy(host, dev, n, hipMemcpyDeviceToHost), "hipMemcpy D2H")) return 0;
  FILE* f = fopen(path, "wb");
  const int ok = f && fwrite(host, 1, n, f) == n;
  if (f) fclose(f);
  free(host);
  return ok;
}

int main(int argc, char** argv) {
  if (argc != 5) {
    fprintf(stderr, "usage: %s IN ROWS COLS OUT_PREFIX\n", argv[0]);
    return 2;
  }
  const int64_t rows = atoll(argv[2]), cols = atoll(argv[3]);
  const size_t n = (size_t)(rows * cols);
  uint16_t* host = malloc(2 * n);
  FILE* f = fopen(argv[1], "rb");
  if (!host || !f || fread(host, 2, n, f) != n) {
    fprintf(stderr, "cannot read %zu bf16 values from %s\n", n, argv[1]);
    return 2;
  }
  fclose(f);
  const size_t nb = (size_t)(rows / 128) * (size_t)(cols / 128); /* per-block scales */
  const int64_t half = cols / 2;                                   /* SwiGLU outputs per row */
  const size_t ns = (size_t)(rows * half);
  const size_t ntr = (size_t)(rows / 128) * (size_t)((cols + 3) / 4 * 4); /* col-major sf */
  void *x, *q, *sf, *qT, *sfT, *q4, *sf4, *qb, *sfb, *qs, *sfs, *qTr, *sfTr;
  if (!hip_ok(hipMalloc(&x, 2 * n), "hipMalloc") || !hip_ok(hipMalloc(&q, n), "hipMalloc") ||
      !hip_ok(hipMalloc(&sf, n / 128 * 4), "hipMalloc") || !hip_ok(hipMalloc(&qT, n), "hipMalloc") ||
      !hip_ok(hipMalloc(&sfT, n / 128 * 4), "hipMalloc") ||
      !hip_ok(hipMalloc(&q4, n / 2), "hipMalloc") || !hip_ok(hipMalloc(&sf4, n / 32 * 4), "hipMalloc") ||
      !hip_ok(hipMalloc(&qb, n), "hipMalloc") || !hip_ok(hipMalloc(&sfb, nb * 4 + 4), "hipMalloc") ||
      !hip_ok(hipMalloc(&qs, ns + 1), "hipMalloc") || !hip_ok(hipMalloc(&sfs, ns / 64 * 4 + 4), "hipMalloc") ||
      !hip_ok(hipMalloc(&qTr, n), "hipMalloc") || !hip_ok(hipMalloc(&sfTr, ntr * 4 + 4), "hipMalloc"))
    return 1;
  if (!hip_ok(hipMemcpy(x, host, 2 * n, hipMemcpyHostToDevice), "hipMemcpy H2D")) return 1;
  int rc = qcast_per_token(x, rows, cols, QCAST_FMT_E4M3, 128, 0.0f, q, (float*)sf, NULL);
  if (rc != QCAST_OK) return fail("qcast_per_token", rc);
  rc = qcast_per_channel_T(x, rows, cols, QCAST_FMT_E4M3, 128, 0.0f, qT, (float*)sfT, NULL);
  if (rc != QCAST_OK) return fail("qcast_per_channel_T", rc);
  rc = qcast_e2m1(x, rows, cols, 32, 0.0f, (uint8_t*)q4, (float*)sf4, NULL);
  if (rc != QCAST_OK) return fail("qcast_e2m1", rc);
  rc = qcast_per_block(x, rows, cols, QCAST_FMT_E4M3, 128, 0.0f, qb, (float*)sfb, NULL);
  if (rc != QCAST_OK) return fail("qcast_per_block", rc);
  rc = qcast_swiglu_per_token(x, rows, half, NULL, QCAST_FMT_E4M3, 64, 0.0f, qs, (float*)sfs, NULL);
  if (rc != QCAST_OK) return fail("qcast_swiglu_per_token", rc);
  rc = qcast_per_channel_T_sf(x, rows, cols, QCAST_FMT_E4M3, 128, 0.0f,
                              QCAST_SF_ROUND_POW2 | QCAST_SF_COL_MAJOR, qTr, sfTr, NULL);
  if (rc != QCAST_OK) return fail("qcast_per_channel_T_sf", rc);
  /* an argument error comes back before anything is launched */
  rc = qcast_per_token(x, rows, cols, QCAST_FMT_E4M3, 100, 0.0f, q, (float*)sf, NULL);
  if (rc != QCAST_ERR_GROUP) return fail("qcast_per_token with group 100", rc);
  if (!hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize")) return 1;
  if (!save(argv[4], "q", q, n) || !save(argv[4], "sf", sf, n / 128 * 4) ||
      !save(argv[4], "qT", qT, n) || !save(argv[4], "sfT", sfT, n / 128 * 4) ||
      !save(argv[4], "q4", q4, n / 2) || !save(argv[4], "sf4", sf4, n / 32 * 4) ||
      !save(argv[4], "qb", qb, n) || !save(argv[4], "sfb", sfb, nb * 4) ||
      !save(argv[4], "qs", qs, ns) || !save(argv[4], "sfs", sfs, ns / 64 * 4) ||
      !save(argv[4], "qTr", qTr, n) || !save(argv[4], "sfTr", sfTr, ntr * 4)) {
    fprintf(stderr, "cannot write the outputs\n");
    return 1;
  }
  hipFree(x); hipFree(q); hipFree(sf); hipFree(qT); hipFree(sfT); hipFree(q4); hipFree(sf4);
  hipFree(qb); hipFree(sfb); hipFree(qs); hipFree(sfs); hipFree(qTr); hipFree(sfTr);
  free(host);
  printf("ok\n");
  return 0;
}
