/*
 * A C99 consumer of the library: include/w4a16.h and the HIP runtime's C API
 * only (no C++, no Python, no PyTorch).  It packs seeded codes on the device,
 * runs the dense product at M = 3 and M = 1, the LM head with argmax and the
 * routed product, and checks every result against the CPU oracle
 * (oracle/oracle.c, linked as test infrastructure):
 *   - packed words bit for bit against the oracle's packing;
 *   - fp32 outputs within 1e-3 * sum_k |w x| of the oracle's fp64 sums;
 *   - each row of the M = 3 call bit for bit equal to the M = 1 call on it;
 *   - the argmax equal to the lowest index of the largest returned logit;
 *   - an unsupported group size rejected with a status string.
 * Exit status 0 and a final line "ok" on success.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "w4a16.h"

/* oracle entry points (oracle/oracle.c) */
int orc_pack_rows(const uint8_t *codes, int64_t N, int64_t K, uint32_t *qw);
int orc_qmm(const uint16_t *x, const uint32_t *qw, const uint16_t *scales, const uint16_t *biases, int64_t M,
            int64_t N, int64_t K, int64_t G, const int32_t *rows, int64_t R, double *y, double *absy);
int orc_qmm_id(const uint16_t *x, int x_per_slot, const uint32_t *qw, const uint16_t *scales,
               const uint16_t *biases, const int32_t *ids, int64_t M, int64_t top_k, int64_t E, int64_t N,
               int64_t K, int64_t G, double *y, double *absy);
uint16_t orc_f64_to_bf16(double v);

#define CHECK_HIP(call)                                                            \
  do {                                                                             \
    hipError_t e_ = (call);                                                        \
    if (e_ != hipSuccess) {                                                        \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_));   \
      exit(2);                                                                     \
    }                                                                              \
  } while (0)
#define CHECK_W4(call)                                                             \
  do {                                                                             \
    w4a16_status_t s_ = (call);                                                    \
    if (s_ != W4A16_OK) {                                                          \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, w4a16_status_str(s_));   \
      exit(3);                                                                     \
    }                                                                              \
  } while (0)
#define FAIL(...)                     \
  do {                                \
    fprintf(stderr, __VA_ARGS__);     \
    fputc('\n', stderr);              \
    exit(1);                          \
  } while (0)

/* splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
   generators", 2014) as the seeded source of every input */
static uint64_t sm_state = 0x243F6A8885A308D3ull;
static uint64_t sm_next(void) {
  uint64_t z = (sm_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static double sm_unit(void) { return (double)(sm_next() >> 11) * 0x1p-53; }

static void *dev_copy(const void *h, size_t bytes) {
  void *d = NULL;
  CHECK_HIP(hipMalloc(&d, bytes));
  CHECK_HIP(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  return d;
}

static float bits_f32(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

/* |y32 - y64| <= 1e-3 * sum|w x| for every element */
static void check_close(const float *y32, const double *y64, const double *absy, size_t n, const char *what) {
  for (size_t i = 0; i < n; ++i)
    if (!(fabs((double)y32[i] - y64[i]) <= 1e-3 * absy[i]))
      FAIL("%s: element %zu: gpu %.9g oracle %.9g bound %.3g", what, i, (double)y32[i], y64[i], 1e-3 * absy[i]);
}

int main(void) {
  enum { M = 3, N = 300, K = 512, G = 64, E = 4, TOPK = 2 };
  const int NG = K / G;

  /* weights of E experts (expert 0 doubles as the dense matrix) */
  const size_t ncode = (size_t)E * N * K, nword = ncode / 8, ngrp = (size_t)E * N * NG;
  uint8_t *codes = malloc(ncode);
  uint32_t *qw_ref = malloc(nword * 4), *qw = malloc(nword * 4);
  uint16_t *sc = malloc(ngrp * 2), *bi = malloc(ngrp * 2), *x = malloc((size_t)M * K * 2);
  for (size_t i = 0; i < ncode; ++i) codes[i] = (uint8_t)(sm_next() & 15u);
  for (size_t i = 0; i < ngrp; ++i) {
    sc[i] = orc_f64_to_bf16(0.002 + 0.018 * sm_unit());
    bi[i] = orc_f64_to_bf16(-8.0 * (double)bits_f32((uint32_t)sc[i] << 16) + 0.002 * (sm_unit() - 0.5));
  }
  for (int i = 0; i < M * K; ++i) x[i] = orc_f64_to_bf16(2.0 * sm_unit() - 1.0);
  if (orc_pack_rows(codes, (int64_t)E * N, K, qw_ref)) FAIL("oracle packing failed");

  /* pack on the device */
  uint8_t *d_codes = dev_copy(codes, ncode);
  uint32_t *d_qw = NULL;
  CHECK_HIP(hipMalloc((void **)&d_qw, nword * 4));
  CHECK_W4(w4a16_pack(d_codes, d_qw, E * N, K, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(qw, d_qw, nword * 4, hipMemcpyDeviceToHost));
  if (memcmp(qw, qw_ref, nword * 4)) FAIL("w4a16_pack differs from the oracle's packing");

  uint16_t *d_s = dev_copy(sc, ngrp * 2), *d_b = dev_copy(bi, ngrp * 2), *d_x = dev_copy(x, (size_t)M * K * 2);

  /* dense product, M = 3 and M = 1 per row */
  double *y64 = malloc(sizeof(double) * M * N * TOPK), *a64 = malloc(sizeof(double) * M * N * TOPK);
  float *y = malloc(sizeof(float) * M * N * TOPK), *y1 = malloc(sizeof(float) * N);
  float *d_y = NULL;
  CHECK_HIP(hipMalloc((void **)&d_y, sizeof(float) * M * N * TOPK));
  CHECK_W4(w4a16_matmul(d_x, d_qw, d_s, d_b, d_y, W4A16_OUT_F32, M, N, K, G, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(y, d_y, sizeof(float) * M * N, hipMemcpyDeviceToHost));
  if (orc_qmm(x, qw_ref, sc, bi, M, N, K, G, NULL, N, y64, a64)) FAIL("oracle qmm failed");
  check_close(y, y64, a64, (size_t)M * N, "dense M = 3");
  for (int m = 0; m < M; ++m) {
    CHECK_W4(w4a16_matmul(d_x + (size_t)m * K, d_qw, d_s, d_b, d_y, W4A16_OUT_F32, 1, N, K, G, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(y1, d_y, sizeof(float) * N, hipMemcpyDeviceToHost));
    for (int n = 0; n < N; ++n)
      if (f32_bits(y1[n]) != f32_bits(y[m * N + n])) FAIL("row %d col %d: M = 1 differs from M = 3", m, n);
  }

  /* LM head with argmax over the same matrix */
  size_t ws_bytes = w4a16_lmhead_argmax_workspace_bytes(M, N, K, G);
  if (!ws_bytes) FAIL("no workspace size");
  void *d_ws = NULL;
  int32_t *d_am = NULL, am[M];
  CHECK_HIP(hipMalloc(&d_ws, ws_bytes));
  CHECK_HIP(hipMalloc((void **)&d_am, sizeof(am)));
  CHECK_W4(w4a16_lmhead_argmax(d_x, d_qw, d_s, d_b, d_y, W4A16_OUT_F32, d_am, d_ws, ws_bytes, M, N, K, G, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(am, d_am, sizeof(am), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(y, d_y, sizeof(float) * M * N, hipMemcpyDeviceToHost));
  check_close(y, y64, a64, (size_t)M * N, "LM head logits");
  for (int m = 0; m < M; ++m) {
    int best = 0;
    for (int n = 1; n < N; ++n)
      if (y[m * N + n] > y[m * N + best]) best = n;
    if (am[m] != best) FAIL("row %d: argmax %d, largest logit at %d", m, am[m], best);
  }

  /* routed product: token m takes experts (m + j) mod E */
  int32_t ids[M * TOPK];
  for (int m = 0; m < M; ++m)
    for (int j = 0; j < TOPK; ++j) ids[m * TOPK + j] = (m + j) % E;
  int32_t *d_ids = dev_copy(ids, sizeof(ids));
  CHECK_W4(w4a16_matmul_id(d_x, 0, d_qw, d_s, d_b, d_ids, d_y, W4A16_OUT_F32, M, TOPK, E, N, K, G, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(y, d_y, sizeof(float) * M * N * TOPK, hipMemcpyDeviceToHost));
  if (orc_qmm_id(x, 0, qw_ref, sc, bi, ids, M, TOPK, E, N, K, G, y64, a64)) FAIL("oracle qmm_id failed");
  check_close(y, y64, a64, (size_t)M * TOPK * N, "routed");

  /* an unsupported group size is refused before anything runs */
  w4a16_status_t st = w4a16_matmul(d_x, d_qw, d_s, d_b, d_y, W4A16_OUT_F32, M, N, K, 32, NULL);
  if (st != W4A16_ERR_UNSUPPORTED || !w4a16_status_str(st)[0]) FAIL("group 32 not refused");

  hipFree(d_codes); hipFree(d_qw); hipFree(d_s); hipFree(d_b); hipFree(d_x); hipFree(d_y);
  hipFree(d_ws); hipFree(d_am); hipFree(d_ids);
  free(codes); free(qw_ref); free(qw); free(sc); free(bi); free(x); free(y64); free(a64); free(y); free(y1);
  puts("ok");
  return 0;
}
