/*
 * abi_check.c - the C ABI of libawq_gfx950 used from plain C (no Python, no C++).
 *
 * One small layer (N = 256, K = 1024, groups of 128, asymmetric format) goes through
 * awq_channel_scale, awq_pack, awq_repack, awq_dequant (both layouts), awq_gemv and
 * awq_gemm on the current HIP device. The host checks, in float64:
 *   - the dequantized weights (q - z) * s rounded to binary16 from the canonical packed
 *     words it reads back, against both device dequantizers, bit for bit;
 *   - y from awq_gemv and awq_gemm against sum_k (x * inv_s_c) * W_d in float64, within
 *     2e-3 of max |y| (the library's stated accuracy);
 *   - error statuses for a few invalid calls (returned before any launch).
 * Exit status 0 and "abi_check: ok" on success.
 *
 * Weights and activations are small integers over powers of two, so every input is an
 * exact binary16 value and the host needs only an exact encoder for them.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "awq.h"

#define N 256
#define K 1024
#define M 3
#define G 128

static int failures = 0;

static void check(int cond, const char* what) {
  if (!cond) {
    fprintf(stderr, "abi_check: FAILED: %s\n", what);
    ++failures;
  }
}

#define HIP(call)                                                              \
  do {                                                                         \
    hipError_t e_ = (call);                                                    \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "abi_check: %s: %s\n", #call, hipGetErrorString(e_));    \
      exit(2);                                                                 \
    }                                                                          \
  } while (0)

/* binary16 bits -> double (every binary16 value is exact in double) */
static double half_to_double(uint16_t h) {
  const int sign = h >> 15, e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24);
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(f | 1024), e - 25);
  }
  return sign ? -v : v;
}

/* double -> binary16 bits, round to nearest, ties to even, subnormals kept */
static uint16_t double_to_half(double v) {
  uint16_t sign = 0;
  if (v < 0 || (v == 0 && signbit(v))) {
    sign = 0x8000;
    v = -v;
  }
  if (isnan(v)) return 0x7E00;
  if (v >= 65520.0) return sign | 0x7C00;
  if (v < ldexp(1.0, -14)) {
    /* subnormal range: units of 2^-24 */
    const double q = v * ldexp(1.0, 24);
    double r = floor(q);
    const double frac = q - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) == 1.0)) r += 1.0;
    return sign | (uint16_t)r;
  }
  int e;
  (void)frexp(v, &e); /* v = m * 2^e, 0.5 <= m < 1 */
  const double ulp = ldexp(1.0, e - 11);
  const double q = v / ulp; /* in [1024, 2048) */
  double r = floor(q);
  const double frac = q - r;
  if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) == 1.0)) r += 1.0;
  int exp16 = e - 1 + 15;
  int man = (int)r;
  if (man == 2048) {
    man = 1024;
    ++exp16;
  }
  if (exp16 >= 31) return sign | 0x7C00;
  return sign | (uint16_t)(exp16 << 10) | (uint16_t)(man - 1024);
}

static uint32_t lcg_state = 12345u;
static int lcg(int range) {
  lcg_state = lcg_state * 1664525u + 1013904223u;
  return (int)((lcg_state >> 8) % (uint32_t)range);
}

int main(void) {
  const char* s0 = awq_status_string(AWQ_OK);
  check(s0 != NULL && strlen(s0) > 0, "status string");
  check(awq_layout_version() > 0, "layout version");

  int ndev = 0;
  HIP(hipGetDeviceCount(&ndev));
  if (ndev < 1) {
    fprintf(stderr, "abi_check: no HIP device\n");
    return 2;
  }

  /* host inputs: exact binary16 values */
  static uint16_t w[N * K], xcal[32 * K], x[M * K];
  for (int i = 0; i < N * K; ++i) w[i] = double_to_half((lcg(61) - 30) / 1024.0);
  for (int i = 0; i < 32 * K; ++i) xcal[i] = double_to_half((lcg(33) - 16) / 8.0);
  for (int i = 0; i < M * K; ++i) x[i] = double_to_half((lcg(33) - 16) / 8.0);

  uint16_t *d_w, *d_xcal, *d_x, *d_sc, *d_inv, *d_scales, *d_y1, *d_y2, *d_wd0, *d_wd1;
  int32_t *d_qw, *d_qz;
  void *d_packed, *d_ws = NULL;
  const size_t packed_bytes = awq_repacked_bytes(N, K, G, AWQ_FMT_ASYM);
  const size_t ws_bytes = awq_workspace_bytes(M, N, K, G);
  check(packed_bytes > 0, "repacked bytes");
  HIP(hipMalloc((void**)&d_w, sizeof w));
  HIP(hipMalloc((void**)&d_xcal, sizeof xcal));
  HIP(hipMalloc((void**)&d_x, sizeof x));
  HIP(hipMalloc((void**)&d_sc, K * 2));
  HIP(hipMalloc((void**)&d_inv, K * 2));
  HIP(hipMalloc((void**)&d_qw, (size_t)N * (K / 8) * 4));
  HIP(hipMalloc((void**)&d_scales, (size_t)(K / G) * N * 2));
  HIP(hipMalloc((void**)&d_qz, (size_t)(K / G) * (N / 8) * 4));
  HIP(hipMalloc(&d_packed, packed_bytes));
  HIP(hipMalloc((void**)&d_y1, (size_t)M * N * 2));
  HIP(hipMalloc((void**)&d_y2, (size_t)M * N * 2));
  HIP(hipMalloc((void**)&d_wd0, (size_t)N * K * 2));
  HIP(hipMalloc((void**)&d_wd1, (size_t)N * K * 2));
  if (ws_bytes > 0) HIP(hipMalloc(&d_ws, ws_bytes));
  HIP(hipMemcpy(d_w, w, sizeof w, hipMemcpyHostToDevice));
  HIP(hipMemcpy(d_xcal, xcal, sizeof xcal, hipMemcpyHostToDevice));
  HIP(hipMemcpy(d_x, x, sizeof x, hipMemcpyHostToDevice));

  hipStream_t st;
  HIP(hipStreamCreate(&st));
  check(awq_channel_scale(d_xcal, 32, K, 0.5, d_sc, d_inv, st) == AWQ_OK, "awq_channel_scale");
  check(awq_pack(d_w, d_sc, N, K, G, AWQ_FMT_ASYM, d_qw, d_scales, d_qz, st) == AWQ_OK, "awq_pack");
  check(awq_repack(d_qw, d_scales, d_qz, N, K, G, AWQ_FMT_ASYM, d_packed, packed_bytes, st) == AWQ_OK,
        "awq_repack");
  check(awq_dequant(d_qw, d_scales, d_qz, AWQ_LAYOUT_CANONICAL, N, K, G, AWQ_FMT_ASYM, d_wd0, st) ==
            AWQ_OK,
        "awq_dequant canonical");
  check(awq_dequant(d_packed, NULL, NULL, AWQ_LAYOUT_GFX950, N, K, G, AWQ_FMT_ASYM, d_wd1, st) == AWQ_OK,
        "awq_dequant gfx950");
  check(awq_gemv(d_x, d_inv, d_packed, M, N, K, G, AWQ_FMT_ASYM, d_y1, d_ws, ws_bytes, st) == AWQ_OK,
        "awq_gemv");
  check(awq_gemm(d_x, d_inv, d_packed, M, N, K, G, AWQ_FMT_ASYM, d_y2, d_ws, ws_bytes, st) == AWQ_OK,
        "awq_gemm");
  /* rejected before any launch */
  check(awq_gemv(d_x, d_inv, d_packed, 17, N, K, G, AWQ_FMT_ASYM, d_y1, d_ws, ws_bytes, st) ==
            AWQ_ERR_UNSUPPORTED,
        "gemv M > 16 rejected");
  check(awq_gemm(d_x, d_inv, d_packed, M, N, K, 96, AWQ_FMT_ASYM, d_y2, d_ws, ws_bytes, st) ==
            AWQ_ERR_INVALID_ARG ||
        awq_gemm(d_x, d_inv, d_packed, M, N, K, 96, AWQ_FMT_ASYM, d_y2, d_ws, ws_bytes, st) ==
            AWQ_ERR_UNSUPPORTED,
        "group 96 rejected");
  check(awq_gemm((const uint16_t*)((const char*)d_x + 2), d_inv, d_packed, M, N, K, G, AWQ_FMT_ASYM,
                 d_y2, d_ws, ws_bytes, st) == AWQ_ERR_MISALIGNED,
        "misaligned x rejected");
  HIP(hipStreamSynchronize(st));

  static int32_t qw[N * (K / 8)], qz[(K / G) * (N / 8)];
  static uint16_t scales[(K / G) * N], inv[K], wd0[N * K], wd1[N * K], y1[M * N], y2[M * N];
  HIP(hipMemcpy(qw, d_qw, sizeof qw, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(qz, d_qz, sizeof qz, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(scales, d_scales, sizeof scales, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(inv, d_inv, sizeof inv, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(wd0, d_wd0, sizeof wd0, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(wd1, d_wd1, sizeof wd1, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(y1, d_y1, sizeof y1, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(y2, d_y2, sizeof y2, hipMemcpyDeviceToHost));

  /* W_d from the canonical words, as the header defines them */
  static double wd[N * K];
  int deq_mismatch = 0;
  for (int n = 0; n < N; ++n) {
    for (int k = 0; k < K; ++k) {
      const uint32_t word = (uint32_t)qw[n * (K / 8) + k / 8];
      const int q = (int)((word >> (4 * (k % 8))) & 15u);
      const int g = k / G;
      const uint32_t zw = (uint32_t)qz[g * (N / 8) + n / 8];
      const int z = (int)((zw >> (4 * (n % 8))) & 15u);
      const double s = half_to_double(scales[g * N + n]);
      const uint16_t h = double_to_half((double)(q - z) * s);
      wd[n * K + k] = half_to_double(h);
      if (wd0[n * K + k] != h || wd1[n * K + k] != h) ++deq_mismatch;
    }
  }
  check(deq_mismatch == 0, "dequantized weights bit-exact in both layouts");

  double maxref = 0.0, err1 = 0.0, err2 = 0.0;
  for (int m = 0; m < M; ++m) {
    for (int n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int k = 0; k < K; ++k) acc += half_to_double(x[m * K + k]) * half_to_double(inv[k]) * wd[n * K + k];
      if (fabs(acc) > maxref) maxref = fabs(acc);
      const double e1 = fabs(half_to_double(y1[m * N + n]) - acc);
      const double e2 = fabs(half_to_double(y2[m * N + n]) - acc);
      if (e1 > err1) err1 = e1;
      if (e2 > err2) err2 = e2;
    }
  }
  err1 /= maxref;
  err2 /= maxref;
  check(maxref > 0.0, "nonzero product");
  check(err1 <= 2e-3, "awq_gemv within 2e-3");
  check(err2 <= 2e-3, "awq_gemm within 2e-3");

  HIP(hipStreamDestroy(st));
  hipFree(d_w); hipFree(d_xcal); hipFree(d_x); hipFree(d_sc); hipFree(d_inv); hipFree(d_qw);
  hipFree(d_scales); hipFree(d_qz); hipFree(d_packed); hipFree(d_y1); hipFree(d_y2);
  hipFree(d_wd0); hipFree(d_wd1);
  if (d_ws) hipFree(d_ws);
  if (failures) return 1;
  printf("abi_check: ok (gemv %.2e, gemm %.2e of max|y|, %d weights bit-exact)\n", err1, err2, N * K);
  return 0;
}
