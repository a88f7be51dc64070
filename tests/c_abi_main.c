/*
 * A plain C caller of the library: include/int8lin.h compiled as C99, the
 * HIP runtime for device memory, the NULL (default) stream, no PyTorch.
 *
 * It runs the integer special cases of the layer, whose results are exact
 * and equal to the textbook integer matrix products (bitsandbytes PR #33:
 * the 127 scale of the dequantization review; forward and memory-efficient
 * backward of the PR description):
 *   - weights W integer-valued in [-127, 127] with +-127 in every row,
 *     quantized by int8_quantize_rowwise with tau off: CB = W, SCB = 127;
 *   - activations A of the same kind (fp32): the forward's codes equal A and
 *     its row scales are 127, so C32 = A W^T exactly and, with tau off and
 *     no bias, out = C32 * 127 * 127 / 127^2 = C32 (exact in fp32 here);
 *   - the backward with SCB = 127 dequantizes Wdq = fp16(CB * fl32(127 *
 *     fl32(1/127))) = CB exactly, so with G in {-1, 0, 1}: grad_A = G W
 *     exactly and grad_bias = the column sums of G;
 *   - the allocation-free forward returns the forward's bits.
 * Shapes span several tiles with ragged tails. Prints "c abi ok" and
 * returns 0 when every element matches.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "int8lin.h"

#define HIP_OK(x)                                                               \
  do {                                                                          \
    hipError_t e_ = (x);                                                        \
    if (e_ != hipSuccess) {                                                     \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                   \
      return 1;                                                                 \
    }                                                                           \
  } while (0)

#define I8L_OK_(x)                                                              \
  do {                                                                          \
    int rc_ = (x);                                                              \
    if (rc_ != I8L_OK) {                                                        \
      fprintf(stderr, "%s: %s\n", #x, int8_linear_strerror(rc_));               \
      return 1;                                                                 \
    }                                                                           \
  } while (0)

/* integer in [-127, 127] from a small hash; column (r * 7) % cols of row r is +-127 */
static float int_value(int64_t r, int64_t c, int64_t cols, uint32_t salt) {
  if (c == (r * 7) % cols) return (r & 1) ? -127.0f : 127.0f;
  uint32_t h = (uint32_t)(r * 2654435761u) ^ (uint32_t)(c * 40503u) ^ salt;
  h ^= h >> 15;
  h *= 2246822519u;
  h ^= h >> 13;
  return (float)((int)(h % 255u) - 127);
}

static int run(int64_t M, int64_t K, int64_t N) {
  printf("case M=%lld K=%lld N=%lld\n", (long long)M, (long long)K, (long long)N);
  fflush(stdout);
  float* hA = malloc((size_t)(M * K) * sizeof(float));
  float* hW = malloc((size_t)(N * K) * sizeof(float));
  float* hG = malloc((size_t)(M * N) * sizeof(float));
  float* hOut = malloc((size_t)(M * N) * sizeof(float));
  float* hOut2 = malloc((size_t)(M * N) * sizeof(float));
  int32_t* hC32 = malloc((size_t)(M * N) * sizeof(int32_t));
  float* hGA = malloc((size_t)(M * K) * sizeof(float));
  float* hGB = malloc((size_t)N * sizeof(float));
  int8_t* hCB = malloc((size_t)(N * K));
  float* hSCB = malloc((size_t)N * sizeof(float));
  if (!hA || !hW || !hG || !hOut || !hOut2 || !hC32 || !hGA || !hGB || !hCB || !hSCB) return 1;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) hA[m * K + k] = int_value(m, k, K, 0x1234u);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) hW[n * K + k] = int_value(n, k, K, 0x9e37u);
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) hG[m * N + n] = (float)((int)((m * 5 + n * 3) % 3) - 1);

  void *dA, *dW, *dG, *dOut, *dOut2, *dC32, *dGA, *dGB, *dCB, *dSCB, *dCnt, *dQws, *dFws, *dBws;
  const size_t qws = int8_quantize_rowwise_workspace_bytes(N, K);
  const int32_t cap = 0;
  const size_t fws = int8_linear_forward_workspace_bytes(M, K, N, cap);
  const size_t bws = int8_linear_backward_workspace_bytes(M, N, 1);
  HIP_OK(hipMalloc(&dA, (size_t)(M * K) * 4));
  HIP_OK(hipMalloc(&dW, (size_t)(N * K) * 4));
  HIP_OK(hipMalloc(&dG, (size_t)(M * N) * 4));
  HIP_OK(hipMalloc(&dOut, (size_t)(M * N) * 4));
  HIP_OK(hipMalloc(&dOut2, (size_t)(M * N) * 4));
  HIP_OK(hipMalloc(&dC32, (size_t)(M * N) * 4));
  HIP_OK(hipMalloc(&dGA, (size_t)(M * K) * 4));
  HIP_OK(hipMalloc(&dGB, (size_t)N * 4));
  HIP_OK(hipMalloc(&dCB, (size_t)(N * K)));
  HIP_OK(hipMalloc(&dSCB, (size_t)N * 4));
  HIP_OK(hipMalloc(&dCnt, 4));
  HIP_OK(hipMalloc(&dQws, qws > 0 ? qws : 1));
  HIP_OK(hipMalloc(&dFws, fws));
  HIP_OK(hipMalloc(&dBws, bws > 0 ? bws : 1));
  HIP_OK(hipMemcpy(dA, hA, (size_t)(M * K) * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dW, hW, (size_t)(N * K) * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dG, hG, (size_t)(M * N) * 4, hipMemcpyHostToDevice));

  /* weights: tau off (threshold 0), no outlier buffers (cap 0) */
  I8L_OK_(int8_quantize_rowwise(dW, I8L_F32, N, K, 0.0f, (int8_t*)dCB, (float*)dSCB, NULL, (int32_t*)dCnt, NULL, 0,
                                dQws, qws, NULL));
  I8L_OK_(int8_linear_forward(dA, I8L_F32, M, K, (const int8_t*)dCB, (const float*)dSCB, N, NULL, 0.0f, cap, dOut,
                              (int32_t*)dC32, dFws, fws, NULL));
  int32_t count = -1;
  I8L_OK_(int8_linear_forward_check(dFws, M, K, N, cap, NULL, &count));
  if (int8_linear_forward_noalloc_bytes(M, K, N) <= int8_linear_forward_noalloc_max_bytes())
    I8L_OK_(int8_linear_forward_noalloc(dA, I8L_F32, M, K, (const int8_t*)dCB, (const float*)dSCB, N, NULL, 0.0f,
                                        dOut2, NULL));
  I8L_OK_(int8_linear_backward_input(dG, I8L_F32, M, N, (const int8_t*)dCB, (const float*)dSCB, K, dGA, dGB, dBws,
                                     bws, NULL));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(hCB, dCB, (size_t)(N * K), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hSCB, dSCB, (size_t)N * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hOut, dOut, (size_t)(M * N) * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hOut2, dOut2, (size_t)(M * N) * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hC32, dC32, (size_t)(M * N) * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hGA, dGA, (size_t)(M * K) * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hGB, dGB, (size_t)N * 4, hipMemcpyDeviceToHost));

  /* the integer operands, for the host products (|sums| < 2^31) */
  int16_t* iA = malloc((size_t)(M * K) * sizeof(int16_t));
  int16_t* iW = malloc((size_t)(N * K) * sizeof(int16_t));
  if (!iA || !iW) return 1;
  for (int64_t i = 0; i < M * K; ++i) iA[i] = (int16_t)hA[i];
  for (int64_t i = 0; i < N * K; ++i) iW[i] = (int16_t)hW[i];
  int64_t bad = 0;
  if (count != 0) { fprintf(stderr, "outlier count %d with tau off\n", count); ++bad; }
  for (int64_t n = 0; n < N; ++n) {
    if (hSCB[n] != 127.0f) ++bad;
    for (int64_t k = 0; k < K; ++k) bad += (float)hCB[n * K + k] != hW[n * K + k];
  }
  if (bad) { fprintf(stderr, "weight codes or scales differ (%lld)\n", (long long)bad); return 1; }
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      const int16_t* a = iA + m * K;
      const int16_t* w = iW + n * K;
      int32_t s = 0;
      for (int64_t k = 0; k < K; ++k) s += (int32_t)a[k] * (int32_t)w[k];
      bad += hC32[m * N + n] != s;
      bad += hOut[m * N + n] != (float)s;
      if (int8_linear_forward_noalloc_bytes(M, K, N) <= int8_linear_forward_noalloc_max_bytes())
        bad += memcmp(&hOut[m * N + n], &hOut2[m * N + n], 4) != 0;
    }
  if (bad) { fprintf(stderr, "forward differs from the integer product (%lld)\n", (long long)bad); return 1; }
  int32_t* row = malloc((size_t)K * sizeof(int32_t));
  if (!row) return 1;
  for (int64_t m = 0; m < M; ++m) {
    memset(row, 0, (size_t)K * sizeof(int32_t));
    for (int64_t n = 0; n < N; ++n) {
      const int32_t g = (int32_t)hG[m * N + n];
      const int16_t* w = iW + n * K;
      if (g != 0)
        for (int64_t k = 0; k < K; ++k) row[k] += g * (int32_t)w[k];
    }
    for (int64_t k = 0; k < K; ++k) bad += hGA[m * K + k] != (float)row[k];
  }
  free(row);
  for (int64_t n = 0; n < N; ++n) {
    int64_t s = 0;
    for (int64_t m = 0; m < M; ++m) s += (int64_t)hG[m * N + n];
    bad += hGB[n] != (float)s;
  }
  if (bad) { fprintf(stderr, "backward differs from the integer product (%lld)\n", (long long)bad); return 1; }

  HIP_OK(hipFree(dA)); HIP_OK(hipFree(dW)); HIP_OK(hipFree(dG)); HIP_OK(hipFree(dOut)); HIP_OK(hipFree(dOut2));
  HIP_OK(hipFree(dC32)); HIP_OK(hipFree(dGA)); HIP_OK(hipFree(dGB)); HIP_OK(hipFree(dCB)); HIP_OK(hipFree(dSCB)); HIP_OK(hipFree(dCnt));
  HIP_OK(hipFree(dQws)); HIP_OK(hipFree(dFws)); HIP_OK(hipFree(dBws));
  free(iA); free(iW); free(hA); free(hW); free(hG); free(hOut); free(hOut2); free(hC32); free(hGA); free(hGB); free(hCB); free(hSCB);
  return 0;
}

int main(void) {
  /* ragged shapes on the generic kernels and on the 256-row tile kernels */
  static const int64_t shapes[][3] = {{300, 520, 260}, {2100, 1032, 2056}};
  for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i)
    if (run(shapes[i][0], shapes[i][1], shapes[i][2]) != 0) return 1;
  printf("c abi ok\n");
  return 0;
}
