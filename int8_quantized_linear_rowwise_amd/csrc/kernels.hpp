// Internal launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8l {

// Quantizer: X (rows x cols, dtype dt) -> codes, scale, outlier list (first
// idx_cap entries; idx_cap < 0 means cap), count, sub (rows x cap fp16: the
// values of the first cap outlier columns). scratch: quant_scratch_words()
// 32-bit words.
// preflags: column flag words ([slabs][words], the layout of the scratch)
// handed over by the producer of X; the flags pass is then skipped.
//
// Columns of the weight's dequantized outlier slice kept for a staging width
// cap: a multiple of 8 (16-byte rows), at most 256.
inline int wsub_width(int cap) {
  if (cap <= 0) return 0;
  const int w = (cap + 7) & ~7;
  return w < 256 ? w : 256;
}
// With ow (forward only), the row pass also writes ow->wsub[n * wcap + j] =
// fp16(CB[n, O[j]] * (SCB[n] * (1/127))) for n < N, j < min(|O|, wcap): the
// dequantized weight values of the outlier columns (cols = the weight's K).
struct OutlierWeights {
  const int8_t* CB;
  const float* SCB;
  int N, K;
  uint16_t* wsub;
  int wcap;
};
size_t quant_scratch_words(int64_t rows, int64_t cols);
hipError_t launch_quantize(int dt, const void* X, int64_t rows, int cols, float tau, int8_t* codes, float* scale,
                           int32_t* idx, int32_t* count, uint16_t* sub, int cap, uint32_t* scratch,
                           hipStream_t st, const uint32_t* preflags = nullptr, int idx_cap = -1,
                           const OutlierWeights* ow = nullptr);

// Producer of a quantizer input: A = D(SiLU(H)) and A's column flag words
// (quant_scratch_words(rows, cols) words) for tau.
hipError_t launch_silu_flags(int dt, const void* H, int64_t rows, int cols, float tau, void* A, uint32_t* flags,
                             hipStream_t st);

// Forward GEMM with fused epilogue: out = D(CA.CB^T * SCA SCB / 127^2
// + A16[:, idx] . Wdq[:, idx]^T + bias); optional int32 export of CA.CB^T.
// The outlier values of the first cap columns come from subA (M x cap fp16),
// those of later columns straight from A (M x K of dt, fp16 cast on the fly);
// the weight values of the first wcap (wsub_width) columns from wsub (N x
// wcap fp16), later ones rebuilt from CB; idx holds all *count columns.
hipError_t launch_gemm_fwd(int dt, const int8_t* CA, const float* SCA, int M, const int8_t* CB, const float* SCB,
                           int N, int K, const uint16_t* subA, int cap, const uint16_t* wsub, int wcap,
                           const void* A, const int32_t* idx, const int32_t* count, const void* bias, void* out,
                           int32_t* c32, hipStream_t st);

// Kernel chosen for a forward / backward GEMM of this shape (operands 16-byte
// aligned): 0 none (empty output), 1 the generic 128 x 128 kernel, 2 the
// large 256 x 256 tile kernel, 3 the large kernel with 256 x 128 tiles.
int gemm_fwd_plan(int dt, int64_t M, int64_t N, int64_t K, bool aligned);
int gemm_bwd_plan(int dt, int64_t M, int64_t N, int64_t K, bool aligned);

// Backward-input GEMM: grad_A = D(fp16(G) . Wdq), Wdq built from CB on the fly.
hipError_t launch_gemm_bwd(int dt, const void* G, int M, int N, const int8_t* CB, const float* SCB, int K,
                           void* grad_A, hipStream_t st);

// Weight gradient of the trainable-weight mode: grad_W = D(fp16(G)^T . fp16(A)).
hipError_t launch_gemm_wgrad(int dt, const void* G, const void* A, int M, int N, int K, void* grad_W,
                             hipStream_t st);

// grad_bias[n] = D(sum_m G[m, n]) (fp32 accumulation, fixed order).
size_t grad_bias_partial_floats(int M, int N);
hipError_t launch_grad_bias(int dt, const void* G, int M, int N, float* partial, void* grad_bias, hipStream_t st);

}  // namespace i8l
