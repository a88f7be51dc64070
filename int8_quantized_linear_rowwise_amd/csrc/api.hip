// C-ABI host layer: argument validation (before any HIP call), workspace
// carving and kernel launches on the caller's stream. No allocation, no
// synchronisation (except int8_linear_forward_check).
#include <limits.h>
#include <stdint.h>

#include <mutex>

#include "../../include/int8lin.h"
#include "kernels.hpp"

// Scratch of int8_linear_forward_noalloc: one copy on every GPU the library
// runs on, held until the process ends. Host code never uses this name as an
// address: the device address of each GPU's copy comes from
// hipGetSymbolAddress (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[I8L_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t ALIGN = 256;

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

bool valid_dtype(int dt) { return dt == I8L_F32 || dt == I8L_F16 || dt == I8L_BF16; }

// quantizer scratch: the column flag words of each row slab ([slabs][ceil(cols / 32)])
size_t quant_scratch_bytes(int64_t rows, int64_t cols) { return align_up(i8l::quant_scratch_words(rows, cols) * 4); }

bool fwd_layout(int64_t M, int64_t K, int64_t N, int32_t cap, i8l_forward_layout* L) {
  if (M < 0 || K < 0 || N < 0 || cap < 0) return false;
  size_t off = 0;
  L->count = off;
  off += ALIGN;
  L->idx = off;
  // the outlier list holds every column that can be one: it never overflows
  off += align_up((size_t)(K > 0 ? K : 1) * 4);
  L->scale = off;
  off += align_up((size_t)(M > 0 ? M : 1) * 4);
  L->codes = off;
  off += align_up((size_t)M * (size_t)K > 0 ? (size_t)M * (size_t)K : 1);
  L->sub = off;
  off += align_up((size_t)M * (size_t)cap * 2 > 0 ? (size_t)M * (size_t)cap * 2 : 2);
  // the dequantized weight columns of the first wsub_width(cap) outlier columns
  // (cap rounded up to a multiple of 8, at most 256)
  const size_t wcap = (size_t)i8l::wsub_width(cap);
  L->wsub = off;
  off += align_up((size_t)N * wcap * 2 > 0 ? (size_t)N * wcap * 2 : 2);
  // quantizer scratch after the layout proper
  off += quant_scratch_bytes(M, K);
  L->total = off;
  return true;
}

int hip_status(hipError_t e) { return e == hipSuccess ? I8L_OK : I8L_EHIP; }

// outlier staging width of the allocation-free forward (further outlier
// columns are read from A by the epilogue)
constexpr int32_t NOALLOC_CAP = 64;
constexpr int MAX_DEVICES = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];

// Device address of the current GPU's copy of `scratch`, looked up once per
// device with that device current and kept for later calls.
hipError_t noalloc_scratch(void** p) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (q == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = q;
  }
  *p = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* int8_linear_strerror(int code) {
  switch (code) {
    case I8L_OK: return "ok";
    case I8L_EINVAL: return "invalid argument (NULL pointer, negative size or misaligned workspace)";
    case I8L_EDTYPE: return "unsupported dtype";
    case I8L_ESHAPE: return "unsupported shape (too large, or K above the int32-accumulator limit)";
    case I8L_EWORKSPACE: return "workspace missing or too small";
    case I8L_EHIP: return "HIP launch or copy failed";
    case I8L_EOVERFLOW: return "more outlier columns than the outlier buffer capacity";
    case I8L_ESCRATCH:
      return "problem too large for the library's static scratch (see int8_linear_forward_noalloc_max_bytes)";
    default: return "unknown error";
  }
}

size_t int8_quantize_rowwise_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return 0;
  return quant_scratch_bytes(rows, cols);
}

int int8_quantize_rowwise(const void* X, int dtype, int64_t rows, int64_t cols, float threshold, int8_t* codes,
                          float* row_scale, int32_t* outlier_idx, int32_t* outlier_count, uint16_t* sub,
                          int32_t cap, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(dtype)) return I8L_EDTYPE;
  if (rows < 0 || cols < 0 || cap < 0) return I8L_EINVAL;
  if (rows > INT32_MAX || cols > I8L_MAX_COLS || rows * cols > ((int64_t)1 << 40)) return I8L_ESHAPE;
  if (outlier_count == nullptr) return I8L_EINVAL;
  if (rows > 0 && (row_scale == nullptr || (cols > 0 && (X == nullptr || codes == nullptr)))) return I8L_EINVAL;
  if (cap > 0 && (outlier_idx == nullptr || (rows > 0 && sub == nullptr))) return I8L_EINVAL;
  const size_t need = quant_scratch_bytes(rows, cols);
  if (ws == nullptr || ws_bytes < need) return I8L_EWORKSPACE;
  if ((uintptr_t)ws % ALIGN) return I8L_EINVAL;
  return hip_status(i8l::launch_quantize(dtype, X, rows, (int)cols, threshold, codes, row_scale, outlier_idx,
                                         outlier_count, sub, cap, static_cast<uint32_t*>(ws), (hipStream_t)stream));
}

size_t int8_linear_forward_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t cap) {
  i8l_forward_layout L;
  if (!fwd_layout(M, K, N, cap, &L)) return 0;
  return L.total;
}

int int8_linear_forward_workspace_layout(int64_t M, int64_t K, int64_t N, int32_t cap, i8l_forward_layout* layout) {
  if (layout == nullptr) return I8L_EINVAL;
  if (!fwd_layout(M, K, N, cap, layout)) return I8L_EINVAL;
  return I8L_OK;
}

static int forward_impl(const void* A, int dtype, int64_t M, int64_t K, const int8_t* CB, const float* SCB,
                        int64_t N, const void* bias, float threshold, const uint32_t* preflags, int32_t cap,
                        void* out, int32_t* c32, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(dtype)) return I8L_EDTYPE;
  if (M < 0 || K < 0 || N < 0 || cap < 0) return I8L_EINVAL;
  if (M > INT32_MAX || N > INT32_MAX || K > I8L_MAX_K || M * K > ((int64_t)1 << 40) ||
      M * N > ((int64_t)1 << 40) || N * K > ((int64_t)1 << 40))
    return I8L_ESHAPE;
  if (M > 0 && N > 0) {
    if (out == nullptr || SCB == nullptr) return I8L_EINVAL;
    if (K > 0 && (A == nullptr || CB == nullptr)) return I8L_EINVAL;
  }
  i8l_forward_layout L;
  fwd_layout(M, K, N, cap, &L);
  if (ws == nullptr || ws_bytes < L.total) return I8L_EWORKSPACE;
  if ((uintptr_t)ws % ALIGN) return I8L_EINVAL;
  if (M == 0 || N == 0) return I8L_OK;
  char* w = static_cast<char*>(ws);
  int32_t* count = reinterpret_cast<int32_t*>(w + L.count);
  int32_t* idx = reinterpret_cast<int32_t*>(w + L.idx);
  float* SCA = reinterpret_cast<float*>(w + L.scale);
  int8_t* CA = reinterpret_cast<int8_t*>(w + L.codes);
  uint16_t* subA = reinterpret_cast<uint16_t*>(w + L.sub);
  uint16_t* wsub = reinterpret_cast<uint16_t*>(w + L.wsub);
  const int wcap = i8l::wsub_width(cap);
  uint32_t* qscratch = reinterpret_cast<uint32_t*>(w + L.total - quant_scratch_bytes(M, K));
  hipStream_t st = (hipStream_t)stream;
  // the first cap outlier columns are staged in subA; the epilogue reads the
  // values of any further ones from A itself
  // the row pass also writes wsub, the weight columns of the outlier columns
  // dequantized (Wdq[n, O[j]], j < wcap), for the epilogue's outlier product
  const i8l::OutlierWeights ow = {CB, SCB, (int)N, (int)K, wsub, wcap};
  hipError_t e = i8l::launch_quantize(dtype, A, M, (int)K, threshold, CA, SCA, idx, count, subA, cap, qscratch, st,
                                      preflags, (int)K, &ow);
  if (e != hipSuccess) return I8L_EHIP;
  e = i8l::launch_gemm_fwd(dtype, CA, SCA, (int)M, CB, SCB, (int)N, (int)K, subA, cap, wsub, wcap, A, idx, count,
                           bias, out, c32, st);
  return hip_status(e);
}

int int8_linear_forward(const void* A, int dtype, int64_t M, int64_t K, const int8_t* CB, const float* SCB,
                        int64_t N, const void* bias, float threshold, int32_t cap, void* out, int32_t* c32,
                        void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(A, dtype, M, K, CB, SCB, N, bias, threshold, nullptr, cap, out, c32, ws, ws_bytes, stream);
}

size_t int8_linear_forward_noalloc_max_bytes(void) { return I8L_NOALLOC_SCRATCH_BYTES; }

size_t int8_linear_forward_noalloc_bytes(int64_t M, int64_t K, int64_t N) {
  i8l_forward_layout L;
  if (M < 0 || K < 0 || N < 0 || !fwd_layout(M, K, N, K < NOALLOC_CAP ? (int32_t)K : NOALLOC_CAP, &L)) return 0;
  return L.total;
}

int int8_linear_forward_noalloc(const void* A, int dtype, int64_t M, int64_t K, const int8_t* CB, const float* SCB,
                                int64_t N, const void* bias, float threshold, void* out, void* stream) {
  // argument errors first, on the host, as in int8_linear_forward
  if (!valid_dtype(dtype)) return I8L_EDTYPE;
  if (M < 0 || K < 0 || N < 0) return I8L_EINVAL;
  if (M > INT32_MAX || N > INT32_MAX || K > I8L_MAX_K || M * K > ((int64_t)1 << 40) ||
      M * N > ((int64_t)1 << 40) || N * K > ((int64_t)1 << 40))
    return I8L_ESHAPE;
  if (M > 0 && N > 0) {
    if (out == nullptr || SCB == nullptr) return I8L_EINVAL;
    if (K > 0 && (A == nullptr || CB == nullptr)) return I8L_EINVAL;
  }
  const int32_t cap = K < NOALLOC_CAP ? (int32_t)K : NOALLOC_CAP;
  i8l_forward_layout L;
  fwd_layout(M, K, N, cap, &L);
  if (L.total > I8L_NOALLOC_SCRATCH_BYTES) return I8L_ESCRATCH;
  if (M == 0 || N == 0) return I8L_OK;
  void* ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess) return I8L_EHIP;
  // no buffer of the call needs to start at zero: the quantizer writes its
  // flag words, list, count, codes and scales before the GEMM reads them
  return forward_impl(A, dtype, M, K, CB, SCB, N, bias, threshold, nullptr, cap, out, nullptr, ws,
                      I8L_NOALLOC_SCRATCH_BYTES, stream);
}

size_t int8_outlier_flags_words(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return 0;
  return i8l::quant_scratch_words(rows, cols);
}

int int8_silu_outlier_flags(const void* H, int dtype, int64_t rows, int64_t cols, float threshold, void* A,
                            uint32_t* flags, size_t flag_words, void* stream) {
  if (!valid_dtype(dtype)) return I8L_EDTYPE;
  if (rows < 0 || cols < 0) return I8L_EINVAL;
  if (rows > INT32_MAX || cols > I8L_MAX_COLS || rows * cols > ((int64_t)1 << 40)) return I8L_ESHAPE;
  if (rows == 0 || cols == 0) return I8L_OK;
  if (H == nullptr || A == nullptr || flags == nullptr) return I8L_EINVAL;
  if (flag_words < i8l::quant_scratch_words(rows, cols)) return I8L_EWORKSPACE;
  return hip_status(i8l::launch_silu_flags(dtype, H, rows, (int)cols, threshold, A, flags, (hipStream_t)stream));
}

int int8_linear_forward_flagged(const void* A, int dtype, int64_t M, int64_t K, const uint32_t* flags,
                                size_t flag_words, const int8_t* CB, const float* SCB, int64_t N, const void* bias,
                                int32_t cap, void* out, int32_t* c32_debug, void* ws, size_t ws_bytes,
                                void* stream) {
  if (M > 0 && K > 0) {
    if (flags == nullptr) return I8L_EINVAL;
    if (M <= INT32_MAX && K <= I8L_MAX_K && flag_words < i8l::quant_scratch_words(M, K)) return I8L_EWORKSPACE;
  }
  return forward_impl(A, dtype, M, K, CB, SCB, N, bias, 0.0f, flags, cap, out, c32_debug, ws, ws_bytes, stream);
}

int int8_linear_forward_check(const void* ws, int64_t M, int64_t K, int64_t N, int32_t cap, void* stream,
                              int32_t* count) {
  i8l_forward_layout L;
  if (ws == nullptr || !fwd_layout(M, K, N, cap, &L)) return I8L_EINVAL;
  int32_t c = 0;
  hipStream_t st = (hipStream_t)stream;
  if (hipMemcpyAsync(&c, static_cast<const char*>(ws) + L.count, sizeof(int32_t), hipMemcpyDeviceToHost, st) !=
      hipSuccess)
    return I8L_EHIP;
  if (hipStreamSynchronize(st) != hipSuccess) return I8L_EHIP;
  if (count) *count = c;
  return I8L_OK;
}

int int8_linear_forward_plan(int dtype, int64_t M, int64_t K, int64_t N) {
  if (!valid_dtype(dtype)) return I8L_EDTYPE;
  if (M < 0 || K < 0 || N < 0) return I8L_EINVAL;
  if (M > INT32_MAX || N > INT32_MAX || K > I8L_MAX_K) return I8L_ESHAPE;
  return i8l::gemm_fwd_plan(dtype, M, N, K, true);
}

int int8_linear_backward_plan(int dtype, int64_t M, int64_t N, int64_t K) {
  if (!valid_dtype(dtype)) return I8L_EDTYPE;
  if (M < 0 || K < 0 || N < 0) return I8L_EINVAL;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return I8L_ESHAPE;
  return i8l::gemm_bwd_plan(dtype, M, N, K, true);
}

size_t int8_linear_backward_workspace_bytes(int64_t M, int64_t N, int with_grad_bias) {
  if (M < 0 || N < 0 || M > INT32_MAX || N > INT32_MAX) return 0;
  if (!with_grad_bias) return 0;
  return align_up(i8l::grad_bias_partial_floats((int)M, (int)N) * sizeof(float));
}

int int8_linear_backward_input(const void* G, int dtype, int64_t M, int64_t N, const int8_t* CB, const float* SCB,
                               int64_t K, void* grad_A, void* grad_bias, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(dtype)) return I8L_EDTYPE;
  if (M < 0 || N < 0 || K < 0) return I8L_EINVAL;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX || M * K > ((int64_t)1 << 40) ||
      M * N > ((int64_t)1 << 40) || N * K > ((int64_t)1 << 40))
    return I8L_ESHAPE;
  if (M > 0 && K > 0) {
    if (grad_A == nullptr) return I8L_EINVAL;
    if (N > 0 && (G == nullptr || CB == nullptr || SCB == nullptr)) return I8L_EINVAL;
  }
  if (grad_bias != nullptr) {
    if (M > 0 && N > 0 && G == nullptr) return I8L_EINVAL;
    const size_t need = int8_linear_backward_workspace_bytes(M, N, 1);
    if (ws == nullptr || ws_bytes < need) return I8L_EWORKSPACE;
    if ((uintptr_t)ws % ALIGN) return I8L_EINVAL;
  }
  hipStream_t st = (hipStream_t)stream;
  if (M > 0 && K > 0) {
    hipError_t e = i8l::launch_gemm_bwd(dtype, G, (int)M, (int)N, CB, SCB, (int)K, grad_A, st);
    if (e != hipSuccess) return I8L_EHIP;
  }
  if (grad_bias != nullptr && N > 0) {
    hipError_t e = i8l::launch_grad_bias(dtype, G, (int)M, (int)N, static_cast<float*>(ws), grad_bias, st);
    if (e != hipSuccess) return I8L_EHIP;
  }
  return I8L_OK;
}

// int8 backward workspace: count | SG (M fp32) | CG (M x N int8) | quantizer
// scratch | grad_bias partial sums (when requested); 256-byte aligned blocks.
struct Bwd8Layout {
  size_t count, sg, cg, qs, gb, total;
};

static bool bwd8_layout(int64_t M, int64_t N, int with_grad_bias, Bwd8Layout* L) {
  if (M < 0 || N < 0 || M > INT32_MAX || N > INT32_MAX) return false;
  size_t off = 0;
  L->count = off;
  off += ALIGN;
  L->sg = off;
  off += align_up((size_t)(M > 0 ? M : 1) * 4);
  L->cg = off;
  off += align_up((size_t)M * (size_t)N > 0 ? (size_t)M * (size_t)N : 1);
  L->qs = off;
  off += quant_scratch_bytes(M, N);
  L->gb = off;
  if (with_grad_bias) off += align_up(i8l::grad_bias_partial_floats((int)M, (int)N) * sizeof(float));
  L->total = off;
  return true;
}

size_t int8_linear_backward_int8_workspace_bytes(int64_t M, int64_t N, int with_grad_bias) {
  Bwd8Layout L;
  if (!bwd8_layout(M, N, with_grad_bias, &L)) return 0;
  return L.total;
}

int int8_linear_backward_input_int8(const void* G, int dtype, int64_t M, int64_t N, const int8_t* CBt,
                                    const float* SCBt, int64_t K, void* grad_A, void* grad_bias, int32_t* c32_debug,
                                    void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(dtype)) return I8L_EDTYPE;
  if (M < 0 || N < 0 || K < 0) return I8L_EINVAL;
  if (M > INT32_MAX || K > INT32_MAX || N > I8L_MAX_K || N > I8L_MAX_COLS || M * K > ((int64_t)1 << 40) ||
      M * N > ((int64_t)1 << 40) || N * K > ((int64_t)1 << 40))
    return I8L_ESHAPE;
  if (M > 0 && K > 0) {
    if (grad_A == nullptr || SCBt == nullptr) return I8L_EINVAL;
    if (N > 0 && (G == nullptr || CBt == nullptr)) return I8L_EINVAL;
  }
  if (grad_bias != nullptr && M > 0 && N > 0 && G == nullptr) return I8L_EINVAL;
  Bwd8Layout L;
  bwd8_layout(M, N, grad_bias != nullptr, &L);
  if (ws == nullptr || ws_bytes < L.total) return I8L_EWORKSPACE;
  if ((uintptr_t)ws % ALIGN) return I8L_EINVAL;
  char* w = static_cast<char*>(ws);
  hipStream_t st = (hipStream_t)stream;
  if (M > 0 && K > 0) {
    int32_t* count = reinterpret_cast<int32_t*>(w + L.count);
    float* SG = reinterpret_cast<float*>(w + L.sg);
    int8_t* CG = reinterpret_cast<int8_t*>(w + L.cg);
    uint32_t* qscratch = reinterpret_cast<uint32_t*>(w + L.qs);
    // G row-wise with the split off (count 0), then the int8 product with the
    // column-quantized weight copy: the forward kernel with K and N exchanged
    hipError_t e = i8l::launch_quantize(dtype, G, M, (int)N, 0.0f, CG, SG, nullptr, count, nullptr, 0, qscratch, st);
    if (e != hipSuccess) return I8L_EHIP;
    e = i8l::launch_gemm_fwd(dtype, CG, SG, (int)M, CBt, SCBt, (int)K, (int)N, nullptr, 0, nullptr, 0, nullptr,
                             nullptr, count, nullptr, grad_A, c32_debug, st);
    if (e != hipSuccess) return I8L_EHIP;
  }
  if (grad_bias != nullptr && N > 0) {
    hipError_t e =
        i8l::launch_grad_bias(dtype, G, (int)M, (int)N, reinterpret_cast<float*>(w + L.gb), grad_bias, st);
    if (e != hipSuccess) return I8L_EHIP;
  }
  return I8L_OK;
}

int int8_linear_backward_weight(const void* G, const void* A, int dtype, int64_t M, int64_t N, int64_t K,
                                void* grad_W, void* stream) {
  if (!valid_dtype(dtype)) return I8L_EDTYPE;
  if (M < 0 || N < 0 || K < 0) return I8L_EINVAL;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX || M * K > ((int64_t)1 << 40) ||
      M * N > ((int64_t)1 << 40) || N * K > ((int64_t)1 << 40))
    return I8L_ESHAPE;
  if (N == 0 || K == 0) return I8L_OK;
  if (grad_W == nullptr) return I8L_EINVAL;
  if (M > 0 && (G == nullptr || A == nullptr)) return I8L_EINVAL;
  return hip_status(i8l::launch_gemm_wgrad(dtype, G, A, (int)M, (int)N, (int)K, grad_W, (hipStream_t)stream));
}

}  // extern "C"
