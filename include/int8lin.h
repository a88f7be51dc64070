/*
 * int8lin.h — C ABI of an LLM.int8-style row-wise quantized linear layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The operations follow bitsandbytes PR #33 "Memory efficient backward"
 * (public pull request page):
 *   - PR description: int8 weights kept row-major; forward on int8; backward
 *     turns the int8 weights into fp16 weights on the fly and multiplies them
 *     with the fp16 output gradient, never storing fp16 weights; inputs are
 *     cast to fp16 and outputs back to the input dtype.
 *   - review "Cast A to fp16" and commit "cast to half before double_quant":
 *     the quantizer sees the fp16 cast of the activation.
 *   - review on the bias add and "4. Mixed-precision decomposition matmul":
 *     dequantized int8 product + bias + fp16 product of the outlier columns.
 *   - author notes: grad_bias from the un-cast gradient; frozen weight (no
 *     weight gradient).
 *   - review on the backward dequantization: CB * (SCB * (1/127)).
 *   - the has_fp16_weights option beside the memory-efficient one (a trainable
 *     weight re-quantized on each forward): int8_linear_backward_weight.
 * and EasyDeL discussion #66 ("Run and find Out": fwd_bits=8, bwd_bits=8), an
 * 8-bit backward dot product: int8_linear_backward_input_int8.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller (the library
 *     never allocates, frees or synchronises, except int8_linear_forward_check
 *     which synchronises by definition). Every call only enqueues work on
 *     `stream` (a hipStream_t passed as void*; NULL = the default stream).
 *   - Tensors are dense and row-major (last dimension contiguous); leading
 *     batch dimensions are flattened into the row count by the caller.
 *   - dtype: I8L_F32, I8L_F16 or I8L_BF16 (bf16 passed as raw 16-bit words).
 *     fp16 casts and narrowing casts round to nearest even.
 *   - Workspaces are caller-owned device buffers of at least the size the
 *     matching *_workspace_bytes() function returns, 256-byte aligned. Their
 *     contents need no initialisation and are overwritten by each call.
 *   - Return value: I8L_OK (0) or a negative error code. Argument errors are
 *     detected on the host BEFORE any HIP call (nothing is enqueued); launch
 *     errors are reported as I8L_EHIP. Faults inside kernels surface, as in
 *     HIP, at the caller's next synchronisation.
 *   - Calls are stateless and reentrant; results are bitwise deterministic.
 *   - Graph capture: every call except int8_linear_forward_check enqueues
 *     kernels only (no allocation, memset or synchronisation), so it can be
 *     recorded by HIP stream capture and replayed; the pointers are captured,
 *     so a replay reads whatever the buffers hold then. The first call of a
 *     kernel family on a device raises that kernel's LDS limit
 *     (hipFuncSetAttribute); make one ordinary call before capturing.
 *   - Outlier threshold tau: a feature column is an outlier column when any
 *     row of the (flattened) input has |fp16(x)| > tau (strict, compared in
 *     fp32). tau <= 0, tau = +inf or NaN disables the split.
 */
#ifndef INT8LIN_H
#define INT8LIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { I8L_F32 = 0, I8L_F16 = 1, I8L_BF16 = 2 } i8l_dtype;

enum {
  I8L_OK = 0,
  I8L_EINVAL = -1,     /* NULL pointer, negative size, misaligned workspace */
  I8L_EDTYPE = -2,     /* dtype not one of i8l_dtype */
  I8L_ESHAPE = -3,     /* size beyond what the kernels index, or K > I8L_MAX_K */
  I8L_EWORKSPACE = -4, /* workspace NULL or smaller than required */
  I8L_EHIP = -5,       /* a HIP launch or copy failed */
  I8L_EOVERFLOW = -6,  /* reserved: no call returns it (the forward handles any number of
                          outlier columns; int8_quantize_rowwise reports |O| > cap
                          through its count) */
  I8L_ESCRATCH = -7    /* problem larger than the static scratch of the allocation-free
                          forward */
};

/* Largest contraction length whose int32 accumulator cannot overflow:
 * 127 * 127 * K < 2^31. */
#define I8L_MAX_K 133144
/* Widest row int8_quantize_rowwise accepts (column flags kept on chip). */
#define I8L_MAX_COLS 262144

/* Short text for an error code (static storage). */
const char* int8_linear_strerror(int code);

/* ------------------------------------------------------------------------ *
 * Row-wise quantization (bitsandbytes PR #33: "Cast A to fp16" review, commit
 * "cast to half before double_quant"; the 127 scale of the dequantization
 * review). For X (rows x cols):
 *   X16       = fp16(X)
 *   O         = ascending outlier columns of X16 (see tau above)
 *   s[r]      = max over c not in O of |X16[r, c]|        (0 if none)
 *   codes     = clamp(rint(fl32(X16 * fl32(127 / s[r]))), -127, 127), 0 on O
 *               and on rows with s[r] = 0; -128 is never produced
 *   sub[r, j] = X16[r, O[j]] for j < min(|O|, cap)
 * Outputs (device): codes rows x cols int8; row_scale rows fp32 (s, exact);
 * outlier_idx cap int32 (first min(|O|, cap) entries written);
 * outlier_count 1 int32 (= |O|, may exceed cap: overflow is then visible);
 * sub rows x cap fp16 bits (leading dimension cap; only columns j < |O| are
 * written). outlier_idx / sub may be NULL when cap = 0.
 * cols <= I8L_MAX_COLS, else I8L_ESHAPE.
 * Weights are quantized with this call and tau off: CB = codes, SCB = s.
 * ------------------------------------------------------------------------ */
size_t int8_quantize_rowwise_workspace_bytes(int64_t rows, int64_t cols);

int int8_quantize_rowwise(const void* X, int dtype, int64_t rows, int64_t cols, float threshold,
                          int8_t* codes, float* row_scale, int32_t* outlier_idx, int32_t* outlier_count,
                          uint16_t* sub, int32_t cap, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ------------------------------------------------------------------------ *
 * Forward (bitsandbytes PR #33, review on the bias add and
 * "4. Mixed-precision decomposition matmul"):
 *   (CA, SCA, O, subA) = quantize(A, tau)                      (as above)
 *   C32[m, n] = sum_k CA[m, k] * CB[n, k]                      (exact int32)
 *   Wdq[n, k] = fp16(fl32(CB[n, k] * fl32(SCB[n] * fl32(1/127))))
 *   out[m, n] = D(C32 * SCA[m] * SCB[n] / 127^2 + sum_j subA[m, j] * Wdq[n, O[j]]
 *                 + bias[n])                                    (fp32 accumulate)
 * A: M x K of `dtype`; CB: N x K int8 row-major; SCB: N fp32; bias: N of
 * `dtype` or NULL; out: M x N of `dtype`; c32_debug: M x N int32 or NULL
 * (exports C32). K <= I8L_MAX_K.
 * cap (>= 0): columns of the workspace's fp16 outlier sub-matrix subA. The
 * values of the first cap outlier columns are staged there by the quantizer;
 * the epilogue reads those of any further outlier column from A itself (the
 * same fp16 cast), so every |O| <= K is handled and the output is complete
 * for any cap. The row pass also writes the dequantized weight values of
 * the first wcap outlier columns, wcap = cap rounded up to a multiple of 8
 * and at most 256 (N x wcap fp16: the weight side of the outlier product,
 * rebuilt from CB on every call), so that the epilogue reads both operands
 * of that product as contiguous rows; the weight values of further columns
 * are rebuilt from CB by the epilogue. A small cap (a few times the expected
 * |O|) keeps the workspace at about M*K + 2*(M + N)*cap bytes.
 * The workspace holds the quantized activation (CA, SCA), the full outlier
 * list (K entries), subA, the weight slice and the quantizer's flag words;
 * its layout is
 * reported by int8_linear_forward_workspace_layout so that tests can read it
 * back. A must stay unchanged until the call has run (it is read twice by the
 * quantizer and again by the epilogue).
 * ------------------------------------------------------------------------ */
typedef struct {
  size_t count;   /* int32 |O| */
  size_t idx;     /* int32[K] outlier columns, ascending (first |O| valid) */
  size_t scale;   /* fp32[M] SCA */
  size_t codes;   /* int8[M*K] CA */
  size_t sub;     /* fp16[M*cap] subA: A16[:, O[j]] for j < min(|O|, cap) */
  size_t wsub;    /* fp16[N*wcap] (wcap above): Wdq[n, O[j]] for j < min(|O|, wcap) */
  size_t total;   /* bytes required */
} i8l_forward_layout;

size_t int8_linear_forward_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t cap);
int int8_linear_forward_workspace_layout(int64_t M, int64_t K, int64_t N, int32_t cap, i8l_forward_layout* layout);

int int8_linear_forward(const void* A, int dtype, int64_t M, int64_t K, const int8_t* CB, const float* SCB,
                        int64_t N, const void* bias, float threshold, int32_t cap, void* out, int32_t* c32_debug,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): int8_linear_forward with the same inputs, outputs, arithmetic
 * and errors, but its workspace is a static array inside the library
 * (I8L_NOALLOC_SCRATCH_BYTES = 64 MiB per GPU, reserved on each GPU the
 * library runs on until the process ends) and the outlier staging width is
 * min(K, 64) (further outlier columns are read from A, as in the forward).
 * The call allocates nothing and calls no allocating routine.
 *   int8_linear_forward_noalloc_bytes(M, K, N): scratch bytes a call needs
 *     (the forward workspace at that staging width);
 *   int8_linear_forward_noalloc_max_bytes(): the limit, I8L_NOALLOC_SCRATCH_BYTES.
 * A problem needing more (about M*K + 128*(M + N) bytes above 64 MiB) is
 * rejected with I8L_ESCRATCH on the host, before any HIP call. The first call
 * on a GPU looks up that GPU's copy of the array (the current device must be
 * the stream's). Every call on one GPU shares that copy: calls that overlap
 * on one GPU (different streams, or different host threads without
 * ordering) race and give wrong results; calls in one stream are ordered and
 * safe. Nothing in the array needs to start at zero.
 * ------------------------------------------------------------------------ */
#define I8L_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

size_t int8_linear_forward_noalloc_bytes(int64_t M, int64_t K, int64_t N);
size_t int8_linear_forward_noalloc_max_bytes(void);

int int8_linear_forward_noalloc(const void* A, int dtype, int64_t M, int64_t K, const int8_t* CB, const float* SCB,
                                int64_t N, const void* bias, float threshold, void* out, void* stream);

/* ------------------------------------------------------------------------ *
 * Outlier flags handed over by the producer of the input (EasyDeL discussion
 * #66, "Run and find Out": Dense -> SiLU -> Dense). The outlier columns of a
 * layer input are a property of all its rows, so the quantizer normally reads
 * the input once to flag them and once to quantize. When the input is made
 * by the activation kernel below, that kernel flags the columns as it writes
 * them and the flagged forward skips the flagging read.
 *
 * int8_outlier_flags_words(rows, cols): size of the flag buffer in uint32
 * words for an input of rows x cols (row slabs x ceil(cols / 32) words).
 *
 * int8_silu_outlier_flags: A = D(SiLU(H)) elementwise, SiLU(x) = x / (1 +
 * exp(-x)) evaluated in fp32 (within four fp32 units in the last place) and
 * rounded once to `dtype`; flags = the
 * outlier-column flags of A for `threshold` (a column is flagged when any row
 * has |fp16(A)| > threshold; threshold <= 0, +inf or NaN flags nothing).
 * H, A: rows x cols of `dtype` (A may not overlap H); flags: the caller's
 * buffer of flag_words >= int8_outlier_flags_words(rows, cols) words, fully
 * overwritten (I8L_EWORKSPACE when smaller).
 *
 * int8_linear_forward_flagged: int8_linear_forward with the outlier columns
 * given by `flags` (from int8_silu_outlier_flags on the same rows x K shape;
 * the threshold is the one the flags were made with) instead of found by a
 * pass over A. Same workspace, outputs and errors as int8_linear_forward;
 * flags NULL (with M, K > 0) is I8L_EINVAL, flag_words below
 * int8_outlier_flags_words(M, K) is I8L_EWORKSPACE.
 * ------------------------------------------------------------------------ */
size_t int8_outlier_flags_words(int64_t rows, int64_t cols);

int int8_silu_outlier_flags(const void* H, int dtype, int64_t rows, int64_t cols, float threshold, void* A,
                            uint32_t* flags, size_t flag_words, void* stream);

int int8_linear_forward_flagged(const void* A, int dtype, int64_t M, int64_t K, const uint32_t* flags,
                                size_t flag_words, const int8_t* CB, const float* SCB, int64_t N, const void* bias,
                                int32_t cap, void* out, int32_t* c32_debug, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Synchronises `stream` and reads the outlier count |O| of the last forward
 * that used `workspace` (laid out for M, K, N, cap) into *count (if non-NULL).
 * Returns I8L_OK, or I8L_EINVAL / I8L_EHIP. The forward's output is complete
 * for every count, so this call is a diagnostic, not a required check. */
int int8_linear_forward_check(const void* workspace, int64_t M, int64_t K, int64_t N, int32_t cap, void* stream,
                              int32_t* count);

/* Which GEMM kernel a call of this shape launches, for operands with the
 * alignment of device allocations (host only: no HIP call, no device
 * memory). int8_linear_forward_plan(dtype, M, K, N) for the forward product
 * (also the int8 backward's, with K and N exchanged) and
 * int8_linear_backward_plan(dtype, M, N, K) for the input gradient:
 * 0 nothing to compute (empty output), 1 the generic 128 x 128 tile kernel,
 * 2 the large pipelined kernel with 256 x 256 tiles, 3 the large kernel with
 * 256 x 128 tiles (chosen where 256 x 256 tiles would fill at most half of the
 * chip's 256 compute units). Negative: the error the call itself would
 * return for these sizes or dtype. Used by tests to check the dispatch. */
int int8_linear_forward_plan(int dtype, int64_t M, int64_t K, int64_t N);
int int8_linear_backward_plan(int dtype, int64_t M, int64_t N, int64_t K);

/* ------------------------------------------------------------------------ *
 * Memory-efficient backward, input gradient only (bitsandbytes PR #33, PR
 * description, backward-dequantization review, author notes):
 *   grad_A[m, k]  = D(sum_n fp16(G[m, n]) * Wdq[n, k])   (fp32 accumulate)
 *   grad_bias[n]  = D(sum_m G[m, n])   on the un-cast G    (fp32 accumulate)
 * G: M x N of `dtype`; CB: N x K int8 row-major; SCB: N fp32; grad_A: M x K
 * of `dtype`; grad_bias: N of `dtype` or NULL (then no workspace is needed).
 * No weight gradient exists: the int8 weight is frozen.
 * ------------------------------------------------------------------------ */
size_t int8_linear_backward_workspace_bytes(int64_t M, int64_t N, int with_grad_bias);

int int8_linear_backward_input(const void* G, int dtype, int64_t M, int64_t N, const int8_t* CB, const float* SCB,
                               int64_t K, void* grad_A, void* grad_bias, void* workspace, size_t workspace_bytes,
                               void* stream);

/* ------------------------------------------------------------------------ *
 * int8 backward variant (EasyDeL discussion #66, "Run and find Out": a Dense
 * layer with fwd_bits=8, bwd_bits=8 computes its backward dot product in 8
 * bits). Not the memory-efficient backward above: here both operands of the
 * input-gradient product are int8, with scales constant along the
 * contraction N:
 *   (CG, SG)     = quantize(G, tau off)                    (row-wise, per token)
 *   C32[m, k]    = sum_n CG[m, n] * CBt[k, n]              (exact int32)
 *   grad_A[m, k] = D(C32 * SG[m] * SCBt[k] / 127^2)        (fp32 arithmetic)
 *   grad_bias[n] = D(sum_m G[m, n])   on the un-cast G       (fp32 accumulate)
 * CBt / SCBt: a second offline int8 copy of the weight, W^T (K x N, row-major)
 * quantized with int8_quantize_rowwise and tau off (one scale per input
 * feature k). G: M x N of `dtype`; grad_A: M x K of `dtype`; grad_bias: N of
 * `dtype` or NULL; c32_debug: M x K int32 or NULL (exports C32).
 * N <= I8L_MAX_K. The workspace holds CG, SG and the quantizer's scratch.
 * ------------------------------------------------------------------------ */
size_t int8_linear_backward_int8_workspace_bytes(int64_t M, int64_t N, int with_grad_bias);

int int8_linear_backward_input_int8(const void* G, int dtype, int64_t M, int64_t N, const int8_t* CBt,
                                    const float* SCBt, int64_t K, void* grad_A, void* grad_bias, int32_t* c32_debug,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Weight gradient of the trainable-weight mode (bitsandbytes PR #33 names a
 * has_fp16_weights option beside the memory-efficient backward; the weight
 * then stays a trainable tensor that is re-quantized on each forward):
 *   grad_W[n, k] = D(sum_m fp16(G[m, n]) * fp16(A[m, k]))   (fp32 accumulate)
 * G: M x N and A: M x K of `dtype` (the output gradient and the layer input,
 * both row-major); grad_W: N x K of `dtype`, row-major (the weight's layout).
 * M = 0 writes zeros. Needs no workspace. Errors: I8L_EDTYPE, I8L_EINVAL
 * (negative size, NULL pointer where data is needed), I8L_ESHAPE (a size
 * beyond INT32_MAX or a product beyond 2^40), I8L_EHIP (launch failure).
 * ------------------------------------------------------------------------ */
int int8_linear_backward_weight(const void* G, const void* A, int dtype, int64_t M, int64_t N, int64_t K,
                                void* grad_W, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* INT8LIN_H */
