// Measurement kernels for the roofline constants of one MI355X (gfx950):
// matrix-core throughput per MFMA instruction with nothing else in the loop,
// the shader clock the chip holds meanwhile, and HBM read / copy bandwidth.
// Built into libi8lpeaks.so, used only by the benchmark's --peaks mode; the
// layer itself never calls it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int CHAINS = 8;   // independent accumulators per wave

// kind: 0 v_mfma_i32_32x32x32_i8, 1 v_mfma_f32_32x32x16_f16 (the two
// instructions of the layer's GEMMs)
template <int KIND>
__global__ __launch_bounds__(256) void k_mfma_loop(int iters, float* __restrict__ sink,
                                                   uint64_t* __restrict__ clk) {
  const int t = threadIdx.x;
  uint64_t c0 = 0, r0 = 0;
  if (t == 0) {
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  float s = 0.0f;
  if constexpr (KIND == 0) {
    constexpr int R = 16;
    typedef int vacc __attribute__((ext_vector_type(R)));
    const v4i a = {t, t + 1, t + 2, t + 3}, b = {3 * t, t ^ 5, t + 7, t * 11};
    vacc acc[CHAINS];
#pragma unroll
    for (int j = 0; j < CHAINS; ++j) acc[j] = vacc{} + j;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < CHAINS; ++j) {
        acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[j], 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < CHAINS; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) s += (float)acc[j][r];
  } else {
    constexpr int R = 16;
    typedef float vacc __attribute__((ext_vector_type(R)));
    v8h a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (_Float16)(float)((t + e) & 7);
      b[e] = (_Float16)(float)((t * 3 + e) & 7);
    }
    vacc acc[CHAINS];
#pragma unroll
    for (int j = 0; j < CHAINS; ++j) acc[j] = vacc{} + (float)j;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < CHAINS; ++j) {
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < CHAINS; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) s += acc[j][r];
  }
  sink[blockIdx.x * 256 + t] = s;
  if (t == 0) {
    clk[4 * blockIdx.x + 0] = c0;
    clk[4 * blockIdx.x + 1] = __builtin_amdgcn_s_memtime();
    clk[4 * blockIdx.x + 2] = r0;
    clk[4 * blockIdx.x + 3] = __builtin_amdgcn_s_memrealtime();
  }
}

// every 16-byte chunk of src read once (sum kept so the loads stay); four
// independent chunks per thread and step keep several loads in flight
constexpr int UNR = 4;
__global__ __launch_bounds__(256) void k_read(const v4u* __restrict__ src, int64_t n16, unsigned* __restrict__ sink) {
  unsigned acc = 0u;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (UNR - 1) * stride < n16; i += UNR * stride) {
    v4u v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < UNR; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const v4u v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;   // practically never: keeps the loads live
}

__global__ __launch_bounds__(256) void k_copy(const v4u* __restrict__ src, v4u* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (UNR - 1) * stride < n16; i += UNR * stride) {
    v4u v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < UNR; ++u) dst[i + u * stride] = v[u];
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

// Launch `blocks` workgroups of 256 threads (four waves, one per SIMD; two
// such workgroups per compute unit give two waves per SIMD), each wave
// issuing iters x 8 independent MFMAs of the chosen kind. sink: blocks * 256
// floats; clk: blocks * 4 uint64 (shader-clock and 100 MHz reference-clock
// stamps of each workgroup's start and end). Returns a hipError_t value.
int i8l_peak_mfma(int kind, int blocks, int iters, float* sink, uint64_t* clk, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  switch (kind) {
    case 0: hipLaunchKernelGGL(k_mfma_loop<0>, dim3(blocks), dim3(256), 0, st, iters, sink, clk); break;
    case 1: hipLaunchKernelGGL(k_mfma_loop<1>, dim3(blocks), dim3(256), 0, st, iters, sink, clk); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// MACs of one instruction of each kind
long long i8l_peak_mfma_macs(int kind) {
  switch (kind) {
    case 0: return 32LL * 32 * 32;
    case 1: return 32LL * 32 * 16;
    default: return 0;
  }
}

// bytes: a multiple of 16; src / dst 16-byte aligned device buffers
int i8l_peak_read(const void* src, long long bytes, unsigned* sink, int blocks, void* stream) {
  hipLaunchKernelGGL(k_read, dim3(blocks), dim3(256), 0, (hipStream_t)stream, static_cast<const v4u*>(src),
                     (int64_t)(bytes / 16), sink);
  return (int)hipGetLastError();
}

int i8l_peak_copy(const void* src, void* dst, long long bytes, int blocks, void* stream) {
  hipLaunchKernelGGL(k_copy, dim3(blocks), dim3(256), 0, (hipStream_t)stream, static_cast<const v4u*>(src),
                     static_cast<v4u*>(dst), (int64_t)(bytes / 16));
  return (int)hipGetLastError();
}

}  // extern "C"
