// Row-wise int8 quantizer with outlier-column split (LLM.int8 style).
//
// bitsandbytes PR #33 "Memory efficient backward" (review "Cast A to fp16",
// commit "cast to half before double_quant"): the activation is cast to fp16
// before quantization; feature columns holding a value whose magnitude
// exceeds the threshold leave the int8 path ("4. Mixed-precision
// decomposition matmul") and are kept as a dense fp16 sub-matrix.
//
// Three kernels, all on the caller's stream:
//   k_zero_words       clears the column bitmask (no memset node, so the
//                      sequence can be captured in a graph);
//   k_outlier_flags    one read of X: per column, the largest magnitude over
//                      a slab of rows, kept in the storage format's own bits
//                      (magnitude bits order like the values), then one fp16
//                      cast + compare per column; set bits are OR-ed into the
//                      bitmask (only for flagged columns, which are rare);
//   k_outlier_compact  one workgroup: per-word exclusive popcount prefix,
//                      ascending outlier index list, count;
//   k_rowquant         second read of X: per row, absmax over non-outlier
//                      columns, inv = 127 / s (IEEE division), codes =
//                      clamp(rint(x * inv), +-127), 0 on outlier columns,
//                      outlier values copied into the dense fp16 sub-matrix.
#include "common.hpp"
#include "kernels.hpp"

namespace i8l {

__global__ void k_zero_words(uint32_t* __restrict__ p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Magnitude bits of 8 consecutive elements, kept in the storage format.
template <int DT> struct MagAcc;

template <> struct MagAcc<DT_F32> {
  uint32_t m[8];
  __device__ void reset() {
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = 0u;
  }
  __device__ void add_vec(const float* p) {
    v4u a = *reinterpret_cast<const v4u*>(p);
    v4u b = *reinterpret_cast<const v4u*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m[e] = max(m[e], a[e] & 0x7fffffffu);
      m[e + 4] = max(m[e + 4], b[e] & 0x7fffffffu);
    }
  }
  __device__ void add_one(const float* p, int e) { m[e] = max(m[e], __float_as_uint(*p) & 0x7fffffffu); }
  __device__ float half_mag(int e) const { return (float)(_Float16)__uint_as_float(m[e]); }
};

template <int DT> struct MagAcc16 {
  uint32_t m[4];  // two 16-bit magnitudes per word
  __device__ void reset() {
#pragma unroll
    for (int e = 0; e < 4; ++e) m[e] = 0u;
  }
  __device__ void add_vec(const void* p) {
    v4u a = *reinterpret_cast<const v4u*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t w = a[e] & 0x7fff7fffu;
      uint32_t lo = max(m[e] & 0xffffu, w & 0xffffu);
      uint32_t hi = max(m[e] >> 16, w >> 16);
      m[e] = lo | (hi << 16);
    }
  }
  __device__ void add_one(const void* p, int e) {
    uint32_t w = (uint32_t)(*reinterpret_cast<const uint16_t*>(p)) & 0x7fffu;
    uint32_t cur = (e & 1) ? (m[e >> 1] >> 16) : (m[e >> 1] & 0xffffu);
    uint32_t nv = max(cur, w);
    m[e >> 1] = (e & 1) ? ((m[e >> 1] & 0xffffu) | (nv << 16)) : ((m[e >> 1] & 0xffff0000u) | nv);
  }
  __device__ float half_mag(int e) const {
    uint16_t b = (uint16_t)((e & 1) ? (m[e >> 1] >> 16) : (m[e >> 1] & 0xffffu));
    if constexpr (DT == DT_F16) return (float)__builtin_bit_cast(_Float16, b);
    else return (float)(_Float16)bf16_to_f32(b);
  }
};
template <> struct MagAcc<DT_F16> : MagAcc16<DT_F16> {};
template <> struct MagAcc<DT_BF16> : MagAcc16<DT_BF16> {};

// grid: x over column groups of 2048 (256 threads x 8 columns), y over row slabs.
template <int DT>
__global__ __launch_bounds__(256) void k_outlier_flags(const typename Elem<DT>::T* __restrict__ X,
                                                       int64_t rows, int cols, float tau,
                                                       int rows_per_slab, int vec,
                                                       uint32_t* __restrict__ mask) {
  typedef typename Elem<DT>::T T;
  const int c0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (c0 >= cols) return;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_slab;
  int64_t r1 = r0 + rows_per_slab;
  if (r1 > rows) r1 = rows;
  MagAcc<DT> acc;
  acc.reset();
  const bool full = vec && (c0 + 8 <= cols);
  if (full) {
    const T* p = X + r0 * (int64_t)cols + c0;
    int64_t r = r0;
    for (; r + 4 <= r1; r += 4, p += 4 * (int64_t)cols) {
      acc.add_vec(p);
      acc.add_vec(p + cols);
      acc.add_vec(p + 2 * (int64_t)cols);
      acc.add_vec(p + 3 * (int64_t)cols);
    }
    for (; r < r1; ++r, p += cols) acc.add_vec(p);
  } else {
    for (int64_t r = r0; r < r1; ++r) {
      const T* p = X + r * (int64_t)cols + c0;
      for (int e = 0; e < 8; ++e)
        if (c0 + e < cols) acc.add_one(p + e, e);
    }
  }
  uint32_t bits = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (c0 + e < cols && acc.half_mag(e) > tau) bits |= 1u << e;
  if (bits) atomicOr(mask + (c0 >> 5), bits << (c0 & 31));
}

// One workgroup of 1024 threads. nwords <= 8 * 1024.
__global__ __launch_bounds__(1024) void k_outlier_compact(const uint32_t* __restrict__ mask, int nwords,
                                                          int32_t* __restrict__ prefix,
                                                          int32_t* __restrict__ idx, int cap,
                                                          int32_t* __restrict__ count) {
  __shared__ int wsum[16];
  const int t = threadIdx.x;
  const int per = (nwords + 1023) / 1024;
  const int w0 = t * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (w0 + i < nwords) local += __popc(mask[w0 + i]);
  // block exclusive scan of `local`
  const int lane = t & 63, wid = t >> 6;
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < wid; ++i) base += wsum[i];
  int run = base + incl - local;
  for (int i = 0; i < per; ++i) {
    int w = w0 + i;
    if (w >= nwords) break;
    uint32_t m = mask[w];
    prefix[w] = run;
    while (m) {
      int b = __ffs(m) - 1;
      if (run < cap) idx[run] = w * 32 + b;
      ++run;
      m &= m - 1;
    }
  }
  if (t == 1023) {
    int total = 0;
    for (int i = 0; i < 16; ++i) total += wsum[i];
    *count = total;
  }
}

// Row quantization. TPR threads per row (64: one wave, 256: one workgroup),
// each thread holding up to NCH chunks of 8 columns in registers; rows wider
// than TPR * 8 * NCH stream twice through the cache instead.
template <int DT, int TPR, int NCH>
__global__ __launch_bounds__(256) void k_rowquant(const typename Elem<DT>::T* __restrict__ X, int64_t rows,
                                                  int cols, int tau_on, const uint32_t* __restrict__ mask,
                                                  const int32_t* __restrict__ prefix, int vec,
                                                  int8_t* __restrict__ codes, float* __restrict__ scale,
                                                  uint16_t* __restrict__ sub, int cap) {
  typedef typename Elem<DT>::T T;
  __shared__ float red[4];
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const bool live = row < rows;
  const int nchunk = (cols + 7) / 8;
  const bool in_regs = nchunk <= TPR * NCH;
  const T* xr = X + (live ? row : 0) * (int64_t)cols;

  auto load_chunk = [&](int ci, float (&v)[8]) {
    const int c0 = ci * 8;
    if (vec && c0 + 8 <= cols) {
      T raw[8];
      load8<DT>(xr + c0, raw);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = half_cast_f32<DT>(raw[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (c0 + e < cols) ? half_cast_f32<DT>(xr[c0 + e]) : 0.0f;
    }
  };
  auto chunk_mask = [&](int ci) -> uint32_t {
    if (!tau_on) return 0u;
    const int c0 = ci * 8;
    return (mask[c0 >> 5] >> (c0 & 31)) & 0xffu;
  };

  float vals[NCH][8];
  float smax = 0.0f;
  if (live) {
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int ci = i * TPR + tid;
        if (ci < nchunk) load_chunk(ci, vals[i]);
      }
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int ci = i * TPR + tid;
        if (ci < nchunk) {
          uint32_t om = chunk_mask(ci);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (!((om >> e) & 1u)) smax = fmaxf(smax, fabsf(vals[i][e]));
        }
      }
    } else {
      for (int ci = tid; ci < nchunk; ci += TPR) {
        float v[8];
        load_chunk(ci, v);
        uint32_t om = chunk_mask(ci);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (!((om >> e) & 1u)) smax = fmaxf(smax, fabsf(v[e]));
      }
    }
  }
  smax = wave_max(smax);
  if constexpr (TPR == 256) {
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = smax;
    __syncthreads();
    smax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  }
  if (!live) return;
  const float s = smax;
  const float inv = (s > 0.0f) ? (127.0f / s) : 0.0f;

  int8_t* cr = codes + row * (int64_t)cols;
  auto emit = [&](int ci, const float (&v)[8]) {
    const int c0 = ci * 8;
    const uint32_t om = chunk_mask(ci);
    int q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float r = rintf(v[e] * inv);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      q[e] = ((om >> e) & 1u) ? 0 : (int)r;
    }
    if (vec && c0 + 8 <= cols) {
      v2u pk;
      pk[0] = (uint32_t)(q[0] & 0xff) | ((uint32_t)(q[1] & 0xff) << 8) | ((uint32_t)(q[2] & 0xff) << 16) |
              ((uint32_t)(q[3] & 0xff) << 24);
      pk[1] = (uint32_t)(q[4] & 0xff) | ((uint32_t)(q[5] & 0xff) << 8) | ((uint32_t)(q[6] & 0xff) << 16) |
              ((uint32_t)(q[7] & 0xff) << 24);
      *reinterpret_cast<v2u*>(cr + c0) = pk;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c0 + e < cols) cr[c0 + e] = (int8_t)q[e];
    }
    if (om) {
      const int w = c0 >> 5;
      const uint32_t mw = mask[w];
      const int base = prefix[w];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if ((om >> e) & 1u) {
          const int c = c0 + e;
          const int j = base + __popc(mw & ((1u << (c & 31)) - 1u));
          if (j < cap) sub[row * (int64_t)cap + j] = __builtin_bit_cast(uint16_t, (_Float16)v[e]);
        }
      }
    }
  };

  if (in_regs) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ci = i * TPR + tid;
      if (ci < nchunk) emit(ci, vals[i]);
    }
  } else {
    for (int ci = tid; ci < nchunk; ci += TPR) {
      float v[8];
      load_chunk(ci, v);
      emit(ci, v);
    }
  }
  if (tid == 0) scale[row] = s;
}

// ---------------------------------------------------------------------------
// host-side launch sequence

static bool aligned(const void* p, int a) { return ((uintptr_t)p % (uintptr_t)a) == 0; }

template <int DT>
static hipError_t launch_quantize_t(const void* Xv, int64_t rows, int cols, float tau, int8_t* codes,
                                    float* scale, int32_t* idx, int32_t* count, uint16_t* sub, int cap,
                                    uint32_t* mask, int32_t* prefix, hipStream_t st) {
  typedef typename Elem<DT>::T T;
  const T* X = static_cast<const T*>(Xv);
  const bool tau_on = (tau > 0.0f) && (tau < __builtin_huge_valf());
  const int nwords = (cols + 31) / 32;
  const int vec = (cols % 8 == 0) && aligned(X, 16) && aligned(codes, 8);
  if (nwords > 0) {
    hipLaunchKernelGGL(k_zero_words, dim3((nwords + 255) / 256), dim3(256), 0, st, mask, nwords);
    if (tau_on && rows > 0) {
      const int gx = (cols + 2047) / 2048;
      // about 2048 workgroups in flight, at least 16 rows per slab
      int64_t want_y = (2048 + gx - 1) / gx;
      int64_t rps = (rows + want_y - 1) / want_y;
      if (rps < 16) rps = 16;
      const int64_t gy = (rows + rps - 1) / rps;
      hipLaunchKernelGGL(k_outlier_flags<DT>, dim3(gx, (unsigned)gy), dim3(256), 0, st, X, rows, cols, tau,
                         (int)rps, vec, mask);
    }
  }
  hipLaunchKernelGGL(k_outlier_compact, dim3(1), dim3(1024), 0, st, mask, nwords, prefix, idx, cap, count);
  if (rows > 0) {
    const int nchunk = (cols + 7) / 8;
    if (nchunk <= 64 * 8) {
      hipLaunchKernelGGL((k_rowquant<DT, 64, 8>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, X, rows,
                         cols, (int)tau_on, mask, prefix, vec, codes, scale, sub, cap);
    } else {
      hipLaunchKernelGGL((k_rowquant<DT, 256, 16>), dim3((unsigned)rows), dim3(256), 0, st, X, rows, cols,
                         (int)tau_on, mask, prefix, vec, codes, scale, sub, cap);
    }
  }
  return hipGetLastError();
}

hipError_t launch_quantize(int dt, const void* X, int64_t rows, int cols, float tau, int8_t* codes, float* scale,
                           int32_t* idx, int32_t* count, uint16_t* sub, int cap, uint32_t* mask, int32_t* prefix,
                           hipStream_t st) {
  switch (dt) {
    case DT_F32: return launch_quantize_t<DT_F32>(X, rows, cols, tau, codes, scale, idx, count, sub, cap, mask, prefix, st);
    case DT_F16: return launch_quantize_t<DT_F16>(X, rows, cols, tau, codes, scale, idx, count, sub, cap, mask, prefix, st);
    default: return launch_quantize_t<DT_BF16>(X, rows, cols, tau, codes, scale, idx, count, sub, cap, mask, prefix, st);
  }
}

}  // namespace i8l
