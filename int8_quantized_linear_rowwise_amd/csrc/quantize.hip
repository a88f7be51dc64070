// Row-wise int8 quantizer with outlier-column split (LLM.int8 style).
//
// bitsandbytes PR #33 "Memory efficient backward" (review "Cast A to fp16",
// commit "cast to half before double_quant"): the activation is cast to fp16
// before quantization; feature columns holding a value whose magnitude
// exceeds the threshold leave the int8 path ("4. Mixed-precision
// decomposition matmul") and are kept as a dense fp16 sub-matrix.
//
// Three kernels on the caller's stream (HBM-bound; the second read of X is
// usually served by the Infinity Cache):
//   k_outlier_flags    one read of X. A workgroup covers a slab of rows and
//                      512 columns; per column it keeps the largest magnitude
//                      in the storage format's own bits (magnitude bits order
//                      like the values, and the fp16 cast is monotone), then
//                      casts once and compares with tau. Each workgroup writes
//                      its own words of a [slab][column-word] bit array, so
//                      nothing needs clearing beforehand.
//   k_outlier_compact  one workgroup: OR over slabs (in LDS), per-word
//                      exclusive popcount prefix, ascending outlier list,
//                      count (an OR and a prefix scan: order-independent).
//   k_rowquant         second read of X, one wave per row: absmax over
//                      non-outlier columns (again on magnitude bits), s as an
//                      fp16 value, inv = 127 / s (IEEE division), codes =
//                      clamp(rint(x * inv), +-127), 0 on outlier columns,
//                      outlier values copied into the dense fp16 sub-matrix.
#include "common.hpp"
#include "kernels.hpp"

namespace i8l {

constexpr int FLAG_COLS = 512;     // columns per flags workgroup (64 lanes x 8)
constexpr int FLAG_SLABS = 256;    // at most this many row slabs in the flags pass
constexpr int FLAG_MAX_WORDS = 8192;  // column words the compaction keeps in LDS (K <= 262144)

// ---------------------------------------------------------------------------
// magnitude bits of 8 consecutive elements (storage format)

template <int DT> struct Mag8;

template <> struct Mag8<DT_F32> {
  uint32_t m[8];
  __device__ void reset() {
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = 0u;
  }
  __device__ void add(const v4u& a, const v4u& b) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m[e] = max(m[e], a[e] & 0x7fffffffu);
      m[e + 4] = max(m[e + 4], b[e] & 0x7fffffffu);
    }
  }
  __device__ float half_mag(int e) const { return (float)(_Float16)__uint_as_float(m[e]); }
};

template <int DT> struct Mag8h {
  uint32_t m[4];  // two 16-bit magnitudes per word
  __device__ void reset() {
#pragma unroll
    for (int e = 0; e < 4; ++e) m[e] = 0u;
  }
  __device__ void add(const v4u& a) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t w = a[e] & 0x7fff7fffu;
      const uint32_t lo = max(m[e] & 0xffffu, w & 0xffffu);
      const uint32_t hi = max(m[e] >> 16, w >> 16);
      m[e] = lo | (hi << 16);
    }
  }
  __device__ float half_mag(int e) const {
    const uint16_t b = (uint16_t)((e & 1) ? (m[e >> 1] >> 16) : (m[e >> 1] & 0xffffu));
    if constexpr (DT == DT_F16) return (float)__builtin_bit_cast(_Float16, b);
    else return (float)(_Float16)bf16_to_f32(b);
  }
};
template <> struct Mag8<DT_F16> : Mag8h<DT_F16> {};
template <> struct Mag8<DT_BF16> : Mag8h<DT_BF16> {};

// Load 8 consecutive elements of row r (cols c0..c0+7) as raw words, zero
// past the end of the row. vec: rows are 16-byte aligned and cols % 8 == 0.
template <int DT>
__device__ __forceinline__ void load_raw8(const typename Elem<DT>::T* __restrict__ row, int c0, int cols, bool vec,
                                          v4u& a, v4u& b) {
  typedef typename Elem<DT>::T T;
  if (vec && c0 + 8 <= cols) {
    a = *reinterpret_cast<const v4u*>(row + c0);
    if constexpr (DT == DT_F32) b = *reinterpret_cast<const v4u*>(row + c0 + 4);
    return;
  }
  uint32_t w[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (c0 + e < cols) {
      if constexpr (DT == DT_F32) {
        w[e] = __float_as_uint(row[c0 + e]);
      } else {
        const uint32_t h = (uint32_t)__builtin_bit_cast(uint16_t, row[c0 + e]);
        w[e >> 1] |= h << (16 * (e & 1));
      }
    }
  }
  a = v4u{w[0], w[1], w[2], w[3]};
  if constexpr (DT == DT_F32) b = v4u{w[4], w[5], w[6], w[7]};
}

// grid: x over column groups of 512, y over row slabs. Four waves split the
// slab's rows (wave w takes rows r0 + w, r0 + w + 4, ...); their flags are
// OR-ed in LDS and the workgroup writes its 16 words of bits[slab][word].
template <int DT>
__global__ __launch_bounds__(256) void k_outlier_flags(const typename Elem<DT>::T* __restrict__ X, int64_t rows,
                                                       int cols, float tau, int64_t rows_per_slab, int vec,
                                                       int nwords, uint32_t* __restrict__ bits) {
  typedef typename Elem<DT>::T T;
  __shared__ uint32_t sw[4][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = blockIdx.x * FLAG_COLS + lane * 8;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_slab;
  int64_t r1 = r0 + rows_per_slab;
  if (r1 > rows) r1 = rows;
  Mag8<DT> acc;
  acc.reset();
  if (c0 < cols) {
    int64_t r = r0 + wave;
    const T* p = X + r * (int64_t)cols;
    const int64_t step = 4 * (int64_t)cols;
    for (; r + 28 < r1; r += 32, p += 8 * step) {
      v4u a[8], b[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) load_raw8<DT>(p + u * step, c0, cols, vec, a[u], b[u]);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if constexpr (DT == DT_F32) acc.add(a[u], b[u]);
        else acc.add(a[u]);
      }
    }
    for (; r < r1; r += 4, p += step) {
      v4u a, b;
      load_raw8<DT>(p, c0, cols, vec, a, b);
      if constexpr (DT == DT_F32) acc.add(a, b);
      else acc.add(a);
    }
  }
  uint32_t byte = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (c0 + e < cols && acc.half_mag(e) > tau) byte |= 1u << e;
  // four lanes form one 32-bit word (columns 32w .. 32w+31)
  uint32_t word = byte << (8 * (lane & 3));
  word |= __shfl_xor(word, 1, 64);
  word |= __shfl_xor(word, 2, 64);
  if ((lane & 3) == 0) sw[wave][lane >> 2] = word;
  __syncthreads();
  if (threadIdx.x < 16) {
    const int w = blockIdx.x * (FLAG_COLS / 32) + threadIdx.x;
    if (w < nwords)
      bits[(int64_t)blockIdx.y * nwords + w] =
          sw[0][threadIdx.x] | sw[1][threadIdx.x] | sw[2][threadIdx.x] | sw[3][threadIdx.x];
  }
}

// One workgroup of 1024 threads: mask = OR over slabs; prefix; list; count.
// nwords <= FLAG_MAX_WORDS (checked on the host).
__global__ __launch_bounds__(1024) void k_outlier_compact(const uint32_t* __restrict__ bits, int slabs,
                                                          int nwords, uint32_t* __restrict__ mask,
                                                          int32_t* __restrict__ prefix, int32_t* __restrict__ idx,
                                                          int cap, int32_t* __restrict__ count) {
  __shared__ int wsum[16];
  __shared__ uint32_t smask[FLAG_MAX_WORDS];
  const int t = threadIdx.x;
  for (int w = t; w < nwords; w += 1024) smask[w] = 0u;
  __syncthreads();
  // parallel OR: thread t takes word t % nwords of slabs t / nwords + k * stride,
  // eight independent loads at a time, then one LDS OR per word and thread
  if (nwords > 0) {
    const int lanes_per_word = max(1, 1024 / nwords);
    const int w = t % nwords, s0 = t / nwords;
    if (t < lanes_per_word * nwords) {
      uint32_t m = 0u;
      int s = s0;
      for (; s + 7 * lanes_per_word < slabs; s += 8 * lanes_per_word) {
        uint32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = bits[(int64_t)(s + u * lanes_per_word) * nwords + w];
#pragma unroll
        for (int u = 0; u < 8; ++u) m |= v[u];
      }
      for (; s < slabs; s += lanes_per_word) m |= bits[(int64_t)s * nwords + w];
      if (m) atomicOr(&smask[w], m);
      // words beyond the first 1024 (nwords > 1024)
      for (int w2 = t + 1024; w2 < nwords; w2 += 1024) {
        uint32_t m2 = 0u;
        for (int s2 = 0; s2 < slabs; ++s2) m2 |= bits[(int64_t)s2 * nwords + w2];
        if (m2) atomicOr(&smask[w2], m2);
      }
    }
  }
  __syncthreads();
  for (int w = t; w < nwords; w += 1024) mask[w] = smask[w];
  const int per = (nwords + 1023) / 1024;
  const int w0 = t * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (w0 + i < nwords) local += __popc(smask[w0 + i]);
  const int lane = t & 63, wid = t >> 6;
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < wid; ++i) base += wsum[i];
  int run = base + incl - local;
  for (int i = 0; i < per; ++i) {
    const int w = w0 + i;
    if (w >= nwords) break;
    uint32_t m = smask[w];
    prefix[w] = run;
    while (m) {
      const int b = __ffs(m) - 1;
      if (run < cap) idx[run] = w * 32 + b;
      ++run;
      m &= m - 1;
    }
  }
  if (t == 1023) {
    int total_count = 0;
    for (int i = 0; i < 16; ++i) total_count += wsum[i];
    *count = total_count;
  }
}

// fp16 value (as fp32) of element e of a raw 8-element chunk
template <int DT>
__device__ __forceinline__ float chunk_val(const v4u& a, const v4u& b, int e) {
  if constexpr (DT == DT_F32) {
    const uint32_t w = (e < 4) ? a[e] : b[e - 4];
    return (float)(_Float16)__uint_as_float(w);
  } else {
    const uint32_t w = a[e >> 1];
    const uint16_t h = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
    if constexpr (DT == DT_F16) return (float)__builtin_bit_cast(_Float16, h);
    else return (float)(_Float16)bf16_to_f32(h);
  }
}

// magnitude bits of element e of a raw chunk, in the storage format
template <int DT>
__device__ __forceinline__ uint32_t chunk_mag(const v4u& a, const v4u& b, int e) {
  if constexpr (DT == DT_F32) return ((e < 4) ? a[e] : b[e - 4]) & 0x7fffffffu;
  else return ((e & 1) ? (a[e >> 1] >> 16) : a[e >> 1]) & 0x7fffu;
}

template <int DT>
__device__ __forceinline__ float mag_to_half_value(uint32_t m) {
  if constexpr (DT == DT_F32) return (float)(_Float16)__uint_as_float(m);
  else if constexpr (DT == DT_F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)m);
  else return (float)(_Float16)bf16_to_f32((uint16_t)m);
}

// Row quantization: one wave per row; a wave walks rows row0, row0 + W, ...
// (W waves in the grid). Rows of at most 64 * NCH chunks of 8 elements stay in
// registers, and the next row's loads are issued before the current row is
// quantized (two register buffers); wider rows stream twice through the
// cache, one row at a time. The column bitmask is staged in LDS.
// Outlier values of one 8-column chunk into the dense fp16 sub-matrix (rare:
// kept out of line so that it adds no registers to the main path).
template <int DT>
__device__ __noinline__ void put_outliers(uint16_t* __restrict__ srow, const uint32_t* __restrict__ smask,
                                          const int32_t* __restrict__ prefix, int c0, uint32_t om, v4u a, v4u b,
                                          int cap) {
  const int w = c0 >> 5;
  const uint32_t mw = smask[w];
  const int base = prefix[w];
  for (int e = 0; e < 8; ++e) {
    if ((om >> e) & 1u) {
      const int c = c0 + e;
      const int j = base + __popc(mw & ((1u << (c & 31)) - 1u));
      if (j < cap) srow[j] = __builtin_bit_cast(uint16_t, (_Float16)chunk_val<DT>(a, b, e));
    }
  }
}

// Row quantization: one wave per row, a wave walks rows row0, row0 + W, ...
// (W waves in the grid). VEC rows (cols % 8 == 0, 16-byte aligned) are read
// with 16-byte loads and written with 8-byte stores; with NCH > 0 a row of at
// most 64 * NCH chunks stays in registers between the absmax and the
// quantization, otherwise it streams twice through the cache. The column
// bitmask is staged in LDS.
template <int DT, int NCH, bool VEC>
__global__ __launch_bounds__(256) void k_rowquant(const typename Elem<DT>::T* __restrict__ X, int64_t rows,
                                                  int cols, int tau_on, const uint32_t* __restrict__ gmask,
                                                  const int32_t* __restrict__ prefix, int8_t* __restrict__ codes,
                                                  float* __restrict__ scale, uint16_t* __restrict__ sub, int cap) {
  typedef typename Elem<DT>::T T;
  extern __shared__ uint32_t smask[];
  const int nwords = (cols + 31) >> 5;
  if (tau_on)
    for (int w = threadIdx.x; w < nwords; w += 256) smask[w] = gmask[w];
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int64_t wstride = (int64_t)gridDim.x * 4;
  const int64_t row0 = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nchunk = (cols + 7) >> 3;

  auto chunk_mask = [&](int ci) -> uint32_t {
    if (!tau_on) return 0u;
    const int c0 = ci * 8;
    return (smask[c0 >> 5] >> (c0 & 31)) & 0xffu;
  };
  auto load = [&](const T* xr, int ci, v4u& a, v4u& b) {
    if constexpr (VEC) {
      a = *reinterpret_cast<const v4u*>(xr + ci * 8);
      if constexpr (DT == DT_F32) b = *reinterpret_cast<const v4u*>(xr + ci * 8 + 4);
    } else {
      load_raw8<DT>(xr, ci * 8, cols, false, a, b);
    }
  };
  auto absmax = [&](const v4u& a, const v4u& b, uint32_t om) -> uint32_t {
    uint32_t mx = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t m = chunk_mag<DT>(a, b, e);
      mx = ((om >> e) & 1u) ? mx : max(mx, m);
    }
    return mx;
  };
  auto emit = [&](int64_t row, int ci, const v4u& a, const v4u& b, float inv) {
    const int c0 = ci * 8;
    const uint32_t om = chunk_mask(ci);
    uint32_t q[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float r = rintf(chunk_val<DT>(a, b, e) * inv);
      r = __builtin_amdgcn_fmed3f(r, -127.0f, 127.0f);
      const uint32_t c = ((om >> e) & 1u) ? 0u : ((uint32_t)(int)r & 0xffu);
      q[e >> 2] |= c << (8 * (e & 3));
    }
    int8_t* cr = codes + row * (int64_t)cols + c0;
    if constexpr (VEC) {
      *reinterpret_cast<v2u*>(cr) = v2u{q[0], q[1]};
    } else {
      for (int e = 0; e < 8; ++e)
        if (c0 + e < cols) cr[e] = (int8_t)((q[e >> 2] >> (8 * (e & 3))) & 0xffu);
    }
    if (om) put_outliers<DT>(sub + row * (int64_t)cap, smask, prefix, c0, om, a, b, cap);
  };
  auto finish = [&](uint32_t mx, float& s, float& inv) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    s = mag_to_half_value<DT>(mx);        // max |fp16(x)| = fp16 cast of the max magnitude
    inv = (s > 0.0f) ? (127.0f / s) : 0.0f;
  };

  for (int64_t row = row0; row < rows; row += wstride) {
    const T* xr = X + row * (int64_t)cols;
    uint32_t mx = 0u;
    float sv, inv;
    if constexpr (NCH > 0) {
      v4u ra[NCH], rb[NCH];
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int ci = i * 64 + lane;
        if (ci < nchunk) load(xr, ci, ra[i], rb[i]);
      }
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int ci = i * 64 + lane;
        if (ci < nchunk) mx = max(mx, absmax(ra[i], rb[i], chunk_mask(ci)));
      }
      finish(mx, sv, inv);
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int ci = i * 64 + lane;
        if (ci < nchunk) emit(row, ci, ra[i], rb[i], inv);
      }
    } else {
      for (int cb = 0; cb < nchunk; cb += 4 * 64) {
        v4u a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int ci = cb + u * 64 + lane;
          if (ci < nchunk) load(xr, ci, a[u], b[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int ci = cb + u * 64 + lane;
          if (ci < nchunk) mx = max(mx, absmax(a[u], b[u], chunk_mask(ci)));
        }
      }
      finish(mx, sv, inv);
      for (int cb = 0; cb < nchunk; cb += 4 * 64) {
        v4u a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int ci = cb + u * 64 + lane;
          if (ci < nchunk) load(xr, ci, a[u], b[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int ci = cb + u * 64 + lane;
          if (ci < nchunk) emit(row, ci, a[u], b[u], inv);
        }
      }
    }
    if (lane == 0) scale[row] = sv;
  }
}

// ---------------------------------------------------------------------------
// host-side launch sequence

static bool aligned(const void* p, int a) { return ((uintptr_t)p % (uintptr_t)a) == 0; }

size_t quant_scratch_words(int64_t rows, int64_t cols) {
  const int64_t nw = (cols + 31) / 32;
  const int64_t slabs = rows < FLAG_SLABS ? (rows > 0 ? rows : 1) : FLAG_SLABS;
  // bits[slabs][nw] + mask[nw] + prefix[nw]
  return (size_t)((slabs + 2) * (nw > 0 ? nw : 1));
}

template <int DT>
static hipError_t launch_quantize_t(const void* Xv, int64_t rows, int cols, float tau, int8_t* codes,
                                    float* scale, int32_t* idx, int32_t* count, uint16_t* sub, int cap,
                                    uint32_t* scratch, hipStream_t st) {
  typedef typename Elem<DT>::T T;
  const T* X = static_cast<const T*>(Xv);
  const bool tau_on = (tau > 0.0f) && (tau < __builtin_huge_valf());
  const int nwords = (cols + 31) / 32;
  const int vec = (cols % 8 == 0) && aligned(X, 16) && aligned(codes, 8);
  const int64_t slabs = tau_on ? (rows < FLAG_SLABS ? (rows > 0 ? rows : 1) : FLAG_SLABS) : 0;
  const int64_t nw1 = nwords > 0 ? nwords : 1;
  uint32_t* bits = scratch;
  uint32_t* mask = scratch + (size_t)(rows < FLAG_SLABS ? (rows > 0 ? rows : 1) : FLAG_SLABS) * nw1;
  int32_t* prefix = reinterpret_cast<int32_t*>(mask + nw1);
  if (tau_on && rows > 0 && cols > 0) {
    // about 1024 workgroups, at least 32 rows per slab (8 per wave)
    const int gx = (cols + FLAG_COLS - 1) / FLAG_COLS;
    int64_t want = (1024 + gx - 1) / gx;
    if (want > slabs) want = slabs;
    int64_t rps = (rows + want - 1) / want;
    if (rps < 32) rps = 32;
    const int64_t gy = (rows + rps - 1) / rps;
    hipLaunchKernelGGL(k_outlier_flags<DT>, dim3(gx, (unsigned)gy), dim3(256), 0, st, X, rows, cols, tau, rps, vec,
                       nwords, bits);
    hipLaunchKernelGGL(k_outlier_compact, dim3(1), dim3(1024), 0, st, bits, (int)gy, nwords, mask, prefix, idx, cap,
                       count);
  } else {
    // no split: empty list, count 0, and no mask reads (tau_on = 0 below)
    hipLaunchKernelGGL(k_outlier_compact, dim3(1), dim3(1024), 0, st, bits, 0, 0, mask, prefix, idx, cap, count);
  }
  if (rows > 0) {
    const int nchunk = (cols + 7) / 8;
    const size_t lds = tau_on ? (size_t)nw1 * 4 : 0;
    const dim3 grid((unsigned)((rows + 3) / 4));   // one row per wave, four waves per workgroup
#define I8L_RQ(NCH, VEC)                                                                                   \
  hipLaunchKernelGGL((k_rowquant<DT, NCH, VEC>), grid, dim3(256), lds, st, X, rows, cols, (int)tau_on, mask, \
                     prefix, codes, scale, sub, cap)
    if (vec) {
      if (nchunk <= 64 * 8) I8L_RQ(8, true);
      else I8L_RQ(0, true);
    } else {
      if (nchunk <= 64 * 8) I8L_RQ(8, false);
      else I8L_RQ(0, false);
    }
#undef I8L_RQ
  }
  return hipGetLastError();
}

hipError_t launch_quantize(int dt, const void* X, int64_t rows, int cols, float tau, int8_t* codes, float* scale,
                           int32_t* idx, int32_t* count, uint16_t* sub, int cap, uint32_t* scratch,
                           hipStream_t st) {
  switch (dt) {
    case DT_F32: return launch_quantize_t<DT_F32>(X, rows, cols, tau, codes, scale, idx, count, sub, cap, scratch, st);
    case DT_F16: return launch_quantize_t<DT_F16>(X, rows, cols, tau, codes, scale, idx, count, sub, cap, scratch, st);
    default: return launch_quantize_t<DT_BF16>(X, rows, cols, tau, codes, scale, idx, count, sub, cap, scratch, st);
  }
}

}  // namespace i8l
