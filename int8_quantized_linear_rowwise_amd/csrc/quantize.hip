// Row-wise int8 quantizer with outlier-column split (LLM.int8 style).
//
// bitsandbytes PR #33 "Memory efficient backward" (review "Cast A to fp16",
// commit "cast to half before double_quant"): the activation is cast to fp16
// before quantization; feature columns holding a value whose magnitude
// exceeds the threshold leave the int8 path ("4. Mixed-precision
// decomposition matmul") and are kept as a dense fp16 sub-matrix.
//
// Two kernels on the caller's stream (HBM-bound; the second read of X is
// usually served by the Infinity Cache):
//   k_colflags   one read of X. A workgroup covers 64 columns of a slab of
//                rows (at most 16 slabs); per column it keeps the largest
//                magnitude in the storage format's own bits (magnitude bits
//                order like the values, and the fp16 cast is monotone), then
//                casts once and compares with tau. Each workgroup writes its
//                own two words of a [slab][column-word] bit array, so nothing
//                needs clearing beforehand.
//   k_rowquant   second read of X. Every workgroup first ORs the slab words
//                into the column mask and computes the per-word popcount
//                prefix in LDS (a few KB from L2); workgroup 0 also writes the
//                ascending outlier list and the count. Then one wave (or, for
//                rows wider than 4096 16-bit values, one workgroup) per row:
//                absmax over non-outlier columns (on magnitude bits), s as an
//                fp16 value, inv = 127 / s (IEEE division), codes =
//                rint(fl32(x * inv)) (|code| <= 127 by construction), 0 on
//                outlier columns, outlier values copied into the dense fp16
//                sub-matrix. In a forward, the workgroups then also write the
//                weight's side of the outlier product (the pages' subB): the
//                dequantized int8 weights of the first outlier columns, as
//                dense fp16 rows, so that the GEMM epilogue never gathers
//                single bytes of the weight once per output tile.

#include "common.hpp"
#include "kernels.hpp"

namespace i8l {

constexpr int CF_COLS = 64;          // columns per flags workgroup (8 lanes x 8 columns)
constexpr int CF_MAX_SLABS = 16;     // row slabs of the flags pass
constexpr int CF_SLAB_WORDS = 2048;  // slabs * words the row kernel ORs per workgroup (at most)
constexpr int RQ_MAX_BLOCKS = 1024;  // row-kernel workgroups (four rows, or one row, at a time each)

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// Slabs of the flags pass for a matrix: enough workgroups to fill the chip,
// few enough words for every row-kernel workgroup to OR them.
static int colflag_slabs(int64_t rows, int64_t cols) {
  const int64_t nw = (cols + 31) / 32;
  int64_t s = CF_SLAB_WORDS / (nw > 0 ? nw : 1);
  if (s > CF_MAX_SLABS) s = CF_MAX_SLABS;
  if (s < 1) s = 1;
  if (s > rows) s = rows > 0 ? rows : 1;
  return (int)s;
}

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

// SiLU of the 8 elements of a raw chunk, rounded to the storage format, as raw
// words (EasyDeL discussion #66: the activation between the MLP's linears).
// fp32 results use the accurate exp and IEEE division; for 16-bit results the
// hardware exp and reciprocal (a few fp32 ulps) are far inside one unit of
// the output format.
template <int DT>
__device__ __forceinline__ void silu_chunk(v4u& a, v4u& b) {
  auto f = [](float x) {
    if constexpr (DT == DT_F32) return x / (1.0f + expf(-x));
    else return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
  };
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      a[d] = __float_as_uint(f(__uint_as_float(a[d])));
      b[d] = __float_as_uint(f(__uint_as_float(b[d])));
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint16_t lo = (uint16_t)(a[d] & 0xffffu), hi = (uint16_t)(a[d] >> 16);
      typedef typename Elem<DT>::T T;
      const T rl = Elem<DT>::from_f32(f(Elem<DT>::to_f32(__builtin_bit_cast(T, lo))));
      const T rh = Elem<DT>::from_f32(f(Elem<DT>::to_f32(__builtin_bit_cast(T, hi))));
      a[d] = (uint32_t)__builtin_bit_cast(uint16_t, rl) | ((uint32_t)__builtin_bit_cast(uint16_t, rh) << 16);
    }
  }
}

// Store a raw 8-element chunk to row[c0 .. c0 + 7], clipped to cols.
template <int DT>
__device__ __forceinline__ void store_raw8(typename Elem<DT>::T* __restrict__ row, int c0, int cols, bool vec,
                                           const v4u& a, const v4u& b) {
  typedef typename Elem<DT>::T T;
  if (vec && c0 + 8 <= cols) {
    *reinterpret_cast<v4u*>(row + c0) = a;
    if constexpr (DT == DT_F32) *reinterpret_cast<v4u*>(row + c0 + 4) = b;
    return;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (c0 + e < cols) {
      if constexpr (DT == DT_F32) {
        row[c0 + e] = __uint_as_float(e < 4 ? a[e] : b[e - 4]);
      } else {
        row[c0 + e] = __builtin_bit_cast(T, (uint16_t)(a[e >> 1] >> (16 * (e & 1))));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// column flags: grid (ceil(cols / 64), slabs), 256 threads. Lane l reads the
// 8-column chunk l & 7 of rows r0 + 8 * wave + (l >> 3) + 32 i; the running
// maximum is kept on magnitude bits (two 16-bit magnitudes per word for fp16
// and bf16). Lanes and waves sharing a chunk are then combined, the maxima
// cast to fp16 once and compared with tau, and the workgroup writes words
// 2 bx and 2 bx + 1 of bits[slab].
// With ACT the kernel is also the producer of its input: it reads H, stores
// X = SiLU(H) (rounded to the storage format) and flags the columns of X.
template <int DT, bool ACT = false>
__global__ __launch_bounds__(256) void k_colflags(const typename Elem<DT>::T* __restrict__ X, int64_t rows,
                                                  int cols, float tau, int64_t rows_per_slab, int vec, int nwords,
                                                  uint32_t* __restrict__ bits,
                                                  typename Elem<DT>::T* __restrict__ act_out = nullptr) {
  typedef typename Elem<DT>::T T;
  constexpr int NW = (DT == DT_F32) ? 8 : 4;   // words of magnitudes per 8-column chunk
  __shared__ uint32_t sm[4][8][NW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cc = lane & 7, ro = lane >> 3;
  const int c0 = blockIdx.x * CF_COLS + cc * 8;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_slab;
  const int64_t r1 = min(rows, r0 + rows_per_slab);

  uint32_t m[NW];
#pragma unroll
  for (int d = 0; d < NW; ++d) m[d] = 0u;
  auto add = [&](const v4u& a, const v4u& b) {
    if constexpr (DT == DT_F32) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        m[d] = max(m[d], a[d] & 0x7fffffffu);
        m[d + 4] = max(m[d + 4], b[d] & 0x7fffffffu);
      }
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d)
        m[d] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, m[d]),
                                                                      __builtin_bit_cast(us2, a[d] & 0x7fff7fffu)));
    }
  };
  if (c0 < cols) {
    const bool fast = vec && c0 + 8 <= cols;
    // with ACT the chunk of row r is activated and stored before it is flagged
    auto consume = [&](int64_t row, v4u& a, v4u& b) {
      if constexpr (ACT) {
        silu_chunk<DT>(a, b);
        store_raw8<DT>(act_out + row * (int64_t)cols, c0, cols, fast, a, b);
      }
      add(a, b);
    };
    int64_t r = r0 + 8 * wave + ro;
    // groups of 8 rows (stride 32); the next group's loads are issued before
    // the current group is reduced
    if (r + 7 * 32 < r1) {
      v4u a[8], b[8], na[8], nb[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) load_raw8<DT>(X + (r + 32 * u) * (int64_t)cols, c0, cols, fast, a[u], b[u]);
      int64_t rg = r;
      for (r += 8 * 32; r + 7 * 32 < r1; r += 8 * 32) {
#pragma unroll
        for (int u = 0; u < 8; ++u) load_raw8<DT>(X + (r + 32 * u) * (int64_t)cols, c0, cols, fast, na[u], nb[u]);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          consume(rg + 32 * u, a[u], b[u]);
          a[u] = na[u];
          b[u] = nb[u];
        }
        rg = r;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) consume(rg + 32 * u, a[u], b[u]);
    }
    for (; r < r1; r += 32) {
      v4u a, b;
      load_raw8<DT>(X + r * (int64_t)cols, c0, cols, fast, a, b);
      consume(r, a, b);
    }
  }
  // lanes with the same chunk: xor over the row-offset bits of the lane id
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {
#pragma unroll
    for (int d = 0; d < NW; ++d) {
      const uint32_t o = (uint32_t)__shfl_xor((int)m[d], off, 64);
      if constexpr (DT == DT_F32) m[d] = max(m[d], o);
      else m[d] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, m[d]),
                                                                         __builtin_bit_cast(us2, o)));
    }
  }
  if (ro == 0)
#pragma unroll
    for (int d = 0; d < NW; ++d) sm[wave][cc][d] = m[d];
  __syncthreads();
  if (threadIdx.x < 8) {
    uint32_t byte = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t mm = 0u;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t v;
        if constexpr (DT == DT_F32) v = sm[w][cc][e];
        else v = (sm[w][cc][e >> 1] >> (16 * (e & 1))) & 0xffffu;
        mm = max(mm, v);
      }
      if (c0 + e < cols && mag_to_half_value<DT>(mm) > tau) byte |= 1u << e;
    }
    // lanes 0..3 -> word 2 bx (columns 0..31 of the group), lanes 4..7 -> word 2 bx + 1
    uint32_t word = byte << (8 * (cc & 3));
    word |= (uint32_t)__shfl_xor((int)word, 1, 64);
    word |= (uint32_t)__shfl_xor((int)word, 2, 64);
    const int w = blockIdx.x * 2 + (cc >> 2);
    if ((cc & 3) == 0 && w < nwords) bits[(int64_t)blockIdx.y * nwords + w] = word;
  }
}

// ---------------------------------------------------------------------------
// Per-chunk pieces of the row kernels (a chunk: 8 consecutive columns).

// column-mask bits of chunk ci
__device__ __forceinline__ uint32_t chunk_mask_bits(const uint32_t* smask, int ci) {
  const int c0 = ci * 8;
  return (smask[c0 >> 5] >> (c0 & 31)) & 0xffu;
}

// largest magnitude (storage-format bits) of the chunk's non-outlier
// elements; om: the chunk's outlier-column bits; any: some lane of the wave
// has an outlier column in this chunk (wave-uniform, so that the common case
// skips all masking)
template <int DT, bool VEC>
__device__ __forceinline__ uint32_t chunk_absmax(const v4u& a, const v4u& b, uint32_t om, bool any) {
  if constexpr (VEC && DT != DT_F32) {
    us2 mx = {0, 0};
    if (!any) {
#pragma unroll
      for (int d = 0; d < 4; ++d) mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, a[d] & 0x7fff7fffu));
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t keep = (((om >> (2 * d)) & 1u) ? 0u : 0x0000ffffu) | (((om >> (2 * d + 1)) & 1u) ? 0u : 0xffff0000u);
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, a[d] & 0x7fff7fffu & keep));
      }
    }
    return max((uint32_t)mx[0], (uint32_t)mx[1]);
  } else {
    uint32_t mx = 0u;
    if (!any) {
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = max(mx, chunk_mag<DT>(a, b, e));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t m = chunk_mag<DT>(a, b, e);
        mx = ((om >> e) & 1u) ? mx : max(mx, m);
      }
    }
    return mx;
  }
}

// codes of one chunk, packed little-endian into two words: x16 = fp16(x),
// code = rint(fl32(x16 * inv)) by the exact fp32 add of 1.5 * 2^23
template <int DT>
__device__ __forceinline__ void chunk_quant8(const v4u& a, const v4u& b, float inv, uint32_t& lo, uint32_t& hi) {
#pragma clang fp contract(off)
  uint32_t h[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    if constexpr (DT == DT_F16) h[d] = a[d];
    else if constexpr (DT == DT_BF16) h[d] = bf16x2_to_f16x2(a[d]);
    else h[d] = f32x2_to_f16x2(__uint_as_float(d < 2 ? a[2 * d] : b[2 * d - 4]),
                               __uint_as_float(d < 2 ? a[2 * d + 1] : b[2 * d - 3]));
  }
  uint32_t q[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const _Float16 x = __builtin_bit_cast(_Float16, (uint16_t)(h[e >> 1] >> (16 * (e & 1))));
    const float p = (float)x * inv;
    q[e] = __float_as_uint(p + 12582912.0f);
  }
  lo = __builtin_amdgcn_perm(q[1], q[0], 0x0c0c0400u) | __builtin_amdgcn_perm(q[3], q[2], 0x04000c0cu);
  hi = __builtin_amdgcn_perm(q[5], q[4], 0x0c0c0400u) | __builtin_amdgcn_perm(q[7], q[6], 0x04000c0cu);
}

// chunk ci of row `row` to memory: codes, 0 on outlier columns, whose fp16
// values go to the dense sub-matrix at their rank among the outlier columns
// (the prefix of the column's mask word plus the set bits below it)
template <int DT, bool VEC>
__device__ __forceinline__ void chunk_emit(int8_t* __restrict__ codes, uint16_t* __restrict__ sub, int cap,
                                           int cols, const uint32_t* smask, const int32_t* sprefix, int64_t row,
                                           int ci, const v4u& a, const v4u& b, float inv, uint32_t om, bool any) {
  const int c0 = ci * 8;
  uint32_t lo, hi;
  chunk_quant8<DT>(a, b, inv, lo, hi);
  if (any && om) {
    uint32_t kl = 0u, kh = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kl |= ((om >> e) & 1u) ? 0u : (0xffu << (8 * e));
      kh |= ((om >> (e + 4)) & 1u) ? 0u : (0xffu << (8 * e));
    }
    lo &= kl;
    hi &= kh;
    uint16_t* srow = sub + row * (int64_t)cap;
    const int w = c0 >> 5;
    const uint32_t mw = smask[w];
    const int base = sprefix[w];
    uint32_t rest = om;
    while (rest) {
      const int e = __ffs(rest) - 1;
      rest &= rest - 1u;
      const int c = c0 + e;
      const int j = base + __popc(mw & ((1u << (c & 31)) - 1u));
      if (j < cap) srow[j] = __builtin_bit_cast(uint16_t, (_Float16)chunk_val<DT>(a, b, e));
    }
  }
  int8_t* cr = codes + row * (int64_t)cols + c0;
  if constexpr (VEC) {
    *reinterpret_cast<v2u*>(cr) = v2u{lo, hi};
  } else {
    for (int e = 0; e < 8; ++e)
      if (c0 + e < cols) cr[e] = (int8_t)(((e < 4 ? lo : hi) >> (8 * (e & 3))) & 0xffu);
  }
}

// With the column mask in LDS (smask, written by the whole workgroup and
// followed by a barrier): the exclusive popcount prefix per word (sprefix,
// LDS). With `list`, the ascending outlier list (first idx_cap entries) and
// the count go to memory; the first wcap columns also go to slist (LDS).
// Called by the whole workgroup; returns |O|.
__device__ __forceinline__ int mask_prefix(const uint32_t* smask, int32_t* sprefix, int* wsum, int nwords,
                                           bool list, int32_t* __restrict__ idx, int idx_cap,
                                           int32_t* __restrict__ count, int* slist, int wcap) {
  const int t = threadIdx.x, lane = t & 63, wid = __builtin_amdgcn_readfirstlane(t >> 6);
  const int per = (nwords + 255) / 256;
  const int w0 = t * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (w0 + i < nwords) local += __popc(smask[w0 + i]);
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  int run = incl - local;
  for (int i = 0; i < wid; ++i) run += wsum[i];
  for (int i = 0; i < per; ++i) {
    const int w = w0 + i;
    if (w >= nwords) break;
    sprefix[w] = run;
    uint32_t mw = smask[w];
    if (list || run < wcap) {
      int j = run;
      while (mw) {
        const int b = __ffs(mw) - 1;
        if (list && j < idx_cap) idx[j] = w * 32 + b;
        if (j < wcap) slist[j] = w * 32 + b;
        ++j;
        mw &= mw - 1u;
      }
    }
    run += __popc(smask[w]);
  }
  const int tot = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  if (list && t == 0) *count = tot;
  __syncthreads();
  return tot;
}

// The weight's side of the outlier product in a forward: wsub[n * wcap + j] =
// fp16(fl32(CB[n, O[j]] * fl32(SCB[n] * fl32(1/127)))) for j < min(tot, wcap),
// the columns listed in slist. Four weight rows per wave and pass, lanes over
// the outlier columns (one byte gather each, every row's values written as
// one contiguous run).
__device__ __forceinline__ void weight_slice(const int8_t* __restrict__ wCB, const float* __restrict__ wSCB, int wN,
                                             int K, uint16_t* __restrict__ wsub, int wcap, const int* slist,
                                             int tot) {
  const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cw = min(tot, wcap);
  const int64_t gw = (int64_t)blockIdx.x * 4 + wid, nwv = (int64_t)gridDim.x * 4;
  for (int jb = 0; jb < cw; jb += 64) {
    const int j = jb + lane;
    const bool jok = j < cw;
    const int col = jok ? slist[j] : 0;
    for (int64_t n = gw * 4; n < wN; n += nwv * 4) {
      int v[4];
      float sg[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool ok = n + u < wN;
        v[u] = (ok && jok) ? (int)wCB[(n + u) * (int64_t)K + col] : 0;
        sg[u] = ok ? wSCB[n + u] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (jok && n + u < wN)
          wsub[(n + u) * (int64_t)wcap + j] =
              __builtin_bit_cast(uint16_t, half_of_f32((float)v[u] * (sg[u] * (1.0f / 127.0f))));
    }
  }
}

// ---------------------------------------------------------------------------
// Row quantization. Prologue of every workgroup (tau on): column mask = OR
// of the slab words, exclusive per-word popcount prefix, both in LDS;
// workgroup 0 writes the ascending outlier list (first cap entries) and the
// count (the first idx_cap entries of the list; the outlier values of the
// first cap columns go to the dense sub-matrix). Then one wave per row, a
// wave walks rows row0, row0 + W, ... (W
// waves in the grid); with WG one workgroup per row instead, walking rows
// blockIdx.x, blockIdx.x + gridDim.x, ... VEC rows (cols % 8 == 0, 16-byte
// aligned) are read with 16-byte loads and written with 8-byte stores; with
// NCH > 0 a row of at most NCH chunks per thread (64 NCH, or 256 NCH with WG)
// stays in registers between the absmax and the quantization, so it is read
// once; otherwise it streams twice through the cache.
//
// Quantization of one element: x16 = fp16(x), p = fl32(x16 * inv),
// code = rint(p). For a non-outlier column |x16| <= s, and fl32(s * fl32(127 /
// s)) rounds to 127 for every fp16 value s, so |code| <= 127 and the clamp to
// [-127, 127] never applies. rint is computed as fl32(p + 1.5 * 2^23), whose
// low byte is the two's-complement code; contraction into an FMA is off so
// that the product is rounded to fp32 first.
template <int DT, int NCH, bool VEC, bool WG = false>
__global__ __launch_bounds__(256) void k_rowquant(const typename Elem<DT>::T* __restrict__ X, int64_t rows,
                                                  int cols, int tau_on, const uint32_t* __restrict__ bits,
                                                  int slabs, int8_t* __restrict__ codes, float* __restrict__ scale,
                                                  int32_t* __restrict__ idx, int idx_cap,
                                                  int32_t* __restrict__ count, uint16_t* __restrict__ sub, int cap,
                                                  const int8_t* __restrict__ wCB, const float* __restrict__ wSCB,
                                                  int wN, uint16_t* __restrict__ wsub, int wcap) {
#pragma clang fp contract(off)
  typedef typename Elem<DT>::T T;
  extern __shared__ uint32_t smem_q[];
  __shared__ int wsum[4];
  __shared__ int slist[256];   // the first wcap outlier columns (weight slice)
  const bool wfill = wsub != nullptr && wcap > 0;
  const int nwords = (cols + 31) >> 5;
  uint32_t* smask = smem_q;
  int32_t* sprefix = reinterpret_cast<int32_t*>(smem_q + nwords);
  const int t = threadIdx.x, lane = t & 63, wid = __builtin_amdgcn_readfirstlane(t >> 6);
  // a row belongs to one wave, or with WG to the whole workgroup (TPR threads)
  constexpr int TPR = WG ? 256 : 64;
  const int me = WG ? t : lane;
  const int64_t wstride = WG ? (int64_t)gridDim.x : (int64_t)gridDim.x * 4;
  const int64_t row0 = WG ? (int64_t)blockIdx.x : (int64_t)blockIdx.x * 4 + wid;
  const int nchunk = (cols + 7) >> 3;
  auto load = [&](const T* xr, int ci, v4u& a, v4u& b) {
    if constexpr (VEC) {
      a = *reinterpret_cast<const v4u*>(xr + ci * 8);
      if constexpr (DT == DT_F32) b = *reinterpret_cast<const v4u*>(xr + ci * 8 + 4);
    } else {
      load_raw8<DT>(xr, ci * 8, cols, false, a, b);
    }
  };
  // slab words of this thread's first column word, requested before the row
  // data (memory requests of a wave complete in order)
  uint32_t sw[CF_MAX_SLABS];
  const bool w0ok = tau_on && t < nwords;
  if (w0ok) {
#pragma unroll
    for (int sl = 0; sl < CF_MAX_SLABS; ++sl) sw[sl] = sl < slabs ? bits[(int64_t)sl * nwords + t] : 0u;
  }
  // register-resident rows (16-bit, VEC) are read through a buffer resource
  // per row: chunks past the row read as zero without a memory access, so the
  // loads need no branch. The first row is requested before the prologue, so
  // that its memory latency overlaps the mask construction.
  constexpr int NR = NCH > 0 ? NCH : 1;
  v4u ra[NR], rb[NR] = {};
  auto load_row = [&](int64_t r, v4u(&a)[NR]) {
    const bool in = r < rows;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(X + (in ? r : 0) * (int64_t)cols, in ? cols * (int)sizeof(T) : 0);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int ci = i * TPR + me;
      a[i] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, ci < nchunk ? ci * 16 : OOB_OFFSET, 0, 0));
    }
  };
  if constexpr (NCH > 0) load_row(row0, ra);

  int tot = 0;
  if (tau_on) {
    if (w0ok) {
      uint32_t mw = 0u;
#pragma unroll
      for (int sl = 0; sl < CF_MAX_SLABS; ++sl) mw |= sw[sl];
      smask[t] = mw;
    }
    for (int w = t + 256; w < nwords; w += 256) {
      uint32_t v[CF_MAX_SLABS];
#pragma unroll
      for (int sl = 0; sl < CF_MAX_SLABS; ++sl) v[sl] = sl < slabs ? bits[(int64_t)sl * nwords + w] : 0u;
      uint32_t mw = 0u;
#pragma unroll
      for (int sl = 0; sl < CF_MAX_SLABS; ++sl) mw |= v[sl];
      smask[w] = mw;
    }
    __syncthreads();
    tot = mask_prefix(smask, sprefix, wsum, nwords, blockIdx.x == 0, idx, idx_cap, count, slist,
                      wfill ? wcap : 0);
  } else if (blockIdx.x == 0 && t == 0) {
    *count = 0;
  }

  auto chunk_mask = [&](int ci) -> uint32_t { return tau_on ? chunk_mask_bits(smask, ci) : 0u; };
  auto absmax = [&](const v4u& a, const v4u& b, uint32_t om, bool any) -> uint32_t {
    return chunk_absmax<DT, VEC>(a, b, om, any);
  };
  auto emit = [&](int64_t row, int ci, const v4u& a, const v4u& b, float inv, uint32_t om, bool any) {
    chunk_emit<DT, VEC>(codes, sub, cap, cols, smask, sprefix, row, ci, a, b, inv, om, any);
  };
  // with WG the wave maxima meet in LDS; the two slots alternate by row, so
  // one barrier per row suffices
  __shared__ uint32_t red[2][4];
  int par = 0;
  auto finish = [&](uint32_t mx, float& s, float& inv) {
    mx = wave_umax(mx);
    if constexpr (WG) {
      if (lane == 0) red[par][wid] = mx;
      __syncthreads();
      mx = max(max(red[par][0], red[par][1]), max(red[par][2], red[par][3]));
      par ^= 1;
    }
    s = mag_to_half_value<DT>(mx);        // max |fp16(x)| = fp16 cast of the max magnitude
    inv = (s > 0.0f) ? (127.0f / s) : 0.0f;
  };

  // the outlier columns are the same for every row: a wave-uniform flag per
  // register chunk (once per wave) lets the common case skip all masking; the
  // chunk masks themselves are re-read from LDS only where a flag is set
  uint32_t anyb = 0u;
  if constexpr (NCH > 0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ci = i * TPR + me;
      const uint32_t om = ci < nchunk ? chunk_mask(ci) : 0u;
      if (__builtin_amdgcn_ballot_w64(om != 0u) != 0) anyb |= 1u << i;
    }
  }
  auto rmask = [&](int i) -> uint32_t {
    const int ci = i * TPR + me;
    return ((anyb >> i) & 1u) && ci < nchunk ? chunk_mask(ci) : 0u;
  };

  if constexpr (NCH > 0) {
    static_assert(VEC && DT != DT_F32, "register-resident rows are 16-bit, 16-byte aligned");
    for (int64_t row = row0; row < rows; row += wstride) {
      if (row != row0) load_row(row, ra);
      uint32_t mx = 0u;
      float sv, inv;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int ci = i * TPR + me;
        if (ci < nchunk) mx = max(mx, absmax(ra[i], rb[i], rmask(i), (anyb >> i) & 1u));
      }
      finish(mx, sv, inv);
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int ci = i * TPR + me;
        if (ci < nchunk) emit(row, ci, ra[i], rb[i], inv, rmask(i), (anyb >> i) & 1u);
      }
      if (me == 0) scale[row] = sv;
    }
  } else {
    for (int64_t row = row0; row < rows; row += wstride) {
      const T* xr = X + row * (int64_t)cols;
      uint32_t mx = 0u;
      float sv, inv;
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
            const uint32_t om = ci < nchunk ? chunk_mask(ci) : 0u;
            const bool any = __builtin_amdgcn_ballot_w64(om != 0u) != 0;
            if (ci < nchunk) mx = max(mx, absmax(a[u], b[u], om, any));
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
            const uint32_t om = ci < nchunk ? chunk_mask(ci) : 0u;
            const bool any = __builtin_amdgcn_ballot_w64(om != 0u) != 0;
            if (ci < nchunk) emit(row, ci, a[u], b[u], inv, om, any);
          }
        }
      if (lane == 0) scale[row] = sv;
    }
  }

  if (tau_on && wfill) weight_slice(wCB, wSCB, wN, cols, wsub, wcap, slist, tot);
}

// ---------------------------------------------------------------------------
// host-side launch sequence

static bool aligned(const void* p, int a) { return ((uintptr_t)p % (uintptr_t)a) == 0; }

size_t quant_scratch_words(int64_t rows, int64_t cols) {
  const int64_t nw = (cols + 31) / 32;
  // bits[slabs][nw]
  return (size_t)(colflag_slabs(rows, cols) * (nw > 0 ? nw : 1));
}

template <int DT>
static hipError_t launch_quantize_t(const void* Xv, int64_t rows, int cols, float tau, int8_t* codes,
                                    float* scale, int32_t* idx, int idx_cap, int32_t* count, uint16_t* sub, int cap,
                                    uint32_t* scratch, const uint32_t* preflags, const OutlierWeights* ow,
                                    hipStream_t st) {
  typedef typename Elem<DT>::T T;
  const T* X = static_cast<const T*>(Xv);
  // column flags handed over by the producer of X replace the flags pass
  const bool tau_on = (preflags != nullptr || ((tau > 0.0f) && (tau < __builtin_huge_valf()))) && rows > 0 &&
                      cols > 0;
  const int nwords = (cols + 31) / 32;
  const int vec = (cols % 8 == 0) && aligned(X, 16) && aligned(codes, 8);
  const int slabs = colflag_slabs(rows, cols);
  const uint32_t* bits = preflags != nullptr ? preflags : scratch;
  // weight slice (forward only)
  const bool wf = ow != nullptr && ow->wsub != nullptr && ow->wcap > 0 && ow->N > 0 && tau_on;
  const int8_t* wCB = wf ? ow->CB : nullptr;
  const float* wSCB = wf ? ow->SCB : nullptr;
  uint16_t* wsub = wf ? ow->wsub : nullptr;
  const int wN = wf ? ow->N : 0, wcap = wf ? ow->wcap : 0;
  if (tau_on && preflags == nullptr) {
    const int gx = (cols + CF_COLS - 1) / CF_COLS;
    const int64_t rps = (rows + slabs - 1) / slabs;
    hipLaunchKernelGGL(k_colflags<DT>, dim3(gx, (unsigned)slabs), dim3(256), 0, st, X, rows, cols, tau, rps, vec,
                       nwords, scratch, nullptr);
  }
  // the row kernel also writes the outlier list and count (count 0 when the split is off)
  // workgroups: four rows at a time (one per wave), or one row at a time
  const int64_t rblocks = rows > 0 ? ((rows + 3) / 4 < RQ_MAX_BLOCKS ? (rows + 3) / 4 : RQ_MAX_BLOCKS) : 1;
  const int64_t wblocks = rows > 0 ? (rows < RQ_MAX_BLOCKS ? rows : RQ_MAX_BLOCKS) : 1;
  // with the weight slice to write, at least one wave per 16 weight rows (up
  // to the cap); the extra workgroups have no rows of X
  const int64_t fblocks = wf ? ((int64_t)ow->N + 15) / 16 : 1;
  const int nchunk = (cols + 7) / 8;
  const size_t lds = tau_on ? (size_t)2 * (nwords > 0 ? nwords : 1) * 4 : 0;
#define I8L_RQ(NCH, VEC, WGM)                                                                                   \
  do {                                                                                                          \
    auto kern = k_rowquant<DT, NCH, VEC, WGM>;                                                                  \
    if (lds > 32768) {                                                                                          \
      hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
      if (e != hipSuccess) return e;                                                                            \
    }                                                                                                           \
    int64_t nb = WGM ? wblocks : rblocks;                                                                       \
    if (fblocks > nb) nb = fblocks < RQ_MAX_BLOCKS ? fblocks : RQ_MAX_BLOCKS;                                   \
    hipLaunchKernelGGL(kern, dim3((unsigned)nb), dim3(256), lds, st, X, rows, cols, (int)tau_on, bits, slabs,   \
                       codes, scale, idx, idx_cap, count, sub, cap, wCB, wSCB, wN, wsub, wcap);                 \
  } while (0)
  // 16-bit rows stay in registers between the absmax and the quantization:
  // rows of up to 4096 values in one wave, up to 32768 values spread over a
  // workgroup (4, 8 or 16 chunks of 8 per thread); fp32, wider, unaligned or
  // ragged rows stream through the cache twice
  bool done = false;
  if constexpr (DT != DT_F32) {
    if (vec && nchunk <= 64 * 8) {
      I8L_RQ(8, true, false);
      done = true;
    } else if (vec && nchunk <= 256 * 4) {
      I8L_RQ(4, true, true);
      done = true;
    } else if (vec && nchunk <= 256 * 8) {
      I8L_RQ(8, true, true);
      done = true;
    } else if (vec && nchunk <= 256 * 16) {
      I8L_RQ(16, true, true);
      done = true;
    }
  }
  if (!done) {
    if (vec) I8L_RQ(0, true, false);
    else I8L_RQ(0, false, false);
  }
#undef I8L_RQ
  return hipGetLastError();
}

hipError_t launch_quantize(int dt, const void* X, int64_t rows, int cols, float tau, int8_t* codes, float* scale,
                           int32_t* idx, int32_t* count, uint16_t* sub, int cap, uint32_t* scratch,
                           hipStream_t st, const uint32_t* preflags, int idx_cap, const OutlierWeights* ow) {
  if (idx_cap < 0) idx_cap = cap;
  if (ow != nullptr && (ow->K != cols || ow->wcap > 256)) return hipErrorInvalidValue;
  switch (dt) {
    case DT_F32:
      return launch_quantize_t<DT_F32>(X, rows, cols, tau, codes, scale, idx, idx_cap, count, sub, cap, scratch,
                                       preflags, ow, st);
    case DT_F16:
      return launch_quantize_t<DT_F16>(X, rows, cols, tau, codes, scale, idx, idx_cap, count, sub, cap, scratch,
                                       preflags, ow, st);
    default:
      return launch_quantize_t<DT_BF16>(X, rows, cols, tau, codes, scale, idx, idx_cap, count, sub, cap, scratch,
                                        preflags, ow, st);
  }
}

template <int DT>
static hipError_t launch_silu_flags_t(const void* Hv, int64_t rows, int cols, float tau, void* Av, uint32_t* flags,
                                      hipStream_t st) {
  typedef typename Elem<DT>::T T;
  const T* H = static_cast<const T*>(Hv);
  T* A = static_cast<T*>(Av);
  if (rows <= 0 || cols <= 0) return hipSuccess;
  // with the split off no column is flagged: compare against +inf
  const bool tau_on = (tau > 0.0f) && (tau < __builtin_huge_valf());
  const int nwords = (cols + 31) / 32;
  const int vec = (cols % 8 == 0) && aligned(H, 16) && aligned(A, 16);
  const int slabs = colflag_slabs(rows, cols);
  const int gx = (cols + CF_COLS - 1) / CF_COLS;
  const int64_t rps = (rows + slabs - 1) / slabs;
  hipLaunchKernelGGL((k_colflags<DT, true>), dim3(gx, (unsigned)slabs), dim3(256), 0, st, H, rows, cols,
                     tau_on ? tau : __builtin_huge_valf(), rps, vec, nwords, flags, A);
  return hipGetLastError();
}

hipError_t launch_silu_flags(int dt, const void* H, int64_t rows, int cols, float tau, void* A, uint32_t* flags,
                             hipStream_t st) {
  switch (dt) {
    case DT_F32: return launch_silu_flags_t<DT_F32>(H, rows, cols, tau, A, flags, st);
    case DT_F16: return launch_silu_flags_t<DT_F16>(H, rows, cols, tau, A, flags, st);
    default: return launch_silu_flags_t<DT_BF16>(H, rows, cols, tau, A, flags, st);
  }
}

}  // namespace i8l
