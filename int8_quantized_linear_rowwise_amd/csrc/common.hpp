// Shared device helpers for the int8 linear kernels (gfx950 / CDNA4).
//
// Storage dtypes: 0 = fp32, 1 = fp16, 2 = bf16 (bf16 handled as raw 16-bit
// patterns). All conversions to fp16 and from fp32 round to nearest even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace i8l {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

// Two bf16 values packed in a word -> two fp16 values packed in a word (RNE).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  const v2f f = {__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, v2h));
}
// fp16 value (RNE) of x after x has been rounded to fp32. A product written
// straight into an fp16 conversion is otherwise compiled to one
// mixed-precision FMA (v_fma_mixlo_f16), even with contraction off, which
// rounds the exact product to fp16 in one step; that differs from rounding it
// to fp32 first whenever the fp32 product lies exactly halfway between two
// fp16 values. The empty asm statement (no instruction) keeps x an fp32
// register value.
__device__ __forceinline__ _Float16 half_of_f32(float x) {
  asm("" : "+v"(x));
  return (_Float16)x;
}

// Two fp32 values -> two fp16 values packed in a word (RNE).
__device__ __forceinline__ uint32_t f32x2_to_f16x2(float a, float b) {
  const v2f f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, v2h));
}

enum DType : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN): the language
// conversion, one v_cvt_pk_bf16_f32 on gfx950. Only the scalar form is used;
// its result equals the bias-and-truncate rounding for every fp32 input.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Element type traits: load 8 consecutive elements as fp32 values of their
// fp16 cast (the fp16 cast is exact for fp16 and RNE for fp32 / bf16).
template <int DT> struct Elem;

template <> struct Elem<DT_F32> {
  typedef float T;
  static constexpr int size = 4;
  __device__ static __forceinline__ float to_f32(T v) { return v; }
  __device__ static __forceinline__ T from_f32(float f) { return f; }
};
template <> struct Elem<DT_F16> {
  typedef _Float16 T;
  static constexpr int size = 2;
  __device__ static __forceinline__ float to_f32(T v) { return (float)v; }
  __device__ static __forceinline__ T from_f32(float f) { return (_Float16)f; }
};
template <> struct Elem<DT_BF16> {
  typedef uint16_t T;
  static constexpr int size = 2;
  __device__ static __forceinline__ float to_f32(T v) { return bf16_to_f32(v); }
  __device__ static __forceinline__ T from_f32(float f) { return f32_to_bf16(f); }
};

// Value of the fp16 cast of element v, as fp32 (exact).
template <int DT>
__device__ __forceinline__ float half_cast_f32(typename Elem<DT>::T v) {
  if constexpr (DT == DT_F16) return (float)v;
  else return (float)(_Float16)Elem<DT>::to_f32(v);
}

template <int DT>
__device__ __forceinline__ _Float16 to_half(typename Elem<DT>::T v) {
  if constexpr (DT == DT_F16) return v;
  else return (_Float16)Elem<DT>::to_f32(v);
}

// Load 8 consecutive elements (vector load; caller guarantees alignment).
template <int DT>
__device__ __forceinline__ void load8(const typename Elem<DT>::T* p, typename Elem<DT>::T (&out)[8]) {
  if constexpr (DT == DT_F32) {
    const v4f* q = reinterpret_cast<const v4f*>(p);
    v4f a = q[0], b = q[1];
    out[0] = a[0]; out[1] = a[1]; out[2] = a[2]; out[3] = a[3];
    out[4] = b[0]; out[5] = b[1]; out[6] = b[2]; out[7] = b[3];
  } else {
    v4u a = *reinterpret_cast<const v4u*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w = a[i];
      uint16_t lo = (uint16_t)(w & 0xffffu), hi = (uint16_t)(w >> 16);
      out[2 * i] = __builtin_bit_cast(typename Elem<DT>::T, lo);
      out[2 * i + 1] = __builtin_bit_cast(typename Elem<DT>::T, hi);
    }
  }
}

__device__ __forceinline__ int ceil_div_i(int a, int b) { return (a + b - 1) / b; }

// LDS tiles of 128-byte rows are stored with their eight 16-byte chunks
// permuted: chunk c of row r lives at position c ^ lds_swz(r). For 16-byte
// accesses by consecutive rows (operand fragment reads) or by eight lanes
// sharing a row (tile writes) the positions hit distinct bank groups, with
// either 32 or 64 four-byte banks. lds_swz depends only on r mod 32, so row
// offsets that are multiples of 32 fold into instruction immediates.
__device__ __forceinline__ int lds_swz(int r) { return (r & 7) ^ ((r >> 3) & 3); }

// Buffer resource for raw (byte-addressed) buffer loads: reads at offsets
// beyond num_bytes return zero without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num_bytes, 0x00020000);
}
constexpr int OOB_OFFSET = 0x7ffffff0;

#define I8L_SGB(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)
enum : int { SG_MFMA = 0x008, SG_VMEM_R = 0x020, SG_DS_R = 0x100, SG_DS_W = 0x200, SG_VALU = 0x002 };

// Output-tile order. Workgroups are handed to the 8 XCDs round-robin; each
// XCD gets one contiguous run of tile ids (so neighbouring tiles share that
// XCD's L2), and within a run tiles go down groups of 8 row-tiles before
// moving to the next column-tile, so concurrently running workgroups share
// operand tiles.
#ifndef I8L_TILE_GRP
#define I8L_TILE_GRP 4
#endif
#ifndef I8L_TILE_XCD
#define I8L_TILE_XCD 1
#endif
__device__ __forceinline__ void tile_coords(int bid, int tiles_r, int tiles_c, int& tr, int& tc) {
  const int nt = tiles_r * tiles_c;
  int pid = bid;
  if (I8L_TILE_XCD) {
    const int x = bid & 7, i = bid >> 3;
    const int base = nt >> 3, rem = nt & 7;
    pid = x * base + (x < rem ? x : rem) + i;
  }
  constexpr int GRP = I8L_TILE_GRP;
  const int group = pid / (GRP * tiles_c);
  const int first = group * GRP;
  const int gsz = min(tiles_r - first, GRP);
  tr = first + (pid % (GRP * tiles_c)) % gsz;
  tc = (pid % (GRP * tiles_c)) / gsz;
}

// Output tiles of 256 x 256 16-bit values are staged in LDS (512 bytes per
// row) so that global stores cover whole rows: lanes holding four
// consecutive columns of 32 different rows write 8 bytes each into LDS, then
// each half-wave stores one 512-byte row. The 16-byte chunk c of row r sits at
// chunk position c ^ (r & 31), which spreads the 32 rows of one LDS write
// over all banks.
__device__ __forceinline__ int otile_off(int row, int chunk) { return row * 512 + 16 * (chunk ^ (row & 31)); }

// Store rows [32 w, 32 w + 32) of an LDS output tile (wave w of eight) to
// dst[(r0 + row) * ld + c0 + col], clipped to R rows and C columns.
template <typename T>
__device__ __forceinline__ void otile_store(const char* ot, T* __restrict__ dst, int64_t ld, int r0, int c0, int R,
                                            int C, int wave, int lane) {
  static_assert(sizeof(T) == 2, "16-bit outputs");
  const int ch = lane & 31;
  const int c = c0 + ch * 8;
  const bool vec = (ld % 8 == 0) && ((uintptr_t)dst % 16 == 0);
#pragma unroll 4
  for (int it = 0; it < 16; ++it) {
    const int row = 32 * wave + 2 * it + (lane >> 5);
    const int r = r0 + row;
    if (r >= R) continue;
    const v4u v = *reinterpret_cast<const v4u*>(ot + otile_off(row, ch));
    T* p = dst + (int64_t)r * ld + c;
    if (c + 8 <= C) {
      if (vec) {
        *reinterpret_cast<v4u*>(p) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[2 * e] = __builtin_bit_cast(T, (uint16_t)(v[e] & 0xffffu));
          p[2 * e + 1] = __builtin_bit_cast(T, (uint16_t)(v[e] >> 16));
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c + e < C) p[e] = __builtin_bit_cast(T, (uint16_t)(v[e >> 1] >> (16 * (e & 1))));
    }
  }
}

// Raises a kernel's dynamic-LDS limit once per device (the attribute is per
// device; the bit mask remembers devices 0..63 already set up).
inline hipError_t lds_limit_once(const void* kern, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Wave-wide reductions (wave64).
// Unsigned maximum over all 64 lanes (every lane active), returned to all
// lanes: DPP within rows of 16 (swap neighbours, swap pairs, mirror halves of
// 8, mirror halves of 16), then the four row results through scalar reads.
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xf, 0xf, false));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xf, 0xf, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xf, 0xf, false));  // row_mirror
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace i8l
