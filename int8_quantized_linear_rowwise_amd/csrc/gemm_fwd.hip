// Forward of the int8 linear layer on gfx950 matrix cores.
//
// bitsandbytes PR #33 "Memory efficient backward", review on _functions.py
// (dequantize, cast, add bias; "4. Mixed-precision decomposition matmul"):
//   y[m, n] = C32[m, n] * SCA[m] * SCB[n] / 127^2
//             + sum_j A16[m, O[j]] * Wdq[n, O[j]]     (fp16 x fp16 -> fp32)
//             + bias[n]
//   out = D(y)
// with C32 = CA . CB^T exact in int32, CA (M x K) and CB (N x K) both int8
// row-major (K contiguous), and Wdq[n, k] = fp16(CB[n, k] * (SCB[n] * (1/127)))
// rebuilt from the int8 weights (no fp16 weights are kept).
//
// One kernel: LDS-staged int8 tiles, double buffered through registers, fed
// to v_mfma_i32_32x32x32_i8; the int32 accumulators are dequantized in
// registers, the outlier product runs on v_mfma_f32_32x32x16_f16 into the
// same fp32 accumulators, then bias, cast and store. The product is computed
// as C^T (weights on the MFMA's row side) so that each lane owns four
// consecutive output features of one token and stores them as one vector.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace i8l {


// Fused epilogue shared by the forward kernels. A wave owns TI x TJ tiles of
// 32 x 32 (n x m); lane (lr, lg) holds, for tile (i, j) and register r,
//   n = nw + i*32 + (r/4)*8 + lg*4 + r%4,   m = mw + j*32 + lr.
//
// opan (optional): LDS panels of the first 16 outlier columns for a 256 x 256
// block tile with origin (tm0, tn0): P[n][16] = Wdq[n, O[j]] at opan, then
// Q[m][16] = A16[m, O[j]] at opan + OPAN_Q (fp16, 32 bytes per row, zero past
// the count); filled by the kernel before its k loop.
//
// With LDS_OUT (16-bit outputs, eight waves over a 256 x 256 block tile whose
// origin is (tm0, tn0)), the results are written to the LDS tile `ot` (row m,
// 16-byte chunk of 8 features) instead of global memory; the caller then
// stores whole rows with otile_store. The call starts with a block barrier.
constexpr int OPAN_Q = 256 * 32;      // Q panel after the 256 x 16 P panel
constexpr int OPAN_BYTES = 2 * 256 * 32;
// lsc (optional): the block tile's SCB[n0 + 0..255], SCA[m0 + 0..255] and
// fp32 bias[n0 + 0..255] in LDS (zero past the matrix), filled by the kernel
// before its k loop.
constexpr int LSC_SCB = 0, LSC_SCA = 256, LSC_BIAS = 512, LSC_BYTES = 768 * 4;

// fp16 bits of outlier value j of row m: the quantizer's staged copy for the
// first cap columns, beyond them the fp16 cast of A[m, idx[j]] read from the
// layer input itself (the same value, so any number of outlier columns is
// handled without a staging buffer of K columns).
template <int DT>
__device__ __forceinline__ uint16_t outlier_half(const uint16_t* __restrict__ subA, int cap,
                                                 const typename Elem<DT>::T* __restrict__ A, int K,
                                                 const int32_t* __restrict__ idx, int m, int j) {
  if (j < cap) return subA[(int64_t)m * cap + j];
  return __builtin_bit_cast(uint16_t, to_half<DT>(A[(int64_t)m * K + idx[j]]));
}

// Outlier values j0 .. j0 + 7 of activation row m as one fp16 operand (zero
// at and past cnt, or for a row outside the matrix): one 16-byte read of the
// staged copy when the staging rows are 16-byte aligned and hold all eight.
template <int DT>
__device__ __forceinline__ v8h outlier_a8(const uint16_t* __restrict__ subA, int cap,
                                          const typename Elem<DT>::T* __restrict__ A, int K,
                                          const int32_t* __restrict__ idx, int m, bool mok, int j0, int cnt) {
  v8h q;
  if (mok && (cap & 7) == 0 && j0 + 8 <= cap) {
    const v8h v = *reinterpret_cast<const v8h*>(subA + (int64_t)m * cap + j0);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = (j0 + e < cnt) ? v[e] : (_Float16)0.0f;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      q[e] = (mok && j0 + e < cnt) ? __builtin_bit_cast(_Float16, outlier_half<DT>(subA, cap, A, K, idx, m, j0 + e))
                                   : (_Float16)0.0f;
  }
  return q;
}

// Dequantized weight values Wdq[n, O[j]], j = j0 .. j0 + 7 (j0 % 8 == 0), as
// one fp16 operand (zero at and past cnt, or for a row outside the matrix):
// one 16-byte read of the slice the row quantizer wrote (wcap columns, a
// multiple of 8), beyond it fp16(CB[n, O[j]] * (SCB[n] * (1/127))) rebuilt
// from the int8 weights.
__device__ __forceinline__ v8h outlier_w8(const uint16_t* __restrict__ wsub, int wcap,
                                          const int8_t* __restrict__ CB, const float* __restrict__ SCB, int K,
                                          const int32_t* __restrict__ idx, int n, bool nok, int j0, int cnt) {
  v8h p;
  if (nok && j0 < wcap) {
    const v8h v = *reinterpret_cast<const v8h*>(wsub + (int64_t)n * wcap + j0);
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = (j0 + e < cnt) ? v[e] : (_Float16)0.0f;
  } else {
    const float sig = nok ? SCB[n] * (1.0f / 127.0f) : 0.0f;
    const int8_t* wrow = CB + (int64_t)(nok ? n : 0) * K;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      p[e] = (nok && j0 + e < cnt) ? half_of_f32((float)wrow[idx[j0 + e]] * sig) : (_Float16)0.0f;
  }
  return p;
}

// Staged outlier operands, 16-byte reads only (the row exists, j0 + 8 is
// within the staged width and the width is a multiple of 8): values j0 ..
// j0 + 7 of activation row m / weight row n, zero at and past cnt.
__device__ __forceinline__ v8h outlier_a8v(const uint16_t* __restrict__ subA, int cap, int m, int j0, int cnt) {
  const v8h v = *reinterpret_cast<const v8h*>(subA + (int64_t)m * cap + j0);
  v8h q;
#pragma unroll
  for (int e = 0; e < 8; ++e) q[e] = (j0 + e < cnt) ? v[e] : (_Float16)0.0f;
  return q;
}
__device__ __forceinline__ v8h outlier_w8v(const uint16_t* __restrict__ wsub, int wcap, int n, int j0, int cnt) {
  const v8h v = *reinterpret_cast<const v8h*>(wsub + (int64_t)n * wcap + j0);
  v8h p;
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = (j0 + e < cnt) ? v[e] : (_Float16)0.0f;
  return p;
}

template <int TI, int TJ, int DT, bool OV, bool LDS_OUT = false>
__device__ __forceinline__ void fwd_epilogue(v16i (&acc)[TI][TJ], int mw, int nw, int lr, int lg, int M, int N, int K,
                                             const float* __restrict__ SCA, const int8_t* __restrict__ CB,
                                             const float* __restrict__ SCB, const uint16_t* __restrict__ subA,
                                             int cap, const uint16_t* __restrict__ wsub, int wcap,
                                             const typename Elem<DT>::T* __restrict__ Asrc,
                                             const int32_t* __restrict__ idx,
                                             const int32_t* __restrict__ count,
                                             const typename Elem<DT>::T* __restrict__ bias,
                                             typename Elem<DT>::T* __restrict__ out, int32_t* __restrict__ c32,
                                             char* ot = nullptr, int tm0 = 0, int tn0 = 0,
                                             const char* opan = nullptr, const float* lsc = nullptr) {
  static_assert(!LDS_OUT || DT != DT_F32, "LDS output staging holds 16-bit values");
  if constexpr (LDS_OUT) __syncthreads();   // the operand stages are no longer read
  typedef typename Elem<DT>::T T;
  const int nb = nw + lg * 4;
  const int mb = mw + lr;

  if (c32 != nullptr) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int m = mb + j * 32;
        if (m >= M) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nb + i * 32 + q * 8;
          int32_t* p = c32 + (int64_t)m * N + n;
          if (OV && n + 3 < N) {
            *reinterpret_cast<v4i*>(p) = v4i{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                             acc[i][j][4 * q + 3]};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < N) p[e] = acc[i][j][4 * q + e];
          }
        }
      }
  }

  float sa[TJ];
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int m = mb + j * 32;
    if (lsc != nullptr) sa[j] = lsc[LSC_SCA + m - tm0];
    else sa[j] = (m < M) ? SCA[m] : 0.0f;
  }
  const int cnt = count != nullptr ? *count : 0;

  // outlier product operands of one step of 16 columns: P (weights, row
  // nw + i*32 + lr) and Q[j] (activations, row mw + j*32 + lr), columns
  // jo + lg*8 .. +7. Steps below jvec read both from the staged copies with
  // one 16-byte read each, requested a step ahead (across slabs too, so the
  // next slab's first step is in flight during its dequantization); later
  // steps gather their values one by one.
  const int jfirst = (opan != nullptr && cnt > 0) ? 16 : 0;
  const int jvec = min(cnt, min(wcap, (cap & 7) == 0 ? cap : 0) & ~15);
  v8h Pn, Qn[TJ];
  auto oload = [&](int i, int jo) {
    const int n = nw + i * 32 + lr;
    Pn = outlier_w8v(wsub, wcap, n < N ? n : 0, jo + lg * 8, cnt);
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int m = mw + j * 32 + lr;
      Qn[j] = outlier_a8v(subA, cap, m < M ? m : 0, jo + lg * 8, cnt);
    }
  };
  if (jfirst < jvec) oload(0, jfirst);

  // one slab of TJ tiles (32 output features) at a time keeps the fp32 copy small
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    float sb[16], bv[16];
    if (lsc != nullptr) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4f v = *reinterpret_cast<const v4f*>(lsc + LSC_SCB + nb - tn0 + i * 32 + q * 8);
        const v4f w = *reinterpret_cast<const v4f*>(lsc + LSC_BIAS + nb - tn0 + i * 32 + q * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sb[4 * q + e] = v[e];
          bv[4 * q + e] = w[e];
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = nb + i * 32 + (r >> 2) * 8 + (r & 3);
        sb[r] = (n < N) ? SCB[n] : 0.0f;
        bv[r] = (bias != nullptr && n < N) ? Elem<DT>::to_f32(bias[n]) : 0.0f;
      }
    }
    // C32 * (SCA * (SCB * fl32(1/127^2))) + bias in one fused multiply-add
    // (the bias joins the accumulator before the outlier product); the scale
    // product is exactly 1 when both scales are 127
#pragma unroll
    for (int r = 0; r < 16; ++r) sb[r] *= (1.0f / 16129.0f);
    v16f accf[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) accf[j][r] = __builtin_fmaf((float)acc[i][j][r], sa[j] * sb[r], bv[r]);

    // outlier columns: fp16 product accumulated into the same fp32 registers,
    // the first 16 columns from the LDS panels when the kernel staged them
    if (jfirst == 16) {
      const v8h P = *reinterpret_cast<const v8h*>(opan + (nw - tn0 + i * 32 + lr) * 32 + lg * 16);
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const v8h Q = *reinterpret_cast<const v8h*>(opan + OPAN_Q + (mw - tm0 + j * 32 + lr) * 32 + lg * 16);
        accf[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(P, Q, accf[j], 0, 0, 0);
      }
    }
    int jo = jfirst;
    for (; jo < jvec; jo += 16) {
      const v8h P = Pn;
      v8h Q[TJ];
#pragma unroll
      for (int j = 0; j < TJ; ++j) Q[j] = Qn[j];
      if (jo + 16 < jvec) oload(i, jo + 16);
      else if (i + 1 < TI) oload(i + 1, jfirst);
#pragma unroll
      for (int j = 0; j < TJ; ++j) accf[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(P, Q[j], accf[j], 0, 0, 0);
    }
    for (; jo < cnt; jo += 16) {
      const int n = nw + i * 32 + lr;
      const v8h P = outlier_w8(wsub, wcap, CB, SCB, K, idx, n, n < N, jo + lg * 8, cnt);
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int m = mw + j * 32 + lr;
        const v8h Q = outlier_a8<DT>(subA, cap, Asrc, K, idx, m, m < M, jo + lg * 8, cnt);
        accf[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(P, Q, accf[j], 0, 0, 0);
      }
    }

    // cast, store
    if constexpr (LDS_OUT) {
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int row = mb + j * 32 - tm0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int chunk = (nw - tn0 + i * 32 + q * 8) >> 3;
          v2u w;
#pragma unroll
          for (int e = 0; e < 2; ++e)
            w[e] = (uint32_t)__builtin_bit_cast(uint16_t, Elem<DT>::from_f32(accf[j][4 * q + 2 * e])) |
                   ((uint32_t)__builtin_bit_cast(uint16_t,
                                                 Elem<DT>::from_f32(accf[j][4 * q + 2 * e + 1]))
                    << 16);
          *reinterpret_cast<v2u*>(ot + otile_off(row, chunk) + 8 * lg) = w;
        }
      }
      continue;
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int m = mb + j * 32;
      if (m >= M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nb + i * 32 + q * 8;
        T* p = out + (int64_t)m * N + n;
        T v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = Elem<DT>::from_f32(accf[j][4 * q + e]);
        if (OV && n + 3 < N) {
          if constexpr (DT == DT_F32) {
            *reinterpret_cast<v4f*>(p) = v4f{v[0], v[1], v[2], v[3]};
          } else {
            v2u w;
            w[0] = (uint32_t)__builtin_bit_cast(uint16_t, v[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, v[1]) << 16);
            w[1] = (uint32_t)__builtin_bit_cast(uint16_t, v[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, v[3]) << 16);
            *reinterpret_cast<v2u*>(p) = w;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) p[e] = v[e];
        }
      }
    }
  }
}


template <int BM, int BN, int BK, int DT, bool KV, bool OV>
__global__ __launch_bounds__(256) void k_gemm_fwd(const int8_t* __restrict__ CA, const float* __restrict__ SCA,
                                                  int M, const int8_t* __restrict__ CB,
                                                  const float* __restrict__ SCB, int N, int K,
                                                  const uint16_t* __restrict__ subA, int cap,
                                                  const uint16_t* __restrict__ wsub, int wcap,
                                                  const typename Elem<DT>::T* __restrict__ Asrc,
                                                  const int32_t* __restrict__ idx,
                                                  const int32_t* __restrict__ count,
                                                  const typename Elem<DT>::T* __restrict__ bias,
                                                  typename Elem<DT>::T* __restrict__ out,
                                                  int32_t* __restrict__ c32) {
  typedef typename Elem<DT>::T T;
  constexpr int LDK = BK + 16;           // padded row pitch (bytes): conflict-free 16-byte reads
  constexpr int WN = BN / 2, WM = BM / 2;
  constexpr int TI = WN / 32, TJ = WM / 32;
  constexpr int CPR = BK / 16;           // 16-byte chunks per tile row
  constexpr int NCB = BN * CPR, NCA = BM * CPR;
  constexpr int CPT = (NCB + NCA) / 256; // chunks per thread per stage
  static_assert((NCB % 256) == 0 && (NCA % 256) == 0, "tile/thread mismatch");

  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  int8_t* sB = smem;                      // [2][BN][LDK]
  int8_t* sA = smem + 2 * BN * LDK;       // [2][BM][LDK]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const int wn = wave & 1, wm = wave >> 1;

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  v4i pre[CPT];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      const bool isB = c < NCB;
      const int cc = isB ? c : c - NCB;
      const int row = cc / CPR, col = (cc % CPR) * 16;
      const int grow = (isB ? n0 : m0) + row;
      const int lim = isB ? N : M;
      const int8_t* base = isB ? CB : CA;
      const int k = kt + col;
      v4i v = {0, 0, 0, 0};
      if (grow < lim) {
        const int8_t* p = base + (int64_t)grow * K + k;
        if constexpr (KV) {
          if (k < K) v = *reinterpret_cast<const v4i*>(p);
        } else {
          uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int b = 0; b < 16; ++b)
            if (k + b < K) w[b >> 2] |= ((uint32_t)(uint8_t)p[b]) << (8 * (b & 3));
          v = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
        }
      }
      pre[i] = v;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      const bool isB = c < NCB;
      const int cc = isB ? c : c - NCB;
      const int row = cc / CPR, col = (cc % CPR) * 16;
      int8_t* dst = (isB ? sB + buf * BN * LDK : sA + buf * BM * LDK) + row * LDK + col;
      *reinterpret_cast<v4i*>(dst) = pre[i];
    }
  };

  v16i acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v16i{};

  const int nk = (K + BK - 1) / BK;
  if (nk > 0) {
    gload(0);
    sstore(0);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const int8_t* bB = sB + cur * BN * LDK + (wn * WN + lr) * LDK + lg * 16;
    const int8_t* bA = sA + cur * BM * LDK + (wm * WM + lr) * LDK + lg * 16;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      v4i P[TI], Q[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) P[i] = *reinterpret_cast<const v4i*>(bB + i * 32 * LDK + ks * 32);
#pragma unroll
      for (int j = 0; j < TJ; ++j) Q[j] = *reinterpret_cast<const v4i*>(bA + j * 32 * LDK + ks * 32);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(P[i], Q[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  fwd_epilogue<TI, TJ, DT, OV>(acc, m0 + wm * WM, n0 + wn * WN, lr, lg, M, N, K, SCA, CB, SCB, subA, cap, wsub, wcap,
                               Asrc, idx, count, bias, out, c32);
}

// Large-tile forward kernel: 256 (m) x BN (n) output tile (BN = 256, or 128
// when 256-wide tiles would leave compute units idle), 8 waves (two per SIMD)
// of BN / 2 (n) x 64 (m), K stepped 128 bytes at a time through two swizzled
// LDS stages of (256 + BN) x 128 bytes. Registers hold the next step's tiles;
// each of the first two quarters of a step writes half of them to the other
// stage and reloads that half two steps ahead. Requires K % 16 == 0.
template <int DT, bool OV, int BN = 256>
__global__ __launch_bounds__(512, 1) void k_gemm_fwd_w8(const int8_t* __restrict__ CA,
                                                        const float* __restrict__ SCA, int M,
                                                        const int8_t* __restrict__ CB,
                                                        const float* __restrict__ SCB, int N, int K,
                                                        const uint16_t* __restrict__ subA, int cap,
                                                        const uint16_t* __restrict__ wsub, int wcap,
                                                        const typename Elem<DT>::T* __restrict__ Asrc,
                                                        const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ count,
                                                        const typename Elem<DT>::T* __restrict__ bias,
                                                        typename Elem<DT>::T* __restrict__ out,
                                                        int32_t* __restrict__ c32) {
  static_assert(BN == 256 || BN == 128, "256- or 128-wide tiles");
  constexpr int BM = 256, BK = 128, TI = BN / 64, TJ = 2;
  constexpr int NB = BN / 64;                  // register slots of the B tile
  constexpr int STAGE = (BM + BN) * BK;        // bytes per LDS stage
  constexpr int AOFF = BN * BK;                // A tile after the B tile
  constexpr int OT = 256 * 512;                // the LDS output tile (rows of 256 16-bit values)
  constexpr int BASE = 2 * STAGE > OT ? 2 * STAGE : OT;   // panels and scales after both
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lg = lane >> 5;
  const int wn = wave & 1, wm = wave >> 1;     // 2 (n) x 4 (m) waves

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const __amdgpu_buffer_rsrc_t rA = make_rsrc(CA + (int64_t)m0 * K, min(BM, M - m0) * K);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(CB + (int64_t)n0 * K, min(BN, N - n0) * K);

  // global -> register slots: chunk lc (16 bytes) of rows lrow + 64 i (i < NB
  // for the B tile, i < 4 for the A tile)
  const int lrow = tid >> 3, lc = tid & 7;
  const int voff = lrow * K + 16 * lc;
  const int woff = lrow * BK + 16 * (lc ^ lds_swz(lrow));
  const int sw = lds_swz(lr);
  int roff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) roff[ks] = lr * BK + 16 * ((2 * ks + lg) ^ sw);
  const int pb = wn * (BN / 2) * BK, qb = AOFF + wm * 64 * BK;

  v4u RB[NB], RA[4];
  // chunks past K (contraction tail) must read as zero: out of range
  auto load_b = [&](int kt) {
    const int v = (kt + 16 * lc < K) ? voff : OOB_OFFSET;
#pragma unroll
    for (int i = 0; i < NB; ++i)
      RB[i] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rB, v, kt + 64 * i * K, 0));
  };
  auto load_a = [&](int kt) {
    const int v = (kt + 16 * lc < K) ? voff : OOB_OFFSET;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      RA[i] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rA, v, kt + 64 * i * K, 0));
  };
  auto write_b = [&](int st) {
#pragma unroll
    for (int i = 0; i < NB; ++i) *reinterpret_cast<v4u*>(smem + st * STAGE + woff + i * 64 * BK) = RB[i];
  };
  auto write_a = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<v4u*>(smem + st * STAGE + AOFF + woff + i * 64 * BK) = RA[i];
  };

  v16i acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v16i{};

  v4i F[2][TI + TJ];
  auto fread = [&](int st, int ks, int b) {
    const int8_t* base = smem + st * STAGE + roff[ks];
#pragma unroll
    for (int i = 0; i < TI; ++i) F[b][i] = *reinterpret_cast<const v4i*>(base + pb + i * 32 * BK);
#pragma unroll
    for (int j = 0; j < TJ; ++j) F[b][TI + j] = *reinterpret_cast<const v4i*>(base + qb + j * 32 * BK);
  };
  auto mma = [&](int b) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(F[b][i], F[b][TI + j], acc[i][j], 0, 0, 0);
  };

  const int nk = (K + BK - 1) / BK;
  load_b(0);
  load_a(0);

  // outlier panels (first 16 outlier columns) for the epilogue, read while
  // the first operand tiles are in flight: thread t covers row t >> 1 of the
  // tile, columns 8 (t & 1) .. +7, of both panels
  char* opan = reinterpret_cast<char*>(smem) + BASE;
  int o16 = 0;
  if (count != nullptr) o16 = min(*count, 16);
  const int orow = tid >> 1, oj = (tid & 1) * 8;
  v8h opP = {}, opQ = {};
  if (o16 > 0) {
    const int n = n0 + orow, m = m0 + orow;
    opP = outlier_w8(wsub, wcap, CB, SCB, K, idx, n, (BN == 256 || orow < BN) && n < N, oj, o16);
    opQ = outlier_a8<DT>(subA, cap, Asrc, K, idx, m, m < M, oj, o16);
  }

  // the tile's scales and bias, likewise (thread t < 256: column n0 + t,
  // thread t >= 256: row m0 + t - 256)
  float* lsc = reinterpret_cast<float*>(opan + OPAN_BYTES);
  float sc0 = 0.0f, bias0 = 0.0f;
  if (tid < 256) {
    const int n = n0 + tid;
    if ((BN == 256 || tid < BN) && n < N) {
      sc0 = SCB[n];
      if (bias != nullptr) bias0 = Elem<DT>::to_f32(bias[n]);
    }
  } else {
    const int m = m0 + tid - 256;
    if (m < M) sc0 = SCA[m];
  }

  write_b(0);
  write_a(0);
  load_b(BK);
  load_a(BK);
  if (tid < 256) {
    lsc[LSC_SCB + tid] = sc0;
    lsc[LSC_BIAS + tid] = bias0;
  } else {
    lsc[LSC_SCA + tid - 256] = sc0;
  }
  if (o16 > 0) {
    *reinterpret_cast<v8h*>(opan + orow * 32 + oj * 2) = opP;
    *reinterpret_cast<v8h*>(opan + OPAN_Q + orow * 32 + oj * 2) = opQ;
  }
  __syncthreads();
  fread(0, 0, 0);
  // instruction interleave inside a phase: each MFMA paired with a fragment
  // read of the next phase and, in the first two phases, with an LDS tile
  // write and a global load
  auto groups_w = [&](auto nwr) {
    constexpr int W = decltype(nwr)::value;
    if constexpr (BN == 256) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        I8L_SGB(SG_MFMA, 1);
        I8L_SGB(SG_DS_R, 1);
        I8L_SGB(SG_DS_W, 1);
        I8L_SGB(SG_VMEM_R, 1);
      }
      I8L_SGB(SG_MFMA, 1);
      I8L_SGB(SG_DS_R, 2);
      I8L_SGB(SG_MFMA, 3);
    } else {
#pragma unroll
      for (int q = 0; q < W; ++q) {
        I8L_SGB(SG_MFMA, 1);
        I8L_SGB(SG_DS_R, 1);
        I8L_SGB(SG_DS_W, 1);
        I8L_SGB(SG_VMEM_R, 1);
      }
#pragma unroll
      for (int q = W; q < TI * TJ; ++q) {
        I8L_SGB(SG_MFMA, 1);
        I8L_SGB(SG_DS_R, 1);
      }
    }
  };
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    const int k2 = (kt + 2) * BK;    // past the end: zeros
    fread(st, 1, 1);
    write_b(st ^ 1);
    load_b(k2);
    mma(0);
    groups_w(std::integral_constant<int, NB>{});
    __builtin_amdgcn_sched_barrier(0);
    fread(st, 2, 0);
    write_a(st ^ 1);
    load_a(k2);
    mma(1);
    groups_w(std::integral_constant<int, 4>{});
    __builtin_amdgcn_sched_barrier(0);
    fread(st, 3, 1);
    mma(0);
    if constexpr (BN == 256) {
#pragma unroll
      for (int q = 0; q < 6; ++q) {
        I8L_SGB(SG_MFMA, 1);
        I8L_SGB(SG_DS_R, 1);
      }
      I8L_SGB(SG_MFMA, 2);
    } else {
#pragma unroll
      for (int q = 0; q < TI * TJ; ++q) {
        I8L_SGB(SG_MFMA, 1);
        I8L_SGB(SG_DS_R, 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    mma(1);
    __syncthreads();
    fread(st ^ 1, 0, 0);
  }

  const char* op = o16 > 0 ? opan : nullptr;
  if constexpr (DT == DT_F32) {
    fwd_epilogue<TI, TJ, DT, OV>(acc, m0 + wm * 64, n0 + wn * (BN / 2), lr, lg, M, N, K, SCA, CB, SCB, subA, cap,
                                 wsub, wcap, Asrc, idx, count, bias, out, c32, nullptr, m0, n0, op, lsc);
  } else {
    // output tile through LDS, stored as whole rows (of the tile's BN columns)
    char* ot = reinterpret_cast<char*>(smem);
    fwd_epilogue<TI, TJ, DT, OV, true>(acc, m0 + wm * 64, n0 + wn * (BN / 2), lr, lg, M, N, K, SCA, CB, SCB, subA,
                                       cap, wsub, wcap, Asrc, idx, count, bias, out, c32, ot, m0, n0, op, lsc);
    __syncthreads();
    otile_store<typename Elem<DT>::T>(ot, out, N, m0, n0, M, BN == 256 ? N : min(N, n0 + BN), wave, lane);
  }
}

template <int DT, bool OV, int BN>
static hipError_t launch_fwd_w8(const int8_t* CA, const float* SCA, int M, const int8_t* CB, const float* SCB,
                                int N, int K, const uint16_t* subA, int cap, const uint16_t* wsub, int wcap,
                                const void* A, const int32_t* idx,
                                const int32_t* count, const void* bias, void* out, int32_t* c32, hipStream_t st) {
  typedef typename Elem<DT>::T T;
  // both stages (or the output tile, if larger), panels, scales
  constexpr size_t stages = (size_t)2 * (256 + BN) * 128, otile = (size_t)256 * 512;
  constexpr size_t lds = (stages > otile ? stages : otile) + OPAN_BYTES + LSC_BYTES;
  auto kern = k_gemm_fwd_w8<DT, OV, BN>;
  static std::atomic<uint64_t> lds_set{0};
  {
    const hipError_t e = lds_limit_once((const void*)kern, (int)lds, lds_set);
    if (e != hipSuccess) return e;
  }
  const int tiles = ((M + 255) / 256) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3(tiles), dim3(512), lds, st, CA, SCA, M, CB, SCB, N, K, subA, cap, wsub, wcap,
                     static_cast<const T*>(A), idx, count, static_cast<const T*>(bias), static_cast<T*>(out), c32);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int DT, bool KV, bool OV>
static hipError_t launch_fwd_cfg(const int8_t* CA, const float* SCA, int M, const int8_t* CB, const float* SCB,
                                 int N, int K, const uint16_t* subA, int cap, const uint16_t* wsub, int wcap,
                                 const void* A, const int32_t* idx,
                                 const int32_t* count, const void* bias, void* out, int32_t* c32, hipStream_t st) {
  typedef typename Elem<DT>::T T;
  constexpr int LDK = BK + 16;
  constexpr size_t lds = (size_t)2 * (BM + BN) * LDK;
  auto kern = k_gemm_fwd<BM, BN, BK, DT, KV, OV>;
  static std::atomic<uint64_t> lds_set{0};
  {
    const hipError_t e = lds_limit_once((const void*)kern, (int)lds, lds_set);
    if (e != hipSuccess) return e;
  }
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3(tiles), dim3(256), lds, st, CA, SCA, M, CB, SCB, N, K, subA, cap, wsub, wcap,
                     static_cast<const T*>(A), idx, count, static_cast<const T*>(bias), static_cast<T*>(out), c32);
  return hipGetLastError();
}

int gemm_fwd_plan(int dt, int64_t M, int64_t N, int64_t K, bool aligned) {
  (void)dt;
  if (M <= 0 || N <= 0) return 0;
  if (aligned && K % 16 == 0) {
    const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
    // 64 to 128 tiles of 256 x 256 would fill at most half of the 256 compute
    // units: half-width tiles take about half the time each and fill them all
    if (big_tiles >= 64 && big_tiles <= 128) return 3;
    if (big_tiles > 128) return 2;
  }
  return 1;
}

template <int DT, bool KV, bool OV>
static hipError_t launch_fwd_dt(const int8_t* CA, const float* SCA, int M, const int8_t* CB, const float* SCB,
                                int N, int K, const uint16_t* subA, int cap, const uint16_t* wsub, int wcap,
                                const void* A, const int32_t* idx,
                                const int32_t* count, const void* bias, void* out, int32_t* c32, hipStream_t st) {
  const int plan = gemm_fwd_plan(DT, M, N, K, KV);
  if constexpr (KV) {
    if (plan == 3)
      return launch_fwd_w8<DT, OV, 128>(CA, SCA, M, CB, SCB, N, K, subA, cap, wsub, wcap, A, idx, count, bias, out,
                                        c32, st);
    if (plan == 2)
      return launch_fwd_w8<DT, OV, 256>(CA, SCA, M, CB, SCB, N, K, subA, cap, wsub, wcap, A, idx, count, bias, out,
                                        c32, st);
  }
  return launch_fwd_cfg<128, 128, 64, DT, KV, OV>(CA, SCA, M, CB, SCB, N, K, subA, cap, wsub, wcap, A, idx, count,
                                                  bias, out, c32, st);
}

hipError_t launch_gemm_fwd(int dt, const int8_t* CA, const float* SCA, int M, const int8_t* CB, const float* SCB,
                           int N, int K, const uint16_t* subA, int cap, const uint16_t* wsub, int wcap,
                           const void* Asrc, const int32_t* idx,
                           const int32_t* count, const void* bias, void* out, int32_t* c32, hipStream_t st) {
  const bool kv = (K % 16 == 0) && ((uintptr_t)CA % 16 == 0) && ((uintptr_t)CB % 16 == 0);
  const int osz = dt == DT_F32 ? 4 : 2;
  const bool ov = (N % 4 == 0) && ((uintptr_t)out % (4 * osz) == 0) && (c32 == nullptr || (uintptr_t)c32 % 16 == 0);
#define I8L_FWD(D, A, B) \
  return launch_fwd_dt<D, A, B>(CA, SCA, M, CB, SCB, N, K, subA, cap, wsub, wcap, Asrc, idx, count, bias, out, c32, st)
  switch (dt) {
    case DT_F32:
      if (kv) { if (ov) I8L_FWD(DT_F32, true, true); else I8L_FWD(DT_F32, true, false); }
      else { if (ov) I8L_FWD(DT_F32, false, true); else I8L_FWD(DT_F32, false, false); }
    case DT_F16:
      if (kv) { if (ov) I8L_FWD(DT_F16, true, true); else I8L_FWD(DT_F16, true, false); }
      else { if (ov) I8L_FWD(DT_F16, false, true); else I8L_FWD(DT_F16, false, false); }
    default:
      if (kv) { if (ov) I8L_FWD(DT_BF16, true, true); else I8L_FWD(DT_BF16, true, false); }
      else { if (ov) I8L_FWD(DT_BF16, false, true); else I8L_FWD(DT_BF16, false, false); }
  }
#undef I8L_FWD
}

}  // namespace i8l
