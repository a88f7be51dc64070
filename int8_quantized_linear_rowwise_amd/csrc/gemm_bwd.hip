// Memory-efficient backward of the int8 linear layer on gfx950 matrix cores.
//
// bitsandbytes PR #33 "Memory efficient backward", PR description and the
// review on the backward dequantization (CB cast, multiplied by
// SCB * (1/127)): the row-major int8 weights are turned into fp16 weights on
// the fly and multiplied with the fp16 output gradient; no fp16 weights are
// stored. The weight is frozen, so only the input gradient is produced:
//   grad_A[m, k] = D( sum_n fp16(G[m, n]) * Wdq[n, k] ),
//   Wdq[n, k]    = fp16( CB[n, k] * fl32(SCB[n] * fl32(1/127)) ).
// The contraction runs along the rows of CB (the strided direction), so each
// int8 tile of CB is dequantized once per workgroup while it is staged into
// LDS, transposed to n-contiguous fp16 rows that feed v_mfma_f32_32x32x16_f16
// directly. The output is computed transposed (weights on the MFMA's row side)
// so that each lane owns four consecutive k of one token.
//
// Author notes of the same PR: grad_bias comes from the un-cast gradient; it
// is a column sum of G in fp32, accumulated in a fixed order (deterministic).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace i8l {


template <int BM, int BK, int BNC, int DT, bool GV, bool WV, bool OV>
__global__ __launch_bounds__(256) void k_gemm_bwd(const typename Elem<DT>::T* __restrict__ G, int M, int N,
                                                  const int8_t* __restrict__ CB, const float* __restrict__ SCB,
                                                  int K, typename Elem<DT>::T* __restrict__ gA) {
  typedef typename Elem<DT>::T T;
  constexpr int LDN = BNC + 8;                 // halfs per LDS row (padded)
  constexpr int WK = BK / 2, WM = BM / 2;
  constexpr int TI = WK / 32, TJ = WM / 32;
  constexpr int GCPR = BNC / 8;                // 8-element chunks per G row
  constexpr int GCPT = BM * GCPR / 256;        // G chunks per thread
  constexpr int KQ = BK / 4;                   // 4-byte k quads per CB row of the tile
  constexpr int UPT = (BNC / 8) * KQ / 256;    // 8(n) x 4(k) CB units per thread
  static_assert(GCPT * 256 == BM * GCPR && UPT * 256 == (BNC / 8) * KQ, "tile/thread mismatch");

  extern __shared__ __attribute__((aligned(16))) _Float16 hsm[];
  _Float16* sW = hsm;                          // [2][BK][LDN]  (k rows, n contiguous)
  _Float16* sG = hsm + 2 * BK * LDN;           // [2][BM][LDN]  (m rows, n contiguous)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const int wk = wave & 1, wm = wave >> 1;

  const int tiles_m = (M + BM - 1) / BM, tiles_k = (K + BK - 1) / BK;
  int tm, tk;
  tile_coords(blockIdx.x, tiles_m, tiles_k, tm, tk);
  const int m0 = tm * BM, k0 = tk * BK;

  // prefetch registers (raw storage words: 4 per 8-element chunk for 16-bit
  // types, 8 for fp32)
  constexpr int GW = (DT == DT_F32) ? 8 : 4;
  uint32_t graw[GCPT][GW];
  uint32_t wraw[UPT][8];
  float wsig[UPT][8];

  auto gload = [&](int nc) {
#pragma unroll
    for (int i = 0; i < GCPT; ++i) {
      const int c = tid + 256 * i;
      const int row = c / GCPR, col = (c % GCPR) * 8;
      const int m = m0 + row, n = nc + col;
      const T* src = G + (int64_t)m * N + n;
      if (GV) {
        if (m < M && n < N) {
          if constexpr (DT == DT_F32) {
            v4u a = *reinterpret_cast<const v4u*>(src);
            v4u b = *reinterpret_cast<const v4u*>(src + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) { graw[i][e] = a[e]; graw[i][e + 4] = b[e]; }
          } else {
            v4u a = *reinterpret_cast<const v4u*>(src);
#pragma unroll
            for (int e = 0; e < 4; ++e) graw[i][e] = a[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < GW; ++e) graw[i][e] = 0u;
        }
      } else {
        if constexpr (DT == DT_F32) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            graw[i][e] = (m < M && n + e < N) ? __float_as_uint(src[e]) : 0u;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint32_t lo = (m < M && n + 2 * e < N) ? (uint32_t)__builtin_bit_cast(uint16_t, src[2 * e]) : 0u;
            uint32_t hi = (m < M && n + 2 * e + 1 < N) ? (uint32_t)__builtin_bit_cast(uint16_t, src[2 * e + 1]) : 0u;
            graw[i][e] = lo | (hi << 16);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int un = tid + 256 * u;
      const int kq = un % KQ, ng = un / KQ;
      const int k = k0 + 4 * kq;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int n = nc + 8 * ng + e;
        uint32_t w = 0u;
        float s = 0.0f;
        if (n < N) {
          s = SCB[n] * (1.0f / 127.0f);
          const int8_t* p = CB + (int64_t)n * K + k;
          if (WV) {
            if (k < K) w = *reinterpret_cast<const uint32_t*>(p);
          } else {
#pragma unroll
            for (int b = 0; b < 4; ++b)
              if (k + b < K) w |= ((uint32_t)(uint8_t)p[b]) << (8 * b);
          }
        }
        wraw[u][e] = w;
        wsig[u][e] = s;
      }
    }
  };
  auto sstore = [&](int buf) {
    _Float16* dG = sG + buf * BM * LDN;
#pragma unroll
    for (int i = 0; i < GCPT; ++i) {
      const int c = tid + 256 * i;
      const int row = c / GCPR, col = (c % GCPR) * 8;
      v8h h;
      if constexpr (DT == DT_F16) {
        h = __builtin_bit_cast(v8h, v4u{graw[i][0], graw[i][1], graw[i][2], graw[i][3]});
      } else if constexpr (DT == DT_BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          h[2 * e] = (_Float16)__uint_as_float(graw[i][e] << 16);
          h[2 * e + 1] = (_Float16)__uint_as_float(graw[i][e] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (_Float16)__uint_as_float(graw[i][e]);
      }
      *reinterpret_cast<v8h*>(dG + row * LDN + col) = h;
    }
    _Float16* dW = sW + buf * BK * LDN;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int un = tid + 256 * u;
      const int kq = un % KQ, ng = un / KQ;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        v8h h;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int b = (int)(int8_t)(wraw[u][e] >> (8 * c));
          h[e] = half_of_f32((float)b * wsig[u][e]);
        }
        *reinterpret_cast<v8h*>(dW + (4 * kq + c) * LDN + 8 * ng) = h;
      }
    }
  };

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v16f{};

  const int nn = (N + BNC - 1) / BNC;
  if (nn > 0) {
    gload(0);
    sstore(0);
    __syncthreads();
  }
  for (int t = 0; t < nn; ++t) {
    const int cur = t & 1;
    if (t + 1 < nn) gload((t + 1) * BNC);
    const _Float16* bW = sW + cur * BK * LDN + (wk * WK + lr) * LDN + lg * 8;
    const _Float16* bG = sG + cur * BM * LDN + (wm * WM + lr) * LDN + lg * 8;
#pragma unroll
    for (int ks = 0; ks < BNC / 16; ++ks) {
      v8h P[TI], Q[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) P[i] = *reinterpret_cast<const v8h*>(bW + i * 32 * LDN + ks * 16);
#pragma unroll
      for (int j = 0; j < TJ; ++j) Q[j] = *reinterpret_cast<const v8h*>(bG + j * 32 * LDN + ks * 16);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(P[i], Q[j], acc[i][j], 0, 0, 0);
    }
    if (t + 1 < nn) sstore(cur ^ 1);
    __syncthreads();
  }

  // lane (lr, lg), register r of tile (i, j):
  //   k = k0 + wk*WK + i*32 + (r/4)*8 + lg*4 + r%4,  m = m0 + wm*WM + j*32 + lr
  const int kb = k0 + wk * WK + lg * 4;
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int m = m0 + wm * WM + j * 32 + lr;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = kb + i * 32 + q * 8;
        T* p = gA + (int64_t)m * K + k;
        T v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = Elem<DT>::from_f32(acc[i][j][4 * q + e]);
        if (OV && k + 3 < K) {
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
            if (k + e < K) p[e] = v[e];
        }
      }
    }
  }
}

// Large-tile backward kernel for 16-bit gradients: 256 (m) x BK (k) output
// tile (BK = 256, or 128 when 256-wide tiles would leave compute units idle),
// 8 waves (two per SIMD, so that one wave's MFMAs run while the other waits)
// of BK / 2 (k) x 64 (m), the contraction over n stepped 64 at a time through
// two swizzled LDS stages (W^T tile: BK k-rows x 64 n, G tile: 256 m-rows x
// 64 n, both fp16). The next stage's int8 weights and gradient come in
// through buffer loads two steps ahead and are dequantized / cast and written
// to the other LDS stage in the first phases of a step, between the MFMAs.
// Requires N % 8 == 0 and K % 4 == 0.
template <int DT, bool OV, int BK = 256>
__global__ __launch_bounds__(512, 1) void k_gemm_bwd_w8(const typename Elem<DT>::T* __restrict__ G, int M, int N,
                                                        const int8_t* __restrict__ CB,
                                                        const float* __restrict__ SCB, int K,
                                                        typename Elem<DT>::T* __restrict__ gA) {
  static_assert(DT == DT_F16 || DT == DT_BF16, "16-bit gradients only");
  static_assert(BK == 256 || BK == 128, "256- or 128-wide tiles");
  constexpr int BM = 256, BNC = 64, TI = BK / 64, TJ = 2;
  // weight rows per lane: 8 (all 64 lanes on 4 k-bytes of each of the wave's
  // 8 rows), or 4 with 128-wide tiles (half-waves on rows 0-3 and 4-7)
  constexpr int WR = BK / 32;
  constexpr int ROW = BNC * 2;                 // bytes per LDS row
  constexpr int STAGE = (BK + BM) * ROW;       // 64 KB
  constexpr int GOFF = BK * ROW;               // G tile after the W^T tile
  extern __shared__ __attribute__((aligned(16))) char bsm[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lg = lane >> 5;
  const int wk = wave & 1, wm = wave >> 1;     // 2 (k) x 4 (m) waves

  const int tiles_m = (M + BM - 1) / BM, tiles_k = (K + BK - 1) / BK;
  int tm, tk;
  tile_coords(blockIdx.x, tiles_m, tiles_k, tm, tk);
  const int m0 = tm * BM, k0 = tk * BK;

  const __amdgpu_buffer_rsrc_t rG = make_rsrc(G + (int64_t)m0 * N, min(BM, M - m0) * N * 2);
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(CB + k0, max(0, N * K - k0));
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(SCB, N * 4);

  // G slots: 16-byte chunk gc of rows grow + 64 i (i < 4)
  const int grow = tid >> 3, gc = tid & 7;
  const int gvoff = grow * N * 2 + 16 * gc;
  const int gwoff = GOFF + grow * ROW + 16 * (gc ^ lds_swz(grow));
  // W unit: rows n8 + wh .. n8 + wh + WR - 1 with n8 = nc + 8*wave (wave-uniform),
  // bytes 4kq .. 4kq+3; the 16-byte LDS chunk of the wave's 8 rows is
  // written whole, or as two 8-byte halves
  const int kq = BK == 256 ? (tid & 63) : (tid & 31);
  const int wh = BK == 256 ? 0 : 4 * ((tid >> 5) & 1);
  const int wvoff = 4 * kq + wh * K;
  int wwoff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int r = 4 * kq + c;
    wwoff[c] = r * ROW + 16 * (wave ^ lds_swz(r)) + 2 * wh;
  }
  const int sw = lds_swz(lr);
  int roff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) roff[ks] = lr * ROW + 16 * ((2 * ks + lg) ^ sw);
  const int pb = wk * (BK / 2) * ROW, qb = GOFF + wm * 64 * ROW;

  v4u RG[4];
  uint32_t RW[WR];
  float SG[WR];

  auto load_w = [&](int nc) {
    const int n8 = nc + 8 * wave;
#pragma unroll
    for (int e = 0; e < WR; ++e) RW[e] = __builtin_amdgcn_raw_buffer_load_b32(rW, wvoff, (n8 + e) * K, 0);
    // N % 8 == 0: the eight rows from n8 are all in the matrix or all past it
    const int so = (n8 < N) ? 4 * (n8 + wh) : OOB_OFFSET;
#pragma unroll
    for (int h = 0; h < WR / 4; ++h) {
      const v4f sv = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rS, so + 16 * h, 0, 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) SG[4 * h + e] = sv[e];
    }
  };
  auto load_g = [&](int nc) {
    const int gv = (nc + 8 * gc < N) ? gvoff : OOB_OFFSET;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      RG[i] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rG, gv, 2 * nc + 128 * i * N, 0));
  };
  auto write_w = [&](int st, int c0) {
    float sg[WR];
#pragma unroll
    for (int e = 0; e < WR; ++e) sg[e] = SG[e] * (1.0f / 127.0f);
#pragma unroll
    for (int c = c0; c < c0 + 2; ++c) {
      uint32_t h[WR / 2];
#pragma unroll
      for (int e = 0; e < WR / 2; ++e) {
        const float w0 = (float)(int)(int8_t)(RW[2 * e] >> (8 * c));
        const float w1 = (float)(int)(int8_t)(RW[2 * e + 1] >> (8 * c));
        h[e] = f32x2_to_f16x2(w0 * sg[2 * e], w1 * sg[2 * e + 1]);
      }
      if constexpr (WR == 8) *reinterpret_cast<v4u*>(bsm + st * STAGE + wwoff[c]) = v4u{h[0], h[1], h[2], h[3]};
      else *reinterpret_cast<v2u*>(bsm + st * STAGE + wwoff[c]) = v2u{h[0], h[1]};
    }
  };
  auto write_g = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v4u v;
      if constexpr (DT == DT_F16) {
        v = RG[i];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = bf16x2_to_f16x2(RG[i][e]);
      }
      *reinterpret_cast<v4u*>(bsm + st * STAGE + gwoff + i * 64 * ROW) = v;
    }
  };

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v16f{};

  v8h F[2][TI + TJ];
  auto fread = [&](int st, int ks, int b) {
    const char* base = bsm + st * STAGE + roff[ks];
#pragma unroll
    for (int i = 0; i < TI; ++i) F[b][i] = *reinterpret_cast<const v8h*>(base + pb + i * 32 * ROW);
#pragma unroll
    for (int j = 0; j < TJ; ++j) F[b][TI + j] = *reinterpret_cast<const v8h*>(base + qb + j * 32 * ROW);
  };
  auto mma = [&](int b) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(F[b][i], F[b][TI + j], acc[i][j], 0, 0, 0);
  };

  const int nn = (N + BNC - 1) / BNC;
  load_w(0);
  load_g(0);
  write_w(0, 0);
  write_w(0, 2);
  write_g(0);
  load_w(BNC);
  load_g(BNC);
  __syncthreads();
  fread(0, 0, 0);
  // phases of one k step
  // Each MFMA of a phase is followed by four vector ALU instructions of the
  // phase's conversions (the weight dequantization, the gradient cast), then
  // by its share of the fragment reads, tile writes and global loads, so that
  // the conversions issue while the matrix core works instead of in runs
  // between MFMA groups. Measured in one process (bit-identical results):
  // 4 per MFMA is 5-8 % faster than the compiler's own order at 4096 x 4096
  // and at a contraction or output of 11008; 5 per MFMA is slower than no
  // grouping, 2-3 faster but less so.
  constexpr int VPM = 4;
  auto spread = [&](auto dsr, auto dsw, auto vm) {
    constexpr int R = decltype(dsr)::value, Wr = decltype(dsw)::value, G = decltype(vm)::value;
#pragma unroll
    for (int q = 0; q < TI * TJ; ++q) {
      I8L_SGB(SG_MFMA, 1);
      I8L_SGB(SG_VALU, VPM);
      if (q < R) I8L_SGB(SG_DS_R, 1);
      if (q < Wr) I8L_SGB(SG_DS_W, 1);
      if (q < G) I8L_SGB(SG_VMEM_R, 1);
    }
  };
  for (int t = 0; t < nn; ++t) {
    const int st = t & 1;
    const int nc2 = (t + 2) * BNC;   // past the end: zeros
    fread(st, 1, 1);
    write_w(st ^ 1, 0);
    mma(0);
    spread(std::integral_constant<int, TI + TJ>{}, std::integral_constant<int, 2>{},
           std::integral_constant<int, 0>{});
    __builtin_amdgcn_sched_barrier(0);
    fread(st, 2, 0);
    write_w(st ^ 1, 2);
    load_w(nc2);
    mma(1);
    spread(std::integral_constant<int, TI + TJ>{}, std::integral_constant<int, 2>{},
           std::integral_constant<int, WR + WR / 4>{});
    __builtin_amdgcn_sched_barrier(0);
    fread(st, 3, 1);
    write_g(st ^ 1);
    load_g(nc2);
    mma(0);
    spread(std::integral_constant<int, TI + TJ>{}, std::integral_constant<int, 4>{},
           std::integral_constant<int, 4>{});
    __builtin_amdgcn_sched_barrier(0);
    mma(1);
    __syncthreads();
    fread(st ^ 1, 0, 0);
  }

  // lane (lr, lg), register r of tile (i, j):
  //   k = k0 + wk*BK/2 + i*32 + (r/4)*8 + lg*4 + r%4,  m = m0 + wm*64 + j*32 + lr
  // The tile goes through LDS (row m, 16-byte chunk of 8 k) and leaves as
  // whole rows.
  typedef typename Elem<DT>::T T;
  __syncthreads();   // every wave is done with the operand stages
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int row = wm * 64 + j * 32 + lr;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v2u w;
#pragma unroll
        for (int e = 0; e < 2; ++e)
          w[e] = (uint32_t)__builtin_bit_cast(uint16_t, Elem<DT>::from_f32(acc[i][j][4 * q + 2 * e])) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, Elem<DT>::from_f32(acc[i][j][4 * q + 2 * e + 1])) << 16);
        *reinterpret_cast<v2u*>(bsm + otile_off(row, wk * (BK / 16) + i * 4 + q) + 8 * lg) = w;
      }
    }
  }
  __syncthreads();
  otile_store<T>(bsm, gA, K, m0, k0, M, BK == 256 ? K : min(K, k0 + BK), wave, lane);
}

template <int DT, bool OV, int BK>
static hipError_t launch_bwd_w8(const void* G, int M, int N, const int8_t* CB, const float* SCB, int K, void* gA,
                                hipStream_t st) {
  typedef typename Elem<DT>::T T;
  // both stages, or the output tile (256 rows of 512 bytes) if larger
  constexpr size_t stages = (size_t)2 * (BK + 256) * 128, otile = (size_t)256 * 512;
  constexpr size_t lds = stages > otile ? stages : otile;
  auto kern = k_gemm_bwd_w8<DT, OV, BK>;
  static std::atomic<uint64_t> lds_set{0};
  {
    const hipError_t e = lds_limit_once((const void*)kern, (int)lds, lds_set);
    if (e != hipSuccess) return e;
  }
  const int tiles = ((M + 255) / 256) * ((K + BK - 1) / BK);
  hipLaunchKernelGGL(kern, dim3(tiles), dim3(512), lds, st, static_cast<const T*>(G), M, N, CB, SCB, K,
                     static_cast<T*>(gA));
  return hipGetLastError();
}

template <int BM, int BK, int BNC, int DT, bool GV, bool WV, bool OV>
static hipError_t launch_bwd_cfg(const void* G, int M, int N, const int8_t* CB, const float* SCB, int K, void* gA,
                                 hipStream_t st) {
  typedef typename Elem<DT>::T T;
  constexpr int LDN = BNC + 8;
  constexpr size_t lds = (size_t)2 * (BK + BM) * LDN * sizeof(_Float16);
  auto kern = k_gemm_bwd<BM, BK, BNC, DT, GV, WV, OV>;
  static std::atomic<uint64_t> lds_set{0};
  {
    const hipError_t e = lds_limit_once((const void*)kern, (int)lds, lds_set);
    if (e != hipSuccess) return e;
  }
  const int tiles = ((M + BM - 1) / BM) * ((K + BK - 1) / BK);
  hipLaunchKernelGGL(kern, dim3(tiles), dim3(256), lds, st, static_cast<const T*>(G), M, N, CB, SCB, K,
                     static_cast<T*>(gA));
  return hipGetLastError();
}

template <int DT, bool GV, bool WV, bool OV>
static hipError_t launch_bwd_dt(const void* G, int M, int N, const int8_t* CB, const float* SCB, int K, void* gA,
                                hipStream_t st) {
  return launch_bwd_cfg<128, 128, 64, DT, GV, WV, OV>(G, M, N, CB, SCB, K, gA, st);
}

// The large-tile kernel needs 16-bit gradients, N % 8 == 0, K % 4 == 0, a
// contraction (N > 0: its prologue reads two weight steps unconditionally)
// and operands its 32-bit buffer offsets can address.
int gemm_bwd_plan(int dt, int64_t M, int64_t N, int64_t K, bool aligned) {
  if (M <= 0 || K <= 0) return 0;
  const bool fits = (N + 128) * K < ((int64_t)1 << 31) - 4096 && N * 2 * 256 < ((int64_t)1 << 31) - 4096;
  const int64_t big_tiles = ((M + 255) / 256) * ((K + 255) / 256);
  if (dt != DT_F32 && aligned && N > 0 && N % 8 == 0 && K % 4 == 0 && fits && big_tiles >= 64) {
    // 64 to 128 tiles of 256 x 256 would fill at most half of the 256 compute
    // units: half-width tiles take about half the time each and fill them all
    return big_tiles <= 128 ? 3 : 2;
  }
  return 1;
}

hipError_t launch_gemm_bwd(int dt, const void* G, int M, int N, const int8_t* CB, const float* SCB, int K,
                           void* gA, hipStream_t st) {
  const int esz = dt == DT_F32 ? 4 : 2;
  const bool gv = (N % 8 == 0) && ((uintptr_t)G % 16 == 0);
  const bool wv = (K % 4 == 0) && ((uintptr_t)CB % 4 == 0);
  const bool ov = (K % 4 == 0) && ((uintptr_t)gA % (4 * esz) == 0);
  const int plan = gemm_bwd_plan(dt, M, N, K, gv && wv && ov);
  if (plan == 3) {
    if (dt == DT_F16) return launch_bwd_w8<DT_F16, true, 128>(G, M, N, CB, SCB, K, gA, st);
    return launch_bwd_w8<DT_BF16, true, 128>(G, M, N, CB, SCB, K, gA, st);
  }
  if (plan == 2) {
    if (dt == DT_F16) return launch_bwd_w8<DT_F16, true, 256>(G, M, N, CB, SCB, K, gA, st);
    return launch_bwd_w8<DT_BF16, true, 256>(G, M, N, CB, SCB, K, gA, st);
  }
#define I8L_BWD(D)                                                                   \
  do {                                                                               \
    if (gv && wv && ov) return launch_bwd_dt<D, true, true, true>(G, M, N, CB, SCB, K, gA, st); \
    return launch_bwd_dt<D, false, false, false>(G, M, N, CB, SCB, K, gA, st);      \
  } while (0)
  switch (dt) {
    case DT_F32: I8L_BWD(DT_F32);
    case DT_F16: I8L_BWD(DT_F16);
    default: I8L_BWD(DT_BF16);
  }
#undef I8L_BWD
}

// ---------------------------------------------------------------------------
// grad_bias: column sums of the un-cast gradient.

constexpr int GB_ROWS = 128;   // rows per partial

template <int DT>
__global__ __launch_bounds__(256) void k_colsum_partial(const typename Elem<DT>::T* __restrict__ G, int M, int N,
                                                        float* __restrict__ partial) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const int r0 = blockIdx.y * GB_ROWS;
  const int r1 = min(M, r0 + GB_ROWS);
  float s = 0.0f;
  for (int r = r0; r < r1; ++r) s += Elem<DT>::to_f32(G[(int64_t)r * N + n]);
  partial[(int64_t)blockIdx.y * N + n] = s;
}

template <int DT>
__global__ __launch_bounds__(256) void k_colsum_final(const float* __restrict__ partial, int nparts, int N,
                                                      typename Elem<DT>::T* __restrict__ gb) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  float s = 0.0f;
  for (int p = 0; p < nparts; ++p) s += partial[(int64_t)p * N + n];
  gb[n] = Elem<DT>::from_f32(s);
}

size_t grad_bias_partial_floats(int M, int N) {
  const int64_t parts = (M + GB_ROWS - 1) / GB_ROWS;
  return (size_t)(parts < 1 ? 1 : parts) * (size_t)(N < 1 ? 1 : N);
}

template <int DT>
static hipError_t launch_gb_t(const void* G, int M, int N, float* partial, void* gb, hipStream_t st) {
  typedef typename Elem<DT>::T T;
  if (N <= 0) return hipSuccess;
  const int parts = (M + GB_ROWS - 1) / GB_ROWS;
  if (parts > 0)
    hipLaunchKernelGGL(k_colsum_partial<DT>, dim3((N + 255) / 256, parts), dim3(256), 0, st,
                       static_cast<const T*>(G), M, N, partial);
  hipLaunchKernelGGL(k_colsum_final<DT>, dim3((N + 255) / 256), dim3(256), 0, st, partial, parts, N,
                     static_cast<T*>(gb));
  return hipGetLastError();
}

hipError_t launch_grad_bias(int dt, const void* G, int M, int N, float* partial, void* gb, hipStream_t st) {
  switch (dt) {
    case DT_F32: return launch_gb_t<DT_F32>(G, M, N, partial, gb, st);
    case DT_F16: return launch_gb_t<DT_F16>(G, M, N, partial, gb, st);
    default: return launch_gb_t<DT_BF16>(G, M, N, partial, gb, st);
  }
}

}  // namespace i8l
