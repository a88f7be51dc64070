// Weight gradient of the trainable-weight mode of the int8 linear layer.
//
// bitsandbytes PR #33 "Memory efficient backward" names a has_fp16_weights
// option beside the memory-efficient one: the weight stays a trainable fp16
// tensor that is re-quantized on each forward. Its gradient is the fp16 weight
// gradient of y = A16 W^T:
//   grad_W[n, k] = D( sum_m fp16(G[m, n]) * fp16(A[m, k]) ),
// accumulated in fp32 on v_mfma_f32_32x32x16_f16 and rounded once.
//
// The contraction runs over the token rows of both G (M x N) and A (M x K),
// the strided direction of both. Tiles of 64 rows are staged in LDS as they
// lie in memory (fp16, 512-byte rows) and the MFMA operands are read
// transposed with ds_read_b64_tr_b16, which hands each lane four
// consecutive rows of one column.
#include "common.hpp"
#include "kernels.hpp"

namespace i8l {

typedef short v4s __attribute__((ext_vector_type(4)));
#define I8L_LDS(p) ((__attribute__((address_space(3))) v4s*)(p))

// 256 (n) x 256 (k) output tile, 8 waves of 64 (n) x 128 (k), the contraction
// over m stepped 64 rows at a time through two LDS stages of 64 KB (A tile
// then G tile, 64 rows x 256 fp16 each). Requires 16-bit D, N % 8 == 0 and
// K % 8 == 0, M >= 1.
template <int DT>
__global__ __launch_bounds__(512, 1) void k_gemm_wgrad(const typename Elem<DT>::T* __restrict__ G,
                                                       const typename Elem<DT>::T* __restrict__ A, int M, int N,
                                                       int K, typename Elem<DT>::T* __restrict__ gW) {
  static_assert(DT == DT_F16 || DT == DT_BF16, "16-bit inputs only");
  constexpr int BN = 256, BK = 256, BMC = 64, TI = 4, TJ = 2;
  constexpr int ROWB = 512;                    // bytes per LDS row (256 fp16)
  constexpr int GOFF = BMC * ROWB;             // G tile after the A tile
  constexpr int STAGE = 2 * BMC * ROWB;        // 64 KB
  extern __shared__ __attribute__((aligned(16))) char wsm[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lg = lane >> 5;
  const int wk = wave & 1, wn = wave >> 1;     // 2 (k) x 4 (n) waves

  const int tiles_n = (N + BN - 1) / BN, tiles_k = (K + BK - 1) / BK;
  int tn, tk;
  tile_coords(blockIdx.x, tiles_n, tiles_k, tn, tk);
  const int n0 = tn * BN, k0 = tk * BK;

  // Rows m >= M lie past the end of both buffers and read as zero; columns
  // past N or K read the next row's values and only reach output rows n >= N
  // or columns k >= K, which are never stored.
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(A + k0, M * K * 2 - 2 * k0);
  const __amdgpu_buffer_rsrc_t rG = make_rsrc(G + n0, M * N * 2 - 2 * n0);

  // staging slot: row (tid >> 5) + 16 p of the chunk, 16-byte piece tid & 31;
  // piece c of LDS row m sits at position c ^ (4 (m & 3))
  const int srow = tid >> 5, sc = tid & 31;
  const int avoff = srow * K * 2 + 16 * sc, gvoff = srow * N * 2 + 16 * sc;
  const int woff = srow * ROWB + 16 * (sc ^ ((srow & 3) << 2));

  // transposed operand reads: lane group g = lane / 16 of the 64 lanes, lane
  // i16 within it; block b of 32 columns, rows m = 16 ks + 8 (g / 2) + 4 h + i16 / 4
  const int g = lane >> 4, i16 = lane & 15;
  const int sw = (i16 >> 2) << 2;
  auto tr_off = [&](int b) {
    const int c = 4 * b + 2 * (g & 1) + ((i16 & 3) >> 1);
    return (8 * (g >> 1) + (i16 >> 2)) * ROWB + 16 * (c ^ sw) + 8 * (i16 & 1);
  };
  int poff[TI], qoff[TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i) poff[i] = tr_off(wk * 4 + i);
#pragma unroll
  for (int j = 0; j < TJ; ++j) qoff[j] = GOFF + tr_off(wn * 2 + j);

  v4u RA[4], RG[4];
  // halves h = 0, 1 of the staging slots (row chunks p = 2h, 2h + 1)
  auto load_a = [&](int mc, int h) {
#pragma unroll
    for (int p = 2 * h; p < 2 * h + 2; ++p)
      RA[p] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rA, avoff, (mc + 16 * p) * K * 2, 0));
  };
  auto load_g = [&](int mc, int h) {
#pragma unroll
    for (int p = 2 * h; p < 2 * h + 2; ++p)
      RG[p] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rG, gvoff, (mc + 16 * p) * N * 2, 0));
  };
  auto to_f16 = [&](v4u v) {
    if constexpr (DT == DT_BF16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = bf16x2_to_f16x2(v[e]);
    }
    return v;
  };
  auto write_a = [&](int st, int h) {
#pragma unroll
    for (int p = 2 * h; p < 2 * h + 2; ++p) *reinterpret_cast<v4u*>(wsm + st * STAGE + woff + p * 16 * ROWB) = to_f16(RA[p]);
  };
  auto write_g = [&](int st, int h) {
#pragma unroll
    for (int p = 2 * h; p < 2 * h + 2; ++p)
      *reinterpret_cast<v4u*>(wsm + st * STAGE + GOFF + woff + p * 16 * ROWB) = to_f16(RG[p]);
  };

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v16f{};

  v8h F[2][TI + TJ];
  // rows m .. m+3 (elements 0-3) and m+4 .. m+7 (elements 4-7) of the lane's column
  auto frag = [&](const char* p) {
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(I8L_LDS(p));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(I8L_LDS(p + 4 * ROWB));
    return __builtin_bit_cast(v8h, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto fread = [&](int st, int ks, int b) {
    const char* base = wsm + st * STAGE + ks * 16 * ROWB;
#pragma unroll
    for (int i = 0; i < TI; ++i) F[b][i] = frag(base + poff[i]);
#pragma unroll
    for (int j = 0; j < TJ; ++j) F[b][TI + j] = frag(base + qoff[j]);
  };
  auto mma = [&](int b) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(F[b][i], F[b][TI + j], acc[i][j], 0, 0, 0);
  };

  const int nn = (M + BMC - 1) / BMC;
  for (int h = 0; h < 2; ++h) {
    load_a(0, h);
    load_g(0, h);
  }
  for (int h = 0; h < 2; ++h) {
    write_a(0, h);
    write_g(0, h);
  }
  for (int h = 0; h < 2; ++h) {
    load_a(BMC, h);
    load_g(BMC, h);
  }
  __syncthreads();
  fread(0, 0, 0);
  // each phase of a step writes a quarter of the next stage: LDS writes run at
  // about a third of the read rate, and spread evenly they cost less (2 %)
  for (int t = 0; t < nn; ++t) {
    const int st = t & 1;
    const int mc2 = (t + 2) * BMC;   // past the end: zeros
    fread(st, 1, 1);
    write_a(st ^ 1, 0);
    load_a(mc2, 0);
    mma(0);
    __builtin_amdgcn_sched_barrier(0);
    fread(st, 2, 0);
    write_a(st ^ 1, 1);
    load_a(mc2, 1);
    mma(1);
    __builtin_amdgcn_sched_barrier(0);
    fread(st, 3, 1);
    write_g(st ^ 1, 0);
    load_g(mc2, 0);
    mma(0);
    __builtin_amdgcn_sched_barrier(0);
    write_g(st ^ 1, 1);
    load_g(mc2, 1);
    mma(1);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    fread(st ^ 1, 0, 0);
  }

  // lane (lr, lg), register r of tile (i, j):
  //   k = k0 + wk*128 + i*32 + (r/4)*8 + lg*4 + r%4,  n = n0 + wn*64 + j*32 + lr
  // The tile goes through LDS (row n, 16-byte chunk of 8 k) and leaves as whole rows.
  typedef typename Elem<DT>::T T;
  __syncthreads();   // every wave is done with the operand stages
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int row = wn * 64 + j * 32 + lr;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v2u w;
#pragma unroll
        for (int e = 0; e < 2; ++e)
          w[e] = (uint32_t)__builtin_bit_cast(uint16_t, Elem<DT>::from_f32(acc[i][j][4 * q + 2 * e])) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, Elem<DT>::from_f32(acc[i][j][4 * q + 2 * e + 1])) << 16);
        *reinterpret_cast<v2u*>(wsm + otile_off(row, wk * 16 + i * 4 + q) + 8 * lg) = w;
      }
    }
  }
  __syncthreads();
  otile_store<T>(wsm, gW, K, n0, k0, N, K, wave, lane);
}

// Any dtype and shape: 64 (n) x 64 (k) output tile, 256 threads of 4 x 4
// outputs, the fp16-cast operands staged 32 rows at a time as fp32 (the
// products of two fp16 values are exact in fp32), fp32 fused multiply-adds.
template <int DT>
__global__ __launch_bounds__(256) void k_wgrad_small(const typename Elem<DT>::T* __restrict__ G,
                                                     const typename Elem<DT>::T* __restrict__ A, int M, int N,
                                                     int K, typename Elem<DT>::T* __restrict__ gW) {
  __shared__ float sG[32][65];
  __shared__ float sA[32][65];
  const int tid = threadIdx.x;
  const int n0 = blockIdx.y * 64, k0 = blockIdx.x * 64;
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int mc = 0; mc < M; mc += 32) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int idx = tid + 256 * e, r = idx >> 6, c = idx & 63, m = mc + r;
      sG[r][c] = (m < M && n0 + c < N) ? half_cast_f32<DT>(G[(int64_t)m * N + n0 + c]) : 0.0f;
      sA[r][c] = (m < M && k0 + c < K) ? half_cast_f32<DT>(A[(int64_t)m * K + k0 + c]) : 0.0f;
    }
    __syncthreads();
#pragma unroll 4
    for (int r = 0; r < 32; ++r) {
      float a[4], gg[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = sA[r][4 * tx + u];
        gg[u] = sG[r][4 * ty + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = __builtin_fmaf(gg[u], a[v], acc[u][v]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int n = n0 + 4 * ty + u;
    if (n >= N) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int k = k0 + 4 * tx + v;
      if (k < K) gW[(int64_t)n * K + k] = Elem<DT>::from_f32(acc[u][v]);
    }
  }
}

template <int DT>
static hipError_t launch_wgrad_big(const void* G, const void* A, int M, int N, int K, void* gW, hipStream_t st) {
  typedef typename Elem<DT>::T T;
  constexpr size_t lds = (size_t)2 * 2 * 64 * 512;   // also holds the 256 x 512-byte output tile
  auto kern = k_gemm_wgrad<DT>;
  static std::atomic<uint64_t> lds_set{0};
  {
    const hipError_t e = lds_limit_once((const void*)kern, (int)lds, lds_set);
    if (e != hipSuccess) return e;
  }
  const int tiles = ((N + 255) / 256) * ((K + 255) / 256);
  hipLaunchKernelGGL(kern, dim3(tiles), dim3(512), lds, st, static_cast<const T*>(G), static_cast<const T*>(A), M, N,
                     K, static_cast<T*>(gW));
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_wgrad_small(const void* G, const void* A, int M, int N, int K, void* gW, hipStream_t st) {
  typedef typename Elem<DT>::T T;
  hipLaunchKernelGGL(k_wgrad_small<DT>, dim3((K + 63) / 64, (N + 63) / 64), dim3(256), 0, st,
                     static_cast<const T*>(G), static_cast<const T*>(A), M, N, K, static_cast<T*>(gW));
  return hipGetLastError();
}

hipError_t launch_gemm_wgrad(int dt, const void* G, const void* A, int M, int N, int K, void* gW, hipStream_t st) {
  if (N <= 0 || K <= 0) return hipSuccess;
  const bool aligned = (uintptr_t)G % 16 == 0 && (uintptr_t)A % 16 == 0 && (uintptr_t)gW % 16 == 0;
  // the large-tile kernel addresses both operands with 32-bit buffer offsets
  const bool fits = ((int64_t)M + 256) * K * 2 < ((int64_t)1 << 31) - 4096 &&
                    ((int64_t)M + 256) * N * 2 < ((int64_t)1 << 31) - 4096;
  const int64_t tiles = (int64_t)((N + 255) / 256) * ((K + 255) / 256);
  if (dt != DT_F32 && M > 0 && N % 8 == 0 && K % 8 == 0 && aligned && fits && tiles >= 16) {
    if (dt == DT_F16) return launch_wgrad_big<DT_F16>(G, A, M, N, K, gW, st);
    return launch_wgrad_big<DT_BF16>(G, A, M, N, K, gW, st);
  }
  if ((N + 63) / 64 > 65535) return hipErrorInvalidValue;
  switch (dt) {
    case DT_F32: return launch_wgrad_small<DT_F32>(G, A, M, N, K, gW, st);
    case DT_F16: return launch_wgrad_small<DT_F16>(G, A, M, N, K, gW, st);
    default: return launch_wgrad_small<DT_BF16>(G, A, M, N, K, gW, st);
  }
}

}  // namespace i8l
