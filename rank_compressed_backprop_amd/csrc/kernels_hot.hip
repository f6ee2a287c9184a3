// Per-step kernels of the INSTANT low-rank backward (notes "INSTANT: Compressing
// Gradients and Activations for Resource-Efficient Training", sections 整体框架 and
// 关键设计 3):
//   proj    x_hat_b = P x_b (forward compression) and, with the stacked [P; Q],
//           P gy_b and Q gy_b from a single read of gy
//   gemm    g_w = sum_b (P gy_b)^T x_hat_b   (contraction over K = B*Rx)
//           g_hat_x = (Q gy) w               (contraction over K = Cy)
//   expand  g_x_b = Q^T g_hat_x_b            (contraction over K = Ry)
// All contractions run on the matrix cores with float32 accumulation.
#include "common.hpp"
#include "launch.hpp"

namespace instant {

// ----------------------------------------------------------------------------- proj
// Out[b][m][c] = sum_{l < L} A[m][l] X[b][l][c] for m < M, c < C.
// A is [>= M rows][ldA] with zero columns from L up to ldA (ldA a multiple of KSTEP).
// Rows m < M0 go to out0 [B][M0][C]; rows M0 <= m < M go to out1 [B][M - M0][C].
// Grid: (ceil(C / 128), B). Each of the NW waves of a block takes every NW-th k-step
// of the same 128-column strip; the partial tiles are summed through LDS in wave order.
template <class T, int MT, int NW, int U>
__global__ __launch_bounds__(NW * WAVE) void proj_kernel(const T* __restrict__ A, int ldA, int M, int M0,
                                                         const T* __restrict__ X, int L, int C,
                                                         T* __restrict__ out0, T* __restrict__ out1) {
  typedef MM<T> mm;
  typedef typename mm::frag frag;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  const int b = blockIdx.y;
  const int col = blockIdx.x * 128 + 8 * (lane & 15);
  const bool col_ok = col < C;
  const T* __restrict__ Xb = X + (size_t)b * L * C;
  const int arow = lane & 15;
  const int kl = mm::G * (lane >> 4);

  f32x4 acc[MT][8];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[t][j] = zero4();

  const int nsteps = (L + mm::KSTEP - 1) / mm::KSTEP;
  for (int s0 = wave; s0 < nsteps; s0 += NW * U) {
    frag bf[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k0 = (s0 + u * NW) * mm::KSTEP + kl;
      load_strip_T<T, 8>(Xb, C, k0, L, col, col_ok, bf[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * NW;
      if (s < nsteps) {
        const int k0 = s * mm::KSTEP + kl;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const int m = 16 * t + arow;
          frag af = load_frag<T>(A + (size_t)m * ldA + k0, m < M);
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[t][j] = mm::mma(af, bf[u][j], acc[t][j]);
        }
      }
    }
  }

  const int Mb = M - M0;
  auto store = [&](int m, const float v[8]) {
    if (m >= M || !col_ok) return;
    T* dst = (m < M0) ? out0 + ((size_t)b * M0 + m) * C + col : out1 + ((size_t)b * Mb + (m - M0)) * C + col;
    store_row<T, 8>(dst, v);
  };

  if constexpr (NW == 1) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = acc[t][j][v];
        store(16 * t + 4 * (lane >> 4) + v, o);
      }
  } else {
    __shared__ float red[NW][8][4][WAVE];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave][j][v][lane] = acc[t][j][v];
      __syncthreads();
      for (int v = wave; v < 4; v += NW) {
        float o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float sum = red[0][j][v][lane];
#pragma unroll
          for (int w = 1; w < NW; ++w) sum += red[w][j][v][lane];
          o[j] = sum;
        }
        store(16 * t + 4 * (lane >> 4) + v, o);
      }
      __syncthreads();
    }
  }
}

// ----------------------------------------------------------------------------- gemm
// Cm[m][n] = sum_{k < K} A(m, k) B[k][n], written in T to Cm [M][ldc] (batch-strided).
// A_TRANS = false: A is [M][lda] (k contiguous); the wave covers 16*MT rows.
// A_TRANS = true : A is [K][lda] (m contiguous); a lane reads 4 adjacent rows as
//                  virtual tiles, the wave covers 64 rows (MT must be 4).
// B is [K][ldb] (n contiguous); the wave covers 128 columns.
// Grid: (ceil(N / 128), ceil(M / rows per wave), batch); the NW waves of a block split K.
template <class T, bool A_TRANS, int MT, int NW>
__global__ __launch_bounds__(NW * WAVE) void gemm_kernel(const T* __restrict__ A, int lda, size_t strideA,
                                                         const T* __restrict__ Bm, int ldb, size_t strideB,
                                                         T* __restrict__ Cm, int ldc, size_t strideC,
                                                         int M, int N, int K) {
  typedef MM<T> mm;
  typedef typename mm::frag frag;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  const int z = blockIdx.z;
  A += z * strideA;
  Bm += z * strideB;
  Cm += z * strideC;
  const int col = blockIdx.x * 128 + 8 * (lane & 15);
  const bool col_ok = col < N;
  constexpr int ROWS = A_TRANS ? 64 : 16 * MT;
  const int m0 = blockIdx.y * ROWS;
  const int kl = mm::G * (lane >> 4);

  f32x4 acc[MT][8];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[t][j] = zero4();

  const int nsteps = (K + mm::KSTEP - 1) / mm::KSTEP;
  for (int s = wave; s < nsteps; s += NW) {
    const int k0 = s * mm::KSTEP + kl;
    frag bf[8];
    load_strip_T<T, 8>(Bm, ldb, k0, K, col, col_ok, bf);
    frag af[MT];
    if constexpr (A_TRANS) {
      static_assert(MT == 4, "transposed A uses 4-wide strips");
      const int acol = m0 + 4 * (lane & 15);
      load_strip_T<T, 4>(A, lda, k0, K, acol, acol < M, af);
    } else {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int m = m0 + 16 * t + (lane & 15);
        // the k tail of a direct operand is masked element-wise only when K is ragged
        if (m < M && k0 + mm::G <= K) {
          af[t] = load_frag<T>(A + (size_t)m * lda + k0, true);
        } else {
          af[t] = zero_frag<T>();
          if (m < M)
            for (int g = 0; g < mm::G; ++g)
              if (k0 + g < K) af[t][g] = A[(size_t)m * lda + k0 + g];
        }
      }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[t][j] = mm::mma(af[t], bf[j], acc[t][j]);
  }

  auto row_of = [&](int t, int v) {
    const int r = 4 * (lane >> 4) + v;  // tile row
    return A_TRANS ? m0 + 4 * r + t : m0 + 16 * t + r;
  };
  auto store = [&](int m, const float o[8]) {
    if (m < M && col_ok) store_row<T, 8>(Cm + (size_t)m * ldc + col, o);
  };

  if constexpr (NW == 1) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = acc[t][j][v];
        store(row_of(t, v), o);
      }
  } else {
    __shared__ float red[NW][8][4][WAVE];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave][j][v][lane] = acc[t][j][v];
      __syncthreads();
      for (int v = wave; v < 4; v += NW) {
        float o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float sum = red[0][j][v][lane];
#pragma unroll
          for (int w = 1; w < NW; ++w) sum += red[w][j][v][lane];
          o[j] = sum;
        }
        store(row_of(t, v), o);
      }
      __syncthreads();
    }
  }
}

// ----------------------------------------------------------------------------- expand
// Out[b][l][c] = sum_{r < R} At[l][r] Bz[b][r][c]: At is [L][ldA] with zero columns
// from R up to ldA = KS * KSTEP; Bz is [B][R][C]. Each wave keeps the B operand of its
// 128-column strip in registers and sweeps MPW row tiles of 16 tokens.
// Grid: (ceil(C / 128), B, ceil(L / (16 * MPW * NW))).
template <class T, int KS, int MPW, int NW>
__global__ __launch_bounds__(NW * WAVE) void expand_kernel(const T* __restrict__ At, int ldA,
                                                           const T* __restrict__ Bz, int R, int L, int C,
                                                           T* __restrict__ out) {
  typedef MM<T> mm;
  typedef typename mm::frag frag;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  const int b = blockIdx.y;
  const int col = blockIdx.x * 128 + 8 * (lane & 15);
  const bool col_ok = col < C;
  const int kl = mm::G * (lane >> 4);
  const T* __restrict__ Bb = Bz + (size_t)b * R * C;

  frag bf[KS][8];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) load_strip_T<T, 8>(Bb, C, ks * mm::KSTEP + kl, R, col, col_ok, bf[ks]);

  const int tile0 = (blockIdx.z * NW + wave) * MPW;
#pragma unroll
  for (int i = 0; i < MPW; ++i) {
    const int l0 = 16 * (tile0 + i);
    if (l0 >= L) break;
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = zero4();
    const int la = l0 + (lane & 15);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      frag af = load_frag<T>(At + (size_t)la * ldA + ks * mm::KSTEP + kl, la < L);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = mm::mma(af, bf[ks][j], acc[j]);
    }
    if (col_ok) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int l = l0 + 4 * (lane >> 4) + v;
        if (l < L) {
          float o[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) o[j] = acc[j][v];
          store_row<T, 8>(out + ((size_t)b * L + l) * C + col, o);
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------- launchers

template <class T, int MT>
static hipError_t proj_mt(const void* A, int ldA, int M, int M0, const void* X, int B, int L, int C,
                          void* out0, void* out1, hipStream_t st) {
  constexpr int NW = 4;
  constexpr int U = MT <= 5 ? 2 : 1;  // keeps the widest stacks free of register spills
  dim3 grid((C + 127) / 128, B);
  hipLaunchKernelGGL((proj_kernel<T, MT, NW, U>), grid, dim3(NW * WAVE), 0, st, (const T*)A, ldA, M, M0,
                     (const T*)X, L, C, (T*)out0, (T*)out1);
  return hipGetLastError();
}

template <class T>
static hipError_t proj_t(const void* A, int ldA, int M, int M0, const void* X, int B, int L, int C,
                         void* out0, void* out1, hipStream_t st) {
  switch ((M + 15) / 16) {
    case 1: return proj_mt<T, 1>(A, ldA, M, M0, X, B, L, C, out0, out1, st);
    case 2: return proj_mt<T, 2>(A, ldA, M, M0, X, B, L, C, out0, out1, st);
    case 3: return proj_mt<T, 3>(A, ldA, M, M0, X, B, L, C, out0, out1, st);
    case 4: return proj_mt<T, 4>(A, ldA, M, M0, X, B, L, C, out0, out1, st);
    case 5: return proj_mt<T, 5>(A, ldA, M, M0, X, B, L, C, out0, out1, st);
    case 6: return proj_mt<T, 6>(A, ldA, M, M0, X, B, L, C, out0, out1, st);
    case 7: return proj_mt<T, 7>(A, ldA, M, M0, X, B, L, C, out0, out1, st);
    case 8: return proj_mt<T, 8>(A, ldA, M, M0, X, B, L, C, out0, out1, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_proj(bool bf16_io, const void* A, int ldA, int M, int M0, const void* X, int B, int L, int C,
                       void* out0, void* out1, hipStream_t st) {
  return bf16_io ? proj_t<bf16>(A, ldA, M, M0, X, B, L, C, out0, out1, st)
                 : proj_t<float>(A, ldA, M, M0, X, B, L, C, out0, out1, st);
}

template <class T, bool AT>
static hipError_t gemm_t(const void* A, int lda, size_t sA, const void* Bm, int ldb, size_t sB, void* Cm, int ldc,
                         size_t sC, int batch, int M, int N, int K, hipStream_t st) {
  constexpr int MT = 4;
  constexpr int NW = 4;
  dim3 grid((N + 127) / 128, (M + 63) / 64, batch);
  hipLaunchKernelGGL((gemm_kernel<T, AT, MT, NW>), grid, dim3(NW * WAVE), 0, st, (const T*)A, lda, sA,
                     (const T*)Bm, ldb, sB, (T*)Cm, ldc, sC, M, N, K);
  return hipGetLastError();
}

hipError_t launch_gemm(bool bf16_io, bool a_trans, const void* A, int lda, size_t sA, const void* Bm, int ldb,
                       size_t sB, void* Cm, int ldc, size_t sC, int batch, int M, int N, int K, hipStream_t st) {
  if (bf16_io)
    return a_trans ? gemm_t<bf16, true>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, st)
                   : gemm_t<bf16, false>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, st);
  return a_trans ? gemm_t<float, true>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, st)
                 : gemm_t<float, false>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, st);
}

template <class T, int KS>
static hipError_t expand_ks(const void* At, int ldA, const void* Bz, int B, int R, int L, int C, void* out,
                            hipStream_t st) {
  constexpr int MPW = 4;
  constexpr int NW = 4;
  dim3 grid((C + 127) / 128, B, (L + 16 * MPW * NW - 1) / (16 * MPW * NW));
  hipLaunchKernelGGL((expand_kernel<T, KS, MPW, NW>), grid, dim3(NW * WAVE), 0, st, (const T*)At, ldA,
                     (const T*)Bz, R, L, C, (T*)out);
  return hipGetLastError();
}

template <class T>
static hipError_t expand_t(const void* At, int ldA, const void* Bz, int B, int R, int L, int C, void* out,
                           hipStream_t st) {
  switch ((R + MM<T>::KSTEP - 1) / MM<T>::KSTEP) {
    case 1: return expand_ks<T, 1>(At, ldA, Bz, B, R, L, C, out, st);
    case 2: return expand_ks<T, 2>(At, ldA, Bz, B, R, L, C, out, st);
    case 3: return expand_ks<T, 3>(At, ldA, Bz, B, R, L, C, out, st);
    case 4: return expand_ks<T, 4>(At, ldA, Bz, B, R, L, C, out, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_expand(bool bf16_io, const void* At, int ldA, const void* Bz, int B, int R, int L, int C,
                         void* out, hipStream_t st) {
  return bf16_io ? expand_t<bf16>(At, ldA, Bz, B, R, L, C, out, st)
                 : expand_t<float>(At, ldA, Bz, B, R, L, C, out, st);
}

}  // namespace instant
