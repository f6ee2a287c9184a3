// Calibration kernels of INSTANT (notes "INSTANT: Compressing Gradients and Activations
// for Resource-Efficient Training", sections 关键设计 1 and 关键设计 2):
//   syrk            running sums S += sum_b t_b t_b^T of the token autocorrelation, on the
//                   matrix cores, upper-triangle 64x64 tiles, deterministic split reduction
//                   into float64
//   build_io        I/O-dtype copies of the published projections
// The eigen-decomposition and truncation live in kernels_eig.hip.
#include "common.hpp"
#include "launch.hpp"

namespace instant {

// ============================================================================ SYRK
constexpr int ST = 64;  // statistics tile edge

int syrk_tiles(int L) {
  const int T = (L + ST - 1) / ST;
  return T * (T + 1) / 2;
}

__device__ inline void upper_tile(int idx, int T, int& ti, int& tj) {
  ti = 0;
  while (idx >= T - ti) {
    idx -= T - ti;
    ++ti;
  }
  tj = ti + idx;
}

// part[s][tile][64*64] = sum over the s-th slice of the (sample, channel-step) range of
// X_b[rows of ti] . X_b[rows of tj]^T. Four waves split the slice; LDS sums them in order.
template <class T>
__global__ __launch_bounds__(256) void syrk_kernel(const T* __restrict__ X, int B, int L, int C, int nsplit,
                                                   float* __restrict__ part) {
  typedef MM<T> mm;
  typedef typename mm::frag frag;
  constexpr int NW = 4;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  const int Tn = (L + ST - 1) / ST;
  const int ntiles = Tn * (Tn + 1) / 2;
  // Workgroups are dealt to the 8 XCDs round-robin by linear id. When there are at least
  // 8 slices, give all tiles of a slice to one XCD so each sample is fetched into one L2.
  int tile, s;
  const int lin = blockIdx.x;
  if (nsplit % 8 == 0) {
    const int xcd = lin % 8, k = lin / 8;
    s = xcd + 8 * (k / ntiles);
    tile = k % ntiles;
  } else {
    s = lin / ntiles;
    tile = lin % ntiles;
  }
  int ti, tj;
  upper_tile(tile, Tn, ti, tj);
  const int steps_c = (C + mm::KSTEP - 1) / mm::KSTEP;
  const long total = (long)B * steps_c;
  const long beg = total * s / nsplit;
  const long end = total * (s + 1) / nsplit;
  const int kl = mm::G * (lane >> 4);

  f32x4 acc[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[t][u] = zero4();

  constexpr int U = 4;  // k-steps whose loads are in flight together
  for (long q0 = beg + wave; q0 < end; q0 += NW * U) {
    frag a[U][4], bb[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long q = q0 + u * NW;
      const bool qok = q < end;
      const int b = qok ? (int)(q / steps_c) : 0;
      const int kk = (int)(q % steps_c) * mm::KSTEP + kl;
      const T* __restrict__ Xb = X + (size_t)b * L * C;
      const bool kok = qok && kk < C;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = ti * ST + 16 * t + (lane & 15);
        a[u][t] = load_frag<T>(Xb + (size_t)r * C + kk, kok && r < L);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = tj * ST + 16 * t + (lane & 15);
        bb[u][t] = load_frag<T>(Xb + (size_t)r * C + kk, kok && r < L);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[t][v] = mm::mma(a[u][t], bb[u][v], acc[t][v]);
  }

  __shared__ float red[NW][4][4][WAVE];
  float* __restrict__ out = part + ((size_t)s * ntiles + tile) * (ST * ST);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][u][v][lane] = acc[t][u][v];
    __syncthreads();
    {
      const int v = wave;  // each wave finishes one of the four rows a lane holds
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float sum = red[0][u][v][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) sum += red[w][u][v][lane];
        const int row = 16 * t + 4 * (lane >> 4) + v;
        const int col = 16 * u + (lane & 15);
        out[row * ST + col] = sum;
      }
    }
    __syncthreads();
  }
}

// S[i][j] += sum_s part[s][tile] in split order, float64, for the upper-triangle tiles.
__global__ __launch_bounds__(256) void syrk_reduce_kernel(const float* __restrict__ part, int nsplit, int ntiles,
                                                          int L, double* __restrict__ S) {
  const int tile = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;
  const int Tn = (L + ST - 1) / ST;
  int ti, tj;
  upper_tile(tile, Tn, ti, tj);
  const int i = ti * ST + e / ST;
  const int j = tj * ST + e % ST;
  if (i >= L || j >= L) return;
  // independent loads, summed in split order
  const float* __restrict__ pp = part + (size_t)tile * (ST * ST) + e;
  const size_t stride = (size_t)ntiles * (ST * ST);
  double acc = 0.0;
  int s = 0;
  for (; s + 4 <= nsplit; s += 4) {
    const float v0 = pp[(s + 0) * stride], v1 = pp[(s + 1) * stride];
    const float v2 = pp[(s + 2) * stride], v3 = pp[(s + 3) * stride];
    acc += (double)v0;
    acc += (double)v1;
    acc += (double)v2;
    acc += (double)v3;
  }
  for (; s < nsplit; ++s) acc += (double)pp[s * stride];
  S[(size_t)i * L + j] += acc;
}

template <class T>
static hipError_t syrk_t(const void* X, int B, int L, int C, int nsplit, float* part, hipStream_t st) {
  dim3 grid(syrk_tiles(L) * nsplit);
  hipLaunchKernelGGL(syrk_kernel<T>, grid, dim3(256), 0, st, (const T*)X, B, L, C, nsplit, part);
  return hipGetLastError();
}

hipError_t launch_syrk(bool bf16_io, const void* X, int B, int L, int C, int nsplit, float* part, hipStream_t st) {
  return bf16_io ? syrk_t<bf16>(X, B, L, C, nsplit, part, st) : syrk_t<float>(X, B, L, C, nsplit, part, st);
}

hipError_t launch_syrk_reduce(const float* part, int nsplit, int L, double* S, hipStream_t st) {
  dim3 grid(syrk_tiles(L), ST * ST / 256);
  hipLaunchKernelGGL(syrk_reduce_kernel, grid, dim3(256), 0, st, part, nsplit, syrk_tiles(L), L, S);
  return hipGetLastError();
}

// I/O-dtype copies: PQ rows [0, Rx) = P, [Rx, Rx+Ry) = Q with ld ldL (zero beyond L), and
// Qt[l][r] = Q[r][l] with ld ldQt (zero beyond Ry). Rows of PQ beyond Rx+Ry are zeroed.
template <class T>
__global__ __launch_bounds__(256) void build_io_kernel(const float* __restrict__ P32, const float* __restrict__ Q32,
                                                       const int* __restrict__ dRx, const int* __restrict__ dRy,
                                                       int L, int ldL, int R_max, T* __restrict__ PQ,
                                                       T* __restrict__ Qt, int ldQt) {
  const int Rx = *dRx, Ry = *dRy;
  const size_t n1 = (size_t)2 * R_max * ldL;
  const size_t n2 = (size_t)L * ldQt;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n1 + n2; e += (size_t)gridDim.x * 256) {
    if (e < n1) {
      const int r = (int)(e / ldL), l = (int)(e % ldL);
      float v = 0.0f;
      if (l < L) {
        if (r < Rx) v = P32[(size_t)r * L + l];
        else if (r < Rx + Ry) v = Q32[(size_t)(r - Rx) * L + l];
      }
      PQ[e] = from_f32<T>(v);
    } else {
      const size_t f = e - n1;
      const int l = (int)(f / ldQt), r = (int)(f % ldQt);
      Qt[f] = from_f32<T>(r < Ry ? Q32[(size_t)r * L + l] : 0.0f);
    }
  }
}

hipError_t launch_build_io(bool bf16_io, const float* P32, const float* Q32, const int* dRx, const int* dRy, int L,
                           int ldL, int R_max, void* PQ, void* Qt, int ldQt, hipStream_t st) {
  const size_t n = (size_t)2 * R_max * ldL + (size_t)L * ldQt;
  const int blocks = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
  if (bf16_io)
    hipLaunchKernelGGL(build_io_kernel<bf16>, dim3(blocks), dim3(256), 0, st, P32, Q32, dRx, dRy, L, ldL, R_max,
                       (bf16*)PQ, (bf16*)Qt, ldQt);
  else
    hipLaunchKernelGGL(build_io_kernel<float>, dim3(blocks), dim3(256), 0, st, P32, Q32, dRx, dRy, L, ldL, R_max,
                       (float*)PQ, (float*)Qt, ldQt);
  return hipGetLastError();
}

__global__ void fill_i32_kernel(int* dst, int n, int v0, int v1, int v2, int v3) {
  const int i = threadIdx.x;
  const int v[4] = {v0, v1, v2, v3};
  if (i < n) dst[i] = v[i];
}

hipError_t launch_fill_i32(int* dst, const int* values, int n, hipStream_t st) {
  if (n > 4) return hipErrorInvalidValue;
  int v[4] = {0, 0, 0, 0};
  for (int i = 0; i < n; ++i) v[i] = values[i];
  hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(64), 0, st, dst, n, v[0], v[1], v[2], v[3]);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_kernel(uint32_t* __restrict__ dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) dst[i] = 0u;
}

hipError_t launch_zero(void* dst, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const size_t want = (n + 255) / 256;
  const int blocks = (int)(want < 2048 ? want : 2048);
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, st, (uint32_t*)dst, n);
  return hipGetLastError();
}

}  // namespace instant

namespace instant {

// C[i][j] = S[min(i,j)][max(i,j)] * inv_n (the running sums hold the upper triangle).
__global__ __launch_bounds__(256) void stat_mean_kernel(const double* __restrict__ S, double inv_n, int L,
                                                        double* __restrict__ out) {
  const size_t n = (size_t)L * L;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256) {
    const int i = (int)(e / L), j = (int)(e % L);
    const int a = i < j ? i : j, b = i < j ? j : i;
    out[e] = S[(size_t)a * L + b] * inv_n;
  }
}

hipError_t launch_stat_mean(const double* S, double inv_n, int L, double* out, hipStream_t st) {
  const size_t n = (size_t)L * L;
  const size_t want = (n + 255) / 256;
  hipLaunchKernelGGL(stat_mean_kernel, dim3((unsigned)(want < 4096 ? want : 4096)), dim3(256), 0, st, S, inv_n, L, out);
  return hipGetLastError();
}

}  // namespace instant
