// Calibration kernels of INSTANT (notes "INSTANT: Compressing Gradients and Activations
// for Resource-Efficient Training", sections 关键设计 1 and 关键设计 2):
//   syrk            running sums S += sum_b t_b t_b^T of the token autocorrelation, on the
//                   matrix cores, upper-triangle 64x64 tiles, deterministic split reduction
//                   into float64
//   jacobi_*        blocked one-sided (Hestenes) Jacobi on C = S / n: columns are
//                   orthogonalised in blocks of 8; each round pairs the blocks by a
//                   round-robin tournament and every pair diagonalises the 16x16 Gram
//                   matrix of its columns and rotates them. At convergence the column
//                   norms are the singular values (= eigenvalues of the PSD C) and the
//                   normalised columns the eigenvectors.
//   truncate_build  descending order, float64 prefix energy, smallest k reaching eps*E,
//                   R = min(k + p, L), compensation c, P = c * U_R^T with a canonical sign
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
  int ti, tj;
  upper_tile(blockIdx.x, Tn, ti, tj);
  const int s = blockIdx.y;
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

  for (long q = beg + wave; q < end; q += NW) {
    const int b = (int)(q / steps_c);
    const int kk = (int)(q % steps_c) * mm::KSTEP + kl;
    const T* __restrict__ Xb = X + (size_t)b * L * C;
    const bool kok = kk < C;
    frag a[4], bb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = ti * ST + 16 * t + (lane & 15);
      a[t] = load_frag<T>(Xb + (size_t)r * C + kk, kok && r < L);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = tj * ST + 16 * u + (lane & 15);
      bb[u] = load_frag<T>(Xb + (size_t)r * C + kk, kok && r < L);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[t][u] = mm::mma(a[t], bb[u], acc[t][u]);
  }

  __shared__ float red[NW][4][4][WAVE];
  float* __restrict__ out = part + ((size_t)s * gridDim.x + blockIdx.x) * (ST * ST);
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
  double acc = 0.0;
  for (int s = 0; s < nsplit; ++s) acc += (double)part[((size_t)s * ntiles + tile) * (ST * ST) + e];
  S[(size_t)i * L + j] += acc;
}

template <class T>
static hipError_t syrk_t(const void* X, int B, int L, int C, int nsplit, float* part, hipStream_t st) {
  dim3 grid(syrk_tiles(L), nsplit);
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

// ============================================================================ Jacobi
// Working matrix W of one side: column-major, column c at W + c * ldw, ldw = L rounded
// up to 16 with zero rows; nb * 8 columns (nb even) with zero columns beyond L.

// W[c][r] = S[min(r,c)][max(r,c)] * inv_n; flags non-finite statistics.
__global__ __launch_bounds__(256) void jacobi_prep_kernel(const double* __restrict__ S, double inv_n, int L, int ldw,
                                                          int ncols, float* __restrict__ W, int* __restrict__ bad) {
  const int c = blockIdx.x;
  for (int r = threadIdx.x; r < ldw; r += 256) {
    float v = 0.0f;
    if (r < L && c < L) {
      const int i = r < c ? r : c;
      const int j = r < c ? c : r;
      const double d = S[(size_t)i * L + j] * inv_n;
      if (!isfinite(d)) atomicOr(bad, 1);
      v = (float)d;
    }
    W[(size_t)c * ldw + r] = v;
  }
  (void)ncols;
}

__device__ inline int tourney(int pos, int round, int nb) {
  // circle method: position 0 fixed, the others rotate by `round`
  return pos == 0 ? 0 : 1 + (pos - 1 + round) % (nb - 1);
}

struct JacobiSide {
  float* W;
  float* offmax;        // max relative off-diagonal seen this sweep (bit pattern of a non-negative float)
  int* active;          // 1 while the side still iterates
  const double* scale;  // ||C||_F^2, invariant under the rotations
};

// Columns whose squared norm is below NOISE_REL * ||C||_F^2 lie under float32 resolution
// (sigma below 1e-5 of the total): their pairings are neither rotated nor counted.
constexpr double NOISE_REL = 1e-10;

// One round: block pair (tourney(p), tourney(nb-1-p)) for p = blockIdx.x, side blockIdx.y.
// The Gram matrix is formed in float32 on the matrix cores; the 16x16 eigenproblem and
// the column update run in float64 so the accumulated rotation stays orthogonal.
__global__ __launch_bounds__(256) void jacobi_round_kernel(JacobiSide s0, JacobiSide s1, int L, int ldw, int nb,
                                                           int round, double rot_tol) {
  const JacobiSide sd = blockIdx.y ? s1 : s0;
  if (*sd.active == 0) return;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  const int ba = tourney(blockIdx.x, round, nb);
  const int bb = tourney(nb - 1 - blockIdx.x, round, nb);
  __shared__ int col[16];
  __shared__ double G[16][17];
  __shared__ double V[16][17];
  __shared__ float part[4][16][17];
  __shared__ int partner[16];
  __shared__ double jd[16], jo[16];
  __shared__ int any_rot;
  if (threadIdx.x < 16) col[threadIdx.x] = (threadIdx.x < 8 ? ba : bb) * 8 + (threadIdx.x & 7);
  __syncthreads();
  const double floor_g = NOISE_REL * *sd.scale;

  // Gram matrix G = Y^T Y of the 16 columns on the matrix cores (fp32). Lane i reads four
  // consecutive rows of column (i % 16); the four waves take alternate 16-row steps.
  {
    const float* __restrict__ cp = sd.W + (size_t)col[lane & 15] * ldw;
    f32x4 acc = zero4();
    for (int r0 = 16 * wave + 4 * (lane >> 4); r0 < ldw; r0 += 64) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(cp + r0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v[0], v[0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v[1], v[1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v[2], v[2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v[3], v[3], acc, 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) part[wave][4 * (lane >> 4) + v][lane & 15] = acc[v];
  }
  __syncthreads();
  {
    const int x = threadIdx.x >> 4, y = threadIdx.x & 15;
    G[x][y] = (double)part[0][x][y] + (double)part[1][x][y] + (double)part[2][x][y] + (double)part[3][x][y];
    V[x][y] = (x == y) ? 1.0 : 0.0;
  }
  __syncthreads();

  // sweep convergence measure: largest |G_xy| / sqrt(G_xx G_yy) over the pair's columns
  if (wave == 0) {
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = lane * 4 + e;
      const int x = idx >> 4, y = idx & 15;
      if (x < y) {
        const double a = G[x][x], d = G[y][y];
        if (a > floor_g && d > floor_g) m = fmaxf(m, (float)(fabs(G[x][y]) / sqrt(a * d)));
      }
    }
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0 && m > 0.0f) atomicMax(reinterpret_cast<unsigned int*>(sd.offmax), __float_as_uint(m));
  }

  // Inner two-sided Jacobi on the 16x16 Gram matrix, accumulating the rotation V.
  for (int isweep = 0; isweep < 6; ++isweep) {
    if (threadIdx.x == 0) any_rot = 0;
    __syncthreads();
    for (int ir = 0; ir < 15; ++ir) {
      if (threadIdx.x < 8) {
        const int p = tourney(threadIdx.x, ir, 16);
        const int q = tourney(15 - threadIdx.x, ir, 16);
        const double a = G[p][p], d = G[q][q], o = G[p][q];
        double c = 1.0, sn = 0.0;
        if (a > floor_g && d > floor_g && fabs(o) > rot_tol * sqrt(a * d)) {
          const double zeta = (d - a) / (2.0 * o);
          const double t = copysign(1.0, zeta) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
          c = 1.0 / sqrt(1.0 + t * t);
          sn = t * c;
          any_rot = 1;
        }
        // new column p = c*p - s*q, new column q = s*p + c*q
        partner[p] = q;
        jd[p] = c;
        jo[p] = -sn;
        partner[q] = p;
        jd[q] = c;
        jo[q] = sn;
      }
      __syncthreads();
      double gn[4], vn[4];
      if (threadIdx.x < 64) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = threadIdx.x * 4 + e;
          const int x = idx >> 4, y = idx & 15;
          const int ox = partner[x], oy = partner[y];
          gn[e] = jd[x] * (jd[y] * G[x][y] + jo[y] * G[x][oy]) + jo[x] * (jd[y] * G[ox][y] + jo[y] * G[ox][oy]);
          vn[e] = V[x][y] * jd[y] + V[x][oy] * jo[y];
        }
      }
      __syncthreads();
      if (threadIdx.x < 64) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = threadIdx.x * 4 + e;
          G[idx >> 4][idx & 15] = gn[e];
          V[idx >> 4][idx & 15] = vn[e];
        }
      }
      __syncthreads();
    }
    const int rotated = any_rot;
    __syncthreads();  // every thread has read the flag before it is cleared again
    if (!rotated) break;
  }

  // Rotate the 16 columns: Y <- Y V (rows split over the block), float64 arithmetic.
  for (int r = threadIdx.x; r < L; r += 256) {
    double y[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) y[q] = (double)sd.W[(size_t)col[q] * ldw + r];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      double acc = 0.0;
#pragma unroll
      for (int p = 0; p < 16; ++p) acc = fma(y[p], V[p][q], acc);
      sd.W[(size_t)col[q] * ldw + r] = (float)acc;
    }
  }
}

// Per side: stop iterating once a whole sweep saw no off-diagonal above tol.
__global__ void jacobi_check_kernel(JacobiSide s0, JacobiSide s1, float tol, int* sweeps, int* converged) {
  const int side = threadIdx.x;
  if (side > 1) return;
  const JacobiSide sd = side ? s1 : s0;
  if (*sd.active) {
    sweeps[side] += 1;
    if (*sd.offmax <= tol) {
      *sd.active = 0;
      converged[side] = 1;
    }
  }
  *sd.offmax = 0.0f;
}

// ||W||_F^2 from the column norms, in a fixed order (one block).
__global__ __launch_bounds__(256) void frob_kernel(const float* __restrict__ nrm, int L, double* __restrict__ out) {
  __shared__ double red[256];
  double acc = 0.0;
  for (int c = threadIdx.x; c < L; c += 256) acc += (double)nrm[c] * (double)nrm[c];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = red[0];
}

// ============================================================================ truncation / build
// Column norms of W: sigma_c = ||W[:, c]||, c < L.
__global__ __launch_bounds__(64) void colnorm_kernel(const float* __restrict__ W, int ldw, int L, float* __restrict__ nrm) {
  const int c = blockIdx.x;
  const int lane = threadIdx.x;
  float acc = 0.0f;
  for (int r = lane; r < L; r += 64) {
    const float v = W[(size_t)c * ldw + r];
    acc += v * v;
  }
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) nrm[c] = sqrtf(acc);
}

// Device-side info block of one side (int32 slots).
// [0] status [1] k [2] R [3] c (float bits) [4..5] kept (double) [6..7] kept_k (double)
constexpr int MAX_L = 4096;
constexpr int INFO_STATUS = 0, INFO_K = 1, INFO_R = 2, INFO_C = 3, INFO_KEPT = 4, INFO_KEPTK = 6;

// One block of 1024 threads: sort the L column norms (descending, ties by column index),
// energy prefix in float64, truncation, compensation and P = c * U_R^T.
__global__ __launch_bounds__(1024) void truncate_build_kernel(const float* __restrict__ W, int ldw, int L,
                                                              const float* __restrict__ nrm, float eps, int p,
                                                              int comp, int R_max, const int* __restrict__ bad,
                                                              const int* __restrict__ converged,
                                                              float* __restrict__ P32, float* __restrict__ sigma_out,
                                                              int* __restrict__ info) {
  __shared__ float key[MAX_L];
  __shared__ int idx[MAX_L];
  __shared__ double prefix_last, prefix_k, prefix_R;
  __shared__ int sk, sR, sstatus;
  __shared__ float sc;
  const int tid = threadIdx.x;
  int Lp2 = 1;
  while (Lp2 < L) Lp2 <<= 1;
  for (int i = tid; i < Lp2; i += 1024) {
    key[i] = i < L ? nrm[i] : -1.0f;  // padding sorts last
    idx[i] = i;
  }
  __syncthreads();
  // bitonic sort, descending by key, ascending index on ties
  for (int size = 2; size <= Lp2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < Lp2; i += 1024) {
        const int jx = i ^ stride;
        if (jx > i) {
          const bool desc = (i & size) == 0;
          const float ki = key[i], kj = key[jx];
          const int ii = idx[i], ij = idx[jx];
          const bool i_first = (ki > kj) || (ki == kj && ii < ij);  // i should precede j
          if (desc ? !i_first : i_first) {
            key[i] = kj;
            key[jx] = ki;
            idx[i] = ij;
            idx[jx] = ii;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < L; i += 1024) sigma_out[i] = key[i];

  if (tid == 0) {
    int status = 0;
    if (*bad) status = 6;            // non-finite statistics
    else if (!*converged) status = 7;  // no convergence
    // ordered float64 prefix of sigma^2
    double run = 0.0;
    for (int i = 0; i < L; ++i) {
      const double sgm = (double)key[i];
      run += sgm * sgm;
    }
    const double E = run;
    int k = 0;
    double Sk = 0.0, SR = 0.0;
    if (status == 0 && !(E > 0.0)) status = (E == 0.0) ? 5 : 6;
    if (status == 0) {
      const double thr = (double)eps * E;
      run = 0.0;
      for (int i = 0; i < L; ++i) {
        const double sgm = (double)key[i];
        run += sgm * sgm;
        if (run >= thr) {
          k = i + 1;
          Sk = run;
          break;
        }
      }
      if (k == 0) {  // rounding made the total fall short of eps*E: only possible at eps == 1
        k = L;
        Sk = E;
      }
    }
    int R = k + p < L ? k + p : L;
    if (status == 0 && R > R_max) status = 4;
    float c = 1.0f;
    if (status == 0) {
      run = 0.0;
      for (int i = 0; i < R; ++i) {
        const double sgm = (double)key[i];
        run += sgm * sgm;
      }
      SR = run;
      if (comp == 0) c = (float)(1.0 / sqrt(SR));
      else if (comp == 2) c = (float)sqrt(E / SR);
    }
    prefix_last = E;
    prefix_k = Sk;
    prefix_R = SR;
    sk = k;
    sR = R;
    sc = c;
    sstatus = status;
  }
  __syncthreads();
  if (sstatus == 0) {
    // P[r][l] = c * W[idx_r][l] / sigma_r, sign fixed so the largest |entry| is positive
    const int R = sR;
    const int wave = tid >> 6, lane = tid & 63;
    for (int r = wave; r < R; r += 16) {
      const int colr = idx[r];
      // a direction with no energy carries no eigenvector information: its row stays zero
      const float inv = key[r] > 0.0f ? 1.0f / key[r] : 0.0f;
      float best = -1.0f;
      int bl = 0x7fffffff;
      float bv = 0.0f;
      for (int l = lane; l < L; l += 64) {
        const float v = W[(size_t)colr * ldw + l];
        const float a = fabsf(v);
        if (a > best || (a == best && l < bl)) {
          best = a;
          bl = l;
          bv = v;
        }
      }
      for (int off = 32; off > 0; off >>= 1) {
        const float ob = __shfl_xor(best, off);
        const int ol = __shfl_xor(bl, off);
        const float ov = __shfl_xor(bv, off);
        if (ob > best || (ob == best && ol < bl)) {
          best = ob;
          bl = ol;
          bv = ov;
        }
      }
      const float sgn = bv < 0.0f ? -1.0f : 1.0f;
      const float scale = sgn * sc * inv;
      for (int l = lane; l < L; l += 64) P32[(size_t)r * L + l] = scale * W[(size_t)colr * ldw + l];
    }
  }
  if (tid == 0) {
    info[INFO_STATUS] = sstatus;
    info[INFO_K] = sk;
    info[INFO_R] = sR;
    info[INFO_C] = __float_as_int(sc);
    const double kept = prefix_last > 0.0 ? prefix_R / prefix_last : 0.0;
    const double keptk = prefix_last > 0.0 ? prefix_k / prefix_last : 0.0;
    *reinterpret_cast<double*>(info + INFO_KEPT) = kept;
    *reinterpret_cast<double*>(info + INFO_KEPTK) = keptk;
  }
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

// ============================================================================ eigen driver
// Both sides iterate together; one launch per round, a convergence check per sweep.
// The host reads the convergence flags once per sweep (a stream synchronisation).
struct EigLayout {
  int ldw, nb, ncols;
  size_t wbytes;
};

static EigLayout eig_layout(int L) {
  EigLayout e;
  e.ldw = (L + 15) / 16 * 16;
  int nb = (L + 7) / 8;
  if (nb < 2) nb = 2;
  if (nb & 1) ++nb;
  e.nb = nb;
  e.ncols = nb * 8;
  e.wbytes = ((size_t)e.ncols * e.ldw * sizeof(float) + 255) / 256 * 256;
  return e;
}

// flags block: [0..1] offmax (float), [2..3] active, [4..5] sweeps, [6..7] converged, [8..9] bad,
// [10..13] the two float64 scales ||C||_F^2
constexpr size_t EIG_FLAGS_BYTES = 256;

size_t eig_workspace_bytes(int L) {
  const EigLayout e = eig_layout(L);
  const size_t nrm = ((size_t)L * sizeof(float) + 255) / 256 * 256;
  return 2 * e.wbytes + 2 * nrm + EIG_FLAGS_BYTES;
}

hipError_t run_eig(const double* SX, const double* SG, double inv_nx, double inv_ng, int L, int max_sweeps,
                   void* work, const EigOut& out, int host_flags[10], hipStream_t st) {
  const EigLayout e = eig_layout(L);
  char* base = (char*)work;
  float* W0 = (float*)base;
  float* W1 = (float*)(base + e.wbytes);
  const size_t nrm_bytes = ((size_t)L * sizeof(float) + 255) / 256 * 256;
  float* n0 = (float*)(base + 2 * e.wbytes);
  float* n1 = (float*)(base + 2 * e.wbytes + nrm_bytes);
  int* flags = (int*)(base + 2 * e.wbytes + 2 * nrm_bytes);
  hipError_t err;
  const int init[4] = {0, 0, 1, 1};
  if ((err = launch_zero(flags, EIG_FLAGS_BYTES, st)) != hipSuccess) return err;
  if ((err = launch_fill_i32(flags, init, 4, st)) != hipSuccess) return err;
  hipLaunchKernelGGL(jacobi_prep_kernel, dim3(e.ncols), dim3(256), 0, st, SX, inv_nx, L, e.ldw, e.ncols, W0, flags + 8);
  hipLaunchKernelGGL(jacobi_prep_kernel, dim3(e.ncols), dim3(256), 0, st, SG, inv_ng, L, e.ldw, e.ncols, W1, flags + 9);
  double* scale = (double*)(flags + 10);
  hipLaunchKernelGGL(colnorm_kernel, dim3(L), dim3(64), 0, st, W0, e.ldw, L, n0);
  hipLaunchKernelGGL(colnorm_kernel, dim3(L), dim3(64), 0, st, W1, e.ldw, L, n1);
  hipLaunchKernelGGL(frob_kernel, dim3(1), dim3(256), 0, st, n0, L, scale);
  hipLaunchKernelGGL(frob_kernel, dim3(1), dim3(256), 0, st, n1, L, scale + 1);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  JacobiSide s0{W0, (float*)(flags + 0), flags + 2, scale};
  JacobiSide s1{W1, (float*)(flags + 1), flags + 3, scale + 1};
  // fp32 Gram entries carry a relative rounding error of about sqrt(L) * 2^-24
  const float tol = fmaxf(1e-6f, 8.0f * sqrtf((float)e.ldw) * 5.96e-8f);
  const double rot_tol = 0.25 * (double)tol;
  for (int sweep = 0; sweep < max_sweeps; ++sweep) {
    for (int round = 0; round < e.nb - 1; ++round)
      hipLaunchKernelGGL(jacobi_round_kernel, dim3(e.nb / 2, 2), dim3(256), 0, st, s0, s1, L, e.ldw, e.nb, round,
                         rot_tol);
    hipLaunchKernelGGL(jacobi_check_kernel, dim3(1), dim3(64), 0, st, s0, s1, tol, flags + 4, flags + 6);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = hipMemcpyAsync(host_flags, flags, 10 * sizeof(int), hipMemcpyDeviceToHost, st)) != hipSuccess) return err;
    if ((err = hipStreamSynchronize(st)) != hipSuccess) return err;
    if (host_flags[2] == 0 && host_flags[3] == 0) break;
  }
  hipLaunchKernelGGL(colnorm_kernel, dim3(L), dim3(64), 0, st, W0, e.ldw, L, n0);
  hipLaunchKernelGGL(colnorm_kernel, dim3(L), dim3(64), 0, st, W1, e.ldw, L, n1);
  hipLaunchKernelGGL(truncate_build_kernel, dim3(1), dim3(1024), 0, st, W0, e.ldw, L, n0, out.eps, out.p, out.comp,
                     out.R_max, flags + 8, flags + 6, out.P32, out.sigma_x, out.info_x);
  hipLaunchKernelGGL(truncate_build_kernel, dim3(1), dim3(1024), 0, st, W1, e.ldw, L, n1, out.eps, out.p, out.comp,
                     out.R_max, flags + 9, flags + 7, out.Q32, out.sigma_g, out.info_g);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if ((err = hipMemcpyAsync(host_flags, flags, 10 * sizeof(int), hipMemcpyDeviceToHost, st)) != hipSuccess) return err;
  return hipStreamSynchronize(st);
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
