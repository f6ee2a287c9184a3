// Eigen-decomposition and truncation of the INSTANT statistics (notes "INSTANT:
// Compressing Gradients and Activations for Resource-Efficient Training", sections
// 关键设计 1: the singular vectors of C_X = E[x x^T] / C_G = E[g_y g_y^T]; 关键设计 2:
// energy threshold, oversampling, compensation).
//
// Blocked one-sided (Hestenes) Jacobi. The columns of W = C V0 (V0 orthogonal: the
// identity on the first calibration, the previous calibration's accumulated rotation
// afterwards) are orthogonalised in blocks of 8. A round pairs the blocks by a
// round-robin tournament; each pair forms the 16x16 Gram matrix of its columns on the
// matrix cores, diagonalises it by cyclic Jacobi in float64 and rotates its columns
// (and the same columns of the accumulated V). At convergence W = U Sigma, so the
// column norms are the singular values of C (its eigenvalues, C being PSD) and the
// normalised columns its eigenvectors; V holds the rotation that starts the next
// calibration.
//
// One cooperative launch runs every sweep. Pairs synchronise through per-block
// version counters (a pair waits only for the two column blocks it reads), and all
// blocks meet once per sweep to agree on convergence. Every wait is bounded: a
// timeout raises a global abort flag that releases every other wait, so the grid
// always drains.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace instant {

constexpr int JB = 8;               // columns per Jacobi block
constexpr int JT = 256;             // threads of a Jacobi workgroup (512 measured no faster)
constexpr int JW = JT / 64;         // its waves
constexpr int JAC_MAX_LDW = 2048;   // the 16 columns of a pair are staged in LDS (128 KB)
// Columns whose squared norm is below NOISE_REL * ||C||_F^2 (sigma under 3.2e-5 of sqrt(E))
// are neither rotated nor counted: the singular values the path reports are accurate to
// 1e-4 of sigma_0, and bf16 inputs carry no resolvable energy at that level.
constexpr double NOISE_REL = 1e-9;
constexpr long SPIN_LIMIT = 1L << 24;  // ~1 s of polling before a wait gives up

struct EigLayout {
  int ldw, nb, ncols;
  size_t wbytes, vbytes, nrmbytes, verbytes, colbytes;
  size_t wnbytes;  // subspace solver: staging of C V, SUB_MAX_COLS columns
};

static size_t al256(size_t n) { return (n + 255) / 256 * 256; }

constexpr int SUB_MAX_COLS = 128;  // widest basis the subspace solver takes

static EigLayout eig_layout(int L) {
  EigLayout e;
  e.ldw = (L + 15) / 16 * 16;
  int nb = (L + JB - 1) / JB;
  if (nb < 2) nb = 2;
  if (nb & 1) ++nb;
  e.nb = nb;
  e.ncols = nb * JB;
  e.wbytes = al256((size_t)e.ncols * e.ldw * sizeof(float));
  e.vbytes = al256((size_t)e.ncols * e.ldw * sizeof(double));
  e.nrmbytes = al256((size_t)L * sizeof(float));
  e.verbytes = al256((size_t)2 * nb * sizeof(int));
  e.colbytes = al256((size_t)e.ncols * sizeof(int));
  e.wnbytes = al256((size_t)SUB_MAX_COLS * e.ldw * sizeof(float));
  return e;
}

// flags block (int32 slots)
constexpr int F_OFFMAX = 0;     // [3 slots][2 sides] float bits
constexpr int F_SWEEPS = 6;     // [2]
constexpr int F_CONV = 8;       // [2]
constexpr int F_BAD = 10;       // [2] non-finite statistics
constexpr int F_SCALE = 12;     // 2 doubles: ||C||_F^2 per side
constexpr int F_BARRIER = 16;   // sweep barrier arrivals
constexpr int F_ABORT = 17;     // a bounded wait timed out
constexpr int F_NALIVE = 18;    // [2] columns above the noise floor
constexpr int F_BARRIER2 = 20;  // Gram check arrivals
constexpr int F_INFO = 24;      // [2][INFO_WORDS] copy of each side's info block
constexpr int F_GMAX = 40;      // [3 slots][2 sides] Gram check maxima (float bits)
constexpr int F_EEXACT = 48;    // 2 doubles: ||C||_F^2 per side from the statistic (subspace solver)
constexpr int F_SUBDONE = 52;   // subspace solver: the basis has converged, later steps do nothing
constexpr size_t EIG_FLAGS_BYTES = 256;

struct EigBufs {
  float* W[2];
  float* Wtmp[2];   // statistic in float32 before the warm start product
  float* V32[2];    // the accumulated rotation in float32, for that product
  double* V[2];
  float* nrm[2];
  int* flags;
  int* version;     // [2][nb]
  int* cols[2];     // [ncols] column order: columns above the noise floor first
  float* res[2];    // subspace solver: Ritz residual ||C v_c - sigma_c v_c|| per column
  double* frob;     // subspace solver: per-block sums of ||C||_F^2 [2][SUB_FROB_BLOCKS]
  struct SubScratch* sub;  // subspace solver: basis completion, one per side
  float* Wn[2];            // subspace solver: C V of a step, copied to W unless the basis has converged
};
constexpr size_t EIG_FROB_BYTES = 2 * 64 * sizeof(double);  // [2][SUB_FROB_BLOCKS]

// Basis completion of the subspace solver (per side): the column lists, the Gram-Schmidt
// coefficients of the live columns against the completed (dead) ones, the dead columns'
// Gram matrix and the inverse of its Cholesky factor.
constexpr int SUB_MAX_DEAD = 32;   // near-null basis columns completed per side and step (the rest are zeroed)
struct SubScratch {
  double coef[SUB_MAX_COLS * SUB_MAX_DEAD];  // [live j][dead d]
  double gram[SUB_MAX_DEAD * SUB_MAX_DEAD];  // [dead i][dead d]
  double li[SUB_MAX_DEAD * SUB_MAX_DEAD];    // inverse of the lower Cholesky factor, [row][col]
  int nl, nd_all;                            // live columns; dead columns (of which at most SUB_MAX_DEAD completed)
  int live[SUB_MAX_COLS], dead[SUB_MAX_COLS];
};
constexpr size_t EIG_SUB_BYTES = 2 * ((sizeof(SubScratch) + 255) / 256 * 256);

static EigBufs eig_bufs(void* work, const EigLayout& e) {
  EigBufs b;
  char* p = (char*)work;
  b.W[0] = (float*)p;
  p += e.wbytes;
  b.W[1] = (float*)p;
  p += e.wbytes;
  for (int s = 0; s < 2; ++s) {
    b.Wtmp[s] = (float*)p;
    p += e.wbytes;
  }
  for (int s = 0; s < 2; ++s) {
    b.V32[s] = (float*)p;
    p += e.wbytes;
  }
  b.V[0] = (double*)p;
  p += e.vbytes;
  b.V[1] = (double*)p;
  p += e.vbytes;
  b.nrm[0] = (float*)p;
  p += e.nrmbytes;
  b.nrm[1] = (float*)p;
  p += e.nrmbytes;
  b.flags = (int*)p;
  p += EIG_FLAGS_BYTES;
  b.version = (int*)p;
  p += e.verbytes;
  b.cols[0] = (int*)p;
  p += e.colbytes;
  b.cols[1] = (int*)p;
  p += e.colbytes;
  b.res[0] = (float*)p;
  p += e.nrmbytes;
  b.res[1] = (float*)p;
  p += e.nrmbytes;
  b.frob = (double*)p;
  p += EIG_FROB_BYTES;
  b.sub = (SubScratch*)p;  // EIG_SUB_BYTES: two of them, 256-byte aligned
  p += EIG_SUB_BYTES;
  b.Wn[0] = (float*)p;
  p += e.wnbytes;
  b.Wn[1] = (float*)p;
  return b;
}

size_t eig_workspace_bytes(int L) {
  const EigLayout e = eig_layout(L);
  return 6 * e.wbytes + 2 * e.vbytes + 4 * e.nrmbytes + EIG_FLAGS_BYTES + e.verbytes + 2 * e.colbytes +
         EIG_FROB_BYTES + EIG_SUB_BYTES + 2 * e.wnbytes;
}

// ---------------------------------------------------------------------------- set-up kernels
// The set-up and read-out kernels treat both statistics in one launch: blockIdx.y (or
// blockIdx.x for the one-block kernels) selects the side, 0 = C_X, 1 = C_G.
struct EigSides {
  const double* S[2];  // statistic sums (upper triangle, row-major L x L)
  double inv[2];       // 1 / samples
  float* Wp[2];        // where the prep kernel writes C (W cold, the staging copy warm)
  float* W[2];
  double* V[2];
  float* V32[2];
  float* nrm[2];
  int* cols[2];
  const int* skip;     // subspace solver: when *skip is set the step's kernels return at once (else null)
};

__device__ inline bool skipped(const int* skip) { return skip != nullptr && *skip != 0; }

// W[c][r] = S[min(r,c)][max(r,c)] * inv_n (column-major, zero padding); flags non-finite sums.
// For a warm start it also rounds column c of the accumulated rotation to float32 (V32):
// rounding V only perturbs W = C V at float32 resolution, the rotation itself stays float64.
__global__ __launch_bounds__(256) void jacobi_prep_kernel(EigSides a, int L, int ldw, int warm,
                                                          int* __restrict__ bad) {
  const int c = blockIdx.x, s = blockIdx.y;
  const double* S = a.S[s];
  float* W = a.Wp[s];
  if (warm)
    for (int r = threadIdx.x; r < ldw; r += 256) a.V32[s][(size_t)c * ldw + r] = (float)a.V[s][(size_t)c * ldw + r];
  for (int r = threadIdx.x; r < ldw; r += 256) {
    float v = 0.0f;
    if (r < L && c < L) {
      const int i = r < c ? r : c;
      const int j = r < c ? c : r;
      const double d = S[(size_t)i * L + j] * a.inv[s];
      if (!isfinite(d)) atomicOr(bad + s, 1);
      v = (float)d;
    }
    W[(size_t)c * ldw + r] = v;
  }
}

// V = I (column-major, ncols x ldw).
__global__ __launch_bounds__(256) void identity_kernel(EigSides a, int ldw) {
  const int c = blockIdx.x;
  double* V = a.V[blockIdx.y];
  for (int r = threadIdx.x; r < ldw; r += 256) V[(size_t)c * ldw + r] = (r == c) ? 1.0 : 0.0;
}

// Column norms of W: sigma_c = ||W[:, c]||, c < L.
__global__ __launch_bounds__(64) void colnorm_kernel(EigSides a, int ldw, int L) {
  if (skipped(a.skip)) return;
  const int c = blockIdx.x;
  const float* W = a.W[blockIdx.y];
  const int lane = threadIdx.x;
  float acc = 0.0f;
  for (int r = lane; r < L; r += 64) {
    const float v = W[(size_t)c * ldw + r];
    acc += v * v;
  }
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) a.nrm[blockIdx.y][c] = sqrtf(acc);
}

// ||W||_F^2 from the column norms in a fixed order, then deflation: columns whose squared
// norm is under the noise floor are left out of the tournament (they would never be
// rotated). cols = [columns above the floor in index order, then the others]; n_alive
// counts the first group. One block of 1024 threads per side (blockIdx.x), ncols <= 2048.
__global__ __launch_bounds__(1024) void frob_alive_kernel(EigSides a, double* __restrict__ scale_out, int L,
                                                          int ncols, int* __restrict__ n_alive_out, double noise_rel) {
  if (skipped(a.skip)) return;
  __shared__ int flag[2048];
  __shared__ int sum[1024];
  __shared__ double fro[1024];
  const int side = blockIdx.x;
  const float* nrm = a.nrm[side];
  int* cols = a.cols[side];
  int* n_alive = n_alive_out + side;
  const int tid = threadIdx.x;
  {
    double acc = 0.0;
    for (int c = tid; c < L; c += 1024) acc += (double)nrm[c] * (double)nrm[c];
    fro[tid] = acc;
    __syncthreads();
    for (int st = 512; st > 0; st >>= 1) {
      if (tid < st) fro[tid] += fro[tid + st];
      __syncthreads();
    }
  }
  const double scale = fro[0];
  if (tid == 0) scale_out[side] = scale;
  const double floor_g = noise_rel * scale;
  // two columns per thread (ncols <= 2048)
  int f[2], own = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = 2 * tid + h;
    const double n = (c < L) ? (double)nrm[c] : 0.0;
    f[h] = (c < ncols && c < L && n * n > floor_g) ? 1 : 0;
    if (c < ncols) flag[c] = f[h];
    own += f[h];
  }
  sum[tid] = own;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan of the per-thread counts
    const int v = tid >= off ? sum[tid - off] : 0;
    __syncthreads();
    sum[tid] += v;
    __syncthreads();
  }
  const int total = sum[1023];
  const int before = sum[tid] - own;              // alive columns before this thread's pair
  const int c0 = 2 * tid;
  int apos = before;                              // position among the alive columns
  int dpos = total + (c0 - before);               // position among the others
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = c0 + h;
    if (c < ncols) {
      if (flag[c]) cols[apos++] = c;
      else cols[dpos++] = c;
    }
  }
  if (tid == 0) *n_alive = total;
}

// ---------------------------------------------------------------------------- Jacobi

__device__ inline int tourney(int pos, int round, int nb) {
  // circle method: position 0 fixed, the others rotate by `round`
  return pos == 0 ? 0 : 1 + (pos - 1 + round) % (nb - 1);
}

struct JacobiArgs {
  float* W[2];
  double* V[2];
  const double* scale;  // [2] ||C||_F^2, invariant under the rotations
  unsigned* offmax;     // [3][2]
  int* out;             // [0..1] sweeps, [2..3] converged
  float* nrm[2];        // final column norms (written at the end)
  int* barrier;
  int* barrier2;        // the Gram check's barrier
  unsigned* gmax;       // [3][2] Gram check maxima (float bits)
  int* abort;
  const int* skip;      // subspace solver: set once the basis has converged (the launch returns at once), else null
  int* version;         // [2][nb]
  const int* cols[2];   // column order per side (alive columns first)
  const int* n_alive;   // [2]
  int L, ldw, nb, max_sweeps;
  int nc;               // columns of W whose final norms are written (L, or the subspace width)
  double noise_rel;     // columns under noise_rel * scale are neither rotated nor counted
  float tol, rot_tol;
};

struct JacobiSmem {
  int col[16];
  float part[JW][16][17];
  double G[16][17];
  double V[16][17];
  float npart[2][4 * JW][16];  // Gram check: column norm partials [A/B][wave * 4 + group][column]
  int need;
  int ok;
};

// LDS ordering inside one wave: every lane's earlier LDS access has completed.
__device__ inline void wave_lds_sync() { __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ inline void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// Wait until *p >= v. Gives up (raising the abort flag) after SPIN_LIMIT polls or as soon
// as another block raised it. The polls are relaxed and one acquire fence follows the
// successful one: an acquire per poll would invalidate the XCD's L2 on every iteration,
// under the feet of the blocks still staging their columns.
__device__ bool wait_geq(const int* p, int v, int* abort) {
  for (long it = 0;; ++it) {
    if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= v) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      return true;
    }
    if (__hip_atomic_load(abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return false;
    if (it > SPIN_LIMIT) {
      __hip_atomic_store(abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// One block pair of one side: stage the 16 columns in LDS, form their Gram matrix on the
// matrix cores (float32), diagonalise it by cyclic Jacobi (one wave, float64), and rotate
// the 16 columns of W and of the accumulated V.
__device__ void jacobi_pair(const JacobiArgs& a, int side, int ba, int bb, int slot, JacobiSmem& sm, float* Y) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  float* __restrict__ W = a.W[side];
  double* __restrict__ Vg = a.V[side];
  if (threadIdx.x < 16) sm.col[threadIdx.x] = a.cols[side][(threadIdx.x < 8 ? ba : bb) * JB + (threadIdx.x & 7)];
  __syncthreads();
  const double floor_g = a.noise_rel * a.scale[side];

  // stage the columns, every load issued before any is used
  {
    const int n4 = a.ldw / 4;
    for (int i0 = threadIdx.x; i0 < 16 * n4; i0 += JT * 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * JT;
        if (i < 16 * n4) v[u] = *reinterpret_cast<const f32x4*>(W + (size_t)sm.col[i / n4] * a.ldw + 4 * (i % n4));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * JT;
        if (i < 16 * n4) *reinterpret_cast<f32x4*>(&Y[(i / n4) * a.ldw + 4 * (i % n4)]) = v[u];
      }
    }
  }
  __syncthreads();

  // The accumulated rotation's entries of this thread's first update row, requested now so
  // that their latency hides behind the Gram and the inner solve.
  const int r0 = threadIdx.x;
  double vpre[16];
  if (r0 < a.ldw) {
#pragma unroll
    for (int q = 0; q < 16; ++q) vpre[q] = Vg[(size_t)sm.col[q] * a.ldw + r0];
  }

  // G = Y^T Y: lane i reads four consecutive rows of column (i % 16), the waves take
  // alternate 16-row steps, LDS sums their partial tiles
  {
    const float* __restrict__ cp = Y + (lane & 15) * a.ldw;
    f32x4 acc = zero4();
    for (int r0 = 16 * wave + 4 * (lane >> 4); r0 < a.ldw; r0 += 16 * JW) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(cp + r0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v[0], v[0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v[1], v[1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v[2], v[2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v[3], v[3], acc, 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) sm.part[wave][4 * (lane >> 4) + v][lane & 15] = acc[v];
  }
  __syncthreads();

  if (wave == 0) {
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = lane * 4 + e;
      const int x = idx >> 4, y = idx & 15;
      double g = 0.0;
#pragma unroll
      for (int w = 0; w < JW; ++w) g += (double)sm.part[w][x][y];
      sm.G[x][y] = g;
      sm.V[x][y] = (x == y) ? 1.0 : 0.0;
    }
    wave_lds_sync();
    // the pair's largest relative off-diagonal (columns above the noise floor only)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = lane * 4 + e;
      const int x = idx >> 4, y = idx & 15;
      if (x < y) {
        const double gx = sm.G[x][x], gy = sm.G[y][y];
        if (gx > floor_g && gy > floor_g) m = fmaxf(m, (float)(fabs(sm.G[x][y]) / sqrt(gx * gy)));
      }
    }
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) {
      if (m > 0.0f) atomicMax(a.offmax + slot * 2 + side, __float_as_uint(m));
      sm.need = m > a.rot_tol;
    }
    wave_lds_sync();

    // Inner cyclic Jacobi, at most two sweeps per visit, in circle-method order: in step ir
    // the 16 indices form 8 disjoint pairs, and lane (a, b) = (lane / 8, lane % 8) owns the
    // 2x2 block rows(pair a) x cols(pair b), which the step updates on its own:
    // G <- J_a^T G J_b, V <- V J_b. The diagonal lanes (a == b) hold their pair's 2x2 and
    // choose its rotation. Angles come from float32 arithmetic; each (c, s) is
    // renormalised in float64 so that every accumulated rotation is orthogonal to float64
    // precision.
    const int pa = lane >> 3, pb = lane & 7;
    const double rt2 = (double)a.rot_tol * (double)a.rot_tol;
    for (int isweep = 0; isweep < 2 && sm.need; ++isweep) {
      int rotated = 0;
      for (int ir = 0; ir < 15; ++ir) {
        const int r0 = tourney(pa, ir, 16), r1 = tourney(15 - pa, ir, 16);
        const int c0 = tourney(pb, ir, 16), c1 = tourney(15 - pb, ir, 16);
        const double g00 = sm.G[r0][c0], g01 = sm.G[r0][c1], g10 = sm.G[r1][c0], g11 = sm.G[r1][c1];
        const double v00 = sm.V[r0][c0], v01 = sm.V[r0][c1], v10 = sm.V[r1][c0], v11 = sm.V[r1][c1];
        double c = 1.0, sn = 0.0;
        if (pa == pb && g00 > floor_g && g11 > floor_g && g01 * g01 > rt2 * g00 * g11) {
          // rotate the pair (p, q) = (r0, r1): new p = c p - s q, new q = s p + c q
          const float zeta = (float)((g11 - g00) * 0.5 * __builtin_amdgcn_rcp(g01));
          const float t = copysignf(1.0f, zeta) / (fabsf(zeta) + sqrtf(1.0f + zeta * zeta));
          const float cf = rsqrtf(1.0f + t * t);
          c = (double)cf;
          sn = (double)(t * cf);
          const double dlt = c * c + sn * sn - 1.0;  // |dlt| ~ 1e-7
          const double nrm = 1.0 - 0.5 * dlt + 0.375 * dlt * dlt;
          c *= nrm;
          sn *= nrm;
          rotated = 1;
        }
        const double ca = __shfl(c, 9 * pa), sa = __shfl(sn, 9 * pa);
        const double cb = __shfl(c, 9 * pb), sb = __shfl(sn, 9 * pb);
        const double h00 = cb * g00 - sb * g01, h01 = sb * g00 + cb * g01;
        const double h10 = cb * g10 - sb * g11, h11 = sb * g10 + cb * g11;
        sm.G[r0][c0] = ca * h00 - sa * h10;
        sm.G[r1][c0] = sa * h00 + ca * h10;
        sm.G[r0][c1] = ca * h01 - sa * h11;
        sm.G[r1][c1] = sa * h01 + ca * h11;
        sm.V[r0][c0] = cb * v00 - sb * v01;
        sm.V[r0][c1] = sb * v00 + cb * v01;
        sm.V[r1][c0] = cb * v10 - sb * v11;
        sm.V[r1][c1] = sb * v10 + cb * v11;
        // the next step's blocks hold entries other lanes wrote in this one
        wave_lds_sync();
      }
      if (__ballot(rotated) == 0) break;  // wave-uniform
      // A second sweep starting with every pair under the rotation threshold would rotate
      // nothing: skip it.
      int left = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = lane * 4 + e;
        const int x = idx >> 4, y = idx & 15;
        if (x < y) {
          const double gx = sm.G[x][x], gy = sm.G[y][y], o = sm.G[x][y];
          if (gx > floor_g && gy > floor_g && o * o > rt2 * gx * gy) left = 1;
        }
      }
      if (__ballot(left) == 0) break;
    }
  }
  __syncthreads();
  if (!sm.need) return;

  // Y <- Y V (W from LDS, float64 arithmetic) and V_acc <- V_acc V (float64 in memory)
  for (int r = r0; r < a.ldw; r += JT) {
    float y[16];
    double vv[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      y[q] = Y[q * a.ldw + r];
      vv[q] = (r == r0) ? vpre[q] : Vg[(size_t)sm.col[q] * a.ldw + r];
    }
    double acc[16], accv[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = accv[q] = 0.0;
#pragma unroll 1
    for (int p = 0; p < 16; ++p) {
      const double yp = (double)y[p], vp = vv[p];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const double vpq = sm.V[p][q];  // LDS broadcast
        acc[q] = fma(yp, vpq, acc[q]);
        accv[q] = fma(vp, vpq, accv[q]);
      }
    }
    // device-scope stores write through the L2, so the release that publishes them has
    // little dirty data to write back
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      __hip_atomic_store(W + (size_t)sm.col[q] * a.ldw + r, (float)acc[q], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(Vg + (size_t)sm.col[q] * a.ldw + r, accv[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Convergence check of one side after a sweep: the largest relative off-diagonal
// |G_pq| / sqrt(G_pp G_qq) of the Gram of its alive columns (pairs above the noise floor),
// tile (ti, tj) of 16 columns each (ti <= tj), folded into *gmax. A sweep that left every
// pair at or under the tolerance has converged the side; without this check only the next
// sweep, which would rotate nothing, could tell.
__device__ void gram_check_tile(const JacobiArgs& a, int side, int ti, int tj, JacobiSmem& sm, unsigned* gmax) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  const float* __restrict__ W = a.W[side];
  const int na = a.n_alive[side];
  const int ca = 16 * ti + (lane & 15), cb = 16 * tj + (lane & 15);
  const bool oka = ca < na, okb = cb < na;
  const float* __restrict__ pa = W + (size_t)(oka ? a.cols[side][ca] : 0) * a.ldw;
  const float* __restrict__ pb = W + (size_t)(okb ? a.cols[side][cb] : 0) * a.ldw;
  f32x4 acc = zero4();
  float sa = 0.0f, sb = 0.0f;
  for (int r0 = 16 * wave + 4 * (lane >> 4); r0 < a.ldw; r0 += 16 * JW) {
    const f32x4 va = oka ? *reinterpret_cast<const f32x4*>(pa + r0) : zero4();
    const f32x4 vb = okb ? *reinterpret_cast<const f32x4*>(pb + r0) : zero4();
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(va[g], vb[g], acc, 0, 0, 0);
      sa += va[g] * va[g];
      sb += vb[g] * vb[g];
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) sm.part[wave][4 * (lane >> 4) + v][lane & 15] = acc[v];
  sm.npart[0][wave * 4 + (lane >> 4)][lane & 15] = sa;
  sm.npart[1][wave * 4 + (lane >> 4)][lane & 15] = sb;
  __syncthreads();
  if (wave == 0) {
    const double floor_g = a.noise_rel * a.scale[side];
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = lane * 4 + e;
      const int x = idx >> 4, y = idx & 15;
      if ((ti != tj || x < y) && 16 * ti + x < na && 16 * tj + y < na) {
        double g = 0.0;
#pragma unroll
        for (int w = 0; w < JW; ++w) g += (double)sm.part[w][x][y];
        double nx = 0.0, ny = 0.0;
#pragma unroll
        for (int k = 0; k < 4 * JW; ++k) {
          nx += (double)sm.npart[0][k][x];
          ny += (double)sm.npart[1][k][y];
        }
        if (nx > floor_g && ny > floor_g) m = fmaxf(m, (float)(fabs(g) / sqrt(nx * ny)));
      }
    }
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0 && m > 0.0f) atomicMax(gmax, __float_as_uint(m));
  }
  __syncthreads();
}

// Tile idx of the upper triangle of a T x T grid of tiles, row by row.
__device__ inline void upper_tile_ij(int idx, int T, int& ti, int& tj) {
  ti = 0;
  while (idx >= T - ti) {
    idx -= T - ti;
    ++ti;
  }
  tj = ti + idx;
}

// Block b handles pair (b mod nb/2) of side (b div nb/2) in every round. Round r of the
// whole run (all sweeps counted) may start on column blocks a, b once their version
// counters reached r; the pair then raises both to r + 1. Once per sweep all blocks meet
// at a counting barrier and read the same per-side maxima, so they take the same
// decisions. The maxima rotate over three slots: slot (s+1) mod 3 is cleared during
// sweep s, after every block has read it at the end of sweep s-2.
__global__ __launch_bounds__(JT) void jacobi_kernel(JacobiArgs a) {
  if (skipped(a.skip)) return;  // the same for every block: none waits on another
  __shared__ JacobiSmem sm;
  extern __shared__ float Ydyn[];  // the pair's 16 columns, 16 * ldw floats
  const int nbmax = a.nb;
  const int side = blockIdx.x / (nbmax / 2);
  const int pair = blockIdx.x % (nbmax / 2);
  // this side's tournament: the alive columns, in blocks of 8, an even number of blocks
  int nbs = (a.n_alive[side] + JB - 1) / JB;
  if (nbs < 2) nbs = 2;
  if (nbs & 1) ++nbs;
  const bool mine = pair < nbs / 2;
  int* ver = a.version + side * nbmax;
  int active[2] = {1, 1};
  int sweeps[2] = {0, 0};
  bool aborted = false;
  int rg = 0;  // this side's round index over the whole run
  int checks = 0;
  for (int sweep = 0; sweep < a.max_sweeps && (active[0] || active[1]); ++sweep) {
    const int slot = sweep % 3;
    if (blockIdx.x == 0 && threadIdx.x < 2) {
      __hip_atomic_store(a.offmax + ((sweep + 1) % 3) * 2 + threadIdx.x, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.gmax + ((sweep + 1) % 3) * 2 + threadIdx.x, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    if (active[side] && mine) {
      for (int round = 0; round < nbs - 1; ++round, ++rg) {
        const int ba = tourney(pair, round, nbs);
        const int bb = tourney(nbs - 1 - pair, round, nbs);
        // thread 0 waits and acquires; the barrier orders the other waves' reads after it
        if (threadIdx.x == 0) sm.ok = wait_geq(&ver[ba], rg, a.abort) && wait_geq(&ver[bb], rg, a.abort);
        __syncthreads();
        if (!sm.ok) {
          aborted = true;
          break;
        }
        jacobi_pair(a, side, ba, bb, slot, sm, Ydyn);
        // every wave's column stores have completed before thread 0 releases them
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (threadIdx.x == 0) {
          // one release for both counters (each release-ordered store would write the
          // L2 back again)
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
          __hip_atomic_store(&ver[ba], rg + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(&ver[bb], rg + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    if (aborted) break;
    // sweep barrier (every block of both sides, working or not)
    __syncthreads();
    if (threadIdx.x == 0) {
      __threadfence();
      __hip_atomic_fetch_add(a.barrier, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      sm.ok = wait_geq(a.barrier, (int)gridDim.x * (sweep + 1), a.abort);
    }
    __syncthreads();
    if (!sm.ok) {
      aborted = true;
      break;
    }
    acquire_agent();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (active[s]) {
        sweeps[s] += 1;
        const unsigned bits = __hip_atomic_load(a.offmax + slot * 2 + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__uint_as_float(bits) <= a.tol) active[s] = 0;
      }
    }
    // Gram check of the sides still active; every block takes a share of the tiles
    if (active[0] || active[1]) {
      int nt[2], ntiles[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        nt[s] = (a.n_alive[s] + 15) / 16;
        ntiles[s] = active[s] ? nt[s] * (nt[s] + 1) / 2 : 0;
      }
      for (int t = blockIdx.x; t < ntiles[0] + ntiles[1]; t += gridDim.x) {
        const int s = t < ntiles[0] ? 0 : 1;
        int ti, tj;
        upper_tile_ij(t - (s ? ntiles[0] : 0), nt[s], ti, tj);
        gram_check_tile(a, s, ti, tj, sm, a.gmax + slot * 2 + s);
      }
      checks += 1;
      __syncthreads();
      if (threadIdx.x == 0) {
        __threadfence();
        __hip_atomic_fetch_add(a.barrier2, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        sm.ok = wait_geq(a.barrier2, (int)gridDim.x * checks, a.abort);
      }
      __syncthreads();
      if (!sm.ok) {
        aborted = true;
        break;
      }
      acquire_agent();
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (active[s]) {
          const unsigned bits = __hip_atomic_load(a.gmax + slot * 2 + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (__uint_as_float(bits) <= a.tol) active[s] = 0;
        }
      }
    }
    __syncthreads();  // sm.ok is rewritten in the next sweep
  }
  // Final column norms of both sides (sigma = ||W[:, c]||, c < nc): every block passed the
  // last sweep barrier, so W is complete; one wave per column.
  if (!aborted) {
    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
    for (int q = blockIdx.x * JW + wave; q < 2 * a.nc; q += gridDim.x * JW) {
      const int s = q / a.nc, c = q - s * a.nc;
      const float* __restrict__ col = a.W[s] + (size_t)c * a.ldw;
      float acc = 0.0f;
      for (int r = lane; r < a.L; r += WAVE) acc += col[r] * col[r];
      for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
      if (lane == 0) a.nrm[s][c] = sqrtf(acc);
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.out[0] = sweeps[0];
    a.out[1] = sweeps[1];
    a.out[2] = !active[0] && !aborted;
    a.out[3] = !active[1] && !aborted;
  }
}

// ---------------------------------------------------------------------------- truncation / build

// Device-side info block of one side (int32 slots).
// [0] status [1] k [2] R [3] c (float bits) [4..5] kept (double) [6..7] kept_k (double)
constexpr int MAX_L = 2048;
constexpr int INFO_STATUS = 0, INFO_K = 1, INFO_R = 2, INFO_C = 3, INFO_KEPT = 4, INFO_KEPTK = 6;

// One block of 1024 threads per side: sort the L column norms (descending, ties by column
// index), energy prefix in float64 (a block scan), truncation, compensation and
// P = c * U_R^T.
struct TruncArgs {
  const float* W[2];
  const float* nrm[2];
  float* P32[2];
  float* sigma[2];
  int* info[2];
  float eps;
  int p, comp, R_max;
  int n;                // column norms to rank: L (full decomposition) or the subspace width
  const double* E_ext;  // [2] total energy ||C||_F^2 when only n < L values are known, else null
  const float* res[2];  // Ritz residuals of the n columns (subspace solver), else null
  float res_tol;        // largest residual of a kept direction, relative to sigma_0
};

__global__ __launch_bounds__(1024) void truncate_build_kernel(TruncArgs a, int ldw, int L, int* __restrict__ flags) {
  const int side = blockIdx.x;
  const float* __restrict__ W = a.W[side];
  const float* __restrict__ nrm = a.nrm[side];
  float* __restrict__ P32 = a.P32[side];
  float* __restrict__ sigma_out = a.sigma[side];
  int* __restrict__ info = a.info[side];
  const float eps = a.eps;
  const int p = a.p, comp = a.comp, R_max = a.R_max;
  __shared__ float key[MAX_L];
  __shared__ int idx[MAX_L];
  __shared__ double pre[MAX_L];
  __shared__ double scan[1024];
  __shared__ double prefix_last, prefix_k, prefix_R;
  __shared__ int sk, sR, sstatus, kfirst;
  __shared__ float sc;
  const int tid = threadIdx.x;
  const int n = a.n;  // ranked entries (the spectrum beyond them is known only through E)
  int Lp2 = 1;
  while (Lp2 < n) Lp2 <<= 1;
  for (int i = tid; i < Lp2; i += 1024) {
    key[i] = i < n ? nrm[i] : -1.0f;  // padding sorts last
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
  for (int i = tid; i < L; i += 1024) sigma_out[i] = i < n ? key[i] : 0.0f;

  // float64 prefix of sigma^2 in sorted order: thread t owns entries 2t and 2t+1 and the
  // block scans the pair sums (pre[i] = sum_{j <= i} sigma_j^2)
  {
    const double a0 = 2 * tid < n ? (double)key[2 * tid] * (double)key[2 * tid] : 0.0;
    const double a1 = 2 * tid + 1 < n ? (double)key[2 * tid + 1] * (double)key[2 * tid + 1] : 0.0;
    scan[tid] = a0 + a1;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const double v = tid >= off ? scan[tid - off] : 0.0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const double before = scan[tid] - (a0 + a1);
    if (2 * tid < n) pre[2 * tid] = before + a0;
    if (2 * tid + 1 < n) pre[2 * tid + 1] = before + a0 + a1;
    if (tid == 0) kfirst = n;
    __syncthreads();
    // k = the smallest j with pre[j - 1] >= eps * E
    const double thr = (double)eps * (a.E_ext ? a.E_ext[side] : pre[n - 1]);
    for (int i = tid; i < n; i += 1024)
      if (pre[i] >= thr && (i == 0 || pre[i - 1] < thr)) atomicMin(&kfirst, i);
    __syncthreads();
  }

  if (tid == 0) {
    int status = 0;
    if (flags[F_BAD + side]) status = 6;        // non-finite statistics
    else if (!flags[F_CONV + side]) status = 7;  // no convergence
    const double E = a.E_ext ? a.E_ext[side] : pre[n - 1];
    int k = 0;
    double Sk = 0.0, SR = 0.0;
    if (status == 0 && !(E > 0.0)) status = (E == 0.0) ? 5 : 6;
    if (status == 0) {
      // With all L values known, E = pre[n - 1] and eps <= 1 put the threshold at or below
      // pre[n - 1] (a product by a float no greater than 1 rounds to at most E), so some
      // index always qualifies. Only a subspace basis can miss it: eps * E then lies beyond
      // the n directions it holds.
      if (kfirst < n) {
        k = kfirst + 1;
        Sk = pre[kfirst];
      } else {
        status = 4;
      }
    }
    int R = k + p < L ? k + p : L;
    if (status == 0 && (R > R_max || R > n)) status = 4;
    if (status == 0 && a.res[side]) {
      // every kept direction must be an eigenvector to the residual tolerance
      float worst = 0.0f;
      for (int r = 0; r < R; ++r) worst = fmaxf(worst, a.res[side][idx[r]]);
      if (!(worst <= a.res_tol * key[0])) status = 7;
    }
    float c = 1.0f;
    if (status == 0) {
      SR = pre[R - 1];
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
    // the info block goes to the caller's buffer and to the flags, which the host reads
    int* dst[2] = {info, flags + F_INFO + INFO_WORDS * side};
    const double kept = prefix_last > 0.0 ? prefix_R / prefix_last : 0.0;
    const double keptk = prefix_last > 0.0 ? prefix_k / prefix_last : 0.0;
    for (int d = 0; d < 2; ++d) {
      dst[d][INFO_STATUS] = sstatus;
      dst[d][INFO_K] = sk;
      dst[d][INFO_R] = sR;
      dst[d][INFO_C] = __float_as_int(sc);
      __builtin_memcpy(dst[d] + INFO_KEPT, &kept, 8);
      __builtin_memcpy(dst[d] + INFO_KEPTK, &keptk, 8);
    }
  }
}


// ---------------------------------------------------------------------------- driver

hipError_t run_eig(const double* SX, const double* SG, double inv_nx, double inv_ng, int L, int max_sweeps,
                   bool warm, void* work, const EigOut& out, int host_flags[EIG_HOST_FLAGS], hipStream_t st,
                   bool wait) {
  if (L > JAC_MAX_LDW) return hipErrorInvalidValue;
  const EigLayout e = eig_layout(L);
  const EigBufs b = eig_bufs(work, e);
  int* flags = b.flags;
  double* scale = (double*)(flags + F_SCALE);
  hipError_t err;
  if ((err = launch_zero(flags, EIG_FLAGS_BYTES + e.verbytes, st)) != hipSuccess) return err;
  EigSides sd;
  sd.skip = nullptr;
  sd.S[0] = SX;
  sd.S[1] = SG;
  sd.inv[0] = inv_nx;
  sd.inv[1] = inv_ng;
  for (int s = 0; s < 2; ++s) {
    sd.Wp[s] = warm ? b.Wtmp[s] : b.W[s];
    sd.W[s] = b.W[s];
    sd.V[s] = b.V[s];
    sd.V32[s] = b.V32[s];
    sd.nrm[s] = b.nrm[s];
    sd.cols[s] = b.cols[s];
  }
  hipLaunchKernelGGL(jacobi_prep_kernel, dim3(e.ncols, 2), dim3(256), 0, st, sd, L, e.ldw, warm ? 1 : 0,
                     flags + F_BAD);
  if (warm) {
    // W[c][r] = sum_k V[k][c] C[k][r]: A = V^T stored [ncols][ldw] (k contiguous), B = C
    // stored [k][r] (r contiguous), both float32, on the matrix cores; one batch per side
    if ((err = launch_gemm(false, false, b.V32[0], e.ldw, (size_t)(b.V32[1] - b.V32[0]), b.Wtmp[0], e.ldw,
                           (size_t)(b.Wtmp[1] - b.Wtmp[0]), b.W[0], e.ldw, (size_t)(b.W[1] - b.W[0]), 2, e.ncols,
                           e.ldw, L, st)) != hipSuccess)
      return err;
  } else {
    hipLaunchKernelGGL(identity_kernel, dim3(e.ncols, 2), dim3(256), 0, st, sd, e.ldw);
  }
  hipLaunchKernelGGL(colnorm_kernel, dim3(L, 2), dim3(64), 0, st, sd, e.ldw, L);
  hipLaunchKernelGGL(frob_alive_kernel, dim3(2), dim3(1024), 0, st, sd, scale, L, e.ncols, flags + F_NALIVE,
                     NOISE_REL);
  if ((err = hipGetLastError()) != hipSuccess) return err;

  JacobiArgs ja;
  ja.W[0] = b.W[0];
  ja.W[1] = b.W[1];
  ja.V[0] = b.V[0];
  ja.V[1] = b.V[1];
  ja.scale = scale;
  ja.offmax = (unsigned*)(flags + F_OFFMAX);
  ja.out = flags + F_SWEEPS;
  ja.nrm[0] = b.nrm[0];
  ja.nrm[1] = b.nrm[1];
  ja.barrier = flags + F_BARRIER;
  ja.barrier2 = flags + F_BARRIER2;
  ja.gmax = (unsigned*)(flags + F_GMAX);
  ja.abort = flags + F_ABORT;
  ja.skip = nullptr;
  ja.version = b.version;
  ja.cols[0] = b.cols[0];
  ja.cols[1] = b.cols[1];
  ja.n_alive = flags + F_NALIVE;
  ja.L = L;
  ja.ldw = e.ldw;
  ja.nb = e.nb;
  ja.max_sweeps = max_sweeps;
  ja.nc = L;
  ja.noise_rel = NOISE_REL;
  // fp32 Gram entries carry a relative rounding error of about sqrt(L) * 2^-24
  ja.tol = fmaxf(1e-6f, 8.0f * sqrtf((float)e.ldw) * 5.96e-8f);
  ja.rot_tol = 0.25f * ja.tol;
  void* kargs[] = {&ja};
  const size_t dyn = (size_t)16 * e.ldw * sizeof(float);
  err = hipLaunchCooperativeKernel((const void*)jacobi_kernel, dim3(e.nb), dim3(JT), kargs, dyn, st);
  if (err != hipSuccess) return err;

  TruncArgs ta;
  for (int s = 0; s < 2; ++s) {
    ta.W[s] = b.W[s];
    ta.nrm[s] = b.nrm[s];
  }
  ta.P32[0] = out.P32;
  ta.P32[1] = out.Q32;
  ta.sigma[0] = out.sigma_x;
  ta.sigma[1] = out.sigma_g;
  ta.info[0] = out.info_x;
  ta.info[1] = out.info_g;
  ta.eps = out.eps;
  ta.p = out.p;
  ta.comp = out.comp;
  ta.R_max = out.R_max;
  ta.n = L;
  ta.E_ext = nullptr;
  ta.res[0] = ta.res[1] = nullptr;
  ta.res_tol = 0.0f;
  hipLaunchKernelGGL(truncate_build_kernel, dim3(2), dim3(1024), 0, st, ta, e.ldw, L, flags);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // work that depends on the outcome is queued by the caller before this read-back
  if (out.before_readback && (err = out.before_readback(out.ctx, st)) != hipSuccess) return err;
  if ((err = hipMemcpyAsync(host_flags, flags, EIG_HOST_FLAGS * sizeof(int), hipMemcpyDeviceToHost, st)) != hipSuccess)
    return err;
  if (!wait) return hipSuccess;  // the caller settles the outcome once the stream has passed here
  if ((err = hipStreamSynchronize(st)) != hipSuccess) return err;
  if (host_flags[F_ABORT]) return hipErrorLaunchTimeOut;  // a bounded wait gave up
  return hipSuccess;
}

int eig_max_L() { return JAC_MAX_LDW; }

// ---------------------------------------------------------------------------- subspace solver
// Only the leading eigenpairs decide P and Q: the truncation needs the top k + p of them,
// and the total energy E = ||C||_F^2 comes from C itself (关键设计 2 states the identity
// sum_i sigma_i^2 = ||C||_F^2). Block subspace iteration keeps an L x m basis V (m a little
// above R_max) and repeats
//     W = C V                      (float32 matrix cores)
//     W J = U Sigma                (the one-sided Jacobi above on the m columns)
//     V <- U
// The Jacobi step is the Rayleigh-Ritz step of this iteration: it diagonalises
// (C V)^T (C V) = V^T C^2 V, whose Ritz vectors are those of C since C is PSD, and it
// orthonormalises the basis. V J is the old basis in the Ritz coordinates, so
// sigma_c ||u_c - (V J)_c|| = ||C (V J)_c - sigma_c (V J)_c|| is the residual of the Ritz
// pair, which the truncation bounds for every kept direction. The basis of one
// finalize starts the next; the first starts from pseudo-random columns.

constexpr float SUB_RES_TOL = 3e-5f;  // kept Ritz residuals, relative to sigma_0

int eig_subspace_width(int L, int R_max) {
  const int m = (R_max + 16 + 15) / 16 * 16;  // 16 more directions than the largest rank, whole blocks
  return m < L ? m : 0;                        // 0: the subspace would be the whole space
}

// ||C||_F^2 = sum_i C_ii^2 + 2 sum_{i<j} C_ij^2 from the float64 upper-triangle sums, in a
// fixed order: block b of a side takes the rows i = b mod SUB_FROB_BLOCKS and writes its sum
// to part[side][b]; stat_frob_fold_kernel adds those in block order.
constexpr int SUB_FROB_BLOCKS = 64;
static_assert(EIG_FROB_BYTES == 2 * SUB_FROB_BLOCKS * sizeof(double), "per-block energy sums");
__global__ __launch_bounds__(256) void stat_frob_kernel(EigSides a, int L, double* __restrict__ part) {
  __shared__ double red[256];
  const int side = blockIdx.y, b = blockIdx.x;
  const double* S = a.S[side];
  const double inv = a.inv[side];
  double acc = 0.0;
  for (int i = b; i < L; i += SUB_FROB_BLOCKS) {
    const double* row = S + (size_t)i * L;
    for (int j = i + threadIdx.x; j < L; j += 256) {
      const double v = row[j] * inv;
      acc += (j == i ? 1.0 : 2.0) * v * v;
    }
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[side * SUB_FROB_BLOCKS + b] = red[0];
}

__global__ void stat_frob_fold_kernel(const double* __restrict__ part, double* __restrict__ out) {
  const int side = threadIdx.x;
  if (side < 2) {
    double e = 0.0;
    for (int b = 0; b < SUB_FROB_BLOCKS; ++b) e += part[side * SUB_FROB_BLOCKS + b];
    out[side] = e;
  }
}

// Pseudo-random starting basis (a counter-based hash of row, column and side, uniform in
// [-1, 1)), zero in the padding rows.
__global__ __launch_bounds__(256) void seed_basis_kernel(EigSides a, int L, int ldw) {
  const int c = blockIdx.x, s = blockIdx.y;
  for (int r = threadIdx.x; r < ldw; r += 256) {
    unsigned h = (unsigned)(r + 1) * 0x9E3779B1u ^ (unsigned)(c + 1) * 0x85EBCA77u ^ (unsigned)(s + 1) * 0xC2B2AE3Du;
    h ^= h >> 15;
    h *= 0x2C1B3C6Du;
    h ^= h >> 12;
    h *= 0x297A2D39u;
    h ^= h >> 15;
    a.V32[s][(size_t)c * ldw + r] = r < L ? (float)(h >> 8) * (2.0f / 16777216.0f) - 1.0f : 0.0f;
  }
}

// Before each Jacobi launch: clear its counters, maxima and outputs, keep the statistics'
// non-finite flags, the exact energies and an abort (a later launch then ends at once and
// the host sees it); copy the basis to the float64 matrix the Jacobi rotates along with W.
__global__ __launch_bounds__(256) void sub_reset_kernel(EigSides a, int* __restrict__ flags, int* __restrict__ version,
                                                        int nver, int ldw) {
  if (skipped(a.skip)) return;
  const int c = blockIdx.x, s = blockIdx.y;
  if (c == 0 && s == 0) {
    for (int i = threadIdx.x; i < F_INFO; i += 256)
      if (i != F_BAD && i != F_BAD + 1 && i != F_ABORT) flags[i] = 0;
    for (int i = threadIdx.x; i < 6; i += 256) flags[F_GMAX + i] = 0;
    for (int i = threadIdx.x; i < nver; i += 256) version[i] = 0;
  }
  for (int r = threadIdx.x; r < ldw; r += 256) a.V[s][(size_t)c * ldw + r] = (double)a.V32[s][(size_t)c * ldw + r];
}

// After each Jacobi launch: the new basis u_c = W[:, c] / sigma_c and the Ritz residual
// sigma_c ||u_c - (V J)_c||. Columns under the noise floor were not rotated: their basis
// column stays as it was, for the completion kernels to make orthogonal to the new one.
__global__ __launch_bounds__(256) void sub_normalize_kernel(EigSides a, const double* __restrict__ scale, float* res0,
                                                            float* res1, int ldw) {
  if (skipped(a.skip)) return;
  __shared__ double part[256];
  const int c = blockIdx.x, s = blockIdx.y;
  const float sig = a.nrm[s][c];
  const bool live = (double)sig * (double)sig > NOISE_REL * scale[s];
  const float inv = sig > 0.0f ? 1.0f / sig : 0.0f;
  double d2 = 0.0;
  for (int r = threadIdx.x; r < ldw; r += 256) {
    const float u = a.W[s][(size_t)c * ldw + r] * inv;
    const double diff = (double)u - a.V[s][(size_t)c * ldw + r];
    d2 += diff * diff;
    if (live) a.V32[s][(size_t)c * ldw + r] = u;
  }
  part[threadIdx.x] = d2;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (threadIdx.x < st) part[threadIdx.x] += part[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) (s ? res1 : res0)[c] = sig * (float)sqrt(part[0]);
}

// Basis completion after a step. The columns under the noise floor ("dead": their
// directions carry no energy, so any orthonormal completion will do) are made orthogonal to
// the live columns by two passes of classical Gram-Schmidt, then orthonormal among
// themselves through the Cholesky factor of their Gram matrix, all in float64. A column
// that falls into the span of the others, and every dead column beyond SUB_MAX_DEAD, becomes
// zero; a zero column stays zero (C 0 = 0) and is never kept. The work is spread over many
// compute units in five short kernels: lists, dots (one block per column), row updates and
// the row transform (blocks of rows), and the factorisation (one wave per side).

// Column lists from the norms the Jacobi left: live columns in index order, then dead ones
// (one wave per side; a ballot gives each column its place).
__global__ __launch_bounds__(WAVE) void sub_lists_kernel(EigSides a, const double* __restrict__ scale, int m,
                                                         SubScratch* __restrict__ sub) {
  if (skipped(a.skip)) return;
  const int side = blockIdx.x, lane = threadIdx.x;
  SubScratch& S = sub[side];
  const double floor_g = NOISE_REL * scale[side];
  const unsigned long long below = (1ull << lane) - 1ull;
  int nl = 0, nd = 0;
  for (int c0 = 0; c0 < m; c0 += WAVE) {
    const int c = c0 + lane;
    const bool in = c < m;
    const double sg = in ? (double)a.nrm[side][c] : 0.0;
    const bool live = in && sg * sg > floor_g;
    const unsigned long long lm = __ballot(live), dm = __ballot(in && !live);
    if (live) S.live[nl + __popcll(lm & below)] = c;
    else if (in) S.dead[nd + __popcll(dm & below)] = c;
    nl += __popcll(lm);
    nd += __popcll(dm);
  }
  if (lane == 0) {
    S.nl = nl;
    S.nd_all = nd;
  }
}

// Dots of one column against every completed dead column: block j takes live column j
// (gram = 0, the Gram-Schmidt coefficients) or dead column j (gram = 1, the Gram matrix).
// Each thread sums its rows in order, each wave by a fixed shuffle tree, the waves in order.
constexpr int SUB_DT = 256;
__global__ __launch_bounds__(SUB_DT) void sub_dots_kernel(EigSides a, SubScratch* __restrict__ sub, int gram, int L,
                                                          int ldw) {
  if (skipped(a.skip)) return;
  const int side = blockIdx.y, j = blockIdx.x;
  SubScratch& S = sub[side];
  const int nd = S.nd_all < SUB_MAX_DEAD ? S.nd_all : SUB_MAX_DEAD;
  const int cnt = gram ? nd : S.nl;
  if (nd == 0 || j >= cnt) return;
  __shared__ int dl[SUB_MAX_DEAD];
  if (threadIdx.x < SUB_MAX_DEAD) dl[threadIdx.x] = threadIdx.x < nd ? S.dead[threadIdx.x] : 0;
  __syncthreads();
  const float* __restrict__ V = a.V32[side];
  const float* __restrict__ x = V + (size_t)(gram ? S.dead[j] : S.live[j]) * ldw;
  double acc[SUB_MAX_DEAD];
#pragma unroll
  for (int d = 0; d < SUB_MAX_DEAD; ++d) acc[d] = 0.0;
  for (int r = threadIdx.x; r < L; r += SUB_DT) {
    const double xr = (double)x[r];
#pragma unroll
    for (int d = 0; d < SUB_MAX_DEAD; ++d)
      if (d < nd) acc[d] += xr * (double)V[(size_t)dl[d] * ldw + r];
  }
  __shared__ double part[SUB_DT / WAVE][SUB_MAX_DEAD];
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
#pragma unroll
  for (int d = 0; d < SUB_MAX_DEAD; ++d) {
    if (d < nd) {  // (the same for every lane; no early exit, so acc stays in registers)
      double v = acc[d];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
      if (lane == 0) part[wave][d] = v;
    }
  }
  __syncthreads();
  if (threadIdx.x < nd) {
    double v = part[0][threadIdx.x];
    for (int w = 1; w < SUB_DT / WAVE; ++w) v += part[w][threadIdx.x];
    (gram ? S.gram : S.coef)[j * SUB_MAX_DEAD + threadIdx.x] = v;
  }
}

// One Gram-Schmidt pass over a block of rows: v_d -= sum_j coef[j][d] u_j, the live columns
// in order, eight loads at a time.
constexpr int SUB_RT = 256;
__global__ __launch_bounds__(SUB_RT) void sub_update_kernel(EigSides a, SubScratch* __restrict__ sub, int L, int ldw) {
  if (skipped(a.skip)) return;
  const int side = blockIdx.y;
  SubScratch& S = sub[side];
  const int nd = S.nd_all < SUB_MAX_DEAD ? S.nd_all : SUB_MAX_DEAD;
  const int nl = S.nl;
  if (nd == 0) return;
  __shared__ double cf[SUB_MAX_COLS * SUB_MAX_DEAD];
  for (int e = threadIdx.x; e < nl * SUB_MAX_DEAD; e += SUB_RT) cf[e] = S.coef[e];
  __syncthreads();
  const int r = blockIdx.x * SUB_RT + threadIdx.x;
  if (r >= L) return;
  float* __restrict__ V = a.V32[side];
  double v[SUB_MAX_DEAD];
#pragma unroll
  for (int d = 0; d < SUB_MAX_DEAD; ++d) v[d] = d < nd ? (double)V[(size_t)S.dead[d] * ldw + r] : 0.0;
  constexpr int JU = 8;
  for (int j0 = 0; j0 < nl; j0 += JU) {
    float u[JU];
#pragma unroll
    for (int q = 0; q < JU; ++q) u[q] = j0 + q < nl ? V[(size_t)S.live[j0 + q] * ldw + r] : 0.0f;
#pragma unroll
    for (int q = 0; q < JU; ++q) {
      if (j0 + q >= nl) break;
#pragma unroll
      for (int d = 0; d < SUB_MAX_DEAD; ++d) v[d] -= cf[(j0 + q) * SUB_MAX_DEAD + d] * (double)u[q];
    }
  }
#pragma unroll
  for (int d = 0; d < SUB_MAX_DEAD; ++d)
    if (d < nd) V[(size_t)S.dead[d] * ldw + r] = (float)v[d];
}

// Cholesky factor of the dead columns' Gram matrix and its inverse, one wave per side. Lane
// i holds row i of the factor, lane c column c of the inverse; the entries they need from
// other lanes are broadcast across the wave. Every entry is formed by the same subtractions
// in the same order as the left-looking factorisation and the forward substitution.
__device__ inline double lane_value(double v, int lane) {  // v of one lane (a uniform index), to every lane
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), lane);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), lane);
  return __hiloint2double(hi, lo);
}

__global__ __launch_bounds__(WAVE) void sub_chol_kernel(SubScratch* __restrict__ sub, const int* __restrict__ skip) {
  if (skipped(skip)) return;
  SubScratch& S = sub[blockIdx.x];
  const int nd = S.nd_all < SUB_MAX_DEAD ? S.nd_all : SUB_MAX_DEAD;
  if (nd == 0) return;
  const int i = threadIdx.x;
  double l[SUB_MAX_DEAD];  // row i of the Gram matrix, then of its lower Cholesky factor
#pragma unroll
  for (int k = 0; k < SUB_MAX_DEAD; ++k) l[k] = (i < nd && k <= i) ? S.gram[i * SUB_MAX_DEAD + k] : 0.0;
#pragma unroll
  for (int j = 0; j < SUB_MAX_DEAD; ++j) {
    if (j < nd) {
      // the columns had unit norm before the projections: a pivot this small means the
      // column lies in the span of the others, and its column of the factor is zero
      const double sjj = lane_value(l[j], j);
      const double ljj = sjj > 1e-8 ? sqrt(sjj) : 0.0;
      if (i == j) l[j] = ljj;
      else if (i > j) l[j] = ljj > 0.0 ? l[j] / ljj : 0.0;
#pragma unroll
      for (int k = 0; k < SUB_MAX_DEAD; ++k) {
        if (k > j && k < nd) {
          const double lkj = lane_value(l[j], k);
          if (i >= k) l[k] -= l[j] * lkj;
        }
      }
    }
  }
  // column c of L^-1 (lane c) by forward substitution, row l_i broadcast from lane i; a zero
  // pivot zeroes its row
  const int c = i;
  double x[SUB_MAX_DEAD];
#pragma unroll
  for (int r = 0; r < SUB_MAX_DEAD; ++r) {
    x[r] = 0.0;
    if (r < nd) {
      double v = r == c ? 1.0 : 0.0;
#pragma unroll
      for (int k = 0; k < SUB_MAX_DEAD; ++k) {
        if (k < r) {
          const double lrk = lane_value(l[k], r);
          if (k >= c) v -= lrk * x[k];
        }
      }
      const double lrr = lane_value(l[r], r);
      if (r >= c) x[r] = lrr > 0.0 ? v / lrr : 0.0;
    }
  }
  if (c < nd)
#pragma unroll
    for (int r = 0; r < SUB_MAX_DEAD; ++r)
      if (r < nd) S.li[r * SUB_MAX_DEAD + c] = x[r];
}

// Rows of the completed dead block times L^-T (every load of a row before any store), and
// the dead columns beyond SUB_MAX_DEAD set to zero.
__global__ __launch_bounds__(SUB_RT) void sub_transform_kernel(EigSides a, SubScratch* __restrict__ sub, int L,
                                                               int ldw) {
  if (skipped(a.skip)) return;
  const int side = blockIdx.y;
  SubScratch& S = sub[side];
  const int nd_all = S.nd_all;
  const int nd = nd_all < SUB_MAX_DEAD ? nd_all : SUB_MAX_DEAD;
  if (nd == 0) return;
  __shared__ double li[SUB_MAX_DEAD * SUB_MAX_DEAD];
  for (int e = threadIdx.x; e < nd * SUB_MAX_DEAD; e += SUB_RT) li[e] = S.li[e];
  __syncthreads();
  const int r = blockIdx.x * SUB_RT + threadIdx.x;
  if (r >= L) return;
  float* __restrict__ V = a.V32[side];
  for (int i = nd; i < nd_all; ++i) V[(size_t)S.dead[i] * ldw + r] = 0.0f;
  double v[SUB_MAX_DEAD];
#pragma unroll
  for (int d = 0; d < SUB_MAX_DEAD; ++d) v[d] = d < nd ? (double)V[(size_t)S.dead[d] * ldw + r] : 0.0;
  for (int d = 0; d < nd; ++d) {
    double y = 0.0;
#pragma unroll
    for (int k = 0; k < SUB_MAX_DEAD; ++k)  // (constant k: v stays in registers)
      if (k <= d) y += li[d * SUB_MAX_DEAD + k] * v[k];
    V[(size_t)S.dead[d] * ldw + r] = (float)y;
  }
}

// W <- C V of this step, unless the basis has already converged (then W, the norms and the
// residuals of the converged step stay as they are for the truncation).
__global__ __launch_bounds__(256) void sub_commit_kernel(EigSides a, float* Wn0, float* Wn1, int ldw) {
  if (skipped(a.skip)) return;
  const int c = blockIdx.x, s = blockIdx.y;
  const float* __restrict__ src = (s ? Wn1 : Wn0) + (size_t)c * ldw;
  float* __restrict__ dst = a.W[s] + (size_t)c * ldw;
  for (int r = threadIdx.x; r < ldw; r += 256) dst[r] = src[r];
}

// After a step: the basis has converged when, on both sides, every column among the R_max
// largest has a Ritz residual within tol * sigma_0 (the truncation keeps at most R_max of
// them and applies the same test to those it keeps). Later steps then do nothing.
__global__ __launch_bounds__(SUB_MAX_COLS) void sub_check_kernel(EigSides a, const float* __restrict__ res0,
                                                                 const float* __restrict__ res1, int m, int R_max,
                                                                 float tol, int* __restrict__ done) {
  if (*done) return;
  __shared__ int fail;
  if (threadIdx.x == 0) fail = 0;
  __syncthreads();
  const int c = threadIdx.x;
  for (int side = 0; side < 2; ++side) {
    const float* __restrict__ nrm = a.nrm[side];
    const float* __restrict__ res = side ? res1 : res0;
    if (c < m) {
      float sig0 = 0.0f;
      int rank = 0;
      const float sc = nrm[c];
      for (int k = 0; k < m; ++k) {
        const float sk = nrm[k];
        sig0 = fmaxf(sig0, sk);
        rank += (sk > sc) || (sk == sc && k < c);
      }
      if (rank < R_max && !(res[c] <= tol * sig0)) fail = 1;  // (a NaN residual fails too)
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && !fail) *done = 1;
}

static hipError_t launch_sub_complete(const EigSides& sd, const double* scale, SubScratch* sub, int m, int L, int ldw,
                                      hipStream_t st) {
  const dim3 rows((L + SUB_RT - 1) / SUB_RT, 2);
  hipLaunchKernelGGL(sub_lists_kernel, dim3(2), dim3(WAVE), 0, st, sd, scale, m, sub);
  for (int pass = 0; pass < 2; ++pass) {
    hipLaunchKernelGGL(sub_dots_kernel, dim3(m, 2), dim3(SUB_DT), 0, st, sd, sub, 0, L, ldw);
    hipLaunchKernelGGL(sub_update_kernel, rows, dim3(SUB_RT), 0, st, sd, sub, L, ldw);
  }
  hipLaunchKernelGGL(sub_dots_kernel, dim3(SUB_MAX_DEAD < m ? SUB_MAX_DEAD : m, 2), dim3(SUB_DT), 0, st, sd, sub, 1,
                     L, ldw);
  hipLaunchKernelGGL(sub_chol_kernel, dim3(2), dim3(WAVE), 0, st, sub, sd.skip);
  hipLaunchKernelGGL(sub_transform_kernel, rows, dim3(SUB_RT), 0, st, sd, sub, L, ldw);
  return hipGetLastError();
}

hipError_t run_eig_subspace(const double* SX, const double* SG, double inv_nx, double inv_ng, int L, int m,
                            int iters, int max_sweeps, bool warm, void* work, const EigOut& out,
                            int host_flags[EIG_HOST_FLAGS], hipStream_t st, bool wait) {
  // (the completion's column lists hold at most SUB_MAX_COLS columns)
  if (L > JAC_MAX_LDW || m < 16 || m % 16 || m >= L || m > SUB_MAX_COLS || iters < 1) return hipErrorInvalidValue;
  const EigLayout e = eig_layout(L);
  const EigBufs b = eig_bufs(work, e);
  int* flags = b.flags;
  double* scale = (double*)(flags + F_SCALE);
  double* eexact = (double*)(flags + F_EEXACT);
  hipError_t err;
  if ((err = launch_zero(flags, EIG_FLAGS_BYTES + e.verbytes, st)) != hipSuccess) return err;
  EigSides sd;
  sd.skip = flags + F_SUBDONE;
  sd.S[0] = SX;
  sd.S[1] = SG;
  sd.inv[0] = inv_nx;
  sd.inv[1] = inv_ng;
  for (int s = 0; s < 2; ++s) {
    sd.Wp[s] = b.Wtmp[s];  // C in float32, kept for every iteration's product
    sd.W[s] = b.W[s];
    sd.V[s] = b.V[s];
    sd.V32[s] = b.V32[s];  // the basis; its first m columns carry over between finalizes
    sd.nrm[s] = b.nrm[s];
    sd.cols[s] = b.cols[s];
  }
  hipLaunchKernelGGL(jacobi_prep_kernel, dim3(e.ncols, 2), dim3(256), 0, st, sd, L, e.ldw, 0, flags + F_BAD);
  hipLaunchKernelGGL(stat_frob_kernel, dim3(SUB_FROB_BLOCKS, 2), dim3(256), 0, st, sd, L, b.frob);
  hipLaunchKernelGGL(stat_frob_fold_kernel, dim3(1), dim3(64), 0, st, (const double*)b.frob, eexact);
  if (!warm) hipLaunchKernelGGL(seed_basis_kernel, dim3(m, 2), dim3(256), 0, st, sd, L, e.ldw);
  if ((err = hipGetLastError()) != hipSuccess) return err;

  const int nb = m / JB;  // even: m is a multiple of 16
  JacobiArgs ja;
  ja.W[0] = b.W[0];
  ja.W[1] = b.W[1];
  ja.V[0] = b.V[0];
  ja.V[1] = b.V[1];
  ja.scale = scale;
  ja.offmax = (unsigned*)(flags + F_OFFMAX);
  ja.out = flags + F_SWEEPS;
  ja.nrm[0] = b.nrm[0];
  ja.nrm[1] = b.nrm[1];
  ja.barrier = flags + F_BARRIER;
  ja.barrier2 = flags + F_BARRIER2;
  ja.gmax = (unsigned*)(flags + F_GMAX);
  ja.abort = flags + F_ABORT;
  ja.skip = flags + F_SUBDONE;
  ja.version = b.version;
  ja.cols[0] = b.cols[0];
  ja.cols[1] = b.cols[1];
  ja.n_alive = flags + F_NALIVE;
  ja.L = L;
  ja.ldw = e.ldw;
  ja.nb = nb;
  ja.nc = m;
  // Columns under the noise floor are not rotated (their near-degenerate directions would
  // keep the tournament busy for nothing); the completion kernels make them orthonormal to the
  // rest afterwards, so the next step's basis is orthonormal.
  ja.noise_rel = NOISE_REL;
  ja.max_sweeps = max_sweeps;
  ja.tol = fmaxf(1e-6f, 8.0f * sqrtf((float)e.ldw) * 5.96e-8f);
  ja.rot_tol = 0.25f * ja.tol;
  void* kargs[] = {&ja};
  const size_t dyn = (size_t)16 * e.ldw * sizeof(float);
  for (int it = 0; it < iters; ++it) {
    hipLaunchKernelGGL(sub_reset_kernel, dim3(m, 2), dim3(256), 0, st, sd, flags, b.version, 2 * nb, e.ldw);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // W[c][r] = sum_k V[k][c] C[k][r]: A = V^T [m][ldw] (k contiguous), B = C [k][r]
    if ((err = launch_gemm(false, false, b.V32[0], e.ldw, (size_t)(b.V32[1] - b.V32[0]), b.Wtmp[0], e.ldw,
                           (size_t)(b.Wtmp[1] - b.Wtmp[0]), b.Wn[0], e.ldw, (size_t)(b.Wn[1] - b.Wn[0]), 2, m, e.ldw,
                           L, st)) != hipSuccess)
      return err;
    hipLaunchKernelGGL(sub_commit_kernel, dim3(m, 2), dim3(256), 0, st, sd, b.Wn[0], b.Wn[1], e.ldw);
    hipLaunchKernelGGL(colnorm_kernel, dim3(m, 2), dim3(64), 0, st, sd, e.ldw, L);
    hipLaunchKernelGGL(frob_alive_kernel, dim3(2), dim3(1024), 0, st, sd, scale, m, m, flags + F_NALIVE,
                       NOISE_REL);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    err = hipLaunchCooperativeKernel((const void*)jacobi_kernel, dim3(nb), dim3(JT), kargs, dyn, st);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(sub_normalize_kernel, dim3(m, 2), dim3(256), 0, st, sd, scale, b.res[0], b.res[1], e.ldw);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = launch_sub_complete(sd, scale, b.sub, m, L, e.ldw, st)) != hipSuccess) return err;
    if (it + 1 < iters)
      hipLaunchKernelGGL(sub_check_kernel, dim3(1), dim3(SUB_MAX_COLS), 0, st, sd, b.res[0], b.res[1], m,
                         out.R_max, SUB_RES_TOL, flags + F_SUBDONE);
  }

  TruncArgs ta;
  for (int s = 0; s < 2; ++s) {
    ta.W[s] = b.W[s];
    ta.nrm[s] = b.nrm[s];
    ta.res[s] = b.res[s];
  }
  ta.P32[0] = out.P32;
  ta.P32[1] = out.Q32;
  ta.sigma[0] = out.sigma_x;
  ta.sigma[1] = out.sigma_g;
  ta.info[0] = out.info_x;
  ta.info[1] = out.info_g;
  ta.eps = out.eps;
  ta.p = out.p;
  ta.comp = out.comp;
  ta.R_max = out.R_max;
  ta.n = m;
  ta.E_ext = eexact;
  ta.res_tol = SUB_RES_TOL;
  hipLaunchKernelGGL(truncate_build_kernel, dim3(2), dim3(1024), 0, st, ta, e.ldw, L, flags);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (out.before_readback && (err = out.before_readback(out.ctx, st)) != hipSuccess) return err;
  if ((err = hipMemcpyAsync(host_flags, flags, EIG_HOST_FLAGS * sizeof(int), hipMemcpyDeviceToHost, st)) != hipSuccess)
    return err;
  if (!wait) return hipSuccess;
  if ((err = hipStreamSynchronize(st)) != hipSuccess) return err;
  if (host_flags[F_ABORT]) return hipErrorLaunchTimeOut;
  return hipSuccess;
}

}  // namespace instant
