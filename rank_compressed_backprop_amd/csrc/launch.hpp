// Host-side launchers of the INSTANT kernels. Each returns the launch status; all
// work is enqueued on `st`. Pointers are device pointers; the I/O dtype is bf16
// when `bf16_io` is true, float32 otherwise.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace instant {

// Out[b][m][c] = sum_l A[m][l] X[b][l][c]; rows m < M0 to out0 [B][M0][C], the rest
// to out1 [B][M-M0][C]. A: [M][ldA], zero beyond column L, ldA a multiple of 32. M <= 128.
// zpad: 16 zero bytes in device memory (bf16 inputs stream through LDS reading it in place
// of out-of-range rows; without it they take the register-blocked kernel).
hipError_t launch_proj(bool bf16_io, const void* A, int ldA, int M, int M0, const void* X, int B, int L, int C,
                       void* out0, void* out1, const void* zpad, hipStream_t st);

// Cm[m][n] = sum_k A(m,k) B[k][n] per batch entry z (pointer strides sA, sB, sC in
// elements). a_trans: A stored [K][lda] instead of [M][lda]. M, N multiples of 4 / 8.
// part (room for part_floats float32) and zpad (16 zero bytes in device memory), when given,
// let a bf16 GEMM whose B is too large for L2 read B once over K slices (gemm_ws_slices).
hipError_t launch_gemm(bool bf16_io, bool a_trans, const void* A, int lda, size_t sA, const void* Bm, int ldb,
                       size_t sB, void* Cm, int ldc, size_t sC, int batch, int M, int N, int K, hipStream_t st,
                       float* part = nullptr, size_t part_floats = 0, const void* zpad = nullptr);
// K slices (0: not used) of that path for these shapes; it needs S * M * N floats of part.
int gemm_ws_slices(bool bf16_io, bool a_trans, int M, int N, int K);
// That path's slices alone (bf16, A [M][lda]): part[z][m][n] for the S = gemm_ws_slices(true,
// false, M, N, K) > 0 slices, left for launch_expand_parts to add; needs S * M * N floats.
hipError_t launch_gemm_ws_parts(const void* A, int lda, const void* Bm, int ldb, float* part, size_t part_floats,
                                int M, int N, int K, const void* zpad, hipStream_t st);

// bf16 C[M][N] = sum_k A(m,k) B[k][n] on LDS-staged 128 x 128 tiles (kernels_gemm.hip).
// a_kmajor: A stored [K][lda] (m contiguous), else [M][lda]; B stored [K][ldb]. N % 8 == 0,
// and M % 8 == 0 (k-major A) or K % 8 == 0 (m-major A). When K is split into S > 1 slices
// (gemm_tiled_slices) the float32 partials need gemm_tiled_part_floats(M, N, K) floats of
// part. zpad: 16 zero bytes in device memory.
int gemm_tiled_slices(int M, int N, int K);
// Whether the tiled kernel is the faster choice for these shapes (and supports them).
bool gemm_tiled_applies(bool a_kmajor, int M, int N, int K);
size_t gemm_tiled_part_floats(int M, int N, int K);
hipError_t launch_gemm_tiled(bool a_kmajor, const void* A, int lda, const void* Bm, int ldb, void* Cm, int ldc, int M,
                             int N, int K, float* part, size_t part_floats, const void* zpad, hipStream_t st);

// Out[b][l][c] = sum_{r<R} At[l][r] Bz[b][r][c]; At: [L][ldA], zero beyond column R.
hipError_t launch_expand(bool bf16_io, const void* At, int ldA, const void* Bz, int B, int R, int L, int C,
                         void* out, hipStream_t st);
// The same (bf16) with Bz given as the S float32 slices part[z][b * R + r][c] of
// launch_gemm_ws_parts, added in slice order and rounded as the slices' reduction would round
// them (identical output). 1 <= S <= 16, R <= 64, C % 8 == 0, ldA >= 64.
hipError_t launch_expand_parts(const void* At, int ldA, const float* part, int S, int B, int R, int L, int C, void* out,
                               hipStream_t st);

// gx[b][l][c] = sum_r At[l][r] (sum_k Qgy[b][r][k] w[k][c]) with g_hat_x kept in LDS
// (rounded to the I/O dtype), and g_w = sum_b Pgy_b^T xhat_b (Pgy [Kw][Cy], xhat [Kw][Cx],
// Kw = B * Rx), in one launch. Applies when w is small enough to stay in L2. `ncu` is the
// device's compute unit count, which sizes the grid.
bool gx_fused_applies(bool bf16_io, int B, int Cx, int Cy);
hipError_t launch_bwd_tail(bool bf16_io, const void* Qgy, const void* w, const void* At, int ldA, int B, int R, int L,
                           int Cy, int Cx, void* gx, const void* Pgy, const void* xhat, void* gw, int Kw, int ncu,
                           hipStream_t st);

// ---- calibration ([KD1], [KD2])

// One statistic of a batch: S += sum_b X_b X_b^T for X [B][L][C] (float64 upper-triangle
// tiles of S), through nsplit slices of the batch*channel reduction whose float32 partial
// tiles go to part [nsplit][ntiles][128*128], summed into S in slice order.
struct SyrkSide {
  const void* X;
  int C, nsplit;
  float* part;
  double* S;
  int overwrite;  // S = the batch's sum instead of S += it (the first batch of a window)
};
// The statistics of one batch: one or two sides in one SYRK launch, then one reduction
// launch. zpad: 256 zero bytes in device memory (read in place of out-of-range data).
hipError_t launch_syrk(bool bf16_io, const SyrkSide* sides, int nsides, int B, int L, const void* zpad,
                       hipStream_t st);
int syrk_tiles(int L);
// With L <= 64 the statistics take one 64 x 64 tile and nsplit is not used: a side's partials
// need syrk_small_part_floats(bf16_io, B, C) floats of its part region.
size_t syrk_small_part_floats(bool bf16_io, int B, int C);

// Eigen-decomposition of both statistics (C = S * inv_n, float64 upper-triangle sums)
// by blocked one-sided Jacobi, then truncation, compensation and the float32
// projections P32 [Rx][L] / Q32 [Ry][L], the descending spectra and the per-side
// device info blocks (int32 slots: status, k, R, c bits, kept (f64), kept_k (f64)).
// warm: start from the rotation accumulated by the previous call (kept in `work`).
// host_flags receives the first EIG_HOST_FLAGS int32 slots of the flags block (see
// kernels_eig.hip) through a copy queued on `st`. wait: synchronise the stream at the end
// and turn an aborted wait into hipErrorLaunchTimeOut; otherwise return once everything is
// queued (host_flags must then be pinned memory, valid after the stream passes the copy,
// and slot EIGF_ABORT tells whether a bounded wait gave up).
struct EigOut {
  float eps;
  int p, comp, R_max;
  float* P32;
  float* Q32;
  float* sigma_x;
  float* sigma_g;
  int* info_x;
  int* info_g;
  // optional: queued on the stream after the decomposition and before the host reads
  // the flags back (the caller's follow-up work that needs no host decision)
  hipError_t (*before_readback)(void* ctx, hipStream_t st) = nullptr;
  void* ctx = nullptr;
};
constexpr int INFO_WORDS = 8;
constexpr int EIG_HOST_FLAGS = 40;
constexpr int EIGF_SWEEPS = 6, EIGF_CONV = 8, EIGF_BAD = 10, EIGF_ABORT = 17, EIGF_NALIVE = 18, EIGF_INFO = 24;
size_t eig_workspace_bytes(int L);
int eig_max_L();
// Subspace width for the top-R solver (0 when it would span the whole space).
int eig_subspace_width(int L, int R_max);
// The same outputs from `iters` steps of block subspace iteration on an L x m basis; the
// truncation takes E = ||C||_F^2 from the statistic and rejects (status 7) kept directions
// whose Ritz residual exceeds its tolerance, and (status 4) thresholds beyond m directions.
hipError_t run_eig_subspace(const double* SX, const double* SG, double inv_nx, double inv_ng, int L, int m,
                            int iters, int max_sweeps, bool warm, void* work, const EigOut& out,
                            int host_flags[EIG_HOST_FLAGS], hipStream_t st, bool wait);
hipError_t run_eig(const double* SX, const double* SG, double inv_nx, double inv_ng, int L, int max_sweeps,
                   bool warm, void* work, const EigOut& out, int host_flags[EIG_HOST_FLAGS], hipStream_t st,
                   bool wait);

// I/O-dtype copies of the active projections: PQ [2*R_max][ldL] (rows [0,Rx) = P,
// [Rx,Rx+Ry) = Q, zero elsewhere) and Qt [L][ldQt] (zero beyond Ry).
hipError_t launch_build_io(bool bf16_io, const float* P32, const float* Q32, const int* dRx, const int* dRy, int L,
                           int ldL, int R_max, void* PQ, void* Qt, int ldQt, hipStream_t st);

// out[i][j] = S[min][max] * inv_n for the full L x L matrix (float64).
hipError_t launch_stat_mean(const double* S, double inv_n, int L, double* out, hipStream_t st);

hipError_t launch_fill_i32(int* dst, const int* values, int n, hipStream_t st);
hipError_t launch_zero(void* dst, size_t bytes, hipStream_t st);

}  // namespace instant
