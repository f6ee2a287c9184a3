// Per-step kernels of the INSTANT low-rank backward (notes "INSTANT: Compressing
// Gradients and Activations for Resource-Efficient Training", sections 整体框架 and
// 关键设计 3); the projection (forward compression and the stacked [P; Q] gy) is in
// kernels_proj.hip:
//   gemm    g_w = sum_b (P gy_b)^T x_hat_b   (contraction over K = B*Rx)
//           g_hat_x = (Q gy) w               (contraction over K = Cy)
//   expand  g_x_b = Q^T g_hat_x_b            (contraction over K = Ry)
// All contractions run on the matrix cores with float32 accumulation.
#include <algorithm>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"
#include "lds_tiles.hpp"

namespace instant {

// ----------------------------------------------------------------------------- gemm
// Cm[m][n] = sum_{k < K} A(m, k) B[k][n], written in T to Cm [M][ldc] (batch-strided).
// A_TRANS = false: A is [M][lda] (k contiguous); the wave covers 16*MT rows.
// A_TRANS = true : A is [K][lda] (m contiguous); a lane reads 4 adjacent rows as
//                  virtual tiles, the wave covers 64 rows (MT must be 4).
// B is [K][ldb] (n contiguous); the wave covers 128 columns.
// Grid: (ceil(N / 128), ceil(M / rows per wave), batch); the NW waves of a block split K,
// each issuing the loads of U steps before any product.
// Block (bx, by, bz) of the grid described above, computed by NW waves numbered `wave` =
// 0 .. NW-1 (all waves of the workgroup call it the same number of times: it holds block
// barriers); `red` is NW * 8 KB of LDS.
template <class T, bool A_TRANS, int MT, int NW, int U, bool NT = false>
__device__ __forceinline__ void gemm_block(const T* __restrict__ A, int lda, size_t strideA,
                                           const T* __restrict__ Bm, int ldb, size_t strideB, T* __restrict__ Cm,
                                           int ldc, size_t strideC, int M, int N, int K, int bx, int by, int bz,
                                           int wave, float (*red)[8][4][WAVE]) {
  typedef MM<T> mm;
  typedef typename mm::frag frag;
  const int lane = threadIdx.x & (WAVE - 1);
    const int z = bz;
  A += z * strideA;
  Bm += z * strideB;
  Cm += z * strideC;
  const int col = bx * 128 + 8 * (lane & 15);
  const bool col_ok = col < N;
  constexpr int ROWS = A_TRANS ? 64 : 16 * MT;
  const int m0 = by * ROWS;
  const int kl = mm::G * (lane >> 4);

  f32x4 acc[MT][8];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[t][j] = zero4();

  const int nsteps = (K + mm::KSTEP - 1) / mm::KSTEP;
  for (int s0 = wave; s0 < nsteps; s0 += NW * U) {
    frag bf[U][8];
    frag af[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * NW;
      const int k0 = s * mm::KSTEP + kl;
      load_strip_T<T, 8>(Bm, ldb, k0, K, col, col_ok, bf[u]);
      if constexpr (A_TRANS) {
        static_assert(MT == 4, "transposed A uses 4-wide strips");
        const int acol = m0 + 4 * (lane & 15);
        load_strip_T<T, 4>(A, lda, k0, K, acol, acol < M, af[u]);
      } else {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const int m = m0 + 16 * t + (lane & 15);
          if (m < M && k0 + mm::G <= K) {
            af[u][t] = load_frag<T>(A + (size_t)m * lda + k0, true);
          } else {
            // ragged k tail of a direct operand: element-wise, zero beyond K
            af[u][t] = zero_frag<T>();
            if (m < M)
              for (int g = 0; g < mm::G; ++g)
                if (k0 + g < K) af[u][t][g] = A[(size_t)m * lda + k0 + g];
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[t][j] = mm::mma(af[u][t], bf[u][j], acc[t][j]);
  }

  auto row_of = [&](int t, int v) {
    const int r = 4 * (lane >> 4) + v;  // tile row
    return A_TRANS ? m0 + 4 * r + t : m0 + 16 * t + r;
  };
  auto store = [&](int m, const float o[8]) {
    if (m < M && col_ok) {
      if constexpr (NT) store_row_nt<T, 8>(Cm + (size_t)m * ldc + col, o);
      else store_row<T, 8>(Cm + (size_t)m * ldc + col, o);
    }
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

// WPE: the fewest waves each SIMD must be able to hold (caps the registers a wave may use);
// NT: non-temporal stores, for an output that neither this launch nor the next one reads.
template <class T, bool A_TRANS, int MT, int NW, int U, int WPE = 1, bool NT = false>
__global__ __launch_bounds__(NW * WAVE) __attribute__((amdgpu_waves_per_eu(WPE, 8))) void gemm_kernel(
    const T* __restrict__ A, int lda, size_t strideA, const T* __restrict__ Bm, int ldb, size_t strideB,
    T* __restrict__ Cm, int ldc, size_t strideC, int M, int N, int K) {
  __shared__ float red[NW][8][4][WAVE];
  // Workgroups go to the XCDs in turn, so consecutive column strips land on different XCDs and
  // each XCD keeps its own strips of B. When A is the larger operand (M > N), the blocks are
  // renumbered row-major in a contiguous run per XCD instead: the strips of a row block then
  // read its A rows through one L2 (measured on gfx950: EfficientFormer g_hat_x, 3712 x 448 x
  // 1792, 17.6 -> 16.4 us; LLM MLP g_w, 11008 x 4096 x 272, 44.3 -> 43.8 us; with M < N the
  // renumbering lost, BERT FFN down g_hat_x, 448 x 3072 x 768, 8.6 -> 11.2 us).
  int bx = blockIdx.x, by = blockIdx.y;
  if (M > N) {
    const int gx = gridDim.x, u = xcd_unit(bx + gx * by, gx * gridDim.y);
    bx = u % gx;
    by = u / gx;
  }
  gemm_block<T, A_TRANS, MT, NW, U, NT>(A, lda, strideA, Bm, ldb, strideB, Cm, ldc, strideC, M, N, K, bx, by,
                                        blockIdx.z, threadIdx.x / WAVE, red);
}

// ---------------------------------------------------------------- g_hat_x with w read once
// C[M][N] = A[M][K] . B[K][N] (A k-contiguous) for a B too large to stay in L2 and few rows
// (g_hat_x = (Q gy) w of an LLM MLP: M = B*Ry = 272, w 90 MB). Blocks computing different row
// ranges of one column strip would each stream the strip from memory again, so a block here
// owns all M rows of a 128-column strip over one K slice (grid: strips x S). A stage (one
// k-step: 32 rows of B x 128 columns, and the row tiles of A x 32 k) goes to LDS by DMA,
// each wave issuing the same 1 + TPW loads (so its wait counts are exact); eight waves own
// the row tiles w, w + 8, ...; the slices write float32 partials [S][M][N], which
// splitk_reduce_kernel sums in slice order. K % 32 == 0, N % 8 == 0, M <= 128 * TPW.
template <int TPW, int STG>
__global__ __launch_bounds__(512) void gemm_ws_kernel(const bf16* __restrict__ A, int lda, const bf16* __restrict__ Bm,
                                                      int ldb, float* __restrict__ part, int M, int N, int K,
                                                      const bf16* __restrict__ zpad) {
  typedef MM<bf16> mm;
  typedef mm::frag frag;
  constexpr int NT = 8 * TPW;             // row tile slots of a stage
  constexpr int STAGE = 1024 * (8 + NT);  // bytes: B chunks [g][lane], then A tiles [t][lane]
  __shared__ __attribute__((aligned(1024))) unsigned char ring[STG][STAGE];
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  // units slice-major, a contiguous run per XCD: with eight slices each XCD reads one K slice of
  // A, which then stays in its L2 for every strip
  const int strips = gridDim.x, S = gridDim.y;
  const int u = xcd_unit(blockIdx.x + strips * blockIdx.y, strips * S);
  const int z = u / strips;
  const int col = (u % strips) * 128 + 8 * (lane & 15);
  const bool col_ok = col < N;
  const int kl = 8 * (lane >> 4);
  const int nsteps = K / mm::KSTEP;
  const int sb = (int)((long)nsteps * z / S), se = (int)((long)nsteps * (z + 1) / S), nq = se - sb;
  // B chunk g = wave: rows k0 + g of the lanes' columns; A tile t = wave + 8j: rows 16t + lane % 16
  auto issue = [&](int s, int slot) {
    const int k0 = s * mm::KSTEP + kl;
    unsigned char* st = ring[slot];
    lds_dma16(col_ok ? (const void*)(Bm + (size_t)(k0 + wave) * ldb + col) : (const void*)zpad, st + 1024 * wave);
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = wave + 8 * j;
      const int m = 16 * t + (lane & 15);
      lds_dma16(m < M ? (const void*)(A + (size_t)m * lda + k0) : (const void*)zpad, st + 1024 * (8 + t));
    }
  };
  f32x4 acc[TPW][8];
#pragma unroll
  for (int j = 0; j < TPW; ++j)
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[j][u] = zero4();
#pragma unroll
  for (int q = 0; q < STG - 1; ++q)
    if (q < nq) issue(sb + q, q);
  for (int i = 0; i < nq; ++i) {
    // stage i has landed once at most the later stages' loads remain (and LDS reads are done)
    const int later = (nq - 1 - i) < (STG - 2) ? (nq - 1 - i) : (STG - 2);
    wait_oldest_stage<1 + TPW, STG - 2>(later);
    bare_barrier();  // every wave's part of stage i; every read of the buffer refilled next
    if (i + STG - 1 < nq) issue(sb + i + STG - 1, (i + STG - 1) % STG);
    const unsigned char* st = ring[i % STG];
    bf16x8 r[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) r[g] = *reinterpret_cast<const bf16x8*>(st + 1024 * g + 16 * lane);
    frag bf[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int g = 0; g < 8; ++g) bf[u][g] = r[g][u];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const frag af = *reinterpret_cast<const frag*>(st + 1024 * (8 + wave + 8 * j) + 16 * lane);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[j][u] = mm::mma(af, bf[u], acc[j][u]);
    }
  }
  float* __restrict__ out = part + (size_t)z * M * N;
#pragma unroll
  for (int j = 0; j < TPW; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 16 * (wave + 8 * j) + 4 * (lane >> 4) + v;
      if (m < M && col_ok) {
        float* p = out + (size_t)m * N + col;
        *reinterpret_cast<f32x4*>(p) = f32x4{acc[j][0][v], acc[j][1][v], acc[j][2][v], acc[j][3][v]};
        *reinterpret_cast<f32x4*>(p + 4) = f32x4{acc[j][4][v], acc[j][5][v], acc[j][6][v], acc[j][7][v]};
      }
    }
}

// C[m][n] = sum_{z < S} part[z][m][n] in slice order (part: S slices of [M][N] float32).
// The same product for up to 288 rows, with the waves tiled in two dimensions and the loads
// issued by waves of their own. Block (128-column strip, K slice); a stage is 64 k: the w tile
// (64 rows x 256 bytes, k-major, read through the transpose read) and the A tile (MA rows x
// 128 bytes, m-major) go to LDS by DMA through a GWS_STAGES-deep ring. Eight compute waves:
// row group rg (RT row tiles of 16) x column half ch (64 columns as two 32-column pairs); four
// loader waves issue every 1 KB load of a stage between them (LDPS each, padded with loads of
// the zero pad, so the waits are exact counts). Against gemm_ws_kernel, whose eight waves each
// hold every row tile of their slot and issue their own loads, at the LLM MLP g_hat_x (272 x
// 4096 x 11008, 8 slices, with the reduction, bit-identical): 56.4 -> 45.8 us on gfx950.
constexpr int GWS_STAGES = 3;

template <int RT, int MA, int STG>
__global__ __launch_bounds__(768) void gemm_ws2_kernel(const bf16* __restrict__ A, int lda, const bf16* __restrict__ Bm,
                                                       int ldb, float* __restrict__ part, int M, int N, int K,
                                                       const bf16* __restrict__ zpad) {
  typedef MM<bf16> mm;
  constexpr int XT = 16384;                // w tile of a stage
  constexpr int TOT = 16 + MA / 8;         // 1 KB loads of a stage
  constexpr int NL = 4;                    // loader waves
  constexpr int LDPS = (TOT + NL - 1) / NL;
  constexpr int STAGE = 1024 * NL * LDPS;  // w tile, A tile, then the padding loads' slots
  static_assert(MA % 8 == 0 && 64 * RT >= MA && LDPS * (STG - 2) <= 63, "row groups cover the rows; vmcnt range");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[STG][STAGE];
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const bool loader = wave >= 8;
  const int li = wave - 8;
  const int ch = wave & 1, rg = wave >> 1;
  const int MT = (M + 15) / 16;
  // units slice-major, a contiguous run per XCD: with eight slices each XCD reads one K slice of
  // A (750 KB at the LLM MLP size), which then stays in its L2 for every strip; in strip order
  // each XCD would need all of A (6 MB, beyond its 4 MB L2) at every stage
  const int strips = gridDim.x, S = gridDim.y;
  const int u = xcd_unit(blockIdx.x + strips * blockIdx.y, strips * S);
  const int n0 = (u % strips) * 128, z = u / strips;
  const int nst = (K + 63) / 64;
  const int sb = (int)((long)nst * z / S), se = (int)((long)nst * (z + 1) / S), nq = se - sb;
  auto issue = [&](int s, int slot) {
    unsigned char* st = ring[slot];
    const int k0 = 64 * s;
#pragma unroll
    for (int i = 0; i < LDPS; ++i) {
      const int J = li + NL * i;
      const void* src;
      if (J < 16) {  // w: rows 4 J + lane / 16, 16 chunks a row
        const int r = 4 * J + (lane >> 4);
        const int lc = (lane & 15) ^ kswz_b(r);
        const int k = k0 + r, n = n0 + 8 * lc;
        src = (k < K && n < N) ? (const void*)(Bm + (size_t)k * ldb + n) : (const void*)zpad;
      } else if (J < TOT) {  // A: rows 8 (J - 16) + lane / 8, 8 chunks a row
        const int r = 8 * (J - 16) + (lane >> 3);
        const int lc = (lane & 7) ^ mswz(r);
        const int kk = k0 + 8 * lc;
        src = (r < M && kk < K) ? (const void*)(A + (size_t)r * lda + kk) : (const void*)zpad;
      } else {
        src = zpad;
      }
      lds_dma16(src, st + 1024 * J);
    }
  };
  f32x4 acc[RT][4];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[t][j] = zero4();
  if (loader) {
#pragma unroll
    for (int q = 0; q < STG - 1; ++q)
      if (q < nq) issue(sb + q, q);
  }
  const int q4 = lane >> 4, l16 = lane & 15;
  const int t0 = rg * RT;
  for (int i = 0; i < nq; ++i) {
    // (compute waves issue no loads and pass the count at once; all wait for their LDS reads)
    const int later = (nq - 1 - i) < (STG - 2) ? (nq - 1 - i) : (STG - 2);
    wait_oldest_stage<LDPS, STG - 2>(later);
    bare_barrier();  // stage i has landed for every wave; the slot refilled next is free
    if (loader) {
      if (i + STG - 1 < nq) issue(sb + i + STG - 1, (i + STG - 1) % STG);
      continue;
    }
    const unsigned char* st = ring[i % STG];
    const unsigned char* ta = st + XT;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      mm::frag xf[4], af[RT];
#pragma unroll
      for (int j = 0; j < 4; ++j) xf[j] = kmajor_frag<true>(st, h, lane, 64 * ch + 32 * (j >> 1), j & 1);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int r = 16 * (t0 + t) + l16;
        af[t] = t0 + t < MT ? *reinterpret_cast<const mm::frag*>(ta + r * 128 + 16 * ((4 * h + q4) ^ mswz(r))) : xf[0];
      }
      // every read of the k-step before its products (left to itself the scheduler waits for
      // each row tile's read in turn)
      __builtin_amdgcn_sched_group_barrier(0x100, RT + 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * RT, 0);
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[t][j] = mm::mma(xf[j], af[t], acc[t][j]);
    }
  }
  if (loader) return;
  // lane: row m of the partial, columns n .. n + 7: the first four from half q4 % 2 of the
  // pair, the last four from the other half (the pair layout of kmajor_frag)
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int m = 16 * (t0 + t) + l16;
    if (t0 + t >= MT || m >= M) continue;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int n = n0 + 64 * ch + 32 * p + 8 * q4;
      if (n >= N) continue;
      const int h0 = q4 & 1;
      float o[8];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        o[v] = h0 ? acc[t][2 * p + 1][v] : acc[t][2 * p][v];
        o[4 + v] = h0 ? acc[t][2 * p][v] : acc[t][2 * p + 1][v];
      }
      float* dst = part + ((size_t)z * M + m) * N + n;
      *reinterpret_cast<f32x4*>(dst) = f32x4{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
    }
  }
}

template <class T>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int S, int M, int N,
                                                            T* __restrict__ Cm, int ldc) {
  const int n4 = N / 4;
  const size_t slice = (size_t)M * N;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < (size_t)M * n4; e += (size_t)gridDim.x * 256) {
    const int m = (int)(e / n4), c = (int)(e % n4) * 4;
    const float* p = part + (size_t)m * N + c;
    f32x4 acc = *reinterpret_cast<const f32x4*>(p);
    for (int z = 1; z < S; ++z) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(p + z * slice);
      acc[0] += v[0];
      acc[1] += v[1];
      acc[2] += v[2];
      acc[3] += v[3];
    }
    const float o[4] = {acc[0], acc[1], acc[2], acc[3]};
    store_row<T, 4>(Cm + (size_t)m * ldc + c, o);
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
  frag af[MPW][KS];
#pragma unroll
  for (int i = 0; i < MPW; ++i) {
    const int la = 16 * (tile0 + i) + (lane & 15);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) af[i][ks] = load_frag<T>(At + (size_t)la * ldA + ks * mm::KSTEP + kl, la < L);
  }
#pragma unroll
  for (int i = 0; i < MPW; ++i) {
    const int l0 = 16 * (tile0 + i);
    if (l0 >= L) break;
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = zero4();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = mm::mma(af[i][ks], bf[ks][j], acc[j]);
    if (col_ok) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int l = l0 + 4 * (lane >> 4) + v;
        if (l < L) {
          float o[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) o[j] = acc[j][v];
          store_row_nt<T, 8>(out + ((size_t)b * L + l) * C + col, o);
        }
      }
    }
  }
}

// The expansion with the split-K reduction of g_hat_x folded in (bf16): g_hat_x arrives as the
// S float32 slices [S][B * R][C] of gemm_ws_kernel / gemm_ws2_kernel. Block (128-column strip,
// sample, token group): its threads first add the S slices of the sample's R x 128 strip in
// slice order, rounded to bf16 as splitk_reduce_kernel would (so the result is the same bit for
// bit), into an LDS operand whose rows R .. KS * KSTEP - 1 are zero; then every wave sweeps its
// 16-token tiles as expand_kernel does, the B operand read from LDS. This saves the reduction's
// launch and the round trip of g_hat_x. Grid: (ceil(C / 128), B, TG); S <= 16, C % 8 == 0.
template <int KS, int NW>
__global__ __launch_bounds__(NW * WAVE) void expand_parts_kernel(const bf16* __restrict__ At, int ldA,
                                                                const float* __restrict__ part, int S, int R,
                                                                int L, int C, bf16* __restrict__ out) {
  typedef MM<bf16> mm;
  typedef mm::frag frag;
  constexpr int KR = KS * mm::KSTEP;  // rows of the LDS operand
  __shared__ __attribute__((aligned(16))) bf16 gs[KR][128];
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int b = blockIdx.y, c0 = blockIdx.x * 128;
  const size_t slice = (size_t)gridDim.y * R * C;  // one slice: B * R rows of C
  // (a thread's slices loaded at once, added in slice order; holding the loads of several
  // elements at once took registers the sweep below needed: slower on gfx950)
  for (int e = threadIdx.x; e < KR * 32; e += NW * WAVE) {
    const int r = e >> 5, c = 4 * (e & 31);
    float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (r < R && c0 + c < C) {
      const float* p = part + ((size_t)b * R + r) * C + c0 + c;
      f32x4 v[16];
#pragma unroll
      for (int z = 0; z < 16; ++z)
        if (z < S) v[z] = *reinterpret_cast<const f32x4*>(p + z * slice);
      f32x4 acc = v[0];
#pragma unroll
      for (int z = 1; z < 16; ++z)
        if (z < S) {
          acc[0] += v[z][0];
          acc[1] += v[z][1];
          acc[2] += v[z][2];
          acc[3] += v[z][3];
        }
      o[0] = acc[0];
      o[1] = acc[1];
      o[2] = acc[2];
      o[3] = acc[3];
    }
    store_row<bf16, 4>(&gs[r][c], o);
  }
  __syncthreads();

  const int col = c0 + 8 * (lane & 15);
  const bool col_ok = col < C;
  const int kl = mm::G * (lane >> 4);
  frag bf[KS][8];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) load_strip_T<bf16, 8>(&gs[0][0], 128, ks * mm::KSTEP + kl, KR, 8 * (lane & 15), true, bf[ks]);
  constexpr int MPW = 4;
  const int ntl = (L + 15) / 16, step = NW * gridDim.z;
  for (int tl0 = blockIdx.z * NW + wave; tl0 < ntl; tl0 += step * MPW) {
    frag af[MPW][KS];
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
      const int tl = tl0 + i * step;
      const int la = 16 * tl + (lane & 15);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        af[i][ks] = load_frag<bf16>(At + (size_t)la * ldA + ks * mm::KSTEP + kl, tl < ntl && la < L);
    }
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
      const int tl = tl0 + i * step;
      if (tl >= ntl) break;
      f32x4 acc[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = mm::mma(af[i][ks], bf[ks][j], acc[j]);
      if (col_ok) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int l = 16 * tl + 4 * (lane >> 4) + v;
          if (l < L) {
            float o[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] = acc[j][v];
            store_row_nt<bf16, 8>(out + ((size_t)b * L + l) * C + col, o);
          }
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------- fused g_x
// For layers whose weight stays resident in L2: block (strip, sample group) first forms
// g_hat_x_b[:, strip] = Qgy_b (Ry x Cy) . w[:, strip] (Cy x 16*SW) on the matrix cores for
// the SPB samples b of its group at once (their Ry-row blocks of Qgy are adjacent, so they
// stack into the 16-row A operand; the NW waves split Cy, LDS sums them), keeps them in
// LDS in the I/O dtype, and then expands g_x_b[:, strip] = Q^T g_hat_x_b[:, strip] over
// all L tokens, one Q^T fragment serving every sample. Stacking samples divides the w
// strip a block streams from L2 by SPB at the same block count. A lane owns SW adjacent
// columns of the strip.
template <class T, int MTA, int KS, int SW>
struct GxShared {
  // rows of the LDS operand: the stacked g_hat_x rows, and the K padding of the last
  // sample's expansion operand (zero)
  static constexpr int GROWS = 16 * MTA > KS * MM<T>::KSTEP ? 16 * MTA : KS * MM<T>::KSTEP;
  T g[GROWS][16 * SW];
};

template <class T, int MTA, int KS, int NW, int SW, int SPB>
__device__ __forceinline__ void gx_fused_block(const T* __restrict__ Qgy, const T* __restrict__ w,
                                               const T* __restrict__ At, int ldA, int R, int L, int Cy, int Cx,
                                               T* __restrict__ out, int strip, int b0, int nb,
                                               float (*red)[SW][4][WAVE], GxShared<T, MTA, KS, SW>& gs) {
  typedef MM<T> mm;
  typedef typename mm::frag frag;
  constexpr int U = 3;  // with 8 waves, the 24 k-steps of Cy = 768 in one round of loads
  constexpr int GROWS = GxShared<T, MTA, KS, SW>::GROWS;
  constexpr int SC = 16 * SW;  // strip columns
  auto& gsm = gs.g;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  const int lc = SW * (lane & 15);  // column within the strip
  const int col = strip * SC + lc;
  const bool col_ok = col < Cx;
  const int kl = mm::G * (lane >> 4);
  const T* __restrict__ Ab = Qgy + (size_t)b0 * R * Cy;
  const int rows = nb * R;  // stacked g_hat_x rows of the group

  for (int e = threadIdx.x; e < GROWS * SC; e += NW * WAVE) (&gsm[0][0])[e] = (T)0.0f;

  // phase 1: g_hat_x tiles of the group
  f32x4 acc[MTA][SW];
#pragma unroll
  for (int t = 0; t < MTA; ++t)
#pragma unroll
    for (int j = 0; j < SW; ++j) acc[t][j] = zero4();
  const int nsteps = (Cy + mm::KSTEP - 1) / mm::KSTEP;
  for (int s0 = wave; s0 < nsteps; s0 += NW * U) {
    frag bf[U][SW];
    frag af[U][MTA];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * NW;
      const int k0 = s * mm::KSTEP + kl;
      load_strip_T<T, SW>(w, Cx, k0, Cy, col, col_ok, bf[u]);
#pragma unroll
      for (int t = 0; t < MTA; ++t) {
        const int m = 16 * t + (lane & 15);
        af[u][t] = load_frag<T>(Ab + (size_t)m * Cy + k0, m < rows && s < nsteps && k0 + mm::G <= Cy);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < MTA; ++t)
#pragma unroll
        for (int j = 0; j < SW; ++j) acc[t][j] = mm::mma(af[u][t], bf[u][j], acc[t][j]);
  }
#pragma unroll
  for (int t = 0; t < MTA; ++t) {
#pragma unroll
    for (int j = 0; j < SW; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][j][v][lane] = acc[t][j][v];
    __syncthreads();
    for (int v = wave; v < 4; v += NW) {
      const int r = 16 * t + 4 * (lane >> 4) + v;
      if (r < rows) {
#pragma unroll
        for (int j = 0; j < SW; ++j) {
          float sum = red[0][j][v][lane];
#pragma unroll
          for (int ww = 1; ww < NW; ++ww) sum += red[ww][j][v][lane];
          gsm[r][lc + j] = from_f32<T>(sum);
        }
      }
    }
    __syncthreads();
  }

  // phase 2: expand over all tokens; each wave takes every NW-th 16-token tile
  frag bz[SPB][KS][SW];
#pragma unroll
  for (int g = 0; g < SPB; ++g)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      load_strip_T<T, SW>(&gsm[g * R][0], SC, ks * mm::KSTEP + kl, g < nb ? R : 0, lc, true, bz[g][ks]);
  constexpr int MPW = SPB == 1 ? 4 : 2;
  const int ntl = (L + 15) / 16;
  for (int tl0 = wave; tl0 < ntl; tl0 += NW * MPW) {
    frag af[MPW][KS];
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
      const int tl = tl0 + i * NW;
      const int la = 16 * tl + (lane & 15);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        af[i][ks] = load_frag<T>(At + (size_t)la * ldA + ks * mm::KSTEP + kl, tl < ntl && la < L);
    }
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
      const int tl = tl0 + i * NW;
      if (tl >= ntl) break;
      const int l0 = 16 * tl;
#pragma unroll
      for (int g = 0; g < SPB; ++g) {
        if (g >= nb) break;
        f32x4 o4[SW];
#pragma unroll
        for (int j = 0; j < SW; ++j) o4[j] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int j = 0; j < SW; ++j) o4[j] = mm::mma(af[i][ks], bz[g][ks][j], o4[j]);
        if (col_ok) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int l = l0 + 4 * (lane >> 4) + v;
            if (l < L) {
              float o[SW];
#pragma unroll
              for (int j = 0; j < SW; ++j) o[j] = o4[j][v];
              store_row_nt<T, SW>(out + ((size_t)(b0 + g) * L + l) * Cx + col, o);
            }
          }
        }
      }
    }
  }
}

// The fused g_x blocks and the g_w blocks in one launch: both depend only on the stacked
// projection, and the g_w tiles fill the compute units the g_x strips leave free.
// Blocks [0, ngx) are g_x (one strip and a group of SPB samples each); each of the rest
// takes two g_w tiles (64 x 128) side by side, half of its waves on each with K split
// over them, which halves the g_w blocks at the latency of one tile.
template <class T, int MTA, int KS, int NW, int SW, int SPB>
__global__ __launch_bounds__(NW * WAVE) void bwd_tail_kernel(const T* __restrict__ Qgy, const T* __restrict__ w,
                                                             const T* __restrict__ At, int ldA, int B, int R,
                                                             int L, int Cy, int Cx, T* __restrict__ gx,
                                                             int nstrip, int ngx, const T* __restrict__ Pgy,
                                                             const T* __restrict__ xhat, T* __restrict__ gw,
                                                             int Kw, int gw_bx, int gw_tiles) {
  __shared__ float red[NW][8][4][WAVE];
  __shared__ __attribute__((aligned(16))) GxShared<T, MTA, KS, SW> gs;
  const int id = blockIdx.x;
  if (id < ngx) {
    // Workgroups are dealt to the XCDs in turn (id % 8). Units in strip-major order, a
    // contiguous run of them per XCD, so that each XCD's L2 holds one or two strips of w
    // rather than all of it.
    const int unit = xcd_unit(id, ngx);
    const int ngroups = ngx / nstrip;
    const int strip = unit / ngroups;
    const int b0 = SPB * (unit % ngroups);
    gx_fused_block<T, MTA, KS, NW, SW, SPB>(Qgy, w, At, ldA, R, L, Cy, Cx, gx, strip, b0,
                                            min(SPB, B - b0),
                                            reinterpret_cast<float (*)[SW][4][WAVE]>(&red[0][0][0][0]), gs);
  } else {
    // g_w = sum_b (P gy_b)^T x_hat_b: M = Cy, N = Cx, K = B*Rx (A stored [K][Cy])
    constexpr int HW = NW / 2;
    const int half = threadIdx.x / (HW * WAVE);
    const int t = 2 * (id - ngx) + half;
    // a missing second tile still takes part in the barriers, with no columns
    gemm_block<T, true, 4, HW, 1>(Pgy, Cy, 0, xhat, Cx, 0, gw, Cx, 0, Cy, t < gw_tiles ? Cx : 0, Kw, t % gw_bx,
                                  t / gw_bx, 0, threadIdx.x / WAVE - half * HW, red + half * HW);
  }
}

// ----------------------------------------------------------------------------- launchers

template <class T, bool AT, int MT, int NW, int U, int WPE = 1, bool NT = false>
static hipError_t gemm_cfg(const void* A, int lda, size_t sA, const void* Bm, int ldb, size_t sB, void* Cm, int ldc,
                           size_t sC, int batch, int M, int N, int K, hipStream_t st) {
  constexpr int ROWS = AT ? 64 : 16 * MT;
  dim3 grid((N + 127) / 128, (M + ROWS - 1) / ROWS, batch);
  hipLaunchKernelGGL((gemm_kernel<T, AT, MT, NW, U, WPE, NT>), grid, dim3(NW * WAVE), 0, st, (const T*)A, lda, sA,
                     (const T*)Bm, ldb, sB, (T*)Cm, ldc, sC, M, N, K);
  return hipGetLastError();
}

constexpr int WS_TPW = 3;  // row tiles per wave of gemm_ws_kernel: up to 384 rows

int gemm_ws_slices(bool bf16_io, bool a_trans, int M, int N, int K) {
  if (!bf16_io || a_trans || M < 1 || M > 128 * WS_TPW || K % 32 || N % 8) return 0;
  if ((double)N * K * 2 < 32.0 * (1 << 20)) return 0;  // B small enough to stay in L2: the row blocks share it
  const int strips = (N + 127) / 128;
  int S = std::max(2, std::min(16, 256 / strips));      // about one block per compute unit
  S = std::min(S, (K / 32) / 16);                        // slices of at least 16 k-steps
  return S >= 2 ? S : 0;
}

// The slices of the read-w-once GEMM (S = gemm_ws_slices(...) > 0): part[z][m][n].
static hipError_t ws_slices_launch(const void* A, int lda, const void* Bm, int ldb, float* part, int S, int M, int N,
                                   int K, const void* zpad, hipStream_t st) {
  const unsigned strips = (unsigned)((N + 127) / 128);
#define WS2(RT, MA)                                                                                                  \
  hipLaunchKernelGGL((gemm_ws2_kernel<RT, MA, GWS_STAGES>), dim3(strips, S), dim3(768), 0, st, (const bf16*)A, lda, \
                     (const bf16*)Bm, ldb, part, M, N, K, (const bf16*)zpad)
  if (M <= 128) WS2(2, 128);
  else if (M <= 192) WS2(3, 192);
  else if (M <= 288) WS2(5, 288);
  else
    hipLaunchKernelGGL((gemm_ws_kernel<WS_TPW, 3>), dim3(strips, S), dim3(512), 0, st, (const bf16*)A, lda,
                       (const bf16*)Bm, ldb, part, M, N, K, (const bf16*)zpad);
#undef WS2
  return hipGetLastError();
}

hipError_t launch_gemm_ws_parts(const void* A, int lda, const void* Bm, int ldb, float* part, size_t part_floats,
                                int M, int N, int K, const void* zpad, hipStream_t st) {
  const int S = gemm_ws_slices(true, false, M, N, K);
  if (!S || !part || !zpad || (size_t)S * M * N > part_floats) return hipErrorInvalidValue;
  return ws_slices_launch(A, lda, Bm, ldb, part, S, M, N, K, zpad, st);
}

template <class T, bool AT>
static hipError_t gemm_t(const void* A, int lda, size_t sA, const void* Bm, int ldb, size_t sB, void* Cm, int ldc,
                         size_t sC, int batch, int M, int N, int K, float* part, size_t part_floats,
                         const void* zpad, hipStream_t st) {
  const int nsteps = (K + MM<T>::KSTEP - 1) / MM<T>::KSTEP;
  constexpr bool BF = MM<T>::KSTEP == 32;
  const long strips = (N + 127) / 128;
  if constexpr (BF && !AT) {
    // (bf16, measured on gfx950) B read once when it is too large for L2 (LLM MLP g_hat_x,
    // 272 x 4096 x 11008: 55.5 us against 71.7 us for row blocks that each stream w again)
    const int S = (part && zpad && batch == 1) ? gemm_ws_slices(true, false, M, N, K) : 0;
    if (S && (size_t)S * M * N <= part_floats) {
      hipError_t e = ws_slices_launch(A, lda, Bm, ldb, part, S, M, N, K, zpad, st);
      if (e != hipSuccess) return e;
      const size_t n4 = (size_t)M * (N / 4);
      hipLaunchKernelGGL(splitk_reduce_kernel<T>, dim3((unsigned)std::min<size_t>((n4 + 255) / 256, 2048)), dim3(256),
                         0, st, (const float*)part, S, M, N, (T*)Cm, ldc);
      return hipGetLastError();
    }
  }
  if constexpr (AT) {
    if constexpr (BF) {
      // (bf16, measured on gfx950) Many 64x128 tiles (g_w of an LLM MLP: 5504 at 11008 x 4096,
      // K = 272): one wave per tile, one step of loads in flight, registers capped so that two
      // waves share a SIMD (one hides the other's loads), non-temporal stores: 44 us, against
      // 73-77 us with one wave per SIMD and three steps in flight, and 122 us for two waves
      // splitting K. Few tiles (BERT FFN, 288 at K = 448; EfficientFormer, 112 at K = 3712):
      // four waves split K, 10.8-11.4 us against 12.0-12.5 us with two, and 34 us against
      // 57 us at the long K with two steps in flight per wave.
      const long tiles = strips * ((M + 63) / 64);
      if (tiles >= 2048)
        return gemm_cfg<T, true, 4, 1, 1, 2, true>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, st);
      if (nsteps <= 16) return gemm_cfg<T, true, 4, 4, 1>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, st);
      return gemm_cfg<T, true, 4, 4, 2>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, st);
    }
    if (nsteps >= 8) return gemm_cfg<T, true, 4, 4, 2>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, st);
    return gemm_cfg<T, true, 4, 2, 2>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, st);
  } else {
    if constexpr (BF) {
      // (bf16, measured on gfx950) Eight waves split K; every row block streams its own pass
      // over the B strip, so the tallest row blocks that still give at least 192 blocks win:
      // LLM MLP (M = 272, K = 11008) 48 rows, 75 us against 114 us with 32 rows; BERT FFN down
      // (M = 448, K = 768) 48 rows, 9.1 us against 10.0 us; BERT FFN up (N = 768, K = 3072)
      // 16 rows, 13.8 against 16.8 us; EfficientFormer (M = 3712, N = 448) 64 rows, 18.4 us
      // against 19.7 us.
      auto blocks = [&](int mt) { return strips * ((M + 16 * mt - 1) / (16 * mt)); };
      if (blocks(4) >= 192) return gemm_cfg<T, false, 4, 8, 1>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, st);
      if (blocks(3) >= 192) return gemm_cfg<T, false, 3, 8, 1>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, st);
      if (blocks(2) >= 192) return gemm_cfg<T, false, 2, 8, 1>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, st);
      return gemm_cfg<T, false, 1, 8, 2>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, st);
    }
    // fp32 (the eigensolver's warm start W = C V): K split over eight waves for long K
    if (nsteps >= 16) return gemm_cfg<T, false, 2, 8, 2>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, st);
    return gemm_cfg<T, false, 2, 4, 2>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, st);
  }
}

hipError_t launch_gemm(bool bf16_io, bool a_trans, const void* A, int lda, size_t sA, const void* Bm, int ldb,
                       size_t sB, void* Cm, int ldc, size_t sC, int batch, int M, int N, int K, hipStream_t st,
                       float* part, size_t part_floats, const void* zpad) {
  if (bf16_io)
    return a_trans
               ? gemm_t<bf16, true>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, part, part_floats, zpad, st)
               : gemm_t<bf16, false>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, part, part_floats, zpad, st);
  return a_trans
             ? gemm_t<float, true>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, part, part_floats, zpad, st)
             : gemm_t<float, false>(A, lda, sA, Bm, ldb, sB, Cm, ldc, sC, batch, M, N, K, part, part_floats, zpad, st);
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

hipError_t launch_expand_parts(const void* At, int ldA, const float* part, int S, int B, int R, int L, int C, void* out,
                               hipStream_t st) {
  if (S < 1 || S > 16 || R < 1 || R > 64 || C % 8 || ldA < 64) return hipErrorInvalidValue;
  // one block a (strip, sample) over every token, eight waves (measured on gfx950 at the LLM MLP
  // size, B = 8, L = 2048, C = 4096, R = 34, 8 slices: 34.2 us against 37.3 us for the slices'
  // reduction and expand_kernel; two token groups 35.3-41.0 us, four waves 34.7 us)
  const dim3 grid((C + 127) / 128, B, 1);
  if (R <= 32)
    hipLaunchKernelGGL((expand_parts_kernel<1, 8>), grid, dim3(512), 0, st, (const bf16*)At, ldA, part, S, R, L, C,
                       (bf16*)out);
  else
    hipLaunchKernelGGL((expand_parts_kernel<2, 8>), grid, dim3(512), 0, st, (const bf16*)At, ldA, part, S, R, L, C,
                       (bf16*)out);
  return hipGetLastError();
}

template <class T, int MTA, int KS, int SW, int SPB>
static hipError_t bwd_tail_cfg(const void* Qgy, const void* w, const void* At, int ldA, int B, int R, int L, int Cy,
                               int Cx, void* gx, const void* Pgy, const void* xhat, void* gw, int Kw,
                               hipStream_t st) {
  constexpr int NW = MTA == 1 ? 8 : 4;
  const int nstrip = (Cx + 16 * SW - 1) / (16 * SW);
  const int ngx = nstrip * ((B + SPB - 1) / SPB);
  const int gw_bx = (Cx + 127) / 128, gw_tiles = gw_bx * ((Cy + 63) / 64);
  const int ngw = (gw_tiles + 1) / 2;
  hipLaunchKernelGGL((bwd_tail_kernel<T, MTA, KS, NW, SW, SPB>), dim3(ngx + ngw), dim3(NW * WAVE), 0, st,
                     (const T*)Qgy, (const T*)w, (const T*)At, ldA, B, R, L, Cy, Cx, (T*)gx, nstrip, ngx,
                     (const T*)Pgy, (const T*)xhat, (T*)gw, Kw, gw_bx, gw_tiles);
  return hipGetLastError();
}

template <class T, int MTA, int KS>
static hipError_t bwd_tail_sw(const void* Qgy, const void* w, const void* At, int ldA, int B, int R, int L, int Cy,
                              int Cx, void* gx, const void* Pgy, const void* xhat, void* gw, int Kw, int ncu,
                              hipStream_t st) {
  if constexpr (MTA == 1) {
    // two samples stacked in the 16-row tile: half the w strip per sample, in 64-column
    // strips so that the block count stays that of one sample in 128-column strips
    if (2 * R <= 16 && B > 1 && Cx > 64)
      return bwd_tail_cfg<T, 1, KS, 4, 2>(Qgy, w, At, ldA, B, R, L, Cy, Cx, gx, Pgy, xhat, gw, Kw, st);
  }
  // 64-column strips only when even they fit the compute units in one round: a second round
  // of g_x blocks costs more than the wider strip's longer pass (measured on gfx950 at
  // B = 32, C = 768: 11.2 us with 128-column strips against 14.7 us with 64-column ones)
  if ((long)((Cx + 63) / 64) * B <= ncu && Cx > 64)
    return bwd_tail_cfg<T, MTA, KS, 4, 1>(Qgy, w, At, ldA, B, R, L, Cy, Cx, gx, Pgy, xhat, gw, Kw, st);
  return bwd_tail_cfg<T, MTA, KS, 8, 1>(Qgy, w, At, ldA, B, R, L, Cy, Cx, gx, Pgy, xhat, gw, Kw, st);
}

template <class T>
static hipError_t bwd_tail_t(const void* Qgy, const void* w, const void* At, int ldA, int B, int R, int L, int Cy,
                             int Cx, void* gx, const void* Pgy, const void* xhat, void* gw, int Kw, int ncu,
                             hipStream_t st) {
  const int mta = (R + 15) / 16;
  const int ks = (R + MM<T>::KSTEP - 1) / MM<T>::KSTEP;
#define BTC(MA, K) \
  if (mta == MA && ks == K) return bwd_tail_sw<T, MA, K>(Qgy, w, At, ldA, B, R, L, Cy, Cx, gx, Pgy, xhat, gw, Kw, ncu, st);
  if constexpr (MM<T>::KSTEP == 32) {
    BTC(1, 1) BTC(2, 1) BTC(3, 2) BTC(4, 2)
  } else {
    BTC(1, 1) BTC(2, 2) BTC(3, 3) BTC(4, 4)
  }
#undef BTC
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_tail(bool bf16_io, const void* Qgy, const void* w, const void* At, int ldA, int B, int R, int L,
                           int Cy, int Cx, void* gx, const void* Pgy, const void* xhat, void* gw, int Kw, int ncu,
                           hipStream_t st) {
  if (ncu < 1) return hipErrorInvalidValue;
  return bf16_io ? bwd_tail_t<bf16>(Qgy, w, At, ldA, B, R, L, Cy, Cx, gx, Pgy, xhat, gw, Kw, ncu, st)
                 : bwd_tail_t<float>(Qgy, w, At, ldA, B, R, L, Cy, Cx, gx, Pgy, xhat, gw, Kw, ncu, st);
}

bool gx_fused_applies(bool bf16_io, int B, int Cx, int Cy) {
  const double wbytes = (double)Cx * Cy * (bf16_io ? 2 : 4);
  return wbytes <= 2.0 * (1 << 20) && B * wbytes <= 64.0 * (1 << 20);
}

}  // namespace instant
