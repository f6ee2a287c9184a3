// LDS-tiled matrix-core GEMM of the INSTANT low-rank backward (notes "INSTANT: Compressing
// Gradients and Activations for Resource-Efficient Training", section 关键设计 3), for the
// unfused path (w too large to stay resident in L2 for the fused g_x kernel):
//   g_w     = sum_b (P gy_b)^T x_hat_b   C[Cy][Cx], A = P gy stored [K = B*Rx][Cy]
//   g_hat_x = (Q gy) w                   C[B*Ry][Cx], A = Q gy stored [B*Ry][K = Cy]
// with B = x_hat [K][Cx] or w [K][Cx]: the B operand is stored k-major ("MN-major": n
// contiguous), and so is A for g_w.
//
// A 128 x 128 block tile is computed by four waves of 64 x 64 over a K slice. Stages of 64 k
// go from memory straight to LDS (global_load_lds, 16 bytes per lane) through a ring, so the
// later stages' loads are in flight while the matrix cores consume the oldest; four loader
// waves issue them, each the same loads per stage, so the waits are exact counts.
//
// Operands in LDS: k-major tiles (64 k rows x 128 columns) are read through the gfx950
// transpose read, m-major tiles (128 rows x 64 k) with one 16-byte read per lane; the layouts
// and swizzles are those of lds_tiles.hpp.
//
// Orientation. The MFMA computes D[n][m] = C[m][n]: the B operand (columns n) takes the
// first operand slot, A (rows m) the second. A lane then holds D rows 4 q + v (q = lane / 16,
// v < 4) of one column m; with the column bases cb of the two tiles (halves hh = 0, 1) of a
// 32-column pair set to 8 a + 4 (hh ^ (a % 2)), those rows of the two tiles are the 8
// consecutive columns n = 8 q .. 8 q + 7 of the pair: results leave as 16-byte stores.
//
// Split K: with grid.z = S > 1 every slice writes float32 partials [S][M][N] that a second
// launch sums in slice order (deterministic).
#include <algorithm>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"
#include "lds_tiles.hpp"

namespace instant {

namespace {

constexpr int GT = 128;        // block tile edge (M and N)
constexpr int GBK = 64;        // k per stage (two MFMA k-steps)
constexpr int KMAJ_BYTES = GBK * GT * 2;   // a k-major tile of a stage: 64 rows x 256 bytes
constexpr int MMAJ_BYTES = GT * GBK * 2;   // an m-major tile of a stage: 128 rows x 128 bytes
constexpr int STAGE_BYTES = KMAJ_BYTES + 16384;  // B tile, then the A tile (16 KB either way)
static_assert(MMAJ_BYTES == 16384 && KMAJ_BYTES == 16384, "tile sizes");

}  // namespace

// C = A . B over k slice blockIdx.z (see the file comment). A_KM: A stored [K][lda]
// (k-major), else [M][lda]. Grid: (tiles, 1, S) with tiles = ceil(M/128) * ceil(N/128).
// K % 8 == 0 when A is m-major; N % 8 == 0 and M % 8 == 0 when A is k-major.
template <bool A_KM, int STG, bool PART, int NLD>
__global__ __launch_bounds__(64 * (4 + NLD)) void gemm_tiled_kernel(const bf16* __restrict__ A, int lda,
                                                         const bf16* __restrict__ Bm, int ldb,
                                                         bf16* __restrict__ Cm, int ldc, float* __restrict__ part,
                                                         int M, int N, int K, const bf16* __restrict__ zpad) {
  typedef MM<bf16> mm;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[STG][STAGE_BYTES];
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  // NLD = 4: four more waves only stream the ring (loader li issues what compute wave li
  // would); NLD = 0: the four compute waves stream it themselves
  const bool loader = NLD ? wave >= 4 : true;
  const bool computer = wave < 4;
  const int li = NLD ? wave - 4 : wave;
  const int mtiles = (M + GT - 1) / GT, ntiles = (N + GT - 1) / GT;
  const int ntile_all = mtiles * ntiles;
  // XCD-aware order: the tiles of one XCD are a contiguous run, m fastest, so they share
  // the B panel (and neighbouring A panels) in that XCD's L2
  const int t = xcd_unit(blockIdx.x, ntile_all);
  const int m0 = (t % mtiles) * GT, n0 = (t / mtiles) * GT;
  const int z = blockIdx.z, S = gridDim.z;
  const int nst = (K + GBK - 1) / GBK;
  const int sb = (int)((long)nst * z / S), se = (int)((long)nst * (z + 1) / S), nq = se - sb;

  // every loader wave issues 8 DMA loads a stage: 4 for the B tile, 4 for the A tile
  auto issue = [&](int s, int slot) {
    unsigned char* st = ring[slot];
    const int k0 = s * GBK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // B: k-major, 64 rows x 16 chunks, 4 rows per wave-load
      const int r = 16 * j + 4 * li + (lane >> 4);
      const int pc = lane & 15, lc = pc ^ kswz_b(r);
      const int k = k0 + r, n = n0 + 8 * lc;
      const void* src = (k < K && n < N) ? (const void*)(Bm + (size_t)k * ldb + n) : (const void*)zpad;
      lds_dma16(src, st + 1024 * (4 * j + li));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const void* src;
      if constexpr (A_KM) {  // A: k-major like B
        const int r = 16 * j + 4 * li + (lane >> 4);
        const int pc = lane & 15, lc = pc ^ kswz_a(r);
        const int k = k0 + r, m = m0 + 8 * lc;
        src = (k < K && m < M) ? (const void*)(A + (size_t)k * lda + m) : (const void*)zpad;
      } else {  // A: m-major, 128 rows x 8 chunks, 8 rows per wave-load
        const int r = 32 * j + 8 * li + (lane >> 3);
        const int pc = lane & 7, lc = pc ^ mswz(r);
        const int m = m0 + r, k = k0 + 8 * lc;
        src = (m < M && k < K) ? (const void*)(A + (size_t)m * lda + k) : (const void*)zpad;
      }
      lds_dma16(src, st + KMAJ_BYTES + 1024 * (4 * j + li));
    }
  };

  const int wm = wave >> 1, wn = wave & 1;  // this wave's 64 x 64 quarter of the tile
  f32x4 acc[4][4];                          // [m tile][n tile]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero4();

  if (loader) {
#pragma unroll
    for (int q = 0; q < STG - 1; ++q)
      if (q < nq) issue(sb + q, q);
  }
  const int q4 = lane >> 4, l16 = lane & 15;
  for (int i = 0; i < nq; ++i) {
    // (waves that issue no loads pass the count at once; all wait for their LDS reads)
    const int later = (nq - 1 - i) < (STG - 2) ? (nq - 1 - i) : (STG - 2);
    wait_oldest_stage<8, STG - 2>(later);
    bare_barrier();  // stage i has landed for every wave; the slot refilled next is free
    if (loader && i + STG - 1 < nq) issue(sb + i + STG - 1, (i + STG - 1) % STG);
    if (!computer) continue;
    const unsigned char* st = ring[i % STG];
    const unsigned char* ta = st + KMAJ_BYTES;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      mm::frag bfr[4], afr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)  // n tiles: the two halves of two 32-column pairs
        bfr[j] = kmajor_frag<true>(st, h, lane, 64 * wn + 32 * (j >> 1), j & 1);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if constexpr (A_KM) {
          afr[mt] = kmajor_frag<false>(ta, h, lane, 64 * wm + 16 * mt, 0);
        } else {
          const int r = 64 * wm + 16 * mt + l16;
          afr[mt] = *reinterpret_cast<const mm::frag*>(ta + r * 128 + 16 * ((4 * h + q4) ^ mswz(r)));
        }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mt][j] = mm::mma(bfr[j], afr[mt], acc[mt][j]);
    }
  }

  if (!computer) return;
  // lane: column m = m0 + 64 wm + 16 mt + l16 of D, rows n = pair base + 8 q4 + (0..7): the
  // first four from half q4 % 2 of the pair, the last four from the other half
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int m = m0 + 64 * wm + 16 * mt + l16;
    if (m >= M) continue;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int n = n0 + 64 * wn + 32 * p + 8 * q4;
      if (n >= N) continue;
      float o[8];
      const int h0 = q4 & 1;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        o[v] = h0 ? acc[mt][2 * p + 1][v] : acc[mt][2 * p][v];
        o[4 + v] = h0 ? acc[mt][2 * p][v] : acc[mt][2 * p + 1][v];
      }
      if constexpr (PART) {
        float* dst = part + ((size_t)z * M + m) * N + n;
        *reinterpret_cast<f32x4*>(dst) = f32x4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
      } else {
        store_row<bf16, 8>(Cm + (size_t)m * ldc + n, o);
      }
    }
  }
}

// C[m][n] = sum_{z < S} part[z][m][n] in slice order.
__global__ __launch_bounds__(256) void gemm_tiled_reduce_kernel(const float* __restrict__ part, int S, int M, int N,
                                                                bf16* __restrict__ Cm, int ldc) {
  const int n8 = N / 8;
  const size_t slice = (size_t)M * N;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < (size_t)M * n8; e += (size_t)gridDim.x * 256) {
    const int m = (int)(e / n8), c = (int)(e % n8) * 8;
    const float* p = part + (size_t)m * N + c;
    f32x4 a0 = *reinterpret_cast<const f32x4*>(p), a1 = *reinterpret_cast<const f32x4*>(p + 4);
    for (int z = 1; z < S; ++z) {
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(p + z * slice);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(p + z * slice + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a0[j] += v0[j];
        a1[j] += v1[j];
      }
    }
    const float o[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    store_row<bf16, 8>(Cm + (size_t)m * ldc + c, o);
  }
}

// Four waves compute, four more only stream the ring (a compute wave that issued its own
// eight loads a stage spent 750 of its 2000 clocks a stage issuing them, per-phase clock
// stamps on gfx950; the data had landed long before it waited for them). With loader waves
// one block fits a compute unit (146 registers a lane), so the ring may be deeper: four
// stages once a slice is long or the tiles alone fill the chip, two otherwise (measured on
// gfx950: EfficientFormer g_w 24.3 -> 19.2 us, BERT FFN g_w 10.8 -> 8.0 us, EfficientFormer
// up g_hat_x 29.1 -> 18.3 us unsplit).
constexpr int GEMM_TILED_LOADERS = 4;

int gemm_tiled_slices(int M, int N, int K) {
  const long tiles = (long)((M + GT - 1) / GT) * ((N + GT - 1) / GT);
  const int nst = (K + GBK - 1) / GBK;
  // Split K while the blocks still fit one to a compute unit and every slice keeps >= 8
  // stages: the partials' write and re-read only pay off against a long K (measured on
  // gfx950 with loader waves and four stages: EfficientFormer g_w, 56 tiles, K = 3712: 32.4 /
  // 23.6 / 19.2 / 26.9 us unsplit / 2 / 4 / 8 slices with the reduction; BERT FFN g_w, 144
  // tiles, K = 448: 8.0 us unsplit, 22 us in two slices).
  int S = 1;
  while (tiles * 2 * S <= 256 && S < 16 && nst / (2 * S) >= 8) S *= 2;
  return S;
}

bool gemm_tiled_applies(bool a_kmajor, int M, int N, int K) {
  const long tiles = (long)((M + GT - 1) / GT) * ((N + GT - 1) / GT);
  if (N % 8 || (a_kmajor ? M % 8 : K % 8)) return false;
  // (measured on gfx950 against the register-blocked GEMM of kernels_hot.hip, same run)
  // g_w (k-major A): ahead wherever the output is not huge (EfficientFormer 34.1 -> 19.5 us
  // with the reduction, BERT FFN 10.5 -> 7.9 us); with >= 2048 tiles and a short K (LLM MLP,
  // 2752 tiles, K = 272) the register-blocked kernel's 43.7 us beat 67.4 us.
  if (a_kmajor) return tiles < 2048;
  // g_hat_x (m-major A, the weight as B): ahead once the tiles alone cover the compute units
  // (EfficientFormer down, 406 tiles: 30.3 -> 15.1 us); with fewer tiles the eight-wave
  // K-splitting blocks of the register-blocked kernel win (EfficientFormer up 17.4 against
  // 19.3 us, BERT FFN 8.5-13.3 against 10.4-15.6 us).
  return tiles >= 256;
}

size_t gemm_tiled_part_floats(int M, int N, int K) {
  const int S = gemm_tiled_slices(M, N, K);
  return S > 1 ? (size_t)S * M * N : 0;
}

hipError_t launch_gemm_tiled(bool a_kmajor, const void* A, int lda, const void* Bm, int ldb, void* Cm, int ldc, int M,
                             int N, int K, float* part, size_t part_floats, const void* zpad, hipStream_t st) {
  if (M < 1 || N < 1 || K < 1 || N % 8 || (a_kmajor ? M % 8 : K % 8) || !zpad) return hipErrorInvalidValue;
  const int S = gemm_tiled_slices(M, N, K);
  if (S > 1 && (!part || (size_t)S * M * N > part_floats)) return hipErrorInvalidValue;
  const unsigned tiles = (unsigned)(((M + GT - 1) / GT) * ((N + GT - 1) / GT));
  const dim3 grid(tiles, 1, S);
  const int nq = (K + GBK - 1) / GBK / S;  // stages of a slice (at least)
  const bool deep = nq >= 12 || tiles >= 256;
  constexpr int NLD = GEMM_TILED_LOADERS;
#define GT_LAUNCH(AK, STG, PT)                                                                                      \
  hipLaunchKernelGGL((gemm_tiled_kernel<AK, STG, PT, NLD>), grid, dim3(64 * (4 + NLD)), 0, st, (const bf16*)A, lda, \
                     (const bf16*)Bm, ldb, (bf16*)Cm, ldc, part, M, N, K, (const bf16*)zpad)
#define GT_STAGES(AK, PT)          \
  if (deep) GT_LAUNCH(AK, 4, PT);  \
  else GT_LAUNCH(AK, 2, PT);
  if (a_kmajor) {
    if (S > 1) { GT_STAGES(true, true) }
    else { GT_STAGES(true, false) }
  } else {
    if (S > 1) { GT_STAGES(false, true) }
    else { GT_STAGES(false, false) }
  }
#undef GT_STAGES
#undef GT_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  const size_t n8 = (size_t)M * (N / 8);
  hipLaunchKernelGGL(gemm_tiled_reduce_kernel, dim3((unsigned)std::min<size_t>((n8 + 255) / 256, 2048)), dim3(256), 0,
                     st, (const float*)part, S, M, N, (bf16*)Cm, ldc);
  return hipGetLastError();
}

}  // namespace instant
