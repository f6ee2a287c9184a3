// Projection kernel of the INSTANT path (notes "INSTANT: Compressing Gradients and
// Activations for Resource-Efficient Training", sections 整体框架 and 关键设计 3):
//   proj    x_hat_b = P x_b (forward compression) and, with the stacked [P; Q],
//           P gy_b and Q gy_b from a single read of gy
// The contraction runs on the matrix cores with float32 accumulation. bf16 inputs stream
// through an LDS ring (proj_lds_kernel); float32 inputs, and bf16 rows not a multiple of 8
// elements, take the register-blocked proj_kernel.
#include <algorithm>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"
#include "lds_tiles.hpp"

namespace instant {
// ----------------------------------------------------------------------------- proj
// Out[b][m][c] = sum_{l < L} A[m][l] X[b][l][c] for m < M, c < C.
// A is [>= M rows][ldA] with zero columns from L up to ldA (ldA a multiple of KSTEP).
// Rows m < M0 go to out0 [B][M0][C]; rows M0 <= m < M go to out1 [B][M - M0][C].
// Grid: (ceil(C / (16 * SW)), B). A lane owns SW adjacent columns; the NW waves of a
// block take every NW-th k-step of the same column strip and issue the loads of U
// steps before any product; the partial tiles are summed through LDS in wave order.
template <class T, int MT, int NW, int U, int SW>
__global__ __launch_bounds__(NW * WAVE) void proj_kernel(const T* __restrict__ A, int ldA, int M, int M0,
                                                         const T* __restrict__ X, int L, int C,
                                                         T* __restrict__ out0, T* __restrict__ out1) {
  typedef MM<T> mm;
  typedef typename mm::frag frag;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  const int b = blockIdx.y;
  const int col = blockIdx.x * (16 * SW) + SW * (lane & 15);
  const bool col_ok = col < C;
  const T* __restrict__ Xb = X + (size_t)b * L * C;
  const int arow = lane & 15;
  const int kl = mm::G * (lane >> 4);

  f32x4 acc[MT][SW];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int j = 0; j < SW; ++j) acc[t][j] = zero4();

  const int nsteps = (L + mm::KSTEP - 1) / mm::KSTEP;
  for (int s0 = wave; s0 < nsteps; s0 += NW * U) {
    frag bf[U][SW];
    frag af[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * NW;
      const int k0 = s * mm::KSTEP + kl;
      load_strip_T<T, SW>(Xb, C, k0, L, col, col_ok, bf[u]);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int m = 16 * t + arow;
        af[u][t] = load_frag<T>(A + (size_t)m * ldA + k0, m < M && s < nsteps);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < SW; ++j) acc[t][j] = mm::mma(af[u][t], bf[u][j], acc[t][j]);
  }

  const int Mb = M - M0;
  auto store = [&](int m, const float v[SW]) {
    if (m >= M || !col_ok) return;
    T* dst = (m < M0) ? out0 + ((size_t)b * M0 + m) * C + col : out1 + ((size_t)b * Mb + (m - M0)) * C + col;
    store_row<T, SW>(dst, v);
  };

  if constexpr (NW == 1) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float o[SW];
#pragma unroll
        for (int j = 0; j < SW; ++j) o[j] = acc[t][j][v];
        store(16 * t + 4 * (lane >> 4) + v, o);
      }
  } else {
    __shared__ float red[NW][SW][4][WAVE];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
      for (int j = 0; j < SW; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave][j][v][lane] = acc[t][j][v];
      __syncthreads();
      for (int v = wave; v < 4; v += NW) {
        float o[SW];
#pragma unroll
        for (int j = 0; j < SW; ++j) {
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

template <class T, int MT, int NW, int SW,
          int U = NW >= 8 ? (MT <= 2 ? 2 : 1) : (MT <= 2 ? 4 : (MT <= 5 ? 2 : 1))>
static hipError_t proj_cfg(const void* A, int ldA, int M, int M0, const void* X, int B, int L, int C, void* out0,
                           void* out1, hipStream_t st) {
  // (U: loads in flight vs registers; with eight waves a strip is already split finely)
  dim3 grid((C + 16 * SW - 1) / (16 * SW), B);
  hipLaunchKernelGGL((proj_kernel<T, MT, NW, U, SW>), grid, dim3(NW * WAVE), 0, st, (const T*)A, ldA, M, M0,
                     (const T*)X, L, C, (T*)out0, (T*)out1);
  return hipGetLastError();
}

template <class T, int MT>
static hipError_t proj_mt(const void* A, int ldA, int M, int M0, const void* X, int B, int L, int C, void* out0,
                          void* out1, hipStream_t st) {
  const int nsteps = (L + MM<T>::KSTEP - 1) / MM<T>::KSTEP;
  // A token axis of one or two k-steps (EfficientFormer's 49 tokens): one wave per block and
  // sample strip, all k-steps in one wave and no reduction across waves; the blocks are small
  // enough to keep every compute unit busy (measured on gfx950 at B = 128, L = 49: 27.0 ->
  // 15.2 us for [P; Q] g_y with C = 1792, 20.4 -> 9.4 us for x_hat with C = 1792, 6.1 -> 4.7 us
  // with C = 448, against two waves splitting the two k-steps)
  // (float32 reaches two k-steps only with L <= 32, so M = Rx + Ry <= 64: MT <= 4)
  if constexpr (sizeof(T) == 2 || MT <= 4) {
    if (nsteps <= 2) return proj_cfg<T, MT, 1, 8, 2>(A, ldA, M, M0, X, B, L, C, out0, out1, st);
  }
  // eight waves per strip keep the most loads in flight per compute unit (measured on
  // gfx950 at B=32, L=512, C=768); narrower strips when 128-column strips would leave
  // compute units idle and the token axis is short
  const bool narrow = (long)((C + 127) / 128) * B < 256 && C > 64 && nsteps < 8;
  // (512-thread blocks leave 256 registers per lane: only the narrow stacks fit)
  if constexpr (MT <= 2) {
    if (nsteps >= 8) return proj_cfg<T, MT, 8, 8>(A, ldA, M, M0, X, B, L, C, out0, out1, st);
  }
  if (nsteps >= 4)
    return narrow ? proj_cfg<T, MT, 4, 4>(A, ldA, M, M0, X, B, L, C, out0, out1, st)
                  : proj_cfg<T, MT, 4, 8>(A, ldA, M, M0, X, B, L, C, out0, out1, st);
  if (nsteps >= 2)
    return narrow ? proj_cfg<T, MT, 2, 4>(A, ldA, M, M0, X, B, L, C, out0, out1, st)
                  : proj_cfg<T, MT, 2, 8>(A, ldA, M, M0, X, B, L, C, out0, out1, st);
  return narrow ? proj_cfg<T, MT, 1, 4>(A, ldA, M, M0, X, B, L, C, out0, out1, st)
                : proj_cfg<T, MT, 1, 8>(A, ldA, M, M0, X, B, L, C, out0, out1, st);
}

// ------------------------------------------------------------------ proj through LDS (bf16)
// The same product for bf16 inputs. Block (128-column strip, sample): stages of 64 tokens x
// 128 columns of X (16 KB, k-major) and the matching 64 columns of every row of A (MA rows of
// 128 bytes, m-major) go from memory straight to LDS (global_load_lds) through a PROJ_STAGES
// deep ring; each of the four compute waves owns 32 columns and all the row tiles, reading X
// fragments with the transpose read and A fragments with 16-byte reads (lds_tiles.hpp), and
// accumulates over every token itself: no cross-wave reduction. Against the register-blocked
// kernel, whose loads wait in registers beside 16 * MT * SW accumulators, the ring keeps three
// stages of X in flight whatever the number of rows (measured on gfx950, bit-identical outputs:
// LLM MLP [P; Q] g_y, 68 rows, 99.7 -> 72.3 us; x_hat, 34 rows, 32.5 -> 27.0 us; BERT FFN
// [P; Q] g_y, 28 rows, 27.0 -> 19.5 us; attention [P; Q] g_y, 16 rows, 7.1 -> 6.1 us).
// With two or more row tiles, four more waves only stream the ring: each issues the 4 + MA / 32
// loads of a stage that one compute wave would (rows and tokens out of range read the zero
// pad), so the waits are exact counts, and the compute waves do not stall on issuing them
// (measured on gfx950, same box: LLM MLP backward 204.1 -> 202.0 us, BERT FFN 52.3 -> 51.8
// us; the kernel alone at the LLM size 81.0 -> 70.7 us). With one row tile the compute waves
// stream it themselves (attention backward 17.09 us against 17.21 us with loaders). The MFMA
// takes the X operand first: a lane then holds 8 consecutive columns of one output row (the
// pair layout of kmajor_frag), stored as 16 bytes. Needs C % 8 == 0 (16-byte rows); A zero from
// column L up to ldA >= the next multiple of 8.
constexpr int PROJ_STAGES = 4;

template <int MTL, int MA, int STG, int NLD>
__global__ __launch_bounds__(64 * (4 + NLD)) void proj_lds_kernel(const bf16* __restrict__ A, int ldA, int M, int M0,
                                                       const bf16* __restrict__ X, int L, int C,
                                                       bf16* __restrict__ out0, bf16* __restrict__ out1,
                                                       const bf16* __restrict__ zpad) {
  typedef MM<bf16> mm;
  constexpr int XT = 16384;             // X tile of a stage: 64 rows x 256 bytes
  constexpr int STAGE = XT + MA * 128;  // then the A tile: MA rows x 128 bytes
  constexpr int LDPS = 4 + MA / 32;     // DMA loads per wave and stage
  static_assert(MA % 32 == 0 && 16 * MTL <= MA && LDPS * (STG - 2) <= 63, "A rows, vmcnt range");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[STG][STAGE];
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  // NLD = 4: four more waves only stream the ring (loader li issues what compute wave li
  // would); NLD = 0: the four compute waves stream it themselves
  const bool loader = NLD ? wave >= 4 : true;
  const bool computer = wave < 4;
  const int li = NLD ? wave - 4 : wave;
  const int n0 = blockIdx.x * 128, b = blockIdx.y;
  const bf16* __restrict__ Xb = X + (size_t)b * L * C;
  const int nq = (L + 63) / 64;
  auto issue = [&](int s, int slot) {
    unsigned char* st = ring[slot];
    const int k0 = 64 * s;
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // X: rows 16 j + 4 wave + lane / 16, 16 chunks a row
      const int r = 16 * j + 4 * li + (lane >> 4);
      const int lc = (lane & 15) ^ kswz_b(r);
      const int k = k0 + r, n = n0 + 8 * lc;
      lds_dma16((k < L && n < C) ? (const void*)(Xb + (size_t)k * C + n) : (const void*)zpad,
                st + 1024 * (4 * j + li));
    }
#pragma unroll
    for (int j = 0; j < MA / 32; ++j) {  // A: rows 32 j + 8 wave + lane / 8, 8 chunks a row
      const int r = 32 * j + 8 * li + (lane >> 3);
      const int lc = (lane & 7) ^ mswz(r);
      const int kk = k0 + 8 * lc;
      lds_dma16((r < M && kk < L) ? (const void*)(A + (size_t)r * ldA + kk) : (const void*)zpad,
                st + XT + 1024 * (4 * j + li));
    }
  };
  f32x4 acc[MTL][2];
#pragma unroll
  for (int t = 0; t < MTL; ++t) acc[t][0] = acc[t][1] = zero4();
  if (loader) {
#pragma unroll
    for (int q = 0; q < STG - 1; ++q)
      if (q < nq) issue(q, q);
  }
  const int q4 = lane >> 4, l16 = lane & 15;
  for (int i = 0; i < nq; ++i) {
    // (waves that issue no loads pass the count at once; all wait for their LDS reads)
    const int later = (nq - 1 - i) < (STG - 2) ? (nq - 1 - i) : (STG - 2);
    wait_oldest_stage<LDPS, STG - 2>(later);
    bare_barrier();  // stage i has landed for every wave; the slot refilled next is free
    if (loader && i + STG - 1 < nq) issue(i + STG - 1, (i + STG - 1) % STG);
    if (!computer) continue;
    const unsigned char* st = ring[i % STG];
    const unsigned char* ta = st + XT;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const mm::frag x0 = kmajor_frag<true>(st, h, lane, 32 * wave, 0);
      const mm::frag x1 = kmajor_frag<true>(st, h, lane, 32 * wave, 1);
#pragma unroll
      for (int t = 0; t < MTL; ++t) {
        const int r = 16 * t + l16;
        const mm::frag af = *reinterpret_cast<const mm::frag*>(ta + r * 128 + 16 * ((4 * h + q4) ^ mswz(r)));
        acc[t][0] = mm::mma(x0, af, acc[t][0]);
        acc[t][1] = mm::mma(x1, af, acc[t][1]);
      }
    }
  }
  // lane: row m = 16 t + l16, columns n .. n + 7: the first four from half q4 % 2 of the
  // wave's column pair, the last four from the other half
  if (!computer) return;
  const int Mb = M - M0;
  const int n = n0 + 32 * wave + 8 * q4;
  if (n >= C) return;
#pragma unroll
  for (int t = 0; t < MTL; ++t) {
    const int m = 16 * t + l16;
    if (m >= M) continue;
    float o[8];
    const int h0 = q4 & 1;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      o[v] = h0 ? acc[t][1][v] : acc[t][0][v];
      o[4 + v] = h0 ? acc[t][0][v] : acc[t][1][v];
    }
    bf16* dst = m < M0 ? out0 + ((size_t)b * M0 + m) * C + n : out1 + ((size_t)b * Mb + (m - M0)) * C + n;
    store_row<bf16, 8>(dst, o);
  }
}

template <int MTL>
static hipError_t proj_lds_mt(const void* A, int ldA, int M, int M0, const void* X, int B, int L, int C, void* out0,
                              void* out1, const void* zpad, hipStream_t st) {
  constexpr int MA = (16 * MTL + 31) / 32 * 32;
  constexpr int NLD = MTL >= 2 ? 4 : 0;
  const dim3 grid((C + 127) / 128, B), block(64 * (4 + NLD));
  // a token axis of one or two stages (EfficientFormer's 49 tokens) takes a two-stage ring: the
  // smaller LDS footprint fits more blocks per compute unit (measured on gfx950 at B = 128,
  // L = 49: [P; Q] g_y 15.1 -> 12.0 us with C = 1792, 6.5 -> 4.7 us with C = 448; x_hat 4.6 ->
  // 3.9 us and 9.3 -> 8.5 us, against the one-wave register-blocked blocks)
  if ((L + 63) / 64 <= 2)
    hipLaunchKernelGGL((proj_lds_kernel<MTL, MA, 2, NLD>), grid, block, 0, st, (const bf16*)A, ldA, M, M0,
                       (const bf16*)X, L, C, (bf16*)out0, (bf16*)out1, (const bf16*)zpad);
  else
    hipLaunchKernelGGL((proj_lds_kernel<MTL, MA, PROJ_STAGES, NLD>), grid, block, 0, st, (const bf16*)A, ldA, M, M0,
                       (const bf16*)X, L, C, (bf16*)out0, (bf16*)out1, (const bf16*)zpad);
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
                       void* out0, void* out1, const void* zpad, hipStream_t st) {
  if (bf16_io && zpad && C % 8 == 0) {
    switch ((M + 15) / 16) {
      case 1: return proj_lds_mt<1>(A, ldA, M, M0, X, B, L, C, out0, out1, zpad, st);
      case 2: return proj_lds_mt<2>(A, ldA, M, M0, X, B, L, C, out0, out1, zpad, st);
      case 3: return proj_lds_mt<3>(A, ldA, M, M0, X, B, L, C, out0, out1, zpad, st);
      case 4: return proj_lds_mt<4>(A, ldA, M, M0, X, B, L, C, out0, out1, zpad, st);
      case 5: return proj_lds_mt<5>(A, ldA, M, M0, X, B, L, C, out0, out1, zpad, st);
      case 6: return proj_lds_mt<6>(A, ldA, M, M0, X, B, L, C, out0, out1, zpad, st);
      case 7: return proj_lds_mt<7>(A, ldA, M, M0, X, B, L, C, out0, out1, zpad, st);
      case 8: return proj_lds_mt<8>(A, ldA, M, M0, X, B, L, C, out0, out1, zpad, st);
      default: return hipErrorInvalidValue;
    }
  }
  return bf16_io ? proj_t<bf16>(A, ldA, M, M0, X, B, L, C, out0, out1, st)
                 : proj_t<float>(A, ldA, M, M0, X, B, L, C, out0, out1, st);
}

}  // namespace instant
