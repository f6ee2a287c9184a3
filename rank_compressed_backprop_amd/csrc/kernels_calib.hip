// Calibration kernels of INSTANT (notes "INSTANT: Compressing Gradients and Activations
// for Resource-Efficient Training", sections 关键设计 1 and 关键设计 2):
//   syrk            running sums S += sum_b t_b t_b^T of the token autocorrelation, on the
//                   matrix cores, upper-triangle 128x128 tiles, deterministic split
//                   reduction into float64
//   build_io        I/O-dtype copies of the published projections
// The eigen-decomposition and truncation live in kernels_eig.hip.
#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

namespace instant {

// ============================================================================ SYRK
// Running sums S += sum_b X_b X_b^T over upper-triangle 128x128 tiles. A block of four
// waves owns one tile and one slice of the (sample, channel) reduction; each wave owns a
// 64x64 quarter. A k-step covers 32 bf16 / 16 fp32 values; a stage of the LDS ring holds
// two k-steps, i.e. 128 bytes (a whole cache line) of every row of the tile's two row
// panels (one panel for diagonal tiles). Stages go straight from memory to LDS
// (global_load_lds, 16 bytes per lane) through a SYRK_STAGES-deep ring, so later stages'
// loads are in flight while the matrix cores consume the oldest. Within a panel, 16-byte
// chunk c of row r sits in slot c ^ (r & 7): the fragment reads of 16 consecutive rows
// then run at the full LDS rate (measured on gfx950; an extra flip of the slot for rows
// 8-15 cost a quarter of it). Lanes whose row or channel is out of range
// read a zeroed pad instead. Slices write float32 partial tiles (in fragment order); a
// second kernel adds them to the float64 sums in slice order.
constexpr int ST = 128;           // statistics tile edge
// LDS ring depth (32 KB a stage). Two stages leave room for two blocks per compute unit,
// whose barriers and fragment reads then overlap the other block's products (measured on
// gfx950: 21.8 against 27.7 us at L = 512, B = 32, C = 768; 578 against 654 us at L = 2048
// with the same slices; rings of 4-8 stages with one block per unit were no faster than 3).
constexpr int SYRK_STAGES = 2;
constexpr int SYRK_LOADERS = 4;   // waves that only stream the ring, besides the four computing

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

constexpr int WPANEL = ST * 128;  // bytes per panel of a stage
__device__ inline int slot_swz(int r) { return r & 7; }

// NLD = 0: the four compute waves also stream the ring; NLD = 4 or 8: that many more waves
// only stream it (a wave sustains about a sixth of a compute unit's L2 read bandwidth).
template <class T, int STAGES, int NLD>
__global__ __launch_bounds__(64 * (4 + NLD)) void syrk_kernel(SyrkSide s0, SyrkSide s1, int B, int L,
                                                              const T* __restrict__ zpad) {
  typedef MM<T> mm;
  typedef typename mm::frag frag;
  constexpr int LOADERS = NLD ? NLD : 4;
  constexpr int HP = 16 / LOADERS;  // wave-loads per panel and loader
  static_assert(STAGES >= 2 && 2 * HP * (STAGES - 2) <= 63, "outstanding loads must fit the vmcnt counter");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[STAGES][2][WPANEL];
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int wave = tid / WAVE;
  const int Tn = (L + ST - 1) / ST;
  const int ntiles = Tn * (Tn + 1) / 2;
  // blocks [0, ntiles * s0.nsplit) serve the first statistic, the rest the second
  int lin = blockIdx.x;
  const bool second = lin >= ntiles * s0.nsplit;
  if (second) lin -= ntiles * s0.nsplit;
  const T* __restrict__ X = (const T*)(second ? s1.X : s0.X);
  const int C = second ? s1.C : s0.C;
  const int nsplit = second ? s1.nsplit : s0.nsplit;
  float* __restrict__ part = second ? s1.part : s0.part;
  int tile, s;
  if (nsplit % 8 == 0) {
    const int xcd = lin % 8, kq = lin / 8;
    s = xcd + 8 * (kq / ntiles);
    tile = kq % ntiles;
  } else {
    s = lin / ntiles;
    tile = lin % ntiles;
  }
  int ti, tj;
  upper_tile(tile, Tn, ti, tj);
  const bool diag = ti == tj;
  const int steps_c = (C + mm::KSTEP - 1) / mm::KSTEP;
  const int pairs_c = (steps_c + 1) / 2;
  const int total = B * pairs_c;
  const int beg = (int)((long)total * s / nsplit);
  const int end = (int)((long)total * (s + 1) / nsplit);
  const int nq = end - beg;

  // A slice is a range of stages in (sample, channel) order; a stage past the last channel
  // reads zeros. Wave-load j = HP * loader + h moves rows 8j .. 8j+7 of a panel (1 KB).
  constexpr int EPC = 16 / (int)sizeof(T);
  const bool loader = NLD ? wave >= 4 : true;
  const bool computer = wave < 4;
  const int li = NLD ? wave - 4 : wave;
  auto issue = [&](int q, int stage) {
    const int b = q / pairs_c;
    const int k0 = (q - b * pairs_c) * 2 * mm::KSTEP;
    const T* __restrict__ Xb = X + (size_t)b * L * C;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (p == 1 && diag) break;
      const int tb = p == 0 ? ti : tj;
#pragma unroll
      for (int h = 0; h < HP; ++h) {
        const int j = HP * li + h;
        const int rloc = 8 * j + (lane >> 3);
        const int chunk = (lane & 7) ^ slot_swz(rloc);
        const int row = tb * ST + rloc;
        const int kk = k0 + chunk * EPC;
        const T* src = (row < L && kk < C) ? Xb + (size_t)row * C + kk : zpad;
        lds_dma16(src, &lds[stage][p][1024 * j]);
      }
    }
  };

  const int wr = wave >> 1, wc = wave & 1;
  f32x4 acc[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[t][u] = zero4();

  if (loader) {
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
      if (st < nq) issue(beg + st, st);
  }
  const int g = lane >> 4;
  for (int i = 0; i < nq; ++i) {
    // (waves that issue no loads pass the count at once; all wait for their LDS reads)
    const int younger = (nq - 1 - i) < (STAGES - 2) ? (nq - 1 - i) : (STAGES - 2);
    if (diag) wait_oldest_stage<HP, STAGES - 2>(younger);
    else wait_oldest_stage<2 * HP, STAGES - 2>(younger);
    bare_barrier();
    if (loader && i + STAGES - 1 < nq) issue(beg + i + STAGES - 1, (i + STAGES - 1) % STAGES);
    if (!computer) continue;
    const unsigned char* pa = lds[i % STAGES][0];
    const unsigned char* pb = diag ? pa : lds[i % STAGES][1];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      frag af[4], bf[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int ra = 64 * wr + 16 * t + (lane & 15);
        const int rb = 64 * wc + 16 * t + (lane & 15);
        af[t] = *reinterpret_cast<const frag*>(pa + ra * 128 + 16 * ((4 * h + g) ^ slot_swz(ra)));
        bf[t] = *reinterpret_cast<const frag*>(pb + rb * 128 + 16 * ((4 * h + g) ^ slot_swz(rb)));
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[t][u] = mm::mma(af[t], bf[u], acc[t][u]);
    }
  }

  if (!computer) return;
  // the partial tile in fragment order: one 16-byte store per lane and 16x16 tile
  float* __restrict__ out = part + ((size_t)s * ntiles + tile) * (ST * ST);
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<f32x4*>(out + (((wave * 16 + t * 4 + u) * WAVE + lane) * 4)) = acc[t][u];
}

// ---------------------------------------------------------------- SYRK, wide blocks
// The same sums for long token axes (bf16): a block owns a 256 x 128 pair of upper-triangle
// tiles, the 128-row tiles 2I and 2I + 1 against the 128-column tile J >= 2I, over one slice.
// Each of its four compute waves owns 128 x 64 (eight row tiles of 16 against four column
// tiles), so a k-step reads 12 fragments for 32 products instead of 8 for 16: a third less
// LDS traffic per product than the 128 x 128 blocks, whose compute units are bound by their
// LDS port. A stage holds 64 channels of the 256-row panel (32 KB) and of the 128-row panel
// (16 KB; none when tile J is one of the pair, which the first panel then holds); four loader
// waves stream a SYRK_WIDE_STAGES-deep ring. The waves write the float32 partials of each of
// their two 128 x 128 tiles in the fragment order of syrk_kernel, so syrk_reduce_kernel adds
// them unchanged, and the sums are the same bit for bit. Below the diagonal (tile 2I + 1
// against J = 2I) and beyond the last tile nothing is written.
constexpr int SYRK_WIDE_STAGES = 3;  // 144 KB of LDS: one block a compute unit
// Token axes of 16 128-row tiles (L > 1920) take the wide blocks (measured on gfx950, SYRK and
// fold a batch, bit-identical sums: LLM MLP, B = 8, L = 2048, C = 4096 / 11008, 790-803 ->
// 702-717 us; C = 4096 / 4096, 440-443 -> 397-406 us; at L = 1024 the 128 x 128 blocks, two a
// compute unit, stay ahead: 50.3 against 51.9 us)
constexpr int WIDE_MIN_TILES = 16;

int syrk_wide_pairs(int L) {
  const int T = (L + ST - 1) / ST, m = T / 2;
  return T % 2 ? (m + 1) * (m + 1) : m * (m + 1);
}

// sum over I < ceil(T / 2) of T - 2I: m (m + 1) for T = 2m, (m + 1)^2 for T = 2m + 1
__device__ inline int syrk_wide_pairs_dev(int T) {
  const int m = T / 2;
  return T % 2 ? (m + 1) * (m + 1) : m * (m + 1);
}

__device__ inline void wide_pair(int idx, int T, int& I, int& J) {
  I = 0;
  while (idx >= T - 2 * I) {
    idx -= T - 2 * I;
    ++I;
  }
  J = 2 * I + idx;
}

__device__ inline int upper_index(int ti, int tj, int T) { return ti * T - ti * (ti - 1) / 2 + (tj - ti); }

template <int STAGES>
__global__ __launch_bounds__(512) void syrk_wide_kernel(SyrkSide s0, SyrkSide s1, int B, int L,
                                                        const bf16* __restrict__ zpad) {
  typedef MM<bf16> mm;
  typedef mm::frag frag;
  constexpr int PA = 2 * WPANEL;  // 256-row panel of a stage
  static_assert(12 * (STAGES - 2) <= 63, "outstanding loads must fit the vmcnt counter");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[STAGES][PA + WPANEL];
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int T = (L + ST - 1) / ST;
  const int ntiles = T * (T + 1) / 2;
  const int npairs = syrk_wide_pairs_dev(T);
  int lin = blockIdx.x;
  const bool second = lin >= npairs * s0.nsplit;
  if (second) lin -= npairs * s0.nsplit;
  const bf16* __restrict__ X = (const bf16*)(second ? s1.X : s0.X);
  const int C = second ? s1.C : s0.C;
  const int nsplit = second ? s1.nsplit : s0.nsplit;
  float* __restrict__ part = second ? s1.part : s0.part;
  int pair, s;
  if (nsplit % 8 == 0) {  // slice s on XCD s % 8, as in syrk_kernel
    const int xcd = lin % 8, kq = lin / 8;
    s = xcd + 8 * (kq / npairs);
    pair = kq % npairs;
  } else {
    s = lin / npairs;
    pair = lin % npairs;
  }
  int I, J;
  wide_pair(pair, T, I, J);
  const bool shared = J < 2 * I + 2;  // tile J is one of the pair: the 256-row panel holds it
  const int pairs_c = ((C + mm::KSTEP - 1) / mm::KSTEP + 1) / 2;
  const int total = B * pairs_c;
  const int beg = (int)((long)total * s / nsplit);
  const int end = (int)((long)total * (s + 1) / nsplit);
  const int nq = end - beg;

  const bool loader = wave >= 4;
  const int li = wave - 4;
  // wave-load j moves rows 8j .. 8j+7 of a panel (1 KB): 32 of the first panel, 16 of the second
  auto issue = [&](int q, int stage) {
    const int b = q / pairs_c;
    const int k0 = (q - b * pairs_c) * 2 * mm::KSTEP;
    const bf16* __restrict__ Xb = X + (size_t)b * L * C;
    auto one = [&](int base_row, int j, unsigned char* dst) {
      const int rloc = 8 * j + (lane >> 3);
      const int chunk = (lane & 7) ^ slot_swz(rloc);
      const int row = base_row + rloc;
      const int kk = k0 + chunk * 8;
      const bf16* src = (row < L && kk < C) ? Xb + (size_t)row * C + kk : zpad;
      lds_dma16(src, dst + 1024 * j);
    };
#pragma unroll
    for (int h = 0; h < 8; ++h) one(2 * ST * I, 8 * li + h, lds[stage]);
    if (!shared) {
#pragma unroll
      for (int h = 0; h < 4; ++h) one(ST * J, 4 * li + h, lds[stage] + PA);
    }
  };

  const int wr = wave >> 1, wc = wave & 1;
  f32x4 acc[8][4];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[t][u] = zero4();

  if (loader) {
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
      if (st < nq) issue(beg + st, st);
  }
  const int g = lane >> 4;
  for (int i = 0; i < nq; ++i) {
    // (compute waves issue no loads and pass the count at once; all wait for their LDS reads)
    const int younger = (nq - 1 - i) < (STAGES - 2) ? (nq - 1 - i) : (STAGES - 2);
    if (shared) wait_oldest_stage<8, STAGES - 2>(younger);
    else wait_oldest_stage<12, STAGES - 2>(younger);
    bare_barrier();
    if (loader) {
      if (i + STAGES - 1 < nq) issue(beg + i + STAGES - 1, (i + STAGES - 1) % STAGES);
      continue;
    }
    const unsigned char* pa = lds[i % STAGES];
    const unsigned char* pb = shared ? pa + WPANEL * (J - 2 * I) : pa + PA;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      frag af[8], bf[4];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int ra = ST * wr + 16 * t + (lane & 15);
        af[t] = *reinterpret_cast<const frag*>(pa + ra * 128 + 16 * ((4 * h + g) ^ slot_swz(ra)));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int rb = 64 * wc + 16 * u + (lane & 15);
        bf[u] = *reinterpret_cast<const frag*>(pb + rb * 128 + 16 * ((4 * h + g) ^ slot_swz(rb)));
      }
      // every read of the k-step before its products (left to the compiler's order: 4-10% slower)
      __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 32, 0);
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[t][u] = mm::mma(af[t], bf[u], acc[t][u]);
    }
  }

  if (loader) return;
  // rows 128 wr .. of the pair: tile ti = 2I + wr against tj = J, upper triangle only
  const int ti = 2 * I + wr, tj = J;
  if (ti >= T || tj < ti) return;
  float* __restrict__ out = part + ((size_t)s * ntiles + upper_index(ti, tj, T)) * (ST * ST);
#pragma unroll
  for (int t8 = 0; t8 < 8; ++t8)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ow = 2 * (t8 >> 2) + wc;  // the 64 x 64 quarter of syrk_kernel's fragment order
      *reinterpret_cast<f32x4*>(out + (((ow * 16 + (t8 & 3) * 4 + u) * WAVE + lane) * 4)) = acc[t8][u];
    }
}

// S[i][j] += sum_s part[s][tile] in split order, float64, for the upper-triangle tiles (or
// S[i][j] = that sum for a statistic's first batch).
__global__ __launch_bounds__(256) void syrk_reduce_kernel(SyrkSide s0, SyrkSide s1, int ntiles, int L) {
  const SyrkSide& sd = blockIdx.z ? s1 : s0;
  const float* __restrict__ part = sd.part;
  const int nsplit = sd.nsplit;
  double* __restrict__ S = sd.S;
  const int tile = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;  // fragment-order index, see syrk_kernel
  const int Tn = (L + ST - 1) / ST;
  int ti, tj;
  upper_tile(tile, Tn, ti, tj);
  const int wave = e >> 12, t = (e >> 10) & 3, u = (e >> 8) & 3, lane = (e >> 2) & 63, v = e & 3;
  const int i = ti * ST + 64 * (wave >> 1) + 16 * t + 4 * (lane >> 4) + v;
  const int j = tj * ST + 64 * (wave & 1) + 16 * u + (lane & 15);
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
  if (sd.overwrite) S[(size_t)i * L + j] = acc;
  else S[(size_t)i * L + j] += acc;
}

// ---------------------------------------------------------------- statistics, L <= 64
// A token axis of at most 64 (EfficientFormer's 49 tokens) fills one 64 x 64 tile; only its
// ten upper 16 x 16 tiles are computed. The (sample, channel) reduction is cut into k-steps;
// each wave takes SMALL_KPW consecutive ones, loads all of them at once (rows beyond L read as
// zero) and multiplies: in S = sum X X^T the same fragments serve as both operands. The four
// waves of a block are summed through LDS in wave order into one float32 partial per block,
// [part][10 tiles][4][64] in fragment order; syrk_small_reduce_kernel adds the partials
// into the float64 sums in a fixed order.
constexpr int SMALL_KPW = 8;
constexpr int SMALL_TILES = 10;  // 16 x 16 tiles (t, u), t <= u < 4
constexpr int SMALL_PART = SMALL_TILES * 4 * WAVE;

__device__ __forceinline__ void small_tile(int k, int& t, int& u) {
  // (0,0) (0,1) (0,2) (0,3) (1,1) (1,2) (1,3) (2,2) (2,3) (3,3)
  t = k < 4 ? 0 : (k < 7 ? 1 : (k < 9 ? 2 : 3));
  const int first = t == 0 ? 0 : (t == 1 ? 4 : (t == 2 ? 7 : 9));
  u = t + (k - first);
}

template <class T>
__global__ __launch_bounds__(256) void syrk_small_kernel(SyrkSide s0, SyrkSide s1, int nb0, int B, int L) {
  typedef MM<T> mm;
  typedef typename mm::frag frag;
  __shared__ float red[4][SMALL_TILES][4][WAVE];
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const bool second = (int)blockIdx.x >= nb0;
  const int p = second ? blockIdx.x - nb0 : blockIdx.x;
  const T* __restrict__ X = (const T*)(second ? s1.X : s0.X);
  const int C = second ? s1.C : s0.C;
  float* __restrict__ part = second ? s1.part : s0.part;
  const int nks = (C + mm::KSTEP - 1) / mm::KSTEP;
  const int total = B * nks;
  const int q0 = (p * 4 + wave) * SMALL_KPW;
  frag f[SMALL_KPW][4];
#pragma unroll
  for (int i = 0; i < SMALL_KPW; ++i) {
    const int q = q0 + i;
    const int b = q / nks;
    const int c0 = (q - b * nks) * mm::KSTEP + mm::G * (lane >> 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int l = 16 * t + (lane & 15);
      f[i][t] = load_frag<T>(X + ((size_t)b * L + l) * C + c0, q < total && l < L && c0 < C);
    }
  }
  f32x4 acc[SMALL_TILES];
#pragma unroll
  for (int k = 0; k < SMALL_TILES; ++k) acc[k] = zero4();
#pragma unroll
  for (int i = 0; i < SMALL_KPW; ++i)
#pragma unroll
    for (int k = 0; k < SMALL_TILES; ++k) {
      int t, u;
      small_tile(k, t, u);
      acc[k] = mm::mma(f[i][t], f[i][u], acc[k]);
    }
#pragma unroll
  for (int k = 0; k < SMALL_TILES; ++k)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][k][v][lane] = acc[k][v];
  __syncthreads();
  float* __restrict__ out = part + (size_t)p * SMALL_PART;
  const float* r = &red[0][0][0][0];
  for (int e = threadIdx.x; e < SMALL_PART; e += 256)
    out[e] = ((r[e] + r[SMALL_PART + e]) + r[2 * SMALL_PART + e]) + r[3 * SMALL_PART + e];
}

// S[i][j] (+)= sum_p part[p][e] (float64), e the fragment-order index of (i, j). Eight
// threads share an entry: thread g sums the parts of its fixed range [g np / 8, (g+1) np / 8)
// in order, four loads in flight, and the eight range sums are added in range order.
constexpr int SMALL_RED_GROUPS = 8;
constexpr int SMALL_RED_ENTRIES = 256 / SMALL_RED_GROUPS;  // entries per block
__global__ __launch_bounds__(256) void syrk_small_reduce_kernel(SyrkSide s0, SyrkSide s1, int np0, int np1, int L) {
  __shared__ double red[SMALL_RED_GROUPS][SMALL_RED_ENTRIES];
  const SyrkSide& sd = blockIdx.y ? s1 : s0;
  const int np = blockIdx.y ? np1 : np0;
  const int g = threadIdx.x / SMALL_RED_ENTRIES, j = threadIdx.x % SMALL_RED_ENTRIES;
  const int e = blockIdx.x * SMALL_RED_ENTRIES + j;  // < SMALL_PART
  const int qb = (int)((long)np * g / SMALL_RED_GROUPS), qe = (int)((long)np * (g + 1) / SMALL_RED_GROUPS);
  const float* __restrict__ pp = sd.part + e;
  double acc = 0.0;
  int q = qb;
  for (; q + 4 <= qe; q += 4) {
    const float v0 = pp[(size_t)(q + 0) * SMALL_PART], v1 = pp[(size_t)(q + 1) * SMALL_PART];
    const float v2 = pp[(size_t)(q + 2) * SMALL_PART], v3 = pp[(size_t)(q + 3) * SMALL_PART];
    acc += (double)v0;
    acc += (double)v1;
    acc += (double)v2;
    acc += (double)v3;
  }
  for (; q < qe; ++q) acc += (double)pp[(size_t)q * SMALL_PART];
  red[g][j] = acc;
  __syncthreads();
  if (g != 0) return;
  double sum = red[0][j];
#pragma unroll
  for (int h = 1; h < SMALL_RED_GROUPS; ++h) sum += red[h][j];
  int t, u;
  small_tile(e >> 8, t, u);
  const int v = (e >> 6) & 3, lane = e & 63;
  const int i = 16 * t + 4 * (lane >> 4) + v, jj = 16 * u + (lane & 15);
  if (i >= L || jj >= L) return;
  double* __restrict__ S = sd.S;
  if (sd.overwrite) S[(size_t)i * L + jj] = sum;
  else S[(size_t)i * L + jj] += sum;
}

int syrk_small_parts(bool bf16_io, int B, int C) {
  const int kstep = bf16_io ? 32 : 16;
  const long total = (long)B * ((C + kstep - 1) / kstep);
  return (int)((total + 4 * SMALL_KPW - 1) / (4 * SMALL_KPW));
}

size_t syrk_small_part_floats(bool bf16_io, int B, int C) {
  return (size_t)syrk_small_parts(bf16_io, B, C) * SMALL_PART;
}

template <class T>
static hipError_t syrk_small_t(const SyrkSide* sides, int nsides, int B, int L, hipStream_t st) {
  const bool bf = sizeof(T) == 2;
  const SyrkSide s0 = sides[0];
  const SyrkSide s1 = nsides > 1 ? sides[1] : SyrkSide{nullptr, 0, 0, nullptr, nullptr, 0};
  const int np0 = syrk_small_parts(bf, B, s0.C), np1 = nsides > 1 ? syrk_small_parts(bf, B, s1.C) : 0;
  hipLaunchKernelGGL(syrk_small_kernel<T>, dim3(np0 + np1), dim3(256), 0, st, s0, s1, np0, B, L);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(syrk_small_reduce_kernel, dim3(SMALL_PART / SMALL_RED_ENTRIES, nsides), dim3(256), 0, st, s0, s1,
                     np0, np1, L);
  return hipGetLastError();
}

template <class T>
static hipError_t syrk_t(const SyrkSide* sides, int nsides, int B, int L, const void* zpad, hipStream_t st) {
  if (L <= 64) return syrk_small_t<T>(sides, nsides, B, L, st);
  const SyrkSide s0 = sides[0];
  const SyrkSide s1 = nsides > 1 ? sides[1] : SyrkSide{nullptr, 0, 0, nullptr, nullptr, 0};
  const int nt = syrk_tiles(L);
  if (sizeof(T) == 2 && (L + ST - 1) / ST >= WIDE_MIN_TILES)
    hipLaunchKernelGGL((syrk_wide_kernel<SYRK_WIDE_STAGES>), dim3(syrk_wide_pairs(L) * (s0.nsplit + s1.nsplit)),
                       dim3(512), 0, st, s0, s1, B, L, (const bf16*)zpad);
  else
    hipLaunchKernelGGL((syrk_kernel<T, SYRK_STAGES, SYRK_LOADERS>), dim3(nt * (s0.nsplit + s1.nsplit)),
                       dim3(64 * (4 + SYRK_LOADERS)), 0, st, s0, s1, B, L, (const T*)zpad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid(nt, ST * ST / 256, nsides);  // 64 blocks of 256 elements per tile and statistic
  hipLaunchKernelGGL(syrk_reduce_kernel, grid, dim3(256), 0, st, s0, s1, nt, L);
  return hipGetLastError();
}

hipError_t launch_syrk(bool bf16_io, const SyrkSide* sides, int nsides, int B, int L, const void* zpad,
                       hipStream_t st) {
  if (nsides < 1 || nsides > 2) return hipErrorInvalidValue;
  return bf16_io ? syrk_t<bf16>(sides, nsides, B, L, zpad, st) : syrk_t<float>(sides, nsides, B, L, zpad, st);
}

// I/O-dtype copies: PQ rows [0, Rx) = P, [Rx, Rx+Ry) = Q with ld ldL (zero beyond L), and
// Qt[l][r] = Q[r][l] with ld ldQt (zero beyond Ry). Rows of PQ beyond Rx+Ry are zeroed.
template <class T>
__global__ __launch_bounds__(256) void build_io_kernel(const float* __restrict__ P32, const float* __restrict__ Q32,
                                                       const int* __restrict__ dRx, const int* __restrict__ dRy,
                                                       int L, int ldL, int R_max, T* __restrict__ PQ,
                                                       T* __restrict__ Qt, int ldQt) {
  // ranks outside [0, R_max] come from a failed truncation; the copies are then unused
  const int Rx = min(max(*dRx, 0), R_max), Ry = min(max(*dRy, 0), R_max);
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
