// Host runtime of the INSTANT C ABI (include/instant.h): argument checks, workspace
// layout, stream-ordered launches of the kernels, calibration bookkeeping.
//
// Method: notes "INSTANT: Compressing Gradients and Activations for Resource-Efficient
// Training" — 整体框架 (forward keeps x_hat = P x; P, Q refreshed every N_t steps),
// 关键设计 1 (statistics C_X, C_G), 关键设计 2 (truncation, oversampling, compensation),
// 关键设计 3 (reordered low-rank products).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <new>

#include "instant.h"
#include "launch.hpp"

#define INSTANT_API extern "C" __attribute__((visibility("default")))

namespace {

using namespace instant;

constexpr int MAX_L = 2048;  // a Jacobi pair stages 16 columns of L floats in LDS
constexpr int MAX_R = 64;
constexpr int LD_QT = 64;
constexpr int SYRK_TARGET_BLOCKS = 4096;  // tile-slices of a batch's statistics (both sides)
constexpr int SYRK_MIN_STAGES = 16;      // shortest slice: the LDS ring's fill stays small
constexpr int SYRK_MAX_SPLIT = 64;
constexpr int SYRK_TILE = 128;

inline size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// K slices of one statistic's SYRK for a batch of B samples. Both statistics get slices of
// about the same length (the launch holds both, and its time is that of its longest
// blocks), long enough to amortise the ring's fill, short enough to give about
// SYRK_TARGET_BLOCKS tile-slices per batch so that the last round of blocks is short.
// Counts of 8 or more are multiples of 8: slice s then stays on accelerator die s % 8 and
// the row panels of its K range are shared in that die's L2 by every tile (measured on
// gfx950 at L = 2048, B = 8, C = 4096 / 11008: 8 / 24 slices 578 us, 4 / 11 slices
// 802 us, 2 / 2 slices 1037 us). The count depends only on the layer's shapes and B, not
// on which statistics a call carries, so split and joint calls sum identically.
int syrk_nsplit(const instant_config& c, int B, int C) {
  const int kstep = c.dtype == INSTANT_BF16 ? 32 : 16;
  auto stages = [&](int ch) { return (long)B * (((ch + kstep - 1) / kstep + 1) / 2); };  // two k-steps a stage
  const long work = (long)syrk_tiles(c.L) * (stages(c.Cx) + stages(c.Cy));
  const long len = std::max<long>(SYRK_MIN_STAGES, (work + SYRK_TARGET_BLOCKS - 1) / SYRK_TARGET_BLOCKS);
  const long st = stages(C);
  long n = (st + len / 2) / len;
  if (n >= 8) n = (n + 4) / 8 * 8;
  n = std::min<long>(std::min<long>(n, SYRK_MAX_SPLIT), st);
  return (int)std::max<long>(1, n);
}

// The most slices one statistic takes at any batch size up to B_max (sizes its partials).
int syrk_split_max(const instant_config& c, int C) {
  int m = 1;
  for (int b = 1; b <= c.B_max; ++b) m = std::max(m, syrk_nsplit(c, b, C));
  return m;
}

bool config_ok(const instant_config* c) {
  if (!c) return false;
  if (c->L < 1 || c->L > MAX_L) return false;
  if (c->Cx < 8 || c->Cy < 8 || (c->Cx % 8) || (c->Cy % 8)) return false;
  if (c->B_max < 1) return false;
  if (c->R_max < 1 || c->R_max > MAX_R || c->R_max > c->L) return false;
  if (c->p < 0 || c->N_t < 0) return false;
  if (!(c->eps > 0.0f && c->eps <= 1.0f)) return false;
  if (c->dtype != INSTANT_FP32 && c->dtype != INSTANT_BF16) return false;
  if (c->comp < INSTANT_COMP_PAPER || c->comp > INSTANT_COMP_RATIO) return false;
  if (c->max_sweeps < 1) return false;
  if (c->solver != INSTANT_SOLVER_JACOBI && c->solver != INSTANT_SOLVER_SUBSPACE) return false;
  if (c->solver == INSTANT_SOLVER_SUBSPACE && c->sub_iters < 1) return false;
  return true;
}

struct Layout {
  size_t SX, SG, zpad, part, part_x_floats, eig, sig_x, sig_g, info, rank, P32[2], Q32[2], PQ[2], Qt[2], Pgy, Qgy,
      gxh, gpart, gpart_floats, total;
  int ldL;
};

Layout layout_of(const instant_config* c) {
  Layout l;
  const size_t esz = c->dtype == INSTANT_BF16 ? 2 : 4;
  const size_t L = c->L;
  l.ldL = (c->L + 31) / 32 * 32;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  l.SX = take(L * L * sizeof(double));
  l.SG = take(L * L * sizeof(double));
  l.zpad = take(256);
  {
    // float32 partials of the statistics, one region per statistic: split K slices of the
    // 128 x 128 tiles, or the per-block partials of the one-tile path at L <= 64
    auto side = [&](int C) {
      size_t f = (size_t)syrk_split_max(*c, C) * syrk_tiles(c->L) * SYRK_TILE * SYRK_TILE;
      if (c->L <= 64)
        for (int b = 1; b <= c->B_max; ++b) f = std::max(f, syrk_small_part_floats(c->dtype == INSTANT_BF16, b, C));
      return f;
    };
    l.part_x_floats = side(c->Cx);
    l.part = take((l.part_x_floats + side(c->Cy)) * sizeof(float));
  }
  l.eig = take(eig_workspace_bytes(c->L));
  l.sig_x = take(L * sizeof(float));
  l.sig_g = take(L * sizeof(float));
  l.info = take(2 * INFO_WORDS * sizeof(int));
  l.rank = take(2 * sizeof(int));
  for (int b = 0; b < 2; ++b) {
    l.P32[b] = take((size_t)c->R_max * L * sizeof(float));
    l.Q32[b] = take((size_t)c->R_max * L * sizeof(float));
    l.PQ[b] = take((size_t)2 * c->R_max * l.ldL * esz);
    l.Qt[b] = take(L * LD_QT * esz);
  }
  // float32 K-slice partials of the unfused path's GEMMs (they run one after the other):
  // g_hat_x = (Q gy) w read once over K slices when w is too large for L2 (M = B Ry rows), or
  // either GEMM on LDS tiles when its K is split
  {
    size_t need = 0;
    const bool bf = c->dtype == INSTANT_BF16;
    for (int m = 1; m <= c->B_max * c->R_max; ++m)
      need = std::max(need, (size_t)gemm_ws_slices(bf, false, m, c->Cx, c->Cy) * m * c->Cx);
    if (bf)
      for (int m = 1; m <= c->B_max * c->R_max; ++m) {
        if (gemm_tiled_applies(true, c->Cy, c->Cx, m))  // g_w, K = B Rx
          need = std::max(need, gemm_tiled_part_floats(c->Cy, c->Cx, m));
        if (!gemm_ws_slices(true, false, m, c->Cx, c->Cy) && gemm_tiled_applies(false, m, c->Cx, c->Cy))
          need = std::max(need, gemm_tiled_part_floats(m, c->Cx, c->Cy));  // g_hat_x, M = B Ry
      }
    l.gpart_floats = need;
    l.gpart = take(need * sizeof(float));
  }
  l.Pgy = take((size_t)c->B_max * c->R_max * c->Cy * esz);
  l.Qgy = take((size_t)c->B_max * c->R_max * c->Cy * esz);
  l.gxh = take((size_t)c->B_max * c->R_max * c->Cx * esz);
  l.total = off;
  return l;
}

// ---- the scratch of instant_backward_static: one file-scope device array per GPU, held by
// every device the library runs on until the process ends. Host code never uses the
// array's name as an address: its device address is looked up once per device (at the first
// instant_create on that device) and kept in scratch_ptr.
constexpr size_t STATIC_SCRATCH_BYTES = INSTANT_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[STATIC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES];
bool scratch_looked_up[MAX_DEVICES];

// The device address of `scratch` on device `dev` (the current device), looked up on the
// first call for that device; nullptr if the lookup failed.
void* scratch_on(int dev) {
  if (dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_looked_up[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();  // leave no sticky error behind for the caller's next call
      p = nullptr;
    }
    scratch_ptr[dev] = p;
    scratch_looked_up[dev] = true;
  }
  return scratch_ptr[dev];
}

}  // namespace

struct instant_layer {
  instant_config cfg;
  bool bf16;
  char* ws;
  Layout lay;
  int active;  // projection buffer in use, -1 before the first one
  bool warm;   // the eigensolver's accumulated rotation from the last finalize is usable
  int Rx, Ry;
  int64_t nx, ng;
  int ncu;  // compute units of the device the handle was created on
  void* scratch;  // device address of the static scratch on that device (null if unavailable)
  instant_info info;
  instant_status last;
  // outcome of the last finalize: copied by the device into pinned host memory; with an
  // asynchronous finalize it is settled once `done` has passed (pending until then)
  int* hflags;
  hipEvent_t done;
  bool pending;
  int pend_t, pend_m;
  int64_t pend_nx, pend_ng;

  double* SX() const { return (double*)(ws + lay.SX); }
  double* SG() const { return (double*)(ws + lay.SG); }
  // partial tiles of the statistics' split reduction, one region per statistic
  float* part(int side) const { return (float*)(ws + lay.part) + (side ? lay.part_x_floats : 0); }
  int* info_dev() const { return (int*)(ws + lay.info); }
  int* rank_dev() const { return (int*)(ws + lay.rank); }
  float* P32(int b) const { return (float*)(ws + lay.P32[b]); }
  float* Q32(int b) const { return (float*)(ws + lay.Q32[b]); }
  void* PQ(int b) const { return ws + lay.PQ[b]; }
  void* Qt(int b) const { return ws + lay.Qt[b]; }
};

namespace {

inline hipStream_t S(void* stream) { return (hipStream_t)stream; }
inline instant_status hip_ok(hipError_t e) { return e == hipSuccess ? INSTANT_OK : INSTANT_E_HIP; }

// Applies the outcome of the last finalize from the flags the device copied back: the new
// projections become active only if both sides succeeded.
instant_status settle(instant_layer* h) {
  const int* flags = h->hflags;
  const int* ix = flags + EIGF_INFO;
  const int* ig = flags + EIGF_INFO + INFO_WORDS;
  instant_status status = (instant_status)(ix[0] != 0 ? ix[0] : ig[0]);
  if (flags[EIGF_ABORT]) status = INSTANT_E_HIP;  // a bounded wait of the eigensolver gave up

  instant_info& I = h->info;
  I.kx = ix[1];
  I.ky = ig[1];
  I.sweeps_x = flags[EIGF_SWEEPS];
  I.sweeps_g = flags[EIGF_SWEEPS + 1];
  I.status = status;
  float c;
  std::memcpy(&c, &ix[3], 4);
  I.cP = c;
  std::memcpy(&c, &ig[3], 4);
  I.cQ = c;
  std::memcpy(&I.kept_x, &ix[4], 8);
  std::memcpy(&I.kept_g, &ig[4], 8);
  I.n_samples_x = h->pend_nx;
  I.n_samples_g = h->pend_ng;
  if (status == INSTANT_OK) {
    h->active = h->pend_t;
    h->Rx = ix[2];
    h->Ry = ig[2];
    I.Rx = h->Rx;
    I.Ry = h->Ry;
    I.generation += 1;
  }
  h->last = status;
  // a failed decomposition may leave the accumulated rotation unusable: restart cold (a
  // subspace basis that has not converged yet is still the best start for the next one)
  h->warm = (status == INSTANT_OK || status == INSTANT_E_RANK) ||
            (h->pend_m > 0 && status == INSTANT_E_NOCONV);
  return status;
}

// Settles an asynchronous finalize whose work has completed (or, with wait, once it has).
void apply_pending(instant_layer* h, bool wait) {
  if (!h->pending) return;
  hipError_t e = wait ? hipEventSynchronize(h->done) : hipEventQuery(h->done);
  if (e == hipErrorNotReady) return;
  h->pending = false;
  if (e != hipSuccess) {
    h->warm = false;
    h->last = INSTANT_E_HIP;
    h->info.status = INSTANT_E_HIP;
    return;
  }
  settle(h);
}

// Both statistics of a batch (either input may be NULL) in one SYRK launch.
instant_status accumulate(instant_layer* h, const void* x, const void* gy, int B, hipStream_t st) {
  SyrkSide sides[2];
  int n = 0;
  // the first batch of a window overwrites the sums, so a finalize need not clear them
  if (x) sides[n++] = SyrkSide{x, h->cfg.Cx, syrk_nsplit(h->cfg, B, h->cfg.Cx), h->part(0), h->SX(), h->nx == 0};
  if (gy) sides[n++] = SyrkSide{gy, h->cfg.Cy, syrk_nsplit(h->cfg, B, h->cfg.Cy), h->part(1), h->SG(), h->ng == 0};
  return hip_ok(launch_syrk(h->bf16, sides, n, B, h->cfg.L, h->ws + h->lay.zpad, st));
}

}  // namespace

INSTANT_API size_t instant_workspace_bytes(const instant_config* cfg) {
  if (!config_ok(cfg)) return 0;
  return layout_of(cfg).total;
}

INSTANT_API instant_status instant_create(instant_layer** h, const instant_config* cfg, void* workspace,
                                          void* stream) {
  if (!h || !config_ok(cfg) || !workspace) return INSTANT_E_ARG;
  if (((uintptr_t)workspace) % 256) return INSTANT_E_ARG;
  instant_layer* L = new (std::nothrow) instant_layer();
  if (!L) return INSTANT_E_ARG;
  L->cfg = *cfg;
  L->bf16 = cfg->dtype == INSTANT_BF16;
  L->ws = (char*)workspace;
  L->lay = layout_of(cfg);
  L->active = -1;
  L->warm = false;
  L->Rx = L->Ry = 0;
  L->nx = L->ng = 0;
  std::memset(&L->info, 0, sizeof(L->info));
  L->last = INSTANT_OK;
  L->pending = false;
  L->pend_t = L->pend_m = 0;
  L->pend_nx = L->pend_ng = 0;
  L->hflags = nullptr;
  L->done = nullptr;
  if (hipHostMalloc((void**)&L->hflags, EIG_HOST_FLAGS * sizeof(int), hipHostMallocDefault) != hipSuccess) {
    delete L;
    return INSTANT_E_HIP;
  }
  std::memset(L->hflags, 0, EIG_HOST_FLAGS * sizeof(int));
  if (hipEventCreateWithFlags(&L->done, hipEventDisableTiming) != hipSuccess) {
    (void)hipHostFree(L->hflags);
    delete L;
    return INSTANT_E_HIP;
  }
  int dev = 0;
  L->ncu = 0;
  L->scratch = nullptr;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&L->ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || L->ncu < 1) {
    (void)hipEventDestroy(L->done);
    (void)hipHostFree(L->hflags);
    delete L;
    return INSTANT_E_HIP;
  }
  L->scratch = scratch_on(dev);
  // statistics start at zero; the rest of the workspace is written before it is read
  hipError_t e = launch_zero(L->SX(), (size_t)cfg->L * cfg->L * sizeof(double), S(stream));
  if (e == hipSuccess) e = launch_zero(L->ws + L->lay.zpad, 256, S(stream));
  if (e == hipSuccess) e = launch_zero(L->SG(), (size_t)cfg->L * cfg->L * sizeof(double), S(stream));
  if (e != hipSuccess) {
    (void)hipEventDestroy(L->done);
    (void)hipHostFree(L->hflags);
    delete L;
    return INSTANT_E_HIP;
  }
  *h = L;
  return INSTANT_OK;
}

INSTANT_API instant_status instant_destroy(instant_layer* h) {
  if (!h) return INSTANT_E_ARG;
  if (h->pending) (void)hipEventSynchronize(h->done);  // the device may still write hflags
  (void)hipEventDestroy(h->done);
  (void)hipHostFree(h->hflags);
  delete h;
  return INSTANT_OK;
}

INSTANT_API instant_status instant_calibrate(instant_layer* h, const void* x, const void* gy, int32_t B,
                                             int32_t finalize, void* stream) {
  if (!h) return INSTANT_E_ARG;
  if (B < 0 || B > h->cfg.B_max) return (B < 0) ? INSTANT_E_ARG : INSTANT_E_SHAPE;
  if ((x || gy) && B < 1) return INSTANT_E_ARG;
  if (!x && !gy && !finalize) return INSTANT_E_ARG;
  if (finalize != 0 && finalize != INSTANT_FINALIZE_SYNC && finalize != INSTANT_FINALIZE_ASYNC) return INSTANT_E_ARG;
  hipStream_t st = S(stream);
  if (finalize) {
    const int64_t nx = h->nx + (x ? B : 0), ng = h->ng + (gy ? B : 0);
    if (nx == 0 || ng == 0) return INSTANT_E_STATE;
  }
  if (x || gy) {
    const instant_status s = accumulate(h, x, gy, B, st);
    if (s != INSTANT_OK) return s;
    if (x) h->nx += B;
    if (gy) h->ng += B;
  }
  if (!finalize) return INSTANT_OK;

  apply_pending(h, true);  // the previous finalize's outcome decides which buffer is free
  const int t = (h->active == 0) ? 1 : 0;
  EigOut out;
  out.eps = h->cfg.eps;
  out.p = h->cfg.p;
  out.comp = h->cfg.comp;
  out.R_max = h->cfg.R_max;
  out.P32 = h->P32(t);
  out.Q32 = h->Q32(t);
  out.sigma_x = (float*)(h->ws + h->lay.sig_x);
  out.sigma_g = (float*)(h->ws + h->lay.sig_g);
  out.info_x = h->info_dev();
  out.info_g = h->info_dev() + INFO_WORDS;
  // Queued before the host reads the outcome, so the finalize costs one round trip: the
  // I/O copies of the new projections go to the inactive buffer t (harmless if the
  // finalize fails: t only becomes active on success). The statistics window is consumed
  // whatever the outcome: the next batch overwrites the sums.
  struct Tail {
    instant_layer* h;
    int t;
  } tail{h, t};
  out.ctx = &tail;
  out.before_readback = [](void* ctx, hipStream_t st) -> hipError_t {
    const Tail& tl = *(const Tail*)ctx;
    instant_layer* hh = tl.h;
    return launch_build_io(hh->bf16, hh->P32(tl.t), hh->Q32(tl.t), hh->info_dev() + 2,
                           hh->info_dev() + INFO_WORDS + 2, hh->cfg.L, hh->lay.ldL, hh->cfg.R_max, hh->PQ(tl.t),
                           hh->Qt(tl.t), LD_QT, st);
  };
  const int m = h->cfg.solver == INSTANT_SOLVER_SUBSPACE ? eig_subspace_width(h->cfg.L, h->cfg.R_max) : 0;
  const bool async = finalize == INSTANT_FINALIZE_ASYNC;
  hipError_t e = m > 0 ? run_eig_subspace(h->SX(), h->SG(), 1.0 / (double)h->nx, 1.0 / (double)h->ng, h->cfg.L, m,
                                          h->cfg.sub_iters, h->cfg.max_sweeps, h->warm, h->ws + h->lay.eig, out,
                                          h->hflags, st, !async)
                       : run_eig(h->SX(), h->SG(), 1.0 / (double)h->nx, 1.0 / (double)h->ng, h->cfg.L,
                                 h->cfg.max_sweeps, h->warm, h->ws + h->lay.eig, out, h->hflags, st, !async);
  if (e == hipSuccess && async) e = hipEventRecord(h->done, st);
  if (e != hipSuccess) {
    // a failed launch, or a bounded eigensolver wait that gave up: latched like any other
    // calibration failure, so instant_query reports it; the previous projections stay active
    h->warm = false;
    h->nx = h->ng = 0;
    h->last = INSTANT_E_HIP;
    h->info.status = INSTANT_E_HIP;
    return INSTANT_E_HIP;
  }
  h->pend_t = t;
  h->pend_m = m;
  h->pend_nx = h->nx;
  h->pend_ng = h->ng;
  h->nx = h->ng = 0;  // the window is consumed whatever the outcome
  if (async) {
    h->pending = true;
    return INSTANT_OK;
  }
  return settle(h);
}

INSTANT_API instant_status instant_compress_fwd(instant_layer* h, const void* x, int32_t B, void* xhat,
                                                void* stream) {
  if (!h || !x || !xhat || B < 1) return INSTANT_E_ARG;
  if (B > h->cfg.B_max) return INSTANT_E_SHAPE;
  // a finished asynchronous finalize takes effect here, at a forward (waited for only when
  // no projections are active yet), so a compress / backward pair uses one set
  apply_pending(h, h->active < 0);
  if (h->active < 0) return INSTANT_E_STATE;
  const int a = h->active;
  return hip_ok(launch_proj(h->bf16, h->PQ(a), h->lay.ldL, h->Rx, h->Rx, x, B, h->cfg.L, h->cfg.Cx, xhat, nullptr,
                            h->ws + h->lay.zpad, S(stream)));
}

namespace {

// Where one backward call keeps its intermediates: P g_y [B][Rx][Cy], Q g_y [B][Ry][Cy],
// g_hat_x [B][Ry][Cx] (I/O dtype) and the float32 K-slice partials of g_hat_x.
struct BwdScratch {
  void* Pgy;
  void* Qgy;
  void* gxh;
  float* gpart;
  size_t gpart_floats;
};

// The low-rank backward of one call (the launches of instant_backward).
instant_status run_backward(instant_layer* h, const void* xhat, const void* gy, const void* w, int B, void* gw,
                            void* gx, const BwdScratch& sc, hipStream_t st) {
  const int a = h->active;
  const int L = h->cfg.L, Cx = h->cfg.Cx, Cy = h->cfg.Cy, Rx = h->Rx, Ry = h->Ry;
  // [P; Q] gy_b from one pass over gy
  const void* zpad = h->ws + h->lay.zpad;
  hipError_t e = launch_proj(h->bf16, h->PQ(a), h->lay.ldL, Rx + Ry, Rx, gy, B, L, Cy, sc.Pgy, sc.Qgy, zpad, st);
  if (gx_fused_applies(h->bf16, B, Cx, Cy)) {
    // g_x_b = Q^T ((Q gy_b) w) with w resident in L2, and g_w, in one launch
    if (e == hipSuccess)
      e = launch_bwd_tail(h->bf16, sc.Qgy, w, h->Qt(a), LD_QT, B, Ry, L, Cy, Cx, gx, sc.Pgy, xhat, gw, B * Rx,
                          h->ncu, st);
  } else {
    // g_w = sum_b (P gy_b)^T x_hat_b: M = Cy, N = Cx, K = B * Rx (LDS-staged tiles or
    // register-blocked, whichever is faster for the shapes)
    if (e == hipSuccess)
      e = h->bf16 && gemm_tiled_applies(true, Cy, Cx, B * Rx)
              ? launch_gemm_tiled(true, sc.Pgy, Cy, xhat, Cx, gw, Cx, Cy, Cx, B * Rx, sc.gpart, sc.gpart_floats,
                                  zpad, st)
              : launch_gemm(h->bf16, true, sc.Pgy, Cy, 0, xhat, Cx, 0, gw, Cx, 0, 1, Cy, Cx, B * Rx, st);
    // g_hat_x = (Q gy) w: M = B * Ry, N = Cx, K = Cy; a w too large for L2 is read once over
    // K slices, whose float32 partials the expansion adds itself; otherwise LDS-staged tiles
    // or register-blocked as for g_w
    const int ws = h->bf16 ? gemm_ws_slices(true, false, B * Ry, Cx, Cy) : 0;
    if (ws && (size_t)ws * B * Ry * Cx <= sc.gpart_floats) {
      // g_x_b = Q^T g_hat_x_b with g_hat_x summed from its slices inside the expansion
      if (e == hipSuccess)
        e = launch_gemm_ws_parts(sc.Qgy, Cy, w, Cx, sc.gpart, sc.gpart_floats, B * Ry, Cx, Cy, zpad, st);
      if (e == hipSuccess) e = launch_expand_parts(h->Qt(a), LD_QT, sc.gpart, ws, B, Ry, L, Cx, gx, st);
      return hip_ok(e);
    }
    if (e == hipSuccess) {
      if (h->bf16 && !ws && gemm_tiled_applies(false, B * Ry, Cx, Cy))
        e = launch_gemm_tiled(false, sc.Qgy, Cy, w, Cx, sc.gxh, Cx, B * Ry, Cx, Cy, sc.gpart, sc.gpart_floats, zpad,
                              st);
      else
        e = launch_gemm(h->bf16, false, sc.Qgy, Cy, 0, w, Cx, 0, sc.gxh, Cx, 0, 1, B * Ry, Cx, Cy, st, sc.gpart,
                        sc.gpart_floats, zpad);
    }
    // g_x_b = Q^T g_hat_x_b
    if (e == hipSuccess) e = launch_expand(h->bf16, h->Qt(a), LD_QT, sc.gxh, B, Ry, L, Cx, gx, st);
  }
  return hip_ok(e);
}

}  // namespace

INSTANT_API instant_status instant_backward(instant_layer* h, const void* xhat, const void* gy, const void* w,
                                            int32_t B, void* gw, void* gx, void* stream) {
  if (!h || !xhat || !gy || !w || !gw || !gx || B < 1) return INSTANT_E_ARG;
  if (B > h->cfg.B_max) return INSTANT_E_SHAPE;
  if (h->active < 0) return INSTANT_E_STATE;
  const BwdScratch sc{h->ws + h->lay.Pgy, h->ws + h->lay.Qgy, h->ws + h->lay.gxh, (float*)(h->ws + h->lay.gpart),
                      h->lay.gpart_floats};
  return run_backward(h, xhat, gy, w, B, gw, gx, sc, S(stream));
}

INSTANT_API instant_status instant_backward_static(instant_layer* h, const void* xhat, const void* gy,
                                                   const void* w, int32_t B, void* gw, void* gx, void* stream) {
  if (!h || !xhat || !gy || !w || !gw || !gx || B < 1) return INSTANT_E_ARG;
  if (B > h->cfg.B_max) return INSTANT_E_SHAPE;
  if (h->active < 0) return INSTANT_E_STATE;
  if (!h->scratch) return INSTANT_E_HIP;  // the device address of the scratch could not be looked up
  const size_t esz = h->bf16 ? 2 : 4;
  const size_t Cx = h->cfg.Cx, Cy = h->cfg.Cy, Rx = h->Rx, Ry = h->Ry;
  // the same intermediates instant_backward keeps in the workspace, packed for this call
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  const size_t o_pgy = take((size_t)B * Rx * Cy * esz);
  const size_t o_qgy = take((size_t)B * Ry * Cy * esz);
  const size_t o_gxh = take((size_t)B * Ry * Cx * esz);
  size_t part_floats = 0;
  if (!gx_fused_applies(h->bf16, B, (int)Cx, (int)Cy)) {
    const int ws = gemm_ws_slices(h->bf16, false, B * (int)Ry, (int)Cx, (int)Cy);
    part_floats = (size_t)ws * B * Ry * Cx;
    if (h->bf16) {
      if (gemm_tiled_applies(true, (int)Cy, (int)Cx, B * (int)Rx))
        part_floats = std::max(part_floats, gemm_tiled_part_floats((int)Cy, (int)Cx, B * (int)Rx));
      if (!ws && gemm_tiled_applies(false, B * (int)Ry, (int)Cx, (int)Cy))
        part_floats = std::max(part_floats, gemm_tiled_part_floats(B * (int)Ry, (int)Cx, (int)Cy));
    }
  }
  const size_t o_part = take(part_floats * sizeof(float));
  if (off > STATIC_SCRATCH_BYTES) return INSTANT_E_SHAPE;
  char* base = (char*)h->scratch;
  const BwdScratch sc{base + o_pgy, base + o_qgy, base + o_gxh, (float*)(base + o_part), part_floats};
  return run_backward(h, xhat, gy, w, B, gw, gx, sc, S(stream));
}

INSTANT_API instant_status instant_query(instant_layer* h, instant_info* out) {
  if (!h || !out) return INSTANT_E_ARG;
  apply_pending(h, true);
  *out = h->info;
  return h->last;
}

INSTANT_API instant_status instant_set_projections(instant_layer* h, const float* P, int32_t Rx, const float* Q,
                                                   int32_t Ry, void* stream) {
  if (!h || !P || !Q) return INSTANT_E_ARG;
  if (Rx < 1 || Ry < 1 || Rx > h->cfg.R_max || Ry > h->cfg.R_max) return INSTANT_E_SHAPE;
  apply_pending(h, true);
  hipStream_t st = S(stream);
  const int t = (h->active == 0) ? 1 : 0;
  const size_t L = h->cfg.L;
  hipError_t e = hipMemcpyAsync(h->P32(t), P, (size_t)Rx * L * sizeof(float), hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(h->Q32(t), Q, (size_t)Ry * L * sizeof(float), hipMemcpyDeviceToDevice, st);
  const int r[2] = {Rx, Ry};
  if (e == hipSuccess) e = launch_fill_i32(h->rank_dev(), r, 2, st);
  if (e == hipSuccess)
    e = launch_build_io(h->bf16, h->P32(t), h->Q32(t), h->rank_dev(), h->rank_dev() + 1, h->cfg.L, h->lay.ldL,
                        h->cfg.R_max, h->PQ(t), h->Qt(t), LD_QT, st);
  if (e != hipSuccess) return INSTANT_E_HIP;
  h->active = t;
  h->Rx = Rx;
  h->Ry = Ry;
  h->info.Rx = Rx;
  h->info.Ry = Ry;
  h->info.generation += 1;
  return INSTANT_OK;
}

INSTANT_API instant_status instant_get_projections(instant_layer* h, float* P, float* Q, float* sigma_x,
                                                   float* sigma_g, void* stream) {
  if (!h) return INSTANT_E_ARG;
  apply_pending(h, true);
  if ((P || Q) && h->active < 0) return INSTANT_E_STATE;
  hipStream_t st = S(stream);
  const size_t L = h->cfg.L;
  hipError_t e = hipSuccess;
  if (P) e = hipMemcpyAsync(P, h->P32(h->active), (size_t)h->Rx * L * sizeof(float), hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && Q)
    e = hipMemcpyAsync(Q, h->Q32(h->active), (size_t)h->Ry * L * sizeof(float), hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && sigma_x)
    e = hipMemcpyAsync(sigma_x, h->ws + h->lay.sig_x, L * sizeof(float), hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && sigma_g)
    e = hipMemcpyAsync(sigma_g, h->ws + h->lay.sig_g, L * sizeof(float), hipMemcpyDeviceToDevice, st);
  return hip_ok(e);
}

INSTANT_API instant_status instant_get_statistics(instant_layer* h, double* C_X, double* C_G, void* stream) {
  if (!h) return INSTANT_E_ARG;
  if ((C_X && h->nx == 0) || (C_G && h->ng == 0)) return INSTANT_E_STATE;
  hipError_t e = hipSuccess;
  if (C_X) e = launch_stat_mean(h->SX(), 1.0 / (double)h->nx, h->cfg.L, C_X, S(stream));
  if (e == hipSuccess && C_G) e = launch_stat_mean(h->SG(), 1.0 / (double)h->ng, h->cfg.L, C_G, S(stream));
  return hip_ok(e);
}

INSTANT_API const char* instant_status_str(instant_status s) {
  switch (s) {
    case INSTANT_OK: return "INSTANT_OK";
    case INSTANT_E_ARG: return "INSTANT_E_ARG";
    case INSTANT_E_SHAPE: return "INSTANT_E_SHAPE";
    case INSTANT_E_STATE: return "INSTANT_E_STATE";
    case INSTANT_E_RANK: return "INSTANT_E_RANK";
    case INSTANT_E_ENERGY: return "INSTANT_E_ENERGY";
    case INSTANT_E_NONFINITE: return "INSTANT_E_NONFINITE";
    case INSTANT_E_NOCONV: return "INSTANT_E_NOCONV";
    case INSTANT_E_HIP: return "INSTANT_E_HIP";
  }
  return "INSTANT_E_UNKNOWN";
}
