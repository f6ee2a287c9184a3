// Device-side building blocks shared by the INSTANT kernels (gfx950, wave64).
//
// Matrix-core convention. Every contraction is issued as 16x16 output tiles of
// v_mfma_f32_16x16x32_bf16 (bf16 operands) or four v_mfma_f32_16x16x4_f32 (fp32
// operands). In one k-step of KSTEP = 4*G values, lane i supplies for its operand
// row or column (i % 16) the G consecutive k values k0 + G*(i/16) .. +G-1, and
// receives output rows 4*(i/16) .. +3 of column (i % 16).
//
// Operands stored with k contiguous ("direct") are read with one 16-byte load per
// lane. Operands stored with the output index contiguous ([K][N] row-major, as x,
// gy, w and every intermediate are) are read as G rows x 8 columns per lane and
// transposed in registers: column j of that 8-wide strip becomes "virtual tile" j,
// whose tile column (i % 16) is the actual column n0 + 8*(i % 16) + j. The same
// lane then owns 8 contiguous output columns, so results leave as 16-byte stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace instant {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int WAVE = 64;
// accelerator dies (XCDs) of the chip, each with its own L2; a launch's workgroups are dealt
// to them in turn by workgroup id
constexpr int XCDS = 8;

// The work unit of workgroup `id` out of `n` such that each XCD takes a contiguous run of units
// (ids past the last full round of XCDS workgroups keep their own number).
__device__ inline int xcd_unit(int id, int n) {
  const int per = n / XCDS;
  return id < per * XCDS ? (id % XCDS) * per + id / XCDS : id;
}

template <class T> struct MM;

template <> struct MM<bf16> {
  static constexpr int G = 8;          // k values per lane per step
  static constexpr int KSTEP = 32;     // k values per wave per step
  typedef bf16x8 frag;
  typedef bf16x8 vec8;                 // 8 consecutive elements (16 bytes)
  __device__ static inline f32x4 mma(const frag& a, const frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct MM<float> {
  static constexpr int G = 4;
  static constexpr int KSTEP = 16;
  typedef f32x4 frag;
  typedef f32x8 vec8;                  // 8 consecutive elements (32 bytes)
  __device__ static inline f32x4 mma(const frag& a, const frag& b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
  }
};

template <class T> __device__ inline T from_f32(float v);
template <> __device__ inline float from_f32<float>(float v) { return v; }
template <> __device__ inline bf16 from_f32<bf16>(float v) { return (bf16)v; }  // round to nearest even

template <class T> __device__ inline float to_f32(T v) { return (float)v; }

template <class T> __device__ inline typename MM<T>::frag zero_frag() {
  typename MM<T>::frag f;
#pragma unroll
  for (int g = 0; g < MM<T>::G; ++g) f[g] = (T)0.0f;
  return f;
}

template <class T> __device__ inline typename MM<T>::vec8 zero_vec8() {
  typename MM<T>::vec8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (T)0.0f;
  return v;
}

// 16-byte load of G consecutive k values (direct operand). `ok` false gives zeros.
template <class T>
__device__ inline typename MM<T>::frag load_frag(const T* __restrict__ p, bool ok) {
  if (ok) return *reinterpret_cast<const typename MM<T>::frag*>(p);
  return zero_frag<T>();
}

// Load G rows (row0 + g, g < G; rows >= nrows read as zero) x W columns starting at
// `col` from a [rows][ld] matrix and transpose: f[j][g] = M[row0 + g][col + j], j < W.
// W is 8 (16-byte bf16 rows, 32-byte fp32 rows) or 4.
template <class T, int W> struct VecW;
template <class T> struct VecW<T, 8> { typedef typename MM<T>::vec8 type; };
template <> struct VecW<bf16, 4> { typedef bf16x4 type; };
template <> struct VecW<float, 4> { typedef f32x4 type; };

template <class T, int W>
__device__ inline void load_strip_T(const T* __restrict__ base, int ld, int row0, int nrows, int col,
                                    bool col_ok, typename MM<T>::frag f[W]) {
  typedef typename VecW<T, W>::type vec;
  vec r[MM<T>::G];
#pragma unroll
  for (int g = 0; g < MM<T>::G; ++g) {
    const int row = row0 + g;
    if (col_ok && row < nrows) {
      r[g] = *reinterpret_cast<const vec*>(base + (size_t)row * ld + col);
    } else {
#pragma unroll
      for (int j = 0; j < W; ++j) r[g][j] = (T)0.0f;
    }
  }
#pragma unroll
  for (int j = 0; j < W; ++j)
#pragma unroll
    for (int g = 0; g < MM<T>::G; ++g) f[j][g] = r[g][j];
}

// Store W consecutive output columns of one row.
template <class T, int W>
__device__ inline void store_row(T* __restrict__ p, const float v[W]) {
  typename VecW<T, W>::type o;
#pragma unroll
  for (int j = 0; j < W; ++j) o[j] = from_f32<T>(v[j]);
  *reinterpret_cast<typename VecW<T, W>::type*>(p) = o;
}

// The same with the non-temporal hint, for a large output that neither this launch nor the
// next one reads: its lines then go on to memory while the launch runs instead of staying
// dirty in L2 until the write-back at the launch's end (1.5 us of an 11 us launch that
// writes 25 MB, measured on gfx950).
template <class T, int W>
__device__ inline void store_row_nt(T* __restrict__ p, const float v[W]) {
  typedef typename VecW<T, W>::type vec;
  vec o;
#pragma unroll
  for (int j = 0; j < W; ++j) o[j] = from_f32<T>(v[j]);
  __builtin_nontemporal_store(o, reinterpret_cast<vec*>(p));
}

__device__ inline f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace instant
