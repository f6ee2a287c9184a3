// LDS tile layouts shared by the ring kernels that feed the matrix cores from LDS (gfx950,
// wave64, bf16): the XOR swizzles of k-major and m-major stage tiles and the transpose read
// that turns a k-major tile into MFMA operands.
//
// A k-major tile (64 k rows x 128 columns, 256 bytes a row) feeds the matrix cores through the
// gfx950 transpose read ds_read_b64_tr_b16: within each group of 16 lanes, destination lane i,
// element j receives element i % 4 of the 8 bytes that source lane i / 4 + 4 j addressed (lane
// layout measured on gfx950). Lane s of a group addresses row k0 + s / 4 (+ 4 for the second
// read) at columns cb(s % 4) .. cb(s % 4) + 3, so lane i ends with the 8 consecutive k of
// column cb(i / 4) + i % 4: an MFMA operand without register shuffles. An m-major tile (rows x
// 64 k, 128 bytes a row) is read with one 16-byte read per lane. 16-byte chunks are
// XOR-swizzled by row so that the reads avoid bank conflicts.
#pragma once

#include "common.hpp"

namespace instant {
namespace {

// k-major tiles: 16-byte chunk c of row r lives at chunk c ^ swz(r). The LDS serves a
// transpose read 16 lanes at a time from a 128-byte bank window (measured on gfx950: a
// swizzle built for 256-byte windows left half the LDS cycles in bank conflicts). The 16
// lanes read 4 consecutive rows (r % 4), each at 4 places:
//   B tiles (pairs of 32 columns, AS = 8): 8 bytes in each of 4 consecutive chunks,
//     alternating halves (see kmajor_frag); XOR with 0, 1, 4, 5 for r % 4 = 0..3 gives the
//     rows disjoint (chunk mod 8, half) slots;
//   A tiles (16 consecutive columns, AS = 4): both halves of 2 consecutive chunks; XOR with
//     0, 2, 4, 6 gives the rows disjoint chunk pairs mod 8.
// Both also flip chunk bit 3 for rows 8-15 of each 16, in case two groups share a window.
__device__ __forceinline__ int kswz_b(int r) { return ((r & 1) | ((r & 2) << 1)) ^ (((r >> 3) & 1) << 3); }
__device__ __forceinline__ int kswz_a(int r) { return (2 * (r & 3)) ^ (((r >> 3) & 1) << 3); }
// m-major tile: chunk c of row r at c ^ (r & 7) (8 chunks a row, one 16-byte read per lane).
__device__ __forceinline__ int mswz(int r) { return r & 7; }

// 4 bf16 of a transpose read (kept whole: the operand is assembled by vector shuffles)
__device__ __forceinline__ bf16x4 tr_read(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)p);
}

// One MFMA operand from a k-major tile: lane (q = lane / 16, i = lane % 16) receives the 8 k
// values 32 h + 8 q .. + 7 of column cb(i / 4) + i % 4. As a source, lane s addresses row
// 32 h + 8 q + s / 4 (+ 4 for the second half) at columns cb(s % 4) .. + 3, where
//   PAIR = false: cb(a) = col0 + 4 a, the 16 consecutive columns col0 .. col0 + 15;
//   PAIR = true : cb(a) = col0 + 8 a + 4 (hh ^ (a % 2)), half hh of the 32-column pair at col0:
//                 quad a of the two halves together covers columns col0 + 8 a .. + 7.
template <bool PAIR>
__device__ __forceinline__ MM<bf16>::frag kmajor_frag(const unsigned char* tile, int h, int lane, int col0, int hh) {
  const int q = lane >> 4, s = lane & 15, a = s & 3;
  const int col = PAIR ? col0 + 8 * a + 4 * (hh ^ (a & 1)) : col0 + 4 * a;
  const int chunk = col >> 3, within = (col & 7) * 2;
  const int r0 = 32 * h + 8 * q + (s >> 2), r1 = r0 + 4;
  const int w0 = PAIR ? kswz_b(r0) : kswz_a(r0), w1 = PAIR ? kswz_b(r1) : kswz_a(r1);
  const bf16x4 lo = tr_read(tile + r0 * 256 + 16 * (chunk ^ w0) + within);
  const bf16x4 hi = tr_read(tile + r1 * 256 + 16 * (chunk ^ w1) + within);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace
}  // namespace instant
