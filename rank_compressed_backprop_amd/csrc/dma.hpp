// Global-to-LDS streaming helpers shared by the ring-buffered kernels (gfx950, wave64): a
// wave's 16-byte-per-lane DMA into LDS, a fence-free workgroup barrier and waits on the
// wave's outstanding vector-memory loads.
#pragma once

#include <hip/hip_runtime.h>

namespace instant {

// 16 bytes per lane from src straight into LDS at lds_wave + 16 * lane (lds_wave uniform
// across the wave; the hardware takes it from M0). Written as inline assembly on purpose: the
// compiler, seeing the intrinsic form write LDS, puts a wait for every outstanding vector
// load in front of each later LDS read (it cannot tell ring slots apart), which empties the
// ring at every stage. Here the kernels' own waits (wait_oldest_stage) order the stages. The
// instruction has no register result; the nop is the wait state a write of M0 needs before
// a DMA reads it.
__device__ inline void lds_dma16(const void* src, void* lds_wave) {
  const unsigned lds = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds_wave;
  __asm__ volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

// Workgroup barrier without a memory fence (waits are explicit around it).
__device__ inline void bare_barrier() {
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Wait until at most N vector-memory loads of this wave are outstanding, and for all of its
// LDS reads: the next barrier may hand their buffer to a refill.
template <int N>
__device__ inline void wait_vmcnt() {
  __asm__ volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}

// Wait for the oldest stage when `younger` (0..Y) later stages of LDPS loads each may stay
// in flight (the count has to be an immediate).
template <int LDPS, int Y>
__device__ inline void wait_oldest_stage(int younger) {
  if constexpr (Y == 0) {
    wait_vmcnt<0>();
  } else {
    if (younger >= Y) wait_vmcnt<Y * LDPS>();
    else wait_oldest_stage<LDPS, Y - 1>(younger);
  }
}

}  // namespace instant
