// Direct global -> LDS copies (global_load_lds_dwordx4) issued from inline
// assembly, and the explicit vmcnt waits that go with them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fipa {

// Number of direct-to-LDS copy instructions each of the W wavefronts issues
// for a tile of BYTES bytes (1 KiB per instruction).
template <int BYTES, int W>
constexpr int dma_per_wave() { return ((BYTES + 1023) / 1024 + W - 1) / W; }

// Copy a tile (BYTES, a multiple of 16) global -> LDS with
// global_load_lds_dwordx4: lane l of a wavefront moves bytes 16l .. 16l+15 of
// one KiB chunk to M0 + 16l.  Every wavefront issues the same number of
// instructions (dma_per_wave) so that the vmcnt waits below are
// compile-time constants; a wavefront with fewer chunks repeats its last one
// (same bytes to the same place).  The copies are issued from inline
// assembly: the compiler does not track them, and the kernel waits for them
// explicitly (vmcnt) before the barrier that precedes the LDS reads.
template <int BYTES, int W>
__device__ __forceinline__ void dma_tile(const char* g, const char* s, int w, int lane) {
  constexpr int nch = (BYTES + 1023) / 1024;
  const uint32_t lbase = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(s);
  // the tile address is uniform; make that explicit for the SGPR operand
  // (readfirstlane returns int: each half goes through uint32_t so that the
  // low word is zero-extended, not sign-extended, when the halves are joined)
  const uint64_t ga = (uint64_t)(uintptr_t)g;
  const uint32_t glo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ga);
  const uint32_t ghi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(ga >> 32));
  g = (const char*)(uintptr_t)(((uint64_t)ghi << 32) | (uint64_t)glo);
#pragma unroll
  for (int k = 0; k < dma_per_wave<BYTES, W>(); ++k) {
    int ch = w + W * k;
    ch = ch < nch ? ch : nch - 1;
    const uint32_t off = (uint32_t)ch * 1024u + (uint32_t)lane * 16u;
    const uint32_t voff = off < (uint32_t)BYTES ? off : (uint32_t)(BYTES - 16);
    const uint32_t m0 = lbase + (uint32_t)ch * 1024u;
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(g), "s"(m0)
                 : "memory", "m0");
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace fipa
