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

// LDS bytes a copied tile occupies: whole KiB chunks (the lanes of a partial
// last chunk land in the rounding).
__host__ __device__ constexpr int dma_lds_bytes(int bytes) { return (bytes + 1023) / 1024 * 1024; }

// The chunk that copy instruction k of wavefront w moves (a wavefront with
// fewer chunks repeats the tile's last one), and, for lane `lane`, the byte
// offset it reads within the tile (clamped to the tile's last 16 bytes) and
// the byte offset it writes within the LDS buffer.
__host__ __device__ constexpr int dma_chunk(int bytes, int W, int w, int k) {
  return w + W * k < (bytes + 1023) / 1024 ? w + W * k : (bytes + 1023) / 1024 - 1;
}
__host__ __device__ constexpr uint32_t dma_src_off(int bytes, int ch, int lane) {
  return (uint32_t)ch * 1024u + (uint32_t)lane * 16u < (uint32_t)bytes ? (uint32_t)ch * 1024u + (uint32_t)lane * 16u
                                                                        : (uint32_t)(bytes - 16);
}
__host__ __device__ constexpr uint32_t dma_dst_off(int ch, int lane) { return (uint32_t)ch * 1024u + (uint32_t)lane * 16u; }

// A 64-bit address from its two 32-bit halves.  Both halves must be unsigned:
// readfirstlane returns int, and an int low word with bit 31 set would be
// sign-extended by the join and fill the high word with ones.
__host__ __device__ constexpr uint64_t join_addr(uint32_t hi, uint32_t lo) { return ((uint64_t)hi << 32) | (uint64_t)lo; }

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
  const uint32_t lbase = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(s);
  // the tile address is uniform; make that explicit for the SGPR operand
  const uint64_t ga = (uint64_t)(uintptr_t)g;
  const uint32_t glo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ga);
  const uint32_t ghi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(ga >> 32));
  g = (const char*)(uintptr_t)join_addr(ghi, glo);
  if constexpr (BYTES % 1024 == 0) {
    // whole chunks: no lane is clamped, so one lane offset (16 l) serves
    // every chunk and the chunk offset goes into the scalar address
    const uint32_t voff = dma_src_off(BYTES, 0, lane);
#pragma unroll
    for (int k = 0; k < dma_per_wave<BYTES, W>(); ++k) {
      const int ch = dma_chunk(BYTES, W, w, k);
      const char* gc = g + (size_t)dma_dst_off(ch, 0);
      const uint32_t m0 = lbase + dma_dst_off(ch, 0);
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gc), "s"(m0)
                   : "memory", "m0");
    }
  } else {
#pragma unroll
    for (int k = 0; k < dma_per_wave<BYTES, W>(); ++k) {
      const int ch = dma_chunk(BYTES, W, w, k);
      const uint32_t voff = dma_src_off(BYTES, ch, lane);
      // the instruction writes lane l's 16 bytes to M0 + 16 l, i.e. at
      // dma_dst_off(ch, l) within the buffer
      const uint32_t m0 = lbase + dma_dst_off(ch, 0);
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(g), "s"(m0)
                   : "memory", "m0");
    }
  }
}

// Copy a tile made of four parts, each a whole number of KiB and each from a
// source of its own, into one LDS buffer (the parts back to back in order):
// chunk c of the C = (B0 + B1 + B2 + B3) / 1024 chunks goes to s + 1024 c.
// Wavefront w moves chunks w, w + W, ... (every wavefront issues
// dma_per_wave<1024 C, W> instructions, repeating the last chunk where it has
// fewer), lane l bytes 16 l .. 16 l + 15 of each.  Which part a chunk comes
// from is decided on scalar registers (uniform per wavefront).
__host__ __device__ constexpr int dma_part_of_chunk(int c, int C0, int C1, int C2) {
  return c < C0 ? 0 : (c < C0 + C1 ? 1 : (c < C0 + C1 + C2 ? 2 : 3));
}
template <int B0, int B1, int B2, int B3, int W>
__device__ __forceinline__ void dma_parts(const char* g0, const char* g1, const char* g2, const char* g3,
                                          const char* s, int w, int lane) {
  static_assert(B0 % 1024 == 0 && B1 % 1024 == 0 && B2 % 1024 == 0 && B3 % 1024 == 0, "parts of whole KiB");
  constexpr int C0 = B0 / 1024, C1 = B1 / 1024, C2 = B2 / 1024, C3 = B3 / 1024;
  constexpr int C = C0 + C1 + C2 + C3;
  __builtin_assume(w >= 0 && w < W);
  const uint32_t lbase = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(s);
  auto uni = [](const char* g) {
    const uint64_t ga = (uint64_t)(uintptr_t)g;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ga);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(ga >> 32));
    return (const char*)(uintptr_t)join_addr(hi, lo);
  };
  g0 = uni(g0); g1 = uni(g1); g2 = uni(g2); g3 = uni(g3);
  const uint32_t voff = (uint32_t)lane * 16u;
#pragma unroll
  for (int k = 0; k < dma_per_wave<C * 1024, W>(); ++k) {
    const int c = w + W * k < C ? w + W * k : C - 1;
    const char* gc;
    if (c < C0) gc = g0 + (size_t)c * 1024;
    else if (c < C0 + C1) gc = g1 + (size_t)(c - C0) * 1024;
    else if (c < C0 + C1 + C2) gc = g2 + (size_t)(c - C0 - C1) * 1024;
    else gc = g3 + (size_t)(c - C0 - C1 - C2) * 1024;
    const uint32_t m0 = lbase + (uint32_t)c * 1024u;
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gc), "s"(m0)
                 : "memory", "m0");
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace fipa
