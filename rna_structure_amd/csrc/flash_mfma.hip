// Kernel 2, matrix-core path: fused masked online-softmax attention over the
// lifted IPA rows on gfx950 MFMA.  No [N,N] tensor is written anywhere.
//
// Per (batch b, head h, query tile): W wavefronts (4 or 8), each owning 32
// queries.  Per 64-key tile staged in LDS by the whole workgroup:
//   S^T (keys x queries) = K~ Q~^T        v_mfma_f32_32x32x16_bf16 over the
//                                         scalar + pair columns,
//                                         v_mfma_f32_32x32x16_f16 over the
//                                         centred point columns (fp16 hi/lo
//                                         split: 3 products per coordinate,
//                                         plus the tile offset, the row term
//                                         minus the running maximum and the
//                                         key mask, see common.h), so S is
//                                         the complete logit times log2 e
//                                         relative to the running maximum
//   masked online softmax in fp32 with exp2, a running maximum that is only
//   raised when it grows by more than 8 (probabilities stay below 2^8) and
//   an fp32 row sum for the log-sum-exp
//   O^T += V~^T P^T                       fp16 probabilities against the fp16
//                                         value tile: values (times 2^-8), the
//                                         centred value points, the centroid
//                                         and ones rows (per head), and the
//                                         pair factors (times 2^-8, shared by
//                                         the heads)
// The accumulator layout of S^T gives every lane one query and 16 keys, so
// the probabilities feed the value product from registers; the value tile is
// stored transposed with its keys permuted to match (lift kernel).
// Normalisation uses the ones rows, i.e. the sums of the rounded
// probabilities actually multiplied into O, so the weights applied to the
// values sum to one to fp32 rounding and the centroid cancels exactly.
// Key and value tiles are copied global -> LDS with direct-to-LDS loads.  A
// tile has four parts (common.h): the head's key rows and value rows, and the
// pair-factor key and value rows that the H heads of a batch element share.
// Two schemes (NBUF): with two buffers the copies of the next tile run
// during the whole of the current tile and one barrier per tile separates
// the two (8 wavefronts, one workgroup per CU: long key ranges); with one
// buffer the copies of a tile go out when every wavefront is done with the
// previous one, and the latency is hidden by a second workgroup on the CU
// (4 wavefronts, two workgroups per CU: short key ranges, where the
// per-workgroup prologue and output also overlap with the other
// workgroup's tiles).  (Refilling the key and value parts of the one buffer
// in turn, so that copies overlap the products, measured no faster.)
#include "lds_copy.h"
#include "mfma_tile.h"

namespace fipa {

struct FlashMfmaArgs {
  Layout L;
  const char* ws;
  float* o;
  float* lse;
  int qtiles;
  int nwg;
  int ks;  // key ranges per query tile (partial results when > 1)
};

template <typename V>
__device__ __forceinline__ float pick16(const V& acc, int r) {
  float v = 0.f;
#pragma unroll
  for (int x = 0; x < 16; ++x) v = (x == r) ? acc[x] : v;
  return v;
}

// Uniform read-only data (per-tile centroids, key-mask words, point
// weights) is read through the constant address space so that it goes
// through scalar loads and never adds to the vector-memory counter that the
// tile copies below are synchronised with.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return *(const __attribute__((address_space(4))) T*)(uintptr_t)join_addr(hi, lo);
}
__device__ __forceinline__ float4 ld_uniform4(const float4* p) {
  const float* f = reinterpret_cast<const float*>(p);
  return make_float4(ld_uniform(f), ld_uniform(f + 1), ld_uniform(f + 2), ld_uniform(f + 3));
}

// First key tile after t with at least one valid key (NT if none); kmb
// points at the key-mask words of the batch element.
__device__ __forceinline__ int next_valid_tile(const uint32_t* kmb, int t, int NT) {
  for (++t; t < NT; ++t)
    if ((ld_uniform(kmb + 2 * t) | ld_uniform(kmb + 2 * t + 1)) != 0u) break;
  return __builtin_amdgcn_readfirstlane(t);
}

// Byte sizes of the four parts of a key/value tile (common.h) and of one LDS
// tile buffer, which holds them back to back in this order.
template <int NQS, int NVB, int GS>
struct TileDims {
  static constexpr int KH = 64 * (16 + 16 * GS + kRowPad) * 2;    // head key rows
  static constexpr int KZ = 64 * (16 * (NQS - 1) + kRowPad) * 2;  // pair-factor key rows
  static constexpr int VH = 64 * kVCols * 2;                      // head value rows (blocks 0, 1)
  static constexpr int VZ = (32 * (NVB - 1) * kVCols * 2 + 1023) / 1024 * 1024;  // pair-factor value rows
  static constexpr int TB = KH + KZ + VH + VZ;
};

// Global addresses of key/value tile 0 of one (batch, head): the head's own
// parts and the shared pair-factor parts.
struct TileSrc {
  const char *kh, *kz, *vh, *vz;
};

// Key and value tile t into LDS buffer buf.
template <int NQS, int NVB, int GS, int W>
__device__ __forceinline__ void copy_kv_tile(const TileSrc& src, char* skv, int t, int buf, int w, int lane) {
  using T = TileDims<NQS, NVB, GS>;
  dma_parts<T::KH, T::KZ, T::VH, T::VZ, W>(src.kh + (size_t)t * T::KH, src.kz + (size_t)t * T::KZ,
                                           src.vh + (size_t)t * T::VH, src.vz + (size_t)t * T::VZ,
                                           skv + buf * T::TB, w, lane);
}

// Second half of the online softmax: p = 2^s (s already relative to the
// running maximum), its fp32 row sum (returned) and the fp16 operand ph of
// the value product.
__device__ __forceinline__ float exp_tile(float* s, f16x8_t* ph) {
  float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int x = 0; x < 32; ++x) {
    s[x] = __builtin_amdgcn_exp2f(s[x]);
    ps[x & 3] += s[x];
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) ph[ks][e] = (_Float16)s[(ks >> 1) * 16 + (ks & 1) * 8 + e];
  return (ps[0] + ps[1]) + (ps[2] + ps[3]);
}

// O^T += V~^T P^T over one 64-key value tile in LDS: 4 K-steps x (NVB + 1)
// value blocks, consecutive MFMAs on different blocks (independent), value
// fragments fetched DEPTH MFMAs ahead of their use so that the LDS latency
// hides behind the preceding MFMAs.  pv_tile_ops emits the reads and MFMAs,
// pv_tile_sched their order (with up to VPER vector-ALU instructions of other
// work after each MFMA).
template <int NVB, int DEPTH>
__device__ __forceinline__ void pv_tile_ops(const char* vrow, const f16x8_t* pc, f32x16_t* oacc) {
  constexpr int NB = NVB + 1;
  constexpr int NS = 4 * NB;
  auto off = [](int st) { return (size_t)((st % NB) * 32 * kVCols) * 2 + (st / NB) * 32; };
  uint4 f[DEPTH];
#pragma unroll
  for (int st = 0; st < DEPTH; ++st) f[st] = *reinterpret_cast<const uint4*>(vrow + off(st));
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const uint4 c = f[st % DEPTH];
    if (st + DEPTH < NS) f[st % DEPTH] = *reinterpret_cast<const uint4*>(vrow + off(st + DEPTH));
    oacc[st % NB] =
        __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, c), pc[st / NB], oacc[st % NB], 0, 0, 0);
  }
}

template <int NS, int DEPTH, int VPER>
__device__ __forceinline__ void pv_tile_sched() {
  __builtin_amdgcn_sched_group_barrier(0x100, DEPTH, 0);
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (st + DEPTH < NS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (VPER > 0) __builtin_amdgcn_sched_group_barrier(0x002, VPER, 0);
  }
}

template <int NVB>
__device__ __forceinline__ void pv_tile(const char* vrow, const f16x8_t* pc, f32x16_t* oacc) {
  pv_tile_ops<NVB, 4>(vrow, pc, oacc);
  pv_tile_sched<4 * (NVB + 1), 4, 0>();
}

// Second half of the online softmax and the value product of one tile in
// one block of instructions: p = 2^s for the first 32-key block (registers
// 0..15 of s) before a scheduling barrier, then the exponentials, row sum
// and fp16 conversion of the second block placed between the 2 (NVB + 1)
// value MFMAs of K-steps 0 and 1 (which need only the first block), then
// the MFMAs of K-steps 2 and 3.  Returns the fp32 row sum.
template <int NVB>
__device__ __forceinline__ float exp_pv_interleaved(const char* vrow, float* s, f16x8_t* ph, f32x16_t* oacc) {
  constexpr int NB = NVB + 1;
  float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    s[x] = __builtin_amdgcn_exp2f(s[x]);
    ps[x & 3] += s[x];
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) ph[ks][e] = (_Float16)s[ks * 8 + e];
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
  // the second block's softmax (independent of K-steps 0 and 1), then the
  // value product; the scheduling groups below interleave the two
#pragma unroll
  for (int x = 16; x < 32; ++x) {
    s[x] = __builtin_amdgcn_exp2f(s[x]);
    ps[x & 3] += s[x];
  }
#pragma unroll
  for (int ks = 2; ks < 4; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) ph[ks][e] = (_Float16)s[16 + (ks - 2) * 8 + e];
  pv_tile_ops<NVB, 4>(vrow, ph, oacc);
  // order: the first DEPTH fragment reads, then per MFMA of K-steps 0 and 1
  // its read DEPTH ahead and two or three vector instructions of the second
  // block's softmax, then the remaining MFMAs with their reads
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int st = 0; st < 4 * NB; ++st) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (st + 4 < 4 * NB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (st < 2 * NB) __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
  }
  __builtin_amdgcn_s_setprio(0);
  return (ps[0] + ps[1]) + (ps[2] + ps[3]);
}

// First half of the online softmax of one tile for the 32 queries of a
// wavefront.  S arrives relative to the running maximum m of each query (m
// rides in the row term of the last geometric K-step); keys that are masked
// out arrive as -16 x 65504 (key-mask column) or are set to -inf here
// (pair-mask bits).  m starts at the maximum of the first tile that holds a
// permitted key of the row: without a pair mask every tile the loop visits
// holds a valid key, which every valid query may attend to; with one, the
// row's permitted keys are exactly its finite entries.  After that m is
// raised only when a row maximum exceeds it by more than 8 (log2 units), so
// the probabilities stay below 2^8 and rescaling is rare.  Leaves s relative
// to the new m and returns the factor by which O and l are to be scaled.
template <bool PM>
__device__ __forceinline__ float softmax_max(const f32x16_t* sacc, uint32_t mw, float& m, bool& init, float* s) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb * 16 + r] = sacc[kb][r];
  if constexpr (PM) {
    if (!__all(mw == 0xFFFFFFFFu)) {
#pragma unroll
      for (int x = 0; x < 32; ++x) s[x] = ((mw >> x) & 1u) ? s[x] : -INFINITY;
    }
  }
  float mt = fmaxf(s[0], s[1]);
#pragma unroll
  for (int x = 2; x < 32; ++x) mt = fmaxf(mt, s[x]);
  {
    // the other half of the wavefront holds the same queries' other 32 keys
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
    mt = fmaxf(mt, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
  }
  // the first tile with a permitted key of the row, or a maximum that grew
  // by more than 8
  const bool need = init ? (mt > 8.0f) : (PM ? (mt > -INFINITY) : true);
  const float shift = need ? mt : 0.f;
  const float alpha = (need && init) ? __builtin_amdgcn_exp2f(-mt) : 1.0f;
  if (__any(need)) {
#pragma unroll
    for (int x = 0; x < 32; ++x) s[x] -= shift;
  }
  m += shift;
  init = init || need;
  return alpha;
}

// Output of 32 queries i0 .. i0+31 none of which is valid: zero rows of O
// and a log-sum-exp of -inf.
__device__ __forceinline__ void zero_rows(const FlashMfmaArgs& a, int b, int h, int s, int i0, int lane) {
  const Layout& L = a.L;
  const int N = L.N, H = L.H, DO = L.DO;
  if (a.ks > 1) {
    // partial result: empty statistics (the combine reads no values then)
    if (lane < 32 && i0 + lane < N) {
      float* rec = reinterpret_cast<float*>(const_cast<char*>(a.ws) + part_rec_off(L, s, b, h, i0 + lane)) + DO;
      rec[0] = -INFINITY; rec[1] = 0.f; rec[2] = 0.f; rec[3] = 0.f;
    }
    return;
  }
  if (lane < 32 && i0 + lane < N) a.lse[((size_t)b * H + h) * N + i0 + lane] = -INFINITY;
  if ((DO & 3) == 0) {
    const int n4 = DO >> 2;
    for (int x = lane; x < 32 * n4; x += 64) {
      const int q = x / n4, j = x - q * n4;
      if (i0 + q < N)
        reinterpret_cast<float4*>(a.o + (((size_t)b * N + i0 + q) * H + h) * DO)[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  } else {
    for (int x = lane; x < 32 * DO; x += 64) {
      const int q = x / DO, c = x - q * DO;
      if (i0 + q < N) a.o[(((size_t)b * N + i0 + q) * H + h) * DO + c] = 0.f;
    }
  }
}

// Final normalisation (or, with several key ranges, the partial result) of
// one block of 32 queries i - l32 .. i - l32 + 31 after its last key tile:
// log-sum-exp, O divided by the ones-row sums, the centroid added back to the
// value points.  Widths that are multiples of 4 are written straight from
// the accumulator registers; others through an LDS slot of the (then free)
// tile buffers, `w` naming the slot (0 .. W-1).  Every wavefront of the
// workgroup calls it the same number of times (the staged path contains a
// barrier; which path runs depends only on the shape).
// Value blocks: 0 = [v 2^-8 (Dv) | 1 | 0], 1 = [x - c_t (3Q) | 1 | c_t | 0],
// 2 .. NVB = pair factors 2^-8 (R Cz rows).  The output row is
// [v (Dv) | pair (R Cz) | points (3Q)], i.e. the blocks in the order
// 0, 2, 3, .., NVB, 1 ("positions" 0 .. NVB below).
template <int NVB>
__device__ __forceinline__ constexpr int block_at(int pos) { return pos == 0 ? 0 : (pos == NVB ? 1 : pos + 1); }

template <int NQS, int NVB, int GS, int W, int NBUF>
__device__ __forceinline__ void finish_rows(const FlashMfmaArgs& a, char* skv, int sp, int b, int h, int i,
                                            bool qin, bool qvalid, int w, int lane, int l32, int half,
                                            const f32x16_t* oacc, float m, float l, bool init) {
  using T = TileDims<NQS, NVB, GS>;
  const Layout& L = a.L;
  const int N = L.N, H = L.H;
  const float ltot = l + __shfl_xor(l, 32);
  const bool nonempty = qvalid && init && ltot > 0.f;
  const bool partial = a.ks > 1;
  if (qin && half == 0 && !partial)
    a.lse[((size_t)b * H + h) * N + i] = nonempty ? (m + log2f(ltot)) * kLn2 : -INFINITY;

  // row d of a 32-row block sits in register 4*(d/8) + d%4 of the lane half (d%8)/4
  const int Dv = L.Dv, RCz = L.RCz, Q3 = 3 * L.Q, DO = L.DO;
  const int d1 = Dv + RCz;
  float lbf, lh, cxyz[3];
  lbf = __shfl(pick16(oacc[0], 4 * (Dv >> 3) + (Dv & 3)), l32 + 32 * ((Dv & 7) >> 2));
  {
    int rr = Q3;
    lh = __shfl(pick16(oacc[1], 4 * (rr >> 3) + (rr & 3)), l32 + 32 * ((rr & 7) >> 2));
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      rr = Q3 + 1 + x;
      cxyz[x] = __shfl(pick16(oacc[1], 4 * (rr >> 3) + (rr & 3)), l32 + 32 * ((rr & 7) >> 2));
    }
  }
  // a partial result keeps the unnormalised sums (values times 2^-8) and
  // its statistics; the combine normalises
  const float ib = nonempty ? (partial ? 1.0f : (1.0f / kVScale) / lbf) : 0.f;  // the value rows hold v 2^-8
  const float ih = nonempty ? (partial ? 1.0f : 1.0f / lh) : 0.f;
  float* prec = reinterpret_cast<float*>(const_cast<char*>(a.ws) + part_rec_off(L, sp, b, h, 0));
  if (partial && qin && half == 0) {
    float* st = prec + (size_t)i * L.PREC + DO;
    st[0] = nonempty ? m : -INFINITY;
    st[1] = nonempty ? ltot : 0.f;
    st[2] = nonempty ? lbf : 0.f;
    st[3] = nonempty ? lh : 0.f;
  }
  // Widths that are multiples of 4 (every instance's standard shape): a
  // lane's registers 4k .. 4k+3 of a block are rows 8k + 4 half .. +3, four
  // consecutive output columns of its query row, written as one 16-byte
  // store straight from the registers (no staging, no barrier); the two
  // lane halves fill 32 consecutive bytes of each of the 32 rows.  The
  // condition is uniform over the workgroup, so either every wavefront takes
  // the barrier of the staged path below or none does.
  const int pitch = partial ? L.PREC : DO;
  if (((Dv | RCz | Q3 | pitch) & 3) == 0) {
    if (!qin) return;
    float* row = partial ? prec + (size_t)i * L.PREC : a.o + (((size_t)b * N + i) * H + h) * DO;
#pragma unroll
    for (int vb = 0; vb <= NVB; ++vb) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int rr = 8 * k + 4 * half;  // first row of the lane's group
        int col;
        bool ok;
        if (vb == 0) {
          col = rr;
          ok = rr < Dv;
        } else if (vb == 1) {
          col = d1 + rr;
          ok = rr < Q3;
        } else {
          const int pr = 32 * (vb - 2) + rr;
          col = Dv + pr;
          ok = pr < RCz;
        }
        float e4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * k + e;
          if (vb != 1) {
            e4[e] = oacc[vb][r] * ib;
          } else {
            // value-point row 8k + e + 4 half: add back centroid coordinate (row % 3)
            const int x0 = (8 * k + e) % 3, x1 = (8 * k + e + 4) % 3;
            const float c0 = x0 == 0 ? cxyz[0] : (x0 == 1 ? cxyz[1] : cxyz[2]);
            const float c1 = x1 == 0 ? cxyz[0] : (x1 == 1 ? cxyz[1] : cxyz[2]);
            e4[e] = (oacc[1][r] + (half ? c1 : c0)) * ih;
          }
        }
        if (ok) *reinterpret_cast<float4*>(row + col) = make_float4(e4[0], e4[1], e4[2], e4[3]);
      }
    }
    return;
  }
  // first and one-past-last output column of position p
  auto col_start = [&](int p) { return p == 0 ? 0 : (p == NVB ? d1 : min(Dv + 32 * (p - 1), d1)); };
  auto col_end = [&](int p) { return p == 0 ? Dv : (p == NVB ? d1 + Q3 : min(Dv + 32 * p, d1)); };
  // O is written through LDS (the tile buffers are free now), BPP positions
  // per pass: every wavefront stores its 32 queries x 32 BPP rows (scaled) in
  // a slot of its own, register by register, then writes the pass's output
  // columns, one contiguous range, 16 bytes per lane with consecutive lanes
  // on consecutive addresses.
  constexpr int NB = NVB + 1;
  constexpr int SLOT = NBUF * T::TB / W;  // bytes per slot
  constexpr int BPP0 = (SLOT / (32 * 4) - 1) / 32;
  constexpr int BPP = BPP0 < NB ? BPP0 : NB;
  static_assert(BPP >= 1, "LDS slots too small for the output staging");
  constexpr int PITCH = 32 * BPP + 1;  // floats per staged query row
  static_assert(32 * PITCH * 4 <= SLOT, "output staging slot");
  float* slot = reinterpret_cast<float*>(skv + (size_t)w * SLOT);
  const int i0 = i - l32;  // first query of this wavefront
  __syncthreads();  // every wave is done with the tile buffers
#pragma unroll
  for (int p = 0; p < (NB + BPP - 1) / BPP; ++p) {
    const int p0 = p * BPP;
    const int p1 = p0 + BPP < NB ? p0 + BPP : NB;
#pragma unroll
    for (int j = 0; j < BPP; ++j) {
      const int pos = p0 + j;
      if (pos < NB) {
        const int vb = block_at<NVB>(pos);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // row of register r in a 32-row block: 8 (r/4) + 4 half + r%4
          const int rb = 8 * (r >> 2) + (r & 3);
          float v;
          if (vb != 1) {
            v = oacc[vb][r] * ib;
          } else {
            // value-point row dd = rb + 4 half: add back the centroid coordinate dd % 3
            const int x0 = rb % 3, x1 = (rb + 4) % 3;
            const float c0 = x0 == 0 ? cxyz[0] : (x0 == 1 ? cxyz[1] : cxyz[2]);
            const float c1 = x1 == 0 ? cxyz[0] : (x1 == 1 ? cxyz[1] : cxyz[2]);
            v = (oacc[1][r] + (half ? c1 : c0)) * ih;
          }
          slot[l32 * PITCH + 32 * j + rb + 4 * half] = v;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    // output columns of this pass: [col_start(p0), col_end(p1 - 1))
    const int cs = col_start(p0), ce = col_end(p1 - 1);
    const int nc = ce - cs, n4 = (nc + 3) >> 2;
    const bool vec = (((partial ? L.PREC : DO) | cs) & 3) == 0;
    for (int x = lane; x < 32 * n4; x += 64) {
      const int q = x / n4, jj = x - q * n4, iq = i0 + q;
      if (iq >= N) continue;
      const float* sr = slot + q * PITCH;
      float e4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = cs + 4 * jj + e;
        // position and row of output column c
        const int pos = c < Dv ? 0 : (c < d1 ? 1 + (c - Dv) / 32 : NVB);
        const int row = c < Dv ? c : (c < d1 ? (c - Dv) % 32 : c - d1);
        e4[e] = c < ce ? sr[32 * (pos - p0) + row] : 0.f;
      }
      float* dst = (partial ? prec + (size_t)iq * L.PREC : a.o + (((size_t)b * N + iq) * H + h) * DO) + cs + 4 * jj;
      if (vec && 4 * jj + 4 <= nc) {
        *reinterpret_cast<float4*>(dst) = make_float4(e4[0], e4[1], e4[2], e4[3]);
      } else {
        for (int e = 0; e < 4 && 4 * jj + e < nc; ++e) dst[e] = e4[e];
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// One key tile t of the main loop, held in LDS buffer BUF (a compile-time
// index, so that every LDS offset is a constant): the point operand with the
// current running maximum; with two buffers the wait for the tile's copies
// (issued one tile earlier), the barrier that makes them visible and frees
// the other buffer, and the copies of the next valid tile into that buffer;
// with one buffer a barrier (every wavefront is done with the previous tile,
// unless t is the first), the copies of tile t, the wait and a barrier; then
// the products and softmax of tile t.  Returns the next tile with a valid key
// (tend if none).
template <int NQS, int NVB, int GS, int W, bool PM, int NBUF, int BUF, bool STK>
__device__ __forceinline__ int attend_tile(const FlashMfmaArgs& a, const TileSrc& src, char* skv,
                                           const uint32_t* kmb, const float4* ckb, int t, int tend, int b, int i,
                                           bool qin, bool qvalid, bool active, int w, int lane, int l32, int half,
                                           float gl, float Pf, const bf16x8_t* bq, f16x8_t* bg, const QueryGeo& qg,
                                           f32x16_t* oacc, float& m, float& l, bool& init, int t_first) {
  using T = TileDims<NQS, NVB, GS>;
  const Layout& L = a.L;
  const int tn = next_valid_tile(kmb, t, tend);
  uint32_t mw = 0xFFFFFFFFu;
  if constexpr (PM) mw = perm_word(L, a.ws, true, b, i, qin, qvalid, t, half);
  if constexpr (STK)
    geo_tile_stacked(qg, m, half, bg);
  else
    geo_tile<GS>(qg, ld_uniform4(ckb + t), gl, Pf, m, half, bg);
  if constexpr (NBUF == 2) {
    // tile t has landed; every wave is done with the previous tile
    wait_vmcnt<0>();
    __syncthreads();
    if constexpr (PM) asm volatile("" ::"v"(mw));  // in registers before the next copies are issued
    if (tn < tend) copy_kv_tile<NQS, NVB, GS, W>(src, skv, tn, 1 - BUF, w, lane);
  } else {
    // the first tile's copies went out before the loop
    if (t != t_first) {
      __syncthreads();  // every wave is done with the previous tile
      copy_kv_tile<NQS, NVB, GS, W>(src, skv, t, 0, w, lane);
    }
    wait_vmcnt<0>();
    __syncthreads();
    if constexpr (PM) asm volatile("" ::"v"(mw));
  }
  if (!active) return tn;
  const char* kt = skv + BUF * T::TB;
  f32x16_t sacc[2];
  __builtin_amdgcn_s_setprio(1);
  s_tile<NQS, GS, 3, STK>(kt, kt + T::KH, bq, bg, l32, half, sacc);
  __builtin_amdgcn_s_setprio(0);

  float s32[32];
  const float alpha = softmax_max<PM>(sacc, mw, m, init, s32);
  if (__any(alpha != 1.0f)) {
#pragma unroll
    for (int vb = 0; vb <= NVB; ++vb) oacc[vb] *= alpha;
  }
  f16x8_t ph[4];
  if constexpr (W == 4) {
    // one wavefront per SIMD (the widest rows): no second wavefront hides
    // the softmax behind its matrix work, so the exponentials of the second
    // 32-key block are issued between the value-product MFMAs of the first
    // (K-steps 0 and 1 use only the first block's probabilities)
    const float ps = exp_pv_interleaved<NVB>(kt + T::KH + T::KZ + (size_t)(l32 * kVCols) * 2 + half * 16, s32, ph,
                                             oacc);
    l = l * alpha + ps;
    return tn;
  }
  const float ps = exp_tile(s32, ph);
  l = l * alpha + ps;

  __builtin_amdgcn_s_setprio(1);
  pv_tile<NVB>(kt + T::KH + T::KZ + (size_t)(l32 * kVCols) * 2 + half * 16, ph, oacc);
  __builtin_amdgcn_s_setprio(0);
  return tn;
}

// Main loop over the key tiles [t, tend) of key range sp and the final
// normalisation (or, with several key ranges, the partial result) for one
// wavefront's 32 queries.  The copy of the first tile t (into buffer 0) was
// issued by the caller.  Key/value tiles alternate between two LDS buffers
// (the loop is unrolled by two so that buffer offsets are constants).  PM
// selects the per-query pair-mask words (a vector load per tile); without a
// pair mask the key mask is inside the key product.
template <int NQS, int NVB, int GS, int W, int NBUF, bool PM, bool STK>
__device__ __forceinline__ void attend(const FlashMfmaArgs& a, const TileSrc& src, char* skv, int t, int tend, int sp,
                                       int b, int h, int i, bool qin, bool qvalid, int w, int lane, int l32, int half,
                                       float gl, float Pf, const bf16x8_t* bq, f16x8_t* bg, const QueryGeo& qg) {
  const Layout& L = a.L;
  const int NT = L.NT;
  const float4* ckb = reinterpret_cast<const float4*>(a.ws + L.off_ck) + (size_t)b * NT;
  const uint32_t* kmb = reinterpret_cast<const uint32_t*>(a.ws + L.off_km) + (size_t)b * NT * 2;
  f32x16_t oacc[NVB + 1];
#pragma unroll
  for (int vb = 0; vb <= NVB; ++vb) oacc[vb] = f32x16_t{};
  float m = 0.f, l = 0.f;
  bool init = false;
  // a wavefront without a valid query keeps copying tiles and meeting the
  // barriers, but does no products
  const bool active = __any(qvalid);
  const int t_first = t;
#define FIPA_TILE(BUFI)                                                                                             \
  attend_tile<NQS, NVB, GS, W, PM, NBUF, BUFI, STK>(a, src, skv, kmb, ckb, t, tend, b, i, qin, qvalid, active, w, lane,   \
                                               l32, half, gl, Pf, bq, bg, qg, oacc, m, l, init, t_first)
  if constexpr (NBUF == 2) {
    while (t < tend) {
      t = FIPA_TILE(0);
      if (t >= tend) break;
      t = FIPA_TILE(1);
    }
  } else {
    while (t < tend) t = FIPA_TILE(0);
  }
#undef FIPA_TILE
  finish_rows<NQS, NVB, GS, W, NBUF>(a, skv, sp, b, h, i, qin, qvalid, w, lane, l32, half, oacc, m, l, init);
}

// NBUF tile buffers, each [head key rows | pair key rows | head value rows |
// pair value rows]; with one buffer two workgroups share a CU (registers
// capped at 256 a lane).
template <int NQS, int NVB, int GS, int W, int NBUF, bool STK = false>
__global__ __launch_bounds__(W * 64, NBUF == 1 ? 2 : 1) void flash_mfma_kernel(FlashMfmaArgs a) {
  using T = TileDims<NQS, NVB, GS>;
  __shared__ __attribute__((aligned(1024))) char skv[NBUF * T::TB];

  const Layout& L = a.L;
  const int N = L.N, H = L.H;
  // Consecutive workgroup ids go round-robin over the 8 XCDs; remap so each
  // XCD works through a contiguous range of (b, h, query tile), keeping the
  // key/value tiles of a head in one L2.
  const int wg = blockIdx.x;
  int logical = wg;
  if ((a.nwg & 7) == 0) logical = (wg & 7) * (a.nwg >> 3) + (wg >> 3);
  const int qt = logical % a.qtiles;
  const int sp = (logical / a.qtiles) % a.ks;  // key range
  const int bh = logical / (a.qtiles * a.ks);
  const int h = bh % H, b = bh / H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront index (uniform)
  const int l32 = lane & 31, half = lane >> 5;
  const int i = qt * (W * 32) + w * 32 + l32;
  const bool qin = i < N;

  const int NT = L.NT;
  const uint32_t* kmb = reinterpret_cast<const uint32_t*>(a.ws + L.off_km) + (size_t)b * NT * 2;
  const TileSrc src{a.ws + kt_tile_off(L, b, h, 0), a.ws + ktz_tile_off(L, b, 0), a.ws + vt_tile_off(L, b, h, 0),
                    a.ws + vtz_tile_off(L, b, 0)};
  // key tiles [tb, te) of key range sp; the copy of the first goes out
  // before anything else is loaded
  const int tb = (int)(((long)NT * sp) / a.ks), te = (int)(((long)NT * (sp + 1)) / a.ks);
  const int t0 = next_valid_tile(kmb, tb - 1, te);
  if (t0 < te) copy_kv_tile<NQS, NVB, GS, W>(src, skv, t0, 0, w, lane);
  {
    // a workgroup none of whose queries is valid (padding) only writes zeros
    const int tq0 = (qt * W * 32) >> 6, tq1 = min(NT, tq0 + W / 2);
    uint32_t any = 0;
    for (int tq = tq0; tq < tq1; ++tq) any |= ld_uniform(kmb + 2 * tq) | ld_uniform(kmb + 2 * tq + 1);
    if (any == 0) {
      wait_vmcnt<0>();  // the tile copy lands before the workgroup's LDS is released
      zero_rows(a, b, h, sp, qt * (W * 32) + w * 32, lane);
      return;
    }
  }

  const Header* hd = reinterpret_cast<const Header*>(a.ws);
  const bool has_pm = ld_uniform(&hd->has_pair_mask) != 0;
  const float gl = ld_uniform(reinterpret_cast<const float*>(a.ws + L.off_gam) + h) * kLog2e;
  const float Pf = (float)L.P;

  // query operand (B of S^T): lane holds query l32, columns half*8 .. +7 of each K-step
  bf16x8_t bq[NQS];
  load_q_operand<NQS>(L, a.ws, b, h, i, qin, half, bq);
  const bool qvalid = query_valid(L, a.ws, b, i, qin);
  f16x8_t bg[GS];
  QueryGeo qg;
  {
    float av[15];
    load_qa(reinterpret_cast<const float4*>(a.ws + qa_row_off(L, b, h, qin ? i : 0)), qin, av);
    if constexpr (STK)
      build_geo_stacked<4>(av, half, bg, &qg);
    else
      build_geo<GS>(L.P, av, qvalid, gl, half, bg, &qg);
  }

  if (has_pm)
    attend<NQS, NVB, GS, W, NBUF, true, STK>(a, src, skv, t0, te, sp, b, h, i, qin, qvalid, w, lane, l32, half, gl, Pf, bq,
                                        bg, qg);
  else
    attend<NQS, NVB, GS, W, NBUF, false, STK>(a, src, skv, t0, te, sp, b, h, i, qin, qvalid, w, lane, l32, half, gl, Pf, bq,
                                         bg, qg);
}

// Merge the partial results of the KS key ranges of every (b, h, query):
// weights 2^(m_s - m) for the range maxima m_s, values divided by the merged
// ones-row sums, log-sum-exp from the merged fp32 sums.  One thread per four
// output columns of a row; every load of a thread (the statistics and four
// values of each range) is issued before any is used, the ranges past KS
// reading range KS - 1 and weighing nothing.
__global__ __launch_bounds__(256) void combine_kernel(Layout L, const float* part, float* o, float* lse) {
  const int DO = L.DO, n4 = (DO + 3) >> 2, H = L.H, N = L.N, KS = L.KS;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)L.B * N * H * n4) return;
  const long row = idx / n4;  // output row (b, i, h)
  const int c4 = (int)(idx - row * n4);
  const int h = (int)(row % H), i = (int)((row / H) % N), b = (int)(row / ((long)H * N));
  const size_t sstride = (size_t)L.B * H * L.NQpad * L.PREC;
  const float* rec0 = part + (((size_t)b * H + h) * L.NQpad + i) * L.PREC;
  float sm[4], sl[4], sb[4], sh[4];
  float4 v[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const float* rec = rec0 + (size_t)min(s, KS - 1) * sstride;
    sm[s] = rec[DO];
    sl[s] = rec[DO + 1];
    sb[s] = rec[DO + 2];
    sh[s] = rec[DO + 3];
    v[s] = *reinterpret_cast<const float4*>(rec + 4 * c4);
  }
  float m = -INFINITY;
#pragma unroll
  for (int s = 0; s < 4; ++s)
    if (s < KS && sl[s] > 0.f) m = fmaxf(m, sm[s]);
  float ls = 0.f, lbf = 0.f, lh = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (m > -INFINITY) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // an empty range (or one past KS) holds no values
      // (its records may be unwritten: selected away, never multiplied)
      if (s < KS && sl[s] > 0.f) {
        const float wgt = __builtin_amdgcn_exp2f(sm[s] - m);
        ls = fmaf(wgt, sl[s], ls);
        lbf = fmaf(wgt, sb[s], lbf);
        lh = fmaf(wgt, sh[s], lh);
        acc[0] = fmaf(wgt, v[s].x, acc[0]); acc[1] = fmaf(wgt, v[s].y, acc[1]);
        acc[2] = fmaf(wgt, v[s].z, acc[2]); acc[3] = fmaf(wgt, v[s].w, acc[3]);
      }
    }
  }
  const bool nonempty = ls > 0.f;
  const int d1 = L.Dv + L.RCz;
  const float ib = nonempty ? (1.0f / kVScale) / lbf : 0.f, ih = nonempty ? 1.0f / lh : 0.f;
  float* orow = o + (size_t)row * DO;
  float r4[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) r4[e] = acc[e] * (4 * c4 + e < d1 ? ib : ih);
  if ((DO & 3) == 0) {
    reinterpret_cast<float4*>(orow)[c4] = make_float4(r4[0], r4[1], r4[2], r4[3]);
  } else {
    for (int e = 0; e < 4 && 4 * c4 + e < DO; ++e) orow[4 * c4 + e] = r4[e];
  }
  if (c4 == 0) lse[((size_t)b * H + h) * N + i] = nonempty ? (m + log2f(ls)) * kLn2 : -INFINITY;
}

// Short chains whose keys are not split (KS = 1, at most kShortRange tiles
// per query tile: the protein-like and short-chain batches) run on one tile
// buffer, four wavefronts (128 queries) per workgroup and two workgroups per
// CU; everything else on two buffers with 8 wavefronts (256 queries), one
// workgroup per CU.  Whole forwards measured 2% faster with one buffer on
// the two batches, 1.5-4% slower at N = 2048 and 4096 (key ranges split over
// more workgroups) and the same at N = 8192.  KS > 1 splits the keys of a
// query tile into ranges (one workgroup each, the combine kernel after).
constexpr int kShortRange = 16;
template <int NQS, int NVB, int GS, bool STK = false>
static hipError_t launch_inst(const Layout& L, const void* ws, float* o, float* lse, hipStream_t st) {
  FlashMfmaArgs a;
  a.L = L;
  a.ws = reinterpret_cast<const char*>(ws);
  a.o = o;
  a.lse = lse;
  a.ks = L.KS;
  if constexpr (NQS > 9) {
    // the widest rows (rank-3 pair factors): four wavefronts, one per SIMD,
    // with the whole register file each
    a.qtiles = (L.N + 127) / 128;
    a.nwg = a.qtiles * L.H * L.B * L.KS;
    hipLaunchKernelGGL((flash_mfma_kernel<NQS, NVB, GS, 4, 2>), dim3(a.nwg), dim3(256), 0, st, a);
  } else {
    if (L.KS == 1 && L.NT <= kShortRange) {
      a.qtiles = (L.N + 127) / 128;
      a.nwg = a.qtiles * L.H * L.B * L.KS;
      hipLaunchKernelGGL((flash_mfma_kernel<NQS, NVB, GS, 4, 1, STK>), dim3(a.nwg), dim3(256), 0, st, a);
    } else {
      a.qtiles = (L.N + 255) / 256;
      a.nwg = a.qtiles * L.H * L.B * L.KS;
      hipLaunchKernelGGL((flash_mfma_kernel<NQS, NVB, GS, 8, 2, STK>), dim3(a.nwg), dim3(512), 0, st, a);
    }
  }
  if (L.KS > 1) {
    const long n = (long)L.B * L.N * L.H * ((L.DO + 3) / 4);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, L,
                       reinterpret_cast<const float*>(reinterpret_cast<const char*>(ws) + L.off_part), o, lse);
  }
  return hipGetLastError();
}

hipError_t launch_flash_mfma(const Layout& L, const void* ws, float* o, float* lse, hipStream_t st) {
  if (L.stacked) {
    // the pages' stacked point columns (comparison): standard widths only
    if (L.GS == 2 && L.NQS == 9 && L.NVB == 5) return launch_inst<9, 5, 2, true>(L, ws, o, lse, st);
    return hipErrorInvalidValue;
  }
  if (L.GS == 3) {
    if (L.NQS == 3 && L.NVB == 2) return launch_inst<3, 2, 3>(L, ws, o, lse, st);
    if (L.NQS == 5 && L.NVB == 3) return launch_inst<5, 3, 3>(L, ws, o, lse, st);
    if (L.NQS == 9 && L.NVB == 5) return launch_inst<9, 5, 3>(L, ws, o, lse, st);
    if (L.NQS == 13 && L.NVB == 7) return launch_inst<13, 7, 3>(L, ws, o, lse, st);
  } else if (L.GS == 4) {
    if (L.NQS == 3 && L.NVB == 2) return launch_inst<3, 2, 4>(L, ws, o, lse, st);
    if (L.NQS == 5 && L.NVB == 3) return launch_inst<5, 3, 4>(L, ws, o, lse, st);
    if (L.NQS == 9 && L.NVB == 5) return launch_inst<9, 5, 4>(L, ws, o, lse, st);
    if (L.NQS == 13 && L.NVB == 7) return launch_inst<13, 7, 4>(L, ws, o, lse, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace fipa
