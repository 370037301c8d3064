// MFMA fragment code of the fused kernel, shared with the diagnostic logit
// kernel so that both evaluate every logit with the identical sequence of
// matrix instructions on the same operands (the diagnostic kernel passes a
// running maximum of zero, so only the rounding of the per-tile row term
// differs between the two).
#pragma once

#include "common.h"

namespace fipa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float f16_round(float x) {
  return (float)(_Float16)fminf(fmaxf(x, -65504.0f), 65504.0f);
}

// A centroid on the 4-angstrom grid, exactly representable in fp16.
__device__ __forceinline__ float grid_round(float x) {
  return f16_round((float)kCentGrid * rintf(x * (1.0f / (float)kCentGrid)));
}

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  return (uint32_t)f32_to_f16_bits(lo) | ((uint32_t)f32_to_f16_bits(hi) << 16);
}

// Query operand of S^T = K~ Q~^T (B operand): lane (l32, half) holds columns
// half*8 .. +7 of every 16-wide K-step of query row i.  K-step 0 holds the
// head's scalar columns (QL), K-steps 1 .. NQS-1 the pair columns
// bf16((w_pair[h] x zl) x kPairScale), formed here from the shared zl rows
// (QZ) and the head's pair weights (WP), both bf16 as given, in fp32 and
// rounded to nearest.
template <int NQS>
__device__ __forceinline__ void load_q_operand(const Layout& L, const char* ws, int b, int h, int i, bool qin,
                                               int half, bf16x8_t* bq) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const uint4* qrow = reinterpret_cast<const uint4*>(ws + ql_row_off(L, b, h, qin ? i : 0));
  const uint4* zrow = reinterpret_cast<const uint4*>(ws + qz_row_off(L, b, qin ? i : 0));
  const uint4* wrow = reinterpret_cast<const uint4*>(ws + wp_row_off(L, h));
  uint4 z[NQS], wv[NQS];
  z[0] = qin ? qrow[half] : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int ks = 1; ks < NQS; ++ks) {
    z[ks] = qin ? zrow[(ks - 1) * 2 + half] : make_uint4(0, 0, 0, 0);
    wv[ks] = wrow[(ks - 1) * 2 + half];
  }
  bq[0] = __builtin_bit_cast(bf16x8_t, z[0]);
  auto prod = [](uint32_t w2, uint32_t z2) {
    const float w0 = __uint_as_float(w2 << 16), w1 = __uint_as_float(w2 & 0xFFFF0000u);
    const float z0 = __uint_as_float(z2 << 16), z1 = __uint_as_float(z2 & 0xFFFF0000u);
    const bf16x2_t v = {(__bf16)(w0 * z0 * kPairScale), (__bf16)(w1 * z1 * kPairScale)};
    return __builtin_bit_cast(uint32_t, v);
  };
#pragma unroll
  for (int ks = 1; ks < NQS; ++ks) {
    const uint4 p = make_uint4(prod(wv[ks].x, z[ks].x), prod(wv[ks].y, z[ks].y), prod(wv[ks].z, z[ks].z),
                               prod(wv[ks].w, z[ks].w));
    bq[ks] = __builtin_bit_cast(bf16x8_t, p);
  }
}

__device__ __forceinline__ void load_qa(const float4* arow, bool qin, float* av) {
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    float4 v = qin ? arow[x] : make_float4(0.f, 0.f, 0.f, 0.f);
    if (4 * x + 0 < 15) av[4 * x + 0] = v.x;
    if (4 * x + 1 < 15) av[4 * x + 1] = v.y;
    if (4 * x + 2 < 15) av[4 * x + 2] = v.z;
    if (4 * x + 3 < 15) av[4 * x + 3] = v.w;
  }
}

// Per-wavefront query geometry: centroid c_w of the valid queries (32
// consecutive residues), split operand u = 2 gl (a - c_w), and the sums
// U = sum_p (a_p - c_w), SA = sum_p |a_p - c_w|^2 used by the per-tile row
// term t' = -gl sum_p |a_p - c_t|^2 = 2 gl delta.U - gl (P |delta|^2 + SA).
struct QueryGeo {
  float cw[3];
  float U[3];
  float SA;
  uint32_t fix0, fix1;  // fixed first two dwords of the last geometric K-step
  uint32_t fix2, fix3;  // stacked layout: its last two dwords (half 0)
};

template <int P, int GS>
__device__ __forceinline__ void build_geo_P(const float* av, bool qvalid, float gl, int half, f16x8_t* bg,
                                            QueryGeo* qg) {
  constexpr int P3 = 3 * P;
  constexpr int base = 16 * (GS - 1);
  // centroid of the valid queries of this wavefront (each half holds the same 32)
  float sx = 0.f, sy = 0.f, sz = 0.f, cnt = qvalid ? 1.f : 0.f;
  if (qvalid) {
#pragma unroll
    for (int p = 0; p < P; ++p) { sx += av[3 * p]; sy += av[3 * p + 1]; sz += av[3 * p + 2]; }
    sx *= 1.0f / P; sy *= 1.0f / P; sz *= 1.0f / P;
  }
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) {
    sx += __shfl_xor(sx, off);
    sy += __shfl_xor(sy, off);
    sz += __shfl_xor(sz, off);
    cnt += __shfl_xor(cnt, off);
  }
  const float inv = cnt > 0.f ? 1.0f / cnt : 0.f;
  qg->cw[0] = grid_round(sx * inv);
  qg->cw[1] = grid_round(sy * inv);
  qg->cw[2] = grid_round(sz * inv);
  float uh[P3], ul[P3];
  float U0 = 0.f, U1 = 0.f, U2 = 0.f, SA = 0.f;
#pragma unroll
  for (int g = 0; g < P3; ++g) {
    const float A = av[g] - qg->cw[g % 3];
    if (g % 3 == 0) U0 += A; else if (g % 3 == 1) U1 += A; else U2 += A;
    SA = fmaf(A, A, SA);
    const float u = 2.f * gl * A;
    uh[g] = f16_round(u);
    ul[g] = f16_round(u - uh[g]);
  }
  qg->U[0] = U0; qg->U[1] = U1; qg->U[2] = U2; qg->SA = SA;
  auto qval = [&](int g) -> float {
    if (g < base + 4) {
      const int c = g;
      if (c < P3) return uh[c];
      if (c < 2 * P3) return uh[c - P3];
      if (c < 3 * P3) return ul[c - 2 * P3];
      return 0.f;
    }
    if (g == base + 4 || g == base + 8 || g == base + 12) return kNormScale;
    return 0.f;  // delta and t' slots, set per key tile
  };
#pragma unroll
  for (int s = 0; s < GS; ++s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v0 = qval(16 * s + e), v1 = qval(16 * s + 8 + e);
      bg[s][e] = (_Float16)(half ? v1 : v0);
    }
  }
  const uint4 last = __builtin_bit_cast(uint4, bg[GS - 1]);
  qg->fix0 = last.x;
  qg->fix1 = last.y;
}

template <int GS>
__device__ __forceinline__ void build_geo(int P, const float* av, bool qvalid, float gl, int half, f16x8_t* bg,
                                          QueryGeo* qg) {
  if constexpr (GS == 3) {
    switch (P) {
      case 1: build_geo_P<1, 3>(av, qvalid, gl, half, bg, qg); break;
      case 2: build_geo_P<2, 3>(av, qvalid, gl, half, bg, qg); break;
      case 3: build_geo_P<3, 3>(av, qvalid, gl, half, bg, qg); break;
      default: build_geo_P<4, 3>(av, qvalid, gl, half, bg, qg); break;
    }
  } else {
    build_geo_P<5, 4>(av, qvalid, gl, half, bg, qg);
  }
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// Query side of the stacked comparison layout (common.h): per point
// [a_p (3) | |a_p|^2 | 1] in bf16 from the global query points, 16 in the
// key-mask column; the -m/16 columns are set per key tile (geo_tile_stacked).
template <int P>
__device__ __forceinline__ void build_geo_stacked(const float* av, int half, f16x8_t* bg, QueryGeo* qg) {
  auto qval = [&](int g) -> float {
    if (g < 5 * P) {
      const int p = g / 5, e = g % 5;
      const float x = av[3 * p], y = av[3 * p + 1], z = av[3 * p + 2];
      return e == 0 ? x : (e == 1 ? y : (e == 2 ? z : (e == 3 ? x * x + y * y + z * z : 1.0f)));
    }
    return g == kStkMaskCol ? 16.0f : 0.f;
  };
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    uint32_t d[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int g0 = 16 * s + 8 * half + 2 * e;
      d[e] = pack_bf16(qval(g0), qval(g0 + 1));
    }
    bg[s] = __builtin_bit_cast(f16x8_t, make_uint4(d[0], d[1], d[2], d[3]));
  }
  const uint4 last = __builtin_bit_cast(uint4, bg[1]);
  qg->fix0 = last.x; qg->fix1 = last.y; qg->fix2 = last.z; qg->fix3 = last.w;
}

// Per key tile (stacked layout): -msub/16 in three bf16 parts in columns
// 29..31 (half 1, elements 5..7), so that the product returns the logit
// minus msub.
__device__ __forceinline__ void geo_tile_stacked(const QueryGeo& qg, float msub, int half, f16x8_t* bg) {
  const float x = -msub * (1.0f / 16.0f);
  const float h1 = bf16_bits_to_f32(f32_to_bf16_bits(x));
  const float r1 = x - h1;
  const float h2 = bf16_bits_to_f32(f32_to_bf16_bits(r1));
  const float h3 = r1 - h2;
  uint4 last = make_uint4(qg.fix0, qg.fix1, qg.fix2, qg.fix3);
  if (half) {
    last.z = (qg.fix2 & 0xFFFFu) | ((uint32_t)f32_to_bf16_bits(h1) << 16);
    last.w = pack_bf16(h2, h3);
  }
  bg[1] = __builtin_bit_cast(f16x8_t, last);
}

// Per key tile: -delta (exact in fp16) in the last K-step, and the row term
// t' - msub (three fp16 parts of (t' - msub)/16) in the slots of half 1, so
// that the product returns the logit minus msub (the running maximum of the
// query in the fused kernel, 0 for plain logits).
template <int GS>
__device__ __forceinline__ void geo_tile(const QueryGeo& qg, float4 ct, float gl, float Pf, float msub, int half,
                                         f16x8_t* bg) {
  const float dx = ct.x - qg.cw[0], dy = ct.y - qg.cw[1], dz = ct.z - qg.cw[2];
  const float dU = fmaf(dx, qg.U[0], fmaf(dy, qg.U[1], dz * qg.U[2]));
  const float d2 = fmaf(dx, dx, fmaf(dy, dy, dz * dz));
  const float tp = 2.f * gl * dU - gl * fmaf(Pf, d2, qg.SA) - msub;
  const float x = fminf(fmaxf(tp * (1.0f / kNormScale), -65504.0f), 65504.0f);
  const float h1 = f16_round(x);
  const float r1 = x - h1;
  const float h2 = f16_round(r1);
  const float h3 = f16_round(r1 - h2);
  uint4 last;
  last.x = half ? pack_f16(kNormScale, h1) : qg.fix0;
  last.y = half ? pack_f16(h2, h3) : qg.fix1;
  last.z = pack_f16(kNormScale, -dx);
  last.w = pack_f16(-dy, -dz);
  bg[GS - 1] = __builtin_bit_cast(f16x8_t, last);
}

// S^T for one 64-key tile: sacc[kb] (keys kb*32 .. +31) x 32 queries.
// khead points at the tile's 64 head rows of KROW = 16 + 16 GS + pad 16-bit
// elements ([k | geometric | pad]), kpair at its 64 shared pair-factor rows
// of KZROW = 16 (NQS - 1) + pad elements (LDS or global memory).  K-step 0
// is the scalar part, K-steps 1 .. NQS-1 the pair part, then GS geometric
// K-steps.  The two key blocks are interleaved so consecutive MFMAs are
// independent, and the operand fragments are fetched DEPTH K-steps ahead of
// their MFMA so that the reads' latency hides behind the preceding MFMAs.
// s_tile_ops emits the reads and MFMAs only; the caller orders them
// (s_tile_sched), so that other work can be placed between them.
template <int NQS, int GS, int DEPTH, bool STK = false>
__device__ __forceinline__ void s_tile_ops(const char* khead, const char* kpair, const bf16x8_t* bq,
                                           const f16x8_t* bg, int l32, int half, f32x16_t* sacc) {
  constexpr int KROW = 16 + 16 * GS + kRowPad;
  constexpr int KZROW = 16 * (NQS - 1) + kRowPad;
  constexpr int NS = NQS + GS;
  const char* h0 = khead + (size_t)(l32 * KROW) * 2 + half * 16;
  const char* h1 = h0 + (size_t)(32 * KROW) * 2;
  const char* z0 = kpair + (size_t)(l32 * KZROW) * 2 + half * 16;
  const char* z1 = z0 + (size_t)(32 * KZROW) * 2;
  // fragment of K-step st for key block kb
  auto frag = [&](int st, int kb) {
    const char* p = st == 0 ? (kb ? h1 : h0)
                            : (st < NQS ? (kb ? z1 : z0) + (st - 1) * 32 : (kb ? h1 : h0) + (16 + (st - NQS) * 16) * 2);
    return *reinterpret_cast<const uint4*>(p);
  };
  uint4 f0[DEPTH], f1[DEPTH];
#pragma unroll
  for (int st = 0; st < DEPTH && st < NS; ++st) {
    f0[st] = frag(st, 0);
    f1[st] = frag(st, 1);
  }
  sacc[0] = f32x16_t{};
  sacc[1] = f32x16_t{};
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const uint4 c0 = f0[st % DEPTH], c1 = f1[st % DEPTH];
    if (st + DEPTH < NS) {
      f0[st % DEPTH] = frag(st + DEPTH, 0);
      f1[st % DEPTH] = frag(st + DEPTH, 1);
    }
    if (st < NQS) {
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, c0), bq[st], sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, c1), bq[st], sacc[1], 0, 0, 0);
    } else if constexpr (STK) {
      // stacked comparison layout: bf16 point columns
      const bf16x8_t g = __builtin_bit_cast(bf16x8_t, bg[st - NQS]);
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, c0), g, sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, c1), g, sacc[1], 0, 0, 0);
    } else {
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, c0), bg[st - NQS], sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, c1), bg[st - NQS], sacc[1], 0, 0, 0);
    }
  }
}

// Instruction order for s_tile_ops: the first DEPTH steps' reads, then per
// step its two MFMAs, the reads DEPTH steps ahead and up to VPER vector-ALU
// instructions of independent work placed in the same region.
template <int NS, int DEPTH, int VPER>
__device__ __forceinline__ void s_tile_sched() {
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * DEPTH, 0);
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    if (st + DEPTH < NS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    if (VPER > 0) __builtin_amdgcn_sched_group_barrier(0x002, VPER, 0);
  }
}

template <int NQS, int GS, int DEPTH = 3, bool STK = false>
__device__ __forceinline__ void s_tile(const char* khead, const char* kpair, const bf16x8_t* bq, const f16x8_t* bg,
                                       int l32, int half, f32x16_t* sacc) {
  s_tile_ops<NQS, GS, DEPTH, STK>(khead, kpair, bq, bg, l32, half, sacc);
  s_tile_sched<NQS + GS, DEPTH, 0>();
}

// Permitted-key word of a lane for key tile t (bit kb*16 + r <-> key
// kb*32 + 8*(r/4) + 4*half + r%4).
__device__ __forceinline__ uint32_t perm_word(const Layout& L, const char* ws, bool has_pm, int b, int i, bool qin,
                                              bool qvalid, int t, int half) {
  const uint32_t* km = reinterpret_cast<const uint32_t*>(ws + L.off_km);
  if (has_pm) {
    const uint32_t* pmw = reinterpret_cast<const uint32_t*>(ws + L.off_pm);
    return qin ? pmw[(((size_t)b * L.NQpad + i) * L.NT + t) * 2 + half] : 0u;
  }
  return qvalid ? km[((size_t)b * L.NT + t) * 2 + half] : 0u;
}

__device__ __forceinline__ bool query_valid(const Layout& L, const char* ws, int b, int i, bool qin) {
  if (!qin) return false;
  const uint32_t* km = reinterpret_cast<const uint32_t*>(ws + L.off_km);
  int hf;
  const int bit = mask_bit_of_key(i & 63, &hf);
  return (km[((size_t)b * L.NT + (i >> 6)) * 2 + hf] >> bit) & 1u;
}

}  // namespace fipa
