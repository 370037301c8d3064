// MFMA fragment code of the fused kernel, shared with the diagnostic logit
// kernel so that both evaluate every logit with the identical instruction
// sequence (and hence bit-identical results).
#pragma once

#include "common.h"

namespace fipa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float f16_round(float x) {
  return (float)(_Float16)fminf(fmaxf(x, -65504.0f), 65504.0f);
}

// value of geometric query column g (0..47) given the split parts
__device__ __forceinline__ float geo_q(int g, const float* uh, const float* ul) {
  if (g < kGeoW) return uh[g];
  if (g < 2 * kGeoW) return uh[g - kGeoW];
  if (g < 3 * kGeoW) return ul[g - 2 * kGeoW];
  if (g < 3 * kGeoW + 2) return kNormScale;
  return 0.f;
}

// Query operand of S^T = K~ Q~^T (B operand): lane (l32, half) holds columns
// half*8 .. +7 of every 16-wide K-step of query row `qrow`.
template <int NQS>
__device__ __forceinline__ void load_q_frag(const uint4* qrow, bool qin, int half, bf16x8_t* bq) {
#pragma unroll
  for (int ks = 0; ks < NQS; ++ks) {
    uint4 v = qin ? qrow[ks * 2 + half] : make_uint4(0, 0, 0, 0);
    bq[ks] = __builtin_bit_cast(bf16x8_t, v);
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

// Query-side geometric operand for a key tile with centroid c:
//   u = 2 gamma log2e (a - c) split into fp16 high/low parts,
//   na = gamma log2e |a - c|^2 (the row term, subtracted after the product).
__device__ __forceinline__ void geo_frag(const float* av, float4 c4, float gl, int P3, int half, f16x8_t* bg,
                                         float* na_out) {
  float uh[15], ul[15];
  float na = 0.f;
#pragma unroll
  for (int g = 0; g < 15; ++g) {
    const float cc = (g % 3 == 0) ? c4.x : ((g % 3 == 1) ? c4.y : c4.z);
    const float d = (g < P3) ? av[g] - cc : 0.f;
    na = fmaf(d, d, na);
    const float u = 2.f * gl * d;
    uh[g] = f16_round(u);
    ul[g] = f16_round(u - uh[g]);
  }
  *na_out = na * gl;
#pragma unroll
  for (int s = 0; s < 3; ++s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v0 = geo_q(s * 16 + e, uh, ul), v1 = geo_q(s * 16 + 8 + e, uh, ul);
      bg[s][e] = (_Float16)(half ? v1 : v0);
    }
  }
}

// S^T for one 64-key tile: sacc[kb] (keys kb*32 .. +31) x 32 queries.
// ktile points at 64 rows of KROW 16-bit elements (LDS or global memory).
template <int NQS>
__device__ __forceinline__ void s_tile(const char* ktile, const bf16x8_t* bq, const f16x8_t* bg, int l32, int half,
                                       f32x16_t* sacc) {
  constexpr int QW = 16 * NQS;
  constexpr int KROW = QW + kGeoCols + kRowPad;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    sacc[kb] = f32x16_t{};
    const char* krow = ktile + (size_t)((kb * 32 + l32) * KROW) * 2;
#pragma unroll
    for (int ks = 0; ks < NQS; ++ks) {
      const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(krow + (ks * 16 + half * 8) * 2);
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bq[ks], sacc[kb], 0, 0, 0);
    }
#pragma unroll
    for (int gs = 0; gs < 3; ++gs) {
      const f16x8_t af = *reinterpret_cast<const f16x8_t*>(krow + (QW + gs * 16 + half * 8) * 2);
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bg[gs], sacc[kb], 0, 0, 0);
    }
  }
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
