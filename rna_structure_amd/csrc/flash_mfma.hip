// Kernel 2, matrix-core path: fused masked online-softmax attention over the
// lifted IPA rows on gfx950 MFMA.  No [N,N] tensor is written anywhere.
//
// Per (batch b, head h, 128-query tile): 4 waves, each owning 32 queries.
// Per 64-key tile staged in LDS by the whole workgroup:
//   S^T (keys x queries) = K~ Q~^T        v_mfma_f32_32x32x16_bf16 over the
//                                         scalar + pair columns,
//                                         v_mfma_f32_32x32x16_f16 over the
//                                         centred point columns (fp16 hi/lo
//                                         split: 3 products per coordinate)
//   s = S - gamma log2e |a_i - c_t|^2     (row term of the expanded distance)
//   masked online softmax in fp32 with exp2 (logits carry a log2 e factor),
//   a running maximum that is only raised when it grows by more than 8
//   (probabilities stay below 2^8) and an fp32 row sum for the log-sum-exp
//   O^T += V~^T P^T                       bf16 probabilities against the
//                                         value and pair-factor rows, fp16
//                                         probabilities against the centred
//                                         value points, the centroid and a
//                                         ones row
// The accumulator layout of S^T gives every lane one query and 16 keys, so
// the probabilities feed the value product from registers; the value tile is
// stored transposed with its keys permuted to match (lift kernel).
// Normalisation uses the ones rows, i.e. the sums of the rounded
// probabilities actually multiplied into O, so the weights applied to the
// values sum to one to fp32 rounding and the centroid cancels exactly.
#include "mfma_tile.h"

namespace fipa {

struct FlashMfmaArgs {
  Layout L;
  const char* ws;
  float* o;
  float* lse;
  int qtiles;
  int nwg;
};

template <typename V>
__device__ __forceinline__ float pick16(const V& acc, int r) {
  float v = 0.f;
#pragma unroll
  for (int x = 0; x < 16; ++x) v = (x == r) ? acc[x] : v;
  return v;
}

template <int NQS, int NVB>
__global__ __launch_bounds__(256, 2) void flash_mfma_kernel(FlashMfmaArgs a) {
  constexpr int QW = 16 * NQS;
  constexpr int KROW = QW + kGeoCols + kRowPad;
  constexpr int KT_BYTES = 64 * KROW * 2;
  constexpr int VROWS = 32 * (NVB + 1);
  constexpr int VT_BYTES = VROWS * kVCols * 2;
  __shared__ __attribute__((aligned(16))) char smem[KT_BYTES + VT_BYTES];

  const Layout& L = a.L;
  const int N = L.N, H = L.H, NT = L.NT;
  // Consecutive workgroup ids go round-robin over the 8 XCDs; remap so each
  // XCD works through a contiguous range of (b, h, query tile), keeping the
  // key/value tiles of a head in one L2.
  const int wg = blockIdx.x;
  int logical = wg;
  if ((a.nwg & 7) == 0) logical = (wg & 7) * (a.nwg >> 3) + (wg >> 3);
  const int qt = logical % a.qtiles;
  const int bh = logical / a.qtiles;
  const int h = bh % H, b = bh / H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int i = qt * kQueryTile + w * 32 + l32;
  const bool qin = i < N;

  const Header* hd = reinterpret_cast<const Header*>(a.ws);
  const bool has_pm = hd->has_pair_mask != 0;
  const float gl = reinterpret_cast<const float*>(a.ws + L.off_gam)[h] * kLog2e;
  const uint32_t* km = reinterpret_cast<const uint32_t*>(a.ws + L.off_km);
  const float4* ck = reinterpret_cast<const float4*>(a.ws + L.off_ck);

  // query operand (B of S^T): lane holds query l32, columns half*8 .. +7 of each K-step
  bf16x8_t bq[NQS];
  load_q_frag<NQS>(reinterpret_cast<const uint4*>(a.ws + L.off_ql) + (((size_t)b * H + h) * L.NQpad + i) * (QW / 8),
                   qin, half, bq);
  float av[15];
  load_qa(reinterpret_cast<const float4*>(a.ws + L.off_qa) + (((size_t)b * H + h) * L.NQpad + i) * 4, qin, av);
  const int P3 = 3 * L.P;
  const bool qvalid = query_valid(L, a.ws, b, i, qin);

  f32x16_t oacc[NVB + 1];
#pragma unroll
  for (int vb = 0; vb <= NVB; ++vb) oacc[vb] = f32x16_t{};
  float m = -INFINITY, l = 0.f;

  const char* ktg0 = a.ws + L.off_kt + ((size_t)b * H + h) * NT * (size_t)KT_BYTES;
  const char* vtg0 = a.ws + L.off_vt + ((size_t)b * H + h) * NT * (size_t)VT_BYTES;

  for (int t = 0; t < NT; ++t) {
    const uint32_t k0 = km[((size_t)b * NT + t) * 2], k1 = km[((size_t)b * NT + t) * 2 + 1];
    if ((k0 | k1) == 0u) continue;  // no valid key in this tile (uniform)
    const uint32_t mw = perm_word(L, a.ws, has_pm, b, i, qin, qvalid, t, half);

    __syncthreads();
    {
      const uint4* kg = reinterpret_cast<const uint4*>(ktg0 + (size_t)t * KT_BYTES);
      const uint4* vg = reinterpret_cast<const uint4*>(vtg0 + (size_t)t * VT_BYTES);
      uint4* s4 = reinterpret_cast<uint4*>(smem);
      for (int c = tid; c < KT_BYTES / 16; c += 256) s4[c] = kg[c];
      for (int c = tid; c < VT_BYTES / 16; c += 256) s4[KT_BYTES / 16 + c] = vg[c];
    }
    __syncthreads();

    // query geometric operand for this key tile (centroid c_t), then S^T = K~ Q~^T
    f16x8_t bg[3];
    float na;
    geo_frag(av, ck[(size_t)b * NT + t], gl, P3, half, bg, &na);
    f32x16_t sacc[2];
    s_tile<NQS>(smem, bq, bg, l32, half, sacc);

    float s[32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb * 16 + r] = sacc[kb][r] - na;
    if (!__all(mw == 0xFFFFFFFFu)) {
#pragma unroll
      for (int x = 0; x < 32; ++x) s[x] = ((mw >> x) & 1u) ? s[x] : -INFINITY;
    }
    float mt = s[0];
#pragma unroll
    for (int x = 1; x < 32; ++x) mt = fmaxf(mt, s[x]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mnew = fmaxf(m, mt);
    if (__any(mnew > m + 8.0f)) {
      const float alpha = (mnew > m) ? exp2f(m - mnew) : 1.0f;
#pragma unroll
      for (int vb = 0; vb <= NVB; ++vb) oacc[vb] *= alpha;
      l *= alpha;
      m = mnew;
    }
    const float mu = (m == -INFINITY) ? 0.f : m;
    float p[32];
    float ps = 0.f;
#pragma unroll
    for (int x = 0; x < 32; ++x) {
      p[x] = exp2f(s[x] - mu);
      ps += p[x];
    }
    l += ps;
    bf16x8_t pb[4];
    f16x8_t ph[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = p[(ks >> 1) * 16 + (ks & 1) * 8 + e];
        pb[ks][e] = (__bf16)v;
        ph[ks][e] = (_Float16)v;
      }

    // O^T += V~^T P^T
    const char* vbase = smem + KT_BYTES;
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      const char* vrow = vbase + (size_t)((vb * 32 + l32) * kVCols) * 2;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(vrow + (ks * 16 + half * 8) * 2);
        oacc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, pb[ks], oacc[vb], 0, 0, 0);
      }
    }
    {
      const char* vrow = vbase + (size_t)((NVB * 32 + l32) * kVCols) * 2;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f16x8_t af = *reinterpret_cast<const f16x8_t*>(vrow + (ks * 16 + half * 8) * 2);
        oacc[NVB] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, ph[ks], oacc[NVB], 0, 0, 0);
      }
    }
  }

  // ---- finalise
  const float ltot = l + __shfl_xor(l, 32);
  const bool nonempty = qvalid && ltot > 0.f;
  const float mu = (m == -INFINITY) ? 0.f : m;
  if (qin && half == 0)
    a.lse[((size_t)b * H + h) * N + i] = nonempty ? (mu + log2f(ltot)) * kLn2 : -INFINITY;

  // row d of a 32-row block sits in register 4*(d/8) + d%4 of the lane half (d%8)/4
  const int Dv = L.Dv, RCz = L.RCz, Q3 = 3 * L.Q, DO = L.DO;
  const int d1 = Dv + RCz;
  float lbf, lh, cxyz[3];
  {
    const int vb1 = d1 >> 5, rr = d1 & 31;
    float v = 0.f;
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      const float pv = pick16(oacc[vb], 4 * (rr >> 3) + (rr & 3));
      v = (vb == vb1) ? pv : v;
    }
    lbf = __shfl(v, l32 + 32 * ((rr & 7) >> 2));
  }
  {
    int rr = Q3;
    lh = __shfl(pick16(oacc[NVB], 4 * (rr >> 3) + (rr & 3)), l32 + 32 * ((rr & 7) >> 2));
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      rr = Q3 + 1 + x;
      cxyz[x] = __shfl(pick16(oacc[NVB], 4 * (rr >> 3) + (rr & 3)), l32 + 32 * ((rr & 7) >> 2));
    }
  }
  if (!qin) return;
  const float ib = nonempty ? 1.0f / lbf : 0.f;
  const float ih = nonempty ? 1.0f / lh : 0.f;
  float* orow = a.o + (((size_t)b * N + i) * H + h) * DO;
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = vb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (d < d1) orow[d] = oacc[vb][r] * ib;
    }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int dd = 8 * (r >> 2) + 4 * half + (r & 3);
    if (dd < Q3) {
      const int x = dd % 3;
      const float c = (x == 0) ? cxyz[0] : ((x == 1) ? cxyz[1] : cxyz[2]);
      orow[d1 + dd] = (oacc[NVB][r] + c) * ih;
    }
  }
}

template <int NQS, int NVB>
static hipError_t launch_inst(const Layout& L, const void* ws, float* o, float* lse, hipStream_t st) {
  FlashMfmaArgs a;
  a.L = L;
  a.ws = reinterpret_cast<const char*>(ws);
  a.o = o;
  a.lse = lse;
  a.qtiles = (L.N + kQueryTile - 1) / kQueryTile;
  a.nwg = a.qtiles * L.H * L.B;
  hipLaunchKernelGGL((flash_mfma_kernel<NQS, NVB>), dim3(a.nwg), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_flash_mfma(const Layout& L, const void* ws, float* o, float* lse, hipStream_t st) {
  if (L.NQS == 3 && L.NVB == 2) return launch_inst<3, 2>(L, ws, o, lse, st);
  if (L.NQS == 5 && L.NVB == 3) return launch_inst<5, 3>(L, ws, o, lse, st);
  if (L.NQS == 9 && L.NVB == 5) return launch_inst<9, 5>(L, ws, o, lse, st);
  return hipErrorInvalidValue;
}

}  // namespace fipa
