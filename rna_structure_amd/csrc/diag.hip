// Diagnostic kernel (tests only): the logits the fused kernel forms, for a
// few query rows, in natural-log units, -inf where the key is not permitted.
// The matrix-core variant runs the fused kernel's own MFMA fragment sequence
// (mfma_tile.h) on the same lifted operands and the same query grouping; the
// fused kernel folds its running maximum into the per-tile row term, which is
// zero here, so the two differ only in the rounding of that term (three fp16
// parts of the row term over 16: a few units of 2^-22 relative).  Together
// with the fused kernel's log-sum-exp these logits give the attention rows
// exp(L - lse).  The fp32
// variant repeats the fp32 kernel's expressions in the same order.
#include "mfma_tile.h"

namespace fipa {

struct DiagArgs {
  Layout L;
  const char* ws;
  int b, h, row0, nrows;
  float* out;
};

// One wavefront per aligned group of 32 query rows (the grouping of the
// fused kernel's wavefronts, which sets the query centroid), all key tiles.
template <int NQS, int GS>
__global__ __launch_bounds__(64) void logit_rows_mfma_kernel(DiagArgs a) {
  const Layout& L = a.L;
  const int lane = threadIdx.x, l32 = lane & 31, half = lane >> 5;
  const int b = a.b, h = a.h, N = L.N, H = L.H, NT = L.NT;
  const int i = (a.row0 / 32 + (int)blockIdx.x) * 32 + l32;
  const bool qin = i < N;
  const bool out_row = qin && i >= a.row0 && i < a.row0 + a.nrows;
  const Header* hd = reinterpret_cast<const Header*>(a.ws);
  const bool has_pm = hd->has_pair_mask != 0;
  const float gl = reinterpret_cast<const float*>(a.ws + L.off_gam)[h] * kLog2e;
  const float4* ck = reinterpret_cast<const float4*>(a.ws + L.off_ck);
  bf16x8_t bq[NQS];
  load_q_operand<NQS>(L, a.ws, b, h, i, qin, half, bq);
  const bool qvalid = query_valid(L, a.ws, b, i, qin);
  f16x8_t bg[GS];
  QueryGeo qg;
  {
    float av[15];
    load_qa(reinterpret_cast<const float4*>(a.ws + L.off_qa) + (((size_t)b * H + h) * L.NQpad + i) * 4, qin, av);
    build_geo<GS>(L.P, av, qvalid, gl, half, bg, &qg);
  }
  for (int t = 0; t < NT; ++t) {
    const uint32_t mw = perm_word(L, a.ws, has_pm, b, i, qin, qvalid, t, half);
    geo_tile<GS>(qg, ck[(size_t)b * NT + t], gl, (float)L.P, 0.f, half, bg);
    f32x16_t sacc[2];
    s_tile<NQS, GS>(a.ws + kt_tile_off(L, b, h, t), a.ws + ktz_tile_off(L, b, t), bq, bg, l32, half, sacc);
    if (!out_row) continue;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = t * 64 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (j < N)
          a.out[(size_t)(i - a.row0) * N + j] = ((mw >> (kb * 16 + r)) & 1u) ? sacc[kb][r] * kLn2 : -INFINITY;
      }
  }
}

__global__ __launch_bounds__(256) void logit_rows_f32_kernel(DiagArgs a) {
  const Layout& L = a.L;
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int ri = blockIdx.y;
  const int i = a.row0 + ri;
  const int b = a.b, h = a.h, N = L.N, H = L.H, NT = L.NT;
  if (j >= N || i >= N) return;
  const Header* hd = reinterpret_cast<const Header*>(a.ws);
  const int t = j >> 6, jj = j & 63;
  int hf;
  const int bit = mask_bit_of_key(jj, &hf);
  const uint32_t mw = perm_word(L, a.ws, hd->has_pair_mask != 0, b, i, true, query_valid(L, a.ws, b, i, true), t, hf);
  float* outp = a.out + (size_t)ri * N + j;
  if (!((mw >> bit) & 1u)) { *outp = -INFINITY; return; }
  const float gl = reinterpret_cast<const float*>(a.ws + L.off_gam)[h] * kLog2e;
  const float4 c4 = reinterpret_cast<const float4*>(a.ws + L.off_ck)[(size_t)b * NT + t];
  const float* arow = reinterpret_cast<const float*>(a.ws + L.off_qa) + (((size_t)b * H + h) * L.NQpad + i) * 16;
  const int P3 = 3 * L.P, DQ = L.D + L.RCz;
  const float* q = reinterpret_cast<const float*>(a.ws + L.off_ql) + (((size_t)b * H + h) * L.NQpad + i) * L.DQP;
  const float* k = reinterpret_cast<const float*>(a.ws + L.off_kt) + (((size_t)b * H + h) * L.NKpad + j) * L.KROW;
  float dA[15];
  for (int g = 0; g < 15; ++g) {
    const float cc = (g % 3 == 0) ? c4.x : ((g % 3 == 1) ? c4.y : c4.z);
    dA[g] = (g < P3) ? arow[g] - cc : 0.f;
  }
  float s = 0.f;
  for (int c = 0; c < DQ; ++c) s = fmaf(q[c], k[c], s);
  float dist = 0.f;
  for (int g = 0; g < P3; ++g) {
    const float df = dA[g] - k[DQ + g];
    dist = fmaf(df, df, dist);
  }
  s = fmaf(-gl, dist, s);
  *outp = s * kLn2;
}

template <int NQS, int GS>
static void launch_m(const DiagArgs& a, hipStream_t st) {
  const int groups = (a.row0 + a.nrows - 1) / 32 - a.row0 / 32 + 1;
  hipLaunchKernelGGL((logit_rows_mfma_kernel<NQS, GS>), dim3(groups), dim3(64), 0, st, a);
}

hipError_t launch_logit_rows(const Layout& L, const void* ws, int b, int h, int row0, int nrows, float* out,
                             hipStream_t st) {
  DiagArgs a;
  a.L = L;
  a.ws = reinterpret_cast<const char*>(ws);
  a.b = b; a.h = h; a.row0 = row0; a.nrows = nrows; a.out = out;
  if (L.mfma) {
    if (L.GS == 3 && L.NQS == 3) launch_m<3, 3>(a, st);
    else if (L.GS == 3 && L.NQS == 5) launch_m<5, 3>(a, st);
    else if (L.GS == 3 && L.NQS == 9) launch_m<9, 3>(a, st);
    else if (L.GS == 3 && L.NQS == 13) launch_m<13, 3>(a, st);
    else if (L.GS == 4 && L.NQS == 3) launch_m<3, 4>(a, st);
    else if (L.GS == 4 && L.NQS == 5) launch_m<5, 4>(a, st);
    else if (L.GS == 4 && L.NQS == 9) launch_m<9, 4>(a, st);
    else if (L.GS == 4 && L.NQS == 13) launch_m<13, 4>(a, st);
    else return hipErrorInvalidValue;
  } else {
    dim3 grid((L.N + 255) / 256, nrows);
    hipLaunchKernelGGL(logit_rows_f32_kernel, grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace fipa
