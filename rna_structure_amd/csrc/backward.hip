// Backward pass of the IPA core (fp32, vector ALU): gradients of
// <update, d_update> + <local_points, d_local> with respect to every input of
// the forward ("Invariant point attention (IPA)" problem page, "Required
// behavior"; pair factors per the FlashIPA rebuttal, paperhub page, Q4/Q5).
// The page's starter code says its suite grades gradients.
//
// Per (b, h) and residue the forward is re-expressed with plain rows:
//   QV_i = [q_i / sqrt(3D) | w_pair[h] * zl_i / sqrt(3)]   (D + R Cz)
//   KV_j = [k_j | zr_j]                                     (D + R Cz)
//   VV_j = [v_j | zr_j | T_j(v_points_j)]                   (Dv + R Cz + 3Q)
//   A_i  = T_i(q_points_i),  B_j = T_j(k_points_j)          (3P each)
//   L_ij = QV_i . KV_j - gamma_h sum |A_i - B_j|^2   (natural log units)
// so the attention core is p = softmax_j(L) over the permitted keys and
// O_i = sum_j p_ij VV_j = [o_scalar | o_zr | g].  With dO from the epilogue's
// backward and Dsum_i = dO_i . O_i the core's gradients are the
// FlashAttention-style recomputation
//   dS_ij = p_ij (dO_i . VV_j - Dsum_i)
//   dQV_i = sum_j dS_ij KV_j,   dA_i = -2 gamma sum_j dS_ij (A_i - B_j)
//   dKV_j = sum_i dS_ij QV_i,   dB_j = +2 gamma sum_i dS_ij (A_i - B_j)
//   dVV_j = sum_i p_ij dO_i,    dgamma = -sum_ij dS_ij |A_i - B_j|^2
// in two passes (one over keys per query, one over queries per key), after a
// forward pass that yields O and the log-sum-exp.
// Precision: dO_i . VV_j - Dsum_i cancels, and for long chains the global
// value points in VV and O are hundreds of angstroms from the origin, so in
// fp32 the two products would carry absolute errors far above their
// difference.  Every 32-residue block k of a sample therefore has a
// reference point c_k (its first residue's translation rounded to whole
// angstroms, so that differences of references are exact): VV_j holds its
// points relative to c of j's block and O_i relative to c of i's block
// (O'_i), and with S_i = sum_q dO_i of the point part (3 components)
//   dO_i . VV_j - Dsum_i = dO_i . VV'_j - (Dsum'_i + S_i . (c_i - c_j))
// where Dsum'_i = dO_i . O'_i.  All products then involve coordinates of the
// size of a block or of the attention's reach.  Four lanes share a row:
// each holds a quarter of the columns and the dot products are summed over
// the quad with DPP.  The epilogue's backward and the weight gradients use a
// tiled fp32 GEMM; a last pass maps the row gradients back to the inputs
// (frames, points, factors) and reduces the per-head parameters.
#include <algorithm>

#include "common.h"

namespace fipa {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBwTile = 32;   // partner rows staged in LDS per step

struct BwLayout {
  int B, N, H, D, Dv, P, Q, Cz, R, Cout, F;
  int DK, DV, P3, NK4, NV4, DKp, DVp;
  int ksplit;
  int psplit;  // inner-loop ranges of the matrix-core pair passes (one workgroup each)
  size_t off_opart, off_xqv, off_xqa, off_xgam, off_xkv, off_xkb, off_xvv;  // their partial results (psplit > 1)
  size_t off_gam, off_qv, off_kv, off_vv, off_qa, off_kb, off_o, off_lse, off_do, off_dd, off_ds, off_feat, off_dfeat,
      off_dqv, off_dqa, off_dgam, off_dkv, off_dkb, off_dvv, off_dzle, off_dre, off_dte, off_dwpart, off_ppart,
      total;
  int bf16;               // inputs are bf16: converted into fp32 copies first
  size_t off_cvt[14];     // fp32 copies of the 14 inputs (bf16 inputs only)
  size_t cvt_n[14];
};

struct BwArgs {
  BwLayout L;
  char* ws;
  // inputs (fp32)
  const float *q, *k, *v, *qp, *kp, *vp, *rot, *tr, *wraw, *wpair, *zl, *zr, *wout, *bout;
  const uint8_t *mask, *pmask;
  const float *dupd, *dloc;
  float eps;
  // outputs
  float *gq, *gk, *gv, *gqp, *gkp, *gvp, *grot, *gtr, *gwraw, *gwpair, *gzl, *gzr, *gwout, *gbout;
};

__device__ __forceinline__ float* wsf(const BwArgs& a, size_t off) { return reinterpret_cast<float*>(a.ws + off); }

__device__ __forceinline__ size_t rowidx(const BwLayout& L, int b, int h, int n) {
  return ((size_t)b * L.H + h) * L.N + n;
}

// sum over the four lanes of a quad (the four parts of one row)
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
  return x;
}

// Reference point of the 32-residue block holding residue n of sample b: the
// block's first translation rounded to whole angstroms (differences of two
// references are exact in fp32).
__device__ __forceinline__ float3 blk_ref(const BwArgs& a, int b, int n) {
  const float* t = a.tr + ((size_t)b * a.L.N + (size_t)(n & ~31)) * 3;
  return make_float3(rintf(t[0]), rintf(t[1]), rintf(t[2]));
}

// e^x as 2^(x log2 e) on v_exp_f32 (two instructions; expf's range reduction
// and special-case selects take about twelve).  The rounding of the product
// adds a relative error of about |x| 2^-24: below 1e-6 for every argument
// whose result is not negligible against the others of its row.  Used by the
// matrix-core passes, whose vector-ALU work does not overlap their fp32
// matrix instructions.
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ __forceinline__ float softplusf(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }

// ------------------------------------------------------------------ prep
// The plain rows QV, KV, VV, A, B of 32 residues of one (b, h) per
// workgroup.  Threads walk the 4-float pieces of the rows, so that
// consecutive lanes read consecutive inputs and store consecutive addresses.
constexpr int kPrepRows = 32;
__global__ __launch_bounds__(256) void bw_prep_kernel(BwArgs a) {
  const BwLayout& L = a.L;
  const int h = blockIdx.y, b = blockIdx.z;
  const int n0 = blockIdx.x * kPrepRows, nr = min(kPrepRows, L.N - n0);
  if (b == 0 && blockIdx.x == 0 && h == 0 && threadIdx.x == 0) {
    for (int hh = 0; hh < L.H; ++hh)
      wsf(a, L.off_gam)[hh] = 0.5f * softplusf(a.wraw[hh]) * sqrtf(2.0f / (27.0f * (float)L.P));
  }
  const float sq = 1.0f / sqrtf(3.0f * (float)L.D), s3 = 1.0f / sqrtf(3.0f);
  const int RCz = L.R * L.Cz;
  // QV = [q / sqrt(3D) | w_pair zl / sqrt(3) | 0], KV = [k | zr | 0]
  const int k4 = L.DKp / 4;
  for (int x = threadIdx.x; x < nr * k4; x += 256) {
    const int rr = x / k4, c4 = x - rr * k4, n = n0 + rr;
    const size_t bn = (size_t)b * L.N + n, ri = rowidx(L, b, h, n);
    float qv[4], kv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 4 * c4 + e;
      if (c < L.D) {
        qv[e] = a.q[(bn * L.H + h) * L.D + c] * sq;
        kv[e] = a.k[(bn * L.H + h) * L.D + c];
      } else if (c < L.D + RCz) {
        const int idx = c - L.D, z = idx % L.Cz;
        qv[e] = a.wpair[h * L.Cz + z] * a.zl[bn * RCz + idx] * s3;
        kv[e] = a.zr[bn * RCz + idx];
      } else {
        qv[e] = kv[e] = 0.f;
      }
    }
    reinterpret_cast<float4*>(wsf(a, L.off_qv) + ri * L.DKp)[c4] = make_float4(qv[0], qv[1], qv[2], qv[3]);
    reinterpret_cast<float4*>(wsf(a, L.off_kv) + ri * L.DKp)[c4] = make_float4(kv[0], kv[1], kv[2], kv[3]);
  }
  // VV = [v | zr | T(v_points) relative to the block reference (t - c
  // first: exact) | 0]
  const int v4 = L.DVp / 4, pbase = L.Dv + RCz, pend = pbase + 3 * L.Q;
  for (int x = threadIdx.x; x < nr * v4; x += 256) {
    const int rr = x / v4, c4 = x - rr * v4, n = n0 + rr;
    const size_t bn = (size_t)b * L.N + n, ri = rowidx(L, b, h, n);
    float vv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 4 * c4 + e;
      if (c < L.Dv) {
        vv[e] = a.v[(bn * L.H + h) * L.Dv + c];
      } else if (c < pbase) {
        vv[e] = a.zr[bn * RCz + (c - L.Dv)];
      } else if (c < pend) {
        const int qq = (c - pbase) / 3, m = (c - pbase) - 3 * qq;
        const float* R = a.rot + bn * 9;
        const float* x3 = a.vp + ((bn * L.H + h) * L.Q + qq) * 3;
        const float3 cr = blk_ref(a, b, n);
        const float tc = a.tr[bn * 3 + m] - (m == 0 ? cr.x : (m == 1 ? cr.y : cr.z));
        vv[e] = R[m * 3 + 0] * x3[0] + R[m * 3 + 1] * x3[1] + R[m * 3 + 2] * x3[2] + tc;
      } else {
        vv[e] = 0.f;
      }
    }
    reinterpret_cast<float4*>(wsf(a, L.off_vv) + ri * L.DVp)[c4] = make_float4(vv[0], vv[1], vv[2], vv[3]);
  }
  // A = T(q_points), B = T(k_points), 16 coordinates each (zero past 3P)
  for (int x = threadIdx.x; x < nr * 4; x += 256) {
    const int rr = x >> 2, c4 = x & 3, n = n0 + rr;
    const size_t bn = (size_t)b * L.N + n, ri = rowidx(L, b, h, n);
    const float* R = a.rot + bn * 9;
    const float* t = a.tr + bn * 3;
    float qa[4], kb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 4 * c4 + e;
      qa[e] = kb[e] = 0.f;
      if (c < 3 * L.P) {
        const int p = c / 3, m = c - 3 * p;
        const float* xq = a.qp + ((bn * L.H + h) * L.P + p) * 3;
        const float* xk = a.kp + ((bn * L.H + h) * L.P + p) * 3;
        qa[e] = R[m * 3 + 0] * xq[0] + R[m * 3 + 1] * xq[1] + R[m * 3 + 2] * xq[2] + t[m];
        kb[e] = R[m * 3 + 0] * xk[0] + R[m * 3 + 1] * xk[1] + R[m * 3 + 2] * xk[2] + t[m];
      }
    }
    reinterpret_cast<float4*>(wsf(a, L.off_qa) + ri * 16)[c4] = make_float4(qa[0], qa[1], qa[2], qa[3]);
    reinterpret_cast<float4*>(wsf(a, L.off_kb) + ri * 16)[c4] = make_float4(kb[0], kb[1], kb[2], kb[3]);
  }
}

// ------------------------------------------------------------------ row passes
// Lane layout of the three pair passes: 256 threads = 64 rows x 4 parts;
// part = lane & 3 holds columns [part*4*NK4, (part+1)*4*NK4) of a DKp row,
// [part*4*NV4, ...) of a DVp row and coordinates [4 part, 4 part + 4) of the
// 16-wide point rows.

template <int NK4>
__device__ __forceinline__ void load_quarter(const float* row, int part, float4 (&out)[NK4]) {
  const float4* p = reinterpret_cast<const float4*>(row) + part * NK4;
#pragma unroll
  for (int u = 0; u < NK4; ++u) out[u] = p[u];
}

template <int NK4>
__device__ __forceinline__ float dot_quarter(const float4 (&x)[NK4], const float* row, int part) {
  const float4* p = reinterpret_cast<const float4*>(row) + part * NK4;
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < NK4; ++u) {
    const float4 y = p[u];
    s = fmaf(x[u].x, y.x, s);
    s = fmaf(x[u].y, y.y, s);
    s = fmaf(x[u].z, y.z, s);
    s = fmaf(x[u].w, y.w, s);
  }
  return s;
}

template <int NK4>
__device__ __forceinline__ void axpy_quarter(float4 (&acc)[NK4], float w, const float* row, int part) {
  const float4* p = reinterpret_cast<const float4*>(row) + part * NK4;
#pragma unroll
  for (int u = 0; u < NK4; ++u) {
    const float4 y = p[u];
    acc[u].x = fmaf(w, y.x, acc[u].x);
    acc[u].y = fmaf(w, y.y, acc[u].y);
    acc[u].z = fmaf(w, y.z, acc[u].z);
    acc[u].w = fmaf(w, y.w, acc[u].w);
  }
}

template <int NK4>
__device__ __forceinline__ void store_quarter(float* row, int part, const float4 (&x)[NK4]) {
  float4* p = reinterpret_cast<float4*>(row) + part * NK4;
#pragma unroll
  for (int u = 0; u < NK4; ++u) p[u] = x[u];
}

// logit of (own row, partner row) for this lane's part, summed over the quad
template <int NK4>
__device__ __forceinline__ float logit_q(const float4 (&own)[NK4], const float* prow, const float4 own_pt,
                                         const float* ppt, float gam, bool own_is_query, float& d2part) {
  float s = dot_quarter<NK4>(own, prow, 0);
  const float4 y = *reinterpret_cast<const float4*>(ppt);
  const float dx = own_is_query ? own_pt.x - y.x : y.x - own_pt.x;
  const float dy = own_is_query ? own_pt.y - y.y : y.y - own_pt.y;
  const float dz = own_is_query ? own_pt.z - y.z : y.z - own_pt.z;
  const float dw = own_is_query ? own_pt.w - y.w : y.w - own_pt.w;
  d2part = dx * dx + dy * dy + dz * dz + dw * dw;
  return quad_sum(s - gam * d2part);
}

// Forward: per query, O and the natural-log lse over the permitted keys.
template <int NK4, int NV4, int ROWS>
__global__ __launch_bounds__(4 * ROWS) void bw_fwd_kernel(BwArgs a) {
  const BwLayout& L = a.L;
  constexpr int KW = 16 * NK4, VW = 16 * NV4;
  __shared__ __align__(16) float sK[kBwTile][KW];
  __shared__ __align__(16) float sB[kBwTile][16];
  __shared__ __align__(16) float sV[kBwTile][VW];
  __shared__ float sM[kBwTile];
  const int tid = threadIdx.x, part = tid & 3, r = tid >> 2;
  const int h = blockIdx.y, b = blockIdx.z;
  const int i = blockIdx.x * ROWS + r;
  const bool qin = i < L.N;
  const int ic = qin ? i : L.N - 1;
  const size_t ri = rowidx(L, b, h, ic);
  const float gam = wsf(a, L.off_gam)[h];
  const bool mq = qin && a.mask[(size_t)b * L.N + ic] != 0;
  float4 qv[NK4];
  load_quarter<NK4>(wsf(a, L.off_qv) + ri * L.DKp, part, qv);
  const float4 qa = reinterpret_cast<const float4*>(wsf(a, L.off_qa) + ri * 16)[part];
  float4 o[NV4];
#pragma unroll
  for (int u = 0; u < NV4; ++u) o[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  float m = -INFINITY, l = 0.f;
  // sum_j p_ij (c_j - c_i): the key blocks' references relative to the query's
  const float3 cq = blk_ref(a, b, ic);
  float cx = 0.f, cy = 0.f, cz = 0.f;
  const uint8_t* pmrow = a.pmask ? a.pmask + ((size_t)b * L.N + ic) * L.N : nullptr;
  for (int j0 = 0; j0 < L.N; j0 += kBwTile) {
    __syncthreads();
    for (int e = tid; e < kBwTile * (KW / 4); e += 4 * ROWS) {
      const int jj = e / (KW / 4), c4 = e - jj * (KW / 4);
      const int j = min(j0 + jj, L.N - 1);
      reinterpret_cast<float4*>(&sK[jj][0])[c4] = reinterpret_cast<const float4*>(wsf(a, L.off_kv) + rowidx(L, b, h, j) * L.DKp)[c4];
    }
    for (int e = tid; e < kBwTile * (VW / 4); e += 4 * ROWS) {
      const int jj = e / (VW / 4), c4 = e - jj * (VW / 4);
      const int j = min(j0 + jj, L.N - 1);
      reinterpret_cast<float4*>(&sV[jj][0])[c4] = reinterpret_cast<const float4*>(wsf(a, L.off_vv) + rowidx(L, b, h, j) * L.DVp)[c4];
    }
    for (int e = tid; e < kBwTile * 4; e += 4 * ROWS) {
      const int jj = e >> 2, c4 = e & 3;
      const int j = min(j0 + jj, L.N - 1);
      reinterpret_cast<float4*>(&sB[jj][0])[c4] = reinterpret_cast<const float4*>(wsf(a, L.off_kb) + rowidx(L, b, h, j) * 16)[c4];
    }
    if (tid < kBwTile) {
      const int j = j0 + tid;
      sM[tid] = (j < L.N && a.mask[(size_t)b * L.N + j] != 0) ? 1.f : 0.f;
    }
    __syncthreads();
    const int nj = min(kBwTile, L.N - j0);
    const float3 ct = blk_ref(a, b, j0);
    const float dcx = ct.x - cq.x, dcy = ct.y - cq.y, dcz = ct.z - cq.z;
    for (int jj = 0; jj < nj; ++jj) {
      float d2;
      const float lg = logit_q<NK4>(qv, &sK[jj][part * 4 * NK4], qa, &sB[jj][part * 4], gam, true, d2);
      const bool ok = mq && sM[jj] != 0.f && (!pmrow || pmrow[j0 + jj] != 0);
      if (!ok) continue;
      if (lg > m) {
        const float c = expf(m - lg);
        l *= c;
        cx *= c;
        cy *= c;
        cz *= c;
#pragma unroll
        for (int u = 0; u < NV4; ++u) {
          o[u].x *= c;
          o[u].y *= c;
          o[u].z *= c;
          o[u].w *= c;
        }
        m = lg;
      }
      const float p = expf(lg - m);
      l += p;
      cx = fmaf(p, dcx, cx);
      cy = fmaf(p, dcy, cy);
      cz = fmaf(p, dcz, cz);
      axpy_quarter<NV4>(o, p, &sV[jj][0], part);
    }
  }
  if (!qin) return;
  const bool empty = !(l > 0.f);
  const float inv = empty ? 0.f : 1.f / l;
  // O' : the value points relative to the query's block reference
  const int pbase = L.Dv + L.R * L.Cz, pend = pbase + 3 * L.Q;
  const float cc[3] = {cx, cy, cz};
#pragma unroll
  for (int u = 0; u < NV4; ++u) {
    float* e4 = reinterpret_cast<float*>(&o[u]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int col = part * 4 * NV4 + 4 * u + e;
      const float add = (col >= pbase && col < pend) ? cc[(col - pbase) % 3] : 0.f;
      e4[e] = (e4[e] + add) * inv;
    }
  }
  store_quarter<NV4>(wsf(a, L.off_o) + ri * L.DVp, part, o);
  if (part == 0) wsf(a, L.off_lse)[ri] = empty ? -INFINITY : m + logf(l);
}

// dQ pass: per query, loop over all keys.
template <int NK4, int NV4, int ROWS>
__global__ __launch_bounds__(4 * ROWS) void bw_query_kernel(BwArgs a) {
  const BwLayout& L = a.L;
  constexpr int KW = 16 * NK4, VW = 16 * NV4;
  __shared__ __align__(16) float sK[kBwTile][KW];
  __shared__ __align__(16) float sB[kBwTile][16];
  __shared__ __align__(16) float sV[kBwTile][VW];
  __shared__ float sM[kBwTile];
  const int tid = threadIdx.x, part = tid & 3, r = tid >> 2;
  const int h = blockIdx.y, b = blockIdx.z;
  const int i = blockIdx.x * ROWS + r;
  const bool qin = i < L.N;
  const int ic = qin ? i : L.N - 1;
  const size_t ri = rowidx(L, b, h, ic);
  const float gam = wsf(a, L.off_gam)[h];
  const float lse = wsf(a, L.off_lse)[ri];
  const float dsum = wsf(a, L.off_dd)[ri];
  const float4 sv = reinterpret_cast<const float4*>(wsf(a, L.off_ds) + ri * 4)[0];
  const float3 cq = blk_ref(a, b, ic);
  const bool mq = qin && a.mask[(size_t)b * L.N + ic] != 0 && lse > -INFINITY;
  float4 qv[NK4], dq[NK4];
  load_quarter<NK4>(wsf(a, L.off_qv) + ri * L.DKp, part, qv);
  float4 dov[NV4];
  load_quarter<NV4>(wsf(a, L.off_do) + ri * L.DVp, part, dov);
  const float4 qa = reinterpret_cast<const float4*>(wsf(a, L.off_qa) + ri * 16)[part];
#pragma unroll
  for (int u = 0; u < NK4; ++u) dq[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 da = make_float4(0.f, 0.f, 0.f, 0.f);
  float dg = 0.f;
  const uint8_t* pmrow = a.pmask ? a.pmask + ((size_t)b * L.N + ic) * L.N : nullptr;
  for (int j0 = 0; j0 < L.N; j0 += kBwTile) {
    __syncthreads();
    for (int e = tid; e < kBwTile * (KW / 4); e += 4 * ROWS) {
      const int jj = e / (KW / 4), c4 = e - jj * (KW / 4);
      const int j = min(j0 + jj, L.N - 1);
      reinterpret_cast<float4*>(&sK[jj][0])[c4] = reinterpret_cast<const float4*>(wsf(a, L.off_kv) + rowidx(L, b, h, j) * L.DKp)[c4];
    }
    for (int e = tid; e < kBwTile * (VW / 4); e += 4 * ROWS) {
      const int jj = e / (VW / 4), c4 = e - jj * (VW / 4);
      const int j = min(j0 + jj, L.N - 1);
      reinterpret_cast<float4*>(&sV[jj][0])[c4] = reinterpret_cast<const float4*>(wsf(a, L.off_vv) + rowidx(L, b, h, j) * L.DVp)[c4];
    }
    for (int e = tid; e < kBwTile * 4; e += 4 * ROWS) {
      const int jj = e >> 2, c4 = e & 3;
      const int j = min(j0 + jj, L.N - 1);
      reinterpret_cast<float4*>(&sB[jj][0])[c4] = reinterpret_cast<const float4*>(wsf(a, L.off_kb) + rowidx(L, b, h, j) * 16)[c4];
    }
    if (tid < kBwTile) {
      const int j = j0 + tid;
      sM[tid] = (j < L.N && a.mask[(size_t)b * L.N + j] != 0) ? 1.f : 0.f;
    }
    __syncthreads();
    const int nj = min(kBwTile, L.N - j0);
    // Dsum'_i + S_i . (c_i - c_t) for this key block
    const float3 ct = blk_ref(a, b, j0);
    const float corr = fmaf(sv.x, cq.x - ct.x, fmaf(sv.y, cq.y - ct.y, fmaf(sv.z, cq.z - ct.z, dsum)));
    for (int jj = 0; jj < nj; ++jj) {
      float d2;
      const float lg = logit_q<NK4>(qv, &sK[jj][part * 4 * NK4], qa, &sB[jj][part * 4], gam, true, d2);
      const float dp = quad_sum(dot_quarter<NV4>(dov, &sV[jj][0], part));
      const bool ok = mq && sM[jj] != 0.f && (!pmrow || pmrow[j0 + jj] != 0);
      if (!ok) continue;
      const float p = expf(lg - lse);
      const float ds = p * (dp - corr);
      axpy_quarter<NK4>(dq, ds, &sK[jj][0], part);
      const float4 y = *reinterpret_cast<const float4*>(&sB[jj][part * 4]);
      const float w = -2.f * gam * ds;
      da.x = fmaf(w, qa.x - y.x, da.x);
      da.y = fmaf(w, qa.y - y.y, da.y);
      da.z = fmaf(w, qa.z - y.z, da.z);
      da.w = fmaf(w, qa.w - y.w, da.w);
      dg = fmaf(-ds, d2, dg);
    }
  }
  dg = quad_sum(dg);
  if (!qin) return;
  store_quarter<NK4>(wsf(a, L.off_dqv) + ri * L.DKp, part, dq);
  reinterpret_cast<float4*>(wsf(a, L.off_dqa) + ri * 16)[part] = da;
  if (part == 0) wsf(a, L.off_dgam)[ri] = dg;
}

// dK / dV pass: per key, loop over all queries.
// MODE 0 accumulates dKV and dB (needs dP, hence the key's VV quarter);
// MODE 1 accumulates dVV (needs only p); MODE 2 does both in one pass.  On
// large grids the two launches of modes 0 and 1 win (each holds few enough
// registers for two wavefronts per SIMD); on small grids the single pass does.
template <int NK4, int NV4, int ROWS, int MODE>
__global__ __launch_bounds__(4 * ROWS) void bw_key_kernel(BwArgs a) {
  const BwLayout& L = a.L;
  constexpr int KW = 16 * NK4, VW = 16 * NV4;
  __shared__ __align__(16) float sQ[kBwTile][KW];
  __shared__ __align__(16) float sA[kBwTile][16];
  __shared__ __align__(16) float sD[kBwTile][VW];
  __shared__ float sL[kBwTile], sS[kBwTile], sSx[kBwTile], sSy[kBwTile], sSz[kBwTile];
  __shared__ uint8_t sPM[kBwTile][ROWS];
  const int tid = threadIdx.x, part = tid & 3, r = tid >> 2;
  const int h = blockIdx.y, b = blockIdx.z;
  const int j = blockIdx.x * ROWS + r;
  const bool kin = j < L.N;
  const int jc = kin ? j : L.N - 1;
  const size_t rj = rowidx(L, b, h, jc);
  const float gam = wsf(a, L.off_gam)[h];
  const bool mk = kin && a.mask[(size_t)b * L.N + jc] != 0;
  const float3 ckey = blk_ref(a, b, jc);
  constexpr bool kDS = MODE != 1, kDV = MODE != 0;
  float4 kv[NK4], dk[kDS ? NK4 : 1];
  load_quarter<NK4>(wsf(a, L.off_kv) + rj * L.DKp, part, kv);
  float4 vv[kDS ? NV4 : 1], dv[kDV ? NV4 : 1];
  if constexpr (kDS) load_quarter<NV4>(wsf(a, L.off_vv) + rj * L.DVp, part, vv);
  const float4 kb = reinterpret_cast<const float4*>(wsf(a, L.off_kb) + rj * 16)[part];
  if constexpr (kDS) {
#pragma unroll
    for (int u = 0; u < NK4; ++u) dk[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if constexpr (kDV) {
#pragma unroll
    for (int u = 0; u < NV4; ++u) dv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float4 db = make_float4(0.f, 0.f, 0.f, 0.f);
  const int kbase = blockIdx.x * ROWS;
  for (int i0 = 0; i0 < L.N; i0 += kBwTile) {
    __syncthreads();
    for (int e = tid; e < kBwTile * (KW / 4); e += 4 * ROWS) {
      const int ii = e / (KW / 4), c4 = e - ii * (KW / 4);
      const int i = min(i0 + ii, L.N - 1);
      reinterpret_cast<float4*>(&sQ[ii][0])[c4] = reinterpret_cast<const float4*>(wsf(a, L.off_qv) + rowidx(L, b, h, i) * L.DKp)[c4];
    }
    for (int e = tid; e < kBwTile * (VW / 4); e += 4 * ROWS) {
      const int ii = e / (VW / 4), c4 = e - ii * (VW / 4);
      const int i = min(i0 + ii, L.N - 1);
      reinterpret_cast<float4*>(&sD[ii][0])[c4] = reinterpret_cast<const float4*>(wsf(a, L.off_do) + rowidx(L, b, h, i) * L.DVp)[c4];
    }
    for (int e = tid; e < kBwTile * 4; e += 4 * ROWS) {
      const int ii = e >> 2, c4 = e & 3;
      const int i = min(i0 + ii, L.N - 1);
      reinterpret_cast<float4*>(&sA[ii][0])[c4] = reinterpret_cast<const float4*>(wsf(a, L.off_qa) + rowidx(L, b, h, i) * 16)[c4];
    }
    if (tid < kBwTile) {
      const int i = i0 + tid;
      const int icl = min(i, L.N - 1);
      const float lse = wsf(a, L.off_lse)[rowidx(L, b, h, icl)];
      const bool ok = i < L.N && a.mask[(size_t)b * L.N + icl] != 0 && lse > -INFINITY;
      sL[tid] = ok ? lse : INFINITY;  // +inf marks a query that takes no key
      sS[tid] = wsf(a, L.off_dd)[rowidx(L, b, h, icl)];
      const float4 sv = reinterpret_cast<const float4*>(wsf(a, L.off_ds) + rowidx(L, b, h, icl) * 4)[0];
      sSx[tid] = sv.x;
      sSy[tid] = sv.y;
      sSz[tid] = sv.z;
    }
    for (int e = tid; e < kBwTile * ROWS; e += 4 * ROWS) {
      const int ii = e / ROWS, jj = e - ii * ROWS;
      const int i = min(i0 + ii, L.N - 1), jn = min(kbase + jj, L.N - 1);
      sPM[ii][jj] = a.pmask ? a.pmask[((size_t)b * L.N + i) * L.N + jn] : (uint8_t)1;
    }
    __syncthreads();
    const int ni = min(kBwTile, L.N - i0);
    // the query block's reference relative to this key's
    const float3 cqb = blk_ref(a, b, i0);
    const float dcx = cqb.x - ckey.x, dcy = cqb.y - ckey.y, dcz = cqb.z - ckey.z;
    for (int ii = 0; ii < ni; ++ii) {
      float d2;
      const float lg = logit_q<NK4>(kv, &sQ[ii][part * 4 * NK4], kb, &sA[ii][part * 4], gam, false, d2);
      if constexpr (kDS) {
        const float dp = quad_sum(dot_quarter<NV4>(vv, &sD[ii][0], part));
        const bool ok = mk && sL[ii] < INFINITY && sPM[ii][r] != 0;
        if (!ok) continue;
        const float p = expf(lg - sL[ii]);
        const float corr = fmaf(sSx[ii], dcx, fmaf(sSy[ii], dcy, fmaf(sSz[ii], dcz, sS[ii])));
        const float ds = p * (dp - corr);
        axpy_quarter<NK4>(dk, ds, &sQ[ii][0], part);
        if constexpr (kDV) axpy_quarter<NV4>(dv, p, &sD[ii][0], part);
        const float4 x = *reinterpret_cast<const float4*>(&sA[ii][part * 4]);
        const float w = 2.f * gam * ds;
        db.x = fmaf(w, x.x - kb.x, db.x);
        db.y = fmaf(w, x.y - kb.y, db.y);
        db.z = fmaf(w, x.z - kb.z, db.z);
        db.w = fmaf(w, x.w - kb.w, db.w);
      } else {
        const bool ok = mk && sL[ii] < INFINITY && sPM[ii][r] != 0;
        if (!ok) continue;
        axpy_quarter<NV4>(dv, expf(lg - sL[ii]), &sD[ii][0], part);
      }
    }
  }
  if (!kin) return;
  if constexpr (kDS) {
    store_quarter<NK4>(wsf(a, L.off_dkv) + rj * L.DKp, part, dk);
    reinterpret_cast<float4*>(wsf(a, L.off_dkb) + rj * 16)[part] = db;
  }
  if constexpr (kDV) store_quarter<NV4>(wsf(a, L.off_dvv) + rj * L.DVp, part, dv);
}

// ------------------------------------------------------------------ matrix-core forward recomputation
// The same O and lse on fp32 matrix cores (v_mfma_f32_32x32x2f32, full fp32
// operands).  A workgroup of four wavefronts takes 128 queries of one
// (b, h); each wavefront owns 32 queries and walks key tiles of 32 staged in
// LDS.  S^T (32 keys x 32 queries) = KV_t QV^T on the matrix cores (DKp/2
// steps of K = 2); the point term -gamma sum |A - B|^2 is added per element
// on the vector ALU from differences (an expanded form on fp32 matrix cores
// loses ~1e-4 of a logit to cancellation), overlapping the matrix work.  The
// accumulator gives each lane one query and 16 keys, so the softmax row work
// stays in the lane (and its partner 32 lanes away); the running maximum is
// raised lazily.  O^T (32 value columns x 32 queries per block) += VV_t^T P^T
// takes the probabilities straight from the accumulator registers: at step s
// lane half h supplies key kappa(s, h) = 8 (s / 4) + 4 h + s % 4, the key its
// register s holds, and reads the value row of that key.
constexpr int kBwKT = 32;  // keys per tile of the matrix-core passes

// Partner rows [*lo, *hi) of inner-loop range sp of the matrix-core pair
// passes: the N / kBwKT partner tiles split into psplit ranges of whole tiles.
__device__ __forceinline__ void split_range(const BwLayout& L, int sp, int* lo, int* hi) {
  const int nt = (L.N + kBwKT - 1) / kBwKT;
  *lo = (int)((long)nt * sp / L.psplit) * kBwKT;
  *hi = min(L.N, (int)((long)nt * (sp + 1) / L.psplit) * kBwKT);
}

// Merge the psplit partial recomputations of a row (one thread per four
// columns): weights e^(m_s - M) over the ranges with a nonzero sum, O' the
// merged values (plus the merged reference offsets on the value points) over
// the merged sum, lse = M + log(sum).  Rows without a permitted key get
// zeros and -inf, as in the unsplit pass.
__global__ __launch_bounds__(256) void bw_merge_o_kernel(BwArgs a) {
  const BwLayout& L = a.L;
  const size_t rows = (size_t)L.B * L.H * L.N;
  const int n4 = L.DVp / 4, REC = L.DVp + 8;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * n4) return;
  const size_t r = idx / n4;
  const int c4 = (int)(idx - r * n4);
  const float* part = wsf(a, L.off_opart);
  float M = -INFINITY;
  for (int s = 0; s < L.psplit; ++s) {
    const float* rec = part + ((size_t)s * rows + r) * REC;
    if (rec[L.DVp + 1] > 0.f) M = fmaxf(M, rec[L.DVp]);
  }
  float lsum = 0.f, cc[3] = {0.f, 0.f, 0.f}, o[4] = {0.f, 0.f, 0.f, 0.f};
  if (M > -INFINITY) {
    for (int s = 0; s < L.psplit; ++s) {
      const float* rec = part + ((size_t)s * rows + r) * REC;
      const float ls = rec[L.DVp + 1];
      if (!(ls > 0.f)) continue;  // an empty range holds no values
      const float wgt = expf(rec[L.DVp] - M);
      lsum = fmaf(wgt, ls, lsum);
      cc[0] = fmaf(wgt, rec[L.DVp + 2], cc[0]);
      cc[1] = fmaf(wgt, rec[L.DVp + 3], cc[1]);
      cc[2] = fmaf(wgt, rec[L.DVp + 4], cc[2]);
      const float4 v = reinterpret_cast<const float4*>(rec)[c4];
      o[0] = fmaf(wgt, v.x, o[0]); o[1] = fmaf(wgt, v.y, o[1]); o[2] = fmaf(wgt, v.z, o[2]); o[3] = fmaf(wgt, v.w, o[3]);
    }
  }
  const bool empty = !(lsum > 0.f);
  const float inv = empty ? 0.f : 1.f / lsum;
  const int pbase = L.Dv + L.R * L.Cz, pend = pbase + 3 * L.Q;
  float e4[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int col = 4 * c4 + e;
    const float add = (col >= pbase && col < pend) ? cc[(col - pbase) % 3] : 0.f;
    e4[e] = (o[e] + add) * inv;
  }
  reinterpret_cast<float4*>(wsf(a, L.off_o) + r * L.DVp)[c4] = make_float4(e4[0], e4[1], e4[2], e4[3]);
  if (c4 == 0) wsf(a, L.off_lse)[r] = empty ? -INFINITY : M + logf(lsum);
}

// out[i] += sum of the ns slabs extra[z n + i] (the partial sums of the
// inner-loop ranges 1 .. psplit-1 of a pair pass).
__global__ __launch_bounds__(256) void bw_add_slabs_kernel(float* out, const float* extra, size_t n, int ns) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v = out[i];
  for (int z = 0; z < ns; ++z) v += extra[(size_t)z * n + i];
  out[i] = v;
}

__device__ __forceinline__ int kappa(int s, int h) { return 8 * (s >> 2) + 4 * h + (s & 3); }

// One tile of 32 rows of F4 float4 pieces, staged through registers by the
// 256 threads of a workgroup: `load` issues every global load of the tile at
// once (so a tile costs one memory round trip, not one per loop trip; and a
// tile can be loaded one step ahead while the current one is in use),
// `store` hands each piece to the caller's LDS write.  Rows past the end
// repeat row N - 1; pieces at or past `valid` read as zero.  Every load
// address is clamped into the rows and pieces of the tensor.
template <int F4>
struct Tile4 {
  static constexpr int K = (32 * F4 + 255) / 256;
  float4 v[K];
  __device__ __forceinline__ void load(const float* base, int stride, int j0, int N, int tid, int valid) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int e = min(tid + 256 * k, 32 * F4 - 1);
      const int jj = e / F4, c4 = e - jj * F4;
      const int j = min(j0 + jj, N - 1);
      // a 32-bit index from the uniform base (scalar base + vector offset)
      const uint32_t idx = (uint32_t)j * (uint32_t)(stride >> 2) + (uint32_t)min(c4, valid - 1);
      const float4 x = reinterpret_cast<const float4*>(base)[idx];
      v[k] = c4 < valid ? x : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  template <typename Fn>
  __device__ __forceinline__ void store(int tid, Fn fn) const {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int e = tid + 256 * k;
      if (e < 32 * F4) {
        const int jj = e / F4, c4 = e - jj * F4;
        fn(jj, c4, v[k]);
      }
    }
  }
};

// Permission bits of one 32-key tile for a query lane: bit r for key
// kappa(r, hf) of the tile (keys past the chain's end, masked keys, and with
// a pair mask the pairs it removes are 0).  Computed once per tile so that
// the per-element work has no branches; the pair-mask loads of a tile go out
// together (their index clamped into the row; the clamped ones are masked
// by the key bits).
__device__ __forceinline__ uint32_t tile_permitted(const float* sM, int nj, const uint8_t* pmrow, int j0, int N,
                                                   int hf) {
  uint32_t okm = 0u;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int kk = kappa(r, hf);
    okm |= (kk < nj && sM[kk] != 0.f) ? (1u << r) : 0u;
  }
  if (pmrow) {
    uint32_t pm = 0u;
#pragma unroll
    for (int r = 0; r < 16; ++r) pm |= pmrow[min(j0 + kappa(r, hf), N - 1)] != 0 ? (1u << r) : 0u;
    okm &= pm;
  }
  return okm;
}

template <int DKH, int NVB, int P3C>
__global__ __launch_bounds__(256) void bw_fwd_mfma_kernel(BwArgs a) {
  const BwLayout& L = a.L;
  constexpr int DKp = 2 * DKH;
  constexpr int VW = 32 * NVB;  // value columns staged (DVp padded with zeros)
  // Pitches: KV is written transposed by threads walking its columns, so a
  // row pitch of 33 words spreads consecutive columns over the banks (32
  // would put them all in one); the value rows are read at rows kappa(s, 0)
  // and kappa(s, 1) = +4 by the two halves of a wavefront, so a pitch of
  // VW + 8 words (4 (VW + 8) = 32 mod 64) gives the halves different banks.
  constexpr int VWP = VW + 8;
  __shared__ float sKT[DKp][kBwKT + 1];
  __shared__ __align__(16) float sBp[kBwKT][16];
  __shared__ __align__(16) float sV[kBwKT][VWP];
  __shared__ float sM[kBwKT];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int qt = blockIdx.x / L.psplit, sp = blockIdx.x - qt * L.psplit;
  const int q = qt * 128 + 32 * w + l32;
  const bool qin = q < L.N;
  const int qc = qin ? q : L.N - 1;
  const size_t rq = rowidx(L, b, h, qc);
  const float gam = wsf(a, L.off_gam)[h];
  const bool mq = qin && a.mask[(size_t)b * L.N + qc] != 0;
  int jb, je;
  split_range(L, sp, &jb, &je);
  // query operand: QV[q][s + DKH hf], s < DKH; point coordinates 8 hf .. +7
  float qv[DKH];
  {
    const float* row = wsf(a, L.off_qv) + rq * L.DKp + DKH * hf;
#pragma unroll
    for (int s4 = 0; s4 < DKH / 4; ++s4) {
      const float4 v = reinterpret_cast<const float4*>(row)[s4];
      qv[4 * s4] = v.x;
      qv[4 * s4 + 1] = v.y;
      qv[4 * s4 + 2] = v.z;
      qv[4 * s4 + 3] = v.w;
    }
#pragma unroll
    for (int s = 4 * (DKH / 4); s < DKH; ++s) qv[s] = row[s];
  }
  float qa[16];  // this lane's query points (both halves of the pair hold all 16)
  {
    const float* row = wsf(a, L.off_qa) + rq * 16;
#pragma unroll
    for (int u = 0; u < 16; ++u) qa[u] = row[u];
  }
  f32x16_t oacc[NVB];
#pragma unroll
  for (int v = 0; v < NVB; ++v) oacc[v] = f32x16_t{};
  float m = -INFINITY, lsum = 0.f;
  // sum_j p_ij (c_j - c_i) over this lane's keys (the wavefront's 32 queries
  // are one block: one reference)
  const float3 cq = blk_ref(a, b, qc);
  float cx = 0.f, cy = 0.f, cz = 0.f;
  const uint8_t* pmrow = a.pmask ? a.pmask + ((size_t)b * L.N + qc) * L.N : nullptr;
  // key tiles: KV (transposed into LDS), VV rows (zero past DVp), centred key
  // points, key mask; the next tile's loads are in flight during the
  // products of the current one
  const float* kvb = wsf(a, L.off_kv) + rowidx(L, b, h, 0) * L.DKp;
  const float* vvb = wsf(a, L.off_vv) + rowidx(L, b, h, 0) * L.DVp;
  const float* kbb = wsf(a, L.off_kb) + rowidx(L, b, h, 0) * 16;
  Tile4<DKp / 4> tk;
  Tile4<VW / 4> tv;
  Tile4<4> tb;
  float tm = 0.f;
  auto issue = [&](int j0) {
    tk.load(kvb, L.DKp, j0, L.N, tid, DKp / 4);
    tv.load(vvb, L.DVp, j0, L.N, tid, L.DVp / 4);
    tb.load(kbb, 16, j0, L.N, tid, 4);
    const int j = min(j0 + (tid & 31), L.N - 1);
    tm = (j0 + (tid & 31) < L.N && a.mask[(size_t)b * L.N + j] != 0) ? 1.f : 0.f;
  };
  issue(jb);
  for (int j0 = jb; j0 < je; j0 += kBwKT) {
    __syncthreads();
    tk.store(tid, [&](int jj, int c4, float4 v) {
      sKT[4 * c4][jj] = v.x;
      sKT[4 * c4 + 1][jj] = v.y;
      sKT[4 * c4 + 2][jj] = v.z;
      sKT[4 * c4 + 3][jj] = v.w;
    });
    tv.store(tid, [&](int jj, int c4, float4 v) { reinterpret_cast<float4*>(&sV[jj][0])[c4] = v; });
    tb.store(tid, [&](int jj, int c4, float4 v) { reinterpret_cast<float4*>(&sBp[jj][0])[c4] = v; });
    if (tid < kBwKT) sM[tid] = tm;
    if (j0 + kBwKT < je) issue(j0 + kBwKT);
    __syncthreads();
    // S^T: A = key tile (row = key l32, k = hf), B = query (k = hf, column = query l32)
    f32x16_t sacc = f32x16_t{};
#pragma unroll
    for (int s = 0; s < DKH; ++s)
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(sKT[s + DKH * hf][l32], qv[s], sacc, 0, 0, 0);
    // logits of this lane's 16 keys (point term from differences), masks, tile maximum
    float lg[16];
    float tmax = -INFINITY;
    const int nj = min(kBwKT, L.N - j0);
    const uint32_t okm = mq ? tile_permitted(sM, nj, pmrow, j0, L.N, hf) : 0u;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = kappa(r, hf);
      float d2 = 0.f;
#pragma unroll
      for (int c4 = 0; c4 < P3C / 4; ++c4) {
        const float4 y = reinterpret_cast<const float4*>(&sBp[kk][0])[c4];
        const float dx = qa[4 * c4] - y.x, dy = qa[4 * c4 + 1] - y.y, dz = qa[4 * c4 + 2] - y.z, dw = qa[4 * c4 + 3] - y.w;
        d2 += dx * dx + dy * dy + dz * dz + dw * dw;
      }
      lg[r] = ((okm >> r) & 1u) ? sacc[r] - gam * d2 : -INFINITY;
      tmax = fmaxf(tmax, lg[r]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    if (tmax > m + 5.0f) {  // raise the running maximum (lazily: values up to e^5 are fine)
      const float c = exp_fast(m - tmax);
      lsum *= c;
      cx *= c;
      cy *= c;
      cz *= c;
#pragma unroll
      for (int v = 0; v < NVB; ++v) oacc[v] *= c;
      m = tmax;
    }
    float pr[16];
    float tsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pr[r] = lg[r] > -INFINITY ? exp_fast(lg[r] - m) : 0.f;
      tsum += pr[r];
    }
    lsum += tsum;
    {
      const float3 ct = blk_ref(a, b, j0);
      cx = fmaf(tsum, ct.x - cq.x, cx);
      cy = fmaf(tsum, ct.y - cq.y, cy);
      cz = fmaf(tsum, ct.z - cq.z, cz);
    }
    // O^T += VV^T P^T
#pragma unroll
    for (int v = 0; v < NVB; ++v)
#pragma unroll
      for (int s = 0; s < 16; ++s)
        oacc[v] = __builtin_amdgcn_mfma_f32_32x32x2f32(sV[kappa(s, hf)][32 * v + l32], pr[s], oacc[v], 0, 0, 0);
  }
  lsum += __shfl_xor(lsum, 32);
  cx += __shfl_xor(cx, 32);
  cy += __shfl_xor(cy, 32);
  cz += __shfl_xor(cz, 32);
  if (!qin) return;
  if (L.psplit > 1) {
    // partial result of this key range: unnormalised O (value points without
    // the reference offset), then m, the sum, and the offset sums
    float* rec = wsf(a, L.off_opart) + ((size_t)sp * L.B * L.H * L.N + rq) * (L.DVp + 8);
#pragma unroll
    for (int v = 0; v < NVB; ++v)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 32 * v + 8 * g + 4 * hf;
        if (c < L.DVp)
          *reinterpret_cast<float4*>(rec + c) =
              make_float4(oacc[v][4 * g], oacc[v][4 * g + 1], oacc[v][4 * g + 2], oacc[v][4 * g + 3]);
      }
    if (hf == 0) {
      *reinterpret_cast<float4*>(rec + L.DVp) = make_float4(m, lsum, cx, cy);
      rec[L.DVp + 4] = cz;
    }
    return;
  }
  const bool empty = !(lsum > 0.f);
  const float inv = empty ? 0.f : 1.f / lsum;
  // O' : the value points relative to the query's block reference
  const int pbase = L.Dv + L.R * L.Cz, pend = pbase + 3 * L.Q;
  const float cc[3] = {cx, cy, cz};
  float* orow = wsf(a, L.off_o) + rq * L.DVp;
#pragma unroll
  for (int v = 0; v < NVB; ++v)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = 32 * v + 8 * g + 4 * hf;
      if (c < L.DVp) {
        float e4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = c + e;
          const float add = (col >= pbase && col < pend) ? cc[(col - pbase) % 3] : 0.f;
          e4[e] = (oacc[v][4 * g + e] + add) * inv;
        }
        *reinterpret_cast<float4*>(orow + c) = make_float4(e4[0], e4[1], e4[2], e4[3]);
      }
    }
  if (hf == 0) wsf(a, L.off_lse)[rq] = empty ? -INFINITY : m + logf(lsum);
}

// ------------------------------------------------------------------ matrix-core query pass
// dQV, dA and the per-row d gamma sums on fp32 matrix cores (standard
// widths).  Same work split as the matrix-core recomputation: four
// wavefronts x 32 queries of one (b, h), key tiles of 32 in LDS.  Per tile:
//   S^T  = KV_t QV^T and dP^T = VV_t dO^T   (their K-steps interleaved, so
//                                            that the two chains of dependent
//                                            MFMAs overlap)
//   p = exp(S - gamma |A - B|^2 - lse), dS = p (dP - Dsum)   vector ALU, the
//   point term from coordinate differences as in the recomputation, with
//   dA += -2 gamma dS (A - B) and dgamma_i += -dS |A - B|^2 per lane
//   dQV^T += KV_t^T dS^T                     dS straight from the accumulator
//                                            layout (lane half h supplies
//                                            key kappa(s, h) at step s)
// KV and VV are staged transposed with a pitch of 33 floats, so that both the
// row reads (S, dP: one key per lane) and the column reads (dQV: one feature
// per lane) are free of bank conflicts.
template <int DKH, int DVH, int NKB, int P3C>
__global__ __launch_bounds__(256) void bw_query_mfma_kernel(BwArgs a) {
  const BwLayout& L = a.L;
  constexpr int DKp = 2 * DKH, DVp = 2 * DVH;
  static_assert(32 * NKB >= DKp, "dQV blocks cover the key row");
  // row-major tiles; the pitches (floats) make 16-byte reads of 8 consecutive
  // lanes' rows fall on distinct banks, and the key rows run to 32 NKB columns
  // so that the dQV blocks read zeros past DKp
  constexpr int KPI = 32 * NKB + 4, VPI = DVp + 4, QPI = DKp + 4;
  __shared__ __align__(16) float sK[kBwKT][KPI];
  __shared__ __align__(16) float sV[kBwKT][VPI];
  __shared__ __align__(16) float sBp[kBwKT][16];
  __shared__ float sM[kBwKT];
  __shared__ __align__(16) float sQ[4][32][QPI];  // each wavefront's 32 query rows QV
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int qt = blockIdx.x / L.psplit, sp = blockIdx.x - qt * L.psplit;
  const int q = qt * 128 + 32 * w + l32;
  const bool qin = q < L.N;
  const int qc = qin ? q : L.N - 1;
  const size_t rq = rowidx(L, b, h, qc);
  const float gam = wsf(a, L.off_gam)[h];
  const float lse = wsf(a, L.off_lse)[rq];
  int jb, je;
  split_range(L, sp, &jb, &je);
  const float dsum = wsf(a, L.off_dd)[rq];
  const float4 sv = reinterpret_cast<const float4*>(wsf(a, L.off_ds) + rq * 4)[0];
  const float3 cq = blk_ref(a, b, qc);
  const bool mq = qin && a.mask[(size_t)b * L.N + qc] != 0 && lse > -INFINITY;
  // key-row columns past DKp read zeros (the tile copies never write them)
  for (int e = tid; e < kBwKT * (KPI - DKp); e += 256) sK[e / (KPI - DKp)][DKp + e % (KPI - DKp)] = 0.f;
  // B operands: QV[q][s + DKH hf] from LDS, dO[q][s + DVH hf] in registers
  for (int e = lane; e < 32 * (DKp / 4); e += 64) {
    const int qq = e / (DKp / 4), c4 = e - qq * (DKp / 4);
    const int qr = min(qt * 128 + 32 * w + qq, L.N - 1);
    const float4 v = reinterpret_cast<const float4*>(wsf(a, L.off_qv) + rowidx(L, b, h, qr) * L.DKp)[c4];
    *reinterpret_cast<float4*>(&sQ[w][qq][4 * c4]) = v;
  }
  const float* qrow = &sQ[w][l32][DKH * hf];
  float dov[DVH];
  {
    const float* drow = wsf(a, L.off_do) + rq * L.DVp + DVH * hf;
#pragma unroll
    for (int s4 = 0; s4 < DVH / 4; ++s4) {
      const float4 v = reinterpret_cast<const float4*>(drow)[s4];
      dov[4 * s4] = v.x; dov[4 * s4 + 1] = v.y; dov[4 * s4 + 2] = v.z; dov[4 * s4 + 3] = v.w;
    }
  }
  float qa[P3C];  // coordinates past 3P are zero on both sides
  {
    const float* row = wsf(a, L.off_qa) + rq * 16;
#pragma unroll
    for (int u = 0; u < P3C; ++u) qa[u] = row[u];
  }
  f32x16_t dq[NKB];
#pragma unroll
  for (int c = 0; c < NKB; ++c) dq[c] = f32x16_t{};
  float da[P3C];
#pragma unroll
  for (int u = 0; u < P3C; ++u) da[u] = 0.f;
  float dg = 0.f;
  const uint8_t* pmrow = a.pmask ? a.pmask + ((size_t)b * L.N + qc) * L.N : nullptr;
  const float* kvb = wsf(a, L.off_kv) + rowidx(L, b, h, 0) * L.DKp;
  const float* vvb = wsf(a, L.off_vv) + rowidx(L, b, h, 0) * L.DVp;
  const float* kbb = wsf(a, L.off_kb) + rowidx(L, b, h, 0) * 16;
  // key tiles: the next tile's loads are in flight during the products of
  // the current one
  Tile4<4> tb;
  Tile4<DKp / 4> tk;
  Tile4<DVp / 4> tv;
  float tm = 0.f;
  auto issue = [&](int j0) {
    tb.load(kbb, 16, j0, L.N, tid, 4);
    tk.load(kvb, L.DKp, j0, L.N, tid, DKp / 4);
    tv.load(vvb, L.DVp, j0, L.N, tid, DVp / 4);
    const int jm = min(j0 + (tid & 31), L.N - 1);
    tm = (j0 + (tid & 31) < L.N && a.mask[(size_t)b * L.N + jm] != 0) ? 1.f : 0.f;
  };
  if (jb < je) issue(jb);
  for (int j0 = jb; j0 < je; j0 += kBwKT) {
    __syncthreads();
    tb.store(tid, [&](int jj, int c4, float4 v) { reinterpret_cast<float4*>(&sBp[jj][0])[c4] = v; });
    tk.store(tid, [&](int jj, int c4, float4 v) { *reinterpret_cast<float4*>(&sK[jj][4 * c4]) = v; });
    tv.store(tid, [&](int jj, int c4, float4 v) { *reinterpret_cast<float4*>(&sV[jj][4 * c4]) = v; });
    if (tid < kBwKT) sM[tid] = tm;
    if (j0 + kBwKT < je) issue(j0 + kBwKT);
    __syncthreads();
    // S and dP steps interleaved: two independent chains of dependent MFMAs
    f32x16_t sa = f32x16_t{}, pa = f32x16_t{};
    {
      // four K-steps per 16-byte read of the key row (A) and the query row (B)
      const float* ka = &sK[l32][DKH * hf];
      const float* va = &sV[l32][DVH * hf];
#pragma unroll
      for (int s4 = 0; s4 < (DKH > DVH ? DKH : DVH) / 4; ++s4) {
        if (4 * s4 < DKH) {
          const float4 x = *reinterpret_cast<const float4*>(ka + 4 * s4);
          const float4 y = *reinterpret_cast<const float4*>(qrow + 4 * s4);
          sa = __builtin_amdgcn_mfma_f32_32x32x2f32(x.x, y.x, sa, 0, 0, 0);
          sa = __builtin_amdgcn_mfma_f32_32x32x2f32(x.y, y.y, sa, 0, 0, 0);
          sa = __builtin_amdgcn_mfma_f32_32x32x2f32(x.z, y.z, sa, 0, 0, 0);
          sa = __builtin_amdgcn_mfma_f32_32x32x2f32(x.w, y.w, sa, 0, 0, 0);
        }
        if (4 * s4 < DVH) {
          const float4 x = *reinterpret_cast<const float4*>(va + 4 * s4);
          pa = __builtin_amdgcn_mfma_f32_32x32x2f32(x.x, dov[4 * s4], pa, 0, 0, 0);
          pa = __builtin_amdgcn_mfma_f32_32x32x2f32(x.y, dov[4 * s4 + 1], pa, 0, 0, 0);
          pa = __builtin_amdgcn_mfma_f32_32x32x2f32(x.z, dov[4 * s4 + 2], pa, 0, 0, 0);
          pa = __builtin_amdgcn_mfma_f32_32x32x2f32(x.w, dov[4 * s4 + 3], pa, 0, 0, 0);
        }
      }
    }
    const int nj = min(kBwKT, L.N - j0);
    // Dsum'_i + S_i . (c_i - c_t) for this key block
    const float3 ct = blk_ref(a, b, j0);
    const float corr = fmaf(sv.x, cq.x - ct.x, fmaf(sv.y, cq.y - ct.y, fmaf(sv.z, cq.z - ct.z, dsum)));
    float ds[16];
    const uint32_t okm = mq ? tile_permitted(sM, nj, pmrow, j0, L.N, hf) : 0u;
    // dS first (the coordinate differences recomputed below rather than held:
    // sixteen keys' differences would not fit beside the accumulators)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = kappa(r, hf);
      float d2 = 0.f;
#pragma unroll
      for (int c4 = 0; c4 < P3C / 4; ++c4) {
        const float4 y = reinterpret_cast<const float4*>(&sBp[kk][0])[c4];
        const float dx = qa[4 * c4] - y.x, dy = qa[4 * c4 + 1] - y.y, dz = qa[4 * c4 + 2] - y.z, dw = qa[4 * c4 + 3] - y.w;
        d2 += dx * dx + dy * dy + dz * dz + dw * dw;
      }
      const float p = ((okm >> r) & 1u) ? exp_fast(sa[r] - gam * d2 - lse) : 0.f;
      ds[r] = p * (pa[r] - corr);
      dg = fmaf(-ds[r], d2, dg);
    }
    // dQV^T += KV_t^T dS^T, with the point term dA (vector ALU, independent
    // of these products) a piece after each matrix instruction
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int kk = kappa(s, hf);
#pragma unroll
      for (int c = 0; c < NKB; ++c) {
        dq[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(sK[kk][32 * c + l32], ds[s], dq[c], 0, 0, 0);
        if (c < P3C / 4) {
          const float4 y = reinterpret_cast<const float4*>(&sBp[kk][0])[c];
          da[4 * c] = fmaf(ds[s], qa[4 * c] - y.x, da[4 * c]);
          da[4 * c + 1] = fmaf(ds[s], qa[4 * c + 1] - y.y, da[4 * c + 1]);
          da[4 * c + 2] = fmaf(ds[s], qa[4 * c + 2] - y.z, da[4 * c + 2]);
          da[4 * c + 3] = fmaf(ds[s], qa[4 * c + 3] - y.w, da[4 * c + 3]);
        }
      }
    }
  }
  // the two halves of the wavefront hold the same queries' two halves of each tile
#pragma unroll
  for (int u = 0; u < P3C; ++u) da[u] += __shfl_xor(da[u], 32);
  dg += __shfl_xor(dg, 32);
  if (!qin) return;
  // key range sp > 0 writes its partial sums to a slab of its own
  const size_t rows = (size_t)L.B * L.H * L.N, xs = (size_t)(sp - 1);
  float* orow = (sp == 0 ? wsf(a, L.off_dqv) : wsf(a, L.off_xqv) + xs * rows * L.DKp) + rq * L.DKp;
#pragma unroll
  for (int c = 0; c < NKB; ++c)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int f = 32 * c + 8 * g + 4 * hf;
      if (f < DKp)
        *reinterpret_cast<float4*>(orow + f) = make_float4(dq[c][4 * g], dq[c][4 * g + 1], dq[c][4 * g + 2], dq[c][4 * g + 3]);
    }
  if (hf == 0) {
    float* arow = (sp == 0 ? wsf(a, L.off_dqa) : wsf(a, L.off_xqa) + xs * rows * 16) + rq * 16;
#pragma unroll
    for (int u4 = 0; u4 < 4; ++u4) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (4 * u4 < P3C)
        v = make_float4(-2.f * gam * da[4 * u4], -2.f * gam * da[4 * u4 + 1], -2.f * gam * da[4 * u4 + 2],
                        -2.f * gam * da[4 * u4 + 3]);
      reinterpret_cast<float4*>(arow)[u4] = v;
    }
    (sp == 0 ? wsf(a, L.off_dgam) : wsf(a, L.off_xgam) + xs * rows)[rq] = dg;
  }
}

// ------------------------------------------------------------------ matrix-core key pass
// dKV, dB and dVV on fp32 matrix cores (standard widths), in two launches
// (below): four wavefronts x
// 32 keys of one (b, h), query tiles of 32 in LDS.  The accumulator layout
// gives every lane one key and 16 queries.  Per tile:
//   S = QV_t KV^T and dP = dO_t VV^T        K-steps interleaved; the keys'
//                                            KV rows sit in LDS, their VV rows
//                                            in registers
//   p = exp(S - gamma |A - B|^2 - lse_i), dS = p (dP - Dsum_i), and
//   dB += 2 gamma dS (A - B) on the vector ALU
//   dKV^T += QV_t^T dS, dVV^T += dO_t^T P   the probabilities and dS straight
//                                            from the accumulator registers
// The query tile's QV and dO are staged transposed (pitch 33 floats): the S
// and dP products read them one query per lane, the dKV and dVV products one
// feature per lane, both without bank conflicts.
// MODE 0: S and dP, accumulating dKV and dB; MODE 1: S only, accumulating dVV
// (one launch each: together they would hold more registers than a lane has).
template <int DKH, int DVH, int NKB, int NVB, int P3C, int MODE>
__global__ __launch_bounds__(256) void bw_key_mfma_kernel(BwArgs a) {
  const BwLayout& L = a.L;
  constexpr bool kDS = MODE == 0, kDV = MODE == 1;
  constexpr int DKp = 2 * DKH, DVp = 2 * DVH;
  static_assert(32 * NKB >= DKp && 32 * NVB >= DVp, "blocks cover the rows");
  __shared__ float sK[4][32][DKp + 1];  // each wavefront's 32 key rows KV
  __shared__ float sQT[32 * NKB][kBwKT + 1];
  __shared__ float sDT[32 * NVB][kBwKT + 1];
  __shared__ __align__(16) float sA[kBwKT][16];
  __shared__ float sL[kBwKT], sS[kBwKT], sSx[kBwKT], sSy[kBwKT], sSz[kBwKT];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int kt = blockIdx.x / L.psplit, sp = blockIdx.x - kt * L.psplit;
  const int j = kt * 128 + 32 * w + l32;
  const bool kin = j < L.N;
  int ib, ie;
  split_range(L, sp, &ib, &ie);
  const int jc = kin ? j : L.N - 1;
  const size_t rj = rowidx(L, b, h, jc);
  const float gam = wsf(a, L.off_gam)[h];
  const bool mk = kin && a.mask[(size_t)b * L.N + jc] != 0;
  const float3 ckey = blk_ref(a, b, jc);
  // rows of the last blocks past DKp / DVp read zeros
  for (int e = tid; e < (32 * NKB - DKp) * (kBwKT + 1); e += 256) sQT[DKp + e / (kBwKT + 1)][e % (kBwKT + 1)] = 0.f;
  for (int e = tid; e < (32 * NVB - DVp) * (kBwKT + 1); e += 256) sDT[DVp + e / (kBwKT + 1)][e % (kBwKT + 1)] = 0.f;
  for (int e = lane; e < 32 * (DKp / 4); e += 64) {
    const int kk = e / (DKp / 4), c4 = e - kk * (DKp / 4);
    const int kr = min(kt * 128 + 32 * w + kk, L.N - 1);
    const float4 v = reinterpret_cast<const float4*>(wsf(a, L.off_kv) + rowidx(L, b, h, kr) * L.DKp)[c4];
    sK[w][kk][4 * c4] = v.x; sK[w][kk][4 * c4 + 1] = v.y; sK[w][kk][4 * c4 + 2] = v.z; sK[w][kk][4 * c4 + 3] = v.w;
  }
  const float* krow = &sK[w][l32][DKH * hf];
  float vv[kDS ? DVH : 1];
  if constexpr (kDS) {
    const float* row = wsf(a, L.off_vv) + rj * L.DVp + DVH * hf;
#pragma unroll
    for (int s4 = 0; s4 < DVH / 4; ++s4) {
      const float4 v = reinterpret_cast<const float4*>(row)[s4];
      vv[4 * s4] = v.x; vv[4 * s4 + 1] = v.y; vv[4 * s4 + 2] = v.z; vv[4 * s4 + 3] = v.w;
    }
  }
  float kb[P3C];
  {
    const float* row = wsf(a, L.off_kb) + rj * 16;
#pragma unroll
    for (int u = 0; u < P3C; ++u) kb[u] = row[u];
  }
  f32x16_t dk[kDS ? NKB : 1], dv[kDV ? NVB : 1];
#pragma unroll
  for (int c = 0; c < (kDS ? NKB : 1); ++c) dk[c] = f32x16_t{};
#pragma unroll
  for (int c = 0; c < (kDV ? NVB : 1); ++c) dv[c] = f32x16_t{};
  float db[P3C];
#pragma unroll
  for (int u = 0; u < P3C; ++u) db[u] = 0.f;
  // query tiles: QV and dO (transposed into LDS), query points, per-query
  // statistics; the tile's loads go out together one tile ahead, in flight
  // during the products of the current one
  const float* qvb = wsf(a, L.off_qv) + rowidx(L, b, h, 0) * L.DKp;
  const float* dob = wsf(a, L.off_do) + rowidx(L, b, h, 0) * L.DVp;
  const float* qab = wsf(a, L.off_qa) + rowidx(L, b, h, 0) * 16;
  Tile4<DKp / 4> tq;
  Tile4<DVp / 4> td;
  Tile4<4> ta;
  float t_lse = 0.f, t_dd = 0.f;
  float4 t_ds = make_float4(0.f, 0.f, 0.f, 0.f);
  bool t_ok = false;
  auto issue = [&](int i0) {
    tq.load(qvb, L.DKp, i0, L.N, tid, DKp / 4);
    td.load(dob, L.DVp, i0, L.N, tid, DVp / 4);
    ta.load(qab, 16, i0, L.N, tid, 4);
    const int i = i0 + (tid & 31);
    const int icl = min(i, L.N - 1);
    t_lse = wsf(a, L.off_lse)[rowidx(L, b, h, icl)];
    t_ok = i < L.N && a.mask[(size_t)b * L.N + icl] != 0;
    t_dd = wsf(a, L.off_dd)[rowidx(L, b, h, icl)];
    t_ds = reinterpret_cast<const float4*>(wsf(a, L.off_ds) + rowidx(L, b, h, icl) * 4)[0];
  };
  auto put_q = [&](int ii, int c4, float4 v) {
    sQT[4 * c4][ii] = v.x; sQT[4 * c4 + 1][ii] = v.y; sQT[4 * c4 + 2][ii] = v.z; sQT[4 * c4 + 3][ii] = v.w;
  };
  auto put_d = [&](int ii, int c4, float4 v) {
    sDT[4 * c4][ii] = v.x; sDT[4 * c4 + 1][ii] = v.y; sDT[4 * c4 + 2][ii] = v.z; sDT[4 * c4 + 3][ii] = v.w;
  };
  auto put_a = [&](int ii, int c4, float4 v) { reinterpret_cast<float4*>(&sA[ii][0])[c4] = v; };
  if (ib < ie) issue(ib);
  for (int i0 = ib; i0 < ie; i0 += kBwKT) {
    __syncthreads();
    tq.store(tid, put_q);
    td.store(tid, put_d);
    ta.store(tid, put_a);
    if (tid < kBwKT) {
      const bool ok = t_ok && t_lse > -INFINITY;
      sL[tid] = ok ? t_lse : INFINITY;  // +inf marks a query that takes no key
      sS[tid] = t_dd;
      sSx[tid] = t_ds.x;
      sSy[tid] = t_ds.y;
      sSz[tid] = t_ds.z;
    }
    if (i0 + kBwKT < ie) issue(i0 + kBwKT);
    __syncthreads();
    // the query block's reference relative to this key's
    const float3 cqb = blk_ref(a, b, i0);
    const float dcx = cqb.x - ckey.x, dcy = cqb.y - ckey.y, dcz = cqb.z - ckey.z;
    f32x16_t sa = f32x16_t{}, pa = f32x16_t{};
    if constexpr (kDS) {
#pragma unroll
      for (int s = 0; s < (DKH > DVH ? DKH : DVH); ++s) {
        if (s < DKH) sa = __builtin_amdgcn_mfma_f32_32x32x2f32(sQT[s + DKH * hf][l32], krow[s], sa, 0, 0, 0);
        if (s < DVH) pa = __builtin_amdgcn_mfma_f32_32x32x2f32(sDT[s + DVH * hf][l32], vv[s], pa, 0, 0, 0);
      }
    } else {
      // one chain: two accumulators over even and odd K-steps
#pragma unroll
      for (int s = 0; s < DKH; s += 2) {
        sa = __builtin_amdgcn_mfma_f32_32x32x2f32(sQT[s + DKH * hf][l32], krow[s], sa, 0, 0, 0);
        if (s + 1 < DKH) pa = __builtin_amdgcn_mfma_f32_32x32x2f32(sQT[s + 1 + DKH * hf][l32], krow[s + 1], pa, 0, 0, 0);
      }
      sa += pa;
    }
    float ds[16], pr[16];
    // permission bits of the tile's queries for this key (bit r: query
    // kappa(r, hf)), once per tile; the pair-mask loads go out together, their
    // row clamped into the chain (queries past it have sL = +inf)
    uint32_t okm = 0u;
#pragma unroll
    for (int r = 0; r < 16; ++r) okm |= sL[kappa(r, hf)] < INFINITY ? (1u << r) : 0u;
    if (a.pmask) {
      uint32_t pm = 0u;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = min(i0 + kappa(r, hf), L.N - 1);
        pm |= a.pmask[((size_t)b * L.N + i) * L.N + jc] != 0 ? (1u << r) : 0u;
      }
      okm &= pm;
    }
    okm = mk ? okm : 0u;
    // probabilities (and dS) first; the coordinate differences are
    // recomputed for dB below rather than held for sixteen queries
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qq = kappa(r, hf);
      float d2 = 0.f;
#pragma unroll
      for (int c4 = 0; c4 < P3C / 4; ++c4) {
        const float4 x = reinterpret_cast<const float4*>(&sA[qq][0])[c4];
        const float dx = x.x - kb[4 * c4], dy = x.y - kb[4 * c4 + 1], dz = x.z - kb[4 * c4 + 2], dw = x.w - kb[4 * c4 + 3];
        d2 += dx * dx + dy * dy + dz * dz + dw * dw;
      }
      pr[r] = ((okm >> r) & 1u) ? exp_fast(sa[r] - gam * d2 - sL[qq]) : 0.f;
      if constexpr (kDS) {
        const float corr = fmaf(sSx[qq], dcx, fmaf(sSy[qq], dcy, fmaf(sSz[qq], dcz, sS[qq])));
        ds[r] = pr[r] * (pa[r] - corr);
      }
    }
    // dKV^T += QV_t^T dS, dVV^T += dO_t^T P; in mode 0 the point term dB
    // (vector ALU, independent of these products) is placed between the
    // matrix instructions
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      if constexpr (kDS) {
        const int qq = kappa(s, hf);
#pragma unroll
        for (int c = 0; c < NKB; ++c) {
          dk[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(sQT[32 * c + l32][qq], ds[s], dk[c], 0, 0, 0);
          if (c < P3C / 4) {
            // a piece of dB for query qq (coordinates 4c .. 4c+3)
            const float4 x = reinterpret_cast<const float4*>(&sA[qq][0])[c];
            db[4 * c] = fmaf(ds[s], x.x - kb[4 * c], db[4 * c]);
            db[4 * c + 1] = fmaf(ds[s], x.y - kb[4 * c + 1], db[4 * c + 1]);
            db[4 * c + 2] = fmaf(ds[s], x.z - kb[4 * c + 2], db[4 * c + 2]);
            db[4 * c + 3] = fmaf(ds[s], x.w - kb[4 * c + 3], db[4 * c + 3]);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < NVB; ++c)
          dv[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(sDT[32 * c + l32][kappa(s, hf)], pr[s], dv[c], 0, 0, 0);
      }
    }
  }
  // the two halves of the wavefront hold the same keys' two halves of each tile
#pragma unroll
  for (int u = 0; u < P3C; ++u) db[u] += __shfl_xor(db[u], 32);
  if (!kin) return;
  // query range sp > 0 writes its partial sums to a slab of its own
  const size_t rows = (size_t)L.B * L.H * L.N, xs = (size_t)(sp - 1);
  float* krw = (sp == 0 ? wsf(a, L.off_dkv) : wsf(a, L.off_xkv) + xs * rows * L.DKp) + rj * L.DKp;
  float* vrw = (sp == 0 ? wsf(a, L.off_dvv) : wsf(a, L.off_xvv) + xs * rows * L.DVp) + rj * L.DVp;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
#pragma unroll
    for (int c = 0; c < (kDS ? NKB : 0); ++c) {
      const int f = 32 * c + 8 * g + 4 * hf;
      if (f < DKp)
        *reinterpret_cast<float4*>(krw + f) = make_float4(dk[c][4 * g], dk[c][4 * g + 1], dk[c][4 * g + 2], dk[c][4 * g + 3]);
    }
#pragma unroll
    for (int c = 0; c < (kDV ? NVB : 0); ++c) {
      const int f = 32 * c + 8 * g + 4 * hf;
      if (f < DVp)
        *reinterpret_cast<float4*>(vrw + f) = make_float4(dv[c][4 * g], dv[c][4 * g + 1], dv[c][4 * g + 2], dv[c][4 * g + 3]);
    }
  }
  if (kDS && hf == 0) {
    float* brow = (sp == 0 ? wsf(a, L.off_dkb) : wsf(a, L.off_xkb) + xs * rows * 16) + rj * 16;
#pragma unroll
    for (int u4 = 0; u4 < 4; ++u4) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (4 * u4 < P3C)
        v = make_float4(2.f * gam * db[4 * u4], 2.f * gam * db[4 * u4 + 1], 2.f * gam * db[4 * u4 + 2],
                        2.f * gam * db[4 * u4 + 3]);
      reinterpret_cast<float4*>(brow)[u4] = v;
    }
  }
}

// ------------------------------------------------------------------ GEMM
// C[m][n] (+)= sum_k A(m,k) B(k,n), fp32, 64x64 tiles, 256 threads x 4x4.
// A(m,k) = A[m*sam + k*sak], B(k,n) = B[k*sbk + n*sbn].  blockIdx.z splits K
// into ksplit ranges, each writing its own C slab (C + z*slab).
struct GemmArgs {
  const float* A;
  const float* Bm;
  float* C;
  int M, N, K, ksplit;
  long sam, sak, sbk, sbn, ldc;
  size_t slab;
};

__global__ __launch_bounds__(256) void bw_gemm_kernel(GemmArgs g) {
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  const int kchunk = (g.K + g.ksplit - 1) / g.ksplit;
  const int kb = blockIdx.z * kchunk, ke = min(g.K, kb + kchunk);
  float acc[4][4] = {};
  for (int k0 = kb; k0 < ke; k0 += 16) {
    __syncthreads();
    for (int e = tid; e < 16 * 64; e += 256) {
      const int kk = e >> 6, mm = e & 63;
      const int m = m0 + mm, k = k0 + kk;
      As[kk][mm] = (m < g.M && k < ke) ? g.A[(long)m * g.sam + (long)k * g.sak] : 0.f;
      const int n = n0 + mm;
      Bs[kk][mm] = (n < g.N && k < ke) ? g.Bm[(long)k * g.sbk + (long)n * g.sbn] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        av[u] = As[kk][ty * 4 + u];
        bv[u] = Bs[kk][tx * 4 + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[u][w] = fmaf(av[u], bv[w], acc[u][w]);
    }
  }
  float* C = g.C + blockIdx.z * g.slab;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int m = m0 + ty * 4 + u, n = n0 + tx * 4 + w;
      if (m < g.M && n < g.N) C[(long)m * g.ldc + n] = acc[u][w];
    }
}

// fp32 copy of a bf16 array
__global__ __launch_bounds__(256) void bw_widen_kernel(const uint16_t* src, float* dst, size_t n) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e < n) dst[e] = bf16_bits_to_f32(src[e]);
}

// out[e] = sum_z part[z*slab + e]
__global__ __launch_bounds__(256) void bw_sum_slabs_kernel(const float* part, float* out, size_t n, int nz, size_t slab) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  float s = 0.f;
  for (int z = 0; z < nz; ++z) s += part[z * slab + e];
  out[e] = s;
}

// ------------------------------------------------------------------ epilogue backward
// One wavefront per residue row (b, i): features (for dW), dO per head,
// Dsum, and the epilogue's own contributions to dzl, dR, dt.  DFEAT holds
// d_update @ w_out^T for the row (computed by the GEMM before this kernel).
__global__ __launch_bounds__(64) void bw_epi_kernel(BwArgs a) {
  const BwLayout& L = a.L;
  const int bn = blockIdx.x;
  const int b = bn / L.N, i = bn - b * L.N;
  const int lane = threadIdx.x;
  const int H = L.H, Dv = L.Dv, Q = L.Q, Cz = L.Cz, R = L.R, F = L.F;
  const float lse0 = wsf(a, L.off_lse)[rowidx(L, b, 0, i)];
  const bool empty = !(lse0 > -INFINITY);
  float* feat = wsf(a, L.off_feat) + (size_t)bn * (F + 1);
  const float* dfeat = wsf(a, L.off_dfeat) + (size_t)bn * F;
  const float* Rm = a.rot + (size_t)bn * 9;
  const float* tv = a.tr + (size_t)bn * 3;
  const float* zlr = a.zl + (size_t)bn * R * Cz;
  float* dzle = wsf(a, L.off_dzle) + (size_t)bn * R * Cz;
  const int oS = 0, oX = H * Dv, oY = oX + H * Q, oZ = oY + H * Q, oLen = oZ + H * Q, oP = oLen + H * Q;
  if (empty) {
    for (int e = lane; e <= F; e += 64) feat[e] = 0.f;
    for (int h = 0; h < H; ++h) {
      const size_t ri = rowidx(L, b, h, i);
      for (int e = lane; e < L.DVp; e += 64) wsf(a, L.off_do)[ri * L.DVp + e] = 0.f;
      if (lane == 0) wsf(a, L.off_dd)[ri] = 0.f;
      if (lane < 4) wsf(a, L.off_ds)[ri * 4 + lane] = 0.f;
    }
    for (int e = lane; e < R * Cz; e += 64) dzle[e] = 0.f;
    if (lane < 9) wsf(a, L.off_dre)[(size_t)bn * 9 + lane] = 0.f;
    if (lane < 3) wsf(a, L.off_dte)[(size_t)bn * 3 + lane] = 0.f;
    return;
  }
  if (lane == 0) feat[F] = 1.f;  // row kept: the last column of dW's product gives db
  // scalar and pair features, dO scalar / pair parts, dzl
  for (int h = 0; h < H; ++h) {
    const size_t ri = rowidx(L, b, h, i);
    const float* O = wsf(a, L.off_o) + ri * L.DVp;
    float* dO = wsf(a, L.off_do) + ri * L.DVp;
    for (int d = lane; d < Dv; d += 64) {
      feat[oS + h * Dv + d] = O[d];
      dO[d] = dfeat[oS + h * Dv + d];
    }
    for (int c = lane; c < Cz; c += 64) {
      float pf = 0.f;
      const float dpf = dfeat[oP + h * Cz + c];
      for (int r = 0; r < R; ++r) {
        pf += zlr[r * Cz + c] * O[Dv + r * Cz + c];
        dO[Dv + r * Cz + c] = zlr[r * Cz + c] * dpf;
      }
      feat[oP + h * Cz + c] = pf;
    }
    for (int e = Dv + R * Cz + 3 * Q + lane; e < L.DVp; e += 64) dO[e] = 0.f;
  }
  for (int e = lane; e < R * Cz; e += 64) {
    const int r = e / Cz, c = e - r * Cz;
    float s = 0.f;
    for (int h = 0; h < H; ++h) s += wsf(a, L.off_o)[rowidx(L, b, h, i) * L.DVp + Dv + r * Cz + c] * dfeat[oP + h * Cz + c];
    dzle[e] = s;
  }
  // points: one lane per (h, q); O holds them relative to the block
  // reference c of residue i, so g - t = O' - (t - c)
  const float3 cr = blk_ref(a, b, i);
  const float tc[3] = {tv[0] - cr.x, tv[1] - cr.y, tv[2] - cr.z};
  float dr[9] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float dt[3] = {0.f, 0.f, 0.f};
  for (int e = lane; e < H * Q; e += 64) {
    const int h = e / Q, qq = e - h * Q;
    const size_t ri = rowidx(L, b, h, i);
    const float* g = wsf(a, L.off_o) + ri * L.DVp + Dv + R * Cz + 3 * qq;
    const float rel[3] = {g[0] - tc[0], g[1] - tc[1], g[2] - tc[2]};
    float loc[3];
    for (int x = 0; x < 3; ++x) loc[x] = Rm[0 * 3 + x] * rel[0] + Rm[1 * 3 + x] * rel[1] + Rm[2 * 3 + x] * rel[2];
    const float len = sqrtf(loc[0] * loc[0] + loc[1] * loc[1] + loc[2] * loc[2] + a.eps);
    feat[oX + h * Q + qq] = loc[0];
    feat[oY + h * Q + qq] = loc[1];
    feat[oZ + h * Q + qq] = loc[2];
    feat[oLen + h * Q + qq] = len;
    const float* dl = a.dloc + (((size_t)bn * H + h) * Q + qq) * 3;
    const float dlen = dfeat[oLen + h * Q + qq] / len;
    const float dlocv[3] = {dfeat[oX + h * Q + qq] + dl[0] + dlen * loc[0], dfeat[oY + h * Q + qq] + dl[1] + dlen * loc[1],
                            dfeat[oZ + h * Q + qq] + dl[2] + dlen * loc[2]};
    float* dg = wsf(a, L.off_do) + ri * L.DVp + Dv + R * Cz + 3 * qq;
    for (int m = 0; m < 3; ++m) {
      const float v = Rm[m * 3 + 0] * dlocv[0] + Rm[m * 3 + 1] * dlocv[1] + Rm[m * 3 + 2] * dlocv[2];
      dg[m] = v;
      dt[m] -= v;
      for (int x = 0; x < 3; ++x) dr[m * 3 + x] += rel[m] * dlocv[x];
    }
  }
  // wave sums of dR, dt
  for (int e = 0; e < 9; ++e) {
    float v = dr[e];
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    dr[e] = v;
  }
  for (int e = 0; e < 3; ++e) {
    float v = dt[e];
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    dt[e] = v;
  }
  if (lane == 0) {
    for (int e = 0; e < 9; ++e) wsf(a, L.off_dre)[(size_t)bn * 9 + e] = dr[e];
    for (int e = 0; e < 3; ++e) wsf(a, L.off_dte)[(size_t)bn * 3 + e] = dt[e];
  }
  __syncthreads();
  // Dsum'_h = dO_h . O'_h, and S_h = the sum of dO_h's point part over the
  // value points (per coordinate)
  for (int h = 0; h < H; ++h) {
    const size_t ri = rowidx(L, b, h, i);
    const float* O = wsf(a, L.off_o) + ri * L.DVp;
    const float* dO = wsf(a, L.off_do) + ri * L.DVp;
    float s = 0.f;
    for (int e = lane; e < L.DV; e += 64) s += O[e] * dO[e];
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) wsf(a, L.off_dd)[ri] = s;
    if (lane < 4) {
      float sc = 0.f;
      if (lane < 3)
        for (int qq = 0; qq < Q; ++qq) sc += dO[Dv + R * Cz + 3 * qq + lane];
      wsf(a, L.off_ds)[ri * 4 + lane] = sc;
    }
  }
}

// ------------------------------------------------------------------ input gradients
// One wavefront per (b, residue): q/k/v, frames, points, factors.  A global
// point gradient g of local point x gives d x = R^T g, dR += g x^T, dt += g.
__global__ __launch_bounds__(64) void bw_inputs_kernel(BwArgs a) {
  const BwLayout& L = a.L;
  const int bn = blockIdx.x, lane = threadIdx.x;
  const int b = bn / L.N, n = bn - b * L.N;
  const int H = L.H, D = L.D, Dv = L.Dv, P = L.P, Q = L.Q, Cz = L.Cz, R = L.R;
  const float* Rm = a.rot + (size_t)bn * 9;
  const float sq = 1.0f / sqrtf(3.0f * (float)D), s3 = 1.0f / sqrtf(3.0f);
  for (int e = lane; e < H * D; e += 64) {
    const int h = e / D, d = e - h * D;
    const size_t ri = rowidx(L, b, h, n);
    a.gq[(size_t)bn * H * D + e] = wsf(a, L.off_dqv)[ri * L.DKp + d] * sq;
    a.gk[(size_t)bn * H * D + e] = wsf(a, L.off_dkv)[ri * L.DKp + d];
  }
  for (int e = lane; e < H * Dv; e += 64) {
    const int h = e / Dv, d = e - h * Dv;
    a.gv[(size_t)bn * H * Dv + e] = wsf(a, L.off_dvv)[rowidx(L, b, h, n) * L.DVp + d];
  }
  float dr[9] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float dt[3] = {0.f, 0.f, 0.f};
  // tasks: (h, p) query points, (h, p) key points, (h, q) value points
  const int nq = H * P, nv = H * Q;
  for (int e = lane; e < 2 * nq + nv; e += 64) {
    const float* g;
    const float* x;
    float* dx;
    if (e < nq) {
      const int h = e / P, pp = e - h * P;
      g = wsf(a, L.off_dqa) + rowidx(L, b, h, n) * 16 + 3 * pp;
      const size_t o = (((size_t)bn * H + h) * P + pp) * 3;
      x = a.qp + o;
      dx = a.gqp + o;
    } else if (e < 2 * nq) {
      const int f = e - nq, h = f / P, pp = f - h * P;
      g = wsf(a, L.off_dkb) + rowidx(L, b, h, n) * 16 + 3 * pp;
      const size_t o = (((size_t)bn * H + h) * P + pp) * 3;
      x = a.kp + o;
      dx = a.gkp + o;
    } else {
      const int f = e - 2 * nq, h = f / Q, qq = f - h * Q;
      g = wsf(a, L.off_dvv) + rowidx(L, b, h, n) * L.DVp + Dv + R * Cz + 3 * qq;
      const size_t o = (((size_t)bn * H + h) * Q + qq) * 3;
      x = a.vp + o;
      dx = a.gvp + o;
    }
    const float g0 = g[0], g1 = g[1], g2 = g[2];
    const float x0 = x[0], x1 = x[1], x2 = x[2];
    for (int c = 0; c < 3; ++c) dx[c] = Rm[0 * 3 + c] * g0 + Rm[1 * 3 + c] * g1 + Rm[2 * 3 + c] * g2;
    const float gg[3] = {g0, g1, g2}, xx[3] = {x0, x1, x2};
    for (int m = 0; m < 3; ++m) {
      dt[m] += gg[m];
      for (int c = 0; c < 3; ++c) dr[m * 3 + c] += gg[m] * xx[c];
    }
  }
  for (int e = 0; e < 9; ++e) {
    float v = dr[e];
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    dr[e] = v;
  }
  for (int e = 0; e < 3; ++e) {
    float v = dt[e];
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    dt[e] = v;
  }
  if (lane < 9) a.grot[(size_t)bn * 9 + lane] = dr[lane] + wsf(a, L.off_dre)[(size_t)bn * 9 + lane];
  if (lane < 3) a.gtr[(size_t)bn * 3 + lane] = dt[lane] + wsf(a, L.off_dte)[(size_t)bn * 3 + lane];
  for (int e = lane; e < R * Cz; e += 64) {
    const int r = e / Cz, c = e - r * Cz;
    float gl = wsf(a, L.off_dzle)[(size_t)bn * R * Cz + e];
    float gr = 0.f;
    for (int h = 0; h < H; ++h) {
      const size_t ri = rowidx(L, b, h, n);
      gl += wsf(a, L.off_dqv)[ri * L.DKp + D + r * Cz + c] * a.wpair[h * Cz + c] * s3;
      gr += wsf(a, L.off_dkv)[ri * L.DKp + D + r * Cz + c] + wsf(a, L.off_dvv)[ri * L.DVp + Dv + r * Cz + c];
    }
    a.gzl[(size_t)bn * R * Cz + e] = gl;
    a.gzr[(size_t)bn * R * Cz + e] = gr;
  }
}

// Per-head parameters: dw_pair[h][c] = sum_{b,i,r} zl[b,i,r,c] dQV[b,h,i,D+rCz+c] / sqrt(3)
// and dgamma[h] = sum_{b,i} dgam[b,h,i] -> d point_weight_raw.  Stage 1: one
// workgroup per (head, chunk of rows) writes partial sums; stage 2 adds the
// chunks of a head.
constexpr int kBwParamChunks = 64;

__global__ __launch_bounds__(256) void bw_params_part_kernel(BwArgs a) {
  const BwLayout& L = a.L;
  const int h = blockIdx.x, ch = blockIdx.y;
  const int tid = threadIdx.x;
  const int BN = L.B * L.N, Cz = L.Cz, R = L.R, D = L.D;
  const int per = (BN + kBwParamChunks - 1) / kBwParamChunks;
  const int r0 = ch * per, r1 = min(BN, r0 + per);
  float* part = wsf(a, L.off_ppart) + ((size_t)h * kBwParamChunks + ch) * (Cz + 1);
  __shared__ float red[256];
  for (int c0 = 0; c0 < Cz; c0 += 64) {
    const int c = c0 + (tid & 63), grp = tid >> 6;
    float s = 0.f;
    if (c < Cz) {
      for (int bn = r0 + grp; bn < r1; bn += 4) {
        const int b = bn / L.N, n = bn - b * L.N;
        const size_t ri = rowidx(L, b, h, n);
        for (int r = 0; r < R; ++r)
          s += a.zl[(size_t)bn * R * Cz + r * Cz + c] * wsf(a, L.off_dqv)[ri * L.DKp + D + r * Cz + c];
      }
    }
    red[tid] = s;
    __syncthreads();
    if (tid < 64 && c < Cz) part[c] = red[tid] + red[tid + 64] + red[tid + 128] + red[tid + 192];
    __syncthreads();
  }
  float s = 0.f;
  for (int bn = r0 + tid; bn < r1; bn += 256) {
    const int b = bn / L.N, n = bn - b * L.N;
    s += wsf(a, L.off_dgam)[rowidx(L, b, h, n)];
  }
  red[tid] = s;
  __syncthreads();
  for (int o = 128; o >= 1; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) part[Cz] = red[0];
}

__global__ __launch_bounds__(256) void bw_params_kernel(BwArgs a) {
  const BwLayout& L = a.L;
  const int h = blockIdx.x;
  const int Cz = L.Cz;
  const float s3 = 1.0f / sqrtf(3.0f);
  const float* part = wsf(a, L.off_ppart) + (size_t)h * kBwParamChunks * (Cz + 1);
  for (int c = threadIdx.x; c <= Cz; c += 256) {
    float s = 0.f;
    for (int ch = 0; ch < kBwParamChunks; ++ch) s += part[(size_t)ch * (Cz + 1) + c];
    if (c < Cz) {
      a.gwpair[h * Cz + c] = s * s3;
    } else {
      const float w = a.wraw[h];
      const float sig = 1.f / (1.f + expf(-w));
      a.gwraw[h] = s * 0.5f * sig * sqrtf(2.0f / (27.0f * (float)L.P));
    }
  }
}

struct BwInst {
  int nk4, nv4;
};
constexpr BwInst kBwInst[] = {{1, 2}, {4, 4}, {9, 11}, {16, 16}};

template <int NK4, int NV4, int ROWS>
hipError_t launch_pairs_rows(const BwArgs& a, int which, hipStream_t st) {
  const BwLayout& L = a.L;
  dim3 grid((L.N + ROWS - 1) / ROWS, L.H, L.B);
  if (which == 0) hipLaunchKernelGGL((bw_fwd_kernel<NK4, NV4, ROWS>), grid, dim3(4 * ROWS), 0, st, a);
  if (which == 1) hipLaunchKernelGGL((bw_query_kernel<NK4, NV4, ROWS>), grid, dim3(4 * ROWS), 0, st, a);
  if (which == 2) {
    if ((long)grid.x * grid.y * grid.z >= 512) {
      hipLaunchKernelGGL((bw_key_kernel<NK4, NV4, ROWS, 0>), grid, dim3(4 * ROWS), 0, st, a);
      hipLaunchKernelGGL((bw_key_kernel<NK4, NV4, ROWS, 1>), grid, dim3(4 * ROWS), 0, st, a);
    } else {
      hipLaunchKernelGGL((bw_key_kernel<NK4, NV4, ROWS, 2>), grid, dim3(4 * ROWS), 0, st, a);
    }
  }
  return hipGetLastError();
}

// 64 rows (256 threads) per workgroup.  (32-row workgroups for small grids
// were measured slower: the staging per row doubles and the key pass is held
// to one wavefront per SIMD by its registers either way.)
template <int NK4, int NV4>
hipError_t launch_pairs(const BwArgs& a, int which, hipStream_t st) {
  return launch_pairs_rows<NK4, NV4, 64>(a, which, st);
}

hipError_t launch_pairs_inst(const BwArgs& a, int which, hipStream_t st) {
  const BwLayout& L = a.L;
  // the matrix-core passes take psplit workgroups per row tile, one per
  // inner-loop range (psplit > 1 only with every pass on the matrix cores)
  const dim3 grid((L.N + 127) / 128 * L.psplit, L.H, L.B);
  const size_t rows = (size_t)L.B * L.H * L.N;
  const int xs = L.psplit - 1;
  auto add = [&](size_t out, size_t extra, size_t n) {
    hipLaunchKernelGGL(bw_add_slabs_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<float*>(a.ws + out), reinterpret_cast<const float*>(a.ws + extra), n, xs);
  };
  if (which == 0 && L.NK4 == 9) {
    // standard shape (D + R Cz <= 144, Dv + R Cz + 3Q <= 176): matrix cores
    // coordinates past 3P are zero on both sides: P < 4 takes the 12-coordinate instance as well
    if (L.P3 <= 12)
      hipLaunchKernelGGL((bw_fwd_mfma_kernel<72, 6, 12>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((bw_fwd_mfma_kernel<72, 6, 16>), grid, dim3(256), 0, st, a);
    if (L.psplit > 1)
      hipLaunchKernelGGL(bw_merge_o_kernel, dim3((unsigned)((rows * (L.DVp / 4) + 255) / 256)), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  if (which == 2 && L.NK4 == 9 && L.DVp == 176 && L.P3 == 12) {
    hipLaunchKernelGGL((bw_key_mfma_kernel<72, 88, 5, 6, 12, 0>), grid, dim3(256), 0, st, a);
    hipLaunchKernelGGL((bw_key_mfma_kernel<72, 88, 5, 6, 12, 1>), grid, dim3(256), 0, st, a);
    if (L.psplit > 1) {
      add(L.off_dkv, L.off_xkv, rows * L.DKp);
      add(L.off_dkb, L.off_xkb, rows * 16);
      add(L.off_dvv, L.off_xvv, rows * L.DVp);
    }
    return hipGetLastError();
  }
  if (which == 1 && L.NK4 == 9 && L.DVp == 176 && L.P3 == 12) {
    hipLaunchKernelGGL((bw_query_mfma_kernel<72, 88, 5, 12>), grid, dim3(256), 0, st, a);
    if (L.psplit > 1) {
      add(L.off_dqv, L.off_xqv, rows * L.DKp);
      add(L.off_dqa, L.off_xqa, rows * 16);
      add(L.off_dgam, L.off_xgam, rows);
    }
    return hipGetLastError();
  }
  if (L.NK4 == 1) return launch_pairs<1, 2>(a, which, st);
  if (L.NK4 == 4) return launch_pairs<4, 4>(a, which, st);
  if (L.NK4 == 9) return launch_pairs<9, 11>(a, which, st);
  return launch_pairs<16, 16>(a, which, st);
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
  dim3 grid((g.M + 63) / 64, (g.N + 63) / 64, g.ksplit);  // rows on x (up to 2^31 tiles)
  hipLaunchKernelGGL(bw_gemm_kernel, grid, dim3(256), 0, st, g);
  return hipGetLastError();
}

}  // namespace

bool bw_layout(const ipa_shape* s, BwLayout* L) {
  L->B = (int)s->B;
  L->N = (int)s->N;
  L->H = (int)s->H;
  L->D = (int)s->D;
  L->Dv = (int)s->Dv;
  L->P = (int)s->P;
  L->Q = (int)s->Q;
  L->Cz = (int)s->Cz;
  L->R = (int)s->R;
  L->Cout = (int)s->Cout;
  L->F = L->H * (L->Dv + 4 * L->Q + L->Cz);
  L->DK = L->D + L->R * L->Cz;
  L->DV = L->Dv + L->R * L->Cz + 3 * L->Q;
  L->P3 = 3 * L->P;
  if (L->P3 > 16) return false;
  int pick = -1;
  for (int e = 0; e < 4; ++e)
    if (16 * kBwInst[e].nk4 >= L->DK && 16 * kBwInst[e].nv4 >= L->DV) {
      pick = e;
      break;
    }
  if (pick < 0) return false;
  L->NK4 = kBwInst[pick].nk4;
  L->NV4 = kBwInst[pick].nv4;
  L->DKp = 16 * L->NK4;
  L->DVp = 16 * L->NV4;
  const size_t rows = (size_t)L->B * L->H * L->N, bn = (size_t)L->B * L->N;
  L->ksplit = (int)std::min<size_t>(64, std::max<size_t>(1, bn / 256));
  // Short chains: the pair passes' grids (128-row tiles x H x B) would leave
  // CUs idle, so each row tile's inner loop is split into psplit ranges of at
  // least 8 partner tiles (up to 4 ranges, while the grid stays within 256
  // workgroups), the partial results merged by small kernels.  Only when all
  // three passes run on the matrix cores (standard widths).
  const bool mfma_all = L->NK4 == 9 && L->DVp == 176 && L->P3 == 12;
  const size_t row_tiles = (size_t)((L->N + 127) / 128) * L->H * L->B;
  L->psplit = 1;
  while (mfma_all && L->psplit < 4 && row_tiles * L->psplit * 2 <= 256 && (size_t)L->N >= (size_t)512 * L->psplit)
    L->psplit *= 2;
  size_t off = 256;
  auto take = [&](size_t floats) {
    const size_t o = off;
    off += ((floats * 4 + 255) / 256) * 256;
    return o;
  };
  L->off_gam = take(L->H);
  L->off_qv = take(rows * L->DKp);
  L->off_kv = take(rows * L->DKp);
  L->off_vv = take(rows * L->DVp);
  L->off_qa = take(rows * 16);
  L->off_kb = take(rows * 16);
  L->off_o = take(rows * L->DVp);
  L->off_lse = take(rows);
  L->off_do = take(rows * L->DVp);
  L->off_dd = take(rows);
  L->off_ds = take(rows * 4);
  L->off_feat = take(bn * (L->F + 1));
  L->off_dfeat = take(bn * L->F);
  L->off_dqv = take(rows * L->DKp);
  L->off_dqa = take(rows * 16);
  L->off_dgam = take(rows);
  L->off_dkv = take(rows * L->DKp);
  L->off_dkb = take(rows * 16);
  L->off_dvv = take(rows * L->DVp);
  L->off_dzle = take(bn * L->R * L->Cz);
  L->off_dre = take(bn * 9);
  L->off_dte = take(bn * 3);
  L->off_dwpart = take((size_t)L->ksplit * (L->F + 1) * L->Cout);
  L->off_ppart = take((size_t)L->H * kBwParamChunks * (L->Cz + 1));
  const size_t xs = (size_t)(L->psplit - 1);
  L->off_opart = L->psplit > 1 ? take((size_t)L->psplit * rows * (L->DVp + 8)) : 0;
  L->off_xqv = xs ? take(xs * rows * L->DKp) : 0;
  L->off_xqa = xs ? take(xs * rows * 16) : 0;
  L->off_xgam = xs ? take(xs * rows) : 0;
  L->off_xkv = xs ? take(xs * rows * L->DKp) : 0;
  L->off_xkb = xs ? take(xs * rows * 16) : 0;
  L->off_xvv = xs ? take(xs * rows * L->DVp) : 0;
  L->bf16 = s->dtype == IPA_BF16;
  const size_t bnh = bn * L->H;
  const size_t cn[14] = {bnh * L->D, bnh * L->D, bnh * L->Dv, bnh * L->P * 3, bnh * L->P * 3, bnh * L->Q * 3, bn * 9,
                         bn * 3, (size_t)L->H, (size_t)L->H * L->Cz, bn * L->R * L->Cz, bn * L->R * L->Cz,
                         (size_t)L->F * L->Cout, (size_t)L->Cout};
  for (int e = 0; e < 14; ++e) {
    L->cvt_n[e] = cn[e];
    L->off_cvt[e] = L->bf16 ? take(cn[e]) : 0;
  }
  L->total = off;
  return true;
}

size_t bw_workspace_bytes(const ipa_shape* s) {
  BwLayout L;
  if (!bw_layout(s, &L)) return 0;
  return L.total;
}

hipError_t launch_backward(const ipa_shape* s, const ipa_lift_in* in, const ipa_epi_in* ep, const float* dupd,
                           const float* dloc, void* ws, ipa_grads* gr, hipStream_t st) {
  BwArgs a;
  if (!bw_layout(s, &a.L)) return hipErrorInvalidValue;
  const BwLayout& L = a.L;
  a.ws = (char*)ws;
  if (L.bf16) {
    // bf16 inputs: widen every input into its fp32 copy, then run the fp32 backward on the copies
    const void* src[14] = {in->q, in->k, in->v, in->q_points, in->k_points, in->v_points, in->rotation,
                           in->translation, in->point_weight_raw, in->w_pair, in->zl, in->zr, ep->w_out, ep->b_out};
    for (int e = 0; e < 14; ++e) {
      const size_t n = L.cvt_n[e];
      hipLaunchKernelGGL(bw_widen_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                         (const uint16_t*)src[e], (float*)(a.ws + L.off_cvt[e]), n);
    }
    hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
  }
  auto inp = [&](int e, const void* p) { return L.bf16 ? (const float*)(a.ws + L.off_cvt[e]) : (const float*)p; };
  a.q = inp(0, in->q);
  a.k = inp(1, in->k);
  a.v = inp(2, in->v);
  a.qp = inp(3, in->q_points);
  a.kp = inp(4, in->k_points);
  a.vp = inp(5, in->v_points);
  a.rot = inp(6, in->rotation);
  a.tr = inp(7, in->translation);
  a.wraw = inp(8, in->point_weight_raw);
  a.wpair = inp(9, in->w_pair);
  a.zl = inp(10, in->zl);
  a.zr = inp(11, in->zr);
  a.wout = inp(12, ep->w_out);
  a.bout = inp(13, ep->b_out);
  a.mask = in->mask;
  a.pmask = in->pair_mask;
  a.dupd = dupd;
  a.dloc = dloc;
  a.eps = s->eps;
  a.gq = gr->q;
  a.gk = gr->k;
  a.gv = gr->v;
  a.gqp = gr->q_points;
  a.gkp = gr->k_points;
  a.gvp = gr->v_points;
  a.grot = gr->rotation;
  a.gtr = gr->translation;
  a.gwraw = gr->point_weight_raw;
  a.gwpair = gr->w_pair;
  a.gzl = gr->zl;
  a.gzr = gr->zr;
  a.gwout = gr->w_out;
  a.gbout = gr->b_out;
  hipError_t e;
  const int BN = L.B * L.N;
  hipLaunchKernelGGL(bw_prep_kernel, dim3((L.N + kPrepRows - 1) / kPrepRows, L.H, L.B), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_pairs_inst(a, 0, st)) != hipSuccess) return e;
  // DFEAT[bn][f] = sum_c dU[bn][c] w_out[f][c]
  GemmArgs g1{dupd, a.wout, (float*)(a.ws + L.off_dfeat), BN, L.F, L.Cout, 1, L.Cout, 1, 1, L.Cout, L.F, 0};
  if ((e = launch_gemm(g1, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(bw_epi_kernel, dim3(BN), dim3(64), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // [dW; db][f][c] = sum_bn FEAT[bn][f] dU[bn][c], split over bn
  const size_t slab = (size_t)(L.F + 1) * L.Cout;
  GemmArgs g2{(const float*)(a.ws + L.off_feat), dupd, (float*)(a.ws + L.off_dwpart), L.F + 1, L.Cout, BN, L.ksplit,
              1, L.F + 1, L.Cout, 1, L.Cout, slab};
  if ((e = launch_gemm(g2, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(bw_sum_slabs_kernel, dim3((unsigned)((slab - L.Cout + 255) / 256)), dim3(256), 0, st,
                     (const float*)(a.ws + L.off_dwpart), a.gwout, slab - L.Cout, L.ksplit, slab);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bw_sum_slabs_kernel, dim3((L.Cout + 255) / 256), dim3(256), 0, st,
                     (const float*)(a.ws + L.off_dwpart) + (slab - L.Cout), a.gbout, (size_t)L.Cout, L.ksplit, slab);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_pairs_inst(a, 1, st)) != hipSuccess) return e;
  if ((e = launch_pairs_inst(a, 2, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(bw_inputs_kernel, dim3(BN), dim3(64), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bw_params_part_kernel, dim3(L.H, kBwParamChunks), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bw_params_kernel, dim3(L.H), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace fipa
