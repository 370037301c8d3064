// Kernel 2, fp32 path: fused masked online-softmax attention over the lifted
// rows, fp32 arithmetic throughout (VALU, no matrix cores).
//
// Logit (log2 units) for query i, key j in key tile t with centroid c_t:
//   s_ij = Qs_i . Ks_j                       scalar + pair columns (lifted rows)
//        - gamma log2e sum_p |(a_ip - c_t) - (b_jp - c_t)|^2
// which equals log2(e) * L_ijh of the IPA page ("Required behavior").  On
// this fp32 VALU path the point term is formed as a difference, then
// squared, from coordinates centred on the key tile: no expansion, hence no
// cancellation between large terms.
// Softmax over the permitted keys uses a running maximum (FlashAttention
// style); value points are aggregated relative to the tile centroid and the
// centroid term sum_j p_j c_t is carried separately.
//
// Grid (ceil(N/64), H, B), 256 threads: 64 queries x 4 column groups; per
// step of 32 keys the four threads of a query form 8 logits each and share
// them through LDS, then each runs the softmax over all 32 and accumulates
// its own output columns.
#include "common.h"

namespace fipa {

struct FlashF32Args {
  Layout L;
  const char* ws;
  float* o;
  float* lse;
};

constexpr int kF32Keys = 32;  // keys staged per step

// MDQ, MDV: compile-time bounds on D + R Cz and on the output row width, so
// that the per-key loops run over the columns a shape has (two instances:
// narrow rows, and up to kF32MaxDQ / kF32MaxDV)
template <int MDQ, int MDV>
__global__ __launch_bounds__(256) void flash_f32_kernel(FlashF32Args a) {
  constexpr int kF32DvPer = MDV / 4;
  const Layout& L = a.L;
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int qi = tid & 63, part = tid >> 6;
  const int i = qb * 64 + qi;
  const int N = L.N, H = L.H, P3 = 3 * L.P, DQ = L.D + L.RCz, KROW = L.KROW, DVP = L.VROWS;
  const int DO = L.DO, DPT = L.Dv + L.RCz;  // points start at DPT

  extern __shared__ float smem[];
  float* sk = smem;                       // [32][KROW]
  float* sv = smem + kF32Keys * KROW;     // [32][DVP]
  float* slog = sv + kF32Keys * DVP;      // [64][33] logits of the step's keys

  const Header* hd = reinterpret_cast<const Header*>(a.ws);
  const bool has_pm = hd->has_pair_mask != 0;
  const float gam = reinterpret_cast<const float*>(a.ws + L.off_gam)[h];
  const float gl = gam * kLog2e;
  const bool qin = i < N;

  float qv[MDQ];
  const float* qrow = reinterpret_cast<const float*>(a.ws + L.off_ql) + (((size_t)b * H + h) * L.NQpad + i) * L.DQP;
#pragma unroll
  for (int d = 0; d < MDQ; ++d) qv[d] = (qin && d < DQ) ? qrow[d] : 0.f;
  float av[15];
  const float* arow = reinterpret_cast<const float*>(a.ws + L.off_qa) + (((size_t)b * H + h) * L.NQpad + i) * 16;
#pragma unroll
  for (int g = 0; g < 15; ++g) av[g] = (qin && g < P3) ? arow[g] : 0.f;

  float ov[kF32DvPer];
#pragma unroll
  for (int e = 0; e < kF32DvPer; ++e) ov[e] = 0.f;
  float cs0 = 0.f, cs1 = 0.f, cs2 = 0.f;  // sum_j p_j c_t
  float m = -INFINITY, l = 0.f;

  const uint32_t* km = reinterpret_cast<const uint32_t*>(a.ws + L.off_km);
  const uint32_t* pmw = reinterpret_cast<const uint32_t*>(a.ws + L.off_pm);
  const float4* ck = reinterpret_cast<const float4*>(a.ws + L.off_ck);
  const float* kbase = reinterpret_cast<const float*>(a.ws + L.off_kt) + ((size_t)b * H + h) * L.NKpad * KROW;
  const float* vbase = reinterpret_cast<const float*>(a.ws + L.off_vt) + ((size_t)b * H + h) * L.NKpad * DVP;

  // query validity: bit of residue i in the key-mask words of its tile
  bool qvalid = false;
  if (qin) {
    int hf;
    const int bit = mask_bit_of_key(i & 63, &hf);
    qvalid = (km[((size_t)b * L.NT + (i >> 6)) * 2 + hf] >> bit) & 1u;
  }

  float dA[15];  // a - c_t for the current key tile
  float4 c4 = make_float4(0.f, 0.f, 0.f, 0.f);
  uint32_t w0 = 0, w1 = 0;
  const int nsteps = L.NKpad / kF32Keys;
  for (int st = 0; st < nsteps; ++st) {
    const int t = st >> 1;
    if ((st & 1) == 0) {
      c4 = ck[(size_t)b * L.NT + t];
#pragma unroll
      for (int g = 0; g < 15; ++g) {
        const float cc = (g % 3 == 0) ? c4.x : ((g % 3 == 1) ? c4.y : c4.z);
        dA[g] = (g < P3) ? av[g] - cc : 0.f;
      }
      if (has_pm) {
        const size_t o = (((size_t)b * L.NQpad + i) * L.NT + t) * 2;
        w0 = qin ? pmw[o] : 0u;
        w1 = qin ? pmw[o + 1] : 0u;
      } else {
        w0 = qvalid ? km[((size_t)b * L.NT + t) * 2] : 0u;
        w1 = qvalid ? km[((size_t)b * L.NT + t) * 2 + 1] : 0u;
      }
    }
    __syncthreads();
    const float* kt = kbase + (size_t)st * kF32Keys * KROW;
    const float* vt = vbase + (size_t)st * kF32Keys * DVP;
    for (int x = tid; x < kF32Keys * KROW / 4; x += 256)
      reinterpret_cast<float4*>(sk)[x] = reinterpret_cast<const float4*>(kt)[x];
    for (int x = tid; x < kF32Keys * DVP / 4; x += 256)
      reinterpret_cast<float4*>(sv)[x] = reinterpret_cast<const float4*>(vt)[x];
    __syncthreads();
    // logits of the step's 32 keys for this thread's query, 8 keys per
    // column group (keys part, part + 4, ...), shared through LDS; -inf for
    // a key that is not permitted
    for (int jl = part; jl < kF32Keys; jl += 4) {
      const int jj = (st & 1) * kF32Keys + jl;
      int hf;
      const int bit = mask_bit_of_key(jj, &hf);
      const bool perm = (((hf ? w1 : w0) >> bit) & 1u) != 0;
      float s = -INFINITY;
      if (perm) {
        const float* kr = sk + jl * KROW;
        // branch-free column loops (the LDS reads then go out together):
        // columns past DQ read column 0 against a zero query column, point
        // coordinates past 3P give a zero difference; four and three
        // independent partial sums
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d = 0; d < MDQ; ++d) s4[d & 3] = fmaf(qv[d], kr[d < DQ ? d : 0], s4[d & 3]);
        float d3[3] = {0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < 15; ++g) {
          const float df = g < P3 ? dA[g] - kr[DQ + (g < P3 ? g : 0)] : 0.f;
          d3[g % 3] = fmaf(df, df, d3[g % 3]);
        }
        s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        s = fmaf(-gl, (d3[0] + d3[1]) + d3[2], s);
      }
      slog[qi * (kF32Keys + 1) + jl] = s;
    }
    __syncthreads();
    for (int jl = 0; jl < kF32Keys; ++jl) {
      const float s = slog[qi * (kF32Keys + 1) + jl];
      if (s == -INFINITY) continue;  // not permitted
      if (s > m) {
        const float alpha = exp2f(m - s);  // m = -inf -> 0
        l *= alpha;
#pragma unroll
        for (int e = 0; e < kF32DvPer; ++e) ov[e] *= alpha;
        cs0 *= alpha; cs1 *= alpha; cs2 *= alpha;
        m = s;
      }
      const float p = exp2f(s - m);
      l += p;
      const float* vr = sv + jl * DVP;
#pragma unroll
      for (int e = 0; e < kF32DvPer; ++e) {
        const int d = e * 4 + part;
        ov[e] = fmaf(d < DO ? p : 0.f, vr[d < DO ? d : 0], ov[e]);
      }
      cs0 = fmaf(p, c4.x, cs0); cs1 = fmaf(p, c4.y, cs1); cs2 = fmaf(p, c4.z, cs2);
    }
  }
  if (!qin) return;
  const bool nonempty = l > 0.f;
  const float inv = nonempty ? 1.0f / l : 0.f;
  float* orow = a.o + (((size_t)b * N + i) * H + h) * DO;
#pragma unroll
  for (int e = 0; e < kF32DvPer; ++e) {
    const int d = e * 4 + part;
    if (d < DO) {
      float val = ov[e];
      if (d >= DPT) {
        const int x = (d - DPT) % 3;
        val += (x == 0) ? cs0 : ((x == 1) ? cs1 : cs2);
      }
      orow[d] = val * inv;
    }
  }
  if (part == 0) a.lse[((size_t)b * H + h) * N + i] = nonempty ? (m + log2f(l)) * kLn2 : -INFINITY;
}

hipError_t launch_flash_f32(const Layout& L, const void* ws, float* o, float* lse, hipStream_t st) {
  FlashF32Args a;
  a.L = L;
  a.ws = reinterpret_cast<const char*>(ws);
  a.o = o;
  a.lse = lse;
  const size_t shm = ((size_t)kF32Keys * (L.KROW + L.VROWS) + 64 * (kF32Keys + 1)) * sizeof(float);
  dim3 grid((L.N + 63) / 64, L.H, L.B);
  if (L.D + L.RCz <= 64 && L.DO <= 96)
    hipLaunchKernelGGL((flash_f32_kernel<64, 96>), grid, dim3(256), shm, st, a);
  else
    hipLaunchKernelGGL((flash_f32_kernel<kF32MaxDQ, kF32MaxDV>), grid, dim3(256), shm, st, a);
  return hipGetLastError();
}

}  // namespace fipa
