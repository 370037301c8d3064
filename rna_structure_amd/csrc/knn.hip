// k-nearest-neighbour distogram of residue positions, streamed block-wise
// over the candidates (FlashIPA rebuttal, paperhub page, answer to Q6: only
// the k nearest neighbours' distances are kept, (B, L, k, n_bins); the
// neighbours may be found block-wise in a streaming fashion).  No L x L
// array exists; memory is the O(L k) output.
//
// One wavefront owns G = 8 consecutive query residues of one sample.  Its 64
// lanes walk the candidates of that sample 64 at a time in increasing index
// order; the G query positions are wave-uniform, so each lane forms the G
// squared distances of its candidate with scalar operands (ALU bound: the
// candidate block is read once per wavefront and reused G times).
//
// Per query the wavefront keeps a threshold tau and an LDS buffer of up to
// 256 candidates that passed it.  A step appends every lane whose d2 passes
// (ballot + prefix count inside one uniform branch per query).  When a buffer
// fills, an exact rank selection keeps its k best keys (d2, then index) in
// order and lowers tau to the k-th one.  Candidates arrive in increasing
// index order, so a later candidate with the same d2 as the k-th kept one
// loses the tie: after a selection the test is d2 < d2_k, written as
// d2 <= tau with tau the float just below d2_k.  Before the walk, tau is the
// k-th smallest d2 of a 64-residue window around the queries, taken
// inclusively (any k candidates bound the final k-th distance from above);
// for chain molecules it is already close to the final value, so the walk
// buffers few candidates.  A last selection orders the survivors.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/flashipa.h"

namespace fipa {
namespace {

constexpr int kKnnG = 8;       // query residues per wavefront
constexpr int kKnnCap = 256;   // buffered candidates per query
constexpr int kKnnWaves = 4;   // wavefronts per workgroup
constexpr int kKnnMaxK = 64;

struct KnnArgs {
  const float* t;        // [B,N,3]
  const uint8_t* mask;   // [B,N] or null
  int32_t* idx;          // [B,N,k]
  float* dist;           // [B,N,k] or null
  void* dgram;           // [B,N,k,nbins] or null
  int N, k, nbins;
  int groups;            // ceil(N / G) query groups per sample
  int waves;             // B * groups
  float width;           // fl32(dmax / nbins)
  int bf16;              // dgram element type
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Order key of a buffered candidate: (d2 bits, index).  d2 >= 0, so its bits
// order like the value; a d2 word of ~0u marks an entry that is not a
// candidate (the query itself) and sorts after every candidate.
__device__ __forceinline__ uint64_t key_of(uint2 e) { return ((uint64_t)e.x << 32) | e.y; }

// fp32 squared distance of candidate (x,y,z) from query (qx,qy,qz):
// ((dx*dx + dy*dy) + dz*dz), each operation rounded on its own.
__device__ __forceinline__ float sqdist(float x, float y, float z, float qx, float qy, float qz) {
#pragma clang fp contract(off)
  const float dx = x - qx, dy = y - qy, dz = z - qz;
  return (dx * dx + dy * dy) + dz * dz;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Keeps the (at most k) smallest candidate keys of buf[0..n), n <= 256,
// sorted at buf[0..); returns how many were kept (wave-uniform).
__device__ int select_topk(uint2* buf, int n, int k, int lane) {
  uint2 e[4];
  uint64_t ke[4];
  int rank[4];
  bool live[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int p = lane + 64 * r;
    e[r] = p < n ? buf[p] : make_uint2(~0u, ~0u);
    ke[r] = key_of(e[r]);
    live[r] = p < n && e[r].x != ~0u;
    rank[r] = 0;
  }
  const int rows = (n + 63) >> 6;
  if (rows <= 1) {
    for (int f = 0; f < n; ++f) rank[0] += key_of(buf[f]) < ke[0] ? 1 : 0;
  } else {
    for (int f = 0; f < n; ++f) {
      const uint64_t v = key_of(buf[f]);
#pragma unroll
      for (int r = 0; r < 4; ++r) rank[r] += v < ke[r] ? 1 : 0;
    }
  }
  int nlive = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) nlive += __popcll(__ballot(live[r]));
  wave_sync();
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (live[r] && rank[r] < k) buf[rank[r]] = e[r];
  wave_sync();
  return __builtin_amdgcn_readfirstlane(nlive < k ? nlive : k);
}

__device__ __forceinline__ void load_candidate(const float* tb, const uint8_t* mb, int j, int N, float& x, float& y,
                                               float& z) {
  const float qnan = __int_as_float(0x7fc00000);
  x = y = z = qnan;  // NaN: fails every d2 <= tau test
  if (j < N && (!mb || mb[j])) {
    const float* p = tb + 3 * (size_t)j;
    x = p[0];
    y = p[1];
    z = p[2];
  }
}

__global__ __launch_bounds__(256) void knn_distogram_kernel(KnnArgs a) {
  __shared__ uint2 s_buf[kKnnWaves][kKnnG][kKnnCap];
  __shared__ int s_bin[kKnnWaves][kKnnMaxK];
  const int lane = threadIdx.x & 63;
  const int wl = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wid = blockIdx.x * kKnnWaves + wl;
  if (wid >= a.waves) return;
  const int N = a.N, k = a.k;
  const int b = wid / a.groups;
  const int i0 = (wid - b * a.groups) * kKnnG;
  const float* tb = a.t + (size_t)b * N * 3;
  const uint8_t* mb = a.mask ? a.mask + (size_t)b * N : nullptr;
  const float inf = __int_as_float(0x7f800000);

  float qx[kKnnG], qy[kKnnG], qz[kKnnG], tau[kKnnG];
  int cnt[kKnnG];
  bool act[kKnnG];
#pragma unroll
  for (int g = 0; g < kKnnG; ++g) {
    const int i = i0 + g;
    act[g] = i < N && (!mb || mb[i]);
    qx[g] = qy[g] = qz[g] = 0.0f;
    if (act[g]) {
      qx[g] = tb[3 * (size_t)i];
      qy[g] = tb[3 * (size_t)i + 1];
      qz[g] = tb[3 * (size_t)i + 2];
    }
    tau[g] = act[g] ? inf : -1.0f;
    cnt[g] = 0;
  }

  // Seed: tau = k-th smallest d2 over the window's candidates (+inf if fewer).
  {
    int w0 = i0 + kKnnG / 2 - 32;
    w0 = w0 < N - 64 ? w0 : N - 64;
    w0 = w0 > 0 ? w0 : 0;
    const int j = w0 + lane;
    float x, y, z;
    load_candidate(tb, mb, j, N, x, y, z);
#pragma unroll
    for (int g = 0; g < kKnnG; ++g) {
      if (!act[g]) continue;
      const float d2 = sqdist(x, y, z, qx[g], qy[g], qz[g]);
      const float v = (j == i0 + g || d2 != d2) ? inf : d2;
      int lt = 0;
      for (int c = 0; c < 64; ++c) lt += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), c)) < v ? 1 : 0;
      const float m = wave_max(lt < k ? v : -inf);
      tau[g] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(m)));
    }
  }

  // Walk all candidates in increasing index order, one block of 64 per step.
  float cx, cy, cz;
  load_candidate(tb, mb, lane, N, cx, cy, cz);
  for (int c0 = 0; c0 < N; c0 += 64) {
    const int j = c0 + lane;
    const float x = cx, y = cy, z = cz;
    load_candidate(tb, mb, j + 64, N, cx, cy, cz);  // next block, in flight during this one
#pragma unroll
    for (int g = 0; g < kKnnG; ++g) {
      const float d2 = sqdist(x, y, z, qx[g], qy[g], qz[g]);
      const bool pass = d2 <= tau[g];
      const uint64_t m = __ballot(pass);
      if (m) {
        uint2* buf = &s_buf[wl][g][0];
        if (pass) buf[cnt[g] + lanes_below(m)] = make_uint2(j == i0 + g ? ~0u : __float_as_uint(d2), (uint32_t)j);
        cnt[g] = __builtin_amdgcn_readfirstlane(cnt[g] + __popcll(m));
        if (cnt[g] > kKnnCap - 64) {
          wave_sync();
          cnt[g] = select_topk(buf, cnt[g], k, lane);
          if (cnt[g] == k) {
            const uint32_t kb = __builtin_amdgcn_readfirstlane(buf[k - 1].x);
            tau[g] = kb == 0u ? -1.0f : __uint_as_float(kb - 1u);
          }
        }
      }
    }
  }

  // Order the survivors and write the k slots of every query residue.
  const int nb = a.nbins;
  const int tot = k * nb;
  const int q64 = 64 / nb, r64 = 64 - q64 * nb;
  const int s_first = lane / nb, c_first = lane - s_first * nb;
#pragma unroll
  for (int g = 0; g < kKnnG; ++g) {
    const int i = i0 + g;
    if (i >= N) break;
    uint2* buf = &s_buf[wl][g][0];
    wave_sync();
    const int n = act[g] ? select_topk(buf, cnt[g], k, lane) : 0;
    const size_t row = (size_t)b * N + i;
    int jj = -1, bin = -1;
    float d = inf;
    if (lane < n) {
      const uint2 e = buf[lane];
      d = sqrtf(__uint_as_float(e.x));
      jj = (int)e.y;
      const float q = d / a.width;
      bin = q >= (float)nb ? nb - 1 : (int)q;
    }
    if (lane < k) {
      a.idx[row * k + lane] = jj;
      if (a.dist) a.dist[row * k + lane] = d;
      s_bin[wl][lane] = bin;
    }
    if (a.dgram) {
      wave_sync();
      int s = s_first, c = c_first;
      if (a.bf16) {
        uint16_t* out = (uint16_t*)a.dgram + row * tot;
        for (int e2 = lane; e2 < tot; e2 += 64) {
          out[e2] = s_bin[wl][s] == c ? (uint16_t)0x3F80 : (uint16_t)0;
          c += r64;
          s += q64;
          if (c >= nb) { c -= nb; ++s; }
        }
      } else {
        float* out = (float*)a.dgram + row * tot;
        for (int e2 = lane; e2 < tot; e2 += 64) {
          out[e2] = s_bin[wl][s] == c ? 1.0f : 0.0f;
          c += r64;
          s += q64;
          if (c >= nb) { c -= nb; ++s; }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_knn(const ipa_knn_shape* s, const float* t, const uint8_t* mask, int32_t* idx, float* dist,
                      void* dgram, hipStream_t st) {
  KnnArgs a;
  a.t = t;
  a.mask = mask;
  a.idx = idx;
  a.dist = dist;
  a.dgram = dgram;
  a.N = (int)s->N;
  a.k = (int)s->k;
  a.nbins = (int)s->nbins;
  a.groups = (int)((s->N + kKnnG - 1) / kKnnG);
  a.waves = (int)(s->B * a.groups);
  a.width = s->dmax / (float)s->nbins;  // fp32 division, correctly rounded
  a.bf16 = s->dgram_dtype == IPA_BF16;
  const int blocks = (a.waves + kKnnWaves - 1) / kKnnWaves;
  hipLaunchKernelGGL(knn_distogram_kernel, dim3(blocks), dim3(64 * kKnnWaves), 0, st, a);
  return hipGetLastError();
}

}  // namespace fipa
