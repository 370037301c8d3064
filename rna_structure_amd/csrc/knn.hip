// k-nearest-neighbour distogram of residue positions, streamed block-wise
// over the candidates (FlashIPA rebuttal, paperhub page, answer to Q6: only
// the k nearest neighbours' distances are kept, (B, L, k, n_bins); the
// neighbours may be found block-wise in a streaming fashion).  No L x L
// array exists; memory is the O(L k) output.
//
// A group of G = 8 consecutive query residues of one sample is owned by S
// wavefronts (S = 1, 2 or 4; more on small grids), each walking 1/S of the
// candidate blocks.  The 64 lanes of a wavefront take the candidates 64 at a
// time in increasing index order and form the 8 squared distances of their
// candidate against the query positions held in registers (ALU bound: a
// candidate block is read once and used 8 times).
//
// Per query a wavefront keeps a threshold tau and an LDS buffer of up to 256
// candidate keys (d2 bits << 32 | index) that passed it.  One ballot per
// query and step finds the passing lanes; only when some lane passes does the
// step append (prefix count), and a buffer past 192 entries is cut by an exact
// rank selection to its k best keys, which lowers tau to the float just below
// the k-th d2: later candidates have larger indices, so an equal d2 loses the
// tie and the strict test stays exact.  Before the walk tau is (just above)
// the k-th smallest d2 among the candidates of a 64-residue window around the
// queries, taken inclusively -- any k candidates bound the final k-th
// distance from above -- found by a bitwise search with 16 lanes per query
// and DPP row sums; for chain molecules sequence neighbours are spatial
// neighbours, so few candidates are ever buffered.  At the end the S buffers
// of a query are gathered and one selection orders them; the rows of the
// group are contiguous in every output and written by flat loops.
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
  int waves;             // B * groups: query groups in the grid
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

// A buffered candidate is its order key, (d2 bits) << 32 | index: d2 >= 0,
// so the key orders like (d2, index).  A d2 word of ~0u marks an entry that
// is not a candidate (the query itself, or padding) and sorts after every
// candidate.
constexpr uint64_t kDeadKey = ~0ull;
__device__ __forceinline__ uint64_t make_key(uint32_t d2bits, uint32_t j) { return ((uint64_t)d2bits << 32) | j; }
__device__ __forceinline__ bool key_live(uint64_t key) { return (uint32_t)(key >> 32) != ~0u; }

// fp32 squared distance of candidate (x,y,z) from query (qx,qy,qz):
// ((dx*dx + dy*dy) + dz*dz), each operation rounded on its own.
__device__ __forceinline__ float sqdist(float x, float y, float z, float qx, float qy, float qz) {
#pragma clang fp contract(off)
  const float dx = x - qx, dy = y - qy, dz = z - qz;
  return (dx * dx + dy * dy) + dz * dz;
}

// Keeps the (at most k) smallest candidate keys of buf[0..n), n <= 256,
// sorted at buf[0..); returns how many were kept (wave-uniform).  Every lane
// ranks its (up to four) entries against all n keys, read as broadcasts.
__device__ __forceinline__ int select_topk(uint64_t* buf, int n, int k, int lane) {
  uint64_t ke[4];
  int rank[4];
  bool live[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int p = lane + 64 * r;
    const uint64_t v = buf[p];
    ke[r] = p < n ? v : kDeadKey;
    live[r] = key_live(ke[r]);
    rank[r] = 0;
  }
  const uint4* b4 = reinterpret_cast<const uint4*>(buf);
  if (n <= 32) {
    // one entry per lane: entries n..31 become dead keys (they rank nothing),
    // then all 32 broadcasts are in flight at once
    if (lane >= n && lane < 32) buf[lane] = kDeadKey;
    wave_sync();
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint4 w = b4[q];
      rank[0] += (((uint64_t)w.y << 32) | w.x) < ke[0] ? 1 : 0;
      rank[0] += (((uint64_t)w.w << 32) | w.z) < ke[0] ? 1 : 0;
    }
  } else if (n <= 64) {
    if (lane >= n) buf[lane] = kDeadKey;
    wave_sync();
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      const uint4 w = b4[q];
      rank[0] += (((uint64_t)w.y << 32) | w.x) < ke[0] ? 1 : 0;
      rank[0] += (((uint64_t)w.w << 32) | w.z) < ke[0] ? 1 : 0;
    }
  } else {
    int f = 0;
    for (; f + 8 <= n; f += 8) {
      uint64_t v[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint4 w = b4[(f >> 1) + u];
        v[2 * u] = ((uint64_t)w.y << 32) | w.x;
        v[2 * u + 1] = ((uint64_t)w.w << 32) | w.z;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) rank[r] += v[u] < ke[r] ? 1 : 0;
    }
    for (; f < n; ++f) {
      const uint64_t v = buf[f];
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
    if (live[r] && rank[r] < k) buf[rank[r]] = ke[r];
  wave_sync();
  return __builtin_amdgcn_readfirstlane(nlive < k ? nlive : k);
}

// Candidate j's position, NaN (fails every d2 <= tau test) when j is past the
// end or masked.  The loads are issued unconditionally for j < N so that the
// mask does not serialise them.
struct Cand {
  float x, y, z;
  uint32_t m;   // mask byte (ignored without a mask)
  bool inb;     // j < N
};

// mp is the mask, or any readable byte array when there is no mask.  The
// loads are issued unconditionally (clamped index) and their results are only
// looked at in use_candidate, so that a prefetch is not waited for at once.
__device__ __forceinline__ Cand fetch_candidate(const float* tb, const uint8_t* mp, int j, int N) {
  const int jc = j < N ? j : N - 1;
  const float* p = tb + 3 * (size_t)jc;
  Cand c;
  c.x = p[0];
  c.y = p[1];
  c.z = p[2];
  c.m = mp[jc];
  c.inb = j < N;
  return c;
}

__device__ __forceinline__ void use_candidate(const Cand& c, bool has_mask, float& x, float& y, float& z) {
  const float qnan = __int_as_float(0x7fc00000);
  const bool ok = c.inb & (!has_mask | (c.m != 0u));
  x = ok ? c.x : qnan;
  y = ok ? c.y : qnan;
  z = ok ? c.z : qnan;
}

// S wavefronts share one group of G query residues, each walking 1/S of the
// candidate blocks (S = 1, 2, 4; more splits when the grid is small), then
// their per-split best k are merged.  A workgroup holds 4 / S groups.
// Per-query state (position, tau, buffer fill) lives in LDS: the hot loop
// keeps the positions in vector registers (loaded once) and re-reads the
// eight thresholds each step; the rare append path walks the queries in a
// plain loop.
template <int S>
__global__ __launch_bounds__(256) void knn_distogram_kernel(KnnArgs a) {
  constexpr int GPW = kKnnWaves / S;
  __shared__ uint64_t s_buf[kKnnWaves][kKnnG][kKnnCap];
  __shared__ int s_cnt[kKnnWaves][kKnnG];
  __shared__ __align__(16) float s_tau[kKnnWaves][kKnnG];
  __shared__ int s_bin[kKnnWaves][kKnnG * kKnnMaxK];
  __shared__ float4 s_q[kKnnWaves][kKnnG];
  const int lane = threadIdx.x & 63;
  const int wl = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gl = wl / S, split = wl - gl * S;
  const int grp = blockIdx.x * GPW + gl;
  const bool live = grp < a.waves;
  if (S == 1 && !live) return;
  const int N = a.N, k = a.k;
  const int b = live ? grp / a.groups : 0;
  const int i0 = (grp - b * a.groups) * kKnnG;
  const float* tb = a.t + (size_t)b * N * 3;
  const uint8_t* mb = a.mask ? a.mask + (size_t)b * N : nullptr;
  const bool has_mask = mb != nullptr;
  const uint8_t* mp = has_mask ? mb : (const uint8_t*)tb;
  const float inf = __int_as_float(0x7f800000);

  // Lane g < G loads query g; act has bit g set when query g is a valid residue.
  uint32_t act = 0;
  if (live) {
    bool ok = false;
    if (lane < kKnnG) {
      const int i = i0 + lane;
      ok = i < N && (!mb || mb[i]);
      float4 q = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (ok) q = make_float4(tb[3 * (size_t)i], tb[3 * (size_t)i + 1], tb[3 * (size_t)i + 2], 0.0f);
      s_q[wl][lane] = q;
      s_tau[wl][lane] = ok ? inf : -1.0f;
      s_cnt[wl][lane] = 0;
    }
    act = (uint32_t)__ballot(ok);
    wave_sync();
  }
  // Seed from a 64-residue window around the queries.
  if (live) {
    int w0 = i0 + kKnnG / 2 - 32;
    w0 = w0 < N - 64 ? w0 : N - 64;
    w0 = w0 > 0 ? w0 : 0;
    const int j = w0 + lane;
    float x, y, z;
    use_candidate(fetch_candidate(tb, mp, j, N), has_mask, x, y, z);
    // Per query: tau = the k-th smallest d2 among the window's candidates
    // (+inf when it holds fewer than k), rounded up to the top 12 bits of its
    // encoding (exponent and 4 mantissa bits: at most 1/16 above): an upper
    // bound of the final k-th d2.  The 8 x 64 keys go through this wave's
    // part of the output-bin area so that 16 lanes serve each query (4 keys
    // per lane, two passes of 4 queries); counts are summed over the 16 lanes
    // of a row with DPP.
    constexpr int kLow = 19;
    uint32_t* sv = reinterpret_cast<uint32_t*>(&s_bin[wl][0]);
#pragma unroll
    for (int g = 0; g < kKnnG; ++g) {
      const float4 q = s_q[wl][g];
      const float d2 = sqdist(x, y, z, q.x, q.y, q.z);
      sv[g * 64 + lane] = __float_as_uint((j == i0 + g || d2 != d2) ? inf : d2) >> kLow;
    }
    wave_sync();
    const int row = lane >> 4, part = lane & 15;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int g = pass * 4 + row;
      const uint4 w = *reinterpret_cast<const uint4*>(&sv[g * 64 + part * 4]);
      uint32_t res = 0;
#pragma unroll
      for (int bit = 30 - kLow; bit >= 0; --bit) {
        const uint32_t lo = res | ((1u << bit) - 1u);
        int c = (w.x <= lo ? 1 : 0) + (w.y <= lo ? 1 : 0) + (w.z <= lo ? 1 : 0) + (w.w <= lo ? 1 : 0);
        c += __builtin_amdgcn_update_dpp(0, c, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
        c += __builtin_amdgcn_update_dpp(0, c, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
        c += __builtin_amdgcn_update_dpp(0, c, 0x124, 0xF, 0xF, false);  // row_ror:4
        c += __builtin_amdgcn_update_dpp(0, c, 0x128, 0xF, 0xF, false);  // row_ror:8 -> row total
        res = c < k ? (res | (1u << bit)) : res;
      }
      uint32_t tl = (res << kLow) | ((1u << kLow) - 1u);
      if (tl >= 0x7f800000u) tl = 0x7f800000u;  // an infinite k-th value stays +inf
      if (part == 0 && ((act >> g) & 1u)) s_tau[wl][g] = __uint_as_float(tl);
    }
    wave_sync();
  }

  if (live) {
    wave_sync();
    float qx[kKnnG], qy[kKnnG], qz[kKnnG];
#pragma unroll
    for (int g = 0; g < kKnnG; ++g) {
      const float4 q = s_q[wl][g];
      qx[g] = q.x;
      qy[g] = q.y;
      qz[g] = q.z;
    }
    // Walk this split's candidate blocks in increasing index order.
    const int nblk = (N + 63) >> 6;
    const int cb = (split * nblk / S) * 64, ce = ((split + 1) * nblk / S) * 64;
    Cand nx = fetch_candidate(tb, mp, cb + lane, N);
    for (int c0 = cb; c0 < ce; c0 += 64) {
      const int j = c0 + lane;
      float x, y, z;
      use_candidate(nx, has_mask, x, y, z);
      nx = fetch_candidate(tb, mp, j + 64, N);  // next block, in flight during this one
      const float4 ta = *(const float4*)&s_tau[wl][0];
      const float4 tc = *(const float4*)&s_tau[wl][4];
      const float tau[kKnnG] = {ta.x, ta.y, ta.z, ta.w, tc.x, tc.y, tc.z, tc.w};
      uint64_t any = 0;
#pragma unroll
      for (int g = 0; g < kKnnG; ++g) any |= __ballot(sqdist(x, y, z, qx[g], qy[g], qz[g]) <= tau[g]);
      if (!any) continue;
      // Append path: the same distances again, one query at a time.
#pragma unroll 1
      for (int g = 0; g < kKnnG; ++g) {
        const float4 q = s_q[wl][g];
        const float d2 = sqdist(x, y, z, q.x, q.y, q.z);
        const bool pass = d2 <= s_tau[wl][g];
        const uint64_t m = __ballot(pass);
        if (!m) continue;
        uint64_t* buf = &s_buf[wl][g][0];
        int n = __builtin_amdgcn_readfirstlane(s_cnt[wl][g]);
        if (pass) buf[n + lanes_below(m)] = make_key(j == i0 + g ? ~0u : __float_as_uint(d2), (uint32_t)j);
        n += __popcll(m);
        if (n > kKnnCap - 64) {
          wave_sync();
          n = select_topk(buf, n, k, lane);
          if (n == k) {
            const uint32_t kb = __builtin_amdgcn_readfirstlane((uint32_t)(buf[k - 1] >> 32));
            if (lane == 0) s_tau[wl][g] = kb == 0u ? -1.0f : __uint_as_float(kb - 1u);
          }
        }
        if (lane == 0) s_cnt[wl][g] = n;
        wave_sync();
      }
    }
  }
  // Final lists.  S = 1: one selection per query.  S > 1: split s takes the
  // queries g with g % S == s and gathers the other splits' buffers behind
  // its own (first cutting every buffer to its best k if they would not fit)
  // before one selection.
  if constexpr (S > 1) __syncthreads();
  if (live) {
    wave_sync();
#pragma unroll 1
    for (int g = split; g < kKnnG; g += S) {
      if (!((act >> g) & 1u)) continue;
      uint64_t* buf = &s_buf[wl][g][0];
      int n = __builtin_amdgcn_readfirstlane(s_cnt[wl][g]);
      if (S > 1) {
        int tot = n;
        for (int o = 1; o < S; ++o) tot += __builtin_amdgcn_readfirstlane(s_cnt[gl * S + (split + o) % S][g]);
        if (tot > kKnnCap) {
          n = select_topk(buf, n, k, lane);
          for (int o = 1; o < S; ++o) {
            const int src = gl * S + (split + o) % S;
            const int ns = select_topk(&s_buf[src][g][0], __builtin_amdgcn_readfirstlane(s_cnt[src][g]), k, lane);
            if (lane == 0) s_cnt[src][g] = ns;
          }
          wave_sync();
        }
        for (int o = 1; o < S; ++o) {
          const int src = gl * S + (split + o) % S;
          const int no = __builtin_amdgcn_readfirstlane(s_cnt[src][g]);
          for (int e = lane; e < no; e += 64) buf[n + e] = s_buf[src][g][e];
          n += no;
        }
        wave_sync();
      }
      n = select_topk(buf, n, k, lane);
      if (lane == 0) s_cnt[wl][g] = n;
    }
  }
  if constexpr (S > 1) __syncthreads();
  if (!live) return;
  wave_sync();

  // Outputs of the group's rows i0 .. i0+gv-1, contiguous in every output
  // array; the S wavefronts of the group share them.  Query g's final list
  // sits in the buffer of split g % S.
  const int gv = N - i0 < kKnnG ? N - i0 : kKnnG;
  const int nb = a.nbins;
  const size_t row0 = (size_t)b * N + i0;
  int* bins = &s_bin[gl][0];
  {
    const int np = gv * k;  // (query, slot) pairs
    int p = split * 64 + lane;
    int g = p / k, sl = p - g * k;
    const int gstep = (S * 64) / k, sstep = S * 64 - gstep * k;
    for (; p < np; p += S * 64) {
      const int owner = gl * S + g % S;
      const int n = ((act >> g) & 1u) ? s_cnt[owner][g] : 0;
      int jj = -1, bin = -1;
      float d = inf;
      if (sl < n) {
        const uint64_t e = s_buf[owner][g][sl];
        d = sqrtf(__uint_as_float((uint32_t)(e >> 32)));
        jj = (int)(uint32_t)e;
        const float q = d / a.width;
        bin = q >= (float)nb ? nb - 1 : (int)q;
      }
      a.idx[row0 * k + p] = jj;
      if (a.dist) a.dist[row0 * k + p] = d;
      bins[p] = bin;
      g += gstep;
      sl += sstep;
      if (sl >= k) { sl -= k; ++g; }
    }
  }
  if (!a.dgram) return;
  if constexpr (S > 1) __syncthreads(); else wave_sync();
  {
    const int ne = gv * k * nb;  // one-hot elements
    int e = split * 64 + lane;
    int p = e / nb, c = e - p * nb;
    const int pstep = (S * 64) / nb, cstep = S * 64 - pstep * nb;
    if (a.bf16) {
      uint16_t* out = (uint16_t*)a.dgram + row0 * k * nb;
#pragma unroll 4
      for (; e < ne; e += S * 64) {
        out[e] = bins[p] == c ? (uint16_t)0x3F80 : (uint16_t)0;
        p += pstep;
        c += cstep;
        if (c >= nb) { c -= nb; ++p; }
      }
    } else {
      float* out = (float*)a.dgram + row0 * k * nb;
#pragma unroll 4
      for (; e < ne; e += S * 64) {
        out[e] = bins[p] == c ? 1.0f : 0.0f;
        p += pstep;
        c += cstep;
        if (c >= nb) { c -= nb; ++p; }
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
  a.waves = (int)(s->B * a.groups);  // query groups in the grid
  a.width = s->dmax / (float)s->nbins;  // fp32 division, correctly rounded
  a.bf16 = s->dgram_dtype == IPA_BF16;
  // split the candidate walk of a group over several wavefronts while the
  // grid has fewer than ~2048 wavefronts (8 per CU) and every split keeps at
  // least 4 blocks of candidates
  const int64_t nblk = (s->N + 63) / 64;
  int S = 1;
  while (S < 4 && (int64_t)a.waves * S * 2 <= 2048 && nblk >= 8 * S) S *= 2;
  const int gpw = kKnnWaves / S;
  const int blocks = (a.waves + gpw - 1) / gpw;
  if (S == 1)
    hipLaunchKernelGGL(knn_distogram_kernel<1>, dim3(blocks), dim3(64 * kKnnWaves), 0, st, a);
  else if (S == 2)
    hipLaunchKernelGGL(knn_distogram_kernel<2>, dim3(blocks), dim3(64 * kKnnWaves), 0, st, a);
  else
    hipLaunchKernelGGL(knn_distogram_kernel<4>, dim3(blocks), dim3(64 * kKnnWaves), 0, st, a);
  return hipGetLastError();
}

}  // namespace fipa
