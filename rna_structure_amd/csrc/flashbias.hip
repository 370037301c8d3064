// Attention with a low-rank bias on gfx950 matrix cores (FlashBias: Fast
// Computation of Attention with Bias, atlas.scime.ai summary, Approach: the
// dense bias b_ij = phi_q(i) . phi_k(j) is carried by two factor tensors
// concatenated onto the queries and keys, so a flash-attention kernel over
// the widened rows never reads an [N, M] bias).
//
//   L_ij = scale q_i . k_j + phi_q(i) . phi_k(j),  O_i = softmax_j(L_ij) v_j
//
// Lifted rows (the key side written to the workspace by a lift pass, the
// query side built in the attention kernel's prologue, each query row being
// read once):
//   Q~_i = [scale log2(e) q_i | per factor r: hi, hi, lo of log2(e) phi_q,r(i)]
//   K~_j = [k_j               | per factor r: hi, lo, hi of phi_k,r(j)]
// in bf16, zero-padded to W = 16 NQS columns, so that Q~_i . K~_j is L_ij in
// log2 units with every factor product taken as hi.hi + hi.lo + lo.hi
// (hi = bf16(x), lo = bf16(x - hi)): a factor keeps ~16 significant bits, so
// exact factors with large entries (ALiBi's key position, squared norms of
// coordinates) stay exact to ~1e-5 relative instead of bf16's 4e-3.  Values
// are stored transposed per 64-key tile, keys permuted within every 16 as
// [0-3, 8-11, 4-7, 12-15] (the order in which a 32x32 accumulator lane holds
// them), plus one mask word per tile and wavefront half.
//
// Attention: a workgroup of four wavefronts takes 128 queries of one
// (batch, head); each wavefront owns 32.  Per 64-key tile staged in LDS:
//   S^T (keys x queries) = K~ Q~^T     v_mfma_f32_32x32x16_bf16, NQS K-steps
//                                      per 32-key block
//   online softmax in fp32 with exp2; the running maximum is raised only
//   when a row maximum exceeds it by more than 8 (log2 units), so the
//   probabilities stay below 2^8 and rescaling is rare
//   O^T += V~^T P^T                    v_mfma_f32_32x32x16_bf16, the
//                                      probabilities (rounded to bf16) taken
//                                      straight from the S^T accumulators
// The next tile's global loads are issued before the current tile's
// arithmetic and land in LDS after it.  Causal attention stops at the tile
// that holds the workgroup's last query.
#include "lds_copy.h"
#include "mfma_tile.h"

namespace fipa {

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr float kBiasLog2e = 1.4426950408889634f;
constexpr float kBiasLn2 = 0.6931471805599453f;
constexpr float kLazyMax = 16777216.0f;  // 2^24: largest per-lane tile weight sum kept without a new maximum

struct BiasLayout {
  int B, N, M, H, D, Dv, R, causal, bf, bfp;
  float scale;
  int NQS, NVB, W, KP, DVP, Npad, Mpad, MT;  // KP: key row pitch (W + 8, as in LDS)
  size_t off_k, off_v, off_m, total;
};

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

int pick_nqs(int w16) {
  const int opts[] = {2, 3, 4, 5, 8, 9, 16};
  for (int o : opts)
    if (w16 <= o) return o;
  return 0;
}
int pick_nvb(int v32) {
  const int opts[] = {1, 2, 4, 8};
  for (int o : opts)
    if (v32 <= o) return o;
  return 0;
}

bool make_bias_layout(const ipa_bias_shape* s, BiasLayout* L) {
  // dimensions were range-checked by the caller (N, M <= 2^30, D + 3R <= 256, Dv <= 256)
  L->B = (int)s->B; L->N = (int)s->N; L->M = (int)s->M; L->H = (int)s->H;
  L->D = (int)s->D; L->Dv = (int)s->Dv; L->R = (int)s->R; L->causal = s->causal != 0;
  L->bf = s->dtype == IPA_BF16;
  L->bfp = s->phi_dtype == IPA_BF16;
  L->scale = s->scale;
  L->NQS = pick_nqs((L->D + 3 * L->R + 15) / 16);
  L->NVB = pick_nvb((L->Dv + 31) / 32);
  if (L->NQS == 0 || L->NVB == 0) return false;
  L->W = 16 * L->NQS;
  L->KP = L->W + 8;
  L->DVP = 32 * L->NVB;
  L->Npad = (s->N + 127) / 128 * 128;
  L->Mpad = (s->M + 63) / 64 * 64;
  L->MT = L->Mpad / 64;
  const size_t BH = (size_t)s->B * s->H;
  size_t off = 0;
  L->off_k = off; off = al256(off + BH * L->Mpad * L->KP * 2);
  L->off_v = off; off = al256(off + BH * L->Mpad * L->DVP * 72 / 64 * 2);
  L->off_m = off; off = al256(off + (size_t)s->B * L->MT * 2 * 4);
  L->total = off;
  return true;
}

// A uniform word through a scalar load (constant address space): it is not
// counted by the vector-memory counter that the tile copies are waited on with.
__device__ __forceinline__ uint32_t ld_scalar_u32(const uint32_t* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return *(const __attribute__((address_space(4))) uint32_t*)(uintptr_t)join_addr(hi, lo);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// Column c of a lifted row.  side 0: query row (q scaled, factors hi hi lo),
// side 1: key row (k, factors hi lo hi).
template <bool BF, bool BFP>
__device__ __forceinline__ float lifted(const BiasLayout& L, int side, const void* x, const void* phi, size_t xrow,
                                        size_t prow, int c) {
  if (c < L.D) {
    const float v = ld<BF>(x, xrow + c);
    return side == 0 ? v * (L.scale * kBiasLog2e) : v;
  }
  const int idx = c - L.D;
  if (idx >= 3 * L.R) return 0.f;
  const int r = idx / 3, part = idx - 3 * r;
  const float f = ld<BFP>(phi, prow + r) * (side == 0 ? kBiasLog2e : 1.0f);
  const float hi = bf16_bits_to_f32(f32_to_bf16_bits(f));
  const bool want_lo = side == 0 ? part == 2 : part == 1;
  return want_lo ? f - hi : hi;
}

// Lifted query (side 0) or key (side 1) rows: one thread per 8 columns.
template <bool BF, bool BFP>
__global__ __launch_bounds__(256) void bias_lift_rows_kernel(BiasLayout L, int side, const void* x, const void* phi,
                                                             char* ws) {
  // 32-bit indices: B H rows c8 < 2^31 (checked on the host)
  const uint32_t rows = side == 0 ? L.Npad : L.Mpad, n = side == 0 ? L.N : L.M;
  const uint32_t c8 = (side == 0 ? L.W : L.KP) / 8;  // key rows carry the 8 pad columns of the LDS tile
  const uint32_t idx = blockIdx.x * 256u + threadIdx.x;
  if (idx >= (uint32_t)L.B * L.H * rows * c8) return;
  const uint32_t rr = idx / c8, cc = idx - rr * c8;
  const uint32_t bh = rr / rows, i = rr - bh * rows;
  const uint32_t b = bh / L.H, h = bh - b * L.H;
  uint4 out = make_uint4(0, 0, 0, 0);
  if (i < n) {
    const size_t xrow = (((size_t)b * n + i) * L.H + h) * L.D;
    const size_t prow = (((size_t)b * n + i) * L.H + h) * L.R;
    const int c0 = 8 * cc;
    float f[8];
    if ((L.D & 7) == 0 && c0 + 8 <= L.D) {
      // eight q or k columns: one 16-byte (bf16) or two 16-byte (fp32) loads
      const float mul = side == 0 ? L.scale * kBiasLog2e : 1.0f;
      if constexpr (BF) {
        const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + xrow + c0);
        const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = __uint_as_float(w4[e] << 16) * mul;
          f[2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u) * mul;
        }
      } else {
        const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + xrow + c0);
        const float4 c = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + xrow + c0 + 4);
        f[0] = a.x * mul; f[1] = a.y * mul; f[2] = a.z * mul; f[3] = a.w * mul;
        f[4] = c.x * mul; f[5] = c.y * mul; f[6] = c.z * mul; f[7] = c.w * mul;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = lifted<BF, BFP>(L, side, x, phi, xrow, prow, c0 + e);
    }
    out = make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7]));
  }
  char* base = ws + L.off_k;  // (side 0, query rows, is lifted inside the attention kernel)
  reinterpret_cast<uint4*>(base)[idx] = out;
}

// Transposed value tiles [b][h][t][c][72] (64 keys and 8 pad columns, the
// LDS tile's layout), keys permuted within every 16
// (column kappa holds key vt_key_of_col(kappa)).  A workgroup takes one
// 64-key tile and 32 value columns of one (b, h): it reads the 64 rows'
// 32-column pieces, transposes them in LDS and writes 32 rows of 64 keys
// (8 threads per row, 16 bytes each).
template <bool BF>
__global__ __launch_bounds__(256) void bias_lift_v_kernel(BiasLayout L, const void* v, char* ws) {
  __shared__ float sT[64][33];
  const int cb = blockIdx.x % (L.DVP / 32);
  const int t = (blockIdx.x / (L.DVP / 32)) % L.MT;
  const int bh = blockIdx.x / ((L.DVP / 32) * L.MT);
  const int h = bh % L.H, b = bh / L.H;
  const int tid = threadIdx.x;
  {
    // thread: 8 consecutive columns of one key (one 16-byte bf16 or two
    // 16-byte fp32 loads when the row allows it)
    const int jj = tid >> 2, c0 = 8 * (tid & 3), j = t * 64 + jj, cg = 32 * cb + c0;
    float f[8];
    const size_t vrow = (((size_t)b * L.M + min(j, L.M - 1)) * L.H + h) * L.Dv;
    if ((L.Dv & 7) == 0 && cg + 8 <= L.Dv && j < L.M) {
      if constexpr (BF) {
        const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(v) + vrow + cg);
        const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = __uint_as_float(w4[e] << 16);
          f[2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u);
        }
      } else {
        const float4 x0 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(v) + vrow + cg);
        const float4 x1 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(v) + vrow + cg + 4);
        f[0] = x0.x; f[1] = x0.y; f[2] = x0.z; f[3] = x0.w; f[4] = x1.x; f[5] = x1.y; f[6] = x1.z; f[7] = x1.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = (cg + e < L.Dv && j < L.M) ? ld<BF>(v, vrow + cg + e) : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sT[jj][c0 + e] = f[e];
  }
  __syncthreads();
  const int cl = tid >> 3, k8 = tid & 7;
  float f[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = sT[vt_key_of_col(8 * k8 + e)][cl];
  // rows of 72 keys' width: 64 keys and the 8 pad columns of the LDS tile
  uint4* dst = reinterpret_cast<uint4*>(ws + L.off_v) + (((size_t)bh * L.MT + t) * L.DVP + 32 * cb + cl) * 9;
  dst[k8] = make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7]));
  if (k8 == 0) dst[8] = make_uint4(0, 0, 0, 0);
}

// Key-mask words: per (b, tile) two words; bit kb*16 + r of word h is key
// kb*32 + 8*(r/4) + 4*h + r%4 (the key that lane half h holds in register r
// of key block kb).
__global__ __launch_bounds__(256) void bias_mask_kernel(BiasLayout L, const uint8_t* km, char* ws) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)L.B * L.MT * 2) return;
  const int hw = (int)(idx & 1);
  const long bt = idx >> 1;
  const int t = (int)(bt % L.MT), b = (int)(bt / L.MT);
  uint32_t w = 0;
  for (int x = 0; x < 32; ++x) {
    const int kb = x >> 4, r = x & 15;
    const int j = t * 64 + kb * 32 + 8 * (r >> 2) + 4 * hw + (r & 3);
    const bool ok = j < L.M && (km == nullptr || km[(size_t)b * L.M + j] != 0);
    w |= (uint32_t)ok << x;
  }
  reinterpret_cast<uint32_t*>(ws + L.off_m)[idx] = w;
}

// Three wavefronts per SIMD where the instance's registers fit (168 each)
// without spilling, else no occupancy constraint (four, at 128 registers,
// measured slower for the D = 64 instance).
constexpr int bias_waves(int nqs, int nvb) {
  return ((nvb <= 2 && nqs <= 5) || (nvb == 1 && nqs <= 9) || (nvb == 4 && nqs == 2)) ? 3 : 1;
}

template <int NQS, int NVB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(bias_waves(NQS, NVB))))
void bias_attn_kernel(BiasLayout L, const char* ws, const void* qin, const void* pqin, float* o, float* lse) {
  constexpr int W = 16 * NQS, DVP = 32 * NVB;
  constexpr int KP = W + 8;   // LDS row pitch of the key tile (bf16)
  constexpr int VP = 64 + 8;  // LDS row pitch of the transposed value tile (bf16)
  // key and value tiles are copied global -> LDS as they lie in the workspace
  // (rows already at the LDS pitches), into two buffers
  constexpr int KT_BYTES = 64 * KP * 2, VT_BYTES = DVP * VP * 2;
  constexpr int KT_LDS = (KT_BYTES + 1023) / 1024 * 1024, VT_LDS = (VT_BYTES + 1023) / 1024 * 1024;
  constexpr int BUF = KT_LDS + VT_LDS, SB = 4 * 32 * 36 * 4;  // SB: output blocks after the last tile
  __shared__ __align__(1024) char smem[2 * BUF > SB ? 2 * BUF : SB];

  // the wavefront index is uniform: say so, so that the copy offsets live in scalar registers
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l32 = lane & 31,
            hf = lane >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  // causal: the query tiles with the most key tiles are launched first
  const int qt = L.causal ? (int)gridDim.x - 1 - (int)blockIdx.x : (int)blockIdx.x;
  const int q0 = qt * 128, i = q0 + w * 32 + l32;
  const size_t bh = (size_t)b * L.H + h;

  // query operand (B of S^T), lifted here from q and phi_q: lane (query i, half
  // hf) holds columns 16 ks + 8 hf .. +7 of [scale log2e q_i | hi hi lo of
  // log2e phi_q(i) per factor], zero for padding rows
  bf16x8_t bq[NQS];
  {
    const size_t xrow = (((size_t)b * L.N + i) * L.H + h) * L.D;
    const size_t prow = (((size_t)b * L.N + i) * L.H + h) * L.R;
    const float mul = L.scale * kBiasLog2e;
#pragma unroll
    for (int ks = 0; ks < NQS; ++ks) {
      const int c0 = 16 * ks + 8 * hf;
      float f[8];
      if (i < L.N && (L.D & 7) == 0 && c0 + 8 <= L.D) {
        // eight q columns: one 16-byte (bf16) or two 16-byte (fp32) loads
        if (L.bf) {
          const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(qin) + xrow + c0);
          const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            f[2 * e] = __uint_as_float(w4[e] << 16) * mul;
            f[2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u) * mul;
          }
        } else {
          const float4 a0 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(qin) + xrow + c0);
          const float4 a1 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(qin) + xrow + c0 + 4);
          f[0] = a0.x * mul; f[1] = a0.y * mul; f[2] = a0.z * mul; f[3] = a0.w * mul;
          f[4] = a1.x * mul; f[5] = a1.y * mul; f[6] = a1.z * mul; f[7] = a1.w * mul;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = c0 + e;
          f[e] = 0.f;
          if (i < L.N) {
            if (L.bf) f[e] = L.bfp ? lifted<true, true>(L, 0, qin, pqin, xrow, prow, c) : lifted<true, false>(L, 0, qin, pqin, xrow, prow, c);
            else f[e] = L.bfp ? lifted<false, true>(L, 0, qin, pqin, xrow, prow, c) : lifted<false, false>(L, 0, qin, pqin, xrow, prow, c);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) bq[ks][e] = (__bf16)f[e];
    }
  }

  const char* ktg = ws + L.off_k + bh * L.MT * (size_t)KT_BYTES;
  const char* vtg = ws + L.off_v + bh * L.MT * (size_t)VT_BYTES;
  const uint32_t* mw = reinterpret_cast<const uint32_t*>(ws + L.off_m) + (size_t)b * L.MT * 2;
  const int tend = L.causal ? min(L.MT, (min(q0 + 127, L.N - 1) >> 6) + 1) : L.MT;

  f32x16_t oacc[NVB];
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[vb][r] = 0.f;
  float m = -INFINITY, l = 0.f;

  // causal attention walks the key tiles from the diagonal back to the first:
  // a bias that grows with the key index (ALiBi) then sets the running maximum
  // on the first tile and hardly ever raises it again
  const int t0 = L.causal ? tend - 1 : 0, dt = L.causal ? -1 : 1;
  dma_tile<KT_BYTES, 4>(ktg + (size_t)t0 * KT_BYTES, smem, w, lane);
  dma_tile<VT_BYTES, 4>(vtg + (size_t)t0 * VT_BYTES, smem + KT_LDS, w, lane);
  for (int it = 0; it < tend; ++it) {
    const int t = t0 + dt * it;
    // tile t has landed (every wavefront waits for its own copies) and every
    // wavefront is done with the previous tile, whose buffer the next copies refill
    wait_vmcnt<0>();
    __syncthreads();
    if (it + 1 < tend) {
      char* nb = smem + ((it + 1) & 1) * BUF;
      dma_tile<KT_BYTES, 4>(ktg + (size_t)(t + dt) * KT_BYTES, nb, w, lane);
      dma_tile<VT_BYTES, 4>(vtg + (size_t)(t + dt) * VT_BYTES, nb + KT_LDS, w, lane);
    }
    const uint16_t* sK = reinterpret_cast<const uint16_t*>(smem + (it & 1) * BUF);
    const uint16_t* sV = reinterpret_cast<const uint16_t*>(smem + (it & 1) * BUF + KT_LDS);

    // causal: a tile whose first key is past the wavefront's last query adds nothing
    if (L.causal && t * 64 > q0 + w * 32 + 31) continue;

    // S^T for the tile's two 32-key blocks
    f32x16_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
      const uint16_t* krow = &sK[(kb * 32 + l32) * KP + 8 * hf];
#pragma unroll
      for (int ks = 0; ks < NQS; ++ks)
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(krow + 16 * ks)), bq[ks], sacc[kb], 0, 0, 0);
    }

    // masks: key mask word of this lane half; causal keys beyond the query
    const uint32_t w0 = ld_scalar_u32(mw + 2 * t), w1 = ld_scalar_u32(mw + 2 * t + 1);
    const uint32_t word = hf ? w1 : w0;
    const bool diag = L.causal && t * 64 + 63 > q0 + w * 32;
    float s[32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb * 16 + r] = sacc[kb][r];
    if ((w0 & w1) != 0xFFFFFFFFu) {
#pragma unroll
      for (int x = 0; x < 32; ++x) s[x] = ((word >> x) & 1u) ? s[x] : -INFINITY;
    }
    if (diag) {
      // key kb*32 + 8*(r/4) + 4*hf + r%4 of the tile is permitted up to query i
      const int lim = i - t * 64 - 4 * hf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[kb * 16 + r] = (kb * 32 + 8 * (r >> 2) + (r & 3) <= lim) ? s[kb * 16 + r] : -INFINITY;
    }
    // Probabilities against the running maximum m as it stands; the row
    // maximum of the tile is only computed (and m raised) when a row has no
    // reference yet (m = -inf) or when the tile's weights of a lane sum to
    // more than kLazyMax (a weight above it, or infinite): the weights then
    // stay below 2^24, which bf16 operands and fp32 sums hold, and most tiles
    // need neither the maximum nor its exchange between the lane halves.
    // l sums the bf16-rounded weights that the value product multiplies
    // (two at a time, v_dot2 against ones, fp32 accumulation), so the weights
    // applied to V sum to one to fp32 rounding; the log-sum-exp then carries
    // their rounding (below 2^-9 relative in l)
    bf16x8_t pb[4];
    float ps;
    auto weights = [&](float ref) {
#pragma unroll
      for (int x = 0; x < 32; ++x) pb[x >> 3][x & 7] = (__bf16)__builtin_amdgcn_exp2f(s[x] - ref);
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[j], pb[j], 0, 1), one2, ps0, false);
        ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[j], pb[j], 2, 3), one2, ps1, false);
        ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[j], pb[j], 4, 5), one2, ps0, false);
        ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[j], pb[j], 6, 7), one2, ps1, false);
      }
      ps = ps0 + ps1;
    };
    bool exact = m == -INFINITY;
    if (!__any(exact)) {
      weights(m);
      exact = !(ps <= kLazyMax);
    }
    if (__any(exact)) {
      float mt = s[0];
#pragma unroll
      for (int x = 1; x < 32; ++x) mt = fmaxf(mt, s[x]);
      {
        // the other lane half holds the same queries' other 32 keys
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
        mt = fmaxf(mt, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
      }
      if (mt > m + 8.0f) {
        // first permitted key of the row, or a maximum that grew by more than 8
        const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mt);
        m = mt;
        l *= alpha;
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[vb][r] *= alpha;
      }
      // while no key of the row has been permitted, m is -inf and so is every
      // s: subtracting 0 instead keeps exp2(-inf) = 0
      weights(m == -INFINITY ? 0.f : m);
    }
    l += ps;

    // O^T += V~^T P^T: K-step j covers keys 16 j .. 16 j + 15 of the tile
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        const uint4 a = *reinterpret_cast<const uint4*>(&sV[(32 * vb + l32) * VP + 16 * j + 8 * hf]);
        oacc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), pb[j], oacc[vb], 0, 0, 0);
      }
  }

  l += __shfl_xor(l, 32);
  const bool empty = !(l > 0.f);
  const float inv = empty ? 0.f : 1.0f / l;
  if (hf == 0 && i < L.N) lse[bh * L.N + i] = empty ? -INFINITY : (m + log2f(l)) * kBiasLn2;
  wait_vmcnt<0>();  // no tile copy is still in flight when the workgroup ends
  if ((L.Dv & 3) == 0) {
    // registers 4g .. 4g+3 of a block are value columns 8g + 4 hf .. +3 of
    // the lane's query: one 16-byte store each, straight from the registers
    // (uniform condition: no wavefront takes the barrier below)
    if (i < L.N) {
      float* orow = o + (((size_t)b * L.N + i) * L.H + h) * L.Dv;
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = 32 * vb + 8 * g + 4 * hf;
          if (c < L.Dv)
            *reinterpret_cast<float4*>(orow + c) = make_float4(oacc[vb][4 * g] * inv, oacc[vb][4 * g + 1] * inv,
                                                               oacc[vb][4 * g + 2] * inv, oacc[vb][4 * g + 3] * inv);
        }
    }
    return;
  }
  // other widths: O^T (value columns x this wavefront's 32 queries) through
  // LDS, one block of 32 columns at a time, so that every query row is
  // written as whole 128-byte pieces of consecutive columns
  __syncthreads();  // the last tile's LDS reads are done in every wavefront
  float* so = reinterpret_cast<float*>(smem) + w * 32 * 36;
  const int cq = lane & 7;  // 16-byte piece of a row
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(&so[l32 * 36 + 8 * g + 4 * hf]) =
          make_float4(oacc[vb][4 * g] * inv, oacc[vb][4 * g + 1] * inv, oacc[vb][4 * g + 2] * inv,
                      oacc[vb][4 * g + 3] * inv);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int qq = 8 * x + (lane >> 3), iq = q0 + w * 32 + qq, c = 32 * vb + 4 * cq;
      const float4 v4 = *reinterpret_cast<const float4*>(&so[qq * 36 + 4 * cq]);
      if (iq < L.N && c < L.Dv) {
        float* orow = o + (((size_t)b * L.N + iq) * L.H + h) * L.Dv;
        if ((L.Dv & 3) == 0) {
          *reinterpret_cast<float4*>(orow + c) = v4;
        } else {
          orow[c] = v4.x;
          if (c + 1 < L.Dv) orow[c + 1] = v4.y;
          if (c + 2 < L.Dv) orow[c + 2] = v4.z;
          if (c + 3 < L.Dv) orow[c + 3] = v4.w;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int NQS, int NVB>
void launch_attn(const BiasLayout& L, const char* ws, const void* q, const void* pq, float* o, float* lse,
                 hipStream_t st) {
  hipLaunchKernelGGL((bias_attn_kernel<NQS, NVB>), dim3(L.Npad / 128, L.H, L.B), dim3(256), 0, st, L, ws, q, pq, o, lse);
}

template <int NQS>
bool dispatch_nvb(const BiasLayout& L, const char* ws, const void* q, const void* pq, float* o, float* lse,
                  hipStream_t st) {
  switch (L.NVB) {
    case 1: launch_attn<NQS, 1>(L, ws, q, pq, o, lse, st); return true;
    case 2: launch_attn<NQS, 2>(L, ws, q, pq, o, lse, st); return true;
    case 4: launch_attn<NQS, 4>(L, ws, q, pq, o, lse, st); return true;
    case 8: launch_attn<NQS, 8>(L, ws, q, pq, o, lse, st); return true;
  }
  return false;
}

}  // namespace

size_t bias_workspace_bytes(const ipa_bias_shape* s) {
  BiasLayout L;
  return make_bias_layout(s, &L) ? L.total : 0;
}

bool bias_supported(const ipa_bias_shape* s) {
  BiasLayout L;
  return make_bias_layout(s, &L);
}

hipError_t launch_bias_attention(const ipa_bias_shape* s, const void* q, const void* k, const void* v,
                                 const void* phi_q, const void* phi_k, const uint8_t* key_mask, float* o, float* lse,
                                 void* ws, hipStream_t st) {
  BiasLayout L;
  if (!make_bias_layout(s, &L)) return hipErrorInvalidValue;
  char* w = reinterpret_cast<char*>(ws);
  // one thread per 16-byte piece of the key rows, KP wide (with the LDS pad columns)
  const long nk = (long)L.B * L.H * L.Mpad * (L.KP / 8);
  const long nv = (long)L.B * L.H * L.MT * (L.DVP / 32), nm = (long)L.B * L.MT * 2;
  auto rows = [&](auto kern) {  // key rows (the query rows are lifted inside the attention kernel)
    hipLaunchKernelGGL(kern, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0, st, L, 1, k, phi_k, w);
  };
  if (L.bf) {
    if (L.bfp) rows(bias_lift_rows_kernel<true, true>); else rows(bias_lift_rows_kernel<true, false>);
    hipLaunchKernelGGL(bias_lift_v_kernel<true>, dim3((unsigned)nv), dim3(256), 0, st, L, v, w);
  } else {
    if (L.bfp) rows(bias_lift_rows_kernel<false, true>); else rows(bias_lift_rows_kernel<false, false>);
    hipLaunchKernelGGL(bias_lift_v_kernel<false>, dim3((unsigned)nv), dim3(256), 0, st, L, v, w);
  }
  hipLaunchKernelGGL(bias_mask_kernel, dim3((unsigned)((nm + 255) / 256)), dim3(256), 0, st, L, key_mask, w);
  bool ok = false;
  switch (L.NQS) {
    case 2: ok = dispatch_nvb<2>(L, w, q, phi_q, o, lse, st); break;
    case 3: ok = dispatch_nvb<3>(L, w, q, phi_q, o, lse, st); break;
    case 4: ok = dispatch_nvb<4>(L, w, q, phi_q, o, lse, st); break;
    case 5: ok = dispatch_nvb<5>(L, w, q, phi_q, o, lse, st); break;
    case 8: ok = dispatch_nvb<8>(L, w, q, phi_q, o, lse, st); break;
    case 9: ok = dispatch_nvb<9>(L, w, q, phi_q, o, lse, st); break;
    case 16: ok = dispatch_nvb<16>(L, w, q, phi_q, o, lse, st); break;
  }
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fipa
