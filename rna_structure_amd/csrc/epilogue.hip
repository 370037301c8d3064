// Kernel 3 (epilogue): per residue i and head h, from the fused kernel's
// aggregates (IPA page, "Required behavior"):
//   local_ihq = R_i^T (g_ihq - t_i)            inverse frame transform
//   length_ihq = sqrt(|local_ihq|^2 + eps)     (zero for an empty neighbourhood)
//   pair_ih = sum_r zl_ir * o_zr_ihr            pair features from the factors
//   features = [scalar (H,Dv) | x (H,Q) | y | z | length (H,Q) | pair (H,Cz)]
//   update = features @ w_out + b_out, zero for an empty neighbourhood.
// Matrix-core path: the features of a block of residues are built in LDS
// (bf16) by coalesced work items and multiplied by w_out on MFMA (bf16
// operands, fp32 accumulation); w_out is first transposed once per call into
// the workspace so that every MFMA operand fragment is one 16-byte load.
// fp32 path: the same features in fp32 and a VALU product.
#include "common.h"
#include "lds_copy.h"

namespace fipa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct EpiArgs {
  Layout L;
  const float* o;
  const float* lse;
  const void *zl, *rot, *trans, *w_out, *b_out;
  const uint16_t* wt;  // [Cout][FP] bf16 (matrix-core path)
  float* update;
  float* local;
  float eps;
  int FP;  // LDS row pitch of the features (elements)
};

// A residue's neighbourhood is empty when no key is permitted to it (key
// mask, pair mask).  The attention kernels decide that from the mask bits
// alone, the same for every head, and then give lse = -inf, so head 0's
// log-sum-exp tells it for the residue.
__device__ __forceinline__ bool row_empty(const EpiArgs& a, int row) {
  const Layout& L = a.L;
  const int b = row / L.N, i = row % L.N;
  return !(a.lse[((size_t)b * L.H) * L.N + i] > -INFINITY);
}

// ---------------------------------------------------------------- w_out transpose
// wt[c][f] = w_out[f][c] (bf16 bits), zero for f in [F, FP).
__global__ __launch_bounds__(256) void transpose_wout_kernel(const uint16_t* w, uint16_t* wt, int F, int FP, int Cout) {
  __shared__ uint16_t tile[64][65];
  const int f0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  uint16_t v[16];  // all 16 loads of a thread in flight together
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int f = f0 + ty + 4 * k, c = c0 + tx;
    v[k] = (f < F && c < Cout) ? w[(size_t)f * Cout + c] : (uint16_t)0;
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) tile[ty + 4 * k][tx] = v[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int c = c0 + ty + 4 * k, f = f0 + tx;
    if (c < Cout && f < FP) wt[(size_t)c * FP + f] = tile[tx][ty + 4 * k];
  }
}

// ---------------------------------------------------------------- features
// Work items of one (row, head): ceil(Dv/4) scalar chunks, ceil(Cz/4) pair
// chunks, Q points; consecutive items read consecutive parts of the row's O.
template <bool BF, typename T>
__device__ __forceinline__ void feature_item(const EpiArgs& a, int row, int h, int it, bool empty, T* frow) {
  const Layout& L = a.L;
  const int H = L.H, Dv = L.Dv, Q = L.Q, Cz = L.Cz, R = L.R, RCz = L.RCz, DO = L.DO;
  const int nS = (Dv + 3) / 4, nP = (Cz + 3) / 4;
  const int offx = H * Dv, offy = offx + H * Q, offz = offy + H * Q, offl = offz + H * Q, offp = offl + H * Q;
  const float* orow = a.o + ((size_t)row * H + h) * DO;
  auto put = [&](int f, float v) {
    if constexpr (sizeof(T) == 2) frow[f] = __builtin_bit_cast(T, f32_to_bf16_bits(v));
    else frow[f] = v;
  };
  if (it < nS) {
    const int d0 = 4 * it;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (d0 + e < Dv) put(h * Dv + d0 + e, empty ? 0.f : orow[d0 + e]);
  } else if (it < nS + nP) {
    const int c0 = 4 * (it - nS);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c0 + e < Cz)
          acc[e] = fmaf(ld<BF>(a.zl, (size_t)row * RCz + r * Cz + c0 + e), orow[Dv + r * Cz + c0 + e], acc[e]);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (c0 + e < Cz) put(offp + h * Cz + c0 + e, empty ? 0.f : acc[e]);
  } else {
    const int q = it - nS - nP;
    const float gx = orow[Dv + RCz + 3 * q] - ld<BF>(a.trans, (size_t)row * 3);
    const float gy = orow[Dv + RCz + 3 * q + 1] - ld<BF>(a.trans, (size_t)row * 3 + 1);
    const float gz = orow[Dv + RCz + 3 * q + 2] - ld<BF>(a.trans, (size_t)row * 3 + 2);
    float Rm[9];
#pragma unroll
    for (int e = 0; e < 9; ++e) Rm[e] = ld<BF>(a.rot, (size_t)row * 9 + e);
    // R^T (g - t): column x of R dotted with (g - t)
    float x = Rm[0] * gx + Rm[3] * gy + Rm[6] * gz;
    float y = Rm[1] * gx + Rm[4] * gy + Rm[7] * gz;
    float z = Rm[2] * gx + Rm[5] * gy + Rm[8] * gz;
    float len = sqrtf(x * x + y * y + z * z + a.eps);
    if (empty) { x = y = z = len = 0.f; }
    float* lp = a.local + (((size_t)row * H + h) * Q + q) * 3;
    lp[0] = x; lp[1] = y; lp[2] = z;
    put(offx + h * Q + q, x);
    put(offy + h * Q + q, y);
    put(offz + h * Q + q, z);
    put(offl + h * Q + q, len);
  }
}

// Features of one (row, head) for the standard dimensions Dv=16, Cz=64,
// Q=8, R=2: the whole attention-output row (168 floats) is read with 42
// independent 16-byte loads and the features go to LDS as 16-byte stores.
constexpr int kFDv = 16, kFCz = 64, kFQ = 8, kFR = 2, kFDO = kFDv + kFR * kFCz + 3 * kFQ;
__host__ __device__ __forceinline__ bool fast_dims(const Layout& L) {
  return L.Dv == kFDv && L.Cz == kFCz && L.Q == kFQ && L.R == kFR;
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}
__device__ __forceinline__ void features_fast(const EpiArgs& a, int row, int h, bool empty, uint16_t* frow) {
  const int H = a.L.H;
  const float4* __restrict__ o4 = reinterpret_cast<const float4*>(a.o + ((size_t)row * H + h) * kFDO);
  float ov[kFDO];
#pragma unroll
  for (int k = 0; k < kFDO / 4; ++k) {
    const float4 v = o4[k];
    ov[4 * k] = v.x; ov[4 * k + 1] = v.y; ov[4 * k + 2] = v.z; ov[4 * k + 3] = v.w;
  }
  const uint4* __restrict__ z4 = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.zl) +
                                                                (size_t)row * kFR * kFCz);
  uint4 zv[kFR * kFCz / 8];
#pragma unroll
  for (int k = 0; k < kFR * kFCz / 8; ++k) zv[k] = z4[k];
  const uint16_t* __restrict__ rt = reinterpret_cast<const uint16_t*>(a.rot) + (size_t)row * 9;
  const uint16_t* __restrict__ tt = reinterpret_cast<const uint16_t*>(a.trans) + (size_t)row * 3;
  float Rm[9], tr[3];
#pragma unroll
  for (int e = 0; e < 9; ++e) Rm[e] = bf16_bits_to_f32(rt[e]);
#pragma unroll
  for (int e = 0; e < 3; ++e) tr[e] = bf16_bits_to_f32(tt[e]);
  const float keep = empty ? 0.f : 1.f;
  const int offx = H * kFDv, offy = offx + H * kFQ, offz = offy + H * kFQ, offl = offz + H * kFQ,
            offp = offl + H * kFQ;
  // scalar
#pragma unroll
  for (int k = 0; k < kFDv / 8; ++k) {
    uint4 v;
    v.x = pack_bf16(keep * ov[8 * k], keep * ov[8 * k + 1]);
    v.y = pack_bf16(keep * ov[8 * k + 2], keep * ov[8 * k + 3]);
    v.z = pack_bf16(keep * ov[8 * k + 4], keep * ov[8 * k + 5]);
    v.w = pack_bf16(keep * ov[8 * k + 6], keep * ov[8 * k + 7]);
    *reinterpret_cast<uint4*>(frow + h * kFDv + 8 * k) = v;
  }
  // pair: sum_r zl_r * o_zr_r
#pragma unroll
  for (int k = 0; k < kFCz / 8; ++k) {
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = 8 * k + e;
      float acc = 0.f;
#pragma unroll
      for (int r = 0; r < kFR; ++r) {
        const uint4 zz = zv[(r * kFCz + c) / 8];
        const uint32_t wd = (e >> 1) == 0 ? zz.x : ((e >> 1) == 1 ? zz.y : ((e >> 1) == 2 ? zz.z : zz.w));
        const float zlv = __uint_as_float((e & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
        acc = fmaf(zlv, ov[kFDv + r * kFCz + c], acc);
      }
      pv[e] = keep * acc;
    }
    uint4 v;
    v.x = pack_bf16(pv[0], pv[1]); v.y = pack_bf16(pv[2], pv[3]);
    v.z = pack_bf16(pv[4], pv[5]); v.w = pack_bf16(pv[6], pv[7]);
    *reinterpret_cast<uint4*>(frow + offp + h * kFCz + 8 * k) = v;
  }
  // points: R^T (g - t), lengths
  float lx[kFQ], ly[kFQ], lz[kFQ], ll[kFQ];
#pragma unroll
  for (int q = 0; q < kFQ; ++q) {
    const float gx = ov[kFDv + kFR * kFCz + 3 * q] - tr[0];
    const float gy = ov[kFDv + kFR * kFCz + 3 * q + 1] - tr[1];
    const float gz = ov[kFDv + kFR * kFCz + 3 * q + 2] - tr[2];
    const float x = Rm[0] * gx + Rm[3] * gy + Rm[6] * gz;
    const float y = Rm[1] * gx + Rm[4] * gy + Rm[7] * gz;
    const float z = Rm[2] * gx + Rm[5] * gy + Rm[8] * gz;
    lx[q] = keep * x; ly[q] = keep * y; lz[q] = keep * z;
    ll[q] = keep * sqrtf(x * x + y * y + z * z + a.eps);
  }
  float4* __restrict__ lp = reinterpret_cast<float4*>(a.local + ((size_t)row * H + h) * kFQ * 3);
#pragma unroll
  for (int k = 0; k < kFQ * 3 / 4; ++k) {
    float t4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = 4 * k + e, q = idx / 3, c = idx % 3;
      t4[e] = c == 0 ? lx[q] : (c == 1 ? ly[q] : lz[q]);
    }
    lp[k] = make_float4(t4[0], t4[1], t4[2], t4[3]);
  }
  auto st8 = [&](int off, const float* v) {
    uint4 u;
    u.x = pack_bf16(v[0], v[1]); u.y = pack_bf16(v[2], v[3]);
    u.z = pack_bf16(v[4], v[5]); u.w = pack_bf16(v[6], v[7]);
    *reinterpret_cast<uint4*>(frow + off) = u;
  };
  st8(offx + h * kFQ, lx);
  st8(offy + h * kFQ, ly);
  st8(offz + h * kFQ, lz);
  st8(offl + h * kFQ, ll);
}

// ---------------------------------------------------------------- matrix-core path
// RPW residues per workgroup, 8 RPW threads (RPW / 8 wavefronts).  Phase 1
// builds the features; phase 2 streams w_out^T through LDS in chunks of 64
// features (double-buffered, loaded cooperatively with 16-byte loads) and
// every wavefront accumulates 32x32 output tiles.
constexpr int kWChunk = 64;                 // features per w_out chunk
constexpr int kWPitch = kWChunk + 8;        // LDS pitch (elements) of a chunk row
template <int RPW>
__global__ __launch_bounds__(RPW * 8) void epilogue_mfma_kernel(EpiArgs a) {
  constexpr int NT_ = RPW * 8;     // threads
  constexpr int NW = NT_ / 64;     // wavefronts
  constexpr int RB = RPW / 32;     // 32-row blocks
  const Layout& L = a.L;
  extern __shared__ __attribute__((aligned(16))) uint16_t efeat[];  // [RPW][FP] then 2 x [Cout][kWPitch]
  __shared__ int s_empty[RPW];
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = blockIdx.x * RPW;
  const int total = L.B * L.N, H = L.H, F = L.F, FP = a.FP, LP = L.FP, Cout = L.Cout;
  uint16_t* wbuf = efeat + (size_t)RPW * FP;
  const uint16_t* __restrict__ wt = a.wt;
  if (tid < RPW) {
    const int row = row0 + tid;
    s_empty[tid] = row < total ? (int)row_empty(a, row) : 1;
  }
  // padding columns [F, LP) of every row are zero
  for (int x = tid; x < RPW * (LP - F); x += NT_) efeat[(x / (LP - F)) * FP + F + x % (LP - F)] = 0;
  // first w_out chunk in flight while the features are built
  const int nchunk = LP / kWChunk + (LP % kWChunk != 0);
  const int cpr = kWChunk / 8;  // 16-byte pieces per chunk row
  auto load_chunk = [&](int c, uint4* reg) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int x = tid + k * NT_;  // piece index
      const int col = x / cpr, f = c * kWChunk + (x % cpr) * 8;
      reg[k] = (col < Cout && f < LP && x < Cout * cpr) ? *reinterpret_cast<const uint4*>(wt + (size_t)col * LP + f)
                                                         : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_chunk = [&](int buf, const uint4* reg) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int x = tid + k * NT_;
      if (x < Cout * cpr)
        *reinterpret_cast<uint4*>(wbuf + (size_t)buf * Cout * kWPitch + (x / cpr) * kWPitch + (x % cpr) * 8) = reg[k];
    }
  };
  // three chunks of w_out in flight in registers (ring), two in LDS
  uint4 wr0[4], wr1[4], wr2[4];
  load_chunk(0, wr0);
  load_chunk(1, wr1);
  load_chunk(2, wr2);
  __syncthreads();
  if (fast_dims(L)) {
    for (int x = tid; x < RPW * H; x += NT_) {
      const int r = x / H, h = x % H, row = row0 + r;
      uint16_t* frow = efeat + (size_t)r * FP;
      if (row < total) {
        features_fast(a, row, h, s_empty[r] != 0, frow);
      } else {
        const uint4 z = make_uint4(0, 0, 0, 0);
        for (int k = 0; k < kFDv / 8; ++k) *reinterpret_cast<uint4*>(frow + h * kFDv + 8 * k) = z;
        for (int k = 0; k < 4; ++k) *reinterpret_cast<uint4*>(frow + H * kFDv + k * H * kFQ + h * kFQ) = z;
        for (int k = 0; k < kFCz / 8; ++k)
          *reinterpret_cast<uint4*>(frow + H * (kFDv + 4 * kFQ) + h * kFCz + 8 * k) = z;
      }
    }
  } else {
  const int nI = (L.Dv + 3) / 4 + (L.Cz + 3) / 4 + L.Q;
  const int items = RPW * H * nI;
#pragma unroll 4
  for (int x = tid; x < items; x += NT_) {
    const int it = x % nI, rh = x / nI;
    const int r = rh / H, h = rh % H, row = row0 + r;
    uint16_t* frow = efeat + (size_t)r * FP;
    if (row < total) {
      feature_item<true, uint16_t>(a, row, h, it, s_empty[r] != 0, frow);
    } else {
      // rows past the end: zero features (their update is not written)
      const int nS = (L.Dv + 3) / 4, nP = (L.Cz + 3) / 4;
      const int offx = H * L.Dv, offp = offx + 4 * H * L.Q;
      if (it < nS) {
        for (int e = 0; e < 4; ++e) if (4 * it + e < L.Dv) frow[h * L.Dv + 4 * it + e] = 0;
      } else if (it < nS + nP) {
        for (int e = 0; e < 4; ++e) if (4 * (it - nS) + e < L.Cz) frow[offp + h * L.Cz + 4 * (it - nS) + e] = 0;
      } else {
        const int q = it - nS - nP;
        for (int k = 0; k < 4; ++k) frow[offx + k * H * L.Q + h * L.Q + q] = 0;
      }
    }
  }
  }
  store_chunk(0, wr0);
  __syncthreads();
  // output tiles: (row block, 32-column block), wavefront w takes tiles w, w+NW, ...
  const int ncb = (Cout + 31) / 32;
  const int ntiles = RB * ncb;
  constexpr int MAXT = 2;  // tiles per wavefront held in registers
  f32x16_t acc[MAXT];
#pragma unroll
  for (int k = 0; k < MAXT; ++k) acc[k] = f32x16_t{};
  auto compute_chunk = [&](int c) {
    const uint16_t* wb = wbuf + (size_t)(c & 1) * Cout * kWPitch;
#pragma unroll
    for (int k = 0; k < MAXT; ++k) {
      const int ti = w + k * NW;
      if (ti < ntiles) {
        const int rb = ti % RB, cb = ti / RB;
        const int colr = min(cb * 32 + l32, Cout - 1);
#pragma unroll
        for (int ks = 0; ks < kWChunk / 16; ++ks) {
          const int f = c * kWChunk + ks * 16;
          if (f < LP) {
            const bf16x8_t af =
                *reinterpret_cast<const bf16x8_t*>(efeat + (size_t)(rb * 32 + l32) * FP + f + half * 8);
            const bf16x8_t bfr = *reinterpret_cast<const bf16x8_t*>(wb + (size_t)colr * kWPitch + ks * 16 + half * 8);
            acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr, acc[k], 0, 0, 0);
          }
        }
      }
    }
  };
  // chunk c is in LDS buffer c & 1; chunk c+1 waits in the ring register set
  // (c+1) % 3 and is stored after chunk c's products; chunk c+3 is then
  // fetched into the set chunk c used
  auto step = [&](int c, uint4* next, uint4* mine) {
    compute_chunk(c);
    if (c + 1 < nchunk) store_chunk((c + 1) & 1, next);
    if (c + 3 < nchunk) load_chunk(c + 3, mine);
    __syncthreads();
  };
  for (int c = 0; c < nchunk; c += 3) {
    step(c, wr1, wr0);
    if (c + 1 < nchunk) step(c + 1, wr2, wr1);
    if (c + 2 < nchunk) step(c + 2, wr0, wr2);
  }
#pragma unroll
  for (int k = 0; k < MAXT; ++k) {
    const int ti = w + k * NW;
    if (ti >= ntiles) continue;
    const int rb = ti % RB, cb = ti / RB;
    const int col = cb * 32 + l32;
    if (col >= Cout) continue;
    const float bo = ld<true>(a.b_out, col);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rr = rb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      const int row = row0 + rr;
      if (row < total) a.update[(size_t)row * Cout + col] = s_empty[rr] ? 0.f : acc[k][r] + bo;
    }
  }
}

// ---------------------------------------------------------------- per-head matrix-core path
// For the standard dimensions (Dv=16, Cz=64, Q=8, R=2) and Cout <= 128 the
// product is summed over heads: update = sum_h features_h @ W_h + b_out with
// W_h the 112 rows of w_out that multiply head h's features.  w_out is packed
// once per call to wh[h][c][k] (k in the head's feature order [scalar 16 |
// x 8 | y 8 | z 8 | length 8 | pair 64], pitch kHeadFeatPitch).  A workgroup
// of 8 M threads takes M residues; per head, 8 lanes read one residue's
// 672-byte block of O with 16-byte loads on consecutive addresses (whole
// cache lines), build its 112 features in LDS, and the wavefronts multiply
// them by W_h on MFMA.  O is loaded two heads ahead, W_h one head ahead.
constexpr int kHeadCoutMax = 128;
// The per-head kernel: Dv = 16, Cz = 64, Q = 8 (112 features per head, for
// any rank R of the pair factors: the pair expansion contracts r), R = 1..3;
// any Cout in 32 .. 128 for R = 2, Cout = 128 for R = 1 and 3.
__host__ __device__ __forceinline__ bool head_path(const Layout& L) {
  if (!(L.mfma && L.Dv == kFDv && L.Cz == kFCz && L.Q == kFQ && L.R >= 1 && L.R <= 3)) return false;
  return L.R == 2 ? (L.Cout % 32 == 0 && L.Cout <= kHeadCoutMax) : L.Cout == 128;
}

// wh[h][c][k] = w_out[f(h, k)][c] (bf16 bits), zero in the pitch padding.
__global__ __launch_bounds__(256) void pack_wout_heads_kernel(const uint16_t* w, uint16_t* wh, int H, int Cout) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)H * Cout * kHeadFeatPitch) return;
  const int k = (int)(idx % kHeadFeatPitch);
  const long hc = idx / kHeadFeatPitch;
  const int c = (int)(hc % Cout), h = (int)(hc / Cout);
  const int offx = H * kFDv, offy = offx + H * kFQ, offz = offy + H * kFQ, offl = offz + H * kFQ,
            offp = offl + H * kFQ;
  int f = -1;
  if (k < 16) f = h * kFDv + k;
  else if (k < 24) f = offx + h * kFQ + (k - 16);
  else if (k < 32) f = offy + h * kFQ + (k - 24);
  else if (k < 40) f = offz + h * kFQ + (k - 32);
  else if (k < 48) f = offl + h * kFQ + (k - 40);
  else if (k < kHeadFeat) f = offp + h * kFCz + (k - 48);
  wh[idx] = f >= 0 ? w[(size_t)f * Cout + c] : (uint16_t)0;
}

// HT > 0: H = HT at compile time (the head loop is unrolled completely, and
// the compiler's waits for the O loads then follow the two-head prefetch).
// R: rank of the pair factors.  The attention-output row of a (residue, head)
// is DO = 16 + 64 R + 24 floats = 4 + 16 R + 6 pieces of 16 bytes; lane j of
// the residue's 8 loads pieces j, j + 8, .., i.e. NPC = 2 R + 2 of them:
// scalar pieces 0..3 (lanes 0..3, k = 0), pair chunk c of rank r at piece
// 4 + 16 r + c, point pieces 4 + 16 R .. 9 + 16 R (lanes 4..7 at k = 2 R,
// lanes 0, 1 at k = 2 R + 1).
template <int M, int COUT, int HT, int R>
__global__ __launch_bounds__(8 * M) void epilogue_head_kernel(EpiArgs a) {
  constexpr int DOR = kFDv + R * kFCz + 3 * kFQ;        // floats per attention-output row
  constexpr int NPC = 2 * R + 2;                         // 16-byte pieces per lane
  constexpr int NT_ = 8 * M;  // threads
  constexpr int NW = NT_ / 64;
  constexpr int KP = kHeadFeatPitch;
  constexpr int WBYTES = COUT * KP * 2;                  // W_h
  constexpr int WLDS = (WBYTES + 1023) / 1024 * 1024;    // room for a partial last copy chunk
  constexpr int WDMA = dma_per_wave<WBYTES, NW>();       // copy instructions per wavefront
  constexpr int RB = M / 32;
  constexpr int NTILE = RB * (COUT / 32);                // 32x32 output tiles
  static_assert(NTILE <= 2 * NW, "two output tiles per wavefront at most");
  __shared__ __attribute__((aligned(1024))) char sW[2 * WLDS];
  __shared__ __attribute__((aligned(16))) uint16_t sF[M * KP];
  __shared__ __attribute__((aligned(16))) float sP[M][28];
  __shared__ int s_empty[M];
  const Layout& L = a.L;
  const int H = HT > 0 ? HT : L.H, total = L.B * L.N;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = tid >> 3, j = tid & 7;  // residue of the workgroup, lane within its 8
  const int row0 = blockIdx.x * M, row = row0 + r;
  int nonempty = 0;
  if (tid < M) {
    s_empty[tid] = row0 + tid < total ? (int)row_empty(a, row0 + tid) : 1;
    nonempty = !s_empty[tid];
  }
  if (!__syncthreads_or(nonempty)) {
    // every residue is padding or has an empty neighbourhood: zeros only
    const int nr = min(M, total - row0);
    const int HQ3 = H * kFQ * 3;
    float4* up = reinterpret_cast<float4*>(a.update + (size_t)row0 * COUT);
    for (int x = tid; x < nr * COUT / 4; x += NT_) up[x] = make_float4(0.f, 0.f, 0.f, 0.f);
    float4* lp = reinterpret_cast<float4*>(a.local + (size_t)row0 * HQ3);
    for (int x = tid; x < nr * HQ3 / 4; x += NT_) lp[x] = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  const bool empty = s_empty[r] != 0;  // also true past the end

  // per-residue constants, the same for every head: frame, and the zl values
  // of this lane's two pair chunks (chunks qa, qb of 4 channels) for every r
  float Rm[9] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, tr[3] = {0.f, 0.f, 0.f};
  const int qa = j >= 4 ? j - 4 : j + 12, qb = j + 4;
  uint2 zla[R], zlb[R];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) zla[rr] = zlb[rr] = make_uint2(0, 0);
  if (!empty) {
    const uint16_t* rt = reinterpret_cast<const uint16_t*>(a.rot) + (size_t)row * 9;
    const uint16_t* tt = reinterpret_cast<const uint16_t*>(a.trans) + (size_t)row * 3;
#pragma unroll
    for (int e = 0; e < 9; ++e) Rm[e] = bf16_bits_to_f32(rt[e]);
#pragma unroll
    for (int e = 0; e < 3; ++e) tr[e] = bf16_bits_to_f32(tt[e]);
    const uint2* z2 = reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.zl) + (size_t)row * R * kFCz);
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      zla[rr] = z2[16 * rr + qa];  // channels 4 qa .. 4 qa + 3 of rank rr
      zlb[rr] = z2[16 * rr + qb];
    }
  }
  // W_h straight into LDS buffer h&1 (direct copies, waited for explicitly);
  // O of a head: this lane's 16-byte pieces j, j+8, ..., j+40 of the
  // residue's 42-piece block, unconditional loads (clamped indices) so that
  // the compiler's own waits count them exactly
  const char* whg = reinterpret_cast<const char*>(a.wt);
  auto copy_w = [&](int h) { dma_tile<WBYTES, NW>(whg + (size_t)h * WBYTES, sW + (h & 1) * WLDS, w, lane); };
  const int rowc = min(row, total - 1);
  auto load_o = [&](int h, float4* v) {
    const float4* o4 = reinterpret_cast<const float4*>(a.o + ((size_t)rowc * H + h) * DOR);
#pragma unroll
    for (int k = 0; k < NPC; ++k) v[k] = o4[min(j + 8 * k, DOR / 4 - 1)];
  };
  auto zl4 = [](uint2 u, int e) {
    const uint32_t wd = (e >> 1) ? u.y : u.x;
    return __uint_as_float((e & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
  };
  auto f4 = [](const float4& v, int e) { return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w)); };

  f32x16_t acc[2] = {f32x16_t{}, f32x16_t{}};
  uint16_t* frow = sF + r * KP;
  // head h: O in cur (loaded two heads ahead), W_h in LDS buffer h&1 (copy
  // issued one head ahead); issues the copy of W_(h+1), then O of head h+2
  // into nb
  auto step = [&](int h, float4(&cur)[NPC], float4(&nb)[NPC]) {
    if (h + 1 < H) copy_w(h + 1);
    if (h + 2 < H) load_o(h + 2, nb);
    // ---- features of head h for residue r (8 lanes); an empty row's O is zero
    if (empty) {
#pragma unroll
      for (int k = 0; k < NPC; ++k) cur[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (j < 4) {  // scalar: piece j
      uint2 u;
      u.x = pack_bf16(cur[0].x, cur[0].y);
      u.y = pack_bf16(cur[0].z, cur[0].w);
      *reinterpret_cast<uint2*>(frow + 4 * j) = u;
    }
    {
      // pair chunk qa of rank r: piece 4 + 16 r + qa, i.e. k = 2 r (lanes 4..7)
      // or 2 r + 2 (lanes 0..3); chunk qb: piece 8 + 16 r + j, k = 2 r + 1
      float pa[4] = {0.f, 0.f, 0.f, 0.f}, pb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        const float4 c0 = cur[2 * rr], c2 = cur[2 * rr + 2];
        const bool hi = j >= 4;
        const float4 ar = make_float4(hi ? c0.x : c2.x, hi ? c0.y : c2.y, hi ? c0.z : c2.z, hi ? c0.w : c2.w);
        const float4 br = cur[2 * rr + 1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pa[e] = fmaf(zl4(zla[rr], e), f4(ar, e), pa[e]);
          pb[e] = fmaf(zl4(zlb[rr], e), f4(br, e), pb[e]);
        }
      }
      uint2 u;
      u.x = pack_bf16(pa[0], pa[1]); u.y = pack_bf16(pa[2], pa[3]);
      *reinterpret_cast<uint2*>(frow + 48 + 4 * qa) = u;
      u.x = pack_bf16(pb[0], pb[1]); u.y = pack_bf16(pb[2], pb[3]);
      *reinterpret_cast<uint2*>(frow + 48 + 4 * qb) = u;
    }
    // points: pieces 4 + 16 R .. 9 + 16 R through LDS, then lane j takes point j
    if (j >= 4) *reinterpret_cast<float4*>(&sP[r][4 * (j - 4)]) = cur[2 * R];
    if (j < 2) *reinterpret_cast<float4*>(&sP[r][16 + 4 * j]) = cur[2 * R + 1];
    __builtin_amdgcn_wave_barrier();
    {
      const float gx = sP[r][3 * j] - tr[0], gy = sP[r][3 * j + 1] - tr[1], gz = sP[r][3 * j + 2] - tr[2];
      // R^T (g - t): column x of R dotted with (g - t)
      float x = Rm[0] * gx + Rm[3] * gy + Rm[6] * gz;
      float y = Rm[1] * gx + Rm[4] * gy + Rm[7] * gz;
      float z = Rm[2] * gx + Rm[5] * gy + Rm[8] * gz;
      float len = sqrtf(x * x + y * y + z * z + a.eps);
      if (empty) { x = y = z = len = 0.f; }
      frow[16 + j] = f32_to_bf16_bits(x);
      frow[24 + j] = f32_to_bf16_bits(y);
      frow[32 + j] = f32_to_bf16_bits(z);
      frow[40 + j] = f32_to_bf16_bits(len);
      if (row < total) {
        float* lp = a.local + (((size_t)row * H + h) * kFQ + j) * 3;
        lp[0] = x; lp[1] = y; lp[2] = z;
      }
    }
    // W_h has landed: at most the copies and loads issued after it (O of
    // h+1, the copy of W_(h+1), O of h+2) may still be in flight
    if (h + 2 < H) wait_vmcnt<2 * NPC + WDMA>();
    else if (h + 1 < H) wait_vmcnt<NPC + WDMA>();
    else wait_vmcnt<0>();
    __syncthreads();  // features of head h and W_h visible
    // ---- update += features_h @ W_h
    const uint16_t* wb = reinterpret_cast<const uint16_t*>(sW + (h & 1) * WLDS);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int ti = w + k * NW;
      if (ti < NTILE) {
        const int rb = ti % RB, cb = ti / RB;
#pragma unroll
        for (int ks = 0; ks < kHeadFeat / 16; ++ks) {
          const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(sF + (rb * 32 + l32) * KP + ks * 16 + half * 8);
          const bf16x8_t bw = *reinterpret_cast<const bf16x8_t*>(wb + (cb * 32 + l32) * KP + ks * 16 + half * 8);
          acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bw, acc[k], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // everyone done with the features of head h and W buffer h&1
  };
  float4 oa[NPC], ob[NPC], oc[NPC];
  copy_w(0);
  load_o(0, oa);
  if (H > 1) load_o(1, ob);
#pragma unroll
  for (int h = 0; h < H; h += 3) {
    step(h, oa, oc);
    if (h + 1 >= H) break;
    step(h + 1, ob, oa);
    if (h + 2 >= H) break;
    step(h + 2, oc, ob);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int ti = w + k * NW;
    if (ti >= NTILE) continue;
    const int rb = ti % RB, cb = ti / RB;
    const int col = cb * 32 + l32;
    const float bo = ld<true>(a.b_out, col);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int rr = rb * 32 + 8 * (q >> 2) + 4 * half + (q & 3);
      const int orow = row0 + rr;
      if (orow < total) a.update[(size_t)orow * COUT + col] = s_empty[rr] ? 0.f : acc[k][q] + bo;
    }
  }
}

// ---------------------------------------------------------------- fp32 path
constexpr int kEpiRowsF32 = 16;

__global__ __launch_bounds__(256) void epilogue_f32_kernel(EpiArgs a) {
  const Layout& L = a.L;
  extern __shared__ float ffeat[];  // [16][FP]
  __shared__ int s_empty[kEpiRowsF32];
  const int tid = threadIdx.x;
  const int row0 = blockIdx.x * kEpiRowsF32;
  const int total = L.B * L.N, H = L.H, F = L.F, FP = a.FP;
  if (tid < kEpiRowsF32) {
    const int row = row0 + tid;
    s_empty[tid] = row < total ? (int)row_empty(a, row) : 1;
  }
  __syncthreads();
  const int nI = (L.Dv + 3) / 4 + (L.Cz + 3) / 4 + L.Q;
  for (int x = tid; x < kEpiRowsF32 * H * nI; x += 256) {
    const int it = x % nI, rh = x / nI;
    const int r = rh / H, h = rh % H, row = row0 + r;
    if (row < total) feature_item<false, float>(a, row, h, it, s_empty[r] != 0, ffeat + (size_t)r * FP);
  }
  __syncthreads();
  const int Cout = L.Cout;
  const float* wo = reinterpret_cast<const float*>(a.w_out);
  const float* bo = reinterpret_cast<const float*>(a.b_out);
  // thread = (column, half of the 16 rows): consecutive threads on
  // consecutive columns, so the w_out loads of a feature are one coalesced
  // row piece and independent of each other from feature to feature; each
  // thread accumulates its 8 rows from LDS broadcasts of the features
  constexpr int RH = kEpiRowsF32 / 2;
  for (int cb = 0; cb < Cout; cb += 128) {
    const int col = cb + (tid & 127), r0 = (tid >> 7) * RH;
    if (col >= Cout) continue;
    float acc[RH];
#pragma unroll
    for (int q = 0; q < RH; ++q) acc[q] = 0.f;
    int f = 0;
    for (; f + 8 <= F; f += 8) {
      float w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = wo[(size_t)(f + e) * Cout + col];
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int q = 0; q < RH; ++q) acc[q] = fmaf(ffeat[(size_t)(r0 + q) * FP + f + e], w[e], acc[q]);
    }
    for (; f < F; ++f) {
      const float w = wo[(size_t)f * Cout + col];
#pragma unroll
      for (int q = 0; q < RH; ++q) acc[q] = fmaf(ffeat[(size_t)(r0 + q) * FP + f], w, acc[q]);
    }
#pragma unroll
    for (int q = 0; q < RH; ++q) {
      const int row = row0 + r0 + q;
      if (row < total) a.update[(size_t)row * Cout + col] = s_empty[r0 + q] ? 0.f : acc[q] + bo[col];
    }
  }
}

template <typename K>
static hipError_t allow_lds(K kernel, size_t shm, size_t* done) {
  if (shm > 64 * 1024 && shm > *done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    *done = shm;
  }
  return hipSuccess;
}

// LDS bytes of the matrix-core epilogue for RPW residues per workgroup:
// features plus two w_out chunks
static inline size_t epi_lds_bytes(const Layout& L, int rpw) {
  return (size_t)rpw * (L.FP + 8) * 2 + 2 * (size_t)L.Cout * kWPitch * 2;
}

// the output tiles of a workgroup must fit MAXT (2) per wavefront, and the
// chunk loads 4 pieces per thread
static inline bool epi_fits(const Layout& L, int rpw) {
  const int nw = rpw / 8, ntiles = (rpw / 32) * ((L.Cout + 31) / 32);
  return epi_lds_bytes(L, rpw) <= 160 * 1024 && ntiles <= 2 * nw && L.Cout * (kWChunk / 8) <= 4 * rpw * 8;
}

bool epilogue_supported(const Layout& L) {
  if (head_path(L)) return true;
  if (L.mfma) return epi_fits(L, 32) || epi_fits(L, 64);
  return (size_t)kEpiRowsF32 * (L.F + 1) * 4 <= 160 * 1024;
}

hipError_t launch_epilogue(const Layout& L, void* ws, const float* o, const float* lse, const ipa_epi_in* in, float eps,
                           float* update, float* local, hipStream_t st) {
  EpiArgs a;
  a.L = L;
  a.o = o; a.lse = lse;
  a.zl = in->zl; a.rot = in->rotation; a.trans = in->translation; a.w_out = in->w_out; a.b_out = in->b_out;
  a.update = update; a.local = local; a.eps = eps;
  a.wt = nullptr;
  const int total = L.B * L.N;
  if (head_path(L)) {
    uint16_t* wh = reinterpret_cast<uint16_t*>(ws);
    const long n = (long)L.H * L.Cout * kHeadFeatPitch;
    hipLaunchKernelGGL(pack_wout_heads_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<const uint16_t*>(in->w_out), wh, L.H, L.Cout);
    a.wt = wh;
    a.FP = kHeadFeatPitch;
    const dim3 g((total + 31) / 32), blk(256);
    if (L.R == 1) {
      if (L.H == 8) hipLaunchKernelGGL((epilogue_head_kernel<32, 128, 8, 1>), g, blk, 0, st, a);
      else hipLaunchKernelGGL((epilogue_head_kernel<32, 128, 0, 1>), g, blk, 0, st, a);
    } else if (L.R == 3) {
      if (L.H == 8) hipLaunchKernelGGL((epilogue_head_kernel<32, 128, 8, 3>), g, blk, 0, st, a);
      else hipLaunchKernelGGL((epilogue_head_kernel<32, 128, 0, 3>), g, blk, 0, st, a);
    } else if (L.Cout == 128 && L.H == 8) {
      hipLaunchKernelGGL((epilogue_head_kernel<32, 128, 8, 2>), g, blk, 0, st, a);
    } else if (L.Cout == 128 && L.H == 12) {
      hipLaunchKernelGGL((epilogue_head_kernel<32, 128, 12, 2>), g, blk, 0, st, a);
    } else {
      switch (L.Cout) {
        case 32: hipLaunchKernelGGL((epilogue_head_kernel<32, 32, 0, 2>), g, blk, 0, st, a); break;
        case 64: hipLaunchKernelGGL((epilogue_head_kernel<32, 64, 0, 2>), g, blk, 0, st, a); break;
        case 96: hipLaunchKernelGGL((epilogue_head_kernel<32, 96, 0, 2>), g, blk, 0, st, a); break;
        default: hipLaunchKernelGGL((epilogue_head_kernel<32, 128, 0, 2>), g, blk, 0, st, a); break;
      }
    }
  } else if (L.mfma) {
    uint16_t* wt = reinterpret_cast<uint16_t*>(ws);
    hipLaunchKernelGGL(transpose_wout_kernel, dim3((L.FP + 63) / 64, (L.Cout + 63) / 64), dim3(256), 0, st,
                       reinterpret_cast<const uint16_t*>(in->w_out), wt, L.F, L.FP, L.Cout);
    a.wt = wt;
    a.FP = L.FP + 8;  // +8 elements: 16-byte row skew for conflict-free fragment reads
    // 64 residues per workgroup when that still gives every CU a workgroup
    if (epi_fits(L, 64) && (total + 63) / 64 >= 256) {
      static size_t done = 0;
      const size_t shm = epi_lds_bytes(L, 64);
      hipError_t e = allow_lds(&epilogue_mfma_kernel<64>, shm, &done);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(epilogue_mfma_kernel<64>, dim3((total + 63) / 64), dim3(512), shm, st, a);
    } else {
      static size_t done = 0;
      const size_t shm = epi_lds_bytes(L, 32);
      hipError_t e = allow_lds(&epilogue_mfma_kernel<32>, shm, &done);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(epilogue_mfma_kernel<32>, dim3((total + 31) / 32), dim3(256), shm, st, a);
    }
  } else {
    a.FP = L.F + 1;
    const size_t shm = (size_t)kEpiRowsF32 * a.FP * 4;
    static size_t done = 0;
    hipError_t e = allow_lds(&epilogue_f32_kernel, shm, &done);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(epilogue_f32_kernel, dim3((total + kEpiRowsF32 - 1) / kEpiRowsF32), dim3(256), shm, st, a);
  }
  return hipGetLastError();
}

}  // namespace fipa
