// Kernel 3 (epilogue): per residue i and head h, from the fused kernel's
// aggregates (IPA page, "Required behavior"):
//   local_ihq = R_i^T (g_ihq - t_i)            inverse frame transform
//   length_ihq = sqrt(|local_ihq|^2 + eps)     (zero for an empty neighbourhood)
//   pair_ih = sum_r zl_ir * o_zr_ihr            pair features from the factors
//   features = [scalar (H,Dv) | x (H,Q) | y | z | length (H,Q) | pair (H,Cz)]
//   update = features @ w_out + b_out, zero for an empty neighbourhood.
// Features of a block of residues are staged in LDS; the projection runs on
// MFMA (bf16 operands, fp32 accumulation) on the matrix-core path and on
// fp32 VALU on the fp32 path.
#include "common.h"

namespace fipa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct EpiArgs {
  Layout L;
  const float* o;
  const float* lse;
  const void *zl, *rot, *trans, *w_out, *b_out;
  float* update;
  float* local;
  float eps;
  int F, FP;  // feature count, LDS row pitch (elements)
};

// Features of (residue row, head h) into an LDS row (element type T).
template <bool BF, typename T>
__device__ void build_features(const EpiArgs& a, int row, int h, bool empty, T* frow) {
  const Layout& L = a.L;
  const int H = L.H, Dv = L.Dv, Q = L.Q, Cz = L.Cz, R = L.R, RCz = L.RCz, DO = L.DO;
  const int offx = H * Dv, offy = offx + H * Q, offz = offy + H * Q, offl = offz + H * Q, offp = offl + H * Q;
  const float* orow = a.o + ((size_t)row * H + h) * DO;
  auto put = [&](int f, float v) {
    if constexpr (sizeof(T) == 2) frow[f] = __builtin_bit_cast(T, f32_to_bf16_bits(v));
    else frow[f] = v;
  };
  for (int d = 0; d < Dv; ++d) put(h * Dv + d, empty ? 0.f : orow[d]);
  float Rm[9], tr[3];
  for (int e = 0; e < 9; ++e) Rm[e] = ld<BF>(a.rot, (size_t)row * 9 + e);
  for (int e = 0; e < 3; ++e) tr[e] = ld<BF>(a.trans, (size_t)row * 3 + e);
  float* lrow = a.local + ((size_t)row * H + h) * Q * 3;
  for (int q = 0; q < Q; ++q) {
    const float gx = orow[Dv + RCz + 3 * q] - tr[0];
    const float gy = orow[Dv + RCz + 3 * q + 1] - tr[1];
    const float gz = orow[Dv + RCz + 3 * q + 2] - tr[2];
    // R^T (g - t): column x of R dotted with (g - t)
    float x = Rm[0] * gx + Rm[3] * gy + Rm[6] * gz;
    float y = Rm[1] * gx + Rm[4] * gy + Rm[7] * gz;
    float z = Rm[2] * gx + Rm[5] * gy + Rm[8] * gz;
    float len = sqrtf(x * x + y * y + z * z + a.eps);
    if (empty) { x = y = z = len = 0.f; }
    lrow[3 * q] = x; lrow[3 * q + 1] = y; lrow[3 * q + 2] = z;
    put(offx + h * Q + q, x);
    put(offy + h * Q + q, y);
    put(offz + h * Q + q, z);
    put(offl + h * Q + q, len);
  }
  for (int c = 0; c < Cz; ++c) {
    float acc = 0.f;
    for (int r = 0; r < R; ++r) acc = fmaf(ld<BF>(a.zl, (size_t)row * RCz + r * Cz + c), orow[Dv + r * Cz + c], acc);
    put(offp + h * Cz + c, empty ? 0.f : acc);
  }
}

// ---------------------------------------------------------------- matrix-core path
constexpr int kEpiRows = 32;

__global__ __launch_bounds__(256) void epilogue_mfma_kernel(EpiArgs a) {
  const Layout& L = a.L;
  extern __shared__ __attribute__((aligned(16))) uint16_t efeat[];  // [32][FP] bf16
  __shared__ int s_empty[kEpiRows];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, half = lane >> 5;
  const int row0 = blockIdx.x * kEpiRows;
  const int total = L.B * L.N, H = L.H, F = a.F, FP = a.FP;
  if (tid < kEpiRows) {
    const int row = row0 + tid;
    int e = 1;
    if (row < total) {
      const int b = row / L.N, i = row % L.N;
      e = !(a.lse[((size_t)b * H) * L.N + i] > -INFINITY);
    }
    s_empty[tid] = e;
  }
  // zero the padded tail columns of every row
  for (int x = tid; x < kEpiRows * (FP - F); x += 256) efeat[(x / (FP - F)) * FP + F + x % (FP - F)] = 0;
  __syncthreads();
  for (int pr = tid; pr < kEpiRows * H; pr += 256) {
    const int r = pr / H, h = pr % H, row = row0 + r;
    uint16_t* frow = efeat + (size_t)r * FP;
    if (row < total) {
      build_features<true, uint16_t>(a, row, h, s_empty[r] != 0, frow);
    } else {
      const int Dv = L.Dv, Q = L.Q, Cz = L.Cz;
      const int offx = H * Dv, offp = offx + 4 * H * Q;
      for (int d = 0; d < Dv; ++d) frow[h * Dv + d] = 0;
      for (int q = 0; q < Q; ++q)
        for (int k = 0; k < 4; ++k) frow[offx + k * H * Q + h * Q + q] = 0;
      for (int c = 0; c < Cz; ++c) frow[offp + h * Cz + c] = 0;
    }
  }
  __syncthreads();
  // update[32 x Cout] = feat[32 x F] @ w_out[F x Cout]; wave w takes column blocks w, w+4, ...
  const int Cout = L.Cout;
  const uint16_t* wo = reinterpret_cast<const uint16_t*>(a.w_out);
  const int nks = FP / 16;
  for (int cb = w; cb * 32 < Cout; cb += 4) {
    const int col = cb * 32 + l32;
    const bool cin = col < Cout;
    f32x16_t acc = f32x16_t{};
    for (int ks = 0; ks < nks; ++ks) {
      const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(efeat + (size_t)l32 * FP + ks * 16 + half * 8);
      uint16_t bw[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int f = ks * 16 + half * 8 + e;
        bw[e] = (cin && f < F) ? wo[(size_t)f * Cout + col] : (uint16_t)0;
      }
      uint4 pk;
      pk.x = bw[0] | ((uint32_t)bw[1] << 16);
      pk.y = bw[2] | ((uint32_t)bw[3] << 16);
      pk.z = bw[4] | ((uint32_t)bw[5] << 16);
      pk.w = bw[6] | ((uint32_t)bw[7] << 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, __builtin_bit_cast(bf16x8_t, pk), acc, 0, 0, 0);
    }
    if (cin) {
      const float bo = ld<true>(a.b_out, col);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = 8 * (r >> 2) + 4 * half + (r & 3);
        const int row = row0 + rr;
        if (row < total) a.update[(size_t)row * Cout + col] = s_empty[rr] ? 0.f : acc[r] + bo;
      }
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
  const int total = L.B * L.N, H = L.H, F = a.F, FP = a.FP;
  if (tid < kEpiRowsF32) {
    const int row = row0 + tid;
    int e = 1;
    if (row < total) {
      const int b = row / L.N, i = row % L.N;
      e = !(a.lse[((size_t)b * H) * L.N + i] > -INFINITY);
    }
    s_empty[tid] = e;
  }
  __syncthreads();
  for (int pr = tid; pr < kEpiRowsF32 * H; pr += 256) {
    const int r = pr / H, h = pr % H, row = row0 + r;
    if (row < total) build_features<false, float>(a, row, h, s_empty[r] != 0, ffeat + (size_t)r * FP);
  }
  __syncthreads();
  const int Cout = L.Cout;
  const float* wo = reinterpret_cast<const float*>(a.w_out);
  const float* bo = reinterpret_cast<const float*>(a.b_out);
  const int r = tid % kEpiRowsF32, cg = tid / kEpiRowsF32;
  const int row = row0 + r;
  if (row >= total) return;
  for (int col = cg; col < Cout; col += 256 / kEpiRowsF32) {
    float acc = 0.f;
    const float* fr = ffeat + (size_t)r * FP;
    for (int f = 0; f < F; ++f) acc = fmaf(fr[f], wo[(size_t)f * Cout + col], acc);
    a.update[(size_t)row * Cout + col] = s_empty[r] ? 0.f : acc + bo[col];
  }
}

hipError_t launch_epilogue(const Layout& L, const float* o, const float* lse, const ipa_epi_in* in, float eps,
                           float* update, float* local, hipStream_t st) {
  EpiArgs a;
  a.L = L;
  a.o = o; a.lse = lse;
  a.zl = in->zl; a.rot = in->rotation; a.trans = in->translation; a.w_out = in->w_out; a.b_out = in->b_out;
  a.update = update; a.local = local; a.eps = eps;
  a.F = L.H * (L.Dv + 4 * L.Q + L.Cz);
  const int total = L.B * L.N;
  if (L.mfma) {
    a.FP = round_up(a.F, 16) + 8;  // +8 elements: 16-byte row skew for conflict-free fragment reads
    // the tail [F, FP) is zeroed in the kernel; the MFMA loop reads FP - 8 columns
    const size_t shm = (size_t)kEpiRows * a.FP * 2;
    if (shm > 160 * 1024) return hipErrorInvalidValue;
    static size_t attr_set = 0;  // largest dynamic LDS size enabled so far
    if (shm > 64 * 1024 && shm > attr_set) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&epilogue_mfma_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
      if (e != hipSuccess) return e;
      attr_set = shm;
    }
    hipLaunchKernelGGL(epilogue_mfma_kernel, dim3((total + kEpiRows - 1) / kEpiRows), dim3(256), shm, st, a);
  } else {
    a.FP = a.F + 1;
    const size_t shm = (size_t)kEpiRowsF32 * a.FP * 4;
    if (shm > 160 * 1024) return hipErrorInvalidValue;
    static size_t attr_set = 0;
    if (shm > 64 * 1024 && shm > attr_set) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&epilogue_f32_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
      if (e != hipSuccess) return e;
      attr_set = shm;
    }
    hipLaunchKernelGGL(epilogue_f32_kernel, dim3((total + kEpiRowsF32 - 1) / kEpiRowsF32), dim3(256), shm, st, a);
  }
  return hipGetLastError();
}

}  // namespace fipa
