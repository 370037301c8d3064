// Kernel 1 (lift): frames -> global points, per-head point weight, and the
// lifted rows whose inner products are the IPA logits.
//
// Logit of the "Invariant point attention (IPA)" page ("Required behavior"):
//   L_ijh = q.k/sqrt(3D) + pair_bias_ijh/sqrt(3) - gamma_h sum_p |a_ip - b_jp|^2
// with a = T_i(q_points), b = T_j(k_points), gamma_h = 1/2 softplus(w_h)
// sqrt(2/(27P)), pair_bias_ijh = sum_c w_pair[h,c] sum_r zl_irc zr_jrc.
// The squared distance is expanded (FlashIPA verdict page, key_machinery)
// about two centroids, that of the key tile holding j and that of the query's
// wavefront (see common.h for the column layout), so that every term is an
// inner product of a query-side and a key-side vector of small magnitude.
// This kernel writes the key side: centred key points w = b - c_t split into
// fp16 high/low parts, -gamma log2e |w|^2, 2 gamma log2e sum_p w_p, and the
// value rows (centred value points, a ones row and the centroid).  All logits
// are carried in log2 units (times log2 e) so that the softmax can use exp2.
//
// One workgroup per (key tile t, head h, batch b), 64 residues.
#include "common.h"

namespace fipa {

struct LiftArgs {
  Layout L;
  const void *q, *k, *v, *qp, *kp, *vp, *rot, *trans, *pwr, *wpair, *zl, *zr;
  const uint8_t* mask;
  const uint8_t* pm;
  char* ws;
};

__device__ __forceinline__ float softplus_f(float x) {
  // log(1 + exp(x)) without overflow
  return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
}

__device__ __forceinline__ float clamp_f16(float x) { return fminf(fmaxf(x, -65504.0f), 65504.0f); }

__device__ __forceinline__ uint16_t hi16(float x) { return f32_to_f16_bits(clamp_f16(x)); }
__device__ __forceinline__ uint16_t lo16(float x) {
  const float c = clamp_f16(x);
  return f32_to_f16_bits(c - f16_bits_to_f32(f32_to_f16_bits(c)));
}

template <bool BF>
__global__ __launch_bounds__(256) void lift_kernel(LiftArgs a) {
  const Layout& L = a.L;
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int N = L.N, H = L.H, P = L.P, Q = L.Q, D = L.D, Dv = L.Dv, RCz = L.RCz, Cz = L.Cz;

  __shared__ float s_tr[64][3];
  __shared__ int s_valid[64];
  __shared__ float s_w[64][16];    // b - c (key points, centred)
  __shared__ float s_x[64][32];    // x - c (value points, centred)
  __shared__ float s_a[64][16];    // a (query points, global)
  __shared__ float s_nb[64];       // -gamma log2e |b - c|^2
  __shared__ float s_ww[64][4];    // 2 gamma log2e sum_p (b_p - c)
  __shared__ float s_c[4];
  __shared__ float s_gam;

  // --- residues of this tile: validity, translation
  if (tid < 64) {
    const int j = t * 64 + tid;
    int valid = 0;
    float tx = 0.f, ty = 0.f, tz = 0.f;
    if (j < N) {
      valid = a.mask[(size_t)b * N + j] != 0;
      const size_t o = ((size_t)b * N + j) * 3;
      tx = ld<BF>(a.trans, o); ty = ld<BF>(a.trans, o + 1); tz = ld<BF>(a.trans, o + 2);
    }
    s_valid[tid] = valid;
    s_tr[tid][0] = tx; s_tr[tid][1] = ty; s_tr[tid][2] = tz;
    // centroid of the valid translations (wave 0 holds the 64 residues)
    float sx = valid ? tx : 0.f, sy = valid ? ty : 0.f, sz = valid ? tz : 0.f, sn = valid ? 1.f : 0.f;
    for (int off = 32; off > 0; off >>= 1) {
      sx += __shfl_xor(sx, off);
      sy += __shfl_xor(sy, off);
      sz += __shfl_xor(sz, off);
      sn += __shfl_xor(sn, off);
    }
    if (tid == 0) {
      float cx = 0.f, cy = 0.f, cz = 0.f;
      if (sn > 0.f) { cx = sx / sn; cy = sy / sn; cz = sz / sn; }
      // The centroid only has to be some fixed point near the tile.  It is
      // put on a 4-angstrom grid, exactly representable in fp16, so that it
      // can ride in an fp16 value column and so that differences of two
      // centroids are exact in fp16.
      const float grid = (float)kCentGrid;
      cx = grid * rintf(cx / grid); cy = grid * rintf(cy / grid); cz = grid * rintf(cz / grid);
      cx = f16_bits_to_f32(hi16(cx)); cy = f16_bits_to_f32(hi16(cy)); cz = f16_bits_to_f32(hi16(cz));
      s_c[0] = cx; s_c[1] = cy; s_c[2] = cz; s_c[3] = 0.f;
      const float g = 0.5f * softplus_f(ld<BF>(a.pwr, h)) * sqrtf(2.0f / (27.0f * (float)P));
      s_gam = g;
    }
  }
  __syncthreads();
  const float cx = s_c[0], cy = s_c[1], cz = s_c[2];
  const float gam = s_gam;
  const float gl = gam * kLog2e;

  // --- global points of the 64 residues for head h
  if (tid < 64) {
    const int j = t * 64 + tid;
    float Rm[9];
    const bool in = j < N;
    for (int e = 0; e < 9; ++e) Rm[e] = in ? ld<BF>(a.rot, ((size_t)b * N + j) * 9 + e) : 0.f;
    const float tx = s_tr[tid][0], ty = s_tr[tid][1], tz = s_tr[tid][2];
    float nb = 0.f, Wx = 0.f, Wy = 0.f, Wz = 0.f;
    for (int p = 0; p < 16; ++p) { s_w[tid][p] = 0.f; s_a[tid][p] = 0.f; }
    for (int p = 0; p < 32; ++p) s_x[tid][p] = 0.f;
    if (in) {
      const size_t base_k = (((size_t)b * N + j) * H + h) * P * 3;
      for (int p = 0; p < P; ++p) {
        const float lx = ld<BF>(a.kp, base_k + 3 * p), ly = ld<BF>(a.kp, base_k + 3 * p + 1),
                    lz = ld<BF>(a.kp, base_k + 3 * p + 2);
        const float gx = Rm[0] * lx + Rm[1] * ly + Rm[2] * lz + tx;
        const float gy = Rm[3] * lx + Rm[4] * ly + Rm[5] * lz + ty;
        const float gz = Rm[6] * lx + Rm[7] * ly + Rm[8] * lz + tz;
        const float wx = gx - cx, wy = gy - cy, wz = gz - cz;
        s_w[tid][3 * p] = wx; s_w[tid][3 * p + 1] = wy; s_w[tid][3 * p + 2] = wz;
        nb += wx * wx + wy * wy + wz * wz;
        Wx += wx; Wy += wy; Wz += wz;
        const float qx = ld<BF>(a.qp, base_k + 3 * p), qy = ld<BF>(a.qp, base_k + 3 * p + 1),
                    qz = ld<BF>(a.qp, base_k + 3 * p + 2);
        s_a[tid][3 * p] = Rm[0] * qx + Rm[1] * qy + Rm[2] * qz + tx;
        s_a[tid][3 * p + 1] = Rm[3] * qx + Rm[4] * qy + Rm[5] * qz + ty;
        s_a[tid][3 * p + 2] = Rm[6] * qx + Rm[7] * qy + Rm[8] * qz + tz;
      }
      const size_t base_v = (((size_t)b * N + j) * H + h) * Q * 3;
      for (int q = 0; q < Q && q < 10; ++q) {
        const float lx = ld<BF>(a.vp, base_v + 3 * q), ly = ld<BF>(a.vp, base_v + 3 * q + 1),
                    lz = ld<BF>(a.vp, base_v + 3 * q + 2);
        s_x[tid][3 * q] = Rm[0] * lx + Rm[1] * ly + Rm[2] * lz + tx - cx;
        s_x[tid][3 * q + 1] = Rm[3] * lx + Rm[4] * ly + Rm[5] * lz + ty - cy;
        s_x[tid][3 * q + 2] = Rm[6] * lx + Rm[7] * ly + Rm[8] * lz + tz - cz;
      }
    }
    s_nb[tid] = -gl * nb;
    s_ww[tid][0] = 2.f * gl * Wx; s_ww[tid][1] = 2.f * gl * Wy; s_ww[tid][2] = 2.f * gl * Wz; s_ww[tid][3] = 0.f;
  }
  // --- small per-tile / per-head records
  if (tid == 0) {
    if (b == 0 && t == 0) reinterpret_cast<float*>(a.ws + L.off_gam)[h] = gam;
    if (h == 0) {
      float4* ck = reinterpret_cast<float4*>(a.ws + L.off_ck);
      ck[(size_t)b * L.NT + t] = make_float4(cx, cy, cz, 0.f);
      if (b == 0 && t == 0) {
        Header* hd = reinterpret_cast<Header*>(a.ws);
        hd->magic = kMagic;
        hd->has_pair_mask = a.pm != nullptr;
      }
    }
  }
  __syncthreads();
  if (h == 0 && tid < 2) {
    uint32_t w = 0;
    for (int jj = 0; jj < 64; ++jj) {
      int hf;
      const int bit = mask_bit_of_key(jj, &hf);
      if (hf == tid && s_valid[jj]) w |= 1u << bit;
    }
    reinterpret_cast<uint32_t*>(a.ws + L.off_km)[((size_t)b * L.NT + t) * 2 + tid] = w;
  }

  const float sq = kLog2e / sqrtf(3.0f * (float)D);
  const float sp = kLog2e / sqrtf(3.0f);

  if constexpr (BF) {
    // ---------------- matrix-core layouts (common.h)
    const int QW = L.QW, KROW = L.KROW, P3 = 3 * P, GS = L.GS;
    const uint16_t* k16 = reinterpret_cast<const uint16_t*>(a.k);
    const uint16_t* zr16 = reinterpret_cast<const uint16_t*>(a.zr);
    const uint16_t* v16 = reinterpret_cast<const uint16_t*>(a.v);
    // head key rows of tile (b,h,t): [k | 0 | geometric 16 GS | pad]
    uint16_t* kt = reinterpret_cast<uint16_t*>(a.ws + kt_tile_off(L, b, h, t));
    const int kchunks = KROW / 8;
    for (int ch = tid; ch < 64 * kchunks; ch += 256) {
      const int row = ch / kchunks, c0 = (ch % kchunks) * 8;
      const int j = t * 64 + row;
      uint16_t out[8];
      for (int e = 0; e < 8; ++e) {
        const int c = c0 + e;
        uint16_t val = 0;
        if (s_valid[row]) {
          if (c < D) {
            val = k16[(((size_t)b * N + j) * H + h) * D + c];
          } else if (c >= 16 && c < 16 + 16 * GS) {
            // geometric columns, layout in common.h
            const int g = c - 16, base = 16 * (GS - 1);
            if (g < base + 4) {
              if (g < P3) val = hi16(s_w[row][g]);
              else if (g < 2 * P3) val = lo16(s_w[row][g - P3]);
              else if (g < 3 * P3) val = hi16(s_w[row][g - 2 * P3]);
            } else {
              const int x = g - base;
              if (x == 4) val = hi16(s_nb[row] * (1.0f / kNormScale));
              else if (x == 12) val = lo16(s_nb[row] * (1.0f / kNormScale));
              else if (x >= 5 && x <= 7) val = hi16(s_ww[row][x - 5]);
              else if (x >= 13) val = lo16(s_ww[row][x - 13]);
              else if (x >= 9 && x <= 11) val = 0x4C00;  // fp16 16.0, multiplies the query's t'/16 parts
            }
          }
        } else if (c == 16 + 16 * (GS - 1) + 8) {
          val = 0xFBFF;  // fp16 -65504 in the key-mask column of a masked key
        }
        out[e] = val;
      }
      uint4 pk;
      pk.x = out[0] | ((uint32_t)out[1] << 16);
      pk.y = out[2] | ((uint32_t)out[3] << 16);
      pk.z = out[4] | ((uint32_t)out[5] << 16);
      pk.w = out[6] | ((uint32_t)out[7] << 16);
      reinterpret_cast<uint4*>(kt + (size_t)row * KROW + c0)[0] = pk;
    }
    // head value rows of tile (b,h,t), transposed (rows d, columns kappa =
    // permuted keys): [v 2^-8 | 1 | 0] and [x - c | 1 | c | 0]
    uint16_t* vt = reinterpret_cast<uint16_t*>(a.ws + vt_tile_off(L, b, h, t));
    const int vchunks = kVCols / 8;
    for (int ch = tid; ch < 64 * vchunks; ch += 256) {
      const int d = ch / vchunks, k0 = (ch % vchunks) * 8;
      uint16_t out[8];
      for (int e = 0; e < 8; ++e) {
        const int kappa = k0 + e;
        uint16_t val = 0;
        if (kappa < 64) {
          const int jj = vt_key_of_col(kappa);
          const int j = t * 64 + jj;
          if (s_valid[jj]) {
            if (d < 32) {
              if (d < Dv) val = f32_to_f16_bits(bf16_bits_to_f32(v16[(((size_t)b * N + j) * H + h) * Dv + d]) * kVScale);
              else if (d == Dv) val = 0x3C00;  // fp16 1.0: weight sum
            } else {
              const int dd = d - 32;
              if (dd < 3 * Q) val = hi16(s_x[jj][dd]);
              else if (dd == 3 * Q) val = 0x3C00;  // fp16 1.0: weight sum
              else if (dd <= 3 * Q + 3) val = hi16(s_c[dd - 3 * Q - 1]);
            }
          }
        }
        out[e] = val;
      }
      uint4 pk;
      pk.x = out[0] | ((uint32_t)out[1] << 16);
      pk.y = out[2] | ((uint32_t)out[3] << 16);
      pk.z = out[4] | ((uint32_t)out[5] << 16);
      pk.w = out[6] | ((uint32_t)out[7] << 16);
      reinterpret_cast<uint4*>(vt + (size_t)d * kVCols + k0)[0] = pk;
    }
    if (h == 0) {
      // pair-factor key rows [zr | 0 | pad] and transposed value rows
      // [zr 2^-8 | 0] of tile (b,t), shared by the heads
      uint16_t* kz = reinterpret_cast<uint16_t*>(a.ws + ktz_tile_off(L, b, t));
      const int KZROW = L.KZROW;
      for (int x = tid; x < 64 * KZROW; x += 256) {
        const int row = x / KZROW, c = x % KZROW;
        kz[x] = (s_valid[row] && c < RCz) ? zr16[((size_t)b * N + t * 64 + row) * RCz + c] : (uint16_t)0;
      }
      uint16_t* vz = reinterpret_cast<uint16_t*>(a.ws + vtz_tile_off(L, b, t));
      const int vzn = (int)(vtz_tile_bytes(L) / 2);
      for (int x = tid; x < vzn; x += 256) {
        const int d = x / kVCols, kappa = x % kVCols;
        uint16_t val = 0;
        if (d < RCz && kappa < 64) {
          const int jj = vt_key_of_col(kappa);
          if (s_valid[jj])
            val = f32_to_f16_bits(bf16_bits_to_f32(zr16[((size_t)b * N + t * 64 + jj) * RCz + d]) * kVScale);
        }
        vz[x] = val;
      }
    }
    // lifted query rows [q sq | 0] for the tile's residues
    uint16_t* ql = reinterpret_cast<uint16_t*>(a.ws + L.off_ql);
    const int qchunks = QW / 8;
    for (int ch = tid; ch < 64 * qchunks; ch += 256) {
      const int row = ch / qchunks, c0 = (ch % qchunks) * 8;
      const int i = t * 64 + row;
      uint16_t out[8];
      for (int e = 0; e < 8; ++e) {
        const int c = c0 + e;
        out[e] = f32_to_bf16_bits(i < N && c < D ? ld<true>(a.q, (((size_t)b * N + i) * H + h) * D + c) * sq : 0.f);
      }
      uint4 pk;
      pk.x = out[0] | ((uint32_t)out[1] << 16);
      pk.y = out[2] | ((uint32_t)out[3] << 16);
      pk.z = out[4] | ((uint32_t)out[5] << 16);
      pk.w = out[6] | ((uint32_t)out[7] << 16);
      reinterpret_cast<uint4*>(ql + (((size_t)b * H + h) * L.NQpad + i) * QW + c0)[0] = pk;
    }
    // the query pair factors [zl | 0] (shared by the heads: head 0 writes
    // them) and this head's pair weights [w_pair[h, c % Cz] | 0]
    const uint16_t* zl16 = reinterpret_cast<const uint16_t*>(a.zl);
    const uint16_t* wp16 = reinterpret_cast<const uint16_t*>(a.wpair);
    const int ZW = L.ZW;
    if (h == 0) {
      uint16_t* qz = reinterpret_cast<uint16_t*>(a.ws + qz_row_off(L, b, t * 64));
      for (int x = tid; x < 64 * ZW; x += 256) {
        const int row = x / ZW, c = x - row * ZW, i = t * 64 + row;
        if (i < N) qz[(size_t)row * ZW + c] = c < RCz ? zl16[((size_t)b * N + i) * RCz + c] : (uint16_t)0;
      }
    }
    if (b == 0 && t == 0) {
      uint16_t* wp = reinterpret_cast<uint16_t*>(a.ws + wp_row_off(L, h));
      for (int c = tid; c < ZW; c += 256) wp[c] = c < RCz ? wp16[(size_t)h * Cz + c % Cz] : (uint16_t)0;
    }
  } else {
    // ---------------- fp32 layouts (row-major per key / query)
    const int KROW = L.KROW, DVP = L.VROWS, DQP = L.DQP, P3 = 3 * P;
    float* kr = reinterpret_cast<float*>(a.ws + L.off_kt);
    float* vr = reinterpret_cast<float*>(a.ws + L.off_vt);
    float* qr = reinterpret_cast<float*>(a.ws + L.off_ql);
    for (int idx = tid; idx < 64 * KROW; idx += 256) {
      const int row = idx / KROW, c = idx % KROW;
      const int j = t * 64 + row;
      float val = 0.f;
      if (s_valid[row]) {
        if (c < D) val = ld<false>(a.k, (((size_t)b * N + j) * H + h) * D + c);
        else if (c < D + RCz) val = ld<false>(a.zr, ((size_t)b * N + j) * RCz + (c - D));
        else if (c < D + RCz + P3) val = s_w[row][c - D - RCz];
      }
      kr[(((size_t)b * H + h) * L.NKpad + j) * KROW + c] = val;
    }
    for (int idx = tid; idx < 64 * DVP; idx += 256) {
      const int row = idx / DVP, d = idx % DVP;
      const int j = t * 64 + row;
      float val = 0.f;
      if (s_valid[row]) {
        if (d < Dv) val = ld<false>(a.v, (((size_t)b * N + j) * H + h) * Dv + d);
        else if (d < Dv + RCz) val = ld<false>(a.zr, ((size_t)b * N + j) * RCz + (d - Dv));
        else if (d < Dv + RCz + 3 * Q) val = s_x[row][d - Dv - RCz];
      }
      vr[(((size_t)b * H + h) * L.NKpad + j) * DVP + d] = val;
    }
    for (int idx = tid; idx < 64 * DQP; idx += 256) {
      const int row = idx / DQP, c = idx % DQP;
      const int i = t * 64 + row;
      float val = 0.f;
      if (i < N) {
        if (c < D) {
          val = ld<false>(a.q, (((size_t)b * N + i) * H + h) * D + c) * sq;
        } else if (c < D + RCz) {
          const int cc = (c - D) % Cz;
          val = ld<false>(a.wpair, (size_t)h * Cz + cc) * ld<false>(a.zl, ((size_t)b * N + i) * RCz + (c - D)) * sp;
        }
      }
      qr[(((size_t)b * H + h) * L.NQpad + i) * DQP + c] = val;
    }
  }
  // query global points (both paths): 16 floats per (b,h,i)
  float* qa = reinterpret_cast<float*>(a.ws + L.off_qa);
  for (int idx = tid; idx < 64 * 16; idx += 256) {
    const int row = idx / 16, c = idx % 16;
    const int i = t * 64 + row;
    qa[(((size_t)b * H + h) * L.NQpad + i) * 16 + c] = (i < N && c < 3 * P) ? s_a[row][c] : 0.f;
  }
  // packed permitted-key words for every query row and this key tile:
  // mask_i && mask_j && pair_mask_ij
  if (a.pm != nullptr && h == 0) {
    uint32_t* pmw = reinterpret_cast<uint32_t*>(a.ws + L.off_pm);
    for (int i = tid; i < L.NQpad; i += 256) {
      uint32_t w0 = 0, w1 = 0;
      if (i < N && a.mask[(size_t)b * N + i]) {
        const uint8_t* row = a.pm + ((size_t)b * N + i) * N + (size_t)t * 64;
        for (int jj = 0; jj < 64; ++jj) {
          if (t * 64 + jj >= N) break;
          if (s_valid[jj] && row[jj]) {
            int hf;
            const int bit = mask_bit_of_key(jj, &hf);
            if (hf) w1 |= 1u << bit; else w0 |= 1u << bit;
          }
        }
      }
      pmw[(((size_t)b * L.NQpad + i) * L.NT + t) * 2] = w0;
      pmw[(((size_t)b * L.NQpad + i) * L.NT + t) * 2 + 1] = w1;
    }
  }
}

// ---------------------------------------------------------------- vectorised matrix-core lift
// Same output as lift_kernel<true> for shapes whose D, Dv and Cz are
// multiples of 8, so that every 8-column chunk of a lifted row comes from one
// 16-byte piece of one input row.  Per key tile there are H + 1 units: one
// per head (key rows [k | geometric], value rows [v | points], query rows,
// query points) and one for the pair-factor rows the heads share (zr key
// rows, zr value rows).  Every global load of a unit is issued up front into
// registers (one memory latency per workgroup instead of one per loop trip);
// rows are then written with 16-byte stores, value tiles are transposed
// through LDS, the query rows are scaled and rounded 8 columns at a time, and
// one thread per key writes that key's geometric columns (their layout is
// fixed by P at compile time).  LDS rows are padded to odd word strides where
// lanes walk down a column.  Units (b, t, u) are handed out so that the H + 1
// units of one key tile run back to back on one XCD and share its L2 for zl
// and the frames.
constexpr int kFastVRows = 64;       // transposed rows per pass: Dv <= 24 (head unit), R Cz in passes of 64 (pair unit)
constexpr int kFastVPitch = 66;      // 16-bit elements per transposed LDS row (33 words)
constexpr int kFastZ = 6;            // 16-byte pieces of a zr / zl tile per thread: 64 R Cz/8 <= 1536
constexpr int kFastK = 1;            // pieces of a k / v / q tile per thread: 64 D/8 <= 256 (D <= 16, Dv <= 24)
constexpr int kFastPts = 5;          // points per thread: 64 (2P + Q) <= 1280
constexpr int kFastPc = 4;           // 8-byte point pieces per thread: 64 (6 + 3Q/4) <= 1024
constexpr int kPrPitch = 13;         // 8-byte pieces per staged point row (odd: rows spread over banks)

// x / d for 0 <= x < 2^16 and 0 < d < 2^16: m = ceil(2^32 / d), which fits
// in 32 bits for d >= 2; d = 1 is passed through
struct FastDiv {
  uint32_t m;
  int d;
};
static inline FastDiv make_fastdiv(int d) {
  return FastDiv{d > 1 ? (uint32_t)(((1ull << 32) + (uint64_t)d - 1) / (uint64_t)d) : 0u, d};
}
__device__ __forceinline__ int fdiv(int x, FastDiv f) { return f.d == 1 ? x : (int)__umulhi((uint32_t)x, f.m); }

__device__ __forceinline__ uint4 pack8(const uint16_t* v) {
  uint4 pk;
  pk.x = v[0] | ((uint32_t)v[1] << 16);
  pk.y = v[2] | ((uint32_t)v[3] << 16);
  pk.z = v[4] | ((uint32_t)v[5] << 16);
  pk.w = v[6] | ((uint32_t)v[7] << 16);
  return pk;
}

struct LiftFastArgs {
  int units, per_xcd, pm_vec;
  int pts_vec;  // P = 4 and Q % 4 == 0: points loaded as 8-byte pieces of whole rows
  FastDiv nz, nk, nv, npc, nkz;
};

// Two floats to packed bf16 (round to nearest even, the hardware conversion).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

static inline bool lift_fast_fits(const Layout& L) {
  return L.mfma && L.D % 8 == 0 && L.Dv % 8 == 0 && L.Cz % 8 == 0 && L.Dv <= kFastVRows && L.Cz <= 192 &&
         64 * (L.RCz / 8) <= 256 * kFastZ && 64 * (L.D / 8) <= 256 * kFastK && 64 * (L.Dv / 8) <= 256 * kFastK &&
         64 * (2 * L.P + L.Q) <= 256 * kFastPts;
}

// Transposed value rows out of LDS: row d of the transposed copy `src`
// (one 16-bit element per key, pitch kFastVPitch) as 8 column chunks of the
// tile row (columns k0 .. k0+7 hold keys j0 .. j0+3 and j0+8 .. j0+11,
// j0 = vt_key_of_col(k0)) plus the 8 zero pad columns 64 .. 71.
__device__ __forceinline__ void store_vt_rows(uint16_t* vt, const uint16_t (*src)[kFastVPitch], int rows, int tid) {
  for (int x = tid; x < rows * 9; x += 256) {
    const int d = x / 9, c = x - 9 * d;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (c < 8) {
      const int j0 = vt_key_of_col(8 * c);
      const uint32_t* row = reinterpret_cast<const uint32_t*>(&src[d][0]);
      val = make_uint4(row[j0 / 2], row[j0 / 2 + 1], row[j0 / 2 + 4], row[j0 / 2 + 5]);
    }
    *reinterpret_cast<uint4*>(vt + (size_t)d * kVCols + 8 * c) = val;
  }
}

template <int P, bool STK = false>
__global__ __launch_bounds__(256, 6) void lift_fast_kernel(LiftArgs a, LiftFastArgs f) {
  constexpr int P3 = 3 * P;
  constexpr int GS = STK ? 2 : (P <= 4 ? 3 : 4);
  const Layout& L = a.L;
  const int N = L.N, H = L.H, Q = L.Q, D = L.D, Dv = L.Dv, RCz = L.RCz, Cz = L.Cz;
  const int u = (int)(blockIdx.x % 8) * f.per_xcd + (int)(blockIdx.x / 8);
  if (u >= f.units) return;
  const int h = u % (H + 1), t = (u / (H + 1)) % L.NT, b = u / ((H + 1) * L.NT);
  const int tid = threadIdx.x;
  const int nk = D / 8, nz = RCz / 8, nv = Dv / 8;
  const int QW = L.QW;
  const int npt = 2 * P + Q;
  const size_t row0 = (size_t)b * N + (size_t)t * 64;     // first residue of the tile
  const int nrow = min(64, N - t * 64);                    // residues of the tile inside the chain

  __shared__ float s_rot[64][9];
  __shared__ float s_tr[64][3];
  __shared__ int s_valid[64];
  __shared__ uint32_t s_vmask[2];  // valid keys, bit jj of word jj / 32
  __shared__ float s_w[64][P3 % 2 ? P3 : P3 + 1];  // b - c (key points, centred), odd row stride
  __shared__ float s_a[64][P3 % 2 ? P3 : P3 + 1];  // a (query points, global), odd row stride
  __shared__ __attribute__((aligned(16))) float s_xT[32][64];  // x - c of valid keys, coordinate-major
  __shared__ __attribute__((aligned(16))) uint16_t s_vzT[kFastVRows][kFastVPitch];  // transposed rows 2^-8 (fp16)
  __shared__ float s_c[4];
  __shared__ float s_gam;

  if (h == H) {
    // ---- pair-factor unit: zr key rows [zr | 0 | pad] and transposed value
    // rows [zr 2^-8 | 0] of tile (b, t), zero for keys that are masked or
    // past the end
    const uint4* zrb4 = reinterpret_cast<const uint4*>(a.zr) + row0 * nz;
    uint4 zr_r[kFastZ];
#pragma unroll
    for (int k = 0; k < kFastZ; ++k) {
      const int x = tid + 256 * k, r = fdiv(x, f.nz), c = x - r * nz;
      zr_r[k] = (x < 64 * nz && r < nrow) ? zrb4[r * nz + c] : make_uint4(0, 0, 0, 0);
    }
    // the query pair factors of the tile's residues, [zl | 0] (read by the
    // fused kernel for every head)
    {
      const uint4* zlb4 = reinterpret_cast<const uint4*>(a.zl) + row0 * nz;
      uint4 zl_r[kFastZ];
#pragma unroll
      for (int k = 0; k < kFastZ; ++k) {
        const int x = tid + 256 * k, r = fdiv(x, f.nz), c = x - r * nz;
        zl_r[k] = (x < 64 * nz && r < nrow) ? zlb4[r * nz + c] : make_uint4(0, 0, 0, 0);
      }
      uint16_t* qz = reinterpret_cast<uint16_t*>(a.ws + qz_row_off(L, b, t * 64));
#pragma unroll
      for (int k = 0; k < kFastZ; ++k) {
        const int x = tid + 256 * k, r = fdiv(x, f.nz), c = x - r * nz;
        if (x < 64 * nz && r < nrow) *reinterpret_cast<uint4*>(qz + (size_t)r * L.ZW + 8 * c) = zl_r[k];
      }
      const int nzq = (L.ZW - RCz) / 8;
      for (int x = tid; x < nrow * nzq; x += 256) {
        const int r = x / nzq;
        *reinterpret_cast<uint4*>(qz + (size_t)r * L.ZW + RCz + 8 * (x - r * nzq)) = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < 64) s_valid[tid] = tid < nrow && a.mask[row0 + tid] != 0;
    __syncthreads();
    const int KZROW = L.KZROW;
    uint16_t* kz = reinterpret_cast<uint16_t*>(a.ws + ktz_tile_off(L, b, t));
    auto vh = [](uint16_t bits) { return f32_to_f16_bits(bf16_bits_to_f32(bits) * kVScale); };
#pragma unroll
    for (int k = 0; k < kFastZ; ++k) {
      const int x = tid + 256 * k, r = fdiv(x, f.nz), c = x - r * nz;
      if (x < 64 * nz) {
        if (!s_valid[r]) zr_r[k] = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(kz + (size_t)r * KZROW + 8 * c) = zr_r[k];
      }
    }
    // zero columns [R Cz, KZROW) of the key rows
    const int nzero = (KZROW - RCz) / 8;
    for (int x = tid; x < 64 * nzero; x += 256) {
      const int r = fdiv(x, f.nkz);
      *reinterpret_cast<uint4*>(kz + (size_t)r * KZROW + RCz + 8 * (x - r * nzero)) = make_uint4(0, 0, 0, 0);
    }
    // value rows: zr 2^-8 transposed through LDS, kFastVRows channels a pass
    uint16_t* vz = reinterpret_cast<uint16_t*>(a.ws + vtz_tile_off(L, b, t));
    for (int d0 = 0; d0 < RCz; d0 += kFastVRows) {
#pragma unroll
      for (int k = 0; k < kFastZ; ++k) {
        const int x = tid + 256 * k, r = fdiv(x, f.nz), c = x - r * nz;
        if (x < 64 * nz && 8 * c >= d0 && 8 * c < d0 + kFastVRows) {
          const uint16_t* e16 = reinterpret_cast<const uint16_t*>(&zr_r[k]);
#pragma unroll
          for (int e = 0; e < 8; ++e) s_vzT[8 * c + e - d0][r] = vh(e16[e]);
        }
      }
      __syncthreads();
      store_vt_rows(vz + (size_t)d0 * kVCols, s_vzT, min(kFastVRows, RCz - d0), tid);
      __syncthreads();
    }
    // zero rows [R Cz, VZROWS) and the KiB rounding of the tile
    const int zrows_end = (int)(vtz_tile_bytes(L) / 16);
    for (int x = RCz * (kVCols / 8) + tid; x < zrows_end; x += 256)
      reinterpret_cast<uint4*>(vz)[x] = make_uint4(0, 0, 0, 0);
    return;
  }

  // ---- head unit.  1. every global load of the workgroup.  Addresses: one
  // 64-bit base per tensor for the tile's first residue (uniform), plus
  // 32-bit offsets within the tile.
  const size_t rh0 = row0 * H + h;                         // its (residue, head) row
  const uint4* kb4 = reinterpret_cast<const uint4*>(a.k) + rh0 * nk;
  const uint4* vb4 = reinterpret_cast<const uint4*>(a.v) + rh0 * nv;
  const uint4* qb4 = reinterpret_cast<const uint4*>(a.q) + rh0 * nk;
  const uint16_t* kpb = reinterpret_cast<const uint16_t*>(a.kp) + rh0 * (3 * P);
  const uint16_t* qpb = reinterpret_cast<const uint16_t*>(a.qp) + rh0 * (3 * P);
  const uint16_t* vpb = reinterpret_cast<const uint16_t*>(a.vp) + rh0 * (3 * Q);
  float fr[13];  // threads 0..63: translation, rotation, mask of residue tid
  if (tid < 64) {
    if (tid < nrow) {
      const uint16_t* tr16 = reinterpret_cast<const uint16_t*>(a.trans) + (row0 + tid) * 3;
      const uint16_t* ro16 = reinterpret_cast<const uint16_t*>(a.rot) + (row0 + tid) * 9;
#pragma unroll
      for (int e = 0; e < 3; ++e) fr[e] = bf16_bits_to_f32(tr16[e]);
#pragma unroll
      for (int e = 0; e < 9; ++e) fr[3 + e] = bf16_bits_to_f32(ro16[e]);
      fr[12] = a.mask[row0 + tid] != 0 ? 1.f : 0.f;
    } else {
#pragma unroll
      for (int e = 0; e < 13; ++e) fr[e] = 0.f;
    }
  }
  const float pwr = ld<true>(a.pwr, h);
  // each loop below covers one tensor, so the lanes of a wavefront never
  // diverge over which tensor a piece comes from
  uint4 k_r[kFastK], q_r[kFastK], v_r[kFastK];
#pragma unroll
  for (int k = 0; k < kFastK; ++k) {
    const int x = tid + 256 * k;
    const int rk = fdiv(x, f.nk), ck = x - rk * nk;
    const bool ink = x < 64 * nk && rk < nrow;
    k_r[k] = ink ? kb4[rk * H * nk + ck] : make_uint4(0, 0, 0, 0);
    q_r[k] = ink ? qb4[rk * H * nk + ck] : make_uint4(0, 0, 0, 0);
    const int rv = fdiv(x, f.nv), cv = x - rv * nv;
    v_r[k] = (x < 64 * nv && rv < nrow) ? vb4[rv * H * nv + cv] : make_uint4(0, 0, 0, 0);
  }
  // points: with pts_vec, 8-byte pieces of each row's [kp | qp | vp] (3 + 3 +
  // 3Q/4 pieces, consecutive lanes on consecutive pieces), staged in LDS
  // below; else one point (3 x bf16) per thread and item
  const int npc = 6 + 3 * Q / 4;
  uint2 ppc[kFastPc];
  float pts[kFastPts][3];
  if (P == 4 && f.pts_vec) {
#pragma unroll
    for (int k = 0; k < kFastPc; ++k) {
      const int x = tid + 256 * k, r = fdiv(x, f.npc), c = x - r * npc;
      const uint16_t* src = c < 3 ? kpb + r * H * 12 + 4 * c
                                  : (c < 6 ? qpb + r * H * 12 + 4 * (c - 3) : vpb + r * H * 3 * Q + 4 * (c - 6));
      ppc[k] = (x < 64 * npc && r < nrow) ? *reinterpret_cast<const uint2*>(src) : make_uint2(0, 0);
    }
  } else {
#pragma unroll
    for (int k = 0; k < kFastPts; ++k) {
      const int x = tid + 256 * k, r = x % 64, it = x / 64;
      pts[k][0] = pts[k][1] = pts[k][2] = 0.f;
      if (x < 64 * npt && r < nrow) {
        const uint16_t* src;
        if (it < P) src = kpb + r * H * 3 * P + 3 * it;
        else if (it < 2 * P) src = qpb + r * H * 3 * P + 3 * (it - P);
        else src = vpb + r * H * 3 * Q + 3 * (it - 2 * P);
        pts[k][0] = bf16_bits_to_f32(src[0]);
        pts[k][1] = bf16_bits_to_f32(src[1]);
        pts[k][2] = bf16_bits_to_f32(src[2]);
      }
    }
  }

  // ---- 2. frames, validity and the tile centroid (wavefront 0)
  if (tid < 64) {
    const int valid = fr[12] != 0.f;
    const float tx = fr[0], ty = fr[1], tz = fr[2];
    s_valid[tid] = valid;
    const uint64_t vm = __ballot(valid);
    if (tid == 0) { s_vmask[0] = (uint32_t)vm; s_vmask[1] = (uint32_t)(vm >> 32); }
    s_tr[tid][0] = tx; s_tr[tid][1] = ty; s_tr[tid][2] = tz;
#pragma unroll
    for (int e = 0; e < 9; ++e) s_rot[tid][e] = fr[3 + e];
    float sx = valid ? tx : 0.f, sy = valid ? ty : 0.f, sz = valid ? tz : 0.f, sn = valid ? 1.f : 0.f;
    for (int off = 32; off > 0; off >>= 1) {
      sx += __shfl_xor(sx, off);
      sy += __shfl_xor(sy, off);
      sz += __shfl_xor(sz, off);
      sn += __shfl_xor(sn, off);
    }
    if (tid == 0) {
      float cx = 0.f, cy = 0.f, cz = 0.f;
      if (sn > 0.f) { cx = sx / sn; cy = sy / sn; cz = sz / sn; }
      // any fixed point near the tile will do; on the 4-angstrom grid it is
      // exact in fp16 and differences of two centroids are exact too
      const float grid = (float)kCentGrid;
      cx = grid * rintf(cx / grid); cy = grid * rintf(cy / grid); cz = grid * rintf(cz / grid);
      cx = f16_bits_to_f32(hi16(cx)); cy = f16_bits_to_f32(hi16(cy)); cz = f16_bits_to_f32(hi16(cz));
      s_c[0] = cx; s_c[1] = cy; s_c[2] = cz; s_c[3] = 0.f;
      s_gam = 0.5f * softplus_f(pwr) * sqrtf(2.0f / (27.0f * (float)P));
    }
  }
  // raw point rows in LDS (the transposition array is free until the points
  // are done): row r at s_praw + kPrPitch r, as bf16 [kp | qp | vp]
  static_assert(64 * kPrPitch * sizeof(uint2) <= sizeof(s_vzT), "staged point rows overflow the transposition array");
  uint2* s_praw = reinterpret_cast<uint2*>(&s_vzT[0][0]);
  if (P == 4 && f.pts_vec) {
#pragma unroll
    for (int k = 0; k < kFastPc; ++k) {
      const int x = tid + 256 * k, r = fdiv(x, f.npc), c = x - r * npc;
      if (x < 64 * npc) s_praw[r * kPrPitch + c] = ppc[k];
    }
  }
  __syncthreads();
  const float cx = s_c[0], cy = s_c[1], cz = s_c[2];
  const float gam = s_gam;
  const float gl = gam * kLog2e;

  if (b == 0 && t == 0) {
    // this head's pair weights [w_pair[h, c % Cz] | 0], bf16 as given
    uint16_t* wp = reinterpret_cast<uint16_t*>(a.ws + wp_row_off(L, h));
    for (int c = tid; c < L.ZW; c += 256)
      wp[c] = c < RCz ? reinterpret_cast<const uint16_t*>(a.wpair)[(size_t)h * Cz + c % Cz] : (uint16_t)0;
  }
  if (tid == 64) {
    if (b == 0 && t == 0) reinterpret_cast<float*>(a.ws + L.off_gam)[h] = gam;
    if (h == 0) {
      *reinterpret_cast<float4*>(a.ws + ck_off(L, b, t)) = make_float4(cx, cy, cz, 0.f);
      if (b == 0 && t == 0) {
        Header* hd = reinterpret_cast<Header*>(a.ws);
        hd->magic = kMagic;
        hd->has_pair_mask = a.pm != nullptr;
      }
    }
  }
  if (tid >= 128 && tid < 130 && h == 0) {
    // word hw holds the keys of the 4-key groups 2k + hw (k = 0..7), group by
    // group (the bit order of mask_bit_of_key)
    const int hw = tid - 128;
    const uint64_t vm = (uint64_t)s_vmask[0] | ((uint64_t)s_vmask[1] << 32);
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) w |= (uint32_t)((vm >> (4 * (2 * k + hw))) & 0xFu) << (4 * k);
    *reinterpret_cast<uint32_t*>(a.ws + km_word_off(L, b, t, hw)) = w;
  }
  // a tile without a valid residue is never read: the fused kernel skips
  // key tiles without a valid key and writes padding queries as zeros
  const bool tile_any = (s_vmask[0] | s_vmask[1]) != 0u;
  if (tile_any) {
    // ---- 3. points, then k straight into the key rows and v transposed
    // into LDS.  Global points: key points (centred), query points, value
    // points (centred, zero for keys that are masked or past the end)
#pragma unroll
    for (int k = 0; k < kFastPts; ++k) {
      const int x = tid + 256 * k, r = x % 64, it = x / 64;
      if (x < 64 * npt) {
        const bool in = t * 64 + r < N;
        const float* Rm = s_rot[r];
        const float tx = s_tr[r][0], ty = s_tr[r][1], tz = s_tr[r][2];
        float lx, ly, lz;
        if (P == 4 && f.pts_vec) {
          // point it of the row is at bf16 3 it of [kp | qp | vp] (3P = 12)
          const uint16_t* pr = reinterpret_cast<const uint16_t*>(s_praw + r * kPrPitch) + 3 * it;
          lx = bf16_bits_to_f32(pr[0]); ly = bf16_bits_to_f32(pr[1]); lz = bf16_bits_to_f32(pr[2]);
          if (r >= nrow) lx = ly = lz = 0.f;
        } else {
          lx = pts[k][0]; ly = pts[k][1]; lz = pts[k][2];
        }
        const float gx = Rm[0] * lx + Rm[1] * ly + Rm[2] * lz + tx;
        const float gy = Rm[3] * lx + Rm[4] * ly + Rm[5] * lz + ty;
        const float gz = Rm[6] * lx + Rm[7] * ly + Rm[8] * lz + tz;
        if (it < P) {
          s_w[r][3 * it] = in ? gx - cx : 0.f;
          s_w[r][3 * it + 1] = in ? gy - cy : 0.f;
          s_w[r][3 * it + 2] = in ? gz - cz : 0.f;
        } else if (it < 2 * P) {
          const int p = it - P;
          s_a[r][3 * p] = gx; s_a[r][3 * p + 1] = gy; s_a[r][3 * p + 2] = gz;
        } else {
          const int q = it - 2 * P;
          const bool v = in && s_valid[r];
          s_xT[3 * q][r] = v ? gx - cx : 0.f;
          s_xT[3 * q + 1][r] = v ? gy - cy : 0.f;
          s_xT[3 * q + 2][r] = v ? gz - cz : 0.f;
        }
      }
    }
    __syncthreads();  // the raw point rows are read; the staging array is free
    uint16_t* kt = reinterpret_cast<uint16_t*>(a.ws + kt_tile_off(L, b, h, t));
    auto vh = [](uint16_t bits) { return f32_to_f16_bits(bf16_bits_to_f32(bits) * kVScale); };
#pragma unroll
    for (int k = 0; k < kFastK; ++k) {
      const int x = tid + 256 * k;
      const int rk = fdiv(x, f.nk), ck = x - rk * nk;
      if (x < 64 * nk)
        *reinterpret_cast<uint4*>(kt + (size_t)rk * L.KROW + 8 * ck) = s_valid[rk] ? k_r[k] : make_uint4(0, 0, 0, 0);
      const int rv = fdiv(x, f.nv), cv = x - rv * nv;
      if (x < 64 * nv) {
        const uint4 val = s_valid[rv] ? v_r[k] : make_uint4(0, 0, 0, 0);
        const uint16_t* e16 = reinterpret_cast<const uint16_t*>(&val);
#pragma unroll
        for (int e = 0; e < 8; ++e) s_vzT[8 * cv + e][rv] = vh(e16[e]);
      }
    }
    // lifted query rows [q sq | 0] (the pair part of the query operand is
    // formed by the fused kernel from the shared zl rows and w_pair)
    {
      const float sq = kLog2e / sqrtf(3.0f * (float)D);
      uint16_t* ql = reinterpret_cast<uint16_t*>(a.ws + ql_row_off(L, b, h, t * 64));
#pragma unroll
      for (int k = 0; k < kFastK; ++k) {
        const int x = tid + 256 * k, r = fdiv(x, f.nk), c = x - r * nk;
        if (x < 64 * nk) {
          const uint16_t* e16 = reinterpret_cast<const uint16_t*>(&q_r[k]);
          uint4 pk;
          pk.x = pack_bf16x2(bf16_bits_to_f32(e16[0]) * sq, bf16_bits_to_f32(e16[1]) * sq);
          pk.y = pack_bf16x2(bf16_bits_to_f32(e16[2]) * sq, bf16_bits_to_f32(e16[3]) * sq);
          pk.z = pack_bf16x2(bf16_bits_to_f32(e16[4]) * sq, bf16_bits_to_f32(e16[5]) * sq);
          pk.w = pack_bf16x2(bf16_bits_to_f32(e16[6]) * sq, bf16_bits_to_f32(e16[7]) * sq);
          *reinterpret_cast<uint4*>(ql + (size_t)r * QW + 8 * c) = pk;
        }
      }
      // zero columns [D, 16)
      const int nz0 = (16 - D) / 8;
      if (nz0 > 0)
        for (int x = tid; x < 64 * nz0; x += 256) {
          const int r = x / nz0, c = x - r * nz0;
          *reinterpret_cast<uint4*>(ql + (size_t)r * QW + D + 8 * c) = make_uint4(0, 0, 0, 0);
        }
    }
    __syncthreads();

    // ---- 4. key rows past k (one thread per key): zeros up to 16, the
    // geometric columns (layout in common.h), 8 pad columns
    {
      // every wavefront: lane = key, chunks w, w + 4, ... of the 16 GS + 8
      // columns after 16; each lane recomputes its key's point sums
      const int r = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
      const bool valid = s_valid[r] != 0;
      float w[P3];
#pragma unroll
      for (int g = 0; g < P3; ++g) w[g] = s_w[r][g];
      float nb = 0.f, Wx = 0.f, Wy = 0.f, Wz = 0.f;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        nb += w[3 * p] * w[3 * p] + w[3 * p + 1] * w[3 * p + 1] + w[3 * p + 2] * w[3 * p + 2];
        Wx += w[3 * p]; Wy += w[3 * p + 1]; Wz += w[3 * p + 2];
      }
      nb = -gl * nb;
      const float ww[3] = {2.f * gl * Wx, 2.f * gl * Wy, 2.f * gl * Wz};
      uint16_t* krow = kt + (size_t)r * L.KROW;
      if (wv == 0)
        for (int c = D; c < 16; c += 8) *reinterpret_cast<uint4*>(krow + c) = make_uint4(0, 0, 0, 0);
      constexpr int base = 16 * (GS - 1);
      constexpr int NCH = (16 * GS + 8) / 8;
      // value of geometric column g of this key (layout in common.h)
      auto geo = [&](int g) -> uint16_t {
        uint16_t val = 0;
        if constexpr (STK) {
          // stacked comparison: global key points b = w + c in bf16
          if (g < 5 * P) {
            const int p = g / 5, e = g % 5;
            const float bx = w[3 * p] + cx, by = w[3 * p + 1] + cy, bz = w[3 * p + 2] + cz;
            if (e < 3) val = f32_to_bf16_bits(2.f * gl * (e == 0 ? bx : (e == 1 ? by : bz)));
            else if (e == 3) val = f32_to_bf16_bits(-gl);
            else val = f32_to_bf16_bits(-gl * (bx * bx + by * by + bz * bz));
          } else if (g > kStkMaskCol && g < 32) {
            val = 0x4180;  // bf16 16.0, multiplies the query's -m/16 parts
          }
          if (!valid) val = g == kStkMaskCol ? (uint16_t)0xC780 : (g > kStkMaskCol && g < 32 ? val : (uint16_t)0);
          return val;
        }
        if (g < base + 4) {
          if (g < P3) val = hi16(w[g]);
          else if (g < 2 * P3) val = lo16(w[g - P3]);
          else if (g < 3 * P3) val = hi16(w[g - 2 * P3]);
        } else if (g < 16 * GS) {
          const int y = g - base;
          if (y == 4) val = hi16(nb * (1.0f / kNormScale));
          else if (y == 12) val = lo16(nb * (1.0f / kNormScale));
          else if (y >= 5 && y <= 7) val = hi16(ww[y - 5]);
          else if (y >= 13) val = lo16(ww[y - 13]);
          else if (y >= 9 && y <= 11) val = 0x4C00;  // fp16 16.0, multiplies the query's t'/16 parts
        }
        // a masked key (or one past the end) is all zeros but for -65504 in
        // the key-mask column, which the query side multiplies by 16
        return valid ? val : (g == base + 8 ? (uint16_t)0xFBFF : (uint16_t)0);
      };
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (c % 4 != wv) continue;
        uint16_t g16[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) g16[e] = geo(8 * c + e);
        *reinterpret_cast<uint4*>(krow + 16 + 8 * c) = pack8(g16);
      }
    }
    // query global points: 16 floats per (b, h, i)
    {
      float4* qa = reinterpret_cast<float4*>(a.ws + qa_row_off(L, b, h, t * 64));
      const int row = tid / 4, c = (tid % 4) * 4;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (row < nrow && c + e < P3) ? s_a[row][c + e] : 0.f;
      qa[tid] = make_float4(v[0], v[1], v[2], v[3]);
    }
    // head value rows, transposed: rows [0, Dv) from the LDS copy of v, the
    // rest computed (ones rows, centred value points, centroid)
    uint16_t* vt = reinterpret_cast<uint16_t*>(a.ws + vt_tile_off(L, b, h, t));
    store_vt_rows(vt, s_vzT, Dv, tid);
    const uint32_t vm0 = s_vmask[0], vm1 = s_vmask[1];
    for (int x = tid; x < (64 - Dv) * 8; x += 256) {
      const int d = Dv + (x >> 3), j0 = vt_key_of_col(8 * (x & 7));
      // valid bits of the 8 keys, in column order
      const uint32_t word = j0 < 32 ? vm0 : vm1;
      const uint32_t bits = ((word >> (j0 & 31)) & 0xFu) | (((word >> ((j0 & 31) + 8)) & 0xFu) << 4);
      uint16_t one = 0;
      const int dd = d - 32;
      if (d == Dv) one = 0x3C00;                          // fp16 1.0: weight sum
      else if (dd == 3 * Q) one = 0x3C00;                 // fp16 1.0: weight sum
      else if (dd > 3 * Q && dd <= 3 * Q + 3) one = hi16(s_c[dd - 3 * Q - 1]);  // centroid
      uint16_t out[8];
      if (dd >= 0 && dd < 3 * Q) {
        const float4 lo = *reinterpret_cast<const float4*>(&s_xT[dd][j0]);
        const float4 hi = *reinterpret_cast<const float4*>(&s_xT[dd][j0 + 8]);
        out[0] = hi16(lo.x); out[1] = hi16(lo.y); out[2] = hi16(lo.z); out[3] = hi16(lo.w);
        out[4] = hi16(hi.x); out[5] = hi16(hi.y); out[6] = hi16(hi.z); out[7] = hi16(hi.w);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = ((bits >> e) & 1u) ? one : (uint16_t)0;
      }
      *reinterpret_cast<uint4*>(vt + (size_t)d * kVCols + 8 * (x & 7)) = pack8(out);
    }
    // pad columns 64 .. 71 of the computed rows
    for (int d = Dv + tid; d < 64; d += 256)
      *reinterpret_cast<uint4*>(vt + (size_t)d * kVCols + 64) = make_uint4(0, 0, 0, 0);
  }

  // ---- 5. permitted-key words of every query row for this key tile
  // (the H workgroups of the tile share the query rows: rows h, h + H, ...)
  if (a.pm != nullptr) {
    for (int i = tid * H + h; i < L.NQpad; i += 256 * H) {
      uint32_t w[2] = {0u, 0u};
      if (tile_any && i < N && a.mask[(size_t)b * N + i]) {
        const uint8_t* row = a.pm + ((size_t)b * N + i) * N + (size_t)t * 64;
        if (f.pm_vec) {
          // N is a multiple of 16 and the rows are 16-byte aligned
          uint4 v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            v[q] = t * 64 + 16 * q < N ? *reinterpret_cast<const uint4*>(row + 16 * q) : make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t wd[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int jj = 16 * q + e;
              int hf;
              const int bit = mask_bit_of_key(jj, &hf);
              if (((wd[e >> 2] >> (8 * (e & 3))) & 0xFFu) && s_valid[jj]) w[hf] |= 1u << bit;
            }
          }
        } else {
          for (int jj = 0; jj < 64; ++jj) {
            if (t * 64 + jj >= N) break;
            if (s_valid[jj] && row[jj]) {
              int hf;
              const int bit = mask_bit_of_key(jj, &hf);
              w[hf] |= 1u << bit;
            }
          }
        }
      }
      *reinterpret_cast<uint32_t*>(a.ws + pm_word_off(L, b, i, t, 0)) = w[0];
      *reinterpret_cast<uint32_t*>(a.ws + pm_word_off(L, b, i, t, 1)) = w[1];
    }
  }
}

hipError_t launch_lift(const Layout& L, const ipa_lift_in* in, void* ws, hipStream_t st) {
  LiftArgs a;
  a.L = L;
  a.q = in->q; a.k = in->k; a.v = in->v;
  a.qp = in->q_points; a.kp = in->k_points; a.vp = in->v_points;
  a.rot = in->rotation; a.trans = in->translation; a.pwr = in->point_weight_raw;
  a.wpair = in->w_pair; a.zl = in->zl; a.zr = in->zr;
  a.mask = in->mask; a.pm = in->pair_mask;
  a.ws = reinterpret_cast<char*>(ws);
  dim3 grid(L.NT, L.H, L.B);
  const bool aligned = (reinterpret_cast<uintptr_t>(in->q) | reinterpret_cast<uintptr_t>(in->k) |
                        reinterpret_cast<uintptr_t>(in->v) | reinterpret_cast<uintptr_t>(in->zl) |
                        reinterpret_cast<uintptr_t>(in->zr)) % 16 == 0;
  if (L.stacked) {
    // the stacked comparison runs on the fast kernel only (P = 4, checked by
    // the caller)
    if (!aligned || !lift_fast_fits(L) || L.P != 4) return hipErrorInvalidValue;
  }
  if (aligned && lift_fast_fits(L)) {
    LiftFastArgs f;
    f.units = L.B * L.NT * (L.H + 1);
    f.per_xcd = (f.units + 7) / 8;
    f.pm_vec = in->pair_mask != nullptr && L.N % 16 == 0 && reinterpret_cast<uintptr_t>(in->pair_mask) % 16 == 0;
    f.nz = make_fastdiv(L.RCz / 8);
    f.nk = make_fastdiv(L.D / 8);
    f.nv = make_fastdiv(L.Dv / 8);
    f.pts_vec = L.P == 4 && L.Q % 4 == 0 && 6 + 3 * L.Q / 4 <= kPrPitch;
    f.npc = make_fastdiv(6 + 3 * L.Q / 4);
    f.nkz = make_fastdiv((L.KZROW - L.RCz) / 8 > 0 ? (L.KZROW - L.RCz) / 8 : 1);
    const dim3 g(8 * f.per_xcd), blk(256);
    switch (L.P) {
      case 1: hipLaunchKernelGGL(lift_fast_kernel<1>, g, blk, 0, st, a, f); break;
      case 2: hipLaunchKernelGGL(lift_fast_kernel<2>, g, blk, 0, st, a, f); break;
      case 3: hipLaunchKernelGGL(lift_fast_kernel<3>, g, blk, 0, st, a, f); break;
      case 4:
        if (L.stacked)
          hipLaunchKernelGGL((lift_fast_kernel<4, true>), g, blk, 0, st, a, f);
        else
          hipLaunchKernelGGL(lift_fast_kernel<4>, g, blk, 0, st, a, f);
        break;
      default: hipLaunchKernelGGL(lift_fast_kernel<5>, g, blk, 0, st, a, f); break;
    }
  } else if (L.mfma)
    hipLaunchKernelGGL(lift_kernel<true>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(lift_kernel<false>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace fipa
