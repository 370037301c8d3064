// Internal definitions shared by the FlashIPA HIP sources: the layout of the
// opaque "lifted" workspace, tile constants and small conversion helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/flashipa.h"

namespace fipa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Key tile: 64 keys.  Query tile of the matrix-core kernel: 4 waves x 32.
constexpr int kKeyTile = 64;
constexpr int kQueryTile = 128;
// Geometric columns of a lifted key row on the matrix-core path: GS MFMA
// K-steps of 16 (GS = 3 for P <= 4, 4 for P = 5).  With c_t the centroid of
// key tile t and c_w the centroid of the queries of one wavefront (both on a
// 4-angstrom grid, so delta = c_t - c_w is exact in fp16), A = a - c_w and
// w = b - c_t, the point term of the logit (log2 units, gl = gamma log2 e) is
//   -gl sum_p |a_p - b_p|^2 = 2 gl A.w  - gl |w|^2  - 2 gl delta.W  + t'
// with W = sum_p w_p and t' = -gl sum_p |a_p - c_t|^2 (per query and tile).
// Columns 0 .. 16(GS-1)+3 hold the 9P cross products of the fp16 hi/lo
// splits (u = 2 gl A against w): pairs [u_hi.w_hi | u_hi.w_lo | u_lo.w_hi].
// The last K-step holds, with base = 16(GS-1) (query value x key value):
//   base+4:  16 x nb_hi      base+12: 16 x nb_lo     (nb = -gl|w|^2 / 16)
//   base+8:  16 x (-65504 for a masked key, 0 otherwise)
//   base+5..7: -delta x WW_hi  base+13..15: -delta x WW_lo  (WW = 2 gl W)
//   base+9..11: (t' - m)/16 in three fp16 parts x 16 (m: the query's running
//               maximum in the fused kernel, 0 for plain logits)
// so that the MFMA itself returns the complete logit.
//
// Stacked layout (the comparison of the pages' own scheme, Layout::stacked):
// the point term as five bf16 columns per point in global coordinates, no
// centring and no hi/lo split, GS = 2 bf16 K-steps.  Key side, point p:
// [2 gl b_p (3) | -gl | -gl |b_p|^2] at columns 5p .. 5p+4; query side
// [a_p (3) | |a_p|^2 | 1], so the product is -gl |a_p - b_p|^2.  Column 28 is
// the key-mask column (key -65536 when masked, query 16) and columns 29..31
// carry the query's -m/16 in three bf16 parts against a key value of 16.
constexpr int kStkMaskCol = 28;
// log2(e) / sqrt(3): the pair bias enters the logit divided by sqrt(3), in
// log2 units
constexpr float kPairScale = (float)(1.4426950408889634 / 1.7320508075688772);
constexpr int kCentGrid = 4;  // angstrom
constexpr float kNormScale = 16.0f;
// The value tile is fp16 throughout (the probabilities multiply it as fp16).
// Values and pair factors enter it times 2^-8: every bf16 value of magnitude
// up to 1.6e7 stays in range, those of magnitude >= 2^-6 convert exactly and
// smaller ones with an absolute error below 2^-17; the fused kernel's
// normalisation multiplies the 2^8 back.
constexpr float kVScale = 1.0f / 256.0f;
__host__ __device__ __forceinline__ int geo_steps(int P) { return P <= 4 ? 3 : 4; }

// Padding (in 16-bit elements) appended to every LDS row so that the
// 16-byte fragment reads of 16 consecutive rows hit distinct banks.
constexpr int kRowPad = 8;
constexpr int kVCols = kKeyTile + kRowPad;  // 72 elements = 144 bytes
constexpr uint32_t kMagic = 0x46495041u;    // "FIPA"

// Matrix-core kernel instances: (NQS, NVB, GS) = number of 16-wide bf16
// K-steps of the scalar+pair query columns (one for the scalar part, NQS - 1
// for the pair part), number of 32-row value blocks besides the one of the
// value points (one for the values, NVB - 1 for the pair part), number of
// fp16 geometric K-steps.
struct MfmaDims {
  int NQS, NVB, GS;
};

// Workspace header, first 256 bytes of the lifted buffer.
struct Header {
  uint32_t magic;
  uint32_t has_pair_mask;
  uint32_t pad[62];
};

// Everything a kernel needs to find its rows in the lifted workspace.
struct Layout {
  int B, N, H, D, Dv, P, Q, Cz, R, Cout;
  int RCz;   // R*Cz
  int NT;    // key tiles of 64
  int NKpad; // NT*64 key rows
  int NQpad; // query rows rounded up to 128
  int mfma;  // 1: matrix-core path (bf16 input), 0: fp32 path
  int stacked;  // 1: the pages' stacked point columns (bf16, global coordinates), comparison only
  int NQS, NVB, GS;
  int QW;     // per-head query row width (elements): mfma 16 (the scalar columns); fp32 D + R Cz padded
  int ZW;     // mfma: query pair columns 16 (NQS - 1), shared by the heads (QZ rows, WP rows)
  int KROW;   // elements per key row (mfma: head part 16 + 16 GS + pad; fp32: DKP)
  int VROWS;  // mfma: rows of the head part of the transposed value tile (64); fp32: DVP (row stride)
  int KZROW;  // mfma: elements per row of the shared pair-factor key tile, 16 (NQS - 1) + pad
  int VZROWS; // mfma: rows of the shared pair-factor value tile, 32 (NVB - 1)
  int DQP;    // fp32 path: padded query row width
  int DO;     // attention output width Dv + R*Cz + 3Q
  int has_pm;
  int F, FP;  // epilogue feature count, padded to 16
  int KS;     // matrix-core path: key ranges the fused kernel splits a query tile over
  int PREC;   // floats per partial-result record (KS > 1): DO values + 4 statistics, padded to 4
  size_t off_ql, off_qz, off_wp, off_qa, off_kt, off_vt, off_ktz, off_vtz, off_ck, off_gam, off_km, off_part, off_pm,
      total;
  size_t epi_ws;  // bytes of the epilogue's own workspace (packed w_out)
};

// Key ranges per query tile of the fused kernel: when (b, h, 256-query tile)
// workgroups do not fill the 256 compute units, the keys are split into KS
// ranges (at most 4, of at least 4 tiles each), one workgroup per range, and
// a combine kernel merges the partial results.
static inline int key_splits(int B, int N, int H, int NT) {
  const long n8 = (long)((N + 255) / 256) * H * B;
  if (n8 >= 256) return 1;
  int ks = (int)((256 + n8 - 1) / n8);
  ks = ks < 4 ? ks : 4;
  ks = ks < NT / 4 ? ks : NT / 4;
  return ks > 1 ? ks : 1;
}

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Choose the smallest compiled matrix-core instance that holds the shape:
// the scalar query/key columns fit one K-step (D <= 16), the values and
// their ones row one value block (Dv + 1 <= 32), the value points, ones row
// and centroid another (3Q + 4 <= 32), and the R Cz pair columns the rest.
// Returns false when none does.
static inline bool pick_mfma_dims(int D, int Dv, int RCz, int P, int Q, MfmaDims* out) {
  static const MfmaDims inst[] = {{3, 2, 0}, {5, 3, 0}, {9, 5, 0}, {13, 7, 0}};
  if (P > 5) return false;
  if (3 * Q + 4 > 32 || D > 16 || Dv + 1 > 32) return false;
  for (const MfmaDims& m : inst) {
    if (RCz <= 16 * (m.NQS - 1) && RCz <= 32 * (m.NVB - 1)) {
      *out = m;
      out->GS = geo_steps(P);
      return true;
    }
  }
  return false;
}

// Epilogue per-head product: the features of one head (Dv=16, 4 x Q=8,
// Cz=64) and their row pitch in LDS and in the packed w_out (elements).
constexpr int kHeadFeat = 112;
constexpr int kHeadFeatPitch = 120;

// Limits of the fp32 kernels (registers sized at compile time).
constexpr int kF32MaxDQ = 160;   // D + R*Cz
constexpr int kF32MaxDV = 192;   // Dv + R*Cz + 3Q (4 threads x 48)
constexpr int kMaxP = 5;   // 3P <= 15 point coordinates per lifted row
constexpr int kMaxQ = 10;  // 3Q <= 30 value-point coordinates

static inline bool make_layout(const ipa_shape* s, int with_pm, Layout* L, int stacked = 0) {
  if (!s) return false;
  L->stacked = stacked ? 1 : 0;
  if (s->B <= 0 || s->N <= 0 || s->H <= 0 || s->D <= 0 || s->Dv <= 0 || s->P <= 0 || s->Q <= 0 ||
      s->Cz <= 0 || s->R <= 0 || s->Cout <= 0)
    return false;
  if (s->N > (1 << 24) || s->B > (1 << 20) || s->H > 64 || s->Cout > 4096) return false;
  L->B = (int)s->B; L->N = (int)s->N; L->H = (int)s->H; L->D = (int)s->D; L->Dv = (int)s->Dv;
  L->P = (int)s->P; L->Q = (int)s->Q; L->Cz = (int)s->Cz; L->R = (int)s->R; L->Cout = (int)s->Cout;
  L->RCz = L->R * L->Cz;
  L->NT = (L->N + kKeyTile - 1) / kKeyTile;
  L->NKpad = L->NT * kKeyTile;
  L->NQpad = round_up(L->N, kQueryTile);
  L->DO = L->Dv + L->RCz + 3 * L->Q;
  L->F = L->H * (L->Dv + 4 * L->Q + L->Cz);
  L->FP = round_up(L->F, 16);
  L->has_pm = with_pm ? 1 : 0;
  if (L->P > kMaxP || L->Q > kMaxQ) return false;
  const size_t B = L->B, H = L->H, NT = L->NT, NQ = L->NQpad, NK = L->NKpad;
  if (s->dtype == IPA_BF16) {
    MfmaDims md;
    if (!pick_mfma_dims(L->D, L->Dv, L->RCz, L->P, L->Q, &md)) return false;
    L->mfma = 1;
    // the stacked comparison is compiled for the standard widths only
    if (stacked) {
      if (md.NQS != 9 || md.NVB != 5 || L->P != 4 || L->D % 8 || L->Dv % 8 || L->Cz % 8) return false;
      md.GS = 2;
    }
    L->NQS = md.NQS; L->NVB = md.NVB; L->GS = md.GS;
    L->QW = 16;
    L->ZW = 16 * (md.NQS - 1);
    L->KROW = 16 + 16 * md.GS + kRowPad;
    L->VROWS = 64;
    L->KZROW = 16 * (md.NQS - 1) + kRowPad;
    L->VZROWS = 32 * (md.NVB - 1);
    L->DQP = 16 * md.NQS;
    L->KS = key_splits(L->B, L->N, L->H, L->NT);
  } else if (s->dtype == IPA_F32) {
    if (stacked) return false;
    if (L->D + L->RCz > kF32MaxDQ || L->DO > kF32MaxDV) return false;
    L->mfma = 0;
    L->NQS = L->NVB = L->GS = 0;
    L->KS = 1;
    L->DQP = round_up(L->D + L->RCz, 4);
    L->QW = L->DQP;
    L->ZW = 0;
    L->KROW = round_up(L->D + L->RCz + 3 * L->P, 4);
    L->VROWS = round_up(L->DO, 4);
    L->KZROW = L->VZROWS = 0;
  } else {
    return false;
  }
  size_t off = 256;  // header
  L->off_ql = off;
  off = align256(off + B * H * NQ * L->QW * (L->mfma ? 2 : 4));
  // matrix-core path: the query pair factors zl, shared by the heads, and the
  // per-head pair weights w_pair, each padded to ZW columns (bf16); the fused
  // kernel forms the pair part of its query operand from them
  L->off_qz = off;
  off = align256(off + B * NQ * (size_t)L->ZW * 2);
  L->off_wp = off;
  off = align256(off + H * (size_t)L->ZW * 2);
  L->off_qa = off;
  off = align256(off + B * H * NQ * 16 * 4);
  L->off_kt = off;
  off = align256(off + B * H * NK * L->KROW * (L->mfma ? 2 : 4));
  L->off_vt = off;
  if (L->mfma)
    off = align256(off + B * H * NT * (size_t)L->VROWS * kVCols * 2);
  else
    off = align256(off + B * H * NK * (size_t)L->VROWS * 4);
  // pair-factor key and value tiles, shared by the H heads (matrix-core path)
  L->off_ktz = off;
  if (L->mfma) off = align256(off + B * NT * (size_t)kKeyTile * L->KZROW * 2);
  L->off_vtz = off;
  if (L->mfma) off = align256(off + B * NT * (((size_t)L->VZROWS * kVCols * 2 + 1023) / 1024 * 1024));
  L->off_ck = off;
  off = align256(off + B * NT * 4 * 4);
  L->off_gam = off;
  off = align256(off + H * 4);
  L->off_km = off;
  off = align256(off + B * NT * 2 * 4);
  // partial results of the key ranges: [KS][B][H][NQpad][PREC] fp32 (before
  // the pair-mask region, whose presence does not move it)
  L->PREC = round_up(L->DO + 4, 4);
  L->off_part = off;
  if (L->KS > 1) off = align256(off + (size_t)L->KS * B * H * NQ * L->PREC * 4);
  L->off_pm = off;
  if (with_pm) off = align256(off + B * NQ * NT * 2 * 4);
  L->total = off;
  // the epilogue's workspace (separate from the lifted rows): the output
  // projection transposed to [Cout][FP] bf16, or per head to
  // [H][Cout][kHeadFeatPitch] bf16 (matrix-core path); none on the fp32 path
  {
    const size_t a1 = (size_t)L->Cout * L->FP, a2 = (size_t)L->H * L->Cout * kHeadFeatPitch;
    L->epi_ws = L->mfma ? align256((a1 > a2 ? a1 : a2) * 2) : 0;
  }
  return true;
}

// Byte offsets of the records of the lifted workspace, used by the kernels
// that write and read them and by the host-side bounds check of the tests.
// Region sizes (make_layout): QL B H NQpad QW e, QZ B NQpad ZW 2, WP H ZW 2,
// QA B H NQpad 64, KT B H NT
// (64 KROW e), VT B H NT (VROWS kVCols 2 | NKpad/NT 64 VROWS 4), KTZ B NT
// (64 KZROW 2), VTZ B NT (VZROWS kVCols 2 rounded up to KiB), CK B NT 16,
// KM B NT 8, PART KS B H NQpad PREC 4, PM B NQpad NT 8 (e = 2 on the
// matrix-core path, 4 on the fp32 path; KTZ and VTZ empty on the fp32 path).
//
// Matrix-core path, query side:
//   QL  (per head)   rows [q log2e/sqrt(3D) (D, zero to 16)], bf16
//   QZ  (shared)     rows [zl (R Cz, zero to ZW)], bf16, the inputs as given
//   WP  (per head)   [w_pair[h, c % Cz] for c < R Cz, zero to ZW], bf16
// the fused kernel's query operand is QL and bf16((WP x QZ) x kPairScale).
// Matrix-core path, one key tile of 64 keys:
//   KT  (per head)   rows [k (D, zero to 16) | geometric 16 GS | pad 8], bf16 / fp16
//   KTZ (shared)     rows [zr (R Cz, zero to 16 (NQS - 1)) | pad 8], bf16
//   VT  (per head)   64 rows x kVCols, fp16, transposed (one column per key):
//                    rows 0..31  [v 2^-8 (Dv) | 1 | 0 ...]
//                    rows 32..63 [x - c_t (3Q) | 1 | c_t (3) | 0 ...]
//   VTZ (shared)     VZROWS rows x kVCols, fp16 [zr 2^-8 (R Cz) | 0 ...]
// The four parts are whole KiB each, and the fused kernel copies them into
// one LDS buffer in this order; the value part then reads as one tile of
// 64 + VZROWS rows (value blocks 0 and 1 per head, 2 .. NVB pair factors).
__host__ __device__ __forceinline__ size_t lifted_elem(const Layout& L) { return L.mfma ? 2 : 4; }
__host__ __device__ __forceinline__ size_t kt_tile_bytes(const Layout& L) {
  return (size_t)kKeyTile * L.KROW * lifted_elem(L);
}
__host__ __device__ __forceinline__ size_t vt_tile_bytes(const Layout& L) {
  return L.mfma ? (size_t)L.VROWS * kVCols * 2 : (size_t)kKeyTile * L.VROWS * 4;
}
__host__ __device__ __forceinline__ size_t ktz_tile_bytes(const Layout& L) { return (size_t)kKeyTile * L.KZROW * 2; }
__host__ __device__ __forceinline__ size_t vtz_tile_bytes(const Layout& L) {
  return ((size_t)L.VZROWS * kVCols * 2 + 1023) / 1024 * 1024;
}
__host__ __device__ __forceinline__ size_t ktz_tile_off(const Layout& L, int b, int t) {
  return L.off_ktz + ((size_t)b * L.NT + t) * ktz_tile_bytes(L);
}
__host__ __device__ __forceinline__ size_t vtz_tile_off(const Layout& L, int b, int t) {
  return L.off_vtz + ((size_t)b * L.NT + t) * vtz_tile_bytes(L);
}
__host__ __device__ __forceinline__ size_t kt_tile_off(const Layout& L, int b, int h, int t) {
  return L.off_kt + (((size_t)b * L.H + h) * L.NT + t) * kt_tile_bytes(L);
}
__host__ __device__ __forceinline__ size_t vt_tile_off(const Layout& L, int b, int h, int t) {
  return L.off_vt + (((size_t)b * L.H + h) * L.NT + t) * vt_tile_bytes(L);
}
__host__ __device__ __forceinline__ size_t ql_row_off(const Layout& L, int b, int h, int i) {
  return L.off_ql + (((size_t)b * L.H + h) * L.NQpad + i) * (size_t)L.QW * lifted_elem(L);
}
__host__ __device__ __forceinline__ size_t qz_row_off(const Layout& L, int b, int i) {
  return L.off_qz + ((size_t)b * L.NQpad + i) * (size_t)L.ZW * 2;
}
__host__ __device__ __forceinline__ size_t wp_row_off(const Layout& L, int h) {
  return L.off_wp + (size_t)h * L.ZW * 2;
}
__host__ __device__ __forceinline__ size_t qa_row_off(const Layout& L, int b, int h, int i) {
  return L.off_qa + (((size_t)b * L.H + h) * L.NQpad + i) * 64;
}
__host__ __device__ __forceinline__ size_t ck_off(const Layout& L, int b, int t) {
  return L.off_ck + ((size_t)b * L.NT + t) * 16;
}
__host__ __device__ __forceinline__ size_t km_word_off(const Layout& L, int b, int t, int half) {
  return L.off_km + (((size_t)b * L.NT + t) * 2 + half) * 4;
}
__host__ __device__ __forceinline__ size_t pm_word_off(const Layout& L, int b, int i, int t, int half) {
  return L.off_pm + ((((size_t)b * L.NQpad + i) * L.NT + t) * 2 + half) * 4;
}
__host__ __device__ __forceinline__ size_t part_rec_off(const Layout& L, int s, int b, int h, int i) {
  return L.off_part + ((((size_t)s * L.B + b) * L.H + h) * L.NQpad + i) * (size_t)L.PREC * 4;
}

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t u) {
  return __uint_as_float(((uint32_t)u) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {  // round to nearest even
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t u) {
  return (float)__builtin_bit_cast(_Float16, u);
}

// Load element i of an input tensor stored as fp32 or bf16.
template <bool BF>
__device__ __forceinline__ float ld(const void* p, size_t i) {
  if constexpr (BF) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  } else {
    return reinterpret_cast<const float*>(p)[i];
  }
}

// Key index inside a 64-key tile that lives in column kappa of a transposed
// value tile.  Within every 16 keys the order is [0-3, 8-11, 4-7, 12-15]:
// this is the order in which an MFMA 32x32 accumulator lane holds the
// probabilities it feeds back as the B operand of the value product.
__host__ __device__ __forceinline__ int vt_key_of_col(int kappa) {
  const int g = kappa >> 4, half = (kappa >> 3) & 1, e = kappa & 7;
  return 16 * g + 8 * (e >> 2) + 4 * half + (e & 3);
}

// Mask words: every 64-key tile has two 32-bit words, one per half of a
// wavefront.  A lane of half h of a 32x32 accumulator holds keys
// kb*32 + 8*(r/4) + 4*h + r%4 (kb = 0..1, r = 0..15) and reads them as bit
// kb*16 + r of word h.  Returns that bit and sets *half_out = h for key jj.
__host__ __device__ __forceinline__ int mask_bit_of_key(int jj, int* half_out) {
  const int kb = jj >> 5, rem = jj & 31;
  *half_out = (rem >> 2) & 1;
  return kb * 16 + 4 * (rem >> 3) + (rem & 3);
}

}  // namespace fipa
