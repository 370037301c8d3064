// Host-side bounds check of the lifted workspace and of the direct
// global -> LDS tile copies, built from the library's own headers (the same
// offset functions and copy arithmetic the kernels use) and run on the CPU.
//
//  1. Copy arithmetic (lds_copy.h) for every tile size the kernels copy: each
//     lane reads inside the tile, writes inside the KiB-rounded LDS buffer,
//     every byte of the tile is copied to the same offset, and a lane whose
//     read is clamped to the tile's last 16 bytes writes past the tile (it
//     never overwrites tile data).  For the fused kernel's four-part tiles
//     (head key rows, shared pair-factor key rows, head value rows, shared
//     pair-factor value rows): every chunk is read inside its part, every
//     LDS byte of the buffer is written exactly from its part, and the
//     operand reads of the key and value products stay inside their parts.
//  2. Address join: a 64-bit address rebuilt from its two 32-bit halves is
//     the address itself, also when bit 31 of the low half is set.  Joining
//     an int low half instead sign-extends it and fills the high word with
//     ones, i.e. a wild address.
//  3. Workspace layout (common.h make_layout) for the benchmark
//     configurations and ragged or odd shapes: the regions are disjoint and
//     in order, inside the total size, and the last record of every region
//     that the lift writes or the fused kernel reads (key and value tiles,
//     query rows and points, centroids, mask words, partial results, pair
//     mask words) ends inside its region; the tile sizes the fused kernel
//     compiles in equal the layout's; the epilogue's workspace holds the
//     packed output projection; key ranges hold at least one tile each;
//     the workgroup remap of the fused kernel is a permutation.
// Prints "layout bounds: N checks ok" and exits 0, or names the first
// failure and exits 1.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../rna_structure_amd/csrc/common.h"
#include "../rna_structure_amd/csrc/lds_copy.h"

using namespace fipa;

static long g_checks = 0;
#define CHECK(cond, ...)                                           \
  do {                                                             \
    ++g_checks;                                                    \
    if (!(cond)) {                                                 \
      std::printf("FAIL %s:%d: %s -- ", __FILE__, __LINE__, #cond); \
      std::printf(__VA_ARGS__);                                    \
      std::printf("\n");                                           \
      std::exit(1);                                                \
    }                                                              \
  } while (0)

// ---------------------------------------------------------------- 1. copies
static void check_copy(int bytes, int W, int per_wave, const char* what) {
  CHECK(bytes % 16 == 0 && bytes >= 16, "%s: %d bytes", what, bytes);
  const int lds = dma_lds_bytes(bytes);
  std::vector<int> hit(bytes, 0);
  for (int w = 0; w < W; ++w)
    for (int k = 0; k < per_wave; ++k) {
      const int ch = dma_chunk(bytes, W, w, k);
      CHECK(ch >= 0 && ch * 1024 < bytes, "%s: chunk %d of %d bytes", what, ch, bytes);
      for (int lane = 0; lane < 64; ++lane) {
        const uint32_t src = dma_src_off(bytes, ch, lane), dst = dma_dst_off(ch, lane);
        CHECK(src + 16 <= (uint32_t)bytes, "%s: read %u of %d", what, src, bytes);
        CHECK(dst + 16 <= (uint32_t)lds, "%s: write %u of %d", what, dst, lds);
        if (src == dst) {
          for (int e = 0; e < 16; ++e) hit[src + e] = 1;
        } else {
          CHECK(dst >= (uint32_t)bytes, "%s: clamped lane writes tile byte %u", what, dst);
        }
      }
    }
  for (int x = 0; x < bytes; ++x) CHECK(hit[x], "%s: byte %d of %d never copied", what, x, bytes);
}

template <int BYTES, int W>
static void check_copy_inst(const char* what) {
  check_copy(BYTES, W, dma_per_wave<BYTES, W>(), what);
}

// The part sizes of flash_mfma_kernel<NQS, NVB, GS, W> (TileDims there).
template <int NQS, int NVB, int GS>
struct FusedParts {
  static constexpr int KH = 64 * (16 + 16 * GS + kRowPad) * 2;
  static constexpr int KZ = 64 * (16 * (NQS - 1) + kRowPad) * 2;
  static constexpr int VH = 64 * kVCols * 2;
  static constexpr int VZ = (32 * (NVB - 1) * kVCols * 2 + 1023) / 1024 * 1024;
};

static void check_parts(const int* bytes, int W, int per_wave, const char* what) {
  int C = 0, start[5];
  for (int p = 0; p < 4; ++p) {
    CHECK(bytes[p] % 1024 == 0 && bytes[p] > 0, "%s: part %d of %d bytes", what, p, bytes[p]);
    start[p] = C;
    C += bytes[p] / 1024;
  }
  start[4] = C;
  CHECK(per_wave == (C + W - 1) / W, "%s: %d copies per wave", what, per_wave);
  std::vector<int> hit(C * 1024, 0);
  for (int w = 0; w < W; ++w)
    for (int k = 0; k < per_wave; ++k) {
      const int c = w + W * k < C ? w + W * k : C - 1;  // as in dma_parts
      const int p = dma_part_of_chunk(c, start[1], start[2] - start[1], start[3] - start[2]);
      CHECK(c >= start[p] && c < start[p + 1], "%s: chunk %d in part %d", what, c, p);
      for (int lane = 0; lane < 64; ++lane) {
        const uint32_t src = (uint32_t)(c - start[p]) * 1024u + 16u * lane, dst = (uint32_t)c * 1024u + 16u * lane;
        CHECK(src + 16 <= (uint32_t)bytes[p], "%s: read %u of part %d (%d bytes)", what, src, p, bytes[p]);
        CHECK(dst + 16 <= (uint32_t)C * 1024u, "%s: write %u", what, dst);
        CHECK(dst - (uint32_t)start[p] * 1024u == src, "%s: part %d lands at its place", what, p);
        for (int e = 0; e < 16; ++e) hit[dst + e] = 1;
      }
    }
  for (int x = 0; x < C * 1024; ++x) CHECK(hit[x], "%s: LDS byte %d never written", what, x);
}

template <int NQS, int NVB, int GS, int W>
static void check_fused_inst() {
  using T = FusedParts<NQS, NVB, GS>;
  const int parts[4] = {T::KH, T::KZ, T::VH, T::VZ};
  constexpr int TB = T::KH + T::KZ + T::VH + T::VZ;
  check_parts(parts, W, dma_per_wave<TB, W>(), "fused tile");
  CHECK(2 * TB <= 160 * 1024, "fused tile buffers %d bytes", 2 * TB);
  // key operand reads (s_tile_ops): lane (l32, half), key block kb; head
  // part at row pitch 16 + 16 GS + pad, pair part at 16 (NQS - 1) + pad
  constexpr int KROW = 16 + 16 * GS + kRowPad, KZROW = 16 * (NQS - 1) + kRowPad;
  for (int st = 0; st < NQS + GS; ++st)
    for (int kb = 0; kb < 2; ++kb)
      for (int l32 : {0, 31})
        for (int half = 0; half < 2; ++half) {
          const int row = 32 * kb + l32;
          if (st >= 1 && st < NQS) {
            const int off = row * KZROW * 2 + half * 16 + (st - 1) * 32;
            CHECK(off >= 0 && off + 16 <= T::KZ, "pair key read %d of %d", off, T::KZ);
            CHECK((st - 1) * 16 + half * 8 + 8 <= 16 * (NQS - 1), "pair key column past the pair part");
          } else {
            const int col = st == 0 ? half * 8 : 16 + (st - NQS) * 16 + half * 8;
            const int off = row * KROW * 2 + col * 2;
            CHECK(off + 16 <= T::KH && col + 8 <= 16 + 16 * GS, "head key read %d of %d", off, T::KH);
          }
        }
  // value operand reads (pv_tile_ops): block vb, K-step ks, lane (l32, half)
  for (int vb = 0; vb <= NVB; ++vb)
    for (int ks = 0; ks < 4; ++ks)
      for (int l32 : {0, 31})
        for (int half = 0; half < 2; ++half) {
          const int off = (l32 * kVCols) * 2 + half * 16 + vb * 32 * kVCols * 2 + ks * 32;
          CHECK(off + 16 <= T::VH + T::VZ, "value read %d of %d", off, T::VH + T::VZ);
          CHECK((ks * 32 + half * 16) / 2 + 8 <= 64, "value read past the 64 key columns");
        }
}

template <int NQS>
static void check_bias_inst() {
  // the tile sizes of bias_attn_kernel<NQS, NVB> (4 wavefronts)
  constexpr int KP = 16 * NQS + 8;
  check_copy_inst<64 * KP * 2, 4>("bias key tile");
  check_copy_inst<32 * 1 * 72 * 2, 4>("bias value tile");
  check_copy_inst<32 * 2 * 72 * 2, 4>("bias value tile");
  check_copy_inst<32 * 4 * 72 * 2, 4>("bias value tile");
  check_copy_inst<32 * 8 * 72 * 2, 4>("bias value tile");
}

static void check_copies() {
  check_fused_inst<3, 2, 3, 4>(); check_fused_inst<3, 2, 3, 8>(); check_fused_inst<3, 2, 4, 4>();
  check_fused_inst<3, 2, 4, 8>(); check_fused_inst<5, 3, 3, 4>(); check_fused_inst<5, 3, 3, 8>();
  check_fused_inst<5, 3, 4, 4>(); check_fused_inst<5, 3, 4, 8>(); check_fused_inst<9, 5, 3, 4>();
  check_fused_inst<9, 5, 3, 8>(); check_fused_inst<9, 5, 4, 4>(); check_fused_inst<9, 5, 4, 8>();
  check_fused_inst<13, 7, 3, 4>(); check_fused_inst<13, 7, 4, 4>();
  // the stacked point layout (comparison): two bf16 geometric K-steps
  check_fused_inst<9, 5, 2, 4>(); check_fused_inst<9, 5, 2, 8>();
  // epilogue: W_h of Cout rows at the head-feature pitch, 4 wavefronts
  check_copy_inst<32 * kHeadFeatPitch * 2, 4>("epilogue w_out head");
  check_copy_inst<64 * kHeadFeatPitch * 2, 4>("epilogue w_out head");
  check_copy_inst<96 * kHeadFeatPitch * 2, 4>("epilogue w_out head");
  check_copy_inst<128 * kHeadFeatPitch * 2, 4>("epilogue w_out head");
  check_bias_inst<2>(); check_bias_inst<3>(); check_bias_inst<4>(); check_bias_inst<5>();
  check_bias_inst<8>(); check_bias_inst<9>(); check_bias_inst<16>();
  // every size a copy can have, on 4 and 8 wavefronts
  for (int bytes = 16; bytes <= 40 * 1024; bytes += 16) {
    check_copy(bytes, 4, ((bytes + 1023) / 1024 + 3) / 4, "any size, W=4");
    check_copy(bytes, 8, ((bytes + 1023) / 1024 + 7) / 8, "any size, W=8");
  }
}

// ---------------------------------------------------------------- 2. join
static void check_join() {
  const uint64_t addrs[] = {0x00007f0000000000ull, 0x00007f1234567890ull, 0x00007f12ffffff00ull,
                            0x00007f1280000000ull, 0x00007f12fffffff0ull, 0x0000000100000000ull,
                            0x000000017fffffffull, 0x0000000180000000ull};
  for (uint64_t a : addrs) {
    const uint32_t lo = (uint32_t)a, hi = (uint32_t)(a >> 32);
    CHECK(join_addr(hi, lo) == a, "join of %llx", (unsigned long long)a);
    // the pitfall: a signed low half
    const int slo = (int)lo;
    const uint64_t wrong = ((uint64_t)hi << 32) | (uint64_t)(int64_t)slo;
    if (lo & 0x80000000u)
      CHECK((wrong >> 32) == 0xffffffffull, "sign extension of %llx", (unsigned long long)a);
    else
      CHECK(wrong == a, "no sign extension for %llx", (unsigned long long)a);
  }
}

// ---------------------------------------------------------------- 3. layout
struct Region {
  const char* name;
  size_t start, end;  // [start, end), end = start of the next region
};

static void check_layout(const ipa_shape& s, int with_pm, int stacked = 0) {
  Layout L;
  if (!make_layout(&s, with_pm, &L, stacked)) return;  // unsupported shape: nothing to check
  char tag[160];
  std::snprintf(tag, sizeof tag, "B%lld N%lld H%lld D%lld Dv%lld P%lld Q%lld Cz%lld R%lld Cout%lld %s pm%d%s",
                (long long)s.B, (long long)s.N, (long long)s.H, (long long)s.D, (long long)s.Dv, (long long)s.P,
                (long long)s.Q, (long long)s.Cz, (long long)s.R, (long long)s.Cout,
                s.dtype == IPA_BF16 ? "bf16" : "f32", with_pm, stacked ? " stacked" : "");
  if (stacked) CHECK(L.GS == 2 && L.NQS == 9 && L.NVB == 5 && L.KROW == 56, "%s: stacked instance", tag);
  const int B = L.B, H = L.H, NT = L.NT;
  const size_t e = lifted_elem(L);
  CHECK(L.NKpad == NT * 64 && L.NKpad <= L.NQpad, "%s: padded rows", tag);
  // region order and sizes
  const Region reg[] = {
      {"QL", L.off_ql, L.off_qz},   {"QZ", L.off_qz, L.off_wp},       {"WP", L.off_wp, L.off_qa},
      {"QA", L.off_qa, L.off_kt},   {"KT", L.off_kt, L.off_vt},
      {"VT", L.off_vt, L.off_ktz},  {"KTZ", L.off_ktz, L.off_vtz},    {"VTZ", L.off_vtz, L.off_ck},
      {"CK", L.off_ck, L.off_gam},  {"GAM", L.off_gam, L.off_km},     {"KM", L.off_km, L.off_part},
      {"PART", L.off_part, L.off_pm}, {"PM", L.off_pm, L.total}};
  enum { rQL, rQZ, rWP, rQA, rKT, rVT, rKTZ, rVTZ, rCK, rGAM, rKM, rPART, rPM };
  CHECK(L.off_ql >= sizeof(Header), "%s: header", tag);
  for (const Region& r : reg) CHECK(r.start <= r.end && r.start % 256 == 0, "%s: region %s", tag, r.name);
  auto inside = [&](const Region& r, size_t off, size_t bytes, const char* what) {
    CHECK(off >= r.start && off + bytes <= r.end, "%s: %s [%zu, %zu) outside %s [%zu, %zu)", tag, what, off,
          off + bytes, r.name, r.start, r.end);
  };
  // per-region sizes the layout reserves, against the records
  CHECK(L.off_qz - L.off_ql >= (size_t)B * H * L.NQpad * L.QW * e, "%s: QL size", tag);
  if (L.mfma) {
    // the query operand: 16 scalar columns per head row, the pair columns
    // (NQS - 1 K-steps of 16) in the shared rows and the weights
    CHECK(L.QW == 16 && L.ZW == 16 * (L.NQS - 1) && L.ZW >= L.RCz && L.ZW % 8 == 0, "%s: query widths", tag);
    for (int b : {0, B - 1})
      for (int i : {0, L.N - 1, L.NKpad - 1, L.NQpad - 1})
        inside(reg[rQZ], qz_row_off(L, b, i), (size_t)L.ZW * 2, "query pair row");
    for (int h : {0, H - 1}) inside(reg[rWP], wp_row_off(L, h), (size_t)L.ZW * 2, "pair weights");
  } else {
    CHECK(L.off_wp == L.off_qz && L.off_qa == L.off_wp, "%s: no shared query rows on the fp32 path", tag);
  }
  const size_t ktb = kt_tile_bytes(L), vtb = vt_tile_bytes(L);
  for (int b : {0, B - 1})
    for (int h : {0, H - 1}) {
      for (int t : {0, NT - 1}) {
        inside(reg[rKT], kt_tile_off(L, b, h, t), ktb, "key tile");
        inside(reg[rVT], vt_tile_off(L, b, h, t), vtb, "value tile");
        if (L.mfma) {
          inside(reg[rKTZ], ktz_tile_off(L, b, t), ktz_tile_bytes(L), "pair key tile");
          inside(reg[rVTZ], vtz_tile_off(L, b, t), vtz_tile_bytes(L), "pair value tile");
        }
      }
      // the lift writes query rows of every key-tile residue (< NKpad), the
      // fused kernel reads rows < N
      for (int i : {0, L.N - 1, L.NKpad - 1, L.NQpad - 1}) {
        inside(reg[rQL], ql_row_off(L, b, h, i), (size_t)L.QW * e, "query row");
        inside(reg[rQA], qa_row_off(L, b, h, i), 64, "query points");
      }
    }
  for (int b : {0, B - 1})
    for (int t : {0, NT - 1}) {
      inside(reg[rCK], ck_off(L, b, t), 16, "centroid");
      for (int hf = 0; hf < 2; ++hf) inside(reg[rKM], km_word_off(L, b, t, hf), 4, "key-mask word");
      if (with_pm)
        for (int i : {0, L.NQpad - 1})
          for (int hf = 0; hf < 2; ++hf) inside(reg[rPM], pm_word_off(L, b, i, t, hf), 4, "pair-mask word");
    }
  inside(reg[rGAM], L.off_gam, (size_t)H * 4, "point weights");
  if (L.mfma) {
    // the part sizes of the fused kernel instance picked for this layout
    const size_t KH = 64 * (size_t)(16 + 16 * L.GS + kRowPad) * 2, KZ = 64 * (size_t)(16 * (L.NQS - 1) + kRowPad) * 2;
    const size_t VH = 64 * (size_t)kVCols * 2, VZ = (32 * (size_t)(L.NVB - 1) * kVCols * 2 + 1023) / 1024 * 1024;
    CHECK(ktb == KH && vtb == VH && ktz_tile_bytes(L) == KZ && vtz_tile_bytes(L) == VZ, "%s: tile part bytes", tag);
    // the columns and rows the lift fills fit the parts
    CHECK(L.D <= 16 && L.RCz <= 16 * (L.NQS - 1) && L.RCz <= L.VZROWS && L.Dv + 1 <= 32 && 3 * L.Q + 4 <= 32,
          "%s: widths vs instance", tag);
    // packed w_out of the epilogue (per head or transposed), in the
    // epilogue's own workspace
    const size_t wt = (size_t)L.H * L.Cout * kHeadFeatPitch * 2, wt2 = (size_t)L.Cout * L.FP * 2;
    CHECK(L.epi_ws >= (wt > wt2 ? wt : wt2), "%s: epilogue workspace %zu", tag, L.epi_ws);
    // key ranges of the fused kernel: [NT s / KS, NT (s + 1) / KS), each nonempty
    CHECK(L.KS >= 1 && L.KS <= 4, "%s: KS %d", tag, L.KS);
    for (int sp = 0; sp < L.KS; ++sp) {
      const int tb = (int)(((long)NT * sp) / L.KS), te = (int)(((long)NT * (sp + 1)) / L.KS);
      CHECK(te > tb, "%s: empty key range %d", tag, sp);
    }
    if (L.KS > 1)
      for (int i : {0, L.NQpad - 1})
        inside(reg[rPART], part_rec_off(L, L.KS - 1, B - 1, H - 1, i), (size_t)L.PREC * 4, "partial record");
    CHECK(L.PREC >= L.DO + 4 && L.PREC % 4 == 0, "%s: PREC", tag);
    // workgroup remap of the fused kernel (8 or 4 wavefronts per workgroup)
    for (int W : {4, 8}) {
      const int qtiles = (L.N + 32 * W - 1) / (32 * W);
      const long nwg = (long)qtiles * H * B * L.KS;
      if (nwg > (1 << 22) || nwg % 8) continue;
      std::vector<char> seen(nwg, 0);
      for (long wg = 0; wg < nwg; ++wg) {
        const long logical = (wg & 7) * (nwg >> 3) + (wg >> 3);
        CHECK(logical >= 0 && logical < nwg && !seen[logical], "%s: remap %ld", tag, wg);
        seen[logical] = 1;
      }
    }
  }
  CHECK(L.total == (with_pm ? align256(L.off_pm + (size_t)B * L.NQpad * NT * 8) : L.off_pm), "%s: total", tag);
}

static ipa_shape shape(long B, long N, long H, long D, long Dv, long P, long Q, long Cz, long R, long Cout, int dt) {
  ipa_shape s;
  s.B = B; s.N = N; s.H = H; s.D = D; s.Dv = Dv; s.P = P; s.Q = Q; s.Cz = Cz; s.R = R; s.Cout = Cout;
  s.dtype = dt;
  s.eps = 1e-8f;
  return s;
}

static void check_layouts() {
  std::vector<ipa_shape> v;
  // the benchmark configurations
  v.push_back(shape(1, 16, 4, 16, 16, 4, 8, 16, 2, 128, IPA_F32));
  v.push_back(shape(8, 256, 8, 16, 16, 4, 8, 64, 2, 128, IPA_BF16));
  v.push_back(shape(1, 2048, 8, 16, 16, 4, 8, 64, 2, 128, IPA_BF16));
  v.push_back(shape(39, 512, 12, 16, 16, 4, 8, 64, 2, 128, IPA_BF16));
  for (long n : {4096L, 8192L, 16384L, 32768L}) v.push_back(shape(1, n, 8, 16, 16, 4, 8, 64, 2, 128, IPA_BF16));
  // ragged lengths, ranks 1..3, every point count, small and odd widths, both paths
  for (long n : {1L, 2L, 63L, 64L, 65L, 127L, 128L, 129L, 200L, 255L, 256L, 257L, 600L, 1000L, 1024L, 1100L, 5000L})
    for (int dt : {IPA_F32, IPA_BF16}) {
      v.push_back(shape(1, n, 8, 16, 16, 4, 8, 64, 2, 128, dt));
      v.push_back(shape(3, n, 3, 16, 16, 4, 8, 64, 3, 128, dt));
      v.push_back(shape(2, n, 2, 8, 8, 5, 9, 48, 1, 64, dt));
      v.push_back(shape(2, n, 3, 4, 3, 2, 2, 5, 2, 6, dt));
      for (long P = 1; P <= 5; ++P) v.push_back(shape(1, n, 2, 8, 16, P, 4, 40, 2, 64, dt));
      v.push_back(shape(2, n, 12, 16, 16, 4, 8, 64, 2, 96, dt));
    }
  for (const ipa_shape& s : v)
    for (int pm : {0, 1})
      for (int stk : {0, 1}) check_layout(s, pm, stk);
}

int main() {
  check_copies();
  check_join();
  check_layouts();
  std::printf("layout bounds: %ld checks ok\n", g_checks);
  return 0;
}
