// C ABI of the FlashIPA library: argument validation, workspace layout and
// kernel launches.  No allocation, no synchronisation: every kernel is
// enqueued on the caller's stream.  Each call is bracketed by a roctx range
// named after it (rocprofv3 --marker-trace shows them); with the environment
// variable FLASHIPA_DEBUG set to a non-zero value every call also waits for
// its kernels and reports a failing one on stderr.
#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <cstdio>
#include <cstdlib>

#include "common.h"

namespace fipa {
hipError_t launch_lift(const Layout& L, const ipa_lift_in* in, void* ws, hipStream_t st);
hipError_t launch_flash_f32(const Layout& L, const void* ws, float* o, float* lse, hipStream_t st);
hipError_t launch_flash_mfma(const Layout& L, const void* ws, float* o, float* lse, hipStream_t st);
hipError_t launch_epilogue(const Layout& L, void* ws, const float* o, const float* lse, const ipa_epi_in* in, float eps,
                           float* update, float* local, hipStream_t st);
bool epilogue_supported(const Layout& L);
hipError_t launch_logit_rows(const Layout& L, const void* ws, int b, int h, int row0, int nrows, float* out,
                             hipStream_t st);
hipError_t launch_knn(const ipa_knn_shape* s, const float* t, const uint8_t* mask, int32_t* idx, float* dist,
                      void* dgram, hipStream_t st);
size_t bw_workspace_bytes(const ipa_shape* s);
size_t bias_workspace_bytes(const ipa_bias_shape* s);
hipError_t launch_bias_attention(const ipa_bias_shape* s, const void* q, const void* k, const void* v,
                                 const void* phi_q, const void* phi_k, const uint8_t* key_mask, float* o, float* lse,
                                 void* ws, hipStream_t st);
hipError_t launch_backward(const ipa_shape* s, const ipa_lift_in* in, const ipa_epi_in* ep, const float* dupd,
                           const float* dloc, void* ws, ipa_grads* gr, hipStream_t st);
}  // namespace fipa

using fipa::Layout;

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static ipa_status shape_status(const ipa_shape* s, int with_pm, Layout* L, int stacked = 0) {
  if (!s) return IPA_ERR_NULL;
  if (s->B <= 0 || s->N <= 0 || s->H <= 0 || s->D <= 0 || s->Dv <= 0 || s->P <= 0 || s->Q <= 0 || s->Cz <= 0 ||
      s->R <= 0 || s->Cout <= 0 || !(s->eps > 0.0f))
    return IPA_ERR_SHAPE;
  if (s->dtype != IPA_F32 && s->dtype != IPA_BF16) return IPA_ERR_UNSUPPORTED;
  if (!fipa::make_layout(s, with_pm, L, stacked)) return IPA_ERR_UNSUPPORTED;
  return IPA_OK;
}

// roctx range over one ABI call
struct Range {
  explicit Range(const char* name) { roctxRangePushA(name); }
  ~Range() { roctxRangePop(); }
};

static bool debug_mode() {
  static const bool on = [] {
    const char* v = std::getenv("FLASHIPA_DEBUG");
    return v != nullptr && v[0] != '\0' && v[0] != '0';
  }();
  return on;
}

// Status of a call whose kernels were enqueued with launch error e.  In debug
// mode the call also waits for its kernels on `stream`, so that an error of a
// kernel (not only of its launch) is reported here, with the call's name.
static ipa_status launch_status(hipError_t e, const char* what, void* stream) {
  if (e == hipSuccess && debug_mode()) {
    e = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = hipGetLastError();
  }
  if (e != hipSuccess && debug_mode()) std::fprintf(stderr, "flashipa: %s: %s\n", what, hipGetErrorString(e));
  return e == hipSuccess ? IPA_OK : IPA_ERR_LAUNCH;
}

extern "C" {

size_t ipa_lifted_bytes(const ipa_shape* s, int with_pair_mask) {
  Layout L;
  if (shape_status(s, with_pair_mask, &L) != IPA_OK) return 0;
  return L.total;
}

int64_t ipa_o_width(const ipa_shape* s) {
  if (!s) return 0;
  return s->Dv + s->R * s->Cz + 3 * s->Q;
}

}  // extern "C"

// ipa_lift and ipa_lift_stacked (which differ only in the point columns of
// the key rows), ipa_flash_fwd and ipa_flash_fwd_stacked
static ipa_status lift_call(const ipa_shape* s, const ipa_lift_in* in, void* lifted, size_t lifted_bytes,
                            void* stream, int stacked, const char* name) {
  if (!s || !in || !lifted) return IPA_ERR_NULL;
  Layout L;
  const int with_pm = in->pair_mask != nullptr;
  ipa_status st = shape_status(s, with_pm, &L, stacked);
  if (st != IPA_OK) return st;
  const void* req[] = {in->q, in->k, in->v, in->q_points, in->k_points, in->v_points, in->rotation,
                       in->translation, in->point_weight_raw, in->w_pair, in->zl, in->zr, in->mask};
  for (const void* p : req)
    if (!p) return IPA_ERR_NULL;
  for (const void* p : req)
    if (!aligned16(p)) return IPA_ERR_ALIGN;
  if (!aligned16(lifted) || (in->pair_mask && !aligned16(in->pair_mask))) return IPA_ERR_ALIGN;
  if (lifted_bytes < L.total) return IPA_ERR_SHAPE;
  const Range range(name);
  return launch_status(fipa::launch_lift(L, in, lifted, reinterpret_cast<hipStream_t>(stream)), name, stream);
}

static ipa_status flash_call(const ipa_shape* s, const void* lifted, float* o, float* lse, void* stream, int stacked,
                             const char* name) {
  if (!s || !lifted || !o || !lse) return IPA_ERR_NULL;
  Layout L;
  // the pair-mask region is at the end of the workspace; its presence is
  // recorded in the workspace header by the lift
  ipa_status st = shape_status(s, 0, &L, stacked);
  if (st != IPA_OK) return st;
  if (!aligned16(lifted) || !aligned16(o) || !aligned16(lse)) return IPA_ERR_ALIGN;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const Range range(name);
  return launch_status(L.mfma ? fipa::launch_flash_mfma(L, lifted, o, lse, hs)
                              : fipa::launch_flash_f32(L, lifted, o, lse, hs), name, stream);
}

extern "C" {

ipa_status ipa_lift(const ipa_shape* s, const ipa_lift_in* in, void* lifted, size_t lifted_bytes, void* stream) {
  return lift_call(s, in, lifted, lifted_bytes, stream, 0, "ipa_lift");
}

ipa_status ipa_flash_fwd(const ipa_shape* s, const void* lifted, float* o, float* lse, void* stream) {
  return flash_call(s, lifted, o, lse, stream, 0, "ipa_flash_fwd");
}

size_t ipa_lifted_bytes_stacked(const ipa_shape* s, int with_pair_mask) {
  Layout L;
  if (shape_status(s, with_pair_mask, &L, 1) != IPA_OK) return 0;
  return L.total;
}

ipa_status ipa_lift_stacked(const ipa_shape* s, const ipa_lift_in* in, void* lifted, size_t lifted_bytes,
                            void* stream) {
  return lift_call(s, in, lifted, lifted_bytes, stream, 1, "ipa_lift_stacked");
}

ipa_status ipa_flash_fwd_stacked(const ipa_shape* s, const void* lifted, float* o, float* lse, void* stream) {
  return flash_call(s, lifted, o, lse, stream, 1, "ipa_flash_fwd_stacked");
}

size_t ipa_epilogue_workspace_bytes(const ipa_shape* s) {
  Layout L;
  if (shape_status(s, 0, &L) != IPA_OK || !fipa::epilogue_supported(L)) return 0;
  return L.epi_ws > 0 ? L.epi_ws : 16;
}

ipa_status ipa_epilogue(const ipa_shape* s, void* workspace, size_t workspace_bytes, const float* o, const float* lse,
                        const ipa_epi_in* in, float* update, float* local_points, void* stream) {
  if (!s || !o || !lse || !in || !update || !local_points) return IPA_ERR_NULL;
  Layout L;
  ipa_status st = shape_status(s, 0, &L);
  if (st != IPA_OK) return st;
  const void* req[] = {in->zl, in->rotation, in->translation, in->w_out, in->b_out};
  for (const void* p : req)
    if (!p) return IPA_ERR_NULL;
  if (L.epi_ws > 0 && !workspace) return IPA_ERR_NULL;
  for (const void* p : req)
    if (!aligned16(p)) return IPA_ERR_ALIGN;
  if ((workspace && !aligned16(workspace)) || !aligned16(o) || !aligned16(lse) || !aligned16(update) ||
      !aligned16(local_points))
    return IPA_ERR_ALIGN;
  if (!fipa::epilogue_supported(L)) return IPA_ERR_UNSUPPORTED;
  if (workspace_bytes < L.epi_ws) return IPA_ERR_SHAPE;
  const Range range("ipa_epilogue");
  return launch_status(fipa::launch_epilogue(L, workspace, o, lse, in, s->eps, update, local_points,
                                             reinterpret_cast<hipStream_t>(stream)), "ipa_epilogue", stream);
}

ipa_status ipa_logit_rows(const ipa_shape* s, const void* lifted, int64_t b, int64_t h, int64_t row0, int64_t nrows,
                          float* out, void* stream) {
  if (!s || !lifted || !out) return IPA_ERR_NULL;
  Layout L;
  ipa_status st = shape_status(s, 0, &L);
  if (st != IPA_OK) return st;
  if (b < 0 || b >= s->B || h < 0 || h >= s->H || row0 < 0 || nrows <= 0 || row0 + nrows > s->N || nrows > 65535)
    return IPA_ERR_SHAPE;
  if (!aligned16(lifted) || !aligned16(out)) return IPA_ERR_ALIGN;
  const Range range("ipa_logit_rows");
  return launch_status(fipa::launch_logit_rows(L, lifted, (int)b, (int)h, (int)row0, (int)nrows, out,
                                               reinterpret_cast<hipStream_t>(stream)), "ipa_logit_rows", stream);
}

static ipa_status bw_shape_status(const ipa_shape* s) {
  if (!s) return IPA_ERR_NULL;
  if (s->B <= 0 || s->N <= 0 || s->H <= 0 || s->D <= 0 || s->Dv <= 0 || s->P <= 0 || s->Q <= 0 || s->Cz <= 0 ||
      s->R <= 0 || s->Cout <= 0 || !(s->eps > 0.0f))
    return IPA_ERR_SHAPE;
  if (s->dtype != IPA_F32 && s->dtype != IPA_BF16) return IPA_ERR_UNSUPPORTED;
  // grid limits: samples on the z dimension (<= 65535), heads on y
  if (s->N > (1 << 26) || s->B > 65535 || s->B * s->N > (1 << 28) || s->H > 1024 || s->Cout > (1 << 16))
    return IPA_ERR_UNSUPPORTED;
  return fipa::bw_workspace_bytes(s) ? IPA_OK : IPA_ERR_UNSUPPORTED;
}

size_t ipa_backward_workspace_bytes(const ipa_shape* s) {
  if (bw_shape_status(s) != IPA_OK) return 0;
  return fipa::bw_workspace_bytes(s);
}

ipa_status ipa_backward(const ipa_shape* s, const ipa_lift_in* in, const ipa_epi_in* epi, const float* d_update,
                        const float* d_local, void* workspace, size_t workspace_bytes, ipa_grads* g, void* stream) {
  if (!s || !in || !epi || !d_update || !d_local || !workspace || !g) return IPA_ERR_NULL;
  const ipa_status st = bw_shape_status(s);
  if (st != IPA_OK) return st;
  const size_t need = fipa::bw_workspace_bytes(s);
  const void* req[] = {in->q, in->k, in->v, in->q_points, in->k_points, in->v_points, in->rotation,
                       in->translation, in->point_weight_raw, in->w_pair, in->zl, in->zr, in->mask,
                       epi->w_out, epi->b_out, g->q, g->k, g->v, g->q_points, g->k_points, g->v_points,
                       g->rotation, g->translation, g->point_weight_raw, g->w_pair, g->zl, g->zr, g->w_out,
                       g->b_out};
  for (const void* p : req)
    if (!p) return IPA_ERR_NULL;
  for (const void* p : req)
    if (!aligned16(p)) return IPA_ERR_ALIGN;
  if (!aligned16(d_update) || !aligned16(d_local) || !aligned16(workspace) ||
      (in->pair_mask && !aligned16(in->pair_mask)))
    return IPA_ERR_ALIGN;
  if (workspace_bytes < need) return IPA_ERR_SHAPE;
  const Range range("ipa_backward");
  return launch_status(
      fipa::launch_backward(s, in, epi, d_update, d_local, workspace, g, (hipStream_t)stream), "ipa_backward", stream);
}

ipa_status ipa_knn_distogram(const ipa_knn_shape* s, const float* translation, const uint8_t* mask,
                             int32_t* nn_index, float* nn_dist, void* dgram, void* stream) {
  if (!s || !translation || !nn_index) return IPA_ERR_NULL;
  if (s->B <= 0 || s->N <= 0 || s->k < 1 || s->k > 64 || s->nbins < 1 || s->nbins > 4096 ||
      !(s->dmax > 0.0f) || !(s->dmax <= 3.4028235e38f))
    return IPA_ERR_SHAPE;
  // query groups of 8 per wavefront must fit the 32-bit wavefront count
  if (s->N > (int64_t)1 << 30 || s->B * ((s->N + 7) / 8) > ((int64_t)1 << 31) - 4) return IPA_ERR_SHAPE;
  if (s->dgram_dtype != IPA_F32 && s->dgram_dtype != IPA_BF16) return IPA_ERR_UNSUPPORTED;
  if (!aligned16(translation) || !aligned16(nn_index) || (mask && !aligned16(mask)) ||
      (nn_dist && !aligned16(nn_dist)) || (dgram && !aligned16(dgram)))
    return IPA_ERR_ALIGN;
  const Range range("ipa_knn_distogram");
  return launch_status(fipa::launch_knn(s, translation, mask, nn_index, nn_dist, dgram, (hipStream_t)stream), "ipa_knn_distogram", stream);
}

static ipa_status bias_shape_status(const ipa_bias_shape* s) {
  if (!s) return IPA_ERR_NULL;
  if (s->B <= 0 || s->N <= 0 || s->M <= 0 || s->H <= 0 || s->D <= 0 || s->Dv <= 0 || s->R < 0 ||
      !(s->scale > -3.4028235e38f && s->scale < 3.4028235e38f))
    return IPA_ERR_SHAPE;
  if (s->causal && s->N != s->M) return IPA_ERR_SHAPE;
  // grid: query tiles of 128 on x, heads on y, samples on z
  if (s->N > (1 << 30) || s->M > (1 << 30) || s->H > 65535 || s->B > 65535) return IPA_ERR_SHAPE;
  // lift grids: one thread per 8 lifted columns (at most 32 per row) of every padded row
  const int64_t rows = (s->N > s->M ? s->N : s->M) + 127;
  if (s->B * s->H * rows > ((int64_t)1 << 26)) return IPA_ERR_SHAPE;
  if (s->dtype != IPA_F32 && s->dtype != IPA_BF16) return IPA_ERR_UNSUPPORTED;
  if (s->phi_dtype != IPA_F32 && s->phi_dtype != IPA_BF16) return IPA_ERR_UNSUPPORTED;
  if (s->Dv > 256 || s->D + 3 * s->R > 256) return IPA_ERR_UNSUPPORTED;
  return IPA_OK;
}

size_t ipa_bias_workspace_bytes(const ipa_bias_shape* s) {
  if (bias_shape_status(s) != IPA_OK) return 0;
  return fipa::bias_workspace_bytes(s);
}

ipa_status ipa_bias_attention(const ipa_bias_shape* s, const void* q, const void* k, const void* v,
                              const void* phi_q, const void* phi_k, const uint8_t* key_mask, float* o, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream) {
  const ipa_status st = bias_shape_status(s);
  if (st != IPA_OK) return st;
  if (!q || !k || !v || !o || !lse || !workspace || (s->R > 0 && (!phi_q || !phi_k))) return IPA_ERR_NULL;
  const size_t need = fipa::bias_workspace_bytes(s);
  if (need == 0) return IPA_ERR_UNSUPPORTED;
  if (workspace_bytes < need) return IPA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) || !aligned16(workspace) ||
      (phi_q && !aligned16(phi_q)) || (phi_k && !aligned16(phi_k)) || (key_mask && !aligned16(key_mask)))
    return IPA_ERR_ALIGN;
  const Range range("ipa_bias_attention");
  return launch_status(fipa::launch_bias_attention(s, q, k, v, phi_q, phi_k, key_mask, o, lse, workspace,
                                                   (hipStream_t)stream), "ipa_bias_attention", stream);
}

const char* ipa_status_string(int status) {
  switch (status) {
    case IPA_OK: return "ok";
    case IPA_ERR_NULL: return "a required pointer is NULL";
    case IPA_ERR_SHAPE: return "invalid shape or workspace size";
    case IPA_ERR_UNSUPPORTED: return "dimensions or dtype not supported by the compiled kernels";
    case IPA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case IPA_ERR_LAUNCH: return "kernel launch failed";
    case IPA_ERR_DEVICE: return "HIP runtime error";
    case IPA_ERR_SCRATCH: return "the shape needs more than the static scratch of ipa_forward_noalloc";
    default: return "unknown status";
  }
}

const char* ipa_version(void) { return "flashipa-gfx950 0.1"; }

}  // extern "C"
