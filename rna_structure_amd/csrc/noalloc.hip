// The forward for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation):
// ipa_forward_noalloc runs ipa_lift, ipa_flash_fwd and ipa_epilogue in one
// call, with every buffer besides the inputs and the two outputs -- the lifted
// rows, the attention output and its log-sum-exp, the packed output
// projection -- in the static device array `scratch` below.
//
// `scratch` is a file-scope __device__ array: each GPU the library runs on
// holds its own copy, allocated when the code object is loaded there and
// kept until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is a stand-in, not a device address); the device
// address is looked up once per device with hipGetSymbolAddress and cached.
// Every call on a GPU shares that GPU's copy, so calls that overlap on one
// GPU (different streams or host threads) race.  No kernel needs the array
// cleared: each launch writes every byte it later reads.
#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <mutex>

#include "common.h"

namespace fipa {
hipError_t launch_lift(const Layout& L, const ipa_lift_in* in, void* ws, hipStream_t st);
hipError_t launch_flash_f32(const Layout& L, const void* ws, float* o, float* lse, hipStream_t st);
hipError_t launch_flash_mfma(const Layout& L, const void* ws, float* o, float* lse, hipStream_t st);
hipError_t launch_epilogue(const Layout& L, void* ws, const float* o, const float* lse, const ipa_epi_in* in, float eps,
                           float* update, float* local, hipStream_t st);
bool epilogue_supported(const Layout& L);
}  // namespace fipa

constexpr size_t kScratchBytes = (size_t)128 << 20;  // 128 MiB per device

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mutex;
char* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The device address of the current device's copy of `scratch`.
hipError_t scratch_address(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = static_cast<char*>(p);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

static ipa_status enqueue(const fipa::Layout& L, const ipa_lift_in* in, const ipa_epi_in* epi, float eps, char* base,
                          size_t off_o, size_t off_lse, size_t off_epi, float* update, float* local_points,
                          void* stream);

extern "C" ipa_status ipa_forward_noalloc(const ipa_shape* s, const ipa_lift_in* in, const ipa_epi_in* epi,
                                          float* update, float* local_points, void* stream) {
  if (!s || !in || !epi || !update || !local_points) return IPA_ERR_NULL;
  if (s->B <= 0 || s->N <= 0 || s->H <= 0 || s->D <= 0 || s->Dv <= 0 || s->P <= 0 || s->Q <= 0 || s->Cz <= 0 ||
      s->R <= 0 || s->Cout <= 0 || !(s->eps > 0.0f))
    return IPA_ERR_SHAPE;
  if (s->dtype != IPA_F32 && s->dtype != IPA_BF16) return IPA_ERR_UNSUPPORTED;
  fipa::Layout L;
  if (!fipa::make_layout(s, in->pair_mask != nullptr, &L) || !fipa::epilogue_supported(L)) return IPA_ERR_UNSUPPORTED;
  const void* req[] = {in->q, in->k, in->v, in->q_points, in->k_points, in->v_points, in->rotation,
                       in->translation, in->point_weight_raw, in->w_pair, in->zl, in->zr, in->mask,
                       epi->zl, epi->rotation, epi->translation, epi->w_out, epi->b_out};
  for (const void* p : req)
    if (!p) return IPA_ERR_NULL;
  for (const void* p : req)
    if (!aligned16(p)) return IPA_ERR_ALIGN;
  if ((in->pair_mask && !aligned16(in->pair_mask)) || !aligned16(update) || !aligned16(local_points))
    return IPA_ERR_ALIGN;
  // [lifted rows | o (B N H DO fp32) | lse (B H N fp32) | epilogue workspace]
  const size_t off_o = align256(L.total);
  const size_t off_lse = off_o + align256((size_t)L.B * L.N * L.H * L.DO * 4);
  const size_t off_epi = off_lse + align256((size_t)L.B * L.H * L.N * 4);
  const size_t need = off_epi + L.epi_ws;
  if (need > kScratchBytes) return IPA_ERR_SCRATCH;

  char* base = nullptr;
  if (scratch_address(&base) != hipSuccess) return IPA_ERR_DEVICE;
  roctxRangePushA("ipa_forward_noalloc");
  const ipa_status st = enqueue(L, in, epi, s->eps, base, off_o, off_lse, off_epi, update, local_points, stream);
  roctxRangePop();
  return st;
}

static ipa_status enqueue(const fipa::Layout& L, const ipa_lift_in* in, const ipa_epi_in* epi, float eps, char* base,
                          size_t off_o, size_t off_lse, size_t off_epi, float* update, float* local_points,
                          void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  float* o = reinterpret_cast<float*>(base + off_o);
  float* lse = reinterpret_cast<float*>(base + off_lse);
  if (fipa::launch_lift(L, in, base, st) != hipSuccess) return IPA_ERR_LAUNCH;
  const hipError_t e = L.mfma ? fipa::launch_flash_mfma(L, base, o, lse, st) : fipa::launch_flash_f32(L, base, o, lse, st);
  if (e != hipSuccess) return IPA_ERR_LAUNCH;
  if (fipa::launch_epilogue(L, base + off_epi, o, lse, epi, eps, update, local_points, st) != hipSuccess)
    return IPA_ERR_LAUNCH;
  return IPA_OK;
}
