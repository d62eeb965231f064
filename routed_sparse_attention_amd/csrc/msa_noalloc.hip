// msa_route_topk_noalloc: routing and top-k with the library's own fixed
// device scratch instead of a caller workspace, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The scratch is one file-scope device array. Every GPU the library runs on
// holds its own copy until the process ends. In host code the array's name is
// only a host-side stand-in, so its device address is looked up once per
// device with hipGetSymbolAddress (with that device current) and kept; every
// launch receives that address, never the name.
//
// The kernels are those of msa_route_topk. Everything they read from the
// workspace they first write in the same call (chunk scores, per-part maxima,
// per-block document maxima), so nothing needs clearing between calls.
#include <mutex>

#include "msa_internal.h"

namespace msa {

constexpr size_t kScratchBytes = (size_t)MSA_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch`, looked up on the first
// call on each device. The stream must belong to the current device.
int scratch_for(hipStream_t s, void** out) {
  int dev = 0;
  MSA_HIP(hipGetDevice(&dev));
  if (s != nullptr) {
    hipDevice_t sdev = 0;
    MSA_HIP(hipStreamGetDevice(s, &sdev));
    if ((int)sdev != dev)
      return fail(MSA_ERR_INVALID_ARG,
                  "route_topk_noalloc: the stream belongs to device %d, device %d is current",
                  (int)sdev, dev);
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MSA_ERR_UNSUPPORTED, "route_topk_noalloc: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                      "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

}  // namespace
}  // namespace msa

using namespace msa;

extern "C" int32_t msa_route_topk_noalloc(const msa_dims* d, const msa_bf16* QR, int32_t B,
                                          int32_t M, const msa_bf16* KRbar,
                                          const int64_t* dco, int32_t n_docs, int64_t n_chunks,
                                          float* doc_scores, int32_t accumulate,
                                          int32_t* topk_ids, float* topk_scores, int32_t* n_sel,
                                          void* stream) {
  clear_error();
  int rc = check_dims(d);
  if (rc) return rc;
  rc = check_route_args(d, QR, B, M, KRbar, dco, n_docs, n_chunks, doc_scores, accumulate,
                        topk_ids, topk_scores, n_sel);
  if (rc) return rc;
  const size_t need = route_topk_ws(B, M, n_chunks, n_docs, d->top_k);
  if (need > kScratchBytes)
    return fail(MSA_ERR_WORKSPACE,
                "route_topk_noalloc: this call needs %zu bytes of scratch, the fixed scratch "
                "holds %zu (use msa_route_topk with a workspace)",
                need, kScratchBytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  rc = scratch_for(s, &ws);
  if (rc) return rc;
  return route_topk_impl(d, QR, B, M, KRbar, dco, n_docs, n_chunks, doc_scores, accumulate,
                         topk_ids, topk_scores, n_sel, ws, kScratchBytes, s);
}
