// gdla_decode_noalloc: gdla_decode for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  The step's workspace is a library-owned device array
// instead of a caller buffer; everything else -- the kernels, the checks, the
// results -- is gdla_decode's.
//
// The array lives in this translation unit only, so the loader sets it aside
// (GDLA_DECODE_NOALLOC_SCRATCH_BYTES per device) only in processes that use
// this entry point.  Host code never passes the array's name to a kernel: in
// host code that name is a host-side stand-in.  The device address is looked
// up once per device with hipGetSymbolAddress, with that device current, and
// kept in a per-device table.
//
// Every decode step writes each workspace byte it later reads (the chunk plan,
// the projections, the per-chunk partials), so nothing has to be cleared
// between calls.  Calls on one device share the array: two calls whose work
// overlaps in time on one GPU (two streams, or two host threads on one
// stream without ordering) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gdla.h"
#include "decode.h"

namespace {

__device__ __align__(256) unsigned char scratch[GDLA_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};   // device address of `scratch` per device, once looked up

// The scratch array's device address on the current device (nullptr and the
// HIP error on failure).
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" gdla_status gdla_decode_noalloc(const gdla_config* cfg, const gdla_weights* w, int32_t B,
                                           const void* x, void* y, void* cache, const int32_t* cache_lens,
                                           int32_t capacity, void* stream) {
  constexpr size_t CAP = (size_t)GDLA_DECODE_NOALLOC_SCRATCH_BYTES;
  // Sizes first: a request beyond the array launches nothing.  Everything
  // else (config, pointers, B < 0, B = 0) is checked by gdla_decode itself;
  // for those calls no scratch is needed, so none is looked up.
  const size_t need = (cfg && B > 0) ? gdla_decode_workspace_size(cfg, B) : 0;
  if (need == 0) return gdla_decode(cfg, w, B, x, y, cache, cache_lens, capacity, nullptr, 0, stream);
  if (need > CAP)
    return gdla::report_error(GDLA_ERR_WORKSPACE,
                              "gdla_decode_noalloc: this shape and batch need %zu bytes of workspace, the "
                              "library's scratch holds %zu (call gdla_decode with a caller workspace)",
                              need, CAP);
  if (stream) {
    int sdev = -1, cur = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess || hipGetDevice(&cur) != hipSuccess)
      return gdla::report_error(GDLA_ERR_INVALID_ARG, "gdla_decode_noalloc: cannot query the stream's device");
    if (sdev != cur)
      return gdla::report_error(GDLA_ERR_INVALID_ARG,
                                "gdla_decode_noalloc: the stream belongs to device %d, the current device is %d",
                                sdev, cur);
  }
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess)
    return gdla::report_error(GDLA_ERR_HIP, "gdla_decode_noalloc: scratch address: %s", hipGetErrorString(e));
  return gdla_decode(cfg, w, B, x, y, cache, cache_lens, capacity, ws, CAP, stream);
}
