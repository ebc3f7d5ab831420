// svt_noalloc.hip - svt_search_noalloc: svt_search with its workspace in a static device array, for
// callers that cannot allocate device memory.  The array is this file's `scratch`; its address on each
// GPU is looked up once (hipGetSymbolAddress, with that GPU current) and kept.  In host code the array's
// name is not a device address: only the looked-up pointer is passed to kernels.

#include <hip/hip_runtime.h>

#include <mutex>

#include "svt.h"
#include "svt_internal.h"

static __device__ __align__(256) unsigned char scratch[SVT_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch` on each GPU, once looked up

// the address of this GPU's array; the device must be current
int scratch_on(int device, void **out) {
  if (device < 0 || device >= kMaxDevices)
    return svt::report(SVT_EUNSUPPORTED, "svt_search_noalloc: device %d beyond %d", device, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return svt::report(SVT_EDEVICE, "svt_search_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return SVT_OK;
}

}  // namespace

extern "C" int svt_search_noalloc(const svt_index *ix, int32_t B, const int8_t *queries, const uint64_t *masks,
                                  const float *query_scales, int32_t nprobe, int32_t k, int64_t *out_ids,
                                  int32_t *out_scores, float *out_fscores, int32_t *out_counts, int64_t *out_stats,
                                  const svt_search_options *opts, void *hip_stream) {
  const char *who = "svt_search_noalloc";
  (void)svt::report(SVT_OK, "%s", "");
  size_t need = 0;
  int ix_device = -1;
  int rc = svt::search_size(ix, B, nprobe, k, opts, who, &need, &ix_device);
  if (rc != SVT_OK) return rc;
  if (B == 0) return SVT_OK;
  if (need > SVT_NOALLOC_SCRATCH_BYTES)
    return svt::report(SVT_EINVAL, "%s: this search needs %zu bytes of workspace, more than the %zu of the static "
                       "scratch (use svt_search with a workspace)", who, need, (size_t)SVT_NOALLOC_SCRATCH_BYTES);
  int device = -1;
  const hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return svt::report(SVT_EDEVICE, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
  if (device != ix_device)
    return svt::report(SVT_EINVAL, "%s: current device %d is not the index's device %d", who, device, ix_device);
  void *ws = nullptr;
  if ((rc = scratch_on(device, &ws)) != SVT_OK) return rc;
  return svt::search_into(ix, B, queries, masks, query_scales, nprobe, k, out_ids, out_scores, out_fscores,
                          out_counts, out_stats, opts, ws, SVT_NOALLOC_SCRATCH_BYTES, hip_stream, false, who);
}
