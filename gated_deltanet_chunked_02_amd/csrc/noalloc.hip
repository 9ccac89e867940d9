// gdn_chunk_fwd_noalloc: gdn_chunk_fwd with the library's own device scratch as the
// workspace, for callers that cannot allocate (code under HIP graph capture, serving loops
// that must not call hipMalloc, harnesses that forbid it).
//
// The scratch is one file-scope device array per GPU the library runs on, held until the
// process ends.  Host code never uses the array's name as an address (on the host it is a
// stand-in symbol): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.  Nothing here allocates.
//
// Every call on one GPU shares that GPU's array: calls that overlap on one GPU (two
// streams, two host threads) race and give unspecified results.  The kernels fully write
// every part of the workspace they later read (chunk and segment tables, segment maps,
// the longest-first order), so the array needs no clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"

namespace {

static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up on the first call there.
gdn_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GDN_ERR_HIP;
  if (dev >= kMaxDevices) return GDN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDN_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return GDN_OK;
}

}  // namespace

extern "C" gdn_status gdn_chunk_fwd_noalloc(const gdn_desc* d, const void* q, const void* k,
                                            const void* v, const float* g, const void* beta,
                                            const float* h0, const int32_t* cu_seqlens,
                                            float scale, void* o, float* ht,
                                            hipStream_t stream) {
  if (!d) return GDN_ERR_INVALID_ARG;
  // a stage stop leaves its results in the workspace, here the library's own scratch
  if (d->stop_after != 0) return GDN_ERR_INVALID_ARG;
  void* ws = nullptr;
  const gdn_status s = scratch_ptr(&ws);
  if (s != GDN_OK) return s;
  gdn_desc dd = *d;
  dd.workspace = ws;
  dd.workspace_bytes = GDN_NOALLOC_SCRATCH_BYTES;
  // a variant needing more than the scratch holds is refused with GDN_ERR_WORKSPACE (AUTO
  // picks what fits, as it does for any workspace)
  return gdn_chunk_fwd(&dd, q, k, v, g, beta, h0, cu_seqlens, scale, o, ht, stream);
}
