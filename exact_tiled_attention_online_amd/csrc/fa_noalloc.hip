// fa_noalloc.hip -- fa_fwd_splitkv_noalloc: the split-key-range forward with
// the per-range partial results (O and LSE of each key range) in a static
// device array of this library instead of a caller's workspace, for callers
// that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  The kernels are fa_fwd_splitkv's.
//
// `scratch` is a file-scope device array: each GPU the library runs on holds
// its own copy, at its own address, from module load to process end.  In host
// code its name is a host-side stand-in, never a device address: the address
// on a device is taken once per device with hipGetSymbolAddress (with that
// device current) and kept; kernels only ever receive that address.  Every
// call on a device shares the array and overwrites what it needs (the split
// kernel writes every range's O and LSE for every query row it is given, so
// nothing carries over from an earlier call); calls that overlap in time on one
// device race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fa.h"

namespace {

__device__ __align__(256) char scratch[FA_SPLITKV_NOALLOC_MAX_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // per device: the device address of `scratch`

// The device address of `scratch` on the device `stream` belongs to (the
// current device for the null stream); FA_ERR_HIP if the runtime fails.
int scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  if (stream) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return FA_ERR_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return FA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return FA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return FA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return FA_OK;
}

}  // namespace

extern "C" int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                      int H, int Nq, int Nk, int d, int causal, float scale, int num_splits,
                                      void* stream, int dtype, int layout) {
  // every argument check of fa_fwd_splitkv, with no HIP call: given no
  // workspace, a call that passes them all stops at the workspace check
  const int st = fa_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, num_splits, nullptr, 0, stream,
                                dtype, layout);
  if (st != FA_ERR_WORKSPACE) return st;
  const size_t need = fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits);
  if (need == 0) return FA_ERR_INVALID;
  if (need > (size_t)FA_SPLITKV_NOALLOC_MAX_BYTES) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  const int r = scratch_address(static_cast<hipStream_t>(stream), &ws);
  if (r != FA_OK) return r;
  return fa_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, num_splits, ws,
                        (size_t)FA_SPLITKV_NOALLOC_MAX_BYTES, stream, dtype, layout);
}
