// fa_decode_noalloc: fa_decode for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  Its split partials live in a fixed file-scope device array
// instead of a caller-provided workspace; the kernels are fa_decode's.
//
// Each GPU the library runs on holds its own copy of the array until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is a stand-in symbol, not a device address): the first call on a
// device looks up that device's address with hipGetSymbolAddress, with the
// device current, and every call passes that pointer as the workspace.
// Every call on a GPU shares the array, so calls that overlap on one GPU
// (other streams, other host threads) race; calls ordered on one stream do
// not.  No part of the array needs clearing: the split kernel writes every
// partial the merge reads (an empty chunk writes its logsumexp as -inf and
// the merge gives it weight 0).
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa.h"
#include "fa_launch.hpp"

// Float32 partial outputs and logsumexps of B * Hq * num_splits (head, split)
// pairs: (D + 1) * 4 bytes each.  32 MiB holds 65,027 such pairs at D = 128
// (the 128-sequence, 32-head, 8-split decode workload needs 32,768).
static constexpr size_t kScratchBytes = size_t(32) << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device.
fa_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fa::set_error(FA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fa::set_error(FA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fa::set_error(FA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s",
                           dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" fa_status fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                       const int* seqlens, void* o, float* lse, int B, int Hq,
                                       int Hkv, int Lk_max, int D, float scale, int num_splits,
                                       fa_dtype dtype, hipStream_t stream) {
  fa_status st = fa::check_decode_args(q, k_cache, v_cache, seqlens, o, lse, B, Hq, Hkv, Lk_max,
                                       D, scale, num_splits, dtype);
  if (st != FA_OK) return st;
  const size_t need = fa::decode_workspace_bytes(B, Hq, D, num_splits);
  if (need > kScratchBytes)
    return fa::set_error(FA_ERR_INVALID_ARGUMENT,
                         "fa_decode_noalloc: B*Hq*num_splits*(D+1)*4 = %zu bytes of partials "
                         "exceed its %zu-byte static scratch; use fa_decode with a workspace",
                         need, kScratchBytes);
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != FA_OK) return st;
  return fa_decode(q, k_cache, v_cache, seqlens, o, lse, B, Hq, Hkv, Lk_max, D, scale, num_splits,
                   ws, kScratchBytes, dtype, stream);
}
