// splash_attn_fwd_split_noalloc: the split-KV forward with its partials in a
// static device array instead of a caller workspace, for callers that cannot
// allocate (code under HIP graph capture, serving loops).  See
// include/splash.h for the contract.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "errors.h"
#include "splash.h"

namespace {

// The partial outputs and lse values of the chunks (what the workspace of
// splash_attn_fwd_split holds).  Each device the library runs on holds its
// own copy until the process ends.  In host code this name stands for the
// symbol, not a device address: kernels get the address from
// hipGetSymbolAddress (scratch_ptr below).
__device__ __align__(256) uint8_t scratch[SPLASH_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<uintptr_t> g_scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device (concurrent first calls store the same value);
// 0 and an error message on failure.
uintptr_t scratch_ptr(const char* fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    splash::fail(SPLASH_EHIP, "%s: no usable current device (%s)", fn,
                 e != hipSuccess ? hipGetErrorString(e) : "device index out of range");
    return 0;
  }
  uintptr_t ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == 0) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      splash::fail(SPLASH_EHIP, "%s: hipGetSymbolAddress of the static scratch failed: %s", fn,
                   hipGetErrorString(e));
      return 0;
    }
    ptr = reinterpret_cast<uintptr_t>(p);
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

}  // namespace

extern "C" int splash_attn_fwd_split_noalloc(const splash_fwd_args* args, int32_t n_split, void* stream) {
  splash::clear_error();
  const char* fn = "splash_attn_fwd_split_noalloc";
  if (!args) return splash::fail(SPLASH_EINVAL, "%s: NULL args", fn);
  if (n_split < 1 || n_split > SPLASH_MAX_SPLIT)
    return splash::fail(SPLASH_EINVAL, "%s: n_split=%d not in [1, %d]", fn, n_split, SPLASH_MAX_SPLIT);
  if (args->B < 0 || args->Hq < 0 || args->L < 0 || args->d_v <= 0)
    return splash::fail(SPLASH_EINVAL, "%s: bad sizes B=%d Hq=%d L=%d d_v=%d", fn, args->B, args->Hq,
                        args->L, args->d_v);
  int64_t need = 0;
  const int rc = splash_split_workspace_bytes(n_split, args->B, args->Hq, args->L, args->d_v, &need);
  if (rc != SPLASH_OK) return rc;
  if (need > SPLASH_STATIC_SCRATCH_BYTES)
    return splash::fail(SPLASH_EINVAL,
                        "%s: the partials need %lld bytes, the static scratch holds %lld "
                        "(use splash_attn_fwd_split with a workspace)",
                        fn, static_cast<long long>(need), static_cast<long long>(SPLASH_STATIC_SCRATCH_BYTES));
  const uintptr_t ptr = scratch_ptr(fn);
  if (ptr == 0) return SPLASH_EHIP;
  return splash_attn_fwd_split(args, n_split, reinterpret_cast<void*>(ptr), SPLASH_STATIC_SCRATCH_BYTES,
                               stream);
}
