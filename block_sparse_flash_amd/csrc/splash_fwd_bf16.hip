// bf16 forward: the 128/128 instances (every variant at the default tile and
// the decode tile, the plain forward at the other tiles of the block-size
// sweep) and the launcher for all head dims.  The kernel is in splash_fwd_bf16_kernel.h.

#include <atomic>

#include "splash_fwd_bf16_kernel.h"

namespace splash {
namespace {

// Compute units of the current device (cached per device; concurrent first
// calls store the same value).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, int d_qk, int d_v, hipStream_t s) {
  const int n_cu = device_cus();
  const Tile def = bf16_default_tile(d_qk, d_v);
  if (p.block_q == def.bq && p.block_kv == def.bkv) {
    if (d_qk == 128 && d_v == 128) return launch_default<128, 128>(p, n_cu, s);
    if (d_qk == 192) return launch_fwd_bf16_d192(p, d_v, n_cu, s);
    return launch_fwd_bf16_d64(p, d_qk, d_v, n_cu, s);
  }
  if (d_qk != 128 || d_v != 128) return hipErrorInvalidValue;
  if (p.block_q == kDecodeTile.bq && p.block_kv == kDecodeTile.bkv)
    return launch_all<128, 128, kDecodeTile.bkv, kDecodeTile.bq / 32>(p, n_cu, s);
  if (p.ws_o || p.row_period > 0) return hipErrorInvalidValue;
  if (p.block_q == 256 && p.block_kv == 64 && !(def.bq == 256 && def.bkv == 64)) return launch_sweep<256, 64>(p, n_cu, s);
  if (p.block_q == 256 && p.block_kv == 128 && !(def.bq == 256 && def.bkv == 128)) return launch_sweep<256, 128>(p, n_cu, s);
  if (p.block_q == 128 && p.block_kv == 64) return launch_sweep<128, 64>(p, n_cu, s);
  if (p.block_q == 128 && p.block_kv == 128) return launch_sweep<128, 128>(p, n_cu, s);
  return hipErrorInvalidValue;
}

}  // namespace splash
