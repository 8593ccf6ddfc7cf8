// splash_attn_bwd: argument validation and launch.  See include/splash.h for
// the contract.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "bwd_params.h"
#include "errors.h"
#include "fwd_params.h"
#include "splash.h"

namespace {

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

}  // namespace

extern "C" int splash_attn_bwd(const splash_bwd_args* args, void* stream) {
  splash::clear_error();
  const char* fn = "splash_attn_bwd";
  if (!args) return splash::fail(SPLASH_EINVAL, "%s: NULL args", fn);
  const splash_bwd_args& a = *args;
  if (a.dtype != SPLASH_F32 && a.dtype != SPLASH_BF16)
    return splash::fail(SPLASH_EDTYPE, "%s: unknown dtype %d", fn, a.dtype);
  if (a.dtype != SPLASH_BF16) return splash::fail(SPLASH_EUNSUPPORTED, "%s: bf16 only", fn);
  if (!splash::bwd_dims_built(a.d_qk, a.d_v))
    return splash::fail(SPLASH_EUNSUPPORTED, "%s: head dims (%d, %d) not built", fn, a.d_qk, a.d_v);
  if (a.B < 0 || a.Hq < 0 || a.L < 0 || a.Hkv <= 0 || a.L_kv < 0 || a.q_offset < 0)
    return splash::fail(SPLASH_EINVAL, "%s: bad sizes B=%d Hq=%d Hkv=%d L=%d L_kv=%d q_offset=%d", fn,
                        a.B, a.Hq, a.Hkv, a.L, a.L_kv, a.q_offset);
  if (a.Hq % a.Hkv != 0)
    return splash::fail(SPLASH_ESHAPE, "%s: Hq=%d is not a multiple of Hkv=%d", fn, a.Hq, a.Hkv);
  if (a.causal != 0 && a.causal != 1) return splash::fail(SPLASH_EINVAL, "%s: causal must be 0 or 1", fn);
  if (a.window_left < -1 || a.window_right < -1)
    return splash::fail(SPLASH_EINVAL, "%s: window must be -1 or >= 0", fn);
  if (!std::isfinite(a.scale) || !(a.scale > 0.0f))
    return splash::fail(SPLASH_EINVAL, "%s: scale must be finite and > 0", fn);
  if (!std::isfinite(a.soft_cap)) return splash::fail(SPLASH_EINVAL, "%s: soft_cap must be finite", fn);
  if (!a.seg_q && a.seg_kv) return splash::fail(SPLASH_EINVAL, "%s: seg_kv given without seg_q", fn);
  const int32_t Lkv = a.L_kv == 0 ? a.L : a.L_kv;
  if (a.seg_q && !a.seg_kv && Lkv != a.L)
    return splash::fail(SPLASH_EINVAL, "%s: seg_kv is NULL but L_kv (%d) != L (%d)", fn, Lkv, a.L);
  if (a.block_q != splash::kBwdBlockQ || a.block_kv != splash::kBwdBlockKV)
    return splash::fail(SPLASH_ESHAPE, "%s: tables built for blocks %dx%d, kernels use %dx%d", fn, a.block_q,
                        a.block_kv, splash::kBwdBlockQ, splash::kBwdBlockKV);
  const int64_t nq = (static_cast<int64_t>(a.L) + a.block_q - 1) / a.block_q;
  const int64_t nkv = (static_cast<int64_t>(Lkv) + a.block_kv - 1) / a.block_kv;
  if (a.n_q_blocks != nq || a.n_kv_blocks != nkv)
    return splash::fail(SPLASH_ESHAPE, "%s: block counts (%d, %d) but L=%d, L_kv=%d need (%lld, %lld)", fn,
                        a.n_q_blocks, a.n_kv_blocks, a.L, Lkv, static_cast<long long>(nq),
                        static_cast<long long>(nkv));
  if (a.n_active < 0) return splash::fail(SPLASH_EINVAL, "%s: negative n_active", fn);
  const int64_t max_len = a.L > Lkv ? a.L : Lkv;
  if (static_cast<int64_t>(a.B) * a.Hq * nq > INT32_MAX || static_cast<int64_t>(a.B) * a.Hkv * nkv > INT32_MAX ||
      (max_len + 2 * a.block_q) * a.d_qk * 2 > INT32_MAX ||
      static_cast<int64_t>(a.q_offset) + a.L + Lkv + 2 * a.block_q > INT32_MAX)
    return splash::fail(SPLASH_ESHAPE, "%s: problem too large", fn);

  const bool any_q = static_cast<int64_t>(a.B) * a.Hq * a.L > 0;
  const bool any_kv = static_cast<int64_t>(a.B) * Lkv > 0;
  if (!any_q && !any_kv) return SPLASH_OK;
  if (any_kv && (!a.dk || !a.dv || !a.k || !a.v || !a.col_ptr))
    return splash::fail(SPLASH_EINVAL, "%s: NULL k, v, dk, dv or col_ptr", fn);
  if (any_q && (!a.q || !a.o || !a.lse || !a.dout || !a.dq || !a.delta || !a.row_ptr))
    return splash::fail(SPLASH_EINVAL, "%s: NULL q, o, lse, dout, dq, delta or row_ptr", fn);
  if (a.n_active > 0 && (!a.active_cols || !a.col_rows))
    return splash::fail(SPLASH_EINVAL, "%s: NULL active_cols or col_rows", fn);
  for (const void* ptr : {a.q, a.k, a.v, a.o, a.dout, static_cast<const void*>(a.dq),
                          static_cast<const void*>(a.dk), static_cast<const void*>(a.dv)})
    if (!aligned16(ptr)) return splash::fail(SPLASH_EINVAL, "%s: q/k/v/o/dout/dq/dk/dv must be 16-byte aligned", fn);

  splash::BwdParams p{};
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.dout = a.dout;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.delta = a.delta;
  p.B = a.B;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.L = a.L;
  p.Lkv = Lkv;
  p.q_off = a.q_offset;
  p.causal = a.causal;
  // Windows wider than the key range restrict nothing; clamping keeps
  // position + window within int32.
  p.window_left = a.window_left > Lkv ? Lkv : a.window_left;
  p.window_right = a.window_right > Lkv ? Lkv : a.window_right;
  p.seg_q = a.seg_q;
  p.seg_kv = a.seg_kv;
  p.n_q_blocks = static_cast<int32_t>(nq);
  p.n_kv_blocks = static_cast<int32_t>(nkv);
  p.row_ptr = a.row_ptr;
  p.row_order = a.row_order;
  p.active_cols = a.active_cols;
  p.col_ptr = a.col_ptr;
  p.col_rows = a.col_rows;
  p.col_order = a.col_order;
  p.scale = a.scale;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.soft_cap = a.soft_cap > 0.0f ? a.soft_cap : 0.0f;
  const hipError_t e = splash::launch_bwd_bf16(p, a.d_qk, a.d_v, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return splash::fail(SPLASH_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return SPLASH_OK;
}
