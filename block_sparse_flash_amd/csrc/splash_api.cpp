// splash_fwd_tile / splash_attn_fwd: argument validation, kernel selection
// and launch.  See include/splash.h for the contract of each call.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>

#include "bwd_params.h"
#include "errors.h"
#include "fwd_params.h"
#include "splash.h"

namespace {

bool dims_supported(int32_t dtype, int32_t d_qk, int32_t d_v) {
  if (dtype == SPLASH_F32) return (d_qk == 64 || d_qk == 128) && (d_v == 64 || d_v == 128);
  if (dtype == SPLASH_BF16)
    return (d_qk == 64 || d_qk == 128 || d_qk == 192) && (d_v == 64 || d_v == 128);
  return false;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Work-group placement: a "unit" is a run of query heads that share one K/V
// head (the whole group, or the largest part of it that still gives a unit
// count divisible by the XCD count); each unit's items stay on one XCD so
// that its K/V is read into that XCD's L2 once.  Without such a split the
// items keep their plain order.
void choose_xcd_units(const splash_fwd_args& a, splash::FwdParams* p) {
  p->xcd_units = 0;
  p->unit_heads = 1;
  const char* env = std::getenv("SPLASH_XCD_MAP");
  if (env && env[0] == '0') return;
  const int group = a.Hq / a.Hkv;
  const int64_t q_heads = static_cast<int64_t>(a.B) * a.Hq;
  for (int d = group; d >= 1; --d) {
    if (group % d != 0) continue;
    const int64_t units = q_heads / d;
    if (units % splash::kNumXcd == 0) {
      p->xcd_units = static_cast<int32_t>(units);
      p->unit_heads = d;
      return;
    }
  }
}

}  // namespace

extern "C" int splash_fwd_tile(int32_t dtype, int32_t d_qk, int32_t d_v, int32_t* block_q,
                               int32_t* block_kv) {
  splash::clear_error();
  if (!block_q || !block_kv) return splash::fail(SPLASH_EINVAL, "splash_fwd_tile: NULL output");
  if (dtype != SPLASH_F32 && dtype != SPLASH_BF16)
    return splash::fail(SPLASH_EDTYPE, "splash_fwd_tile: unknown dtype %d", dtype);
  if (!dims_supported(dtype, d_qk, d_v))
    return splash::fail(SPLASH_EUNSUPPORTED, "splash_fwd_tile: head dims (%d, %d) not built for dtype %d",
                        d_qk, d_v, dtype);
  if (dtype == SPLASH_F32) {
    *block_q = splash::kF32BlockQ;
    *block_kv = splash::kF32BlockKV;
  } else {
    const splash::Tile t = splash::bf16_default_tile(d_qk, d_v);
    *block_q = t.bq;
    *block_kv = t.bkv;
  }
  return SPLASH_OK;
}

extern "C" int splash_fwd_tiles(int32_t dtype, int32_t d_qk, int32_t d_v, int32_t* block_q,
                                int32_t* block_kv, int32_t capacity, int32_t* count) {
  splash::clear_error();
  if (!count || capacity < 0 || (capacity > 0 && (!block_q || !block_kv)))
    return splash::fail(SPLASH_EINVAL, "splash_fwd_tiles: NULL output or negative capacity");
  int32_t def_q = 0, def_kv = 0;
  const int rc = splash_fwd_tile(dtype, d_qk, d_v, &def_q, &def_kv);
  if (rc != SPLASH_OK) return rc;
  int32_t n = 0;
  auto put = [&](int32_t q, int32_t kv) {
    if (n < capacity) {
      block_q[n] = q;
      block_kv[n] = kv;
    }
    ++n;
  };
  put(def_q, def_kv);
  if (dtype == SPLASH_BF16) {
    for (const splash::Tile& t : splash::kSweepTiles)
      if (!(t.bq == def_q && t.bkv == def_kv) && splash::bf16_tile_built(d_qk, d_v, t.bq, t.bkv, false))
        put(t.bq, t.bkv);
    const splash::Tile t = splash::kDecodeTile;
    if (!(t.bq == def_q && t.bkv == def_kv) && splash::bf16_tile_built(d_qk, d_v, t.bq, t.bkv, false))
      put(t.bq, t.bkv);
  }
  *count = n;
  return SPLASH_OK;
}

extern "C" int splash_bwd_tile(int32_t dtype, int32_t d_qk, int32_t d_v, int32_t* block_q,
                               int32_t* block_kv) {
  splash::clear_error();
  if (!block_q || !block_kv) return splash::fail(SPLASH_EINVAL, "splash_bwd_tile: NULL output");
  if (dtype != SPLASH_F32 && dtype != SPLASH_BF16)
    return splash::fail(SPLASH_EDTYPE, "splash_bwd_tile: unknown dtype %d", dtype);
  if (dtype != SPLASH_BF16 || !splash::bwd_dims_built(d_qk, d_v))
    return splash::fail(SPLASH_EUNSUPPORTED, "splash_bwd_tile: no backward for dtype %d, head dims (%d, %d)",
                        dtype, d_qk, d_v);
  *block_q = splash::kBwdBlockQ;
  *block_kv = splash::kBwdBlockKV;
  return SPLASH_OK;
}

namespace {

// Validates *args (errors prefixed with `fn`) and fills *p for the launch.
// Returns SPLASH_OK, an error code, or -1 for a problem with nothing to
// compute (B, Hq or L equal to 0).
int prepare(const splash_fwd_args* args, const char* fn, bool split, splash::FwdParams* out) {
  if (!args) return splash::fail(SPLASH_EINVAL, "%s: NULL args", fn);
  const splash_fwd_args& a = *args;
  if (a.dtype != SPLASH_F32 && a.dtype != SPLASH_BF16)
    return splash::fail(SPLASH_EDTYPE, "%s: unknown dtype %d", fn, a.dtype);
  if (a.B < 0 || a.Hq < 0 || a.L < 0 || a.Hkv <= 0)
    return splash::fail(SPLASH_EINVAL, "%s: bad sizes B=%d Hq=%d Hkv=%d L=%d", fn, a.B, a.Hq,
                        a.Hkv, a.L);
  if (a.Hq % a.Hkv != 0)
    return splash::fail(SPLASH_ESHAPE, "%s: Hq=%d is not a multiple of Hkv=%d", fn, a.Hq, a.Hkv);
  if (!dims_supported(a.dtype, a.d_qk, a.d_v))
    return splash::fail(SPLASH_EUNSUPPORTED, "%s: head dims (%d, %d) not built for dtype %d", fn,
                        a.d_qk, a.d_v, a.dtype);
  if (a.causal != 0 && a.causal != 1)
    return splash::fail(SPLASH_EINVAL, "%s: causal must be 0 or 1", fn);
  if (a.window_left < -1 || a.window_right < -1)
    return splash::fail(SPLASH_EINVAL, "%s: window must be -1 or >= 0", fn);
  if (a.mask_mode != SPLASH_MASK_COMPUTED && a.mask_mode != SPLASH_MASK_STORED)
    return splash::fail(SPLASH_EINVAL, "%s: unknown mask_mode %d", fn, a.mask_mode);
  if (!std::isfinite(a.scale) || !(a.scale > 0.0f))
    return splash::fail(SPLASH_EINVAL, "%s: scale must be finite and > 0", fn);
  if (std::isnan(a.soft_cap) || std::isinf(a.soft_cap))
    return splash::fail(SPLASH_EINVAL, "%s: soft_cap must be finite", fn);
  if (a.use_max_logit != 0 && a.use_max_logit != 1)
    return splash::fail(SPLASH_EINVAL, "%s: use_max_logit must be 0 or 1", fn);
  if (a.use_max_logit && !std::isfinite(a.max_logit))
    return splash::fail(SPLASH_EINVAL, "%s: max_logit must be finite", fn);
  if (!a.seg_q && a.seg_kv) return splash::fail(SPLASH_EINVAL, "%s: seg_kv given without seg_q", fn);
  if (a.L_kv < 0 || a.q_offset < 0)
    return splash::fail(SPLASH_EINVAL, "%s: negative L_kv=%d or q_offset=%d", fn, a.L_kv, a.q_offset);
  const int32_t Lkv = a.L_kv == 0 ? a.L : a.L_kv;
  const bool decode = Lkv != a.L || a.q_offset != 0;
  if (decode && a.dtype != SPLASH_BF16)
    return splash::fail(SPLASH_EUNSUPPORTED, "%s: L_kv != L or q_offset != 0 needs bf16", fn);
  if (a.seg_q && !a.seg_kv && Lkv != a.L)
    return splash::fail(SPLASH_EINVAL, "%s: seg_kv is NULL but L_kv (%d) != L (%d)", fn, Lkv, a.L);

  int32_t bq = 0, bkv = 0;
  splash_fwd_tile(a.dtype, a.d_qk, a.d_v, &bq, &bkv);
  const bool default_tile = a.block_q == bq && a.block_kv == bkv;
  if (!default_tile) {
    if (a.dtype != SPLASH_BF16 || !splash::bf16_tile_built(a.d_qk, a.d_v, a.block_q, a.block_kv, split))
      return splash::fail(SPLASH_ESHAPE, "%s: no kernel for tables of %dx%d blocks (default tile %dx%d)", fn,
                          a.block_q, a.block_kv, bq, bkv);
    bq = a.block_q;
    bkv = a.block_kv;
  }
  const int64_t nq = (static_cast<int64_t>(a.L) + bq - 1) / bq;
  if (a.n_q_blocks != nq)
    return splash::fail(SPLASH_ESHAPE, "%s: n_q_blocks=%d but L=%d needs %lld", fn, a.n_q_blocks,
                        a.L, static_cast<long long>(nq));
  if (a.n_active < 0 || a.n_patterns < 0)
    return splash::fail(SPLASH_EINVAL, "%s: negative table size", fn);

  const int64_t n_heads = static_cast<int64_t>(a.B) * a.Hq;
  if (n_heads == 0 || a.L == 0) return -1;  // nothing to compute
  const int64_t n_wg = n_heads * nq;
  const int64_t max_d = a.d_qk > a.d_v ? a.d_qk : a.d_v;
  // Byte offsets inside one head's q, k or v (buffer ranges) and key
  // positions q_offset + row (+ window) stay within int32.
  const int64_t max_len = a.L > Lkv ? a.L : Lkv;
  if (n_wg > INT32_MAX || n_heads * max_len > (int64_t{1} << 46) / max_d ||
      (max_len + 2 * bq) * max_d * 2 > INT32_MAX ||
      static_cast<int64_t>(a.q_offset) + a.L + Lkv + 2 * bq > INT32_MAX)
    return splash::fail(SPLASH_ESHAPE, "%s: problem too large", fn);

  if (!a.q || !a.k || !a.v || !a.o) return splash::fail(SPLASH_EINVAL, "%s: NULL q/k/v/o", fn);
  if (!aligned16(a.q) || !aligned16(a.k) || !aligned16(a.v) || !aligned16(a.o))
    return splash::fail(SPLASH_EINVAL, "%s: q/k/v/o must be 16-byte aligned", fn);
  if (!a.row_ptr || !a.row_order)
    return splash::fail(SPLASH_EINVAL, "%s: NULL row_ptr or row_order", fn);
  if (a.n_active > 0 && (!a.active_cols || !a.block_code || !a.mask_next))
    return splash::fail(SPLASH_EINVAL, "%s: NULL active_cols, block_code or mask_next", fn);
  if (a.mask_mode == SPLASH_MASK_STORED && a.n_active > 0 && a.n_patterns > 0 &&
      !a.partial_mask_blocks)
    return splash::fail(SPLASH_EINVAL, "%s: stored mask mode needs partial_mask_blocks", fn);

  splash::FwdParams p{};
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.B = a.B;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.L = a.L;
  p.Lkv = Lkv;
  p.q_off = a.q_offset;
  p.group = a.Hq / a.Hkv;
  p.causal = a.causal;
  // Windows wider than the key range restrict nothing; clamping them keeps
  // position + window within int32 in the kernels.
  p.window_left = a.window_left > Lkv ? Lkv : a.window_left;
  p.window_right = a.window_right > Lkv ? Lkv : a.window_right;
  p.seg_q = a.seg_q;
  p.seg_kv = a.seg_kv;
  p.mask_stored = a.mask_mode == SPLASH_MASK_STORED ? 1 : 0;
  p.block_q = bq;
  p.block_kv = bkv;
  p.n_q_blocks = static_cast<int32_t>(nq);
  p.row_ptr = a.row_ptr;
  p.row_order = a.row_order;
  p.active_cols = a.active_cols;
  p.block_code = a.block_code;
  p.mask_next = a.mask_next;
  p.patterns = a.partial_mask_blocks;
  p.scale = a.scale;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.soft_cap = a.soft_cap > 0.0f ? a.soft_cap : 0.0f;
  p.mle = a.use_max_logit;
  p.mle_log2 = a.use_max_logit ? a.max_logit * 1.4426950408889634f : 0.0f;
  p.n_split = 1;
  p.ws_o = nullptr;
  p.ws_lse = nullptr;
  p.row_period = 0;
  p.Lseg = a.L;
  splash_fwd_args placed = a;
  const bool decode_tile = bq == splash::kDecodeTile.bq && bkv == splash::kDecodeTile.bkv;
  if (a.dtype == SPLASH_BF16 && p.group > 1 && a.L < bq && (default_tile || decode_tile)) {
    // All query rows fit one table row: pack the query heads of each K/V
    // group into one row space ([B, Hq, L, d] is [B, Hkv, group L, d]), so
    // that an item's row tile holds group * L rows instead of L.
    p.row_period = a.L;
    p.L = p.group * a.L;
    p.Hq = a.Hkv;
    p.group = 1;
    p.n_q_blocks = static_cast<int32_t>((static_cast<int64_t>(p.L) + bq - 1) / bq);
    placed.Hq = a.Hkv;
  }
  choose_xcd_units(placed, &p);
  *out = p;
  return SPLASH_OK;
}

int64_t split_workspace_bytes(int64_t n_split, int64_t B, int64_t Hq, int64_t L, int64_t d_v) {
  return n_split * B * Hq * L * (d_v + 1) * static_cast<int64_t>(sizeof(float));
}

}  // namespace

extern "C" int splash_attn_fwd(const splash_fwd_args* args, void* stream) {
  splash::clear_error();
  splash::FwdParams p{};
  const int rc = prepare(args, "splash_attn_fwd", false, &p);
  if (rc == -1) return SPLASH_OK;
  if (rc != SPLASH_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = args->dtype == SPLASH_F32 ? splash::launch_fwd_f32(p, args->d_qk, args->d_v, s)
                                                 : splash::launch_fwd_bf16(p, args->d_qk, args->d_v, s);
  if (e != hipSuccess)
    return splash::fail(SPLASH_EHIP, "splash_attn_fwd: launch failed: %s", hipGetErrorString(e));
  return SPLASH_OK;
}

extern "C" int splash_split_workspace_bytes(int32_t n_split, int32_t B, int32_t Hq, int32_t L,
                                            int32_t d_v, int64_t* bytes) {
  splash::clear_error();
  if (!bytes) return splash::fail(SPLASH_EINVAL, "splash_split_workspace_bytes: NULL output");
  if (n_split < 1 || n_split > SPLASH_MAX_SPLIT || B < 0 || Hq < 0 || L < 0 || d_v <= 0)
    return splash::fail(SPLASH_EINVAL,
                        "splash_split_workspace_bytes: bad sizes n_split=%d B=%d Hq=%d L=%d d_v=%d",
                        n_split, B, Hq, L, d_v);
  *bytes = split_workspace_bytes(n_split, B, Hq, L, d_v);
  return SPLASH_OK;
}

extern "C" int splash_attn_fwd_split(const splash_fwd_args* args, int32_t n_split, void* workspace,
                                     int64_t workspace_bytes, void* stream) {
  splash::clear_error();
  splash::FwdParams p{};
  const int rc = prepare(args, "splash_attn_fwd_split", true, &p);
  if (rc != SPLASH_OK && rc != -1) return rc;
  if (args->dtype != SPLASH_BF16)
    return splash::fail(SPLASH_EUNSUPPORTED, "splash_attn_fwd_split: bf16 only");
  if (n_split < 1 || n_split > SPLASH_MAX_SPLIT)
    return splash::fail(SPLASH_EINVAL, "splash_attn_fwd_split: n_split=%d not in [1, %d]", n_split,
                        SPLASH_MAX_SPLIT);
  if (rc == -1) return SPLASH_OK;
  const int64_t need = split_workspace_bytes(n_split, args->B, args->Hq, args->L, args->d_v);
  if (!workspace || workspace_bytes < need)
    return splash::fail(SPLASH_EINVAL, "splash_attn_fwd_split: workspace of %lld bytes needed, %lld given",
                        static_cast<long long>(need), static_cast<long long>(workspace_bytes));
  if (!aligned16(workspace))
    return splash::fail(SPLASH_EINVAL, "splash_attn_fwd_split: workspace must be 16-byte aligned");
  if (static_cast<int64_t>(p.B) * p.Hq * p.n_q_blocks * n_split > INT32_MAX)
    return splash::fail(SPLASH_ESHAPE, "splash_attn_fwd_split: problem too large");
  const int64_t rows = static_cast<int64_t>(p.B) * p.Hq * p.L;
  p.n_split = n_split;
  p.ws_o = static_cast<float*>(workspace);
  p.ws_lse = p.ws_o + n_split * rows * args->d_v;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = splash::launch_fwd_bf16(p, args->d_qk, args->d_v, s);
  if (e == hipSuccess) e = splash::launch_split_merge_bf16(p, args->d_v, s);
  if (e != hipSuccess)
    return splash::fail(SPLASH_EHIP, "splash_attn_fwd_split: launch failed: %s", hipGetErrorString(e));
  return SPLASH_OK;
}
