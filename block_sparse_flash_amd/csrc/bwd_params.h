// Launch parameters of the backward kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace splash {

// Head dims (d_qk, d_v) the bf16 backward is built for.
constexpr bool bwd_dims_built(int d_qk, int d_v) {
  return (d_qk == 64 && d_v == 64) || (d_qk == 128 && d_v == 128) || (d_qk == 192 && d_v == 128);
}

struct BwdParams {
  const void* q;        // bf16 [B, Hq, L, d_qk]
  const void* k;        // bf16 [B, Hkv, Lkv, d_qk]
  const void* v;        // bf16 [B, Hkv, Lkv, d_v]
  const void* o;        // bf16 [B, Hq, L, d_v]
  const float* lse;     // [B, Hq, L]
  const void* dout;     // bf16 [B, Hq, L, d_v]
  float* dq;            // [B, Hq, L, d_qk]
  float* dk;            // [B, Hkv, Lkv, d_qk]
  float* dv;            // [B, Hkv, Lkv, d_v]
  float* delta;         // [B, Hq, L]
  int32_t B, Hq, Hkv, group, L, Lkv, q_off;
  int32_t causal, window_left, window_right;  // windows clamped to Lkv
  const int32_t* seg_q;   // [B, L] or null
  const int32_t* seg_kv;  // [B, Lkv] or null (then seg_q, Lkv = L)
  int32_t n_q_blocks, n_kv_blocks;
  const int32_t* row_ptr;
  const int32_t* row_order;  // rows longest first, or null (natural order)
  const int32_t* active_cols;
  const int32_t* col_ptr;
  const int32_t* col_rows;
  const int32_t* col_order;  // columns most active blocks first, or null (natural order)
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  float soft_cap;    // > 0 when the cap is on
};

// Launches delta, then dk/dv, then dq on stream s (returns the first
// launch error).
hipError_t launch_bwd_bf16(const BwdParams& p, int d_qk, int d_v, hipStream_t s);

}  // namespace splash
