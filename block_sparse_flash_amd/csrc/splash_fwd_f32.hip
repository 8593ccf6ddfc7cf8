// Float32 block-sparse attention forward for gfx950 (vector ALU, no MFMA).
//
// The float32 path exists for exactness (fp32 storage and arithmetic), not
// for speed.  One work-group = one wave = one 64-query block of one head; each
// lane owns one query row and keeps its q vector, running max m, running sum
// l and output accumulator o in registers ("Lecture 13 - Pallas Kernels and
// Splash Attention", section 5.2: m, l and o stay resident for the whole KV
// loop; the divide o / l happens once at the end).  The work-group walks the
// active kv blocks of its q-block row from the execution table (section 6.3:
// a grid over active blocks only; empty blocks are never loaded).  Each
// 64-key block is staged in LDS and consumed in sub-blocks of 16 keys
// (section 5.3 "bkv_compute" micro-tiling), each sub-block doing one online-
// softmax update (section 5.1):
//   m_new = max(m, max_j z_j); alpha = 2^(m - m_new); p_j = 2^(z_j - m_new);
//   l = alpha * l + sum_j p_j; o = alpha * o + sum_j p_j v_j
// with z = log2(e) * logit so that exp becomes the hardware exp2 (section 6.6
// "use_base2_exp").

#include <hip/hip_runtime.h>
#include <math.h>

#include "fwd_params.h"

namespace splash {
namespace {

constexpr int BQ = kF32BlockQ;
constexpr int BKV = kF32BlockKV;
constexpr int SUB = 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// log2(e) * cap * tanh(x / cap) with tanh(y) = 1 - 2 / (e^{2y} + 1).
__device__ __forceinline__ float capped_log2(float logit, float cap) {
  const float t = fast_exp2(logit * (2.0f * kLog2e / cap));
  return cap * kLog2e * (1.0f - 2.0f / (t + 1.0f));
}

template <int DQK, int DV>
__global__ __launch_bounds__(64) void splash_fwd_f32_kernel(FwdParams p) {
  __shared__ float ks[BKV][DQK];
  __shared__ float vs[BKV][DV];

  int head, rank;
  map_workgroup(p, blockIdx.x, &head, &rank);
  const int b = head / p.Hq;
  const int hq = head - b * p.Hq;
  const int hkv = hq / p.group;
  const int r = p.row_order[rank];
  const int lane = threadIdx.x;
  const int L = p.L;
  const int qi = r * BQ + lane;
  const bool row_valid = qi < L;

  const float* qg = static_cast<const float*>(p.q) + ((int64_t)head * L) * DQK;
  const float* kg = static_cast<const float*>(p.k) + ((int64_t)(b * p.Hkv + hkv) * L) * DQK;
  const float* vg = static_cast<const float*>(p.v) + ((int64_t)(b * p.Hkv + hkv) * L) * DV;

  float q[DQK];
#pragma unroll
  for (int d = 0; d < DQK; ++d) q[d] = row_valid ? qg[(int64_t)qi * DQK + d] : 0.0f;

  float o[DV];
#pragma unroll
  for (int d = 0; d < DV; ++d) o[d] = 0.0f;
  // Running max of z (log2 units); with the max logit estimate a constant.
  const bool mle = p.mle != 0;
  float m = mle ? p.mle_log2 : -INFINITY;
  float l = 0.0f;

  const int32_t* segq = p.seg_q ? p.seg_q + (int64_t)b * L : nullptr;
  const int32_t* segk = p.seg_kv ? p.seg_kv + (int64_t)b * L : segq;
  const int my_seg = (segq && row_valid) ? segq[qi] : 0;
  const bool capped = p.soft_cap > 0.0f;

  const int g0 = p.row_ptr[r];
  const int g1 = p.row_ptr[r + 1];
  for (int g = g0; g < g1; ++g) {
    const int c = p.active_cols[g];
    const bool partial = p.block_code[g] == 1;
    const int k0 = c * BKV;
    __syncthreads();  // previous block fully consumed
    for (int e = lane; e < BKV * DQK; e += 64) {
      const int kr = e / DQK, kd = e % DQK;
      ks[kr][kd] = (k0 + kr < L) ? kg[(int64_t)(k0 + kr) * DQK + kd] : 0.0f;
    }
    for (int e = lane; e < BKV * DV; e += 64) {
      const int kr = e / DV, kd = e % DV;
      vs[kr][kd] = (k0 + kr < L) ? vg[(int64_t)(k0 + kr) * DV + kd] : 0.0f;
    }
    __syncthreads();
    const uint8_t* pat = (partial && p.mask_stored)
                             ? p.patterns + (int64_t)p.mask_next[g] * (BQ * BKV) + lane * BKV
                             : nullptr;
#pragma unroll 1
    for (int s0 = 0; s0 < BKV; s0 += SUB) {
      float z[SUB];
      float zmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < SUB; ++j) {
        float dot = 0.0f;
#pragma unroll
        for (int d = 0; d < DQK; ++d) dot = fmaf(q[d], ks[s0 + j][d], dot);
        float zz = capped ? capped_log2(dot * p.scale, p.soft_cap) : dot * p.scale_log2;
        if (partial) {
          const int kj = k0 + s0 + j;
          bool ok;
          if (pat) {
            ok = pat[s0 + j] != 0;
          } else {
            ok = kj < L;
            if (p.causal) ok = ok && (kj <= qi);
            if (p.window_left >= 0) ok = ok && (qi - kj <= p.window_left);
            if (p.window_right >= 0) ok = ok && (kj - qi <= p.window_right);
            if (segq && kj < L) ok = ok && (segk[kj] == my_seg);
          }
          zz = ok ? zz : -INFINITY;
        }
        z[j] = zz;
        zmax = fmaxf(zmax, zz);
      }
      const float m_new = mle ? m : fmaxf(m, zmax);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = fast_exp2(m - m_use);
      float psum = 0.0f;
#pragma unroll
      for (int j = 0; j < SUB; ++j) {
        z[j] = fast_exp2(z[j] - m_use);
        psum += z[j];
      }
      l = l * alpha + psum;
      m = m_new;
#pragma unroll
      for (int d = 0; d < DV; ++d) {
        float acc = o[d] * alpha;
#pragma unroll
        for (int j = 0; j < SUB; ++j) acc = fmaf(z[j], vs[s0 + j][d], acc);
        o[d] = acc;
      }
    }
  }

  if (!row_valid) return;
  float* og = static_cast<float*>(p.o) + ((int64_t)head * L + qi) * DV;
  const float inv = (l > 0.0f) ? 1.0f / l : 0.0f;
#pragma unroll
  for (int d = 0; d < DV; ++d) og[d] = o[d] * inv;
  if (p.lse) {
    p.lse[(int64_t)head * L + qi] = (l > 0.0f) ? (m + __log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int DQK, int DV>
hipError_t launch(const FwdParams& p, hipStream_t s) {
  const int64_t n_wg = (int64_t)p.B * p.Hq * p.n_q_blocks;
  hipLaunchKernelGGL((splash_fwd_f32_kernel<DQK, DV>), dim3((unsigned)n_wg), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, int d_qk, int d_v, hipStream_t s) {
  if (d_qk == 64 && d_v == 64) return launch<64, 64>(p, s);
  if (d_qk == 128 && d_v == 128) return launch<128, 128>(p, s);
  if (d_qk == 64 && d_v == 128) return launch<64, 128>(p, s);
  if (d_qk == 128 && d_v == 64) return launch<128, 64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace splash
