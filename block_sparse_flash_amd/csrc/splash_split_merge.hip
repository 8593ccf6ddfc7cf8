// Merge of split-KV partial results into the attention output.
//
// Each of the n_split chunks s of a query row's active kv blocks produced
// its own normalised output o_s and log-sum-exp lse_s (the softmax over that
// chunk's keys alone).  The exact result over all keys follows from the
// order-free merge rule of "Lecture 13 - Pallas Kernels and Splash
// Attention" (CMU 11-868 notes), section 5.1 (partial (m, l, o) results of
// separate key ranges combine exactly, as in split-KV inference), written
// with the log-sum-exp residual as on the joto.ai page on core LLM
// operators, section "LSE and online softmax" (split-K reduction):
//   lse = log sum_s e^{lse_s},   o = sum_s e^{lse_s - lse} o_s.
// A chunk with no allowed key has lse_s = -inf and weight 0; a row with no
// allowed key at all gets o = 0 and lse = -inf.
//
// gfx950 layout: one wave per query row, lane i holding output elements
// i and i + 64 (d_v = 64 or 128: two or one of them); the n_split lse
// values are read once per wave, and every load and store is coalesced
// over the row.  The kernel is HBM-bound (it reads n_split * (d_v + 1)
// floats and writes d_v bf16 values and one float per row).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fwd_params.h"

namespace splash {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kRowsPerBlock = 4;   // waves per work-group, one row each

__device__ __forceinline__ uint16_t to_bf16(float x) {
  const __bf16 b = (__bf16)x;   // round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}

template <int DV>
__global__ __launch_bounds__(64 * kRowsPerBlock) void split_merge_bf16_kernel(FwdParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t n_rows = (int64_t)p.B * p.Hq * p.L;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const int S = p.n_split;
  // Largest partial lse of the row (-inf if no chunk saw an allowed key).
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, p.ws_lse[(int64_t)s * n_rows + row]);
  float acc0 = 0.0f, acc1 = 0.0f, den = 0.0f;
  if (mx != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float ls = p.ws_lse[(int64_t)s * n_rows + row];
      const float wgt = __builtin_amdgcn_exp2f((ls - mx) * kLog2e);   // 0 for ls = -inf
      den += wgt;
      const float* os = p.ws_o + ((int64_t)s * n_rows + row) * DV;
      acc0 += wgt * os[lane];
      if constexpr (DV > 64) acc1 += wgt * os[lane + 64];
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  uint16_t* o = static_cast<uint16_t*>(p.o) + row * DV;
  o[lane] = to_bf16(acc0 * inv);
  if constexpr (DV > 64) o[lane + 64] = to_bf16(acc1 * inv);
  if (p.lse && lane == 0) p.lse[row] = den > 0.0f ? mx + __log2f(den) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_split_merge_bf16(const FwdParams& p, int d_v, hipStream_t s) {
  const int64_t n_rows = (int64_t)p.B * p.Hq * p.L;
  const int64_t grid = (n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (grid == 0) return hipSuccess;
  if (d_v == 128)
    hipLaunchKernelGGL(split_merge_bf16_kernel<128>, dim3((unsigned)grid), dim3(64 * kRowsPerBlock), 0, s, p);
  else if (d_v == 64)
    hipLaunchKernelGGL(split_merge_bf16_kernel<64>, dim3((unsigned)grid), dim3(64 * kRowsPerBlock), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace splash
