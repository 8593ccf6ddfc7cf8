// bf16 block-sparse attention forward for gfx950 on MFMA.
//
// Method ("Lecture 13 - Pallas Kernels and Splash Attention", CMU 11-868
// notes): for every query row keep a running max m, a running sum l and an
// un-normalised output o (section 5.2); per kv block compute the scores,
// soft-cap and mask them (5.2, 5.4), update m, rescale l and o by
// alpha = e^(m_old - m_new), add the block's e^(s - m_new) and its weighted
// V rows (5.1), and divide o by l once after the last block (deferred
// normalisation, 5.2).  Only the active blocks of the execution table are
// visited; a partial block gets an element mask, a full block none (6.1-6.3).
// The residual lse = m + ln l is written with o (joto.ai page, "LSE and
// online softmax").
//
// gfx950 design (this file's own; the pages' TPU kernel is prior art):
//   * One work-group = 4 waves = one 128-query block of one head; wave w owns
//     32 query rows.  The work-group walks its row's active blocks (CSR list),
//     64 keys per block.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (fp32 accumulation): the accumulator then holds
//     one query per lane and 32 keys per lane (16 per 32x32 tile, two tiles),
//     so the row max / row sum are in-lane reductions plus one exchange
//     between the two half-waves; m and l are per-lane scalars.
//   * O^T = V^T P^T on the same MFMA.  The probabilities never leave the
//     registers (section 5.3 hands scores from the MXU to the VPU and back):
//     the accumulator items of S^T are reused directly as the B operand after
//     a bf16 conversion; the key order this implies is absorbed by storing V^T
//     in LDS in the matching permuted key order (the contraction over keys is
//     order-free).
//   * K and V tiles are double-buffered in LDS: the next block's global loads
//     are issued before this block's MFMAs and written to the other buffer
//     after them (section 3.1), one barrier per block.  Global loads are
//     16-byte vectors, coalesced along the head dimension; V is transposed in
//     registers (4 keys x 8 dims per thread, v_perm) on its way to LDS.
//     LDS rows are XOR-swizzled in 16-byte chunks so that the 32 rows read by
//     one MFMA operand fetch fall in distinct banks.
//   * exp is the hardware exp2 with log2(e) folded into the scale (section 6.6
//     "use_base2_exp").  With a soft cap, tanh(y) = 1 - 2 / (e^{2y} + 1).
//   * Waves whose 32 rows see none of a partial block skip it; waves for which
//     a partial block is entirely allowed skip the element mask (causal and
//     window bounds are intervals, so this is decided from the corners).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fwd_params.h"

namespace splash {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = kBf16BlockQ;   // 128 queries per work-group
constexpr int BN = kBf16BlockKV;  // 64 keys per block
constexpr int NT = 256;           // threads per work-group (4 waves)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <int DQK, int DV>
struct Smem {
  static constexpr int kElems = BN * DQK;  // K tile, u16 elements
  static constexpr int vElems = DV * BN;   // V^T tile
  static constexpr int bytes = 2 * (kElems + vElems) * 2;
};

template <int DQK, int DV, bool CAP>
__global__ __launch_bounds__(NT) void splash_fwd_bf16_kernel(FwdParams p) {
  static_assert(DQK % 16 == 0 && DV % 32 == 0, "head dims");
  constexpr int KS = DQK / 16;         // MFMA k-steps for S^T
  constexpr int DT = DV / 32;          // O^T row tiles
  constexpr int KCH = DQK / 8;         // 16-byte chunks per K row
  constexpr int KPT = BN * KCH / NT;   // K chunks loaded per thread
  constexpr int VUNITS = (BN / 4) * (DV / 8);  // 4-key x 8-dim V units
  static_assert(BN * KCH % NT == 0 && VUNITS <= NT, "tile split");

  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* ks = smem;                                // [2][BN][DQK]   swizzled
  uint16_t* vs = smem + 2 * Smem<DQK, DV>::kElems;   // [2][DV][BN]    swizzled

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int head, rank;
  map_workgroup(p, blockIdx.x, &head, &rank);
  const int b = head / p.Hq;
  const int hq = head - b * p.Hq;
  const int kvh = b * p.Hkv + hq / p.group;
  const int L = p.L;
  const int r = p.row_order[rank];
  const int qw = r * BM + wave * 32;  // first query row of this wave
  const int qi = qw + l32;            // this lane's query row
  const bool row_valid = qi < L;

  const uint16_t* qg = static_cast<const uint16_t*>(p.q) + (int64_t)head * L * DQK;
  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + (int64_t)kvh * L * DQK;
  const uint16_t* vg = static_cast<const uint16_t*>(p.v) + (int64_t)kvh * L * DV;

  // Q^T as the B operand: lane (l32, hi) holds Q[qi][16 s + 8 hi + 0..7].
  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (row_valid) w = *reinterpret_cast<const u32x4*>(qg + (int64_t)qi * DQK + 16 * s + 8 * hi);
    qf[s] = __builtin_bit_cast(bf16x8, w);
  }

  // Staging registers for the next tile.
  u32x4 kst[KPT];
  u32x4 vst[4];

  auto load_tile = [&](int c) {
    const int k0 = c * BN;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int ci = tid + NT * j;
      const int key = ci / KCH;
      const int cc = ci - key * KCH;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (k0 + key < L) w = *reinterpret_cast<const u32x4*>(kg + (int64_t)(k0 + key) * DQK + cc * 8);
      kst[j] = w;
    }
    if (tid < VUNITS) {
      const int kq = tid & 15;  // group of 4 keys
      const int dc = tid >> 4;  // 8-dim chunk
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 4 * kq + i;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (k0 + key < L) w = *reinterpret_cast<const u32x4*>(vg + (int64_t)(k0 + key) * DV + dc * 8);
        vst[i] = w;
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* kb = ks + buf * Smem<DQK, DV>::kElems;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int ci = tid + NT * j;
      const int key = ci / KCH;
      const int cc = ci - key * KCH;
      *reinterpret_cast<u32x4*>(kb + key * DQK + ((cc ^ (key & 7)) * 8)) = kst[j];
    }
    if (tid < VUNITS) {
      uint16_t* vb = vs + buf * Smem<DQK, DV>::vElems;
      const int kq = tid & 15;
      const int dc = tid >> 4;
      // Key 4kq+i goes to permuted position pos(4kq)+i of its V^T row, where
      // within each 16-key group key k sits at 8*((k/4)%2) + 4*(k/8) + k%4.
      const int chunk = 2 * (kq >> 2) + (kq & 1);
      const int within = 4 * ((kq & 3) >> 1);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const uint32_t lo01 = __builtin_amdgcn_perm(vst[1][jj], vst[0][jj], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(vst[3][jj], vst[2][jj], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(vst[1][jj], vst[0][jj], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(vst[3][jj], vst[2][jj], 0x07060302u);
        const int d0 = 8 * dc + 2 * jj;
        const int d1 = d0 + 1;
        u32x2 w0 = {lo01, lo23};
        u32x2 w1 = {hi01, hi23};
        *reinterpret_cast<u32x2*>(vb + d0 * BN + ((chunk ^ (d0 & 7)) * 8) + within) = w0;
        *reinterpret_cast<u32x2*>(vb + d1 * BN + ((chunk ^ (d1 & 7)) * 8) + within) = w1;
      }
    }
  };

  // Softmax state: z values are in log2 units after multiplying by zc.
  //   no cap: z = q.k,                          zc = scale * log2(e)
  //   cap:    z = log2(e) cap tanh(scale q.k / cap), zc = 1
  const float zc = CAP ? 1.0f : p.scale_log2;
  float m = -INFINITY;
  float l = 0.0f;
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.0f;

  const bool has_seg = p.seg_q != nullptr;
  const int32_t* segq = has_seg ? p.seg_q + (int64_t)b * L : nullptr;
  const int32_t* segk = has_seg ? (p.seg_kv ? p.seg_kv + (int64_t)b * L : segq) : nullptr;
  const int my_seg = (has_seg && row_valid) ? segq[qi] : 0;
  // Allowed key interval of this lane's row before the segment test.
  int klo = 0, khi = L - 1;
  if (p.causal) khi = min(khi, qi);
  if (p.window_left >= 0) klo = max(klo, qi - p.window_left);
  if (p.window_right >= 0) khi = min(khi, qi + p.window_right);
  const int qa = qw;
  const int qb = min(qw + 31, L - 1);

  const int g0 = p.row_ptr[r];
  const int g1 = p.row_ptr[r + 1];

  if (g0 < g1) {
    load_tile(p.active_cols[g0]);
    store_tile(0);
  }
  __syncthreads();

  for (int g = g0, it = 0; g < g1; ++g, ++it) {
    const int buf = it & 1;
    const bool has_next = g + 1 < g1;
    if (has_next) load_tile(p.active_cols[g + 1]);

    const int c = p.active_cols[g];
    const int code = p.block_code[g];
    const int ka = c * BN;
    const int kb = ka + BN - 1;
    // Per-wave class: 0 = nothing allowed for these rows, 1 = element mask,
    // 2 = every element allowed.
    int wcls;
    if (qa >= L) {
      wcls = 0;
    } else if (code == 2) {
      wcls = 2;
    } else if (p.mask_stored) {
      wcls = 1;
    } else {
      const int kbv = min(kb, L - 1);
      const bool none = (p.causal && ka > qb) || (p.window_left >= 0 && qa - kbv > p.window_left) ||
                        (p.window_right >= 0 && ka - qb > p.window_right);
      const bool all = !has_seg && kb < L && (!p.causal || kb <= qa) &&
                       (p.window_left < 0 || qb - ka <= p.window_left) &&
                       (p.window_right < 0 || kb - qa <= p.window_right);
      wcls = none ? 0 : (all ? 2 : 1);
    }

    if (wcls != 0) {
      const uint16_t* kb_lds = ks + buf * Smem<DQK, DV>::kElems;
      const uint16_t* vb_lds = vs + buf * Smem<DQK, DV>::vElems;

      // S^T tile t covers keys 32t..32t+31 of the block; lane (l32, hi)
      // item E holds key 32t + 8(E/4) + 4hi + E%4 for query qi.
      f32x16 sacc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[t][e] = 0.0f;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int key = 32 * t + l32;
          const int chunk = 2 * s + hi;
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb_lds + key * DQK + ((chunk ^ (key & 7)) * 8));
          sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[t], 0, 0, 0);
        }
      }

      if (CAP) {
        const float k2 = 2.0f * kLog2e * p.scale / p.soft_cap;
        const float A = p.soft_cap * kLog2e;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float ex = fast_exp2(sacc[t][e] * k2);
            sacc[t][e] = A - 2.0f * A * __builtin_amdgcn_rcpf(ex + 1.0f);
          }
      }

      if (wcls == 1) {
        if (p.mask_stored) {
          const uint8_t* pat = p.patterns + (int64_t)p.mask_next[g] * (BM * BN) + (wave * 32 + l32) * BN;
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const uint32_t bits = *reinterpret_cast<const uint32_t*>(pat + 32 * t + 8 * q4 + 4 * hi);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (((bits >> (8 * e)) & 0xffu) == 0u) sacc[t][4 * q4 + e] = -INFINITY;
            }
        } else {
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int key = ka + 32 * t + 8 * q4 + 4 * hi + e;
                bool ok = key >= klo && key <= khi;
                if (has_seg) ok = ok && segk[min(key, L - 1)] == my_seg;
                if (!ok) sacc[t][4 * q4 + e] = -INFINITY;
              }
        }
      }

      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[t][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);
      const float mc = (m_new == -INFINITY) ? 0.0f : m_new * zc;
      const float alpha = fast_exp2(m * zc - mc);
      m = m_new;

      // P^T as bf16 B operands: instruction (t, c2) takes items 8c2..8c2+7.
      bf16x8 pb[2][2];
      float psum = 0.0f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          u32x4 w;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const float p0 = fast_exp2(fmaf(sacc[t][8 * c2 + 2 * e2], zc, -mc));
            const float p1 = fast_exp2(fmaf(sacc[t][8 * c2 + 2 * e2 + 1], zc, -mc));
            psum += p0 + p1;
            w[e2] = pack_bf16(p0, p1);
          }
          pb[t][c2] = __builtin_bit_cast(bf16x8, w);
        }
      l = l * alpha + psum;

#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;

#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 32 * dt + l32;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) {
            const int chunk = 2 * (2 * t + c2) + hi;
            const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vb_lds + d * BN + ((chunk ^ (d & 7)) * 8));
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[t][c2], oacc[dt], 0, 0, 0);
          }
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: deferred normalisation o / l and lse = (m zc + log2 l) ln 2.
  const float lt = l + __shfl_xor(l, 32);
  if (!row_valid) return;
  const float inv = (lt > 0.0f) ? 1.0f / lt : 0.0f;
  uint16_t* og = static_cast<uint16_t*>(p.o) + ((int64_t)head * L + qi) * DV;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      // items 4q4..4q4+3 of tile dt are dims 32dt + 8q4 + 4hi + 0..3
      u32x2 w = {pack_bf16(oacc[dt][4 * q4] * inv, oacc[dt][4 * q4 + 1] * inv),
                 pack_bf16(oacc[dt][4 * q4 + 2] * inv, oacc[dt][4 * q4 + 3] * inv)};
      *reinterpret_cast<u32x2*>(og + 32 * dt + 8 * q4 + 4 * hi) = w;
    }
  if (p.lse && hi == 0)
    p.lse[(int64_t)head * L + qi] = (lt > 0.0f) ? (m * zc + __log2f(lt)) * kLn2 : -INFINITY;
}

template <int DQK, int DV, bool CAP>
hipError_t launch(const FwdParams& p, hipStream_t s) {
  const int64_t n_wg = (int64_t)p.B * p.Hq * p.n_q_blocks;
  const int bytes = Smem<DQK, DV>::bytes;
  auto fn = splash_fwd_bf16_kernel<DQK, DV, CAP>;
  if (bytes > 65536) {
    // Opt in to more than 64 KiB of dynamic LDS (gfx950 has 160 KiB per CU).
    // Setting the attribute again is harmless; a failure shows up at launch.
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                              hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    (void)hipGetLastError();
  }
  hipLaunchKernelGGL(fn, dim3((unsigned)n_wg), dim3(NT), bytes, s, p);
  return hipGetLastError();
}

template <int DQK, int DV>
hipError_t launch_cap(const FwdParams& p, hipStream_t s) {
  return p.soft_cap > 0.0f ? launch<DQK, DV, true>(p, s) : launch<DQK, DV, false>(p, s);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, int d_qk, int d_v, hipStream_t s) {
  if (d_qk == 128 && d_v == 128) return launch_cap<128, 128>(p, s);
  if (d_qk == 192 && d_v == 128) return launch_cap<192, 128>(p, s);
  if (d_qk == 64 && d_v == 64) return launch_cap<64, 64>(p, s);
  if (d_qk == 128 && d_v == 64) return launch_cap<128, 64>(p, s);
  if (d_qk == 64 && d_v == 128) return launch_cap<64, 128>(p, s);
  if (d_qk == 192 && d_v == 64) return launch_cap<192, 64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace splash
