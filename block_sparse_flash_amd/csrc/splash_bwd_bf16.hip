// bf16 block-sparse attention backward for gfx950 on MFMA.
//
// Method: the forward keeps only o and the per-row logsumexp residual
// ("Lecture 13 - Pallas Kernels and Splash Attention", section 6.3); the
// backward rebuilds the probabilities on chip as p = e^(logit - lse) (joto.ai
// page on core LLM operators, "LSE and online softmax": read q and k,
// recompute the dot product, subtract the stored lse scalar, exponentiate).
// With y = scale q.k, logit z = cap tanh(y / cap) (z = y without a cap),
// D_i = do_i . o_i and dp_ij = do_i . v_j, the chain rule through the softmax
// gives dy_ij = p_ij (dp_ij - D_i) dz/dy, and
//   dv_j = sum_i p_ij do_i,  dk_j = scale sum_i dy_ij q_i,  dq_i = scale sum_j dy_ij k_j.
// Only the active blocks of the execution table are visited; the element
// mask (causal, window, segment ids, padding) is evaluated from positions on
// every visited block.
//
// gfx950 design:
//   * The dq kernel runs first and also computes D_i from o and do for its
//     rows, writing it for the dk/dv kernel.
//   * dk/dv kernel: one work-group (4 waves) per (K/V head, 64-key block)
//     walks the block's column of the table (the q blocks that read it) for
//     every query head of the GQA group, in 64-row sub-tiles, so dk and dv
//     are summed in registers with no atomics.  Wave w owns keys
//     32 (w % 2) .. + 31 and accumulates dV (w < 2) or dK (w >= 2) over all
//     rows: 64 accumulator registers per wave, so two work-groups fit per
//     CU (both dK and dV in one wave take 128 and spill).  Each wave
//     computes S = Q K^T, dP = dO V^T, P and dS only for its half of the
//     sub-tile's rows (rows 32 (w / 2) .. + 31), so every element is
//     computed once; the two waves of a key half then swap the part the
//     other needs (P to the dV wave, dS to the dK wave) through LDS.
//     S and dP come out of v_mfma_f32_32x32x16_bf16 with one key per lane
//     and 16 rows per lane; those accumulator items, rounded to bf16, are
//     directly the A operand of dV += P^T dO or dK += dS^T Q (the MFMA's
//     reduction index runs over the rows in the order the accumulator holds
//     them; the partner's lane of the same index holds its rows in the same
//     order), and the B operands are read transposed from the row-major Q
//     and dO tiles with ds_read_b64_tr_b16 (four consecutive rows of one
//     column per lane, the row grouping the accumulator implies).
//   * dq kernel: one work-group (8 waves, 32 rows each) per (query head,
//     256-row q block) walks the row's active kv blocks; S^T = K Q^T and
//     dP^T = V dO^T hold one row per lane, and dS^T feeds dQ += dS K the same
//     way, with K read transposed.
//   * LDS tiles are row-major; 128-wide rows take an XOR swizzle of their
//     16-byte chunks and other widths a 16-byte row pad, so that operand and
//     transposing reads fall in distinct banks (see Lay).
//   * 192-wide q/k heads (with 128-wide v): S takes 12 k-steps and dP 8, dK
//     6 accumulator tiles and dV 4; the dk/dv kernel then runs one work-group
//     per CU with one inlined copy of its body per role, and the dq kernel
//     keeps Q in LDS.
//   * Gradients are accumulated and written in float32.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "bwd_params.h"
#include "fwd_params.h"

namespace splash {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) float lds_f32;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
typedef __attribute__((address_space(3))) int32_t lds_i32;

constexpr int BQ = kBwdBlockQ;   // rows per q block of the tables
constexpr int BK = kBwdBlockKV;  // keys per kv block of the tables
constexpr int SUB = 64;           // rows per sub-tile in the dk/dv kernel
constexpr float kLog2e = 1.4426950408889634f;

// LDS layout of a row-major tile with D bf16 columns, in 16-byte chunks.
// Two reads must be bank-conflict free: an operand read, where 16 lanes
// take one chunk of 16 consecutive rows, and a transposing read, where 32
// lanes take 64 bytes of each of 4 consecutive rows.  With 256-byte rows
// (D = 128) chunk c of row r is stored at chunk c ^ 4 (r % 4) ^ (r / 4) % 4:
// 16 consecutive rows get 16 distinct chunks, and 4 consecutive rows put
// each 64-byte group into a different quarter of the banks.  Other tiles
// (and kernels that cannot spare the registers for the address arithmetic)
// pad each row by 16 bytes instead.
template <int D, bool SWIZZLE>
struct Lay {
  static constexpr bool SWZ = SWIZZLE && D == 128;
  static constexpr int ROW = SWZ ? D : D + 8;  // elements per row
  // Element offset of chunk c of row r.
  __device__ static __forceinline__ int off(int r, int c) {
    return r * ROW + 8 * (SWZ ? (c ^ ((r & 3) << 2) ^ ((r >> 2) & 3)) : c);
  }
  // Element offset of element `col` of row r (col % 8 stays in its chunk).
  __device__ static __forceinline__ int at(int r, int col) {
    return SWZ ? off(r, col >> 3) + (col & 7) : r * ROW + col;
  }
};

// Raw buffer resource over `bytes` bytes from `base` (a wave-uniform
// address): loads past the end return zero, with no branch per load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}

// Table entry t[i] read through the scalar cache: the tables are read-only
// for the whole launch and i is wave-uniform.
__device__ __forceinline__ int32_t sload(const int32_t* t, int i) {
  return ((const __attribute__((address_space(4))) int32_t*)t)[__builtin_amdgcn_readfirstlane(i)];
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}


__device__ __forceinline__ bf16x8 ld_op(const lds_u16* ptr) { return *reinterpret_cast<const lds_bf16x8*>(ptr); }

// Operand of 8 rows of one column from a row-major tile: in each group of
// 16 lanes, lane j addresses row base + j / 4 at columns 4 (j % 4) .. + 3 of
// the group's 16 columns, and ds_read_b64_tr_b16 hands lane i of the group
// rows base .. base + 3 of column i; `lo` and `hi` are the lane's addresses
// in the two 4-row runs (rows base and base + 8).
__device__ __forceinline__ bf16x8 ld_tr(const lds_u16* lo, const lds_u16* hi) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)lo);
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)hi);
  const u32x2 a2 = __builtin_bit_cast(u32x2, a);
  const u32x2 b2 = __builtin_bit_cast(u32x2, b);
  const u32x4 v = {a2[0], a2[1], b2[0], b2[1]};
  return __builtin_bit_cast(bf16x8, v);
}

// Work-group w -> (unit, index inside the unit) for n_units units of n_per
// items each.  Consecutive work-group ids go round-robin over the 8 XCDs;
// when the unit count divides over them, all items of a unit (one head's
// blocks, which read the same Q/dO or K/V) run on one XCD and share its L2;
// with fewer units than XCDs (a divisor of 8), each unit gets 8 / n_units
// XCDs of its own.
__device__ __forceinline__ void xcd_map(int w, int n_units, int n_per, int* unit, int* idx) {
  const int xcd = w % kNumXcd;
  const int slot = w / kNumXcd;
  if (n_units % kNumXcd == 0) {
    const int u = slot / n_per;
    *unit = u * kNumXcd + xcd;
    *idx = slot - u * n_per;
  } else if (kNumXcd % n_units == 0 && (n_units * n_per) % kNumXcd == 0) {
    const int share = kNumXcd / n_units;  // XCDs per unit
    *unit = xcd % n_units;
    *idx = slot * share + xcd / n_units;
  } else {
    *unit = w / n_per;
    *idx = w - *unit * n_per;
  }
}

// The dq kernel's order: as xcd_map, but the q blocks of a unit are taken
// by rank (0 = the longest row), and on an XCD with several units the ranks
// of two units at a time interleave (unit pair g: rank 0 of both, rank 1 of
// both, ...).  With one work-group per item and the hardware handing items
// to CUs in order, the longest rows then start first, as in a
// longest-processing-time-first schedule, while only two units' K/V are in
// flight per XCD (units in plain order, each shortest row first, left the
// longest causal rows to run last: a 29% tail in a simulation of the
// dispatch).
__device__ __forceinline__ void xcd_map_ranked(int w, int n_units, int n_per, int* unit, int* rank) {
  if (n_units % kNumXcd == 0) {
    constexpr int G = 2;
    const int xcd = w % kNumXcd;
    const int slot = w / kNumXcd;
    const int U = n_units / kNumXcd;            // units on this XCD
    const int g = slot / (G * n_per);           // unit pair
    const int gsz = min(G, U - g * G);          // units in it (1 for an odd last one)
    const int rem = slot - g * G * n_per;
    const int rk = rem / gsz;
    *unit = (g * G + (rem - rk * gsz)) * kNumXcd + xcd;
    *rank = rk;
  } else {
    xcd_map(w, n_units, n_per, unit, rank);
  }
}

// Runs N unrolled steps: step i's operands are loaded by ld(i) DIST steps
// before use(i, operands) consumes them, with scheduling fences so that the
// compiler keeps the loads that far ahead (left alone it moves every LDS
// read to just before its MFMA, which then waits out the LDS latency).
template <int N, int DIST, typename Ld, typename Use>
__device__ __forceinline__ void pipelined(Ld ld, Use use) {
  using Op = decltype(ld(0));
  Op buf[DIST + 1];
#pragma unroll
  for (int i = 0; i < DIST && i < N; ++i) buf[i] = ld(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + DIST < N) buf[(i + DIST) % (DIST + 1)] = ld(i + DIST);
    __builtin_amdgcn_sched_barrier(0);
    use(i, buf[i % (DIST + 1)]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

struct Op2 {
  bf16x8 a, b;
};
struct Op4 {
  bf16x8 a, b, c, d;
};

// Whether every pair of query rows [r0, r0 + nr) and keys [k0, k0 + nk) is
// allowed by position (causal, window, bounds; segment ids aside).
__device__ __forceinline__ bool pos_allowed(const BwdParams& p, int r0, int nr, int k0, int nk) {
  const int pa = p.q_off + r0;  // smallest row position
  const int pz = pa + nr - 1;   // largest
  const int kz = k0 + nk - 1;   // largest key
  return r0 + nr <= p.L && kz < p.Lkv && (!p.causal || kz <= pa) &&
         (p.window_left < 0 || pz - k0 <= p.window_left) && (p.window_right < 0 || kz - pa <= p.window_right);
}

// Whether `id` is the same in every lane of the wave and equals `ref`
// (wave-uniform result).
__device__ __forceinline__ bool all_equal(int id, int ref) { return __all(id == ref) != 0; }

// Copies rows row0 .. row0 + 63 of a row-major [n_valid, D] bf16 matrix
// into LDS (zeros past n_valid), laid out by Lay<D, SWZ>.
template <int D, int NTHR, bool SWZ>
__device__ __forceinline__ void load_tile(const uint16_t* g, int row0, int n_valid, lds_u16* rm, int tid) {
  constexpr int CH = D / 8;
  constexpr int TOTAL = 64 * CH;
  static_assert(TOTAL % NTHR == 0, "whole chunks per thread");
#pragma unroll
  for (int it = 0; it < TOTAL / NTHR; ++it) {
    const int x = it * NTHR + tid;
    const int r = x / CH;
    const int c = x - r * CH;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (row0 + r < n_valid) val = *reinterpret_cast<const u32x4*>(g + (int64_t)(row0 + r) * D + c * 8);
    *reinterpret_cast<lds_u32x4*>(rm + Lay<D, SWZ>::off(r, c)) = val;
  }
}

// Rows row0 .. row0 + 63 of a row-major [n_valid, D] bf16 matrix staged in
// registers (zeros past n_valid): fetched from global memory while the
// previous tile is being used, stored to LDS after the next barrier.
template <int D, int NTHR, bool SWZ>
struct TileRegs {
  static constexpr int CH = D / 8;
  static constexpr int N = 64 * CH / NTHR;
  static_assert(64 * CH % NTHR == 0, "whole chunks per thread");
  u32x4 v[N];
  // `rs` covers the n_valid rows of the matrix: rows past them read as zero.
  __device__ __forceinline__ void fetch(__amdgpu_buffer_rsrc_t rs, int row0, int tid) {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int x = it * NTHR + tid;
      const int r = x / CH;
      const int c = x - r * CH;
      v[it] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rs, (uint32_t)(((row0 + r) * D + c * 8) * 2), 0, 0));
    }
  }
  __device__ __forceinline__ void store(lds_u16* rm, int tid) const {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int x = it * NTHR + tid;
      const int r = x / CH;
      const int c = x - r * CH;
      *reinterpret_cast<lds_u32x4*>(rm + Lay<D, SWZ>::off(r, c)) = v[it];
    }
  }
};

// Probability and score gradient of one (row, key) pair from its raw dot
// product s, the row's lse (log2 units), its D and dP.
template <bool CAP>
__device__ __forceinline__ void p_and_ds(const BwdParams& p, bool ok, float s, float lse2, float dpv,
                                         float dlt, float* pe, float* ds) {
  float z2, fac = 1.0f;
  if constexpr (CAP) {
    // t = tanh(y / cap) = 1 - 2 / (e^{2y/cap} + 1), y = scale s.
    const float u = 1.0f / (__builtin_amdgcn_exp2f(2.0f * kLog2e * p.scale / p.soft_cap * s) + 1.0f);
    const float t = 1.0f - 2.0f * u;
    z2 = p.soft_cap * kLog2e * t;
    fac = 1.0f - t * t;
  } else {
    z2 = p.scale_log2 * s;
  }
  const float e = ok ? __builtin_amdgcn_exp2f(z2 - lse2) : 0.0f;
  *pe = e;
  *ds = e * (dpv - dlt) * fac;
}

template <int DQK, int DV>
struct DkdvLds {
  static constexpr int NQ = DQK / 32, NV = DV / 32;
  static constexpr int RK = Lay<DQK, true>::ROW;
  static constexpr int RV = Lay<DV, true>::ROW;
  static constexpr int K_OFF = 0;                          // K [64][RK]
  static constexpr int V_OFF = K_OFF + 64 * RK * 2;        // V [64][RV]
  static constexpr int Q_OFF = V_OFF + 64 * RV * 2;        // Q [64][RK]
  static constexpr int O_OFF = Q_OFF + 64 * RK * 2;        // dO [64][RV]
  static constexpr int LSE_OFF = O_OFF + 64 * RV * 2;      // lse * log2(e) [64]
  static constexpr int D_OFF = LSE_OFF + 64 * 4;           // D [64]
  static constexpr int SEG_OFF = D_OFF + 64 * 4;           // row segment ids [64]
  static constexpr int X_OFF = SEG_OFF + 64 * 4;           // P or dS handed over [4 waves][2][64 lanes][8 bf16]
  static constexpr int BYTES = X_OFF + 4 * 64 * 32;
  static_assert(BYTES <= 163840, "fits the LDS of a CU");
};

template <int DQK, int DV, bool CAP>
// Two work-groups per CU where their LDS fits (then 256 registers per
// lane), else one with the whole register file.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DkdvLds<DQK, DV>::BYTES <= 81920 ? 2 : 1,
                                                                     DkdvLds<DQK, DV>::BYTES <= 81920 ? 2 : 1)))
void bwd_dkdv_kernel(BwdParams p) {
  using M = DkdvLds<DQK, DV>;
  using LQ = Lay<DQK, true>;
  using LV = Lay<DV, true>;
  constexpr int NQ = DQK / 32, NV = DV / 32;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  lds_u8* lds = (lds_u8*)smem;
  lds_u16* Ks = (lds_u16*)(lds + M::K_OFF);
  lds_u16* Vs = (lds_u16*)(lds + M::V_OFF);
  lds_u16* Qs = (lds_u16*)(lds + M::Q_OFF);
  lds_u16* Os = (lds_u16*)(lds + M::O_OFF);
  lds_f32* lse2s = (lds_f32*)(lds + M::LSE_OFF);
  lds_f32* Ds = (lds_f32*)(lds + M::D_OFF);
  lds_i32* segqs = (lds_i32*)(lds + M::SEG_OFF);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int kh = wave & 1;   // key half of the block
  const int rh = wave >> 1;  // row half of each 64-row sub-tile whose S and dP this wave computes
  const bool dk_wave = rh != 0;  // wave-uniform: accumulates dK (else dV)
  // This wave's hand-over slots (two 16-byte runs per lane, laid out
  // [wave][run][lane] so that a wave's write or read covers consecutive
  // 16-byte words) and its partner's: the wave of the same keys and the
  // other row half.
  lds_u32x4* xme = (lds_u32x4*)(lds + M::X_OFF) + wave * 128 + lane;
  const lds_u32x4* xpart = (const lds_u32x4*)(lds + M::X_OFF) + (wave ^ 2) * 128 + lane;
  // Transposed-read address of this lane: row 4 hi + (lane % 16) / 4 of a
  // 16-row step, columns 16 ((lane / 16) % 2) + 4 (lane % 4) of a 32-column tile.
  const int trow = 4 * hi + ((lane & 15) >> 2);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  int c, bk;  // kv block, b * Hkv + kv head
  xcd_map(blockIdx.x, p.B * p.Hkv, p.n_kv_blocks, &bk, &c);
  if (p.col_order) c = p.col_order[c];  // the longest columns first
  const int b = bk / p.Hkv;
  const int kvh = bk - b * p.Hkv;
  const int key0 = c * BK;
  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + (int64_t)bk * p.Lkv * DQK;
  const uint16_t* vg = static_cast<const uint16_t*>(p.v) + (int64_t)bk * p.Lkv * DV;
  load_tile<DQK, 256, true>(kg, key0, p.Lkv, Ks, tid);
  load_tile<DV, 256, true>(vg, key0, p.Lkv, Vs, tid);

  const bool has_seg = p.seg_q != nullptr;
  const int my_key = key0 + 32 * kh + l32;
  const int32_t* segk = has_seg ? (p.seg_kv ? p.seg_kv + (int64_t)b * p.Lkv : p.seg_q + (int64_t)b * p.L) : nullptr;
  const int kseg = (has_seg && my_key < p.Lkv) ? segk[my_key] : 0;
  // The wave's 32 keys in one segment (its id kseg0): then a tile whose rows
  // are all in that segment needs no element test for the ids.
  const int kseg0 = __builtin_amdgcn_readfirstlane(kseg);
  const bool kseg_one = !has_seg || all_equal(kseg, kseg0);
  // Rows allowed to see this lane's key by position: causal pos >= key,
  // window pos - key <= left and key - pos <= right, pos = q_off + row.
  int rlo = 0, rhi = my_key < p.Lkv ? p.L - 1 : -1;
  if (p.causal) rlo = max(rlo, my_key - p.q_off);
  if (p.window_right >= 0) rlo = max(rlo, my_key - p.window_right - p.q_off);
  if (p.window_left >= 0) rhi = min(rhi, my_key + p.window_left - p.q_off);

  // The rest of the kernel for role ROLE: 0 = chosen per wave at run time
  // (dK and dV of the same shape), 1 = dK, 2 = dV.  With different shapes
  // (192/128) each role runs its own copy, so that each keeps one
  // accumulator shape (one array used with both shapes makes the compiler
  // shuffle it between register files).
  auto body = [&](auto role_) __attribute__((always_inline)) {
    constexpr int ROLE = decltype(role_)::value;
    const bool dkw = ROLE == 1 ? true : ROLE == 2 ? false : dk_wave;  // accumulates dK (else dV)
    constexpr int NA = NQ > NV ? NQ : NV;
    f32x16 acc[NA];  // dK (NQ tiles) or dV (NV tiles) of this wave's 32 keys
#pragma unroll
    for (int i = 0; i < NA; ++i) acc[i] = f32x16{};

    const int x0 = p.col_ptr[c];
    const int x1 = p.col_ptr[c + 1];
    const int32_t* sq = has_seg ? p.seg_q + (int64_t)b * p.L : nullptr;
    // Cursor over the work-group's sub-tiles: query head cg of the group,
    // entry cx of the column, sub-tile cs of that q block.  The sub-tiles
    // whose positions allow a pair with this kv block form one run per entry
    // (every bound below is monotone in the row): rows row_lo .. row_hi, so
    // cs runs from cs to chi, both set once per entry from its first row crow.
    static_assert(SUB == 64, "sub-tile index by shift");
    int row_lo = 0, row_hi = p.L - 1;
    if (p.causal) row_lo = max(row_lo, key0 - p.q_off - SUB + 1);                      // q_off + row + SUB - 1 >= key0
    if (p.window_right >= 0) row_lo = max(row_lo, key0 - p.window_right - p.q_off - SUB + 1);
    if (p.window_left >= 0) row_hi = min(row_hi, key0 + BK - 1 + p.window_left - p.q_off);
    int cg = 0, cx = x0, cs = 0, chi = -1, crow = 0;
    auto enter = [&]() __attribute__((always_inline)) {
      crow = sload(p.col_rows, cx) * BQ;
      cs = max(0, (row_lo - crow + SUB - 1) >> 6);          // ceil((row_lo - crow) / SUB)
      chi = min(BQ / SUB - 1, (row_hi - crow) >> 6);        // floor((row_hi - crow) / SUB)
    };
    if (x0 < x1) enter();
    auto next = [&](int* g_out, int* row0_out) __attribute__((always_inline)) -> bool {
      if (x0 >= x1) return false;
      while (cs > chi) {
        if (++cx >= x1) {
          if (++cg >= p.group) return false;
          cx = x0;
        }
        enter();
      }
      *g_out = cg;
      *row0_out = crow + cs * SUB;
      ++cs;
      return true;
    };
    // The next sub-tile's Q, dO, lse, D and segment ids are fetched into
    // registers while the current one is computed.
    TileRegs<DQK, 256, true> q_next;
    TileRegs<DV, 256, true> o_next;
    float lse_next = 0.0f, d_next = 0.0f;
    int seg_next = 0;
    auto fetch = [&](int g, int row0) __attribute__((always_inline)) {
      const int64_t head = b * p.Hq + kvh * p.group + g;
      q_next.fetch(buffer_rsrc(static_cast<const uint16_t*>(p.q) + head * p.L * DQK, (uint32_t)p.L * DQK * 2),
                   row0, tid);
      o_next.fetch(buffer_rsrc(static_cast<const uint16_t*>(p.dout) + head * p.L * DV, (uint32_t)p.L * DV * 2),
                   row0, tid);
      if (tid < SUB) {
        const int qi = row0 + tid;
        const bool in = qi < p.L;
        lse_next = in ? p.lse[head * p.L + qi] * kLog2e : INFINITY;
        d_next = in ? p.delta[head * p.L + qi] : 0.0f;
        seg_next = (has_seg && in) ? sq[qi] : 0;
      }
    };
    int next_g = 0, next_row0 = 0;
    bool have = next(&next_g, &next_row0);
    if (have) fetch(next_g, next_row0);
    while (have) {
      const int row0 = next_row0;
      __syncthreads();  // the previous sub-tile is consumed
      q_next.store(Qs, tid);
      o_next.store(Os, tid);
      if (tid < SUB) {
        lse2s[tid] = lse_next;
        Ds[tid] = d_next;
        segqs[tid] = seg_next;
      }
      __syncthreads();
      have = next(&next_g, &next_row0);
      if (have) fetch(next_g, next_row0);

      // S = Q K^T and dP = dO V^T on rows 32 rh .. + 31 of the sub-tile and
      // the wave's 32 keys (two interleaved chains; S takes DQK / 16 k-steps,
      // dP DV / 16): one key per lane, rows 32 rh + items.
      f32x16 s = f32x16{}, dp = f32x16{};
      pipelined<(DQK > DV ? DQK : DV) / 16, 1>(
          [&](int st) {
            Op4 o{};
            if (st < DQK / 16) {
              o.a = ld_op(Qs + LQ::off(32 * rh + l32, 2 * st + hi));
              o.b = ld_op(Ks + LQ::off(32 * kh + l32, 2 * st + hi));
            }
            if (st < DV / 16) {
              o.c = ld_op(Os + LV::off(32 * rh + l32, 2 * st + hi));
              o.d = ld_op(Vs + LV::off(32 * kh + l32, 2 * st + hi));
            }
            return o;
          },
          [&](int st, const Op4& o) {
            if (st < DQK / 16) s = mfma(o.a, o.b, s);
            if (st < DV / 16) dp = mfma(o.c, o.d, dp);
          });

      // Row data of the 16 rows 32 rh + 8 (e / 4) + 4 hi + e % 4 (four runs of 4).
      float pv[16], dsv[16];
      const bool all_ok = pos_allowed(p, row0 + 32 * rh, 32, key0 + 32 * kh, 32) &&
                          (!has_seg || (kseg_one && all_equal(segqs[32 * rh + l32], kseg0)));  // wave-uniform
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int rl0 = 32 * rh + 8 * q4 + 4 * hi;
        const f32x4 l4 = *reinterpret_cast<const lds_f32x4*>(lse2s + rl0);
        const f32x4 d4 = *reinterpret_cast<const lds_f32x4*>(Ds + rl0);
        if (all_ok) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            p_and_ds<CAP>(p, true, s[4 * q4 + j], l4[j], dp[4 * q4 + j], d4[j], &pv[4 * q4 + j], &dsv[4 * q4 + j]);
        } else {
          const i32x4 s4 = *reinterpret_cast<const lds_i32x4*>(segqs + rl0);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int row = row0 + rl0 + j;
            const bool ok = (row >= rlo) & (row <= rhi) & (s4[j] == kseg);  // ids 0 without segments
            p_and_ds<CAP>(p, ok, s[4 * q4 + j], l4[j], dp[4 * q4 + j], d4[j], &pv[4 * q4 + j], &dsv[4 * q4 + j]);
          }
        }
      }
      // P and dS of these 32 rows as bf16 A operands (two k-steps of 16 rows
      // each).  The dV wave keeps P and hands dS to the dK wave of its keys;
      // the dK wave keeps dS and hands P over.
      bf16x8 pa[2], da[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pa[ks][j] = (__bf16)pv[8 * ks + j];
          da[ks][j] = (__bf16)dsv[8 * ks + j];
        }
      const bf16x8 keep0 = dkw ? da[0] : pa[0], keep1 = dkw ? da[1] : pa[1];
      xme[0] = __builtin_bit_cast(u32x4, dkw ? pa[0] : da[0]);
      xme[64] = __builtin_bit_cast(u32x4, dkw ? pa[1] : da[1]);
      __syncthreads();
      const bf16x8 got0 = __builtin_bit_cast(bf16x8, xpart[0]);
      const bf16x8 got1 = __builtin_bit_cast(bf16x8, xpart[64]);
      // dV += P^T dO (dV waves) or dK += dS^T Q (dK waves) over the 64 rows:
      // k-steps 0, 1 on this wave's rows, 2, 3 on the partner's, NT tiles each;
      // the B operand rows are read transposed from the Q or dO tile (layout LB).
      auto accumulate = [&](auto nt_, auto lay_, const lds_u16* src) __attribute__((always_inline)) {
        constexpr int NT = decltype(nt_)::value;
        using LB = decltype(lay_);
        pipelined<4 * NT, 1>(
            [&](int i) {
              const int ks = i / NT;
              const int rr = 32 * (ks < 2 ? rh : rh ^ 1) + 16 * (ks & 1) + trow;
              const int col = 32 * (i % NT) + tcol;
              return ld_tr(src + LB::at(rr, col), src + LB::at(rr + 8, col));
            },
            [&](int i, const bf16x8& bo) {
              const int ks = i / NT;
              const bf16x8 a = ks == 0 ? keep0 : ks == 1 ? keep1 : ks == 2 ? got0 : got1;
              acc[i % NT] = mfma(a, bo, acc[i % NT]);
            });
      };
      if constexpr (DQK == DV) {
        accumulate(std::integral_constant<int, NQ>{}, LQ{}, dkw ? Qs : Os);
      } else if (dkw) {
        accumulate(std::integral_constant<int, NQ>{}, LQ{}, Qs);
      } else {
        accumulate(std::integral_constant<int, NV>{}, LV{}, Os);
      }
    }

    // Each wave writes its 32 keys: dK (times the scale, D = DQK) or dV (D = DV).
    auto write = [&](auto d_, float* outg, float osc) __attribute__((always_inline)) {
      constexpr int D = decltype(d_)::value;
      outg += (int64_t)bk * p.Lkv * D;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = key0 + 32 * kh + 8 * (e / 4) + 4 * hi + (e % 4);
        if (key < p.Lkv) {
#pragma unroll
          for (int t = 0; t < D / 32; ++t) outg[(int64_t)key * D + 32 * t + l32] = osc * acc[t][e];
        }
      }
    };
    if constexpr (DQK == DV) {
      write(std::integral_constant<int, DQK>{}, dkw ? p.dk : p.dv, dkw ? p.scale : 1.0f);
    } else if (dkw) {
      write(std::integral_constant<int, DQK>{}, p.dk, p.scale);
    } else {
      write(std::integral_constant<int, DV>{}, p.dv, 1.0f);
    }

  };
  if constexpr (DQK == DV)
    body(std::integral_constant<int, 0>{});
  else if (dk_wave)
    body(std::integral_constant<int, 1>{});
  else
    body(std::integral_constant<int, 2>{});
}

template <int DQK, int DV>
struct DqLds {
  // Q rows of 192-wide heads wait in LDS rather than in registers, which
  // cannot hold them next to dO and the dQ accumulators at 8 waves per CU.
  static constexpr bool Q_IN_LDS = DQK > 128;
  static constexpr int RK = Lay<DQK, true>::ROW;
  static constexpr int RV = Lay<DV, true>::ROW;
  // One buffer of a kv block: K, V and key segment ids (offsets inside it).
  static constexpr int K_OFF = 0;                      // K [64][RK]
  static constexpr int V_OFF = K_OFF + 64 * RK * 2;    // V [64][RV]
  static constexpr int SEG_OFF = V_OFF + 64 * RV * 2;  // key segment ids [64]
  static constexpr int BUF = SEG_OFF + 64 * 4;
  // Two buffers where they fit beside Q (heads up to 128 wide): block x+1 is
  // stored while no wave reads its buffer any more, so one barrier per block
  // orders both the reuse and the visibility.
  static constexpr int NBUF = Q_IN_LDS ? 1 : 2;
  static constexpr int Q_OFF = NBUF * BUF;             // Q [BQ][RK] when Q_IN_LDS
  static constexpr int BYTES = Q_OFF + (Q_IN_LDS ? BQ * RK * 2 : 0);
  static_assert(BYTES <= 163840, "fits the LDS of a CU");
};

template <int DQK, int DV, bool CAP>
__global__ __launch_bounds__(512) void bwd_dq_kernel(BwdParams p) {
  using M = DqLds<DQK, DV>;
  using LQ = Lay<DQK, true>;
  using LV = Lay<DV, true>;
  constexpr int NQ = DQK / 32;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  lds_u8* lds = (lds_u8*)smem;
  lds_u16* Qs = (lds_u16*)(lds + M::Q_OFF);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int trow = 4 * hi + ((lane & 15) >> 2);  // transposed-read address (see the dk/dv kernel)
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  int r, head;  // q block, b * Hq + h
  xcd_map_ranked(blockIdx.x, p.B * p.Hq, p.n_q_blocks, &head, &r);
  if (p.row_order) r = p.row_order[r];
  const int b = head / p.Hq;
  const int h = head - b * p.Hq;
  const int bk = b * p.Hkv + h / p.group;
  const int qi = r * BQ + 32 * wave + l32;  // this lane's row
  const bool in = qi < p.L;

  const uint16_t* qg = static_cast<const uint16_t*>(p.q) + (int64_t)head * p.L * DQK;
  const uint16_t* og = static_cast<const uint16_t*>(p.dout) + (int64_t)head * p.L * DV;
  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + (int64_t)bk * p.Lkv * DQK;
  const uint16_t* vg = static_cast<const uint16_t*>(p.v) + (int64_t)bk * p.Lkv * DV;

  // Q and dO of this lane's row as B operands: k-step s -> elements 16s + 8hi .. + 7.
  // With Q in LDS each lane stores the chunks it reads back later (row
  // 32 wave + l32, chunks 2s + hi), so no barrier orders them.
  constexpr bool QL = M::Q_IN_LDS;
  bf16x8 qf[QL ? 1 : DQK / 16], df[DV / 16];
#pragma unroll
  for (int st = 0; st < DQK / 16; ++st) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (in) v = *reinterpret_cast<const u32x4*>(qg + (int64_t)qi * DQK + 16 * st + 8 * hi);
    if constexpr (QL)
      *reinterpret_cast<lds_u32x4*>(Qs + LQ::off(32 * wave + l32, 2 * st + hi)) = v;
    else
      qf[st] = __builtin_bit_cast(bf16x8, v);
  }
#pragma unroll
  for (int st = 0; st < DV / 16; ++st) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (in) v = *reinterpret_cast<const u32x4*>(og + (int64_t)qi * DV + 16 * st + 8 * hi);
    df[st] = __builtin_bit_cast(bf16x8, v);
  }
  const float lse2 = in ? p.lse[(int64_t)head * p.L + qi] * kLog2e : INFINITY;
  // D_i = do_i . o_i: each lane holds half of its row's do (above) and reads
  // the same half of o; the two halves meet across the half-waves.  Written
  // for the dk/dv kernel, which runs after this one.
  float dlt;
  {
    const uint16_t* ogr = static_cast<const uint16_t*>(p.o) + (int64_t)head * p.L * DV;
    float acc = 0.0f;
#pragma unroll
    for (int st = 0; st < DV / 16; ++st) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (in) v = *reinterpret_cast<const u32x4*>(ogr + (int64_t)qi * DV + 16 * st + 8 * hi);
      const u32x4 d = __builtin_bit_cast(u32x4, df[st]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = fmaf(__uint_as_float(d[j] << 16), __uint_as_float(v[j] << 16), acc);
        acc = fmaf(__uint_as_float(d[j] & 0xffff0000u), __uint_as_float(v[j] & 0xffff0000u), acc);
      }
    }
    dlt = acc + __shfl_xor(acc, 32);
    if (in && hi == 0) p.delta[(int64_t)head * p.L + qi] = dlt;
  }
  const bool has_seg = p.seg_q != nullptr;
  const int qseg = (has_seg && in) ? p.seg_q[(int64_t)b * p.L + qi] : 0;
  // The wave's 32 rows in one segment (its id qseg0); see the dk/dv kernel.
  const int qseg0 = __builtin_amdgcn_readfirstlane(qseg);
  const bool qseg_one = !has_seg || all_equal(qseg, qseg0);
  const int32_t* segk = has_seg ? (p.seg_kv ? p.seg_kv + (int64_t)b * p.Lkv : p.seg_q + (int64_t)b * p.L) : nullptr;
  // Keys allowed to this lane's row by position (before segment ids).
  const int qpos = p.q_off + qi;
  int klo = 0, khi = in ? p.Lkv - 1 : -1;
  if (p.causal) khi = min(khi, qpos);
  if (p.window_left >= 0) klo = max(klo, qpos - p.window_left);
  if (p.window_right >= 0) khi = min(khi, qpos + p.window_right);

  f32x16 dqacc[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) dqacc[i] = f32x16{};

  const int x0 = p.row_ptr[r];
  const int x1 = p.row_ptr[r + 1];
  // The next block's K, V and key segment ids are fetched into registers
  // while the current one is computed.
  TileRegs<DQK, 512, true> k_next;
  TileRegs<DV, 512, true> v_next;
  int seg_next = 0;
  const __amdgpu_buffer_rsrc_t k_rs = buffer_rsrc(kg, (uint32_t)p.Lkv * DQK * 2);
  const __amdgpu_buffer_rsrc_t v_rs = buffer_rsrc(vg, (uint32_t)p.Lkv * DV * 2);
  auto fetch = [&](int x) __attribute__((always_inline)) {
    const int key0 = p.active_cols[x] * BK;
    k_next.fetch(k_rs, key0, tid);
    v_next.fetch(v_rs, key0, tid);
    if (tid < BK) seg_next = (has_seg && key0 + tid < p.Lkv) ? segk[key0 + tid] : 0;
  };
  auto store_next = [&](int buf) __attribute__((always_inline)) {
    k_next.store((lds_u16*)(lds + buf * M::BUF + M::K_OFF), tid);
    v_next.store((lds_u16*)(lds + buf * M::BUF + M::V_OFF), tid);
    if (tid < BK) ((lds_i32*)(lds + buf * M::BUF + M::SEG_OFF))[tid] = seg_next;
  };
  constexpr bool DB = M::NBUF == 2;
  if (x0 < x1) fetch(x0);
  if constexpr (DB) {
    // Double buffering: block x+1 goes into the buffer of block x-1, which
    // every wave finished reading before the barrier that closed block x-1;
    // the barrier that closes block x makes it visible.
    if (x0 < x1) {
      store_next(0);
      if (x0 + 1 < x1) fetch(x0 + 1);
    }
    __syncthreads();
  }
  for (int x = x0; x < x1; ++x) {
    const int key0 = p.active_cols[x] * BK;
    const int cur = DB ? (x - x0) & 1 : 0;
    if constexpr (!DB) {
      __syncthreads();  // the previous block is consumed
      store_next(0);
      __syncthreads();
      if (x + 1 < x1) fetch(x + 1);
    }
    const lds_u16* Ks = (const lds_u16*)(lds + cur * M::BUF + M::K_OFF);
    const lds_u16* Vs = (const lds_u16*)(lds + cur * M::BUF + M::V_OFF);
    const lds_i32* segks = (const lds_i32*)(lds + cur * M::BUF + M::SEG_OFF);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // S^T = K Q^T and dP^T = V dO^T (interleaved chains): keys 32t + items, row l32.
      f32x16 s = f32x16{}, dp = f32x16{};
      // S takes DQK / 16 k-steps, dP DV / 16.
      pipelined<(DQK > DV ? DQK : DV) / 16, 1>(
          [&](int st) {
            Op4 o{};
            if (st < DQK / 16) o.a = ld_op(Ks + LQ::off(32 * t + l32, 2 * st + hi));
            if (st < DV / 16) o.b = ld_op(Vs + LV::off(32 * t + l32, 2 * st + hi));
            if (QL && st < DQK / 16) o.c = ld_op(Qs + LQ::off(32 * wave + l32, 2 * st + hi));
            return o;
          },
          [&](int st, const Op4& o) {
            if (st < DQK / 16) s = mfma(o.a, QL ? o.c : qf[QL || st >= DQK / 16 ? 0 : st], s);
            if (st < DV / 16) dp = mfma(o.b, df[st < DV / 16 ? st : 0], dp);
          });
      // Keys 32 t + 8 (e / 4) + 4 hi + e % 4 of this lane's row: four runs of
      // 4.  Segment ids are 0 on both sides without segments.
      float pv[16], dsv[16];
      const bool all_ok = pos_allowed(p, r * BQ + 32 * wave, 32, key0 + 32 * t, 32) &&
                          (!has_seg || (qseg_one && all_equal(segks[32 * t + l32], qseg0)));  // wave-uniform
      if (all_ok) {
#pragma unroll
        for (int e = 0; e < 16; ++e) p_and_ds<CAP>(p, true, s[e], lse2, dp[e], dlt, &pv[e], &dsv[e]);
      } else {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int kl0 = 32 * t + 8 * q4 + 4 * hi;
          const i32x4 s4 = *reinterpret_cast<const lds_i32x4*>(segks + kl0);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int e = 4 * q4 + j;
            const int key = key0 + kl0 + j;
            const bool ok = (key >= klo) & (key <= khi) & (s4[j] == qseg);
            p_and_ds<CAP>(p, ok, s[e], lse2, dp[e], dlt, &pv[e], &dsv[e]);
          }
        }
      }
      // dQ += dS K over this tile's 32 keys: two k-steps of NQ tiles.
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 da8;
#pragma unroll
        for (int j = 0; j < 8; ++j) da8[j] = (__bf16)dsv[8 * ks + j];
        pipelined<NQ, 2>(
            [&](int dt) {
              const int kr = 32 * t + 16 * ks + trow;
              return ld_tr(Ks + LQ::at(kr, 32 * dt + tcol), Ks + LQ::at(kr + 8, 32 * dt + tcol));
            },
            [&](int dt, const bf16x8& b) { dqacc[dt] = mfma(da8, b, dqacc[dt]); });
      }
    }
    if constexpr (DB) {
      if (x + 1 < x1) {
        store_next(cur ^ 1);
        if (x + 2 < x1) fetch(x + 2);
      }
      __syncthreads();
    }
  }

  // dq rows 32 wave + items, columns 32 dt + l32.
  float* dqg = p.dq + (int64_t)head * p.L * DQK;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int row = r * BQ + 32 * wave + 8 * (e / 4) + 4 * hi + (e % 4);
    if (row < p.L) {
#pragma unroll
      for (int t = 0; t < NQ; ++t) dqg[(int64_t)row * DQK + 32 * t + l32] = p.scale * dqacc[t][e];
    }
  }
}

template <int DQK, int DV, bool CAP>
hipError_t launch_all(const BwdParams& p, hipStream_t s) {
  // dq first: it also writes D_i (p.delta), which the dk/dv kernel reads.
  const int64_t n_q_items = (int64_t)p.B * p.Hq * p.n_q_blocks;
  if (n_q_items > 0) {
    constexpr int bytes = DqLds<DQK, DV>::BYTES;
    auto fn = bwd_dq_kernel<DQK, DV, CAP>;
    if (bytes > 65536) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3((unsigned)n_q_items), dim3(512), bytes, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t n_kv_items = (int64_t)p.B * p.Hkv * p.n_kv_blocks;
  if (n_kv_items > 0) {
    const int bytes = DkdvLds<DQK, DV>::BYTES;
    auto fn = bwd_dkdv_kernel<DQK, DV, CAP>;
    if (bytes > 65536) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3((unsigned)n_kv_items), dim3(256), bytes, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int DQK, int DV>
hipError_t launch_cap(const BwdParams& p, hipStream_t s) {
  return p.soft_cap > 0.0f ? launch_all<DQK, DV, true>(p, s) : launch_all<DQK, DV, false>(p, s);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, int d_qk, int d_v, hipStream_t s) {
  if (d_qk == 128 && d_v == 128) return launch_cap<128, 128>(p, s);
  if (d_qk == 64 && d_v == 64) return launch_cap<64, 64>(p, s);
  if (d_qk == 192 && d_v == 128) return launch_cap<192, 128>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace splash
