// bf16 block-sparse attention forward for gfx950 on MFMA: the kernel and
// launch templates, instantiated by splash_fwd_bf16*.hip (one file per group
// of head dims, so the instances compile in parallel).
//
// Method ("Lecture 13 - Pallas Kernels and Splash Attention", CMU 11-868
// notes): every query row keeps a running max m, a running sum l and an
// un-normalised output o (section 5.2).  Per kv block the scores are computed,
// soft-capped and masked (5.2, 5.4), l and o are rescaled by
// alpha = e^(m_old - m_new) when the max moves, the block's e^(s - m) and its
// weighted V rows are added (5.1), and o is divided by l once after the last
// block (deferred normalisation, 5.2).  Only the active blocks of the
// execution table are visited; a partial block gets an element mask, a full
// block none (6.1-6.3).  The residual lse = m + ln l is written with o (joto.ai
// page, "LSE and online softmax").
//
// gfx950 design (this file's own; the pages' TPU kernel is prior art):
//   * One work-group = 8 waves = a 256-query block of one head; each wave owns
//     32 query rows.  Registers stay within 256 per lane, so the work-group
//     fills a CU with two waves per SIMD (waves w and w + 4 share a SIMD).
//     Every K/V tile copied into LDS serves 256 queries.
//   * Ping-pong schedule (default loop): waves 0-3 and 4-7 form two groups
//     with one wave per SIMD each.  They alternate, half a block apart,
//     between a matrix phase (O += P V of the previous block, S = Q K^T of
//     this one) and a softmax phase, so on every SIMD one wave feeds the matrix pipe
//     while the other uses the vector unit (section 5.3: the vector work must
//     hide behind the matrix work).  On gfx950 a matrix-only wave and a
//     vector-only wave overlap almost perfectly, while one wave mixing both
//     does not.
//   * The work-group walks its row's active blocks (CSR list), 64 keys per
//     block.  Scores are computed transposed, S^T = K Q^T, on
//     v_mfma_f32_32x32x16_bf16 as two 32-key tiles (two independent
//     accumulation chains): each lane holds one query and 16 keys per tile, so
//     row max / row sum are in-lane reductions plus one half-wave exchange
//     (v_permlane32_swap).
//   * O^T = V^T P^T on the same MFMA.  P never leaves registers (5.3): the
//     S^T accumulator items are the B operand after bf16 conversion, and the
//     V^T A operand is read from row-major V in LDS with ds_read_b64_tr_b16,
//     which returns four consecutive keys of one head dim per lane - the key
//     grouping the accumulator layout implies.
//   * K/V tiles stream HBM -> LDS with buffer_load ... lds (rows past the
//     sequence end read as zero) into double buffers (section 3.1).  LDS rows
//     are XOR-swizzled in 16-byte chunks so that both the K operand reads and
//     the transposing V reads are bank-conflict free at 256 bytes per clock.
//   * exp is the hardware exp2 with log2(e) folded into the scale (6.6
//     "use_base2_exp").  The reference max used in the exponent only moves
//     when a row's block max exceeds it by more than 2^8; the constant cancels
//     in o / l (section 5.4: any constant that keeps exp in range gives the
//     same softmax), so almost every block skips the O rescale, and P is
//     computed with the current reference while the block max is reduced.

#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include <stdint.h>
#include <stdlib.h>

#include "fwd_params.h"

namespace splash {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;      // log2 of the largest p allowed before a rescale
constexpr float kPsum = 256.0f;   // 2^kTau
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit dwords

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Tile geometry of one instance: BN keys per kv block (64 or 128).
template <int DQK, int DV, int BN>
struct Cfg {
  static constexpr int KS = DQK / 16;          // MFMA k-steps for S^T
  static constexpr int DT = DV / 32;           // O^T row tiles
  static constexpr int KROW = DQK * 2;         // bytes per K row in LDS
  static constexpr int VROW = DV * 2;          // bytes per V row in LDS
  static constexpr int KTILE = BN * KROW;      // bytes per K tile
  static constexpr int VTILE = BN * VROW;      // bytes per V tile
  static constexpr int KCHUNKS = KTILE / 16;   // 16-byte chunks per K tile
  static constexpr int VCHUNKS = VTILE / 16;
  static constexpr int NBUF = 2;               // tile buffers per operand
  static constexpr int SEG_OFF = NBUF * (KTILE + VTILE);  // key segment-id ring
  static constexpr int SEG_SLOTS = 3;          // ids of one block per slot
  static constexpr int LDS_BYTES = SEG_OFF + SEG_SLOTS * BN * 4;
  static_assert(LDS_BYTES <= 163840, "fits the LDS of a CU");
};

// Physical 16-byte chunk of logical chunk c in LDS row r (an involution
// that stays inside the row).  The gfx950 LDS serves 256 bytes (64 banks)
// per clock: a ds_read_b128 takes 16 lanes per clock, which read 16
// consecutive K rows at one logical chunk, and a ds_read_b64_tr_b16 takes
// 32 lanes, which read 64 bytes from each of 4 consecutive V rows.  The XOR
// spreads each of those groups over all 64 banks:
//   K, 256-byte rows: chunk ^ (r & 15);   K, 128/384-byte rows: rows pair up
//   in bank halves, chunk ^ ((r >> 1) & 7);
//   V, 256-byte rows: 64-byte group ^ (r & 3);  V, 128-byte rows: chunk ^ 2(r & 3).
template <int ROWB>
__device__ __forceinline__ int kswz(int r, int c) {
  static_assert(ROWB % 128 == 0 && ROWB >= 128, "K rows are 128-byte multiples");
  if constexpr (ROWB % 256 == 0)
    return c ^ (r & 15);
  else
    return c ^ ((r >> 1) & 7);
}
template <int ROWB>
__device__ __forceinline__ int vswz(int r, int c) {
  static_assert(ROWB == 128 || ROWB == 256, "V rows are 128 or 256 bytes");
  if constexpr (ROWB == 256)
    return c ^ (4 * (r & 3));
  else
    return c ^ (2 * (r & 3));
}

// Compile-time register-buffer index (keeps the double-buffered accumulator
// arrays statically indexed).
template <int N>
struct Idx {
  static constexpr int value = N;
};

// Fully unrolled loop with a compile-time index: f(Idx<I>{}) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void sfor(F&& f) {
  if constexpr (B < E) {
    f(Idx<B>{});
    sfor<B + 1, E>(f);
  }
}
#define SIDX(tag) decltype(tag)::value

// One 16-byte-per-lane HBM -> LDS copy: lane i's 16 bytes at byte offset
// voff of the buffer land at LDS address lds_addr + 16 i.  Issued as inline
// assembly so that the compiler does not treat later LDS reads of *other*
// buffers as dependent on it; completion is tracked explicitly with vmcnt.
// M0 (the LDS base of the copy) is set here and declared clobbered.  clang
// warns that it does not preserve a clobbered M0 for its own uses; these
// kernels make none (a CPU test scans the generated code: M0 is written
// only right before these copies), so the warning is silenced here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t lds_addr, int voff) {
  const uint32_t base = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr);
  const u32x4 rs = {(uint32_t)__builtin_amdgcn_readfirstlane(rsrc[0]),
                    (uint32_t)__builtin_amdgcn_readfirstlane(rsrc[1]),
                    (uint32_t)__builtin_amdgcn_readfirstlane(rsrc[2]),
                    (uint32_t)__builtin_amdgcn_readfirstlane(rsrc[3])};
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(base), "v"(voff), "s"(rs)
      : "memory", "m0");
}

// One 4-byte-per-lane HBM -> LDS copy (lane i's dword lands at
// lds_addr + 4 i); otherwise as dma16.
__device__ __forceinline__ void dma4(u32x4 rsrc, uint32_t lds_addr, int voff) {
  const uint32_t base = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr);
  const u32x4 rs = {(uint32_t)__builtin_amdgcn_readfirstlane(rsrc[0]),
                    (uint32_t)__builtin_amdgcn_readfirstlane(rsrc[1]),
                    (uint32_t)__builtin_amdgcn_readfirstlane(rsrc[2]),
                    (uint32_t)__builtin_amdgcn_readfirstlane(rsrc[3])};
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(base), "v"(voff), "s"(rs)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N tile copies of this wave are in flight and all LDS
// reads are done, then synchronise the work-group.
template <int N>
__device__ __forceinline__ void wait_copies_and_barrier() {
  static_assert(N >= 0 && N <= 63, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Read-only table entry through the constant address space: with a
// wave-uniform index this is a scalar load (lgkmcnt, not vmcnt).
template <typename T>
__device__ __forceinline__ T ld_table(const T* base, int i) {
  return ((const __attribute__((address_space(4))) T*)base)[__builtin_amdgcn_readfirstlane(i)];
}

// The value of lane 0 in every lane, held in scalar registers.
__device__ __forceinline__ u32x4 uniform(u32x4 v) {
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)v[0]), (uint32_t)__builtin_amdgcn_readfirstlane((int)v[1]),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)v[2]), (uint32_t)__builtin_amdgcn_readfirstlane((int)v[3])};
}

__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32), bytes, (uint32_t)kRsrcWord3};
}

// Issue order of the matrix phase.  Score MFMA x (of NQ) is k-step
// x / NTILE of 32-key tile x % NTILE; O MFMA x (of NP) is key group
// x / DT of head-dim tile x % DT.
//   Two score tiles (64-key blocks): O and score MFMAs alternate, score
//   first, so consecutive MFMAs never feed the same accumulator; the longer
//   list finishes the sequence.
//   Four score tiles (128-key blocks): the O MFMAs, which read P of the
//   previous block, are interleaved evenly with the scores of tiles 2 and 3;
//   the scores of tiles 0 and 1 follow once P is consumed, so they can reuse
//   its registers (two independent accumulation chains keep the matrix pipe
//   at full rate).
template <int NP, int NQ, int NTILE>
struct MatOrder {
  static_assert(NTILE == 2 || NTILE == 4, "64- or 128-key blocks");
  static constexpr int N = NP + NQ;
  static constexpr int NMIN = NP < NQ ? NP : NQ;
  static constexpr bool kSplit = NTILE == 4 && NP > 0 && NQ > 0;
  static constexpr int SA = NQ / 2;        // scores of tiles 2, 3 (split order)
  static constexpr int A = NP + SA;        // length of the interleaved part
  // Position m of the interleaved part holds a score iff the count of scores
  // placed so far steps up at m.
  static constexpr int s_before(int m) { return m * SA / A; }
  static constexpr bool is_s(int m) {
    if constexpr (kSplit)
      return m >= A || s_before(m + 1) > s_before(m);
    else if constexpr (NTILE == 2)
      return m < 2 * NMIN ? (m % 2 == 0) : (NQ > NP);
    else
      return NQ > 0;
  }
  static constexpr int idx(int m) {
    if constexpr (kSplit) {
      if (m >= A) {  // tiles 0, 1 in k-step order
        const int j = m - A;
        return (j / 2) * NTILE + (j % 2);
      }
      if (!is_s(m)) return m - s_before(m);
      const int j = s_before(m);   // tiles 2, 3 in k-step order
      return (j / 2) * NTILE + 2 + (j % 2);
    } else if constexpr (NTILE == 2) {
      return m < 2 * NMIN ? m / 2 : NMIN + (m - 2 * NMIN);
    } else {
      return m;
    }
  }
};

// Reduction of N values with a three-input operation f (maximum or minimum)
// as a tree: groups of three, then of the group results, and so on.
template <int N, typename F>
__device__ __forceinline__ float tree3(const float* v, F f) {
  if constexpr (N == 1) {
    return v[0];
  } else {
    constexpr int M = (N + 2) / 3;
    float w[M];
    sfor<0, M>([&](auto j_) {
      constexpr int j = SIDX(j_);
      if constexpr (3 * j + 2 < N)
        w[j] = f(v[3 * j], v[3 * j + 1], v[3 * j + 2]);
      else if constexpr (3 * j + 1 < N)
        w[j] = f(v[3 * j], v[3 * j + 1], v[3 * j + 1]);
      else
        w[j] = v[3 * j];
    });
    return tree3<M>(w, f);
  }
}

// Wait for this wave's LDS reads, then synchronise the work-group.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One item: the 32 NW query rows of q-block row r of query head `head`
// (flattened b * Hq + h), over chunk `split` of the row's active kv blocks
// (the whole row when there is no split).
template <int DQK, int DV, int BN, int NW, bool CAP, bool SPLIT, bool PACK>
__device__ __forceinline__ void item_fwd(const FwdParams& p, int head, int r, int split) {
  using C = Cfg<DQK, DV, BN>;
  constexpr int BM = 32 * NW;       // query rows per item: 32 per wave
  constexpr int NTILE = BN / 32;    // 32-key score tiles per block
  constexpr int KS = C::KS;
  constexpr int DT = C::DT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  lds_u8* lds = (lds_u8*)smem;  // address-space cast to LDS
  // Layout: [K buf 0, 1][V buf 0, 1]; block x lives in buffer x % 2.
  auto kbuf = [&](int i) { return lds + i * C::KTILE; };
  auto vbuf = [&](int i) { return lds + C::NBUF * C::KTILE + i * C::VTILE; };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int b = head / p.Hq;
  const int hq = head - b * p.Hq;
  const int kvh = b * p.Hkv + hq / p.group;
  const int L = p.L;      // query rows
  const int Lk = p.Lkv;   // key positions
  const int qw = r * BM + wave * 32;  // first query row of this wave
  const int qi = qw + l32;            // this lane's query row
  // Position of the row inside its query head (packed GQA rows repeat with
  // the period) and its key position for the causal and window tests.
  const int qrow = PACK ? qi % p.row_period : qi;
  const int qp = p.q_off + qrow;

  const uint16_t* qg = static_cast<const uint16_t*>(p.q) + (int64_t)head * L * DQK;
  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + (int64_t)kvh * Lk * DQK;
  const uint16_t* vg = static_cast<const uint16_t*>(p.v) + (int64_t)kvh * Lk * DV;
  // Buffer resources: reads past the sequence end return zero.
  const uint64_t qaddr = reinterpret_cast<uint64_t>(qg);
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(qaddr >> 32)) << 32) |
              (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)qaddr)),
      (short)0, __builtin_amdgcn_readfirstlane(L * DQK * 2), kRsrcWord3);
  const u32x4 krs = uniform(make_rsrc(kg, (uint32_t)(Lk * DQK * 2)));
  const u32x4 vrs = uniform(make_rsrc(vg, (uint32_t)(Lk * DV * 2)));

  // No LDS initialisation: every tile copy covers its whole tile (rows past
  // the sequence end read as zero through the buffer range check) and the
  // segment-id ring is only read where it was copied.  Without a barrier
  // here the Q loads below and the first tile copies are in flight together.

  // Q^T as B operands: k-step s -> Q[qi][16s + 8hi + 0..7].
  bf16x8 qf[KS];
  sfor<0, KS>([&](auto s_) {
    constexpr int s = SIDX(s_);
    const int off = (qi * DQK + 16 * s + 8 * hi) * 2;
    qf[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
  });

  // Softmax state (z in log2 units after multiplying by zc):
  //   no cap: z = q.k, zc = scale log2(e);  cap: z = log2(e) cap tanh(scale q.k / cap), zc = 1.
  // With the cap the score registers hold u = 1 / (e^{2y} + 1), y = scale q.k / cap,
  // from which z = A - 2A u (A = log2(e) cap) is folded into later
  // multiply-adds; z is decreasing in u, so a masked pair holds u = +inf.
  const float zc = CAP ? 1.0f : p.scale_log2;
  constexpr float kMasked = CAP ? INFINITY : -INFINITY;
  // Reference max (z units).  With the max logit estimate (section 5.4) it
  // is the given constant and never moves: no max reduction, no rescale.
  const bool mle = p.mle != 0;
  float mref = mle ? p.mle_log2 / zc : -INFINITY;
  float lsum = 0.0f;
  f32x16 oacc[DT];
  sfor<0, DT>([&](auto i_) { oacc[SIDX(i_)] = f32x16{}; });

  const bool has_seg = p.seg_q != nullptr;
  const int32_t* segq = has_seg ? p.seg_q + (int64_t)b * (PACK ? p.Lseg : L) : nullptr;
  const int32_t* segk = has_seg ? (p.seg_kv ? p.seg_kv + (int64_t)b * Lk : segq) : nullptr;
  const int my_seg = (has_seg && qi < L) ? segq[qrow] : 0;
  // Allowed key interval of this lane's row before the segment test.
  int klo = 0, khi = Lk - 1;
  if (p.causal) khi = min(khi, qp);
  if (p.window_left >= 0) klo = max(klo, qp - p.window_left);
  if (p.window_right >= 0) khi = min(khi, qp + p.window_right);
  // Key positions bounding this wave's valid query rows (packed rows: the
  // whole period).
  const int qa = p.q_off + (PACK ? 0 : qw);
  const int qb = p.q_off + (PACK ? p.row_period - 1 : min(qw + 31, L - 1));

  // Blocks [row_ptr[r] + lo, row_ptr[r] + hi) of the active list: chunk
  // `split` of n_split near-equal contiguous chunks.
  const int tab_r = PACK ? 0 : r;  // table row of these query rows
  const int row0 = ld_table(p.row_ptr, tab_r);
  const int n_row = ld_table(p.row_ptr, tab_r + 1) - row0;
  const int lo = SPLIT ? (int)(((int64_t)n_row * split) / p.n_split) : 0;
  const int hi_blk = SPLIT ? (int)(((int64_t)n_row * (split + 1)) / p.n_split) : n_row;
  const int g0 = row0 + lo;
  const int n = hi_blk - lo;
  const int32_t* cols = p.active_cols + g0;
  auto colc = [&](int x) { return ld_table(cols, min(x, n - 1)); };

  // V^T transposed reads: lane j of 16-lane group G supplies key row
  // 32t + 16c2 + 8e4 + 4(G/2) + j/4 and dims 32dt + 16(G%2) + 4(j%4) .. +3;
  // lane 16G + i receives keys 32t + 16c2 + 8e4 + 4(G/2) + 0..3 of dim
  // 32dt + l32: items 4e4 .. 4e4+3 of the MFMA A operand for (t, c2).
  const int grp = lane >> 4;
  const int jj = lane & 15;
  const int vrow0 = 4 * (grp >> 1) + (jj >> 2);
  const int vcol0 = 2 * (grp & 1) + ((jj & 3) >> 1);

  // Element mask of a partial block for this wave: item E of tile t is key
  // k0 + 32t + 8(E/4) + 4hi + E%4 of query qi.
  auto apply_mask = [&](f32x16* sv, int pat, int c) __attribute__((always_inline)) {
    const int ka = c * BN;
    const int kz = ka + BN - 1;
    if (p.mask_stored) {
      // Pattern row = the row inside the table's q block (packed rows: the
      // row inside its query head, all of them in table row 0).
      const uint8_t* prow = p.patterns + (int64_t)pat * (BM * BN) +
                            (PACK ? qrow : wave * 32 + l32) * BN;
      sfor<0, 4 * NTILE>([&](auto i_) {
        constexpr int t = SIDX(i_) / 4;
        constexpr int q4 = SIDX(i_) % 4;
        const uint32_t bits = *reinterpret_cast<const uint32_t*>(prow + 32 * t + 8 * q4 + 4 * hi);
        sfor<0, 4>([&](auto e_) {
          constexpr int e = SIDX(e_);
          sv[t][4 * q4 + e] = ((bits >> (8 * e)) & 0xffu) ? sv[t][4 * q4 + e] : kMasked;
        });
      });
      return;
    }
    // Corner tests on this wave's rows: no element mask when all are allowed.
    const bool all = !has_seg && kz < Lk && (!p.causal || kz <= qa) &&
                     (p.window_left < 0 || qb - ka <= p.window_left) &&
                     (p.window_right < 0 || kz - qa <= p.window_right);
    if (all) return;
    if (has_seg) {
      sfor<0, 16 * NTILE>([&](auto i_) {
        constexpr int t = SIDX(i_) / 16;
        constexpr int i = SIDX(i_) % 16;
        const int key = ka + 32 * t + 8 * (i / 4) + 4 * hi + (i % 4);
        const bool ok = (key >= klo) & (key <= khi) & (segk[min(key, Lk - 1)] == my_seg);
        sv[t][i] = ok ? sv[t][i] : kMasked;
      });
    } else {
      // Key offset minus 4 hi against the shifted interval (constants on one side).
      const int base = ka + 4 * hi;
      const int lo = klo - base, up = khi - base;
      sfor<0, 16 * NTILE>([&](auto i_) {
        constexpr int t = SIDX(i_) / 16;
        constexpr int i = SIDX(i_) % 16;
        constexpr int r = 32 * t + 8 * (i / 4) + (i % 4);
        const bool ok = (r >= lo) & (r <= up);
        sv[t][i] = ok ? sv[t][i] : kMasked;
      });
    }
  };

  // ---------------------------------------------------------------------
  // Ping-pong loop.  Waves w and w + NW/2 run on the same SIMD, so waves
  // [0, NW/2) (group 0) and [NW/2, NW) (group 1) each hold one wave per SIMD.
  // Both groups run the same sequence MM(0) SM(0) MM(1) SM(1) ... MM(n), but
  // group 1 half a step later.  MM(i) is the matrix phase
  // (O += P_{i-1} V_{i-1} for i >= 1, S_i = Q K_i^T for i < n), SM(i) the
  // softmax phase (S_i -> P_i, l, lazy O rescale).  So in every half-step
  // one wave of each SIMD feeds the matrix pipe while the other works on the
  // vector unit:
  //   half-step 2i:     group 0 MM(i)      group 1 SM(i-1)
  //   half-step 2i+1:   group 0 SM(i)      group 1 MM(i)
  // The tiles of block i+2 (K) and i+1 (V) are copied in half-step 2i+2,
  // into the buffers of K_i and V_{i-1} (last read by MM(i) in half-steps 2i
  // and 2i+1), and MM(i+2) reads them from half-step 2i+4 (see run below for
  // which group issues them).
  auto pingpong_loop = [&]() __attribute__((always_inline)) {
    static_assert(NW % 2 == 0, "two wave groups");
    if (n == 0) return;
    constexpr int GW = NW / 2;               // waves per group
    const bool grp1 = wave >= GW;
    const int gw = wave - (grp1 ? GW : 0);   // wave index inside its group
    float mc = mle ? p.mle_log2 : 0.0f;  // reference exponent offset m zc (0 while m = -inf)
    float mthr = -INFINITY;       // m + kTau / zc: block maxima above it move m
    // A lane's partial row sum of p above it may mean a move: -1 until the
    // row has a reference (every block then checks), then 2^kTau.
    float psthr = -1.0f;

    // Key segment ids of a block, for the element mask of partial blocks,
    // are copied into an LDS ring (slot = block index mod 3) by one wave of
    // group 1 together with the block's K tile; the mask then reads them
    // with four-key LDS loads instead of one global load per key.
    const bool seg_lds = has_seg && !p.mask_stored;
    const u32x4 srs = uniform(make_rsrc(segk, (uint32_t)(has_seg ? Lk * 4 : 0)));
    auto segbuf = [&](int slot) { return lds + C::SEG_OFF + slot * (BN * 4); };
    auto seg_copy = [&](int c, int slot) __attribute__((always_inline)) {
      if (seg_lds && gw == 0) {
        sfor<0, BN / 64>([&](auto h_) {
          constexpr int h = SIDX(h_);
          dma4(srs, (uint32_t)(uintptr_t)(segbuf(slot) + 256 * h), (c * BN + 64 * h + lane) * 4);
        });
      }
    };
    // Element mask of a partial block with segments: item E of tile t is key
    // k0 + 32t + 8(E/4) + 4hi + E%4 of query qi.
    auto apply_mask_seg_lds = [&](f32x16* sv, int c, int slot) __attribute__((always_inline)) {
      // Key offset inside the block minus this half-wave's 4 hi, against the
      // lane's allowed interval shifted the same way: compile-time constants
      // on one side.
      const int base = c * BN + 4 * hi;
      const int lo = klo - base, up = khi - base;
      const lds_u8* st = segbuf(slot) + 16 * hi;
      sfor<0, 4 * NTILE>([&](auto j_) {
        constexpr int t = SIDX(j_) / 4;
        constexpr int q4 = SIDX(j_) % 4;
        const u32x4 ids = *reinterpret_cast<const lds_u32x4*>(st + (32 * t + 8 * q4) * 4);
        sfor<0, 4>([&](auto e_) {
          constexpr int e = SIDX(e_);
          constexpr int r = 32 * t + 8 * q4 + e;
          const bool ok = (r >= lo) & (r <= up) & ((int)ids[e] == my_seg);
          sv[t][4 * q4 + e] = ok ? sv[t][4 * q4 + e] : kMasked;
        });
      });
    };
    f32x16 sacc[NTILE];   // S^T of the current block: 32-key tiles
    bf16x8 pb[NTILE][2];  // P^T of the previous block: [key tile][key half]
    sfor<0, 2 * NTILE>([&](auto i_) { pb[SIDX(i_) / 2][SIDX(i_) % 2] = bf16x8{}; });

    // Tile copies split over the 4 waves of group 1.
    // HBM byte offset, inside a K (V) tile, of the 16-byte chunk that lane
    // `lane` moves in copy k of this wave: chunk slot = (k GW + gw) 64 + lane
    // of the tile, stored at its swizzled place.
    auto koff_in_tile = [&](int k) __attribute__((always_inline)) {
      const int slot = (k * GW + gw) * 64 + lane;
      const int row = slot / (DQK / 8);
      const int pc = slot - row * (DQK / 8);
      return (row * DQK + kswz<C::KROW>(row, pc) * 8) * 2;
    };
    auto voff_in_tile = [&](int k) __attribute__((always_inline)) {
      const int slot = (k * GW + gw) * 64 + lane;
      const int row = slot / (DV / 8);
      const int pc = slot - row * (DV / 8);
      return (row * DV + vswz<C::VROW>(row, pc) * 8) * 2;
    };
    // When the rows one copy spans are a multiple of the swizzle period (16
    // rows for K, 4 for V), a lane's chunk column is the same in every copy:
    // copy k's offset is the lane's offset of copy 0 plus a uniform step, so
    // one register per operand serves every copy.
    constexpr int KROWS = 64 % (DQK / 8) == 0 ? GW * 64 / (DQK / 8) : 0;   // rows per copy
    constexpr int VROWS = 64 % (DV / 8) == 0 ? GW * 64 / (DV / 8) : 0;
    constexpr bool KINV = KROWS > 0 && KROWS % 16 == 0;
    constexpr bool VINV = VROWS > 0 && VROWS % 4 == 0;
    const int koff0 = koff_in_tile(0);
    const int voff0 = voff_in_tile(0);
    // Offset of copy k of block c (the block part is uniform: a scalar, added
    // to the lane part in one vector add per copy).
    auto kcopy_off = [&](int k, int c) __attribute__((always_inline)) {
      const int su = __builtin_amdgcn_readfirstlane(c * (BN * DQK * 2) + (KINV ? k * KROWS * DQK * 2 : 0));
      return (KINV ? koff0 : koff_in_tile(k)) + su;
    };
    auto vcopy_off = [&](int k, int c) __attribute__((always_inline)) {
      const int su = __builtin_amdgcn_readfirstlane(c * (BN * DV * 2) + (VINV ? k * VROWS * DV * 2 : 0));
      return (VINV ? voff0 : voff_in_tile(k)) + su;
    };
    auto g1_load_k = [&](int c, int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < C::KCHUNKS / (64 * GW); ++t)
        dma16(krs, (uint32_t)(uintptr_t)(kbuf(buf) + (t * GW + gw) * 64 * 16), kcopy_off(t, c));
    };
    auto g1_load_v = [&](int c, int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < C::VCHUNKS / (64 * GW); ++t)
        dma16(vrs, (uint32_t)(uintptr_t)(vbuf(buf) + (t * GW + gw) * 64 * 16), vcopy_off(t, c));
    };
    static_assert(C::KCHUNKS % (64 * GW) == 0 && C::VCHUNKS % (64 * GW) == 0, "tile split");

    // Operand addresses.  With 256-byte rows the swizzle is an XOR of the
    // address bits below 256, so every read is one base register XOR a
    // constant (tiles and rows start at multiples of 256 bytes).
    auto kfrag = [&](const lds_u8* kb, int s, int t) __attribute__((always_inline)) {
      if constexpr (C::KROW % 256 == 0) {
        const uint32_t base = (uint32_t)(uintptr_t)kb + l32 * C::KROW + 16 * (hi ^ (l32 & 15));
        const uint32_t a = (base ^ (uint32_t)(32 * s)) + (uint32_t)(32 * t * C::KROW);
        return *reinterpret_cast<const lds_bf16x8*>((lds_u8*)(uintptr_t)a);
      } else {
        const int key = 32 * t + l32;
        return *reinterpret_cast<const lds_bf16x8*>(kb + key * C::KROW + kswz<C::KROW>(key, 2 * s + hi) * 16);
      }
    };
    auto vfrag = [&](const lds_u8* vb, int t, int c2, int dt) __attribute__((always_inline)) {
      const int row = 32 * t + 16 * c2 + vrow0;
      const int row2 = row + 8;
      i16x4 lo, up;
      if constexpr (C::VROW == 256) {
        // chunk 4dt + vcol0 of row r sits at chunk 4(dt ^ (r & 3)) + vcol0.
        const uint32_t base = (uint32_t)(uintptr_t)vb + vrow0 * C::VROW +
                              ((64 * (vrow0 & 3)) | (16 * vcol0) | (8 * (jj & 1)));
        const uint32_t a = (base ^ (uint32_t)(64 * dt)) + (uint32_t)((32 * t + 16 * c2) * C::VROW);
        lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a);
        up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(a + 8 * C::VROW));
      } else {
        const int lc = 4 * dt + vcol0;
        lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vb + row * C::VROW + vswz<C::VROW>(row, lc) * 16 + 8 * (jj & 1)));
        up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vb + row2 * C::VROW + vswz<C::VROW>(row2, lc) * 16 + 8 * (jj & 1)));
      }
      const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
      const u32x2 up2 = __builtin_bit_cast(u32x2, up);
      return __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], up2[0], up2[1]});
    };

    // One tile-copy instruction of a group's share: k < KL copies part of a
    // K tile (with the block's segment ids first), the rest part of a V tile.
    constexpr int KL = C::KCHUNKS / (64 * GW);
    constexpr int VL = C::VCHUNKS / (64 * GW);
    auto copy_part = [&](auto k_, int ck, int kbf, int cv, int vbf, int sslot) __attribute__((always_inline)) {
      constexpr int k = SIDX(k_);
      if constexpr (k == 0) seg_copy(ck, sslot);
      if constexpr (k < KL)
        dma16(krs, (uint32_t)(uintptr_t)(kbuf(kbf) + (k * GW + gw) * 64 * 16), kcopy_off(k, ck));
      else
        dma16(vrs, (uint32_t)(uintptr_t)(vbuf(vbf) + ((k - KL) * GW + gw) * 64 * 16), vcopy_off(k - KL, cv));
    };
    auto no_copy = [&](auto) __attribute__((always_inline)) {};

    // Matrix phase MM(i); the tags select the O product and the scores.
    // copy(Idx<k>) issues tile-copy instruction k of NCOPY, spread between
    // the MFMAs: issuing a copy holds the wave for tens of cycles, which the
    // matrix pipe spends on the MFMAs already issued.
    auto mm = [&](int i, auto pv_tag, auto sc_tag, auto copy, auto ncopy_tag) __attribute__((always_inline)) {
      constexpr int NP = SIDX(pv_tag) ? (BN / 16) * DT : 0;
      constexpr int NQ = SIDX(sc_tag) ? NTILE * KS : 0;
      constexpr int NCOPY = SIDX(ncopy_tag);
      using O = MatOrder<NP, NQ, NTILE>;
      // Operand reads run this many MFMAs ahead (fewer with 192-wide heads,
      // whose Q fragments leave fewer registers).  Each step below is fenced
      // with a scheduling barrier: left to itself the compiler sinks every LDS
      // read to just before its MFMA, which exposes the LDS latency on most
      // of the phase's MFMAs.
      constexpr int DIST = DQK > 128 ? 3 : (BN > 64 ? 4 : 6);
      const lds_u8* kb = kbuf(i & 1);         // K_i
      const lds_u8* vb = vbuf((i + 1) & 1);   // V_{i-1}
      bf16x8 opnd[O::N];
      auto read_opnd = [&](auto m_) __attribute__((always_inline)) {
        constexpr int m = SIDX(m_);
        constexpr int x = O::idx(m);
        if constexpr (O::is_s(m)) {
          opnd[m] = kfrag(kb, x / NTILE, x % NTILE);
        } else {
          constexpr int tc = x / DT;
          opnd[m] = vfrag(vb, tc / 2, tc % 2, x % DT);
        }
      };
      auto issue = [&](auto m_) __attribute__((always_inline)) {
        constexpr int m = SIDX(m_);
        if constexpr (m + DIST < O::N) read_opnd(Idx<m + DIST>{});
        constexpr int x = O::idx(m);
        if constexpr (O::is_s(m)) {
          constexpr int s = x / NTILE, t = x % NTILE;
          if constexpr (s == 0) {
            const f32x16 zero = {};
            sacc[t] = mfma(opnd[m], qf[0], zero);
          } else {
            sacc[t] = mfma(opnd[m], qf[s], sacc[t]);
          }
        } else {
          constexpr int tc = x / DT, dt = x % DT;
          oacc[dt] = mfma(opnd[m], pb[tc / 2][tc % 2], oacc[dt]);
        }
      };
      // The matrix wave wins the SIMD's issue arbitration over the softmax
      // wave sharing its SIMD, so its MFMAs and operand reads are not held
      // behind vector instructions (about 1.5% on dense causal).
      __builtin_amdgcn_s_setprio(3);
      sfor<0, (DIST < O::N ? DIST : O::N)>([&](auto m_) { read_opnd(m_); });
      sfor<0, O::N>([&](auto m_) __attribute__((always_inline)) {
        constexpr int m = SIDX(m_);
        issue(m_);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr ((m + 1) * NCOPY / O::N > m * NCOPY / O::N) {
          sfor<m * NCOPY / O::N, (m + 1) * NCOPY / O::N>(copy);
          __builtin_amdgcn_sched_barrier(0);
        }
      });
      __builtin_amdgcn_s_setprio(0);
      // The scores stay in this half-step (not sunk past the barrier).
      if constexpr (NQ > 0) {
        sfor<0, NTILE>([&](auto t_) {
          const f32x16 a = sacc[SIDX(t_)];
          asm volatile("" ::"v"(a));
        });
      }
    };

    // Softmax phase SM(i): S_i -> P_i (bf16), l, lazy reference and O rescale.
    // copy(Idx<k>) issues tile-copy instruction k of NCOPY; they are spread
    // between the exponentials so that the vector-memory queue drains while
    // the wave keeps computing.  With the lazy reference the exponent offset
    // almost never moves, so P is computed with the current offset while the
    // block max is reduced (a tree, in parallel); only when some row's max
    // passes its threshold does the wave move the reference and recompute.
    // Exponent of an item: z zc - mc, as one multiply-add (cap: (A - mc) - 2A u).
    const float capA = CAP ? p.soft_cap * kLog2e : 0.0f;
    const float ea = CAP ? -2.0f * capA : zc;
    auto exps = [&](f32x16* sv, float mcv, auto copy, auto ncopy_tag) __attribute__((always_inline)) {
      constexpr int NCOPY = SIDX(ncopy_tag);
      const float eb = CAP ? capA - mcv : -mcv;
      float ps[4];
      sfor<0, 2 * NTILE>([&](auto i_) {
        constexpr int t = SIDX(i_) / 2;
        constexpr int c2 = SIDX(i_) % 2;
        u32x4 w;
        sfor<0, 4>([&](auto e_) {
          constexpr int e2 = SIDX(e_);
          constexpr int q = 4 * SIDX(i_) + e2;   // pair index 0..15
          const float p0 = fast_exp2(fmaf(sv[t][8 * c2 + 2 * e2], ea, eb));
          const float p1 = fast_exp2(fmaf(sv[t][8 * c2 + 2 * e2 + 1], ea, eb));
          if constexpr (q < 4)
            ps[q] = p0 + p1;
          else
            ps[q & 3] += p0 + p1;
          w[e2] = pack_bf16(p0, p1);
          if constexpr ((q + 1) * NCOPY / (8 * NTILE) > q * NCOPY / (8 * NTILE)) {
            // Keep each copy at its place between the exponentials.
            __builtin_amdgcn_sched_barrier(0);
            sfor<q * NCOPY / (8 * NTILE), (q + 1) * NCOPY / (8 * NTILE)>(copy);
            __builtin_amdgcn_sched_barrier(0);
          }
        });
        pb[t][c2] = __builtin_bit_cast(bf16x8, w);
      });
      return (ps[0] + ps[1]) + (ps[2] + ps[3]);
    };
    // P values stay where they were computed (not sunk past a branch or barrier).
    auto keep_p = [&]() __attribute__((always_inline)) {
      sfor<0, 2 * NTILE>([&](auto j_) {
        const bf16x8 q = pb[SIDX(j_) / 2][SIDX(j_) % 2];
        asm volatile("" ::"v"(q));
      });
    };
    auto sm = [&](int i, int mn, int ci, auto copy, auto ncopy_tag) __attribute__((always_inline)) {
      f32x16* sv = sacc;
      if constexpr (CAP) {
        // z = log2(e) cap tanh(y), tanh y = 1 - 2 / (e^{2y} + 1): keep u = 1 / (e^{2y} + 1).
        const float k2 = 2.0f * kLog2e * p.scale / p.soft_cap;
        sfor<0, 16 * NTILE>([&](auto i_) {
          constexpr int t = SIDX(i_) / 16;
          constexpr int e = SIDX(i_) % 16;
          sv[t][e] = __builtin_amdgcn_rcpf(fast_exp2(sv[t][e] * k2) + 1.0f);
        });
      }
      // Partial block <=> it has a pattern (mask_next >= 0); after the cap,
      // which would map a masked -inf to -cap.
      if (mn >= 0) {
        if (seg_lds)
          apply_mask_seg_lds(sv, ci, i % 3);
        else
          apply_mask(sv, mn, ci);
      }
      float ps = exps(sv, mc, copy, ncopy_tag);
      {
        // Computed here, overlapping the max below (not sunk into its branch).
        keep_p();
        asm volatile("" ::"v"(ps));
      }
      // With the max logit estimate the reference is fixed: no max at all.
      // Otherwise the row max is needed only when some p of the block
      // exceeds 2^kTau, and then the lane's partial sum of its p (all >= 0)
      // does too: that one compare stands in for the max tree on almost every
      // block.  A sum above the bound without such a p only costs the tree.
      if (!mle && __any(ps > psthr)) {
        // Row max: a tree of three-input maxima over the lane's 16 NTILE scores
        // (32 -> 11 -> 4 -> 2 -> 1, 16 instructions for one 64-key block),
        // then the other half-wave; with the cap a tree of minima over u,
        // z = A - 2A min u.
        auto max3 = [](float a, float b, float c) __attribute__((always_inline)) {
          if constexpr (CAP)
            return __builtin_fminf(__builtin_fminf(a, b), c);
          else
            return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
        };
        float vals[16 * NTILE];
        sfor<0, 16 * NTILE>([&](auto k_) { vals[SIDX(k_)] = sv[SIDX(k_) / 16][SIDX(k_) % 16]; });
        float mx = tree3<16 * NTILE>(vals, max3);
        if constexpr (CAP) mx = fmaf(mx, -2.0f * capA, capA);
        {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
          mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        // Lazy reference: a row moves only when its block max exceeds the
        // reference by more than 2^kTau in the exponent (mthr = m + kTau / zc).
        if (__any(mx > mthr)) {
          const float mnew = (mx > mthr) ? mx : mref;
          const float alpha = (mnew == mref) ? 1.0f : fast_exp2((mref - mnew) * zc);
          mref = mnew;
          mc = (mnew == -INFINITY) ? 0.0f : mnew * zc;
          mthr = mnew + kTau / zc;
          psthr = (mnew == -INFINITY) ? -1.0f : kPsum;
          ps = exps(sv, mc, [&](auto) __attribute__((always_inline)) {}, Idx<0>{});
          lsum *= alpha;
          sfor<0, DT>([&](auto i_) { oacc[SIDX(i_)] *= alpha; });
        }
      }
      lsum += ps;
      // P and l stay in this half-step (not sunk past the barrier).
      {
        keep_p();
        const float l0 = lsum;
        asm volatile("" ::"v"(l0));
      }
    };


    // Each group runs its own copy of the sequence (no per-phase branches).
    // Barriers: one work-group barrier per step, X_i between half-steps 2i+1
    // and 2i+2 (group 0: after SM(i); group 1: after MM(i)), plus the two
    // that open the first step.  X_i is the only ordering the data needs: the
    // copies into the buffers of K_i and V_{i-1} start after it (every MM(i)
    // is done), and the copies of K_{i+1} and V_i issued before it are waited
    // for in it (both groups' MM(i+1) read them after it).  Inside a step the
    // groups keep their half-step offset by themselves, since the two phases
    // take about equally long; a barrier in the middle of the step as well
    // cost 1-3%.  Per item both groups pass n + 2 barriers.
    // Group 1 copies the first tiles (K_0, then K_1 and V_0).  From then on
    // K_{i+2} and V_{i+1} are copied in half-step 2i+2 into the buffers of K_i
    // and V_{i-1} (last read by MM(i) in half-steps 2i and 2i+1) and waited
    // for in X_{i+1}, before MM(i+2) of group 0 (half-step 2i+4):
    //   heads up to 128 wide: by group 0 during its MM(i+1), where issuing a
    //     copy costs little (the matrix pipe works meanwhile);
    //   192-wide heads: by group 1 during its SM(i), since the copy addresses
    //     do not fit beside the wider Q fragments in the matrix phase.
    constexpr bool kCopyInMM = DQK <= 128;
    // Table entries (mask_next of block i, active columns i .. i+3) are read
    // one softmax phase ahead: the scalar loads for step i+1 are issued at the
    // start of SM(i) and complete at its closing barrier.  A scalar load in
    // flight while a phase waits for its LDS reads would force a full wait
    // (both share one counter and scalar loads return out of order).
    struct TabWin {
      int mn, c0, c1, c2, c3;   // mask_next[i], cols[i .. i+3] (clamped to the row)
    };
    auto tab_start = [&]() __attribute__((always_inline)) {
      TabWin t{ld_table(p.mask_next, g0), colc(0), colc(1), colc(2), colc(3)};
      // Resolved here, before the loop (the compiler does not see the waits
      // inside the barrier assembly and would otherwise wait for them in the
      // loop, after the next step's loads were issued).
      asm volatile("" ::"s"(t.mn), "s"(t.c0), "s"(t.c1), "s"(t.c2), "s"(t.c3));
      return t;
    };
    // Issue the loads that advance the window from step i to i+1.
    auto tab_issue = [&](int i, int* nmn, int* c4) __attribute__((always_inline)) {
      *nmn = ld_table(p.mask_next, g0 + min(i + 1, n - 1));
      *c4 = colc(i + 4);
    };
    // Their values are needed before the barrier (which waits for them anyway).
    auto tab_advance = [&](TabWin& t, int nmn, int c4) __attribute__((always_inline)) {
      asm volatile("" ::"s"(nmn), "s"(c4));
      t = TabWin{nmn, t.c1, t.c2, t.c3, c4};
    };
    auto run = [&](auto g1_tag) __attribute__((always_inline)) {
      constexpr bool G1 = SIDX(g1_tag) != 0;
      TabWin tw = tab_start();
      if constexpr (G1) {
        g1_load_k(tw.c0, 0);
        seg_copy(tw.c0, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      lds_barrier();
      if constexpr (G1) {
        if (n > 1) {
          g1_load_k(tw.c1, 1);
          seg_copy(tw.c1, 1);
        }
        g1_load_v(tw.c0, 0);
        lds_barrier();   // group 1 starts one half-step late
      }
      mm(0, Idx<0>{}, Idx<1>{}, no_copy, Idx<0>{});
      if constexpr (!G1) lds_barrier();   // group 1's second barrier (K_1, V_0 issued)
      for (int i = 0; i + 1 < n; ++i) {
        int nmn, c4;
        // X_i: group 1 passes it after MM(i), group 0 after SM(i).
        if constexpr (G1) wait_copies_and_barrier<0>();
        tab_issue(i, &nmn, &c4);
        if constexpr (G1 && !kCopyInMM) {
          // K_{i+2} (past the end: a repeat of K_{n-1} into the free buffer)
          // and V_{i+1}; the segment ids of block i+2 go to ring slot
          // (i+2) % 3, last read by SM(i-1).
          const int ck = tw.c2, cv = tw.c1;
          const int kbf = i & 1, vbf = (i + 1) & 1, sslot = (i + 2) % 3;
          sm(i, tw.mn, tw.c0,
             [&](auto k_) __attribute__((always_inline)) { copy_part(k_, ck, kbf, cv, vbf, sslot); },
             Idx<KL + VL>{});
        } else {
          sm(i, tw.mn, tw.c0, no_copy, Idx<0>{});
        }
        tab_advance(tw, nmn, c4);
        if constexpr (G1) {
          mm(i + 1, Idx<1>{}, Idx<1>{}, no_copy, Idx<0>{});
        } else {
          wait_copies_and_barrier<0>();
          if constexpr (kCopyInMM) {
            // The same copies, issued between the MFMAs (tw has advanced).
            const int ck = tw.c1, cv = tw.c0;
            const int kbf = i & 1, vbf = (i + 1) & 1, sslot = (i + 2) % 3;
            mm(i + 1, Idx<1>{}, Idx<1>{},
               [&](auto k_) __attribute__((always_inline)) { copy_part(k_, ck, kbf, cv, vbf, sslot); },
               Idx<KL + VL>{});
          } else {
            mm(i + 1, Idx<1>{}, Idx<1>{}, no_copy, Idx<0>{});
          }
        }
      }
      if constexpr (G1) wait_copies_and_barrier<0>();
      sm(n - 1, tw.mn, tw.c0, no_copy, Idx<0>{});
      if constexpr (!G1) wait_copies_and_barrier<0>();
      mm(n, Idx<1>{}, Idx<0>{}, no_copy, Idx<0>{});
    };
    if (grp1)
      run(Idx<1>{});
    else
      run(Idx<0>{});
  };

  pingpong_loop();

  // Epilogue: o = O / l, lse = (m zc + log2 l) ln 2.
  const float lt = lsum + __shfl_xor(lsum, 32);
  if constexpr (SPLIT) {
    // Split-KV partial: o and lse of this chunk alone, in float32 (an empty
    // chunk gives o = 0, lse = -inf, which the merge weighs by 0).
    if (qi < L) {
      const float inv = (lt > 0.0f) ? 1.0f / lt : 0.0f;
      const int64_t row = ((int64_t)split * p.B * p.Hq + head) * L + qi;
      float* og = p.ws_o + row * DV;
      sfor<0, DT * 4>([&](auto i_) {
        constexpr int dt = SIDX(i_) / 4;
        constexpr int q4 = SIDX(i_) % 4;
        const f32x4 w = {oacc[dt][4 * q4] * inv, oacc[dt][4 * q4 + 1] * inv, oacc[dt][4 * q4 + 2] * inv,
                         oacc[dt][4 * q4 + 3] * inv};
        *reinterpret_cast<f32x4*>(og + 32 * dt + 8 * q4 + 4 * hi) = w;
      });
      if (hi == 0) p.ws_lse[row] = (lt > 0.0f) ? (mref * zc + __log2f(lt)) * kLn2 : -INFINITY;
    }
    return;
  }
  if (qi < L) {
    const float inv = (lt > 0.0f) ? 1.0f / lt : 0.0f;
    uint16_t* og = static_cast<uint16_t*>(p.o) + ((int64_t)head * L + qi) * DV;
    sfor<0, DT * 4>([&](auto i_) {
      constexpr int dt = SIDX(i_) / 4;
      constexpr int q4 = SIDX(i_) % 4;
      u32x2 w = {pack_bf16(oacc[dt][4 * q4] * inv, oacc[dt][4 * q4 + 1] * inv),
                 pack_bf16(oacc[dt][4 * q4 + 2] * inv, oacc[dt][4 * q4 + 3] * inv)};
      *reinterpret_cast<u32x2*>(og + 32 * dt + 8 * q4 + 4 * hi) = w;
    });
    if (p.lse && hi == 0)
      p.lse[(int64_t)head * L + qi] = (lt > 0.0f) ? (mref * zc + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

// Work-group schedule (persistent): the grid has at most one work-group per
// CU; work-group w processes items w, w + G, w + 2G, ... (G = grid size) of
// the XCD-aware, longest-row-first item order, one after another.  Odd
// rounds run backwards inside each XCD, so that a work-group that took one
// of the longest rows in one round takes one of the shortest in the next:
// the per-CU sums of causal row lengths come out equal.  A CU thus never
// waits for a work-group launch between items.
__device__ __forceinline__ int item_of_round(int k, int w, int G, bool snake) {
  if (snake && (k & 1)) {
    const int S = G / kNumXcd;
    return k * G + kNumXcd * (S - 1 - w / kNumXcd) + w % kNumXcd;
  }
  return k * G + w;
}

template <int DQK, int DV, int BN, int NW, bool CAP, bool SPLIT, bool PACK>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void splash_fwd_bf16_kernel(FwdParams p) {
  const int w = blockIdx.x;
  const int G = gridDim.x;
  // Items: (head, q-block row) x split, split-major, so that the items of
  // one split keep the XCD placement of the unsplit order.
  const int T0 = p.B * p.Hq * p.n_q_blocks;
  const int T = SPLIT ? T0 * p.n_split : T0;
  const bool snake = (G % kNumXcd) == 0;
  for (int k = 0; k * G < T; ++k) {
    const int t = item_of_round(k, w, G, snake);
    if (t >= T) continue;
    const int split = SPLIT ? t / T0 : 0;
    int head, rank;
    map_workgroup(p, t - split * T0, &head, &rank);
    item_fwd<DQK, DV, BN, NW, CAP, SPLIT, PACK>(p, head, PACK ? rank : ld_table(p.row_order, rank), split);
  }
}

// Grid size: one work-group per CU slot (8 waves per CU: one 8-wave work-group
// or several smaller ones, as many as the LDS holds) for masks whose rows cost what their block counts say
// (causal, windows), where the static round schedule is balanced; with
// segment ids, rows mix partial and full blocks unevenly and the hardware's
// dynamic dispatch of one work-group per item balances better (a grid of one
// work-group per item is the same kernel with one round).
template <int DQK, int DV, int BN, int NW, bool CAP, bool SPLIT, bool PACK>
hipError_t launch(const FwdParams& p, int n_cu, hipStream_t s) {
  const int64_t n_items = (int64_t)p.B * p.Hq * p.n_q_blocks * (SPLIT ? p.n_split : 1);
  const bool persistent = p.seg_q == nullptr;
  // Work-groups a CU holds at once: 8 waves, and the LDS (160 KiB).
  constexpr int kPerCu = (8 / NW) < (163840 / Cfg<DQK, DV, BN>::LDS_BYTES) ? (8 / NW)
                                                                          : (163840 / Cfg<DQK, DV, BN>::LDS_BYTES);
  const int64_t slots = (int64_t)n_cu * kPerCu;
  const int64_t grid = (persistent && n_items > slots) ? slots : n_items;
  const int bytes = Cfg<DQK, DV, BN>::LDS_BYTES;
  auto fn = splash_fwd_bf16_kernel<DQK, DV, BN, NW, CAP, SPLIT, PACK>;
  if (bytes > 65536) {
    // Opt in to more than 64 KiB of dynamic LDS (gfx950 has 160 KiB per CU).
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(64 * NW), bytes, s, p);
  return hipGetLastError();
}

template <int DQK, int DV, int BN, int NW, bool PACK>
hipError_t launch_cap(const FwdParams& p, int n_cu, hipStream_t s) {
  if (p.ws_o)
    return p.soft_cap > 0.0f ? launch<DQK, DV, BN, NW, true, true, PACK>(p, n_cu, s)
                             : launch<DQK, DV, BN, NW, false, true, PACK>(p, n_cu, s);
  return p.soft_cap > 0.0f ? launch<DQK, DV, BN, NW, true, false, PACK>(p, n_cu, s)
                           : launch<DQK, DV, BN, NW, false, false, PACK>(p, n_cu, s);
}

// Every variant (split-KV, packed GQA rows) at one tile; packed rows use
// their own instances, so that the unpacked kernels keep their registers.
template <int DQK, int DV, int BN, int NW>
hipError_t launch_all(const FwdParams& p, int n_cu, hipStream_t s) {
  return p.row_period > 0 ? launch_cap<DQK, DV, BN, NW, true>(p, n_cu, s)
                          : launch_cap<DQK, DV, BN, NW, false>(p, n_cu, s);
}

// Every variant at the head dims' default tile.
template <int DQK, int DV>
hipError_t launch_default(const FwdParams& p, int n_cu, hipStream_t s) {
  constexpr Tile t = bf16_default_tile(DQK, DV);
  return launch_all<DQK, DV, t.bkv, t.bq / 32>(p, n_cu, s);
}

// The plain forward (no split, no packing) of 128/128 heads at the other
// tiles of the block-size sweep.
template <int BQ, int BKV>
hipError_t launch_sweep(const FwdParams& p, int n_cu, hipStream_t s) {
  return p.soft_cap > 0.0f ? launch<128, 128, BKV, BQ / 32, true, false, false>(p, n_cu, s)
                           : launch<128, 128, BKV, BQ / 32, false, false, false>(p, n_cu, s);
}

}  // namespace
}  // namespace splash
