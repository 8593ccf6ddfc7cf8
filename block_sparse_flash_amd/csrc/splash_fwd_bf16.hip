// bf16 block-sparse attention forward for gfx950 on MFMA.
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
//   * One work-group = 4 waves = a 256-query block of one head; each wave owns
//     64 query rows as two 32-row q-tiles, so every K/V operand fetched from
//     LDS feeds two MFMAs (LDS read bandwidth, not MFMA, would bind at 32
//     rows per wave).  The work-group walks its row's active blocks (CSR
//     list) in 32-key blocks.
//   * Scores are computed transposed, S^T = K Q^T, on
//     v_mfma_f32_32x32x16_bf16: the accumulator holds one query per lane and
//     16 keys per lane, so row max / row sum are in-lane reductions plus one
//     exchange between the two half-waves.
//   * O^T = V^T P^T on the same MFMA.  P never leaves registers (section 5.3
//     hands scores between the matrix and vector units without memory): the
//     S^T accumulator items are the B operand after bf16 conversion.  The V^T
//     A operand is read from row-major V in LDS with ds_read_b64_tr_b16,
//     which returns four consecutive keys of one head dim per lane - exactly
//     the key grouping the accumulator layout implies.
//   * Software pipeline inside each wave: while the vector unit runs the
//     softmax of block j, the matrix unit runs S_{j+1} = Q K_{j+1}^T and
//     O += P_{j-1} V_{j-1}.  Tiles stream HBM -> LDS with buffer_load ... lds
//     (no staging registers; rows past the sequence end read as zero),
//     K two blocks ahead and V one block ahead, one barrier per block.
//   * LDS rows are XOR-swizzled in 16-byte chunks so that both the K operand
//     reads and the transposing V reads are bank-conflict free.
//   * exp is the hardware exp2 with log2(e) folded into the scale (6.6
//     "use_base2_exp").  The reference max used in the exponent only moves
//     when a row's block max exceeds it by more than 2^8; the constant cancels
//     in o / l (section 5.4: any constant that keeps exp in range gives the
//     same softmax), so most blocks skip the O rescale.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fwd_params.h"

namespace splash {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = kBf16BlockQ;   // 256 queries per work-group
constexpr int BN = kBf16BlockKV;  // 32 keys per block
constexpr int NT = 256;           // 4 waves
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;      // log2 of the largest p allowed before a rescale
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit dwords

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int DQK, int DV>
struct Cfg {
  static constexpr int KS = DQK / 16;          // MFMA k-steps for S^T
  static constexpr int DT = DV / 32;           // O^T row tiles
  static constexpr int KROW = DQK * 2;         // bytes per K row in LDS
  static constexpr int VROW = DV * 2;          // bytes per V row in LDS
  static constexpr int KTILE = BN * KROW;      // bytes per K tile
  static constexpr int VTILE = BN * VROW;      // bytes per V tile
  static constexpr int KCHUNKS = KTILE / 16;   // 16-byte chunks per K tile
  static constexpr int VCHUNKS = VTILE / 16;
  static constexpr int NBUF = 3;                // tile buffers per operand
  static constexpr int LDS_BYTES = NBUF * (KTILE + VTILE);
  static constexpr int KLOADS = KCHUNKS / NT;   // tile-load instructions per wave
  static constexpr int VLOADS = VCHUNKS / NT;
  static_assert(KCHUNKS % NT == 0 && VCHUNKS % NT == 0, "tile chunks split over 256 threads");
};

// Physical 16-byte chunk of logical chunk c in LDS row r.
__device__ __forceinline__ int kswz(int r, int c) { return c ^ (r & 7); }
__device__ __forceinline__ int vswz(int r, int c) { return c ^ (2 * (r & 3)); }

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
// M0 (the LDS base of the copy) is saved and restored around it.
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t lds_addr, int voff) {
  const uint32_t base = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr);
  const u32x4 rs = {(uint32_t)__builtin_amdgcn_readfirstlane(rsrc[0]),
                    (uint32_t)__builtin_amdgcn_readfirstlane(rsrc[1]),
                    (uint32_t)__builtin_amdgcn_readfirstlane(rsrc[2]),
                    (uint32_t)__builtin_amdgcn_readfirstlane(rsrc[3])};
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "v"(voff), "s"(rs)
      : "memory");
}

// Wait until at most N tile copies of this wave are in flight and all LDS
// reads are done, then synchronise the work-group.
template <int N>
__device__ __forceinline__ void wait_copies_and_barrier() {
  static_assert(N >= 0 && N <= 6, "vmcnt immediate");
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if constexpr (N == 1) asm volatile("s_waitcnt vmcnt(1) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if constexpr (N == 3) asm volatile("s_waitcnt vmcnt(3) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if constexpr (N == 5) asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if constexpr (N == 6) asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Read-only table entry through the constant address space: with a
// wave-uniform index this is a scalar load (lgkmcnt, not vmcnt).
template <typename T>
__device__ __forceinline__ T ld_table(const T* base, int i) {
  return ((const __attribute__((address_space(4))) T*)base)[__builtin_amdgcn_readfirstlane(i)];
}

__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32), bytes, (uint32_t)kRsrcWord3};
}

template <int DQK, int DV, bool CAP>
__global__ __launch_bounds__(NT) void splash_fwd_bf16_kernel(FwdParams p) {
  using C = Cfg<DQK, DV>;
  constexpr int KS = C::KS;
  constexpr int DT = C::DT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  lds_u8* lds = (lds_u8*)smem;  // address-space cast to LDS
  // Layout: [K buf 0..2][V buf 0..2]; block x lives in buffer x % 3.
  auto kbuf = [&](int i) { return lds + i * C::KTILE; };
  auto vbuf = [&](int i) { return lds + C::NBUF * C::KTILE + i * C::VTILE; };

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
  const int r = ld_table(p.row_order, rank);
  const int qw = r * BM + wave * 64;  // first query row of this wave

  const uint16_t* qg = static_cast<const uint16_t*>(p.q) + (int64_t)head * L * DQK;
  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + (int64_t)kvh * L * DQK;
  const uint16_t* vg = static_cast<const uint16_t*>(p.v) + (int64_t)kvh * L * DV;
  // Buffer resources: reads past the sequence end return zero.
  const __amdgpu_buffer_rsrc_t qrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)qg, (short)0, L * DQK * 2, kRsrcWord3);
  const u32x4 krs = make_rsrc(kg, (uint32_t)(L * DQK * 2));
  const u32x4 vrs = make_rsrc(vg, (uint32_t)(L * DV * 2));

  // Zero both tile buffers once so that a stale buffer read by the
  // pipeline's edge steps holds finite values.
  for (int i = tid; i < C::LDS_BYTES / 16; i += NT)
    *reinterpret_cast<lds_u32x4*>(lds + 16 * i) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();  // the zero stores land before any wave's tile loads

  // Q^T as B operands: q-tile a, k-step s -> Q[qw + 32a + l32][16s + 8hi + 0..7].
  bf16x8 qf[2][KS];
  sfor<0, 2 * KS>([&](auto i_) {
    constexpr int a = SIDX(i_) / KS;
    constexpr int s = SIDX(i_) % KS;
    const int off = ((qw + 32 * a + l32) * DQK + 16 * s + 8 * hi) * 2;
    qf[a][s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
  });

  // Tile copies HBM -> LDS.  Each wave instruction writes 64 consecutive
  // 16-byte LDS chunks; lane i fetches the global chunk that belongs in
  // physical slot i of the swizzled layout.
  auto load_k = [&](int c, int buf) __attribute__((always_inline)) {
    const int k0 = c * BN;
#pragma unroll
    for (int t = 0; t < C::KCHUNKS / NT; ++t) {
      const int slot0 = (t * 4 + wave) * 64;  // first slot of this wave instruction
      const int slot = slot0 + lane;
      const int row = slot / (DQK / 8);
      const int pc = slot - row * (DQK / 8);
      const int off = ((k0 + row) * DQK + kswz(row, pc) * 8) * 2;
      dma16(krs, (uint32_t)(uintptr_t)(kbuf(buf) + slot0 * 16), off);
    }
  };
  auto load_v = [&](int c, int buf) __attribute__((always_inline)) {
    const int k0 = c * BN;
#pragma unroll
    for (int t = 0; t < C::VCHUNKS / NT; ++t) {
      const int slot0 = (t * 4 + wave) * 64;
      const int slot = slot0 + lane;
      const int row = slot / (DV / 8);
      const int pc = slot - row * (DV / 8);
      const int off = ((k0 + row) * DV + vswz(row, pc) * 8) * 2;
      dma16(vrs, (uint32_t)(uintptr_t)(vbuf(buf) + slot0 * 16), off);
    }
  };

  // Softmax state per q-tile (z in log2 units after multiplying by zc):
  //   no cap: z = q.k, zc = scale log2(e);  cap: z = log2(e) cap tanh(scale q.k / cap), zc = 1.
  const float zc = CAP ? 1.0f : p.scale_log2;
  float mref[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.0f, 0.0f};
  f32x16 oacc[2][DT];
  sfor<0, 2 * DT>([&](auto i_) { oacc[SIDX(i_) / DT][SIDX(i_) % DT] = f32x16{}; });

  const bool has_seg = p.seg_q != nullptr;
  const int32_t* segq = has_seg ? p.seg_q + (int64_t)b * L : nullptr;
  const int32_t* segk = has_seg ? (p.seg_kv ? p.seg_kv + (int64_t)b * L : segq) : nullptr;
  int my_seg[2] = {0, 0};
  int klo[2], khi[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int qi = qw + 32 * a + l32;
    if (has_seg && qi < L) my_seg[a] = segq[qi];
    klo[a] = 0;
    khi[a] = L - 1;
    if (p.causal) khi[a] = min(khi[a], qi);
    if (p.window_left >= 0) klo[a] = max(klo[a], qi - p.window_left);
    if (p.window_right >= 0) khi[a] = min(khi[a], qi + p.window_right);
  }
  const int qa = qw;
  const int qb = min(qw + 63, L - 1);

  const int g0 = ld_table(p.row_ptr, r);
  const int n = ld_table(p.row_ptr, r + 1) - g0;
  const int32_t* cols = p.active_cols + g0;

  // V^T transposed reads: lane j of 16-lane group G supplies row
  // 16 c2 + 8 e4 + 4 (G/2) + j/4 and dims 32 dt + 16 (G%2) + 4 (j%4) .. +3;
  // lane 16 G + i receives keys 16 c2 + 8 e4 + 4 (G/2) + 0..3 of dim
  // 32 dt + l32, which are items 4 e4 .. 4 e4 + 3 of the MFMA A operand.
  const int grp = lane >> 4;
  const int jj = lane & 15;
  const int vrow0 = 4 * (grp >> 1) + (jj >> 2);

  f32x16 sacc[2][2];   // [buffer][q-tile]: S^T of the current / next block
  bf16x8 pb[2][2][2];  // [buffer][q-tile][c2]: P^T of the current / previous block

  auto compute_s = [&](f32x16* sdst, int buf) __attribute__((always_inline)) {
    const lds_u8* kb = kbuf(buf);
    sfor<0, KS>([&](auto s_) {
      constexpr int s = SIDX(s_);
      const bf16x8 kf = *reinterpret_cast<const lds_bf16x8*>(kb + l32 * C::KROW + kswz(l32, 2 * s + hi) * 16);
      if constexpr (s == 0) {
        const f32x16 zero = {};
        sdst[0] = mfma(kf, qf[0][0], zero);
        sdst[1] = mfma(kf, qf[1][0], zero);
      } else {
        sdst[0] = mfma(kf, qf[0][s], sdst[0]);
        sdst[1] = mfma(kf, qf[1][s], sdst[1]);
      }
    });
  };

  auto compute_pv = [&](bf16x8 (*pprev)[2], int buf) __attribute__((always_inline)) {
    const lds_u8* vb = vbuf(buf);
    sfor<0, DT * 2>([&](auto i_) {
        constexpr int dt = SIDX(i_) / 2;
        constexpr int c2 = SIDX(i_) % 2;
        const int row = 16 * c2 + vrow0;
        const int row2 = row + 8;
        const int lc = 4 * dt + 2 * (grp & 1) + ((jj & 3) >> 1);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vb + row * C::VROW + vswz(row, lc) * 16 + 8 * (jj & 1)));
        const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vb + row2 * C::VROW + vswz(row2, lc) * 16 + 8 * (jj & 1)));
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 up2 = __builtin_bit_cast(u32x2, up);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], up2[0], up2[1]});
        oacc[0][dt] = mfma(vf, pprev[0][c2], oacc[0][dt]);
        oacc[1][dt] = mfma(vf, pprev[1][c2], oacc[1][dt]);
    });
  };

  // Element mask of a partial block for this wave: item E of q-tile a is key
  // k0 + 8(E/4) + 4hi + E%4 of query qw + 32a + l32.
  auto apply_mask = [&](f32x16* sv, int g, int c) __attribute__((always_inline)) {
    const int ka = c * BN;
    const int kz = ka + BN - 1;
    if (p.mask_stored) {
      const uint8_t* pat = p.patterns + (int64_t)ld_table(p.mask_next, g0 + g) * (BM * BN);
      sfor<0, 8>([&](auto i_) {
        constexpr int a = SIDX(i_) / 4;
        constexpr int q4 = SIDX(i_) % 4;
        const uint32_t bits =
            *reinterpret_cast<const uint32_t*>(pat + (wave * 64 + 32 * a + l32) * BN + 8 * q4 + 4 * hi);
        sfor<0, 4>([&](auto e_) {
          constexpr int e = SIDX(e_);
          sv[a][4 * q4 + e] = ((bits >> (8 * e)) & 0xffu) ? sv[a][4 * q4 + e] : -INFINITY;
        });
      });
      return;
    }
    // Corner tests on this wave's rows: no element mask when all are allowed.
    const bool all = !has_seg && kz < L && (!p.causal || kz <= qa) &&
                     (p.window_left < 0 || qb - ka <= p.window_left) &&
                     (p.window_right < 0 || kz - qa <= p.window_right);
    if (all) return;
    // Branch-free element test; the 16 keys of a lane are shared by both q-tiles.
    if (has_seg) {
      int sk[16];
      sfor<0, 16>([&](auto i_) {
        constexpr int i = SIDX(i_);
        sk[i] = segk[min(ka + 8 * (i / 4) + 4 * hi + (i % 4), L - 1)];
      });
      sfor<0, 32>([&](auto i_) {
        constexpr int a = SIDX(i_) / 16;
        constexpr int i = SIDX(i_) % 16;
        const int key = ka + 8 * (i / 4) + 4 * hi + (i % 4);
        const bool ok = (key >= klo[a]) & (key <= khi[a]) & (sk[i] == my_seg[a]);
        sv[a][i] = ok ? sv[a][i] : -INFINITY;
      });
    } else {
      sfor<0, 32>([&](auto i_) {
        constexpr int a = SIDX(i_) / 16;
        constexpr int i = SIDX(i_) % 16;
        const int key = ka + 8 * (i / 4) + 4 * hi + (i % 4);
        const bool ok = (key >= klo[a]) & (key <= khi[a]);
        sv[a][i] = ok ? sv[a][i] : -INFINITY;
      });
    }
  };


  // Block x's K and V tiles live in buffer x % 3.  Copies run two steps
  // ahead: step j issues K_{j+3} and V_{j+1} and, before its closing barrier,
  // waits only for the copies issued one step earlier (K_{j+2}, V_j).
  // Past the end of the row the copies repeat the last block (same count
  // every step, landing in a buffer nobody reads).
  constexpr int NL = C::KLOADS + C::VLOADS;  // copy instructions per wave per step
  // Column of block x (clamped); the index is made provably wave-uniform so
  // the read is a scalar load, which does not wait behind the tile copies.
  auto colc = [&](int x) { return ld_table(cols, min(x, n - 1)); };
  // P of the (non-existent) block before the first: zero.
  sfor<0, 4>([&](auto i_) { pb[1][SIDX(i_) / 2][SIDX(i_) % 2] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u}); });
  if (n > 0) {
    load_k(cols[0], 0);
    load_k(colc(1), 1);
    wait_copies_and_barrier<0>();
    compute_s(sacc[0], 0);
    wait_copies_and_barrier<0>();  // every wave is done with K buffer 0
    load_k(colc(2), 2);
    load_v(cols[0], 0);
  }

  // Iteration j: issue loads of K_{j+2} (buffer j%2) and V_j (buffer j%2);
  // softmax(S_j) on the vector unit while the matrix unit computes S_{j+1}
  // (K buffer (j+1)%2) and P_{j-1} V_{j-1} (V buffer (j+1)%2); rescale O if a
  // reference max moved; wait for the loads; barrier.
  //
  // The softmax is cut into NSLICE vector-instruction slices and the NM MFMAs
  // are spread evenly between them; sched_barrier fences keep that order, so
  // each MFMA (32 cycles on the matrix pipe) runs while the following slice
  // issues on the vector pipe.
  constexpr int NM = 2 * KS + 4 * DT;           // MFMAs per step
  constexpr int NSLICE = (CAP ? 4 : 0) + 4 + 16;
  auto step = [&](int j, auto cur_tag) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_tag)::value;
    constexpr int nxt = cur ^ 1;
    const int c = colc(j);
    // Partial block <=> it has a pattern (mask_next >= 0); int32, so a scalar load.
    if (ld_table(p.mask_next, g0 + j) >= 0) apply_mask(sacc[cur], j, c);
    const int jm = j % 3;
    const int jm1 = jm == 2 ? 0 : jm + 1;   // (j + 1) % 3
    const int jm2 = jm1 == 2 ? 0 : jm1 + 1; // (j + 2) % 3 == (j - 1) % 3
    load_k(colc(j + 3), jm);
    load_v(colc(j + 1), jm1);

    const lds_u8* kb = kbuf(jm1);   // K_{j+1}
    const lds_u8* vb = vbuf(jm2);   // V_{j-1}

    // Operand fragments: frag f < KS is K k-step f (B of S^T); frag KS + i is
    // V^T for (d-tile i/2, key half i%2).  Frag f feeds MFMAs 2f and 2f+1
    // (one per q-tile) and is read from LDS LA frags (2 LA MFMAs) ahead.
    constexpr int NF = KS + 2 * DT;
    constexpr int LA = 2;
    bf16x8 frag[NF];
    auto read_frag = [&](auto f_) __attribute__((always_inline)) {
      constexpr int f = SIDX(f_);
      if constexpr (f < KS) {
        frag[f] = *reinterpret_cast<const lds_bf16x8*>(kb + l32 * C::KROW + kswz(l32, 2 * f + hi) * 16);
      } else {
        constexpr int dt = (f - KS) / 2;
        constexpr int c2 = (f - KS) % 2;
        const int row = 16 * c2 + vrow0;
        const int row2 = row + 8;
        const int lc = 4 * dt + 2 * (grp & 1) + ((jj & 3) >> 1);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vb + row * C::VROW + vswz(row, lc) * 16 + 8 * (jj & 1)));
        const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vb + row2 * C::VROW + vswz(row2, lc) * 16 + 8 * (jj & 1)));
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 up2 = __builtin_bit_cast(u32x2, up);
        frag[f] = __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], up2[0], up2[1]});
      }
    };
    sfor<0, LA>(read_frag);

    // MFMA m: S_{j+1} for m < 2 KS (k-step m/2, q-tile m%2), then
    // P_{j-1} V_{j-1} (d-tile, key half c2, q-tile).  Before the first MFMA
    // of a frag, the frag LA ahead is requested from LDS.
    auto issue = [&](auto m_) __attribute__((always_inline)) {
      constexpr int m = SIDX(m_);
      constexpr int f = m / 2;
      if constexpr (m % 2 == 0 && f + LA < NF) read_frag(Idx<f + LA>{});
      if constexpr (m < 2 * KS) {
        constexpr int a = m % 2;
        if constexpr (f == 0) {
          const f32x16 zero = {};
          sacc[nxt][a] = mfma(frag[0], qf[a][0], zero);
        } else {
          sacc[nxt][a] = mfma(frag[f], qf[a][f], sacc[nxt][a]);
        }
      } else {
        constexpr int mm = m - 2 * KS;
        constexpr int dt = mm / 4;
        constexpr int c2 = (mm / 2) % 2;
        constexpr int a = mm % 2;
        oacc[a][dt] = mfma(frag[f], pb[nxt][a][c2], oacc[a][dt]);
      }
    };

    f32x16* sv = sacc[cur];
    float alpha[2], mx[2], mc[2];
    float ps[2] = {0.0f, 0.0f};
    u32x4 w[2][2];  // packed bf16 pairs of P, per q-tile and key half
    auto slice = [&](auto i_) __attribute__((always_inline)) {
      constexpr int i0 = SIDX(i_);
      constexpr int cap_slices = CAP ? 4 : 0;
      if constexpr (i0 < cap_slices) {
        // Soft cap of 8 scores: cap tanh(x scale / cap) in log2 units.
        constexpr int a = i0 / 2;
        constexpr int e0 = (i0 % 2) * 8;
        const float k2 = 2.0f * kLog2e * p.scale / p.soft_cap;
        const float A = p.soft_cap * kLog2e;
        sfor<e0, e0 + 8>([&](auto e_) {
          constexpr int e = SIDX(e_);
          const float x = sv[a][e];
          const float ex = fast_exp2(x * k2);
          const float t = A - 2.0f * A * __builtin_amdgcn_rcpf(ex + 1.0f);
          sv[a][e] = (x == -INFINITY) ? -INFINITY : t;
        });
      } else {
        constexpr int i = i0 - cap_slices;
        if constexpr (i < 2) {
          // Row max of q-tile i: in-lane, then across the two half-waves.
          constexpr int a = i;
          float m0 = sv[a][0];
          sfor<1, 16>([&](auto e_) { m0 = fmaxf(m0, sv[a][SIDX(e_)]); });
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m0), __float_as_uint(m0), false, false);
          mx[a] = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        } else if constexpr (i < 4) {
          // Lazy reference update and rescale factor of q-tile i - 2.
          constexpr int a = i - 2;
          const bool need = mx[a] * zc > mref[a] * zc + kTau;
          const float mnew = need ? mx[a] : mref[a];
          alpha[a] = (mnew == mref[a]) ? 1.0f : fast_exp2((mref[a] - mnew) * zc);
          mref[a] = mnew;
          mc[a] = (mnew == -INFINITY) ? 0.0f : mnew * zc;
        } else {
          // p for one pair of scores, packed into the bf16 B operand.
          constexpr int k = i - 4;
          constexpr int a = k / 8;
          constexpr int c2 = (k / 4) % 2;
          constexpr int e2 = k % 4;
          const float p0 = fast_exp2(fmaf(sv[a][8 * c2 + 2 * e2], zc, -mc[a]));
          const float p1 = fast_exp2(fmaf(sv[a][8 * c2 + 2 * e2 + 1], zc, -mc[a]));
          ps[a] += p0 + p1;
          w[a][c2][e2] = pack_bf16(p0, p1);
          if constexpr (e2 == 3) pb[cur][a][c2] = __builtin_bit_cast(bf16x8, w[a][c2]);
          if constexpr (k == 7 || k == 15) lsum[a] = lsum[a] * alpha[a] + ps[a];
        }
      }
    };

    sfor<0, NSLICE>([&](auto i_) {
      constexpr int i = SIDX(i_);
      constexpr int m0 = i * NM / NSLICE;
      constexpr int m1 = (i + 1) * NM / NSLICE;
      sfor<m0, m1>(issue);
      slice(i_);
      __builtin_amdgcn_sched_barrier(0);
    });
    // Keep P and l computed here, beside the MFMAs, rather than sunk past the
    // branch and barrier below.
    {
      const bf16x8 p00 = pb[cur][0][0], p01 = pb[cur][0][1], p10 = pb[cur][1][0], p11 = pb[cur][1][1];
      const float l0 = lsum[0], l1 = lsum[1];
      asm volatile("" ::"v"(p00), "v"(p01), "v"(p10), "v"(p11), "v"(l0), "v"(l1));
    }

    if (__any(alpha[0] != 1.0f || alpha[1] != 1.0f)) {
      sfor<0, 2 * DT>([&](auto i_) {
        constexpr int a = SIDX(i_) / DT;
        constexpr int dt = SIDX(i_) % DT;
        oacc[a][dt] *= alpha[a];
      });
    }
    wait_copies_and_barrier<NL>();
  };

  for (int j = 0; j < n; j += 2) {
    step(j, Idx<0>{});
    if (j + 1 < n) step(j + 1, Idx<1>{});
  }
  // Last block's P V (V_{n-1} landed before the final barrier).
  if (n > 0) {
    if ((n - 1) & 1)
      compute_pv(pb[1], (n - 1) % 3);
    else
      compute_pv(pb[0], (n - 1) % 3);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the trailing copies

  // Epilogue: o = O / l, lse = (m zc + log2 l) ln 2.
  sfor<0, 2>([&](auto a_) {
    constexpr int a = SIDX(a_);
    const float lt = lsum[a] + __shfl_xor(lsum[a], 32);
    const int qi = qw + 32 * a + l32;
    if (qi < L) {
      const float inv = (lt > 0.0f) ? 1.0f / lt : 0.0f;
      uint16_t* og = static_cast<uint16_t*>(p.o) + ((int64_t)head * L + qi) * DV;
      sfor<0, DT * 4>([&](auto i_) {
        constexpr int dt = SIDX(i_) / 4;
        constexpr int q4 = SIDX(i_) % 4;
        u32x2 w = {pack_bf16(oacc[a][dt][4 * q4] * inv, oacc[a][dt][4 * q4 + 1] * inv),
                   pack_bf16(oacc[a][dt][4 * q4 + 2] * inv, oacc[a][dt][4 * q4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(og + 32 * dt + 8 * q4 + 4 * hi) = w;
      });
      if (p.lse && hi == 0)
        p.lse[(int64_t)head * L + qi] = (lt > 0.0f) ? (mref[a] * zc + __log2f(lt)) * kLn2 : -INFINITY;
    }
  });
}

template <int DQK, int DV, bool CAP>
hipError_t launch(const FwdParams& p, hipStream_t s) {
  const int64_t n_wg = (int64_t)p.B * p.Hq * p.n_q_blocks;
  const int bytes = Cfg<DQK, DV>::LDS_BYTES;
  auto fn = splash_fwd_bf16_kernel<DQK, DV, CAP>;
  if (bytes > 65536) {
    // Opt in to more than 64 KiB of dynamic LDS (gfx950 has 160 KiB per CU).
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
