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
//   * One work-group = 4 waves = a 128-query block of one head; each wave owns
//     32 query rows.  Registers stay within 256 per lane and LDS within 80 KiB
//     per work-group, so two work-groups share a CU and each SIMD runs two
//     waves: the matrix pipe of one wave overlaps the softmax of the other
//     (section 5.3: the vector work must hide behind the matrix work).
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
//     sequence end read as zero) one block ahead into the other of two
//     buffers (section 3.1), waited with vmcnt before one barrier per block.
//     LDS rows are XOR-swizzled in 16-byte chunks so both the K operand reads
//     and the transposing V reads are bank-conflict free.
//   * exp is the hardware exp2 with log2(e) folded into the scale (6.6
//     "use_base2_exp").  The reference max used in the exponent only moves
//     when a row's block max exceeds it by more than 2^8; the constant cancels
//     in o / l (section 5.4: any constant that keeps exp in range gives the
//     same softmax), so almost every block skips the O rescale.

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

constexpr int BM = kBf16BlockQ;   // 128 queries per work-group
constexpr int BN = kBf16BlockKV;  // 64 keys per block
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
  static constexpr int NBUF = 2;               // tile buffers per operand
  static constexpr int LDS_BYTES = NBUF * (KTILE + VTILE);
  static constexpr int KLOADS = KCHUNKS / NT;  // tile-copy instructions per wave
  static constexpr int VLOADS = VCHUNKS / NT;
  static_assert(KCHUNKS % NT == 0 && VCHUNKS % NT == 0, "tile chunks split over 256 threads");
  static_assert(LDS_BYTES <= 81920, "two work-groups per CU");
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
  static_assert(N >= 0 && N <= 63, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
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
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void splash_fwd_bf16_kernel(FwdParams p) {
  using C = Cfg<DQK, DV>;
  constexpr int KS = C::KS;
  constexpr int DT = C::DT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  lds_u8* lds = (lds_u8*)smem;  // address-space cast to LDS
  // Layout: [K buf 0, 1][V buf 0, 1]; block x lives in buffer x % 2.
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
  const int qw = r * BM + wave * 32;  // first query row of this wave
  const int qi = qw + l32;            // this lane's query row

  const uint16_t* qg = static_cast<const uint16_t*>(p.q) + (int64_t)head * L * DQK;
  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + (int64_t)kvh * L * DQK;
  const uint16_t* vg = static_cast<const uint16_t*>(p.v) + (int64_t)kvh * L * DV;
  // Buffer resources: reads past the sequence end return zero.
  const __amdgpu_buffer_rsrc_t qrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)qg, (short)0, L * DQK * 2, kRsrcWord3);
  const u32x4 krs = make_rsrc(kg, (uint32_t)(L * DQK * 2));
  const u32x4 vrs = make_rsrc(vg, (uint32_t)(L * DV * 2));

  // Zero the tile buffers once: a tile that hangs over the sequence end is
  // then finite everywhere (its masked keys get zero weight).
  for (int i = tid; i < C::LDS_BYTES / 16; i += NT)
    *reinterpret_cast<lds_u32x4*>(lds + 16 * i) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();  // the zero stores land before any wave's tile copies

  // Q^T as B operands: k-step s -> Q[qi][16s + 8hi + 0..7].
  bf16x8 qf[KS];
  sfor<0, KS>([&](auto s_) {
    constexpr int s = SIDX(s_);
    const int off = (qi * DQK + 16 * s + 8 * hi) * 2;
    qf[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
  });

  // Tile copies HBM -> LDS.  Each wave instruction writes 64 consecutive
  // 16-byte LDS chunks; lane i fetches the global chunk that belongs in
  // physical slot i of the swizzled layout.
  auto load_k = [&](int c, int buf) __attribute__((always_inline)) {
    const int k0 = c * BN;
#pragma unroll
    for (int t = 0; t < C::KLOADS; ++t) {
      const int slot0 = (t * 4 + wave) * 64;
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
    for (int t = 0; t < C::VLOADS; ++t) {
      const int slot0 = (t * 4 + wave) * 64;
      const int slot = slot0 + lane;
      const int row = slot / (DV / 8);
      const int pc = slot - row * (DV / 8);
      const int off = ((k0 + row) * DV + vswz(row, pc) * 8) * 2;
      dma16(vrs, (uint32_t)(uintptr_t)(vbuf(buf) + slot0 * 16), off);
    }
  };

  // Softmax state (z in log2 units after multiplying by zc):
  //   no cap: z = q.k, zc = scale log2(e);  cap: z = log2(e) cap tanh(scale q.k / cap), zc = 1.
  const float zc = CAP ? 1.0f : p.scale_log2;
  float mref = -INFINITY;
  float lsum = 0.0f;
  f32x16 oacc[DT];
  sfor<0, DT>([&](auto i_) { oacc[SIDX(i_)] = f32x16{}; });

  const bool has_seg = p.seg_q != nullptr;
  const int32_t* segq = has_seg ? p.seg_q + (int64_t)b * L : nullptr;
  const int32_t* segk = has_seg ? (p.seg_kv ? p.seg_kv + (int64_t)b * L : segq) : nullptr;
  const int my_seg = (has_seg && qi < L) ? segq[qi] : 0;
  // Allowed key interval of this lane's row before the segment test.
  int klo = 0, khi = L - 1;
  if (p.causal) khi = min(khi, qi);
  if (p.window_left >= 0) klo = max(klo, qi - p.window_left);
  if (p.window_right >= 0) khi = min(khi, qi + p.window_right);
  const int qa = qw;
  const int qb = min(qw + 31, L - 1);

  const int g0 = ld_table(p.row_ptr, r);
  const int n = ld_table(p.row_ptr, r + 1) - g0;
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
  auto apply_mask = [&](f32x16* sv, int g, int c) __attribute__((always_inline)) {
    const int ka = c * BN;
    const int kz = ka + BN - 1;
    if (p.mask_stored) {
      const uint8_t* prow = p.patterns + (int64_t)ld_table(p.mask_next, g0 + g) * (BM * BN) +
                            (wave * 32 + l32) * BN;
      sfor<0, 8>([&](auto i_) {
        constexpr int t = SIDX(i_) / 4;
        constexpr int q4 = SIDX(i_) % 4;
        const uint32_t bits = *reinterpret_cast<const uint32_t*>(prow + 32 * t + 8 * q4 + 4 * hi);
        sfor<0, 4>([&](auto e_) {
          constexpr int e = SIDX(e_);
          sv[t][4 * q4 + e] = ((bits >> (8 * e)) & 0xffu) ? sv[t][4 * q4 + e] : -INFINITY;
        });
      });
      return;
    }
    // Corner tests on this wave's rows: no element mask when all are allowed.
    const bool all = !has_seg && kz < L && (!p.causal || kz <= qa) &&
                     (p.window_left < 0 || qb - ka <= p.window_left) &&
                     (p.window_right < 0 || kz - qa <= p.window_right);
    if (all) return;
    if (has_seg) {
      sfor<0, 32>([&](auto i_) {
        constexpr int t = SIDX(i_) / 16;
        constexpr int i = SIDX(i_) % 16;
        const int key = ka + 32 * t + 8 * (i / 4) + 4 * hi + (i % 4);
        const bool ok = (key >= klo) & (key <= khi) & (segk[min(key, L - 1)] == my_seg);
        sv[t][i] = ok ? sv[t][i] : -INFINITY;
      });
    } else {
      sfor<0, 32>([&](auto i_) {
        constexpr int t = SIDX(i_) / 16;
        constexpr int i = SIDX(i_) % 16;
        const int key = ka + 32 * t + 8 * (i / 4) + 4 * hi + (i % 4);
        const bool ok = (key >= klo) & (key <= khi);
        sv[t][i] = ok ? sv[t][i] : -INFINITY;
      });
    }
  };

  if (n > 0) {
    load_k(cols[0], 0);
    load_v(cols[0], 0);
  }

  for (int j = 0; j < n; ++j) {
    const int buf = j & 1;
    // Block j's copies (issued one iteration earlier) have landed and every
    // wave is past iteration j-1, so buffer buf^1 is free: copy block j+1
    // into it while block j is computed.
    wait_copies_and_barrier<0>();
    if (j + 1 < n) {
      load_k(colc(j + 1), buf ^ 1);
      load_v(colc(j + 1), buf ^ 1);
    }

    const lds_u8* kb = kbuf(buf);
    const lds_u8* vb = vbuf(buf);

    // S^T for the two 32-key tiles (two independent accumulation chains).
    f32x16 sv[2];
    sfor<0, KS>([&](auto s_) {
      constexpr int s = SIDX(s_);
      sfor<0, 2>([&](auto t_) {
        constexpr int t = SIDX(t_);
        const int key = 32 * t + l32;
        const bf16x8 kf = *reinterpret_cast<const lds_bf16x8*>(kb + key * C::KROW + kswz(key, 2 * s + hi) * 16);
        if constexpr (s == 0) {
          const f32x16 zero = {};
          sv[t] = mfma(kf, qf[0], zero);
        } else {
          sv[t] = mfma(kf, qf[s], sv[t]);
        }
      });
    });

    if constexpr (CAP) {
      const float k2 = 2.0f * kLog2e * p.scale / p.soft_cap;
      const float A = p.soft_cap * kLog2e;
      sfor<0, 32>([&](auto i_) {
        constexpr int t = SIDX(i_) / 16;
        constexpr int e = SIDX(i_) % 16;
        const float ex = fast_exp2(sv[t][e] * k2);
        sv[t][e] = A - 2.0f * A * __builtin_amdgcn_rcpf(ex + 1.0f);
      });
    }
    // Partial block <=> it has a pattern (mask_next >= 0); int32 scalar load.
    if (ld_table(p.mask_next, g0 + j) >= 0) apply_mask(sv, j, colc(j));

    // Row max: in-lane over 32 keys, then across the two half-waves.
    float mx = sv[0][0];
    sfor<1, 32>([&](auto i_) { mx = fmaxf(mx, sv[SIDX(i_) / 16][SIDX(i_) % 16]); });
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // Lazy reference update: move only when the block max exceeds it by > 2^kTau.
    const bool need = mx * zc > mref * zc + kTau;
    const float mnew = need ? mx : mref;
    const float alpha = (mnew == mref) ? 1.0f : fast_exp2((mref - mnew) * zc);
    mref = mnew;
    const float mc = (mnew == -INFINITY) ? 0.0f : mnew * zc;

    // p = 2^(z zc - m zc), packed as bf16 B operands: tile t, key half c2.
    bf16x8 pb[2][2];
    float ps = 0.0f;
    sfor<0, 4>([&](auto i_) {
      constexpr int t = SIDX(i_) / 2;
      constexpr int c2 = SIDX(i_) % 2;
      u32x4 w;
      sfor<0, 4>([&](auto e_) {
        constexpr int e2 = SIDX(e_);
        const float p0 = fast_exp2(fmaf(sv[t][8 * c2 + 2 * e2], zc, -mc));
        const float p1 = fast_exp2(fmaf(sv[t][8 * c2 + 2 * e2 + 1], zc, -mc));
        ps += p0 + p1;
        w[e2] = pack_bf16(p0, p1);
      });
      pb[t][c2] = __builtin_bit_cast(bf16x8, w);
    });
    lsum = lsum * alpha + ps;
    if (__any(alpha != 1.0f)) {
      sfor<0, DT>([&](auto i_) { oacc[SIDX(i_)] *= alpha; });
    }

    // O^T += V^T P^T; key-half-major order keeps the DT accumulators
    // independent between consecutive MFMAs.
    sfor<0, 4>([&](auto tc_) {
      constexpr int t = SIDX(tc_) / 2;
      constexpr int c2 = SIDX(tc_) % 2;
      const int row = 32 * t + 16 * c2 + vrow0;
      const int row2 = row + 8;
      sfor<0, DT>([&](auto dt_) {
        constexpr int dt = SIDX(dt_);
        const int lc = 4 * dt + vcol0;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vb + row * C::VROW + vswz(row, lc) * 16 + 8 * (jj & 1)));
        const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vb + row2 * C::VROW + vswz(row2, lc) * 16 + 8 * (jj & 1)));
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 up2 = __builtin_bit_cast(u32x2, up);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], up2[0], up2[1]});
        oacc[dt] = mfma(vf, pb[t][c2], oacc[dt]);
      });
    });
  }

  // Epilogue: o = O / l, lse = (m zc + log2 l) ln 2.
  const float lt = lsum + __shfl_xor(lsum, 32);
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
