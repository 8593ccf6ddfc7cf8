// Launch parameters of the forward kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace splash {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;          // may be null
  int32_t B, Hq, Hkv, L, group;  // L: query rows; group = Hq / Hkv
  int32_t Lkv;            // key/value positions
  int32_t q_off;          // query row i sits at key position q_off + i
  // Packed GQA rows: when row_period > 0 the query heads of a K/V group are
  // packed into one row space (Hq, L above are then Hkv and group * L):
  // row R is row R % row_period of query head R / row_period, at key
  // position q_off + R % row_period, and every row uses table row 0.
  int32_t row_period;
  int32_t Lseg;           // rows per batch element of seg_q
  // mask
  int32_t causal, window_left, window_right;
  const int32_t* seg_q;   // [B, Lseg] or null
  const int32_t* seg_kv;  // [B, Lkv] or null (then seg_q is used, Lkv = L)
  int32_t mask_stored;    // 1: partial blocks read patterns
  // tables (compiled for block_q x block_kv blocks: the kernel's tile)
  int32_t block_q, block_kv;
  int32_t n_q_blocks;
  const int32_t* row_ptr;
  const int32_t* row_order;
  const int32_t* active_cols;
  const int8_t* block_code;
  const int32_t* mask_next;
  const uint8_t* patterns;
  // arithmetic
  float scale;        // softmax scale
  float scale_log2;   // scale * log2(e)
  float soft_cap;     // > 0 when the cap is on
  int32_t mle;        // 1: constant max logit instead of the running max
  float mle_log2;     // that constant times log2(e)
  // work-group -> (head, row) mapping
  int32_t xcd_units;      // number of units spread over XCDs (0: plain order)
  int32_t unit_heads;     // query heads per unit
  // split-KV: each row's active blocks are cut into n_split contiguous
  // chunks, each an item of its own writing a partial o (float32, divided
  // by its own l) and lse to ws_o [n_split, B*Hq, L, d_v] and
  // ws_lse [n_split, B*Hq, L]; ws_o == null: plain forward (n_split = 1).
  int32_t n_split;
  float* ws_o;
  float* ws_lse;
};

// Launchers (return the hipError_t of the launch).
hipError_t launch_fwd_f32(const FwdParams& p, int d_qk, int d_v, hipStream_t s);
hipError_t launch_fwd_bf16(const FwdParams& p, int d_qk, int d_v, hipStream_t s);
// Its parts for 192-wide q/k heads and for the 64-wide head dims (64/64,
// 64/128, 128/64), at the default tile; n_cu = compute units of the device.
hipError_t launch_fwd_bf16_d192(const FwdParams& p, int d_v, int n_cu, hipStream_t s);
hipError_t launch_fwd_bf16_d64(const FwdParams& p, int d_qk, int d_v, int n_cu, hipStream_t s);
// Merge of the split-KV partials of p.ws_o / p.ws_lse into p.o (bf16) and
// p.lse.
hipError_t launch_split_merge_bf16(const FwdParams& p, int d_v, hipStream_t s);

// Block sizes used by each kernel family.
constexpr int kF32BlockQ = 64;
constexpr int kF32BlockKV = 64;
// The bf16 backward's tables.
constexpr int kBwdBlockQ = 256;
constexpr int kBwdBlockKV = 64;

// A bf16 forward tile: bq query rows (32 per wave) by bkv keys per block.
struct Tile {
  int32_t bq, bkv;
};
// The tile every bf16 forward variant (split-KV, packed GQA rows) is built
// for, per head dims: the fastest of the block-size sweep where it fits the
// LDS (two 128-key K/V buffers of 192-wide heads do not).
constexpr Tile bf16_default_tile(int d_qk, int d_v) {
  return (d_qk <= 128 && d_v <= 128) ? Tile{256, 64} : Tile{256, 64};
}
// Tiles of the plain forward (no split-KV, no packing) of 128/128 heads:
// the block-size sweep of 128 or 256 rows by 64 or 128 keys.
constexpr Tile kSweepTiles[4] = {{256, 64}, {256, 128}, {128, 64}, {128, 128}};
// The decode tile of 128/128 heads: 64 query rows (two waves) by 64 keys,
// with every variant (split-KV, packed GQA rows), for shapes with few query
// rows per K/V head, where a 256-row tile would be mostly padding.
constexpr Tile kDecodeTile = {64, 64};

// Whether a bf16 forward instance exists for these head dims and tile.
inline bool bf16_tile_built(int d_qk, int d_v, int bq, int bkv, bool split) {
  const Tile d = bf16_default_tile(d_qk, d_v);
  if (bq == d.bq && bkv == d.bkv) return true;
  if (d_qk != 128 || d_v != 128) return false;
  if (bq == kDecodeTile.bq && bkv == kDecodeTile.bkv) return true;
  if (split) return false;
  for (const Tile& t : kSweepTiles)
    if (t.bq == bq && t.bkv == bkv) return true;
  return false;
}

// Number of XCDs of an MI355X; consecutive work-group ids are dispatched
// round-robin over them.
constexpr int kNumXcd = 8;

// Maps a linear item id to (flattened head b*Hq+h, q-block row rank).
// When xcd_units > 0, all items of one unit (a K/V head group or a single
// query head) land on the same XCD so that they share its L2.  Within an
// XCD the items go unit by unit, each unit's rows longest-first with the
// query heads of a K/V group side by side: the few units in flight at a
// time keep their K/V in the XCD's L2.
__device__ __forceinline__ void map_workgroup(const FwdParams& p, int wg, int* head, int* rank) {
  const int n_heads = p.B * p.Hq;
  if (p.xcd_units > 0) {
    const int xcd = wg % kNumXcd;
    const int slot = wg / kNumXcd;
    const int per_unit = p.n_q_blocks * p.unit_heads;
    const int unit_local = slot / per_unit;
    const int rem = slot - unit_local * per_unit;
    const int rk = rem / p.unit_heads;
    const int sub = rem - rk * p.unit_heads;
    *head = (unit_local * kNumXcd + xcd) * p.unit_heads + sub;
    *rank = rk;
  } else {
    *rank = wg / n_heads;
    *head = wg - *rank * n_heads;
  }
}

}  // namespace splash
