/*
 * splash.h - C ABI of block-sparse (Splash) attention, forward and
 * backward, for AMD Instinct MI355X (gfx950).
 *
 * These operations cross this boundary:
 *
 *   attn_mask_compile  host-side preprocessing of a causal / local-window /
 *                      segment-id mask (and their AND) into the MaskInfo
 *                      block-sparse execution table.  Defined by "Lecture 13 -
 *                      Pallas Kernels and Splash Attention" (CMU 11-868
 *                      notes), sections 6.1 (empty / full / partial blocks),
 *                      6.2 (block_mask, active rows and columns,
 *                      partial_mask_blocks, mask_next, bounds_start /
 *                      bounds_end), 6.4 (segment ids, AND of masks) and 6.6
 *                      (one byte per pattern element).
 *
 *   splash_attn_fwd    the attention forward over the active blocks only:
 *                      running max m, running sum l and output accumulator o
 *                      per query row, the alpha = e^(m_old - m_new) rescale,
 *                      and a single divide o / l after the last block
 *                      (deferred normalisation), returning o and the
 *                      log-sum-exp residual lse = m + ln l.  Defined by
 *                      Lecture 13 sections 5.1-5.2 (online softmax, kernel
 *                      body), 5.2 (MHA / GQA heads), 5.4 (logit soft cap
 *                      cap * tanh(x / cap)), 6.3 (Splash kernel: inputs q, k,
 *                      v, segment ids, patterns; outputs O and logsumexp), and
 *                      by the joto.ai page on core LLM operators, section
 *                      "LSE and online softmax" (lse = m + log l).
 *
 *   splash_attn_fwd_split  the same forward with each query row's active
 *                      kv blocks cut into n_split contiguous chunks computed
 *                      as separate work items, then merged exactly through
 *                      their log-sum-exp residuals (split-KV).  Defined by
 *                      Lecture 13 section 5.1 (partial (m, l, o) results of
 *                      separate key ranges merge in any order, as in split-KV
 *                      inference) and the joto.ai page, section "LSE and
 *                      online softmax" (split-K: lse = log sum_s e^{lse_s},
 *                      o = sum_s e^{lse_s - lse} o_s).
 *
 *   splash_attn_bwd    the gradients dq, dk, dv of the forward's o, with
 *                      the probabilities rebuilt on chip from the stored lse
 *                      (Lecture 13 section 6.3: the forward keeps lse for the
 *                      backward; joto.ai page, section "LSE and online
 *                      softmax": p is recomputed from q, k and lse).  Its K/V
 *                      side walks the table by kv-block column
 *                      (attn_mask_columns).
 *
 * Query rows may sit at key positions q_offset + i against a longer key
 * sequence (decoding, chunked prefill): splash_mask_desc.q_offset and
 * splash_fwd_args.L_kv / q_offset.
 *
 * Conventions for every call:
 *   - Return value: SPLASH_OK (0) or one of the SPLASH_E* codes below.  On an
 *     error nothing is written to any output and no kernel is launched;
 *     splash_last_error() returns a message for the calling thread.
 *   - No call allocates memory that outlives it or throws across the ABI,
 *     and the caller owns every buffer.  State kept between calls: the
 *     per-thread error message, a per-device cache of the compute-unit count
 *     (read once from the runtime), and splash_attn_fwd_split_noalloc's
 *     static device scratch.  The environment variable SPLASH_XCD_MAP=0
 *     turns off the XCD-aware work-group order of the forward (for
 *     comparisons; results are identical).
 *   - "host" pointers are CPU memory; "device" pointers are HIP device memory
 *     on the current device.
 */
#ifndef SPLASH_H_
#define SPLASH_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPLASH_VERSION 111

/* Largest n_split of splash_attn_fwd_split. */
#define SPLASH_MAX_SPLIT 64

/* Bytes of the static device scratch of splash_attn_fwd_split_noalloc
 * (16 MiB per device). */
#define SPLASH_STATIC_SCRATCH_BYTES (16 << 20)

enum splash_status {
  SPLASH_OK = 0,
  SPLASH_EINVAL = 1,        /* NULL pointer, negative size, bad flag value */
  SPLASH_ESHAPE = 2,        /* inconsistent shapes or tables */
  SPLASH_EDTYPE = 3,        /* unknown dtype */
  SPLASH_EUNSUPPORTED = 4,  /* head dimension not built for this dtype */
  SPLASH_ENOMEM = 5,        /* host scratch allocation failed */
  SPLASH_EHIP = 6,          /* the HIP runtime reported an error */
  SPLASH_EINTERNAL = 7      /* unexpected internal failure */
};

enum splash_dtype {
  SPLASH_F32 = 0,   /* float32 storage, float32 arithmetic */
  SPLASH_BF16 = 1   /* bfloat16 storage, bf16 MFMA with float32 accumulation */
};

enum splash_mask_mode {
  /* Partial blocks build their element mask in the kernel from the query and
   * key positions and the segment ids (Lecture 13 section 6.6 suggests this
   * in place of stored patterns). */
  SPLASH_MASK_COMPUTED = 0,
  /* Partial blocks read partial_mask_blocks[mask_next[g]] (section 6.3). */
  SPLASH_MASK_STORED = 1
};

/* Library version (SPLASH_VERSION of the build). */
int splash_version(void);

/* Message describing the last error on the calling thread ("" if none).
 * The string is owned by the library and valid until the next call made by
 * the same thread. */
const char* splash_last_error(void);

/* ------------------------------------------------------------------------
 * Mask preprocessing (MaskInfo).
 * ---------------------------------------------------------------------- */

/* The mask: element (i, j) (query row i, key position j) is allowed iff
 *   i < L_q and j < L_kv                      (padding of ragged blocks)
 *   and (!causal or j <= p)
 *   and (window_left  < 0 or p - j <= window_left)
 *   and (window_right < 0 or j - p <= window_right)
 *   and (seg_q == NULL or seg_q[i] == seg_kv[j]),
 * where p = q_offset + i is the key position of query row i.
 * The blocks are block_q x block_kv; the last block row / column may hang
 * over the sequence end (ragged L), its padded elements count as masked. */
typedef struct splash_mask_desc {
  int32_t L_q;            /* number of query positions, >= 0 */
  int32_t L_kv;           /* number of key positions, >= 0 */
  int32_t block_q;        /* > 0 */
  int32_t block_kv;       /* > 0 */
  int32_t causal;         /* 0 or 1 */
  int32_t window_left;    /* -1 (unbounded) or >= 0 */
  int32_t window_right;   /* -1 (unbounded) or >= 0 */
  const int32_t* seg_q;   /* host [L_q] segment ids, or NULL: no segment mask */
  const int32_t* seg_kv;  /* host [L_kv], or NULL: same array as seg_q
                             (then L_kv must equal L_q) */
  int32_t q_offset;       /* >= 0: query row i sits at key position
                             q_offset + i in the causal and window tests
                             (0: aligned; decoding the last L_q of L_kv
                             positions: L_kv - L_q) */
} splash_mask_desc;

typedef struct splash_mask_sizes {
  int32_t n_q_blocks;     /* ceil(L_q / block_q) */
  int32_t n_kv_blocks;    /* ceil(L_kv / block_kv) */
  int32_t n_active;       /* blocks with at least one allowed element */
  int32_t n_partial;      /* active blocks that are not full */
  int32_t n_patterns;     /* distinct partial patterns */
} splash_mask_sizes;

/* Host output arrays, all caller-owned.  Any pointer may be NULL to skip
 * that array.  Active blocks are listed in row-major order (q-block row, then
 * kv-block column ascending). */
typedef struct splash_mask_tables {
  int8_t* block_mask;        /* [n_q_blocks * n_kv_blocks] 0 empty, 1 partial,
                                2 full; row-major */
  int32_t* active_rows;      /* [n_active] q-block row of each active block */
  int32_t* active_cols;      /* [n_active] kv-block column */
  int8_t* block_code;        /* [n_active] 1 partial, 2 full */
  int32_t* mask_next;        /* [n_active] pattern index of a partial block
                                (patterns numbered by first appearance in
                                active order), -1 for a full block */
  uint8_t* bounds;           /* [n_active] bit0 = bounds_start (first active
                                block of its row), bit1 = bounds_end (last) */
  int32_t* row_ptr;          /* [n_q_blocks + 1] CSR offsets into the active
                                list */
  int32_t* row_order;        /* [n_q_blocks] rows sorted by active count,
                                longest first, ties by ascending row: the
                                launch order of the forward */
  uint8_t* partial_mask_blocks; /* [n_patterns * block_q * block_kv] 1 =
                                allowed, one byte per element, each pattern
                                row-major [block_q][block_kv] */
} splash_mask_tables;

/* Two-phase call.  With tables == NULL: validates desc and fills *sizes.
 * With tables != NULL: *sizes must hold the values of the first phase for
 * the same desc (SPLASH_ESHAPE otherwise), and the non-NULL arrays are
 * filled.  Deterministic; thread-safe; touches no device.
 * Errors: SPLASH_EINVAL (NULL desc/sizes, negative length, block <= 0,
 * window < -1, seg_kv NULL with L_kv != L_q), SPLASH_ESHAPE (sizes do not
 * match), SPLASH_ENOMEM. */
int attn_mask_compile(const splash_mask_desc* desc, splash_mask_sizes* sizes,
                      splash_mask_tables* tables);

/* Column-major view of the active list (host arrays), for work that owns
 * one kv-block column: the backward sums the gradients of a K/V block over
 * the q-block rows that read it.  From row_ptr [n_q_blocks + 1] and
 * active_cols [n_active] of attn_mask_compile, fills col_ptr
 * [n_kv_blocks + 1] (CSR offsets per column), col_rows [n_active] (the rows
 * of each column, ascending) and col_entry [n_active] (the row-major index
 * of each block, for block_code / mask_next).  Caller-owned arrays.
 * Errors: SPLASH_EINVAL (negative size, NULL array, row_ptr not running
 * from 0 to n_active or decreasing, a row's columns not ascending within
 * [0, n_kv_blocks)). */
int attn_mask_columns(int32_t n_q_blocks, int32_t n_kv_blocks, int32_t n_active,
                      const int32_t* row_ptr, const int32_t* active_cols,
                      int32_t* col_ptr, int32_t* col_rows, int32_t* col_entry);

/* The kv-block columns ordered by their number of active blocks, most
 * first, ties in column order (a stable sort): the order in which the
 * backward's dK/dV kernel takes its columns (splash_bwd_args.col_order),
 * so that the longest columns start first.  From col_ptr [n_kv_blocks + 1]
 * of attn_mask_columns; writes the host array col_order [n_kv_blocks].
 * Errors: SPLASH_EINVAL (negative size, NULL array, col_ptr not starting at
 * 0 or decreasing). */
int attn_mask_column_order(int32_t n_kv_blocks, const int32_t* col_ptr, int32_t* col_order);

/* ------------------------------------------------------------------------
 * Forward.
 * ---------------------------------------------------------------------- */

/* Default block sizes (block_q, block_kv) of the forward kernel for this
 * dtype and head dimensions: the tile every forward variant is built for
 * (split-KV, packed GQA rows), and the one to compile tables with.  Lecture
 * 13 section 5.3 (block sizes of the tiled kernel) and 6.5 (the block-size
 * trade-off).  Errors: SPLASH_EDTYPE, SPLASH_EUNSUPPORTED, SPLASH_EINVAL
 * (NULL outputs). */
int splash_fwd_tile(int32_t dtype, int32_t d_qk, int32_t d_v,
                    int32_t* block_q, int32_t* block_kv);

/* Every (block_q, block_kv) for which splash_attn_fwd (no split-KV) has a
 * kernel for this dtype and head dims, the default tile first: bf16 128/128
 * heads also have the block-size sweep's other tiles of 128 or 256 query rows
 * by 64 or 128 keys (Lecture 13 sections 5.3 and 6.5).  Writes up to
 * `capacity` pairs to the host arrays block_q / block_kv and the total count
 * to *count (call with capacity 0 to size them).  Tables of a non-default
 * tile are accepted by splash_attn_fwd only; packed GQA rows are then not
 * used.  Errors: as splash_fwd_tile, SPLASH_EINVAL (NULL count, negative
 * capacity, NULL arrays with capacity > 0). */
int splash_fwd_tiles(int32_t dtype, int32_t d_qk, int32_t d_v,
                     int32_t* block_q, int32_t* block_kv, int32_t capacity,
                     int32_t* count);

typedef struct splash_fwd_args {
  int32_t dtype;         /* SPLASH_F32 or SPLASH_BF16: q, k, v and o */
  int32_t B;             /* batch, >= 0 */
  int32_t Hq;            /* query heads, >= 0 */
  int32_t Hkv;           /* key/value heads, >= 1, divides Hq; query head h
                            reads kv head h / (Hq / Hkv) */
  int32_t L;             /* query rows (also key positions unless L_kv is
                            set, see below), >= 0 */
  int32_t d_qk;          /* q/k head dim: f32 {64, 128}; bf16 {64, 128, 192} */
  int32_t d_v;           /* v head dim:   f32 {64, 128}; bf16 {64, 128} */
  const void* q;         /* device [B, Hq,  L, d_qk] contiguous, 16-B aligned */
  const void* k;         /* device [B, Hkv, L_kv, d_qk] contiguous, 16-B aligned */
  const void* v;         /* device [B, Hkv, L_kv, d_v]  contiguous, 16-B aligned */
  void* o;               /* device [B, Hq,  L, d_v]  output, same dtype as q,
                            16-B aligned; rows with no allowed key get 0 */
  float* lse;            /* device [B, Hq, L] float32 natural-log lse of the
                            scaled (and capped) logits, -inf for rows with no
                            allowed key; or NULL */
  /* Mask parameters (as in splash_mask_desc) used by SPLASH_MASK_COMPUTED
   * for the element mask of partial blocks.  They must describe the same
   * mask the tables were compiled from, for every batch element. */
  int32_t causal;
  int32_t window_left;
  int32_t window_right;
  const int32_t* seg_q;  /* device [B, L] or NULL */
  const int32_t* seg_kv; /* device [B, L_kv] or NULL (NULL: same as seg_q) */
  /* Execution table (device copies of attn_mask_compile output for
   * L_q = L, this call's L_kv and q_offset and its block sizes). */
  int32_t block_q;       /* a tile of splash_fwd_tiles (splash_attn_fwd) or
                            splash_fwd_tile's (splash_attn_fwd_split) */
  int32_t block_kv;
  int32_t n_q_blocks;    /* ceil(L / block_q) */
  int32_t n_active;
  int32_t n_patterns;
  const int32_t* row_ptr;      /* device [n_q_blocks + 1] */
  const int32_t* row_order;    /* device [n_q_blocks] */
  const int32_t* active_cols;  /* device [n_active] */
  const int8_t* block_code;    /* device [n_active] */
  const int32_t* mask_next;    /* device [n_active]; also marks partial blocks
                                  (>= 0) for the kernels */
  const uint8_t* partial_mask_blocks; /* device [n_patterns, block_q,
                                         block_kv] (SPLASH_MASK_STORED) */
  int32_t mask_mode;     /* splash_mask_mode */
  float scale;           /* softmax scale, finite and > 0 (e.g. 1/sqrt(d_qk)) */
  float soft_cap;        /* logit soft cap; <= 0 disables it; logits are
                            cap * tanh(scale * q.k / cap) */
  /* Max Logit Estimate (Lecture 13 section 5.4).  use_max_logit = 1: the
   * constant max_logit (logit units: after the scale and the cap) replaces
   * the running row max, so p = e^(logit - max_logit) with no max reduction
   * and no rescale.  The constant cancels in o = sum p v / sum p, so o and
   * lse = max_logit + ln(sum p) are those of the exact softmax as long as
   * no exponent leaves the float32 range: max_logit must exceed the largest
   * logit minus 88.7 (else p overflows) and stay below every row's largest
   * logit plus 87.3 (else that row underflows to o = 0, lse = -inf).  With a
   * soft cap, max_logit = soft_cap can never overflow.  0 = running max. */
  int32_t use_max_logit;
  float max_logit;       /* finite when use_max_logit = 1 */
  /* Decoding shapes.  L counts the query rows; the keys and values have
   * L_kv positions, and query row i sits at key position q_offset + i in the
   * causal and window tests (as in splash_mask_desc; decoding the last L of
   * L_kv positions: q_offset = L_kv - L).  Then k and v are
   * [B, Hkv, L_kv, d], seg_kv is [B, L_kv] (required with seg_q when
   * L_kv != L), q, o, lse and seg_q keep L, and the tables come from
   * attn_mask_compile with L_q = L, this L_kv and this q_offset.  A
   * zero-initialised pair (L_kv = 0, q_offset = 0) means L_kv = L, so a
   * query set with no keys at all is given by tables without active blocks.
   * L_kv != L or q_offset != 0 is bf16 only. */
  int32_t L_kv;          /* >= 0; 0: equal to L */
  int32_t q_offset;      /* >= 0 */
} splash_fwd_args;

/* Enqueue the forward on `stream` (a hipStream_t; NULL = the default
 * stream) and return without waiting.  Validation errors are returned
 * synchronously: SPLASH_EINVAL (NULL args or buffers, misaligned pointer,
 * bad flag, scale <= 0 or not finite, soft_cap not finite, max_logit not
 * finite with use_max_logit = 1, negative L_kv or q_offset, seg_q without
 * seg_kv when L_kv != L), SPLASH_ESHAPE
 * (Hq % Hkv != 0, block sizes or n_q_blocks not matching, size overflow),
 * SPLASH_EDTYPE, SPLASH_EUNSUPPORTED (head dims; L_kv != L or q_offset != 0
 * with f32), SPLASH_EHIP (the launch
 * failed).  B, Hq or L equal to 0 is a no-op.  Device-side faults surface at
 * the caller's next synchronisation. */
int splash_attn_fwd(const splash_fwd_args* args, void* stream);

/* ------------------------------------------------------------------------
 * Split-KV forward.
 * ---------------------------------------------------------------------- */

/* Bytes of device workspace splash_attn_fwd_split needs for these sizes:
 * n_split * B * Hq * L * (d_v + 1) * 4 (float32 partial outputs and
 * log-sum-exp values).  Errors: SPLASH_EINVAL (NULL bytes, n_split not in
 * [1, SPLASH_MAX_SPLIT], negative size, d_v <= 0). */
int splash_split_workspace_bytes(int32_t n_split, int32_t B, int32_t Hq, int32_t L,
                                 int32_t d_v, int64_t* bytes);

/* The forward of splash_attn_fwd (same arguments, same results up to
 * float32 rounding order) with every query row's active kv blocks cut into
 * n_split near-equal contiguous chunks, each processed as a separate work
 * item: more items for shapes with few heads or q blocks.  Each chunk's
 * normalised output and lse go to `workspace` (device, 16-B aligned,
 * caller-owned, at least splash_split_workspace_bytes; its contents on entry
 * are ignored and on return are scratch); a second kernel on the same
 * stream merges them into args->o and args->lse (a chunk with no allowed
 * key has weight 0).  bf16 only.  Errors: those of splash_attn_fwd, plus
 * SPLASH_EUNSUPPORTED (f32), SPLASH_EINVAL (n_split not in
 * [1, SPLASH_MAX_SPLIT], NULL, misaligned or too small workspace),
 * SPLASH_ESHAPE (items beyond int32).  Calls that share a workspace must be
 * ordered on one stream. */
int splash_attn_fwd_split(const splash_fwd_args* args, int32_t n_split, void* workspace,
                          int64_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops, harnesses that forbid it): splash_attn_fwd_split
 * with the workspace replaced by a static device array of
 * SPLASH_STATIC_SCRATCH_BYTES that the library holds on each device it runs
 * on until the process ends.  The caller still passes every input and
 * output; nothing is allocated.  The first call on a device looks up that
 * device's array (with the device current).  Every call on a device shares
 * its array: calls that overlap on one device (other streams, other host
 * threads) race and give wrong results; calls ordered on one stream do not.
 * Nothing in the array needs clearing between calls.  Errors: those of
 * splash_attn_fwd_split, plus SPLASH_EINVAL when the partials
 * (splash_split_workspace_bytes) exceed SPLASH_STATIC_SCRATCH_BYTES and
 * SPLASH_EHIP when the array's address cannot be obtained. */
int splash_attn_fwd_split_noalloc(const splash_fwd_args* args, int32_t n_split, void* stream);

/* ------------------------------------------------------------------------
 * Backward.
 *
 * Gradients of the forward's o with respect to q, k and v, given the
 * upstream gradient do = dLoss/do and the forward's residual lse.  The
 * probabilities are rebuilt on chip from the stored lse, p = e^(logit - lse)
 * (Lecture 13 section 6.3: the forward writes the per-row logsumexp for the
 * backward; joto.ai "LSE and online softmax": the backward recomputes p from
 * q, k and the lse scalar of each row), so no attention matrix is stored.
 * With y = scale q.k, logit z = cap tanh(y / cap) (z = y without a cap):
 *   dv_j = sum_i p_ij do_i,   dp_ij = do_i . v_j,   D_i = do_i . o_i,
 *   dy_ij = p_ij (dp_ij - D_i) (1 - tanh^2(y_ij / cap) with a cap),
 *   dq_i = scale sum_j dy_ij k_j,   dk_j = scale sum_i dy_ij q_i,
 * summed over the query heads of a K/V group for dk and dv.
 * ---------------------------------------------------------------------- */

/* Block sizes (block_q, block_kv) of the backward kernels, which its tables
 * (and their column view) must be compiled with; they may differ from the
 * forward's default tile.  Errors: SPLASH_EDTYPE, SPLASH_EUNSUPPORTED (not
 * bf16 with head dims (64, 64), (128, 128) or (192, 128)), SPLASH_EINVAL
 * (NULL outputs). */
int splash_bwd_tile(int32_t dtype, int32_t d_qk, int32_t d_v,
                    int32_t* block_q, int32_t* block_kv);

typedef struct splash_bwd_args {
  int32_t dtype;         /* SPLASH_BF16 (q, k, v, o, dout) */
  int32_t B, Hq, Hkv;    /* as in splash_fwd_args */
  int32_t L;             /* query rows */
  int32_t L_kv;          /* key positions; 0: equal to L */
  int32_t q_offset;      /* query row i sits at key position q_offset + i */
  int32_t d_qk, d_v;     /* (64, 64), (128, 128) or (192, 128) */
  const void* q;         /* device [B, Hq, L, d_qk] */
  const void* k;         /* device [B, Hkv, L_kv, d_qk] */
  const void* v;         /* device [B, Hkv, L_kv, d_v] */
  const void* o;         /* device [B, Hq, L, d_v]: the forward's output */
  const float* lse;      /* device [B, Hq, L]: the forward's lse */
  const void* dout;      /* device [B, Hq, L, d_v]: upstream gradient */
  float* dq;             /* device [B, Hq, L, d_qk] float32 output */
  float* dk;             /* device [B, Hkv, L_kv, d_qk] float32 output */
  float* dv;             /* device [B, Hkv, L_kv, d_v] float32 output */
  float* delta;          /* device [B, Hq, L] float32 scratch, caller-owned:
                            receives D_i = do_i . o_i */
  /* Mask (as in splash_fwd_args; the element mask is computed from
   * positions and segment ids on every active block). */
  int32_t causal;
  int32_t window_left;
  int32_t window_right;
  const int32_t* seg_q;  /* device [B, L] or NULL */
  const int32_t* seg_kv; /* device [B, L_kv] or NULL (NULL: same as seg_q) */
  /* Tables for L_q = L, L_kv, q_offset at the backward's block sizes: the
   * row-major list of attn_mask_compile and its column view from
   * attn_mask_columns, as device copies. */
  int32_t block_q;       /* splash_bwd_tile's block_q for (bf16, d_qk, d_v) */
  int32_t block_kv;      /* splash_bwd_tile's block_kv */
  int32_t n_q_blocks;    /* ceil(L / block_q) */
  int32_t n_kv_blocks;   /* ceil(L_kv / block_kv) */
  int32_t n_active;
  const int32_t* row_ptr;      /* device [n_q_blocks + 1] */
  const int32_t* row_order;    /* device [n_q_blocks]: the rows longest first
                                  (attn_mask_compile's row_order, a
                                  permutation of 0 .. n_q_blocks - 1), the
                                  order in which the dq kernel takes them;
                                  NULL: row order 0, 1, ... (slower where
                                  row lengths differ) */
  const int32_t* active_cols;  /* device [n_active] */
  const int32_t* col_ptr;      /* device [n_kv_blocks + 1] */
  const int32_t* col_rows;     /* device [n_active] */
  const int32_t* col_order;    /* device [n_kv_blocks]: the columns in the
                                  order of attn_mask_column_order (a
                                  permutation of 0 .. n_kv_blocks - 1), the
                                  order in which the dK/dV kernel takes
                                  them; NULL: column order 0, 1, ... */
  float scale;           /* as in the forward */
  float soft_cap;        /* as in the forward; <= 0 disables it */
} splash_bwd_args;

/* Enqueue the backward on `stream` (a hipStream_t; NULL = the default
 * stream): a kernel for dq (one work-group per query head and q block,
 * looping over the row's kv blocks), which also writes delta, then one for
 * dk and dv (one work-group per K/V head and kv block, looping over the
 * column's q blocks and the group's query heads: no atomics).  Every element of dq, dk
 * and dv is written (0 where no allowed pair reaches it).  Validation
 * errors are returned synchronously: SPLASH_EINVAL (NULL or misaligned
 * buffers, bad flag or window, scale, soft_cap, negative sizes),
 * SPLASH_ESHAPE (Hq % Hkv, block sizes or block counts not matching,
 * size overflow), SPLASH_EDTYPE, SPLASH_EUNSUPPORTED (f32, head dims),
 * SPLASH_EHIP (a launch failed).  B, Hq or L equal to 0 writes dk and dv
 * only if it has keys (zeros); all sizes 0 is a no-op. */
int splash_attn_bwd(const splash_bwd_args* args, void* stream);

/* ------------------------------------------------------------------------
 * Clock probe (measurement only; not part of the attention computation).
 * The MFMA peak scales with the shader clock, which the chip lowers under
 * load; these two calls let a caller measure the mean clock over a run of
 * kernels and price its throughput against the peak at that clock.
 * ---------------------------------------------------------------------- */

/* Enqueue on `stream` (a hipStream_t; NULL = the default stream) n_groups
 * work-groups of one wave.  Work-group g writes out[3g] = the shader clock
 * counter (s_memtime: core clock cycles of the CU it ran on), out[3g + 1] =
 * the constant-rate real-time counter (s_memrealtime) and out[3g + 2] = where
 * it ran: (XCD id << 16) | (HW_ID bits 15:8: CU, shader array, shader
 * engine).  `out`: caller-owned device memory of 3 * n_groups uint64 values.
 * The cycle counters of different CUs are not in step, so two probes
 * enqueued before and after a run of kernels give a CU's mean clock over the
 * run only from records of the same location: (cycles after - cycles before)
 * / (real after - real before) times the real-time counter's rate
 * (splash_realtime_khz).  Which CUs a probe's work-groups land on is up to
 * the dispatcher; with n_groups = 256 on an MI355X most CUs are stamped by
 * both probes.  Errors: SPLASH_EINVAL (NULL out, n_groups outside 1..4096),
 * SPLASH_EHIP (launch failed). */
int splash_clock_probe(uint64_t* out, int n_groups, void* stream);

/* Rate of the current device's real-time counter in kHz
 * (hipDeviceAttributeWallClockRate) into *khz.  Errors: SPLASH_EINVAL (NULL),
 * SPLASH_EHIP. */
int splash_realtime_khz(int* khz);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* SPLASH_H_ */
