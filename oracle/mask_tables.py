"""Reference MaskInfo tables by a per-element scan of the mask.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Lecture 13, sections 6.1-6.3: the [L, L] mask is cut into (block_q x
block_kv) blocks; a block with no allowed element is empty (skipped), one
with every element allowed is full (no mask work), anything else is partial
(needs an element mask).  The sparse execution table lists the active
(non-empty) blocks; partial blocks that share a pattern share one stored
pattern, selected through ``mask_next``; ``bounds_start``/``bounds_end`` mark
the first/last active block of a query-block row (initialise / finalise).

Encodings (the pages name the arrays but not their encodings, so these are
readings of them):

* ``block_mask`` [nq, nkv] int8: 0 empty, 1 partial, 2 full.
* Active blocks in row-major order (q-block row, then kv-block column
  ascending): ``active_rows``, ``active_cols`` int32 and ``block_code`` int8
  (the ``block_mask`` value of each active block).
* ``bounds`` uint8 per active block: bit 0 = first active block of its row
  (bounds_start), bit 1 = last (bounds_end).
* ``row_ptr`` int32 [nq + 1]: CSR offsets of each row's active blocks.
* ``mask_next`` int32: for a partial block, the index of its pattern among the
  unique patterns numbered by first appearance in active order; -1 for full.
* ``partial_mask_blocks`` uint8 [n_patterns, block_q, block_kv]: one byte per
  element, 1 = allowed (section 6.6 prices a 1024 x 1024 pattern at 1 MiB).
* ``row_order`` int32 [nq]: q-block rows sorted by active-block count,
  longest first, ties by ascending row (a stable sort); the launch order.

Positions at or beyond the sequence lengths (padding of a ragged last block)
count as masked, so a block that touches padding is never full.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .attention import allowed


def mask_tables_ref(L_q: int, L_kv: int, block_q: int, block_kv: int, *,
                    causal: bool = False, window_left: int = -1,
                    window_right: int = -1,
                    seg_q: Optional[np.ndarray] = None,
                    seg_kv: Optional[np.ndarray] = None, q_offset: int = 0) -> dict:
    """Build every MaskInfo array by scanning the element mask block row by
    block row (query row i at key position q_offset + i).  Returns a dict of
    numpy arrays plus the size counters."""
    nq = -(-L_q // block_q)
    nkv = -(-L_kv // block_kv)
    full_count = block_q * block_kv
    block_mask = np.zeros((nq, nkv), dtype=np.int8)
    kv_pos = np.arange(nkv * block_kv)[None, :]
    patterns = {}          # pattern bytes -> pattern index
    pattern_list = []
    active_rows, active_cols, block_code, mask_next, bounds = [], [], [], [], []
    row_ptr = [0]
    for r in range(nq):
        q_pos = np.arange(r * block_q, (r + 1) * block_q)[:, None]
        m = allowed(q_pos, kv_pos, L_q=L_q, L_kv=L_kv, causal=causal,
                    window_left=window_left, window_right=window_right,
                    seg_q=seg_q, seg_kv=seg_kv, q_offset=q_offset)
        blocks = m.reshape(block_q, nkv, block_kv)
        counts = blocks.sum(axis=(0, 2))
        row_active = []
        for c in range(nkv):
            if counts[c] == 0:
                continue
            code = 2 if counts[c] == full_count else 1
            block_mask[r, c] = code
            row_active.append(c)
            active_rows.append(r)
            active_cols.append(c)
            block_code.append(code)
            if code == 1:
                pat = np.ascontiguousarray(blocks[:, c, :]).astype(np.uint8)
                key = pat.tobytes()
                if key not in patterns:
                    patterns[key] = len(pattern_list)
                    pattern_list.append(pat)
                mask_next.append(patterns[key])
            else:
                mask_next.append(-1)
        n = len(row_active)
        for t in range(n):
            bounds.append((1 if t == 0 else 0) | (2 if t == n - 1 else 0))
        row_ptr.append(row_ptr[-1] + n)
    row_ptr = np.asarray(row_ptr, dtype=np.int32)
    lengths = np.diff(row_ptr)
    # Stable sort, longest first: key (-length, row).
    row_order = np.asarray(sorted(range(nq), key=lambda r: (-int(lengths[r]), r)),
                           dtype=np.int32)
    if pattern_list:
        pmb = np.stack(pattern_list).astype(np.uint8)
    else:
        pmb = np.zeros((0, block_q, block_kv), dtype=np.uint8)
    n_active = len(active_rows)
    return {
        "n_q_blocks": nq,
        "n_kv_blocks": nkv,
        "n_active": n_active,
        "n_partial": int(sum(1 for c in block_code if c == 1)),
        "n_patterns": len(pattern_list),
        "block_mask": block_mask,
        "active_rows": np.asarray(active_rows, dtype=np.int32),
        "active_cols": np.asarray(active_cols, dtype=np.int32),
        "block_code": np.asarray(block_code, dtype=np.int8),
        "mask_next": np.asarray(mask_next, dtype=np.int32),
        "bounds": np.asarray(bounds, dtype=np.uint8),
        "row_ptr": row_ptr,
        "row_order": row_order,
        "partial_mask_blocks": pmb,
    }


def column_tables_ref(block_mask: np.ndarray):
    """Column-major view of the active blocks, for work items that own one
    kv-block column (the gradients of K and V sum over the q-block rows that
    read a kv block).  From the block classes by definition:

    * ``col_ptr`` int32 [nkv + 1]: CSR offsets per kv-block column;
    * ``col_rows`` int32 [n_active]: for each column c in ascending order, the
      rows r with ``block_mask[r, c] != 0``, ascending;
    * ``col_entry`` int32 [n_active]: the index of block (r, c) in the
      row-major active order of ``mask_tables_ref`` (so its ``block_code``
      and ``mask_next`` can be looked up).
    """
    bm = np.asarray(block_mask)
    nq, nkv = bm.shape
    index = {}
    for r in range(nq):
        for c in range(nkv):
            if bm[r, c] != 0:
                index[(r, c)] = len(index)
    col_ptr, col_rows, col_entry = [0], [], []
    for c in range(nkv):
        for r in range(nq):
            if bm[r, c] != 0:
                col_rows.append(r)
                col_entry.append(index[(r, c)])
        col_ptr.append(len(col_rows))
    return {"col_ptr": np.asarray(col_ptr, dtype=np.int32),
            "col_rows": np.asarray(col_rows, dtype=np.int32),
            "col_entry": np.asarray(col_entry, dtype=np.int32)}
