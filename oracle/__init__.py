"""Float64 CPU oracle for the block-sparse (Splash) attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the test suite, the smoke check and the
``cpu_baseline`` leg of the benchmark use it.  It shares no code with the HIP
path: it materialises the full score matrix (in row panels), applies the mask
element by element from its definition, and normalises with a library-free
numpy softmax.

Sources (pages cited by title and section):

* "Lecture 13 - Pallas Kernels and Splash Attention" (CMU 11-868 notes,
  semidirectx.com), sections 5.1-5.2 (online softmax, merge rule, kernel body
  and deferred normalisation), 5.4 (soft cap), 6.1-6.4 (block classes,
  MaskInfo, bounds, segment ids and AND-combined masks), 6.6 (one byte per
  pattern element), exercises 7, 11, 12 and their answers.
* "拆解大模型几项核心操作背后的数学与 Infra 优化逻辑" (joto.ai blog), sections
  "Causal Mask", "Online Softmax" and "LSE 与 Online Softmax" (lse = m + log l,
  the split-K merge of per-range outputs through their lse, and the backward
  rebuilding p = exp(s - lse) from the stored lse).

Parity pins: every function here is pinned by tests under ``tests/`` against
worked examples printed on the pages (``tests/golden/``), closed forms,
library routines (scipy) and brute-force scalar loops.  ``row_order`` (the
longest-row-first schedule) is this build's own addition; it is pinned by its
definition (a stable sort) and by a brute-force check.
"""

from .attention import (
    allowed,
    attention_ref,
    attention_brute,
    online_softmax_steps,
    merge_partials,
    merge_lse,
    mle_safe_range,
)
from .backward import attention_bwd_ref
from .mask_tables import column_tables_ref, mask_tables_ref

__all__ = [
    "allowed",
    "attention_ref",
    "attention_brute",
    "online_softmax_steps",
    "merge_partials",
    "merge_lse",
    "mle_safe_range",
    "mask_tables_ref",
    "column_tables_ref",
    "attention_bwd_ref",
]
