"""Float64 reference attention: the plain definition, written out.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Nothing here is
blocked, fused or reordered beyond what the definition states: the score
matrix is materialised (in row panels of at most ``panel`` rows, each over
every key), the mask is applied element by element, and the softmax is taken
over the allowed keys of each row.

Readings of the pages taken here:

* Scale first, then the soft cap: ``s = cap * tanh(scale * q.k / cap)``;
  ``cap <= 0`` means no cap.  (Lecture 13, section 5.2 kernel body: the cap
  acts on the logits that the dot product produced; section 5.4 defines
  ``logits = cap * tanh(qk / cap)``.)
* A masked pair has exactly zero weight (the -inf reading of the causal-mask
  section of the joto.ai page).  A row with no allowed key returns o = 0 and
  lse = -inf (the pages are silent on this case).
* Window ``(left, right)`` with ``-1`` meaning unbounded, as in the vLLM
  wrapper on the gsyq.cn page: key j is allowed for query i only if
  ``i - j <= left`` and ``j - i <= right``.
* GQA: query head h reads K/V head ``h // (Hq // Hkv)`` (contiguous groups;
  Lecture 13 section 5.2 says several query heads share one K/V group).
* lse is the natural log-sum-exp over the allowed, scaled and capped logits
  (joto.ai, "LSE 与 Online Softmax": lse = m + log l).
* Positions at or beyond the sequence length (the zero padding of a ragged
  last block, Lecture 13 section 2.3) are masked.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np


def allowed(i, j, *, L_q: int, L_kv: int, causal: bool = False,
            window_left: int = -1, window_right: int = -1,
            seg_q: Optional[np.ndarray] = None,
            seg_kv: Optional[np.ndarray] = None, q_offset: int = 0) -> np.ndarray:
    """Element mask: True where query row ``i`` may attend key ``j``.

    ``i`` and ``j`` are integer arrays that broadcast against each other
    (typically a column and a row of positions).  The mask is the logical
    AND of the causal, local-window and segment-id (document) masks
    (Lecture 13 section 6.4; causal mask: joto.ai "Causal Mask" section),
    and of ``i < L_q`` and ``j < L_kv`` (padding is masked).  Query row i
    sits at key position ``q_offset + i`` for the causal and window tests
    (0: queries and keys aligned; decoding the last L_q of L_kv positions
    uses L_kv - L_q); segment ids are looked up by row and key index.
    """
    i = np.asarray(i, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    ok = (i < L_q) & (j < L_kv) & (i >= 0) & (j >= 0)
    pos = i + int(q_offset)
    if causal:
        ok = ok & (j <= pos)
    if window_left >= 0:
        ok = ok & (pos - j <= window_left)
    if window_right >= 0:
        ok = ok & (j - pos <= window_right)
    if seg_q is not None:
        sq = np.asarray(seg_q, dtype=np.int64)
        skv = sq if seg_kv is None else np.asarray(seg_kv, dtype=np.int64)
        ii = np.clip(i, 0, L_q - 1)
        jj = np.clip(j, 0, L_kv - 1)
        ok = ok & (sq[ii] == skv[jj])
    return ok


def _seg_for_batch(seg, b):
    if seg is None:
        return None
    seg = np.asarray(seg)
    return seg[b] if seg.ndim == 2 else seg


def attention_ref(q, k, v, *, scale: float, soft_cap: float = 0.0,
                  causal: bool = False, window_left: int = -1,
                  window_right: int = -1, seg_q=None, seg_kv=None,
                  rows: Optional[Sequence[int]] = None,
                  heads: Optional[Iterable[tuple]] = None,
                  panel: int = 512, max_logit: Optional[float] = None,
                  q_offset: int = 0):
    """Exact masked attention forward in float64.

    Shapes: ``q`` [B, Hq, L_q, d_qk], ``k`` [B, Hkv, L_kv, d_qk],
    ``v`` [B, Hkv, L_kv, d_v]; any real dtype (the stored values are read
    and widened to float64).  ``seg_q``/``seg_kv`` are [L] or [B, L]
    integer ids (``seg_kv`` defaults to ``seg_q``).  ``rows`` restricts the
    computation to those query positions (sampled outputs); ``heads`` to
    those (b, h) pairs.  ``q_offset``: key position of query row 0 (see
    ``allowed``).

    Returns ``(o, lse)``: o [B, Hq, n_rows, d_v] and lse [B, Hq, n_rows] in
    float64.  Heads not in ``heads`` are left as NaN.

    For each query row i (Lecture 13 sections 5.2 and 6.4; joto.ai "LSE"):
      s_ij = scale * sum_d q_id k_jd, then s_ij <- cap * tanh(s_ij / cap);
      A_i  = { j allowed by causal AND window AND segment };
      m_i  = max_{j in A_i} s_ij;  p_ij = exp(s_ij - m_i) on A_i, else 0;
      l_i  = sum_j p_ij;  o_i = sum_j p_ij v_j / l_i;  lse_i = m_i + ln l_i.

    ``max_logit`` = c selects the Max Logit Estimate (Lecture 13 section
    5.4): the constant c takes the place of m_i in every row (p_ij =
    exp(s_ij - c), lse_i = c + ln l_i).  In exact arithmetic c cancels, so
    the result equals the one above; float64 keeps every exp in range for
    |s - c| < 700.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, Hq, L_q, d_qk = q.shape
    Bk, Hkv, L_kv, d_k = k.shape
    d_v = v.shape[3]
    if Bk != B or d_k != d_qk or v.shape[:3] != k.shape[:3]:
        raise ValueError("q/k/v shapes do not agree")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    row_idx = np.arange(L_q) if rows is None else np.asarray(rows, np.int64)
    n_rows = row_idx.shape[0]
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    o = np.full((B, Hq, n_rows, d_v), np.nan)
    lse = np.full((B, Hq, n_rows), np.nan)
    kv_pos = np.arange(L_kv)[None, :]
    for (b, h) in heads:
        kh = h // group
        kf = k[b, kh].astype(np.float64)
        vf = v[b, kh].astype(np.float64)
        sq = _seg_for_batch(seg_q, b)
        skv = _seg_for_batch(seg_kv, b)
        for p0 in range(0, n_rows, panel):
            sel = row_idx[p0:p0 + panel]
            qf = q[b, h, sel].astype(np.float64)
            s = scale * (qf @ kf.T)
            if soft_cap > 0:
                s = soft_cap * np.tanh(s / soft_cap)
            a = allowed(sel[:, None], kv_pos, L_q=L_q, L_kv=L_kv,
                        causal=causal, window_left=window_left,
                        window_right=window_right, seg_q=sq, seg_kv=skv,
                        q_offset=q_offset)
            s_a = np.where(a, s, -np.inf)
            has = a.any(axis=1)
            if max_logit is None:
                m = s_a.max(axis=1)
                m_safe = np.where(has, m, 0.0)
            else:
                m_safe = np.full(sel.shape[0], float(max_logit))
            p = np.where(a, np.exp(s_a - m_safe[:, None]), 0.0)
            l = p.sum(axis=1)
            l_safe = np.where(has, l, 1.0)
            o[b, h, p0:p0 + sel.shape[0]] = np.where(
                has[:, None], (p @ vf) / l_safe[:, None], 0.0)
            lse[b, h, p0:p0 + sel.shape[0]] = np.where(
                has, m_safe + np.log(l_safe), -np.inf)
    return o, lse


# float32 limits of exp: e^x overflows above ln(FLT_MAX) and leaves the
# normal range below ln(FLT_MIN) = ln(2^-126).
LN_FLT_MAX = math.log(3.4028234663852886e38)
LN_FLT_MIN = math.log(2.0 ** -126)


def mle_safe_range(max_logit: float, min_row_max: float):
    """Open interval of Max Logit Estimate constants c that keep float32
    exp(s - c) finite for the largest logit and keep at least each row's
    largest term normal (Lecture 13 section 5.4, exercise 10): the largest
    logit minus c stays below ln(FLT_MAX) (88.72), and c minus the smallest
    row maximum stays below -ln(FLT_MIN) (87.34)."""
    return (float(max_logit) - LN_FLT_MAX, float(min_row_max) - LN_FLT_MIN)


def attention_brute(q, k, v, *, scale: float, soft_cap: float = 0.0,
                    causal: bool = False, window_left: int = -1,
                    window_right: int = -1, seg_q=None, seg_kv=None, q_offset: int = 0):
    """Scalar-loop attention for tiny inputs (a pin for ``attention_ref``).

    Uses the plain definition without the max shift: w_ij = e^{s_ij} /
    sum_{j in A_i} e^{s_ij}, o_i = sum_j w_ij v_j, lse_i = ln sum e^{s_ij},
    with every sum taken by ``math.fsum``.  Only for small |s| (no overflow).
    Returns nested Python lists [B][Hq][L][d_v] and [B][Hq][L].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, L_q, d_qk = q.shape
    Hkv, L_kv, d_v = k.shape[1], k.shape[2], v.shape[3]
    group = Hq // Hkv
    out, lses = [], []
    for b in range(B):
        ob, lb = [], []
        sq = _seg_for_batch(seg_q, b)
        skv = _seg_for_batch(seg_kv, b)
        if skv is None:
            skv = sq
        for h in range(Hq):
            kh = h // group
            oh, lh = [], []
            for i in range(L_q):
                exps, idx = [], []
                pos = i + q_offset
                for j in range(L_kv):
                    ok = True
                    if causal and j > pos:
                        ok = False
                    if window_left >= 0 and pos - j > window_left:
                        ok = False
                    if window_right >= 0 and j - pos > window_right:
                        ok = False
                    if sq is not None and int(sq[i]) != int(skv[j]):
                        ok = False
                    if not ok:
                        continue
                    dot = math.fsum(float(q[b, h, i, d]) * float(k[b, kh, j, d])
                                    for d in range(d_qk))
                    s = scale * dot
                    if soft_cap > 0:
                        s = soft_cap * math.tanh(s / soft_cap)
                    exps.append(math.exp(s))
                    idx.append(j)
                if not idx:
                    oh.append([0.0] * d_v)
                    lh.append(-math.inf)
                    continue
                z = math.fsum(exps)
                oh.append([math.fsum(e * float(v[b, kh, j, d])
                                     for e, j in zip(exps, idx)) / z
                           for d in range(d_v)])
                lh.append(math.log(z))
            ob.append(oh)
            lb.append(lh)
        out.append(ob)
        lses.append(lb)
    return out, lses


def online_softmax_steps(x, block: int):
    """Online softmax over ``x`` in blocks (Lecture 13 section 5.1).

    Keeps the running maximum m and the sum l of exponentials relative to m;
    for each block: m_new = max(m, max(block)),
    l <- l * e^{m - m_new} + sum e^{block - m_new}.
    Returns the list of (m, l) after each block and the final softmax
    e^{x - m} / l.
    """
    x = [float(t) for t in x]
    m, l = -math.inf, 0.0
    steps = []
    for s in range(0, len(x), block):
        blk = x[s:s + block]
        m_new = max(m, max(blk))
        alpha = 0.0 if m == -math.inf else math.exp(m - m_new)
        l = l * alpha + math.fsum(math.exp(t - m_new) for t in blk)
        m = m_new
        steps.append((m, l))
    return steps, [math.exp(t - m) / l for t in x]


def merge_partials(part1, part2):
    """Merge two partial softmax-weighted sums (Lecture 13 section 5.1).

    Each part is (m_k, l_k, u_k) where u_k = sum_{j in part k} e^{x_j - m_k}
    v_j is the un-normalised accumulator.  Returns (m, l, o) with
    m = max(m1, m2), l = l1 e^{m1-m} + l2 e^{m2-m} and
    o = (u1 e^{m1-m} + u2 e^{m2-m}) / l.  The rule is order-independent.
    """
    m1, l1, u1 = part1
    m2, l2, u2 = part2
    m = max(m1, m2)
    a1 = 0.0 if m1 == -math.inf else math.exp(m1 - m)
    a2 = 0.0 if m2 == -math.inf else math.exp(m2 - m)
    l = l1 * a1 + l2 * a2
    o = (np.asarray(u1, np.float64) * a1 + np.asarray(u2, np.float64) * a2) / l
    return m, l, o


def merge_lse(o_parts, lse_parts):
    """Merge the outputs of attention over disjoint key ranges (split-K).

    ``o_parts[s]`` is the normalised output over key range s and
    ``lse_parts[s]`` its natural-log log-sum-exp (-inf for a range with no
    allowed key).  Per the joto.ai page, section "LSE 与 Online Softmax"
    (split-K reduction; also Lecture 13 section 5.1: partial results of
    separate key ranges combine in any order):
        lse = log sum_s e^{lse_s},    o = sum_s e^{lse_s - lse} o_s.
    A row whose ranges are all empty gets o = 0, lse = -inf.
    Shapes: o_parts [S, ..., d], lse_parts [S, ...]; float64 throughout.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    mx = lse_parts.max(axis=0)
    empty = np.isneginf(mx)
    shift = np.where(empty, 0.0, mx)
    w = np.exp(lse_parts - shift[None])             # e^{-inf} = 0
    den = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, shift + np.log(np.where(empty, 1.0, den)))
    o = (w[..., None] * o_parts).sum(axis=0) / np.where(empty, 1.0, den)[..., None]
    o = np.where(empty[..., None], 0.0, o)
    return o, lse
