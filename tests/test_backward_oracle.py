"""Pins of the backward oracle (``oracle.attention_bwd_ref``) and of the
column-major tables (``oracle.column_tables_ref``), independent of the
formulas they implement:

* central finite differences of the forward oracle ``attention_ref`` (the
  loss sum(do * o)), on tiny cases that cover every mask kind, GQA, the soft
  cap and decode positions;
* closed forms: a constant value vector makes o independent of q and k
  (dq = dk = 0, dv_j = sum_i p_ij do_i); do = 0 gives zero gradients;
* invariants: shifting every key by one vector leaves all gradients
  unchanged (softmax shift invariance, no cap); GQA equals MHA with the K/V
  heads repeated and their gradients summed;
* a hand-worked column table of a 4 x 4 causal block mask, and the column
  view against the row-major active list of ``mask_tables_ref``.
"""

import numpy as np
import pytest

from oracle import (allowed, attention_bwd_ref, attention_ref, column_tables_ref,
                    mask_tables_ref)


def _case(seed, B=1, Hq=2, Hkv=1, Lq=6, Lkv=8, dqk=3, dv=2, std=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Lq, dqk)) * std
    k = rng.standard_normal((B, Hkv, Lkv, dqk)) * std
    v = rng.standard_normal((B, Hkv, Lkv, dv))
    do = rng.standard_normal((B, Hq, Lq, dv))
    return q, k, v, do


def _loss(q, k, v, do, kw):
    o, _ = attention_ref(q, k, v, **kw)
    return float(np.sum(do * o))


def _fd_grad(x, f, eps=1e-5):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        x[idx] = old + eps
        fp = f()
        x[idx] = old - eps
        fm = f()
        x[idx] = old
        g[idx] = (fp - fm) / (2 * eps)
    return g


FD_CASES = [
    # (name, case kwargs, attention kwargs)
    ("dense", dict(Lq=5, Lkv=5), dict()),
    ("causal", dict(Lq=6, Lkv=6), dict(causal=True)),
    ("window", dict(Lq=7, Lkv=7), dict(window_left=2, window_right=1)),
    ("segments", dict(Lq=7, Lkv=7), dict(causal=True, seg_q=np.array([0, 0, 0, 1, 1, 2, 2]))),
    ("cap", dict(Lq=6, Lkv=6, std=2.0), dict(causal=True, soft_cap=1.5)),
    ("gqa", dict(Hq=4, Hkv=2, Lq=5, Lkv=5), dict(causal=True)),
    ("decode", dict(Lq=3, Lkv=8), dict(causal=True, window_left=4, q_offset=5)),
    ("empty_rows", dict(Lq=4, Lkv=6), dict(causal=True, window_left=1, q_offset=6)),
]


@pytest.mark.parametrize("name,ck,ak", FD_CASES, ids=[c[0] for c in FD_CASES])
def test_gradients_match_finite_differences(name, ck, ak):
    q, k, v, do = _case(11 + len(name), **ck)
    kw = dict(scale=0.7, **ak)
    dq, dk, dv = attention_bwd_ref(q, k, v, do, **kw)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        fd = _fd_grad(x, lambda: _loss(q, k, v, do, kw))
        np.testing.assert_allclose(g, fd, rtol=0, atol=2e-7)
    assert np.abs(dq).max() > 1e-3 or name == "empty_rows"


def test_empty_rows_have_zero_gradients():
    q, k, v, do = _case(3, Lq=4, Lkv=6)
    kw = dict(scale=0.5, causal=True, window_left=1, q_offset=6)
    # rows at positions 6..9 see keys [pos-1, 5]: row 0 sees key 5, rows 1.. see none
    a = allowed(np.arange(4)[:, None], np.arange(6)[None, :], L_q=4, L_kv=6, causal=True,
                window_left=1, q_offset=6)
    assert a[0].sum() == 1 and not a[1:].any()
    dq, dk, dv = attention_bwd_ref(q, k, v, do, **kw)
    assert np.all(dq[0, :, 1:] == 0)
    # one allowed key: p = 1, so dz = 0, dq = dk = 0 and dv_5 = do_0
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv[0, 0, 5], do[0, 0, 0] + do[0, 1, 0], atol=1e-15)
    assert np.all(dv[0, 0, :5] == 0)


def test_constant_values_closed_form():
    q, k, v, do = _case(5, Lq=6, Lkv=6)
    v[:] = np.array([0.3, -1.2])
    kw = dict(scale=0.9, causal=True)
    dq, dk, dv = attention_bwd_ref(q, k, v, do, **kw)
    np.testing.assert_allclose(dq, 0, atol=1e-12)
    np.testing.assert_allclose(dk, 0, atol=1e-12)
    # dv_j = sum_i p_ij do_i with p the causal softmax
    s = 0.9 * np.einsum("hid,jd->hij", q[0], k[0, 0])
    a = np.tril(np.ones((6, 6), bool))
    e = np.where(a, np.exp(s - s.max(axis=2, keepdims=True)), 0)
    p = e / e.sum(axis=2, keepdims=True)
    np.testing.assert_allclose(dv[0, 0], np.einsum("hij,hid->jd", p, do[0]), atol=1e-12)


def test_zero_upstream_gradient():
    q, k, v, do = _case(6)
    dq, dk, dv = attention_bwd_ref(q, k, v, np.zeros_like(do), scale=1.0, causal=True)
    assert not dq.any() and not dk.any() and not dv.any()


def test_key_shift_invariance():
    q, k, v, do = _case(7, Lq=7, Lkv=7)
    kw = dict(scale=0.8, window_left=3)
    g0 = attention_bwd_ref(q, k, v, do, **kw)
    g1 = attention_bwd_ref(q, k + np.array([0.5, -2.0, 1.0]), v, do, **kw)
    for a, b in zip(g0, g1):
        np.testing.assert_allclose(a, b, atol=1e-12)


def test_gqa_equals_repeated_mha():
    q, k, v, do = _case(8, Hq=4, Hkv=2, Lq=6, Lkv=6)
    kw = dict(scale=0.6, causal=True, soft_cap=2.0)
    dq, dk, dv = attention_bwd_ref(q, k, v, do, **kw)
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    dq1, dk1, dv1 = attention_bwd_ref(q, kr, vr, do, **kw)
    np.testing.assert_allclose(dq, dq1, atol=1e-12)
    np.testing.assert_allclose(dk, dk1.reshape(1, 2, 2, 6, 3).sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(dv, dv1.reshape(1, 2, 2, 6, 2).sum(axis=2), atol=1e-12)


def test_column_tables_hand_example():
    """4 x 4 causal block mask (full below the diagonal, partial on it).
    Row-major active order: (0,0)=0 (1,0)=1 (1,1)=2 (2,0)=3 (2,1)=4 (2,2)=5
    (3,0)=6 (3,1)=7 (3,2)=8 (3,3)=9."""
    bm = np.array([[1, 0, 0, 0], [2, 1, 0, 0], [2, 2, 1, 0], [2, 2, 2, 1]], np.int8)
    t = column_tables_ref(bm)
    assert t["col_ptr"].tolist() == [0, 4, 7, 9, 10]
    assert t["col_rows"].tolist() == [0, 1, 2, 3, 1, 2, 3, 2, 3, 3]
    assert t["col_entry"].tolist() == [0, 1, 3, 6, 2, 4, 7, 5, 8, 9]


@pytest.mark.parametrize("seed", range(6))
def test_column_tables_against_row_major_list(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(40, 200))
    kw = dict(causal=bool(rng.integers(0, 2)), window_left=int(rng.integers(-1, 60)))
    t = mask_tables_ref(L, L, 16, 8, **kw)
    c = column_tables_ref(t["block_mask"])
    assert c["col_ptr"][-1] == t["n_active"]
    # every active block appears once, at its row-major index
    seen = np.zeros(t["n_active"], bool)
    for col in range(t["n_kv_blocks"]):
        for x in range(c["col_ptr"][col], c["col_ptr"][col + 1]):
            e = c["col_entry"][x]
            assert t["active_rows"][e] == c["col_rows"][x] and t["active_cols"][e] == col
            seen[e] = True
    assert seen.all()
