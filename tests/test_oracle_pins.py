"""Pins of the float64 attention oracle against things other than itself:
the pages' worked examples, closed forms, scipy routines and brute force."""

import math

import numpy as np
import pytest
import scipy.special
from hypothesis import given, settings, strategies as st

from oracle import (allowed, attention_brute, attention_ref, merge_lse, merge_partials,
                    mle_safe_range, online_softmax_steps)
from tests.conftest import read_golden


def _floats(s):
    return [float(t) for t in s.split()]


@pytest.mark.parametrize("name", ["online_softmax_x6.txt",
                                  "online_softmax_exercise7.txt"])
def test_online_softmax_worked_examples(name):
    g = read_golden(name)
    x = _floats(g["x"])
    steps, sm = online_softmax_steps(x, int(g["block"]))
    dec = int(g["decimals"])
    assert [round(m, dec) for m, _ in steps] == _floats(g["steps_m"])
    assert [round(l, dec) for _, l in steps] == _floats(g["steps_l"])
    direct = scipy.special.softmax(np.asarray(x))
    assert np.max(np.abs(np.asarray(sm) - direct)) < 1e-15
    if "softmax" in g:
        assert [round(t, dec) for t in sm] == _floats(g["softmax"])


def test_online_softmax_shift_invariance():
    rng = np.random.default_rng(7)
    x = rng.normal(size=37) * 4
    _, a = online_softmax_steps(x, 5)
    _, b = online_softmax_steps(x + 123.25, 5)
    assert np.max(np.abs(np.asarray(a) - np.asarray(b))) < 1e-14


def test_merge_matches_whole_row():
    rng = np.random.default_rng(11)
    x = rng.normal(size=20) * 3
    v = rng.normal(size=(20, 5))
    cut = 8

    def part(xs, vs):
        m = xs.max()
        e = np.exp(xs - m)
        return m, e.sum(), e @ vs

    m, l, o = merge_partials(part(x[:cut], v[:cut]), part(x[cut:], v[cut:]))
    w = scipy.special.softmax(x)
    assert abs(m - x.max()) == 0
    assert abs(l - np.exp(x - x.max()).sum()) < 1e-13
    assert np.max(np.abs(o - w @ v)) < 1e-14
    # Order independence.
    m2, l2, o2 = merge_partials(part(x[cut:], v[cut:]), part(x[:cut], v[:cut]))
    assert m2 == m and abs(l2 - l) < 1e-14 and np.max(np.abs(o2 - o)) < 1e-15


@pytest.mark.parametrize("S", [1, 2, 3, 7])
def test_merge_lse_matches_whole_rows(S):
    """Split-K merge (joto.ai "LSE 与 Online Softmax"): outputs and lse of
    disjoint key ranges, each taken with scipy on its own range, merge into
    scipy's softmax and logsumexp of the whole masked row; ranges with no
    allowed key weigh nothing, and a row with none at all stays empty."""
    rng = np.random.default_rng(100 + S)
    R, N, d = 6, 23, 4
    x = rng.normal(size=(R, N)) * 4
    allowed_ = rng.random((R, N)) < 0.6
    allowed_[1, 5:] = False            # keys only in the first range(s)
    allowed_[4, :] = False             # a row with no allowed key
    v = rng.normal(size=(N, d))
    cuts = np.linspace(0, N, S + 1).astype(int)
    o_parts, lse_parts = [], []
    for s in range(S):
        a, b = cuts[s], cuts[s + 1]
        xs = np.where(allowed_[:, a:b], x[:, a:b], -np.inf)
        lse_s = scipy.special.logsumexp(xs, axis=1)
        w = np.zeros_like(xs)
        ok = np.isfinite(lse_s)
        w[ok] = scipy.special.softmax(xs[ok], axis=1)
        o_parts.append(w @ v[a:b])
        lse_parts.append(lse_s)
    o, lse = merge_lse(o_parts, lse_parts)
    xf = np.where(allowed_, x, -np.inf)
    full = np.isfinite(scipy.special.logsumexp(xf, axis=1))
    assert np.array_equal(full, np.isfinite(lse))
    ref_w = scipy.special.softmax(xf[full], axis=1)
    assert np.max(np.abs(o[full] - ref_w @ v)) < 1e-13
    assert np.max(np.abs(lse[full] - scipy.special.logsumexp(xf[full], axis=1))) < 1e-13
    assert np.all(o[~full] == 0) and np.all(np.isneginf(lse[~full]))


def _rand_case(seed, B, Hq, Hkv, L, dqk, dv, std=1.0):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(B, Hq, L, dqk)) * std
    k = rng.normal(size=(B, Hkv, L, dqk)) * std
    v = rng.normal(size=(B, Hkv, L, dv))
    return q, k, v


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 10_000),
       L=st.integers(1, 11),
       dqk=st.integers(1, 4), dv=st.integers(1, 4),
       group=st.sampled_from([1, 2]), Hkv=st.sampled_from([1, 2]),
       B=st.sampled_from([1, 2]),
       causal=st.booleans(),
       wl=st.integers(-1, 5), wr=st.integers(-1, 5),
       use_seg=st.booleans(), cap=st.sampled_from([0.0, 0.7, 3.0]))
def test_ref_matches_brute_force(seed, L, dqk, dv, group, Hkv, B, causal, wl,
                                 wr, use_seg, cap):
    Hq = Hkv * group
    q, k, v = _rand_case(seed, B, Hq, Hkv, L, dqk, dv)
    rng = np.random.default_rng(seed + 1)
    seg = rng.integers(0, 3, size=(B, L)) if use_seg else None
    kw = dict(scale=0.8, soft_cap=cap, causal=causal, window_left=wl,
              window_right=wr, seg_q=seg, seg_kv=seg)
    o, lse = attention_ref(q, k, v, panel=3, **kw)
    ob, lb = attention_brute(q, k, v, **kw)
    ob = np.asarray(ob)
    lb = np.asarray(lb)
    assert np.array_equal(np.isinf(lse), np.isinf(lb))
    fin = np.isfinite(lb)
    assert np.max(np.abs(lse[fin] - lb[fin]), initial=0) < 1e-12
    assert np.max(np.abs(o - ob)) < 1e-12


def test_probability_rows_sum_to_one_and_o_in_hull():
    q, k, v = _rand_case(3, 1, 2, 2, 64, 8, 4)
    ones = np.ones_like(v)
    o, _ = attention_ref(q, k, ones, scale=0.5, causal=True, window_left=9)
    assert np.max(np.abs(o - 1.0)) < 1e-14
    o, _ = attention_ref(q, k, v, scale=0.5, causal=True, window_left=9)
    for d in range(v.shape[3]):
        assert np.all(o[..., d] <= v[..., d].max() + 1e-12)
        assert np.all(o[..., d] >= v[..., d].min() - 1e-12)


def test_causal_first_row_is_v0():
    q, k, v = _rand_case(4, 1, 3, 3, 40, 16, 8)
    scale = 1 / math.sqrt(16)
    o, lse = attention_ref(q, k, v, scale=scale, causal=True)
    assert np.array_equal(o[0, :, 0, :], v[0, :, 0, :])
    s00 = scale * np.einsum("hd,hd->h", q[0, :, 0], k[0, :, 0])
    assert np.max(np.abs(lse[0, :, 0] - s00)) < 1e-14


def test_dense_equals_scipy_softmax():
    q, k, v = _rand_case(5, 1, 2, 2, 50, 16, 12)
    scale = 0.3
    o, lse = attention_ref(q, k, v, scale=scale, panel=7)
    for h in range(2):
        s = scale * q[0, h] @ k[0, h].T
        assert np.max(np.abs(o[0, h] - scipy.special.softmax(s, axis=1) @ v[0, h])) < 1e-13
        assert np.max(np.abs(lse[0, h] - scipy.special.logsumexp(s, axis=1))) < 1e-13


def test_lse_matches_scipy_logsumexp_on_masked_rows():
    q, k, v = _rand_case(6, 1, 1, 1, 70, 8, 8)
    seg = np.repeat(np.arange(5), 14)
    scale, cap = 0.9, 2.5
    _, lse = attention_ref(q, k, v, scale=scale, soft_cap=cap, causal=True,
                           window_left=20, seg_q=seg)
    s = cap * np.tanh(scale * (q[0, 0] @ k[0, 0].T) / cap)
    for i in range(70):
        js = [j for j in range(70) if j <= i and i - j <= 20 and seg[i] == seg[j]]
        assert abs(lse[0, 0, i] - scipy.special.logsumexp(s[i, js])) < 1e-13


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v = _rand_case(8, 2, 8, 2, 33, 8, 8)
    kw = dict(scale=0.4, causal=True, window_left=12)
    o, lse = attention_ref(q, k, v, **kw)
    o2, lse2 = attention_ref(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), **kw)
    assert np.max(np.abs(o - o2)) == 0 and np.max(np.abs(lse - lse2)) == 0
    # Head 5 reads kv head 1 (contiguous groups of 4): differs from kv head 0.
    o3, _ = attention_ref(q[:, 5:6], k[:, 1:2], v[:, 1:2], **kw)
    assert np.max(np.abs(o3[:, 0] - o[:, 5])) == 0


def test_soft_cap_bounds_and_limit():
    q, k, v = _rand_case(9, 1, 1, 1, 30, 8, 8, std=3.0)
    cap = 2.0
    _, lse = attention_ref(q, k, v, scale=1.0, soft_cap=cap, causal=True)
    # lse_i = ln sum_{j<=i} e^{s_ij} with |s_ij| < cap:
    n = np.arange(1, 31)
    assert np.all(lse[0, 0] < cap + np.log(n))
    assert np.all(lse[0, 0] > -cap + np.log(n))
    o_inf, lse_inf = attention_ref(q, k, v, scale=1.0, causal=True)
    # cap * tanh(s / cap) = s - s^3 / (3 cap^2) + ...: at cap 1e8 and
    # |s| < 100 the difference is below 1e-10.
    o_big, lse_big = attention_ref(q, k, v, scale=1.0, soft_cap=1e8, causal=True)
    assert np.max(np.abs(o_big - o_inf)) < 1e-9
    assert np.max(np.abs(lse_big - lse_inf)) < 1e-9


def test_rows_subset_and_empty_rows():
    q, k, v = _rand_case(10, 1, 2, 1, 48, 8, 8)
    seg_q = np.repeat(np.arange(4), 12)
    seg_kv = seg_q.copy()
    seg_kv[seg_kv == 2] = 9    # queries of document 2 see no key
    kw = dict(scale=0.5, causal=True, seg_q=seg_q, seg_kv=seg_kv)
    o, lse = attention_ref(q, k, v, **kw)
    rows = np.array([47, 0, 25, 13])
    o2, lse2 = attention_ref(q, k, v, rows=rows, **kw)
    assert np.array_equal(o[:, :, rows], o2) and np.array_equal(lse[:, :, rows], lse2)
    empty = seg_q == 2
    assert np.all(np.isneginf(lse[:, :, empty])) and np.all(o[:, :, empty] == 0)
    assert np.all(np.isfinite(lse[:, :, ~empty]))


def test_allowed_definition_examples():
    i = np.arange(6)[:, None]
    j = np.arange(6)[None, :]
    a = allowed(i, j, L_q=6, L_kv=6, causal=True, window_left=2)
    expect = np.array([[1 if (jj <= ii and ii - jj <= 2) else 0
                        for jj in range(6)] for ii in range(6)], bool)
    assert np.array_equal(a, expect)
    # padding beyond the lengths is masked
    a = allowed(np.arange(8)[:, None], np.arange(8)[None, :], L_q=5, L_kv=6)
    assert a[:5, :6].all() and not a[5:, :].any() and not a[:, 6:].any()
    # right window only
    a = allowed(i, j, L_q=6, L_kv=6, window_right=1)
    assert a[0, 1] and not a[0, 2] and a[5, 0]


# ---------------------------------------------------------- max logit estimate


def test_mle_safe_range_exercise10():
    """The safe interval of the Max Logit Estimate constant against the
    worked answer of Lecture 13 exercise 10 (section 5.4)."""
    g = read_golden("mle_exercise10.txt")
    lo, hi = mle_safe_range(float(g["max_logit"]), float(g["min_row_max"]))
    assert abs(lo - float(g["lower"])) < 0.05      # 40 - 88.72
    assert abs(hi - float(g["upper"])) < 0.5       # -30 + 87.34 (page rounds to 87)
    # The float32 limits it uses are those of numpy's float32.
    assert abs((40 - lo) - math.log(float(np.finfo(np.float32).max))) < 1e-12
    assert abs((hi + 30) + math.log(float(np.finfo(np.float32).tiny))) < 1e-12


@pytest.mark.parametrize("c", [-20.0, 0.0, 3.0, 60.0])
@pytest.mark.parametrize("mask", [dict(causal=True), dict(causal=True, window_left=5),
                                  dict(causal=False, seg="split"), dict(causal=True, cap=2.5)])
def test_mle_constant_cancels(c, mask):
    """Section 5.4: any constant in place of the row max gives the same
    softmax; lse carries the constant back (lse = c + ln l)."""
    rng = np.random.default_rng(7)
    B, H, L, d = 2, 2, 24, 8
    q = rng.standard_normal((B, H, L, d))
    k = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    kw = dict(scale=0.5, causal=mask.get("causal", False),
              window_left=mask.get("window_left", -1), soft_cap=mask.get("cap", 0.0))
    if mask.get("seg") == "split":
        kw["seg_q"] = np.repeat(np.arange(3), 8).astype(np.int32)
    o0, l0 = attention_ref(q, k, v, **kw)
    o1, l1 = attention_ref(q, k, v, max_logit=c, **kw)
    assert np.max(np.abs(o1 - o0)) < 1e-12
    assert np.max(np.abs(l1 - l0)) < 1e-10
    # The unshifted brute-force definition agrees too.
    ob, lb = attention_brute(q, k, v, **kw)
    assert np.max(np.abs(o1 - np.asarray(ob))) < 1e-12
    assert np.max(np.abs(l1 - np.asarray(lb))) < 1e-10


@pytest.mark.parametrize("mk", [dict(causal=True), dict(causal=True, window_left=9),
                                dict(window_left=5, window_right=3), dict(causal=True, segs=True)])
def test_decode_rows_are_rows_of_aligned_attention(mk):
    """Queries at key positions q_offset + i (decoding the last L_q of L_kv
    positions, q_offset = L_kv - L_q) see exactly what those rows see in
    the aligned attention over all L_kv positions."""
    B, H, L, Lq, d = 2, 3, 37, 5, 4
    q, k, v = _rand_case(5, B, H, H, L, d, d)
    mk = dict(mk)
    seg = None
    if mk.pop("segs", False):
        seg = np.repeat(np.arange(5), 8)[:L].astype(np.int64)
    o_full, l_full = attention_ref(q, k, v, scale=0.7, seg_q=seg, **mk)
    o_dec, l_dec = attention_ref(q[:, :, L - Lq:], k, v, scale=0.7, q_offset=L - Lq,
                                 seg_q=None if seg is None else seg[L - Lq:], seg_kv=seg, **mk)
    assert np.max(np.abs(o_dec - o_full[:, :, L - Lq:])) < 1e-12
    assert np.max(np.abs(l_dec - l_full[:, :, L - Lq:])) < 1e-12


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 10_000), Lq=st.integers(1, 6), Lkv=st.integers(1, 11),
       off=st.integers(0, 12), causal=st.booleans(), wl=st.integers(-1, 5),
       wr=st.integers(-1, 5), cap=st.sampled_from([0.0, 2.0]))
def test_ref_matches_brute_force_with_offsets(seed, Lq, Lkv, off, causal, wl, wr, cap):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(1, 2, Lq, 3))
    k = rng.normal(size=(1, 1, Lkv, 3))
    v = rng.normal(size=(1, 1, Lkv, 2))
    kw = dict(scale=0.9, soft_cap=cap, causal=causal, window_left=wl, window_right=wr,
              q_offset=off)
    o, lse = attention_ref(q, k, v, panel=2, **kw)
    ob, lb = attention_brute(q, k, v, **kw)
    assert np.max(np.abs(o - np.asarray(ob))) < 1e-12
    lb = np.asarray(lb)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    assert np.max(np.abs(lse[fin] - lb[fin]), initial=0.0) < 1e-12
