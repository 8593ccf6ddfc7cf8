"""Pins of the reference MaskInfo tables: the pages' worked examples and a
brute-force element scan written with plain loops."""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import mask_tables_ref
from tests.conftest import read_golden

CODE = {".": 0, "P": 1, "F": 2}


def _grid(g):
    return np.array([[CODE[c] for c in row] for row in g["grid"]], dtype=np.int8)


def _tables_from_golden(g):
    L = int(g["L"])
    kw = dict(causal=bool(int(g.get("causal", "0"))))
    if "doc_lengths" in g:
        lens = [int(t) for t in g["doc_lengths"].split()]
        kw["seg_q"] = np.repeat(np.arange(len(lens)), lens).astype(np.int32)
    return mask_tables_ref(L, L, int(g["block_q"]), int(g["block_kv"]), **kw)


@pytest.mark.parametrize("name", ["classes_causal_L8_b2.txt",
                                  "maskinfo_causal_4096_1024x2048.txt",
                                  "maskinfo_exercise11.txt",
                                  "maskinfo_exercise12.txt"])
def test_block_classes_match_pages(name):
    g = read_golden(name)
    t = _tables_from_golden(g)
    assert np.array_equal(t["block_mask"], _grid(g))
    codes = t["block_code"]
    for key, val in (("n_active", len(codes)),
                     ("n_partial", int((codes == 1).sum())),
                     ("n_full", int((codes == 2).sum())),
                     ("n_patterns", t["n_patterns"])):
        if key in g:
            assert val == int(g[key]), key


def test_maskinfo_section_6_2_bounds_and_patterns():
    g = read_golden("maskinfo_causal_4096_1024x2048.txt")
    t = _tables_from_golden(g)
    bs = [bool(b & 1) for b in t["bounds"]]
    be = [bool(b & 2) for b in t["bounds"]]
    assert bs == [c == "T" for c in g["bounds_start"].split()]
    assert be == [c == "T" for c in g["bounds_end"].split()]
    pos = {(int(r), int(c)): n for n, (r, c) in
           enumerate(zip(t["active_rows"], t["active_cols"]))}
    for pair in g["same_pattern"].split():
        a, b = pair.split("=")
        ra, ca = map(int, a.split(","))
        rb, cb = map(int, b.split(","))
        assert t["mask_next"][pos[(ra, ca)]] == t["mask_next"][pos[(rb, cb)]]
    assert sorted(set(t["mask_next"][t["block_code"] == 1].tolist())) == [0, 1]


def test_pattern_counts_section_6_6():
    g = read_golden("pattern_counts_16384_b1024.txt")
    L, b = int(g["L"]), int(g["block_q"])
    t = mask_tables_ref(L, L, b, int(g["block_kv"]), causal=True)
    assert t["n_patterns"] == int(g["causal_patterns"])
    assert t["partial_mask_blocks"].nbytes == int(g["causal_pattern_bytes"])
    t = mask_tables_ref(L, L, b, int(g["block_kv"]), causal=True,
                        window_left=int(g["window_left"]))
    assert t["n_patterns"] == int(g["window_patterns"])
    assert t["partial_mask_blocks"].nbytes == int(g["window_pattern_bytes"])


def _brute_tables(L_q, L_kv, bq, bkv, causal, wl, wr, seg_q, seg_kv, q_offset=0):
    """Independent scan with scalar loops (no numpy mask algebra)."""
    nq = (L_q + bq - 1) // bq
    nkv = (L_kv + bkv - 1) // bkv

    def ok(i, j):
        if i >= L_q or j >= L_kv:
            return False
        pos = i + q_offset
        if causal and j > pos:
            return False
        if wl >= 0 and pos - j > wl:
            return False
        if wr >= 0 and j - pos > wr:
            return False
        if seg_q is not None and seg_q[i] != seg_kv[j]:
            return False
        return True

    classes, pats, order, nxt = [], [], [], []
    for r in range(nq):
        row = []
        for c in range(nkv):
            bits = tuple(tuple(1 if ok(r * bq + a, c * bkv + b) else 0
                               for b in range(bkv)) for a in range(bq))
            n = sum(map(sum, bits))
            code = 0 if n == 0 else (2 if n == bq * bkv else 1)
            row.append(code)
            if code == 1:
                if bits not in pats:
                    pats.append(bits)
                nxt.append(pats.index(bits))
            elif code == 2:
                nxt.append(-1)
        classes.append(row)
    return classes, pats, nxt


@settings(max_examples=80, deadline=None)
@given(L=st.integers(1, 40), bq=st.sampled_from([1, 2, 3, 4, 8]),
       bkv=st.sampled_from([1, 2, 4, 5, 8]), causal=st.booleans(),
       wl=st.integers(-1, 9), wr=st.integers(-1, 9), use_seg=st.booleans(),
       seed=st.integers(0, 1000))
def test_tables_match_brute_scan(L, bq, bkv, causal, wl, wr, use_seg, seed):
    seg = None
    if use_seg:
        seg = np.random.default_rng(seed).integers(0, 3, size=L).astype(np.int32)
    t = mask_tables_ref(L, L, bq, bkv, causal=causal, window_left=wl,
                        window_right=wr, seg_q=seg, seg_kv=seg)
    classes, pats, nxt = _brute_tables(L, L, bq, bkv, causal, wl, wr, seg, seg)
    assert t["block_mask"].tolist() == classes
    assert t["mask_next"].tolist() == nxt
    assert t["n_patterns"] == len(pats)
    for p, bits in zip(t["partial_mask_blocks"], pats):
        assert p.tolist() == [list(r) for r in bits]
    # CSR, active lists, bounds and launch order from their definitions.
    rows = [r for r in range(len(classes)) for c in range(len(classes[r]))
            if classes[r][c]]
    cols = [c for r in range(len(classes)) for c in range(len(classes[r]))
            if classes[r][c]]
    assert t["active_rows"].tolist() == rows and t["active_cols"].tolist() == cols
    lens = [sum(1 for c in row if c) for row in classes]
    assert t["row_ptr"].tolist() == [sum(lens[:r]) for r in range(len(lens) + 1)]
    exp_bounds = []
    for n in lens:
        exp_bounds += [(1 if a == 0 else 0) | (2 if a == n - 1 else 0)
                       for a in range(n)]
    assert t["bounds"].tolist() == exp_bounds
    order = t["row_order"].tolist()
    assert sorted(order) == list(range(len(lens)))
    for a, b in zip(order, order[1:]):
        assert lens[a] > lens[b] or (lens[a] == lens[b] and a < b)


@settings(max_examples=60, deadline=None)
@given(Lq=st.integers(1, 20), Lkv=st.integers(1, 40), off=st.integers(0, 30),
       bq=st.sampled_from([1, 2, 4]), bkv=st.sampled_from([1, 3, 8]), causal=st.booleans(),
       wl=st.integers(-1, 9), wr=st.integers(-1, 9), use_seg=st.booleans(),
       seed=st.integers(0, 1000))
def test_tables_match_brute_scan_with_offsets(Lq, Lkv, off, bq, bkv, causal, wl, wr, use_seg,
                                              seed):
    """Queries at key positions q_offset + i (decode shapes, L_q != L_kv)."""
    sq = skv = None
    if use_seg:
        rng = np.random.default_rng(seed)
        sq = rng.integers(0, 3, size=Lq).astype(np.int32)
        skv = rng.integers(0, 3, size=Lkv).astype(np.int32)
    t = mask_tables_ref(Lq, Lkv, bq, bkv, causal=causal, window_left=wl, window_right=wr,
                        seg_q=sq, seg_kv=skv, q_offset=off)
    classes, pats, nxt = _brute_tables(Lq, Lkv, bq, bkv, causal, wl, wr, sq, skv, off)
    assert t["block_mask"].tolist() == classes
    assert t["mask_next"].tolist() == nxt
    for p, bits in zip(t["partial_mask_blocks"], pats):
        assert p.tolist() == [list(r) for r in bits]
