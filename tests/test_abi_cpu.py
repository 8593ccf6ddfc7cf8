"""CPU tests of the C ABI: exported symbols, bit-exact mask tables against
the oracle, and the documented error codes (no GPU needed: validation runs
before any device call and attn_mask_compile is host code)."""

import ctypes
import math
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from block_sparse_flash_amd import _lib, compile_mask, fwd_tile
from block_sparse_flash_amd.inputs import WORKLOADS, segment_ids
from oracle import mask_tables_ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TABLE_FIELDS = ["block_mask", "active_rows", "active_cols", "block_code",
                "mask_next", "bounds", "row_ptr", "row_order",
                "partial_mask_blocks"]


def _declared_functions():
    names = []
    for h in os.listdir(os.path.join(ROOT, "include")):
        if not h.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, re.M):
            if not m.group(0).lstrip().startswith(("typedef", "#", "enum", "struct")):
                names.append(m.group(1))
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTED), declared
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.splash_version() == 111


def _assert_tables_equal(t, ref):
    for key in ("n_q_blocks", "n_kv_blocks", "n_active", "n_partial", "n_patterns"):
        assert getattr(t, key) == ref[key], key
    for name in TABLE_FIELDS:
        a, b = getattr(t, name), ref[name]
        assert a.dtype == b.dtype and a.shape == b.shape, name
        assert np.array_equal(a, b), name


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_tables_bit_exact_on_workloads(name):
    w = WORKLOADS[name]
    bq, bkv = fwd_tile(w.dtype, w.d_qk, w.d_v)
    seg = segment_ids(w.L, w.seed, w.seg_min, w.seg_max) if w.segments else None
    kw = dict(causal=w.causal, window_left=w.window_left,
              window_right=w.window_right, seg_q=seg, seg_kv=seg)
    t = compile_mask(w.L, bq, bkv, **kw)
    _assert_tables_equal(t, mask_tables_ref(w.L, w.L, bq, bkv, **kw))


@settings(max_examples=150, deadline=None)
@given(Lq=st.integers(0, 150), dL=st.integers(-20, 20),
       bq=st.sampled_from([1, 2, 3, 8, 16, 64]), bkv=st.sampled_from([1, 4, 5, 16, 64]),
       causal=st.booleans(), wl=st.integers(-1, 40), wr=st.integers(-1, 40),
       seg_mode=st.sampled_from(["none", "same", "split", "noncontig"]),
       seed=st.integers(0, 10_000))
def test_tables_bit_exact_random(Lq, dL, bq, bkv, causal, wl, wr, seg_mode, seed):
    rng = np.random.default_rng(seed)
    Lkv = Lq if seg_mode in ("same",) else max(0, Lq + dL)
    sq = skv = None
    if seg_mode == "same" and Lq > 0:
        sq = np.sort(rng.integers(0, 5, size=Lq)).astype(np.int32)
    elif seg_mode == "split" and Lq > 0 and Lkv > 0:
        sq = np.sort(rng.integers(0, 4, size=Lq)).astype(np.int32)
        skv = np.sort(rng.integers(0, 4, size=Lkv)).astype(np.int32)
    elif seg_mode == "noncontig" and Lq > 0 and Lkv > 0:
        sq = rng.integers(0, 3, size=Lq).astype(np.int32)
        skv = rng.integers(0, 3, size=Lkv).astype(np.int32)
    kw = dict(causal=causal, window_left=wl, window_right=wr, seg_q=sq, seg_kv=skv)
    t = compile_mask(Lq, bq, bkv, L_kv=Lkv, **kw)
    _assert_tables_equal(t, mask_tables_ref(Lq, Lkv, bq, bkv, **kw))


@settings(max_examples=100, deadline=None)
@given(Lq=st.integers(1, 80), Lkv=st.integers(1, 200), off=st.integers(0, 150),
       bq=st.sampled_from([1, 4, 16, 64]), bkv=st.sampled_from([1, 5, 16, 64]),
       causal=st.booleans(), wl=st.integers(-1, 40), wr=st.integers(-1, 40),
       use_seg=st.booleans(), seed=st.integers(0, 10_000))
def test_tables_bit_exact_with_offsets(Lq, Lkv, off, bq, bkv, causal, wl, wr, use_seg, seed):
    """Decode shapes: query row i at key position q_offset + i."""
    rng = np.random.default_rng(seed)
    sq = skv = None
    if use_seg:
        sq = rng.integers(0, 3, size=Lq).astype(np.int32)
        skv = np.sort(rng.integers(0, 3, size=Lkv)).astype(np.int32)
    kw = dict(causal=causal, window_left=wl, window_right=wr, seg_q=sq, seg_kv=skv)
    t = compile_mask(Lq, bq, bkv, L_kv=Lkv, q_offset=off, **kw)
    _assert_tables_equal(t, mask_tables_ref(Lq, Lkv, bq, bkv, q_offset=off, **kw))


def test_empty_and_no_allowed_mask():
    t = compile_mask(0, 64, 64, causal=True)
    assert t.n_q_blocks == 0 and t.n_active == 0 and t.row_ptr.tolist() == [0]
    # Every query in its own segment, keys in another: nothing is allowed.
    t = compile_mask(100, 16, 16, seg_q=np.zeros(100, np.int32),
                     seg_kv=np.ones(100, np.int32))
    assert t.n_active == 0 and t.row_ptr.tolist() == [0] * (t.n_q_blocks + 1)


# ---------------------------------------------------------------- errors


def _compile_raw(desc, tables=False, sizes=None):
    lib = _lib.load()
    sz = sizes or _lib.MaskSizes()
    tabs = _lib.MaskTablesC() if tables else None
    return lib.attn_mask_compile(ctypes.byref(desc) if desc else None,
                                 ctypes.byref(sz), ctypes.byref(tabs) if tabs else None)


def test_mask_compile_errors():
    lib = _lib.load()
    assert lib.attn_mask_compile(None, None, None) == 1
    bad = [
        _lib.MaskDesc(-1, 10, 4, 4, 0, -1, -1, None, None),
        _lib.MaskDesc(10, 10, 0, 4, 0, -1, -1, None, None),
        _lib.MaskDesc(10, 10, 4, -3, 0, -1, -1, None, None),
        _lib.MaskDesc(10, 10, 4, 4, 2, -1, -1, None, None),
        _lib.MaskDesc(10, 10, 4, 4, 0, -2, -1, None, None),
        _lib.MaskDesc(10, 10, 4, 4, 0, -1, -7, None, None),
        _lib.MaskDesc(10, 10, 4, 4, 1, -1, -1, None, None, -1),
    ]
    for d in bad:
        assert _compile_raw(d) == 1
        assert lib.splash_last_error()
    seg = np.zeros(10, np.int32)
    d = _lib.MaskDesc(10, 12, 4, 4, 0, -1, -1, seg.ctypes.data_as(ctypes.c_void_p), None)
    assert _compile_raw(d) == 1     # seg_kv NULL needs L_kv == L_q
    d = _lib.MaskDesc(10, 10, 4, 4, 0, -1, -1, None, seg.ctypes.data_as(ctypes.c_void_p))
    assert _compile_raw(d) == 1     # seg_kv without seg_q
    # Phase 2 with sizes that do not belong to this mask.
    d = _lib.MaskDesc(64, 64, 8, 8, 1, -1, -1, None, None)
    sizes = _lib.MaskSizes(8, 8, 1, 1, 1)
    assert _compile_raw(d, tables=True, sizes=sizes) == 2
    assert b"do not match" in lib.splash_last_error()


def test_fwd_tile_errors_and_values():
    lib = _lib.load()
    a, b = ctypes.c_int32(), ctypes.c_int32()
    assert lib.splash_fwd_tile(7, 128, 128, ctypes.byref(a), ctypes.byref(b)) == 3
    assert lib.splash_fwd_tile(1, 96, 128, ctypes.byref(a), ctypes.byref(b)) == 4
    assert lib.splash_fwd_tile(0, 192, 128, ctypes.byref(a), ctypes.byref(b)) == 4
    assert lib.splash_fwd_tile(1, 128, 128, None, ctypes.byref(b)) == 1
    assert fwd_tile("bf16", 128, 128) == (256, 64)
    assert fwd_tile("bf16", 192, 128) == (256, 64)
    assert fwd_tile("f32", 64, 64) == (64, 64)


def test_fwd_tiles_and_bwd_tile():
    """The block-size sweep (Lecture 13 sections 5.3 and 6.5): 128/128 bf16
    heads have kernels for 128 or 256 rows by 64 or 128 keys, the default
    first; other head dims and f32 have their default tile only."""
    from block_sparse_flash_amd import bwd_tile, fwd_tiles
    lib = _lib.load()
    t = fwd_tiles("bf16", 128, 128)
    assert t[0] == fwd_tile("bf16", 128, 128)
    assert sorted(t) == [(64, 64), (128, 64), (128, 128), (256, 64), (256, 128)]
    for dims in [(192, 128), (192, 64), (64, 64), (128, 64), (64, 128)]:
        assert fwd_tiles("bf16", *dims) == [fwd_tile("bf16", *dims)]
    assert fwd_tiles("f32", 128, 128) == [(64, 64)]
    n = ctypes.c_int32()
    assert lib.splash_fwd_tiles(1, 128, 128, None, None, 0, ctypes.byref(n)) == 0 and n.value == 5
    assert lib.splash_fwd_tiles(1, 128, 128, None, None, 2, ctypes.byref(n)) == 1
    assert lib.splash_fwd_tiles(1, 128, 128, None, None, 0, None) == 1
    assert lib.splash_fwd_tiles(1, 96, 128, None, None, 0, ctypes.byref(n)) == 4
    assert bwd_tile("bf16", 128, 128) == (256, 64) and bwd_tile("bf16", 64, 64) == (256, 64)
    a, b = ctypes.c_int32(), ctypes.c_int32()
    assert lib.splash_bwd_tile(1, 192, 128, ctypes.byref(a), ctypes.byref(b)) == 0
    assert (a.value, b.value) == (256, 64)
    assert lib.splash_bwd_tile(1, 192, 64, ctypes.byref(a), ctypes.byref(b)) == 4
    assert lib.splash_bwd_tile(1, 128, 64, ctypes.byref(a), ctypes.byref(b)) == 4
    assert lib.splash_bwd_tile(0, 128, 128, ctypes.byref(a), ctypes.byref(b)) == 4
    assert lib.splash_bwd_tile(3, 128, 128, ctypes.byref(a), ctypes.byref(b)) == 3


@pytest.mark.parametrize("bq,bkv,d,code", [
    (256, 128, 128, 0), (128, 64, 128, 0), (128, 128, 128, 0),   # sweep tiles of 128/128
    (64, 64, 128, 0),                                            # decode tile
    (256, 128, 64, 2), (128, 64, 64, 2),                         # not built for 64/64
    (64, 64, 64, 2), (512, 64, 128, 2), (256, 32, 128, 2),
])
def test_forward_accepts_built_tiles_only(bq, bkv, d, code):
    """Validation accepts tables of any tile with a kernel and rejects the
    rest before touching device memory (the fake pointers are never read:
    B = 0 makes an accepted call a no-op)."""
    lib = _lib.load()
    args = _good_args(B=0, d_qk=d, d_v=d, block_q=bq, block_kv=bkv, n_q_blocks=(256 + bq - 1) // bq)
    assert lib.splash_attn_fwd(ctypes.byref(args), None) == code


def _good_args(**over):
    """Arguments that pass validation (with fake, aligned device pointers);
    each test changes one field so that validation must reject it before
    any pointer is used."""
    fake = 0x10000
    a = dict(dtype=1, B=1, Hq=2, Hkv=1, L=256, d_qk=128, d_v=128,
             q=fake, k=fake, v=fake, o=fake, lse=None,
             causal=1, window_left=-1, window_right=-1, seg_q=None, seg_kv=None,
             block_q=256, block_kv=64, n_q_blocks=1, n_active=3, n_patterns=1,
             row_ptr=fake, row_order=fake, active_cols=fake, block_code=fake,
             mask_next=fake, partial_mask_blocks=fake, mask_mode=0,
             scale=0.088, soft_cap=0.0)
    a.update(over)
    return _lib.FwdArgs(**a)


@pytest.mark.parametrize("over,code", [
    (dict(dtype=5), 3),
    (dict(B=-1), 1),
    (dict(Hkv=0), 1),
    (dict(Hq=3, Hkv=2), 2),
    (dict(d_qk=96), 4),
    (dict(dtype=0, d_qk=192), 4),
    (dict(causal=3), 1),
    (dict(window_left=-2), 1),
    (dict(mask_mode=9), 1),
    (dict(scale=0.0), 1),
    (dict(scale=-1.0), 1),
    (dict(scale=math.nan), 1),
    (dict(scale=math.inf), 1),
    (dict(soft_cap=math.nan), 1),
    (dict(soft_cap=math.inf), 1),
    (dict(block_kv=32), 2),
    (dict(n_q_blocks=2), 2),
    (dict(q=None), 1),
    (dict(o=0x10008), 1),
    (dict(row_ptr=None), 1),
    (dict(active_cols=None), 1),
    (dict(mask_next=None), 1),
    (dict(mask_mode=1, partial_mask_blocks=None), 1),
    (dict(seg_kv=0x10000), 1),
    (dict(n_active=-1), 1),
    (dict(use_max_logit=2), 1),
    (dict(use_max_logit=1, max_logit=math.nan), 1),
    (dict(use_max_logit=1, max_logit=math.inf), 1),
    (dict(Hq=1 << 20, L=1 << 20, n_q_blocks=4096), 2),   # items beyond int32
    (dict(L_kv=-1), 1),
    (dict(q_offset=-1), 1),
    (dict(dtype=0, block_q=64, n_q_blocks=4, L_kv=300), 4),    # decode shapes: bf16 only
    (dict(dtype=0, block_q=64, n_q_blocks=4, q_offset=8), 4),
    (dict(L_kv=512, seg_q=0x10000), 1),                        # seg_kv needed
    (dict(L_kv=1 << 24), 2),                                   # key bytes beyond int32
    (dict(q_offset=(1 << 31) - 300), 2),                       # positions beyond int32
])
def test_forward_validation_errors(over, code):
    lib = _lib.load()
    args = _good_args(**over)
    assert lib.splash_attn_fwd(ctypes.byref(args), None) == code
    assert len(lib.splash_last_error()) > 0


def test_forward_null_args_and_noops():
    lib = _lib.load()
    assert lib.splash_attn_fwd(None, None) == 1
    # B == 0, Hq == 0 or L == 0 is valid and launches nothing.
    assert lib.splash_attn_fwd(ctypes.byref(_good_args(B=0)), None) == 0
    assert lib.splash_attn_fwd(ctypes.byref(_good_args(Hq=0)), None) == 0
    assert lib.splash_attn_fwd(ctypes.byref(_good_args(L=0, n_q_blocks=0)), None) == 0
    assert lib.splash_last_error() == b""


def test_split_workspace_bytes():
    lib = _lib.load()
    nb = ctypes.c_int64()
    assert lib.splash_split_workspace_bytes(3, 2, 4, 1000, 128, ctypes.byref(nb)) == 0
    assert nb.value == 3 * 2 * 4 * 1000 * (128 + 1) * 4
    for bad in [(0, 1, 1, 1, 64), (_lib.SPLASH_MAX_SPLIT + 1, 1, 1, 1, 64), (2, -1, 1, 1, 64),
                (2, 1, 1, 1, 0)]:
        assert lib.splash_split_workspace_bytes(*bad, ctypes.byref(nb)) == 1
    assert lib.splash_split_workspace_bytes(2, 1, 1, 1, 64, None) == 1


@pytest.mark.parametrize("over,n_split,ws,ws_bytes,code", [
    (dict(dtype=0, block_q=64, n_q_blocks=4), 2, 0x20000, 1 << 30, 4),  # f32: bf16 only
    (dict(), 0, 0x20000, 1 << 30, 1),                 # n_split < 1
    (dict(), 65, 0x20000, 1 << 30, 1),                # n_split > SPLASH_MAX_SPLIT
    (dict(), 2, None, 1 << 30, 1),                    # no workspace
    (dict(), 2, 0x20000, 1024, 1),                    # workspace too small
    (dict(), 2, 0x20008, 1 << 30, 1),                 # misaligned workspace
    (dict(Hq=3, Hkv=2), 2, 0x20000, 1 << 30, 2),      # errors of splash_attn_fwd apply
    (dict(scale=0.0), 2, 0x20000, 1 << 30, 1),
    (dict(block_kv=128), 2, 0x20000, 1 << 30, 2),     # split-KV: default and decode tiles only
])
def test_split_forward_validation_errors(over, n_split, ws, ws_bytes, code):
    lib = _lib.load()
    args = _good_args(**over)
    assert lib.splash_attn_fwd_split(ctypes.byref(args), n_split, ws, ws_bytes, None) == code
    assert len(lib.splash_last_error()) > 0


def test_split_forward_noops():
    lib = _lib.load()
    assert lib.splash_attn_fwd_split(None, 2, None, 0, None) == 1
    assert lib.splash_attn_fwd_split(ctypes.byref(_good_args(B=0)), 2, None, 0, None) == 0
    assert lib.splash_last_error() == b""


@settings(max_examples=60, deadline=None)
@given(Lq=st.integers(1, 300), Lkv=st.integers(1, 300), off=st.integers(0, 100),
       bq=st.sampled_from([4, 16, 64]), bkv=st.sampled_from([5, 16, 64]),
       causal=st.booleans(), wl=st.integers(-1, 60), wr=st.integers(-1, 60))
def test_columns_bit_exact(Lq, Lkv, off, bq, bkv, causal, wl, wr):
    """attn_mask_columns against the oracle's column view of the block mask."""
    from oracle import column_tables_ref
    t = compile_mask(Lq, bq, bkv, L_kv=Lkv, q_offset=off, causal=causal, window_left=wl,
                     window_right=wr)
    got = t.columns()
    ref = column_tables_ref(t.block_mask)
    for name in ("col_ptr", "col_rows", "col_entry"):
        assert np.array_equal(got[name], ref[name]), name


def test_columns_errors():
    lib = _lib.load()
    P = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    row_ptr = np.array([0, 2, 3], np.int32)
    cols = np.array([0, 1, 1], np.int32)
    cp, cr, ce = np.zeros(3, np.int32), np.zeros(3, np.int32), np.zeros(3, np.int32)
    assert lib.attn_mask_columns(2, 2, 3, P(row_ptr), P(cols), P(cp), P(cr), P(ce)) == 0
    assert cp.tolist() == [0, 1, 3] and cr.tolist() == [0, 0, 1] and ce.tolist() == [0, 1, 2]
    assert lib.attn_mask_columns(-1, 2, 3, P(row_ptr), P(cols), P(cp), P(cr), P(ce)) == 1
    assert lib.attn_mask_columns(2, 2, 3, None, P(cols), P(cp), P(cr), P(ce)) == 1
    assert lib.attn_mask_columns(2, 2, 4, P(row_ptr), P(cols), P(cp), P(cr), P(ce)) == 1
    bad = np.array([1, 0, 1], np.int32)          # columns not ascending in row 0
    assert lib.attn_mask_columns(2, 2, 3, P(row_ptr), P(bad), P(cp), P(cr), P(ce)) == 1
    out = np.array([0, 2, 1], np.int32)          # column out of range
    assert lib.attn_mask_columns(2, 2, 3, P(row_ptr), P(out), P(cp), P(cr), P(ce)) == 1
    assert len(lib.splash_last_error()) > 0


def test_column_order():
    """attn_mask_column_order: columns by active-block count, most first,
    ties in column order (numpy's stable argsort of the negated counts)."""
    lib = _lib.load()
    P = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    cp = np.array([0, 2, 7, 12, 13, 13], np.int32)   # counts 2, 5, 5, 1, 0
    out = np.full(5, -1, np.int32)
    assert lib.attn_mask_column_order(5, P(cp), P(out)) == 0
    assert out.tolist() == [1, 2, 0, 3, 4]
    rng = np.random.default_rng(7)
    for n in (1, 3, 64, 513):
        counts = rng.integers(0, 6, n).astype(np.int32)
        cp = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        out = np.zeros(n, np.int32)
        assert lib.attn_mask_column_order(n, P(cp), P(out)) == 0
        assert out.tolist() == np.argsort(-counts, kind="stable").tolist()
    assert lib.attn_mask_column_order(0, P(np.zeros(1, np.int32)), None) == 0
    assert lib.attn_mask_column_order(-1, P(cp), P(out)) == 1
    assert lib.attn_mask_column_order(2, None, P(out)) == 1
    assert lib.attn_mask_column_order(2, P(np.array([1, 2, 3], np.int32)), P(out)) == 1
    assert lib.attn_mask_column_order(2, P(np.array([0, 2, 1], np.int32)), P(out)) == 1
    assert len(lib.splash_last_error()) > 0


def _good_bwd(**over):
    fake = 0x10000
    a = dict(dtype=1, B=1, Hq=2, Hkv=1, L=256, L_kv=0, q_offset=0, d_qk=128, d_v=128,
             q=fake, k=fake, v=fake, o=fake, lse=fake, dout=fake, dq=fake, dk=fake, dv=fake,
             delta=fake, causal=1, window_left=-1, window_right=-1, seg_q=None, seg_kv=None,
             block_q=256, block_kv=64, n_q_blocks=1, n_kv_blocks=4, n_active=4,
             row_ptr=fake, active_cols=fake, col_ptr=fake, col_rows=fake,
             scale=0.088, soft_cap=0.0)
    a.update(over)
    return _lib.BwdArgs(**a)


@pytest.mark.parametrize("over,code", [
    (dict(dtype=5), 3),
    (dict(dtype=0), 4),                         # bf16 only
    (dict(d_qk=192, d_v=64), 4),
    (dict(d_qk=128, d_v=192), 4),
    (dict(d_qk=64, d_v=128), 4),
    (dict(B=-1), 1),
    (dict(Hkv=0), 1),
    (dict(Hq=3, Hkv=2), 2),
    (dict(L_kv=-1), 1),
    (dict(q_offset=-1), 1),
    (dict(causal=2), 1),
    (dict(window_right=-3), 1),
    (dict(scale=0.0), 1),
    (dict(soft_cap=math.inf), 1),
    (dict(seg_kv=0x10000), 1),
    (dict(L_kv=300, n_kv_blocks=5, seg_q=0x10000), 1),
    (dict(block_q=128), 2),
    (dict(n_q_blocks=2), 2),
    (dict(n_kv_blocks=3), 2),
    (dict(n_active=-1), 1),
    (dict(dq=None), 1),
    (dict(delta=None), 1),
    (dict(col_ptr=None), 1),
    (dict(col_rows=None), 1),
    (dict(dk=0x10004), 1),
    (dict(L_kv=1 << 24, n_kv_blocks=(1 << 24) // 64), 2),
])
def test_backward_validation_errors(over, code):
    lib = _lib.load()
    assert lib.splash_attn_bwd(ctypes.byref(_good_bwd(**over)), None) == code
    assert len(lib.splash_last_error()) > 0


def test_backward_null_args_and_noop():
    lib = _lib.load()
    assert lib.splash_attn_bwd(None, None) == 1
    assert lib.splash_attn_bwd(ctypes.byref(_good_bwd(B=0)), None) == 0
    assert lib.splash_last_error() == b""


def test_tables_refuse_another_mask():
    """Tables remember the mask they were compiled for (Lecture 13 section
    6.2: the table is computed once for one mask); the binding refuses them
    for a call with another causal flag, window or segment ids."""
    from block_sparse_flash_amd.api import _check_tables, _mask_key
    L = 700
    bq, bkv = fwd_tile("bf16", 128, 128)
    seg = segment_ids(L, 3, 40, 300)
    t = compile_mask(L, bq, bkv, causal=True, window_left=100, seg_q=seg)
    same = _mask_key(True, 100, -1, seg, None, 0)
    _check_tables(t, bq, bkv, L, L, same)
    # explicit key ids equal to the query ids are the same mask
    _check_tables(t, bq, bkv, L, L, _mask_key(True, 100, -1, seg, seg.copy(), 0))
    other_seg = seg.copy()
    other_seg[L // 2:] += 1
    for key, what in [(_mask_key(False, 100, -1, seg, None, 0), "causal"),
                      (_mask_key(True, 99, -1, seg, None, 0), "window_left"),
                      (_mask_key(True, 100, 5, seg, None, 0), "window_right"),
                      (_mask_key(True, 100, -1, None, None, 0), "segment ids"),
                      (_mask_key(True, 100, -1, other_seg, None, 0), "segment ids")]:
        with pytest.raises(ValueError, match=what):
            _check_tables(t, bq, bkv, L, L, key)
    with pytest.raises(ValueError, match="block_q"):
        _check_tables(t, bq, bkv, L + 1, L + 1, same)


def test_segment_ids_are_cached_per_tables():
    """The binding's segment-id handling: host rows, the per-batch flag, the
    digest the table check uses, and reuse of the device copies while the
    ids stay the same (no copy, synchronisation or hashing per call)."""
    from block_sparse_flash_amd.api import _seg_digest, _segments
    L = 300
    seg = segment_ids(L, 7, 20, 90)
    cache = {}
    a = _segments(seg, None, 2, L, L, "cpu", cache)
    assert not a["per_batch"] and a["hq"].shape == (1, L) and a["hkv"] is None
    assert tuple(a["dev_q"].shape) == (2, L) and (a["dev_q"].numpy() == seg).all()
    # the kernels read [B, L] row-major through the raw pointer
    assert a["dev_q"].is_contiguous() and a["dev_q"].stride() == (L, 1)
    assert a["digest0"] == _seg_digest(seg, None) == _seg_digest(seg, seg)
    assert _segments(seg.copy(), None, 2, L, L, "cpu", cache) is a          # same ids: cached
    other = seg.copy()
    other[L // 2:] += 1
    b = _segments(other, None, 2, L, L, "cpu", cache)
    assert b is not a and b["digest0"] != a["digest0"] and cache["seg"] is b
    c = _segments(np.stack([seg, other]), None, 2, L, L, "cpu", cache)
    assert c["per_batch"] and c["hq"].shape == (2, L)
    assert c["dev_q"].stride() == (L, 1) and (c["dev_q"].numpy()[1] == other).all()
    e = _segments(seg, other, 3, L, L, "cpu", None)
    assert e["dev_kv"].stride() == (L, 1) and (e["dev_kv"].numpy() == other).all()
    d = _segments(np.stack([seg, seg]), None, 2, L, L, "cpu", None)
    assert not d["per_batch"]
    assert _segments(None, None, 2, L, L, "cpu", cache) is None
    with pytest.raises(ValueError, match="seg_kv given without seg_q"):
        _segments(None, seg, 2, L, L, "cpu")
    with pytest.raises(ValueError, match="seg_kv is required"):
        _segments(seg, None, 2, L, L + 5, "cpu")
    with pytest.raises(ValueError, match="must be"):
        _segments(np.stack([seg, seg, seg]), None, 2, L, L, "cpu")
    with pytest.raises(ValueError, match="must be"):
        _segments(seg[:-1], None, 2, L, L, "cpu")
