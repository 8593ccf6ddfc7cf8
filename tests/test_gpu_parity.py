"""GPU parity: the HIP forward (through the C ABI) against the float64 oracle.

Tolerances (max-abs): fp32 o and lse 1e-5; bf16 o 2e-2 and lse 1e-3.
Small cases compare every output element; the full-size workloads compare
sampled rows (first/last rows, rows around block edges and random rows of a
few heads), each of which the oracle computes exactly.
"""

import math
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_sparse_flash_amd import compile_mask, fwd_tile, splash_fwd
from block_sparse_flash_amd.inputs import (EXTRA_WORKLOADS, WORKLOADS, as_f64, draw_qkv,
                                           make_inputs, segment_ids, stored)
from oracle import allowed, attention_ref, mle_safe_range

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-3)}


def _announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _run(q, k, v, dev="cuda", **kw):
    o, lse = splash_fwd(q.to(dev), k.to(dev), v.to(dev), **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _compare(o, lse, o_ref, lse_ref, dtype):
    to, tl = TOL[dtype]
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), "rows with no allowed key differ"
    fin = np.isfinite(lse_ref)
    err_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    err_l = float(np.max(np.abs(lse[fin] - lse_ref[fin]))) if fin.any() else 0.0
    assert np.all(np.isfinite(o)), "non-finite output"
    assert err_o <= to, f"o max-abs error {err_o:.3g} > {to}"
    assert err_l <= tl, f"lse max-abs error {err_l:.3g} > {tl}"
    return err_o, err_l



def _lane_keys():
    """Keys of a 64-key block held by the lanes of each half-wave in the
    bf16 forward (two 32-key score tiles; item e of tile t is key
    32 t + 8 (e / 4) + 4 hi + e % 4)."""
    return [[32 * t + 8 * (e // 4) + 4 * hi + e % 4 for t in range(2) for e in range(16)] for hi in range(2)]


def _reference_moves(q, k, scale, rows):
    """A float64 model of the forward's lazy reference on causal rows at the
    256x64 tile: a block's row max is taken when some lane's partial sum of
    p exceeds 2^8 (or the row has no reference yet) and moves the reference
    when it exceeds it by more than 8 in log2 units.  Returns (moves after a
    row's first block, blocks whose sum passed the bound without a move)."""
    lanes = _lane_keys()
    moves = no_move = 0
    for h in range(q.shape[0]):
        s = (q[h] @ k[h].T) * scale / math.log(2.0)
        for i in rows:
            mc, seen = 0.0, False
            for b in range(i // 64 + 1):
                keys = np.arange(64 * b, 64 * b + 64)
                x = np.where(keys <= i, s[i, np.minimum(keys, s.shape[1] - 1)], -np.inf) - mc
                p = np.exp2(x)
                if seen and max(p[lanes[0]].sum(), p[lanes[1]].sum()) <= 256.0:
                    continue
                mx = x.max()
                if (not seen and mx > -np.inf) or mx > 8.0:
                    moves += seen
                    mc, seen = mc + mx, True
                elif seen:
                    no_move += 1
    return moves, no_move


def test_rising_and_falling_logits_move_the_reference():
    """Logits that rise along the keys (head 0: fast, then slowly) and fall
    (head 1), up to about 120, causal: on head 0 a row's exponent reference
    moves again and again after its first block, and some blocks' partial
    sums of p pass 2^8 without any p doing so (the guard takes the row max
    and nothing moves); on head 1 the first block's reference holds.  Every
    element against the oracle."""
    _announce("rising and falling logits")
    L, d = 1024, 128
    rng = np.random.default_rng(11)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = np.stack([4.0 * u + 0.05 * rng.standard_normal((L, d)) for _ in range(2)])
    j = np.arange(L)
    rise = np.where(j < L // 2, 0.25 * j, 0.25 * (L // 2) + 0.07 * (j - L // 2))
    g = np.stack([rise, rise[::-1].copy()]) * math.sqrt(d) / 4.0 * math.log(2.0)
    k = g[:, :, None] * u[None, None, :] + 0.3 * rng.standard_normal((2, L, d))
    v = rng.standard_normal((2, L, d))
    qs, ks, vs = (stored(torch.from_numpy(a[None].astype(np.float32)), "bf16") for a in (q, k, v))
    scale = 1.0 / math.sqrt(d)
    moves, no_move = _reference_moves(as_f64(qs)[0], as_f64(ks)[0], scale, range(0, L, 7))
    assert moves > 100 and no_move > 10, (moves, no_move)
    o, lse = _run(qs, ks, vs, scale=scale, causal=True)
    o_ref, lse_ref = attention_ref(as_f64(qs), as_f64(ks), as_f64(vs), scale=scale, causal=True)
    assert float(lse_ref.max()) > 100.0
    eo, el = _compare(o, lse, o_ref, lse_ref, "bf16")
    _announce(f"  moves {moves}, guard without move {no_move}; max-abs o {eo:.3g} lse {el:.3g}")


RISING = [
    # (name, Hq, Hkv, L_q, L_kv, q_offset, d_qk, d_v, soft_cap, n_split)
    ("d64", 2, 2, 700, 700, 0, 64, 64, 0.0, 1),
    ("d192x128", 2, 2, 700, 700, 0, 192, 128, 0.0, 1),
    ("cap30", 2, 2, 700, 700, 0, 128, 128, 30.0, 1),
    ("decode-gqa-split3", 8, 2, 16, 2000, 1984, 128, 128, 0.0, 3),
]


@pytest.mark.parametrize("case", RISING, ids=lambda c: c[0])
def test_rising_logits_other_instances(case):
    """The rising-logit inputs (the exponent reference moves block after
    block) on the other kernel instances that share the guarded row max:
    64- and 192-wide heads, the soft cap (logits capped at 30), and a decode
    shape (16 rows at the end of 2000 keys, packed GQA rows, split-KV in
    three chunks, the 64-row decode tile).  Every element against the
    oracle."""
    name, Hq, Hkv, Lq, Lkv, off, dqk, dv, cap, S = case
    _announce(f"rising logits {name}")
    rng = np.random.default_rng(12)
    u = rng.standard_normal(dqk)
    u /= np.linalg.norm(u)
    j = np.arange(Lkv)
    # logits rise by up to 0.25 (log2 units) per key, to about 120 at the last key
    g = (0.25 * min(1.0, 700 / Lkv) * j) * math.sqrt(dqk) / 4.0 * math.log(2.0)
    q = 4.0 * u + 0.05 * rng.standard_normal((Hq, Lq, dqk))
    k = g[None, :, None] * u[None, None, :] + 0.3 * rng.standard_normal((Hkv, Lkv, dqk))
    v = rng.standard_normal((Hkv, Lkv, dv))
    qs, ks, vs = (stored(torch.from_numpy(a[None].astype(np.float32)), "bf16") for a in (q, k, v))
    scale = 1.0 / math.sqrt(dqk)
    o, lse = _run(qs, ks, vs, scale=scale, soft_cap=cap, causal=True, q_offset=off, n_split=S)
    o_ref, lse_ref = attention_ref(as_f64(qs), as_f64(ks), as_f64(vs), scale=scale, soft_cap=cap,
                                   causal=True, q_offset=off)
    assert float(lse_ref.max()) > (20.0 if cap else 100.0)
    eo, el = _compare(o, lse, o_ref, lse_ref, "bf16")
    _announce(f"  max-abs o {eo:.3g} lse {el:.3g}")

SMALL = [
    # (dtype, B, Hq, Hkv, L, d_qk, d_v, mask kwargs, soft_cap, mask_mode)
    ("f32", 1, 1, 1, 256, 64, 64, dict(causal=True), 0.0, "computed"),
    ("f32", 2, 4, 2, 200, 128, 128, dict(causal=True, window_left=37), 0.0, "computed"),
    ("f32", 1, 2, 1, 333, 64, 128, dict(causal=True, segs=(20, 90)), 5.0, "computed"),
    ("f32", 1, 2, 2, 190, 128, 64, dict(window_left=50, window_right=20), 0.0, "stored"),
    ("bf16", 1, 2, 2, 256, 128, 128, dict(causal=True), 0.0, "computed"),
    ("bf16", 2, 4, 4, 640, 128, 128, dict(), 0.0, "computed"),
    ("bf16", 1, 4, 1, 1000, 128, 128, dict(causal=True, window_left=200), 0.0, "computed"),
    ("bf16", 1, 4, 2, 777, 128, 128, dict(causal=True, segs=(40, 300)), 50.0, "computed"),
    ("bf16", 1, 4, 2, 777, 128, 128, dict(causal=True, segs=(40, 300)), 50.0, "stored"),
    ("bf16", 1, 2, 2, 520, 192, 128, dict(causal=True), 0.0, "computed"),
    ("bf16", 1, 2, 1, 300, 64, 64, dict(window_left=70, window_right=33), 3.0, "computed"),
    ("bf16", 1, 2, 1, 300, 64, 64, dict(window_left=70, window_right=33), 3.0, "stored"),
    ("bf16", 1, 3, 1, 450, 128, 64, dict(segs=(10, 200)), 0.0, "computed"),
    ("bf16", 1, 2, 2, 130, 64, 128, dict(causal=True), 0.0, "computed"),
    ("bf16", 1, 2, 2, 96, 192, 64, dict(causal=True, window_left=5), 0.0, "computed"),
    # GQA with fewer than 256 rows: the query heads of a group share a row tile
    ("bf16", 2, 8, 2, 100, 128, 128, dict(causal=True, segs=(10, 40)), 0.0, "computed"),
    ("bf16", 1, 8, 2, 200, 64, 64, dict(window_left=30), 2.0, "stored"),
    ("bf16", 1, 6, 1, 50, 192, 128, dict(causal=True), 0.0, "computed"),
    # 192-wide heads with a soft cap (the DeepSeek-V3 head shape, Lecture 13
    # section 6.6, with the section 5.4 cap): plain, stored masks, packed rows
    ("bf16", 1, 2, 2, 520, 192, 128, dict(causal=True), 30.0, "computed"),
    ("bf16", 1, 4, 2, 777, 192, 128, dict(causal=True, segs=(40, 300)), 50.0, "stored"),
    ("bf16", 1, 2, 1, 300, 192, 64, dict(window_left=70, window_right=33), 5.0, "computed"),
    ("bf16", 1, 6, 1, 50, 192, 128, dict(causal=True), 20.0, "computed"),
    ("bf16", 1, 8, 2, 100, 192, 64, dict(causal=True, segs=(10, 40)), 10.0, "computed"),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c[0]}-B{c[1]}H{c[2]}/{c[3]}-L{c[4]}-d{c[5]}x{c[6]}-{c[9]}"
                         + ("-cap" if c[8] else "") + "-" + "-".join(sorted(c[7])))
def test_small_cases_every_element(case):
    dtype, B, Hq, Hkv, L, dqk, dv, mk, cap, mode = case
    _announce(f"small {case}")
    seed = 1000 + L + dqk
    q, k, v = draw_qkv(B, Hq, Hkv, L, dqk, dv, seed, qk_std=1.5 if cap else 1.0)
    q, k, v = stored(q, dtype), stored(k, dtype), stored(v, dtype)
    mk = dict(mk)
    seg = None
    if "segs" in mk:
        lo, hi = mk.pop("segs")
        seg = segment_ids(L, seed, lo, hi)
    scale = 1.0 / math.sqrt(dqk)
    o, lse = _run(q, k, v, scale=scale, soft_cap=cap, seg_q=seg, mask_mode=mode, **mk)
    o_ref, lse_ref = attention_ref(as_f64(q), as_f64(k), as_f64(v), scale=scale,
                                   soft_cap=cap, seg_q=seg, **mk)
    eo, el = _compare(o, lse, o_ref, lse_ref, dtype)
    _announce(f"  max-abs o {eo:.3g} lse {el:.3g}")


TILE_CASES = [
    # (B, Hq, Hkv, L, mask kwargs, soft_cap, mask_mode)
    (1, 4, 2, 777, dict(causal=True, segs=(40, 300)), 50.0, "computed"),
    (1, 4, 2, 777, dict(causal=True, segs=(40, 300)), 50.0, "stored"),
    (2, 4, 4, 640, dict(), 0.0, "computed"),
    (1, 4, 1, 1000, dict(causal=True, window_left=200), 0.0, "computed"),
    (1, 2, 2, 300, dict(window_left=70, window_right=33), 3.0, "stored"),
    (2, 36, 6, 1000, dict(causal=True, window_left=300), 0.0, "computed"),  # several rounds
]
SWEEP_TILES = [(256, 128), (128, 64), (128, 128)]


@pytest.mark.parametrize("tile", SWEEP_TILES, ids=lambda t: f"{t[0]}x{t[1]}")
@pytest.mark.parametrize("case", TILE_CASES, ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}-L{c[3]}-{c[6]}"
                         + ("-cap" if c[5] else "") + "-" + "-".join(sorted(c[4])))
def test_sweep_tiles_every_element(tile, case):
    """The plain forward at the other tiles of the block-size sweep (Lecture
    13 sections 5.3 and 6.5): tables compiled at that tile, every element
    against the oracle."""
    B, Hq, Hkv, L, mk, cap, mode = case
    bq, bkv = tile
    _announce(f"tile {bq}x{bkv} {case}")
    seed = 3000 + L + Hq
    q, k, v = (stored(a, "bf16") for a in draw_qkv(B, Hq, Hkv, L, 128, 128, seed, qk_std=1.5 if cap else 1.0))
    mk = dict(mk)
    seg = None
    if "segs" in mk:
        lo, hi = mk.pop("segs")
        seg = segment_ids(L, seed, lo, hi)
    t = compile_mask(L, bq, bkv, seg_q=seg, **mk)
    scale = 1.0 / math.sqrt(128)
    o, lse = _run(q, k, v, scale=scale, soft_cap=cap, seg_q=seg, mask_mode=mode, tables=t, **mk)
    o_ref, lse_ref = attention_ref(as_f64(q), as_f64(k), as_f64(v), scale=scale,
                                   soft_cap=cap, seg_q=seg, **mk)
    eo, el = _compare(o, lse, o_ref, lse_ref, "bf16")
    _announce(f"  max-abs o {eo:.3g} lse {el:.3g}")


def _logit_extremes(q, k, scale, cap, mk, seg):
    """Largest allowed logit and smallest row maximum (float64)."""
    qf, kf = as_f64(q), as_f64(k)
    B, Hq, L, _ = qf.shape
    group = Hq // kf.shape[1]
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    a = allowed(i, j, L_q=L, L_kv=L, causal=mk.get("causal", False),
                window_left=mk.get("window_left", -1), window_right=mk.get("window_right", -1),
                seg_q=seg)
    smax, rmin = -np.inf, np.inf
    for b in range(B):
        for h in range(Hq):
            s = scale * (qf[b, h] @ kf[b, h // group].T)
            if cap > 0:
                s = cap * np.tanh(s / cap)
            s = np.where(a, s, -np.inf)
            rm = s.max(axis=1)
            rm = rm[np.isfinite(rm)]
            smax, rmin = max(smax, rm.max()), min(rmin, rm.min())
    return float(smax), float(rmin)


MLE_CASES = [
    # (dtype, L, d_qk, d_v, mask kwargs, soft_cap, how the constant is chosen)
    ("bf16", 777, 128, 128, dict(causal=True, segs=(40, 300)), 0.0, "max"),
    ("bf16", 777, 128, 128, dict(causal=True, segs=(40, 300)), 0.0, "low"),
    ("bf16", 777, 128, 128, dict(causal=True, segs=(40, 300)), 0.0, "high"),
    ("bf16", 600, 128, 128, dict(causal=True, window_left=100), 20.0, "cap"),
    ("bf16", 520, 192, 128, dict(causal=True), 0.0, "max"),
    ("bf16", 300, 64, 64, dict(window_left=70, window_right=33), 0.0, "low"),
    ("f32", 333, 64, 128, dict(causal=True, segs=(20, 90)), 5.0, "cap"),
    ("f32", 256, 128, 128, dict(causal=True), 0.0, "high"),
]


@pytest.mark.parametrize("case", MLE_CASES, ids=lambda c: f"{c[0]}-L{c[1]}-d{c[2]}x{c[3]}-{c[6]}")
def test_max_logit_estimate(case):
    """Lecture 13 section 5.4: a constant in place of the running max gives
    the softmax of the oracle (its running-max definition) as long as the
    constant is inside the float32 safe range; "low" / "high" sit 60 inside
    the overflow / underflow edges."""
    dtype, L, dqk, dv, mk, cap, how = case
    _announce(f"max logit estimate {case}")
    seed = 4000 + L + dqk
    q, k, v = (stored(a, dtype) for a in draw_qkv(1, 4, 2, L, dqk, dv, seed, qk_std=1.5 if cap else 1.0))
    mk = dict(mk)
    seg = None
    if "segs" in mk:
        lo, hi = mk.pop("segs")
        seg = segment_ids(L, seed, lo, hi)
    scale = 1.0 / math.sqrt(dqk)
    smax, rmin = _logit_extremes(q, k, scale, cap, mk, seg)
    c = {"max": smax, "low": smax - 60.0, "high": rmin + 60.0, "cap": cap}[how]
    lo_c, hi_c = mle_safe_range(smax, rmin)
    assert lo_c < c < hi_c
    o, lse = _run(q, k, v, scale=scale, soft_cap=cap, seg_q=seg, max_logit=c, **mk)
    o_ref, lse_ref = attention_ref(as_f64(q), as_f64(k), as_f64(v), scale=scale,
                                   soft_cap=cap, seg_q=seg, **mk)
    eo, el = _compare(o, lse, o_ref, lse_ref, dtype)
    _announce(f"  c {c:.3f} (safe {lo_c:.1f}..{hi_c:.1f}) max-abs o {eo:.3g} lse {el:.3g}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rows_without_allowed_keys(dtype):
    _announce(f"empty rows {dtype}")
    B, H, L, d = 1, 2, 200, 64
    q, k, v = (stored(a, dtype) for a in draw_qkv(B, H, H, L, d, d, 77))
    seg_q = np.repeat(np.arange(4), 50).astype(np.int32)
    seg_kv = seg_q.copy()
    seg_kv[seg_kv == 1] = 7          # queries of segment 1 see nothing
    o, lse = _run(q, k, v, causal=True, seg_q=seg_q, seg_kv=seg_kv)
    o_ref, lse_ref = attention_ref(as_f64(q), as_f64(k), as_f64(v), scale=1 / 8,
                                   causal=True, seg_q=seg_q, seg_kv=seg_kv)
    _compare(o, lse, o_ref, lse_ref, dtype)
    assert np.all(o[:, :, 50:100] == 0) and np.all(np.isneginf(lse[:, :, 50:100]))


def test_per_batch_segments_and_gqa():
    _announce("per-batch segments, GQA 6/2")
    B, Hq, Hkv, L, d = 3, 6, 2, 384, 128
    q, k, v = (stored(a, "bf16") for a in draw_qkv(B, Hq, Hkv, L, d, d, 5))
    seg = np.stack([segment_ids(L, s, 30, 200) for s in range(B)])
    o, lse = _run(q, k, v, causal=True, seg_q=seg)
    o_ref, lse_ref = attention_ref(as_f64(q), as_f64(k), as_f64(v), scale=d ** -0.5,
                                   causal=True, seg_q=seg)
    _compare(o, lse, o_ref, lse_ref, "bf16")


def test_more_items_than_work_groups():
    """288 (head, q-block row) items on at most one work-group per CU: two
    rounds, the second partial and run in reverse order inside each XCD;
    every output element is checked."""
    _announce("persistent rounds: B=2 Hq=36 Hkv=6 L=1000 d=64, causal + window 300")
    B, Hq, Hkv, L, d = 2, 36, 6, 1000, 64
    q, k, v = (stored(a, "bf16") for a in draw_qkv(B, Hq, Hkv, L, d, d, 31))
    mk = dict(causal=True, window_left=300)
    o, lse = _run(q, k, v, **mk)
    o_ref, lse_ref = attention_ref(as_f64(q), as_f64(k), as_f64(v), scale=d ** -0.5, **mk)
    eo, el = _compare(o, lse, o_ref, lse_ref, "bf16")
    _announce(f"  max-abs o {eo:.3g} lse {el:.3g}")


def test_persistent_rounds_items_of_one_to_many_blocks():
    """The ping-pong loop passes n + 2 work-group barriers per item of n
    blocks, the same count in both wave groups.  The 64-row decode tile on
    causal L=700 gives items of 1 to 11 blocks; 2 x 24 heads make 528 items,
    more than the 512 persistent work-groups (two per CU), so work-groups
    chain items of different lengths (one-block items included).  Every
    output element is checked."""
    _announce("persistent rounds, 64x64 tile: B=2 Hq=24 Hkv=8 L=700 d=128, causal")
    B, Hq, Hkv, L, d = 2, 24, 8, 700, 128
    q, k, v = (stored(a, "bf16") for a in draw_qkv(B, Hq, Hkv, L, d, d, 37))
    t = compile_mask(L, 64, 64, causal=True)
    rows = np.diff(t.row_ptr)
    assert rows.min() == 1 and rows.max() == 11
    o, lse = _run(q, k, v, causal=True, tables=t)
    o_ref, lse_ref = attention_ref(as_f64(q), as_f64(k), as_f64(v), scale=d ** -0.5, causal=True)
    eo, el = _compare(o, lse, o_ref, lse_ref, "bf16")
    _announce(f"  max-abs o {eo:.3g} lse {el:.3g}")


SPLIT_CASES = [
    # (B, Hq, Hkv, L, d_qk, d_v, mask kwargs, soft_cap, n_split)
    (1, 2, 2, 1000, 128, 128, dict(causal=True), 0.0, 2),
    (1, 4, 2, 777, 128, 128, dict(causal=True, window_left=200), 0.0, 5),
    (1, 4, 1, 900, 128, 64, dict(causal=True, segs=(40, 300)), 50.0, 3),
    (2, 2, 2, 520, 192, 128, dict(causal=True), 0.0, 4),
    (1, 2, 1, 300, 64, 64, dict(window_left=70, window_right=33), 3.0, 7),
    (1, 2, 2, 640, 64, 128, dict(), 0.0, 64),   # more chunks than blocks: empty chunks
    (1, 2, 2, 600, 192, 128, dict(causal=True), 30.0, 3),
    (1, 4, 1, 500, 192, 64, dict(causal=True, segs=(40, 200)), 20.0, 2),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}-L{c[3]}-d{c[4]}x{c[5]}-s{c[8]}"
                         + ("-cap" if c[7] else "") + "-" + "-".join(sorted(c[6])))
def test_split_kv_every_element(case):
    """splash_attn_fwd_split: chunks of each row's active blocks merged
    through their lse (split-K) give the oracle's attention."""
    B, Hq, Hkv, L, dqk, dv, mk, cap, S = case
    _announce(f"split-KV {case}")
    seed = 7000 + L + S
    q, k, v = (stored(a, "bf16") for a in draw_qkv(B, Hq, Hkv, L, dqk, dv, seed, qk_std=1.5 if cap else 1.0))
    mk = dict(mk)
    seg = None
    if "segs" in mk:
        lo, hi = mk.pop("segs")
        seg = segment_ids(L, seed, lo, hi)
    scale = 1.0 / math.sqrt(dqk)
    o, lse = _run(q, k, v, scale=scale, soft_cap=cap, seg_q=seg, n_split=S, **mk)
    o_ref, lse_ref = attention_ref(as_f64(q), as_f64(k), as_f64(v), scale=scale,
                                   soft_cap=cap, seg_q=seg, **mk)
    eo, el = _compare(o, lse, o_ref, lse_ref, "bf16")
    _announce(f"  max-abs o {eo:.3g} lse {el:.3g}")


DECODE_CASES = [
    # (B, Hq, Hkv, L_q, L_kv, q_offset, d_qk, d_v, mask kwargs, soft_cap, mask_mode, n_split)
    (2, 8, 2, 1, 3000, 2999, 128, 128, dict(causal=True), 0.0, "computed", 1),     # one new token
    (2, 8, 2, 1, 3000, 2999, 128, 128, dict(causal=True), 0.0, "computed", 8),
    (1, 4, 1, 16, 1000, 984, 128, 128, dict(causal=True, window_left=300, segs=(50, 400)), 0.0,
     "computed", 1),
    (1, 4, 1, 16, 1000, 984, 128, 128, dict(causal=True, window_left=300, segs=(50, 400)), 0.0,
     "stored", 3),
    (1, 2, 2, 300, 777, 477, 192, 128, dict(causal=True), 0.0, "computed", 1),    # chunked prefill
    (1, 4, 4, 5, 4100, 4095, 64, 64, dict(causal=True, window_left=1000), 30.0, "computed", 4),
    (1, 2, 1, 40, 500, 0, 128, 64, dict(window_right=100), 0.0, "computed", 1),
    (1, 2, 2, 300, 100, 0, 64, 128, dict(), 0.0, "computed", 2),                  # L_kv < L_q
    # rows past the last key; those beyond position 949 see no key at all
    (1, 2, 2, 64, 700, 900, 128, 128, dict(causal=True, window_left=250), 0.0, "computed", 1),
    (1, 2, 2, 64, 700, 900, 128, 128, dict(causal=True, window_left=250), 0.0, "computed", 5),
]


@pytest.mark.parametrize("case", DECODE_CASES,
                         ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}-Lq{c[3]}-Lkv{c[4]}-off{c[5]}-d{c[6]}x{c[7]}"
                         f"-{c[10]}-s{c[11]}" + ("-cap" if c[9] else "") + "-" + "-".join(sorted(c[8])))
def test_decode_shapes_every_element(case):
    """L_q != L_kv with query row i at key position q_offset + i (decoding
    and chunked prefill), with and without split-KV, against the oracle."""
    B, Hq, Hkv, Lq, Lkv, off, dqk, dv, mk, cap, mode, S = case
    _announce(f"decode {case}")
    seed = 9000 + Lq + Lkv + S
    q, k, v = (stored(a, "bf16")
               for a in draw_qkv(B, Hq, Hkv, Lq, dqk, dv, seed, qk_std=1.5 if cap else 1.0, L_kv=Lkv))
    mk = dict(mk)
    seg_q = seg_kv = None
    if "segs" in mk:
        lo, hi = mk.pop("segs")
        seg_kv = segment_ids(Lkv, seed, lo, hi)
        seg_q = seg_kv[off:off + Lq].copy()     # the new rows continue the cached documents
    scale = 1.0 / math.sqrt(dqk)
    o, lse = _run(q, k, v, scale=scale, soft_cap=cap, seg_q=seg_q, seg_kv=seg_kv, q_offset=off,
                  mask_mode=mode, n_split=S, **mk)
    o_ref, lse_ref = attention_ref(as_f64(q), as_f64(k), as_f64(v), scale=scale, soft_cap=cap,
                                   seg_q=seg_q, seg_kv=seg_kv, q_offset=off, **mk)
    eo, el = _compare(o, lse, o_ref, lse_ref, "bf16")
    _announce(f"  max-abs o {eo:.3g} lse {el:.3g}")


DECODE_TILE_CASES = [c for c in DECODE_CASES if c[6] == 128 and c[7] == 128] + [
    # (B, Hq, Hkv, L_q, L_kv, q_offset, d_qk, d_v, mask kwargs, soft_cap, mask_mode, n_split)
    (1, 8, 1, 40, 2000, 1960, 128, 128, dict(causal=True), 0.0, "computed", 4),   # 320 packed rows
    (1, 4, 4, 16, 2000, 1984, 128, 128, dict(causal=True, window_left=500), 10.0, "computed", 3),  # MHA
    (1, 4, 1, 64, 1500, 1436, 128, 128, dict(causal=True, segs=(50, 400)), 0.0, "stored", 1),
]


@pytest.mark.parametrize("case", DECODE_TILE_CASES,
                         ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}-Lq{c[3]}-Lkv{c[4]}-off{c[5]}"
                         f"-{c[10]}-s{c[11]}" + ("-cap" if c[9] else "") + "-" + "-".join(sorted(c[8])))
def test_decode_tile_every_element(case):
    """The 64-row decode tile (packed GQA rows, split-KV) against the oracle."""
    B, Hq, Hkv, Lq, Lkv, off, dqk, dv, mk, cap, mode, S = case
    _announce(f"decode tile {case}")
    seed = 9500 + Lq + Lkv + S
    q, k, v = (stored(a, "bf16")
               for a in draw_qkv(B, Hq, Hkv, Lq, dqk, dv, seed, qk_std=1.5 if cap else 1.0, L_kv=Lkv))
    mk = dict(mk)
    seg_q = seg_kv = None
    if "segs" in mk:
        lo, hi = mk.pop("segs")
        seg_kv = segment_ids(Lkv, seed, lo, hi)
        seg_q = seg_kv[off:off + Lq].copy()
    t = compile_mask(Lq, 64, 64, L_kv=Lkv, seg_q=seg_q, seg_kv=seg_kv, q_offset=off, **mk)
    scale = 1.0 / math.sqrt(dqk)
    o, lse = _run(q, k, v, scale=scale, soft_cap=cap, seg_q=seg_q, seg_kv=seg_kv, q_offset=off,
                  mask_mode=mode, n_split=S, tables=t, **mk)
    o_ref, lse_ref = attention_ref(as_f64(q), as_f64(k), as_f64(v), scale=scale, soft_cap=cap,
                                   seg_q=seg_q, seg_kv=seg_kv, q_offset=off, **mk)
    eo, el = _compare(o, lse, o_ref, lse_ref, "bf16")
    _announce(f"  max-abs o {eo:.3g} lse {el:.3g}")


def test_decode_full_length_gqa_split():
    """Decoding 16 new rows against a 32768-key cache: B=4, GQA 32/8, causal,
    q_offset = L_kv - L_q, split into 16 chunks; every row against the
    oracle, and the unsplit forward agrees."""
    B, Hq, Hkv, Lq, Lkv, d = 4, 32, 8, 16, 32768, 128
    _announce(f"decode full length B={B} Hq={Hq} Hkv={Hkv} L_q={Lq} L_kv={Lkv}")
    q, k, v = (stored(a, "bf16") for a in draw_qkv(B, Hq, Hkv, Lq, d, d, 77, L_kv=Lkv))
    off = Lkv - Lq
    o, lse = _run(q, k, v, causal=True, q_offset=off, n_split=16)
    heads = [(b, h) for b in range(B) for h in (0, 9, Hq - 1)]
    o_ref, lse_ref = attention_ref(as_f64(q), as_f64(k), as_f64(v), scale=1.0 / math.sqrt(d),
                                   causal=True, q_offset=off, heads=heads)
    sel = (np.array([b for b, _ in heads]), np.array([h for _, h in heads]))
    eo, el = _compare(o[sel], lse[sel], o_ref[sel], lse_ref[sel], "bf16")
    o1, lse1 = _run(q, k, v, causal=True, q_offset=off)
    assert float(np.max(np.abs(o1 - o))) <= 2e-2 and float(np.max(np.abs(lse1 - lse))) <= 1e-3
    _announce(f"  max-abs o {eo:.3g} lse {el:.3g}")


def test_decode_mismatched_tables_rejected():
    """Tables compiled for another L_kv or q_offset are refused by the
    binding before any launch."""
    q, k, v = (stored(a, "bf16") for a in draw_qkv(1, 2, 2, 8, 128, 128, 5, L_kv=600))
    bq, bkv = fwd_tile("bf16", 128, 128)
    t = compile_mask(8, bq, bkv, L_kv=600, causal=True, q_offset=500)
    with pytest.raises(ValueError):
        splash_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True, q_offset=592, tables=t)
    with pytest.raises(ValueError, match="another mask"):
        splash_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True, window_left=64, q_offset=500, tables=t)
    with pytest.raises(ValueError, match="out must be"):
        splash_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True, q_offset=500, tables=t,
                   out=torch.empty((1, 2, 8, 64), dtype=torch.bfloat16, device="cuda"))
    o, _ = splash_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True, q_offset=500, tables=t)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()


def test_ragged_full_length_persistent():
    """L = 32768 - 37 (a ragged last q block and kv block) with GQA 16/4 and
    a causal 4096-key window: 2048 items over the persistent rounds; sampled
    rows (both ends of every edge block class) against the oracle."""
    B, Hq, Hkv, L, d = 1, 16, 4, 32768 - 37, 128
    _announce(f"ragged full length B={B} Hq={Hq} Hkv={Hkv} L={L}")
    q, k, v = (stored(a, "bf16") for a in draw_qkv(B, Hq, Hkv, L, d, d, 41))
    mk = dict(causal=True, window_left=4095)
    o, lse = splash_fwd(q.cuda(), k.cuda(), v.cuda(), **mk)
    torch.cuda.synchronize()
    rng = np.random.default_rng(41)
    rows = _sample_rows(L, 256, rng)
    heads = [(0, 0), (0, 5), (0, Hq - 1)]
    o_ref, lse_ref = attention_ref(as_f64(q), as_f64(k), as_f64(v), scale=d ** -0.5, rows=rows,
                                   heads=heads, **mk)
    o_np = o.float().cpu().numpy()
    lse_np = lse.cpu().numpy()
    for (b, h) in heads:
        _compare(o_np[b, h, rows].astype(np.float64), lse_np[b, h, rows].astype(np.float64),
                 o_ref[b, h], lse_ref[b, h], "bf16")
    assert bool(torch.isfinite(lse).all())


def test_split_kv_rows_without_keys_and_reuse():
    """Rows with no allowed key stay o = 0, lse = -inf through the merge;
    one workspace serves two calls in a row, the second smaller."""
    _announce("split-KV empty rows + workspace reuse")
    from block_sparse_flash_amd import split_workspace_bytes
    B, H, L, d = 1, 2, 600, 128
    q, k, v = (stored(a, "bf16") for a in draw_qkv(B, H, H, L, d, d, 78))
    seg_q = np.repeat(np.arange(6), 100).astype(np.int32)
    seg_kv = seg_q.copy()
    seg_kv[seg_kv == 2] = 9
    ws = torch.empty(split_workspace_bytes(4, B, H, L, d), dtype=torch.uint8, device="cuda")
    o, lse = _run(q, k, v, causal=True, seg_q=seg_q, seg_kv=seg_kv, n_split=4, workspace=ws)
    o_ref, lse_ref = attention_ref(as_f64(q), as_f64(k), as_f64(v), scale=d ** -0.5,
                                   causal=True, seg_q=seg_q, seg_kv=seg_kv)
    _compare(o, lse, o_ref, lse_ref, "bf16")
    assert np.all(o[:, :, 200:300] == 0) and np.all(np.isneginf(lse[:, :, 200:300]))
    L2 = 300
    q2, k2, v2 = (stored(a, "bf16") for a in draw_qkv(B, H, H, L2, d, d, 79))
    o2, l2 = _run(q2, k2, v2, causal=True, n_split=3, workspace=ws)
    o2_ref, l2_ref = attention_ref(as_f64(q2), as_f64(k2), as_f64(v2), scale=d ** -0.5, causal=True)
    _compare(o2, l2, o2_ref, l2_ref, "bf16")


def test_empty_problem_is_noop():
    _announce("empty problem")
    q = torch.zeros((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    o, lse = splash_fwd(q, q, q, causal=True)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0, 128) and lse.shape == (1, 2, 0)


def test_deterministic_and_modes_agree():
    _announce("determinism + stored == computed")
    B, H, L, d = 1, 4, 1024, 128
    q, k, v = (stored(a, "bf16").cuda() for a in draw_qkv(B, H, H, L, d, d, 9))
    seg = segment_ids(L, 9, 60, 400)
    kw = dict(causal=True, window_left=300, seg_q=seg, soft_cap=20.0)
    o1, l1 = splash_fwd(q, k, v, **kw)
    o2, l2 = splash_fwd(q, k, v, **kw)
    o3, l3 = splash_fwd(q, k, v, mask_mode="stored", **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def _sample_rows(L, bq, rng, n_random=24):
    edges = []
    for r0 in (0, bq, L // 2 - (L // 2) % bq, L - bq):
        edges += [r0, r0 + 1, r0 + 31, r0 + 32, r0 + bq - 1]
    rows = set(x for x in edges if 0 <= x < L)
    rows |= set(rng.integers(0, L, size=n_random).tolist())
    rows.add(L - 1)
    return np.array(sorted(rows))


FULL_SIZE = [(name, 1) for name in WORKLOADS] + \
    [(name, w.n_split if w.n_split > 1 else 4) for name, w in EXTRA_WORKLOADS.items()]


@pytest.mark.parametrize("name,n_split", FULL_SIZE, ids=lambda x: str(x))
def test_full_size_workloads_sampled(name, n_split):
    w = {**WORKLOADS, **EXTRA_WORKLOADS}[name]
    _announce(f"full-size {name} n_split={n_split}")
    q, k, v, seg = make_inputs(w)
    # The tile the bench times this workload at.
    bq, bkv = w.tile if w.tile else fwd_tile(w.dtype, w.d_qk, w.d_v)
    tabs = compile_mask(w.L, bq, bkv, L_kv=w.keys, causal=w.causal, window_left=w.window_left,
                        window_right=w.window_right, seg_q=seg, q_offset=w.q_offset)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o, lse = splash_fwd(qd, kd, vd, scale=w.softmax_scale, soft_cap=w.soft_cap,
                        causal=w.causal, window_left=w.window_left,
                        window_right=w.window_right, seg_q=seg, tables=tabs, n_split=n_split,
                        q_offset=w.q_offset)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed + 7)
    n_heads = w.B * w.Hq
    pick = sorted(set([0, n_heads - 1] + rng.integers(0, n_heads, size=2).tolist()))
    heads = [(hh // w.Hq, hh % w.Hq) for hh in pick]
    rows = _sample_rows(w.L, bq, rng)
    if seg is not None:
        # Both sides of every document boundary (Lecture 13 section 6.4: the
        # segment mask ANDed with the causal one), where a row's allowed keys
        # start over.
        starts = np.flatnonzero(np.diff(np.asarray(seg)) != 0) + 1
        near = np.concatenate([starts - 2, starts - 1, starts, starts + 1, starts + 63])
        rows = np.union1d(rows, near[(near >= 0) & (near < w.L)])
    qf, kf, vf = q.float().numpy(), k.float().numpy(), v.float().numpy()
    o_ref, lse_ref = attention_ref(qf, kf, vf, scale=w.softmax_scale, soft_cap=w.soft_cap,
                                   causal=w.causal, window_left=w.window_left,
                                   window_right=w.window_right, seg_q=seg, rows=rows,
                                   heads=heads, q_offset=w.q_offset)
    o_np = o.float().cpu().numpy()
    lse_np = lse.cpu().numpy()
    worst = (0.0, 0.0)
    for (b, h) in heads:
        got_o = o_np[b, h, rows].astype(np.float64)
        got_l = lse_np[b, h, rows].astype(np.float64)
        eo, el = _compare(got_o, got_l, o_ref[b, h], lse_ref[b, h], w.dtype)
        worst = (max(worst[0], eo), max(worst[1], el))
    # Every output row is finite (all workloads are causal: each row sees itself).
    assert bool(torch.isfinite(lse).all()) and bool(torch.isfinite(o.float()).all())
    _announce(f"  {len(heads)} heads x {len(rows)} rows: max-abs o {worst[0]:.3g} lse {worst[1]:.3g}")


# Every bf16 forward instance the library compiles at the default tile: head
# dims x soft cap x split-KV x packed GQA rows (all query rows of a K/V group
# in one row tile when L is below the tile's rows), and the same for the
# 64-row decode tile of 128/128 heads (chosen for L <= 64).
INSTANCE_SHAPES = {
    # name: (B, Hq, Hkv, L, mask kwargs)
    "plain": (1, 2, 2, 300, dict(causal=True, window_left=120)),
    "packed": (1, 4, 1, 90, dict(causal=True)),
    "decode-tile": (1, 2, 2, 40, dict(causal=True)),
    "decode-tile-packed": (1, 4, 1, 40, dict(causal=True, window_left=25)),
}
INSTANCES = [(dims, shape, cap, n_split)
             for dims in [(128, 128), (64, 64), (64, 128), (128, 64), (192, 128), (192, 64)]
             for shape in ("plain", "packed")
             for cap in (0.0, 10.0)
             for n_split in (1, 3)]
INSTANCES += [((128, 128), shape, cap, n_split)
              for shape in ("decode-tile", "decode-tile-packed")
              for cap in (0.0, 10.0)
              for n_split in (1, 3)]


@pytest.mark.parametrize("case", INSTANCES, ids=lambda c: f"d{c[0][0]}x{c[0][1]}-{c[1]}"
                         + ("-cap" if c[2] else "") + f"-s{c[3]}")
def test_every_kernel_instance(case):
    """Each compiled variant of the bf16 forward (cap, split-KV, packed rows,
    decode tile) against the oracle, element by element (Lecture 13 section
    5.2 kernel body, section 5.4 cap; split-K merge through the lse, joto.ai
    "LSE and online softmax")."""
    (dqk, dv), shape, cap, n_split = case
    B, Hq, Hkv, L, mk = INSTANCE_SHAPES[shape]
    _announce(f"instance {case}")
    seed = 9000 + L + dqk + dv + n_split + int(cap)
    q, k, v = (stored(a, "bf16") for a in draw_qkv(B, Hq, Hkv, L, dqk, dv, seed, qk_std=1.5 if cap else 1.0))
    scale = 1.0 / math.sqrt(dqk)
    o, lse = _run(q, k, v, scale=scale, soft_cap=cap, n_split=n_split, **mk)
    o_ref, lse_ref = attention_ref(as_f64(q), as_f64(k), as_f64(v), scale=scale, soft_cap=cap, **mk)
    eo, el = _compare(o, lse, o_ref, lse_ref, "bf16")
    _announce(f"  max-abs o {eo:.3g} lse {el:.3g}")
