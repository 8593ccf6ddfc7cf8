"""The allocation-free split-KV forward (splash_attn_fwd_split_noalloc,
static device scratch) against splash_attn_fwd_split with a caller
workspace, through the C ABI: two calls in a row on one stream, the second
smaller, and the oracle for both; plus the size limit, checked before any
device work."""

import ctypes
import math
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_sparse_flash_amd import _lib, splash_fwd, split_workspace_bytes
from block_sparse_flash_amd.inputs import as_f64, draw_qkv, segment_ids, stored
from oracle import attention_ref

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


CALLS = [
    # (B, Hq, Hkv, L, L_kv, q_offset, d, mask kwargs, soft_cap, n_split, segments)
    (1, 8, 2, 600, 600, 0, 128, dict(causal=True, window_left=300), 0.0, 4, (40, 250)),
    (1, 4, 1, 16, 3000, 2984, 128, dict(causal=True), 20.0, 3, None),     # decode, smaller
]


def test_noalloc_matches_workspace_split_twice():
    outs = []
    for B, Hq, Hkv, L, Lkv, off, d, mk, cap, S, segs in CALLS:
        _announce(f"no-alloc split B={B} Hq={Hq} Hkv={Hkv} L={L} L_kv={Lkv} n_split={S}")
        q, k, v = (stored(a, "bf16").cuda()
                   for a in draw_qkv(B, Hq, Hkv, L, d, d, 600 + L, qk_std=1.5 if cap else 1.0, L_kv=Lkv))
        seg_q = seg_kv = None
        if segs is not None:
            seg_q = segment_ids(L, 600 + L, *segs)
        kw = dict(scale=1.0 / math.sqrt(d), soft_cap=cap, seg_q=seg_q, seg_kv=seg_kv, q_offset=off,
                  n_split=S, **mk)
        ws = torch.empty(split_workspace_bytes(S, B, Hq, L, d), dtype=torch.uint8, device="cuda")
        o_ws, l_ws = splash_fwd(q, k, v, workspace=ws, **kw)
        o_na, l_na = splash_fwd(q, k, v, no_alloc=True, **kw)
        torch.cuda.synchronize()
        # Same kernels on the same inputs: identical results.
        assert torch.equal(o_ws, o_na) and torch.equal(l_ws, l_na)
        o_ref, l_ref = attention_ref(as_f64(q), as_f64(k), as_f64(v), scale=1.0 / math.sqrt(d),
                                     soft_cap=cap, seg_q=seg_q, seg_kv=seg_kv, q_offset=off, **mk)
        o = o_na.float().cpu().numpy().astype(np.float64)
        lse = l_na.cpu().numpy().astype(np.float64)
        eo = float(np.max(np.abs(o - o_ref)))
        el = float(np.max(np.abs(lse - l_ref)))
        assert eo <= 2e-2 and el <= 1e-3, (eo, el)
        _announce(f"  max-abs o {eo:.3g} lse {el:.3g}")
        outs.append(o_na)
    assert all(bool(torch.isfinite(t.float()).all()) for t in outs)


def test_noalloc_rejects_partials_beyond_the_scratch():
    """n_split x B x Hq x L x (d_v + 1) x 4 bytes beyond the static scratch:
    refused before any device work (no launch, message names both sizes)."""
    lib = _lib.load()
    fake = 0x10000
    args = _lib.FwdArgs(dtype=1, B=4, Hq=32, Hkv=8, L=4096, d_qk=128, d_v=128,
                        q=fake, k=fake, v=fake, o=fake, lse=None, causal=1, window_left=-1,
                        window_right=-1, seg_q=None, seg_kv=None, block_q=256, block_kv=64,
                        n_q_blocks=16, n_active=1, n_patterns=0, row_ptr=fake, row_order=fake,
                        active_cols=fake, block_code=fake, mask_next=fake, partial_mask_blocks=fake,
                        mask_mode=0, scale=0.088, soft_cap=0.0)
    assert lib.splash_attn_fwd_split_noalloc(ctypes.byref(args), 4, None) == 1
    assert b"static scratch" in lib.splash_last_error()
    assert lib.splash_attn_fwd_split_noalloc(ctypes.byref(args), 0, None) == 1
    assert lib.splash_attn_fwd_split_noalloc(None, 4, None) == 1
