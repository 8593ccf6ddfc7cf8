"""CPU checks of bench.py's bookkeeping: the unmasked pair count behind the
TFLOP/s figure equals the number of pairs the oracle's mask definition
allows, for the named workloads (decoding included)."""

import importlib.util
import os

import numpy as np
import pytest

from block_sparse_flash_amd.inputs import ALL_WORKLOADS, segment_ids
from oracle import allowed

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    import sys
    if "bench" not in sys.modules:
        spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
        mod = importlib.util.module_from_spec(spec)
        sys.modules["bench"] = mod   # the oracle pool's workers are looked up by module name
        spec.loader.exec_module(mod)
    return sys.modules["bench"]


def _allowed_count(w, seg):
    j = np.arange(w.keys)[None, :]
    total = 0
    for r0 in range(0, w.L, 2048):
        i = np.arange(r0, min(r0 + 2048, w.L))[:, None]
        a = allowed(i, j, L_q=w.L, L_kv=w.keys, causal=w.causal, window_left=w.window_left,
                    window_right=w.window_right, seg_q=seg, q_offset=w.q_offset)
        total += int(np.count_nonzero(a))
    return total


@pytest.mark.parametrize("name", [n for n, w in ALL_WORKLOADS.items() if w.L * w.keys <= 1 << 26])
def test_pair_count_matches_mask_definition(name):
    w = ALL_WORKLOADS[name]
    seg = segment_ids(w.L, w.seed, w.seg_min, w.seg_max) if w.segments else None
    assert _bench().unmasked_pairs(None, w, seg) == _allowed_count(w, seg)


def test_pair_count_decode_closed_form():
    """16 causal rows at the last 16 of 32768 positions: row i sees
    32768 - 16 + i + 1 keys."""
    w = ALL_WORKLOADS["decode_gqa_bf16_Lq16_Lkv32768"]
    assert _bench().unmasked_pairs(None, w, None) == sum(32768 - 16 + i + 1 for i in range(16))


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_median_min():
    b = _bench()
    assert b.median_min([3.0, 1.0, 2.0]) == (2.0, 1.0)
    assert b.median_min([4.0, 1.0, 2.0, 3.0]) == (2.5, 1.0)


def test_causal_only_pairs_of_masked_workloads():
    """The sparsity leg's causal-only pair count is the causal count of the
    same shape: L (L + 1) / 2 per (b, h)."""
    b = _bench()
    for name in ("gqa_window_bf16_L32768", "gqa_docs_cap_bf16_L32768"):
        w = ALL_WORKLOADS[name]
        seg = segment_ids(w.L, w.seed, w.seg_min, w.seg_max) if w.segments else None
        assert b.unmasked_pairs(None, w, seg, causal_only=True) == w.L * (w.L + 1) // 2
        assert b.unmasked_pairs(None, w, seg) < w.L * (w.L + 1) // 2


def test_cpu_baseline_pool_bookkeeping():
    """The oracle baseline runs as a pool of single-threaded workers and
    reports the cores it used, the host's core count and CPU model, and an
    effective rate over the unmasked FLOPs of the sample it timed."""
    from block_sparse_flash_amd.inputs import make_inputs
    b = _bench()
    w = ALL_WORKLOADS["causal_f32_L256_d64"]
    q, k, v, seg = make_inputs(w)
    r = b.cpu_baseline(w, q, k, v, seg, budget_s=0.5, max_workers=2)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0
    assert r["cores"] == min(2, r["nproc"]) and r["nproc"] >= 1 and isinstance(r["cpu_model"], str)
    assert "work items" in r["sample"]
    rb = b.cpu_baseline(w, q, k, v, seg, budget_s=0.5, backward=True, max_workers=2)
    assert rb["value"] > 0 and "backward" in rb["sample"]
