"""Seeded synthetic inputs and the named workloads.

This module only draws random numbers and describes shapes: it holds none of
the attention arithmetic, so both the HIP path and the float64 oracle can be
fed from it.  Every tensor is drawn on the host with numpy's PCG64
``default_rng(seed)`` as float32 standard normals in the order q, k, v, then
stored in the workload's dtype (bf16 by round-to-nearest-even).  Segment ids
are drawn from their own stream ``default_rng(seed + 1000)``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, asdict
from typing import Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One attention-forward problem: shapes, mask and input distribution."""

    name: str
    dtype: str              # "f32" or "bf16": storage and input dtype
    B: int
    Hq: int
    Hkv: int
    L: int
    d_qk: int
    d_v: int
    causal: bool = True
    window_left: int = -1   # -1 = unbounded
    window_right: int = -1
    segments: bool = False  # segment ids with lengths U[seg_min, seg_max]
    seg_min: int = 512
    seg_max: int = 8192
    soft_cap: float = 0.0   # <= 0: no cap
    qk_std: float = 1.0     # q and k ~ N(0, qk_std^2); v ~ N(0, 1)
    seed: int = 0
    scale: Optional[float] = None   # None: 1/sqrt(d_qk)
    L_kv: Optional[int] = None      # key positions; None: L
    q_offset: int = 0               # query row i sits at key position q_offset + i
    n_split: int = 1                # split-KV chunks the bench uses by default
    tile: Optional[Tuple[int, int]] = None   # forward tile the bench uses (None: default)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.d_qk)

    @property
    def keys(self) -> int:
        return self.L if self.L_kv is None else self.L_kv

    def asdict(self):
        d = asdict(self)
        d["scale"] = self.softmax_scale
        return d


# The five problems of the block-sparse attention forward: a tiny fp32 causal
# case, dense causal MHA at L=4096 (d=128 and the 192/128 wide head), GQA with
# a 4096-key sliding window at L=32768, and GQA with a document mask plus a
# logit soft cap at L=32768.
WORKLOADS = {
    "causal_f32_L256_d64": Workload(
        "causal_f32_L256_d64", "f32", 1, 1, 1, 256, 64, 64,
        causal=True, seed=1),
    "causal_mha_bf16_L4096_d128": Workload(
        "causal_mha_bf16_L4096_d128", "bf16", 2, 32, 32, 4096, 128, 128,
        causal=True, seed=2),
    "causal_mha_bf16_L4096_d192": Workload(
        "causal_mha_bf16_L4096_d192", "bf16", 1, 128, 128, 4096, 192, 128,
        causal=True, seed=3),
    "gqa_window_bf16_L32768": Workload(
        "gqa_window_bf16_L32768", "bf16", 1, 32, 8, 32768, 128, 128,
        causal=True, window_left=4095, seed=4, tile=(256, 128)),
    "gqa_docs_cap_bf16_L32768": Workload(
        "gqa_docs_cap_bf16_L32768", "bf16", 1, 16, 4, 32768, 128, 128,
        causal=True, segments=True, soft_cap=50.0, qk_std=math.sqrt(2.0),
        seed=5),
}

# Tiles (None: the default 256x64): the block-size sweep's fastest for each
# workload, except that the documents workload keeps 256 rows (128-row tiles
# were 1% faster there but read each K/V block for twice as many items, 1.6x
# the HBM bytes); 128 keys per block pay off only for the long window.
WORKLOAD_ORDER = list(WORKLOADS)

# A shape for the split-KV forward: two heads of causal attention at
# L=32768, 256 (head, q-block row) items of 4 to 512 active blocks, so that
# without splitting the longest rows set the time on 256 CUs.
EXTRA_WORKLOADS = {
    "causal_bf16_L32768_H2": Workload(
        "causal_bf16_L32768_H2", "bf16", 1, 2, 2, 32768, 128, 128,
        causal=True, seed=6),
    # Decoding 16 new rows per sequence (speculative or multi-token decode)
    # against a 32768-position K/V cache: GQA 32/8, causal, the new rows at
    # the last 16 positions; the 4 query heads of a K/V head packed into one
    # 64-row decode tile, split-KV into 4 chunks per row.
    "decode_gqa_bf16_Lq16_Lkv32768": Workload(
        "decode_gqa_bf16_Lq16_Lkv32768", "bf16", 8, 32, 8, 16, 128, 128,
        causal=True, seed=7, L_kv=32768, q_offset=32768 - 16, n_split=4, tile=(64, 64)),
}
ALL_WORKLOADS = {**WORKLOADS, **EXTRA_WORKLOADS}


def segment_ids(L: int, seed: int, lo: int = 512, hi: int = 8192) -> np.ndarray:
    """Contiguous document ids 0, 1, 2, ... with lengths drawn uniformly from
    [lo, hi] (inclusive) until they cover L; the last one is cut at L."""
    rng = np.random.default_rng(seed + 1000)
    ids = np.empty(L, dtype=np.int32)
    pos, doc = 0, 0
    while pos < L:
        n = int(rng.integers(lo, hi, endpoint=True))
        n = min(n, L - pos)
        ids[pos:pos + n] = doc
        pos += n
        doc += 1
    return ids


def draw_qkv(B, Hq, Hkv, L, d_qk, d_v, seed, qk_std=1.0, L_kv=None):
    """float32 q [B,Hq,L,d_qk], k [B,Hkv,L_kv,d_qk], v [B,Hkv,L_kv,d_v]."""
    L_kv = L if L_kv is None else L_kv
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, L, d_qk), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, L_kv, d_qk), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, L_kv, d_v), dtype=np.float32)
    if qk_std != 1.0:
        q *= np.float32(qk_std)
        k *= np.float32(qk_std)
    return q, k, v


def stored(arr: np.ndarray, dtype: str):
    """The tensor as stored for the kernel: a contiguous torch CPU tensor in
    ``dtype`` ("f32" or "bf16", the latter rounded to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if dtype == "bf16":
        return t.to(torch.bfloat16).contiguous()
    if dtype == "f32":
        return t.to(torch.float32).contiguous()
    raise ValueError(f"unknown dtype {dtype}")


def as_f64(t) -> np.ndarray:
    """Decode a stored torch tensor to float64 numpy (exact widening)."""
    return t.detach().to("cpu").float().numpy().astype(np.float64)


def make_inputs(w: Workload):
    """(q, k, v, seg) for a workload: q/k/v stored torch CPU tensors, seg an
    int32 numpy array [L] or None."""
    q, k, v = draw_qkv(w.B, w.Hq, w.Hkv, w.L, w.d_qk, w.d_v, w.seed, w.qk_std, L_kv=w.keys)
    if w.segments and (w.keys != w.L or w.q_offset):
        raise ValueError("segment ids are drawn for L_q = L_kv workloads only")
    seg = segment_ids(w.L, w.seed, w.seg_min, w.seg_max) if w.segments else None
    return stored(q, w.dtype), stored(k, w.dtype), stored(v, w.dtype), seg
