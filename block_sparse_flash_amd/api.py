"""Python binding of the C ABI: ``compile_mask`` and ``splash_fwd``.

Argument marshalling only: the mask tables come from ``attn_mask_compile``
(host C++) and the forward runs in the library's HIP kernels.  PyTorch
provides device memory, host<->device copies and the current stream.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from . import _lib

_DTYPES = {"f32": _lib.SPLASH_F32, "bf16": _lib.SPLASH_BF16}
_MASK_MODES = {"computed": _lib.SPLASH_MASK_COMPUTED, "stored": _lib.SPLASH_MASK_STORED}


def _ptr(arr: Optional[np.ndarray]):
    return None if arr is None else arr.ctypes.data_as(ctypes.c_void_p)


def _seg_array(seg, L):
    if seg is None:
        return None
    a = np.ascontiguousarray(np.asarray(seg).reshape(-1), dtype=np.int32)
    if a.shape[0] != L:
        raise ValueError(f"segment ids have length {a.shape[0]}, expected {L}")
    return a


def _seg_digest(seg_q, seg_kv):
    """Digest of one row of query and key segment ids (key ids default to
    the query ids)."""
    import hashlib
    h = hashlib.sha256()
    sq = np.ascontiguousarray(np.asarray(seg_q).reshape(-1), dtype=np.int32)
    skv = sq if seg_kv is None else np.ascontiguousarray(np.asarray(seg_kv).reshape(-1), dtype=np.int32)
    h.update(sq.tobytes())
    h.update(b"|")
    h.update(skv.tobytes())
    return h.hexdigest()


def _mask_key(causal, window_left, window_right, seg_q, seg_kv, q_offset, digest=None):
    """What a table was compiled for: the mask parameters and a digest of
    the segment ids (``digest``, or computed from seg_q / seg_kv)."""
    if digest is None and seg_q is not None:
        digest = _seg_digest(seg_q, seg_kv)
    return (bool(causal), int(window_left), int(window_right), digest, int(q_offset))


def _host_rows(seg, n, name):
    """Segment ids ([n] or [rows, n], numpy or torch) as a host int32 array
    [rows, n]."""
    a = seg.detach().cpu().numpy() if hasattr(seg, "detach") else np.asarray(seg)
    a = np.ascontiguousarray(a, dtype=np.int32)
    if a.ndim not in (1, 2) or a.shape[-1] != n:
        raise ValueError(f"{name} must be [{n}] or [B, {n}]; got shape {tuple(a.shape)}")
    return a.reshape(-1, n)


def _segments(seg_q, seg_kv, B, L, L_kv, device, cache=None):
    """The segment ids of a call: host rows ``hq`` / ``hkv`` (1 or B rows),
    whether the batch rows differ (``per_batch``), device copies
    ``dev_q`` [B, L] / ``dev_kv`` [B, L_kv] and the digest of row 0
    (``digest0``); None without segment ids.  With ``cache`` (the dict of the
    MaskTables the call uses) a call with the same ids as the previous one
    reuses its device copies and digest: no host-device copy, no
    synchronisation and no hashing per call."""
    import torch
    if seg_q is None:
        if seg_kv is not None:
            raise ValueError("seg_kv given without seg_q")
        return None
    hq = _host_rows(seg_q, L, "seg_q")
    hkv = None if seg_kv is None else _host_rows(seg_kv, L_kv, "seg_kv")
    if hkv is None and L_kv != L:
        raise ValueError("seg_kv is required when L_kv != L")
    if hq.shape[0] not in (1, B) or (hkv is not None and hkv.shape[0] not in (1, B)):
        raise ValueError("segment ids must be [L] or [B, L] ([L_kv] or [B, L_kv] for seg_kv)")
    dkey = str(torch.device(device))
    if cache is not None:
        c = cache.get("seg")
        if (c is not None and c["B"] == B and c["device"] == dkey and np.array_equal(c["hq"], hq)
                and ((hkv is None and c["hkv"] is None)
                     or (hkv is not None and c["hkv"] is not None and np.array_equal(c["hkv"], hkv)))):
            return c
    per_batch = B > 1 and (bool((hq != hq[:1]).any()) or (hkv is not None and bool((hkv != hkv[:1]).any())))
    # A row-major copy: numpy's default order would follow the broadcast's
    # zero stride and lay [1, n] ids broadcast to [B, n] out column-major.
    up = lambda h, n: torch.from_numpy(np.array(np.broadcast_to(h, (B, n)), dtype=np.int32, order="C")).to(device)
    rec = {"B": B, "device": dkey, "hq": hq.copy(), "hkv": None if hkv is None else hkv.copy(),
           "per_batch": per_batch, "dev_q": up(hq, L), "dev_kv": None if hkv is None else up(hkv, L_kv),
           "digest0": _seg_digest(hq[0], None if hkv is None else hkv[0])}
    for t in (rec["dev_q"], rec["dev_kv"]):
        if t is not None and not t.is_contiguous():
            raise RuntimeError("segment ids must reach the kernels row-major")
    if cache is not None:
        cache["seg"] = rec
    return rec


def _seg_row(h, b):
    """Row b of host segment ids held as 1 or B rows (None stays None)."""
    return None if h is None else h[b if h.shape[0] > 1 else 0]


def _check_tables(tabs, bq, bkv, L, L_kv, key):
    got = (tabs.block_q, tabs.block_kv, tabs.L_q, tabs.L_kv, tabs.q_offset)
    if got != (bq, bkv, L, L_kv, key[4]):
        raise ValueError(f"tables were compiled for (block_q, block_kv, L_q, L_kv, q_offset)="
                         f"{got}; need {(bq, bkv, L, L_kv, key[4])}")
    if tabs.mask_key is not None and tabs.mask_key != key:
        names = ("causal", "window_left", "window_right", "segment ids", "q_offset")
        diff = [n for n, a, b in zip(names, tabs.mask_key, key) if a != b]
        raise ValueError("tables were compiled for another mask (differs in " + ", ".join(diff) + ")")


def _check_out(t, name, shape, dtype, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}; "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}"
                         + ("" if t.is_contiguous() else " (not contiguous)"))


@dataclass
class MaskTables:
    """Host copy of the MaskInfo execution table (see include/splash.h)."""

    L_q: int
    L_kv: int
    block_q: int
    block_kv: int
    n_q_blocks: int
    n_kv_blocks: int
    n_active: int
    n_partial: int
    n_patterns: int
    block_mask: np.ndarray
    active_rows: np.ndarray
    active_cols: np.ndarray
    block_code: np.ndarray
    mask_next: np.ndarray
    bounds: np.ndarray
    row_ptr: np.ndarray
    row_order: np.ndarray
    partial_mask_blocks: np.ndarray
    q_offset: int = 0
    # (causal, window_left, window_right, segment-id digest, q_offset) the
    # tables were compiled for; calls with another mask are refused.
    mask_key: Optional[tuple] = None
    _device: dict = field(default_factory=dict, repr=False)
    _columns: Optional[dict] = field(default=None, repr=False)

    def columns(self):
        """Column-major view of the active list (``attn_mask_columns``):
        host arrays ``col_ptr`` [n_kv_blocks + 1], ``col_rows`` and
        ``col_entry`` [n_active], and ``col_order`` [n_kv_blocks], the
        columns most active blocks first (``attn_mask_column_order``)."""
        if self._columns is None:
            lib = _lib.load()
            cols = {"col_ptr": np.zeros(self.n_kv_blocks + 1, np.int32),
                    "col_rows": np.zeros(self.n_active, np.int32),
                    "col_entry": np.zeros(self.n_active, np.int32)}
            row_ptr = np.ascontiguousarray(self.row_ptr, dtype=np.int32)
            active_cols = np.ascontiguousarray(self.active_cols, dtype=np.int32)
            _lib.check(lib.attn_mask_columns(self.n_q_blocks, self.n_kv_blocks, self.n_active,
                                             _ptr(row_ptr), _ptr(active_cols),
                                             _ptr(cols["col_ptr"]), _ptr(cols["col_rows"]),
                                             _ptr(cols["col_entry"])))
            cols["col_order"] = np.zeros(self.n_kv_blocks, np.int32)
            _lib.check(lib.attn_mask_column_order(self.n_kv_blocks, _ptr(cols["col_ptr"]),
                                                  _ptr(cols["col_order"])))
            self._columns = cols
        return self._columns

    def device_columns(self, device):
        """Device copies (torch tensors) of ``col_ptr``, ``col_rows`` and
        ``col_order``."""
        import torch
        key = "cols:" + str(torch.device(device))
        if key not in self._device:
            cols = self.columns()
            def up(a):
                t = torch.from_numpy(np.ascontiguousarray(a)).to(torch.int32)
                return (t if t.numel() else torch.zeros(1, dtype=torch.int32)).to(device)
            self._device[key] = {k: up(cols[k]) for k in ("col_ptr", "col_rows", "col_order")}
        return self._device[key]

    def device(self, device):
        """Device copies (torch tensors) of the arrays the forward reads."""
        import torch
        key = str(torch.device(device))
        if key not in self._device:
            def up(a, dt):
                t = torch.from_numpy(np.ascontiguousarray(a)).to(dt)
                if t.numel() == 0:   # keep a valid, non-null allocation
                    t = torch.zeros(1, dtype=dt)
                return t.to(device)
            self._device[key] = {
                "row_ptr": up(self.row_ptr, torch.int32),
                "row_order": up(self.row_order, torch.int32),
                "active_cols": up(self.active_cols, torch.int32),
                "block_code": up(self.block_code, torch.int8),
                "mask_next": up(self.mask_next, torch.int32),
                "partial_mask_blocks": up(self.partial_mask_blocks.reshape(-1), torch.uint8),
            }
        return self._device[key]


def compile_mask(L_q: int, block_q: int, block_kv: int, *, L_kv: Optional[int] = None,
                 causal: bool = False, window_left: int = -1, window_right: int = -1,
                 seg_q=None, seg_kv=None, q_offset: int = 0) -> MaskTables:
    """Run ``attn_mask_compile`` (both phases) and return the host tables.
    Query row i sits at key position ``q_offset + i``."""
    lib = _lib.load()
    L_kv = L_q if L_kv is None else L_kv
    sq = _seg_array(seg_q, L_q)
    skv = _seg_array(seg_kv, L_kv) if seg_kv is not None else None
    desc = _lib.MaskDesc(L_q, L_kv, block_q, block_kv, int(bool(causal)), window_left,
                         window_right, _ptr(sq), _ptr(skv), int(q_offset))
    sizes = _lib.MaskSizes()
    _lib.check(lib.attn_mask_compile(ctypes.byref(desc), ctypes.byref(sizes), None))
    nq, nkv, na, npat = sizes.n_q_blocks, sizes.n_kv_blocks, sizes.n_active, sizes.n_patterns
    arrays = {
        "block_mask": np.zeros(nq * nkv, np.int8),
        "active_rows": np.zeros(na, np.int32),
        "active_cols": np.zeros(na, np.int32),
        "block_code": np.zeros(na, np.int8),
        "mask_next": np.zeros(na, np.int32),
        "bounds": np.zeros(na, np.uint8),
        "row_ptr": np.zeros(nq + 1, np.int32),
        "row_order": np.zeros(nq, np.int32),
        "partial_mask_blocks": np.zeros(npat * block_q * block_kv, np.uint8),
    }
    tabs = _lib.MaskTablesC(*(_ptr(arrays[name]) for name, _ in _lib.MaskTablesC._fields_))
    _lib.check(lib.attn_mask_compile(ctypes.byref(desc), ctypes.byref(sizes), ctypes.byref(tabs)))
    arrays["block_mask"] = arrays["block_mask"].reshape(nq, nkv)
    arrays["partial_mask_blocks"] = arrays["partial_mask_blocks"].reshape(npat, block_q, block_kv)
    return MaskTables(L_q, L_kv, block_q, block_kv, nq, nkv, na, sizes.n_partial, npat, **arrays,
                      q_offset=int(q_offset),
                      mask_key=_mask_key(causal, window_left, window_right, sq, skv, q_offset))


def fwd_tile(dtype: str, d_qk: int, d_v: int):
    """(block_q, block_kv) the forward kernel uses for this dtype and head dims."""
    lib = _lib.load()
    bq, bkv = ctypes.c_int32(), ctypes.c_int32()
    _lib.check(lib.splash_fwd_tile(_DTYPES[dtype], d_qk, d_v, ctypes.byref(bq), ctypes.byref(bkv)))
    return bq.value, bkv.value


def fwd_tiles(dtype: str, d_qk: int, d_v: int):
    """Every (block_q, block_kv) the plain forward has a kernel for, the
    default tile first (``splash_fwd_tiles``)."""
    lib = _lib.load()
    n = ctypes.c_int32()
    _lib.check(lib.splash_fwd_tiles(_DTYPES[dtype], d_qk, d_v, None, None, 0, ctypes.byref(n)))
    bq = np.zeros(n.value, np.int32)
    bkv = np.zeros(n.value, np.int32)
    _lib.check(lib.splash_fwd_tiles(_DTYPES[dtype], d_qk, d_v, _ptr(bq), _ptr(bkv), n.value,
                                    ctypes.byref(n)))
    return [(int(a), int(b)) for a, b in zip(bq, bkv)]


def bwd_tile(dtype: str, d_qk: int, d_v: int):
    """(block_q, block_kv) the backward's tables are compiled with."""
    lib = _lib.load()
    bq, bkv = ctypes.c_int32(), ctypes.c_int32()
    _lib.check(lib.splash_bwd_tile(_DTYPES[dtype], d_qk, d_v, ctypes.byref(bq), ctypes.byref(bkv)))
    return bq.value, bkv.value


def pick_tile(dtype: str, d_qk: int, d_v: int, L: int, group: int):
    """The tile ``splash_fwd`` compiles tables for when none are given: the
    64-row decode tile for few query rows per K/V head (its query heads are
    packed into one row space when L is below the tile), else the default."""
    if L <= 64 and (64, 64) in fwd_tiles(dtype, d_qk, d_v):
        return (64, 64)
    return fwd_tile(dtype, d_qk, d_v)


def _torch_dtype_name(t):
    import torch
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.float32:
        return "f32"
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.float32 or torch.bfloat16")


def splash_fwd(q, k, v, *, scale: Optional[float] = None, soft_cap: float = 0.0,
               causal: bool = False, window_left: int = -1, window_right: int = -1,
               seg_q=None, seg_kv=None, tables: Optional[MaskTables] = None,
               mask_mode: str = "computed", out=None, lse=None, return_lse: bool = True,
               max_logit: Optional[float] = None, n_split: int = 1, workspace=None,
               q_offset: int = 0, no_alloc: bool = False, stream=None):
    """Block-sparse attention forward on the GPU.

    q [B, Hq, L, d_qk], k [B, Hkv, L_kv, d_qk], v [B, Hkv, L_kv, d_v]:
    contiguous torch tensors on one GPU, all float32 or all bfloat16.  Query
    row i sits at key position ``q_offset + i`` (decoding the last L of L_kv
    positions: ``q_offset = L_kv - L``); L_kv != L or q_offset != 0 is bf16
    only.  ``seg_q``: segment ids [L] (shared by the batch) or [B, L];
    ``seg_kv``: [L_kv] or [B, L_kv] (required when L_kv != L).  ``tables``:
    a MaskTables compiled for this mask at the kernel's block sizes
    (``fwd_tile``); compiled here when omitted.  ``max_logit``: the Max Logit
    Estimate constant (logit units) used instead of the running row max, or
    None.  Returns (o, lse) with o like q but with d_v, lse float32 [B, Hq, L]
    (None if ``return_lse`` is False).  ``n_split`` > 1 (bf16 only): each
    row's active kv blocks are cut into that many chunks computed as separate
    items and merged through their log-sum-exp (``splash_attn_fwd_split``);
    ``workspace`` is a device tensor of at least ``split_workspace_bytes``
    bytes, allocated here when omitted.  ``no_alloc`` (with ``n_split`` > 1):
    the partials go to the library's static device scratch instead
    (``splash_attn_fwd_split_noalloc``; no workspace, calls on one device
    must not overlap).
    """
    import torch
    lib = _lib.load()
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k and v must be GPU tensors")
    dt = _torch_dtype_name(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, Hq, L, d_qk = q.shape
    Hkv, L_kv = k.shape[1], k.shape[2]
    d_v = v.shape[3]
    if tuple(k.shape) != (B, Hkv, L_kv, d_qk) or tuple(v.shape[:3]) != (B, Hkv, L_kv):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    if scale is None:
        scale = 1.0 / float(d_qk) ** 0.5
    # Tables given: their tile (the library checks a kernel exists for it);
    # else the default tile.
    bq, bkv = ((tables.block_q, tables.block_kv) if tables is not None
               else pick_tile(dt, d_qk, d_v, L, Hq // max(Hkv, 1)))

    segs = _segments(seg_q, seg_kv, B, L, L_kv, q.device,
                     None if tables is None else tables._device)
    seg_q_dev = None if segs is None else segs["dev_q"]
    seg_kv_dev = None if segs is None else segs["dev_kv"]
    per_batch = segs is not None and segs["per_batch"]

    _check_out(out, "out", (B, Hq, L, d_v), q.dtype, q.device)
    _check_out(lse, "lse", (B, Hq, L), torch.float32, q.device)
    if out is None:
        out = torch.empty((B, Hq, L, d_v), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream

    ws_ptr, ws_bytes = None, 0
    if no_alloc and (n_split == 1 or workspace is not None):
        raise ValueError("no_alloc is for the split-KV forward (n_split > 1) without a workspace")
    if n_split != 1 and not no_alloc:
        need = split_workspace_bytes(n_split, 1 if per_batch else B, Hq, L, d_v)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        if workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous tensor on {q.device}")
        have = workspace.numel() * workspace.element_size()
        if have < need:
            raise ValueError(f"workspace holds {have} bytes, {need} needed")
        ws_ptr, ws_bytes = workspace.data_ptr(), have

    batches = range(B) if per_batch else [None]
    for bsel in batches:
        ids_q = None if segs is None else _seg_row(segs["hq"], bsel or 0)
        ids_kv = None if segs is None else _seg_row(segs["hkv"], bsel or 0)
        if tables is None or per_batch:
            tabs = compile_mask(L, bq, bkv, L_kv=L_kv, causal=causal, window_left=window_left,
                                window_right=window_right, seg_q=ids_q, seg_kv=ids_kv,
                                q_offset=q_offset)
            digest = None
        else:
            tabs = tables
            digest = None if segs is None else segs["digest0"]
        _check_tables(tabs, bq, bkv, L, L_kv,
                      _mask_key(causal, window_left, window_right, ids_q, ids_kv, q_offset, digest))
        dev = tabs.device(q.device)
        if bsel is None:
            qb, kb, vb, ob = q, k, v, out
            lb = lse
            sqb, skb, nb = seg_q_dev, seg_kv_dev, B
        else:
            sl = slice(bsel, bsel + 1)
            qb, kb, vb, ob = q[sl], k[sl], v[sl], out[sl]
            lb = None if lse is None else lse[sl]
            sqb = seg_q_dev[sl]
            skb = None if seg_kv_dev is None else seg_kv_dev[sl]
            nb = 1
        args = _lib.FwdArgs(
            _DTYPES[dt], nb, Hq, Hkv, L, d_qk, d_v,
            qb.data_ptr(), kb.data_ptr(), vb.data_ptr(), ob.data_ptr(),
            None if lb is None else lb.data_ptr(),
            int(bool(causal)), window_left, window_right,
            None if sqb is None else sqb.data_ptr(),
            None if skb is None else skb.data_ptr(),
            bq, bkv, tabs.n_q_blocks, tabs.n_active, tabs.n_patterns,
            dev["row_ptr"].data_ptr(), dev["row_order"].data_ptr(),
            dev["active_cols"].data_ptr(), dev["block_code"].data_ptr(),
            dev["mask_next"].data_ptr(), dev["partial_mask_blocks"].data_ptr(),
            _MASK_MODES[mask_mode], float(scale), float(soft_cap),
            0 if max_logit is None else 1, 0.0 if max_logit is None else float(max_logit),
            L_kv, int(q_offset))
        if n_split == 1:
            _lib.check(lib.splash_attn_fwd(ctypes.byref(args), ctypes.c_void_p(stream)))
        elif no_alloc:
            _lib.check(lib.splash_attn_fwd_split_noalloc(ctypes.byref(args), int(n_split),
                                                         ctypes.c_void_p(stream)))
        else:
            _lib.check(lib.splash_attn_fwd_split(ctypes.byref(args), int(n_split),
                                                 ctypes.c_void_p(ws_ptr), ctypes.c_int64(ws_bytes),
                                                 ctypes.c_void_p(stream)))
    return out, (lse if return_lse else None)


def split_workspace_bytes(n_split: int, B: int, Hq: int, L: int, d_v: int) -> int:
    """Device workspace bytes of a split-KV forward (``splash_split_workspace_bytes``)."""
    lib = _lib.load()
    nb = ctypes.c_int64()
    _lib.check(lib.splash_split_workspace_bytes(int(n_split), int(B), int(Hq), int(L), int(d_v),
                                                ctypes.byref(nb)))
    return nb.value


def clock_probe(out, n_groups: int = 8, stream=None) -> None:
    """Enqueue ``splash_clock_probe``: ``n_groups`` single-wave work-groups
    write (shader-clock cycles, real-time counter, XCD id) into ``out``, an
    int64 device tensor of at least 3 * n_groups elements (measurement only),
    on ``stream`` (a raw stream handle; None: torch's current stream)."""
    import torch
    lib = _lib.load()
    if out.dtype != torch.int64 or not out.is_cuda or not out.is_contiguous() or out.numel() < 3 * n_groups:
        raise ValueError("out must be a contiguous int64 device tensor of >= 3 * n_groups elements")
    if stream is None:
        stream = torch.cuda.current_stream(out.device).cuda_stream
    _lib.check(lib.splash_clock_probe(ctypes.c_void_p(out.data_ptr()), int(n_groups),
                                      ctypes.c_void_p(stream)))


def realtime_khz() -> int:
    """Rate of the current device's real-time counter in kHz (``splash_realtime_khz``)."""
    lib = _lib.load()
    khz = ctypes.c_int32()
    _lib.check(lib.splash_realtime_khz(ctypes.byref(khz)))
    return khz.value


def splash_bwd(q, k, v, o, lse, dout, *, scale: Optional[float] = None, soft_cap: float = 0.0,
               causal: bool = False, window_left: int = -1, window_right: int = -1,
               seg_q=None, seg_kv=None, q_offset: int = 0, tables: Optional[MaskTables] = None,
               stream=None, natural_order: bool = False):
    """Block-sparse attention backward on the GPU (``splash_attn_bwd``).

    q, k, v, ``o`` (the forward's output) and ``dout`` (the upstream
    gradient, shaped like o) are contiguous bfloat16 GPU tensors with the
    forward's shapes; ``lse`` is the forward's float32 lse [B, Hq, L]; the
    mask arguments are those of the forward.  Returns (dq, dk, dv) as float32
    tensors shaped like q, k and v.  Head dims (64, 64), (128, 128) or
    (192, 128).  ``natural_order`` passes no row and column orders, so the
    kernels take their items in table order instead of longest first (the
    results are the same; it is slower where rows or columns differ in
    length).
    """
    import torch
    lib = _lib.load()
    for t in (q, k, v, o, dout):
        if not t.is_cuda or t.dtype != torch.bfloat16:
            raise TypeError("q, k, v, o and dout must be bfloat16 GPU tensors")
    if not lse.is_cuda or lse.dtype != torch.float32:
        raise TypeError("lse must be a float32 GPU tensor")
    B, Hq, L, d_qk = q.shape
    Hkv, L_kv = k.shape[1], k.shape[2]
    d_v = v.shape[3]
    if (tuple(k.shape) != (B, Hkv, L_kv, d_qk) or tuple(v.shape[:3]) != (B, Hkv, L_kv)
            or tuple(o.shape) != (B, Hq, L, d_v) or tuple(dout.shape) != (B, Hq, L, d_v)
            or tuple(lse.shape) != (B, Hq, L)):
        raise ValueError("shape mismatch among q, k, v, o, lse, dout")
    q, k, v, o, dout, lse = (t.contiguous() for t in (q, k, v, o, dout, lse))
    if scale is None:
        scale = 1.0 / float(d_qk) ** 0.5
    bq, bkv = bwd_tile("bf16", d_qk, d_v)
    segs = _segments(seg_q, seg_kv, B, L, L_kv, q.device,
                     None if tables is None else tables._device)
    sq = None if segs is None else segs["dev_q"]
    skv = None if segs is None else segs["dev_kv"]
    per_batch = segs is not None and segs["per_batch"]
    dq = torch.empty((B, Hq, L, d_qk), dtype=torch.float32, device=q.device)
    dk = torch.empty((B, Hkv, L_kv, d_qk), dtype=torch.float32, device=q.device)
    dv = torch.empty((B, Hkv, L_kv, d_v), dtype=torch.float32, device=q.device)
    delta = torch.empty((B, Hq, max(L, 1)), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    for bsel in (range(B) if per_batch else [None]):
        b0 = bsel or 0
        ids_q = None if segs is None else _seg_row(segs["hq"], b0)
        ids_kv = None if segs is None else _seg_row(segs["hkv"], b0)
        if tables is None or per_batch:
            tabs = compile_mask(L, bq, bkv, L_kv=L_kv, causal=causal, window_left=window_left,
                                window_right=window_right, q_offset=q_offset,
                                seg_q=ids_q, seg_kv=ids_kv)
            digest = None
        else:
            tabs = tables
            digest = None if segs is None else segs["digest0"]
        _check_tables(tabs, bq, bkv, L, L_kv,
                      _mask_key(causal, window_left, window_right, ids_q, ids_kv, q_offset, digest))
        dev = tabs.device(q.device)
        cdev = tabs.device_columns(q.device)
        sl = slice(None) if bsel is None else slice(bsel, bsel + 1)
        nb = B if bsel is None else 1
        ptr = lambda t: None if t is None else t[sl].data_ptr()
        args = _lib.BwdArgs(
            _DTYPES["bf16"], nb, Hq, Hkv, L, L_kv, int(q_offset), d_qk, d_v,
            ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), ptr(dout), ptr(dq), ptr(dk), ptr(dv),
            ptr(delta), int(bool(causal)), window_left, window_right, ptr(sq), ptr(skv),
            bq, bkv, tabs.n_q_blocks, tabs.n_kv_blocks, tabs.n_active,
            dev["row_ptr"].data_ptr(), None if natural_order else dev["row_order"].data_ptr(),
            dev["active_cols"].data_ptr(), cdev["col_ptr"].data_ptr(), cdev["col_rows"].data_ptr(),
            None if natural_order else cdev["col_order"].data_ptr(),
            float(scale), float(soft_cap))
        _lib.check(lib.splash_attn_bwd(ctypes.byref(args), ctypes.c_void_p(stream)))
    return dq, dk, dv
