"""Benchmark of the block-sparse attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one forward (``splash_attn_fwd``: every active block of every
head) over the workload's resident inputs; the MaskInfo table is compiled
once before timing (its time is reported as ``mask_compile_ms``).  Prints
one JSON line with the effective TFLOP/s over unmasked pairs, the roofline
figures of the forward kernel, and the float64 oracle timed on the host CPU
over a bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "causal_mha_bf16_L4096_d128"
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}   # dense MFMA bf16; fp32 vector
PEAK_HBM_GBS = 8000.0                           # HBM3E
PEAK_CLOCK_HZ = 2.4e9                           # clock of the published peaks (256 CUs)
KERNEL_SOURCES = {"bf16": ("splash_fwd_bf16_kernel.h", "splash_fwd_bf16.hip"),
                  "f32": ("splash_fwd_f32.hip",)}


def unmasked_pairs(tabs, w, seg, causal_only=False):
    """Exact count of allowed (query, key) pairs per (b, h), from the mask
    definition, summed row by row with interval arithmetic (segments: the
    allowed keys of a row are the part of its interval inside its segment,
    segments being contiguous here).  ``causal_only``: the same shape under
    the causal mask alone."""
    return int(pairs_per_row(w, None if causal_only else seg, causal_only).sum())


def pairs_per_row(w, seg, causal_only=False):
    """Allowed keys of every query row (numpy int64 [L])."""
    import numpy as np
    L = w.L
    i = w.q_offset + np.arange(L, dtype=np.int64)   # key positions of the query rows
    lo = np.zeros(L, np.int64)
    hi = np.full(L, w.keys - 1, np.int64)
    if w.causal:
        hi = np.minimum(hi, i)
    if w.window_left >= 0 and not causal_only:
        lo = np.maximum(lo, i - w.window_left)
    if w.window_right >= 0 and not causal_only:
        hi = np.minimum(hi, i + w.window_right)
    if seg is not None:
        seg = np.asarray(seg)
        assert np.all(np.diff(seg) >= 0), "pair count assumes contiguous segments"
        starts = np.searchsorted(seg, seg, side="left")
        ends = np.searchsorted(seg, seg, side="right") - 1
        lo = np.maximum(lo, starts)
        hi = np.minimum(hi, ends)
    return np.maximum(hi - lo + 1, 0)


def kernel_sha(dtype):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_flash_amd", "csrc")
    for name in (*KERNEL_SOURCES[dtype], "fwd_params.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(workload, dtype):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"splash_fwd_{dtype}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"kernel_sha256_16:\s*([0-9a-f]+)", text)
    tb = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not tb or sha.group(1) != kernel_sha(dtype):
        return None
    return float(tb.group(1))


def host_cpu():
    """(usable cores, CPU model name) of this host."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return n, model


# Inputs of the oracle workers: set in the parent before the pool forks, so
# the children share them copy-on-write (no pickling of the arrays).
_ORACLE = {}


def _limit_threads():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _oracle_fwd_item(item):
    """One work item of the forward baseline: rows [r0, r1) of head (b, h)."""
    from oracle import attention_ref
    b, h, r0, r1 = item
    w, seg = _ORACLE["w"], _ORACLE["seg"]
    t0 = time.perf_counter()
    attention_ref(_ORACLE["q"], _ORACLE["k"], _ORACLE["v"], scale=w.softmax_scale,
                  soft_cap=w.soft_cap, causal=w.causal, window_left=w.window_left,
                  window_right=w.window_right, seg_q=seg, heads=[(b, h)],
                  rows=list(range(r0, r1)), q_offset=w.q_offset)
    return time.perf_counter() - t0


def _oracle_bwd_item(item):
    """One work item of the backward baseline: the gradients of head (b, h)
    alone (its own K/V head, a seeded upstream gradient)."""
    import numpy as np
    from oracle import attention_bwd_ref
    b, h = item
    w, seg = _ORACLE["w"], _ORACLE["seg"]
    kh = h // (w.Hq // w.Hkv)
    do = np.random.default_rng(w.seed + 2 + b * w.Hq + h).standard_normal((1, 1, w.L, w.d_v))
    q, k, v = _ORACLE["q"], _ORACLE["k"], _ORACLE["v"]
    t0 = time.perf_counter()
    attention_bwd_ref(q[b:b + 1, h:h + 1], k[b:b + 1, kh:kh + 1], v[b:b + 1, kh:kh + 1], do,
                      scale=w.softmax_scale, soft_cap=w.soft_cap, causal=w.causal,
                      window_left=w.window_left, window_right=w.window_right, seg_q=seg,
                      q_offset=w.q_offset)
    return time.perf_counter() - t0


def cpu_baseline(w, q, k, v, seg, budget_s, backward=False, max_workers=16):
    """The float64 oracle as it stands, timed on the host: a process pool
    (one single-threaded BLAS per worker, as many workers as usable cores,
    at most ``max_workers``) over work items of the same workload - row
    panels of 512 rows of a (batch, head) for the forward, whole (batch,
    head) gradients for the backward.  One item is timed first to size the
    sample to about ``budget_s`` seconds of wall time; the sample is then
    timed with perf_counter around the pool (input generation excluded).
    Returns the baseline dict (None when one backward head would not fit in
    memory)."""
    import multiprocessing as mp
    import numpy as np
    nproc, model = host_cpu()
    workers = max(1, min(nproc, max_workers))
    if backward and w.L * w.keys * 8 * 12 > (4 << 30):
        return None
    _ORACLE.update(w=w, seg=seg, q=q.float().numpy(), k=k.float().numpy(), v=v.float().numpy())
    rows = pairs_per_row(w, seg)
    flop_pair = 2.0 * ((3 * w.d_qk + 2 * w.d_v) if backward else (w.d_qk + w.d_v))
    if backward:
        items = [(b, h) for b in range(w.B) for h in range(w.Hq)]
        item_flop = lambda it: flop_pair * float(rows.sum())
        fn = _oracle_bwd_item
    else:
        panel = 512
        # Every (batch, head) cut into row panels, in a fixed pseudo-random
        # order: the oracle's work per panel is the same (it scores all keys),
        # and a sample drawn this way carries the workload's mix of unmasked
        # pairs per panel.
        items = [(b, h, r0, min(r0 + panel, w.L)) for b in range(w.B) for h in range(w.Hq)
                 for r0 in range(0, w.L, panel)]
        items = [items[i] for i in np.random.default_rng(0).permutation(len(items))]
        item_flop = lambda it: flop_pair * float(rows[it[2]:it[3]].sum())
        fn = _oracle_fwd_item
    _limit_threads()
    t1 = fn(items[0])          # serial probe (warm caches, size the sample)
    n = int(min(len(items), max(workers, round(budget_s * workers / max(t1, 1e-3)))))
    n = max(1, (n // workers) * workers) if n >= workers else n
    sample = items[:n]
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_limit_threads) as pool:
        t0 = time.perf_counter()
        pool.map(fn, sample, chunksize=1)
        dt = time.perf_counter() - t0
    flop = sum(item_flop(it) for it in sample)
    _ORACLE.clear()
    what = (f"backward of {n} of {len(items)} (batch, head) pairs" if backward else
            f"{n} of {len(items)} work items (512-row panels of a (batch, head), against all "
            f"{w.keys} keys)")
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": workers,
            "kind": "oracle",
            "sample": f"{what}, float64 numpy, {workers} single-threaded worker processes, "
                      f"{dt:.1f} s wall; effective FLOPs = unmasked pairs x {int(flop_pair)}",
            "nproc": nproc, "cpu_model": model}


def median_min(xs):
    """(median, min) of a non-empty list."""
    srt = sorted(xs)
    return 0.5 * (srt[(len(srt) - 1) // 2] + srt[len(srt) // 2]), srt[0]


class ClockProbe:
    """Mean shader clock of the CUs over the timed steps: the library's clock
    probe (single-wave work-groups that record their CU's core-clock cycle
    counter, the constant-rate real-time counter and their location)
    enqueued on the launch stream just before and just after them.  The
    cycle counters of different CUs are not in step, so only a CU stamped by
    both probes gives a clock."""

    N = 256   # work-groups per probe (the dispatcher spreads them over the CUs)

    def __init__(self, dev, stream):
        import torch
        from block_sparse_flash_amd.api import clock_probe, realtime_khz
        self._probe = clock_probe
        self.buf = torch.zeros((2, 3 * self.N), dtype=torch.int64, device=dev)
        self.stream = stream
        self.khz = realtime_khz()

    def __call__(self, i):
        self._probe(self.buf[i], self.N, self.stream.cuda_stream)

    def per_cu_hz(self):
        """{location: mean clock in Hz} for the CUs stamped once by each probe."""
        b = self.buf.cpu().numpy().reshape(2, self.N, 3)
        out = {}
        for loc in set(int(x) for x in b[0, :, 2]) & set(int(x) for x in b[1, :, 2]):
            r0 = b[0][b[0, :, 2] == loc]
            r1 = b[1][b[1, :, 2] == loc]
            if len(r0) != 1 or len(r1) != 1:
                continue   # two work-groups on one CU: which came first is unknown
            dc, dr = int(r1[0, 0]) - int(r0[0, 0]), int(r1[0, 1]) - int(r0[0, 1])
            if dc > 0 and dr > 0:
                out[loc] = dc / (dr / (self.khz * 1e3))
        return out


def time_steps(step, stream, steps, warmup, probe=None):
    """Run ``warmup`` untimed steps, then ``steps`` timed ones with a HIP
    event pair around each call (on the launch stream) and one pair around
    all of them; ``probe`` (a ClockProbe) is enqueued just outside that
    pair.  Returns (total ms, per-call ms list, wall s)."""
    import torch
    for _ in range(warmup):
        step()
    if probe is not None:
        probe(0)   # first launch of the probe kernel outside the timed region
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    if probe is not None:
        probe(0)
    ev0.record(stream)
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    ev1.record(stream)
    if probe is not None:
        probe(1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return ev0.elapsed_time(ev1), [a.elapsed_time(b) for a, b in ev], wall


def time_cold(step, stream, dev, scratch_mib=512):
    """One call right after writing a scratch buffer of ``scratch_mib`` MiB
    (which evicts the inputs from the L2 and the last-level cache); ms."""
    import torch
    scratch = torch.empty(scratch_mib << 20, dtype=torch.uint8, device=dev)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    scratch.fill_(1)
    a.record(stream)
    step()
    b.record(stream)
    torch.cuda.synchronize()
    del scratch
    return a.elapsed_time(b)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # After the GPU idles, the first ~100 launches run slower while its
    # power management settles (dense causal L=4096: 305 us mean over the
    # first 50, 273 over the next 50, then 266-267 for 1500 more); the
    # default warm-up runs past that so the timed steps see the sustained rate.
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--mask-mode", default="computed", choices=["computed", "stored"])
    ap.add_argument("--max-logit", type=float, default=None,
                    help="Max Logit Estimate constant (logit units) in place of the running "
                         "row max; the default is the running max")
    ap.add_argument("--n-split", type=int, default=None,
                    help="split-KV: chunks per row merged through their lse (bf16; 1 = plain "
                         "forward); default: the workload's own (1 except for decoding)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (dq, dk, dv from o, lse and a random upstream "
                         "gradient) instead of the forward")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run one device-to-device copy of this many MiB "
                         "(a plain copy of known size, for scaling HBM counters)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds (wall) of oracle work for cpu_baseline (0: skip)")
    ap.add_argument("--no-sparsity", action="store_true",
                    help="skip the causal-only timing of masked workloads")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache call")
    ap.add_argument("--tile", default=None,
                    help="forward tile BQxBKV (one of fwd_tiles); default: the workload's tuned "
                         "tile, else the library's default")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_flash_amd import compile_mask, fwd_tile, splash_fwd
    from block_sparse_flash_amd.inputs import ALL_WORKLOADS, make_inputs

    w = ALL_WORKLOADS[args.workload]
    if args.n_split is None:
        args.n_split = w.n_split
    q, k, v, seg = make_inputs(w)
    if args.backward and (w.dtype != "bf16" or args.n_split != 1):
        raise SystemExit("--backward runs bf16 workloads without split-KV")
    # The oracle baseline runs first, before this process touches the GPU,
    # so that its worker processes fork from a process without a device.
    cpu = None
    if args.cpu_budget > 0:
        cpu = cpu_baseline(w, q, k, v, seg, args.cpu_budget, backward=args.backward)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    if args.tile:
        bq, bkv = (int(x) for x in args.tile.lower().split("x"))
    elif w.tile and not args.backward:
        bq, bkv = w.tile
    else:
        bq, bkv = fwd_tile(w.dtype, w.d_qk, w.d_v)
    mask_kw = dict(causal=w.causal, window_left=w.window_left, window_right=w.window_right)
    t0 = time.perf_counter()
    tabs = compile_mask(w.L, bq, bkv, L_kv=w.keys, seg_q=seg, q_offset=w.q_offset, **mask_kw)
    mask_ms = (time.perf_counter() - t0) * 1e3
    out = torch.empty((w.B, w.Hq, w.L, w.d_v), dtype=qd.dtype, device=dev)
    lse = torch.empty((w.B, w.Hq, w.L), dtype=torch.float32, device=dev)
    kw = dict(scale=w.softmax_scale, soft_cap=w.soft_cap, seg_q=seg, tables=tabs,
              mask_mode=args.mask_mode, out=out, lse=lse, max_logit=args.max_logit,
              q_offset=w.q_offset, **mask_kw)
    if args.n_split != 1:
        from block_sparse_flash_amd import split_workspace_bytes
        ws = torch.empty(split_workspace_bytes(args.n_split, w.B, w.Hq, w.L, w.d_v),
                         dtype=torch.uint8, device=dev)
        kw.update(n_split=args.n_split, workspace=ws)

    if args.backward:
        from block_sparse_flash_amd import bwd_tile, splash_bwd
        splash_fwd(qd, kd, vd, **kw)
        bq, bkv = bwd_tile(w.dtype, w.d_qk, w.d_v)
        tabs = compile_mask(w.L, bq, bkv, L_kv=w.keys, seg_q=seg, q_offset=w.q_offset, **mask_kw)
        g = torch.Generator().manual_seed(w.seed + 1)
        dod = torch.randn(out.shape, generator=g).to(torch.bfloat16).to(dev)
        bkw = dict(scale=w.softmax_scale, soft_cap=w.soft_cap, seg_q=seg, tables=tabs,
                   q_offset=w.q_offset, **mask_kw)
        step = lambda: splash_bwd(qd, kd, vd, out, lse, dod, **bkw)
    else:
        step = lambda: splash_fwd(qd, kd, vd, **kw)
    stream = torch.cuda.current_stream(dev)
    probe = ClockProbe(dev, stream)
    ms_total, per_call, wall = time_steps(step, stream, args.steps, args.warmup, probe)
    clock_hz = probe.per_cu_hz()
    ms_per_step = ms_total / args.steps
    ms_median, ms_min = median_min(per_call)
    ms_cold = None if args.no_cold else time_cold(step, stream, dev)

    pairs = unmasked_pairs(tabs, w, seg)
    # Algorithmic FLOP per unmasked pair: forward S = QK^T and PV; backward
    # S, dP = dO V^T, dV = P^T dO, dK = dS^T Q and dQ = dS K.
    flop_pair = 2.0 * (3 * w.d_qk + 2 * w.d_v) if args.backward else 2.0 * (w.d_qk + w.d_v)
    flop_per_step = flop_pair * pairs * w.B * w.Hq
    tflops = flop_per_step / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    traffic = None if args.backward else committed_traffic(w.name, w.dtype)
    decode = w.keys != w.L or w.q_offset != 0
    if decode and not args.backward:
        # Decoding: a few query rows against a long K/V cache; the forward
        # streams K and V once per K/V head and is bound by HBM.  Algorithmic
        # bytes: K and V of every K/V head, q and o of every query head, lse.
        elt = 2 if w.dtype == "bf16" else 4
        algo_bytes = (elt * (w.B * w.Hkv * w.keys * (w.d_qk + w.d_v) + w.B * w.Hq * w.L * (w.d_qk + w.d_v))
                      + 4 * w.B * w.Hq * w.L)
        gbs = algo_bytes / (ms_per_step * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                    "algorithmic_bytes": algo_bytes}
    else:
        roofline = {"bound": "mfma" if w.dtype == "bf16" else "alu",
                    "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(tflops / peak, 4), "traffic": traffic}

    # The shader clock over the timed steps (median over the CUs stamped by
    # both probes).  The matrix and vector peaks scale with it (the published
    # ones assume 2.4 GHz on 256 CUs); HBM bandwidth does not.
    clock = None
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    if len(clock_hz) >= n_cu // 4:
        ghz = sorted(clock_hz.values())
        f = 0.5 * (ghz[(len(ghz) - 1) // 2] + ghz[len(ghz) // 2])
        clock = {"ghz": round(f / 1e9, 3), "cu_p10_ghz": round(ghz[len(ghz) // 10] / 1e9, 3),
                 "cu_p90_ghz": round(ghz[(9 * len(ghz)) // 10] / 1e9, 3), "n_cu_stamped": len(ghz),
                 "n_cu": n_cu,
                 "method": "per-CU core-clock cycles over real time between two clock "
                           "probes enqueued around the timed steps"}
        if roofline["bound"] != "hbm":
            peak_clk = peak * (n_cu / 256.0) * (f / PEAK_CLOCK_HZ)
            roofline["peak_at_clock"] = round(peak_clk, 1)
            roofline["frac_at_clock"] = round(tflops / peak_clk, 4)

    # Skipped-block speedup against mask sparsity (Lecture 13 section 6.4):
    # the same shape and inputs under the causal mask alone.
    sparsity = None
    masked = w.window_left >= 0 or w.window_right >= 0 or w.segments
    if masked and w.causal and not decode and not args.no_sparsity and not args.backward:
        ctabs = compile_mask(w.L, bq, bkv, L_kv=w.keys, causal=True, q_offset=w.q_offset)
        ckw = dict(kw, tables=ctabs, seg_q=None, window_left=-1, window_right=-1)
        cstep = lambda: splash_fwd(qd, kd, vd, **ckw)
        c_steps = max(1, min(args.steps, 20))
        c_total, _, _ = time_steps(cstep, stream, c_steps, min(args.warmup, 3))
        c_ms = c_total / c_steps
        pairs_c = unmasked_pairs(None, w, seg, causal_only=True)
        sparsity = {"t_causal_ms": round(c_ms, 5), "t_masked_ms": round(ms_per_step, 5),
                    "speedup": round(c_ms / ms_per_step, 3),
                    "active_blocks_causal": ctabs.n_active, "active_blocks_masked": tabs.n_active,
                    "block_ratio": round(ctabs.n_active / max(1, tabs.n_active), 3),
                    "pair_ratio": round(pairs_c / max(1, pairs), 3),
                    "block": [bq, bkv], "causal_steps": c_steps}

    mask = "causal" if w.causal else "dense"
    if w.window_left >= 0 or w.window_right >= 0:
        mask += f"+window({w.window_left},{w.window_right})"
    if w.segments:
        mask += f"+segments U[{w.seg_min},{w.seg_max}]"
    rec = {
        "metric": ("effective attention backward TFLOP/s (unmasked FLOPs) and % of bf16 MFMA peak"
                   if args.backward else
                   "effective attention TFLOP/s (unmasked FLOPs) and % of bf16 MFMA peak"),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_median": round(ms_median, 5),
        "ms_min": round(ms_min, 5),
        "ms_cold": None if ms_cold is None else round(ms_cold, 5),
        "value_median": round(flop_per_step / (ms_median * 1e-3) / 1e12, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "L": w.L,
                   "L_kv": w.keys, "q_offset": w.q_offset,
                   "d_qk": w.d_qk, "d_v": w.d_v, "mask": mask, "soft_cap": w.soft_cap,
                   "scale": w.softmax_scale, "block_q": bq, "block_kv": bkv,
                   "mask_mode": args.mask_mode, "max_logit": args.max_logit,
                   "n_split": args.n_split, "pass": "backward" if args.backward else "forward",
                   "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "pct_of_peak_at_clock": roofline.get("frac_at_clock") and round(100.0 * roofline["frac_at_clock"], 2),
        "clock": clock,
        "unmasked_tflop_per_step": flop_per_step / 1e12,
        "active_blocks": tabs.n_active, "partial_blocks": tabs.n_partial,
        "mask_compile_ms": round(mask_ms, 3),
        "wall_s_timed_region": round(wall, 4),
        "timing": "HIP events on the launch stream around each call and around all "
                  "calls; inputs resident, no cache flush (ms_cold: one call after "
                  "writing 512 MiB of scratch)",
        "roofline": roofline,
        "sparsity": sparsity,
        "cpu_baseline": cpu,
    }
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20)
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_calibration_bytes"] = n
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
