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
KERNEL_SOURCES = {"bf16": "splash_fwd_bf16.hip", "f32": "splash_fwd_f32.hip"}


def unmasked_pairs(tabs, w, seg):
    """Exact count of allowed (query, key) pairs per (b, h), from the mask
    definition, summed row by row with interval arithmetic (segments: the
    allowed keys of a row are the part of its interval inside its segment,
    segments being contiguous here)."""
    import numpy as np
    L = w.L
    i = w.q_offset + np.arange(L, dtype=np.int64)   # key positions of the query rows
    lo = np.zeros(L, np.int64)
    hi = np.full(L, w.keys - 1, np.int64)
    if w.causal:
        hi = np.minimum(hi, i)
    if w.window_left >= 0:
        lo = np.maximum(lo, i - w.window_left)
    if w.window_right >= 0:
        hi = np.minimum(hi, i + w.window_right)
    if seg is not None:
        seg = np.asarray(seg)
        assert np.all(np.diff(seg) >= 0), "pair count assumes contiguous segments"
        starts = np.searchsorted(seg, seg, side="left")
        ends = np.searchsorted(seg, seg, side="right") - 1
        lo = np.maximum(lo, starts)
        hi = np.minimum(hi, ends)
    return int(np.maximum(hi - lo + 1, 0).sum())


def kernel_sha(dtype):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_flash_amd", "csrc")
    for name in (KERNEL_SOURCES[dtype], "fwd_params.h"):
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


def cpu_baseline(w, q, k, v, seg, budget_s):
    """The float64 oracle on the host over whole (batch, head) pairs, in
    order, adding heads until about budget_s of work or the whole workload;
    returns the baseline dict."""
    from oracle import attention_ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    qf, kf, vf = q.float().numpy(), k.float().numpy(), v.float().numpy()
    pairs = unmasked_pairs(None, w, seg)
    done = 0
    t0 = time.perf_counter()
    while done < w.B * w.Hq and (time.perf_counter() - t0) < budget_s:
        b, h = divmod(done, w.Hq)
        attention_ref(qf, kf, vf, scale=w.softmax_scale, soft_cap=w.soft_cap,
                      causal=w.causal, window_left=w.window_left,
                      window_right=w.window_right, seg_q=seg, heads=[(b, h)],
                      q_offset=w.q_offset)
        done += 1
    dt = time.perf_counter() - t0
    flop = 2.0 * (w.d_qk + w.d_v) * pairs * done
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {w.B * w.Hq} (batch, head) pairs in order, all {w.L} "
                      f"rows each (against {w.keys} keys), float64 numpy, {dt:.1f} s"}


def cpu_baseline_bwd(w, q, k, v, seg, budget_s):
    """The float64 backward oracle on the host over whole (batch, head) pairs
    in order (each with its own K/V head and a seeded upstream gradient),
    adding heads until about budget_s of work; returns the baseline dict."""
    import numpy as np
    from oracle import attention_bwd_ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    qf, kf, vf = q.float().numpy(), k.float().numpy(), v.float().numpy()
    group = w.Hq // w.Hkv
    rng = np.random.default_rng(w.seed + 2)
    pairs = unmasked_pairs(None, w, seg)
    done = 0
    t0 = time.perf_counter()
    while done < w.B * w.Hq and (time.perf_counter() - t0) < budget_s:
        b, h = divmod(done, w.Hq)
        kh = h // group
        do = rng.standard_normal((1, 1, w.L, w.d_v))
        attention_bwd_ref(qf[b:b + 1, h:h + 1], kf[b:b + 1, kh:kh + 1], vf[b:b + 1, kh:kh + 1], do,
                          scale=w.softmax_scale, soft_cap=w.soft_cap, causal=w.causal,
                          window_left=w.window_left, window_right=w.window_right, seg_q=seg,
                          q_offset=w.q_offset)
        done += 1
    dt = time.perf_counter() - t0
    flop = 2.0 * (3 * w.d_qk + 2 * w.d_v) * pairs * done
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"backward of {done} of {w.B * w.Hq} (batch, head) pairs in order, all "
                      f"{w.L} rows each, float64 numpy, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
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
                    help="seconds of oracle work for cpu_baseline (0: skip)")
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
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    q, k, v, seg = make_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
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
        from block_sparse_flash_amd import splash_bwd
        if w.dtype != "bf16" or args.n_split != 1:
            raise SystemExit("--backward runs bf16 workloads without split-KV")
        splash_fwd(qd, kd, vd, **kw)
        g = torch.Generator().manual_seed(w.seed + 1)
        dod = torch.randn(out.shape, generator=g).to(torch.bfloat16).to(dev)
        bkw = dict(scale=w.softmax_scale, soft_cap=w.soft_cap, seg_q=seg, tables=tabs,
                   q_offset=w.q_offset, **mask_kw)
        step = lambda: splash_bwd(qd, kd, vd, out, lse, dod, **bkw)
    else:
        step = lambda: splash_fwd(qd, kd, vd, **kw)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_events = ev0.elapsed_time(ev1)
    ms_per_step = ms_events / args.steps

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

    cpu = None
    if args.cpu_budget > 0:
        cpu = (cpu_baseline_bwd if args.backward else cpu_baseline)(w, q, k, v, seg, args.cpu_budget)

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
        "unmasked_tflop_per_step": flop_per_step / 1e12,
        "active_blocks": tabs.n_active, "partial_blocks": tabs.n_partial,
        "mask_compile_ms": round(mask_ms, 3),
        "wall_s_timed_region": round(wall, 4),
        "roofline": roofline,
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
