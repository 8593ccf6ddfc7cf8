"""GPU parity of the backward (``splash_attn_bwd`` through the C ABI) against
the float64 oracle gradients ``attention_bwd_ref``.

Inputs are the stored bf16 q, k, v and upstream gradient; o and lse come from
this library's forward, as a training step would use them.  Tolerance: the
max-abs error of each gradient tensor at most TOL times that tensor's
max-abs reference value.  The kernels round p and dS to bf16 (8 significant
bits, relative error up to 2^-9) as MFMA operands and take D = do . o from
the bf16 forward output, so each product term carries a relative error of a
few 2^-9; TOL = 2^-5 leaves a factor of about 5 over that for the sums.
"""

import math
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_sparse_flash_amd import compile_mask, fwd_tile, splash_bwd, splash_fwd
from block_sparse_flash_amd.inputs import as_f64, draw_qkv, segment_ids, stored
from oracle import attention_bwd_ref

pytestmark = pytest.mark.gpu

TOL = 2.0 ** -5


def _announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _check(name, got, ref):
    got = got.detach().float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite gradient"
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert err <= TOL * scale + 1e-6, f"{name}: max-abs error {err:.3g} > {TOL} x {scale:.3g}"
    return err / scale if scale > 0 else 0.0


def _run_case(B, Hq, Hkv, Lq, Lkv, d, mk, cap, seed, q_offset=0, seg_q=None, seg_kv=None):
    """d: the head dim of q, k and v, or a pair (d_qk, d_v)."""
    d_qk, d_v = (d, d) if isinstance(d, int) else d
    q, k, v = (stored(a, "bf16") for a in draw_qkv(B, Hq, Hkv, Lq, d_qk, d_v, seed,
                                                   qk_std=1.5 if cap else 1.0, L_kv=Lkv))
    rng = np.random.default_rng(seed + 99)
    do = stored(rng.standard_normal((B, Hq, Lq, d_v), dtype=np.float32), "bf16")
    scale = 1.0 / math.sqrt(d_qk)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = splash_fwd(qd, kd, vd, scale=scale, soft_cap=cap, seg_q=seg_q, seg_kv=seg_kv,
                        q_offset=q_offset, **mk)
    dq, dk, dv = splash_bwd(qd, kd, vd, o, lse, dod, scale=scale, soft_cap=cap, seg_q=seg_q,
                            seg_kv=seg_kv, q_offset=q_offset, **mk)
    torch.cuda.synchronize()
    rdq, rdk, rdv = attention_bwd_ref(as_f64(q), as_f64(k), as_f64(v), as_f64(do), scale=scale,
                                      soft_cap=cap, seg_q=seg_q, seg_kv=seg_kv,
                                      q_offset=q_offset, **mk)
    e = (_check("dq", dq, rdq), _check("dk", dk, rdk), _check("dv", dv, rdv))
    _announce(f"  relative max-abs errors dq {e[0]:.3g} dk {e[1]:.3g} dv {e[2]:.3g}")


CASES = [
    # (B, Hq, Hkv, L, d, mask kwargs, soft_cap, segments (lo, hi) or None)
    (1, 2, 2, 256, 128, dict(causal=True), 0.0, None),
    (2, 4, 2, 700, 128, dict(causal=True, window_left=200), 0.0, None),
    (1, 4, 1, 600, 64, dict(causal=True), 20.0, (40, 250)),
    (1, 2, 2, 333, 128, dict(), 0.0, None),
    (1, 2, 1, 300, 64, dict(window_left=70, window_right=33), 3.0, None),
    (1, 8, 2, 2048, 128, dict(causal=True), 0.0, None),
    # d = 128 with documents and the cap (the build of the documents workload)
    (1, 4, 1, 900, 128, dict(causal=True), 50.0, (40, 300)),
    (1, 4, 2, 640, 128, dict(causal=True, window_left=150), 20.0, (30, 200)),
    # 192-wide q/k heads with 128-wide v
    (1, 4, 2, 700, (192, 128), dict(causal=True), 0.0, None),
    (2, 2, 1, 333, (192, 128), dict(), 0.0, None),
    (1, 4, 1, 900, (192, 128), dict(causal=True), 50.0, (40, 300)),
    (1, 2, 2, 600, (192, 128), dict(causal=True, window_left=120, window_right=7), 0.0, None),
]


def _dims(d):
    return f"d{d}" if isinstance(d, int) else f"d{d[0]}x{d[1]}"


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}-L{c[3]}-{_dims(c[4])}"
                         + ("-cap" if c[6] else "") + ("-seg" if c[7] else "") + "-"
                         + "-".join(sorted(c[5])))
def test_backward_every_element(case):
    B, Hq, Hkv, L, d, mk, cap, segs = case
    _announce(f"backward {case}")
    seg = None if segs is None else segment_ids(L, 500 + L, *segs)
    _run_case(B, Hq, Hkv, L, L, d, mk, cap, 500 + L + (d if isinstance(d, int) else sum(d)), seg_q=seg)


def test_backward_decode_positions_and_empty_rows():
    """Query rows at key positions q_offset + i, with L_q != L_kv; in the
    second case rows past position 949 see no key (zero gradients)."""
    _announce("backward decode Lq=40 Lkv=900 off=860")
    _run_case(1, 4, 2, 40, 900, 128, dict(causal=True), 0.0, 61, q_offset=860)
    _announce("backward rows without keys Lq=64 Lkv=700 off=900")
    _run_case(1, 2, 2, 64, 700, 64, dict(causal=True, window_left=250), 0.0, 62, q_offset=900)
    _announce("backward decode d192x128 Lq=100 Lkv=800 off=700")
    _run_case(1, 4, 1, 100, 800, (192, 128), dict(causal=True), 0.0, 63, q_offset=700)


def test_backward_per_batch_segments():
    """Different document boundaries per batch element (the binding runs one
    table per batch element)."""
    _announce("backward per-batch segments")
    L = 500
    seg = np.stack([segment_ids(L, 71, 30, 200), segment_ids(L, 72, 50, 300)])
    _run_case(2, 2, 1, L, L, 64, dict(causal=True), 0.0, 73, seg_q=seg)


def test_backward_deterministic():
    """No atomics: two calls give bit-identical gradients."""
    q, k, v = (stored(a, "bf16").cuda() for a in draw_qkv(1, 4, 2, 900, 128, 128, 81))
    do = torch.randn(1, 4, 900, 128, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).cuda()
    o, lse = splash_fwd(q, k, v, causal=True)
    g1 = splash_bwd(q, k, v, o, lse, do, causal=True)
    g2 = splash_bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_backward_item_order_changes_nothing():
    """The kernels' item orders (longest q blocks and kv columns first, from
    the tables) against table order (NULL orders through the C ABI): a
    schedule only, so the gradients are bit-identical.  GQA with documents,
    16 query heads (two per XCD, interleaved by the dq kernel) and uneven
    columns."""
    _announce("backward item order")
    L = 1500
    seg = segment_ids(L, 91, 40, 600)
    q, k, v = (stored(a, "bf16").cuda() for a in draw_qkv(2, 8, 2, L, 128, 128, 92))
    do = torch.randn(2, 8, L, 128, generator=torch.Generator().manual_seed(93)).to(torch.bfloat16).cuda()
    mk = dict(causal=True, seg_q=seg)
    o, lse = splash_fwd(q, k, v, **mk)
    g1 = splash_bwd(q, k, v, o, lse, do, **mk)
    g2 = splash_bwd(q, k, v, o, lse, do, natural_order=True, **mk)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_backward_full_size_sampled_heads():
    """The bench's backward workload (dense causal L=4096, B=2, Hq=Hkv=32,
    d=128) at full size: every gradient element of three heads against the
    oracle (with Hq = Hkv a head's dq, dk and dv depend on that head only)."""
    from block_sparse_flash_amd.inputs import ALL_WORKLOADS, make_inputs
    w = ALL_WORKLOADS["causal_mha_bf16_L4096_d128"]
    _announce(f"backward full size {w.name}")
    q, k, v, _ = make_inputs(w)
    g = torch.Generator().manual_seed(w.seed + 1)
    do = torch.randn((w.B, w.Hq, w.L, w.d_v), generator=g).to(torch.bfloat16)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = splash_fwd(qd, kd, vd, causal=True)
    dq, dk, dv = splash_bwd(qd, kd, vd, o, lse, dod, causal=True)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (1, 17), (1, 31)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        rdq, rdk, rdv = attention_bwd_ref(as_f64(q[sl]), as_f64(k[sl]), as_f64(v[sl]), as_f64(do[sl]),
                                          scale=w.softmax_scale, causal=True)
        e = (_check("dq", dq[sl], rdq), _check("dk", dk[sl], rdk), _check("dv", dv[sl], rdv))
        _announce(f"  head ({b}, {h}): relative max-abs errors dq {e[0]:.3g} dk {e[1]:.3g} dv {e[2]:.3g}")
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())


def test_backward_documents_workload_whole_documents():
    """The documents workload (GQA 16/4, L = 32768, causal AND segment ids,
    cap 50) at full size.  Under the segment mask a document's keys are
    reached only by its own rows, so every gradient element of a document
    equals the backward of that document alone with a causal mask: checked
    for two documents (the shortest one and the one holding row L/2) on the
    query heads of two K/V heads."""
    from block_sparse_flash_amd.inputs import ALL_WORKLOADS, make_inputs
    w = ALL_WORKLOADS["gqa_docs_cap_bf16_L32768"]
    _announce(f"backward full size {w.name}")
    q, k, v, seg = make_inputs(w)
    g = torch.Generator().manual_seed(w.seed + 1)
    do = torch.randn((w.B, w.Hq, w.L, w.d_v), generator=g).to(torch.bfloat16)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    mk = dict(causal=True, soft_cap=w.soft_cap, scale=w.softmax_scale, seg_q=seg)
    o, lse = splash_fwd(qd, kd, vd, **mk)
    dq, dk, dv = splash_bwd(qd, kd, vd, o, lse, dod, **mk)
    torch.cuda.synchronize()
    seg = np.asarray(seg)
    starts = np.concatenate([[0], np.flatnonzero(np.diff(seg) != 0) + 1])
    ends = np.concatenate([starts[1:], [w.L]])
    lens = ends - starts
    docs = sorted({int(np.argmin(lens)), int(seg[w.L // 2] - seg[0])})
    group = w.Hq // w.Hkv
    for di in docs:
        s0, s1 = int(starts[di]), int(ends[di])
        for kh in (0, w.Hkv - 1):
            hs = slice(kh * group, (kh + 1) * group)
            sub = lambda t, hsl: as_f64(t[:, hsl, s0:s1])
            rdq, rdk, rdv = attention_bwd_ref(sub(q, hs), sub(k, slice(kh, kh + 1)),
                                              sub(v, slice(kh, kh + 1)), sub(do, hs),
                                              scale=w.softmax_scale, soft_cap=w.soft_cap,
                                              causal=True)
            e = (_check("dq", dq[:, hs, s0:s1], rdq), _check("dk", dk[:, kh:kh + 1, s0:s1], rdk),
                 _check("dv", dv[:, kh:kh + 1, s0:s1], rdv))
            _announce(f"  document {di} rows [{s0}, {s1}) K/V head {kh}: relative max-abs errors "
                      f"dq {e[0]:.3g} dk {e[1]:.3g} dv {e[2]:.3g}")
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())


def test_backward_wide_head_full_size_sampled_heads():
    """The 192/128 dense causal workload (L=4096, B=1, Hq=Hkv=128) at full
    size: every gradient element of two heads against the oracle."""
    from block_sparse_flash_amd.inputs import ALL_WORKLOADS, make_inputs
    w = ALL_WORKLOADS["causal_mha_bf16_L4096_d192"]
    _announce(f"backward full size {w.name}")
    q, k, v, _ = make_inputs(w)
    g = torch.Generator().manual_seed(w.seed + 1)
    do = torch.randn((w.B, w.Hq, w.L, w.d_v), generator=g).to(torch.bfloat16)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = splash_fwd(qd, kd, vd, causal=True)
    dq, dk, dv = splash_bwd(qd, kd, vd, o, lse, dod, causal=True)
    torch.cuda.synchronize()
    assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape
    for b, h in [(0, 5), (0, 127)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        rdq, rdk, rdv = attention_bwd_ref(as_f64(q[sl]), as_f64(k[sl]), as_f64(v[sl]), as_f64(do[sl]),
                                          scale=w.softmax_scale, causal=True)
        e = (_check("dq", dq[sl], rdq), _check("dk", dk[sl], rdk), _check("dv", dv[sl], rdv))
        _announce(f"  head ({b}, {h}): relative max-abs errors dq {e[0]:.3g} dk {e[1]:.3g} dv {e[2]:.3g}")
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())
