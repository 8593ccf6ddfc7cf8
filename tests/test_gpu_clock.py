"""GPU test of the clock probe (measurement only): stamps carry their CU's
location, and two probes around a run of forwards give every CU stamped by
both a clock in the chip's range."""

import numpy as np
import pytest
import torch

from block_sparse_flash_amd import api
from block_sparse_flash_amd.inputs import ALL_WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

N = 256


def test_clock_probe_gives_a_plausible_clock_per_cu():
    dev = torch.device("cuda:0")
    w = ALL_WORKLOADS["causal_mha_bf16_L4096_d128"]
    q, k, v, _ = make_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    bq, bkv = api.fwd_tile(w.dtype, w.d_qk, w.d_v)
    kw = dict(scale=w.softmax_scale, causal=True,
              tables=api.compile_mask(w.L, bq, bkv, causal=True))   # no host work per call
    o, lse = api.splash_fwd(qd, kd, vd, **kw)
    buf = torch.zeros((2, 3 * N), dtype=torch.int64, device=dev)
    for _ in range(100):   # past the clock's settling after idle
        api.splash_fwd(qd, kd, vd, out=o, lse=lse, **kw)
    api.clock_probe(buf[0], N)
    for _ in range(50):
        api.splash_fwd(qd, kd, vd, out=o, lse=lse, **kw)
    api.clock_probe(buf[1], N)
    torch.cuda.synchronize()
    b = buf.cpu().numpy().reshape(2, N, 3)
    xcd = b[:, :, 2] >> 16
    assert xcd.min() >= 0 and xcd.max() <= 7
    khz = api.realtime_khz()
    assert khz > 0
    ghz = []
    for loc in set(b[0, :, 2].tolist()) & set(b[1, :, 2].tolist()):
        r0, r1 = b[0][b[0, :, 2] == loc], b[1][b[1, :, 2] == loc]
        if len(r0) == 1 and len(r1) == 1:
            dc, dr = int(r1[0, 0] - r0[0, 0]), int(r1[0, 1] - r0[0, 1])
            assert dc > 0 and dr > 0
            ghz.append(dc / (dr / (khz * 1e3)) / 1e9)
    print(f"{len(ghz)} CUs stamped twice; GHz min {min(ghz):.3f} median {np.median(ghz):.3f} max {max(ghz):.3f}")
    assert len(ghz) >= N // 4
    assert all(0.3 < g < 3.0 for g in ghz), sorted(ghz)


def test_clock_probe_rejects_bad_arguments():
    dev = torch.device("cuda:0")
    buf = torch.zeros(24, dtype=torch.int64, device=dev)
    with pytest.raises(ValueError):
        api.clock_probe(buf, 9)            # needs 27 elements
    with pytest.raises(ValueError):
        api.clock_probe(buf.to(torch.int32), 8)
