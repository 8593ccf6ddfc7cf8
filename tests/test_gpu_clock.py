"""GPU test of the clock probe (measurement only): every XCD is stamped
once per probe, and two probes around a run of forwards give a clock in the
chip's range."""

import numpy as np
import pytest
import torch

from block_sparse_flash_amd import api
from block_sparse_flash_amd.inputs import ALL_WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def test_clock_probe_stamps_every_xcd_and_gives_a_plausible_clock():
    dev = torch.device("cuda:0")
    w = ALL_WORKLOADS["causal_mha_bf16_L4096_d128"]
    q, k, v, _ = make_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = api.splash_fwd(qd, kd, vd, scale=w.softmax_scale, causal=True)
    buf = torch.zeros((2, 24), dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    api.clock_probe(buf[0], 8)
    for _ in range(20):
        api.splash_fwd(qd, kd, vd, scale=w.softmax_scale, causal=True, out=o, lse=lse)
    api.clock_probe(buf[1], 8)
    torch.cuda.synchronize()
    b = buf.cpu().numpy().reshape(2, 8, 3)
    for p in range(2):
        assert sorted(int(x) for x in b[p, :, 2]) == list(range(8))
    khz = api.realtime_khz()
    assert khz > 0
    pre = {int(r[2]): r for r in b[0]}
    ghz = []
    for r1 in b[1]:
        r0 = pre[int(r1[2])]
        dc, dr = int(r1[0] - r0[0]), int(r1[1] - r0[1])
        assert dc > 0 and dr > 0
        ghz.append(dc / (dr / (khz * 1e3)) / 1e9)
    print("per-XCD GHz", np.round(ghz, 3), "real-time counter kHz", khz)
    assert all(0.3 < g < 3.0 for g in ghz), ghz


def test_clock_probe_rejects_bad_arguments():
    dev = torch.device("cuda:0")
    buf = torch.zeros(24, dtype=torch.int64, device=dev)
    with pytest.raises(ValueError):
        api.clock_probe(buf, 9)            # needs 27 elements
    with pytest.raises(ValueError):
        api.clock_probe(buf.to(torch.int32), 8)
