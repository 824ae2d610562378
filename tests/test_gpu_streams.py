"""Two independent decode steps (their own inputs, outputs and workspaces) on
two streams at once give the same bits as run one after the other: the
library keeps no state outside the buffers a call is given."""
from __future__ import annotations

import pytest
import torch

from mla_decode_context_amd import workloads as WL
from mla_decode_context_amd.runner import DeviceWorkload
from tests._gpu import log, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.mark.parametrize("H", [16, 128])
def test_two_streams_match_sequential(H):
    log(f"two streams H={H}")
    a = DeviceWorkload(WL.make_custom(f"streams_a_{H}", [700, 90, 2, 1500], [2, 1, 2, 4], H=H, W=2, P=64, seed=121))
    b = DeviceWorkload(WL.make_custom(f"streams_b_{H}", [300, 2, 1, 900, 65], [2, 1, 1, 3, 4], H=H, W=4, P=16,
                                      seed=122))
    a.step()
    b.step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (a.outs, a.out, b.outs, b.out)]
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()       # default priority
    for _ in range(5):
        for t in (a.outs, a.out, b.outs, b.out):
            t.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(sa):
            a.step()
        with torch.cuda.stream(sb):
            b.step()
        torch.cuda.synchronize()
        for t, r in zip((a.outs, a.out, b.outs, b.out), ref):
            assert torch.equal(t, r)
