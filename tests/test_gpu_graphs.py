"""HIP-graph capture of the paths the other graph tests do not cover: the FP8
cache, fp32 partials, the two-stage step and the allocation-free entry point.

Each step is captured once and replayed three times, with the program's own
eager work (zeroing the outputs) and a synchronisation between replays; every
replay must equal the eager run bit for bit.
"""
from __future__ import annotations

import pytest
import torch

from mla_decode_context_amd import binding as mla
from mla_decode_context_amd import workloads as WL
from mla_decode_context_amd.runner import DeviceWorkload
from tests._gpu import log, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]

S = [300, 2, 1, 700, 65]
Q = [2, 1, 1, 3, 4]


def _replay_matches(run, outputs):
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(3):
        for t in outputs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (t, r) in enumerate(zip(outputs, ref)):
            assert torch.equal(t, r), f"replay {i}: output {k} differs from the eager run"


@pytest.mark.parametrize("name,H,W,P,fp8,f32,splits", [
    ("fp8_h16_balanced", 16, 4, 16, True, False, 0),
    ("fp8_h16_fixed_splits", 16, 2, 64, True, False, 3),
    ("f32_h16_balanced", 16, 4, 16, False, True, 0),
    ("f32_h128_ordered", 128, 2, 64, False, True, 0),
    ("f32_h128_split", 128, 2, 64, False, True, 4),
    ("h64_ordered", 64, 2, 64, False, False, 0),
])
def test_graph_replay_step(name, H, W, P, fp8, f32, splits):
    log(f"graph {name}")
    wl = WL.make_custom(name, S, Q, H=H, W=W, P=P, seed=111, kv_scale=WL.FP8_SCALE if fp8 else None)
    dw = DeviceWorkload(wl, num_splits=splits, partial_dtype=torch.float32 if f32 else None)
    _replay_matches(dw.step, [dw.outs, dw.lses, dw.valid, dw.out, dw.out_lse])


@pytest.mark.parametrize("H", [16, 128])
def test_graph_replay_two_stage(H):
    log(f"graph two-stage H={H}")
    wl = WL.make_custom(f"graph_two_{H}", S, Q, H=H, W=2, P=16, seed=112)
    dw = DeviceWorkload(wl)
    dw.setup_two_stage()
    _replay_matches(dw.two_stage_step, [dw.outs2, dw.lses2, dw.valid2, dw.out, dw.out_lse])


@pytest.mark.parametrize("H", [16, 128])
def test_graph_replay_noalloc(H):
    log(f"graph noalloc H={H}")
    wl = WL.make_custom(f"graph_noalloc_{H}", S, Q, H=H, W=2, P=16, seed=113)
    dw = DeviceWorkload(wl)

    def run():
        for r in range(wl.W):
            mla.mla_decode_partial_noalloc(dw.q_nope, dw.q_pe, dw.caches[r], dw.tables[r], dw.seq_lens, dw.qsl,
                                           wl.W, r, dw.scale, dw.outs[r], dw.lses[r],
                                           max_query_len=dw.max_query_len, max_seq_len=dw.max_seq_len,
                                           row_keys=dw.valid[r])
        dw.merge()

    _replay_matches(run, [dw.outs, dw.lses, dw.valid, dw.out, dw.out_lse])
