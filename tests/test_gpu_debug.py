"""MLA_DEBUG=1: mla_decode_partial checks its device-side contract on host
copies before launching anything.

Only violations that are harmless if a kernel did run are used on the GPU
(upper bounds that are too small); the block-id checks are covered on the CPU
through mla_check_decode_metadata, since a bad block id that slipped through
would make a kernel read outside the cache.
"""
from __future__ import annotations

import pytest
import torch

from mla_decode_context_amd import binding as mla
from mla_decode_context_amd import workloads as WL
from mla_decode_context_amd.runner import DeviceWorkload
from tests._gpu import log, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]


def _call(dw, r, out, lse, **kw):
    args = dict(max_query_len=dw.max_query_len, max_seq_len=dw.max_seq_len, workspace=dw.workspace,
                cp_interleave=dw.I)
    args.update(kw)
    mla.mla_decode_partial(dw.q_nope, dw.q_pe, dw.caches[r], dw.tables[r], dw.seq_lens, dw.qsl, dw.W, r,
                           dw.scale, out, lse, **args)


@pytest.mark.parametrize("H", [16, 128])
def test_debug_mode_valid_call_matches(monkeypatch, H):
    log(f"MLA_DEBUG valid call H={H}")
    wl = WL.make_custom("dbg", [40, 300, 7], [2, 1, 3], H=H, W=2, P=16, seed=3)
    dw = DeviceWorkload(wl)
    dw.partial(1)
    torch.cuda.synchronize()
    ref_o, ref_l = dw.outs[1].clone(), dw.lses[1].clone()
    monkeypatch.setenv("MLA_DEBUG", "1")
    out = torch.full_like(ref_o, float("nan"))
    lse = torch.full_like(ref_l, float("nan"))
    _call(dw, 1, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)


@pytest.mark.parametrize("bad", [dict(max_query_len=2), dict(max_seq_len=299)])
def test_debug_mode_rejects_before_launch(monkeypatch, bad):
    log(f"MLA_DEBUG rejects {bad}")
    wl = WL.make_custom("dbg", [40, 300, 7], [2, 1, 3], H=16, W=2, P=16, seed=3)
    dw = DeviceWorkload(wl)
    out = torch.full_like(dw.outs[0], 7.0)
    lse = torch.full_like(dw.lses[0], 7.0)
    monkeypatch.setenv("MLA_DEBUG", "1")
    with pytest.raises(mla.MlaError, match="MLA_ERR_SHAPE"):
        _call(dw, 0, out, lse, **bad)
    torch.cuda.synchronize()
    # nothing was enqueued: the outputs keep their fill
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)
    # without MLA_DEBUG the same call is not checked (these bounds only size the grid)
    monkeypatch.delenv("MLA_DEBUG")
    _call(dw, 0, out, lse, **bad)
    torch.cuda.synchronize()
    assert not torch.all(out == 7.0)


def test_debug_mode_refuses_capture(monkeypatch):
    log("MLA_DEBUG during capture")
    wl = WL.make_custom("dbg", [40, 30], [2, 1], H=16, W=1, P=16, seed=4)
    dw = DeviceWorkload(wl)
    dw.partial(0)
    torch.cuda.synchronize()
    monkeypatch.setenv("MLA_DEBUG", "1")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.graph(g, stream=s):
        try:
            _call(dw, 0, dw.outs[0], dw.lses[0])
        except mla.MlaError as e:
            err = str(e)
        dw.outs.add_(0)       # the captured graph holds one ordinary node
    assert err is not None and "MLA_ERR_CAPTURE" in err, err
