"""GPU parity at the long end of the context range: a request of 131 074
tokens (past 2^16 and 2^17 keys per row, where 16- or 17-bit index and offset
arithmetic would wrap), beside short ones.

* 128 heads, two shards: about 65 500 keys per row and shard, so the dispatch
  splits the long rows into fixed-size pieces merged by the combine kernel.
* 16 heads, one shard: the balanced schedule cuts the long row into pieces
  held by most of the workers (more than eight pieces per row, so the split
  combine's loop over pieces runs more than once), bf16 and FP8 caches.

Every row against the oracle's partial, and the merged rows against the
oracle's unsharded attention.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from mla_decode_context_amd import workloads as WL
from mla_decode_context_amd.runner import DeviceWorkload
from oracle import mla_oracle as O
from tests._gpu import check_rows, log, needs_gpu, oracle_valid

pytestmark = [pytest.mark.gpu, needs_gpu]

LONG = 131074


def _oracle(wl, toks, kv, unsharded=False):
    def gkv(b):
        if b not in kv:
            kv[b] = wl.global_kv(b)
        return kv[b]

    if unsharded:
        return O.decode_partial(wl.seq_lens, wl.query_start_loc, wl.q_nope, wl.q_pe, gkv, wl.scale, 1, 0,
                                tokens=toks, kv_scale=wl.kv_scale)
    parts = [O.decode_partial(wl.seq_lens, wl.query_start_loc, wl.q_nope, wl.q_pe, gkv, wl.scale, wl.W, r,
                              tokens=toks, I=wl.I, kv_scale=wl.kv_scale) for r in range(wl.W)]
    return np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts])


@pytest.mark.parametrize("name,S,Q,H,W,P,fp8", [
    ("h128_w2_131k", [LONG, 300], [2, 1], 128, 2, 64, False),
    ("h16_w1_131k", [LONG, 40, 5000], [1, 1, 1], 16, 1, 16, False),
    ("h16_w1_131k_fp8", [LONG, 40, 5000], [1, 1, 1], 16, 1, 16, True),
])
def test_long_context_rows(name, S, Q, H, W, P, fp8):
    log(f"[{name}] generating inputs")
    wl = WL.make_custom(name, S, Q, H=H, W=W, P=P, seed=97, kv_scale=WL.FP8_SCALE if fp8 else None)
    dw = DeviceWorkload(wl)
    log(f"[{name}] T={wl.T}; running")
    dw.outs.fill_(float("nan"))
    dw.step()
    torch.cuda.synchronize()
    toks = list(range(wl.T))
    kv = {}
    log(f"[{name}] oracle")
    ref_o, ref_l = _oracle(wl, toks, kv)
    for r in range(W):
        st = check_rows(dw.outs[r], dw.lses[r], ref_o[r], ref_l[r], f"{name} r={r}")
        log(f"[{name}] rank {r}: {st}")
    assert np.array_equal(dw.valid.cpu().numpy(), oracle_valid(wl, toks))
    if W > 1:
        full_o, full_l = _oracle(wl, toks, kv, unsharded=True)
        st = check_rows(dw.out, dw.out_lse, full_o, full_l, f"{name} merged")
        log(f"[{name}] merged vs unsharded: {st}")
