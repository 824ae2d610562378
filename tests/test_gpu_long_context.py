"""GPU parity at the size extremes.

A request of 131 074 tokens (past 2^16 and 2^17 keys per row, where 16- or
17-bit index and offset arithmetic would wrap), beside short ones:

* 128 heads, two shards: about 65 500 keys per row and shard, so the dispatch
  splits the long rows into fixed-size pieces merged by the combine kernel.
* 16 heads, one shard: the balanced schedule cuts the long row into pieces
  held by most of the workers (more than eight pieces per row, so the split
  combine's loop over pieces runs more than once), bf16 and FP8 caches.

Every row against the oracle's partial, and the merged rows against the
oracle's unsharded attention.  Many rows per call: a 4096-row prefill chunk
at 128 heads (8192 work items per shard for the dispatch order; sampled rows)
and 2048 single-row requests at 16 heads (every row).
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
    ("h64_w2_131k", [LONG, 300], [2, 1], 64, 2, 64, False),
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


def test_many_rows_prefill_chunk_h128():
    # A 4096-row prefill chunk (8192 work items per shard for the dispatch
    # order) beside a single decode row; sampled rows of both.
    name = "h128_chunk4096"
    wl = WL.make_custom(name, [8192, 40], [4096, 1], H=128, W=2, P=64, seed=98)
    dw = DeviceWorkload(wl)
    log(f"[{name}] T={wl.T}; running")
    dw.outs.fill_(float("nan"))
    dw.step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    toks = sorted({0, 1, 2, 2047, 2048, 4094, 4095, 4096} | set(int(x) for x in rng.integers(0, wl.T, 16)))
    kv = {}
    ref_o, ref_l = _oracle(wl, toks, kv)
    idx = torch.tensor(toks, device="cuda")
    for r in range(wl.W):
        st = check_rows(dw.outs[r][idx], dw.lses[r][idx], ref_o[r], ref_l[r], f"{name} r={r}")
        log(f"[{name}] rank {r}: {st}")
    full_o, full_l = _oracle(wl, toks, kv, unsharded=True)
    check_rows(dw.out[idx], dw.out_lse[idx], full_o, full_l, f"{name} merged")
    assert np.array_equal(dw.valid.cpu().numpy(), np.stack(
        [O.row_counts(wl.seq_lens, wl.query_start_loc, wl.W, r, wl.I) for r in range(wl.W)]))


def test_many_requests_h16():
    # 2048 short requests: the balanced schedule's per-wave scan runs over 32
    # chunks of 64 requests; every row checked.
    name = "h16_b2048"
    rng = np.random.default_rng(6)
    S = [int(x) for x in rng.integers(1, 600, 2048)]
    wl = WL.make_custom(name, S, [1] * 2048, H=16, W=1, P=16, seed=99)
    dw = DeviceWorkload(wl)
    log(f"[{name}] T={wl.T}; running")
    dw.outs.fill_(float("nan"))
    dw.step()
    torch.cuda.synchronize()
    toks = list(range(wl.T))
    ref_o, ref_l = _oracle(wl, toks, {})
    st = check_rows(dw.outs[0], dw.lses[0], ref_o[0], ref_l[0], f"{name}")
    log(f"[{name}] every row: {st}")
