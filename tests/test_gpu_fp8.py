"""GPU parity of the FP8 E4M3 latent cache (one fp32 scale per cache) in the
16-head decode against the fp64 oracle's dequantised decode.

The cache rows hold E4M3 codes; the oracle takes each element as code value x
scale.  The kernel expands each stage to bf16 exactly and applies the scale in
fp32, so the tolerances are those of the bf16 cache."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from mla_decode_context_amd import binding as mla
from mla_decode_context_amd import workloads as WL
from mla_decode_context_amd.runner import DeviceWorkload
from oracle import mla_oracle as O
from tests._gpu import check_rows, log, needs_gpu, oracle_valid

pytestmark = [pytest.mark.gpu, needs_gpu]

KS = WL.FP8_SCALE


def _oracle(wl, toks, kv=None, unsharded=False):
    kv = {} if kv is None else kv

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


CASES = [
    # name, seq_lens, query_lens, H, W, P, I, num_splits
    ("h16_w1_p64", [1100, 31, 33, 700], [1, 1, 1, 1], 16, 1, 64, 1, 0),
    ("h16_w2_p16", [6, 37, 128, 255], [4, 4, 4, 4], 16, 2, 16, 1, 0),
    ("h16_w2_split3", [6, 37, 128, 255], [4, 4, 4, 4], 16, 2, 16, 1, 3),
    ("h16_w3_p7_ragged", [9, 2, 70, 33, 400], [3, 2, 1, 5, 2], 16, 3, 7, 1, 0),
    ("h8_w2_p1", [40, 5, 17], [2, 1, 3], 8, 2, 1, 1, 0),
    ("h1_w1_unsplit", [300, 5, 40], [1, 2, 3], 1, 1, 16, 1, 1),
    ("h16_w4_pages", [700, 64, 129, 5], [2, 2, 1, 3], 16, 4, 16, 16, 0),
    ("h16_w16_sparse", [40, 3, 100, 17], [2, 1, 3, 4], 16, 16, 16, 1, 0),
]


@pytest.mark.parametrize("name,S,Q,H,W,P,I,splits", CASES, ids=[c[0] for c in CASES])
def test_fp8_cache_small(name, S, Q, H, W, P, I, splits):
    log(f"fp8 {name}")
    wl = WL.make_custom(name, S, Q, H=H, W=W, P=P, seed=71, I=I, kv_scale=KS)
    toks = list(range(wl.T))
    ref_o, ref_l = _oracle(wl, toks)
    full_o, full_l = _oracle(wl, toks, unsharded=True)
    dw = DeviceWorkload(wl, num_splits=splits)
    assert dw.caches[0].dtype == torch.uint8
    dw.outs.fill_(float("nan"))
    dw.step()
    torch.cuda.synchronize()
    for r in range(W):
        check_rows(dw.outs[r], dw.lses[r], ref_o[r], ref_l[r], f"{name} fp8 r={r}")
    assert np.array_equal(dw.valid.cpu().numpy(), oracle_valid(wl, toks))
    check_rows(dw.out, dw.out_lse, full_o, full_l, f"{name} fp8 merged")


def test_fp8_cache_f32_partials_and_two_stage():
    wl = WL.make_custom("fp8_two", [300, 17, 64, 2, 129], [2, 3, 1, 2, 4], H=16, W=2, P=16, seed=72, kv_scale=KS)
    toks = list(range(wl.T))
    full_o, full_l = _oracle(wl, toks, unsharded=True)
    dw = DeviceWorkload(wl, partial_dtype=torch.float32)
    dw.step()
    torch.cuda.synchronize()
    check_rows(dw.out, dw.out_lse, full_o, full_l, "fp8 fp32-partials merged")
    dw.setup_two_stage()
    dw.two_stage_step()
    torch.cuda.synchronize()
    check_rows(dw.out, dw.out_lse, full_o, full_l, "fp8 two-stage merged")


def test_fp8_plain_full_size_every_row():
    wl = WL.make_workload("plain_fp8", threads=16)
    log(f"plain_fp8 T={wl.T}")
    dw = DeviceWorkload(wl)
    dw.outs.fill_(float("nan"))
    dw.step()
    torch.cuda.synchronize()
    toks = list(range(wl.T))
    ref_o, ref_l = _oracle(wl, toks)
    st = check_rows(dw.outs[0], dw.lses[0], ref_o[0], ref_l[0], "plain_fp8 every row")
    log(f"plain_fp8 every row: {st}")


def test_fp8_cache_needs_at_most_16_heads():
    wl = WL.make_custom("fp8_h128", [100, 20], [2, 1], H=128, W=1, P=64, seed=73, kv_scale=KS)
    dw = DeviceWorkload(wl)
    out = torch.full_like(dw.outs[0], 7.0)
    with pytest.raises(mla.MlaError, match="MLA_ERR_UNSUPPORTED"):
        mla.mla_decode_partial(dw.q_nope, dw.q_pe, dw.caches[0], dw.tables[0], dw.seq_lens, dw.qsl, 1, 0,
                               dw.scale, out, dw.lses[0], max_query_len=2, max_seq_len=100, kv_scale=KS)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
