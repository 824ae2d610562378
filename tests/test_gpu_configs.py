"""GPU parity at the full sizes of the large workloads, in the launch
configuration the benchmark times.

Plain and the two MTP DCP4 workloads are checked on every row (the plain
decode's balanced schedule cuts every row into pieces at worker boundaries, so
all its piece boundaries are covered); the long DCP8 and mixed workloads on
sampled rows the oracle computes one by one: the first and last rows, the
shortened and prefill-chunk requests, every row of the four longest requests
(the first items of the longest-first dispatch order) and seeded random rows.

A 64-head batch at the MTP DCP4 shape (a 128-head model on two
tensor-parallel ranks) is checked on every row as well.

For each workload: every rank's partial against the oracle's partial, the
merged rows against the oracle's unsharded attention (merge(shards) ==
unsharded), valid counts bit-exact, and for the mixed batch the fused merge +
W_UV against the oracle's project-then-merge.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from mla_decode_context_amd import workloads as WL
from mla_decode_context_amd.runner import DeviceWorkload
from oracle import mla_oracle as O
from tests._gpu import (check_proj, check_rows, log, needs_gpu, oracle_partials, oracle_unsharded,
                        oracle_valid, sample_tokens, to_f64)

pytestmark = [pytest.mark.gpu, needs_gpu]

SHORT = {"long_dcp8": (0, 64, 128, 192), "mixed_wuv": (96, 97)}


@pytest.mark.parametrize("name", ["plain", "mtp_dcp4", "long_dcp8", "mixed_wuv", "mtp_dcp4_pages"])
def test_full_config_sampled_rows(name):
    log(f"[{name}] generating inputs")
    wl = WL.make_workload(name, threads=16)
    log(f"[{name}] T={wl.T} B={wl.B} W={wl.W}; uploading and running")
    dw = DeviceWorkload(wl)
    dw.outs.fill_(float("nan"))
    dw.step()
    torch.cuda.synchronize()
    if name in ("plain", "mtp_dcp4", "mtp_dcp4_pages"):
        toks = list(range(wl.T))
    else:
        longest = [int(b) for b in np.argsort(-np.asarray(wl.seq_lens))[:4]]
        toks = sample_tokens(wl, n_random=10, extra_requests=tuple(SHORT.get(name, ())) + tuple(longest))
    log(f"[{name}] oracle on {len(toks)} sampled tokens")
    kv = {}
    ref_o, ref_l = oracle_partials(wl, toks, kv)
    idx = torch.tensor(toks, device="cuda")
    for r in range(wl.W):
        st = check_rows(dw.outs[r][idx], dw.lses[r][idx], ref_o[r], ref_l[r], f"{name} r={r}")
        log(f"[{name}] rank {r}: {st}")
    assert np.array_equal(dw.valid.cpu().numpy()[:, toks], oracle_valid(wl, toks))
    assert np.array_equal(dw.valid.cpu().numpy(), np.stack(
        [O.row_counts(wl.seq_lens, wl.query_start_loc, wl.W, r, wl.I) for r in range(wl.W)]))
    if wl.w_uv is None:
        if wl.W > 1:
            full_o, full_l = oracle_unsharded(wl, toks, kv)
            st = check_rows(dw.out[idx], dw.out_lse[idx], full_o, full_l, f"{name} merged")
            log(f"[{name}] merged vs unsharded: {st}")
    else:
        wuv = O.bf16_bits_to_f64(wl.w_uv)
        ref_y, ref_yl = O.project_then_merge(ref_o, ref_l, oracle_valid(wl, toks), wuv)
        st = check_proj(dw.out_proj[idx], ref_y, f"{name} merge_v_up")
        assert np.max(np.abs(to_f64(dw.out_lse[idx]) - ref_yl)) <= 1e-3
        log(f"[{name}] merge+W_UV vs project-then-merge: {st}")
    # whole-output properties at full size: finite everywhere, empty rows exact
    for r in range(wl.W):
        lse = dw.lses[r]
        empty = dw.valid[r] == 0
        assert torch.isfinite(dw.outs[r]).all()
        assert torch.all(lse[empty] == float("-inf")) and torch.all(dw.outs[r][empty] == 0)
        assert torch.isfinite(lse[~empty]).all()


def test_h64_at_the_mtp_dcp4_shape():
    # 64 heads (a 128-head model on two tensor-parallel ranks) at the MTP DCP4
    # batch shape: 128 requests of two query rows, contexts 1024..4096, four
    # shards, pages of 64.  The 128-head kernel serves it with one 64-head block
    # per row and the dispatch order; every row against the oracle.
    name = "h64_mtp_dcp4_shape"
    rng = np.random.default_rng(44)
    S = [int(x) for x in rng.integers(1024, 4097, 128)]
    wl = WL.make_custom(name, S, [2] * 128, H=64, W=4, P=64, seed=44, threads=16)
    log(f"[{name}] T={wl.T}; running")
    dw = DeviceWorkload(wl)
    dw.outs.fill_(float("nan"))
    dw.step()
    torch.cuda.synchronize()
    toks = list(range(wl.T))
    kv = {}
    ref_o, ref_l = oracle_partials(wl, toks, kv)
    for r in range(wl.W):
        st = check_rows(dw.outs[r], dw.lses[r], ref_o[r], ref_l[r], f"{name} r={r}")
        log(f"[{name}] rank {r}: {st}")
    assert np.array_equal(dw.valid.cpu().numpy(), oracle_valid(wl, toks))
    full_o, full_l = oracle_unsharded(wl, toks, kv)
    st = check_rows(dw.out, dw.out_lse, full_o, full_l, f"{name} merged")
    log(f"[{name}] merged vs unsharded: {st}")
