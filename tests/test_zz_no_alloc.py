"""mla_decode_partial_noalloc: the decode without a workspace (the library's
per-GPU scratch array holds the split partials, tickets and dispatch order),
against mla_decode_partial with a caller workspace on the same inputs.

Every case makes two calls in a row on the same GPU, the second with a smaller
input, so the second call runs on scratch the first one left behind; the
outputs must equal those of mla_decode_partial bit for bit (same plan, same
kernels), and the smaller call is also checked against the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from mla_decode_context_amd import binding as mla
from mla_decode_context_amd import workloads as WL
from mla_decode_context_amd.runner import DeviceWorkload
from tests._gpu import check_rows, log, needs_gpu, oracle_partials

pytestmark = [pytest.mark.gpu, needs_gpu]

LIMIT = 64 << 20            # MLA_NOALLOC_SCRATCH_BYTES


def _noalloc(dw, r, out, lse):
    mla.mla_decode_partial_noalloc(dw.q_nope, dw.q_pe, dw.caches[r], dw.tables[r], dw.seq_lens, dw.qsl, dw.W, r,
                                   dw.scale, out, lse, max_query_len=dw.max_query_len, max_seq_len=dw.max_seq_len,
                                   num_splits=dw.num_splits, cp_interleave=dw.I)


CASES = [
    # name, (large S, Q), (small S, Q), H, W, P, num_splits, partial dtype
    ("h16_balanced", ([3000, 700, 5000, 64, 2100, 9000, 33, 1500], [1, 1, 1, 1, 1, 1, 1, 1]),
     ([40, 700, 3], [1, 1, 1]), 16, 1, 64, 0, torch.bfloat16),
    ("h16_dcp2_mtp", ([3000, 700, 5000, 2100], [2, 2, 2, 2]), ([90, 7], [2, 3]), 16, 2, 16, 0, torch.bfloat16),
    ("h16_fixed_splits_tickets", ([4000, 900, 2500], [1, 2, 1]), ([700, 30], [1, 2]), 16, 2, 16, 3, torch.bfloat16),
    ("h48_generic_tickets", ([3000, 130, 64], [2, 1, 5]), ([300, 5], [2, 3]), 48, 2, 33, 0, torch.bfloat16),
    ("h128_ordered", ([1500, 700, 90, 2, 2200], [2, 2, 1, 2, 4]), ([300, 65], [2, 1]), 128, 2, 64, 0,
     torch.bfloat16),
    ("h128_split", ([5000, 900], [1, 2]), ([1200, 3], [1, 3]), 128, 2, 64, 4, torch.bfloat16),
    ("h64_ordered", ([1500, 700, 90, 2, 2200], [2, 2, 1, 2, 4]), ([300, 65], [2, 1]), 64, 2, 64, 0,
     torch.bfloat16),
    ("h16_fp32_partials", ([3000, 700, 5000], [1, 2, 1]), ([40, 70], [2, 1]), 16, 2, 16, 0, torch.float32),
]


@pytest.mark.parametrize("name,large,small,H,W,P,splits,dt", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_call(name, large, small, H, W, P, splits, dt):
    for k, (S, Q) in enumerate((large, small)):
        log(f"noalloc {name} call {k} (S={S}, Q={Q})")
        wl = WL.make_custom(f"{name}_{k}", S, Q, H=H, W=W, P=P, seed=51 + k)
        dw = DeviceWorkload(wl, num_splits=splits, partial_dtype=dt)
        need = mla.workspace_size(wl.B, wl.T, H, wl.max_query_len, wl.max_seq_len, W, splits)
        assert need <= LIMIT, (name, need)
        for r in range(W):
            dw.partial(r)                                   # with the caller's workspace
            out = torch.full_like(dw.outs[r], float("nan"))
            lse = torch.full_like(dw.lses[r], float("nan"))
            _noalloc(dw, r, out, lse)
            torch.cuda.synchronize()
            assert torch.equal(out, dw.outs[r]) and torch.equal(lse, dw.lses[r]), f"{name} call {k} r={r}"
        if k == 1:
            ref_o, ref_l = oracle_partials(wl, list(range(wl.T)))
            for r in range(W):
                check_rows(dw.outs[r], dw.lses[r], ref_o[r], ref_l[r], f"{name} small r={r}")


def test_noalloc_rejects_plans_beyond_the_limit():
    # Two 128-head rows of 100k tokens split 200 ways: 400 split partials of
    # 256 KiB, over the 64 MiB limit; nothing is enqueued.
    wl = WL.make_custom("noalloc_big", [3000], [2], H=128, W=1, P=64, seed=3)
    dw = DeviceWorkload(wl, num_splits=1)
    need = mla.workspace_size(1, 2, 128, 2, 100000, 1, 200)
    assert need > LIMIT
    out = torch.full_like(dw.outs[0], 7.0)
    lse = torch.full_like(dw.lses[0], 7.0)
    with pytest.raises(mla.MlaError, match="MLA_ERR_WORKSPACE"):
        mla.mla_decode_partial_noalloc(dw.q_nope, dw.q_pe, dw.caches[0], dw.tables[0], dw.seq_lens, dw.qsl, 1, 0,
                                       dw.scale, out, lse, max_query_len=2, max_seq_len=100000, num_splits=200)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)
