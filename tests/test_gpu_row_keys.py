"""GPU check of the per-row key counts mla_decode_partial writes into
`row_keys`: bit-exact against the oracle's per-rank seqlen_k (the pages' per-row
count) and against mla_dcp_local_seqlens, on every kernel path (16-head
balanced schedule and fixed splits, the generic kernel, the 128-head kernel
with and without its dispatch order, the allocation-free entry point), both
mask modes and the run layout, with rows that see no key."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from mla_decode_context_amd import binding as mla
from mla_decode_context_amd import workloads as WL
from mla_decode_context_amd.runner import DeviceWorkload
from oracle import mla_oracle as O
from tests._gpu import log, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]

CASES = [
    # name, seq_lens, query_lens, H, W, P, I, num_splits, workspace
    ("h16_balanced", [300, 2, 1, 700, 65], [2, 1, 1, 3, 4], 16, 4, 16, 1, 0, True),
    ("h16_fixed_splits", [300, 2, 1, 700, 65], [2, 1, 1, 3, 4], 16, 4, 16, 1, 3, True),
    ("h16_unsplit", [40, 1, 130], [3, 1, 1], 16, 2, 64, 1, 1, False),
    ("h48_generic", [130, 64, 9, 2], [2, 1, 5, 2], 48, 3, 33, 1, 0, True),
    ("h128_ordered", [700, 90, 2, 1500, 3], [2, 1, 2, 4, 3], 128, 8, 64, 1, 0, True),
    ("h128_token_order", [700, 90, 2, 1500, 3], [2, 1, 2, 4, 3], 128, 8, 64, 1, 0, False),
    ("h128_split", [5000, 900, 3], [1, 2, 3], 128, 2, 64, 1, 4, True),
    ("h16_runs", [700, 64, 129, 5], [2, 2, 1, 3], 16, 4, 16, 16, 0, True),
    ("h128_runs", [700, 64, 129, 5], [2, 2, 1, 3], 128, 4, 64, 64, 0, True),
    ("h64_ordered", [700, 90, 2, 1500, 3], [2, 1, 2, 4, 3], 64, 8, 64, 1, 0, True),
    ("h64_split", [5000, 900, 3], [1, 2, 3], 64, 2, 64, 1, 4, True),
]


def _oracle_counts(wl, mode):
    qsl = wl.query_start_loc
    out = []
    for r in range(wl.W):
        if mode == mla.MASK_CAUSAL:
            out.append(O.row_counts(wl.seq_lens, qsl, wl.W, r, wl.I))
        else:
            c = []
            for b in range(wl.B):
                Q = int(qsl[b + 1] - qsl[b])
                c += [O.context_count(int(wl.seq_lens[b]), Q, wl.W, r, wl.I)] * Q
            out.append(np.array(c, dtype=np.int64))
    return np.stack(out).astype(np.int32)


@pytest.mark.parametrize("mode", [mla.MASK_CAUSAL, mla.MASK_CONTEXT], ids=["causal", "context"])
@pytest.mark.parametrize("name,S,Q,H,W,P,I,splits,use_ws", CASES, ids=[c[0] for c in CASES])
def test_decode_writes_row_keys(name, S, Q, H, W, P, I, splits, use_ws, mode):
    log(f"row_keys {name} mode={mode}")
    wl = WL.make_custom(name, S, Q, H=H, W=W, P=P, seed=81, I=I)
    dw = DeviceWorkload(wl, num_splits=splits)
    ws = dw.workspace if use_ws else None
    keys = torch.full((W, wl.T), -7, dtype=torch.int32, device="cuda")
    ref = torch.full((W, wl.T), -7, dtype=torch.int32, device="cuda")
    for r in range(W):
        mla.mla_decode_partial(dw.q_nope, dw.q_pe, dw.caches[r], dw.tables[r], dw.seq_lens, dw.qsl, W, r, dw.scale,
                               dw.outs[r], dw.lses[r], max_query_len=dw.max_query_len, max_seq_len=dw.max_seq_len,
                               workspace=ws, num_splits=splits, cp_interleave=I, mask_mode=mode, row_keys=keys[r])
        mla.mla_dcp_local_seqlens(dw.seq_lens, dw.qsl, wl.T, W, r, row_seqlen=ref[r], cp_interleave=I,
                                  mask_mode=mode)
    torch.cuda.synchronize()
    got = keys.cpu().numpy()
    assert np.array_equal(got, _oracle_counts(wl, mode)), name
    assert np.array_equal(got, ref.cpu().numpy()), name
    if mode == mla.MASK_CAUSAL:
        assert (got == 0).any(), "the cases include rows that see no key on some rank"


def test_noalloc_writes_row_keys():
    wl = WL.make_custom("row_keys_noalloc", [300, 2, 1, 700, 65], [2, 1, 1, 3, 4], H=128, W=4, P=64, seed=82)
    dw = DeviceWorkload(wl)
    keys = torch.full((wl.W, wl.T), -7, dtype=torch.int32, device="cuda")
    for r in range(wl.W):
        mla.mla_decode_partial_noalloc(dw.q_nope, dw.q_pe, dw.caches[r], dw.tables[r], dw.seq_lens, dw.qsl, wl.W, r,
                                       dw.scale, dw.outs[r], dw.lses[r], max_query_len=dw.max_query_len,
                                       max_seq_len=dw.max_seq_len, row_keys=keys[r])
    torch.cuda.synchronize()
    assert np.array_equal(keys.cpu().numpy(), _oracle_counts(wl, mla.MASK_CAUSAL))


def test_step_counts_come_from_the_decode():
    """The runner's step takes the merge's valid counts from the decode calls."""
    wl = WL.make_custom("row_keys_step", [300, 2, 1, 700, 65], [2, 1, 1, 3, 4], H=16, W=4, P=16, seed=83)
    dw = DeviceWorkload(wl)
    dw.valid.fill_(-7)
    dw.step()
    torch.cuda.synchronize()
    assert np.array_equal(dw.valid.cpu().numpy(), _oracle_counts(wl, mla.MASK_CAUSAL))
