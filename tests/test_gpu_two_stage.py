"""GPU parity of the two-stage decode (query rows > 1): the context stage of
every rank (MLA_MASK_CONTEXT: all rows of a request see the rank's share of
its tokens before the query tokens, no causal mask), the query stage over the
query tokens' own KV (ordinary causal call, one rank), and the merge of the
W + 1 partials, against the fp64 oracle's two stages and against unsharded
attention."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from mla_decode_context_amd import workloads as WL
from mla_decode_context_amd.runner import DeviceWorkload
from oracle import mla_oracle as O
from tests._gpu import check_proj, check_rows, log, needs_gpu, oracle_unsharded, sample_tokens, to_f64

pytestmark = [pytest.mark.gpu, needs_gpu]


def _oracle_stages(wl, toks, kv=None):
    kv = {} if kv is None else kv

    def gkv(b):
        if b not in kv:
            kv[b] = wl.global_kv(b)
        return kv[b]

    ctx = [O.decode_context_part(wl.seq_lens, wl.query_start_loc, wl.q_nope, wl.q_pe, gkv, wl.scale, wl.W, r,
                                 tokens=toks, I=wl.I) for r in range(wl.W)]
    qp = O.decode_query_part(wl.seq_lens, wl.query_start_loc, wl.q_nope, wl.q_pe, gkv, wl.scale, tokens=toks)
    return ctx, qp


def _context_counts(wl):
    qsl = wl.query_start_loc
    out = []
    for r in range(wl.W):
        c = []
        for b in range(wl.B):
            Q = int(qsl[b + 1] - qsl[b])
            c += [O.context_count(int(wl.seq_lens[b]), Q, wl.W, r, wl.I)] * Q
        out.append(c)
    return np.array(out, dtype=np.int32).reshape(wl.W, wl.T)


CASES = [
    # name, seq_lens, query_lens, H, W, P, I, num_splits
    ("h16_w2", [6, 37, 128, 255], [4, 4, 4, 4], 16, 2, 16, 1, 0),
    ("h16_w4_split3", [300, 17, 64, 5, 129], [2, 3, 1, 5, 4], 16, 4, 16, 1, 3),
    ("h16_w1", [100, 3, 700], [2, 3, 1], 16, 1, 64, 1, 0),
    ("h48_w3", [130, 64, 9], [2, 1, 5], 48, 3, 33, 1, 0),
    ("h128_w2", [700, 90, 2, 1500], [2, 1, 2, 4], 128, 2, 64, 1, 0),
    ("h128_w8_short", [2, 3, 5, 7, 200], [2, 3, 1, 2, 4], 128, 8, 64, 1, 0),
    ("h128_w4_pages", [700, 64, 129, 5], [2, 2, 1, 3], 128, 4, 64, 64, 0),
    ("h128_split", [5000, 900, 3], [1, 2, 3], 128, 2, 64, 1, 4),
    ("h64_w2", [700, 90, 2, 1500], [2, 1, 2, 4], 64, 2, 64, 1, 0),
    ("h64_w4_pages_split", [3000, 64, 129, 5], [2, 2, 1, 3], 64, 4, 64, 64, 3),
    ("h8_q_equals_s", [3, 5, 40, 1], [3, 5, 2, 1], 8, 2, 16, 1, 0),
]


@pytest.mark.parametrize("name,S,Q,H,W,P,I,splits", CASES, ids=[c[0] for c in CASES])
def test_two_stage_small(name, S, Q, H, W, P, I, splits):
    log(f"two-stage {name}")
    wl = WL.make_custom(name, S, Q, H=H, W=W, P=P, seed=61, I=I)
    toks = list(range(wl.T))
    (ctx, qp) = _oracle_stages(wl, toks)
    full_o, full_l = oracle_unsharded(wl, toks)
    dw = DeviceWorkload(wl, num_splits=splits)
    dw.setup_two_stage()
    dw.outs2.fill_(float("nan"))
    dw.two_stage_step()
    torch.cuda.synchronize()
    assert np.array_equal(dw.valid2[:W].cpu().numpy(), _context_counts(wl)), name
    assert np.array_equal(dw.valid2[W].cpu().numpy(),
                          np.concatenate([np.arange(1, q + 1) for q in wl.query_lens]).astype(np.int32)), name
    for r in range(W):
        check_rows(dw.outs2[r], dw.lses2[r], ctx[r][0], ctx[r][1], f"{name} context r={r}")
    check_rows(dw.outs2[W], dw.lses2[W], qp[0], qp[1], f"{name} query part")
    check_rows(dw.out, dw.out_lse, full_o, full_l, f"{name} merged")
    # the one-stage path on the same inputs agrees with it
    dw.step()
    torch.cuda.synchronize()
    check_rows(dw.out, dw.out_lse, full_o, full_l, f"{name} one-stage merged")


def test_two_stage_f32_partials():
    wl = WL.make_custom("two_stage_f32", [700, 90, 2, 1500], [2, 1, 2, 4], H=128, W=2, P=64, seed=62)
    toks = list(range(wl.T))
    ctx, qp = _oracle_stages(wl, toks)
    full_o, full_l = oracle_unsharded(wl, toks)
    dw = DeviceWorkload(wl, partial_dtype=torch.float32)
    dw.setup_two_stage()
    dw.two_stage_step()
    torch.cuda.synchronize()
    assert dw.outs2.dtype == torch.float32
    for r in range(wl.W):
        check_rows(dw.outs2[r], dw.lses2[r], ctx[r][0], ctx[r][1], f"f32 context r={r}")
    check_rows(dw.outs2[wl.W], dw.lses2[wl.W], qp[0], qp[1], "f32 query part")
    check_rows(dw.out, dw.out_lse, full_o, full_l, "f32 merged")


SHORT = {"long_dcp8": (0, 64, 128, 192), "mixed_wuv": (96, 97)}


@pytest.mark.parametrize("name", ["mtp_dcp4", "long_dcp8", "mixed_wuv"])
def test_two_stage_full_size_sampled(name):
    """The two-stage path at the full sizes of the DCP workloads, on sampled rows
    (first and last rows, the shortened requests, the prefill chunks' first and
    last rows, seeded random rows)."""
    log(f"[{name}] generating inputs")
    wl = WL.make_workload(name, threads=16)
    dw = DeviceWorkload(wl)
    dw.setup_two_stage()
    dw.outs2.fill_(float("nan"))
    log(f"[{name}] T={wl.T}: two-stage step")
    dw.two_stage_step()
    torch.cuda.synchronize()
    assert np.array_equal(dw.valid2[:wl.W].cpu().numpy(), _context_counts(wl))
    toks = sample_tokens(wl, n_random=8, extra_requests=SHORT.get(name, ()))
    log(f"[{name}] oracle on {len(toks)} sampled tokens")
    kv = {}
    ctx, qp = _oracle_stages(wl, toks, kv)
    idx = torch.tensor(toks, device="cuda")
    for r in range(wl.W):
        check_rows(dw.outs2[r][idx], dw.lses2[r][idx], ctx[r][0], ctx[r][1], f"{name} context r={r}")
    check_rows(dw.outs2[wl.W][idx], dw.lses2[wl.W][idx], qp[0], qp[1], f"{name} query part")
    valid = np.concatenate([dw.valid2.cpu().numpy()[:, toks]])
    if wl.w_uv is None:
        full_o, full_l = oracle_unsharded(wl, toks, kv)
        check_rows(dw.out[idx], dw.out_lse[idx], full_o, full_l, f"{name} merged")
    else:
        outs = np.stack([c[0] for c in ctx] + [qp[0]])
        lses = np.stack([c[1] for c in ctx] + [qp[1]])
        ref_y, ref_yl = O.project_then_merge(outs, lses, valid, O.bf16_bits_to_f64(wl.w_uv))
        check_proj(dw.out_proj[idx], ref_y, f"{name} merge_v_up")
        assert np.max(np.abs(to_f64(dw.out_lse[idx]) - ref_yl)) <= 1e-3
