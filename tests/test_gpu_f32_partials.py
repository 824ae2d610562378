"""fp32 partials: mla_decode_partial writing the normalised fp32 accumulator and
the merges (and the exchange's pack) reading fp32 partials, against the fp64
oracle at the stated tolerances.

With bf16 partials a merged row is rounded to bf16 twice (the partial, then the
merged output); with fp32 partials once.  Both decode outputs come from the same
fp32 accumulator, so the bf16 partial must be exactly the fp32 partial rounded
to nearest even.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from mla_decode_context_amd import binding as mla
from mla_decode_context_amd import workloads as WL
from mla_decode_context_amd.runner import DeviceWorkload
from oracle import mla_oracle as O
from tests._gpu import (check_proj, check_rows, log, needs_gpu, oracle_partials, oracle_unsharded, oracle_valid,
                        sample_tokens, to_f64)

pytestmark = [pytest.mark.gpu, needs_gpu]

F32 = torch.float32


def _both(wl, num_splits=0):
    """The same step with bf16 and with fp32 partials."""
    out = []
    for dt in (torch.bfloat16, F32):
        dw = DeviceWorkload(wl, num_splits=num_splits, partial_dtype=dt)
        dw.outs.fill_(float("nan"))
        dw.step()
        torch.cuda.synchronize()
        out.append(dw)
    return out


CASES = [
    # name, seq_lens, query_lens, H, W, P, I, num_splits
    ("tiny_h16", [6, 37, 128, 255], [4, 4, 4, 4], 16, 2, 16, 1, 0),
    ("tiny_h16_split3", [6, 37, 128, 255], [4, 4, 4, 4], 16, 2, 16, 1, 3),
    ("h16_unsplit", [100, 3, 700], [1, 2, 1], 16, 3, 16, 1, 1),
    ("h48_generic", [130, 64, 5], [2, 0, 5], 48, 4, 33, 1, 0),
    ("h128_ordered", [700, 90, 2, 1500], [2, 1, 2, 4], 128, 2, 64, 1, 0),
    ("h128_split", [5000, 900, 3], [1, 2, 3], 128, 2, 64, 1, 4),
    ("h128_pages", [700, 64, 129, 5], [2, 2, 1, 3], 128, 4, 64, 64, 0),
    ("h64_ordered", [700, 90, 2, 1500], [2, 1, 2, 4], 64, 2, 64, 1, 0),
    ("h8_w8_empty_rows", [2, 3, 5, 7, 60], [2, 3, 1, 2, 4], 8, 8, 16, 1, 0),
]


@pytest.mark.parametrize("name,S,Q,H,W,P,I,splits", CASES, ids=[c[0] for c in CASES])
def test_f32_partials_and_merge(name, S, Q, H, W, P, I, splits):
    log(f"fp32 partials {name}")
    wl = WL.make_custom(name, S, Q, H=H, W=W, P=P, seed=41, I=I)
    toks = list(range(wl.T))
    ref_o, ref_l = oracle_partials(wl, toks)
    full_o, full_l = oracle_unsharded(wl, toks)
    d16, d32 = _both(wl, splits)
    assert d32.outs.dtype == F32
    for r in range(W):
        check_rows(d32.outs[r], d32.lses[r], ref_o[r], ref_l[r], f"{name} fp32 r={r}")
        # one accumulator, two roundings of it: bf16 partial == RNE(fp32 partial), LSE identical
        assert torch.equal(d16.outs[r], d32.outs[r].to(torch.bfloat16)), f"{name} r={r}"
        assert torch.equal(d16.lses[r], d32.lses[r]), f"{name} r={r}"
    assert np.array_equal(d32.valid.cpu().numpy(), oracle_valid(wl, toks))
    check_rows(d32.out, d32.out_lse, full_o, full_l, f"{name} fp32 merged")


@pytest.mark.parametrize("H,W", [(16, 2), (128, 3)])
def test_many_short_requests_f32_all_rows(H, W):
    """Requests of 0-60 tokens (plus a few of 700): with fp32 partials every merged
    row, including rows that see a handful of keys (values up to ~4.5), is held
    to max-abs 2e-2, rel-L2 5e-3 and LSE 1e-3 against unsharded attention."""
    rng = np.random.default_rng(21 + H + W)
    B = 240
    Q = rng.integers(0, 4, size=B)
    S = Q + rng.integers(0, 60, size=B)
    S[::37] = Q[::37] + 700
    log(f"many short requests, fp32 partials, H={H} W={W} T={int(Q.sum())}")
    wl = WL.make_custom("many_short", S, Q, H=H, W=W, P=16, seed=13)
    toks = list(range(wl.T))
    ref_o, ref_l = oracle_partials(wl, toks)
    full_o, full_l = oracle_unsharded(wl, toks)
    dw = DeviceWorkload(wl, partial_dtype=F32)
    dw.outs.fill_(float("nan"))
    dw.step()
    torch.cuda.synchronize()
    for r in range(W):
        check_rows(dw.outs[r], dw.lses[r], ref_o[r], ref_l[r], f"many_short fp32 H={H} r={r}")
    st = check_rows(dw.out, dw.out_lse, full_o, full_l, f"many_short fp32 H={H} merged")
    log(f"merged (all {wl.T} rows): {st}")


def _random_partials_f32(W, T, H, seed, p_invalid=0.25):
    rng = np.random.default_rng(seed)
    outs = (rng.standard_normal((W, T, H, 512)) * 0.3).astype(np.float32)
    lses = (rng.standard_normal((W, T, H)) * 2 + 3).astype(np.float32)
    valid = (rng.random((W, T)) > p_invalid).astype(np.int32) * rng.integers(1, 50, size=(W, T)).astype(np.int32)
    valid[:, 0] = 0
    valid[0, 1] = 5
    valid[1:, 1] = 0
    return outs, lses, valid


@pytest.mark.parametrize("W,T,H", [(2, 37, 16), (4, 19, 128), (8, 9, 128), (13, 6, 2), (5, 41, 9), (1, 5, 16)])
def test_lse_merge_f32_inputs(W, T, H):
    log(f"merge fp32 W={W} T={T} H={H}")
    outs, lses, valid = _random_partials_f32(W, T, H, seed=W * 100 + T)
    ref_o, ref_l = O.lse_merge(outs.astype(np.float64), lses.astype(np.float64), valid)
    outs_p, lses_p = outs.copy(), lses.copy()
    outs_p[valid <= 0] = np.nan          # ranks that take no part are never read
    lses_p[valid <= 0] = np.nan
    out = torch.full((T, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    out_lse = torch.full((T, H), float("nan"), dtype=F32, device="cuda")
    mla.mla_lse_merge(torch.from_numpy(outs_p).cuda(), torch.from_numpy(lses_p).cuda(),
                      torch.from_numpy(valid).cuda(), out, out_lse)
    torch.cuda.synchronize()
    check_rows(out, out_lse, ref_o, ref_l, f"merge fp32 W={W}")
    # one rounding: the merged output is within half a bf16 ulp of the fp64
    # merge of the same fp32 inputs, plus the fp32 arithmetic (absolute: a value
    # near zero can come from partials of size ~1, whose fp32 error is ~1e-7)
    go = to_f64(out)
    live = np.isfinite(ref_l)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref_o[live]), 2.0 ** -126))) - 7)
    assert np.all(np.abs(go[live] - ref_o[live]) <= 0.5 * ulp + 2e-6)
    # without counts: ranks that take no part carry -inf (and zeros)
    lses_m = lses.copy()
    lses_m[np.broadcast_to((valid <= 0)[:, :, None], lses.shape)] = -np.inf
    outs_z = outs.copy()
    outs_z[valid <= 0] = 0
    out2 = torch.full_like(out, float("nan"))
    lse2 = torch.full_like(out_lse, float("nan"))
    mla.mla_lse_merge(torch.from_numpy(outs_z).cuda(), torch.from_numpy(lses_m).cuda(), None, out2, lse2)
    torch.cuda.synchronize()
    check_rows(out2, lse2, ref_o, ref_l, f"merge fp32 W={W} valid=None")


@pytest.mark.parametrize("W,T,H", [(4, 70, 128), (1, 16, 16), (2, 130, 24), (8, 3, 128), (3, 2, 8)])
def test_merge_v_up_proj_f32_inputs(W, T, H):
    log(f"merge_v_up fp32 W={W} T={T} H={H}")
    outs, lses, valid = _random_partials_f32(W, T, H, seed=W * 7 + T)
    rng = np.random.default_rng(3)
    wuv_t = torch.from_numpy((0.02 * rng.standard_normal((H, 512, 128))).astype(np.float32)).to(torch.bfloat16)
    wuv = to_f64(wuv_t)
    ref_y, ref_l = O.project_then_merge(outs.astype(np.float64), lses.astype(np.float64), valid, wuv)
    outs_p = outs.copy()
    outs_p[valid <= 0] = np.nan
    y = torch.full((T, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    yl = torch.full((T, H), float("nan"), dtype=F32, device="cuda")
    mla.mla_merge_v_up_proj(torch.from_numpy(outs_p).cuda(), torch.from_numpy(lses).cuda(),
                            torch.from_numpy(valid).cuda(), wuv_t.cuda(), y, yl)
    torch.cuda.synchronize()
    dead = valid.sum(axis=0) == 0
    assert np.all(to_f64(y)[dead] == 0) and np.all(to_f64(yl)[dead] == -np.inf)
    check_proj(y[torch.from_numpy(~dead)], ref_y[~dead], f"merge_v_up fp32 W={W}")
    assert np.max(np.abs(to_f64(yl)[~dead] - ref_l[~dead])) <= 1e-3


@pytest.mark.parametrize("W", [2, 4])
def test_pack_f32_partials(W):
    """The exchange's pack reading fp32 partials: against the oracle's pack of the
    same partials, and its receivers' combine against project-then-merge."""
    log(f"exchange pack fp32 W={W}")
    wl = WL.make_custom("xf32", [300, 17, 64, 2, 129], [2, 3, 1, 2, 4], H=128, W=W, P=16, seed=17, w_uv=True)
    dw = DeviceWorkload(wl, partial_dtype=F32)
    for r in range(W):
        dw.partial(r)
    dw.valid_counts()
    torch.cuda.synchronize()
    valid = dw.valid.cpu().numpy()
    for r in range(W):
        dead = torch.tensor(valid[r] == 0, device="cuda")
        dw.outs[r][dead] = float("nan")
    T, H = wl.T, wl.H
    Hs = H // W
    wuv = O.bf16_bits_to_f64(wl.w_uv)
    send_y = torch.full((W, W, T, Hs, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    send_l = torch.full((W, W, T, Hs), float("nan"), dtype=F32, device="cuda")
    for r in range(W):
        mla.mla_dcp_a2a_pack(dw.outs[r], dw.lses[r], dw.valid[r], dw.w_uv, send_y[r], send_l[r], W)
    out = torch.empty((W, T, Hs, 128), dtype=torch.bfloat16, device="cuda")
    out_l = torch.empty((W, T, Hs), dtype=F32, device="cuda")
    for q in range(W):
        mla.mla_dcp_a2a_combine(send_y[:, q], send_l[:, q], out[q], out_l[q])
    torch.cuda.synchronize()
    outs64, lses64 = np.nan_to_num(to_f64(dw.outs)), to_f64(dw.lses)
    for r in range(W):
        ref_y, _ = O.a2a_pack(outs64[r], np.nan_to_num(lses64[r]), valid[r], wuv, W)
        err = np.abs(to_f64(send_y[r]) - ref_y)
        assert np.all(err <= 1e-2 * np.maximum(1.0, np.abs(ref_y))), (r, float(err.max()))
    full_y, full_l = O.project_then_merge(outs64, np.nan_to_num(lses64), valid, wuv)
    for q in range(W):
        check_proj(out[q], full_y[:, q * Hs:(q + 1) * Hs], f"pack fp32 dest={q}")


def test_full_mixed_batch_f32_partials():
    """The mixed batch (96 decodes + two 512-row chunks, W = 4, merge fused with
    W_UV) at full size with fp32 partials, on sampled rows."""
    wl = WL.make_workload("mixed_wuv", threads=16)
    log(f"mixed_wuv fp32 partials T={wl.T}")
    dw = DeviceWorkload(wl, partial_dtype=F32)
    dw.outs.fill_(float("nan"))
    dw.step()
    torch.cuda.synchronize()
    toks = sample_tokens(wl, n_random=10, extra_requests=(96, 97))
    kv = {}
    ref_o, ref_l = oracle_partials(wl, toks, kv)
    idx = torch.tensor(toks, device="cuda")
    for r in range(wl.W):
        check_rows(dw.outs[r][idx], dw.lses[r][idx], ref_o[r], ref_l[r], f"mixed fp32 r={r}")
    ref_y, ref_yl = O.project_then_merge(ref_o, ref_l, oracle_valid(wl, toks), O.bf16_bits_to_f64(wl.w_uv))
    check_proj(dw.out_proj[idx], ref_y, "mixed fp32 merge_v_up")
    assert np.max(np.abs(to_f64(dw.out_lse[idx]) - ref_yl)) <= 1e-3
