"""GPU parity of mla_lse_merge and mla_merge_v_up_proj against the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from mla_decode_context_amd import binding as mla
from oracle import mla_oracle as O
from tests._gpu import check_proj, check_rows, log, needs_gpu, to_f64

pytestmark = [pytest.mark.gpu, needs_gpu]


def _bf16_round(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)


def _random_partials(W, T, H, seed, p_invalid=0.25):
    rng = np.random.default_rng(seed)
    outs = _bf16_round(rng.standard_normal((W, T, H, 512)) * 0.3)
    lses = (rng.standard_normal((W, T, H)) * 2 + 3).astype(np.float32)
    valid = (rng.random((W, T)) > p_invalid).astype(np.int32) * rng.integers(1, 50, size=(W, T)).astype(np.int32)
    valid[:, 0] = 0          # a row no rank takes part in
    valid[0, 1] = 5          # a row with exactly one rank
    valid[1:, 1] = 0
    return outs, lses, valid


def _oracle_merge(outs_t, lses, valid):
    return O.lse_merge(to_f64(outs_t), lses.astype(np.float64), valid)


@pytest.mark.parametrize("W,T,H", [(1, 5, 16), (2, 37, 16), (4, 19, 128), (8, 9, 128), (3, 70, 20), (13, 6, 2),
                                   (8, 2, 128), (2, 3, 1), (5, 41, 9)])
def test_lse_merge_random(W, T, H):
    log(f"merge W={W} T={T} H={H}")
    outs_t, lses, valid = _random_partials(W, T, H, seed=W * 100 + T)
    ref_o, ref_l = _oracle_merge(outs_t, lses, valid)
    # poison everything that does not take part: the kernel must not read it
    outs_p = outs_t.clone()
    lses_p = lses.copy()
    for w in range(W):
        for t in range(T):
            if valid[w, t] <= 0:
                outs_p[w, t] = float("nan")
                lses_p[w, t] = np.nan
    d_outs = outs_p.cuda()
    d_lses = torch.from_numpy(lses_p).cuda()
    d_valid = torch.from_numpy(valid).cuda()
    out = torch.full((T, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    out_lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_lse_merge(d_outs, d_lses, d_valid, out, out_lse)
    torch.cuda.synchronize()
    check_rows(out, out_lse, ref_o, ref_l, f"merge W={W}")
    # without counts: invalid ranks are marked by lse = -inf instead
    lses_m = lses.copy()
    lses_m[np.broadcast_to((valid <= 0)[:, :, None], lses.shape)] = -np.inf
    out2 = torch.full_like(out, float("nan"))
    lse2 = torch.full_like(out_lse, float("nan"))
    mla.mla_lse_merge(d_outs.clone().nan_to_num_(0.0), torch.from_numpy(lses_m).cuda(), None, out2, lse2)
    torch.cuda.synchronize()
    check_rows(out2, lse2, ref_o, ref_l, f"merge W={W} valid=None")


def test_merge_identities():
    W, T, H = 4, 8, 16
    outs_t, lses, _ = _random_partials(W, T, H, seed=9, p_invalid=0.0)
    ones = np.ones((W, T), dtype=np.int32)
    # W copies of one partial: same output, LSE + ln W
    same = outs_t[:1].repeat(W, 1, 1, 1).cuda()
    same_l = torch.from_numpy(np.repeat(lses[:1], W, axis=0)).cuda()
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    ol = torch.empty((T, H), dtype=torch.float32, device="cuda")
    mla.mla_lse_merge(same, same_l, torch.from_numpy(ones).cuda(), out, ol)
    torch.cuda.synchronize()
    assert np.max(np.abs(to_f64(out) - to_f64(outs_t[0]))) <= 2 ** -7
    assert np.max(np.abs(to_f64(ol) - (lses[0] + np.log(W)))) <= 1e-5
    # shard order does not matter (up to fp32 summation order)
    perm = [2, 0, 3, 1]
    out_a = torch.empty_like(out)
    out_b = torch.empty_like(out)
    la = torch.empty_like(ol)
    lb = torch.empty_like(ol)
    d = outs_t.cuda()
    dl = torch.from_numpy(lses).cuda()
    dv = torch.from_numpy(ones).cuda()
    mla.mla_lse_merge(d, dl, dv, out_a, la)
    mla.mla_lse_merge(d[perm].contiguous(), dl[perm].contiguous(), dv[perm].contiguous(), out_b, lb)
    torch.cuda.synchronize()
    assert np.max(np.abs(to_f64(out_a) - to_f64(out_b))) <= 2 ** -7
    assert np.max(np.abs(to_f64(la) - to_f64(lb))) <= 1e-5


@pytest.mark.parametrize("W,T,H", [(4, 70, 128), (1, 16, 16), (2, 130, 24), (8, 3, 128), (3, 2, 8), (12, 17, 4)])
def test_merge_v_up_proj_random(W, T, H):
    log(f"merge_v_up W={W} T={T} H={H}")
    outs_t, lses, valid = _random_partials(W, T, H, seed=W * 7 + T)
    rng = np.random.default_rng(3)
    wuv_t = _bf16_round(0.02 * rng.standard_normal((H, 512, 128)))
    wuv = to_f64(wuv_t)
    ref_y, ref_l = O.project_then_merge(to_f64(outs_t), lses.astype(np.float64), valid, wuv)
    ref_y2, _ = O.merge_then_project(to_f64(outs_t), lses.astype(np.float64), valid, wuv)
    assert np.allclose(ref_y, ref_y2, atol=1e-12)
    outs_p = outs_t.clone()
    for w in range(W):
        for t in range(T):
            if valid[w, t] <= 0:
                outs_p[w, t] = float("nan")
    y = torch.full((T, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    yl = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_merge_v_up_proj(outs_p.cuda(), torch.from_numpy(lses).cuda(), torch.from_numpy(valid).cuda(),
                            wuv_t.cuda(), y, yl)
    torch.cuda.synchronize()
    gy = to_f64(y)
    # rows with no taking-part rank project to exactly 0
    dead = valid.sum(axis=0) == 0
    assert np.all(gy[dead] == 0) and np.all(to_f64(yl)[dead] == -np.inf)
    check_proj(y[torch.from_numpy(~dead)], ref_y[~dead], f"merge_v_up W={W}")
    assert np.max(np.abs(to_f64(yl)[~dead] - ref_l[~dead])) <= 1e-3
    # Without counts the LSE decides: ranks that do not take part carry -inf
    # (and NaN partials, which must not reach the result).
    lses_m = lses.copy()
    lses_m[np.broadcast_to((valid <= 0)[:, :, None], lses.shape)] = -np.inf
    y2 = torch.full((T, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    yl2 = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_merge_v_up_proj(outs_p.cuda(), torch.from_numpy(lses_m).cuda(), None, wuv_t.cuda(), y2, yl2)
    torch.cuda.synchronize()
    assert torch.equal(y2, y) and torch.equal(yl2, yl), f"merge_v_up W={W} valid=None"


def test_merge_v_up_proj_hip_graph_replay():
    """mla_merge_v_up_proj captured alone in a HIP graph: every replay, with
    eager work and synchronisations between the replays, reproduces the eager
    result bit for bit."""
    W, T, H = 4, 70, 128
    outs_t, lses, valid = _random_partials(W, T, H, seed=91)
    rng = np.random.default_rng(5)
    wuv = _bf16_round(0.02 * rng.standard_normal((H, 512, 128))).cuda()
    d_outs, d_lses, d_valid = outs_t.cuda(), torch.from_numpy(lses).cuda(), torch.from_numpy(valid).cuda()
    y = torch.empty((T, H, 128), dtype=torch.bfloat16, device="cuda")
    yl = torch.empty((T, H), dtype=torch.float32, device="cuda")
    mla.mla_merge_v_up_proj(d_outs, d_lses, d_valid, wuv, y, yl)
    torch.cuda.synchronize()
    ref_y, ref_l = y.clone(), yl.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mla.mla_merge_v_up_proj(d_outs, d_lses, d_valid, wuv, y, yl, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mla.mla_merge_v_up_proj(d_outs, d_lses, d_valid, wuv, y, yl)
    for k in range(4):
        y.fill_(float("nan"))
        yl.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref_y) and torch.equal(yl, ref_l), f"replay {k}"
        del junk
