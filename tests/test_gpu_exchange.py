"""GPU parity of the projected exchange of the merge (the part one GPU holds).

Every rank packs its partial (projected through W_UV, by destination head
slice), the all-to-all is stood in for by addressing: destination q reads slice
q of every rank's send buffer in place, through the combine's per-source
stride; the combine merges them.  Checked against the oracle's pack and
combine, against the head slice of project-then-merge, and against the fused
merge + W_UV call on the same partials.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from mla_decode_context_amd import binding as mla
from mla_decode_context_amd import workloads as WL
from mla_decode_context_amd.runner import DeviceWorkload
from oracle import mla_oracle as O
from tests._gpu import check_proj, log, needs_gpu, to_f64

pytestmark = [pytest.mark.gpu, needs_gpu]


def _exchange(dw, W, valid=True):
    T, H = dw.T, dw.H
    Hs = H // W
    send_y = torch.full((W, W, T, Hs, 128), float("nan"), dtype=torch.bfloat16, device="cuda")   # [src, dest, ...]
    send_l = torch.full((W, W, T, Hs), float("nan"), dtype=torch.float32, device="cuda")
    for r in range(W):
        mla.mla_dcp_a2a_pack(dw.outs[r], dw.lses[r], dw.valid[r] if valid else None, dw.w_uv, send_y[r], send_l[r], W)
    out = torch.full((W, T, Hs, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    out_l = torch.full((W, T, Hs), float("nan"), dtype=torch.float32, device="cuda")
    for q in range(W):
        mla.mla_dcp_a2a_combine(send_y[:, q], send_l[:, q], out[q], out_l[q])
    torch.cuda.synchronize()
    return send_y, send_l, out, out_l


@pytest.mark.parametrize("name,S,Q,H,W,I", [
    ("w4_h128", [300, 17, 64, 2, 129], [2, 3, 1, 2, 4], 128, 4, 1),
    ("w2_h16", [90, 5, 33], [3, 1, 2], 16, 2, 1),
    ("w8_h128_short", [3, 5, 700, 9], [2, 3, 4, 1], 128, 8, 1),
    ("w4_h128_pages", [400, 70], [2, 3], 128, 4, 64),
])
def test_pack_exchange_combine(name, S, Q, H, W, I):
    log(f"exchange {name}")
    wl = WL.make_custom(name, S, Q, H=H, W=W, P=16, seed=17, I=I, w_uv=True)
    dw = DeviceWorkload(wl)
    dw.outs.fill_(float("nan"))
    for r in range(W):
        dw.partial(r)
    dw.valid_counts()
    torch.cuda.synchronize()
    valid = dw.valid.cpu().numpy()
    # Rows a rank does not take part in are poisoned: the pack must not read them.
    for r in range(W):
        dead = torch.tensor(valid[r] == 0, device="cuda")
        dw.outs[r][dead] = float("nan")
        dw.lses[r][dead] = float("nan")
    wuv = O.bf16_bits_to_f64(wl.w_uv)
    Hs = H // W
    outs64, lses64 = to_f64(dw.outs), to_f64(dw.lses)
    send_y, send_l, out, out_l = _exchange(dw, W)
    for r in range(W):
        ref_y, ref_l = O.a2a_pack(np.nan_to_num(outs64[r]), np.nan_to_num(lses64[r]), valid[r], wuv, W)
        got_y = to_f64(send_y[r])
        err = np.abs(got_y - ref_y)
        assert np.all(err <= 1e-2 * np.maximum(1.0, np.abs(ref_y))), (name, r, float(err.max()))
        got_l = to_f64(send_l[r])
        assert np.array_equal(np.isinf(got_l), np.isinf(ref_l)) and np.allclose(got_l[np.isfinite(got_l)], ref_l[np.isfinite(ref_l)], atol=1e-5)
    # Receivers against the head slices of project-then-merge of the same partials.
    full_y, full_l = O.project_then_merge(np.nan_to_num(outs64), np.nan_to_num(lses64), valid, wuv)
    for q in range(W):
        check_proj(out[q], full_y[:, q * Hs:(q + 1) * Hs], f"{name} dest={q}")
        got_l = to_f64(out_l[q])
        ref_l = full_l[:, q * Hs:(q + 1) * Hs]
        assert np.array_equal(np.isinf(got_l), np.isinf(ref_l))
        assert np.max(np.abs(got_l[np.isfinite(got_l)] - ref_l[np.isfinite(ref_l)]), initial=0.0) <= 1e-3
    # ... and against the fused merge + W_UV on the device (merge first, then project).
    dw.merge_v_up()
    torch.cuda.synchronize()
    fused = to_f64(dw.out_proj)
    exch = np.concatenate([to_f64(out[q]) for q in range(W)], axis=1)
    assert np.max(np.abs(exch - fused)) <= 2e-2 and np.linalg.norm(exch - fused) <= 1e-2 * np.linalg.norm(fused)


def test_pack_without_counts_and_combine_identity():
    # Without counts a rank takes part iff its LSE is finite; one rank's slices
    # combined alone give back exactly what it packed.
    wl = WL.make_custom("ident", [40, 3], [2, 2], H=16, W=2, P=16, seed=19, w_uv=True)
    dw = DeviceWorkload(wl)
    for r in range(2):
        dw.partial(r)
    dw.valid_counts()
    _, _, out_a, out_la = _exchange(dw, 2, valid=True)
    send_y, send_l, out_b, out_lb = _exchange(dw, 2, valid=False)
    assert torch.equal(out_a, out_b) and torch.equal(out_la, out_lb)
    one = torch.empty_like(out_a[0])
    one_l = torch.empty_like(out_la[0])
    mla.mla_dcp_a2a_combine(send_y[1, 0:1], send_l[1, 0:1], one, one_l)
    torch.cuda.synchronize()
    fin = torch.isfinite(send_l[1, 0])
    assert torch.equal(one[fin], send_y[1, 0][fin]) and torch.equal(one_l[fin], send_l[1, 0][fin])
    assert torch.all(one[~fin] == 0) and torch.all(torch.isinf(one_l[~fin]))


@pytest.mark.parametrize("W,T,Hs", [(13, 37, 3), (9, 5, 16), (1, 20, 7)])
def test_combine_many_sources_padded(W, T, Hs):
    # More sources than one load batch (8), odd slice sizes, sources padded
    # apart in one allocation, and rows that some or all sources leave empty.
    rng = np.random.default_rng(W * 100 + T)
    pad = 3 * 128                                     # elements between a slice's end and the next
    buf = torch.full((W, T * Hs * 128 + pad), float("nan"), dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((W, T * Hs + 5), float("nan"), dtype=torch.float32, device="cuda")
    y = (rng.standard_normal((W, T, Hs, 128)) * 0.5).astype(np.float32)
    l = (rng.standard_normal((W, T, Hs)) * 4).astype(np.float32)
    l[rng.random((W, T, Hs)) < 0.3] = -np.inf
    l[:, 0, 0] = -np.inf                              # a row no source takes part in
    buf[:, :T * Hs * 128] = torch.tensor(y.reshape(W, -1)).to(torch.bfloat16).cuda()
    lbuf[:, :T * Hs] = torch.tensor(l.reshape(W, -1)).cuda()
    recv_y = buf[:, :T * Hs * 128].view(W, T, Hs, 128)
    recv_l = lbuf[:, :T * Hs].view(W, T, Hs)
    out = torch.empty((T, Hs, 128), dtype=torch.bfloat16, device="cuda")
    out_l = torch.empty((T, Hs), dtype=torch.float32, device="cuda")
    mla.mla_dcp_a2a_combine(recv_y, recv_l, out, out_l)
    torch.cuda.synchronize()
    ref_y, ref_l = O.a2a_combine(to_f64(recv_y), l.astype(np.float64))
    got_l = to_f64(out_l)
    assert np.array_equal(np.isinf(got_l), np.isinf(ref_l))
    assert np.max(np.abs(got_l[np.isfinite(got_l)] - ref_l[np.isfinite(ref_l)]), initial=0.0) <= 1e-4
    check_proj(out, ref_y, f"combine W={W}")
    assert torch.all(out[0, 0] == 0)


def test_hip_graph_replay_exchange():
    # Pack of every rank and combine of every destination captured in one HIP
    # graph; every replay (with eager work and synchronisation in between)
    # reproduces the eager result bit for bit.
    W = 4
    wl = WL.make_custom("graph", [300, 17, 64, 2, 129], [2, 3, 1, 2, 4], H=128, W=W, P=16, seed=23, w_uv=True)
    dw = DeviceWorkload(wl)
    for r in range(W):
        dw.partial(r)
    dw.valid_counts()
    torch.cuda.synchronize()
    T, Hs = dw.T, dw.H // W
    send_y = torch.zeros((W, W, T, Hs, 128), dtype=torch.bfloat16, device="cuda")
    send_l = torch.zeros((W, W, T, Hs), dtype=torch.float32, device="cuda")
    out = torch.zeros((W, T, Hs, 128), dtype=torch.bfloat16, device="cuda")
    out_l = torch.zeros((W, T, Hs), dtype=torch.float32, device="cuda")

    def exchange():
        for r in range(W):
            mla.mla_dcp_a2a_pack(dw.outs[r], dw.lses[r], dw.valid[r], dw.w_uv, send_y[r], send_l[r], W)
        for q in range(W):
            mla.mla_dcp_a2a_combine(send_y[:, q], send_l[:, q], out[q], out_l[q])

    exchange()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (send_y, send_l, out, out_l)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        exchange()             # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        exchange()
    for _ in range(3):
        for x in (send_y, send_l, out, out_l):
            x.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip((send_y, send_l, out, out_l), ref):
            assert torch.equal(x, y)
