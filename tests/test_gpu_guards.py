"""Guard bytes around every output and around the workspace: each entry point,
on each kernel path, writes only inside the buffers it is given.

This is the check an address sanitizer would make (none is available for GPU
code here).  Every output (and the decode's workspace) is a view into a larger
byte buffer whose 4 KiB before and after it hold a fixed pattern; after the
call the pattern must be intact, and the guarded outputs must equal, bit for
bit, what the same call writes into ordinary tensors.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from mla_decode_context_amd import binding as mla
from mla_decode_context_amd import workloads as WL
from mla_decode_context_amd.runner import DeviceWorkload
from tests._gpu import log, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]

GUARD = 4096          # bytes on each side; a multiple of 256 keeps the view aligned
PATTERN = 0xA5


class Guarded:
    """A tensor of `shape` and `dtype` inside a byte buffer with guards around it."""

    def __init__(self, shape, dtype, fill=None):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.n = n
        self.buf = torch.full((n + 2 * GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD:GUARD + n].view(dtype).view(*shape)
        if fill is not None:
            self.t.fill_(fill)

    def intact(self) -> bool:
        return bool((self.buf[:GUARD] == PATTERN).all()) and bool((self.buf[GUARD + self.n:] == PATTERN).all())


def _same(a, b) -> bool:
    return torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                       b.view(torch.uint8) if b.dtype != torch.uint8 else b)


CASES = [
    # name, seq_lens, query_lens, H, W, P, I, num_splits, workspace, fp8, fp32 partials
    ("h16_balanced", [300, 2, 1, 700, 65], [2, 1, 1, 3, 4], 16, 4, 16, 1, 0, True, False, False),
    ("h16_fixed_splits", [300, 2, 1, 700, 65], [2, 1, 1, 3, 4], 16, 4, 16, 1, 3, True, False, False),
    ("h16_unsplit", [40, 1, 130], [3, 1, 1], 16, 2, 64, 1, 1, False, False, False),
    ("h16_fp8_p7", [9, 2, 70, 33, 400], [3, 2, 1, 5, 2], 16, 3, 7, 1, 0, True, True, False),
    ("h16_fp32_partials", [300, 2, 1, 700, 65], [2, 1, 1, 3, 4], 16, 4, 16, 1, 0, True, False, True),
    ("h48_generic", [130, 64, 9, 2], [2, 1, 5, 2], 48, 3, 33, 1, 0, True, False, False),
    ("h128_ordered", [700, 90, 2, 1500, 3], [2, 1, 2, 4, 3], 128, 8, 64, 1, 0, True, False, False),
    ("h128_token_order", [700, 90, 2, 1500, 3], [2, 1, 2, 4, 3], 128, 8, 64, 1, 0, False, False, False),
    ("h128_split", [5000, 900, 3], [1, 2, 3], 128, 2, 64, 1, 4, True, False, False),
    ("h128_fp32_partials", [700, 90, 2, 1500, 3], [2, 1, 2, 4, 3], 128, 8, 64, 1, 0, True, False, True),
    ("h128_runs", [700, 64, 129, 5], [2, 2, 1, 3], 128, 4, 64, 64, 0, True, False, False),
    ("h64_ordered", [700, 90, 2, 1500, 3], [2, 1, 2, 4, 3], 64, 8, 64, 1, 0, True, False, False),
    ("h64_split_f32", [5000, 900, 3], [1, 2, 3], 64, 2, 64, 1, 4, True, False, True),
]


@pytest.mark.parametrize("name,S,Q,H,W,P,I,splits,use_ws,fp8,f32", CASES, ids=[c[0] for c in CASES])
def test_decode_writes_inside_its_buffers(name, S, Q, H, W, P, I, splits, use_ws, fp8, f32):
    log(f"guards decode {name}")
    kw = dict(kv_scale=0.37) if fp8 else {}
    wl = WL.make_custom(name, S, Q, H=H, W=W, P=P, seed=91, I=I, **kw)
    dw = DeviceWorkload(wl, num_splits=splits, partial_dtype=torch.float32 if f32 else None)
    ws_bytes = dw.workspace.numel() if (use_ws and dw.workspace is not None) else 0
    pdt = torch.float32 if f32 else torch.bfloat16
    for r in range(W):
        out = Guarded((wl.T, H, 512), pdt, fill=float("nan"))
        lse = Guarded((wl.T, H), torch.float32, fill=float("nan"))
        keys = Guarded((wl.T,), torch.int32, fill=-7)
        ws = None
        if ws_bytes:
            ws = Guarded((ws_bytes,), torch.uint8, fill=0)       # zero-filled before its first use
        mla.mla_decode_partial(dw.q_nope, dw.q_pe, dw.caches[r], dw.tables[r], dw.seq_lens, dw.qsl, W, r,
                               dw.scale, out.t, lse.t, max_query_len=dw.max_query_len,
                               max_seq_len=dw.max_seq_len, workspace=ws.t if ws else None, num_splits=splits,
                               cp_interleave=I, row_keys=keys.t, kv_scale=wl.kv_scale if fp8 else None)
        ref_keys = torch.full((wl.T,), -7, dtype=torch.int32, device="cuda")
        mla.mla_decode_partial(dw.q_nope, dw.q_pe, dw.caches[r], dw.tables[r], dw.seq_lens, dw.qsl, W, r,
                               dw.scale, dw.outs[r], dw.lses[r], max_query_len=dw.max_query_len,
                               max_seq_len=dw.max_seq_len, workspace=dw.workspace if ws_bytes else None,
                               num_splits=splits, cp_interleave=I, row_keys=ref_keys,
                               kv_scale=wl.kv_scale if fp8 else None)
        torch.cuda.synchronize()
        for g, what in ((out, "out"), (lse, "lse"), (keys, "row_keys")) + (((ws, "workspace"),) if ws else ()):
            assert g.intact(), f"{name} r={r}: a write outside {what}"
        assert _same(out.t, dw.outs[r]) and _same(lse.t, dw.lses[r]) and _same(keys.t, ref_keys), \
            f"{name} r={r}: the guarded call differs from the plain one"


def test_noalloc_decode_writes_inside_its_buffers():
    log("guards noalloc")
    wl = WL.make_custom("guards_noalloc", [700, 90, 2, 1500, 3], [2, 1, 2, 4, 3], H=128, W=4, P=64, seed=92)
    dw = DeviceWorkload(wl)
    for r in range(wl.W):
        out = Guarded((wl.T, 128, 512), torch.bfloat16, fill=float("nan"))
        lse = Guarded((wl.T, 128), torch.float32, fill=float("nan"))
        keys = Guarded((wl.T,), torch.int32, fill=-7)
        mla.mla_decode_partial_noalloc(dw.q_nope, dw.q_pe, dw.caches[r], dw.tables[r], dw.seq_lens, dw.qsl, wl.W, r,
                                       dw.scale, out.t, lse.t, max_query_len=dw.max_query_len,
                                       max_seq_len=dw.max_seq_len, row_keys=keys.t)
        dw.partial(r)
        torch.cuda.synchronize()
        assert out.intact() and lse.intact() and keys.intact(), f"noalloc r={r}"
        assert _same(out.t, dw.outs[r]) and _same(lse.t, dw.lses[r])


@pytest.mark.parametrize("name,S,Q,H,W,f32", [
    ("w3_h16", [90, 5, 33], [3, 1, 2], 16, 3, False),
    ("w8_h128", [3, 5, 700, 9], [2, 3, 4, 1], 128, 8, False),
    ("w13_h16", [40, 3, 100, 17], [2, 1, 3, 4], 16, 13, False),
    ("w4_h128_f32", [300, 17, 64, 2, 129], [2, 3, 1, 2, 4], 128, 4, True),
])
def test_merges_write_inside_their_buffers(name, S, Q, H, W, f32):
    log(f"guards merge {name}")
    wl = WL.make_custom(name, S, Q, H=H, W=W, P=16, seed=93, w_uv=True)
    dw = DeviceWorkload(wl, partial_dtype=torch.float32 if f32 else None)
    dw.step()
    dw.valid_counts()
    torch.cuda.synchronize()
    T = wl.T
    for valid in (dw.valid, None):
        out = Guarded((T, H, 512), torch.bfloat16, fill=float("nan"))
        out_l = Guarded((T, H), torch.float32, fill=float("nan"))
        ref = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
        ref_l = torch.empty((T, H), dtype=torch.float32, device="cuda")
        mla.mla_lse_merge(dw.outs, dw.lses, valid, out.t, out_l.t)
        mla.mla_lse_merge(dw.outs, dw.lses, valid, ref, ref_l)
        y = Guarded((T, H, 128), torch.bfloat16, fill=float("nan"))
        y_l = Guarded((T, H), torch.float32, fill=float("nan"))
        ref_y = torch.empty((T, H, 128), dtype=torch.bfloat16, device="cuda")
        ref_yl = torch.empty((T, H), dtype=torch.float32, device="cuda")
        mla.mla_merge_v_up_proj(dw.outs, dw.lses, valid, dw.w_uv, y.t, y_l.t)
        mla.mla_merge_v_up_proj(dw.outs, dw.lses, valid, dw.w_uv, ref_y, ref_yl)
        torch.cuda.synchronize()
        tag = f"{name} valid={'counts' if valid is not None else 'None'}"
        for g, what in ((out, "merge out"), (out_l, "merge lse"), (y, "merge+W_UV out"), (y_l, "merge+W_UV lse")):
            assert g.intact(), f"{tag}: a write outside {what}"
        assert _same(out.t, ref) and _same(out_l.t, ref_l) and _same(y.t, ref_y) and _same(y_l.t, ref_yl), tag


def test_exchange_writes_inside_its_buffers():
    log("guards exchange")
    W, H = 4, 128
    wl = WL.make_custom("guards_exchange", [300, 17, 64, 2, 129], [2, 3, 1, 2, 4], H=H, W=W, P=16, seed=94,
                        w_uv=True)
    dw = DeviceWorkload(wl)
    dw.step()
    dw.valid_counts()
    torch.cuda.synchronize()
    T, Hs = wl.T, H // W
    send = torch.empty((W, W, T, Hs, 128), dtype=torch.bfloat16, device="cuda")
    send_l = torch.empty((W, W, T, Hs), dtype=torch.float32, device="cuda")
    for r in range(W):
        gy = Guarded((W, T, Hs, 128), torch.bfloat16, fill=float("nan"))
        gl = Guarded((W, T, Hs), torch.float32, fill=float("nan"))
        mla.mla_dcp_a2a_pack(dw.outs[r], dw.lses[r], dw.valid[r], dw.w_uv, gy.t, gl.t, W)
        mla.mla_dcp_a2a_pack(dw.outs[r], dw.lses[r], dw.valid[r], dw.w_uv, send[r], send_l[r], W)
        torch.cuda.synchronize()
        assert gy.intact() and gl.intact(), f"pack r={r}"
        assert _same(gy.t, send[r]) and _same(gl.t, send_l[r]), f"pack r={r}"
    for q in range(W):
        out = Guarded((T, Hs, 128), torch.bfloat16, fill=float("nan"))
        out_l = Guarded((T, Hs), torch.float32, fill=float("nan"))
        ref = torch.empty((T, Hs, 128), dtype=torch.bfloat16, device="cuda")
        ref_l = torch.empty((T, Hs), dtype=torch.float32, device="cuda")
        mla.mla_dcp_a2a_combine(send[:, q], send_l[:, q], out.t, out_l.t)
        mla.mla_dcp_a2a_combine(send[:, q], send_l[:, q], ref, ref_l)
        torch.cuda.synchronize()
        assert out.intact() and out_l.intact(), f"combine q={q}"
        assert _same(out.t, ref) and _same(out_l.t, ref_l), f"combine q={q}"


def test_local_seqlens_writes_inside_its_buffers():
    log("guards local seqlens")
    wl = WL.make_custom("guards_seqlens", [700, 64, 129, 5, 1], [2, 2, 1, 3, 1], H=16, W=4, P=16, seed=95, I=16)
    dw = DeviceWorkload(wl)
    for r in range(wl.W):
        rs = Guarded((wl.T,), torch.int32, fill=-7)
        sl = Guarded((wl.B,), torch.int32, fill=-7)
        mla.mla_dcp_local_seqlens(dw.seq_lens, dw.qsl, wl.T, wl.W, r, row_seqlen=rs.t, shard_len=sl.t,
                                  cp_interleave=wl.I)
        torch.cuda.synchronize()
        assert rs.intact() and sl.intact(), f"local seqlens r={r}"
        assert bool((rs.t >= 0).all()) and bool((sl.t >= 0).all())
