"""Shared helpers for the GPU parity tests (compare HIP results with the oracle)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O

# Tolerances for bf16 inputs with fp32 accumulation: per-row outputs within
# max-abs 2e-2 and relative L2 5e-3 of the fp64 oracle, LSE within 1e-3.
OUT_MAX_ABS = 2e-2
OUT_REL_L2 = 5e-3
LSE_ABS = 1e-3

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def log(msg: str):
    print(msg, flush=True)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_rows(gpu_out, gpu_lse, ref_out, ref_lse, tag=""):
    """Compare per-row outputs and LSEs; rows the oracle calls empty must be exact."""
    go = to_f64(gpu_out) if isinstance(gpu_out, torch.Tensor) else gpu_out
    gl = to_f64(gpu_lse) if isinstance(gpu_lse, torch.Tensor) else gpu_lse
    ref_out = np.asarray(ref_out, dtype=np.float64)
    ref_lse = np.asarray(ref_lse, dtype=np.float64)
    assert go.shape == ref_out.shape, (tag, go.shape, ref_out.shape)
    empty = ~np.isfinite(ref_lse)
    if empty.any():
        assert np.all(gl[empty] == -np.inf), f"{tag}: empty rows must have lse = -inf"
        assert np.all(go[empty] == 0), f"{tag}: empty rows must have out = 0"
    ne = ~empty
    if not ne.any():
        return dict(max_abs=0.0, rel_l2=0.0, lse_abs=0.0)
    diff = go[ne] - ref_out[ne]
    stats = dict(max_abs=float(np.abs(diff).max()),
                 rel_l2=float(np.linalg.norm(diff) / max(np.linalg.norm(ref_out[ne]), 1e-300)),
                 lse_abs=float(np.abs(gl[ne] - ref_lse[ne]).max()))
    assert np.all(np.isfinite(go[ne])), f"{tag}: non-finite output"
    assert stats["max_abs"] <= OUT_MAX_ABS, (tag, stats)
    assert stats["rel_l2"] <= OUT_REL_L2, (tag, stats)
    assert stats["lse_abs"] <= LSE_ABS, (tag, stats)
    return stats


def check_proj(gpu_y, ref_y, tag=""):
    gy = to_f64(gpu_y)
    ref_y = np.asarray(ref_y, dtype=np.float64)
    diff = gy - ref_y
    stats = dict(max_abs=float(np.abs(diff).max()),
                 rel_l2=float(np.linalg.norm(diff) / max(np.linalg.norm(ref_y), 1e-300)))
    assert stats["max_abs"] <= OUT_MAX_ABS, (tag, stats)
    assert stats["rel_l2"] <= OUT_REL_L2, (tag, stats)
    return stats


def oracle_partials(wl, tokens, kv_bits=None):
    """Oracle partials of every rank for the listed tokens: out [W,n,H,512], lse [W,n,H]."""
    kv = kv_bits if kv_bits is not None else {}

    def gkv(b):
        if b not in kv:
            kv[b] = wl.global_kv(b)
        return kv[b]

    parts = [O.decode_partial(wl.seq_lens, wl.query_start_loc, wl.q_nope, wl.q_pe, gkv, wl.scale,
                              wl.W, r, tokens=tokens, I=wl.I) for r in range(wl.W)]
    return np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts])


def oracle_unsharded(wl, tokens, kv_bits=None):
    kv = kv_bits if kv_bits is not None else {}

    def gkv(b):
        if b not in kv:
            kv[b] = wl.global_kv(b)
        return kv[b]

    return O.decode_partial(wl.seq_lens, wl.query_start_loc, wl.q_nope, wl.q_pe, gkv, wl.scale, 1, 0,
                            tokens=tokens)


def oracle_valid(wl, tokens):
    return np.stack([O.row_counts(wl.seq_lens, wl.query_start_loc, wl.W, r, wl.I)[tokens] for r in range(wl.W)])


def sample_tokens(wl, n_random=12, seed=123, extra_requests=()):
    """First/last token, first/last row of every listed request, plus seeded random tokens."""
    qsl = wl.query_start_loc
    picks = {0, wl.T - 1}
    for b in extra_requests:
        if qsl[b + 1] > qsl[b]:
            picks.update({int(qsl[b]), int(qsl[b + 1]) - 1})
    rng = np.random.default_rng(seed)
    picks.update(int(x) for x in rng.integers(0, wl.T, size=n_random))
    return sorted(picks)
