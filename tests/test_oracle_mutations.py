"""Plant plausible mistakes in the oracle (on the CPU) and check the pins see them.

Each mutant replaces one oracle function with a wrong variant; at least one pin
must then fail.  This guards the pins themselves against being too weak.
"""
import math

import numpy as np
import pytest

from oracle import mla_oracle as O
from tests import _pins


def _count_drop_plus_one(p, W, r, I=1):     # forgets that key p itself is visible
    n = p - r
    return 0 if n <= 0 else (n + W - 1) // W


def _count_floor(p, W, r, I=1):             # floor instead of ceil
    n = p + 1 - r
    return 0 if n <= 0 else n // W


def _count_runs_unscaled_rank(p, W, r, I=1):  # shard r's run taken to start at position r, not rI
    rounds, m = divmod(p + 1, W * I)
    return rounds * I + min(max(m - r, 0), I)


def _holder_offset_in_run(k, W, I=1):        # deals by the offset inside the run
    return (k % I) % W if I > 1 else k % W


def _local_index_interleaved(k, W, I=1):     # local index as if the layout were interleaved
    return k // W


_real_pack = O.a2a_pack


def _pack_interleaved_heads(o_r, lse_r, valid_r, w_uv, W):   # destination q gets heads q, q+W, ...
    y, l = _real_pack(o_r, lse_r, valid_r, w_uv, W)
    T, H = np.asarray(lse_r).shape
    Hs = H // W
    perm = [h for q in range(W) for h in range(q, H, W)]     # head order the mutant sends
    flat_y = y.transpose(1, 0, 2, 3).reshape(T, H, -1)[:, np.argsort(perm)]
    flat_l = l.transpose(1, 0, 2).reshape(T, H)[:, np.argsort(perm)]
    return (flat_y.reshape(T, W, Hs, -1).transpose(1, 0, 2, 3), flat_l.reshape(T, W, Hs).transpose(1, 0, 2))


def _rows_top_left(seq_lens, qsl):          # query rows at the first Q positions
    rows = []
    for b in range(len(seq_lens)):
        for i in range(int(qsl[b + 1]) - int(qsl[b])):
            rows.append((b, i, i))
    return rows


def _keys_wrong_residue(p, W, r, I=1):      # shard r holds p mod W == W-1-r
    return [k for k in range(p + 1) if k % W == (W - 1 - r)]


_real_attend = O.attend


def _attend_no_pe(q_nope, q_pe, keys, scale):    # drops the rope term
    return _real_attend(q_nope, np.zeros_like(q_pe), keys, scale)


def _attend_double_scale(q_nope, q_pe, keys, scale):
    return _real_attend(q_nope, q_pe, keys, 2 * scale)


def _attend_log2(q_nope, q_pe, keys, scale):     # LSE in base 2
    out, lse = _real_attend(q_nope, q_pe, keys, scale)
    return out, lse / math.log(2)


def _merge_wrong_sign(outs, lses, valid=None):
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    W, T, H = lses.shape
    out = np.zeros(outs.shape[1:])
    lse = np.full((T, H), -np.inf)
    for t in range(T):
        for h in range(H):
            used = [w for w in range(W) if (valid[w][t] > 0 if valid is not None else np.isfinite(lses[w, t, h]))]
            if not used:
                continue
            m = max(lses[w, t, h] for w in used)
            total = m + math.log(sum(math.exp(lses[w, t, h] - m) for w in used))
            lse[t, h] = total
            out[t, h] = sum(math.exp(total - lses[w, t, h]) * outs[w, t, h] for w in used) / W
    return out, lse


def _vup_transposed(o, w_uv):               # uses W_UV[h]^T-like indexing
    return np.einsum("thk,hkn->thn", o, w_uv[:, :, ::-1])


def _vup_heads_swapped(o, w_uv):            # head h projected by W_UV of head H-1-h
    return np.einsum("thk,hkn->thn", o, w_uv[::-1])


def _vup_k_misindexed(o, w_uv):             # latent dim k paired with row 511-k of W_UV[h]
    return np.einsum("thk,hkn->thn", o, w_uv[:, ::-1, :])


def _vup_heads_rolled(o, w_uv):             # off by one head
    return np.einsum("thk,hkn->thn", o, np.roll(w_uv, 1, axis=0))


def _widen_as_fp16(bits):                   # reads the bits as IEEE half
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _widen_shift15(bits):                   # one bit too few in the shift
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
    return b.view(np.float32).astype(np.float64)


def _widen_flush_subnormals(bits):          # flushes subnormals to zero
    x = _real_widen(bits)
    return np.where(np.abs(x) < 2.0 ** -126, 0.0 * x, x)


_real_widen = O.bf16_bits_to_f64


def _fp8_bias8(bits):                        # the FNUZ exponent bias
    c = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    e, f = (c >> 3) & 15, (c & 7).astype(np.float64)
    v = np.where(e == 0, np.ldexp(f / 8.0, -7), np.ldexp(1.0 + f / 8.0, e - 8))
    return np.where(c >> 7, -v, v)


_real_fp8 = O.fp8_e4m3_bits_to_f64


def _fp8_subnormal_as_normal(bits):          # subnormals given an implicit leading one
    c = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    v = _real_fp8(bits)
    e, f = (c >> 3) & 15, (c & 7).astype(np.float64)
    return np.where(e == 0, np.where(c >> 7, -1.0, 1.0) * np.ldexp(1.0 + f / 8.0, -6), v)


def _kv_scale_ignored(rows, kv_scale=None):  # FP8 codes used without the cache's scale
    return O.bf16_bits_to_f64(rows) if kv_scale is None else _real_fp8(rows)


def _query_part_shifted(S, Q, i):            # the query part one position late
    return list(range(S - Q + 1, S - Q + i + 2))


def _query_part_exclusive(S, Q, i):          # a row does not see its own token
    return list(range(S - Q, S - Q + i))


def _context_includes_first_query(S, Q, W, r, I=1):   # context runs through the first query token
    return [k for k in range(S - Q + 1) if (k // I) % W == r]


def _context_count_interleaved_only(S, Q, W, r, I=1):  # ignores the run length
    n = S - Q
    return 0 if n <= r else (n - r + W - 1) // W


MUTANTS = [
    ("visible_count", _count_drop_plus_one),
    ("visible_count", _count_floor),
    ("query_rows", _rows_top_left),
    ("visible_keys", _keys_wrong_residue),
    ("visible_count", _count_runs_unscaled_rank),
    ("holder", _holder_offset_in_run),
    ("local_index", _local_index_interleaved),
    ("a2a_pack", _pack_interleaved_heads),
    ("attend", _attend_no_pe),
    ("attend", _attend_double_scale),
    ("attend", _attend_log2),
    ("lse_merge", _merge_wrong_sign),
    ("v_up_proj", _vup_transposed),
    ("v_up_proj", _vup_heads_swapped),
    ("v_up_proj", _vup_k_misindexed),
    ("v_up_proj", _vup_heads_rolled),
    ("bf16_bits_to_f64", _widen_as_fp16),
    ("bf16_bits_to_f64", _widen_shift15),
    ("bf16_bits_to_f64", _widen_flush_subnormals),
    ("fp8_e4m3_bits_to_f64", _fp8_bias8),
    ("fp8_e4m3_bits_to_f64", _fp8_subnormal_as_normal),
    ("kv_rows_to_f64", _kv_scale_ignored),
    ("query_part_keys", _query_part_shifted),
    ("query_part_keys", _query_part_exclusive),
    ("context_keys", _context_includes_first_query),
    ("context_count", _context_count_interleaved_only),
]


@pytest.mark.parametrize("name,fn", MUTANTS, ids=[f"{n}:{f.__name__}" for n, f in MUTANTS])
def test_pins_catch_mutant(monkeypatch, name, fn):
    monkeypatch.setattr(O, name, fn)
    results = {c.__name__: _safe(c) for c in _pins.ALL_CHECKS
               if c not in (_pins.check_counts_bruteforce, _pins.check_runs_bruteforce, _pins.check_two_stage_keys)}
    results["check_counts_bruteforce"] = _safe(lambda: _pins.check_counts_bruteforce(5, 30, 5))
    results["check_runs_bruteforce"] = _safe(lambda: _pins.check_runs_bruteforce(4, 5, 40))
    results["check_two_stage_keys"] = _safe(lambda: _pins.check_two_stage_keys(4, 3, 25, 5))
    assert not all(results.values()), f"no pin failed for mutant {name}:{fn.__name__}"


def test_pins_catch_projection_mutant(monkeypatch):
    # the projection only enters the commute check through v_up_proj's definition
    monkeypatch.setattr(O, "v_up_proj", _vup_transposed)
    assert not _pins.check_wuv_commutes()


def _safe(check):
    try:
        return bool(check())
    except Exception:
        return False
