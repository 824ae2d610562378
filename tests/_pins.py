"""Checks that pin the fp64 oracle to facts outside itself.

Each check returns True when the oracle passes it.  The oracle tests assert that
every check passes; the mutation tests plant a plausible mistake in the oracle and
assert that at least one check then fails, which shows the checks can see it.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

from oracle import mla_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bits(x):
    """float64 -> bf16 bits by truncating float32 (inputs here are chosen bf16-exact)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16)


def _torch_widen(bits) -> np.ndarray:
    """bf16 storage bits -> float64 through torch's bfloat16 dtype (a library
    route independent of the oracle's own widening)."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


# bf16 bit patterns and the values the binary32 format gives them (bf16 is the
# upper half of an IEEE-754 binary32: sign, 8 exponent bits with bias 127, 7
# fraction bits): 1.0, -2.5, pi rounded to 8 significant bits, the smallest
# subnormal 2^-133, the smallest normal 2^-126, the largest finite
# (2 - 2^-7) * 2^127, +0, -0, +inf and -inf.
BF16_FIXED = [
    (0x3F80, 1.0), (0xC020, -2.5), (0x4049, 3.140625), (0x0001, 2.0 ** -133), (0x0080, 2.0 ** -126),
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127), (0x0000, 0.0), (0x8000, -0.0), (0x7F80, math.inf),
    (0xFF80, -math.inf), (0x3C00, 2.0 ** -7), (0x4300, 128.0), (0xBF81, -(1.0 + 2.0 ** -7)), (0xBF01, -0.50390625),
]


def check_bf16_widening() -> bool:
    """The oracle's exact widening of bf16 bits against fixed patterns whose
    values follow from the binary32 format (signs of zero included), NaN
    patterns staying NaN, and torch's bf16 dtype on every one of the 65536
    patterns."""
    bits = np.array([b for b, _ in BF16_FIXED], dtype=np.uint16)
    got = O.bf16_bits_to_f64(bits)
    for g, (b, want) in zip(got, BF16_FIXED):
        if not (g == want and np.signbit(g) == np.signbit(want)):
            return False
    if not np.all(np.isnan(O.bf16_bits_to_f64(np.array([0x7FC0, 0xFFC1, 0x7F81], dtype=np.uint16)))):
        return False
    every = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    a, b = O.bf16_bits_to_f64(every), _torch_widen(every)
    same = (a == b) | (np.isnan(a) & np.isnan(b))
    return bool(np.all(same) and np.array_equal(np.signbit(a), np.signbit(b)))


def check_v_up_proj_closed_forms(seed=7) -> bool:
    """y[t,h,:] = o[t,h,:] @ W_UV[h] against projections whose result is known
    without a matrix product: (i) W_UV[h] picks latent dim sel(h,n) into column
    n with a factor c_h of its own, so y[t,h,n] = c_h * o[t,h,sel(h,n)];
    (ii) two picks per column add; (iii) a rank-one W_UV[h] = u_h v_h^T gives
    y[t,h,:] = (sum_k o[t,h,k] u_h[k]) * v_h, the inner sum taken term by term."""
    rng = np.random.default_rng(seed)
    T, H, K, N = 3, 4, 512, 128
    o = rng.standard_normal((T, H, K))
    c = np.array([1.0, -2.0, 0.5, 3.0])
    sel = np.array([[(7 * n + 61 * h + 3) % K for n in range(N)] for h in range(H)])
    w = np.zeros((H, K, N))
    for h in range(H):
        for n in range(N):
            w[h, sel[h, n], n] = c[h]
    y = O.v_up_proj(o, w)
    if y.shape != (T, H, N):
        return False
    for t in range(T):
        for h in range(H):
            for n in range(N):
                if y[t, h, n] != c[h] * o[t, h, sel[h, n]]:
                    return False
    sel2 = (sel + 100) % K
    w2 = w.copy()
    for h in range(H):
        for n in range(N):
            w2[h, sel2[h, n], n] = 0.25
    y2 = O.v_up_proj(o, w2)
    for t in range(T):
        for h in range(H):
            for n in range(N):
                if abs(y2[t, h, n] - (c[h] * o[t, h, sel[h, n]] + 0.25 * o[t, h, sel2[h, n]])) > 1e-14:
                    return False
    u = rng.standard_normal((H, K))
    v = rng.standard_normal((H, N))
    y3 = O.v_up_proj(o, u[:, :, None] * v[:, None, :])
    for t in range(T):
        for h in range(H):
            dot = math.fsum(o[t, h, k] * u[h, k] for k in range(K))
            if not np.allclose(y3[t, h], dot * v[h], rtol=1e-12, atol=1e-12):
                return False
    return True


# FP8 E4M3 (OCP "fn") codes and the values the format gives them: sign bit,
# exponent bias 7, 3 fraction bits, subnormals f/8 * 2^-6, S.1111.111 NaN.
FP8_FIXED = [
    (0x38, 1.0), (0xB8, -1.0), (0x40, 2.0), (0x3C, 1.5), (0x30, 0.5), (0x7E, 448.0), (0xFE, -448.0),
    (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x00, 0.0), (0x80, -0.0), (0x77, 240.0),
    (0x4D, 6.5), (0x29, 0.28125),
]


def _torch_widen_fp8(codes) -> np.ndarray:
    """E4M3 codes -> float64 through torch's float8_e4m3fn dtype."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def check_fp8_widening() -> bool:
    """The oracle's E4M3 decoding against fixed codes, both NaN codes, and
    torch's float8_e4m3fn on all 256 codes; positive codes are increasing."""
    got = O.fp8_e4m3_bits_to_f64(np.array([c for c, _ in FP8_FIXED], dtype=np.uint8))
    for g, (c, want) in zip(got, FP8_FIXED):
        if not (g == want and np.signbit(g) == np.signbit(want)):
            return False
    if not np.all(np.isnan(O.fp8_e4m3_bits_to_f64(np.array([0x7F, 0xFF], dtype=np.uint8)))):
        return False
    every = np.arange(256).astype(np.uint8)
    a, b = O.fp8_e4m3_bits_to_f64(every), _torch_widen_fp8(every)
    num = ~np.isnan(b)                       # a NaN's sign carries nothing
    if not (np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[num], b[num])
            and np.array_equal(np.signbit(a[num]), np.signbit(b[num]))):
        return False
    return bool(np.all(np.diff(a[:0x7F]) > 0))


def check_fp8_decode(seed=10) -> bool:
    """Decode over an FP8 cache: (i) against torch SDPA on the values torch's
    float8_e4m3fn dtype gives the codes times the scale; (ii) with a power-of-two
    scale the values are bf16-exact, and the result equals the decode of the
    same values stored as bf16; (iii) q = 0 gives the mean of code * scale."""
    rng = np.random.default_rng(seed)
    scale = 1 / math.sqrt(192)
    for (S, Q, H, W, ks) in [(9, 3, 2, 2, 0.0137), (13, 4, 3, 1, 0.05), (20, 2, 2, 3, 1.7)]:
        codes = rng.integers(0, 256, size=(S, 576)).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x3A           # no NaN codes in the rows
        qn = _bits(rng.standard_normal((Q, H, 512)).astype(np.float32))
        qp = _bits(rng.standard_normal((Q, H, 64)).astype(np.float32))
        kv = _torch_widen_fp8(codes) * ks
        q = torch.from_numpy(np.concatenate([_torch_widen(qn), _torch_widen(qp)], axis=-1)).permute(1, 0, 2)
        for r in range(W):
            out, lse = O.decode_partial([S], [0, Q], qn, qp, lambda b: codes, scale, W, r, kv_scale=ks)
            mask = torch.from_numpy(O.dense_mask(S, Q, W, r))
            ne = mask.any(dim=1).numpy()
            ref = torch.nn.functional.scaled_dot_product_attention(
                q.unsqueeze(0), torch.from_numpy(kv).expand(1, H, S, 576), torch.from_numpy(kv[:, :512]).expand(1, H, S, 512),
                attn_mask=mask.expand(1, H, Q, S), scale=scale)[0].permute(1, 0, 2).numpy()
            if not np.allclose(out[ne], ref[ne], rtol=1e-12, atol=1e-12):
                return False
        # power-of-two scale: bf16-exact values, same result as a bf16 cache
        bf = _bits((_torch_widen_fp8(codes) * 0.125).astype(np.float32))
        o8, l8 = O.decode_partial([S], [0, Q], qn, qp, lambda b: codes, scale, 1, 0, kv_scale=0.125)
        o16, l16 = O.decode_partial([S], [0, Q], qn, qp, lambda b: bf, scale, 1, 0)
        if not (np.array_equal(o8, o16) and np.array_equal(l8, l16)):
            return False
        # q = 0: every visible key weighs the same
        z = np.zeros_like(qn)
        zp = np.zeros_like(qp)
        oz, lz = O.decode_partial([S], [0, Q], z, zp, lambda b: codes, scale, 1, 0, kv_scale=ks)
        for i in range(Q):
            n = S - Q + i + 1
            if not (np.allclose(oz[i], kv[:n, :512].mean(axis=0)[None], atol=1e-12)
                    and np.allclose(lz[i], math.log(n), atol=1e-14)):
                return False
    return True


def load_worked_masks():
    out = []
    with open(os.path.join(GOLDEN, "pr24453_worked_masks.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, W, r, keys, rows = line.split()
            out.append(dict(name=name, W=int(W), r=0 if r == "-" else int(r),
                            keys=[int(k) for k in keys.split(",")],
                            rows=[[c == "1" for c in row] for row in rows.split(",")]))
    return out


def check_worked_masks() -> bool:
    """The oracle's masks and counts reproduce the page's 6-key, 4-row, dcp=2 matrices."""
    S, Q = 6, 4
    for m in load_worked_masks():
        W, r = m["W"], m["r"]
        dense = O.dense_mask(S, Q, W, r)
        # the page lists only the keys this rank holds, in column order
        if [k for k in range(S) if k % W == r] != m["keys"]:
            return False
        sub = dense[:, m["keys"]]
        want = np.array(m["rows"])
        if sub.shape != want.shape or not np.array_equal(sub, want):
            return False
        # closed-form counts and explicit visible sets agree with the matrix rows
        rows = O.query_rows([S], [0, Q])
        for i, (_, _, p) in enumerate(rows):
            if O.visible_count(p, W, r) != int(want[i].sum()):
                return False
            if O.visible_keys(p, W, r) != [k for k, on in zip(m["keys"], want[i]) if on]:
                return False
        if list(O.row_counts([S], [0, Q], W, r)) != [int(x) for x in want.sum(axis=1)]:
            return False
    return True


def check_ab_example() -> bool:
    """dcp=2, query_len=2 over a 2-token request: rank 0 sees {1,1}, rank 1 sees {0,1}."""
    with open(os.path.join(GOLDEN, "pr24453_ab_example.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            r, counts = line.split()
            want = [int(c) for c in counts.split(",")]
            if list(O.row_counts([2], [0, 2], 2, int(r))) != want:
                return False
    return True


def check_counts_bruteforce(max_w=8, max_s=80, max_q=9) -> bool:
    """Closed-form counts == explicit enumeration, and the shards partition the keys."""
    for W in range(1, max_w + 1):
        for S in range(1, max_s):
            for Q in range(1, min(max_q, S) + 1):
                rows = O.query_rows([S], [0, Q])
                tot = np.zeros(Q, dtype=np.int64)
                for r in range(W):
                    dm = O.dense_mask(S, Q, W, r) if (S < 24 and Q < 5) else None
                    for i, (_, _, p) in enumerate(rows):
                        n = O.visible_count(p, W, r)
                        if n != sum(1 for k in range(p + 1) if k % W == r):
                            return False
                        if dm is not None and n != int(dm[i].sum()):
                            return False
                        tot[i] += n
                    if O.shard_length(S, W, r) != len(range(r, S, W)):
                        return False
                if list(tot) != [p + 1 for (_, _, p) in rows]:
                    return False
    return True


def _rand_case(rng, S, Q, H, zero_q=False):
    kv = rng.standard_normal((S, 576)).astype(np.float32)
    qn = rng.standard_normal((Q, H, 512)).astype(np.float32)
    qp = rng.standard_normal((Q, H, 64)).astype(np.float32)
    if zero_q:
        qn[:] = 0
        qp[:] = 0
    return _bits(kv), _bits(qn), _bits(qp)


def check_against_sdpa(seed=0) -> bool:
    """Unsharded and sharded oracle outputs == torch SDPA (fp64, CPU, explicit mask)."""
    rng = np.random.default_rng(seed)
    scale = 1 / math.sqrt(192)
    for (S, Q, H, W) in [(6, 4, 3, 1), (9, 3, 2, 2), (13, 5, 4, 3), (31, 1, 2, 1), (40, 7, 2, 4)]:
        kvb, qnb, qpb = _rand_case(rng, S, Q, H)
        # inputs widened by torch's own bf16 dtype, not by the oracle's widening
        kv = _torch_widen(kvb)
        q = np.concatenate([_torch_widen(qnb), _torch_widen(qpb)], axis=-1)  # [Q,H,576]
        for r in range(W):
            out, lse = O.decode_partial([S], [0, Q], qnb, qpb, lambda b: kvb, scale, W, r)
            mask = torch.from_numpy(O.dense_mask(S, Q, W, r))  # [Q, S]
            nonempty = mask.any(dim=1).numpy()
            qt = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)            # [1,H,Q,576]
            kt = torch.from_numpy(kv).expand(1, H, S, 576)
            vt = torch.from_numpy(kv[:, :512]).expand(1, H, S, 512)
            ref = torch.nn.functional.scaled_dot_product_attention(
                qt, kt, vt, attn_mask=mask.expand(1, H, Q, S), scale=scale)
            ref = ref[0].permute(1, 0, 2).numpy()                              # [Q,H,512]
            if not np.allclose(out[nonempty], ref[nonempty], rtol=1e-12, atol=1e-12):
                return False
            if np.any(out[~nonempty] != 0) or np.any(lse[~nonempty] != -np.inf):
                return False
            # LSE through SDPA: with one-hot values SDPA returns the softmax weights
            # w[j]; then lse = score[j] - ln w[j] for any visible key j.
            eye = torch.eye(S, dtype=torch.float64).expand(1, H, S, S)
            wts = torch.nn.functional.scaled_dot_product_attention(
                qt, kt, eye, attn_mask=mask.expand(1, H, Q, S), scale=scale)[0].numpy()  # [H,Q,S]
            scores = scale * np.einsum("qhd,sd->hqs", q, kv)
            for i in np.nonzero(nonempty)[0]:
                j = int(np.nonzero(mask[i].numpy())[0][-1])
                want = scores[:, i, j] - np.log(wts[:, i, j])
                if not np.allclose(lse[i], want, rtol=0, atol=1e-10):
                    return False
    return True


def check_closed_forms(seed=1) -> bool:
    """q = 0 gives lse = ln(count) and the mean of the visible latents; one key gives c_0."""
    rng = np.random.default_rng(seed)
    scale = 1 / math.sqrt(192)
    S, Q, H, W = 23, 4, 2, 3
    kvb, qnb, qpb = _rand_case(rng, S, Q, H, zero_q=True)
    kv = _torch_widen(kvb)
    for r in range(W):
        out, lse = O.decode_partial([S], [0, Q], qnb, qpb, lambda b: kvb, scale, W, r)
        for i in range(Q):
            p = S - Q + i
            keys = [k for k in range(p + 1) if k % W == r]
            if not np.allclose(lse[i], math.log(len(keys)), atol=1e-14):
                return False
            if not np.allclose(out[i], kv[keys, :512].mean(axis=0)[None], atol=1e-13):
                return False
    # one visible key: out is that key's latent exactly, lse its scaled score
    kvb, qnb, qpb = _rand_case(rng, 1, 1, H)
    out, lse = O.decode_partial([1], [0, 1], qnb, qpb, lambda b: kvb, scale, 1, 0)
    kv = _torch_widen(kvb)
    s0 = scale * (_torch_widen(qnb[0]) @ kv[0, :512] + _torch_widen(qpb[0]) @ kv[0, 512:])
    return np.array_equal(out[0], np.repeat(kv[:1, :512], H, axis=0)) and np.allclose(lse[0], s0, atol=1e-13)


def _sharded_case(rng, seq_lens, q_lens, H, W):
    qsl = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    T = int(qsl[-1])
    kvs = [_bits(rng.standard_normal((s, 576)).astype(np.float32)) for s in seq_lens]
    qnb = _bits(rng.standard_normal((T, H, 512)).astype(np.float32))
    qpb = _bits(rng.standard_normal((T, H, 64)).astype(np.float32))
    return qsl, kvs, qnb, qpb


def check_merge_equals_unsharded(seed=2) -> bool:
    """merge over the W shards' partials == attention over all keys (fp64 exact algebra)."""
    rng = np.random.default_rng(seed)
    scale = 1 / math.sqrt(192)
    for seq_lens, q_lens, H, W in [([6, 9], [4, 3], 2, 2), ([2, 3, 17], [2, 3, 5], 2, 4),
                                   ([12, 30], [1, 6], 3, 8), ([5], [5], 1, 3)]:
        qsl, kvs, qnb, qpb = _sharded_case(rng, seq_lens, q_lens, H, W)
        full, full_lse = O.decode_partial(seq_lens, qsl, qnb, qpb, lambda b: kvs[b], scale, 1, 0)
        parts = [O.decode_partial(seq_lens, qsl, qnb, qpb, lambda b: kvs[b], scale, W, r)
                 for r in range(W)]
        outs = np.stack([p[0] for p in parts])
        lses = np.stack([p[1] for p in parts])
        valid = np.stack([O.row_counts(seq_lens, qsl, W, r) for r in range(W)])
        for v in (valid, None):
            m, ml = O.lse_merge(outs, lses, v)
            if not (np.allclose(m, full, atol=1e-12) and np.allclose(ml, full_lse, atol=1e-12)):
                return False
    return True


def check_merge_identities(seed=3) -> bool:
    """Single valid shard is the identity; W copies add ln W; shard order is irrelevant;
    invalid partials are ignored whatever they hold."""
    rng = np.random.default_rng(seed)
    W, T, H, D = 4, 3, 2, 8
    outs = rng.standard_normal((W, T, H, D))
    lses = rng.standard_normal((W, T, H)) * 3
    valid = np.ones((W, T), dtype=np.int32)
    m1, l1 = O.lse_merge(outs[:1], lses[:1], valid[:1])
    if not (np.allclose(m1, outs[0], atol=1e-15) and np.allclose(l1, lses[0], atol=1e-15)):
        return False
    same = np.repeat(outs[:1], W, axis=0)
    same_l = np.repeat(lses[:1], W, axis=0)
    m2, l2 = O.lse_merge(same, same_l, valid)
    if not (np.allclose(m2, outs[0], atol=1e-13) and np.allclose(l2, lses[0] + math.log(W), atol=1e-13)):
        return False
    perm = rng.permutation(W)
    m3, l3 = O.lse_merge(outs, lses, valid)
    m4, l4 = O.lse_merge(outs[perm], lses[perm], valid[perm])
    if not (np.allclose(m3, m4, atol=1e-13) and np.allclose(l3, l4, atol=1e-13)):
        return False
    # poison shard 1 of row 0 and mark it invalid: result equals merging the rest
    po, pl = outs.copy(), lses.copy()
    po[1, 0] = np.nan
    pl[1, 0] = np.nan
    v = valid.copy()
    v[1, 0] = 0
    m5, l5 = O.lse_merge(po, pl, v)
    keep = [0, 2, 3]
    m6, l6 = O.lse_merge(outs[keep][:, :1], lses[keep][:, :1], valid[keep][:, :1])
    if not (np.allclose(m5[0], m6[0], atol=1e-13) and np.allclose(l5[0], l6[0], atol=1e-13)):
        return False
    # a row with no valid shard: out 0, lse -inf
    v0 = valid.copy()
    v0[:, 2] = 0
    m7, l7 = O.lse_merge(po, pl, v0)
    if np.any(m7[2] != 0) or np.any(l7[2] != -np.inf):
        return False
    # hand-computed 2-shard case: lse_w = ln 1, ln 3 -> weights 1/4, 3/4, LSE = ln 4
    o2 = np.array([[[[1.0, 0.0]]], [[[0.0, 1.0]]]])
    l2w = np.log(np.array([[[1.0]], [[3.0]]]))
    m8, l8 = O.lse_merge(o2, l2w, None)
    return np.allclose(m8[0, 0], [0.25, 0.75], atol=1e-15) and abs(l8[0, 0] - math.log(4)) < 1e-15


def check_wuv_commutes(seed=4) -> bool:
    """merge-then-project == project-then-merge, and the projection is o @ W_UV[h]."""
    rng = np.random.default_rng(seed)
    W, T, H = 3, 4, 2
    outs = rng.standard_normal((W, T, H, 512))
    lses = rng.standard_normal((W, T, H))
    valid = (rng.random((W, T)) > 0.3).astype(np.int32)
    valid[0] = 1
    w_uv = 0.02 * rng.standard_normal((H, 512, 128))
    a, la = O.merge_then_project(outs, lses, valid, w_uv)
    b, lb = O.project_then_merge(outs, lses, valid, w_uv)
    if not (np.allclose(a, b, atol=1e-12) and np.array_equal(la, lb)):
        return False
    y = O.v_up_proj(outs[0], w_uv)
    return np.allclose(y[1, 1], outs[0, 1, 1] @ w_uv[1], atol=1e-13)


def _dealt_holders(S: int, W: int, I: int) -> list[int]:
    """Shard of each of the tokens 0..S-1 when runs of I consecutive tokens are
    dealt to the shards 0, 1, .., W-1, 0, .. in turn (simulated with counters)."""
    out, cur, used = [], 0, 0
    for _ in range(S):
        if used == I:
            cur, used = (cur + 1) % W, 0
        out.append(cur)
        used += 1
    return out


def check_runs_bruteforce(max_w=5, max_i=7, max_s=70) -> bool:
    """Run-dealt layout (runs of I tokens per shard): holder, visible keys, counts,
    local indices and shard lengths == a simulation of the dealing; the shards
    partition the keys; I = 1 is the interleaved p mod W layout; with I = page
    size every page sits whole on one shard, consecutive pages on consecutive
    shards."""
    for W in range(1, max_w + 1):
        for I in range(1, max_i + 1):
            hold = _dealt_holders(max_s, W, I)
            for k in range(max_s):
                if O.holder(k, W, I) != hold[k]:
                    return False
                if O.local_index(k, W, I) != sum(1 for j in range(k) if hold[j] == hold[k]):
                    return False
                if I == 1 and hold[k] != k % W:
                    return False
            for p in range(max_s):
                tot = 0
                for r in range(W):
                    keys = [k for k in range(p + 1) if hold[k] == r]
                    if O.visible_keys(p, W, r, I) != keys or O.visible_count(p, W, r, I) != len(keys):
                        return False
                    if O.shard_length(p + 1, W, r, I) != len(keys):
                        return False
                    tot += len(keys)
                if tot != p + 1:
                    return False
    for P, W in ((4, 3), (16, 2)):
        hold = _dealt_holders(8 * P, W, P)
        for g in range(8):
            if set(hold[g * P:(g + 1) * P]) != {g % W}:
                return False
    for S, Q, W, I in ((13, 4, 2, 3), (20, 2, 3, 4), (9, 9, 4, 2)):
        rows = O.query_rows([S], [0, Q])
        for r in range(W):
            dm = O.dense_mask(S, Q, W, r, I)
            if [int(x) for x in dm.sum(axis=1)] != [O.visible_count(p, W, r, I) for (_, _, p) in rows]:
                return False
    return True


def check_runs_merge_equals_unsharded(seed=5) -> bool:
    """Run-dealt layout: the merge of the W shards' partials == attention over all keys."""
    rng = np.random.default_rng(seed)
    scale = 1 / math.sqrt(192)
    for seq_lens, q_lens, H, W, I in [([7, 19], [4, 3], 2, 2, 3), ([2, 3, 40], [2, 3, 5], 2, 4, 16),
                                      ([33], [6], 1, 3, 5), ([12, 30], [1, 6], 2, 8, 2)]:
        qsl, kvs, qnb, qpb = _sharded_case(rng, seq_lens, q_lens, H, W)
        full, full_lse = O.decode_partial(seq_lens, qsl, qnb, qpb, lambda b: kvs[b], scale, 1, 0)
        parts = [O.decode_partial(seq_lens, qsl, qnb, qpb, lambda b: kvs[b], scale, W, r, I=I)
                 for r in range(W)]
        outs = np.stack([p[0] for p in parts])
        lses = np.stack([p[1] for p in parts])
        valid = np.stack([O.row_counts(seq_lens, qsl, W, r, I) for r in range(W)])
        for v in (valid, None):
            m, ml = O.lse_merge(outs, lses, v)
            if not (np.allclose(m, full, atol=1e-12) and np.allclose(ml, full_lse, atol=1e-12)):
                return False
    return True


def check_a2a_pack_combine(seed=6) -> bool:
    """Projected exchange: every rank packs, the all-to-all hands destination q
    the slice q of every rank, and q's combine == the head slice q of
    project-then-merge (itself pinned to merge-then-project); rows with valid
    count 0 hold NaN and never reach the result."""
    rng = np.random.default_rng(seed)
    for W, T, H in ((4, 5, 8), (2, 3, 4), (8, 2, 16)):
        outs = rng.standard_normal((W, T, H, 512))
        lses = rng.standard_normal((W, T, H)) * 3
        valid = rng.integers(0, 3, size=(W, T))
        valid[:, 0] = 0                      # a row no rank takes part in
        valid[0, 1] = 5
        for w in range(W):
            for t in range(T):
                if valid[w, t] == 0:
                    outs[w, t] = np.nan
                    lses[w, t] = np.nan
        wuv = rng.standard_normal((H, 512, 128)) * 0.02
        Hs = H // W
        sends = [O.a2a_pack(outs[r], lses[r], valid[r], wuv, W) for r in range(W)]
        ref_y, ref_l = O.project_then_merge(np.nan_to_num(outs), np.nan_to_num(lses), valid, wuv)
        for q in range(W):
            recv_y = np.stack([sends[r][0][q] for r in range(W)])
            recv_l = np.stack([sends[r][1][q] for r in range(W)])
            y, l = O.a2a_combine(recv_y, recv_l)
            if not (np.allclose(y, ref_y[:, q * Hs:(q + 1) * Hs], atol=1e-12)
                    and np.array_equal(np.isinf(l), np.isinf(ref_l[:, q * Hs:(q + 1) * Hs]))
                    and np.allclose(l[np.isfinite(l)], ref_l[:, q * Hs:(q + 1) * Hs][np.isfinite(l)], atol=1e-12)):
                return False
        # one rank, one slice: the pack is the plain projection of the valid rows
        y0, l0 = O.a2a_pack(np.nan_to_num(outs[0]), np.nan_to_num(lses[0]), None, wuv, 1)
        if not np.allclose(y0[0], np.einsum("thk,hkn->thn", np.nan_to_num(outs[0]), wuv), atol=1e-12):
            return False
    return True


def check_two_stage_keys(max_w=5, max_i=4, max_s=40, max_q=7) -> bool:
    """Two-stage split: the context count is the size of the explicit context set;
    for every row the shards' context keys and the row's query-part keys
    partition 0..p exactly once; the context part is the same for every row of a
    request."""
    for W in range(1, max_w + 1):
        for I in range(1, max_i + 1):
            for S in range(1, max_s):
                for Q in range(1, min(max_q, S) + 1):
                    ctx = []
                    for r in range(W):
                        keys = O.context_keys(S, Q, W, r, I)
                        if keys != [k for k in range(S - Q) if (k // I) % W == r]:
                            return False
                        if O.context_count(S, Q, W, r, I) != len(keys):
                            return False
                        ctx += keys
                    if sorted(ctx) != list(range(S - Q)):
                        return False
                    for i in range(Q):
                        p = S - Q + i
                        qk = O.query_part_keys(S, Q, i)
                        if sorted(ctx + qk) != list(range(p + 1)) or len(qk) != i + 1:
                            return False
    return True


def check_two_stage_against_sdpa(seed=8) -> bool:
    """Stage 1 on each shard == torch SDPA without a mask over that shard's
    context keys; stage 2 == torch SDPA with is_causal=True over the request's
    Q query tokens' own KV (square Q x Q causal: row i sees keys 0..i)."""
    rng = np.random.default_rng(seed)
    scale = 1 / math.sqrt(192)
    for (S, Q, H, W, I) in [(9, 3, 2, 2, 1), (13, 5, 3, 3, 1), (20, 4, 2, 2, 3), (6, 6, 2, 2, 1), (7, 1, 2, 4, 1)]:
        kvb, qnb, qpb = _rand_case(rng, S, Q, H)
        kv = _torch_widen(kvb)
        q = torch.from_numpy(np.concatenate([_torch_widen(qnb), _torch_widen(qpb)], axis=-1)).permute(1, 0, 2)
        qsl = [0, Q]
        for r in range(W):
            out, lse = O.decode_context_part([S], qsl, qnb, qpb, lambda b: kvb, scale, W, r, I=I)
            keys = [k for k in range(S - Q) if (k // I) % W == r]
            if not keys:
                if np.any(out != 0) or np.any(lse != -np.inf):
                    return False
                continue
            kt = torch.from_numpy(kv[keys]).expand(H, len(keys), 576).unsqueeze(0)
            vt = torch.from_numpy(kv[keys, :512]).expand(H, len(keys), 512).unsqueeze(0)
            ref = torch.nn.functional.scaled_dot_product_attention(q.unsqueeze(0), kt, vt, scale=scale)[0]
            if not np.allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12):
                return False
        out, lse = O.decode_query_part([S], qsl, qnb, qpb, lambda b: kvb, scale)
        new = kv[S - Q:]
        kt = torch.from_numpy(new).expand(H, Q, 576).unsqueeze(0)
        vt = torch.from_numpy(new[:, :512]).expand(H, Q, 512).unsqueeze(0)
        ref = torch.nn.functional.scaled_dot_product_attention(q.unsqueeze(0), kt, vt, scale=scale, is_causal=True)[0]
        if not np.allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12):
            return False
        # one query row: the query part is that token's own row exactly, LSE its score
        if Q == 1:
            s0 = scale * (_torch_widen(qnb[0]) @ kv[S - 1, :512] + _torch_widen(qpb[0]) @ kv[S - 1, 512:])
            if not (np.array_equal(out[0], np.repeat(kv[S - 1:, :512], H, axis=0)) and np.allclose(lse[0], s0)):
                return False
    return True


def check_two_stage_merge(seed=9) -> bool:
    """merge(W context partials + the query partial) == unsharded attention ==
    merge of the one-stage shard partials (fp64), for several requests,
    layouts and query lengths, including requests with no context (Q = S)."""
    rng = np.random.default_rng(seed)
    scale = 1 / math.sqrt(192)
    for seq_lens, q_lens, H, W, I in [([6, 9], [4, 3], 2, 2, 1), ([2, 3, 17], [2, 3, 5], 2, 4, 1),
                                      ([30, 12], [6, 1], 2, 8, 2), ([5, 40], [5, 2], 1, 3, 4)]:
        qsl, kvs, qnb, qpb = _sharded_case(rng, seq_lens, q_lens, H, W)
        gkv = lambda b: kvs[b]
        full, full_lse = O.decode_partial(seq_lens, qsl, qnb, qpb, gkv, scale, 1, 0)
        ctx = [O.decode_context_part(seq_lens, qsl, qnb, qpb, gkv, scale, W, r, I=I) for r in range(W)]
        qp = O.decode_query_part(seq_lens, qsl, qnb, qpb, gkv, scale)
        outs = np.stack([c[0] for c in ctx] + [qp[0]])
        lses = np.stack([c[1] for c in ctx] + [qp[1]])
        m, ml = O.lse_merge(outs, lses, None)
        if not (np.allclose(m, full, atol=1e-12) and np.allclose(ml, full_lse, atol=1e-12)):
            return False
        one = [O.decode_partial(seq_lens, qsl, qnb, qpb, gkv, scale, W, r, I=I) for r in range(W)]
        m1, ml1 = O.lse_merge(np.stack([o[0] for o in one]), np.stack([o[1] for o in one]), None)
        if not (np.allclose(m, m1, atol=1e-12) and np.allclose(ml, ml1, atol=1e-12)):
            return False
    return True


ALL_CHECKS = [check_bf16_widening, check_fp8_widening, check_fp8_decode, check_worked_masks, check_ab_example, check_counts_bruteforce,
              check_against_sdpa, check_closed_forms, check_merge_equals_unsharded, check_merge_identities,
              check_wuv_commutes, check_v_up_proj_closed_forms, check_runs_bruteforce,
              check_runs_merge_equals_unsharded, check_a2a_pack_combine, check_two_stage_keys,
              check_two_stage_against_sdpa, check_two_stage_merge]
