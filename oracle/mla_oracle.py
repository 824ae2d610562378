"""fp64 CPU oracle for absorbed-MLA decode under decode context parallelism (DCP).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module; the product library never does, and
this module imports nothing from the product (it shares no kernels, helpers,
tables or constants with it).  It is the plain definition written out in fp64
with NumPy, slow on purpose and meant to be checked by eye against the pages:

* "[Attention] add DCP support for FLASH_ATTN_MLA backend" (vLLM PR #24453),
  review thread: the "Normal" causal mask with the query rows as the last tokens,
  and the "DCP Rank 0 / DCP Rank 1" interleaved masks (keys {0,2,4} and {1,3,5});
  the dcp=2, query_len=2 "AB" example where a row can have seqlen_k = 0.
* "vllm.v1.attention.backends.mla.flashattn_mla" API page, ``_forward_decode``:
  the absorbed form (q_pe against k_pe, q_nope against the latent c_kv, the
  latent as the value), one softmax scale, causal, the LSE returned per
  (token, head) in [B, H] order.
* "[Attention] DCP sparse MLA output-merge optimizations" (vLLM PR #48196):
  the exact LSE-weighted merge of the per-rank partials, per-row valid counts,
  and the W_UV projection that commutes with the merge.
* The same PR #24453 thread's alternative for query_len > 1: a two-stage
  decode, the context KV without a causal mask and the query KV with one,
  merged by LSE.

Readings where the pages are silent (all listed in the design notes):
``seq_lens`` holds the global total S_b including the request's query tokens;
query row i of a request with Q_b rows sits at global position S_b - Q_b + i;
the LSE is the natural log of the sum of exp(scaled score); an empty row has
output 0 and LSE -inf; a shard's partial counts as valid iff its per-row count
(or, without counts, its LSE) is positive (finite).

Parity of every function here is pinned by the CPU tests (worked masks printed on
the PR #24453 page, brute force, torch's SDPA, closed forms and the merge
identities); nothing in this file is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

D_LATENT = 512
D_ROPE = 64


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 storage bits (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def fp8_e4m3_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of FP8 E4M3 codes (uint8), the OCP "fn" variant: sign bit,
    4 exponent bits with bias 7, 3 fraction bits; exponent field 0 holds the
    subnormals f/8 * 2^-6; the code S.1111.111 is NaN and there are no
    infinities (largest finite 448).

    The pages give no convention for an FP8 latent cache (the "flashattn_mla"
    API page rejects an FP8 KV cache as unsupported).  Reading: each cached element is an
    E4M3 code, and the cache carries one fp32 scale; the element's value is
    code value * scale.
    """
    c = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    f = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(f / 8.0, -6), np.ldexp(1.0 + f / 8.0, e - 7))
    return np.where((e == 15) & (f == 7), np.nan, sign * mag)


def kv_rows_to_f64(rows: np.ndarray, kv_scale=None) -> np.ndarray:
    """Cache rows as stored -> float64 values: bf16 bits widened exactly, or
    (kv_scale given) FP8 E4M3 codes times the cache's scale."""
    if kv_scale is None:
        return bf16_bits_to_f64(rows)
    return fp8_e4m3_bits_to_f64(rows) * float(kv_scale)


# ---------------------------------------------------------------------------
# Where the query rows sit, and which keys each row sees on each shard
# ---------------------------------------------------------------------------

def query_rows(seq_lens, query_start_loc):
    """For every query token t: (request b, row i within b, global position p).

    PR #24453 thread, "Normal" mask: the Q query rows of a request are its last Q
    tokens, so row i of request b is at global position S_b - Q_b + i and sees
    keys 0..p (bottom-right causal alignment).
    """
    seq_lens = [int(s) for s in seq_lens]
    qsl = [int(x) for x in query_start_loc]
    rows = []
    for b in range(len(seq_lens)):
        q_b = qsl[b + 1] - qsl[b]
        for i in range(q_b):
            rows.append((b, i, seq_lens[b] - q_b + i))
    return rows


def holder(k: int, W: int, I: int = 1) -> int:
    """DCP shard that stores global token k.

    PR #24453 thread: with the interleaved layout token k lives on shard k mod W
    (key A on rank 0, B on rank 1, ...).  The same thread mentions the other
    layout, contiguous runs of tokens (whole pages) per shard; with runs of I
    tokens dealt to the shards in turn, token k lives on shard (k div I) mod W.
    I = 1 is the interleaved layout.
    """
    return (k // I) % W


def visible_keys(p: int, W: int, r: int, I: int = 1) -> list[int]:
    """Global positions a query row at position p attends to on shard r.

    PR #24453 thread, "DCP Rank 0/1" masks: shard r holds the keys of its own
    (holder(k) == r), and the causal rule keeps those at or before p.  Listed in
    ascending position, which is the shard-local order.
    """
    return [k for k in range(p + 1) if holder(k, W, I) == r]


def visible_count(p: int, W: int, r: int, I: int = 1) -> int:
    """Closed form of len(visible_keys(p, W, r, I)): the per-row, per-shard seqlen_k.

    The n = p + 1 positions 0..p hold n div (W*I) whole rounds of the shards'
    runs, I tokens of shard r each, and a last partial round of m = n mod (W*I)
    positions in which shard r's run covers positions rI .. rI + I - 1, i.e.
    min(max(m - rI, 0), I) of them.  With I = 1: ceil((p + 1 - r) / W) when
    p >= r, else 0.
    """
    n = p + 1
    if n <= 0:
        return 0
    rounds, m = divmod(n, W * I)
    return rounds * I + min(max(m - r * I, 0), I)


def local_index(k: int, W: int, I: int = 1) -> int:
    """Shard-local index of global token k on its holder: the number of the
    holder's tokens before k (whole rounds of I tokens, then the offset in the run)."""
    return (k // (W * I)) * I + k % I


def shard_length(S: int, W: int, r: int, I: int = 1) -> int:
    """Tokens of a request with S global tokens stored on shard r (= visible_count(S-1))."""
    return visible_count(S - 1, W, r, I) if S > 0 else 0


def dense_mask(S: int, Q: int, W: int = 1, r: int = 0, I: int = 1) -> np.ndarray:
    """Boolean [Q, S] mask over GLOBAL key positions, built entry by entry.

    mask[i, k] is True iff key k is causally visible to query row i (k <= S-Q+i)
    and key k is stored on shard r ((k div I) mod W == r).  With W = 1 this is the
    "Normal" matrix of the PR #24453 thread; with I = 1 its columns restricted to
    one shard's keys give the "DCP Rank r" matrices.
    """
    m = np.zeros((Q, S), dtype=bool)
    for i in range(Q):
        for k in range(S):
            m[i, k] = (k <= S - Q + i) and ((k // I) % W == r)
    return m


def row_counts(seq_lens, query_start_loc, W: int, r: int, I: int = 1) -> np.ndarray:
    """Per query token t, its seqlen_k on shard r (int32 [T])."""
    return np.array([visible_count(p, W, r, I) for (_, _, p) in query_rows(seq_lens, query_start_loc)],
                    dtype=np.int32)


def shard_lengths(seq_lens, W: int, r: int, I: int = 1) -> np.ndarray:
    """Per request, the number of its tokens stored on shard r (int32 [B])."""
    return np.array([shard_length(int(s), W, r, I) for s in seq_lens], dtype=np.int32)


# ---------------------------------------------------------------------------
# Attention of one query token over a set of keys
# ---------------------------------------------------------------------------

def attend(q_nope: np.ndarray, q_pe: np.ndarray, keys: np.ndarray, scale: float):
    """Absorbed-MLA attention of one query token (all heads) over the given key rows.

    q_nope [H,512], q_pe [H,64], keys [n,576] (c_kv | k_pe), all float64.
    Score of head h and key j: scale * (q_nope[h].c_kv[j] + q_pe[h].k_pe[j])
    (flashattn_mla page: q=q_pe against k=k_pe, q_v=q_nope against v=c_kv, one
    softmax_scale).  The value is c_kv itself.  Returns out [H,512] (softmax-
    weighted sum of c_kv) and lse [H] = ln sum_j exp(score).  With no keys the row
    is empty: out = 0, lse = -inf.
    """
    H = q_nope.shape[0]
    n = keys.shape[0]
    if n == 0:
        return np.zeros((H, D_LATENT)), np.full(H, -np.inf)
    c = keys[:, :D_LATENT]
    k_pe = keys[:, D_LATENT:]
    s = scale * (q_nope @ c.T + q_pe @ k_pe.T)          # [H, n]
    m = s.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    p = np.exp(s - lse[:, None])
    return p @ c, lse


def decode_partial(seq_lens, query_start_loc, q_nope_bits, q_pe_bits, global_kv, scale: float,
                   W: int = 1, r: int = 0, tokens=None, I: int = 1, kv_scale=None):
    """Shard r's partial attention for every query token (or the listed ones).

    ``global_kv(b)`` returns request b's global token rows [S_b, 576] as stored:
    bf16 bits, or FP8 E4M3 codes when ``kv_scale`` (the cache's scale) is given.
    Each row attends to visible_keys(p, W, r, I).  Returns out [n,H,512], lse [n,H]
    (float64) for the selected tokens in the order given.
    """
    rows = query_rows(seq_lens, query_start_loc)
    sel = range(len(rows)) if tokens is None else [int(t) for t in tokens]
    H = q_nope_bits.shape[1]
    outs = np.zeros((len(sel), H, D_LATENT))
    lses = np.zeros((len(sel), H))
    cache = {}
    for n_out, t in enumerate(sel):
        b, _, p = rows[t]
        if b not in cache:
            cache.clear()
            cache[b] = kv_rows_to_f64(global_kv(b), kv_scale)
        keys = cache[b][visible_keys(p, W, r, I)]
        outs[n_out], lses[n_out] = attend(bf16_bits_to_f64(q_nope_bits[t]),
                                          bf16_bits_to_f64(q_pe_bits[t]), keys, scale)
    return outs, lses


# ---------------------------------------------------------------------------
# The two-stage split of a decode with more than one query row
# ---------------------------------------------------------------------------
#
# PR #24453 review thread (youzhedian): with query_len > 1 the DCP decode can
# be run in two stages instead of with the interleaved mask -- the context KV
# with causal=False and the query KV with causal=True -- so that no backend
# needs a custom mask.  Reading: the context of a request is its tokens before
# its Q query tokens (global positions 0 .. S-Q-1); every query row sees all of
# them, and each DCP rank attends to the ones it stores.  The query KV is the
# request's own Q tokens (positions S-Q .. S-1), which a causal mask restricted
# to them makes row i see the first i+1 of; it is one dense block, attended
# once (not per rank).  The W context partials and the query partial merge by
# LSE into the unsharded result.

def context_keys(S: int, Q: int, W: int, r: int, I: int = 1) -> list[int]:
    """Global positions of the context part that shard r stores: the request's
    tokens before its Q query tokens.  Every query row of the request sees all
    of them (no causal mask inside the context)."""
    return [k for k in range(S - Q) if holder(k, W, I) == r]


def query_part_keys(S: int, Q: int, i: int) -> list[int]:
    """Global positions of the query part that query row i sees: the request's
    own query tokens S-Q .. S-Q+i (the causal mask among its Q tokens)."""
    return list(range(S - Q, S - Q + i + 1))


def context_count(S: int, Q: int, W: int, r: int, I: int = 1) -> int:
    """Closed form of len(context_keys(...)): what shard r stores of the first
    S - Q positions (the same for every query row of the request)."""
    return shard_length(S - Q, W, r, I)


def decode_context_part(seq_lens, query_start_loc, q_nope_bits, q_pe_bits, global_kv, scale: float,
                        W: int = 1, r: int = 0, tokens=None, I: int = 1, kv_scale=None):
    """Stage 1 on shard r: every query row attends, without a causal mask, to
    the context keys shard r stores.  Returns out [n,H,512], lse [n,H] (empty
    context: out 0, lse -inf)."""
    rows = query_rows(seq_lens, query_start_loc)
    qsl = [int(x) for x in query_start_loc]
    sel = range(len(rows)) if tokens is None else [int(t) for t in tokens]
    H = q_nope_bits.shape[1]
    outs = np.zeros((len(sel), H, D_LATENT))
    lses = np.zeros((len(sel), H))
    cache = {}
    for n_out, t in enumerate(sel):
        b, _, _ = rows[t]
        if b not in cache:
            cache.clear()
            cache[b] = kv_rows_to_f64(global_kv(b), kv_scale)
        S, Q = int(seq_lens[b]), qsl[b + 1] - qsl[b]
        keys = cache[b][context_keys(S, Q, W, r, I)]
        outs[n_out], lses[n_out] = attend(bf16_bits_to_f64(q_nope_bits[t]), bf16_bits_to_f64(q_pe_bits[t]),
                                          keys, scale)
    return outs, lses


def decode_query_part(seq_lens, query_start_loc, q_nope_bits, q_pe_bits, global_kv, scale: float, tokens=None,
                      kv_scale=None):
    """Stage 2, once for all ranks: query row i of a request attends causally to
    the request's own query tokens 0..i (global positions S-Q .. S-Q+i)."""
    rows = query_rows(seq_lens, query_start_loc)
    sel = range(len(rows)) if tokens is None else [int(t) for t in tokens]
    H = q_nope_bits.shape[1]
    outs = np.zeros((len(sel), H, D_LATENT))
    lses = np.zeros((len(sel), H))
    qsl = [int(x) for x in query_start_loc]
    cache = {}
    for n_out, t in enumerate(sel):
        b, i, _ = rows[t]
        if b not in cache:
            cache.clear()
            cache[b] = kv_rows_to_f64(global_kv(b), kv_scale)
        S, Q = int(seq_lens[b]), qsl[b + 1] - qsl[b]
        keys = cache[b][query_part_keys(S, Q, i)]
        outs[n_out], lses[n_out] = attend(bf16_bits_to_f64(q_nope_bits[t]), bf16_bits_to_f64(q_pe_bits[t]),
                                          keys, scale)
    return outs, lses


# ---------------------------------------------------------------------------
# Merge of per-shard partials, and the W_UV up-projection
# ---------------------------------------------------------------------------

def lse_merge(outs: np.ndarray, lses: np.ndarray, valid=None):
    """Exact LSE-weighted merge over shards (PR #48196, _dcp_lse_merge).

    outs [W,T,H,D], lses [W,T,H]; valid [W,T] per-row counts (a shard is used for
    row t iff valid[w,t] > 0) or None (used iff its lse is finite).  Invalid
    partials are never read, whatever they hold.  Merged LSE = ln sum_w exp(lse_w)
    over the used shards; merged out = sum_w exp(lse_w - LSE) * out_w.  A row with
    no used shard gives out 0 and LSE -inf.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    W, T, H = lses.shape
    out = np.zeros(outs.shape[1:])
    lse = np.full((T, H), -np.inf)
    for t in range(T):
        for h in range(H):
            used = [w for w in range(W)
                    if (valid[w][t] > 0 if valid is not None else np.isfinite(lses[w, t, h]))]
            if not used:
                continue
            m = max(lses[w, t, h] for w in used)
            total = m + math.log(sum(math.exp(lses[w, t, h] - m) for w in used))
            lse[t, h] = total
            out[t, h] = sum(math.exp(lses[w, t, h] - total) * outs[w, t, h] for w in used)
    return out, lse


def v_up_proj(o: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """Per-head up-projection y[t,h,:] = o[t,h,:] @ W_UV[h] (512 -> 128)."""
    return np.einsum("thk,hkn->thn", o, w_uv)


def merge_then_project(outs, lses, valid, w_uv):
    """Merge the latent partials, then project by W_UV."""
    o, lse = lse_merge(outs, lses, valid)
    return v_up_proj(o, w_uv), lse


def project_then_merge(outs, lses, valid, w_uv):
    """Project every shard's partial by W_UV, then merge (PR #48196's order)."""
    outs = np.asarray(outs, dtype=np.float64)
    proj = np.stack([v_up_proj(outs[w], w_uv) for w in range(outs.shape[0])])
    return lse_merge(proj, lses, valid)


# ---------------------------------------------------------------------------
# The exchange layout of the projected merge (one GPU's share of it)
# ---------------------------------------------------------------------------

def a2a_pack(o_r: np.ndarray, lse_r: np.ndarray, valid_r, w_uv: np.ndarray, W: int):
    """Rank r's send buffers for the all-to-all of the projected merge.

    PR #48196: each rank projects its partial through W_UV before the exchange
    (the payload per head shrinks from 512 to 128 values), and empty rows are
    handled in the pack from the per-row valid counts.  Reading (the pages name
    no layout): destination q owns the contiguous head slice q*Hs .. q*Hs+Hs-1,
    Hs = H / W, and receives y[t, h] = o_r[t, h] @ W_UV[h] with its LSE for those
    heads; a row whose valid count is 0 (or, without counts, whose LSE is -inf)
    is sent as y = 0, LSE = -inf, and its partial is never read.

    o_r [T,H,512], lse_r [T,H], valid_r [T] or None, w_uv [H,512,128].
    Returns send_y [W,T,Hs,128] and send_lse [W,T,Hs] (float64).
    """
    o_r = np.asarray(o_r, dtype=np.float64)
    lse_r = np.asarray(lse_r, dtype=np.float64)
    T, H = lse_r.shape
    assert H % W == 0
    Hs = H // W
    send_y = np.zeros((W, T, Hs, w_uv.shape[2]))
    send_lse = np.full((W, T, Hs), -np.inf)
    for t in range(T):
        for h in range(H):
            used = valid_r[t] > 0 if valid_r is not None else np.isfinite(lse_r[t, h])
            if not used:
                continue
            q, hh = divmod(h, Hs)
            send_y[q, t, hh] = o_r[t, h] @ w_uv[h]
            send_lse[q, t, hh] = lse_r[t, h]
    return send_y, send_lse


def a2a_combine(recv_y: np.ndarray, recv_lse: np.ndarray):
    """Receiver side: merge the W ranks' slices [W,T,Hs,128] / [W,T,Hs] of one
    destination; an empty row arrives as LSE -inf and takes no part (the same
    LSE-weighted merge as lse_merge, over the projected rows)."""
    return lse_merge(recv_y, recv_lse, None)
