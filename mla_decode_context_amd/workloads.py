"""Seeded synthetic inputs for absorbed-MLA decode under decode context parallelism.

This module only draws numbers and lays them out in memory.  It holds none of the
attention arithmetic: no scores, no softmax, no masks, no merge.  Both the fp64
oracle (``oracle/``) and the HIP path consume what it produces, so a layout bug
here shows up as a parity failure rather than being hidden.

Shapes follow the workload the pages describe:

* every cache token row is ``c_kv[512] | k_pe[64]`` in bf16, 1152 bytes
  ("flashattn_mla" API page, ``_forward_decode``: the cache is sliced at
  ``kv_lora_rank`` into the latent and rope parts);
* queries come as ``q_nope [T,H,512]`` and ``q_pe [T,H,64]`` bf16 (same page,
  the tuple/split of ``q``);
* the KV of one request is paged: ``block_table[b][j // P]`` names the physical
  block of local token ``j`` and ``j % P`` its slot (same page, ``block_table``
  passed to the varlen kernel);
* under DCP the global token ``p`` of a request is stored on shard ``p mod W`` at
  shard-local index ``p div W`` (PR #24453 review thread: with dcp=2 key A lives on
  rank 0 and key B on rank 1).  With a run length ``I`` > 1 (the same thread's
  mention of contiguous whole pages per shard), runs of ``I`` consecutive tokens
  go to the shards in turn: token ``p`` on shard ``(p div I) mod W``, each shard
  keeping its tokens in ascending position.  Each shard owns a separate paged
  cache with its own randomly permuted physical block ids.

Random streams (NumPy PCG64), one per purpose so that any request's tokens can be
regenerated on demand without replaying the others:

* ``default_rng(seed)``          sequence lengths, then (mixed batch) query lengths
* ``default_rng([seed, 1])``     q_nope, then q_pe
* ``default_rng([seed, 2, b])``  the global KV rows of request ``b``
* ``default_rng([seed, 3, r])``  the physical block permutation of shard ``r``
* ``default_rng([seed, 4])``     W_UV

Values are ``standard_normal`` in float32 rounded to bf16 (round to nearest even);
W_UV is ``0.02 * standard_normal``.  Unused cache slots, spare blocks and the tail
of each request's last page hold the bf16 quiet NaN 0x7FC0, and unused block-table
entries hold -1, so a kernel that reads outside a request's tokens poisons its
result instead of passing by accident.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

D_LATENT = 512          # kv_lora_rank: width of c_kv and of the output
D_ROPE = 64             # qk_rope_head_dim: width of k_pe / q_pe
D_ROW = D_LATENT + D_ROPE
D_V = 128               # v_head_dim: width after the W_UV up-projection
BF16_NAN = 0x7FC0
FP8_NAN = 0x7F          # E4M3 (OCP "fn") NaN code
FP8_SCALE = 0.0137      # scale of the FP8 caches: values are code * FP8_SCALE

# The five workloads.  Lengths are global totals S_b including the request's own
# query tokens; "lo..hi" draws are inclusive integer uniforms.
CONFIGS = {
    "tiny_dcp": dict(
        desc="4 requests, total seq lens {6,37,128,255}, Q=4, H=16, W=2, page 16",
        B=4, seq_lens=[6, 37, 128, 255], q_len=4, H=16, W=2, P=16, seed=0),
    "plain": dict(
        desc="batch 64, Q=1, H=16, W=1, context 1024..8192, page 64",
        B=64, seq_range=(1024, 8192), q_len=1, H=16, W=1, P=64, seed=1),
    "mtp_dcp4": dict(
        desc="batch 128, Q=2, H=128, W=4, context 1024..4096, page 64",
        B=128, seq_range=(1024, 4096), q_len=2, H=128, W=4, P=64, seed=2),
    "long_dcp8": dict(
        desc="batch 256, Q=2, H=128, W=8, context 8192..32768, page 64; "
             "requests 0,64,128,192 shortened to 2,3,5,7 tokens so that some "
             "shards hold empty rows",
        B=256, seq_range=(8192, 32768), q_len=2, H=128, W=8, P=64, seed=3,
        overrides={0: 2, 64: 3, 128: 5, 192: 7}),
    "mixed_wuv": dict(
        desc="96 decodes (Q in {1,2,4}) then 2 prefill chunks of 512 rows, H=128, "
             "W=4, context 512..16384, page 64, W_UV [128,512,128] ~ 0.02*N(0,1)",
        B=98, n_decode=96, decode_q=(1, 2, 4), chunk_q=512, seq_range=(512, 16384),
        H=128, W=4, P=64, seed=4, w_uv=True),
    "plain_fp8": dict(
        desc="plain with an FP8 E4M3 latent cache (one scale per cache): batch 64, Q=1, H=16, W=1, "
             "context 1024..8192, page 64",
        B=64, seq_range=(1024, 8192), q_len=1, H=16, W=1, P=64, seed=1, kv_fp8=True),
    "mtp_dcp4_pages": dict(
        desc="mtp_dcp4 with whole pages per shard: runs of 64 tokens (one page) "
             "dealt to the 4 shards in turn",
        B=128, seq_range=(1024, 4096), q_len=2, H=128, W=4, P=64, seed=2, I=64),
}
CONFIG_ORDER = ["tiny_dcp", "plain", "mtp_dcp4", "long_dcp8", "mixed_wuv", "mtp_dcp4_pages", "plain_fp8"]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 storage (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def _e4m3_magnitudes() -> np.ndarray:
    """Values of the non-negative finite E4M3 codes 0x00 .. 0x7E, ascending."""
    c = np.arange(0x7F)
    e, f = c >> 3, (c & 7).astype(np.float64)
    return np.where(e == 0, np.ldexp(f / 8.0, -6), np.ldexp(1.0 + f / 8.0, e - 7))


def f64_to_fp8_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round to the nearest E4M3 (OCP "fn") value, ties to the even code,
    saturating at +-448; returns uint8 codes.  Input drawing only (the
    synthetic FP8 caches), not part of the decode."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    vals = _e4m3_magnitudes()
    hi = np.clip(np.searchsorted(vals, a), 1, 126)
    lo = hi - 1
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    code = np.where(a >= vals[126], 126, code)
    return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def _normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def shard_token_rows(S: int, W: int, r: int, I: int = 1) -> np.ndarray:
    """Positions among 0..S-1 that shard r stores, ascending (its local order),
    when runs of I tokens go to the shards in turn (I = 1: p mod W == r).

    This is storage bookkeeping for building the caches (which rows shard r
    holds), not the per-query-row mask.
    """
    pos = np.arange(S, dtype=np.int64)
    return pos[(pos // I) % W == r]


def shard_token_count(S: int, W: int, r: int, I: int = 1) -> int:
    """How many of the tokens 0..S-1 shard r stores."""
    return int(shard_token_rows(S, W, r, I).shape[0])


@dataclass
class Shard:
    """One DCP shard's paged latent cache."""
    cache: np.ndarray          # uint16 [num_blocks, P, 576] (bf16 bits)
    block_table: np.ndarray    # int32 [B, max_blocks], -1 where unused
    token_counts: np.ndarray   # int32 [B], rows of request b stored on this shard


@dataclass
class Workload:
    name: str
    B: int
    H: int
    W: int
    P: int
    seed: int
    scale: float
    seq_lens: np.ndarray       # int32 [B], global S_b including the query tokens
    query_lens: np.ndarray     # int32 [B]
    query_start_loc: np.ndarray  # int32 [B+1]
    q_nope: np.ndarray         # uint16 [T,H,512]
    q_pe: np.ndarray           # uint16 [T,H,64]
    shards: list = field(default_factory=list)
    w_uv: np.ndarray | None = None   # uint16 [H,512,128]
    I: int = 1                       # shard run length: token p on shard (p div I) mod W
    kv_scale: float | None = None    # FP8 caches: uint8 E4M3 codes, value = code * kv_scale

    @property
    def T(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.B else 0

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.B else 0

    def global_kv(self, b: int) -> np.ndarray:
        """Regenerate the global KV rows [S_b, 576] of request b as stored: bf16
        bits, or E4M3 codes for an FP8 cache."""
        return _request_kv(self.seed, b, int(self.seq_lens[b]), self.kv_scale)


def query_part_layout(wl: Workload):
    """The query tokens' own KV rows laid out for the query stage of the
    two-stage decode: rows [T, 576] (row t = the KV row of query token t, i.e.
    global position S_b - Q_b + i of its request), a block table [B, max Q]
    naming row qsl[b] + j as block j of request b when the rows are read as a
    cache of one-token pages (-1 past Q_b), and the per-request lengths Q_b.
    Pure layout: copies rows, computes no attention."""
    T, B = wl.T, wl.B
    rows = np.empty((T, D_ROW), dtype=np.uint8 if wl.kv_scale is not None else np.uint16)
    qsl = wl.query_start_loc
    for b in range(B):
        q0, q1 = int(qsl[b]), int(qsl[b + 1])
        if q1 > q0:
            S = int(wl.seq_lens[b])
            rows[q0:q1] = wl.global_kv(b)[S - (q1 - q0):S]
    mq = max(1, wl.max_query_len)
    table = np.full((B, mq), -1, dtype=np.int32)
    for b in range(B):
        q0, q1 = int(qsl[b]), int(qsl[b + 1])
        table[b, :q1 - q0] = np.arange(q0, q1, dtype=np.int32)
    return rows, table, wl.query_lens.astype(np.int32).copy()


def _request_kv(seed: int, b: int, S: int, kv_scale=None) -> np.ndarray:
    rng = np.random.default_rng([seed, 2, b])
    if kv_scale is None:
        return _normal_bf16(rng, (S, D_ROW))
    x = rng.standard_normal((S, D_ROW), dtype=np.float32)
    return f64_to_fp8_e4m3_bits(x.astype(np.float64) / kv_scale)


def _draw_lengths(cfg: dict, seed: int):
    rng = np.random.default_rng(seed)
    B = cfg["B"]
    if "seq_lens" in cfg:
        S = np.array(cfg["seq_lens"], dtype=np.int64)
    else:
        lo, hi = cfg["seq_range"]
        S = rng.integers(lo, hi, size=B, endpoint=True)
    if "n_decode" in cfg:
        nd = cfg["n_decode"]
        Q = np.empty(B, dtype=np.int64)
        Q[:nd] = rng.choice(np.array(cfg["decode_q"]), size=nd)
        Q[nd:] = cfg["chunk_q"]
    else:
        Q = np.full(B, cfg["q_len"], dtype=np.int64)
    for b, s in cfg.get("overrides", {}).items():
        S[b] = s
    Q = np.minimum(Q, S)       # a request cannot have more query rows than tokens
    return S.astype(np.int32), Q.astype(np.int32)


def build_shard(seed: int, r: int, W: int, P: int, seq_lens: np.ndarray,
                kv_rows_of, spare_frac: float = 0.05, I: int = 1, fp8: bool = False) -> Shard:
    """Lay shard r's tokens of every request (p = r, r+W, ... when I = 1) into its pages.

    ``kv_rows_of(b)`` returns the shard-local rows of request b ([n, 576] bf16 bits)
    in local order.  Logical blocks are numbered request by request; physical ids
    are a random permutation of the pool, which has ``spare_frac`` extra blocks.
    """
    B = len(seq_lens)
    counts = np.array([shard_token_count(int(s), W, r, I) for s in seq_lens], dtype=np.int32)
    nblk = np.array([math.ceil(int(c) / P) for c in counts], dtype=np.int64)
    n_logical = int(nblk.sum())
    pool = n_logical + max(1, int(math.ceil(spare_frac * n_logical)))
    perm = np.random.default_rng([seed, 3, r]).permutation(pool).astype(np.int32)
    max_blocks = max(1, int(nblk.max()) if B else 1)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    cache = np.full((pool, P, D_ROW), FP8_NAN, dtype=np.uint8) if fp8 else \
        np.full((pool, P, D_ROW), BF16_NAN, dtype=np.uint16)
    off = 0
    for b in range(B):
        nb = int(nblk[b])
        if nb == 0:
            continue
        phys = perm[off:off + nb]
        table[b, :nb] = phys
        rows = kv_rows_of(b)
        n = rows.shape[0]
        full = n // P
        if full:
            cache[phys[:full]] = rows[:full * P].reshape(full, P, D_ROW)
        if n % P:
            cache[phys[full], :n % P] = rows[full * P:]
        off += nb
    return Shard(cache=cache, block_table=table, token_counts=counts)


def make_workload(name: str, *, threads: int = 8, seed: int | None = None,
                  seq_lens=None, query_lens=None, H: int | None = None,
                  W: int | None = None, P: int | None = None, I: int | None = None) -> Workload:
    """Build one of the named workloads (or a variant with some fields replaced)."""
    cfg = dict(CONFIGS[name])
    seed = cfg["seed"] if seed is None else seed
    S, Q = _draw_lengths(cfg, seed)
    if seq_lens is not None:
        S = np.asarray(seq_lens, dtype=np.int32)
        Q = np.full(len(S), cfg.get("q_len", 1), dtype=np.int32) if query_lens is None else Q
    if query_lens is not None:
        Q = np.asarray(query_lens, dtype=np.int32)
    H = cfg["H"] if H is None else H
    W = cfg["W"] if W is None else W
    P = cfg["P"] if P is None else P
    I = cfg.get("I", 1) if I is None else I
    return make_custom(name, S, Q, H=H, W=W, P=P, seed=seed,
                       w_uv=cfg.get("w_uv", False), threads=threads, I=I,
                       kv_scale=FP8_SCALE if cfg.get("kv_fp8") else None)


def make_custom(name: str, seq_lens, query_lens, *, H: int, W: int, P: int, seed: int,
                w_uv: bool = False, threads: int = 8, scale: float | None = None, I: int = 1,
                kv_scale: float | None = None) -> Workload:
    """Build a workload from explicit per-request lengths (an FP8 E4M3 cache
    with that scale when kv_scale is given)."""
    S = np.asarray(seq_lens, dtype=np.int32)
    Q = np.asarray(query_lens, dtype=np.int32)
    assert S.shape == Q.shape and np.all(Q >= 0) and np.all(Q <= S)
    B = len(S)
    qsl = np.zeros(B + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(Q)
    T = int(qsl[-1])
    rq = np.random.default_rng([seed, 1])
    q_nope = _normal_bf16(rq, (T, H, D_LATENT))
    q_pe = _normal_bf16(rq, (T, H, D_ROPE))
    wl = Workload(name=name, B=B, H=H, W=W, P=P, seed=seed, I=I, kv_scale=kv_scale,
                  scale=(1.0 / math.sqrt(D_V + D_ROPE)) if scale is None else scale,
                  seq_lens=S, query_lens=Q, query_start_loc=qsl, q_nope=q_nope, q_pe=q_pe)
    # Global KV is generated per request (in parallel: each request has its own
    # stream, so the result does not depend on scheduling) and scattered to shards.
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        kv = list(ex.map(lambda b: _request_kv(seed, b, int(S[b]), kv_scale), range(B)))
        wl.shards = list(ex.map(
            lambda r: build_shard(seed, r, W, P, S, lambda b: kv[b][shard_token_rows(int(S[b]), W, r, I)], I=I,
                                  fp8=kv_scale is not None),
            range(W)))
    del kv
    if w_uv:
        wl.w_uv = _normal_bf16(np.random.default_rng([seed, 4]), (H, D_LATENT, D_V), std=0.02)
    return wl
