"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments with status codes before touching a device.
No call here enqueues GPU work."""
import ctypes

import pytest

from mla_decode_context_amd import binding

lib = binding.load_library()

OK, NULL, SHAPE, UNSUP, WS, HIP, CAPTURE = 0, -1, -2, -3, -4, -5, -6
P = ctypes.c_void_p(16 * 1024)          # a dummy, aligned non-null "device" address (never dereferenced)


def test_exports_every_declared_symbol():
    names = binding.header_functions()
    assert set(names) == {"mla_status_string", "mla_decode_partial", "mla_decode_workspace_size",
                          "mla_lse_merge", "mla_merge_v_up_proj", "mla_dcp_local_seqlens",
                          "mla_dcp_a2a_pack", "mla_dcp_a2a_combine", "mla_check_decode_metadata",
                          "mla_decode_partial_noalloc",
                          "mla_calib_hbm_read", "mla_calib_hbm_gather", "mla_calib_mfma_bf16",
                          "mla_calib_mfma_flops"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in (OK, NULL, SHAPE, UNSUP, WS, HIP, CAPTURE):
        s = lib.mla_status_string(code).decode()
        assert s.startswith("MLA_")
    assert "unknown" in lib.mla_status_string(7).decode()


def _decode(**kw):
    a = dict(q_nope=P, qn_t=16 * 512, qn_h=512, q_pe=P, qp_t=16 * 64, qp_h=64, kv=P, kv_bs=16 * 576, page=16,
             bt=P, bt_stride=4, seq=P, qsl=P, B=2, T=4, H=16, mq=2, ms=100, W=2, r=0, I=1, mask=0, scale=0.07,
             splits=0, out=P, dtype=0, lse=P, ws=None, ws_bytes=0, kvt=0, kvs=1.0)
    a.update(kw)
    return lib.mla_decode_partial(a["q_nope"], a["qn_t"], a["qn_h"], a["q_pe"], a["qp_t"], a["qp_h"], a["kv"],
                                  a["kvt"], a["kvs"], a["kv_bs"], a["page"], a["bt"], a["bt_stride"], a["seq"], a["qsl"], a["B"],
                                  a["T"], a["H"], a["mq"], a["ms"], a["W"], a["r"], a["I"], a["mask"], a["scale"],
                                  a["splits"],
                                  a["out"], a["dtype"], a["lse"], None, a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(H=0), SHAPE), (dict(H=129), SHAPE), (dict(B=-1), SHAPE), (dict(T=-1), SHAPE),
    (dict(W=0), SHAPE), (dict(r=2), SHAPE), (dict(r=-1), SHAPE), (dict(page=0), SHAPE),
    (dict(scale=float("nan")), SHAPE), (dict(scale=float("inf")), SHAPE), (dict(splits=-1), SHAPE),
    (dict(scale=0.0), SHAPE), (dict(scale=-0.07), SHAPE),
    (dict(B=0, T=3), SHAPE),
    (dict(q_nope=None), NULL), (dict(kv=None), NULL), (dict(bt=None), NULL), (dict(lse=None), NULL),
    (dict(qn_h=500), SHAPE), (dict(qn_t=512), SHAPE), (dict(qp_h=60), SHAPE), (dict(kv_bs=575 * 16), SHAPE),
    (dict(q_nope=ctypes.c_void_p(16 * 1024 + 2)), SHAPE), (dict(bt_stride=0), SHAPE),
    (dict(T=0), OK), (dict(B=0, T=0), OK), (dict(T=0, q_nope=None), OK),
    (dict(I=0), SHAPE), (dict(I=-3), SHAPE), (dict(W=4, I=1 << 29), SHAPE),
    (dict(W=2, I=1 << 28, T=0), OK),
    (dict(dtype=2), SHAPE), (dict(dtype=-1), SHAPE), (dict(dtype=1, T=0), OK),
    (dict(mask=2), SHAPE), (dict(mask=-1), SHAPE), (dict(mask=1, T=0), OK),
    (dict(kvt=1), SHAPE), (dict(kvt=3), SHAPE), (dict(kvt=2, kvs=0.0), SHAPE), (dict(kvt=2, kvs=-1.0), SHAPE),
    (dict(kvt=2, kvs=float("nan")), SHAPE), (dict(kvt=2, kv_bs=16 * 576 + 8), SHAPE),
    (dict(kvt=0, kvs=float("nan"), T=0), OK), (dict(kvt=2, kvs=0.01, T=0), OK),
])
def test_decode_argument_checks(kw, code):
    assert _decode(**kw) == code


def _ws(B, T, H, mq, ms, W, splits, I=1):
    return lib.mla_decode_workspace_size(B, T, H, mq, ms, W, I, splits)


def test_workspace_size_host_logic():
    ws = _ws
    bad = ctypes.c_size_t(-1).value
    assert ws(2, 4, 0, 1, 100, 1, 0) == bad
    assert ws(2, 4, 16, 1, 100, 0, 0) == bad
    assert ws(0, 0, 16, 1, 100, 1, 0) == 0
    assert ws(4, 4, 16, 1, 100, 1, 1) == 0                   # never split
    # a long row split 4 ways needs 4 fp32 partial rows + LSE per (t, h)
    n = ws(1, 1, 16, 1, 4096, 1, 4)
    assert n >= 4 * 16 * (512 + 1) * 4
    assert ws(64, 64, 16, 1, 8192, 1, 0) > 0                 # the batch-64 decode splits automatically
    assert ws(64, 64, 16, 1, 8192, 1, 2) < ws(64, 64, 16, 1, 8192, 1, 16)
    # 128 heads, never split: only the dispatch order (one int32 item and one
    # int2 {request, keys} per token and 64-head block, each array in 256-byte
    # units) plus the alignment slack
    assert ws(2, 4, 128, 2, 100, 1, 1) == 256 + 256 + 256
    assert ws(300, 600, 128, 2, 4000, 4, 1) == 4864 + 9728 + 256     # 600 * 2 * {4, 8} bytes, rounded up
    # more (split, request) units than the order kernel sorts: no order, no workspace
    assert ws(9000, 9000, 128, 1, 4000, 4, 1) == 0
    # run layout: invalid run lengths are rejected; the split plan follows the
    # longest shard (rank 0 holds a whole first run of every round): 100 tokens
    # in runs of 64 over 2 ranks put 64 on rank 0, more than ceil(100 / 2) = 50
    assert ws(2, 4, 16, 1, 100, 2, 0, I=0) == bad
    assert ws(2, 4, 16, 1, 100, 4, 0, I=1 << 29) == bad          # W * I above 2^30
    assert ws(1, 1, 16, 1, 8192, 4, 4, I=64) == ws(1, 1, 16, 1, 8192, 4, 4, I=1)
    assert ws(1, 1, 128, 1, 100, 2, 0, I=64) >= ws(1, 1, 128, 1, 100, 2, 0, I=1)


def test_merge_argument_checks():
    m = lib.mla_lse_merge
    assert m(P, 0, P, None, 0, 4, 16, P, None, None) == SHAPE
    assert m(P, 0, P, None, 2, 4, 0, P, None, None) == SHAPE
    assert m(None, 0, P, None, 2, 4, 16, P, None, None) == NULL
    assert m(P, 0, P, None, 2, 0, 16, P, None, None) == OK
    assert m(P, 1, P, None, 2, 0, 16, P, None, None) == OK
    assert m(P, 3, P, None, 2, 4, 16, P, None, None) == SHAPE     # unknown partial dtype
    v = lib.mla_merge_v_up_proj
    assert v(P, 0, P, None, 2, 4, 16, None, P, None, None) == NULL
    assert v(P, 0, P, None, 2, -1, 16, P, P, None, None) == SHAPE
    assert v(P, 7, P, None, 2, 4, 16, P, P, None, None) == SHAPE
    s = lib.mla_dcp_local_seqlens
    assert s(P, P, 2, 4, 2, 2, 1, 0, P, P, None) == SHAPE
    assert s(P, P, 2, 4, 2, 1, 0, 0, P, P, None) == SHAPE
    assert s(P, P, 2, 4, 2, 1, 1, 5, P, P, None) == SHAPE          # unknown mask mode
    assert s(None, P, 2, 4, 2, 1, 1, 0, P, P, None) == NULL
    assert s(P, P, 0, 0, 2, 1, 16, 1, P, P, None) == OK


def test_exchange_argument_checks():
    pk = lib.mla_dcp_a2a_pack
    assert pk(P, 0, P, None, 4, 128, 3, P, P, P, None) == SHAPE       # H % W != 0
    assert pk(P, 0, P, None, 4, 0, 1, P, P, P, None) == SHAPE
    assert pk(P, 0, P, None, -1, 16, 2, P, P, P, None) == SHAPE
    assert pk(P, 0, P, None, 4, 16, 2, None, P, P, None) == NULL      # W_UV missing
    assert pk(P, 0, P, None, 4, 16, 2, P, P, None, None) == NULL      # send_lse missing
    assert pk(P, 0, P, None, 0, 16, 2, None, None, None, None) == OK  # T == 0
    assert pk(P, 2, P, None, 4, 16, 2, P, P, P, None) == SHAPE        # unknown partial dtype
    cb = lib.mla_dcp_a2a_combine
    rows = 4 * 8
    assert cb(P, rows * 128, P, rows, 0, 4, 8, P, None, None) == SHAPE
    assert cb(P, rows * 128 - 8, P, rows, 2, 4, 8, P, None, None) == SHAPE    # slices overlap
    assert cb(P, rows * 128, P, rows - 1, 2, 4, 8, P, None, None) == SHAPE
    assert cb(P, rows * 128 + 4, P, rows, 2, 4, 8, P, None, None) == SHAPE    # not 16-byte aligned
    assert cb(None, rows * 128, P, rows, 2, 4, 8, P, None, None) == NULL
    assert cb(P, rows * 128, P, rows, 2, 0, 8, P, None, None) == OK


def test_calibration_argument_checks():
    assert lib.mla_calib_hbm_read(P, 0, 0, None, None) == OK           # nothing to read
    assert lib.mla_calib_hbm_read(None, 1024, 0, P, None) == NULL
    assert lib.mla_calib_hbm_read(P, 1000, 0, P, None) == SHAPE        # not whole 16-byte words
    assert lib.mla_calib_hbm_read(ctypes.c_void_p(16 * 1024 + 4), 1024, 0, P, None) == SHAPE
    assert lib.mla_calib_hbm_gather(P, 0, 8, P, None) == OK            # nothing to move
    assert lib.mla_calib_hbm_gather(None, 1024, 8, P, None) == NULL
    assert lib.mla_calib_hbm_gather(P, 1024, 8, None, None) == NULL
    assert lib.mla_calib_hbm_gather(P, 1000, 8, P, None) == SHAPE      # not whole 16-byte words
    assert lib.mla_calib_hbm_gather(P, 1024, 3, P, None) == SHAPE      # 1, 2, 4 or 8 inputs
    assert lib.mla_calib_hbm_gather(ctypes.c_void_p(16 * 1024 + 4), 1024, 8, P, None) == SHAPE
    assert lib.mla_calib_mfma_bf16(-1, P, None) == SHAPE
    assert lib.mla_calib_mfma_bf16(10, None, None) == NULL
    # 512 workgroups x 4 waves x iters x 8 chains x 16384 flop per MFMA
    assert lib.mla_calib_mfma_flops(10) == 512 * 4 * 10 * 8 * 16384.0
    assert lib.mla_calib_mfma_flops(-1) == -1.0


# ---------------------------------------------------------------------------
# mla_check_decode_metadata: the device-side contract on host copies (what
# MLA_DEBUG=1 checks before a decode call launches anything)
# ---------------------------------------------------------------------------

def _meta(**kw):
    """A valid metadata set: 3 requests, W = 2, rank 1, page 4, 40 blocks."""
    m = dict(S=[9, 2, 17], qsl=[0, 2, 3, 7], bt=None, bt_stride=3, T=7, mq=4, ms=17, P=4, W=2, r=1, I=1, mode=0,
             nblk=40)
    m.update(kw)
    if m["bt"] is None:
        m["bt"] = [0, 1, -1, 2, -1, -1, 3, 4, 5]     # rank 1 holds 4, 1, 8 tokens -> 1, 1, 2 blocks
    return m


def _check_meta(m):
    S = (ctypes.c_int32 * len(m["S"]))(*m["S"])
    q = (ctypes.c_int32 * len(m["qsl"]))(*m["qsl"])
    bt = (ctypes.c_int32 * len(m["bt"]))(*m["bt"])
    why = ctypes.create_string_buffer(256)
    st = lib.mla_check_decode_metadata(S, q, bt, m["bt_stride"], len(m["S"]), m["T"], m["mq"], m["ms"], m["P"],
                                       m["W"], m["r"], m["I"], m["mode"], m["nblk"], why, 256)
    return st, why.value.decode()


@pytest.mark.parametrize("kw,fragment", [
    (dict(qsl=[1, 2, 3, 7]), "query_start_loc[0]"),
    (dict(qsl=[0, 3, 2, 7]), "decreases"),
    (dict(qsl=[0, 2, 3, 6]), "not T"),
    (dict(mq=3), "max_query_len"),
    (dict(S=[9, 0, 17]), "query rows"),                 # Q_b > S_b
    (dict(ms=16), "max_seq_len"),
    (dict(bt=[0, 1, -1, 2, -1, -1, 3, -1, 5]), "block_table entry 1 = -1"),
    (dict(bt=[0, 1, -1, 40, -1, -1, 3, 4, 5]), "block_table entry 0 = 40"),
    (dict(bt=[0, 1, 2, 3, 4, 5], bt_stride=2, S=[9, 2, 33], ms=33), "blocks on rank"),
])
def test_check_metadata_violations(kw, fragment):
    st, why = _check_meta(_meta(**kw))
    assert st == SHAPE and fragment in why, (st, why)


def test_check_metadata_accepts_valid_sets():
    assert _check_meta(_meta()) == (OK, "")
    # unused entries past a request's blocks are never looked at, whatever they hold
    assert _check_meta(_meta(bt=[0, 1, -99, 2, 12345, -7, 3, 4, 5]))[0] == OK
    # unknown pool size: ids only need to be >= 0
    assert _check_meta(_meta(bt=[0, 10 ** 6, -1, 2, -1, -1, 3, 4, 5], nblk=-1))[0] == OK
    # whole-page runs (I = 4): rank 1 holds 4, 0, 8 tokens; request 1 needs no block
    assert _check_meta(_meta(I=4, bt=[0, -1, -1, -1, -1, -1, 3, 4, -1]))[0] == OK
    # rank 0 of W = 1 holds everything: 9, 2, 17 tokens -> 3, 1, 5 blocks (stride 5)
    bt = [0, 1, 2, -1, -1, 3, -1, -1, -1, -1, 4, 5, 6, 7, 8]
    assert _check_meta(_meta(W=1, r=0, bt=bt, bt_stride=5))[0] == OK
    assert _check_meta(_meta(S=[], qsl=[0], bt=[0], T=0))[0] == OK
    # context mode reads only the first S - Q tokens' share: request 2 (S 17,
    # Q 4) holds 6 of its 13 context tokens on rank 1 -> 2 blocks, request 0
    # (S 9, Q 2) 3 of 7 -> 1 block, request 1 none; entries past them unread
    assert _check_meta(_meta(mode=1, bt=[0, -1, -1, -1, -1, -1, 3, 4, -1]))[0] == OK
    assert _check_meta(_meta(mode=0, bt=[0, -1, -1, -1, -1, -1, 3, 4, -1]))[0] == SHAPE
    assert _check_meta(_meta(mode=2))[0] == SHAPE
    assert _check_meta(_meta(S=[], qsl=[0], bt=[0], T=2))[0] == SHAPE
