"""Thin Python binding of libmla (argument marshalling only).

Every function here takes torch tensors that already live on the GPU, checks
dtype/shape/contiguity on the host, and forwards raw device pointers, strides
and sizes to the C ABI declared in ``include/mla.h``.  No step of the
computation happens here; there is no fallback path.  If the shared library has
not been built, loading it raises immediately.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla.so")
INCLUDE = os.path.join(os.path.dirname(_PKG), "include")
HEADER = os.path.join(INCLUDE, "mla.h")

MLA_OK = 0
D_LATENT, D_ROPE, D_ROW, D_V = 512, 64, 576, 128
DTYPE_BF16, DTYPE_F32 = 0, 1          # MLA_DTYPE_BF16 / MLA_DTYPE_F32
MASK_CAUSAL, MASK_CONTEXT = 0, 1       # MLA_MASK_CAUSAL / MLA_MASK_CONTEXT
DTYPE_FP8_E4M3 = 2                     # MLA_DTYPE_FP8_E4M3 (cache elements)

_lib = None

_c_void_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class MlaError(RuntimeError):
    pass


def load_library():
    """Load libmla.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MlaError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_status_string.argtypes = [_i32]
    lib.mla_decode_partial.restype = _i32
    lib.mla_decode_partial.argtypes = [
        _c_void_p, _i64, _i64, _c_void_p, _i64, _i64, _c_void_p, _i32, ctypes.c_float, _i64, _i32,
        _c_void_p, _i32, _c_void_p, _c_void_p,
        _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _i32,
        _c_void_p, _i32, _c_void_p, _c_void_p, _c_void_p, ctypes.c_size_t, _c_void_p]
    lib.mla_decode_partial_noalloc.restype = _i32
    lib.mla_decode_partial_noalloc.argtypes = [
        _c_void_p, _i64, _i64, _c_void_p, _i64, _i64, _c_void_p, _i32, ctypes.c_float, _i64, _i32,
        _c_void_p, _i32, _c_void_p, _c_void_p,
        _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _i32,
        _c_void_p, _i32, _c_void_p, _c_void_p, _c_void_p]
    lib.mla_decode_workspace_size.restype = ctypes.c_size_t
    lib.mla_decode_workspace_size.argtypes = [_i32] * 8
    lib.mla_lse_merge.restype = _i32
    lib.mla_lse_merge.argtypes = [_c_void_p, _i32, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                  _c_void_p, _c_void_p, _c_void_p]
    lib.mla_merge_v_up_proj.restype = _i32
    lib.mla_merge_v_up_proj.argtypes = [_c_void_p, _i32, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                        _c_void_p, _c_void_p, _c_void_p, _c_void_p]
    lib.mla_dcp_a2a_pack.restype = _i32
    lib.mla_dcp_a2a_pack.argtypes = [_c_void_p, _i32, _c_void_p, _c_void_p, _i32, _i32, _i32, _c_void_p,
                                     _c_void_p, _c_void_p, _c_void_p]
    lib.mla_dcp_a2a_combine.restype = _i32
    lib.mla_dcp_a2a_combine.argtypes = [_c_void_p, _i64, _c_void_p, _i64, _i32, _i32, _i32,
                                        _c_void_p, _c_void_p, _c_void_p]
    lib.mla_dcp_local_seqlens.restype = _i32
    lib.mla_dcp_local_seqlens.argtypes = [_c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32,
                                          _c_void_p, _c_void_p, _c_void_p]
    lib.mla_check_decode_metadata.restype = _i32
    lib.mla_check_decode_metadata.argtypes = [_c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _i32,
                                              _i32, _i32, _i32, _i32, _i32, _i64, ctypes.c_char_p, ctypes.c_size_t]
    lib.mla_calib_hbm_read.restype = _i32
    lib.mla_calib_hbm_read.argtypes = [_c_void_p, ctypes.c_size_t, _i32, _c_void_p, _c_void_p]
    lib.mla_calib_hbm_gather.restype = _i32
    lib.mla_calib_hbm_gather.argtypes = [_c_void_p, ctypes.c_size_t, _i32, _c_void_p, _c_void_p]
    lib.mla_calib_mfma_bf16.restype = _i32
    lib.mla_calib_mfma_bf16.argtypes = [_i32, _c_void_p, _c_void_p]
    lib.mla_calib_mfma_flops.restype = ctypes.c_double
    lib.mla_calib_mfma_flops.argtypes = [_i32]
    _lib = lib
    return lib


def header_functions() -> list[str]:
    """Names of the functions declared in the headers under include/."""
    names = []
    for f in sorted(os.listdir(INCLUDE)):
        if f.endswith(".h"):
            text = open(os.path.join(INCLUDE, f)).read()
            names += re.findall(r"^\s*(?:mla_status|size_t|double|const char\*)\s+(mla_\w+)\s*\(", text, re.M)
    return names


def _check(status: int, what: str):
    if status != MLA_OK:
        msg = load_library().mla_status_string(status).decode()
        raise MlaError(f"{what} failed: {msg} ({status})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, name, dims=None):
    if t.dtype != dtype:
        raise MlaError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise MlaError(f"{name}: must be a GPU tensor")
    if dims is not None and t.dim() != dims:
        raise MlaError(f"{name}: expected {dims} dims, got shape {tuple(t.shape)}")


def _partial_dtype(t, name):
    """ABI code of a partial-output tensor's element type (bf16 or fp32)."""
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise MlaError(f"{name}: expected bfloat16 or float32 partials, got {t.dtype}")


def _kv_dtype(kv_cache, kv_scale):
    """ABI code and scale of a cache tensor: bf16, or FP8 E4M3 codes (uint8 or
    float8_e4m3fn) with their scale."""
    if kv_cache.dtype == torch.bfloat16:
        return DTYPE_BF16, 1.0
    if kv_cache.dtype in (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8)):
        if kv_scale is None:
            raise MlaError("kv_cache: an FP8 E4M3 cache needs kv_scale")
        return DTYPE_FP8_E4M3, float(kv_scale)
    raise MlaError(f"kv_cache: expected bfloat16 or FP8 E4M3 codes, got {kv_cache.dtype}")


def workspace_size(B, T, H, max_query_len, max_seq_len, cp_world, num_splits=0, cp_interleave=1) -> int:
    n = load_library().mla_decode_workspace_size(B, T, H, max_query_len, max_seq_len, cp_world,
                                                 cp_interleave, num_splits)
    if n == ctypes.c_size_t(-1).value:
        raise MlaError("mla_decode_workspace_size: invalid arguments")
    return int(n)


def mla_decode_partial(q_nope, q_pe, kv_cache, block_table, seq_lens, query_start_loc,
                       cp_world, cp_rank, scale, out, lse, *, max_query_len, max_seq_len,
                       workspace=None, num_splits=0, stream=None, cp_interleave=1, mask_mode=MASK_CAUSAL,
                       kv_scale=None, row_keys=None):
    """One DCP rank's partial attention; writes ``out`` [T,H,512] (bf16, or fp32
    partials when ``out`` is a float32 tensor) and ``lse`` [T,H] fp32, and when
    given ``row_keys`` [T] int32 (every row's visible local key count).
    ``cp_interleave``: tokens per run of the shard layout (1 = token p on rank p mod W)."""
    lib = load_library()
    _need(q_nope, torch.bfloat16, "q_nope", 3)
    _need(q_pe, torch.bfloat16, "q_pe", 3)
    kv_dtype, kv_sc = _kv_dtype(kv_cache, kv_scale)
    _need(kv_cache, kv_cache.dtype, "kv_cache", 3)
    _need(block_table, torch.int32, "block_table", 2)
    _need(seq_lens, torch.int32, "seq_lens", 1)
    _need(query_start_loc, torch.int32, "query_start_loc", 1)
    out_dtype = _partial_dtype(out, "out")
    _need(out, out.dtype, "out", 3)
    _need(lse, torch.float32, "lse", 2)
    T, H, dn = q_nope.shape
    if dn != D_LATENT or tuple(q_pe.shape) != (T, H, D_ROPE):
        raise MlaError("q_nope/q_pe: expected [T,H,512] / [T,H,64]")
    if T == 0:
        # nothing to compute; the C call is a no-op but still validates the scalars
        qn_st, qn_sh, qp_st, qp_sh = H * D_LATENT, D_LATENT, H * D_ROPE, D_ROPE
    else:
        if q_nope.stride(2) != 1 or q_pe.stride(2) != 1:
            raise MlaError("q_nope/q_pe: the last dim must be contiguous")
        qn_st, qn_sh, qp_st, qp_sh = q_nope.stride(0), q_nope.stride(1), q_pe.stride(0), q_pe.stride(1)
    nblk, page, row = kv_cache.shape
    if row != D_ROW or kv_cache.stride(2) != 1 or kv_cache.stride(1) != D_ROW:
        raise MlaError("kv_cache: expected [num_blocks, page_size, 576] with contiguous rows")
    B = seq_lens.shape[0]
    if query_start_loc.shape[0] != B + 1 or block_table.shape[0] != B or block_table.stride(1) != 1:
        raise MlaError("seq_lens/query_start_loc/block_table sizes disagree")
    if tuple(out.shape) != (T, H, D_LATENT) or (T and not out.is_contiguous()):
        raise MlaError("out: expected contiguous [T,H,512]")
    if tuple(lse.shape) != (T, H) or (T and not lse.is_contiguous()):
        raise MlaError("lse: expected contiguous [T,H]")
    if not (seq_lens.is_contiguous() and query_start_loc.is_contiguous()):
        raise MlaError("seq_lens/query_start_loc must be contiguous")
    _row_keys_ok(row_keys, T)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.mla_decode_partial(
        _ptr(q_nope), qn_st, qn_sh,
        _ptr(q_pe), qp_st, qp_sh,
        _ptr(kv_cache), kv_dtype, kv_sc, kv_cache.stride(0), page,
        _ptr(block_table), block_table.stride(0),
        _ptr(seq_lens), _ptr(query_start_loc),
        B, T, H, int(max_query_len), int(max_seq_len), int(cp_world), int(cp_rank), int(cp_interleave),
        int(mask_mode), float(scale),
        int(num_splits), _ptr(out), out_dtype, _ptr(lse), _ptr(row_keys), _ptr(workspace), ws_bytes,
        _stream(stream))
    _check(st, "mla_decode_partial")


def _row_keys_ok(row_keys, T):
    if row_keys is None:
        return
    _need(row_keys, torch.int32, "row_keys", 1)
    if row_keys.shape[0] != T or not row_keys.is_contiguous():
        raise MlaError("row_keys: expected contiguous int32 [T]")


def mla_decode_partial_noalloc(q_nope, q_pe, kv_cache, block_table, seq_lens, query_start_loc,
                               cp_world, cp_rank, scale, out, lse, *, max_query_len, max_seq_len,
                               num_splits=0, stream=None, cp_interleave=1, mask_mode=MASK_CAUSAL, kv_scale=None,
                               row_keys=None):
    """mla_decode_partial without a workspace (the library's per-GPU scratch array
    holds the split partials): for callers that cannot allocate."""
    lib = load_library()
    out_dtype = _partial_dtype(out, "out")
    kv_dtype, kv_sc = _kv_dtype(kv_cache, kv_scale)
    for t, dt, n, d in ((q_nope, torch.bfloat16, "q_nope", 3), (q_pe, torch.bfloat16, "q_pe", 3),
                        (kv_cache, kv_cache.dtype, "kv_cache", 3), (block_table, torch.int32, "block_table", 2),
                        (seq_lens, torch.int32, "seq_lens", 1), (query_start_loc, torch.int32, "query_start_loc", 1),
                        (out, out.dtype, "out", 3), (lse, torch.float32, "lse", 2)):
        _need(t, dt, n, d)
    T, H, _ = q_nope.shape
    nblk, page, row = kv_cache.shape
    if row != D_ROW or kv_cache.stride(1) != D_ROW or tuple(out.shape) != (T, H, D_LATENT) or tuple(lse.shape) != (T, H):
        raise MlaError("mla_decode_partial_noalloc: shapes disagree")
    if T and not (out.is_contiguous() and lse.is_contiguous() and q_nope.stride(2) == 1 and q_pe.stride(2) == 1):
        raise MlaError("mla_decode_partial_noalloc: out/lse contiguous, q rows contiguous")
    _row_keys_ok(row_keys, T)
    B = seq_lens.shape[0]
    st = lib.mla_decode_partial_noalloc(
        _ptr(q_nope), q_nope.stride(0), q_nope.stride(1), _ptr(q_pe), q_pe.stride(0), q_pe.stride(1),
        _ptr(kv_cache), kv_dtype, kv_sc, kv_cache.stride(0), page, _ptr(block_table), block_table.stride(0),
        _ptr(seq_lens), _ptr(query_start_loc), B, T, H, int(max_query_len), int(max_seq_len),
        int(cp_world), int(cp_rank), int(cp_interleave), int(mask_mode), float(scale), int(num_splits),
        _ptr(out), out_dtype, _ptr(lse), _ptr(row_keys), _stream(stream))
    _check(st, "mla_decode_partial_noalloc")


def mla_lse_merge(outs, lses, valid, out, out_lse=None, stream=None):
    """Merge W partials: outs [W,T,H,512] bf16 or fp32, lses [W,T,H] fp32, valid [W,T] int32 or None."""
    lib = load_library()
    outs_dtype = _partial_dtype(outs, "outs")
    _need(outs, outs.dtype, "outs", 4)
    _need(lses, torch.float32, "lses", 3)
    W, T, H, d = outs.shape
    if d != D_LATENT or tuple(lses.shape) != (W, T, H) or (T and not (outs.is_contiguous() and lses.is_contiguous())):
        raise MlaError("outs/lses: expected contiguous [W,T,H,512] / [W,T,H]")
    if valid is not None:
        _need(valid, torch.int32, "valid", 2)
        if tuple(valid.shape) != (W, T) or not valid.is_contiguous():
            raise MlaError("valid: expected contiguous [W,T]")
    _need(out, torch.bfloat16, "out", 3)
    if tuple(out.shape) != (T, H, D_LATENT) or not out.is_contiguous():
        raise MlaError("out: expected contiguous [T,H,512]")
    if out_lse is not None:
        _need(out_lse, torch.float32, "out_lse", 2)
        if tuple(out_lse.shape) != (T, H) or not out_lse.is_contiguous():
            raise MlaError("out_lse: expected contiguous [T,H]")
    st = lib.mla_lse_merge(_ptr(outs), outs_dtype, _ptr(lses), _ptr(valid), W, T, H, _ptr(out), _ptr(out_lse),
                           _stream(stream))
    _check(st, "mla_lse_merge")


def mla_merge_v_up_proj(outs, lses, valid, W_UV, out, out_lse=None, stream=None):
    """Merge W partials (bf16 or fp32) and project by W_UV [H,512,128]: out [T,H,128] bf16."""
    lib = load_library()
    outs_dtype = _partial_dtype(outs, "outs")
    _need(outs, outs.dtype, "outs", 4)
    _need(lses, torch.float32, "lses", 3)
    _need(W_UV, torch.bfloat16, "W_UV", 3)
    W, T, H, d = outs.shape
    if d != D_LATENT or tuple(lses.shape) != (W, T, H) or (T and not (outs.is_contiguous() and lses.is_contiguous())):
        raise MlaError("outs/lses: expected contiguous [W,T,H,512] / [W,T,H]")
    if tuple(W_UV.shape) != (H, D_LATENT, D_V) or not W_UV.is_contiguous():
        raise MlaError("W_UV: expected contiguous [H,512,128]")
    if valid is not None:
        _need(valid, torch.int32, "valid", 2)
        if tuple(valid.shape) != (W, T) or not valid.is_contiguous():
            raise MlaError("valid: expected contiguous [W,T]")
    _need(out, torch.bfloat16, "out", 3)
    if tuple(out.shape) != (T, H, D_V) or not out.is_contiguous():
        raise MlaError("out: expected contiguous [T,H,128]")
    if out_lse is not None:
        _need(out_lse, torch.float32, "out_lse", 2)
        if tuple(out_lse.shape) != (T, H) or not out_lse.is_contiguous():
            raise MlaError("out_lse: expected contiguous [T,H]")
    st = lib.mla_merge_v_up_proj(_ptr(outs), outs_dtype, _ptr(lses), _ptr(valid), W, T, H, _ptr(W_UV), _ptr(out),
                                 _ptr(out_lse), _stream(stream))
    _check(st, "mla_merge_v_up_proj")


def mla_dcp_a2a_pack(out_r, lse_r, valid_r, W_UV, send_y, send_lse, cp_world, stream=None):
    """Rank r's projected send buffers: send_y [W,T,H/W,128] bf16, send_lse [W,T,H/W] fp32."""
    lib = load_library()
    out_dtype = _partial_dtype(out_r, "out_r")
    _need(out_r, out_r.dtype, "out_r", 3)
    _need(lse_r, torch.float32, "lse_r", 2)
    _need(W_UV, torch.bfloat16, "W_UV", 3)
    _need(send_y, torch.bfloat16, "send_y", 4)
    _need(send_lse, torch.float32, "send_lse", 3)
    T, H, dn = out_r.shape
    W = int(cp_world)
    if dn != D_LATENT or W < 1 or H % W or tuple(lse_r.shape) != (T, H) or tuple(W_UV.shape) != (H, D_LATENT, 128):
        raise MlaError("mla_dcp_a2a_pack: expected out_r [T,H,512], lse_r [T,H], W_UV [H,512,128], H % W == 0")
    if tuple(send_y.shape) != (W, T, H // W, 128) or tuple(send_lse.shape) != (W, T, H // W):
        raise MlaError("mla_dcp_a2a_pack: send_y [W,T,H/W,128] / send_lse [W,T,H/W] expected")
    for t, n in ((out_r, "out_r"), (lse_r, "lse_r"), (W_UV, "W_UV"), (send_y, "send_y"), (send_lse, "send_lse")):
        if T and not t.is_contiguous():
            raise MlaError(f"{n}: must be contiguous")
    if valid_r is not None:
        _need(valid_r, torch.int32, "valid_r", 1)
        if valid_r.shape[0] != T or not valid_r.is_contiguous():
            raise MlaError("valid_r: expected contiguous [T]")
    st = lib.mla_dcp_a2a_pack(_ptr(out_r), out_dtype, _ptr(lse_r), _ptr(valid_r), T, H, W, _ptr(W_UV), _ptr(send_y),
                              _ptr(send_lse), _stream(stream))
    _check(st, "mla_dcp_a2a_pack")


def mla_dcp_a2a_combine(recv_y, recv_lse, out, out_lse=None, stream=None):
    """Merge the W received slices recv_y [W,T,Hs,128] / recv_lse [W,T,Hs] (any stride
    along W, each slice contiguous) into out [T,Hs,128] and out_lse [T,Hs]."""
    lib = load_library()
    _need(recv_y, torch.bfloat16, "recv_y", 4)
    _need(recv_lse, torch.float32, "recv_lse", 3)
    _need(out, torch.bfloat16, "out", 3)
    W, T, Hs, dv = recv_y.shape
    if dv != 128 or tuple(recv_lse.shape) != (W, T, Hs) or tuple(out.shape) != (T, Hs, 128):
        raise MlaError("mla_dcp_a2a_combine: recv_y [W,T,Hs,128], recv_lse [W,T,Hs], out [T,Hs,128] expected")
    if T and Hs and not (recv_y[0].is_contiguous() and recv_lse[0].is_contiguous() and out.is_contiguous()):
        raise MlaError("mla_dcp_a2a_combine: every slice and out must be contiguous")
    if out_lse is not None:
        _need(out_lse, torch.float32, "out_lse", 2)
        if tuple(out_lse.shape) != (T, Hs) or not out_lse.is_contiguous():
            raise MlaError("out_lse: expected contiguous [T,Hs]")
    st = lib.mla_dcp_a2a_combine(_ptr(recv_y), recv_y.stride(0), _ptr(recv_lse), recv_lse.stride(0), W, T, Hs,
                                 _ptr(out), _ptr(out_lse), _stream(stream))
    _check(st, "mla_dcp_a2a_combine")


SINK_WORDS = 1 << 20          # MLA_CALIB_SINK_WORDS


def calib_hbm_read(buf, sink, nontemporal=False, stream=None):
    """Read every byte of the GPU tensor ``buf`` once (calibration of the HBM
    read rate); ``sink`` is an int32/uint32 GPU tensor of at least 2^20 words."""
    lib = load_library()
    if not buf.is_cuda or not buf.is_contiguous() or not sink.is_cuda or sink.numel() * sink.element_size() < 4 * SINK_WORDS:
        raise MlaError("calib_hbm_read: contiguous GPU buffer and a 2^20-word GPU sink expected")
    _check(lib.mla_calib_hbm_read(_ptr(buf), buf.numel() * buf.element_size(), int(bool(nontemporal)), _ptr(sink),
                                  _stream(stream)), "mla_calib_hbm_read")


def calib_hbm_gather(buf, bytes_per_input, inputs, stream=None) -> int:
    """Read ``inputs`` consecutive buffers of ``bytes_per_input`` bytes at the
    start of the GPU tensor ``buf`` and write their xor right after them (the
    merges' pattern); returns the bytes moved."""
    lib = load_library()
    need = (inputs + 1) * bytes_per_input
    if not buf.is_cuda or not buf.is_contiguous() or buf.numel() * buf.element_size() < need:
        raise MlaError("calib_hbm_gather: a contiguous GPU buffer of (inputs + 1) * bytes_per_input bytes expected")
    base = buf.data_ptr()
    _check(lib.mla_calib_hbm_gather(ctypes.c_void_p(base), int(bytes_per_input), int(inputs),
                                    ctypes.c_void_p(base + inputs * bytes_per_input), _stream(stream)),
           "mla_calib_hbm_gather")
    return need


def calib_mfma_bf16(iters, sink, stream=None) -> float:
    """Enqueue the register-resident bf16 MFMA loop; returns the flops it performs."""
    lib = load_library()
    if not sink.is_cuda or sink.numel() * sink.element_size() < 4 * SINK_WORDS:
        raise MlaError("calib_mfma_bf16: a 2^20-word GPU sink expected")
    _check(lib.mla_calib_mfma_bf16(int(iters), _ptr(sink), _stream(stream)), "mla_calib_mfma_bf16")
    return float(lib.mla_calib_mfma_flops(int(iters)))


def mla_dcp_local_seqlens(seq_lens, query_start_loc, T, cp_world, cp_rank, row_seqlen=None,
                          shard_len=None, stream=None, cp_interleave=1, mask_mode=MASK_CAUSAL):
    """Per-row visible key counts [T] and per-request stored token counts [B] on rank cp_rank."""
    lib = load_library()
    _need(seq_lens, torch.int32, "seq_lens", 1)
    _need(query_start_loc, torch.int32, "query_start_loc", 1)
    B = seq_lens.shape[0]
    if row_seqlen is not None:
        _need(row_seqlen, torch.int32, "row_seqlen", 1)
        if row_seqlen.shape[0] != T:
            raise MlaError("row_seqlen: expected [T]")
    if shard_len is not None:
        _need(shard_len, torch.int32, "shard_len", 1)
        if shard_len.shape[0] != B:
            raise MlaError("shard_len: expected [B]")
    st = lib.mla_dcp_local_seqlens(_ptr(seq_lens), _ptr(query_start_loc), B, int(T), int(cp_world),
                                   int(cp_rank), int(cp_interleave), int(mask_mode), _ptr(row_seqlen),
                                   _ptr(shard_len), _stream(stream))
    _check(st, "mla_dcp_local_seqlens")
