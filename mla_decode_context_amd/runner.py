"""Drive one DCP decode step on one GPU through the C ABI.

All W ranks' paged caches live on the same GPU as separate tensors.  One step
is: every rank's partial attention (``mla_decode_partial`` with cp_rank = r),
the per-row valid counts of every rank (``mla_dcp_local_seqlens``), then the
merge -- ``mla_lse_merge``, or ``mla_merge_v_up_proj`` when W_UV is given.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as mla


def _bf16(a: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bits (host) -> bf16 tensor on the device."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


def _i32(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


class DeviceWorkload:
    """Device copies of a ``workloads.Workload`` plus output buffers."""

    def __init__(self, wl, device="cuda", num_splits: int = 0, partial_dtype=None):
        self.wl = wl
        self.device = torch.device(device)
        dev = self.device
        self.B, self.T, self.H, self.W = wl.B, wl.T, wl.H, wl.W
        self.I = wl.I                  # shard run length of the layout
        self.scale = wl.scale
        self.max_query_len = wl.max_query_len
        self.max_seq_len = wl.max_seq_len
        self.num_splits = num_splits
        self.q_nope = _bf16(wl.q_nope, dev)
        self.q_pe = _bf16(wl.q_pe, dev)
        self.seq_lens = _i32(wl.seq_lens, dev)
        self.qsl = _i32(wl.query_start_loc, dev)
        # bf16 caches, or FP8 E4M3 codes (uint8) with the cache's scale
        self.kv_scale = wl.kv_scale
        self.caches = [_bf16(sh.cache, dev) if wl.kv_scale is None else torch.from_numpy(sh.cache).to(dev)
                       for sh in wl.shards]
        self.tables = [_i32(sh.block_table, dev) for sh in wl.shards]
        self.w_uv = _bf16(wl.w_uv, dev) if wl.w_uv is not None else None
        T, H, W = self.T, self.H, self.W
        # per-rank partials: bf16 by default, fp32 when asked for
        self.outs = torch.empty((W, T, H, 512), dtype=partial_dtype or torch.bfloat16, device=dev)
        self.lses = torch.empty((W, T, H), dtype=torch.float32, device=dev)
        self.valid = torch.empty((W, T), dtype=torch.int32, device=dev)
        self.out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
        self.out_proj = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev) if self.w_uv is not None else None
        self.out_lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        self.alloc_workspace(num_splits)

    def alloc_workspace(self, num_splits: int):
        self.num_splits = num_splits
        n = mla.workspace_size(self.B, self.T, self.H, self.max_query_len, self.max_seq_len, self.W, num_splits,
                               cp_interleave=self.I)
        # zero-filled once: the split tickets must start at zero (calls reset them)
        self.workspace = torch.zeros(n, dtype=torch.uint8, device=self.device) if n else None

    def decode_kernel_name(self) -> str:
        """Kernels one mla_decode_partial call launches for this shape (with the
        automatic split plan), joined by "+"."""
        if self.H % 64 == 0:
            page32 = "true" if self.wl.P % 32 == 0 else "false"
            runs = "true" if self.I != 1 else "false"
            name = f"decode_kernel_h128<{page32}, {runs}>"
            if self.workspace is None:
                return name
            # the workspace holds the dispatch order (one int32 item and one int2
            # {request, keys} per token and 64-head block, each 256-byte aligned)
            # and, when rows are split, the partials
            hb = self.H // 64
            order_only = -(-self.T * hb * 4 // 256) * 256 + -(-self.T * hb * 8 // 256) * 256 + 256
            name = "h128_order_kernel+" + name
            return name + "+combine_fixed_kernel" if self.workspace.numel() > order_only else name
        page16 = "true" if self.wl.P % 16 == 0 else "false"
        fp8 = "true" if self.kv_scale is not None else "false"
        if self.H <= 16:
            if self.num_splits == 0 and self.workspace is not None:
                runs = "true" if self.I != 1 or (fp8 == "true" and page16 == "false") else "false"
                return f"decode_kernel_h16<{page16}, true, {runs}, {fp8}>+split_combine_kernel"
            return f"decode_kernel_h16<{page16}, false, true, {fp8}>"
        return f"decode_kernel<2, 3, {page16}>"

    def partial(self, r: int, stream=None):
        """Rank r's partial, and its rows' key counts into valid[r] (the merge's
        valid counts, written by the decode's own launches)."""
        mla.mla_decode_partial(
            self.q_nope, self.q_pe, self.caches[r], self.tables[r], self.seq_lens, self.qsl,
            self.W, r, self.scale, self.outs[r], self.lses[r],
            max_query_len=self.max_query_len, max_seq_len=self.max_seq_len,
            workspace=self.workspace, num_splits=self.num_splits, stream=stream, cp_interleave=self.I,
            kv_scale=self.kv_scale, row_keys=self.valid[r])

    def valid_counts(self, stream=None):
        """The same counts through mla_dcp_local_seqlens (one launch per rank)."""
        for r in range(self.W):
            mla.mla_dcp_local_seqlens(self.seq_lens, self.qsl, self.T, self.W, r,
                                      row_seqlen=self.valid[r], stream=stream, cp_interleave=self.I)

    # ---- the two-stage decode (query rows > 1): context stage per rank, one
    # query stage over the query tokens' own KV, merge of the W + 1 partials ----

    def setup_two_stage(self):
        from . import workloads as WL
        rows, table, qlens = WL.query_part_layout(self.wl)
        dev = self.device
        T, H, W = self.T, self.H, self.W
        self.qkv = (_bf16(rows, dev) if self.kv_scale is None else torch.from_numpy(rows).to(dev)).view(T, 1, 576)
        self.q_table = _i32(table, dev)
        self.q_lens = _i32(qlens, dev)
        dt = self.outs.dtype
        self.outs2 = torch.empty((W + 1, T, H, 512), dtype=dt, device=dev)
        self.lses2 = torch.empty((W + 1, T, H), dtype=torch.float32, device=dev)
        self.valid2 = torch.empty((W + 1, T), dtype=torch.int32, device=dev)
        n = mla.workspace_size(self.B, T, H, self.max_query_len, self.max_query_len, 1, self.num_splits)
        self.q_workspace = torch.zeros(n, dtype=torch.uint8, device=dev) if n else None

    def context_partial(self, r: int, stream=None):
        mla.mla_decode_partial(
            self.q_nope, self.q_pe, self.caches[r], self.tables[r], self.seq_lens, self.qsl,
            self.W, r, self.scale, self.outs2[r], self.lses2[r],
            max_query_len=self.max_query_len, max_seq_len=self.max_seq_len, workspace=self.workspace,
            num_splits=self.num_splits, stream=stream, cp_interleave=self.I, mask_mode=mla.MASK_CONTEXT,
            kv_scale=self.kv_scale, row_keys=self.valid2[r])

    def query_partial(self, stream=None):
        mla.mla_decode_partial(
            self.q_nope, self.q_pe, self.qkv, self.q_table, self.q_lens, self.qsl, 1, 0, self.scale,
            self.outs2[self.W], self.lses2[self.W], max_query_len=self.max_query_len,
            max_seq_len=self.max_query_len, workspace=self.q_workspace, num_splits=self.num_splits, stream=stream,
            kv_scale=self.kv_scale, row_keys=self.valid2[self.W])

    def two_stage_counts(self, stream=None):
        """The two stages' counts through mla_dcp_local_seqlens (the partials
        already write them)."""
        for r in range(self.W):
            mla.mla_dcp_local_seqlens(self.seq_lens, self.qsl, self.T, self.W, r, row_seqlen=self.valid2[r],
                                      stream=stream, cp_interleave=self.I, mask_mode=mla.MASK_CONTEXT)
        mla.mla_dcp_local_seqlens(self.q_lens, self.qsl, self.T, 1, 0, row_seqlen=self.valid2[self.W],
                                  stream=stream)

    def two_stage_step(self, stream=None):
        """The two-stage path: every rank's context partial, the query partial,
        their counts and the merge of the W + 1 partials into out / out_lse
        (or out_proj with W_UV)."""
        for r in range(self.W):
            self.context_partial(r, stream)
        self.query_partial(stream)
        if self.w_uv is not None:
            mla.mla_merge_v_up_proj(self.outs2, self.lses2, self.valid2, self.w_uv, self.out_proj, self.out_lse,
                                    stream=stream)
        else:
            mla.mla_lse_merge(self.outs2, self.lses2, self.valid2, self.out, self.out_lse, stream=stream)

    def merge(self, stream=None):
        mla.mla_lse_merge(self.outs, self.lses, self.valid, self.out, self.out_lse, stream=stream)

    def merge_v_up(self, stream=None):
        mla.mla_merge_v_up_proj(self.outs, self.lses, self.valid, self.w_uv, self.out_proj, self.out_lse,
                                stream=stream)

    def step(self, stream=None):
        """One pass of the whole path: all ranks' partials (with their valid
        counts), merge."""
        for r in range(self.W):
            self.partial(r, stream)
        if self.w_uv is not None:
            self.merge_v_up(stream)
        else:
            self.merge(stream)
