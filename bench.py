"""Benchmark of the absorbed-MLA DCP decode path on one MI355X.

Default workload (the headline line): long-context DCP decode, batch 256, two
query rows per request (MTP), 128 heads, W = 8 shards simulated on the one GPU,
contexts drawn uniformly from 8192..32768 tokens (four requests shortened so
that some shards hold empty rows), page 64 with permuted physical blocks.  One
step = one pass of the whole path over that batch: every shard's
mla_decode_partial (row seqlens, paged gather, scores, masked online softmax,
PV, split-K where the plan splits, finalise; each call also writes its rows'
valid counts), and the LSE merge of the eight partials.

Other workloads (reported under "configs", not in the headline value): the
plain 16-head decode (W = 1, no merge), the MTP DCP4 step, the mixed batch
whose merge is fused with W_UV, and the whole-page DCP4 layout.  Merge figures
time the merge where a step runs it, right after the shard decodes;
``merge_*_back_to_back`` repeats the merge alone, which for partials that fit
in the 256 MB last-level cache reads them from there.  The W_UV workload also
times the projected exchange's two kernels.

Printed: one JSON line.  ``value`` is KV-cache GB/s of the whole step (bytes of
cache rows the method must read once, divided by the step time) with inputs
already resident in HBM.  ``roofline`` is the dominant kernel's algorithmic
flops (or bytes, for an HBM-bound workload) per call over its average call
duration, measured with HIP events on the launch stream: for a one-call step
(the plain workloads) the timed region's own pair of events, otherwise one
pair around `steps` passes over every shard's decode, issued back to back as a
step issues them (events between the calls of the timed region would idle the
GPU a few microseconds each); ``calibration`` holds what a streaming
read and a register-resident MFMA loop reach on the same GPU (the roofline is
also given as a fraction of those); ``cpu_baseline`` times the fp64 oracle on
the host for a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "MLA decode KV GB/s (% of HBM peak) + query-tokens/s; merge GB/s"


def workload_bytes(wl, valid):
    """Algorithmic bytes and flops of one step, per shard call.

    valid [W,T] holds every row's visible key count on every rank (from the
    library's own mla_dcp_local_seqlens).  Bytes: each stored cache row once
    (1152 B), q once (H*1152 B per row), out + LSE once (H*1028 B per row).
    Flops: 2176 per visible (key, head, row) -- 1152 for the scores, 1024 for PV.
    """
    per_shard = []
    row_bytes = 576 if wl.kv_scale is not None else 1152      # FP8 E4M3 or bf16 cache rows
    for r in range(wl.W):
        kv_tokens = int(sum(sh for sh in wl.shards[r].token_counts))
        flops = float(valid[r].astype(np.float64).sum()) * wl.H * 2176.0
        kv = kv_tokens * row_bytes
        q = wl.T * wl.H * 1152
        out = wl.T * wl.H * 1028
        per_shard.append(dict(kv=kv, q=q, out=out, flops=flops, total=kv + q + out))
    return per_shard


def merge_bytes(wl, valid, proj: bool):
    """Bytes the merge must move: participating partials + LSEs read, result written."""
    n_part = int((valid > 0).sum()) * wl.H      # participating (rank, t, h) rows
    read = n_part * (1024 + 4)
    write = wl.T * wl.H * ((256 if proj else 1024) + 4)
    wuv = wl.H * 512 * 128 * 2 if proj else 0
    flops = wl.T * wl.H * 2.0 * 512 * 128 if proj else 0.0
    return read + write + wuv, flops


# Sources that build each measured kernel: a traffic record stays valid while
# the sources it names are unchanged.
DECODE16_SOURCES = ["mla_api.hip", "mla_common.h", "mla_decode.hip", "mla_device.h", "mla_kernels.h"]
H128_SOURCES = ["mla_api.hip", "mla_common.h", "mla_decode_h128.hip", "mla_device.h", "mla_kernels.h"]
MERGE_SOURCES = ["mla_api.hip", "mla_common.h", "mla_merge.hip", "mla_device.h", "mla_kernels.h"]


def strip_comments(src: str) -> str:
    """C/C++ source without its comments, whitespace runs collapsed: what the
    compiler sees, so that an edit of comments alone keeps a measurement valid."""
    out = []
    i, n = 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":                      # string or character literal, kept whole
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(files=None) -> str:
    """Hash of the given kernel sources (file names under the package's csrc/;
    all of them when None), comments and whitespace left out."""
    csrc = os.path.join(ROOT, "mla_decode_context_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(files if files is not None else os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(strip_comments(fh.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM traffic measured with rocprofv3 counters for this kernel source, if any."""
    path = os.path.join(ROOT, "profiles", f"decode_kernel_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash(rec.get("kernel_sources")):
        return None
    return rec.get("bytes_per_launch")


def time_workload(name, steps, warmup, torch, wl=None, headline=False, cold=True, alternate=False):
    from mla_decode_context_amd import workloads as WL
    from mla_decode_context_amd.runner import DeviceWorkload

    if wl is None:
        wl = WL.make_workload(name, threads=16)
    dw = DeviceWorkload(wl)
    dw.valid_counts()
    per_shard = workload_bytes(wl, dw.valid.cpu().numpy())
    proj = wl.w_uv is not None
    merging = wl.W > 1

    def step(evs=None):
        for r in range(wl.W):
            if evs is not None:
                evs[r][0].record()
            dw.partial(r)                 # also writes rank r's valid counts
            if evs is not None:
                evs[r][1].record()
        if merging:
            if evs is not None:
                evs[wl.W][0].record()
            dw.merge_v_up() if proj else dw.merge()
            if evs is not None:
                evs[wl.W][1].record()

    # With `alternate`, a second copy of every shard's cache: the timed steps
    # alternate between the two copies, so no call can find the rows that the
    # previous call read still in the 256 MB last-level cache (the copies hold
    # the same rows under the same block tables, so results are identical).
    # Workloads whose shards together exceed that cache need no copy.
    spare = [dw.caches[r].clone() for r in range(wl.W)] if alternate else None

    def swap():
        if spare is not None:
            for r in range(wl.W):
                dw.caches[r], spare[r] = spare[r], dw.caches[r]

    for _ in range(warmup):
        step()
        swap()
    torch.cuda.synchronize()
    # Timed region: the steps back to back, as a serving loop issues them, with
    # one pair of events around the whole region (on the launch stream, the
    # current stream).  Events between the steps' calls are left out: each one
    # costs the GPU a few microseconds of idle time (measured 12 us per 70 us
    # plain step).
    ev_a, ev_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_a.record()
    for k in range(steps):
        step()
        swap()
    ev_b.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    ev_ms_step = ev_a.elapsed_time(ev_b) / steps
    same_cache_ms = None
    if spare is not None:
        # The same steps on one cache copy (rows may survive in the last-level
        # cache between calls): reported beside the value, never as it.
        a2, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        step()
        a2.record()
        for k in range(steps):
            step()
        b2.record()
        torch.cuda.synchronize()
        same_cache_ms = a2.elapsed_time(b2) / steps
    # Breakdown: each operation of a step on its own, `steps` calls back to back
    # between two events (markers around every single call would add a few
    # microseconds to each): every shard's decode, then the merge.
    def loop_ms(op):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        op()
        a.record()
        for _ in range(steps):
            op()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    # With a spare cache copy the calls alternate between the copies here too.
    def partial_alt(r):
        dw.partial(r)
        swap()

    dec_avg = np.array([loop_ms(lambda r=r: partial_alt(r)) for r in range(wl.W)])   # per shard, ms
    # Every shard's decode back to back, as a step issues them (consecutive
    # calls read different shards' caches, so a shard whose cache fits in the
    # last-level cache gains nothing from the previous call): ms per shard.
    dec_step = loop_ms(lambda: [dw.partial(r) for r in range(wl.W)] + [swap()]) / wl.W
    spare = None                          # either copy holds the same rows
    mg_ms = mg_step_ms = None
    if merging:
        dw.valid_counts()
        mg_ms = loop_ms(dw.merge_v_up if proj else dw.merge)
        # The merge as a step runs it: right after every shard's decode, whose
        # partials it reads (events around the merge only).  Merges repeated
        # back to back re-read partials that a small step leaves in the 256 MB
        # last-level cache, so that figure is reported beside this one.
        mevs = []
        for _ in range(steps):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(wl.W + 1)]
            step(evs)
            mevs.append(evs[wl.W])
        torch.cuda.synchronize()
        mg_step_ms = float(np.median([a.elapsed_time(b) for a, b in mevs]))
    xchg = exchange_times(dw, wl, steps, torch) if merging and proj and wl.H % wl.W == 0 else None
    # The two-stage path (query rows > 1): every rank's context stage, the query
    # stage over the query tokens' own KV, the merge of the W + 1 partials;
    # timed as a whole step and per stage, beside the one-stage step above.
    two = None
    if wl.max_query_len > 1:
        dw.setup_two_stage()
        dw.two_stage_step()
        two = {"two_stage_ms_per_step": loop_ms(dw.two_stage_step),
               "two_stage_context_ms_per_shard": loop_ms(lambda: [dw.context_partial(r) for r in range(wl.W)]) / wl.W,
               "two_stage_query_ms": loop_ms(dw.query_partial)}
        two["two_stage_vs_one_stage"] = two["two_stage_ms_per_step"] / float(ev_ms_step)
    res = dict(workload=name, T=wl.T, B=wl.B, H=wl.H, W=wl.W, ms_per_step=ms_step)
    if xchg is not None:
        res.update(xchg)
    if two is not None:
        res.update(two)
    kv_total = sum(p["kv"] for p in per_shard)
    res["kv_GBps"] = kv_total / (ms_step * 1e-3) / 1e9
    res["query_tokens_per_s"] = wl.T / (ms_step * 1e-3)
    res["decode_ms_per_shard"] = [round(float(x), 4) for x in dec_avg]   # one shard's calls repeated
    res["decode_ms_per_shard_in_step"] = round(float(dec_step), 4)
    alg_bytes = np.array([p["total"] for p in per_shard], dtype=np.float64)
    alg_flops = np.array([p["flops"] for p in per_shard], dtype=np.float64)
    dec_all = dec_step * wl.W        # ms for every shard's decode of one step
    res["decode_alg_GBps"] = float(alg_bytes.sum() / (dec_all * 1e-3) / 1e9)
    res["decode_kv_GBps"] = float(sum(p["kv"] for p in per_shard) / (dec_all * 1e-3) / 1e9)
    res["decode_TFLOPs"] = float(alg_flops.sum() / (dec_all * 1e-3) / 1e12)
    res["decode_pct_bf16_peak"] = 100.0 * res["decode_TFLOPs"] / BF16_PEAK_TFLOPS
    res["decode_pct_hbm_peak"] = 100.0 * res["decode_alg_GBps"] / HBM_PEAK_GBPS
    # Roofline fraction of the decode calls: the longer of the two roofline
    # times (bytes at the HBM peak, flops at the dense bf16 peak) over the
    # measured time, summed over the shards.
    t_roof = np.maximum(alg_bytes / (HBM_PEAK_GBPS * 1e9), alg_flops / (BF16_PEAK_TFLOPS * 1e12))
    res["decode_roofline_frac"] = float(t_roof.sum() / (dec_all * 1e-3))
    res["decode_bound"] = "mfma" if alg_flops.sum() / (BF16_PEAK_TFLOPS * 1e12) > \
        alg_bytes.sum() / (HBM_PEAK_GBPS * 1e9) else "hbm"
    # one-rank view: the slowest rank's partial plus the merge (excludes the exchange)
    if merging:
        valid = dw.valid.cpu().numpy()
        mbytes, mflops = merge_bytes(wl, valid, proj)
        res["merge_kind"] = "merge+W_UV" if proj else "lse_merge"
        res["merge_ms"] = float(mg_step_ms)
        res["merge_GBps"] = mbytes / (mg_step_ms * 1e-3) / 1e9
        res["merge_pct_hbm_peak"] = 100.0 * res["merge_GBps"] / HBM_PEAK_GBPS
        res["merge_ms_back_to_back"] = float(mg_ms)
        res["merge_GBps_back_to_back"] = mbytes / (mg_ms * 1e-3) / 1e9
        res["query_tokens_per_s_one_rank"] = wl.T / ((dec_avg.max() + mg_step_ms) * 1e-3)
    res["ms_per_step_events"] = float(ev_ms_step)
    if same_cache_ms is not None:
        res["kv_GBps_same_cache"] = sum(p["kv"] for p in per_shard) / (same_cache_ms * 1e-3) / 1e9
    # Roofline of the decode calls (the dominant kernels): algorithmic bytes
    # and flops of the average call over its average duration (a call launches
    # the kernels decode_kernel_name() lists).  The duration: with one rank and
    # no merge a step is exactly one call, so the timed region's events over
    # the steps; otherwise a timed loop of `steps` passes over every shard's
    # decode, back to back as a step issues them, between one pair of events.
    res["_alg_bytes_per_launch"] = float(alg_bytes.mean())
    res["_alg_flops_per_launch"] = float(alg_flops.mean())
    res["_decode_avg_ms"] = float(ev_ms_step) if not merging else float(dec_step)
    res["_kernel"] = dw.decode_kernel_name()
    if headline:
        res["_cold_kv_GBps"] = cold_kv(dw, wl, per_shard, torch) if cold else None
    del dw
    torch.cuda.empty_cache()
    return res, wl


def exchange_times(dw, wl, steps, torch):
    """The projected exchange of the merge, the part one GPU holds: every rank's
    pack (projection by W_UV, by destination head slice), then every
    destination's combine of the slices it would receive, addressed in place in
    the ranks' send buffers (the transport between GPUs is not part of it).
    Timed where a step runs them, right after the shard decodes (median over
    `steps`, events around each phase)."""
    from mla_decode_context_amd import binding as mla
    W, T, H = wl.W, wl.T, wl.H
    Hs = H // W
    send_y = torch.empty((W, W, T, Hs, 128), dtype=torch.bfloat16, device="cuda")
    send_l = torch.empty((W, W, T, Hs), dtype=torch.float32, device="cuda")
    out = torch.empty((W, T, Hs, 128), dtype=torch.bfloat16, device="cuda")
    out_l = torch.empty((W, T, Hs), dtype=torch.float32, device="cuda")
    marks = []
    for _ in range(steps + 1):
        for r in range(W):
            dw.partial(r)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        for r in range(W):
            mla.mla_dcp_a2a_pack(dw.outs[r], dw.lses[r], dw.valid[r], dw.w_uv, send_y[r], send_l[r], W)
        ev[1].record()
        for q in range(W):
            mla.mla_dcp_a2a_combine(send_y[:, q], send_l[:, q], out[q], out_l[q])
        ev[2].record()
        marks.append(ev)
    torch.cuda.synchronize()
    marks = marks[1:]
    pack_ms = float(np.median([e[0].elapsed_time(e[1]) for e in marks])) / W
    comb_ms = float(np.median([e[1].elapsed_time(e[2]) for e in marks])) / W
    valid = dw.valid.cpu().numpy()
    rows_in = float((valid > 0).sum()) / W                  # participating rows per rank
    pack_bytes = rows_in * H * (1024 + 4) + T * H * (256 + 4) + H * 512 * 128 * 2
    comb_bytes = W * T * Hs * (256 + 4) + T * Hs * (256 + 4)
    return {"a2a_pack_ms_per_rank": pack_ms, "a2a_pack_GBps": pack_bytes / (pack_ms * 1e-3) / 1e9,
            "a2a_combine_ms_per_rank": comb_ms, "a2a_combine_GBps": comb_bytes / (comb_ms * 1e-3) / 1e9,
            "a2a_payload_bytes_per_peer": T * Hs * (256 + 4)}


def cold_kv(dw, wl, per_shard, torch, reps=7):
    """KV GB/s of one step started from an idle GPU whose 256 MB last-level
    cache was just flushed by reading 1 GiB (a read leaves no dirty lines whose
    write-back would compete with the decode)."""
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dw.device)
    times = []
    for _ in range(reps):
        float(flush.sum())
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for r in range(wl.W):
            dw.partial(r)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    del flush
    kv = sum(p["kv"] for p in per_shard)
    return kv / (float(np.median(times)) * 1e-3) / 1e9


def cpu_baseline(wl, budget_s=12.0):
    """The fp64 oracle on the host for the same workload: passes over the batch,
    request by request (every rank), until about budget_s seconds of oracle time
    are spent.  Generating the inputs is not timed."""
    from oracle import mla_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    qsl = wl.query_start_loc
    done_tokens = done_kv = reqs = 0
    spent = 0.0
    kv_cache = {}
    while spent < budget_s:
        for b in range(wl.B):
            if b not in kv_cache:
                kv_cache[b] = wl.global_kv(b)
            kv = kv_cache[b]
            toks = list(range(int(qsl[b]), int(qsl[b + 1])))
            t0 = time.perf_counter()
            for r in range(wl.W):
                O.decode_partial(wl.seq_lens, qsl, wl.q_nope, wl.q_pe, lambda _b: kv, wl.scale, wl.W, r,
                                 tokens=toks)
            spent += time.perf_counter() - t0
            done_tokens += len(toks)
            done_kv += int(sum(len(range(r, int(wl.seq_lens[b]), wl.W)) for r in range(wl.W))) * 1152
            reqs += 1
            if spent >= budget_s:
                break
    return dict(value=round(done_kv / spent / 1e9, 4), unit="GB/s", cores=int(threads), kind="oracle",
                cpu_model=cpu_model(),
                sample=f"fp64 oracle over {reqs} requests ({reqs / wl.B:.2f} passes over the {wl.B}-request "
                       f"batch, {done_tokens} query rows, every rank) in {spent:.1f} s; "
                       f"query-tokens/s {done_tokens / spent:.3g}",
                query_tokens_per_s=round(done_tokens / spent, 2))


def cpu_model() -> str:
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def calibrate(torch, reps=5):
    """What this GPU reaches for a streaming read of 4 GiB (plain and
    non-temporal loads; 16x the last-level cache) and for a register-resident
    bf16 MFMA loop.  Best of `reps` timed calls after one untimed call."""
    from mla_decode_context_amd import binding as mla
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(mla.SINK_WORDS, dtype=torch.int32, device="cuda")

    def best_ms(op):
        op()
        times = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            op()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        return min(times), float(np.median(times))

    rd, rd_med = best_ms(lambda: mla.calib_hbm_read(buf, sink, nontemporal=False))
    rn, rn_med = best_ms(lambda: mla.calib_hbm_read(buf, sink, nontemporal=True))
    # The merges' pattern: eight streams of 72 MiB read (2.3x the last-level
    # cache together), one written.
    gb = 72 << 20
    gbytes = (8 + 1) * gb
    rg, rg_med = best_ms(lambda: mla.calib_hbm_gather(buf, gb, 8))
    del buf
    iters = 40000
    flops = mla.calib_mfma_bf16(iters, sink)
    mf, mf_med = best_ms(lambda: mla.calib_mfma_bf16(iters, sink))
    del sink
    torch.cuda.empty_cache()
    return {"hbm_read_GBps": round(nbytes / (rd * 1e-3) / 1e9, 1),
            "hbm_read_GBps_median": round(nbytes / (rd_med * 1e-3) / 1e9, 1),
            "hbm_read_nt_GBps": round(nbytes / (rn * 1e-3) / 1e9, 1),
            "hbm_read_nt_GBps_median": round(nbytes / (rn_med * 1e-3) / 1e9, 1),
            "hbm_8read_1write_GBps": round(gbytes / (rg * 1e-3) / 1e9, 1),
            "hbm_8read_1write_GBps_median": round(gbytes / (rg_med * 1e-3) / 1e9, 1),
            "mfma_bf16_TFLOPs": round(flops / (mf * 1e-3) / 1e12, 1),
            "mfma_bf16_TFLOPs_median": round(flops / (mf_med * 1e-3) / 1e12, 1),
            "method": "mla_calib_hbm_read over 4 GiB (plain / non-temporal loads), mla_calib_hbm_gather "
                      "(8 x 72 MiB read, 72 MiB written), mla_calib_mfma_bf16 "
                      f"({iters} rounds of 8 chains of v_mfma_f32_16x16x32_bf16, 2 waves per SIMD); "
                      f"best of {reps} event-timed calls"}


def make_roofline(res, workload, calib=None):
    """Roofline object of a workload's decode calls: MFMA-bound when its flops
    at the bf16 peak take longer than its bytes at the HBM peak."""
    t_mem = res["_alg_bytes_per_launch"] / (HBM_PEAK_GBPS * 1e9)
    t_mfma = res["_alg_flops_per_launch"] / (BF16_PEAK_TFLOPS * 1e12)
    sec = res["_decode_avg_ms"] * 1e-3
    if t_mfma > t_mem:
        ach = res["_alg_flops_per_launch"] / sec / 1e12
        rl = {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
              "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": load_traffic(workload)}
        meas = calib.get("mfma_bf16_TFLOPs") if calib else None
    else:
        ach = res["_alg_bytes_per_launch"] / sec / 1e9
        rl = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
              "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": load_traffic(workload)}
        meas = calib.get("hbm_read_nt_GBps") if calib else None
    if meas:
        rl["achievable"] = meas
        rl["frac_of_achievable"] = round(ach / meas, 4)
    rl.update({"kernel": res["_kernel"], "avg_launch_ms": round(res["_decode_avg_ms"], 5),
               "alg_bytes_per_launch": int(res["_alg_bytes_per_launch"]),
               "alg_flops_per_launch": int(res["_alg_flops_per_launch"])})
    return rl


def copy_probe(torch, mib: int):
    """One plain device-to-device copy of mib MiB: the known-size kernel that HBM
    traffic counters are scaled by."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps first (the GPU's clocks settle over the first few thousand calls; "
                         "300 long_dcp8 steps are about 1 s)")
    ap.add_argument("--workload", default="long_dcp8")
    ap.add_argument("--configs", default="plain,plain_fp8,mtp_dcp4,mixed_wuv,mtp_dcp4_pages",
                    help="comma-separated secondary workloads ('' for none)")
    ap.add_argument("--config-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the flushed-cache (cold) decode timing")
    ap.add_argument("--no-calib", action="store_true", help="skip the HBM / MFMA calibration kernels")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run one plain copy of this many MiB (scale for traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (all DCP ranks are simulated on it); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch
    from mla_decode_context_amd import binding
    from mla_decode_context_amd import workloads as WL

    binding.load_library()
    torch.cuda.set_device(0)
    if args.copy_probe_mib > 0:
        copy_probe(torch, args.copy_probe_mib)
    calib = None
    if not args.no_calib:
        # First, so that the GPU has left its idle clocks before any workload
        # is timed (the calibration is a second or so of streaming reads and
        # MFMA loops).
        print("[bench] calibration: streaming read and MFMA loop", file=sys.stderr, flush=True)
        calib = calibrate(torch)
        print(f"[bench] calibration: {json.dumps(calib)}", file=sys.stderr, flush=True)
    print(f"[bench] {args.workload}: generating inputs", file=sys.stderr, flush=True)
    head, wl = time_workload(args.workload, args.steps, args.warmup, torch, headline=True,
                             cold=not args.no_cold, alternate=args.workload.startswith("plain"))
    print(f"[bench] {args.workload}: {head['ms_per_step']:.4f} ms/step, {head['kv_GBps']:.1f} GB/s",
          file=sys.stderr, flush=True)
    configs = {}
    for name in [c for c in args.configs.split(",") if c and c != args.workload]:
        print(f"[bench] {name}: generating inputs", file=sys.stderr, flush=True)
        plain_like = name.startswith("plain")      # 70 us steps: more of them
        res, _ = time_workload(name, 20 * args.config_steps if plain_like else args.config_steps,
                               300 if plain_like else 3, torch, alternate=plain_like)
        res["roofline"] = make_roofline(res, name, calib)
        if calib and res.get("merge_GBps"):
            res["merge_frac_of_achievable"] = res["merge_GBps"] / calib["hbm_8read_1write_GBps"]
        configs[name] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in res.items()
                         if not k.startswith("_")}
        print(f"[bench] {name}: {json.dumps(configs[name])}", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on the host", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl)
    roofline = make_roofline(head, args.workload, calib)
    cfg = WL.CONFIGS[args.workload]
    line = {
        "metric": METRIC,
        "value": round(head["kv_GBps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "desc": cfg["desc"], "batch": wl.B, "query_rows": wl.T,
                   "heads": wl.H, "dcp_world": wl.W, "page_size": wl.P, "seed": wl.seed},
        "pct_hbm_peak": round(100.0 * head["kv_GBps"] / HBM_PEAK_GBPS, 2),
        "query_tokens_per_s": round(head["query_tokens_per_s"], 1),
        "decode_ms_per_shard_in_step": head["decode_ms_per_shard_in_step"],
        "decode_pct_bf16_peak": round(head["decode_pct_bf16_peak"], 2),
        "kv_GBps_cold_llc": None if head.get("_cold_kv_GBps") is None else round(head["_cold_kv_GBps"], 2),
        "roofline": roofline,
        "merge_kind": head.get("merge_kind"),
        "merge_ms": None if head.get("merge_ms") is None else round(head["merge_ms"], 5),
        "merge_GBps": None if head.get("merge_GBps") is None else round(head["merge_GBps"], 1),
        "merge_pct_hbm_peak": None if head.get("merge_pct_hbm_peak") is None else round(head["merge_pct_hbm_peak"], 2),
        "merge_frac_of_achievable": None if not (calib and head.get("merge_GBps")) else
        round(head["merge_GBps"] / calib["hbm_8read_1write_GBps"], 4),
        "calibration": calib,
        "cpu_baseline": cpu,
        "configs": configs,
    }
    if "kv_GBps_same_cache" in head:
        line["kv_GBps_same_cache"] = round(head["kv_GBps_same_cache"], 2)
    for k in ("two_stage_ms_per_step", "two_stage_context_ms_per_shard", "two_stage_query_ms", "two_stage_vs_one_stage"):
        if k in head:
            line[k] = round(head[k], 5)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
