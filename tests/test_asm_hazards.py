"""Hazard checks on the gfx950 assembly of every kernel source (CPU only).

The direct-to-LDS loads are issued through inline asm, inside which the
compiler inserts no wait states of its own.  Two hardware rules apply to them:

* a VMEM instruction may read an SGPR only five wait states after a VALU
  instruction wrote it (the SGPR base of ``global_load_lds_dwordx4 v, s[a:b]``
  is assembled with ``v_readfirstlane``);
* the LDS address of the load comes from M0, which needs one wait state after
  the ``s_mov_b32 m0`` that sets it.

M0 is also not a clobber LLVM honours, so the asm may only own it if nothing
else in the compiled kernels reads or writes it.  This test compiles each
source to assembly with the library's own flags and checks all three.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

import pytest

from mla_decode_context_amd import build as B

# Instructions that read M0 implicitly (besides the LDS-DMA loads themselves).
_IMPLICIT_M0 = ("s_movrel", "v_movrel", "s_set_gpr_idx", "v_interp", "s_sendmsg", "s_ttracedata",
                "ds_gws", "ds_ordered", "buffer_load_lds", "s_buffer_load_lds")


def _compile(src: str, out: str):
    extra = dict(B.SOURCES)[src]
    cmd = [B.hipcc(), *B.HIPCC_FLAGS, *extra, "-I", os.path.join(B.ROOT, "include"), "-I", B.CSRC,
           "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read()


def _instructions(text: str):
    """(mnemonic, operands, is_label) for every instruction and label line."""
    out = []
    for line in text.splitlines():
        s = line.split(";")[0].strip()
        if not s or s.startswith("."):
            continue
        if s.endswith(":"):
            out.append((None, s, True))
            continue
        parts = s.split(None, 1)
        out.append((parts[0], parts[1] if len(parts) > 1 else "", False))
    return out


def _sgprs(op: str):
    """SGPR numbers named by one operand (sN or s[a:b])."""
    m = re.fullmatch(r"s(\d+)", op)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def _wait_states(mn: str, ops: str) -> int:
    if mn == "s_nop":
        return int(ops.strip(), 0) + 1
    return 1


def _check(text: str):
    ins = _instructions(text)
    n_lds_dma = 0
    for k, (mn, ops, lab) in enumerate(ins):
        if lab:
            continue
        if mn.startswith("global_load_lds"):
            n_lds_dma += 1
            # M0 set by the instruction two before, with a nop in between.
            assert k >= 2 and ins[k - 1][0] == "s_nop" and ins[k - 2][0] == "s_mov_b32" \
                and ins[k - 2][1].startswith("m0,"), f"LDS-DMA load {k} without 's_mov_b32 m0; s_nop' before it"
            args = [a.strip() for a in ops.split(",")]
            base = _sgprs(args[1].split()[0]) if len(args) > 1 else set()   # drop modifiers (nt, ...)
            if base:
                # Walk back to the last VALU write of a base SGPR.
                ws, j = 0, k - 1
                while j >= 0 and ws < 5:
                    pmn, pops, plab = ins[j]
                    if plab:
                        break
                    if pmn.startswith("v_"):
                        dst = pops.split(",")[0].strip()
                        assert not (_sgprs(dst) & base), \
                            f"{pmn} writes {dst} {ws} wait states before {mn} {ops} (needs 5)"
                    ws += _wait_states(pmn, pops)
                    j -= 1
                assert ws >= 5, f"{mn} {ops}: only {ws} wait states known before it (label reached)"
        # M0: written only by the loads' own s_mov, read only by the loads.
        if re.search(r"\bm0\b", ops):
            assert mn == "s_mov_b32" and ops.startswith("m0,") and k + 2 < len(ins) \
                and ins[k + 2][0] is not None and ins[k + 2][0].startswith("global_load_lds"), \
                f"M0 used outside the LDS-DMA asm: {mn} {ops}"
        assert not mn.startswith(_IMPLICIT_M0), f"{mn} reads M0 implicitly"
    return n_lds_dma


@pytest.mark.parametrize("src", [s for s, _ in B.SOURCES])
def test_lds_dma_wait_states_and_m0(src):
    with tempfile.TemporaryDirectory() as d:
        text = _compile(src, os.path.join(d, "k.s"))
    n = _check(text)
    if src in ("mla_decode.hip", "mla_decode_h128.hip", "mla_merge.hip"):
        assert n > 0, "expected LDS-DMA loads in this source"


def test_checker_sees_a_short_gap():
    # The pattern the compiler produced before the fix: a readfirstlane two
    # wait states before the load that reads its SGPR.
    bad = ("\tv_readfirstlane_b32 s79, v3\n\tv_readfirstlane_b32 s78, v2\n\ts_mov_b32 m0, s99\n"
           "\ts_nop 0\n\tglobal_load_lds_dwordx4 v212, s[78:79] nt\n")
    with pytest.raises(AssertionError):
        _check(bad)
    good = bad.replace("s_nop 0", "s_nop 4")
    assert _check(good) == 1
    with pytest.raises(AssertionError):
        _check("\ts_mov_b32 m0, s1\n\tv_mov_b32 v0, m0\n")


def _vector_load_waits_before_dma(text: str, window: int = 40):
    """Places where a 32-bit vector load is waited for with vmcnt(0) within
    `window` instructions before an LDS-DMA load: the shape of a block id read
    through the vector memory path, whose wait also waits for every stage load
    in flight.  Block ids are read with scalar loads, so there must be none."""
    ins = [(mn, ops) for mn, ops, lab in _instructions(text) if not lab]
    found = []
    for k, (mn, ops) in enumerate(ins):
        if not mn.startswith("global_load_lds"):
            continue
        seen_wait = False
        for j in range(k - 1, max(k - window, -1), -1):
            pmn, pops = ins[j]
            if pmn.startswith("global_load_lds"):
                break                      # an earlier load of the same stage
            if pmn == "s_waitcnt" and "vmcnt(0)" in pops:
                seen_wait = True
            elif pmn == "global_load_dword" and seen_wait:
                found.append(k)
                break
    return found


@pytest.mark.parametrize("src", ["mla_decode.hip", "mla_decode_h128.hip"])
def test_stage_issue_reads_block_ids_with_scalar_loads(src):
    with tempfile.TemporaryDirectory() as d:
        text = _compile(src, os.path.join(d, "k.s"))
    assert _vector_load_waits_before_dma(text) == []


def test_vector_block_id_check_sees_the_old_shape():
    bad = ("\tglobal_load_dword v3, v[84:85], off\n\tv_mul_lo_u32 v2, v2, s56\n\ts_waitcnt vmcnt(0)\n"
           "\tv_readfirstlane_b32 s88, v2\n\ts_mov_b32 m0, s4\n\ts_nop 0\n"
           "\tglobal_load_lds_dwordx4 v212, s[88:89] nt\n")
    assert _vector_load_waits_before_dma(bad) == [6]
    good = bad.replace("global_load_dword v3, v[84:85], off", "s_load_dword s3, s[84:85], 0x0")
    assert _vector_load_waits_before_dma(good) == []
