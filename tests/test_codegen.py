"""Code-generation guards (CPU only).

1. No MFMA may be issued while EXEC is narrowed by a divergent branch.
   MFMA instructions do not honour EXEC: an MFMA on a path that a wave skips
   through exec masking still runs and still writes (and accumulates into)
   its destination.  The kernels keep every branch around MFMAs
   wave-uniform (the wave index is read into a scalar register), so that
   the compiler emits scalar jumps there.  The check is a may-analysis over
   the basic blocks of the assembly: EXEC counts as narrowed at a block's
   entry if it is narrowed at the end of any predecessor (fallthrough or
   branch, loops iterated to a fixpoint); a saveexec narrows it, and an
   explicit restore of EXEC (s_or_b64 / s_mov_b64 into exec) ends it.

2. The recurrence's LDS-DMA inline assembly writes M0, which the compiler
   owns: it saves M0 to a scratch SGPR first and restores it after the load
   has issued.  The guard checks that every write of M0 in the recurrence
   kernels is one of those save / set / restore sequences around a
   buffer_load ... lds, so no value of the compiler's is ever lost."""

import os
import re
import shutil
import subprocess

import pytest

from chunked_kda_prefill_amd import build

KERNELS = ["kda_intra.hip", "kda_recurrence.hip"]

_BRANCH = re.compile(r"^s_(cbranch_\w+|branch)$")


def _instructions(asm: str):
    """(line number, opcode, text) of instructions and labels, in order."""
    out = []
    for i, line in enumerate(asm.split("\n")):
        # comments first: the compiler annotates labels (".LBB1_5:  ; in Loop")
        s = line.split(";")[0].strip()
        if not s or (s.startswith(".") and not s.endswith(":")):
            continue
        out.append((i + 1, s.split()[0], s))
    return out


def _narrows(op, text):
    return "saveexec" in op or (op in ("s_andn2_b64", "s_and_b64", "s_xor_b64")
                                and text.split()[1].rstrip(",") == "exec")


def _restores(op, text):
    if op == "s_or_b64" and re.match(r"s_or_b64\s+exec,\s*exec,", text):
        return True
    return op == "s_mov_b64" and text.split()[1].rstrip(",") == "exec"


def mfma_under_masked_exec(asm: str) -> list:
    """Line numbers of MFMAs that may issue while EXEC is narrowed."""
    ins = _instructions(asm)
    # basic blocks: split at labels and after branches / s_endpgm
    blocks, labels, cur = [], {}, []
    for item in ins:
        _, op, _ = item
        if op.endswith(":"):
            if cur:
                blocks.append(cur)
            cur = []
            labels[op[:-1]] = len(blocks)
            continue
        cur.append(item)
        if _BRANCH.match(op) or op == "s_endpgm":
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    # labels map to the next block created after them
    succ = []
    for b, blk in enumerate(blocks):
        s = []
        last = blk[-1] if blk else None
        if last and _BRANCH.match(last[1]):
            tgt = last[2].split()[1] if len(last[2].split()) > 1 else None
            if tgt in labels:
                s.append(labels[tgt])
            if last[1] != "s_branch" and b + 1 < len(blocks):
                s.append(b + 1)
        elif not last or last[1] != "s_endpgm":
            if b + 1 < len(blocks):
                s.append(b + 1)
        succ.append(s)
    entry = [False] * len(blocks)
    changed = True
    while changed:
        changed = False
        for b, blk in enumerate(blocks):
            st = entry[b]
            for _, op, text in blk:
                if _narrows(op, text):
                    st = True
                elif _restores(op, text):
                    st = False
            for t in succ[b]:
                if st and not entry[t]:
                    entry[t] = True
                    changed = True
    bad = []
    for b, blk in enumerate(blocks):
        st = entry[b]
        for ln, op, text in blk:
            if _narrows(op, text):
                st = True
            elif _restores(op, text):
                st = False
            elif op.startswith("v_mfma") and st:
                bad.append(ln)
    return sorted(bad)


def test_scanner_flags_masked_mfma():
    asm = "\n".join(["k:", "  s_and_saveexec_b64 s[0:1], vcc",
                     "  v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
                     "  s_or_b64 exec, exec, s[0:1]",
                     "  v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0"])
    assert mfma_under_masked_exec(asm) == [3]


def test_scanner_follows_labels_and_loops():
    # an MFMA at a loop header (a label) that is entered with EXEC narrowed,
    # and one in a branch target reached only from a narrowed block
    asm = "\n".join([
        "k:",
        "  s_and_saveexec_b64 s[0:1], vcc",      # 2
        ".LBB0_1:",
        "  v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",   # 4: loop header, narrowed
        "  s_cbranch_scc1 .LBB0_1",
        "  s_cbranch_vccnz .LBB0_3",
        "  s_or_b64 exec, exec, s[0:1]",
        "  s_branch .LBB0_4",
        ".LBB0_3:",
        "  v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",   # 10: reached narrowed
        "  s_or_b64 exec, exec, s[0:1]",
        ".LBB0_4:",
        "  v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",   # 13: restored on both paths
        "  s_endpgm"])
    assert mfma_under_masked_exec(asm) == [4, 10]
    # a backward branch from a narrowed block makes the loop header narrowed
    asm = "\n".join([
        "k:",
        ".LBB1_1:",
        "  v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",   # 3
        "  s_and_saveexec_b64 s[0:1], vcc",
        "  s_cbranch_execnz .LBB1_1",
        "  s_or_b64 exec, exec, s[0:1]",
        "  s_endpgm"])
    assert mfma_under_masked_exec(asm) == [3]


def _compile(src, tmp_path):
    hip = os.path.join(build.CSRC, src)
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    out = tmp_path / (src + ".s")
    cmd = ["hipcc", *flags, "-S", "--cuda-device-only", "-I", os.path.join(build.ROOT, "include"),
           "-I", build.CSRC, hip, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text(), res.stderr


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
@pytest.mark.parametrize("src", KERNELS)
def test_no_mfma_under_masked_exec(src, tmp_path):
    asm, _ = _compile(src, tmp_path)
    bad = mfma_under_masked_exec(asm)
    assert not bad, f"{src}: MFMAs under a narrowed EXEC at assembly lines {bad[:10]}"


# a scalar register the compiler may hand the asm: s<n>, vcc_lo / vcc_hi, ...
_SREG = r"(?:s\d+|vcc_lo|vcc_hi|ttmp\d+|flat_scratch_lo|flat_scratch_hi)"


def m0_writes_outside_dma(asm: str) -> list:
    """Line numbers of instructions writing M0 that are not part of a
    save (s_mov_b32 sX, m0) / set (s_mov_b32 m0, sY) / s_nop / buffer_load
    ... lds / restore (s_mov_b32 m0, sX) sequence."""
    ins = [x for x in _instructions(asm) if not x[1].endswith(":")]
    bad = []
    i = 0
    while i < len(ins):
        ln, op, text = ins[i]
        writes_m0 = len(text.split()) > 1 and text.split()[1].rstrip(",") == "m0"
        save = re.match(rf"s_mov_b32\s+({_SREG}),\s*m0$", text)
        if op == "s_mov_b32" and save:
            saved = save.group(1)
            seq = ins[i + 1:i + 5]
            ok = (len(seq) == 4 and re.match(rf"s_mov_b32\s+m0,\s*{_SREG}$", seq[0][2])
                  and seq[1][1] == "s_nop"
                  and seq[2][1].startswith("buffer_load") and seq[2][2].rstrip().endswith("lds")
                  and re.match(rf"s_mov_b32\s+m0,\s*{saved}$", seq[3][2]))
            if not ok:
                bad.append(ln)
                i += 1
                continue
            i += 5
            continue
        if writes_m0 or (op.startswith("buffer_load") and text.endswith(" lds")):
            bad.append(ln)
        i += 1
    return bad


def test_m0_scanner():
    good = "\n".join(["s_mov_b32 s9, m0", "s_mov_b32 m0, s4", "s_nop 0",
                      "buffer_load_dwordx4 v1, s[0:3], s5 offen lds", "s_mov_b32 m0, s9"])
    assert m0_writes_outside_dma(good) == []
    assert m0_writes_outside_dma(good.replace("s9", "vcc_hi")) == []
    assert m0_writes_outside_dma("s_mov_b32 m0, s4\nbuffer_load_dwordx4 v1, s[0:3], s5 offen lds") == [1, 2]
    # a restore from the wrong register breaks the sequence: every M0 write
    # and the DMA itself are reported
    assert m0_writes_outside_dma(good.replace("s_mov_b32 m0, s9", "s_mov_b32 m0, s8")) == [1, 2, 4, 5]


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_recurrence_m0_is_preserved(tmp_path):
    asm, err = _compile("kda_recurrence.hip", tmp_path)
    assert "clobber list contains reserved registers" not in err
    assert "lds" in asm
    bad = m0_writes_outside_dma(asm)
    assert not bad, f"M0 written outside the save/restore DMA sequence at lines {bad[:10]}"


def waterfall_loops(asm: str) -> list:
    """Line numbers of vector memory instructions issued from inside a
    waterfall loop: a loop whose body reads a value with v_readfirstlane,
    narrows EXEC to the lanes that match it, issues the access and clears
    those lanes (s_xor_b64 exec, exec, ...) before branching back while any
    remain.  The compiler emits one when a buffer resource or scalar operand
    lives in vector registers; its s_waitcnt vmcnt(0) then waits for every
    load and store in flight."""
    ins = _instructions(asm)
    labels = {text[:-1]: k for k, (_, op, text) in enumerate(ins) if text.endswith(":")}
    bad = []
    for k, (ln, op, text) in enumerate(ins):
        if op != "s_cbranch_execnz":
            continue
        target = labels.get(text.split()[1])
        if target is None or target > k:
            continue
        body = ins[target + 1:k]
        ops = [b[1] for b in body]
        if ("v_readfirstlane_b32" in ops and any(o.startswith("s_and_saveexec") for o in ops)
                and any(b[2].startswith("s_xor_b64 exec, exec") for b in body)):
            bad += [b[0] for b in body if b[1].startswith(("buffer_", "global_"))]
    return bad


def test_waterfall_scanner():
    asm = "\n".join([
        ".LBB0_5:",
        "  v_readfirstlane_b32 s36, v36",
        "  s_waitcnt vmcnt(0)",
        "  v_cmp_eq_u64_e32 vcc, s[36:37], v[36:37]",
        "  s_and_saveexec_b64 s[0:1], vcc",
        "  buffer_load_dword v0, v38, s[36:39], 0 offen",   # 6
        "  s_xor_b64 exec, exec, s[0:1]",
        "  s_cbranch_execnz .LBB0_5",
        "  s_endpgm"])
    assert waterfall_loops(asm) == [6]
    # a forward if/else over EXEC is not a loop
    assert waterfall_loops(asm.replace(".LBB0_5:\n", "").replace("  s_endpgm", ".LBB0_5:\n  s_endpgm")) == []


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
@pytest.mark.parametrize("src", KERNELS)
def test_no_waterfall_loops(src, tmp_path):
    asm, _ = _compile(src, tmp_path)
    bad = waterfall_loops(asm)
    assert not bad, f"{src}: memory access inside a waterfall loop at assembly lines {bad[:10]}"
