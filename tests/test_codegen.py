"""Code-generation guard (CPU only): no MFMA may be issued while EXEC is
narrowed by a divergent branch.

MFMA instructions do not honour EXEC: an MFMA on a path that a wave skips
through exec masking still runs and still writes (and accumulates into) its
destination.  The kernels keep every branch around MFMAs wave-uniform (the
wave index is read into a scalar register), so that the compiler emits
scalar jumps there.  This test compiles the kernels to gfx950 assembly and
checks, block by block, that no MFMA follows a saveexec before EXEC is
restored."""

import os
import shutil
import subprocess

import pytest

from chunked_kda_prefill_amd import build

KERNELS = ["kda_intra.hip", "kda_recurrence.hip"]


def mfma_under_masked_exec(asm: str) -> list:
    """Line numbers of MFMAs issued after a saveexec in the same basic block
    (straight-line code after the mask is narrowed, before it is restored)."""
    bad = []
    narrowed = False
    for i, line in enumerate(asm.split("\n")):
        tok = line.strip().split()
        if not tok or tok[0].startswith(";"):
            continue
        op = tok[0]
        if op.endswith(":"):            # a new basic block
            narrowed = False
        elif "saveexec" in op:
            narrowed = True
        elif op.startswith("s_or_b64") and "exec, exec" in line:
            narrowed = False
        elif line.strip().startswith("s_mov_b64 exec"):
            narrowed = False
        elif op.startswith("v_mfma") and narrowed:
            bad.append(i + 1)
    return bad


def test_scanner_flags_masked_mfma():
    asm = "\n".join(["k:", "  s_and_saveexec_b64 s[0:1], vcc",
                     "  v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
                     "  s_or_b64 exec, exec, s[0:1]",
                     "  v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0"])
    assert mfma_under_masked_exec(asm) == [3]


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
@pytest.mark.parametrize("src", KERNELS)
def test_no_mfma_under_masked_exec(src, tmp_path):
    hip = os.path.join(build.CSRC, src)
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    out = tmp_path / (src + ".s")
    cmd = ["hipcc", *flags, "-S", "--cuda-device-only", "-I", os.path.join(build.ROOT, "include"),
           "-I", build.CSRC, hip, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    bad = mfma_under_masked_exec(out.read_text())
    assert not bad, f"{src}: MFMAs under a narrowed EXEC at assembly lines {bad[:10]}"
