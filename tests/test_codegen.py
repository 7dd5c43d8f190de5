"""Checks on the gfx950 assembly of the matrix-core decode kernels (CPU only).

The transposed V reads are issued as inline assembly and their completion is
awaited with an explicit lgkmcnt wait that names the destination registers.
The compiler does not see the reads as asynchronous, so nothing but this test
guarantees that it never reads, copies or overwrites a destination register
between the read and its wait.  The test also checks that no decode kernel
keeps anything in scratch memory.
"""

import os
import re
import shutil
import subprocess

import pytest

from paged_kv_cache_447_amd import build as B

SRC = os.path.join(B.CSRC, "decode_mfma.hip")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = B.hipcc()
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "decode_mfma.s"
    cmd = [hipcc, "-x", "hip", *B.COMMON, *B.DEVICE, "--offload-device-only", "-S", SRC, "-o", str(out)]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr[-2000:]
    text = out.read_text()
    kernels = {}
    for name in re.findall(r"^(_Z\S*decode_mfma\S*):", text, re.M):
        i = text.index(name + ":")
        kernels[name] = text[i:text.index(".Lfunc_end", i)].split("\n")
    assert kernels, "no decode kernels found in the assembly"
    return kernels


def _regs(line):
    regs = {int(x) for x in re.findall(r"\bv(\d+)\b", line)}
    for lo, hi in re.findall(r"v\[(\d+):(\d+)\]", line):
        regs.update(range(int(lo), int(hi) + 1))
    return regs


def test_no_scratch(asm):
    for name, body in asm.items():
        used = [l.strip() for l in body if re.match(r"\s+scratch_", l)]
        assert not used, f"{name} uses scratch: {used[:3]}"


def test_transposed_reads_untouched_until_waited(asm):
    n = 0
    for name, body in asm.items():
        for k, line in enumerate(body):
            m = re.match(r"\s+ds_read_b64_tr_b16 v\[(\d+):(\d+)\]", line)
            if not m:
                continue
            n += 1
            dst = set(range(int(m.group(1)), int(m.group(2)) + 1))
            for later in body[k + 1:]:
                if re.match(r"\s+s_waitcnt", later) and "lgkmcnt" in later:
                    break
                if "ds_read_b64_tr_b16" in later:
                    continue
                assert not (_regs(later) & dst), f"{name}: {line.strip()} touched by {later.strip()} before its wait"
            else:
                raise AssertionError(f"{name}: {line.strip()} never waited for")
    assert n > 0, "no transposed reads found"
