"""Checks on the gfx950 assembly of the matrix-core kernels (CPU only).

The transposed V reads are issued as inline assembly and their completion is
awaited with an explicit lgkmcnt wait that names the destination registers.
The compiler does not see the reads as asynchronous, so nothing but this test
guarantees that it never reads, copies or overwrites a destination register
between the read and its wait.  The test also checks that no matrix-core
kernel (decode, prefill) keeps anything in scratch memory.
"""

import os
import re
import shutil
import subprocess

import pytest

from paged_kv_cache_447_amd import build as B

SOURCES = ["decode_mfma.hip", "prefill_mfma.hip"]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = B.hipcc()
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("asm")
    procs = []
    for src in SOURCES:  # both files compile at once
        out = d / (src + ".s")
        cmd = [hipcc, "-x", "hip", *B.COMMON, *B.DEVICE, "--offload-device-only", "-S", os.path.join(B.CSRC, src),
               "-o", str(out)]
        procs.append((src, out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    kernels = {}
    for src, out, p in procs:
        _, err = p.communicate()
        assert p.returncode == 0, err[-2000:]
        text = out.read_text()
        stem = src.split(".")[0]
        found = re.findall(r"^(_Z\S*" + stem + r"\S*):", text, re.M)
        assert found, f"no {stem} kernels found in the assembly"
        for name in found:
            i = text.index(name + ":")
            kernels[name] = text[i:text.index(".Lfunc_end", i)].split("\n")
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
