"""Checks on the gfx950 assembly of the kernels (CPU only).

The transposed V reads are issued as inline assembly and their completion is
awaited with an explicit lgkmcnt wait that names the destination registers.
The compiler does not see the reads as asynchronous, so nothing but this test
guarantees that it never reads, copies or overwrites a destination register
between the read and its wait.  The test also checks that no kernel (both
decode kernels, the no-allocation decode, prefill) keeps anything in scratch
memory, and that every decode kernel publishes a cut context's partial in
the order its merge relies on: the partial's device-coherent (sc1) stores,
then a full wait (s_waitcnt vmcnt(0)), then the counter's atomic add; and
the merge's coherent loads only after the atomic's returned value is read.
"""

import os
import re
import shutil
import subprocess

import pytest

from paged_kv_cache_447_amd import build as B

SOURCES = ["decode_mfma.hip", "decode_valu.hip", "decode_static.hip", "prefill_mfma.hip"]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = B.hipcc()
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("asm")
    procs = []
    for src in SOURCES:  # the files compile in parallel
        out = d / (src + ".s")
        cmd = [hipcc, "-x", "hip", *B.COMMON, *B.DEVICE, "--offload-device-only", "-S", os.path.join(B.CSRC, src),
               "-o", str(out)]
        procs.append((src, out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    kernels = {}
    for src, out, p in procs:
        _, err = p.communicate()
        assert p.returncode == 0, err[-2000:]
        text = out.read_text()
        stem = {"decode_static": "clear_scratch"}.get(src.split(".")[0], src.split(".")[0])
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


def publication_violations(body):
    """Violations of the partial-publication order in one kernel body (lines of
    assembly, in layout order): a counter atomic (global_atomic_add returning
    its value) with a coherent partial store (buffer_store ... sc1) before it
    and no full vmcnt wait in between; a coherent merge load (buffer_load ...
    sc1) not preceded, since the last counter atomic, by a read of that
    atomic's returned register."""
    bad = []
    atomics = [k for k, l in enumerate(body) if re.match(r"\s+global_atomic_add\S* v\d+", l) and "sc0" in l]
    for k in atomics:
        for j in range(k - 1, -1, -1):
            l = body[j]
            if re.match(r"\s+s_waitcnt", l) and ("vmcnt(0)" in l or re.match(r"\s+s_waitcnt\s+0\s*$", l)):
                break
            if re.match(r"\s+buffer_store\S*", l) and "sc1" in l:
                bad.append(f"line {k}: counter atomic after a partial store with no full wait ({l.strip()})")
                break
    for k, l in enumerate(body):
        if not (re.match(r"\s+buffer_load\S*", l) and "sc1" in l):
            continue
        prev = [a for a in atomics if a < k]
        if not prev:
            bad.append(f"line {k}: merge load with no counter atomic before it")
            continue
        a = prev[-1]
        dst = re.match(r"\s+global_atomic_add\S* (v\d+)", body[a]).group(1)
        used = any(re.search(r"\b" + dst + r"\b", body[j]) and ("readfirstlane" in body[j] or "readlane" in body[j])
                   for j in range(a + 1, k))
        if not used:
            bad.append(f"line {k}: merge load before the counter's returned value ({dst}) is read")
    return bad


def _decode_bodies(asm):
    return {n: b for n, b in asm.items() if "decode_valu" in n or "decode_mfma" in n}


def test_partials_published_in_order(asm):
    bodies = _decode_bodies(asm)
    assert len(bodies) > 10
    n_atomics = 0
    for name, body in bodies.items():
        n_atomics += sum(1 for l in body if re.match(r"\s+global_atomic_add", l))
        bad = publication_violations(body)
        assert not bad, f"{name}: {bad[:3]}"
    assert n_atomics > 0, "no counter atomics found"


def test_publication_check_catches_a_planted_reorder(asm):
    """The check above rejects a body whose full wait before the counter's
    atomic was removed, and one whose merge load was hoisted above the read of
    the counter's value (both planted in a copy of the assembly text)."""
    name, body = next((n, b) for n, b in _decode_bodies(asm).items() if "decode_valu" in n)
    k = next(k for k, l in enumerate(body) if re.match(r"\s+global_atomic_add", l) and "sc0" in l)
    w = max(j for j in range(k) if re.match(r"\s+s_waitcnt", body[j]) and "vmcnt(0)" in body[j])
    assert not publication_violations(body)
    no_wait = body[:w] + body[w + 1:]
    assert publication_violations(no_wait), "removing the wait before the counter atomic went unnoticed"
    m = next(j for j in range(k, len(body)) if re.match(r"\s+buffer_load\S*", body[j]) and "sc1" in body[j])
    hoisted = body[:k + 1] + [body[m]] + body[k + 1:m] + body[m + 1:]
    assert publication_violations(hoisted), "a merge load ahead of the counter's value went unnoticed"
