"""Host sanitizer runs (CPU only).

The oracle (``oracle/oracle.c``) and the host side of the C ABI
(``csrc/pa_api.cpp``, ``csrc/pa_validate.cpp``) are compiled with
AddressSanitizer and UndefinedBehaviorSanitizer, with every finding fatal, and
driven through their entry points by ``tests/sanitize/oracle_driver.c`` and
``tests/sanitize/abi_driver.cpp``.  A copy of the oracle with a planted heap
overflow goes through the same build and must be reported, so that a clean run
means the sanitizers were really watching.  The ABI driver links the kernels'
objects as the library build leaves them; it calls nothing that reaches a
device (every call fails its checks first).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "oracle.c")
SAN_DIR = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "paged_kv_cache_447_amd", "csrc")
BUILD_DIR = os.path.join(ROOT, "paged_kv_cache_447_amd", "_build")
KERNEL_OBJECTS = ["decode_valu.hip.o", "decode_mfma.hip.o", "decode_static.hip.o", "prefill_mfma.hip.o",
                  "cache_write.hip.o", "block_copy.hip.o", "stream_read.hip.o"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

SANITIZE = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _need(tool):
    if not shutil.which(tool):
        pytest.skip(f"{tool} not found")


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)


def _build_oracle(src, exe):
    subprocess.run(["gcc", "-std=c11", *SANITIZE, "-ffp-contract=off", str(src),
                    os.path.join(SAN_DIR, "oracle_driver.c"), "-o", str(exe), "-lm", "-lpthread"],
                   check=True, capture_output=True, text=True)


def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    _need("gcc")
    exe = tmp_path / "oracle_driver"
    _build_oracle(ORACLE_C, exe)
    r = _run(exe)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "all entry points clean" in r.stdout


def test_a_planted_overflow_in_the_oracle_is_reported(tmp_path):
    _need("gcc")
    text = open(ORACLE_C).read()
    exact = "double *s = (double *)malloc(sizeof(double) * (size_t)(cap + 1));"
    assert exact in text
    # the decode's score buffer, sized for half the longest context
    bad = tmp_path / "oracle_planted.c"
    bad.write_text(text.replace(exact, "double *s = (double *)malloc(sizeof(double) * (size_t)(cap / 2));", 1))
    exe = tmp_path / "oracle_planted"
    _build_oracle(bad, exe)
    r = _run(exe)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


def test_abi_host_side_is_clean_under_asan_and_ubsan(tmp_path):
    _need("g++")
    objs = [os.path.join(BUILD_DIR, o) for o in KERNEL_OBJECTS]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("the library's objects are not built (python -m paged_kv_cache_447_amd.build)")
    exe = tmp_path / "abi_driver"
    proc = subprocess.run(["g++", "-std=c++17", *SANITIZE, "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
                           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", os.path.join(SAN_DIR, "abi_driver.cpp"),
                           os.path.join(CSRC, "pa_api.cpp"), os.path.join(CSRC, "pa_validate.cpp"), *objs,
                           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", str(exe)],
                          capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr[-4000:]
    r = _run(exe)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "all checks clean" in r.stdout
