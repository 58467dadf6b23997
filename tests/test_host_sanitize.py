"""The C ABI's host code (argument validation, layout and size arithmetic)
under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's sources are compiled for the host only (the kernels' device
code is left out, so every launch fails and the entry points report
RDKV_ERR_HIP), with the sanitizers on the host code, and linked with
tests/sanitize/driver.cpp, which calls every entry point with valid, NULL,
misaligned, short and tampered arguments and then with random and extreme
shapes, budgets and lengths.  The sanitizers abort on their first finding.
CPU only; needs hipcc."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "decode_attention_rdkv_amd", "csrc")
SOURCES = ["api", "k_decode", "k_pack", "k_alloc", "k_score", "k_rollover", "scratch"]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    # an empty device binary stands in for the kernels' code objects
    empty = tmp_path / "empty.hip"
    empty.write_text("\n")
    fatbin = tmp_path / "empty.fatbin"
    subprocess.run([hipcc, "--offload-arch=gfx950", "--cuda-device-only", "-c", str(empty), "-o", str(fatbin)],
                   check=True, capture_output=True)
    procs, objs = [], []
    for s in SOURCES:
        o = tmp_path / f"{s}.o"
        objs.append(str(o))
        procs.append(subprocess.Popen(
            [hipcc, "--offload-host-only", "-std=c++17", "-O1", "-g", *san, "-Xclang", "-fcuda-include-gpubinary",
             "-Xclang", str(fatbin), *inc, "-c", os.path.join(CSRC, s + ".hip"), "-o", str(o)],
            stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out[-4000:]
    drv = tmp_path / "driver"
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc)))
    host_inc = ["-I", os.path.join(rocm, "include"), "-D__HIP_PLATFORM_AMD__"]   # the HIP runtime header, host side
    r = subprocess.run([hipcc, "-std=c++17", "-O1", "-g", *san[1::2], *inc, *host_inc,
                        "-x", "c++", os.path.join(HERE, "sanitize", "driver.cpp"), "-x", "none", *objs,
                        "-o", str(drv)], capture_output=True, text=True)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="")
    r = subprocess.run([str(drv)], capture_output=True, text=True, env=env, timeout=600)
    log = r.stdout + r.stderr
    assert r.returncode == 0, log[-4000:]
    assert "runtime error" not in log and "AddressSanitizer" not in log, log[-4000:]
    assert " 0 failed" in r.stdout
