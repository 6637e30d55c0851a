"""The C ABI's host-side checks under AddressSanitizer and
UndefinedBehaviorSanitizer.

Every library source is compiled with both sanitizers on its host code only
(each -fsanitize flag behind -Xarch_host; the device code is built as usual
and never runs here), linked with abi_sanitize/abi_host_checks.cpp, and run.
That program calls every entry point with arguments its host checks refuse
(the cases of test_abi_host.py and a few more at extreme sizes) and checks
each status code; a read outside a struct or host array, or undefined
arithmetic in the size checks, aborts it with the sanitizer's report.  No
call reaches a device.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_expert_ffn_top_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
DRIVER = os.path.join(ROOT, "tests", "abi_sanitize", "abi_host_checks.cpp")

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]
FLAGS = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc not found")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout[-3000:]}\n{res.stderr[-3000:]}"


def test_abi_host_checks_under_asan_and_ubsan(tmp_path):
    hipcc = _hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [DRIVER]
    objs = [str(tmp_path / (os.path.basename(s).rsplit(".", 1)[0] + ".o")) for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda so: _run([hipcc, *FLAGS, *SAN, "-c", so[0], "-o", so[1]]),
                    zip(srcs, objs)))
    exe = str(tmp_path / "abi_host_checks")
    _run([hipcc, "--offload-arch=gfx950", *SAN, *objs, "-o", exe])
    env = dict(os.environ)
    # the HIP runtime keeps allocations until exit: leaks are not checked
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300,
                         cwd=str(tmp_path))
    out = res.stdout + res.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert "abi host checks:" in out and ", 0 failed" in out, out[-4000:]
    n = int(out.split("abi host checks:")[1].split("passed")[0])
    assert n >= 140, out
