"""The library's host code (argument checks, work plans, workspace arithmetic)
under AddressSanitizer and UndefinedBehaviorSanitizer, without a GPU.

A copy of libhla.so is built into a temporary directory with both sanitizers on
its host code only (device code is compiled as usual), and tests/sanitize/
abi_grid.cpp calls every entry point over a grid of shapes (-1 to 2^63-1 per
dimension), head dims, dtype codes and arguments, each call with one invalid
argument or an empty tensor so that validation returns before any HIP call.
Any sanitizer report aborts the driver; the test checks its exit status and
call count.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "softmax_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["hla_api.hip", "linear_bf16.hip", "linear_f32.hip", "anchor_bf16.hip", "anchor_f32.hip",
           "attnres.hip"]
# sanitizers on the host side of each hipcc compile only
HOST_SAN = ["-Xarch_host", "-fsanitize=address",
            "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all",
            "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_argument_checks_under_asan_and_ubsan(tmp_path):
    objs = []
    procs = []
    for src in SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-command-line-argument", *HOST_SAN, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        objs.append(obj)
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out
    lib = str(tmp_path / "libhla_san.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN, *objs, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    # the host code is instrumented: it calls the sanitizers' report hooks
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle_" in syms
    exe = str(tmp_path / "abi_grid")
    r = subprocess.run([HIPCC, "-O1", "-g", *HOST_SAN, "-x", "c++",
                        os.path.join(ROOT, "tests", "sanitize", "abi_grid.cpp"), "-x", "none", lib,
                        f"-Wl,-rpath,{tmp_path}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "failures 0" in r.stdout
    calls = int(r.stdout.split("calls ")[1].split()[0])
    assert calls > 100_000, r.stdout
    print(r.stdout.strip())
