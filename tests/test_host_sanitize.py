"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

The library's sources are compiled with the sanitizers on their host code
only (each -fsanitize= behind -Xarch_host; device code is built as usual) and
linked into a separate shared library; a C++ driver built with the same
sanitizers calls every ABI entry point whose arguments are rejected, or whose
answer is computed, before any HIP call: configuration validation over the
supported set and its edges, status strings, load-time argument checks and
calls on a null layer.  Any sanitizer report, or a failed expectation, fails
the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_moe_relu_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
SOURCES = ["host.hip", "pack.hip", "decode.hip", "prefill.hip", "backward.hip"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if r.returncode != 0:
        raise AssertionError(f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}")
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not installed")
def test_host_code_under_asan_ubsan(tmp_path):
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             f"-I{os.path.join(ROOT, 'include')}", *SAN]
    procs, objs = [], []
    for src in SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p, src in zip(procs, SOURCES):
        out, _ = p.communicate()
        assert p.returncode == 0, f"hipcc failed on {src}:\n{out[-3000:]}"
    lib = str(tmp_path / "libdeco_moe_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, "-o", lib, *objs])
    exe = str(tmp_path / "host_checks")
    _run([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          f"-I{os.path.join(ROOT, 'include')}", os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"),
          lib, f"-Wl,-rpath,{tmp_path}", "-o", exe])
    env = dict(os.environ)
    # leaks of the uninstrumented HIP runtime at exit are not this code's
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    log = r.stdout + r.stderr
    assert r.returncode == 0, log[-4000:]
    assert "host checks passed" in r.stdout
    assert "ERROR: AddressSanitizer" not in log and "runtime error" not in log, log[-4000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
