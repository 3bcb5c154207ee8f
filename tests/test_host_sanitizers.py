"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* The library's host code: api.hip (argument validation, kernel choice, split plans and
  workspace arithmetic of every entry point) compiled host-only with the sanitizers on
  the host side, linked with the library's kernel objects and
  tests/host_checks/abi_host_check.c, and run (nothing launches a kernel).
* The float64 oracle: oracle/gqa_oracle.c with tests/host_checks/oracle_host_check.c,
  every code path on small shapes, built with gcc's sanitizers.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "grouped_query_attention_amd", "csrc")
CHECKS = os.path.join(ROOT, "tests", "host_checks")
OUT = os.path.join(ROOT, "_build", "host_sanitizers")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
# sanitizers on the host side only, each flag behind -Xarch_host
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


def _kernel_objects():
    """Objects of the kernel sources from the library build (grouped_query_attention_amd/
    build.py writes them to _build/); built here when absent."""
    build_dir = os.path.join(ROOT, "_build")
    srcs = [os.path.basename(p)[:-4] for p in glob.glob(os.path.join(CSRC, "*.hip"))]
    objs = [os.path.join(build_dir, s + ".o") for s in srcs if s != "api"]
    if not all(os.path.exists(o) for o in objs):
        import importlib.util
        spec = importlib.util.spec_from_file_location("gqa_build", os.path.join(ROOT, "grouped_query_attention_amd",
                                                                                 "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return objs


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_library_host_code_under_sanitizers():
    """api.hip (every entry point's validation, kernel choice and plan arithmetic) is
    compiled host-only with the sanitizers and linked with the library's kernel objects
    (whose host parts are the launchers and the decode split plan)."""
    os.makedirs(OUT, exist_ok=True)
    api = os.path.join(OUT, "api.o")
    _run([HIPCC, "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fPIC"] + SAN +
         ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, "api.hip"), "-o", api])
    drv = os.path.join(OUT, "abi_host_check.o")
    _run([HIPCC, "-x", "c", "-O1", "-g"] + SAN + ["-I", os.path.join(ROOT, "include"), "-c",
                                                  os.path.join(CHECKS, "abi_host_check.c"), "-o", drv])
    exe = os.path.join(OUT, "abi_host_check")
    _run([HIPCC, "--offload-arch=gfx950"] + SAN + [drv, api] + _kernel_objects() + ["-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "0 failures" in r.stdout, r.stdout
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_host_check")
    _run(["gcc", "-O1", "-g", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
          os.path.join(CHECKS, "oracle_host_check.c"), os.path.join(ROOT, "oracle", "gqa_oracle.c"),
          "-o", exe, "-lm", "-lpthread"])
    r = _run([exe], env=ENV, timeout=300)
    assert "0 failures" in r.stdout, r.stdout
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
