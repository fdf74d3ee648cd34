"""The host layer of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer,
on the CPU: api.hip is compiled with host-side sanitizers (device code as usual),
linked with the library's other objects, and a C driver (tests/asan/abi_checks.c)
calls every entry point with arguments that must be refused before anything
reaches HIP, queries workspace sizes at extreme shapes, and refuses calls from
four threads at once. Any sanitizer report or unexpected return fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="hipcc / clang not installed")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_abi_argument_checks_under_sanitizers(tmp_path):
    from block_sparse_attention_softmax_amd import build as B
    objs = [os.path.join(B.BUILD, os.path.basename(s) + ".o") for s in B.sources()
            if not s.endswith("api.hip")]
    if not all(os.path.exists(o) for o in objs):
        B.build(verbose=False)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
    api = str(tmp_path / "api_san.o")
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g"]
    _run([HIPCC, *flags, *san, "-c", os.path.join(B.CSRC, "api.hip"), "-o", api])
    lib = str(tmp_path / "libsparge_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, api, "-o", lib])
    nm = _run(["nm", "-D", "--undefined-only", lib]).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm, "host code is not instrumented"
    drv = str(tmp_path / "abi_checks")
    _run([CLANG, "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-g", "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "tests", "asan", "abi_checks.c"), "-L", str(tmp_path),
          "-lsparge_san", f"-Wl,-rpath,{tmp_path}", "-lpthread", "-lm", "-o", drv])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([drv], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "abi checks ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
