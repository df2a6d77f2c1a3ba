"""Host-side sanitizer builds (CPU only, no GPU needed):

* the fp64 oracle (oracle/oracle.c) built with AddressSanitizer and UndefinedBehaviorSanitizer,
  driven by tests/c/oracle_driver.c over every entry point (threaded attention, row subsets,
  windows, grouped heads) with closed-form checks;
* the library's host validation (csrc/capi.hip) built with host-only ASan/UBSan
  (-Xarch_host, so no device code is instrumented) against stand-in launchers that record launches
  instead of touching a GPU, driven by the plain C client tests/c/abi_check.c: every call there is
  rejected before launch or is an empty no-op, so the stand-ins must report zero launches.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CDIR = os.path.join(ROOT, "tests", "c")
CSRC = os.path.join(ROOT, "head_attention_streaming_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "oracle_san")
    _run([gcc, "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-pthread", os.path.join(CDIR, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", exe])
    r = _run([exe], timeout=120, env=SAN_ENV)
    assert r.stdout.strip() == "ok"
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr


def test_host_validation_under_asan_and_ubsan(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not all(os.path.exists(p) for p in (hipcc, clang, clangxx)):
        pytest.skip("no ROCm toolchain")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", INCLUDE, "-I", CSRC]
    objs = []
    for src in (os.path.join(CSRC, "capi.hip"), os.path.join(CDIR, "host_stubs.hip")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([hipcc, *common, *san, "-c", src, "-o", obj])
        objs.append(obj)
    client = str(tmp_path / "abi_check.o")
    _run([clang, "-std=c99", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I", INCLUDE, "-c", os.path.join(CDIR, "abi_check.c"), "-o", client])
    exe = str(tmp_path / "abi_san")
    _run([clangxx, "-fsanitize=address,undefined", client, *objs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe])
    r = _run([exe], timeout=120, env=SAN_ENV)
    assert r.stdout.strip() == "ok"
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr
    assert "stub launches: 0" in r.stderr, r.stderr
