"""The boundary from plain C: tests/c/abi_check.c is compiled as C99 against include/streamattn.h
alone (no C++, no torch), linked to libstreamattn.so and run; it checks the host-only cache
functions and argument validation (no device work)."""
import os
import shutil
import subprocess

import pytest
import torch

from head_attention_streaming_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="host-side validation checks (no GPU)")


def test_plain_c_client_compiles_links_and_passes(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    lib = binding.library_path()
    assert os.path.exists(lib), "build the library first"
    exe = tmp_path / "abi_check"
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_check.c"), lib, f"-Wl,-rpath,{os.path.dirname(lib)}",
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"
