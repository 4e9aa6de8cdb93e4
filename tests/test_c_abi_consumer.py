"""The boundary is a C ABI: a plain C99 program built with gcc against
include/echo.h and linked to the built library must compile without warnings
and see the documented sizes and argument checks (no GPU needed: every call
it makes returns before any HIP work)."""
import os
import shutil
import subprocess

import pytest

from error_compensated_bit_amd import build as eb

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_c99_consumer_builds_and_runs(tmp_path):
    lib = eb.library_path()
    if not os.path.exists(lib):
        pytest.skip("library not built")
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(lib)
    name = os.path.basename(lib)[3:-3]     # libecho_amd.so -> echo_amd
    cmd = ["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c_abi", "consumer.c"),
           "-L", libdir, f"-l{name}", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok"
