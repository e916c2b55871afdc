"""The C ABI from plain C: tests/c/abi_from_c.c is compiled with gcc as C11
(-pedantic, warnings as errors) against include/triattn.h, linked to the
built library and run.  It makes only host-side calls (workspace sizes,
pyramid budgets, status strings, argument errors), so no GPU is needed."""
import os
import shutil
import subprocess

import pytest

import rope_aware_key_amd as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_header_and_library_from_c(tmp_path):
    exe = tmp_path / "abi_from_c"
    lib_dir = os.path.dirname(R.LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_from_c.c"),
           "-L", lib_dir, "-ltriattn", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failure(s)" in r.stdout
