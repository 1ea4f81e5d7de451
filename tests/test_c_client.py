"""The C ABI from plain C: include/rs.h compiles as C99 (gcc, warnings as
errors) and a C program linked against librs.so sizes layers and gets the
host-side error codes, with no Python in between. No device call is made."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "ssm_decode_checkpoint_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c99_client_links_and_runs(tmp_path):
    exe = tmp_path / "abi_host"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_host.c"), "-L", LIB_DIR, "-lrs", f"-Wl,-rpath,{LIB_DIR}",
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "FAIL" not in run.stdout and run.stdout.count("ok ") >= 10
