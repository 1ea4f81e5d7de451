"""The C ABI's host side (rs_host.cpp: validation, buffer layout, argument
blocks) built on its own with AddressSanitizer and UndefinedBehaviorSanitizer
against a recording stand-in for the kernel files, and driven by the plain C
clients: tests/c/abi_host.c (the client test_c_client.py links against
librs.so) and tests/c/abi_dispatch.c (every entry point dispatches exactly
once on valid arguments and not at all on invalid ones). CPU only; the host
compiler builds it, no GPU code is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ssm_decode_checkpoint_amd", "csrc")
INC = os.path.join(ROOT, "include")
C_DIR = os.path.join(ROOT, "tests", "c")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.fixture(scope="module")
def objs(tmp_path_factory):
    if shutil.which("g++") is None or shutil.which("gcc") is None:
        pytest.skip("no host compiler")
    d = tmp_path_factory.mktemp("san")
    out = []
    for src, cc, std in (("rs_host.cpp", "g++", "-std=c++17"), ("dispatch_stub.cpp", "g++", "-std=c++17")):
        path = os.path.join(CSRC if src == "rs_host.cpp" else C_DIR, src)
        o = str(d / (src + ".o"))
        r = subprocess.run([cc, std, *SAN, "-Wall", "-Wextra", "-Werror", f"-I{INC}", f"-I{CSRC}", "-c", path, "-o", o],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        out.append(o)
    return d, out


def _run_client(objs, name):
    d, base = objs
    o = str(d / (name + ".o"))
    r = subprocess.run(["gcc", "-std=c99", *SAN, "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{INC}", "-c",
                        os.path.join(C_DIR, name + ".c"), "-o", o], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(d / name)
    r = subprocess.run(["g++", *SAN, *base, o, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    return run


def test_abi_host_client_under_sanitizers(objs):
    run = _run_client(objs, "abi_host")
    assert run.returncode == 0, run.stdout + run.stderr
    assert "FAIL" not in run.stdout and "runtime error" not in run.stderr


def test_every_entry_point_dispatches_or_refuses(objs):
    run = _run_client(objs, "abi_dispatch")
    assert run.returncode == 0, run.stdout + run.stderr
    assert "runtime error" not in run.stderr and "ERROR: AddressSanitizer" not in run.stderr
    lines = run.stdout.splitlines()
    assert lines[-1] == "0 failed" and sum(l.startswith("ok ") for l in lines) >= 60, run.stdout
