"""The boundary from plain C: include/sinkroute.h compiles as C99 under
-Wall -Wextra -Werror -pedantic, and a C program linked against the built
library gets the struct sizes the Python binding assumes, the workspace and
launch-policy introspection, and the argument errors that return before
anything is enqueued (tests/c_abi_check.c; no GPU is touched)."""
import ctypes
import os
import shutil
import subprocess

import pytest

from kv_cache_routing_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "kv_cache_routing_amd")


def test_header_and_library_from_c99(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("needs gcc")
    # the C side checks these sizes; the binding's ctypes mirrors must agree
    assert (ctypes.sizeof(N.SrShape), ctypes.sizeof(N.SrLaunch), ctypes.sizeof(N.SrPart)) == \
        (56, 16, 40)
    exe = str(tmp_path / "c_abi_check")
    build = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
             f"-I{os.path.join(ROOT, 'include')}", os.path.join(ROOT, "tests", "c_abi_check.c"),
             f"-L{LIB_DIR}", "-lsinkroute", f"-Wl,-rpath,{LIB_DIR}", "-o", exe]
    r = subprocess.run(build, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout[-2000:], r.stderr[-2000:])
