"""The work-division arithmetic that the decode kernels and sr_plan_parts
share (kv_cache_routing_amd/csrc/sr_internal.h), fuzzed on the CPU under the
undefined-behaviour and address sanitizers: 200000 random launch layouts over
the supported envelope, every signed overflow or bad access fatal, and the
ranges and item parts checked to tile the active chunks in order."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"


def test_plan_arithmetic_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(os.path.join(ROCM_INCLUDE, "hip")):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path / "plan_fuzz")
    src = os.path.join(ROOT, "tests", "plan_fuzz.cpp")
    build = [gxx, "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INCLUDE}",
             f"-I{os.path.join(ROOT, 'include')}",
             f"-I{os.path.join(ROOT, 'kv_cache_routing_amd', 'csrc')}",
             "-fsanitize=undefined,address", "-fno-sanitize-recover=undefined", src, "-o", exe]
    r = subprocess.run(build, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0")
    r = subprocess.run([exe, "200000"], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "200000 layouts ok" in r.stdout


def test_rotary_angle_sincos_matches_the_c_library(tmp_path):
    # sr::angle_sincos (the rotary angles' sine and cosine, shared by host and
    # device code) against glibc's sin and cos over rotary angles, random
    # arguments and quadrant boundaries, under the undefined-behaviour
    # sanitizer: largest absolute error at most 4e-16.
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(os.path.join(ROCM_INCLUDE, "hip")):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path / "angle_check")
    src = os.path.join(ROOT, "tests", "angle_check.cpp")
    build = [gxx, "-std=c++17", "-O2", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INCLUDE}",
             f"-I{os.path.join(ROOT, 'kv_cache_routing_amd', 'csrc')}",
             "-fsanitize=undefined", "-fno-sanitize-recover=undefined", src, "-o", exe]
    r = subprocess.run(build, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "max abs error" in r.stdout
