"""Build libsinkroute.so in-tree for gfx950 with hipcc.

    python kv_cache_routing_amd/build.py        # or __graft_entry__.build()

Every HIP source under csrc/ is compiled to an object and linked into
kv_cache_routing_amd/libsinkroute.so.  Always rebuilds.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsinkroute.so")
ARCH = os.environ.get("SR_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 vector ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
    # per-kernel register / scratch report, checked below
    "-Rpass-analysis=kernel-resource-usage",
]


def scratch_kernels(remarks: str) -> list:
    """Kernels the compiler gave per-lane scratch (private memory).  The
    kernels keep all their state in registers and LDS; scratch appears when
    a register array or struct is indexed at run time or registers spill,
    and it slows the streaming loops by whole percents, so it fails the
    build."""
    bad, name = [], None
    for ln in remarks.splitlines():
        if "Function Name:" in ln:
            name = ln.split("Function Name:")[1].split("[")[0].strip()
        elif "ScratchSize [bytes/lane]:" in ln and name:
            n = int(ln.split("ScratchSize [bytes/lane]:")[1].split("[")[0])
            if n > 0:
                bad.append(f"{name} ({n} bytes/lane)")
    return bad


# LDS per workgroup on gfx950, and the most dynamic LDS a decode launch adds
# (the fused rotary step: cos/sin of d/2 = 64 angles in fp64 and the rotated
# queries of 64 heads of d = 128 in fp32, rope_lds_bytes in sr_internal.h).
LDS_LIMIT = 160 * 1024
ROPE_LDS_MAX = 64 * 2 * 8 + 64 * 128 * 4


def lds_overflows(remarks: str) -> list:
    """Decode kernels whose static LDS plus the largest dynamic LDS of a fused
    rotary launch would not fit a workgroup: such a launch would fail."""
    bad, name = [], None
    for ln in remarks.splitlines():
        if "Function Name:" in ln:
            name = ln.split("Function Name:")[1].split("[")[0].strip()
        elif "LDS Size [bytes/block]:" in ln and name and "k_decode" in name:
            n = int(ln.split("LDS Size [bytes/block]:")[1].split("[")[0])
            if n + ROPE_LDS_MAX > LDS_LIMIT:
                bad.append(f"{name} ({n} + {ROPE_LDS_MAX} bytes)")
    return bad


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    bad = scratch_kernels(r.stderr or "")
    if bad:
        raise RuntimeError(f"{src}: kernels use scratch memory: " + "; ".join(bad))
    bad = lds_overflows(r.stderr or "")
    if bad:
        raise RuntimeError(f"{src}: LDS over {LDS_LIMIT} bytes with the rotary step: "
                           + "; ".join(bad))
    noise, in_remark = [], False
    for ln in (r.stderr or "").splitlines():
        if "remark:" in ln:  # the resource report and the source lines it quotes
            in_remark = True
            continue
        if in_remark and (ln.lstrip().startswith("|") or ln.split("|")[0].strip().isdigit()):
            continue
        in_remark = False
        if "packed-fp32-ops" not in ln and ln.strip():
            noise.append(ln)
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
