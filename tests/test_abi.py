"""Host-side checks of the C ABI: the library loads, exports every function
include/sinkroute.h declares, and rejects bad arguments before launching
anything (each case here fails validation, so no kernel is ever enqueued)."""
import ctypes
import os
import re

import pytest

from kv_cache_routing_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation


def header_functions():
    with open(os.path.join(ROOT, "include", "sinkroute.h")) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(sr_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    declared = header_functions()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(N.lib, name), name
    assert set(declared) == set(N.EXPORTS)


def test_version_and_status_strings():
    assert N.lib.sr_version() >= 100
    for s in (0, 1, 2, 3):
        assert N.status_string(s)
    assert "unsupported" in N.status_string(2)


def shape(B=1, Hq=32, Hkv=8, d=128, T=4096, dt=N.SR_KV_BF16, st=None, reserved=0):
    st = st or d
    return N.SrShape(B, Hq, Hkv, d, T, Hkv * T * st, T * st, st, dt, reserved)


def p(x=FAKE):
    return ctypes.c_void_p(x)


def decode(s, launch=None, ws_bytes=1 << 30, q=FAKE, k=FAKE, v=FAKE, out=FAKE, ws=FAKE,
           v0=FAKE, wl=FAKE, na=FAKE):
    lp = None if launch is None else ctypes.byref(launch)
    return N.lib.sr_decode_attn(ctypes.byref(s), lp, p(q), p(k), p(v), p(v0), p(wl), p(na), 0.0,
                                p(ws), ws_bytes, p(out), None)


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=34, Hkv=8), N.SR_ERR_INVALID_ARG),    # Hq not a multiple of Hkv
    (dict(Hq=136, Hkv=8), N.SR_ERR_UNSUPPORTED),   # G = 17
    (dict(d=96), N.SR_ERR_UNSUPPORTED),
    (dict(d=256), N.SR_ERR_UNSUPPORTED),
    (dict(T=0), N.SR_ERR_INVALID_ARG),
    (dict(B=0), N.SR_ERR_INVALID_ARG),
    (dict(dt=7), N.SR_ERR_INVALID_ARG),
    (dict(reserved=1), N.SR_ERR_INVALID_ARG),
    (dict(B=8193, Hkv=8, Hq=8), N.SR_ERR_UNSUPPORTED),  # > 32768 items
])
def test_shape_envelope(kw, status):
    assert decode(shape(**kw)) == status
    assert N.lib.sr_workspace_bytes(ctypes.byref(shape(**kw)), None) == 0


def test_stride_and_alignment_checks():
    s = shape(st=130)       # 260-byte rows are not 16-byte aligned for bf16
    assert decode(s) == N.SR_ERR_INVALID_ARG
    s = shape(st=120)       # stride_t < d
    assert decode(s) == N.SR_ERR_INVALID_ARG
    assert decode(shape(), k=FAKE + 8) == N.SR_ERR_INVALID_ARG
    assert decode(shape(), q=FAKE + 4) == N.SR_ERR_INVALID_ARG


@pytest.mark.parametrize("which", ["q", "k", "v", "out", "ws", "v0", "wl", "na"])
def test_null_pointers(which):
    assert decode(shape(), **{which: 0}) == N.SR_ERR_INVALID_ARG


def test_dense_needs_no_routing_pointers_but_checks_the_rest():
    s = shape()
    r = N.lib.sr_dense_decode(ctypes.byref(s), None, p(), p(0), p(), 0.0, p(), 1 << 30, p(), None)
    assert r == N.SR_ERR_INVALID_ARG


def test_workspace_too_small():
    s = shape()
    need = N.lib.sr_workspace_bytes(ctypes.byref(s), None)
    assert need > 0
    assert decode(s, ws_bytes=need - 1) == N.SR_ERR_INVALID_ARG


def test_launch_policy_checks():
    s = shape()
    assert decode(s, launch=N.SrLaunch(-1, 0, 0, 0)) == N.SR_ERR_INVALID_ARG
    assert decode(s, launch=N.SrLaunch(0, 9, 0, 0)) == N.SR_ERR_INVALID_ARG
    assert decode(s, launch=N.SrLaunch(0, 0, 0, 5)) == N.SR_ERR_INVALID_ARG   # 5 waves
    assert decode(s, launch=N.SrLaunch(0, 0, -1, 0)) == N.SR_ERR_INVALID_ARG
    f32 = shape(dt=N.SR_KV_F32)
    assert decode(f32, launch=N.SrLaunch(0, N.SR_KERNEL_MFMA, 0, 0)) == N.SR_ERR_UNSUPPORTED


def test_split_policy_host_math():
    s = shape(T=131072)
    fixed = N.SrLaunch(37, 0, 0, 0)
    assert N.lib.sr_grid_size(ctypes.byref(s), ctypes.byref(fixed)) == 8 * 37
    assert N.lib.sr_splits_for(ctypes.byref(s), ctypes.byref(fixed), 3) == 37
    adaptive = N.SrLaunch(0, 0, 2, 0)
    grid = N.lib.sr_grid_size(ctypes.byref(s), ctypes.byref(adaptive))
    assert grid >= 8
    for n_act in (1, 2, 4, 8):
        S = N.lib.sr_splits_for(ctypes.byref(s), ctypes.byref(adaptive), n_act)
        assert 1 <= S and S * n_act <= grid
        assert S <= -(-131072 // 512)
    small = shape(T=100)
    assert N.lib.sr_splits_for(ctypes.byref(small), ctypes.byref(adaptive), 1) == 1


def test_workspace_grows_with_splits():
    s = shape(T=131072)
    a = N.lib.sr_workspace_bytes(ctypes.byref(s), ctypes.byref(N.SrLaunch(8, 0, 0, 0)))
    b = N.lib.sr_workspace_bytes(ctypes.byref(s), ctypes.byref(N.SrLaunch(64, 0, 0, 0)))
    assert 0 < a < b
    # partials: per workgroup 3*GP + GP*d floats, GP = 4
    assert b - a >= 8 * 56 * (3 * 4 + 4 * 128) * 4


def test_route_and_record_validation():
    s = shape()
    r = N.lib.sr_route(ctypes.byref(s), p(), p(), ctypes.c_float(0.5), p(), p(), p(), p(0), None)
    assert r == N.SR_ERR_INVALID_ARG
    r = N.lib.sr_route(ctypes.byref(s), p(), p(), ctypes.c_float(float("nan")), p(), p(), p(), p(),
                       None)
    assert r == N.SR_ERR_INVALID_ARG
    r = N.lib.sr_record_sink(ctypes.byref(s), p(), p(), p(0), p(), None)
    assert r == N.SR_ERR_INVALID_ARG
    r = N.lib.sr_record_sink(None, p(), p(), p(), p(), None)
    assert r == N.SR_ERR_INVALID_ARG
    assert N.lib.sr_workspace_init(p(0), 16, None) == N.SR_ERR_INVALID_ARG


def test_stream_read_validation():
    def rd(flags=0, unroll=4, grid=256, buf=FAKE, nbytes=1 << 20):
        return N.lib.sr_stream_read(p(buf), nbytes, grid, unroll, flags, p(), None)
    assert rd(flags=4) == N.SR_ERR_INVALID_ARG
    assert rd(flags=-1) == N.SR_ERR_INVALID_ARG
    assert rd(unroll=3) == N.SR_ERR_INVALID_ARG
    assert rd(grid=0) == N.SR_ERR_INVALID_ARG
    assert rd(buf=FAKE + 8) == N.SR_ERR_INVALID_ARG
    assert rd(nbytes=8) == N.SR_ERR_INVALID_ARG


def test_header_constants_match_binding():
    with open(os.path.join(ROOT, "include", "sinkroute.h")) as f:
        text = f.read()
    defines = dict(re.findall(r"#define\s+(SR_[A-Z_0-9]+)\s+(\d+)", text))
    assert int(defines["SR_READ_BLOCKED"]) == N.SR_READ_BLOCKED
    assert int(defines["SR_READ_NONTEMPORAL"]) == N.SR_READ_NONTEMPORAL


def test_fused_route_decode_validation():
    s = shape()

    def fused(s, k0=FAKE, v0=FAKE, tau=0.5, ws_bytes=1 << 30):
        return N.lib.sr_route_decode(ctypes.byref(s), None, p(), p(), p(), p(k0), p(v0),
                                     ctypes.c_float(tau), 0.0, p(0), p(0), p(0), p(0), p(),
                                     ws_bytes, p(), None)
    assert fused(s, k0=0) == N.SR_ERR_INVALID_ARG
    assert fused(s, v0=0) == N.SR_ERR_INVALID_ARG
    assert fused(s, tau=float("nan")) == N.SR_ERR_INVALID_ARG
    assert fused(s, ws_bytes=16) == N.SR_ERR_INVALID_ARG
    big = shape(B=1024, Hq=8, Hkv=8)            # 8192 items > 4096
    assert fused(big) == N.SR_ERR_UNSUPPORTED
