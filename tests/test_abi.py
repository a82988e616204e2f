"""Host-side checks of the C ABI: the library loads, exports every function
include/sinkroute.h declares, and rejects bad arguments before launching
anything (each case here fails validation, so no kernel is ever enqueued).
The work division the decode kernel uses is checked through sr_plan_parts,
which runs the same arithmetic on the host."""
import ctypes
import os
import re

import numpy as np
import pytest

from kv_cache_routing_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation
OUT = 0x40000000  # a different fake for out, which must not overlap q


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


def decode(s, launch=None, ws_bytes=1 << 30, q=FAKE, k=FAKE, v=FAKE, out=OUT, ws=FAKE,
           v0=FAKE, wl=FAKE, na=FAKE, sm_scale=0.0):
    lp = None if launch is None else ctypes.byref(launch)
    return N.lib.sr_decode_attn(ctypes.byref(s), lp, p(q), p(k), p(v), p(v0), p(wl), p(na),
                                sm_scale, p(ws), ws_bytes, p(out), None)


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
    assert decode(shape(), out=FAKE + 4096) == N.SR_ERR_INVALID_ARG  # out overlaps q


@pytest.mark.parametrize("scale", [float("nan"), float("inf"), float("-inf")])
def test_non_finite_softmax_scale(scale):
    # NaN and infinities are refused (a NaN is not "<= 0", which selects 1/sqrt(d))
    assert decode(shape(), sm_scale=scale) == N.SR_ERR_INVALID_ARG
    s = shape()
    assert N.lib.sr_dense_decode(ctypes.byref(s), None, p(), p(), p(), scale, p(), 1 << 30,
                                 p(OUT), None) == N.SR_ERR_INVALID_ARG


@pytest.mark.parametrize("which", ["q", "k", "v", "out", "ws", "v0", "wl", "na"])
def test_null_pointers(which):
    assert decode(shape(), **{which: 0}) == N.SR_ERR_INVALID_ARG


def test_dense_needs_no_routing_pointers_but_checks_the_rest():
    s = shape()
    r = N.lib.sr_dense_decode(ctypes.byref(s), None, p(), p(0), p(), 0.0, p(), 1 << 30, p(OUT),
                              None)
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


def test_adaptive_split_cap_values():
    # The lane count that minimises ceil(C / S) chunk times (32 KiB of bf16
    # K and V per 64-position chunk at 36 GB/s: 0.91 us) plus one merge round
    # (3 us) per started multiple of the merge's round size, capped by the
    # chunk count and the grid (256 workgroups when no GPU is visible).
    adaptive = N.SrLaunch(0, 0, 0, 0)
    cases = [  # (Hq, Hkv, d, T, dtype, expected cap)
        # 2048 chunks, rounds of 64: S = 64/128/192/256 cost 32.1/20.6/19.0/19.3 us
        (32, 8, 128, 131072, N.SR_KV_BF16, 192),
        # groups of 8, rounds of 32: S = 96/128/160 cost 29.0/26.6/26.8 us
        (64, 8, 128, 131072, N.SR_KV_BF16, 128),
        # one head per group, rounds of 256: one round reaches the grid
        (8, 8, 128, 524288, N.SR_KV_BF16, 256),
        # 64 fp32 chunks of 64 positions, rounds of 256: every chunk its own lane
        (4, 2, 64, 4096, N.SR_KV_F32, 64),
        (32, 8, 128, 100, N.SR_KV_BF16, 2),        # two chunks
        (32, 8, 128, 1, N.SR_KV_BF16, 1),
    ]
    grid = N.lib.sr_grid_size(ctypes.byref(shape()), ctypes.byref(adaptive))
    for Hq, Hkv, d, T, dt, want in cases:
        s = shape(Hq=Hq, Hkv=Hkv, d=d, T=T, dt=dt)
        got = N.lib.sr_split_cap(ctypes.byref(s), ctypes.byref(adaptive))
        if grid == 256:
            assert got == want, (Hq, d, T)
        assert 1 <= got <= min(grid, max(1, T))
    caps = [N.lib.sr_split_cap(ctypes.byref(shape(T=T)), ctypes.byref(adaptive))
            for T in (64, 1000, 4096, 8192, 65536, 1 << 20)]
    assert caps == sorted(caps)
    assert N.lib.sr_split_cap(ctypes.byref(shape(Hq=33)), ctypes.byref(adaptive)) == 0
    # a huge grid and cache: the search stays short and the cap in range
    import time
    huge = shape(T=(1 << 31) - 1)
    big_grid = N.SrLaunch(0, 0, 1 << 20, 0)
    t0 = time.perf_counter()
    cap = N.lib.sr_split_cap(ctypes.byref(huge), ctypes.byref(big_grid))
    assert time.perf_counter() - t0 < 0.05
    assert 1 <= cap <= N.lib.sr_grid_size(ctypes.byref(huge), ctypes.byref(big_grid))


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
        assert S <= N.lib.sr_split_cap(ctypes.byref(s), ctypes.byref(adaptive))
    assert N.lib.sr_split_cap(ctypes.byref(s), ctypes.byref(fixed)) == 37
    # 100 positions are two 64-position chunks: at most two lanes
    small = shape(T=100)
    assert N.lib.sr_split_cap(ctypes.byref(small), ctypes.byref(adaptive)) == 2
    assert N.lib.sr_splits_for(ctypes.byref(small), ctypes.byref(adaptive), 1) == 2


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
    for q, k0 in ((FAKE + 4, FAKE), (FAKE, FAKE + 8)):  # q and k0 are read as float4
        r = N.lib.sr_route(ctypes.byref(s), p(q), p(k0), ctypes.c_float(0.5), p(), p(), p(), p(),
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
    assert rd(flags=8) == N.SR_ERR_INVALID_ARG
    assert rd(flags=-1) == N.SR_ERR_INVALID_ARG
    assert rd(flags=N.SR_READ_LDS, unroll=32) == N.SR_ERR_INVALID_ARG
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
    assert int(defines["SR_READ_LDS"]) == N.SR_READ_LDS


def test_fused_route_decode_validation():
    s = shape()

    def fused(s, k0=FAKE, v0=FAKE, tau=0.5, ws_bytes=1 << 30):
        return N.lib.sr_route_decode(ctypes.byref(s), None, p(), p(), p(), p(k0), p(v0),
                                     ctypes.c_float(tau), 0.0, p(0), p(0), p(0), p(0), p(),
                                     ws_bytes, p(OUT), None)
    assert fused(s, k0=0) == N.SR_ERR_INVALID_ARG
    assert fused(s, v0=0) == N.SR_ERR_INVALID_ARG
    assert fused(s, tau=float("nan")) == N.SR_ERR_INVALID_ARG
    assert fused(s, ws_bytes=16) == N.SR_ERR_INVALID_ARG
    big = shape(B=4096, Hq=8, Hkv=8)            # 32768 items: the routing kernel's maximum
    assert fused(big, ws_bytes=16) == N.SR_ERR_INVALID_ARG  # runs as two launches; ws too small
    assert fused(shape(B=4097, Hq=8, Hkv=8)) == N.SR_ERR_UNSUPPORTED


def test_static_scratch_route_decode_validation():
    # The no-allocation form checks its arguments like sr_route_decode and
    # rejects, before anything is enqueued, a shape whose workspace would not
    # fit its fixed scratch.
    def call(s, launch=None, k0=FAKE, v0=FAKE, tau=0.5, q=FAKE, out=OUT):
        lp = None if launch is None else ctypes.byref(launch)
        return N.lib.sr_route_decode_static(ctypes.byref(s), lp, p(q), p(), p(), p(k0), p(v0),
                                            ctypes.c_float(tau), 0.0, p(0), p(0), p(0), p(0),
                                            p(out), None)
    s = shape()
    assert call(s, k0=0) == N.SR_ERR_INVALID_ARG
    assert call(s, v0=0) == N.SR_ERR_INVALID_ARG
    assert call(s, q=0) == N.SR_ERR_INVALID_ARG
    assert call(s, tau=float("nan")) == N.SR_ERR_INVALID_ARG
    assert call(s, out=FAKE + 64) == N.SR_ERR_INVALID_ARG     # out overlaps q
    assert call(shape(Hq=136)) == N.SR_ERR_UNSUPPORTED        # G = 17
    # 1024 KV groups of 16 heads at 4 workgroups per CU need just over 16 MiB
    big = shape(B=128, Hq=128, Hkv=8, T=64)
    lau = N.SrLaunch(0, 0, 4, 0)
    need = N.lib.sr_workspace_bytes(ctypes.byref(big), ctypes.byref(lau))
    assert need > N.SR_STATIC_SCRATCH_BYTES
    assert call(big, launch=lau) == N.SR_ERR_UNSUPPORTED
    # fixed split counts grow the workspace too
    lau = N.SrLaunch(4096, 0, 0, 0)
    assert N.lib.sr_workspace_bytes(ctypes.byref(s), ctypes.byref(lau)) > N.SR_STATIC_SCRATCH_BYTES
    assert call(s, launch=lau) == N.SR_ERR_UNSUPPORTED


def test_static_scratch_holds_8b_and_70b_layers():
    # The no-allocation form's fixed scratch takes every Llama-3.1-8B-shaped
    # (32 query / 8 KV heads) or 70B-shaped (64 / 8) layer of up to 64 KV
    # groups, at any context length and cache dtype, under the adaptive policy
    # at 1 to 8 workgroups per CU (the host sizes grids for 256 CUs when it
    # sees no GPU, MI355X's count), and under the default launch.
    sizes = []
    for Hq in (32, 64):
        for B in (1, 2, 4, 8):
            for T in (1, 4096, 131072, 524288, 1 << 24):
                for dt in (N.SR_KV_BF16, N.SR_KV_F32):
                    s = shape(B=B, Hq=Hq, Hkv=8, T=T, dt=dt)
                    for lau in [None] + [N.SrLaunch(0, 0, c, 0) for c in range(1, 9)]:
                        lp = None if lau is None else ctypes.byref(lau)
                        need = N.lib.sr_workspace_bytes(ctypes.byref(s), lp)
                        assert 0 < need <= N.SR_STATIC_SCRATCH_BYTES, (Hq, B, T, dt, lau)
                        sizes.append(need)
    # the largest of them is close enough to the limit that the check means something
    assert max(sizes) > N.SR_STATIC_SCRATCH_BYTES // 2


def test_rope_route_decode_validation():
    def call(s, kn=FAKE, vn=FAKE, f=FAKE, q_out=0, q=FAKE):
        return N.lib.sr_rope_route_decode(ctypes.byref(s), None, p(q), p(kn), p(vn), p(f),
                                          p(q_out), p(), p(), p(), p(), ctypes.c_float(0.5), 0.0,
                                          p(0), p(0), p(0), p(0), p(), 1 << 30, p(OUT), None)
    s = shape()
    assert call(s, kn=0) == N.SR_ERR_INVALID_ARG
    assert call(s, vn=0) == N.SR_ERR_INVALID_ARG
    assert call(s, f=0) == N.SR_ERR_INVALID_ARG
    assert call(shape(T=1)) == N.SR_ERR_INVALID_ARG            # position 0 is the sink key
    assert call(s, q_out=FAKE + 4096) == N.SR_ERR_INVALID_ARG  # overlaps q_new
    assert call(s, q_out=OUT + 64) == N.SR_ERR_INVALID_ARG     # overlaps out
    assert call(shape(B=3, Hq=32, Hkv=8)) == N.SR_ERR_INVALID_ARG  # 96 heads need q_out


# --- work division (host-side model of what the decode kernel streams) ----------
def plan(s, launch, n_active):
    """{wg: [sr_part, ...]} over the whole grid."""
    grid = N.lib.sr_grid_size(ctypes.byref(s), ctypes.byref(launch))
    buf = (N.SrPart * 2)()
    out = {}
    for wg in range(grid):
        r = N.lib.sr_plan_parts(ctypes.byref(s), ctypes.byref(launch), n_active, wg, buf, 2)
        assert 0 <= r <= 2, (wg, r)
        out[wg] = [N.SrPart.from_buffer_copy(buf[i]) for i in range(r)]
    return grid, out


def lane_major_chunks(first, end, C, S):
    """Chunks of lane-major positions [first, end): lane l holds chunks
    l, l + S, ... (Q + (l < rem) of them), lanes in order."""
    Q, rem = divmod(C, S)
    chunks, q = [], 0
    for lane in range(S):
        for k in range(Q + (lane < rem)):
            if first <= q < end:
                chunks.append(lane + k * S)
            q += 1
    return chunks


@pytest.mark.parametrize("kw,n_active,launch", [
    (dict(B=8, Hq=64, Hkv=8, T=131072), 29, (0, 2, 0, 0)),   # 70B shape, 29 of 64 active
    (dict(B=1, Hq=32, Hkv=8, T=524288), 4, (0, 2, 0, 0)),    # divides the grid: lanes
    (dict(B=4, Hq=32, Hkv=8, T=262144), 24, (0, 1, 0, 0)),   # VALU chunking
    (dict(B=2, Hq=8, Hkv=8, T=40000), 11, (0, 2, 2, 0)),     # 2 workgroups per CU
    (dict(B=1, Hq=32, Hkv=8, T=3000), 3, (0, 2, 0, 0)),      # split cap binds: lanes
    (dict(B=1, Hq=8, Hkv=2, T=200), 2, (7, 1, 0, 0)),        # fixed splits
    (dict(B=1, Hq=8, Hkv=2, T=70), 2, (9, 2, 0, 0)),         # more lanes than chunks
    (dict(B=40, Hq=8, Hkv=8, T=65536), 257, (0, 2, 0, 8)),   # >256 items, 8 waves
])
def test_plan_covers_every_chunk_once(kw, n_active, launch):
    s = shape(**kw)
    lau = N.SrLaunch(*launch)
    grid, parts = plan(s, lau, n_active)
    seen = {}
    per_wg, n_parts = [], {}
    for wg, ps in parts.items():
        total = 0
        for p in ps:
            S, chunk = p.lanes, p.chunk
            C = -(-kw["T"] // chunk)
            assert 0 <= p.item < n_active and 0 <= p.first <= p.end <= C
            n_parts.setdefault(p.item, set()).add((p.part, p.parts, wg))
            for c in lane_major_chunks(p.first, p.end, C, S):
                assert (p.item, c) not in seen, ("chunk twice", p.item, c)
                seen[(p.item, c)] = wg
            total += p.end - p.first
        if ps:
            per_wg.append(total)
    C = -(-kw["T"] // parts_chunk(parts))
    assert len(seen) == n_active * C                     # every chunk of every item
    for item, ps in n_parts.items():
        (count,) = {pp for _, pp, _ in ps}
        assert sorted(p for p, _, _ in ps) == list(range(count))
        wgs = sorted(w for _, _, w in ps)
        assert wgs == list(range(wgs[0], wgs[0] + count))  # parts are consecutive workgroups
    S = N.lib.sr_splits_for(ctypes.byref(s), ctypes.byref(lau), n_active)
    balanced = (launch[0] == 0 and n_active * S < grid
                and S < N.lib.sr_split_cap(ctypes.byref(s), ctypes.byref(lau)))
    if balanced:
        assert len(per_wg) == grid and max(per_wg) - min(per_wg) <= 1
    else:  # one lane of one item per workgroup
        assert all(len(ps) <= 1 for ps in parts.values())
        assert sum(1 for ps in parts.values() if ps) == n_active * S


def parts_chunk(parts):
    return next(p.chunk for ps in parts.values() for p in ps)


def test_plan_parts_rejects_bad_arguments():
    s = shape()
    lau = N.SrLaunch(0, 0, 0, 0)
    buf = (N.SrPart * 2)()
    grid = N.lib.sr_grid_size(ctypes.byref(s), ctypes.byref(lau))
    call = lambda n, wg, m=2: N.lib.sr_plan_parts(ctypes.byref(s), ctypes.byref(lau), n, wg, buf, m)
    assert call(-1, 0) == -1 and call(9, 0) == -1
    assert call(4, -1) == -1 and call(4, grid) == -1
    assert call(4, 0, 1) == -1
    assert call(0, 0) == 0                                  # nothing active: no cache work


def test_plan_random_layouts_tile_every_item():
    """Random shapes, kernels, grids and active counts: each item's parts,
    in workgroup order, tile its lane-major chunk sequence [0, C) exactly
    (lane-major positions are one-to-one with chunks), part numbers run
    0..parts-1, and balanced shares differ by at most one chunk."""
    rng = np.random.default_rng(2024)
    buf = (N.SrPart * 2)()
    for _ in range(150):
        Hkv = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.integers(1, 9))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        d = int(rng.choice([64, 128]))
        T = int(rng.integers(1, 400000))
        kern = int(rng.choice([1, 2]))
        waves = int(rng.choice([4, 8]))
        fixed = int(rng.choice([0, 0, 0, int(rng.integers(1, 40))]))
        per_cu = int(rng.choice([0, 1, 2, 3]))
        dt = int(rng.choice([N.SR_KV_BF16, N.SR_KV_F32]))
        s = shape(B=B, Hq=Hkv * G, Hkv=Hkv, d=d, T=T, dt=dt)
        lau = N.SrLaunch(fixed, kern, per_cu, waves)
        grid = N.lib.sr_grid_size(ctypes.byref(s), ctypes.byref(lau))
        n_act = int(rng.integers(0, B * Hkv + 1))
        items, totals = {}, []
        for wg in range(grid):
            r = N.lib.sr_plan_parts(ctypes.byref(s), ctypes.byref(lau), n_act, wg, buf, 2)
            assert 0 <= r <= 2
            tot = 0
            for i in range(r):
                p = N.SrPart.from_buffer_copy(buf[i])
                items.setdefault(p.item, []).append((wg, p.part, p.parts, p.first, p.end, p.chunk))
                tot += p.end - p.first
            if r:
                totals.append(tot)
        assert sorted(items) == list(range(n_act))
        for item, ps in items.items():
            ps.sort()
            C = -(-T // ps[0][5])
            assert [p[1] for p in ps] == list(range(len(ps))) and {p[2] for p in ps} == {len(ps)}
            assert ps[0][3] == 0 and ps[-1][4] == C
            for a, b in zip(ps, ps[1:]):
                assert a[4] == b[3] and b[0] == a[0] + 1
        S = N.lib.sr_splits_for(ctypes.byref(s), ctypes.byref(lau), n_act)
        if (fixed == 0 and n_act and n_act * S < grid
                and S < N.lib.sr_split_cap(ctypes.byref(s), ctypes.byref(lau))):
            assert len(totals) == grid and max(totals) - min(totals) <= 1


def test_binding_plan_parts_matches_the_abi():
    import kv_cache_routing_amd as sr
    s = shape(B=8, Hq=64, Hkv=8, T=131072)
    lau = N.SrLaunch(0, 2, 0, 0)
    got = sr.plan_parts(s, lau, 29, 7)
    buf = (N.SrPart * 2)()
    r = N.lib.sr_plan_parts(ctypes.byref(s), ctypes.byref(lau), 29, 7, buf, 2)
    assert len(got) == r >= 1
    assert got[0]["item"] == buf[0].item and got[0]["end"] == buf[0].end
    with pytest.raises(sr.SinkRouteError):
        sr.plan_parts(s, lau, 65, 0)


def test_build_rejects_kernels_with_scratch():
    from kv_cache_routing_amd.build import scratch_kernels
    report = "\n".join([
        "a.hip:1:1: remark: Function Name: k_good [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark: Function Name: k_spills [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     ScratchSize [bytes/lane]: 96 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert scratch_kernels(report) == ["k_spills (96 bytes/lane)"]
    assert scratch_kernels("") == []


def test_build_checks_lds_for_the_rotary_step():
    from kv_cache_routing_amd.build import LDS_LIMIT, ROPE_LDS_MAX, lds_overflows
    fits = LDS_LIMIT - ROPE_LDS_MAX
    report = "\n".join([
        "a.hip:1:1: remark: Function Name: k_decode_mfma_a [-Rpass-analysis=kernel-resource-usage]",
        f"a.hip:1:1: remark:     LDS Size [bytes/block]: {fits} [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark: Function Name: k_decode_mfma_b [-Rpass-analysis=kernel-resource-usage]",
        f"a.hip:9:1: remark:     LDS Size [bytes/block]: {fits + 1} [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark: Function Name: k_route [-Rpass-analysis=kernel-resource-usage]",
        f"a.hip:9:1: remark:     LDS Size [bytes/block]: {LDS_LIMIT} [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert [b.split(" ")[0] for b in lds_overflows(report)] == ["k_decode_mfma_b"]


def test_build_lds_bound_follows_the_fused_head_limit():
    # the build's dynamic-LDS bound is rope_lds_bytes at the largest fused
    # launch: kMaxFusedHeads query rows of the largest head size (128)
    from kv_cache_routing_amd.build import CSRC, ROPE_LDS_MAX
    src = open(os.path.join(CSRC, "sr_internal.h")).read()
    heads = int(re.search(r"kMaxFusedHeads\s*=\s*(\d+)", src).group(1))
    assert "static_cast<size_t>(d / 2) * 2 * sizeof(double)" in src
    assert "static_cast<size_t>(q_rows) * d * sizeof(float)" in src
    assert ROPE_LDS_MAX == 128 // 2 * 2 * 8 + heads * 128 * 4
