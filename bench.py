#!/usr/bin/env python3
"""Benchmark of the sink-routed decode layer-step on one MI355X.

A step is one pass of the whole hot path on one layer's cache: the routing
(cosine scores, group decision, compacted work list) and the decode (sink
bypass + split-K flash-decode of the active groups with the in-kernel merge),
timed both as one sr_route_decode call and as the two-call form (sr_route,
then sr_decode_attn); each figure reports the faster form and names it.

The headline workload (the JSON line's `value`) is the Llama-3.1-8B decode
layer at 524288 cached positions (B=1, 32 query / 8 KV heads, d=128, bf16
K/V, 4 of 8 KV groups planted as sinks), the shape the SinkRouter pages
quote their 512K speedup on.  The line's `configs` list then times every
layer shape of the suite the same way: the 4096-position fp32 layer, the 8B
layer at 131072 positions, the 8B layer at 262144 positions with B=4 at sink
fractions 0/25/50/75/100 %, the 512K layer, and the 70B-shaped layer at
131072 positions with B=8.  Caches are drawn on the device (seeded, same
recipe as the parity tests' host generator) and enough layer copies are
rotated that nothing of a step's working set is still in the 256 MB Infinity
Cache from the step before (at least 4 GiB).  Every figure is the median of
--loops loops of --steps back-to-back steps after a settling warmup.

Prints ONE JSON line (the metric: effective HBM GB/s of the routed
layer-step, with us per layer-step, the dense baseline and the speedup), the
decode kernel's roofline position measured live with HIP events, and the
fp64 CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps 50] [--warmup 20] [--loops 5] [--settle 0.5]
                    [--no-configs] [--no-sweep] [--no-cpu-baseline]
Environment knobs (no rebuild needed): SR_TAU, SR_SPLITS, SR_WGS_PER_CU,
SR_KERNEL (auto|valu|mfma).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
KERNEL_IDS = {"auto": 0, "valu": 1, "mfma": 2}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """Source text without comments and whitespace, so that editing a comment
    does not invalidate counters taken on the same code."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return re.sub(r"\s+", "", text)


def decode_sources_digest() -> str:
    """Digest of the kernel sources' code (comments and whitespace ignored)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_routing_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(csrc, f)) as fh:
                h.update(f.encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def traffic_record(kernel_name: str, workload: str, path: str = TRAFFIC_JSON):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; otherwise None."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        recs = json.load(f)
    rec = recs.get(f"{kernel_name}@{workload}")
    if not rec or rec.get("sources") != decode_sources_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


CAL_BYTES = 256 << 20  # calibration buffer of the traffic counters


def _pmc_rows(path, counter):
    """{dispatch id: (kernel name, value)} from a rocprofv3 counter_collection csv."""
    import csv
    rows = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            rows[int(r["Dispatch_Id"])] = (r["Kernel_Name"], float(r["Counter_Value"]))
    return rows


def calibrate_counters(sr, torch, dev):
    """Kernels of known traffic for the counter scale, launched before the
    measured ones (`--calibrate`): the library's read probe with the decode
    kernels' access shape (16-byte non-temporal loads, 8 in flight per lane,
    256 workgroups), over CAL_BYTES once grid-strided and once per-workgroup
    blocked, then the library's fill kernel writing CAL_BYTES
    (sr_workspace_init)."""
    import ctypes
    from kv_cache_routing_amd import _native as N
    buf = torch.empty(CAL_BYTES, dtype=torch.uint8, device=dev)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for blocked in (0, N.SR_READ_BLOCKED):
        N.check(N.lib.sr_stream_read(ctypes.c_void_p(buf.data_ptr()), CAL_BYTES, 256, 8,
                                     N.SR_READ_NONTEMPORAL | blocked,
                                     ctypes.c_void_p(sink.data_ptr()), stream), "sr_stream_read")
    N.check(N.lib.sr_workspace_init(ctypes.c_void_p(buf.data_ptr()), CAL_BYTES, stream),
            "sr_workspace_init")
    torch.cuda.synchronize()
    del buf


def summarize_counters(fetch_csv, write_csv, workload: str, out_path: str = TRAFFIC_JSON):
    """HBM bytes per decode launch of one workload from two rocprofv3 --pmc
    runs of `bench.py --roofline-only --calibrate`: counter (KiB) x 1024 x
    scale, where FETCH_SIZE's scale is CAL_BYTES over its reading on the read
    probe's two calibration launches (the decode kernels' load shape) and
    WRITE_SIZE's is CAL_BYTES over its reading on the fill kernel.  Merged
    into out_path under kernel@workload."""
    fetch, write = _pmc_rows(fetch_csv, "FETCH_SIZE"), _pmc_rows(write_csv, "WRITE_SIZE")
    target = CAL_BYTES / 1024.0
    probe = sorted(d for d, (k, _) in fetch.items() if "k_stream_read" in k)
    fill = sorted(d for d, (k, _) in write.items() if "k_zero" in k)
    assert len(probe) == 2 and fill, "calibration launches not found"
    fill = [d for d in fill if abs(write[d][1] - target) < 0.05 * target] or fill[-1:]
    cal = {"FETCH_SIZE": {"kernel": "k_stream_read<8, true> (grid-strided, blocked)",
                          "kib": [fetch[d][1] for d in probe]},
           "WRITE_SIZE": {"kernel": "k_zero", "kib": [write[fill[-1]][1]]}}
    for c in cal.values():
        c["scale"] = CAL_BYTES / (sum(c["kib"]) / len(c["kib"]) * 1024.0)
    recs = {}
    if os.path.exists(out_path):
        with open(out_path) as f:
            recs = json.load(f)
    for kname in ("k_decode_valu", "k_decode_mfma", "k_route"):
        per = {}
        for counter, rows in (("FETCH_SIZE", fetch), ("WRITE_SIZE", write)):
            vals = [v for k, v in rows.values() if kname in k]
            if vals:
                kib = sum(vals) / len(vals)
                per[counter] = {"kib_per_dispatch": kib, "dispatches": len(vals),
                                "scale": cal[counter]["scale"],
                                "bytes_per_dispatch": kib * 1024.0 * cal[counter]["scale"]}
        if len(per) == 2:
            recs[f"{kname}@{workload}"] = {
                "sources": decode_sources_digest(), "calibration": cal,
                "hbm_bytes_per_launch": round(per["FETCH_SIZE"]["bytes_per_dispatch"]
                                              + per["WRITE_SIZE"]["bytes_per_dispatch"]),
                "fetch": per["FETCH_SIZE"], "write": per["WRITE_SIZE"]}
    with open(out_path, "w") as f:
        json.dump(recs, f, indent=1, sort_keys=True)
    print(json.dumps({k: v for k, v in recs.items() if k.endswith("@" + workload)}, indent=1))
    return recs


def algorithmic_bytes(wl, n_active: int) -> int:
    """KV bytes of the active groups + q/out + k0/v0 (per layer-step)."""
    es = 2 if wl.kv_dtype == "bf16" else 4
    kv = n_active * 2 * wl.seq_len * wl.head_dim * es
    io = wl.batch * wl.num_q_heads * wl.head_dim * 4 * 2
    sink = wl.batch * wl.num_kv_heads * wl.head_dim * 4 * 2
    return kv + io + sink


def time_launches(fn, steps, stream):
    """Average duration of one launch: an event pair around every launch, so
    the gaps between launches are not counted (comparable with a profiler's
    per-kernel duration)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        fn(i)
        b.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / steps  # ms


def read_ceiling(tensors, stream, grids=(256, 512, 1024), unrolls=(4, 8), lds=(0,)):
    """Best read bandwidth of the library's streaming probe over the given
    device tensors (16-byte loads per lane, the decode kernels' access width),
    grid-strided and per-workgroup-blocked, default and non-temporal loads,
    into registers or (lds=(0, 1)) staged through LDS by direct-to-LDS loads."""
    import ctypes

    import torch

    from kv_cache_routing_amd import _native as N
    sink = torch.zeros(max(grids), dtype=torch.int32, device=tensors[0].device)
    total = sum(t.numel() * t.element_size() for t in tensors)
    best, rows = 0.0, []
    shapes = [(st, nt, bl, grid, un) for st in lds for nt in (0, 1) for bl in (0, 1)
              for grid in grids for un in unrolls]
    for staged, nontemporal, blocked, grid, un in shapes:
        flags = (blocked * N.SR_READ_BLOCKED + nontemporal * N.SR_READ_NONTEMPORAL
                 + staged * N.SR_READ_LDS)

        def f(i, flags=flags, grid=grid, un=un):
            for t in tensors:
                N.check(N.lib.sr_stream_read(
                    ctypes.c_void_p(t.data_ptr()), t.numel() * t.element_size(), grid, un, flags,
                    ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream)),
                    "sr_stream_read")
        f(0)
        ms = time_loop(f, 5, stream)
        gbs = total / (ms * 1e-3) / 1e9
        rows.append({"lds": staged, "nontemporal": nontemporal, "blocked": blocked, "grid": grid,
                     "unroll": un, "gbs": round(gbs, 1)})
        if not staged:
            best = max(best, gbs)
    return best, rows


def warm_up(fns, steps, settle_s):
    """At least `steps` untimed rounds of every step form, and more until
    settle_s seconds of wall time have passed: the first tens of milliseconds
    of sustained load run several per cent slower while the clocks settle
    (measured: the first 30-step loop after a 12 ms warmup ran 318.7 us per
    step at 70B against 301-302 us in later loops).  Returns the rounds run."""
    import torch
    t0 = time.time()
    i = 0
    while i < steps or time.time() - t0 < settle_s:
        for fn in fns:
            fn(i)
        i += 1
        if i % 4 == 0:
            torch.cuda.synchronize()  # the wall clock follows the GPU, not the queue
    torch.cuda.synchronize()
    return i


def time_loop(fn, steps, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms


def cpu_baseline(wl, q, k0, slabs, tau, budget_s=12.0, chunk=32768, gpu_out=None):
    """The fp64 oracle on one routed layer-step of the workload, on the host
    cores: a thread pool over (active group, chunk of `chunk` positions), each
    piece the oracle's split partial of its chunk (oracle.split_partials with
    one split), merged per group in ascending chunk order by
    oracle.merge_partials (the oracle's split algebra, exact attention up to
    rounding), plus the oracle's routing of every head.  BLAS runs one thread
    per worker.  Passes repeat until budget_s of wall time; the median pass
    is the layer-step time.  slabs: {item: (q rows [G][d], K [T][d], V [T][d])}
    as host float32 arrays (exact copies of the bf16 caches)."""
    import concurrent.futures as cf
    import statistics

    import numpy as np

    import oracle
    blas, limits = "unknown", None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} "
                         f"({i.get('threading_layer', '')})" for i in threadpool_info()) or blas
        limits = threadpool_limits
    except Exception:  # pragma: no cover
        pass
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    scale = 1.0 / math.sqrt(wl.head_dim)
    items = sorted(slabs)
    tasks = [(j, t0) for j in items for t0 in range(0, wl.seq_len, chunk)]

    def piece(task):
        j, t0 = task
        qg, kk, vv = slabs[j]
        return oracle.split_partials(qg, kk[t0:t0 + chunk], vv[t0:t0 + chunk], scale, 1)[0]

    passes, outs = [], {}
    ctx = limits(limits=1) if limits else None
    if ctx:
        ctx.__enter__()
    try:
        cpu0, wall0 = time.process_time(), time.perf_counter()
        with cf.ThreadPoolExecutor(threads) as ex:
            while not passes or sum(passes) < budget_s:
                t0 = time.perf_counter()
                oracle.route(q, k0, tau)
                parts = list(ex.map(piece, tasks))
                for j in items:
                    outs[j] = oracle.merge_partials([p for (jj, _), p in zip(tasks, parts)
                                                     if jj == j])
                passes.append(time.perf_counter() - t0)
        cpu_s, wall_s = time.process_time() - cpu0, time.perf_counter() - wall0
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    step_s = statistics.median(passes)
    kv_bytes = len(items) * 2 * wl.seq_len * wl.head_dim * (2 if wl.kv_dtype == "bf16" else 4)
    rep = {
        "value": round(kv_bytes / step_s / 1e9, 4), "unit": "GB/s", "cores": threads,
        "kind": "oracle",
        "sample": (f"{len(passes)} routed layer-steps of {wl.name} ({len(items)} active KV "
                   f"groups of {wl.seq_len} positions, G={wl.group_size}, fp64 numpy; "
                   f"{len(tasks)} pieces of {chunk} positions per step on {threads} threads) "
                   f"in {sum(passes):.1f} s; median step {step_s * 1e3:.0f} ms"),
        "us_per_layer_step": round(step_s * 1e6, 1),
        "passes": len(passes),
        "seconds": round(sum(passes), 2),
        "cpu_seconds_per_wall_second": round(cpu_s / wall_s, 2),
        "cpu_model": _cpu_model(),
        "host_cpus": len(os.sched_getaffinity(0)),
        "numpy": np.__version__,
        "blas": blas,
    }
    if gpu_out is not None:  # the same step's GPU output, as a check of the sample
        G = wl.group_size
        err = 0.0
        for j in items:
            b, g = divmod(j, wl.num_kv_heads)
            err = max(err, float(np.abs(gpu_out[b, g * G:(g + 1) * G] - outs[j]).max()))
        rep["max_abs_vs_gpu"] = err
    return rep


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def envelope_report(sr, torch, args):
    """Dense-decode bandwidth over the supported envelope: bf16 and fp32 caches,
    d = 64 and 128, G = 1..16, B = 1, 8 KV heads, T sized for ~1 GiB of K + V
    (synthetic normal values).  Each kernel (automatic choice, vector ALU,
    matrix cores) is timed interleaved with the others after a settling time,
    as the median of 12 loops of 8 launches."""
    import statistics
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(5)
    rows = []
    for dt in ("bf16", "f32"):
        for d in (64, 128):
            for G in (1, 2, 4, 8, 16):
                Hkv, es = 8, (2 if dt == "bf16" else 4)
                T = (1 << 30) // (Hkv * d * es * 2)
                tdt = torch.bfloat16 if dt == "bf16" else torch.float32
                K = torch.randn((1, Hkv, T, d), generator=gen, device=dev).to(tdt)
                V = torch.randn((1, Hkv, T, d), generator=gen, device=dev).to(tdt)
                q = torch.randn((1, Hkv * G, d), generator=gen, device=dev)
                shape = sr.make_shape(q, K, V)
                nbytes = 2 * K.numel() * K.element_size()
                fns = {}
                for name in ("auto", "valu", "mfma"):
                    lau = sr.make_launch(0, KERNEL_IDS[name], 0, 0)
                    ws = sr.Workspace(shape, lau, dev)
                    out = torch.empty_like(q)
                    fns[name] = (lambda lau=lau, ws=ws, out=out:
                                 sr.dense_decode(q, K, V, launch=lau, ws=ws, out=out))
                t0 = time.time()
                while time.time() - t0 < args.settle:
                    for f in fns.values():
                        f()
                    torch.cuda.synchronize()
                res = {n: [] for n in fns}
                for _ in range(12):
                    for n, f in fns.items():
                        a = torch.cuda.Event(enable_timing=True)
                        b = torch.cuda.Event(enable_timing=True)
                        a.record()
                        for _ in range(8):
                            f()
                        b.record()
                        torch.cuda.synchronize()
                        res[n].append(a.elapsed_time(b) * 1e3 / 8)
                row = {"dtype": dt, "d": d, "G": G, "T": T, "bytes": nbytes}
                for n, v in res.items():
                    us = statistics.median(v)
                    row[n] = {"us": round(us, 1), "gbs": round(nbytes / us / 1e3, 1)}
                rows.append(row)
                log(f"{dt} d={d} G={G}: " + "  ".join(
                    f"{n} {row[n]['us']} us {row[n]['gbs']} GB/s" for n in res))
                del K, V
                torch.cuda.empty_cache()
    print(json.dumps({"envelope": rows}), flush=True)
    return 0


def decode_layers_report(sr, torch, args):
    """Per-token attention over a stack of layers: each layer rotates the new
    token's q and k and appends k, v (sr_rope_append), then runs routed
    attention (sr_route_decode) inside the gated layer range and dense
    attention (sr_dense_decode) outside it; timed again with each layer as
    one sr_rope_route_decode launch.  Caches come from the seeded GPU
    generator (timing only; every kernel's parity is tested elsewhere).  Sink
    groups' queries are built in the rotated frame (0.9 k0/|k0| + 0.05 noise)
    and turned back by -pos on the host, so the routing sees planted sinks."""
    import statistics

    from workloads import rope_inv_freq
    from workloads.synth import K0_NORM
    L, T0, N = args.decode_layers, args.context, args.tokens
    B, Hq, Hkv, d = 1, 32, 8, 128
    G = Hq // Hkv
    start, end = args.layer_range if args.layer_range else (0, L - 1)
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(9000)
    cap = T0 + N
    caches = []
    for layer in range(L):
        k = torch.randn((B, Hkv, cap, d), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((B, Hkv, cap, d), generator=gen, device=dev).to(torch.bfloat16)
        k0 = k[:, :, 0].float()
        k[:, :, 0] = (k0 * (K0_NORM / k0.norm(dim=-1, keepdim=True))).to(torch.bfloat16)
        caches.append((k, v))
    inv_freq = rope_inv_freq(d)
    f64 = inv_freq.double()
    hgen = torch.Generator().manual_seed(9001)
    plans = []  # per (token, layer): q_pre, k_new, v_new
    sinks = torch.zeros((L, Hkv), dtype=torch.bool)
    for layer in range(L):
        sinks[layer, torch.randperm(Hkv, generator=hgen)[:Hkv // 2]] = True
    for t in range(N):
        pos = T0 + t
        ang = -pos * f64
        c, s = torch.cos(ang), torch.sin(ang)
        row = []
        for layer in range(L):
            k0 = caches[layer][0][0, :, 0].double().cpu()
            target = torch.randn((B, Hq, d), generator=hgen, dtype=torch.float64)
            for h in range(Hq):
                if sinks[layer, h // G]:
                    target[0, h] = 0.9 * k0[h // G] / k0[h // G].norm() + 0.05 * target[0, h]
            lo, hi = target[..., : d // 2], target[..., d // 2:]
            q_pre = torch.cat([lo * c - hi * s, hi * c + lo * s], dim=-1).float()
            kn = torch.randn((B, Hkv, d), generator=hgen)
            vn = torch.randn((B, Hkv, d), generator=hgen)
            row.append((q_pre.to(dev), kn.to(dev), vn.to(dev)))
        plans.append(row)
    freq = inv_freq.to(dev)
    k0v0 = [sr.record_sink(k[:, :, :T0], v[:, :, :T0]) for k, v in caches]
    lau = sr.make_launch()
    shape = sr.make_shape(plans[0][0][0], caches[0][0][:, :, :cap], caches[0][1][:, :, :cap])
    ws = sr.Workspace(shape, lau, dev)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    q_rot = torch.empty_like(out)
    n_active = torch.zeros(L, dtype=torch.int32, device=dev)
    routing = [sr.Routing(torch.empty((B, Hq), device=dev), torch.empty((B, Hkv), dtype=torch.uint8,
                                                                          device=dev),
                          torch.empty(B * Hkv, dtype=torch.int32, device=dev), n_active[i:i + 1])
               for i in range(L)]

    q_rots = [[torch.empty_like(out) for _ in range(L)] for _ in range(N)]

    # --model-step: the rest of a Llama-3.1-8B decoder layer around the
    # attention, with random-init bf16 weights (timing only): QKV projection,
    # O projection and SwiGLU MLP as library M = 1 products, the residual adds
    # folded into them.  Each weight is stored in the layout whose product
    # streamed faster on MI355X (QKV and down as [out][in], O and gate/up as
    # [in][out]).  RMSNorm is left out (two vector ops per layer, fused in a
    # serving engine).  The new key and value come from the projection; the
    # attention keeps the planted rotated-frame queries, so that half of the
    # groups still route as sinks (a projected random query would make every
    # group active).
    Hd, Ff = Hq * d, 14336
    wts, hid = [], None
    if args.model_step:
        wgen = torch.Generator(device=dev).manual_seed(9002)

        def weight(rows, cols, fan_in):
            return (torch.randn((rows, cols), generator=wgen, device=dev)
                    * fan_in ** -0.5).to(torch.bfloat16)
        for _ in range(L):
            wts.append({"qkv": weight(Hd + 2 * Hkv * d, Hd, Hd), "o": weight(Hd, Hd, Hd),
                        "gu": weight(Hd, 2 * Ff, Hd), "down": weight(Hd, Ff, Ff)})
        hid = torch.randn((1, Hd), generator=wgen, device=dev).to(torch.bfloat16)

    def token(t, routed=True, attend=True, append=True, fused=False, model=False):
        pos = T0 + t
        for layer in range(L):
            k, v = caches[layer]
            qp, kn, vn = plans[t][layer]
            q_rot = q_rots[t][layer]
            if model:
                kvn = torch.nn.functional.linear(hid, wts[layer]["qkv"])[:, Hd:].float()
                kn = kvn[:, :Hkv * d].view(B, Hkv, d)
                vn = kvn[:, Hkv * d:].view(B, Hkv, d)
            if fused:  # one launch per layer; tau > 1 gives the dense result
                k0, v0 = k0v0[layer]
                tau = 0.5 if routed and start <= layer <= end else 2.0
                if attend:
                    sr.rope_route_decode(qp, kn, vn, k[:, :, :pos + 1], v[:, :, :pos + 1], k0,
                                         v0, freq, tau, launch=lau, ws=ws, out=out,
                                         routing=routing[layer], q_out=q_rot)
                if model:
                    w = wts[layer]
                    hid.addmm_(out.view(1, Hd).to(torch.bfloat16), w["o"])
                    gu = hid @ w["gu"]
                    act = torch.nn.functional.silu(gu[:, :Ff]) * gu[:, Ff:]
                    hid.addmm_(act, w["down"].t())
                continue
            if append:
                sr.rope_append(qp, kn, vn, k, v, pos, freq, q_out=q_rot)
            if not attend:
                continue
            kv = (k[:, :, :pos + 1], v[:, :, :pos + 1])
            if routed and start <= layer <= end:
                k0, v0 = k0v0[layer]
                sr.route_decode(q_rot, *kv, k0, v0, 0.5, launch=lau, ws=ws, out=out,
                                routing=routing[layer])
            else:
                sr.dense_decode(q_rot, *kv, launch=lau, ws=ws, out=out)

    # Eager pass: appends every token, fills the rotated queries.
    for t in range(N):
        token(t)
    torch.cuda.synchronize()
    active = int(n_active.sum())

    # One HIP graph per token and per variant, replayed like a serving loop
    # (host launch overhead out of the measurement).  Replays rewrite the same
    # cache positions with the same values.
    def graphs(**kw):
        gs = []
        for t in range(N):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                token(t, **kw)
            gs.append(g)
        return gs

    stream = torch.cuda.current_stream()

    def run(gs, reps=3):
        for g in gs:
            g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            for g in gs:
                g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (reps * len(gs)) * 1e3  # us per token

    variants = {"routed": dict(routed=True), "dense": dict(routed=False),
                "append_only": dict(attend=False),
                "attend_routed": dict(routed=True, append=False),
                "attend_dense": dict(routed=False, append=False),
                "routed_one": dict(routed=True, fused=True),
                "dense_one": dict(routed=False, fused=True)}
    if args.model_step:
        for kw in (dict(routed=True), dict(routed=False), dict(attend=False)):
            token(0, fused=True, model=True, **kw)  # eager first: library handles, workspaces
        torch.cuda.synchronize()
        variants.update({"full_routed": dict(routed=True, fused=True, model=True),
                         "full_dense": dict(routed=False, fused=True, model=True),
                         "rest": dict(attend=False, fused=True, model=True)})
    captured = {name: graphs(**kw) for name, kw in variants.items()}
    # Interleaved: every loop replays every variant once, so clock drift over
    # the run falls on all of them alike; each figure is the median of the loops.
    times = {name: [] for name in captured}
    for _ in range(args.loops):
        for name, gs in captured.items():
            times[name].append(run(gs))
    med = {name: statistics.median(v) for name, v in times.items()}
    routed, dense, append_only = med["routed"], med["dense"], med["append_only"]
    attend_routed, attend_dense = med["attend_routed"], med["attend_dense"]
    routed_one, dense_one = med["routed_one"], med["dense_one"]
    model_rep = None
    if args.model_step:
        full_routed, full_dense, rest = med["full_routed"], med["full_dense"], med["rest"]
        model_rep = {
            "layer": "Llama-3.1-8B decoder layer, random-init bf16 weights "
                     f"({sum(x.numel() for w in wts for x in w.values()) * 2 / 2 ** 30:.1f} GiB "
                     "for all layers): QKV, attention (one launch), O, SwiGLU MLP as library "
                     "M = 1 products, residual adds folded in, RMSNorm left out",
            "us_per_token_routed": round(full_routed, 1),
            "us_per_token_dense": round(full_dense, 1),
            "speedup": round(full_dense / full_routed, 4),
            "composition_us_per_token": {"projections_mlp": round(rest, 1),
                                         "attention_routed": round(full_routed - rest, 1),
                                         "attention_dense": round(full_dense - rest, 1)}}
    gated = sum(1 for layer in range(L) if start <= layer <= end)
    rep = {"decode_layers": {
        "layers": L, "context": T0, "tokens": N, "routed_layers": [start, end],
        "shape": f"B={B} Hq={Hq} Hkv={Hkv} d={d} bf16 K/V, half of the groups planted as sinks",
        "timing": "one HIP graph per token (rotary + append + attention for every layer); "
                  f"median of {args.loops} interleaved loops of 3 replays of every token",
        "active_groups_last_token": active, "groups_routed_layers": gated * B * Hkv,
        "us_per_token_routed": round(routed, 1), "us_per_token_dense": round(dense, 1),
        "speedup": round(dense / routed, 4),
        "composition_us_per_token": {"rope_append": round(append_only, 1),
                                     "attention_routed": round(attend_routed, 1),
                                     "attention_dense": round(attend_dense, 1)},
        "one_launch_per_layer": {  # sr_rope_route_decode (dense layers at tau > 1)
            "us_per_token_routed": round(routed_one, 1),
            "us_per_token_dense": round(dense_one, 1),
            "speedup": round(dense_one / routed_one, 4)},
        **({"model_step": model_rep} if model_rep else {}),
        "kv_gib_per_token_dense": round(L * 2 * B * Hkv * T0 * d * 2 / 2 ** 30, 2)}}
    print(json.dumps(rep), flush=True)
    return 0


# --- routing proxy against position-0 attention mass (evaluation only) -------
# The pith.science rendering of arXiv 2604.16883 (Figure 10 caption) scores
# cos(q, K_BOS) as a predictor of an "oracle" sink event defined from the
# full-attention weight of the first position, per KV group, across the
# threshold tau.  Predictions here are the HIP routing mask at each tau;
# events come from the HIP dense decode's alpha_0.  Reading for the event
# threshold, which the pages do not print: a group is an event when every
# one of its heads puts at least `event_mass` of its attention on position 0.
def sink_events(alpha0, num_kv_heads: int, event_mass: float):
    """[B][Hkv] bool tensor: every head of the group has alpha_0 >= event_mass."""
    B, Hq = alpha0.shape
    return (alpha0 >= event_mass).view(B, num_kv_heads, Hq // num_kv_heads).all(dim=-1)


def precision_recall(predicted, events):
    """(precision, recall, F1); precision is 1 when nothing is predicted,
    recall 1 when there is no event, F1 0 when both are 0."""
    p = predicted.reshape(-1).bool()
    e = events.reshape(-1).bool()
    tp = int((p & e).sum())
    fp = int((p & ~e).sum())
    fn = int((~p & e).sum())
    prec = tp / (tp + fp) if tp + fp else 1.0
    rec = tp / (tp + fn) if tp + fn else 1.0
    f1 = 2 * prec * rec / (prec + rec) if prec + rec else 0.0
    return prec, rec, f1


def proxy_sweep(predict, events, taus):
    """Precision / recall / F1 of the routing decision at every tau;
    predict(tau) returns the [B][Hkv] sink mask."""
    rows = []
    for tau in taus:
        p, r, f = precision_recall(predict(float(tau)), events)
        rows.append({"tau": float(tau), "precision": p, "recall": r, "f1": f})
    return rows


def bos_proxy_report(sr, torch):
    """Routing proxy vs position-0 attention mass, from GPU outputs only."""
    from workloads import L8B_128K, make_layer
    dev = torch.device("cuda:0")
    taus = [round(0.05 * i, 2) for i in range(21)]
    report = []
    for k0_norm in (30.0, 120.0, 400.0):
        wl = L8B_128K.with_(name=f"llama8b-32k-b4-k0norm{int(k0_norm)}", batch=4, seq_len=32768,
                            seed=7000 + int(k0_norm), k0_norm=k0_norm)
        layer = make_layer(wl)
        q, k, v = layer.q.to(dev), layer.k.to(dev), layer.v.to(dev)
        k0, _ = sr.record_sink(k, v)
        _, a0 = sr.dense_decode_alpha0(q, k, v)
        torch.cuda.synchronize()
        ev = sink_events(a0, wl.num_kv_heads, 0.5)

        def predict(tau, q=q, k0=k0):
            return sr.route(q, k0, tau).mask.bool()
        report.append({"layer": wl.name, "planted_sinks": int(layer.planted.sum()),
                       "events": int(ev.sum()), "groups": wl.batch * wl.num_kv_heads,
                       "alpha0_planted_mean": float(a0.view(wl.batch, wl.num_kv_heads, -1)[
                           layer.planted.to(dev)].mean()),
                       "sweep": proxy_sweep(predict, ev, taus)})
        log(f"bos proxy {wl.name}: events {int(ev.sum())}")
    print(json.dumps({"bos_proxy": report}), flush=True)
    return 0


def device_clocks():
    """GPU clocks as rocm-smi reports them (best effort; None if unavailable)."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                           text=True, timeout=30)
        data = json.loads(r.stdout)
        return {card: {k.rstrip(":"): v for k, v in vals.items() if "clk" in k.lower()}
                for card, vals in data.items() if isinstance(vals, dict)}
    except Exception as e:  # pragma: no cover
        return {"unavailable": type(e).__name__}


def sclk_now():
    """The GPU core clock level marked current in sysfs (MHz), if readable."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                for ln in f:
                    if ln.rstrip().endswith("*"):
                        return ln.split(":", 1)[1].strip().rstrip("*").strip()
        except OSError:
            continue
    return None


def rotation(wl, rotate: int) -> int:
    """Layer copies rotated over the timed steps: enough for >= 4 GiB, so no
    step finds the previous step's data in the 256 MB Infinity Cache."""
    if rotate > 0:
        return rotate
    es = 2 if wl.kv_dtype == "bf16" else 4
    layer_bytes = 2 * wl.batch * wl.num_kv_heads * wl.seq_len * wl.head_dim * es
    return max(1, min(8, -(-(4 << 30) // layer_bytes)))


def device_layers(sr, torch, wl, R, dev):
    """R device copies (k, v, k0, v0) of the workload's caches, drawn on the
    device (timing only: the parity tests use the host generator)."""
    from workloads import make_caches_device
    k, v = make_caches_device(wl, dev)
    caches = []
    for r in range(R):
        kk, vv = (k, v) if r == 0 else (k.clone(), v.clone())
        caches.append((kk, vv, *sr.record_sink(kk, vv)))
    return caches


def same_size_read(sr, torch, nbytes: int, R: int, args, stream):
    """The library's read probe over `nbytes` in one launch (the decode's
    grid of 256 workgroups of 4 waves, 16-byte non-temporal loads, 8 in
    flight), best of grid-strided and blocked, timed like the decode kernel
    (back-to-back launches between one event pair, median of --loops loops),
    over R rotated buffers.  The bare-read time of the decode kernel's bytes."""
    import ctypes
    import statistics

    from kv_cache_routing_amd import _native as N
    nbytes = nbytes // 16 * 16
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    best = None
    for blocked in (0, N.SR_READ_BLOCKED):
        def f(i, blocked=blocked):
            N.check(N.lib.sr_stream_read(ctypes.c_void_p(bufs[i % R].data_ptr()), nbytes, 256, 8,
                                         N.SR_READ_NONTEMPORAL | blocked,
                                         ctypes.c_void_p(sink.data_ptr()),
                                         ctypes.c_void_p(stream.cuda_stream)), "sr_stream_read")
        warm_up([f], args.warmup, 0.1)
        us = statistics.median(time_loop(f, args.steps, stream) for _ in range(args.loops)) * 1e3
        best = us if best is None else min(best, us)
    del bufs
    return best


def capture_graph(torch, fn, steps):
    """`steps` steps of `fn` captured in one HIP graph (after one eager call),
    replayed once: replaying it gives the GPU's own time per step, without the
    host's launch rate and argument checks."""
    fn(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, steps, stream):
    """ms per step of one replay of a graph of `steps` steps."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def measure(sr, torch, wl, lau, tau, args, caches, q, *, dense=True, decode=True, probe=True,
            dense_us=None):
    """One workload's layer-step, each form timed as the median of --loops
    loops of --steps back-to-back steps (HIP events on the launch stream)
    after the settling warmup: sr_route_decode (one call), sr_route +
    sr_decode_attn (two calls), sr_dense_decode, the one-call and dense steps
    again replayed from a HIP graph; the decode kernel alone, back to back
    (the roofline figure) and with an event pair per launch; and the bare
    read of the same bytes."""
    import statistics
    stream = torch.cuda.current_stream()
    R = len(caches)
    shape = sr.make_shape(q, caches[0][0], caches[0][1])
    ws = sr.Workspace(shape, lau, q.device)
    out = torch.empty_like(q)
    routes = [sr.route(q, c[2], tau) for c in caches]
    torch.cuda.synchronize()
    n_items = wl.batch * wl.num_kv_heads
    n_active = int(routes[0].n_active.item())

    def fused(i):
        k, v, k0, v0 = caches[i % R]
        sr.route_decode(q, k, v, k0, v0, tau, launch=lau, ws=ws, out=out, routing=routes[i % R])

    def two_calls(i):
        k, v, k0, v0 = caches[i % R]
        r = routes[i % R]
        sr.route(q, k0, tau, out=r)
        sr.decode_attn(q, k, v, v0, r.work_list, r.n_active, launch=lau, ws=ws, out=out)

    def dense_step(i):
        k, v, _, _ = caches[i % R]
        sr.dense_decode(q, k, v, launch=lau, ws=ws, out=out)

    def decode_only(i):
        k, v, k0, v0 = caches[i % R]
        r = routes[i % R]
        sr.decode_attn(q, k, v, v0, r.work_list, r.n_active, launch=lau, ws=ws, out=out)

    forms = {"fused": fused, "two_calls": two_calls}
    if dense:
        forms["dense"] = dense_step
    warm = warm_up(list(forms.values()) + ([decode_only] if decode else []), args.warmup,
                   args.settle)
    # the graph-replayed forms are timed inside the same loops as the eager
    # ones, so that a drift of the GPU's speed during the run affects both
    graphs = {"fused": capture_graph(torch, fused, args.steps)}
    if dense:
        graphs["dense"] = capture_graph(torch, dense_step, args.steps)
    runs = {name: [] for name in forms}
    graph_runs = {name: [] for name in graphs}
    dec, dec_b2b = [], []
    for _ in range(args.loops):
        for name, fn in forms.items():
            runs[name].append(time_loop(fn, args.steps, stream) * 1e3)
        for name, g in graphs.items():
            graph_runs[name].append(time_graph(torch, g, args.steps, stream) * 1e3)
        if decode:
            dec.append(time_launches(decode_only, args.steps, stream) * 1e3)
            dec_b2b.append(time_loop(decode_only, args.steps, stream) * 1e3)
    del graphs
    med = {name: statistics.median(v) for name, v in runs.items()}
    graph = {name: statistics.median(v) for name, v in graph_runs.items()}
    step = min(med["fused"], med["two_calls"])
    alg = algorithmic_bytes(wl, n_active)
    rep = {"workload": wl.name,
           "shape": f"B={wl.batch} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} d={wl.head_dim} "
                    f"T={wl.seq_len} {wl.kv_dtype}",
           "tau": tau, "groups": n_items, "n_active": n_active,
           "sink_ratio": round(1 - n_active / n_items, 4),
           "us_per_layer_step": round(step, 2),
           "form": "sr_route_decode" if med["fused"] <= med["two_calls"] else
                   "sr_route + sr_decode_attn",
           "us_fused": round(med["fused"], 2), "us_two_calls": round(med["two_calls"], 2),
           "us_fused_graph": round(graph["fused"], 2),
           "us_loops": {k: [round(x, 2) for x in v] for k, v in runs.items()},
           "algorithmic_bytes": alg, "step_gbs": round(alg / step / 1e3, 1),
           "loops": args.loops, "steps": args.steps, "warmup_rounds_run": warm,
           "rotated_layers": R}
    d_us = med.get("dense", dense_us)
    if d_us is not None:
        rep["us_dense"] = round(d_us, 2)
        if "dense" in graph:
            rep["us_dense_graph"] = round(graph["dense"], 2)
        rep["speedup_vs_dense"] = round(d_us / step, 4)
        rep["pages_fields"] = {"context_length": wl.seq_len, "baseline_latency_us": round(d_us, 2),
                               "sinkrouter_latency_us": round(step, 2),
                               "throughput": round(1e6 / step, 1),
                               "sink_ratio": rep["sink_ratio"],
                               "speedup": round(d_us / step, 4)}
    if decode:
        # back to back: includes the gap between launches, so it errs low;
        # it matched rocprof's per-dispatch average within 0.2 % at 512K, while
        # an event pair per launch adds the events' own ~2.5 us
        d = statistics.median(dec_b2b)
        rep["decode_kernel_us"] = round(d, 2)
        rep["decode_kernel_us_event_pairs"] = round(statistics.median(dec), 2)
        rep["decode_gbs"] = round(alg / d / 1e3, 1)
        rep["decode_frac_of_8tbs"] = round(alg / d / 1e3 / HBM_PEAK_GBS, 4)
        if probe and n_active:
            kv = alg - algorithmic_bytes(wl, 0)
            r_us = same_size_read(sr, torch, kv, R, args, stream)
            rep["same_size_read_us"] = round(r_us, 2)
            rep["same_size_read_gbs"] = round(kv / r_us / 1e3, 1)
            rep["decode_frac_of_same_size_read"] = round(r_us / d, 4)
    rep["sclk_after"] = sclk_now()
    del ws, out, routes
    return rep


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--loops", type=int, default=5,
                    help="timed loops of --steps steps per form; the median is reported")
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed warmup at least (beyond --warmup steps)")
    ap.add_argument("--workload", default="llama8b-512k",
                    help="headline workload: llama8b-512k (default), llama8b-128k, "
                         "llama8b-256k-b4-sink{0,25,50,75,100}, llama70b-128k-b8, tiny-4k-f32")
    ap.add_argument("--rotate", type=int, default=0,
                    help="layer copies rotated over steps (0 = enough for >= 4 GiB)")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the headline workload, not every configuration")
    ap.add_argument("--no-sweep", action="store_true", help="skip the 512K sink-fraction sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-compare", action="store_true",
                    help="skip timing the decode kernel under each kernel variant")
    ap.add_argument("--bos-proxy", action="store_true",
                    help="precision/recall of the cosine routing rule against position-0 "
                         "attention-mass events (alpha_0 >= 0.5 in every head) over a tau "
                         "sweep, on synthetic 8B-shaped layers at several k0 norms, and exit")
    ap.add_argument("--decode-layers", type=int, default=0, metavar="L",
                    help="per-token decode over L layers (rotary + append, then routed or "
                         "dense attention per layer) and exit")
    ap.add_argument("--context", type=int, default=131072, help="context of --decode-layers")
    ap.add_argument("--tokens", type=int, default=8, help="decode steps of --decode-layers")
    ap.add_argument("--model-step", action="store_true",
                    help="--decode-layers also runs each layer's projections and MLP "
                         "(random-init Llama-3.1-8B weights) around the attention")
    ap.add_argument("--layer-range", type=int, nargs=2, default=None, metavar=("START", "END"),
                    help="layers routed by --decode-layers (inclusive); the rest run dense")
    ap.add_argument("--envelope", action="store_true",
                    help="dense-decode bandwidth of every kernel over the envelope "
                         "(bf16/fp32, d = 64/128, G = 1..16, ~1 GiB each) and exit")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="print the HBM read-probe sweep over the layer caches and exit")
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the routed decode launches of the roofline measurement "
                         "(the command the committed rocprofv3 summaries profile)")
    ap.add_argument("--calibrate", action="store_true",
                    help="with --roofline-only: first run the counter calibration kernels "
                         f"(the read probe and the fill kernel over {CAL_BYTES >> 20} MiB)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --roofline-only --calibrate --workload W` into "
                         "profiles/traffic.json and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.workload)
        return 0

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the decode path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}). Run with --gpus 1.", flush=True)
        return 2

    import statistics

    import torch

    import kv_cache_routing_amd as sr
    from workloads import CONFIGS, L8B_256K_B4, SINK_FRACTIONS, make_queries, sweep

    if args.bos_proxy:
        return bos_proxy_report(sr, torch)
    if args.envelope:
        return envelope_report(sr, torch, args)
    if args.decode_layers:
        return decode_layers_report(sr, torch, args)

    names = {w.name: w for w in CONFIGS}
    names.update({sweep(L8B_256K_B4, f).name: sweep(L8B_256K_B4, f) for f in SINK_FRACTIONS})
    if args.workload not in names:
        print(f"unknown workload {args.workload}; choose from {sorted(names)}", flush=True)
        return 2
    wl = names[args.workload]
    tau = float(os.environ.get("SR_TAU", wl.tau))
    kernel = os.environ.get("SR_KERNEL", "auto")
    lau = sr.make_launch(int(os.environ.get("SR_SPLITS", "0")), KERNEL_IDS[kernel],
                         int(os.environ.get("SR_WGS_PER_CU", "0")))
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    kname = "k_decode_valu" if kernel == "valu" else "k_decode_mfma"

    if args.roofline_only:
        if args.calibrate:
            calibrate_counters(sr, torch, dev)
        caches = device_layers(sr, torch, wl, rotation(wl, args.rotate), dev)
        q = make_queries(wl)[0].to(dev)
        R = len(caches)
        routes = [sr.route(q, c[2], tau) for c in caches]
        ws = sr.Workspace(sr.make_shape(q, caches[0][0], caches[0][1]), lau, dev)
        out = torch.empty_like(q)
        torch.cuda.synchronize()
        n_active = int(routes[0].n_active.item())

        def decode_only(i):
            k, v, k0, v0 = caches[i % R]
            r = routes[i % R]
            sr.decode_attn(q, k, v, v0, r.work_list, r.n_active, launch=lau, ws=ws, out=out)
        warm_up([decode_only], args.warmup, args.settle)
        us = time_loop(decode_only, args.steps, stream) * 1e3
        alg = algorithmic_bytes(wl, n_active)
        print(json.dumps({"roofline_only": True, "workload": wl.name, "kernel": kname,
                          "decode_kernel_us": round(us, 2),
                          "achieved_gbs": round(alg / us / 1e3, 1),
                          "algorithmic_bytes_per_launch": alg, "launches": args.steps}),
              flush=True)
        return 0

    t0 = time.time()
    caches = device_layers(sr, torch, wl, rotation(wl, args.rotate), dev)
    q_cpu = make_queries(wl)[0]
    q = q_cpu.to(dev)
    log(f"generated {wl.name} x{len(caches)} on the device in {time.time() - t0:.1f} s")
    if args.read_ceiling:
        best, rows = read_ceiling([t for c in caches for t in c[:2]], stream,
                                  unrolls=(4, 8, 16), lds=(0, 1))
        print(json.dumps({"read_ceiling_gbs": round(best, 1), "bytes": sum(
            t.numel() * t.element_size() for c in caches for t in c[:2]), "sweep": rows}),
            flush=True)
        return 0

    head = measure(sr, torch, wl, lau, tau, args, caches, q)
    log(f"{wl.name}: {json.dumps({k: head[k] for k in ('us_per_layer_step', 'us_dense', 'decode_kernel_us')})}")
    R = len(caches)
    shape = sr.make_shape(q, caches[0][0], caches[0][1])
    n_active = head["n_active"]

    compare = {}
    if not args.no_compare:
        for name in ("valu", "mfma"):
            lk = sr.make_launch(lau.num_splits, KERNEL_IDS[name], lau.wgs_per_cu)
            wsk = sr.Workspace(shape, lk, dev)
            outk = torch.empty_like(q)
            rk = [sr.route(q, c[2], tau) for c in caches]

            def dk(i, lk=lk, wsk=wsk, outk=outk, rk=rk):
                k, v, k0, v0 = caches[i % R]
                r = rk[i % R]
                sr.decode_attn(q, k, v, v0, r.work_list, r.n_active, launch=lk, ws=wsk, out=outk)

            def dd(i, lk=lk, wsk=wsk, outk=outk):
                k, v, _, _ = caches[i % R]
                sr.dense_decode(q, k, v, launch=lk, ws=wsk, out=outk)
            warm_up([dk, dd], args.warmup, 0.1)
            compare[name] = {
                "routed_decode_us": round(statistics.median(
                    time_loop(dk, args.steps, stream) for _ in range(args.loops)) * 1e3, 2),
                "dense_decode_us": round(statistics.median(
                    time_loop(dd, args.steps, stream) for _ in range(args.loops)) * 1e3, 2)}
            log(f"kernel {name}: {compare[name]}")

    sweep_rows = []
    if not args.no_sweep:
        for f in SINK_FRACTIONS:
            swl = sweep(wl, f)
            row = measure(sr, torch, swl, lau, tau, args, caches,
                          make_queries(swl)[0].to(dev), dense=False, decode=False,
                          probe=False, dense_us=head["us_dense"])
            sweep_rows.append({"sink_fraction": f, "n_active": row["n_active"],
                               "us": row["us_per_layer_step"], "form": row["form"],
                               "us_fused_graph": row["us_fused_graph"],
                               "t_over_t_dense": round(row["us_per_layer_step"] / head["us_dense"], 4),
                               "active_fraction": round(1 - row["sink_ratio"], 4),
                               "gbs": row["step_gbs"]})
            log(f"sweep f={f}: {row['us_per_layer_step']} us (n_active={row['n_active']})")
        t_full = sweep_rows[0]["us"]
        for row in sweep_rows:
            row["t_over_t0"] = round(row["us"] / t_full, 4)
            row["dev_from_linear"] = round(row["us"] / t_full - (1 - row["sink_fraction"]), 4)

    ceiling, _ = read_ceiling([t for c in caches for t in c[:2]], stream, grids=(256, 512),
                              unrolls=(8,))

    cpu = None
    if not args.no_cpu_baseline:
        # host copies of the active groups (exact: bf16 widens to fp32)
        from workloads import as_numpy
        k, v, k0, v0 = caches[0]
        r = sr.route(q, k0, tau)
        out = sr.route_decode(q, k, v, k0, v0, tau, launch=lau)[0]
        torch.cuda.synchronize()
        active = [int(j) for j in r.work_list.cpu().tolist()[:n_active]]
        G = wl.group_size
        q_np = as_numpy(q_cpu)
        slabs = {}
        for j in active:
            b, g = divmod(j, wl.num_kv_heads)
            slabs[j] = (q_np[b, g * G:(g + 1) * G], as_numpy(k[b, g].cpu()),
                        as_numpy(v[b, g].cpu()))
        cpu = cpu_baseline(wl, q_np, as_numpy(k0.cpu()), slabs, tau, args.cpu_budget,
                           gpu_out=out.cpu().numpy())
        del slabs
        log(f"cpu baseline: {cpu['sample']}")
    del caches
    torch.cuda.empty_cache()

    configs = []
    if not args.no_configs:
        for cwl in CONFIGS:
            if cwl.name == wl.name:
                configs.append(head)
                continue
            cc = device_layers(sr, torch, cwl, rotation(cwl, args.rotate), dev)
            ctau = float(os.environ.get("SR_TAU", cwl.tau))
            if cwl.name == L8B_256K_B4.name:  # five sink fractions on the same caches
                for i, f in enumerate(SINK_FRACTIONS):
                    swl = sweep(cwl, f)
                    rep = measure(sr, torch, swl, lau, ctau, args, cc,
                                  make_queries(swl)[0].to(dev), dense=i == 0,
                                  dense_us=configs[-1]["us_dense"] if i else None)
                    configs.append(rep)
                    log(f"{swl.name}: {rep['us_per_layer_step']} us")
            else:
                rep = measure(sr, torch, cwl, lau, ctau, args, cc, make_queries(cwl)[0].to(dev))
                if cwl.kv_dtype == "f32" and cwl.seq_len <= 4096:
                    rep["note"] = "launch-bound layer (4 MiB of cache): the time in us is the figure"
                configs.append(rep)
                log(f"{cwl.name}: {rep['us_per_layer_step']} us")
            del cc
            torch.cuda.empty_cache()
    for rep in configs:
        rep["traffic"] = traffic_record(kname, rep["workload"])

    props = torch.cuda.get_device_properties(dev)
    device = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
              "compute_units": props.multi_processor_count,
              "hbm_gib": round(props.total_memory / 2**30, 1), "hip": torch.version.hip,
              "torch": torch.__version__, "clocks": device_clocks()}
    splits = sr.splits_for(shape, lau, n_active)
    grid = sr.grid_size(shape, lau)
    parts0 = sr.plan_parts(shape, lau, n_active, 0)
    balanced = n_active * splits < grid and splits < sr.split_cap(shape, lau)
    launch_info = {"waves_per_wg": lau.waves_per_wg or 4, "grid": grid,
                   "lanes_per_active_group": splits,
                   "positions_per_lane": -(-wl.seq_len // splits),
                   "chunk_positions": parts0[0]["chunk"] if parts0 else 0,
                   "mode": "balanced" if balanced else "lanes"}
    ms_step = head["us_per_layer_step"] / 1e3
    dec_gbs = head["decode_gbs"]
    line = {
        "metric": "decode-attn µs/layer-step + effective HBM GB/s at 512K ctx bf16, vs dense path",
        "workload": wl.name,
        "value": head["step_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "loops": args.loops,
        "timing": (f"median of {args.loops} loops of {args.steps} back-to-back layer-steps, "
                   "HIP events on the launch stream, after a settling warmup"),
        "settle_s": args.settle,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.kv_dtype,
        "data": "synthetic (seeded N(0,1) caches drawn on the device, planted sink queries)",
        "config": {"workload": f"{wl.name}: B={wl.batch} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
                               f"d={wl.head_dim} T={wl.seq_len} {wl.kv_dtype} K/V, "
                               f"{head['groups'] - n_active}/{head['groups']} groups sink, "
                               f"tau={tau}",
                   "global_batch": wl.batch, "seq_len": wl.seq_len, "parallelism": "none (1 GPU)",
                   "rotated_layers": head["rotated_layers"]},
        "us_per_layer_step": head["us_per_layer_step"],
        "us_per_layer_step_fused": head["us_fused"],
        "us_per_layer_step_two_calls": head["us_two_calls"],
        "us_per_layer_step_dense": head["us_dense"],
        "speedup_vs_dense": head["speedup_vs_dense"],
        "step": f"{head['form']}, the faster of the one-call and two-call forms",
        "sink_ratio": head["sink_ratio"],
        "decode_kernel_us": head["decode_kernel_us"],
        "splits_per_active_group": splits,
        "kernel": kernel,
        "launch": launch_info,
        "device": device,
        "pages_fields": head["pages_fields"],
        "roofline": {"bound": "hbm", "achieved": dec_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_record(kname, wl.name), "kernel": kname,
                     "algorithmic_bytes_per_launch": head["algorithmic_bytes"],
                     "launch_us": head["decode_kernel_us"],
                     "timing": (f"{args.steps} decode launches back to back between one event "
                                "pair on the launch stream, median of the loops"),
                     "measured_read_ceiling_gbs": round(ceiling, 1),
                     "frac_of_measured_ceiling": round(dec_gbs / ceiling, 4),
                     "same_size_read_us": head.get("same_size_read_us"),
                     "frac_of_same_size_read": head.get("decode_frac_of_same_size_read")},
        "cpu_baseline": cpu,
        "configs": configs,
        "sink_fraction_sweep": sweep_rows,
        "sink_fraction_sweep_max_dev_from_linear": (
            max(abs(r["dev_from_linear"]) for r in sweep_rows) if sweep_rows else None),
        "kernel_compare": compare,
        "context": "pages report 2.03x decode speedup at 512K (hardware not stated)",
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
