#!/usr/bin/env python3
"""Benchmark of one sink-routed decode layer-step on one MI355X.

A step is one pass of the whole hot path on one layer's cache: sr_route
(cosine scores, group decision, compacted work list) followed by
sr_decode_attn (sink bypass + split-K flash-decode of the active groups with
the in-kernel merge).  The default workload is the Llama-3.1-8B decode layer
at 524288 cached positions (B=1, 32 query / 8 KV heads, d=128, bf16 K/V,
4 of 8 KV groups planted as sinks), the shape the SinkRouter pages quote
their 512K speedup on.  Two copies of the layer are rotated so nothing of a
step's working set is still in the 256 MB Infinity Cache from the step before.

Prints ONE JSON line (the metric: effective HBM GB/s of the routed
layer-step, with us per layer-step, the dense baseline and the speedup), plus
the decode kernel's roofline position, measured live with HIP events, and
the fp64 CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps 50] [--warmup 5] [--no-sweep] [--no-cpu-baseline]
Environment knobs (no rebuild needed): SR_TAU, SR_SPLITS, SR_WGS_PER_CU,
SR_KERNEL (auto|valu|mfma).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
KERNEL_IDS = {"auto": 0, "valu": 1, "mfma": 2}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def decode_sources_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_routing_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_record(kernel_name: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        recs = json.load(f)
    rec = recs.get(f"{kernel_name}@{workload}")
    if not rec or rec.get("sources") != decode_sources_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def algorithmic_bytes(wl, n_active: int) -> int:
    """KV bytes of the active groups + q/out + k0/v0 (per layer-step)."""
    es = 2 if wl.kv_dtype == "bf16" else 4
    kv = n_active * 2 * wl.seq_len * wl.head_dim * es
    io = wl.batch * wl.num_q_heads * wl.head_dim * 4 * 2
    sink = wl.batch * wl.num_kv_heads * wl.head_dim * 4 * 2
    return kv + io + sink


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


def cpu_baseline(layer, n_active_items, budget_s=12.0):
    """The fp64 oracle on whole active items of the same layer, until about
    budget_s of CPU work; reported as effective GB/s of KV processed."""
    import numpy as np

    import oracle
    from workloads import as_numpy
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    wl = layer.wl
    G = wl.group_size
    q = as_numpy(layer.q)
    scale = 1.0 / math.sqrt(wl.head_dim)
    done, t_total, bytes_total = 0, 0.0, 0
    for j in n_active_items:
        b, g = divmod(int(j), wl.num_kv_heads)
        ks, vs = as_numpy(layer.k[b, g]), as_numpy(layer.v[b, g])
        t0 = time.perf_counter()
        oracle.attend_group(q[b, g * G:(g + 1) * G], ks, vs, scale)
        t_total += time.perf_counter() - t0
        bytes_total += 2 * wl.seq_len * wl.head_dim * 2
        done += 1
        if t_total >= budget_s:
            break
    t0 = time.perf_counter()
    oracle.route(q, as_numpy(layer.k[:, :, 0]), wl.tau)
    t_route = time.perf_counter() - t0
    per_item = t_total / done
    step_s = per_item * len(n_active_items) + t_route
    return {
        "value": round(bytes_total / t_total / 1e9, 4), "unit": "GB/s", "cores": int(cores),
        "kind": "oracle",
        "sample": (f"{done} of {len(n_active_items)} active KV groups of one "
                   f"{wl.name} layer-step (fp64 numpy, {wl.seq_len} positions, G={G}), "
                   f"{t_total:.1f} s; routed layer-step extrapolates to {step_s * 1e3:.0f} ms"),
        "us_per_layer_step": round(step_s * 1e6, 1),
        "seconds": round(t_total, 2),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rotate", type=int, default=2, help="layer caches rotated over steps")
    ap.add_argument("--no-sweep", action="store_true", help="skip the sink-fraction sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the decode path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}). Run with --gpus 1.", flush=True)
        return 2

    import torch

    import kv_cache_routing_amd as sr
    from workloads import L8B_512K, SINK_FRACTIONS, make_caches, make_queries, sweep

    wl = L8B_512K
    tau = float(os.environ.get("SR_TAU", wl.tau))
    kernel = os.environ.get("SR_KERNEL", "auto")
    lau = sr.make_launch(int(os.environ.get("SR_SPLITS", "0")), KERNEL_IDS[kernel],
                         int(os.environ.get("SR_WGS_PER_CU", "0")))
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    t0 = time.time()
    k_cpu, v_cpu = make_caches(wl)
    q_cpu, planted = make_queries(wl)
    log(f"generated {wl.name} in {time.time() - t0:.1f} s")
    caches = []
    for r in range(args.rotate):
        k = k_cpu.to(dev) if r == 0 else caches[0][0].clone()
        v = v_cpu.to(dev) if r == 0 else caches[0][1].clone()
        k0, v0 = sr.record_sink(k, v)
        caches.append((k, v, k0, v0))
    q = q_cpu.to(dev)
    shape = sr.make_shape(q, caches[0][0], caches[0][1])
    ws = sr.Workspace(shape, lau, dev)
    routes = [sr.route(q, c[2], tau) for c in caches]
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    n_active = int(routes[0].n_active.cpu()[0])
    active_items = routes[0].work_list.cpu().tolist()[:n_active]
    R = len(caches)

    def routed_step(i):
        k, v, k0, v0 = caches[i % R]
        r = routes[i % R]
        sr.route(q, k0, tau, out=r)
        sr.decode_attn(q, k, v, v0, r.work_list, r.n_active, launch=lau, ws=ws, out=out)

    def decode_only(i):
        k, v, k0, v0 = caches[i % R]
        r = routes[i % R]
        sr.decode_attn(q, k, v, v0, r.work_list, r.n_active, launch=lau, ws=ws, out=out)

    def dense_step(i):
        k, v, _, _ = caches[i % R]
        sr.dense_decode(q, k, v, launch=lau, ws=ws, out=out)

    for i in range(args.warmup):
        routed_step(i)
        dense_step(i)
    ms_routed = time_loop(routed_step, args.steps, stream)
    ms_decode = time_loop(decode_only, args.steps, stream)
    ms_dense = time_loop(dense_step, args.steps, stream)

    alg = algorithmic_bytes(wl, n_active)
    alg_dense = algorithmic_bytes(wl, wl.batch * wl.num_kv_heads)
    gbs = alg / (ms_routed * 1e-3) / 1e9
    dec_gbs = alg / (ms_decode * 1e-3) / 1e9
    dense_gbs = alg_dense / (ms_dense * 1e-3) / 1e9
    splits = sr.splits_for(shape, lau, n_active)
    kname = "k_decode_mfma" if (kernel == "mfma") else "k_decode_valu"
    traffic = traffic_record(kname, wl.name)

    sweep_rows = []
    if not args.no_sweep:
        k, v, k0, v0 = caches[0]
        for f in SINK_FRACTIONS:
            swl = sweep(wl, f)
            qf = make_queries(swl)[0].to(dev)
            rf = sr.route(qf, k0, tau)
            torch.cuda.synchronize()
            na = int(rf.n_active.cpu()[0])

            def st(i, qf=qf, rf=rf):
                kk, vv, kk0, vv0 = caches[i % R]
                sr.route(qf, kk0, tau, out=rf)
                sr.decode_attn(qf, kk, vv, vv0, rf.work_list, rf.n_active, launch=lau, ws=ws,
                               out=out)
            for i in range(args.warmup):
                st(i)
            ms = time_loop(st, args.steps, stream)
            sweep_rows.append({"sink_fraction": f, "n_active": na, "us": round(ms * 1e3, 2),
                               "t_over_t_dense": round(ms / ms_dense, 4),
                               "active_fraction": round(na / 8, 4),
                               "gbs": round(algorithmic_bytes(wl, na) / (ms * 1e-3) / 1e9, 1)})
            log(f"sweep f={f}: {ms * 1e3:.1f} us (n_active={na})")

    cpu = None
    if not args.no_cpu_baseline:
        layer = type("L", (), {})()
        layer.wl, layer.q, layer.k, layer.v = wl, q_cpu, k_cpu, v_cpu
        cpu = cpu_baseline(layer, active_items, args.cpu_budget)

    line = {
        "metric": "decode-attn µs/layer-step + effective HBM GB/s at 512K ctx bf16, vs dense path",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_routed, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: B={wl.batch} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
                               f"d={wl.head_dim} T={wl.seq_len} bf16 K/V, 4/8 groups sink, tau={tau}",
                   "global_batch": wl.batch, "seq_len": wl.seq_len, "parallelism": "none (1 GPU)",
                   "rotated_layers": R},
        "us_per_layer_step": round(ms_routed * 1e3, 2),
        "us_per_layer_step_dense": round(ms_dense * 1e3, 2),
        "speedup_vs_dense": round(ms_dense / ms_routed, 4),
        "sink_ratio": round(1 - n_active / (wl.batch * wl.num_kv_heads), 4),
        "dense_gbs": round(dense_gbs, 1),
        "decode_kernel_us": round(ms_decode * 1e3, 2),
        "splits_per_active_group": splits,
        "kernel": kernel,
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": kname,
                     "algorithmic_bytes_per_launch": alg},
        "cpu_baseline": cpu,
        "sweep_512k": sweep_rows,
        "context": "pages report 2.03x decode speedup at 512K (hardware not stated)",
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
