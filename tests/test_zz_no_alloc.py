"""The no-allocation decode step, sr_route_decode_static, through the C ABI.

Its scratch is the library's own per-device array, so it is compared, bit for
bit, with sr_route_decode on a caller workspace (the same kernels under the
same launch policy): output, scores, mask, work list and active count.  The
calls run in a row through the one shared array with layers of different
sizes (larger, then smaller, then many more groups, then small again), so
each call finds the previous call's partials in the array and must still
start from zeroed tickets.  The first layers are also checked against the
fp64 oracle.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from parity import assert_outputs, assert_route, log, oracle_inputs, sink_rows_exact, upload
from workloads import Workload, make_layer, make_layer_bulk

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import kv_cache_routing_amd as sr
    from kv_cache_routing_amd import _native as N
else:  # collected on CPU only to be deselected by -m "not gpu"
    sr = N = None


def route_decode_static(q, k, v, k0, v0, tau, launch=None):
    shape = sr.make_shape(q, k, v)
    B, Hkv = k.shape[0], k.shape[1]
    dev = q.device
    out = torch.empty_like(q)
    r = sr.Routing(torch.empty((B, q.shape[1]), dtype=torch.float32, device=dev),
                   torch.empty((B, Hkv), dtype=torch.uint8, device=dev),
                   torch.empty((B * Hkv,), dtype=torch.int32, device=dev),
                   torch.empty((1,), dtype=torch.int32, device=dev))
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = N.lib.sr_route_decode_static(
        ctypes.byref(shape), None if launch is None else ctypes.byref(launch), P(q), P(k), P(v),
        P(k0), P(v0), ctypes.c_float(tau), ctypes.c_float(0.0), P(r.scores), P(r.mask),
        P(r.work_list), P(r.n_active), P(out),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    N.check(st, "sr_route_decode_static")
    return out, r


# In call order: 128 query heads (the routing kernel then the decode), a
# smaller 32-head layer (one launch), 1032 KV groups (the routing kernel's
# ticketed partition, tickets far past the first layers'), a fixed split
# count, then the small fp32 layer.
SEQUENCE = [
    (Workload("na-128-heads", 2, 64, 8, 128, 6000, "bf16", seed=301,
              sink_plan=("bernoulli", 0.5)), None, True),
    (Workload("na-32-heads", 1, 32, 8, 128, 3000, "bf16", seed=302, sink_plan=("count", 4)),
     None, True),
    (Workload("na-1032-groups", 129, 8, 8, 64, 16, "bf16", seed=303,
              sink_plan=("bernoulli", 0.5)), None, False),
    (Workload("na-fixed-splits", 1, 32, 8, 128, 5000, "bf16", seed=304, sink_plan=("count", 3)),
     (13, 0, 0, 0), False),
    (Workload("na-tiny-f32", 1, 4, 2, 64, 4096, "f32", seed=0, sink_plan=("tiny",)), None, True),
]


def _run(wl, lau_fields, with_oracle):
    layer = make_layer_bulk(wl) if wl.batch * wl.num_kv_heads > 64 else make_layer(wl)
    q, k, v = upload(layer)
    lau = None if lau_fields is None else sr.make_launch(*lau_fields)
    k0, v0 = sr.record_sink(k, v)
    ref, r_ref = sr.route_decode(q, k, v, k0, v0, wl.tau, launch=lau)
    got, r = route_decode_static(q, k, v, k0, v0, wl.tau, launch=lau)
    torch.cuda.synchronize()
    log(f"{wl.name}: {wl.batch * wl.num_kv_heads} groups, "
        f"{int(r.n_active.item())} active")
    assert torch.equal(got, ref), wl.name
    for name in ("scores", "mask", "work_list", "n_active"):
        assert torch.equal(getattr(r, name), getattr(r_ref, name)), (wl.name, name)
    if with_oracle:
        q_np, k_np, v_np = oracle_inputs(layer)
        k0_ref, v0_ref = oracle.record_sink(k_np, v_np)
        mask, n_active = assert_route(r, q_np, k0_ref, wl.tau)
        g = got.cpu().numpy()
        sink_rows_exact(g, v0_ref, mask, wl.group_size)
        ref_np = oracle.routed_decode(q_np, k_np, v_np, v0_ref, mask)
        if n_active:
            act = np.repeat(mask == 0, wl.group_size, axis=1)
            assert_outputs(g[act], ref_np[act], f"{wl.name} static scratch")
    return got


def test_static_scratch_calls_in_a_row_match_the_workspace_form():
    first = None
    for i, (wl, lau, with_oracle) in enumerate(SEQUENCE):
        got = _run(wl, lau, with_oracle)
        if i == 0:
            first = got.clone()
    # the first layer again, after every other size has passed through the array
    again = _run(*SEQUENCE[0])
    assert torch.equal(again, first)


def test_static_scratch_second_call_smaller():
    # two calls in a row, the second with a smaller layer
    _run(SEQUENCE[0][0].with_(name="na-large", seed=311), None, True)
    _run(SEQUENCE[1][0].with_(name="na-small", seq_len=1000, seed=312), None, True)
