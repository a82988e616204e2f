"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every test draws its layer from the seeded generator, runs record -> route ->
decode on cuda:0 and checks: routing mask and work list bit-exact, sink rows
bit-exact v0, active rows within max-abs 1e-2 / mean-abs 1e-3 / per-row
rel-L2 1e-3 of the oracle (plus a tighter 2e-4 precision check).
Small layers are checked in full, and so is every group of the full-size layers.
"""
import functools
import math
import os

import numpy as np
import pytest
import torch

import oracle
from parity import (assert_outputs, assert_route, log, oracle_inputs, route_ticket,
                    sink_rows_exact, ticket_region, upload)
from workloads import (CONFIGS, L70B_128K_B8, L8B_128K, L8B_256K_B4, L8B_512K, SINK_FRACTIONS,
                       TINY, Workload, as_numpy, make_caches, make_layer, make_layer_bulk,
                       make_queries, sweep)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import kv_cache_routing_amd as sr
else:  # collected on CPU only to be deselected by -m "not gpu"
    sr = None

BF16_KERNELS = ["valu", "mfma"]
KERNEL_ID = {"valu": 1, "mfma": 2, "auto": 0}


def launch(kernel="auto", splits=0, per_cu=0, waves=0):
    return sr.make_launch(splits, KERNEL_ID[kernel], per_cu, waves)


def run_routed(q, k, v, tau, lau):
    k0, v0 = sr.record_sink(k, v)
    r = sr.route(q, k0, tau)
    out = sr.decode_attn(q, k, v, v0, r.work_list, r.n_active, launch=lau)
    return k0, v0, r, out


def full_check(layer, lau, tau=None, check_dense=True):
    wl = layer.wl
    tau = wl.tau if tau is None else tau
    G = wl.group_size
    q_np, k_np, v_np = oracle_inputs(layer)
    q, k, v = upload(layer)
    k0, v0, r, out = run_routed(q, k, v, tau, lau)
    torch.cuda.synchronize()
    k0_ref, v0_ref = oracle.record_sink(k_np, v_np)
    assert np.array_equal(k0.cpu().numpy(), k0_ref) and np.array_equal(v0.cpu().numpy(), v0_ref)
    mask, n_active = assert_route(r, q_np, k0_ref, tau)
    got = out.cpu().numpy()
    ref = oracle.routed_decode(q_np, k_np, v_np, v0_ref, mask)
    n_sink = sink_rows_exact(got, v0_ref, mask, G)
    log(f"{wl.name} T={wl.seq_len} G={G} n_active={n_active} sink_rows={n_sink}")
    if n_active:
        act = np.repeat(mask == 0, G, axis=1)
        assert_outputs(got[act], ref[act], "routed active rows")
    if check_dense:
        dense = sr.dense_decode(q, k, v, launch=lau).cpu().numpy()
        assert_outputs(dense, oracle.dense_decode(q_np, k_np, v_np), "dense")
    return got


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
def test_tiny_layer_full_parity(kernel):
    log(f"tiny {kernel}")
    full_check(make_layer(TINY), launch(kernel))


REDUCED = [
    Workload("8b-ragged", 1, 32, 8, 128, 12345, "bf16", seed=11, sink_plan=("count", 4)),
    Workload("70b-shape", 2, 64, 8, 128, 6000, "bf16", seed=12, sink_plan=("bernoulli", 0.5)),
    Workload("d64-g2", 2, 8, 4, 64, 3001, "bf16", seed=13, sink_plan=("count", 2)),
    Workload("g3-nonpow2", 1, 12, 4, 128, 2100, "bf16", seed=14, sink_plan=("count", 1)),
    Workload("mha-g1", 1, 8, 8, 128, 5000, "bf16", seed=15, sink_plan=("count", 3)),
    Workload("g16-d64", 1, 32, 2, 64, 2000, "bf16", seed=16, sink_plan=("count", 1)),
    Workload("g6-d64", 3, 12, 2, 64, 999, "bf16", seed=17, sink_plan=("bernoulli", 0.5)),
    Workload("f32-d128-g4", 1, 16, 4, 128, 3333, "f32", seed=18, sink_plan=("count", 2)),
    Workload("f32-g8-d64", 2, 16, 2, 64, 700, "f32", seed=19, sink_plan=("count", 1)),
    # fp32 groups of 16 heads: 4 elements per lane (lane groups of 32 at d = 128)
    Workload("f32-g16-d128", 1, 32, 2, 128, 2999, "f32", seed=20, sink_plan=("count", 1)),
    Workload("f32-g16-d64", 2, 16, 1, 64, 1001, "f32", seed=23, sink_plan=("bernoulli", 0.5)),
]


@pytest.mark.parametrize("wl", REDUCED, ids=lambda w: w.name)
@pytest.mark.parametrize("kernel", ["auto"] + BF16_KERNELS)
def test_reduced_layers(wl, kernel):
    log(f"reduced {wl.name} kernel={kernel}")
    full_check(make_layer(wl), launch(kernel))


# The paper's operating threshold (pith.science, Figure 10 caption: tau =
# 0.55) on the reduced layers: both kernels, two calls against the oracle,
# and the one-call form bitwise equal to them.
@pytest.mark.parametrize("wl", REDUCED, ids=lambda w: w.name)
@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_reduced_layers_at_tau_055(wl, kernel):
    log(f"reduced {wl.name} kernel={kernel} tau=0.55")
    layer = make_layer(wl)
    lau = launch(kernel)
    got = full_check(layer, lau, tau=0.55, check_dense=False)
    q, k, v = upload(layer)
    k0, v0 = sr.record_sink(k, v)
    fused, rf = sr.route_decode(q, k, v, k0, v0, 0.55, launch=lau)
    torch.cuda.synchronize()
    assert torch.equal(fused.cpu(), torch.from_numpy(got))
    q_np, k_np, v_np = oracle_inputs(layer)
    assert_route(rf, q_np, oracle.record_sink(k_np, v_np)[0], 0.55)


# Groups of 8 and 16 heads take the PV product on the matrix cores (keys as
# the A operand, value tile transposed through LDS): padded head counts,
# ragged tails, one and seventeen positions, both head sizes, 4 and 8 waves.
MFMA_PV = [
    Workload("pv-g8-d64", 2, 16, 2, 64, 3001, "bf16", seed=31, sink_plan=("count", 1)),
    Workload("pv-g16-d128", 1, 32, 2, 128, 4099, "bf16", seed=32, sink_plan=("count", 1)),
    Workload("pv-g5-d128", 2, 10, 2, 128, 2500, "bf16", seed=33, sink_plan=("bernoulli", 0.5)),
    Workload("pv-g12-d64", 1, 24, 2, 64, 1500, "bf16", seed=34, sink_plan=("count", 1)),
    Workload("pv-g8-t1", 2, 16, 2, 128, 1, "bf16", seed=35, sink_plan=("none",)),
    Workload("pv-g16-t17", 2, 16, 1, 64, 17, "bf16", seed=36, sink_plan=("none",)),
]


@pytest.mark.parametrize("wl", MFMA_PV, ids=lambda w: w.name)
@pytest.mark.parametrize("waves", [4, 8])
def test_matrix_core_pv_groups(wl, waves):
    log(f"mfma pv {wl.name} waves={waves}")
    full_check(make_layer(wl), launch("mfma", waves=waves))


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_split_count_sweep(kernel):
    wl = Workload("8b-splits", 1, 32, 8, 128, 8192 + 77, "bf16", seed=21, sink_plan=("count", 4))
    layer = make_layer(wl)
    q_np, k_np, v_np = oracle_inputs(layer)
    ref = oracle.dense_decode(q_np, k_np, v_np)
    q, k, v = upload(layer)
    for S in (1, 2, 3, 7, 64, 129, 300):
        got = sr.dense_decode(q, k, v, launch=launch(kernel, splits=S)).cpu().numpy()
        assert_outputs(got, ref, f"dense S={S}")
    for per_cu in (1, 2, 4, 8):
        got = sr.dense_decode(q, k, v, launch=launch(kernel, per_cu=per_cu)).cpu().numpy()
        assert_outputs(got, ref, f"dense adaptive {per_cu}/CU")


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_more_splits_than_positions(kernel):
    wl = Workload("short", 1, 8, 2, 128, 200, "bf16", seed=22)
    layer = make_layer(wl)
    q, k, v = upload(layer)
    ref = oracle.dense_decode(*oracle_inputs(layer))
    got = sr.dense_decode(q, k, v, launch=launch(kernel, splits=205)).cpu().numpy()
    assert_outputs(got, ref, "S = T + 5")


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_tau_above_one_matches_dense_bitwise_and_repeats(kernel):
    wl = L8B_128K.with_(seq_len=20000, name="8b-20k")
    layer = make_layer(wl)
    q, k, v = upload(layer)
    for lau in (launch(kernel), launch(kernel, splits=17)):
        k0, v0, r, out = run_routed(q, k, v, 2.0, lau)
        assert int(r.n_active.cpu()[0]) == 8
        dense = sr.dense_decode(q, k, v, launch=lau)
        assert torch.equal(out, dense)
    # repeated calls on one workspace: bitwise identical, tickets back to zero
    lau = launch(kernel)
    shape = sr.make_shape(q, k, v)
    ws = sr.Workspace(shape, lau, q.device)
    k0, v0 = sr.record_sink(k, v)
    r = sr.route(q, k0, wl.tau)
    first = sr.decode_attn(q, k, v, v0, r.work_list, r.n_active, launch=lau, ws=ws).clone()
    for _ in range(200):
        again = sr.decode_attn(q, k, v, v0, r.work_list, r.n_active, launch=lau, ws=ws)
        assert torch.equal(again, first)
    torch.cuda.synchronize()
    assert int(ticket_region(ws, 8).abs().sum()) == 0


@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_fixed_splits_routed_rows_equal_dense_rows(kernel):
    wl = L8B_128K.with_(seq_len=9000, name="8b-9k")
    layer = make_layer(wl)
    q, k, v = upload(layer)
    lau = launch(kernel, splits=11)
    k0, v0, r, out = run_routed(q, k, v, wl.tau, lau)
    dense = sr.dense_decode(q, k, v, launch=lau)
    act = (r.mask == 0).repeat_interleave(4, dim=1)
    assert torch.equal(out[act], dense[act])


def test_special_cases_single_position_zero_query_fixed_point():
    # T = 1: the output is v0 exactly (one weight of 1)
    wl = Workload("t1", 2, 8, 2, 128, 1, "bf16", seed=31)
    layer = make_layer(wl)
    q, k, v = upload(layer)
    for kernel in BF16_KERNELS:
        out = sr.dense_decode(q, k, v, launch=launch(kernel)).cpu()
        assert torch.equal(out, layer.v[:, :, 0].float().repeat_interleave(4, dim=1))
    # q = 0: uniform weights, output is the mean of V; every score is 0 -> active
    wl = Workload("q0", 1, 8, 2, 64, 3000, "bf16", seed=32)
    layer = make_layer(wl)
    q, k, v = upload(layer)
    q.zero_()
    k0, v0, r, out = run_routed(q, k, v, 0.5, launch("auto"))
    assert int(r.n_active.cpu()[0]) == 2 and float(r.scores.abs().max()) == 0.0
    ref = np.repeat(as_numpy(layer.v).astype(np.float64).mean(axis=2), 4, axis=1)
    assert_outputs(out.cpu().numpy(), ref, "q=0 mean of V")
    # fixed point: all softmax mass at position 0 -> the output is v0
    d, T = 64, 4096
    gen = torch.Generator().manual_seed(33)
    kk = torch.randn((1, 1, T, d), generator=gen)
    vv = torch.randn((1, 1, T, d), generator=gen)
    kk[0, 0, 0] *= 400.0 / kk[0, 0, 0].norm()
    qq = (kk[0, 0, 0] / kk[0, 0, 0].norm()).reshape(1, 1, d).contiguous()
    out = sr.dense_decode(qq.cuda(), kk.cuda(), vv.cuda()).cpu()[0, 0]
    err = (out - vv[0, 0, 0]).abs().max().item()
    log(f"  fixed point: |dense - v0|_inf = {err:.3e}")
    assert err <= 1e-5


def test_all_sinks_and_no_sinks():
    wl = Workload("edges", 2, 16, 4, 128, 4000, "bf16", seed=41, sink_plan=("count", 2))
    layer = make_layer(wl)
    q, k, v = upload(layer)
    k0, v0, r, out = run_routed(q, k, v, -2.0, launch("auto"))   # every cosine >= -2
    assert int(r.n_active.cpu()[0]) == 0
    assert torch.equal(out, v0.repeat_interleave(4, dim=1))
    q_np, k_np, v_np = oracle_inputs(layer)
    k0, v0, r, out = run_routed(q, k, v, 1.5, launch("auto"))    # nothing reaches 1.5
    assert int(r.n_active.cpu()[0]) == 8
    assert_outputs(out.cpu().numpy(), oracle.dense_decode(q_np, k_np, v_np), "tau 1.5")


@functools.lru_cache(maxsize=None)
def _sharp_layer(dtype):
    return make_layer(Workload(f"sharp-{dtype}", 1, 32, 8, 128, 20000, dtype, seed=77,
                               sink_plan=("count", 4)))


# Softmax scales above the default 1/sqrt(d) (Eq. (1) with the scale as the
# decode call's parameter; the oracle takes the same one): the distribution
# turns peaky, the split partials' maxima then differ by hundreds, most merge
# weights underflow to zero, and the rounding of the logits grows with their
# size.  Routed (one call) and dense, against the oracle at the tight bound;
# one split per item and the adaptive split must both hold it.
@pytest.mark.parametrize("mult", [4, 16, 64])
@pytest.mark.parametrize("kernel", BF16_KERNELS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sharp_softmax_scales_against_oracle(dtype, kernel, mult):
    layer = _sharp_layer(dtype)
    sc = mult / math.sqrt(128)
    log(f"sharp softmax {dtype} kernel={kernel} scale={mult}/sqrt(d)")
    q_np, k_np, v_np = oracle_inputs(layer)
    k0_ref, v0_ref = oracle.record_sink(k_np, v_np)
    q, k, v = upload(layer)
    k0, v0 = sr.record_sink(k, v)
    dense_ref = oracle.dense_decode(q_np, k_np, v_np, scale=sc)
    for splits in (0, 1):
        lau = launch(kernel, splits=splits)
        out, r = sr.route_decode(q, k, v, k0, v0, 0.5, sm_scale=sc, launch=lau)
        dense = sr.dense_decode(q, k, v, sm_scale=sc, launch=lau)
        torch.cuda.synchronize()
        mask = assert_route(r, q_np, k0_ref, 0.5)[0]
        got = out.cpu().numpy()
        sink_rows_exact(got, v0_ref, mask, 4)
        ref = oracle.routed_decode(q_np, k_np, v_np, v0_ref, mask, scale=sc)
        act = np.repeat(mask == 0, 4, axis=1)
        assert_outputs(got[act], ref[act], f"routed, splits={splits}")
        assert_outputs(dense.cpu().numpy(), dense_ref, f"dense, splits={splits}")


@pytest.mark.parametrize("wl,kernel", [
    (Workload("strided", 2, 16, 4, 128, 3000, "bf16", seed=51, sink_plan=("count", 2)), "mfma"),
    (Workload("strided", 2, 16, 4, 128, 3000, "bf16", seed=51, sink_plan=("count", 2)), "valu"),
    (Workload("strided-d64-g8", 2, 16, 2, 64, 2000, "bf16", seed=52, sink_plan=("count", 1)), "mfma"),
    (Workload("strided-f32-g16", 1, 32, 2, 128, 1800, "f32", seed=53, sink_plan=("count", 1)), "mfma"),
    (Workload("strided-f32-g4", 2, 16, 4, 64, 2100, "f32", seed=54, sink_plan=("count", 2)), "valu"),
], ids=lambda x: x.name if hasattr(x, "name") else x)
def test_strided_cache_views(wl, kernel):
    """Caches viewed out of larger buffers (position stride > d): rows past T
    hold poison that must never be read."""
    layer = make_layer(wl)
    B, Hkv, T, d = layer.k.shape
    big_k = torch.zeros((B, Hkv, T + 333, d), dtype=layer.k.dtype)
    big_v = torch.zeros_like(big_k)
    big_k[:, :, :T] = layer.k
    big_v[:, :, :T] = layer.v
    big_k[:, :, T:] = 1e4   # poison: must never be read
    big_v[:, :, T:] = float("nan")
    k = big_k.cuda()[:, :, :T]
    v = big_v.cuda()[:, :, :T]
    q = layer.q.cuda()
    k0, v0, r, out = run_routed(q, k, v, wl.tau, launch(kernel))
    torch.cuda.synchronize()
    q_np, k_np, v_np = oracle_inputs(layer)
    # every reference from the oracle on the unpadded host arrays
    k0_ref, v0_ref = oracle.record_sink(k_np, v_np)
    assert np.array_equal(k0.cpu().numpy(), k0_ref) and np.array_equal(v0.cpu().numpy(), v0_ref)
    mask, n_active = assert_route(r, q_np, k0_ref, wl.tau)
    assert 0 < n_active < wl.batch * wl.num_kv_heads
    got = out.cpu().numpy()
    sink_rows_exact(got, v0_ref, mask, wl.group_size)
    ref = oracle.routed_decode(q_np, k_np, v_np, v0_ref, mask)
    act = np.repeat(mask == 0, wl.group_size, axis=1)
    assert_outputs(got[act], ref[act], f"strided routed {kernel}")
    dense = sr.dense_decode(q, k, v, launch=launch(kernel)).cpu().numpy()
    assert_outputs(dense, oracle.dense_decode(q_np, k_np, v_np), f"strided dense {kernel}")


# --- full-size layers, every item --------------------------------------------
# The oracle finishes a whole routed layer-step of these layers in about a
# second, so every active group is compared with it (and every group of the
# dense path), not a sample.
def _item_refs(layer, items):
    """Oracle attention of the listed items j = b*Hkv + g: {j: [G][d]}."""
    wl = layer.wl
    G = wl.group_size
    q_np = as_numpy(layer.q)
    scale = 1.0 / math.sqrt(wl.head_dim)
    refs = {}
    for j in items:
        b, g = divmod(int(j), wl.num_kv_heads)
        refs[int(j)] = oracle.attend_group(q_np[b, g * G:(g + 1) * G], as_numpy(layer.k[b, g]),
                                           as_numpy(layer.v[b, g]), scale)
    return refs


def _check_items(got, refs, wl, what):
    G = wl.group_size
    rows_got, rows_ref = [], []
    for j, ref in sorted(refs.items()):
        b, g = divmod(j, wl.num_kv_heads)
        rows_got.append(got[b, g * G:(g + 1) * G])
        rows_ref.append(ref)
    if rows_got:
        assert_outputs(np.concatenate(rows_got), np.concatenate(rows_ref),
                       f"{what}: {len(refs)} groups")


def full_size_check(layer, q, k, v, lau, tau, check_dense=True):
    """Two calls and the one-call form on a full-size layer: routing bit-exact
    against the oracle, the two forms bitwise equal, sink rows exactly v0,
    every active group (and, with check_dense, every group of the dense
    path) against the oracle."""
    wl = layer.wl
    G = wl.group_size
    k0, v0, r, out = run_routed(q, k, v, tau, lau)
    out1, rf = sr.route_decode(q, k, v, k0, v0, tau, launch=lau)
    torch.cuda.synchronize()
    k0_ref = as_numpy(layer.k[:, :, 0]).astype(np.float64)
    v0_ref = as_numpy(layer.v[:, :, 0]).astype(np.float64)
    assert np.array_equal(k0.cpu().numpy(), k0_ref) and np.array_equal(v0.cpu().numpy(), v0_ref)
    mask, n_active = assert_route(r, as_numpy(layer.q), k0_ref, tau)
    for name in ("scores", "mask", "work_list", "n_active"):
        assert torch.equal(getattr(rf, name), getattr(r, name)), name
    assert torch.equal(out1, out), "one-call form differs from two calls"
    got = out.cpu().numpy()
    n_sink = sink_rows_exact(got, v0_ref, mask, G)
    active = [int(j) for j in r.work_list.cpu().numpy()[:n_active]]
    log(f"{wl.name} tau={tau}: n_active={n_active} sink_rows={n_sink}")
    refs = _item_refs(layer, active)
    _check_items(got, refs, wl, f"{wl.name} routed")
    if check_dense:
        dense = sr.dense_decode(q, k, v, launch=lau).cpu().numpy()
        rest = [j for j in range(wl.batch * wl.num_kv_heads) if j not in refs]
        refs.update(_item_refs(layer, rest))
        _check_items(dense, refs, wl, f"{wl.name} dense")
    return r


@pytest.mark.parametrize("wl", [L8B_128K, L8B_512K, L70B_128K_B8], ids=lambda w: w.name)
def test_full_size_layers_every_item(wl):
    log(f"full-size {wl.name}")
    layer = make_layer(wl)
    q, k, v = upload(layer)
    full_size_check(layer, q, k, v, launch("auto"), wl.tau)


# The paper's operating threshold (pith.science, Figure 10 caption: tau =
# 0.55) on the full 128K layer, both decode kernels, both call forms.
@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_full_size_128k_at_tau_055(kernel):
    layer = make_layer(L8B_128K)
    q, k, v = upload(layer)
    r = full_size_check(layer, q, k, v, launch(kernel), 0.55, check_dense=False)
    assert int(r.n_active.cpu()[0]) == 4


def test_full_size_256k_b4_sink_fraction_sweep():
    base = L8B_256K_B4
    log(f"full-size {base.name} sweep")
    k_cpu, v_cpu = make_caches(base)
    k, v = k_cpu.cuda(), v_cpu.cuda()
    from workloads import Layer
    for i, f in enumerate(SINK_FRACTIONS):
        wl = sweep(base, f)
        q_cpu, planted = make_queries(wl)
        layer = Layer(wl, q_cpu, k_cpu, v_cpu, planted)
        r = full_size_check(layer, q_cpu.cuda(), k, v, launch("auto"), wl.tau,
                            check_dense=i == 0)
        assert int(r.n_active.cpu()[0]) == round((1 - f) * 8) * 4


# --- fused route + decode (one launch) ------------------------------------------
FUSED_CASES = [
    Workload("f-8b-ragged", 1, 32, 8, 128, 12345, "bf16", seed=61, sink_plan=("count", 4)),
    Workload("f-70b", 2, 64, 8, 128, 6000, "bf16", seed=62, sink_plan=("bernoulli", 0.5)),
    Workload("f-g3", 3, 12, 4, 64, 2100, "bf16", seed=63, sink_plan=("bernoulli", 0.5)),
    Workload("f-f32", 1, 16, 4, 128, 3333, "f32", seed=64, sink_plan=("count", 2)),
    # the fused decisions are one 64-bit ballot: every bit, one short of it, G = 16
    Workload("f-64-items-g1", 8, 8, 8, 64, 3000, "bf16", seed=65, sink_plan=("bernoulli", 0.5)),
    Workload("f-63-items-g1", 9, 7, 7, 64, 2000, "bf16", seed=66, sink_plan=("bernoulli", 0.5)),
    Workload("f-g16", 4, 16, 1, 128, 2500, "bf16", seed=67, sink_plan=("bernoulli", 0.5)),
]


@pytest.mark.parametrize("wl", FUSED_CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("kernel", ["auto", "valu", "mfma"])
def test_fused_route_decode_matches_two_calls_bitwise(wl, kernel):
    layer = make_layer(wl)
    q, k, v = upload(layer)
    lau = launch(kernel)
    k0, v0, r, out2 = run_routed(q, k, v, wl.tau, lau)
    out1, rf = sr.route_decode(q, k, v, k0, v0, wl.tau, launch=lau)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    assert torch.equal(rf.scores, r.scores)
    assert torch.equal(rf.mask, r.mask)
    assert torch.equal(rf.work_list, r.work_list)
    assert torch.equal(rf.n_active, r.n_active)
    q_np, k_np, v_np = oracle_inputs(layer)
    mask = assert_route(rf, q_np, as_numpy(layer.k[:, :, 0]), wl.tau)[0]
    ref = oracle.routed_decode(q_np, k_np, v_np, as_numpy(layer.v[:, :, 0]), mask)
    assert_outputs(out1.cpu().numpy(), ref, f"fused {wl.name}")


def test_one_workspace_serves_calls_of_other_shapes():
    # The tickets sit at fixed offsets, so partials that a call of one shape
    # left in a workspace never land where a call of another shape keeps its
    # tickets: each call through one shared workspace is bitwise the call
    # through a fresh one, and the ticket region is zero after each.
    cases = [
        (Workload("ws-big", 2, 64, 8, 128, 40000, "bf16", seed=75, sink_plan=("count", 3)),
         launch(splits=300)),
        (Workload("ws-72-items", 9, 8, 8, 128, 3000, "bf16", seed=76,
                  sink_plan=("bernoulli", 0.5)), launch()),
        (Workload("ws-small", 1, 16, 4, 128, 3000, "bf16", seed=77, sink_plan=("count", 2)),
         launch()),
    ]
    runs = []
    for wl, lau in cases:
        q, k, v = upload(make_layer(wl))
        k0, v0 = sr.record_sink(k, v)
        fresh = sr.Workspace(sr.make_shape(q, k, v), lau, q.device)
        ref, _ = sr.route_decode(q, k, v, k0, v0, wl.tau, launch=lau, ws=fresh)
        runs.append((wl, lau, (q, k, v, k0, v0), ref))
    shared = max((sr.Workspace(sr.make_shape(*t[:3]), lau, t[0].device)
                  for _, lau, t, _ in runs), key=lambda w: w.nbytes)
    for wl, lau, t, ref in runs + runs[::-1]:
        out, _ = sr.route_decode(*t, wl.tau, launch=lau, ws=shared)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), wl.name
        assert int(ticket_region(shared).abs().sum()) == 0, wl.name


def test_default_workspace_is_reused_per_stream():
    # calls without a workspace reuse one per (device, stream): bitwise the
    # explicit-workspace result, no new workspace on a repeat, a larger one
    # for a longer layer, and a separate one on a side stream
    wl = Workload("ws-default", 1, 16, 4, 128, 3000, "bf16", seed=71, sink_plan=("count", 2))
    layer = make_layer(wl)
    q, k, v = upload(layer)
    k0, v0 = sr.record_sink(k, v)
    ws = sr.Workspace(sr.make_shape(q, k, v), None, q.device)
    ref, _ = sr.route_decode(q, k, v, k0, v0, wl.tau, ws=ws)
    a, _ = sr.route_decode(q, k, v, k0, v0, wl.tau)
    key = (q.device.index, sr._stream())
    first = sr._default_ws[key]
    b, _ = sr.route_decode(q, k, v, k0, v0, wl.tau)
    torch.cuda.synchronize()
    assert sr._default_ws[key] is first
    assert torch.equal(a, ref) and torch.equal(b, ref)
    big_wl = wl.with_(batch=2, num_q_heads=64, num_kv_heads=8, seq_len=40000, name="ws-default-big")
    big = upload(make_layer(big_wl))
    big_launch = launch(splits=300)
    assert not first.fits(sr.make_shape(*big), big_launch)
    bk0, bv0 = sr.record_sink(big[1], big[2])
    sr.route_decode(*big, bk0, bv0, wl.tau, launch=big_launch)
    assert sr._default_ws[key].fits(sr.make_shape(*big), big_launch)
    assert sr._default_ws[key].nbytes > first.nbytes
    assert any(w is first for w in sr._replaced_ws)  # kept for graphs that captured it
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        c, _ = sr.route_decode(q, k, v, k0, v0, wl.tau)
    torch.cuda.synchronize()
    assert torch.equal(c, ref)
    assert sr._default_ws[(q.device.index, side.cuda_stream)] is not sr._default_ws[key]


def test_fused_edges_all_sinks_no_sinks_and_repeats():
    wl = Workload("f-edges", 2, 16, 4, 128, 4000, "bf16", seed=65, sink_plan=("count", 2))
    layer = make_layer(wl)
    q, k, v = upload(layer)
    k0, v0 = sr.record_sink(k, v)
    out, r = sr.route_decode(q, k, v, k0, v0, -2.0)
    assert int(r.n_active.cpu()[0]) == 0
    assert torch.equal(out, v0.repeat_interleave(4, dim=1))
    out, r = sr.route_decode(q, k, v, k0, v0, 1.5)
    assert int(r.n_active.cpu()[0]) == 8
    assert torch.equal(out, sr.dense_decode(q, k, v))
    lau = launch("auto")
    ws = sr.Workspace(sr.make_shape(q, k, v), lau, q.device)
    first, _ = sr.route_decode(q, k, v, k0, v0, wl.tau, launch=lau, ws=ws)
    first = first.clone()
    for _ in range(100):
        again, _ = sr.route_decode(q, k, v, k0, v0, wl.tau, launch=lau, ws=ws)
        assert torch.equal(again, first)
    torch.cuda.synchronize()
    assert int(ticket_region(ws, 8).abs().sum()) == 0


# --- sr_route_decode picks one launch (<= 64 query heads) or two ----------------
@pytest.mark.parametrize("wl", [
    Workload("rd-64-heads", 2, 32, 8, 128, 9000, "bf16", seed=171, sink_plan=("count", 4)),
    Workload("rd-72-heads", 9, 8, 8, 128, 3000, "bf16", seed=172, sink_plan=("bernoulli", 0.5)),
], ids=lambda w: w.name)
def test_route_decode_forms_match_two_calls(wl):
    layer = make_layer(wl)
    q, k, v = upload(layer)
    k0, v0, r, out2 = run_routed(q, k, v, wl.tau, launch("auto"))
    out1, rf = sr.route_decode(q, k, v, k0, v0, wl.tau)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    for name in ("scores", "mask", "work_list", "n_active"):
        assert torch.equal(getattr(rf, name), getattr(r, name)), name


@pytest.mark.parametrize("wl", [
    Workload("rd-null-128-heads", 4, 32, 8, 128, 5000, "bf16", seed=173, sink_plan=("count", 4)),
    Workload("rd-null-512-heads", 16, 32, 8, 128, 3000, "bf16", seed=174,
             sink_plan=("bernoulli", 0.5)),
], ids=lambda w: w.name)
def test_route_decode_two_launch_form_without_routing_outputs(wl):
    """Large layer, every routing output NULL: the list, the count and the
    flags live in the workspace; the output equals the two calls'."""
    import ctypes
    from kv_cache_routing_amd import _native as N
    layer = make_layer(wl)
    q, k, v = upload(layer)
    k0, v0, _, ref = run_routed(q, k, v, wl.tau, launch("auto"))
    shape = sr.make_shape(q, k, v)
    ws = sr.Workspace(shape, None, q.device)
    out = torch.empty_like(q)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = N.lib.sr_route_decode(ctypes.byref(shape), None, P(q), P(k), P(v), P(k0), P(v0),
                               ctypes.c_float(wl.tau), 0.0, None, None, None, None, P(ws.buf),
                               ws.nbytes, P(out),
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    N.check(st, "sr_route_decode")
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


# --- many items: every branch of the routing partition ----------------------------
# Layers of many items through both calls and sr_route_decode (whose large
# layers take the routing kernel's ticketed form), on both sides of the
# routing kernel's partition tiles and at the envelope maximum (32768 items,
# two calls).
MANY_ITEMS = [
    Workload("items-256", 32, 8, 8, 128, 24, "bf16", seed=141, sink_plan=("bernoulli", 0.5)),
    Workload("items-264-g2", 33, 16, 8, 128, 40, "bf16", seed=142, sink_plan=("bernoulli", 0.5)),
    Workload("items-1024", 128, 8, 8, 64, 16, "bf16", seed=143, sink_plan=("bernoulli", 0.5)),
    Workload("items-1032", 129, 8, 8, 64, 16, "bf16", seed=144, sink_plan=("bernoulli", 0.5)),
    Workload("items-4096", 512, 8, 8, 64, 8, "bf16", seed=145, sink_plan=("bernoulli", 0.5)),
]


def _many_items_check(wl, got, r):
    layer_np = _many_items_check.cache[wl.name]
    q_np, k_np, v_np = layer_np
    mask = assert_route(r, q_np, k_np[:, :, 0], wl.tau)[0]
    ref = oracle.routed_decode(q_np, k_np, v_np, v_np[:, :, 0], mask)
    sink_rows_exact(got, v_np[:, :, 0].astype(np.float32), mask, wl.group_size)
    assert_outputs(got, ref, wl.name)


_many_items_check.cache = {}


@pytest.mark.parametrize("wl", MANY_ITEMS, ids=lambda w: w.name)
def test_many_items_two_call_and_fused(wl):
    layer = make_layer(wl)
    _many_items_check.cache[wl.name] = oracle_inputs(layer)
    q, k, v = upload(layer)
    log(f"{wl.name}: {wl.batch * wl.num_kv_heads} items")
    k0, v0, r, out2 = run_routed(q, k, v, wl.tau, launch("auto"))
    _many_items_check(wl, out2.cpu().numpy(), r)
    out1, rf = sr.route_decode(q, k, v, k0, v0, wl.tau, launch=launch("auto"))
    torch.cuda.synchronize()
    assert torch.equal(rf.mask, r.mask) and torch.equal(rf.work_list, r.work_list)
    assert torch.equal(rf.n_active, r.n_active) and torch.equal(rf.scores, r.scores)
    assert torch.equal(out1, out2)
    _many_items_check.cache.pop(wl.name)


def test_route_at_item_envelope_maximum():
    wl = Workload("items-32768", 4096, 8, 8, 128, 2, "bf16", seed=146,
                  sink_plan=("bernoulli", 0.5))
    layer = make_layer_bulk(wl)
    _many_items_check.cache[wl.name] = oracle_inputs(layer)
    q, k, v = upload(layer)
    log(f"{wl.name}: {wl.batch * wl.num_kv_heads} items")
    _, _, r, out = run_routed(q, k, v, wl.tau, launch("auto"))
    _many_items_check(wl, out.cpu().numpy(), r)
    _many_items_check.cache.pop(wl.name)


# --- routing kernel forms --------------------------------------------------------
# The routing kernel spreads its scoring over one 256-thread workgroup per 16
# items (at most 1024 workgroups, which then stride).  One workgroup also
# partitions; with more, the partition runs in a second launch (sr_route: 256
# threads up to 1024 items, 1024 above) or in the workgroup that draws the
# last ticket (sr_route_decode's two-launch form).  The partition places 4
# items per thread in tiles of 4 x its threads (1024 items for 256 threads,
# 4096 for 1024).  These layers sit on both sides of each boundary; seq_len
# is tiny since only the routing is under test.
ROUTE_FORMS = [
    Workload("rt-16-items-1wg", 2, 128, 8, 64, 2, "bf16", seed=181, sink_plan=("bernoulli", 0.5)),
    Workload("rt-17-items-2wg", 17, 16, 1, 64, 2, "bf16", seed=182, sink_plan=("bernoulli", 0.5)),
    Workload("rt-1024-items", 128, 16, 8, 128, 2, "bf16", seed=183, sink_plan=("bernoulli", 0.5)),
    Workload("rt-1025-items", 205, 5, 5, 64, 2, "bf16", seed=184, sink_plan=("bernoulli", 0.5)),
    Workload("rt-4096-items", 512, 8, 8, 64, 2, "bf16", seed=185, sink_plan=("bernoulli", 0.5)),
    Workload("rt-4097-items", 241, 17, 17, 128, 2, "bf16", seed=186, sink_plan=("bernoulli", 0.5)),
    Workload("rt-16400-items-strided", 2050, 8, 8, 64, 2, "bf16", seed=187,
             sink_plan=("bernoulli", 0.5)),
]


@pytest.mark.parametrize("wl", ROUTE_FORMS, ids=lambda w: w.name)
def test_routing_kernel_forms(wl):
    """sr_route against the oracle; sr_route_decode's routing outputs equal
    sr_route's bit for bit, on two different layers in a row through one
    workspace, and the routing ticket is back at zero after each."""
    n_items = wl.batch * wl.num_kv_heads
    log(f"{wl.name}: {n_items} items, {n_items * wl.group_size} heads")
    ws = None
    for rep in range(2):
        layer = make_layer_bulk(wl.with_(seed=wl.seed + 1000 * rep))
        q_np, k_np, _ = oracle_inputs(layer)
        q, k, v = upload(layer)
        k0, v0 = sr.record_sink(k, v)
        r = sr.route(q, k0, wl.tau)
        assert_route(r, q_np, k_np[:, :, 0], wl.tau)
        if ws is None:
            ws = sr.Workspace(sr.make_shape(q, k, v), None, q.device)
        out, rf = sr.route_decode(q, k, v, k0, v0, wl.tau, ws=ws)
        torch.cuda.synchronize()
        for name in ("scores", "mask", "work_list", "n_active"):
            assert torch.equal(getattr(rf, name), getattr(r, name)), (rep, name)
        assert torch.equal(out, sr.decode_attn(q, k, v, v0, r.work_list, r.n_active))
        assert route_ticket(ws) == 0


# --- balanced work division ------------------------------------------------------
# When the active count does not divide the grid, each workgroup takes an
# equal share of all active items' chunks (a share may span two lanes or two
# items); these layers are long enough (T / 512 above grid / n_active) for
# that mode and small enough for the oracle in full.
BALANCED = [
    Workload("bal-3of4-g4", 1, 16, 4, 128, 65536, "bf16", seed=151, sink_plan=("count", 1)),
    Workload("bal-10of16-g2", 2, 16, 8, 128, 32768, "bf16", seed=152, sink_plan=("count", 3)),
    Workload("bal-7of8-g1-d64", 1, 8, 8, 64, 40000, "bf16", seed=153, sink_plan=("count", 1)),
]


@pytest.mark.parametrize("wl", BALANCED, ids=lambda w: w.name)
@pytest.mark.parametrize("kernel", ["valu", "mfma"])
def test_balanced_division_full_parity(wl, kernel):
    layer = make_layer(wl)
    lau = launch(kernel)
    q, k, v = upload(layer)
    grid = sr.grid_size(sr.make_shape(q, k, v), lau)
    n_act = wl.batch * (wl.num_kv_heads - wl.sink_plan[1])
    S = sr.splits_for(sr.make_shape(q, k, v), lau, n_act)
    cap = sr.split_cap(sr.make_shape(q, k, v), lau)
    assert n_act * S < grid and S < cap, "layer must divide in balanced mode"
    got = full_check(layer, lau, check_dense=False)
    k0, v0 = sr.record_sink(k, v)
    fused, _ = sr.route_decode(q, k, v, k0, v0, wl.tau, launch=lau)
    assert torch.equal(fused.cpu(), torch.from_numpy(got))
    routed_all = sr.decode_attn(q, k, v, v0, *_route_all_active(q, k0), launch=lau)
    assert torch.equal(routed_all, sr.dense_decode(q, k, v, launch=lau))


def _route_all_active(q, k0):
    r = sr.route(q, k0, 2.0)  # tau > 1: every item active, the identity list
    return r.work_list, r.n_active


def test_balanced_dense_alpha0():
    wl = Workload("bal-dense-6", 1, 12, 6, 128, 40000, "bf16", seed=154)
    layer = make_layer(wl)
    q, k, v = upload(layer)
    out, a0 = sr.dense_decode_alpha0(q, k, v)
    q_np, k_np, v_np = oracle_inputs(layer)
    assert_outputs(out.cpu().numpy(), oracle.dense_decode(q_np, k_np, v_np), "balanced dense")
    ref = oracle.bos_mass(q_np, k_np)
    rel = np.abs(a0.cpu().numpy().astype(np.float64) - ref) / ref
    assert rel.max() <= 1e-4


# --- eight-wave workgroups -------------------------------------------------------
EIGHT_WAVES = [
    Workload("w8-8b", 1, 32, 8, 128, 12345, "bf16", seed=161, sink_plan=("count", 4)),
    Workload("w8-g16-d64", 1, 32, 2, 64, 2000, "bf16", seed=162, sink_plan=("count", 1)),
    Workload("w8-f32", 1, 16, 4, 128, 3333, "f32", seed=163, sink_plan=("count", 2)),
    Workload("w8-f32-g16", 1, 32, 2, 128, 1500, "f32", seed=165, sink_plan=("count", 1)),
    Workload("w8-bal-3of4", 1, 16, 4, 128, 65536, "bf16", seed=164, sink_plan=("count", 1)),
]


@pytest.mark.parametrize("wl", EIGHT_WAVES, ids=lambda w: w.name)
@pytest.mark.parametrize("kernel", ["valu", "mfma"])
def test_eight_wave_workgroups(wl, kernel):
    layer = make_layer(wl)
    got = full_check(layer, launch(kernel, waves=8))
    q, k, v = upload(layer)
    k0, v0 = sr.record_sink(k, v)
    fused, _ = sr.route_decode(q, k, v, k0, v0, wl.tau, launch=launch(kernel, waves=8))
    assert torch.equal(fused.cpu(), torch.from_numpy(got))


# --- attention weight of position 0 (alpha_0) -----------------------------------
ALPHA_CASES = [
    Workload("a-8b", 1, 32, 8, 128, 9000, "bf16", seed=81, sink_plan=("count", 4)),
    Workload("a-70b", 2, 64, 8, 128, 3000, "bf16", seed=82, sink_plan=("bernoulli", 0.5)),
    Workload("a-g3-d64", 1, 12, 4, 64, 777, "bf16", seed=83, sink_plan=("count", 1)),
    Workload("a-f32", 1, 8, 2, 128, 2048, "f32", seed=84, sink_plan=("count", 1)),
]


@pytest.mark.parametrize("wl", ALPHA_CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("splits", [0, 1, 7])
def test_dense_alpha0_matches_oracle(wl, kernel, splits):
    layer = make_layer(wl)
    q, k, v = upload(layer)
    lau = launch(kernel, splits=splits)
    out, a0 = sr.dense_decode_alpha0(q, k, v, launch=lau)
    assert torch.equal(out, sr.dense_decode(q, k, v, launch=lau))
    q_np, k_np, _ = oracle_inputs(layer)
    ref = oracle.bos_mass(q_np, k_np)
    got = a0.cpu().numpy().astype(np.float64)
    rel = np.abs(got - ref) / ref
    log(f"  alpha0 {wl.name} {kernel} S={splits}: max rel err {rel.max():.2e}, "
        f"range [{ref.min():.2e}, {ref.max():.2e}]")
    assert rel.max() <= 1e-4


def test_alpha0_fixed_point_bound_on_gpu():
    d, T = 64, 4096
    gen = torch.Generator().manual_seed(85)
    kk = torch.randn((1, 2, T, d), generator=gen)
    vv = torch.randn((1, 2, T, d), generator=gen)
    kk[0, :, 0] *= (40.0 / kk[0, :, 0].norm(dim=-1))[:, None]
    # head 0 of each group aligned with k0 (alpha_0 near 1), head 1 random
    qq = torch.randn((1, 4, d), generator=gen)
    qq[0, 0] = kk[0, 0, 0] / kk[0, 0, 0].norm() * 2.0
    qq[0, 2] = kk[0, 1, 0] / kk[0, 1, 0].norm() * 2.0
    out, a0 = sr.dense_decode_alpha0(qq.cuda(), kk.cuda(), vv.cuda())
    out, a0 = out.cpu().double(), a0.cpu().double()
    for h in range(4):
        g = h // 2
        spread = (vv[0, g, 1:] - vv[0, g, 0]).norm(dim=-1).max().double()
        lhs = (out[0, h] - vv[0, g, 0].double()).norm()
        assert lhs <= (1 - a0[0, h]) * spread * (1 + 1e-4) + 1e-6, (h, lhs, a0[0, h])
    assert a0[0, 0] > 0.5 and a0[0, 2] > 0.5


@pytest.mark.parametrize("kernel", BF16_KERNELS)
@pytest.mark.parametrize("splits", [0, 13])
def test_alternating_layers_on_one_workspace(kernel, splits):
    # Two different layers through the same workspace, interleaved: a split
    # partial that is not yet visible to the merging workgroup would be read
    # from the other layer's previous call and change the result.
    wls = [Workload(f"alt{i}", 1, 32, 8, 128, 20000 + 37 * i, "bf16", seed=91 + i,
                    sink_plan=("count", 3)) for i in range(2)]
    layers = [make_layer(w) for w in wls]
    dev = [upload(L) for L in layers]
    lau = launch(kernel, splits=splits)
    T = max(w.seq_len for w in wls)
    shape = sr.make_shape(dev[0][0], dev[0][1], dev[0][2])
    ws = sr.Workspace(shape, lau, dev[0][0].device)
    k0v0 = [sr.record_sink(k, v) for _, k, v in dev]
    refs = [sr.route_decode(q, k, v, k0, v0, 0.5, launch=lau, ws=ws)[0].clone()
            for (q, k, v), (k0, v0) in zip(dev, k0v0)]
    dense_refs = [sr.dense_decode(q, k, v, launch=lau, ws=ws).clone() for q, k, v in dev]
    for it in range(150):
        i = it % 2
        q, k, v = dev[i]
        k0, v0 = k0v0[i]
        out, _ = sr.route_decode(q, k, v, k0, v0, 0.5, launch=lau, ws=ws)
        assert torch.equal(out, refs[i]), it
        assert torch.equal(sr.dense_decode(q, k, v, launch=lau, ws=ws), dense_refs[i]), it
    for (q, k, v), L, r in zip(dev, layers, refs):
        q_np, k_np, v_np = oracle_inputs(L)
        ref = oracle.dense_decode(q_np, k_np, v_np)
        assert_outputs(sr.dense_decode(q, k, v, launch=lau, ws=ws).cpu().numpy(), ref, "alt dense")


# --- decode-step neighbours: rotary embedding and cache append -------------------
from workloads import rope_inv_freq  # noqa: E402


def _bf16_ulp(x):
    return np.ldexp(1.0, np.frexp(np.abs(x))[1] - 8)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128)])
@pytest.mark.parametrize("pos", [0, 1, 777, 131071])
def test_rope_append_matches_oracle(dtype, d, pos):
    B, Hq, Hkv, T = 2, 16, 4, 131072 if pos == 131071 else 1024
    gen = torch.Generator().manual_seed(111 + pos)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = torch.randn((B, Hkv, T, d), generator=gen).to(tdt)
    vc = torch.randn((B, Hkv, T, d), generator=gen).to(tdt)
    qn, kn, vn = (torch.randn((B, H, d), generator=gen) for H in (Hq, Hkv, Hkv))
    f = rope_inv_freq(d)
    kd, vd = kc.cuda(), vc.cuda()
    q_rot = sr.rope_append(qn.cuda(), kn.cuda(), vn.cuda(), kd, vd, pos, f.cuda()).cpu()
    ref_q = oracle.rope(qn.numpy(), pos, f.numpy())
    err = np.abs(q_rot.numpy().astype(np.float64) - ref_q)
    assert (err <= np.abs(ref_q) * 2 ** -23 + 1e-30).all(), err.max()
    if pos == 0:
        assert torch.equal(q_rot, qn)
    kd_np, vd_np = as_numpy(kd.cpu()).astype(np.float64), as_numpy(vd.cpu()).astype(np.float64)
    ref_k = oracle.rope(kn.numpy(), pos, f.numpy())
    if dtype == "bf16":
        assert (np.abs(kd_np[:, :, pos] - ref_k) <= _bf16_ulp(ref_k)).all()
        assert np.array_equal(vd_np[:, :, pos], oracle.round_bf16(vn.numpy().astype(np.float64)))
    else:
        assert (np.abs(kd_np[:, :, pos] - ref_k) <= np.abs(ref_k) * 2 ** -23 + 1e-30).all()
        assert np.array_equal(vd_np[:, :, pos], vn.numpy().astype(np.float64))
    keep = torch.ones(T, dtype=torch.bool)
    keep[pos] = False
    assert torch.equal(kd.cpu()[:, :, keep], kc[:, :, keep])
    assert torch.equal(vd.cpu()[:, :, keep], vc[:, :, keep])


def test_decode_steps_with_append_match_oracle():
    # three decode steps: rotate + append the new token, then routed decode
    # over the grown cache; compare with the oracle stepping the same way
    wl = Workload("steps", 1, 32, 8, 128, 3000, "bf16", seed=121, sink_plan=("count", 4))
    layer = make_layer(wl)
    cap = wl.seq_len + 8
    kc = torch.zeros((1, 8, cap, 128), dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    kc[:, :, :wl.seq_len] = layer.k
    vc[:, :, :wl.seq_len] = layer.v
    kd, vd = kc.cuda(), vc.cuda()
    f = rope_inv_freq(128)
    k_np, v_np = as_numpy(kc).astype(np.float64), as_numpy(vc).astype(np.float64)
    gen = torch.Generator().manual_seed(122)
    k0, v0 = sr.record_sink(kd[:, :, :wl.seq_len], vd[:, :, :wl.seq_len])
    for step in range(3):
        pos = wl.seq_len + step
        qn, kn, vn = (torch.randn((1, H, 128), generator=gen) for H in (32, 8, 8))
        q_rot = sr.rope_append(qn.cuda(), kn.cuda(), vn.cuda(), kd, vd, pos, f.cuda())
        T = pos + 1
        out, r = sr.route_decode(q_rot, kd[:, :, :T], vd[:, :, :T], k0, v0, 0.5)
        q_ref, k_np, v_np = oracle.rope_append(qn.numpy(), kn.numpy(), vn.numpy(), k_np, v_np,
                                               pos, f.numpy(), bf16=True)
        # the device's rotation and append within their bounds (its appended
        # key may differ from the oracle's by one bf16 ulp) ...
        k_dev = as_numpy(kd.cpu()).astype(np.float64)
        assert (np.abs(k_dev[:, :, pos] - k_np[:, :, pos]) <= _bf16_ulp(k_np[:, :, pos])).all()
        assert np.array_equal(as_numpy(vd.cpu()).astype(np.float64)[:, :, pos], v_np[:, :, pos])
        q_dev = q_rot.cpu().numpy().astype(np.float64)
        assert (np.abs(q_dev - q_ref) <= np.abs(q_ref) * 2 ** -23 + 1e-30).all()
        # ... and the routing and output against the oracle stepping its own
        # caches, with its own rotated query
        mask = assert_route(r, q_ref, k_np[:, :, 0], 0.5)[0]
        ref = oracle.routed_decode(q_ref, k_np[:, :, :T], v_np[:, :, :T], v_np[:, :, 0], mask)
        assert_outputs(out.cpu().numpy(), ref, f"step {step} T={T}")


# (name, B, Hq, Hkv, d, dtype, T, sink groups per sequence, tau, kernel, waves, splits)
ROPE_FUSED = [
    ("8b-lanes", 1, 32, 8, 128, "bf16", 4097, 4, 0.5, "auto", 0, 0),
    ("8b-balanced", 1, 32, 8, 128, "bf16", 100000, 5, 0.5, "auto", 0, 0),
    ("8b-last-row-valu", 1, 32, 8, 128, "bf16", 4096, 4, 0.5, "valu", 0, 0),
    ("d64-b2", 2, 8, 4, 64, "bf16", 3001, 1, 0.5, "auto", 0, 0),
    ("f32-g8", 1, 16, 2, 128, "f32", 5000, 1, 0.5, "auto", 0, 0),
    ("g16-64-heads", 1, 64, 4, 128, "bf16", 2049, 2, 0.5, "auto", 0, 0),
    ("mha", 1, 8, 8, 128, "bf16", 1500, 3, 0.5, "auto", 0, 0),
    ("dense-tau-above-one", 1, 32, 8, 128, "bf16", 4097, 0, 2.0, "auto", 0, 0),
    ("all-sinks", 1, 32, 8, 128, "bf16", 4097, 8, -2.0, "auto", 0, 0),
    ("fixed-splits", 1, 32, 8, 128, "bf16", 20000, 4, 0.5, "mfma", 0, 7),
    ("waves8-f32-d64", 1, 32, 8, 64, "f32", 3000, 2, 0.5, "auto", 8, 0),
    ("valu-f32-g16", 1, 32, 2, 64, "f32", 2500, 1, 0.5, "valu", 0, 0),
    ("two-positions", 1, 32, 8, 128, "bf16", 2, 4, 0.5, "auto", 0, 0),
    ("g3-ragged", 1, 24, 8, 128, "bf16", 7777, 3, 0.5, "auto", 0, 0),
    ("g6-b2-d64", 2, 24, 4, 64, "bf16", 5001, 1, 0.5, "auto", 0, 0),
    ("g12-f32-valu", 1, 48, 4, 128, "f32", 3333, 2, 0.5, "valu", 0, 0),
    ("g5-waves8", 1, 40, 8, 128, "bf16", 6000, 5, 0.5, "mfma", 8, 0),
    # above 64 query heads: the routing kernel rotates and appends, then the decode
    ("128-heads", 2, 64, 8, 128, "bf16", 9000, 4, 0.5, "auto", 0, 0),
    ("70b-shape-512-heads", 8, 64, 8, 128, "bf16", 3000, 4, 0.5, "auto", 0, 0),
    ("g16-f32-256-heads", 4, 64, 4, 64, "f32", 2000, 2, 0.5, "valu", 0, 0),
    ("1024-items", 128, 8, 8, 64, "bf16", 700, 3, 0.5, "mfma", 0, 0),
    ("large-dense", 4, 32, 8, 128, "bf16", 4097, 0, 2.0, "auto", 0, 0),
    # 4800 groups: more than 1024 routing workgroups of 4, so a workgroup rotates
    # and scores several rounds
    ("multi-round-4800-groups", 600, 8, 8, 128, "bf16", 40, 3, 0.5, "auto", 0, 0),
]


@pytest.mark.parametrize("case", ROPE_FUSED, ids=[c[0] for c in ROPE_FUSED])
def test_rope_route_decode_matches_append_then_route_decode(case):
    # One launch (rotate + append + route + decode) against sr_rope_append
    # followed by sr_route_decode on a copy of the caches: every output, the
    # rotated query and the whole cache storage bitwise equal; the output
    # also against the oracle on the appended cache.
    _rope_step_check(case, planted=True)


def _rope_step_check(case, planted):
    # planted: the case's routing must come out as planted (n_sink sinks per
    # sequence); random cases skip that check (a random target can clear tau).
    name, B, Hq, Hkv, d, dtype, T, n_sink, tau, kernel, waves, splits = case
    G = Hq // Hkv
    pos, cap = T - 1, T + 5
    gen = torch.Generator().manual_seed(170 + T + Hq)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = torch.randn((B, Hkv, cap, d), generator=gen).to(tdt)
    vc = torch.randn((B, Hkv, cap, d), generator=gen).to(tdt)
    kc[:, :, pos:] = 7.0  # rows from T - 1 on: only the append may change them
    vc[:, :, pos:] = 7.0
    k0 = kc[:, :, 0].float()
    f = rope_inv_freq(d)
    kn, vn = (torch.randn((B, Hkv, d), generator=gen) for _ in range(2))
    # sinks: the rotated query of every head in the first n_sink groups lies
    # near k0 (planted by turning the target back by the new position)
    target = torch.randn((B, Hq, d), generator=gen, dtype=torch.float64)
    for b in range(B):
        for g in range(n_sink):
            u = k0[b, g].double() / k0[b, g].double().norm()
            for h in range(g * G, (g + 1) * G):
                target[b, h] = 0.9 * u * target[b, h].norm() + 0.05 * target[b, h]
    qn = torch.from_numpy(oracle.rope(target.numpy(), -pos, f.numpy())).float()
    lau = launch(kernel, splits=splits, waves=waves)
    kA, vA = kc.cuda(), vc.cuda()
    kB, vB = kc.cuda(), vc.cuda()
    k0d, v0d = sr.record_sink(kA[:, :, :T], vA[:, :, :T])
    qn_d, kn_d, vn_d, f_d = qn.cuda(), kn.cuda(), vn.cuda(), f.cuda()

    q_rot = sr.rope_append(qn_d, kn_d, vn_d, kA, vA, pos, f_d)
    out_a, r_a = sr.route_decode(q_rot, kA[:, :, :T], vA[:, :, :T], k0d, v0d, tau, launch=lau)
    ws = sr.Workspace(sr.make_shape(qn_d, kB[:, :, :T], vB[:, :, :T]), lau, qn_d.device)
    for rep in range(2):  # the second call reuses the workspace and rewrites the same row
        out_b, r_b, q_b = sr.rope_route_decode(qn_d, kn_d, vn_d, kB[:, :, :T], vB[:, :, :T],
                                               k0d, v0d, f_d, tau, launch=lau, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(q_b, q_rot), f"{name}: rotated query"
        assert torch.equal(out_b, out_a), f"{name}: output (call {rep})"
        for fld in ("scores", "mask", "work_list", "n_active"):
            assert torch.equal(getattr(r_b, fld), getattr(r_a, fld)), f"{name}: {fld}"
        assert torch.equal(kB, kA) and torch.equal(vB, vA), f"{name}: caches"
    n_active = int(r_b.n_active.item())
    expect = B * Hkv if tau > 1 else (0 if tau < -1 else B * (Hkv - n_sink))
    assert n_active == expect or not planted, f"{name}: planted routing gave {n_active} active"
    shape = sr.make_shape(qn_d, kB[:, :, :T], vB[:, :, :T])
    grid, lanes = sr.grid_size(shape, lau), sr.splits_for(shape, lau, n_active)
    balanced = splits == 0 and n_active * lanes < grid and lanes < sr.split_cap(shape, lau)
    log(f"{name}: n_active={n_active} grid={grid} lanes={lanes} balanced={balanced}")
    if name == "8b-balanced":
        assert balanced  # the appended row's owner found from the workgroup's range
    if name == "8b-lanes":
        assert not balanced and n_active > 0  # found from the workgroup's lane

    # The reference comes from the oracle alone: its own rotation of the new
    # query and key and its own append (rounded to the cache dtype), then
    # routing and attention over positions 0 .. T - 1.  The device's rotated
    # query and appended row are held to their own bounds first.
    q_ref, k_ref, v_ref = oracle.rope_append(qn.numpy(), kn.numpy(), vn.numpy(), as_numpy(kc),
                                             as_numpy(vc), pos, f.numpy(), bf16=dtype == "bf16")
    k_ref, v_ref = k_ref[:, :, :T], v_ref[:, :, :T]
    q_dev = q_b.cpu().numpy().astype(np.float64)
    assert (np.abs(q_dev - q_ref) <= np.abs(q_ref) * 2 ** -23 + 1e-30).all(), f"{name}: q_out"
    k_dev = as_numpy(kB[:, :, :T].cpu()).astype(np.float64)
    v_dev = as_numpy(vB[:, :, :T].cpu()).astype(np.float64)
    ulp = _bf16_ulp(k_ref[:, :, pos]) if dtype == "bf16" else np.abs(k_ref[:, :, pos]) * 2 ** -23
    assert (np.abs(k_dev[:, :, pos] - k_ref[:, :, pos]) <= ulp + 1e-30).all(), f"{name}: key row"
    assert np.array_equal(v_dev[:, :, pos], v_ref[:, :, pos]), f"{name}: value row"
    assert np.array_equal(k_dev[:, :, :pos], k_ref[:, :, :pos]), f"{name}: other key rows"
    scores, mask, wl_ref, n_ref = oracle.route(q_ref, k_ref[:, :, 0], tau)
    assert np.abs(scores - tau).min() >= 1e-4, f"{name}: a score within 1e-4 of tau"
    assert np.array_equal(r_b.mask.cpu().numpy(), mask), f"{name}: mask"
    assert np.array_equal(r_b.work_list.cpu().numpy(), wl_ref) and n_active == n_ref
    assert np.abs(r_b.scores.cpu().numpy() - scores).max() <= 2e-5
    ref = oracle.routed_decode(q_ref, k_ref, v_ref, v_ref[:, :, 0], mask)
    sink_rows_exact(out_b.cpu().numpy(), v_ref[:, :, 0].astype(np.float32), mask, G)
    assert_outputs(out_b.cpu().numpy(), ref, f"{name} T={T}")


def test_graph_replay_matches_eager():
    # The decode calls allocate nothing and never wait for the host, so they
    # can be captured; replay several times with eager work in between and
    # compare every replay with the eager result.
    wl = Workload("graph", 1, 32, 8, 128, 10000, "bf16", seed=131, sink_plan=("count", 4))
    layer = make_layer(wl)
    q, k, v = upload(layer)
    lau = launch("auto")
    ws = sr.Workspace(sr.make_shape(q, k, v), lau, q.device)
    k0, v0 = sr.record_sink(k, v)
    r = sr.route(q, k0, wl.tau)
    out_f = torch.empty_like(q)
    out_t = torch.empty_like(q)
    out_d = torch.empty_like(q)
    rf = sr.route(q, k0, wl.tau)
    eager_f = sr.route_decode(q, k, v, k0, v0, wl.tau, launch=lau, ws=ws, routing=rf)[0].clone()
    sr.route(q, k0, wl.tau, out=r)
    eager_t = sr.decode_attn(q, k, v, v0, r.work_list, r.n_active, launch=lau, ws=ws).clone()
    eager_d = sr.dense_decode(q, k, v, launch=lau, ws=ws).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sr.route_decode(q, k, v, k0, v0, wl.tau, launch=lau, ws=ws, out=out_f, routing=rf)
        sr.route(q, k0, wl.tau, out=r)
        sr.decode_attn(q, k, v, v0, r.work_list, r.n_active, launch=lau, ws=ws, out=out_t)
        sr.dense_decode(q, k, v, launch=lau, ws=ws, out=out_d)
    for it in range(5):
        out_f.zero_()
        out_t.zero_()
        out_d.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_f, eager_f), it
        assert torch.equal(out_t, eager_t), it
        assert torch.equal(out_d, eager_d), it
        sr.dense_decode(q, k, v, launch=lau, ws=ws)  # eager work between replays
        torch.cuda.synchronize()
    assert int(ticket_region(ws, 8).abs().sum()) == 0


@pytest.mark.parametrize("n_active", [3, 99, -4])
def test_foreign_work_list_stays_inside_the_buffers(n_active):
    # A work list not made by sr_route, with entries and counts out of range:
    # the kernels clamp them, so every access stays inside the buffers (the
    # output's guard region is untouched) and group 0, which appears only as
    # an active item, still gets exact attention.
    wl = Workload("foreign-list", 1, 32, 8, 128, 3000, "bf16", seed=195)
    layer = make_layer(wl)
    q, k, v = upload(layer)
    k0, v0 = sr.record_sink(k, v)
    n = q.numel()
    big = torch.full((n + 8192,), 123.0, device=q.device)
    out = big[:n].view(q.shape)
    wl_dev = torch.tensor([5, 100, -5, 1000000, 3, 3, 6, 6], dtype=torch.int32, device=q.device)
    na = torch.tensor([n_active], dtype=torch.int32, device=q.device)
    for kernel in ("mfma", "valu"):
        sr.decode_attn(q, k, v, v0, wl_dev, na, launch=launch(kernel), out=out)
        torch.cuda.synchronize()
        assert torch.all(big[n:] == 123.0), kernel
        assert torch.isfinite(out).all(), kernel
        if n_active == 3:  # group 0 comes from the clamped -5, active only
            q_np, k_np, v_np = oracle_inputs(layer)
            ref = oracle.dense_decode(q_np, k_np, v_np)
            assert_outputs(out.cpu().numpy()[:, :4], ref[:, :4], f"group 0 {kernel}")


@pytest.mark.parametrize("dtype,Hq", [("bf16", 32), ("f32", 128)])
def test_rope_step_on_padded_cache_rows(dtype, Hq):
    # Cache rows d + 8 elements apart (views of padded storage): the one-call
    # step equals the two calls bitwise and never writes the padding.
    B, Hkv, d, T = 1, 8, 128, 3001
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator().manual_seed(200 + Hq)
    store = torch.randn((B, Hkv, T + 2, d + 8), generator=gen).to(tdt)
    store[..., d:] = -3.0  # the padding
    vstore = torch.randn((B, Hkv, T + 2, d + 8), generator=gen).to(tdt)
    vstore[..., d:] = -3.0
    qn, kn, vn = (torch.randn((B, H, d), generator=gen).cuda() for H in (Hq, Hkv, Hkv))
    f = rope_inv_freq(d).cuda()
    kA, vA, kB, vB = store.cuda(), vstore.cuda(), store.cuda(), vstore.cuda()
    view = lambda t: t[:, :, :T, :d]
    assert view(kA).stride(2) == d + 8
    k0, v0 = sr.record_sink(view(kA), view(vA))
    q_rot = sr.rope_append(qn, kn, vn, kA[..., :d], vA[..., :d], T - 1, f)
    out_a, r_a = sr.route_decode(q_rot, view(kA), view(vA), k0, v0, 0.0)
    out_b, r_b, q_b = sr.rope_route_decode(qn, kn, vn, view(kB), view(vB), k0, v0, f, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(q_b, q_rot) and torch.equal(out_b, out_a)
    assert torch.equal(r_b.work_list, r_a.work_list)
    assert torch.equal(kB, kA) and torch.equal(vB, vA)  # padding included
    assert torch.all(kB[..., d:] == -3.0) and torch.all(vB[..., d:] == -3.0)


def test_rope_step_graph_replay_matches_eager():
    # A captured one-launch decode step, replayed with the new row of the
    # caches reset by eager work in between: every replay writes the row
    # again and reproduces the eager output, rotated query and caches.
    B, Hq, Hkv, d, T = 1, 32, 8, 128, 9000
    gen = torch.Generator().manual_seed(190)
    kc = torch.randn((B, Hkv, T + 3, d), generator=gen).to(torch.bfloat16)
    vc = torch.randn((B, Hkv, T + 3, d), generator=gen).to(torch.bfloat16)
    qn, kn, vn = (torch.randn((B, H, d), generator=gen).cuda() for H in (Hq, Hkv, Hkv))
    f = rope_inv_freq(d).cuda()
    lau = launch("auto")
    kA, vA, kB, vB = kc.cuda(), vc.cuda(), kc.cuda(), vc.cuda()
    k0, v0 = sr.record_sink(kA[:, :, :T], vA[:, :, :T])
    ws = sr.Workspace(sr.make_shape(qn, kA[:, :, :T], vA[:, :, :T]), lau, qn.device)
    out_e, r_e, q_e = sr.rope_route_decode(qn, kn, vn, kA[:, :, :T], vA[:, :, :T], k0, v0, f,
                                           0.0, launch=lau, ws=ws)
    out_e, q_e = out_e.clone(), q_e.clone()
    out_g, q_g = torch.empty_like(qn), torch.empty_like(qn)
    r_g = sr.Routing(torch.empty_like(r_e.scores), torch.empty_like(r_e.mask),
                     torch.empty_like(r_e.work_list), torch.empty_like(r_e.n_active))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sr.rope_route_decode(qn, kn, vn, kB[:, :, :T], vB[:, :, :T], k0, v0, f, 0.0,
                             launch=lau, ws=ws, out=out_g, routing=r_g, q_out=q_g)
    for it in range(5):
        out_g.zero_()
        q_g.zero_()
        kB[:, :, T - 1] = 7.0
        vB[:, :, T - 1] = 7.0
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e) and torch.equal(q_g, q_e), it
        assert torch.equal(r_g.work_list, r_e.work_list), it
        assert torch.equal(kB, kA) and torch.equal(vB, vA), it
        sr.dense_decode(q_e, kA[:, :, :T], vA[:, :, :T], launch=lau, ws=ws)  # eager work
        torch.cuda.synchronize()
    assert int(r_e.n_active.item()) > 0  # tau = 0: planted nothing, some groups active
    assert int(ticket_region(ws, B * Hkv).abs().sum()) == 0


# --- randomized layers --------------------------------------------------------------
@functools.lru_cache(maxsize=None)
def _random_layers(n, seed):
    """n seeded random small layers over the whole envelope (any G up to 16,
    both head sizes and dtypes, ragged lengths, 0-100 % sinks), each with a
    random kernel, wave count and split policy.  A layer whose generated
    scores fall within 0.05 of tau is redrawn, so every decision is clear."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.integers(1, 17))
        B = int(rng.integers(1, 4))
        d = int(rng.choice([64, 128]))
        T = int(rng.integers(1, 5000))
        dt = str(rng.choice(["bf16", "f32"]))
        frac = float(rng.choice([0.0, 0.3, 0.5, 1.0]))
        wl = Workload(f"rand{len(out)}", B, Hkv * G, Hkv, d, T, dt, seed=int(rng.integers(1, 1 << 30)),
                      sink_plan=("bernoulli", frac))
        kernel = str(rng.choice(["auto", "valu", "mfma"]))
        waves = int(rng.choice([4, 8]))
        splits = int(rng.choice([0, 0, int(rng.integers(1, 40))]))
        layer = make_layer(wl)
        q_np, k_np, _ = oracle_inputs(layer)
        scores = oracle.route(q_np, k_np[:, :, 0], wl.tau)[0]
        if np.abs(scores - wl.tau).min() < 0.05:
            continue
        out.append((layer, kernel, waves, splits))
    return out


# Counts of the randomized tests; larger sweeps run with, e.g.,
# SR_FUZZ_LAYERS=5000 SR_FUZZ_STEPS=2000 [SR_FUZZ_SEED=n] python -m pytest tests -m gpu -k randomized
N_RANDOM_LAYERS = int(os.environ.get("SR_FUZZ_LAYERS", "48"))
N_RANDOM_STEPS = int(os.environ.get("SR_FUZZ_STEPS", "24"))
FUZZ_SEED = int(os.environ.get("SR_FUZZ_SEED", "7001"))


@pytest.mark.parametrize("i", range(N_RANDOM_LAYERS))
def test_randomized_layers_against_oracle(i):
    layer, kernel, waves, splits = _random_layers(N_RANDOM_LAYERS, FUZZ_SEED)[i]
    wl = layer.wl
    log(f"{wl.name}: B={wl.batch} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} d={wl.head_dim} "
        f"T={wl.seq_len} {wl.kv_dtype} {wl.sink_plan} kernel={kernel} waves={waves} splits={splits}")
    lau = launch(kernel, splits=splits, waves=waves)
    got = full_check(layer, lau)
    q, k, v = upload(layer)
    k0, v0 = sr.record_sink(k, v)
    fused, _ = sr.route_decode(q, k, v, k0, v0, wl.tau, launch=lau)
    assert torch.equal(fused.cpu(), torch.from_numpy(got))


@functools.lru_cache(maxsize=None)
def _random_rope_steps(n, seed):
    """n seeded random one-call decode steps: up to 512 query heads (one launch
    up to 64, two above), any G up to 16, both head sizes and dtypes, T from 2
    to 20000, any number of
    planted sink groups, routed, dense (tau > 1) or all-sink (tau < -1), every
    kernel, wave count and split policy."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        Hkv, G, B = int(rng.choice([1, 2, 4, 8])), int(rng.integers(1, 17)), int(rng.integers(1, 9))
        if B * Hkv * G > 512:
            continue
        out.append((f"step{len(out)}", B, Hkv * G, Hkv, int(rng.choice([64, 128])),
                    str(rng.choice(["bf16", "f32"])), int(rng.integers(2, 20000)),
                    int(rng.integers(0, Hkv + 1)), float(rng.choice([0.5, 0.5, 2.0, -2.0])),
                    str(rng.choice(["auto", "valu", "mfma"])), int(rng.choice([4, 8])),
                    int(rng.choice([0, 0, int(rng.integers(1, 40))]))))
    return out


@pytest.mark.parametrize("i", range(N_RANDOM_STEPS))
def test_randomized_rope_steps(i):
    _rope_step_check(_random_rope_steps(N_RANDOM_STEPS, FUZZ_SEED + 1)[i], planted=False)


def test_host_arrays_are_refused_before_any_launch():
    # Every array a call hands over is checked to be on the device (a host
    # pointer would be read by the kernels as device memory): each refusal
    # names the array, and nothing is launched.
    wl = Workload("host-args", 1, 16, 4, 128, 600, "bf16", seed=81, sink_plan=("count", 1))
    q, k, v = upload(make_layer(wl))
    k0, v0 = sr.record_sink(k, v)
    r = sr.route(q, k0, wl.tau)
    cpu_routing = sr.Routing(r.scores.cpu(), r.mask, r.work_list, r.n_active)
    with pytest.raises(ValueError, match="k0 is a host tensor"):
        sr.route_decode(q, k, v, k0.cpu(), v0)
    with pytest.raises(ValueError, match="v0 is a host tensor"):
        sr.decode_attn(q, k, v, v0.cpu(), r.work_list, r.n_active)
    with pytest.raises(ValueError, match="n_active is a host tensor"):
        sr.decode_attn(q, k, v, v0, r.work_list, r.n_active.cpu())
    with pytest.raises(ValueError, match="out is a host tensor"):
        sr.dense_decode(q, k, v, out=torch.empty(q.shape))
    with pytest.raises(ValueError, match="scores is a host tensor"):
        sr.route(q, k0, wl.tau, out=cpu_routing)
    with pytest.raises(ValueError, match="scores is a host tensor"):
        sr.route_decode(q, k, v, k0, v0, routing=cpu_routing)
    f = rope_inv_freq(128).cuda()
    kn = torch.zeros_like(k0)
    with pytest.raises(ValueError, match="q_out is a host tensor"):
        sr.rope_route_decode(q, kn, kn, k, v, k0, v0, f, q_out=torch.empty(q.shape))
    with pytest.raises(ValueError, match="inv_freq is a host tensor"):
        sr.rope_append(q, kn, kn, k, v, 5, f.cpu())
    torch.cuda.synchronize()


@pytest.mark.parametrize("B", [2, 5], ids=["one-launch", "two-launch"])
def test_degenerate_heads_and_keys_route_as_the_oracle(B):
    # A NaN or infinite query element leaves that head's cosine undefined: the
    # score is NaN and the head dissents at every tau, so its group is active
    # even at tau = -2.  A zero position-0 key scores its group's heads 0: a
    # sink at tau <= 0 only.  Checked in sr_route and in both forms of
    # sr_route_decode (one launch up to 64 query heads, two above) against the
    # oracle: scores (NaN where the oracle's are), mask, list and count exactly;
    # sink rows exactly v0; every active row of a finite query within the
    # tolerance (attention of a non-finite query is undefined: not compared).
    wl = Workload(f"degenerate-b{B}", B, 16, 4, 128, 700, "bf16", seed=90 + B,
                  sink_plan=("count", 2))
    layer = make_layer(wl)
    G = wl.group_size
    q_np, k_np, v_np = oracle_inputs(layer)
    k0_ref, _ = oracle.record_sink(k_np, v_np)
    _, mask0, _, _ = oracle.route(q_np, k0_ref, wl.tau)
    sinks = [tuple(int(x) for x in s) for s in zip(*np.nonzero(mask0))]
    (b1, g1), (b2, g2), (b3, g3) = sinks[0], sinks[1], sinks[-1]
    q = layer.q.clone()
    k = layer.k.clone()
    q[b1, g1 * G + 1, 5] = float("nan")
    q[b2, g2 * G + 2, 9] = float("inf")
    k[b3, g3, 0, :] = 0
    q_np, k_np = as_numpy(q), as_numpy(k)
    k0_ref, v0_ref = oracle.record_sink(k_np, v_np)
    qd, kd, vd = q.cuda(), k.cuda(), layer.v.cuda()
    k0, v0 = sr.record_sink(kd, vd)
    for tau in (0.5, 0.0, -2.0):
        scores, mask, wl_ref, n_act = oracle.route(q_np, k0_ref, tau)
        assert mask[b1, g1] == 0 and mask[b2, g2] == 0
        assert mask[b3, g3] == (1 if tau <= 0 else 0)
        r = sr.route(qd, k0, tau)
        out, rf = sr.route_decode(qd, kd, vd, k0, v0, tau)
        torch.cuda.synchronize()
        for got in (r, rf):
            s = got.scores.cpu().numpy()
            assert np.array_equal(np.isnan(s), np.isnan(scores)), tau
            fin = ~np.isnan(scores)
            assert np.abs(s[fin] - scores[fin]).max() <= 2e-5, tau
            assert np.array_equal(got.mask.cpu().numpy(), mask), tau
            assert np.array_equal(got.work_list.cpu().numpy(), wl_ref), tau
            assert int(got.n_active.cpu()[0]) == n_act, tau
        with np.errstate(invalid="ignore"):  # the non-finite heads' rows
            ref = oracle.routed_decode(q_np, k_np, v_np, v0_ref, mask)
        o = out.cpu().numpy()
        sink_rows_exact(o, v0_ref, mask, G)
        rows = np.isfinite(q_np).all(axis=-1)
        assert rows.sum() == B * 16 - 2
        assert_outputs(o[rows], ref[rows], f"{wl.name} tau={tau}")


# --- the longest contexts: cache offsets past 32 bits -----------------------------
@pytest.mark.parametrize("dtype,d,T,B,kernel", [("bf16", 64, 36_000_000, 1, "auto"),
                                                 ("bf16", 64, 36_000_000, 1, "valu"),
                                                 ("f32", 128, 17_000_000, 1, "auto"),
                                                 ("bf16", 64, 18_000_000, 2, "auto")],
                         ids=["bf16-d64-36m", "bf16-d64-36m-valu", "f32-d128-17m",
                              "bf16-d64-18m-b2"])
def test_context_with_offsets_past_32_bits(dtype, d, T, B, kernel):
    # Cache rows 2.2e9-4.6e9 elements (4.6e9-9.2e9 bytes) from the cache base,
    # past any 32-bit element or byte index: the last rows of a 36M-position
    # (bf16) or 17M-position (fp32, d = 128) item, or the second sequence of a
    # batch of two 18M-position items.  Each item's cache spans hundreds of
    # lanes.  One group per sequence is planted as a sink and one is active
    # (G = 2): routing, k0/v0 and the sink rows exact, every active group
    # against the oracle, one call bitwise equal to two calls.
    from workloads import make_caches_device
    wl = Workload(f"ctx-{dtype}-{T // 1_000_000}m-b{B}", B, 4, 2, d, T, dtype, seed=97,
                  sink_plan=("count", 1))
    assert max((T - 1) * d, (B - 1) * 2 * T * d) > 2 ** 31
    dev = torch.device("cuda")
    k, v = make_caches_device(wl, dev)
    q_cpu, planted = make_queries(wl)
    q = q_cpu.to(dev)
    lau = launch(kernel)
    k0, v0, r, out = run_routed(q, k, v, wl.tau, lau)
    out1, rf = sr.route_decode(q, k, v, k0, v0, wl.tau, launch=lau)
    torch.cuda.synchronize()
    k0_ref = as_numpy(k[:, :, 0].cpu()).astype(np.float64)
    v0_ref = as_numpy(v[:, :, 0].cpu()).astype(np.float64)
    assert np.array_equal(k0.cpu().numpy(), k0_ref) and np.array_equal(v0.cpu().numpy(), v0_ref)
    q_np = as_numpy(q_cpu)
    mask, n_active = assert_route(r, q_np, k0_ref, wl.tau)
    assert n_active == B and mask.tolist() == planted.to(torch.uint8).tolist()
    for name in ("scores", "mask", "work_list", "n_active"):
        assert torch.equal(getattr(rf, name), getattr(r, name)), name
    assert torch.equal(out1, out)
    got = out.cpu().numpy()
    sink_rows_exact(got, v0_ref, mask, 2)
    log(f"{wl.name}: grid {sr.grid_size(sr.make_shape(q, k, v), None)}")
    for j in r.work_list.cpu().numpy()[:n_active]:
        b, g = divmod(int(j), 2)
        ref = oracle.attend_group(q_np[b, 2 * g:2 * g + 2], as_numpy(k[b, g].cpu()),
                                  as_numpy(v[b, g].cpu()), 1.0 / math.sqrt(d))
        assert_outputs(got[b, 2 * g:2 * g + 2], ref, f"{wl.name} active group {b}, {g}")


def test_rope_step_at_a_position_past_32_bit_offsets():
    # One whole decode step (sr_rope_route_decode) whose new token lands at
    # position 35,999,999 of a 36M-position bf16 layer (d = 64): the rotary
    # angles reach 3.6e7 radians and the appended rows sit 2.3e9 elements past
    # the cache base.  Against the oracle's own rotation and append: rotated
    # query within 1 fp32 ulp, appended key within 1 bf16 ulp, value exact;
    # then routing (one group planted as a sink through its rotated queries)
    # and the active group's attention over the cache holding the oracle's rows.
    from workloads import make_caches_device
    wl = Workload("rope-36m", 1, 4, 2, 64, 36_000_000, "bf16", seed=98, sink_plan=("none",))
    T, d, G, pos = wl.seq_len, wl.head_dim, 2, wl.seq_len - 1
    dev = torch.device("cuda")
    k, v = make_caches_device(wl, dev)
    k0d, v0d = sr.record_sink(k, v)
    k0_ref = as_numpy(k[:, :, 0].cpu()).astype(np.float64)
    v0_ref = as_numpy(v[:, :, 0].cpu()).astype(np.float64)
    f = rope_inv_freq(d)
    gen = torch.Generator().manual_seed(4242)
    kn, vn = (torch.randn((1, 2, d), generator=gen) for _ in range(2))
    target = torch.randn((1, 4, d), generator=gen, dtype=torch.float64)
    u = torch.from_numpy(k0_ref[0, 0]) / float(np.linalg.norm(k0_ref[0, 0]))
    for h in range(G):  # group 0's rotated queries lie near its k0: a sink
        target[0, h] = 0.9 * u * target[0, h].norm() + 0.05 * target[0, h]
    qn = torch.from_numpy(oracle.rope(target.numpy(), -pos, f.numpy())).float()
    out, r, q_rot = sr.rope_route_decode(qn.to(dev), kn.to(dev), vn.to(dev), k, v, k0d, v0d,
                                         f.to(dev), wl.tau)
    torch.cuda.synchronize()
    q_ref = oracle.rope(qn.numpy(), pos, f.numpy())
    assert (np.abs(q_rot.cpu().numpy() - q_ref) <= np.abs(q_ref) * 2 ** -23 + 1e-30).all()
    k_row = oracle.round_bf16(oracle.rope(kn.numpy(), pos, f.numpy()))
    v_row = oracle.round_bf16(vn.numpy())
    k_dev = as_numpy(k[:, :, pos].cpu()).astype(np.float64)
    assert (np.abs(k_dev - k_row) <= _bf16_ulp(k_row) + 1e-30).all(), "appended key row"
    assert np.array_equal(as_numpy(v[:, :, pos].cpu()).astype(np.float64), v_row)
    scores, mask, wl_ref, n_act = oracle.route(q_ref, k0_ref, wl.tau)
    assert mask.tolist() == [[1, 0]] and n_act == 1
    assert np.array_equal(r.mask.cpu().numpy(), mask)
    assert np.array_equal(r.work_list.cpu().numpy(), wl_ref)
    assert int(r.n_active.cpu()[0]) == 1
    assert np.abs(r.scores.cpu().numpy() - scores).max() <= 2e-5
    got = out.cpu().numpy()
    sink_rows_exact(got, v0_ref, mask, G)
    ks = as_numpy(k[0, 1].cpu())
    vs = as_numpy(v[0, 1].cpu())
    ks[pos], vs[pos] = k_row[0, 1], v_row[0, 1]  # the oracle's own appended rows
    ref = oracle.attend_group(q_ref[0, 2:4], ks, vs, 1.0 / math.sqrt(d))
    assert_outputs(got[0, 2:4], ref, "rope-36m active group")


def test_calls_on_two_streams_at_once_match_their_sequential_results():
    # Two layers decoded on two streams at the same time, each through the
    # default workspace of its own stream: no state is shared between the
    # calls, so each result is bitwise the one its layer gives alone.
    wls = [Workload("stream-a", 1, 32, 8, 128, 200_000, "bf16", seed=201, sink_plan=("count", 4)),
           Workload("stream-b", 2, 16, 4, 128, 150_000, "bf16", seed=202, sink_plan=("count", 1))]
    layers = [upload(make_layer(wl)) for wl in wls]
    sinks = [sr.record_sink(k, v) for _, k, v in layers]
    alone = []
    for wl, (q, k, v), (k0, v0) in zip(wls, layers, sinks):
        out, r = sr.route_decode(q, k, v, k0, v0, wl.tau)
        alone.append((out.clone(), r.work_list.clone()))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    results = [None, None]
    for _ in range(3):
        for i, (wl, (q, k, v), (k0, v0)) in enumerate(zip(wls, layers, sinks)):
            with torch.cuda.stream(streams[i]):
                results[i] = sr.route_decode(q, k, v, k0, v0, wl.tau)
        torch.cuda.synchronize()
        for (out, r), (ref, ref_list) in zip(results, alone):
            assert torch.equal(out, ref) and torch.equal(r.work_list, ref_list)
