"""The seeded generator: reproducible, shaped like the five layers, and every
head's routing score kept >= 0.05 away from tau (checked with the oracle)."""
import numpy as np
import pytest
import torch

import oracle
from workloads import (CONFIGS, L8B_128K, L8B_256K_B4, L8B_512K, L70B_128K_B8, SINK_FRACTIONS,
                       TINY, as_numpy, make_caches, make_k0, make_layer, make_queries,
                       planted_sinks, sweep)

MARGIN = 0.05


def _bf16_valued(t):
    return torch.equal(t, t.to(torch.bfloat16).to(torch.float32))


@pytest.mark.parametrize("wl", CONFIGS, ids=lambda w: w.name)
def test_margin_and_planted_mask_match_oracle(wl):
    q, planted = make_queries(wl)
    k0 = make_k0(wl)
    scores, mask, lst, n_active = oracle.route(as_numpy(q), as_numpy(k0), wl.tau)
    assert np.abs(scores - wl.tau).min() >= MARGIN
    assert np.array_equal(mask.astype(bool), planted.numpy())
    assert torch.allclose(k0.norm(dim=-1), torch.full(k0.shape[:2], 30.0), rtol=1e-2)
    if wl.kv_dtype == "bf16":
        assert _bf16_valued(q) and _bf16_valued(k0)


@pytest.mark.parametrize("f", SINK_FRACTIONS)
def test_sweep_margins_and_counts(f):
    for base in (L8B_512K, L8B_256K_B4):
        wl = sweep(base, f)
        q, planted = make_queries(wl)
        assert (planted.sum(dim=1) == round(f * wl.num_kv_heads)).all()
        scores, mask, _, _ = oracle.route(as_numpy(q), as_numpy(make_k0(wl)), wl.tau)
        assert np.abs(scores - wl.tau).min() >= MARGIN
        assert np.array_equal(mask.astype(bool), planted.numpy())


def test_tiny_is_the_stated_layer():
    L = make_layer(TINY)
    assert L.k.shape == (1, 2, 4096, 64) and L.k.dtype == torch.float32
    assert L.q.shape == (1, 4, 64)
    assert L.planted.tolist() == [[True, False]]
    assert torch.equal(L.k[:, :, 0], make_k0(TINY))


def test_reproducible_and_thread_count_independent():
    wl = L8B_128K.with_(seq_len=3000)
    k1, v1 = make_caches(wl, threads=1)
    k2, v2 = make_caches(wl, threads=7)
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    assert k1.dtype == torch.bfloat16 and k1.shape == (1, 8, 3000, 128)
    q1, _ = make_queries(wl)
    q2, _ = make_queries(wl)
    assert torch.equal(q1, q2)
    other = wl.with_(seed=wl.seed + 1)
    assert not torch.equal(make_caches(other)[0], k1)


def test_bernoulli_plan_varies_per_item():
    p = planted_sinks(L70B_128K_B8)
    assert p.shape == (8, 8)
    assert 0 < int(p.sum()) < 64
    assert len({tuple(r.tolist()) for r in p}) > 1


def test_cache_entries_look_standard_normal():
    wl = L8B_128K.with_(seq_len=20000)
    k, v = make_caches(wl)
    vv = v.float()
    assert abs(vv.mean().item()) < 5e-3 and abs(vv.std().item() - 1.0) < 5e-3
    kk = k[:, :, 1:].float()
    assert abs(kk.std().item() - 1.0) < 5e-3


def test_bulk_layer_has_the_same_recipe():
    from workloads import Workload, make_layer_bulk
    wl = Workload("bulk", 512, 16, 8, 128, 4, "bf16", seed=7, sink_plan=("bernoulli", 0.5))
    L = make_layer_bulk(wl)
    assert L.k.shape == (512, 8, 4, 128) and L.k.dtype == torch.bfloat16
    assert L.q.shape == (512, 16, 128) and L.q.dtype == torch.float32
    assert torch.equal(L.q, L.q.to(torch.bfloat16).to(torch.float32))
    k0 = L.k[:, :, 0].float()
    assert torch.allclose(k0.norm(dim=-1), torch.full((512, 8), 30.0), rtol=2e-3)
    frac = L.planted.float().mean().item()
    assert 0.45 < frac < 0.55
    # planted heads point along their group's k0, the others are isotropic
    unit = (k0 / k0.norm(dim=-1, keepdim=True)).repeat_interleave(2, dim=1)
    cos = (L.q * unit).sum(-1) / L.q.norm(dim=-1)
    planted = L.planted.repeat_interleave(2, dim=1)
    assert cos[planted].min().item() > 0.7
    assert cos[~planted].abs().max().item() < 0.45
    again = make_layer_bulk(wl)
    assert torch.equal(again.k, L.k) and torch.equal(again.q, L.q)
    assert not torch.equal(make_layer_bulk(wl.with_(seed=8)).k, L.k)
