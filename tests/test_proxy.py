"""The product-side proxy evaluation (torch) against the oracle's counting."""
import numpy as np
import torch

import oracle
from kv_cache_routing_amd import proxy


def test_proxy_counts_match_oracle():
    rng = np.random.default_rng(3)
    for _ in range(30):
        B, Hkv, G = 3, 8, 4
        scores = rng.uniform(-1, 1, size=(B, Hkv * G))
        alpha0 = rng.uniform(0, 1, size=(B, Hkv * G)) ** 3
        taus = np.linspace(-1, 1, 9)
        ev_ref = oracle.oracle_sink_events(alpha0, Hkv, 0.3)
        ev = proxy.sink_events(torch.from_numpy(alpha0), Hkv, 0.3)
        assert np.array_equal(ev.numpy(), ev_ref)
        ref = oracle.threshold_sweep(scores, ev_ref, Hkv, taus)
        got = proxy.threshold_sweep(torch.from_numpy(scores), torch.from_numpy(alpha0), Hkv, taus, 0.3)
        for (tau, p, r, f), row in zip(ref, got):
            assert (row["tau"], row["precision"], row["recall"]) == (tau, p, r)
            assert abs(row["f1"] - f) < 1e-15
