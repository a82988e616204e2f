"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test names the pin it checks: brute force on tiny inputs, a library
routine (torch's scaled_dot_product_attention in fp64, scipy's cosine
distance, Python's stable sort), closed forms (T = 1, q = 0, the fixed-point
bound of Eq. (1)), invariants (split count, permutation of positions 1..T-1,
GQA = repeated-KV MHA) and hand-built routing cases with closed-form cosines
(tests/golden/route_cases.json).  The last block plants plausible mistakes in
copies of the oracle and checks that some pin catches each one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import sinkrouter as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_layer(seed, B, Hq, Hkv, T, d, k0_norm=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    if k0_norm is not None:
        k[:, :, 0] *= k0_norm / np.linalg.norm(k[:, :, 0], axis=-1, keepdims=True)
    return q, k, v


# --- p1: brute force ---------------------------------------------------------
def brute_force(q, k, v, scale):
    """Triple loop with math.exp and math.fsum, one head at a time."""
    B, Hq, d = q.shape
    Hkv, T = k.shape[1], k.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            z = [scale * math.fsum(q[b, h, i] * k[b, g, t, i] for i in range(d)) for t in range(T)]
            zm = max(z)
            w = [math.exp(x - zm) for x in z]
            den = math.fsum(w)
            for i in range(d):
                out[b, h, i] = math.fsum(w[t] * v[b, g, t, i] for t in range(T)) / den
    return out


@pytest.mark.parametrize("B,Hq,Hkv,T,d", [(1, 2, 2, 1, 4), (2, 4, 2, 17, 8), (1, 8, 2, 64, 8),
                                          (1, 4, 1, 33, 5)])
def test_p1_dense_equals_brute_force(B, Hq, Hkv, T, d):
    q, k, v = rand_layer(1 + T, B, Hq, Hkv, T, d)
    s = 0.37
    np.testing.assert_allclose(oracle.dense_decode(q, k, v, s), brute_force(q, k, v, s),
                               rtol=0, atol=1e-12)


# --- p2: library routine -----------------------------------------------------
@pytest.mark.parametrize("B,Hq,Hkv,T,d", [(2, 8, 2, 300, 64), (1, 32, 8, 129, 128), (3, 4, 4, 50, 16)])
def test_p2_dense_equals_torch_sdpa_fp64(B, Hq, Hkv, T, d):
    q, k, v = rand_layer(7 + d, B, Hq, Hkv, T, d, k0_norm=30.0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None, :], torch.from_numpy(k), torch.from_numpy(v),
        enable_gqa=True).squeeze(2).numpy()
    np.testing.assert_allclose(oracle.dense_decode(q, k, v), ref, rtol=0, atol=1e-12)


# --- p3: GQA equals MHA with repeated KV heads ------------------------------
def test_p3_gqa_equals_repeated_kv_mha():
    q, k, v = rand_layer(3, 2, 8, 2, 77, 16)
    G = 4
    k_rep = np.repeat(k, G, axis=1)
    v_rep = np.repeat(v, G, axis=1)
    np.testing.assert_allclose(oracle.dense_decode(q, k, v),
                               oracle.dense_decode(q, k_rep, v_rep), rtol=0, atol=1e-14)


# --- p4: routed sink rows are v0 exactly ------------------------------------
def test_p4_sink_rows_are_v0_bit_exact():
    q, k, v = rand_layer(4, 2, 8, 4, 40, 16)
    k0, v0 = oracle.record_sink(k, v)
    mask = np.array([[1, 0, 1, 0], [0, 1, 1, 1]], dtype=np.uint8)
    out = oracle.routed_decode(q, k, v, v0, mask)
    dense = oracle.dense_decode(q, k, v)
    for b in range(2):
        for g in range(4):
            rows = out[b, 2 * g:2 * g + 2]
            if mask[b, g]:
                assert np.array_equal(rows, np.stack([v[b, g, 0]] * 2))
            else:
                assert np.array_equal(rows, dense[b, 2 * g:2 * g + 2])


# --- p5: fixed point of Eq. (1) ---------------------------------------------
def test_p5_fixed_point_bound():
    d, T = 64, 4096
    rng = np.random.default_rng(5)
    k = rng.standard_normal((1, 1, T, d))
    v = rng.standard_normal((1, 1, T, d))
    k[0, 0, 0] *= 400.0 / np.linalg.norm(k[0, 0, 0])
    q = (k[0, 0, 0] / np.linalg.norm(k[0, 0, 0]))[None, None, :]
    out = oracle.dense_decode(q, k, v)[0, 0]
    z = (k[0, 0] @ q[0, 0]) / 8.0
    delta = z[0] - z[1:].max()
    assert delta > 45.0
    spread = np.abs(v[0, 0, 1:] - v[0, 0, 0]).max()
    bound = (T - 1) * math.exp(-delta) * spread
    err = np.abs(out - v[0, 0, 0]).max()
    assert err <= bound + 1e-15
    # general form: |u - v0| <= (1 - alpha_0) max_t |v_t - v0|
    w = np.exp(z - z.max())
    alpha0 = w[0] / w.sum()
    assert err <= (1 - alpha0) * spread * (1 + 1e-9) + 1e-15


def test_p5_general_bound_moderate_dominance():
    d, T = 16, 500
    rng = np.random.default_rng(55)
    k = rng.standard_normal((1, 1, T, d))
    v = rng.standard_normal((1, 1, T, d))
    k[0, 0, 0] *= 12.0 / np.linalg.norm(k[0, 0, 0])
    q = (k[0, 0, 0] / np.linalg.norm(k[0, 0, 0]))[None, None, :] * 2.0
    out = oracle.dense_decode(q, k, v)[0, 0]
    z = (k[0, 0] @ q[0, 0]) / 4.0
    w = np.exp(z - z.max())
    alpha0 = w[0] / w.sum()
    assert 0.0 < alpha0 < 1.0
    dev = v[0, 0, 1:] - v[0, 0, 0]
    lhs = np.linalg.norm(out - v[0, 0, 0])
    assert lhs <= (1 - alpha0) * np.linalg.norm(dev, axis=1).max() * (1 + 1e-12)


# --- p6: T = 1 ----------------------------------------------------------------
def test_p6_single_position_returns_v0_exactly():
    q, k, v = rand_layer(6, 2, 6, 3, 1, 32)
    out = oracle.dense_decode(q, k, v)
    assert np.array_equal(out, np.repeat(v[:, :, 0], 2, axis=1))


# --- p7: q = 0 ----------------------------------------------------------------
def test_p7_zero_query_is_uniform_average_and_active():
    q, k, v = rand_layer(7, 1, 4, 2, 123, 16)
    q[:] = 0.0
    out = oracle.dense_decode(q, k, v)
    np.testing.assert_allclose(out, np.repeat(v.mean(axis=2), 2, axis=1), rtol=0, atol=1e-14)
    scores, mask, wl, n_active = oracle.route(q, k[:, :, 0], 0.5)
    assert np.array_equal(scores, np.zeros_like(scores))
    assert mask.sum() == 0 and n_active == 2


def test_p7_degenerate_scores_reading():
    # The cosine of a zero vector is read as 0 and an undefined one (a NaN or
    # infinite element) stays NaN, which fails ">= tau" at every tau: such a
    # head keeps its group active.  A zero k0 makes its whole group score 0,
    # a sink exactly when tau <= 0.
    rng = np.random.default_rng(71)
    q = rng.standard_normal((1, 8, 16))
    k0 = rng.standard_normal((1, 4, 16))
    k0[0, 1] = 0.0                      # group 1: zero position-0 key
    q[0, 4, 3] = np.nan                 # group 2, head 0: a NaN element
    q[0, 7, 0] = np.inf                 # group 3, head 1: an infinite element
    scores = oracle.route_scores(q, k0)
    assert np.array_equal(scores[0, 2:4], [0.0, 0.0])
    assert np.isnan(scores[0, 4]) and np.isnan(scores[0, 7])
    finite = [0, 1, 5, 6]
    np.testing.assert_allclose(scores[0, finite],
                               [float(orc.cosine(q[0, h], k0[0, h // 2])) for h in finite],
                               rtol=0, atol=0)
    for tau, want in ((0.5, [0, 0, 0, 0]), (0.0, [0, 1, 0, 0]), (-2.0, [1, 1, 0, 0])):
        _, mask, wl, n_active = oracle.route(q, k0, tau)
        assert mask[0].tolist() == want, tau
        assert n_active == 4 - sum(want)
        assert set(wl[:n_active].tolist()) >= {2, 3}   # the NaN groups stay active


# --- p8: split-K invariance ---------------------------------------------------
@pytest.mark.parametrize("S", [1, 2, 3, 7, 64, 100, 105])
def test_p8_split_count_invariance(S):
    q, k, v = rand_layer(8, 1, 8, 2, 100, 16, k0_norm=30.0)
    ref = oracle.dense_decode(q, k, v)
    got = oracle.split_k_decode(q, k, v, S)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_p8_per_token_partials_are_exact_softmax_terms():
    # S = T: each split holds one position, so m = z_t, l = 1, acc = v_t
    q, k, v = rand_layer(88, 1, 2, 1, 9, 4)
    parts = oracle.split_partials(q[0], k[0, 0], v[0, 0], 0.5, 9)
    for t, (m, l, acc) in enumerate(parts):
        np.testing.assert_allclose(m, 0.5 * (q[0] @ k[0, 0, t]), rtol=0, atol=1e-15)
        assert np.array_equal(l, np.ones(2))
        assert np.array_equal(acc, np.stack([v[0, 0, t]] * 2))


# --- p9: permutation invariance ----------------------------------------------
def test_p9_permuting_positions_after_0():
    q, k, v = rand_layer(9, 2, 8, 2, 200, 32, k0_norm=30.0)
    perm = np.concatenate([[0], 1 + np.random.default_rng(0).permutation(199)])
    np.testing.assert_allclose(oracle.dense_decode(q, k[:, :, perm], v[:, :, perm]),
                               oracle.dense_decode(q, k, v), rtol=0, atol=1e-13)
    r1 = oracle.route(q, k[:, :, 0], 0.5)
    r2 = oracle.route(q, k[:, :, perm][:, :, 0], 0.5)
    assert np.array_equal(r1[1], r2[1])


# --- p10: cosine closed forms and a library routine --------------------------
def test_p10_cosine_identities():
    import scipy.spatial.distance as ssd
    rng = np.random.default_rng(10)
    for _ in range(20):
        a, b = rng.standard_normal(64), rng.standard_normal(64)
        c = oracle.cosine(a, b)
        assert abs(c - (1.0 - ssd.cosine(a, b))) < 1e-14
        assert abs(oracle.cosine(3.5 * a, 0.25 * b) - c) < 1e-14
        assert abs(oracle.cosine(a, a) - 1.0) < 1e-15
        assert abs(oracle.cosine(-a, a) + 1.0) < 1e-15
    assert oracle.cosine(np.zeros(8), np.ones(8)) == 0.0
    e = np.eye(4)
    assert oracle.cosine(e[0], e[1]) == 0.0


def test_p10_route_scores_per_head_group_map():
    # head h of a group of G reads k0 of group h // G
    rng = np.random.default_rng(11)
    k0 = rng.standard_normal((2, 3, 16))
    q = np.zeros((2, 6, 16))
    for b in range(2):
        for h in range(6):
            q[b, h] = k0[b, h // 2] * (h + 1)
    scores = oracle.route_scores(q, k0)
    np.testing.assert_allclose(scores, np.ones((2, 6)), rtol=0, atol=1e-14)


# --- routing golden cases (closed-form cosines) ------------------------------
def _golden_cases():
    with open(os.path.join(GOLDEN, "route_cases.json")) as f:
        return json.load(f)["cases"]


def build_golden(case):
    B, Hq, Hkv, d = case["batch"], case["num_q_heads"], case["num_kv_heads"], case["head_dim"]
    k0 = np.zeros((B, Hkv, d))
    q = np.zeros((B, Hq, d))
    for b in range(B):
        for g in range(Hkv):
            k0[b, g, 0] = case["k0_scale"][b][g]
        for h in range(Hq):
            a, c = case["q_ab"][b][h]
            q[b, h, 0], q[b, h, 1] = a, c
    return q, k0


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_route_golden_cases(case):
    q, k0 = build_golden(case)
    scores, mask, wl, n_active = oracle.route(q, k0, case["tau"])
    np.testing.assert_allclose(scores, np.array(case["expect_scores"]), rtol=0, atol=1e-15)
    assert mask.tolist() == case["expect_mask"]
    assert wl.tolist() == case["expect_work_list"]
    assert n_active == case["expect_n_active"]


def test_work_list_is_python_stable_sort_by_sink_flag():
    rng = np.random.default_rng(12)
    for _ in range(50):
        mask = (rng.random((3, 8)) < rng.random()).astype(np.uint8)
        wl, n_active = oracle.work_list(mask)
        flat = mask.reshape(-1).tolist()
        assert wl.tolist() == sorted(range(len(flat)), key=lambda j: flat[j])
        assert n_active == flat.count(0)


def test_record_sink_takes_position_zero():
    q, k, v = rand_layer(13, 2, 4, 2, 10, 8)
    k0, v0 = oracle.record_sink(k, v)
    assert np.array_equal(k0, k[:, :, 0]) and np.array_equal(v0, v[:, :, 0])


def test_rope_at_position_zero_is_identity():
    # The recorded key is the same before and after rotary embedding: every
    # rotation angle at position 0 is 0 (reading of the README's pre/post-RoPE
    # wording; the routing score does not depend on which one is kept).
    d = 128
    x = np.random.default_rng(14).standard_normal(d)
    inv_freq = 500000.0 ** (-np.arange(0, d, 2) / d)
    ang = 0 * inv_freq
    cos, sin = np.cos(np.concatenate([ang, ang])), np.sin(np.concatenate([ang, ang]))
    rot = np.concatenate([-x[d // 2:], x[:d // 2]])
    assert np.array_equal(x * cos + rot * sin, x)


# --- planted mistakes: each one must trip a pin -----------------------------
def _mut_wrong_group_map(q, k, v, scale):
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            g = h % Hkv  # wrong: interleaved head->group map
            out[b, h] = orc.attend_group(q[b, h:h + 1], k[b, g], v[b, g], scale)[0]
    return out


def _mut_no_scale(q, k, v, scale):
    return oracle.dense_decode(q, k, v, 1.0)


def _mut_transposed(q, k, v, scale):
    return oracle.dense_decode(q, v, k, scale)  # K and V swapped


def _mut_skip_position0(q, k, v, scale):
    return oracle.dense_decode(q, k[:, :, 1:], v[:, :, 1:], scale)


def _mut_no_normalise(q, k, v, scale):
    out = np.zeros(q.shape)
    B, Hq, d = q.shape
    G = Hq // k.shape[1]
    for b in range(B):
        for h in range(Hq):
            z = scale * (k[b, h // G] @ q[b, h])
            out[b, h] = np.exp(z - z.max()) @ v[b, h // G]
    return out


@pytest.mark.parametrize("mutant", [_mut_wrong_group_map, _mut_no_scale, _mut_transposed,
                                    _mut_skip_position0, _mut_no_normalise])
def test_planted_attention_mistakes_fail_sdpa_pin(mutant):
    q, k, v = rand_layer(21, 1, 8, 2, 60, 16, k0_norm=30.0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None, :], torch.from_numpy(k), torch.from_numpy(v),
        enable_gqa=True).squeeze(2).numpy()
    assert np.abs(mutant(q, k, v, 0.25) - ref).max() > 1e-6


def test_planted_routing_mistakes_fail_golden():
    cases = _golden_cases()

    def any_rule(scores, Hkv, tau):  # "any head" instead of "every head"
        B, Hq = scores.shape
        G = Hq // Hkv
        return np.array([[int(any(scores[b, g * G + i] >= tau for i in range(G)))
                          for g in range(Hkv)] for b in range(B)], dtype=np.uint8)

    caught = {"any": False, "unstable": False}
    for case in cases:
        q, k0 = build_golden(case)
        sc = oracle.route_scores(q, k0)
        if any_rule(sc, k0.shape[1], case["tau"]).tolist() != case["expect_mask"]:
            caught["any"] = True
        mask = np.array(case["expect_mask"], dtype=np.uint8)
        reversed_sinks = [j for j in range(mask.size) if not mask.flat[j]] + \
            [j for j in reversed(range(mask.size)) if mask.flat[j]]
        if reversed_sinks != case["expect_work_list"]:
            caught["unstable"] = True
    assert all(caught.values()), caught


def test_threshold_tie_counts_as_sink():
    # Reading: "cosine >= tau" (ties route to the sink side).  Generated
    # layers keep every score at least 0.05 away from tau, so ties never occur.
    assert orc.group_mask(np.array([[0.5, 0.5]]), 1, 0.5).tolist() == [[1]]
    assert orc.group_mask(np.array([[0.5, np.nextafter(0.5, 0.0)]]), 1, 0.5).tolist() == [[0]]


# --- oracle sink events (hand-built weights, tests/golden/sink_event_cases.json) --
def _event_cases():
    with open(os.path.join(GOLDEN, "sink_event_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _event_cases(), ids=lambda c: c["name"])
def test_oracle_sink_events_golden(case):
    a0 = np.array(case["alpha0"], dtype=np.float64)
    assert a0.shape == (case["batch"], case["num_q_heads"])
    ev = oracle.oracle_sink_events(a0, case["num_kv_heads"], case["event_mass"])
    assert ev.dtype == bool and ev.tolist() == case["expect_events"]


def test_oracle_sink_events_from_closed_form_weights():
    # End to end with alpha_0 from the oracle's own softmax, on layers whose
    # weights are known in closed form: one head of each group aligned with a
    # norm-400 position-0 key (alpha_0 > 1 - (T-1) e^-delta, near 1), the other
    # head a zero query (alpha_0 = 1/T exactly).
    d, T = 32, 64
    rng = np.random.default_rng(76)
    k = rng.standard_normal((1, 2, T, d))
    k[0, :, 0] *= (400.0 / np.linalg.norm(k[0, :, 0], axis=-1))[:, None]
    q = np.zeros((1, 4, d))
    q[0, 0] = k[0, 0, 0] / np.linalg.norm(k[0, 0, 0])  # group 0: aligned + zero query
    q[0, 2] = k[0, 1, 0] / np.linalg.norm(k[0, 1, 0])  # group 1: aligned ...
    q[0, 3] = k[0, 1, 0] / np.linalg.norm(k[0, 1, 0])  # ... twice
    a0 = oracle.bos_mass(q, k)
    assert a0[0, 1] == 1.0 / T and a0[0, 0] > 0.999 and a0[0, 2] > 0.999
    assert oracle.oracle_sink_events(a0, 2, 0.5).tolist() == [[False, True]]
    # at a mass below 1/T every head qualifies
    assert oracle.oracle_sink_events(a0, 2, 1.0 / T).tolist() == [[True, True]]


def test_planted_event_mistakes_fail_golden():
    # Each plausible misreading of the event rule, applied to the golden
    # weights, must disagree with the stated events somewhere.
    def rule(combine, cmp, interleaved=False):
        def events(a0, Hkv, mass):
            B, Hq = a0.shape
            G = Hq // Hkv
            heads = (lambda g: range(g, Hq, Hkv)) if interleaved else \
                (lambda g: range(g * G, (g + 1) * G))
            return np.array([[combine([cmp(a0[b, h], mass) for h in heads(g)], a0[b, list(heads(g))], mass)
                              for g in range(Hkv)] for b in range(B)])
        return events

    every = lambda flags, vals, mass: all(flags)
    mutants = {
        "any head": rule(lambda f, v, m: any(f), lambda x, m: x >= m),
        "strict >": rule(every, lambda x, m: x > m),
        "mean of heads": rule(lambda f, v, m: float(np.mean(v)) >= m, lambda x, m: x >= m),
        "interleaved head map": rule(every, lambda x, m: x >= m, interleaved=True),
    }
    exact = rule(every, lambda x, m: x >= m)
    for name, mut in mutants.items():
        wrong = 0
        for case in _event_cases():
            a0 = np.array(case["alpha0"], dtype=np.float64)
            args = (a0, case["num_kv_heads"], case["event_mass"])
            assert exact(*args).tolist() == case["expect_events"]  # the harness itself
            wrong += mut(*args).tolist() != case["expect_events"]
        assert wrong, f"mutant '{name}' passes every golden case"


# --- position-0 attention mass and the proxy's precision/recall --------------
def test_bos_mass_against_torch_softmax_weights():
    q, k, v = rand_layer(71, 2, 8, 2, 150, 32, k0_norm=20.0)
    a0 = oracle.bos_mass(q, k)
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(np.repeat(k, 4, axis=1))
    w = torch.softmax((qt[:, :, None, :] @ kt.transpose(-1, -2)).squeeze(2) / math.sqrt(32), dim=-1)
    np.testing.assert_allclose(a0, w[..., 0].numpy(), rtol=0, atol=1e-14)


def test_bos_mass_closed_forms():
    q, k, v = rand_layer(72, 1, 4, 2, 1, 16)
    assert np.array_equal(oracle.bos_mass(q, k), np.ones((1, 4)))       # T = 1
    q, k, v = rand_layer(73, 1, 4, 2, 37, 16)
    q[:] = 0.0
    np.testing.assert_allclose(oracle.bos_mass(q, k), np.full((1, 4), 1 / 37), rtol=0, atol=1e-15)
    # dominant position 0: 1 - alpha_0 = sum_{t>=1} alpha_t <= (T-1) e^{-delta}
    d, T = 64, 2048
    rng = np.random.default_rng(74)
    k = rng.standard_normal((1, 1, T, d))
    k[0, 0, 0] *= 300.0 / np.linalg.norm(k[0, 0, 0])
    q = (k[0, 0, 0] / np.linalg.norm(k[0, 0, 0]))[None, None, :]
    z = (k[0, 0] @ q[0, 0]) / 8.0
    delta = z[0] - z[1:].max()
    assert 1.0 - oracle.bos_mass(q, k)[0, 0] <= (T - 1) * math.exp(-delta) + 1e-15


def test_precision_recall_hand_counts():
    pred = np.array([[1, 1, 0, 0], [1, 0, 1, 0]], dtype=bool)
    ev = np.array([[1, 0, 0, 1], [1, 0, 1, 1]], dtype=bool)
    # tp = 3 (00, 10, 12), fp = 1 (01), fn = 2 (03, 13)
    p, r, f = oracle.proxy_precision_recall(pred, ev)
    assert (p, r) == (0.75, 0.6)
    assert abs(f - 2 * 0.75 * 0.6 / 1.35) < 1e-15
    assert oracle.proxy_precision_recall(np.zeros(3, bool), np.zeros(3, bool)) == (1.0, 1.0, 1.0)
    assert oracle.proxy_precision_recall(np.zeros(3, bool), np.ones(3, bool))[:2] == (1.0, 0.0)


def test_threshold_sweep_is_monotone_in_predictions():
    # raising tau can only remove predicted sinks: recall never increases
    rng = np.random.default_rng(75)
    scores = rng.uniform(-1, 1, size=(4, 16))
    events = rng.random((4, 8)) < 0.5
    rows = oracle.threshold_sweep(scores, events, 8, np.linspace(-1, 1, 21))
    recalls = [r[2] for r in rows]
    assert all(a >= b - 1e-15 for a, b in zip(recalls, recalls[1:]))
    assert rows[0][2] == 1.0          # tau = -1: every group predicted


# --- rotary embedding and cache append ------------------------------------------
def _inv_freq(d, base=500000.0):
    return base ** (-np.arange(0, d, 2) / d)


def test_rope_identity_norm_and_complex_form():
    rng = np.random.default_rng(101)
    x = rng.standard_normal((3, 5, 128))
    f = _inv_freq(128)
    assert np.array_equal(oracle.rope(x, 0, f), x)                        # position 0
    y = oracle.rope(x, 12345, f)
    np.testing.assert_allclose(np.hypot(y[..., :64], y[..., 64:]),
                               np.hypot(x[..., :64], x[..., 64:]), rtol=1e-13)
    z = (x[..., :64] + 1j * x[..., 64:]) * np.exp(1j * 12345 * f)         # complex form
    np.testing.assert_allclose(y, np.concatenate([z.real, z.imag], axis=-1), rtol=0, atol=1e-12)


def test_rope_relative_position_and_composition():
    rng = np.random.default_rng(102)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    f = _inv_freq(64, 10000.0)
    a = oracle.rope(q, 700, f) @ oracle.rope(k, 650, f)
    b = oracle.rope(q, 50, f) @ k
    assert abs(a - b) < 1e-11
    np.testing.assert_allclose(oracle.rope(oracle.rope(q, 300, f), 400, f), oracle.rope(q, 700, f),
                               rtol=0, atol=1e-12)


def test_round_bf16_matches_torch_on_float32_values_and_ties():
    rng = np.random.default_rng(103)
    x = rng.standard_normal(100000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), ref)
    # exact ties round to even; one step avoids double rounding
    assert oracle.round_bf16(np.array([1.0 + 2 ** -8]))[0] == 1.0
    assert oracle.round_bf16(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6
    assert oracle.round_bf16(np.array([1.0 + 2 ** -8 + 2 ** -40]))[0] == 1.0 + 2 ** -7


def test_rope_append_writes_only_position_pos():
    rng = np.random.default_rng(104)
    B, Hq, Hkv, T, d = 2, 8, 2, 10, 32
    q, k, v = (rng.standard_normal((B, H, d)) for H in (Hq, Hkv, Hkv))
    kc = rng.standard_normal((B, Hkv, T, d))
    vc = rng.standard_normal((B, Hkv, T, d))
    f = _inv_freq(d)
    q_rot, kc2, vc2 = oracle.rope_append(q, k, v, kc, vc, 7, f, bf16=False)
    keep = [t for t in range(T) if t != 7]
    assert np.array_equal(kc2[:, :, keep], kc[:, :, keep]) and np.array_equal(vc2[:, :, keep], vc[:, :, keep])
    np.testing.assert_allclose(kc2[:, :, 7], oracle.rope(k, 7, f).astype(np.float32), rtol=0, atol=0)
    np.testing.assert_allclose(q_rot, oracle.rope(q, 7, f), rtol=0, atol=0)
