"""Plain fp64 CPU oracle for SinkRouter's sink-aware GQA decode attention.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
statement of what the decode path computes.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
(the HIP library and its Python binding) never does, and the two share no
code.  Every array is read as its exact stored value and widened to float64.

Sources (the method is described on these pages):
  * SinkRouter GitHub README (github.com/streamer-AP/SinkRouter), the list of
    decode-time steps in its introduction: the key at position 0 is kept
    from prefill; at decode the rotated query is compared with it; the
    decision is taken per GQA KV group ahead of any read of the long cache;
    a sink group answers with the value at position 0; the other groups run
    ordinary tiled attention with an online softmax, split over the context
    and merged inside the kernel.  Its configuration section calls the
    threshold a cosine threshold, 0.5 by default.
  * SinkRouter paper (arXiv 2604.16883) as rendered by pith.science: Eq. (1)
    in the Figure 1 caption defines the head update as the attention-weighted
    sum of the cached values; the Figure 10 caption scores the routing proxy
    as cos(q, K_BOS) at the KV-group level.

Readings where the pages are silent:
  * a group is a sink only when every one of its query heads scores >= tau;
  * a zero-norm query or key scores 0 (so the group stays active unless
    tau <= 0); a NaN or infinite element leaves the cosine undefined: the
    score is NaN, which fails ">= tau" at every tau (the head dissents);
  * query head h reads KV head h // G (the Hugging Face repeat_kv layout);
  * the softmax scale is 1/sqrt(d) unless given;
  * split s covers positions [s*L, min((s+1)*L, T)) with L = ceil(T/S), an
    empty split contributes nothing, and splits are merged in ascending s.

Shapes: q [B][Hq][d]; caches [B][Hkv][T][d]; k0, v0 [B][Hkv][d];
out [B][Hq][d]; scores [B][Hq]; mask [B][Hkv] (1 = sink).
"""
from __future__ import annotations

import math

import numpy as np

# Caches are walked in chunks of this many positions so the fp64 copies of a
# long (512K-position) slab never sit in memory whole.
_CHUNK = 1 << 16


def _f64(x) -> np.ndarray:
    """Exact widening of a float16/bfloat16-as-float32/float32 array to float64."""
    return np.asarray(x, dtype=np.float64)


def default_scale(head_dim: int) -> float:
    """Softmax scale of standard Llama attention, 1/sqrt(d)."""
    return 1.0 / math.sqrt(head_dim)


# ---------------------------------------------------------------------------
# Step 1: prefill keeps the position-0 key and value.
# README, decode-time steps: the prefill path is unchanged apart from keeping
# the key at position 0; sink groups later answer with the value there.
# ---------------------------------------------------------------------------
def record_sink(k_cache, v_cache):
    """Return (k0, v0) = (K[:, :, 0, :], V[:, :, 0, :]) widened to fp64."""
    k = np.asarray(k_cache)
    v = np.asarray(v_cache)
    if k.ndim != 4 or v.shape != k.shape:
        raise ValueError("caches must both be [B][Hkv][T][d]")
    return _f64(k[:, :, 0, :]).copy(), _f64(v[:, :, 0, :]).copy()


# ---------------------------------------------------------------------------
# Step 2: routing score, cos(q, k0) per query head.
# README configuration section (cosine routing threshold); pith.science
# Figure 10 caption (cos(q, K_BOS) as the routing proxy).
# ---------------------------------------------------------------------------
def cosine(a, b) -> float:
    """cos(a, b) = <a, b> / (|a| |b|); 0 when either vector is zero."""
    a = _f64(a)
    b = _f64(b)
    denom = math.sqrt(float(np.dot(a, a))) * math.sqrt(float(np.dot(b, b)))
    if denom == 0.0:
        return 0.0
    return float(np.dot(a, b)) / denom


def route_scores(q, k0):
    """scores[b, h] = cos(q[b, h], k0[b, h // G])."""
    q = _f64(q)
    k0 = _f64(k0)
    B, Hq, d = q.shape
    Bk, Hkv, dk = k0.shape
    if Bk != B or dk != d or Hq % Hkv != 0:
        raise ValueError("q [B][Hq][d] and k0 [B][Hkv][d] disagree")
    G = Hq // Hkv
    scores = np.zeros((B, Hq), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            scores[b, h] = cosine(q[b, h], k0[b, h // G])
    return scores


# ---------------------------------------------------------------------------
# Step 3: group decision and the compacted work list.
# README decode-time steps: the decision is per GQA KV group, taken before
# the cache is read.  Reading: a group is a sink only if all its heads clear
# tau.
# ---------------------------------------------------------------------------
def group_mask(scores, num_kv_heads: int, tau: float):
    """mask[b, g] = 1 iff scores[b, h] >= tau for every head h of group g."""
    scores = np.asarray(scores, dtype=np.float64)
    B, Hq = scores.shape
    G = Hq // num_kv_heads
    mask = np.zeros((B, num_kv_heads), dtype=np.uint8)
    for b in range(B):
        for g in range(num_kv_heads):
            heads = scores[b, g * G:(g + 1) * G]
            mask[b, g] = 1 if all(c >= tau for c in heads) else 0
    return mask


def work_list(mask):
    """Items j = b*Hkv + g: active ones in ascending j, then sinks ascending.

    Returns (list as int32 array, number of active items)."""
    flat = np.asarray(mask).reshape(-1)
    active = [j for j in range(flat.size) if flat[j] == 0]
    sinks = [j for j in range(flat.size) if flat[j] != 0]
    return np.array(active + sinks, dtype=np.int32), len(active)


def route(q, k0, tau: float):
    """Full routing step: (scores, mask, work_list, n_active)."""
    scores = route_scores(q, k0)
    mask = group_mask(scores, np.asarray(k0).shape[1], tau)
    wl, n_active = work_list(mask)
    return scores, mask, wl, n_active


# ---------------------------------------------------------------------------
# Step 4 (active groups): exact softmax attention, Eq. (1) of the paper
# (pith.science, Figure 1 caption): u = sum_i alpha_i v_i with alpha the
# softmax of the scaled query-key products over every cached position.
# ---------------------------------------------------------------------------
def attend_group(q_heads, k_slab, v_slab, scale: float):
    """Attention of G query heads [G][d] over one KV slab [T][d] -> [G][d].

    Two passes over T: logits and their maximum, then the max-subtracted
    exponentials and the weighted sum of values, normalised at the end."""
    qg = _f64(q_heads)
    T = np.asarray(k_slab).shape[0]
    if T < 1:
        raise ValueError("need at least one cached position")
    logits = np.empty((qg.shape[0], T), dtype=np.float64)
    for t0 in range(0, T, _CHUNK):
        kc = _f64(k_slab[t0:t0 + _CHUNK])
        logits[:, t0:t0 + kc.shape[0]] = scale * (qg @ kc.T)
    zmax = logits.max(axis=1, keepdims=True)
    weights = np.exp(logits - zmax)
    denom = weights.sum(axis=1)
    out = np.zeros_like(qg)
    for t0 in range(0, T, _CHUNK):
        vc = _f64(v_slab[t0:t0 + _CHUNK])
        out += weights[:, t0:t0 + vc.shape[0]] @ vc
    return out / denom[:, None]


def dense_decode(q, k_cache, v_cache, scale: float | None = None):
    """Routing disabled: every group attends over its whole cache."""
    q = np.asarray(q)
    B, Hq, d = q.shape
    Hkv = np.asarray(k_cache).shape[1]
    G = Hq // Hkv
    s = default_scale(d) if scale is None else scale
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            out[b, g * G:(g + 1) * G] = attend_group(
                q[b, g * G:(g + 1) * G], k_cache[b, g], v_cache[b, g], s)
    return out


# ---------------------------------------------------------------------------
# Step 5: routed decode.  README decode-time steps: a sink group answers with
# the position-0 value without touching the cache; active groups take step 4.
# ---------------------------------------------------------------------------
def routed_decode(q, k_cache, v_cache, v0, mask, scale: float | None = None):
    """The routed step (README decode-time steps): a sink group (mask 1)
    answers every one of its heads with v0 of the group; any other group
    attends over its whole cache as Eq. (1) states (attend_group)."""
    q = np.asarray(q)
    B, Hq, d = q.shape
    Hkv = np.asarray(k_cache).shape[1]
    G = Hq // Hkv
    s = default_scale(d) if scale is None else scale
    v0 = _f64(v0)
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            rows = slice(g * G, (g + 1) * G)
            if mask[b, g]:
                out[b, rows] = v0[b, g][None, :]
            else:
                out[b, rows] = attend_group(q[b, rows], k_cache[b, g], v_cache[b, g], s)
    return out


# ---------------------------------------------------------------------------
# Split-K algebra (README decode-time steps: the context is split across
# programs and the pieces are merged inside the kernel).  Used only to show the result does not depend on S;
# device outputs are always compared with the exact attention above.
# ---------------------------------------------------------------------------
def split_partials(q_heads, k_slab, v_slab, scale: float, num_splits: int):
    """Per split s: (m_s [G], l_s [G], acc_s [G][d]) over positions
    [s*L, min((s+1)*L, T)), L = ceil(T/S).  Empty splits give m=-inf, l=0, acc=0."""
    qg = _f64(q_heads)
    T = np.asarray(k_slab).shape[0]
    L = -(-T // num_splits)
    parts = []
    for s in range(num_splits):
        t0, t1 = s * L, min((s + 1) * L, T)
        if t0 >= t1:
            parts.append((np.full(qg.shape[0], -np.inf), np.zeros(qg.shape[0]),
                          np.zeros_like(qg)))
            continue
        z = scale * (qg @ _f64(k_slab[t0:t1]).T)
        m = z.max(axis=1)
        p = np.exp(z - m[:, None])
        parts.append((m, p.sum(axis=1), p @ _f64(v_slab[t0:t1])))
    return parts


def merge_partials(parts):
    """Combine split partials in ascending s: M = max m_s,
    l = sum e^(m_s - M) l_s, out = sum e^(m_s - M) acc_s / l."""
    m_all = np.stack([p[0] for p in parts])          # [S][G]
    M = m_all.max(axis=0)
    G, d = parts[0][2].shape
    l = np.zeros(G)
    acc = np.zeros((G, d))
    for m, ls, a in parts:
        w = np.where(np.isneginf(m), 0.0, np.exp(m - M))
        l += w * ls
        acc += w[:, None] * a
    return acc / l[:, None]


def split_k_decode(q, k_cache, v_cache, num_splits: int, scale: float | None = None):
    """Every group through the split algebra above: its partials over
    num_splits contiguous ranges, merged in ascending order.  Equal to
    dense_decode up to rounding for any split count (the invariance pins)."""
    q = np.asarray(q)
    B, Hq, d = q.shape
    Hkv = np.asarray(k_cache).shape[1]
    G = Hq // Hkv
    s = default_scale(d) if scale is None else scale
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            rows = slice(g * G, (g + 1) * G)
            out[b, rows] = merge_partials(split_partials(
                q[b, rows], k_cache[b, g], v_cache[b, g], s, num_splits))
    return out


# ---------------------------------------------------------------------------
# Position-0 attention mass and the routing proxy's precision/recall.
# pith.science rendering of arXiv 2604.16883: Eq. (1) (Figure 1 caption)
# gives the weights alpha_i; the Figure 10 caption scores cos(q, K_BOS) as a
# predictor of an "oracle" sink event defined from the full-attention weight
# on the first position, per KV group, as a function of the threshold tau
# (Figure 8 sweeps that threshold).  The event threshold is not printed:
# reading taken here: a group is an oracle sink when every head puts at least
# `event_mass` of its attention on position 0.
# ---------------------------------------------------------------------------
def bos_mass(q, k_cache, scale: float | None = None):
    """alpha_0[b, h]: softmax weight of position 0 for every query head."""
    q = np.asarray(q)
    B, Hq, d = q.shape
    Hkv, T = np.asarray(k_cache).shape[1], np.asarray(k_cache).shape[2]
    G = Hq // Hkv
    s = default_scale(d) if scale is None else scale
    out = np.zeros((B, Hq))
    for b in range(B):
        for g in range(Hkv):
            qg = _f64(q[b, g * G:(g + 1) * G])
            logits = np.empty((G, T))
            for t0 in range(0, T, _CHUNK):
                kc = _f64(k_cache[b, g, t0:t0 + _CHUNK])
                logits[:, t0:t0 + kc.shape[0]] = s * (qg @ kc.T)
            zmax = logits.max(axis=1)
            w = np.exp(logits - zmax[:, None])
            out[b, g * G:(g + 1) * G] = w[:, 0] / w.sum(axis=1)
    return out


def oracle_sink_events(alpha0, num_kv_heads: int, event_mass: float):
    """[B][Hkv] bool: every head of the group has alpha_0 >= event_mass."""
    a = np.asarray(alpha0)
    B, Hq = a.shape
    G = Hq // num_kv_heads
    return np.array([[all(a[b, g * G + i] >= event_mass for i in range(G))
                      for g in range(num_kv_heads)] for b in range(B)])


def proxy_precision_recall(predicted, events):
    """Precision, recall and F1 of predicted sinks against oracle events.
    Conventions: precision = 1 when nothing is predicted, recall = 1 when
    there is no event, F1 = 0 when precision + recall = 0."""
    p = np.asarray(predicted, dtype=bool).reshape(-1)
    e = np.asarray(events, dtype=bool).reshape(-1)
    tp = int(np.sum(p & e))
    fp = int(np.sum(p & ~e))
    fn = int(np.sum(~p & e))
    precision = tp / (tp + fp) if tp + fp else 1.0
    recall = tp / (tp + fn) if tp + fn else 1.0
    f1 = 2 * precision * recall / (precision + recall) if precision + recall else 0.0
    return precision, recall, f1


def threshold_sweep(scores, events, num_kv_heads: int, taus):
    """(tau, precision, recall, F1) of the group rule at every tau."""
    rows = []
    for tau in taus:
        pred = group_mask(scores, num_kv_heads, float(tau)).astype(bool)
        rows.append((float(tau), *proxy_precision_recall(pred, events)))
    return rows


# ---------------------------------------------------------------------------
# Decode-step neighbours: rotary position embedding of the new token's query
# and key, and the append of its key and value to the caches.  README
# decode-time steps: routing compares the *RoPE* query with the position-0
# key, so the query is rotated first.  Reading (the pages do not print the
# rotary form): the Hugging Face Llama "rotate half" convention, element i
# paired with element i + d/2, angle pos * inv_freq[i], in exact arithmetic.
# ---------------------------------------------------------------------------
def rope(x, pos: int, inv_freq):
    """Rotate the last axis of x (..., d) to position pos (fp64)."""
    x = _f64(x)
    d = x.shape[-1]
    f = _f64(inv_freq)
    ang = float(pos) * f
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def round_bf16(x):
    """fp64 -> bf16 value (as fp64), rounding to nearest even in one step."""
    x = _f64(x)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    scaled = np.ldexp(m, 8)                 # 8 significant bits before the point
    return np.ldexp(np.round(scaled), e - 8)  # np.round is round-half-even


def rope_append(q_new, k_new, v_new, k_cache, v_cache, pos: int, inv_freq, bf16: bool):
    """Return (rotated q fp64, caches with the rotated key and the value
    written at position pos, rounded to bf16 when the caches are bf16)."""
    q_rot = rope(q_new, pos, inv_freq)
    k_rot = rope(k_new, pos, inv_freq)
    v = _f64(v_new)
    kc = _f64(k_cache).copy()
    vc = _f64(v_cache).copy()
    kc[:, :, pos] = round_bf16(k_rot) if bf16 else k_rot.astype(np.float32)
    vc[:, :, pos] = round_bf16(v) if bf16 else v.astype(np.float32)
    return q_rot, kc, vc
