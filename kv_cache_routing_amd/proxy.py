"""Evaluation of the cosine routing proxy against position-0 attention mass.

The pith.science rendering of arXiv 2604.16883 (Figure 10 caption) scores
cos(q, K_BOS) as a predictor of an "oracle" sink event defined from the
full-attention weight of the first position, per KV group, across the
threshold tau (Figure 8 calibrates that threshold).  These helpers take the
device outputs of `route` (scores) and `dense_decode_alpha0` (alpha_0 per
head) and count.  Reading for the event threshold, which the pages do not
print: a group is an event when every one of its heads puts at least
`event_mass` of its attention on position 0.  Evaluation only: nothing here
is on the decode path.
"""
from __future__ import annotations

import torch


def sink_events(alpha0: torch.Tensor, num_kv_heads: int, event_mass: float) -> torch.Tensor:
    """[B][Hkv] bool: every head of the group has alpha_0 >= event_mass."""
    B, Hq = alpha0.shape
    return (alpha0 >= event_mass).view(B, num_kv_heads, Hq // num_kv_heads).all(dim=-1)


def predicted_sinks(scores: torch.Tensor, num_kv_heads: int, tau: float) -> torch.Tensor:
    """[B][Hkv] bool: the routing rule (every head's cosine >= tau)."""
    B, Hq = scores.shape
    return (scores >= tau).view(B, num_kv_heads, Hq // num_kv_heads).all(dim=-1)


def precision_recall(predicted: torch.Tensor, events: torch.Tensor):
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


def threshold_sweep(scores: torch.Tensor, alpha0: torch.Tensor, num_kv_heads: int, taus,
                    event_mass: float = 0.5):
    """Precision / recall / F1 of the routing rule at every tau."""
    events = sink_events(alpha0, num_kv_heads, event_mass)
    rows = []
    for tau in taus:
        p, r, f = precision_recall(predicted_sinks(scores, num_kv_heads, float(tau)), events)
        rows.append({"tau": float(tau), "precision": p, "recall": r, "f1": f})
    return rows
