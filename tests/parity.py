"""Shared helpers of the GPU parity tests: run the HIP path through the
binding on a seeded layer and compare it with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from workloads import as_numpy

# The bar (fp32 accumulation over bf16/fp32 caches against the fp64 oracle):
MAX_ABS = 1e-2       # stated tolerance
MEAN_ABS = 1e-3      # stated tolerance
ROW_REL_L2 = 1e-3    # per output row; a zero or garbage row fails it at any T
# Expected error of a correct kernel is ~1e-6 relative (fp32 sums, exact bf16
# products, ~2^-16 relative split of the query for the MFMA logits); this
# tighter bound flags precision regressions long before the bar.
ROW_REL_L2_TIGHT = 2e-4
SCORE_ATOL = 2e-5    # fp32 cosine against fp64


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def upload(layer, device="cuda"):
    return (layer.q.to(device), layer.k.to(device), layer.v.to(device))


def out_stats(got: np.ndarray, ref: np.ndarray) -> dict:
    err = np.abs(got.astype(np.float64) - ref)
    rows_ref = ref.reshape(-1, ref.shape[-1])
    rows_err = (got.astype(np.float64) - ref).reshape(-1, ref.shape[-1])
    rel = np.linalg.norm(rows_err, axis=1) / np.maximum(np.linalg.norm(rows_ref, axis=1), 1e-30)
    return {"max_abs": float(err.max()), "mean_abs": float(err.mean()),
            "max_row_rel_l2": float(rel.max())}


def assert_outputs(got: np.ndarray, ref: np.ndarray, what: str, tight: bool = True) -> dict:
    st = out_stats(got, ref)
    log(f"  {what}: max_abs={st['max_abs']:.3e} mean_abs={st['mean_abs']:.3e} "
        f"row_rel_l2={st['max_row_rel_l2']:.3e}")
    assert st["max_abs"] <= MAX_ABS, (what, st)
    assert st["mean_abs"] <= MEAN_ABS, (what, st)
    assert st["max_row_rel_l2"] <= ROW_REL_L2, (what, st)
    if tight:
        assert st["max_row_rel_l2"] <= ROW_REL_L2_TIGHT, (what, st)
    return st


def assert_route(r, q_np, k0_np, tau):
    scores, mask, wl, n_active = oracle.route(q_np, k0_np, tau)
    assert np.abs(scores - tau).min() >= 0.05, "generated scores too close to tau"
    got_scores = r.scores.cpu().numpy()
    assert np.abs(got_scores - scores).max() <= SCORE_ATOL
    assert np.array_equal(r.mask.cpu().numpy(), mask), "mask differs"
    assert np.array_equal(r.work_list.cpu().numpy(), wl), "work list differs"
    assert int(r.n_active.cpu()[0]) == n_active
    return mask, n_active


def sink_rows_exact(out: np.ndarray, v0: np.ndarray, mask: np.ndarray, G: int) -> int:
    n = 0
    B, Hkv = mask.shape
    for b in range(B):
        for g in range(Hkv):
            if mask[b, g]:
                for h in range(G):
                    assert np.array_equal(out[b, g * G + h], v0[b, g]), (b, g, h)
                    n += 1
    return n


def oracle_inputs(layer):
    return as_numpy(layer.q), as_numpy(layer.k), as_numpy(layer.v)


# A workspace starts with a ticket region of fixed size: one int32 ticket for
# each of the envelope's 32768 items, then the routing kernel's ticket.
MAX_ITEMS = 32768


def ticket_region(ws, n_items: int = MAX_ITEMS + 1) -> torch.Tensor:
    return ws.buf[: 4 * n_items].view(torch.int32)


def route_ticket(ws) -> int:
    """The routing kernel's ticket, after the item tickets."""
    off = 4 * MAX_ITEMS
    return int(ws.buf[off:off + 4].view(torch.int32).cpu()[0])
