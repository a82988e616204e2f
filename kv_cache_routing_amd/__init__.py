"""Python binding of libsinkroute (sink-routed GQA decode attention, gfx950).

Argument marshalling only: every step of the decode path runs in the HIP
library.  torch supplies device memory and the current stream.

    k0, v0 = record_sink(k, v)                   # prefill side
    r = route(q, k0, tau=0.5)                    # scores, mask, work_list, n_active
    out = decode_attn(q, k, v, v0, r.work_list, r.n_active)
    ref = dense_decode(q, k, v)                  # routing off

Shapes: q [B][Hq][d] fp32; caches [B][Hkv][T][d] (bf16 or fp32, d contiguous,
any T_max >= T via a narrowed view); k0, v0 [B][Hkv][d] fp32.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _native as N
from ._native import (SR_KERNEL_AUTO, SR_KERNEL_MFMA, SR_KERNEL_VALU,  # noqa: F401
                      SinkRouteError)

__all__ = ["record_sink", "route", "decode_attn", "route_decode", "dense_decode",
           "dense_decode_alpha0", "rope_append", "rope_route_decode", "Workspace",
           "make_shape", "make_launch", "splits_for", "split_cap", "grid_size", "plan_parts",
           "SinkRouteError", "Routing", "SR_KERNEL_AUTO", "SR_KERNEL_VALU", "SR_KERNEL_MFMA"]


# Every call below runs these on the host before its launch, so they are kept
# lean: the ctypes signatures convert plain ints and floats, and torch's raw
# stream getter (where it exists) skips building a Stream object, which alone
# cost ~3 us a call; a small layer's eager step is bound by this host time.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream():
    if _raw_stream is not None:
        return _raw_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


# Counting devices does not initialise the GPU.
_SEVERAL_GPUS = torch.cuda.device_count() > 1


def _on_device(t: torch.Tensor, name: str):
    """The library launches on the current device and its stream: every
    array must live there (a host pointer or another GPU's would be read by
    the kernels as this GPU's memory)."""
    dev = t.get_device()
    if dev < 0:
        raise ValueError(f"libsinkroute takes device tensors ({name} is a host tensor)")
    if _SEVERAL_GPUS and dev != torch.cuda.current_device():
        raise ValueError(f"libsinkroute takes tensors on the current device: {name} is on "
                         f"cuda:{dev}, the current device is cuda:{torch.cuda.current_device()}")


def _expect(t: torch.Tensor, name: str, shape: tuple, dtype: torch.dtype):
    """The kernels index these arrays densely from the cache shape: anything
    else would read or write outside them; and they must be on the device.
    (Kept cheap: it runs on every call, and launch-bound steps pay for it.)"""
    if t.shape != shape or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")
    _on_device(t, name)


def _expect_q(q: torch.Tensor, k: torch.Tensor):
    qs, ks = q.shape, k.shape
    if len(qs) != 3 or len(ks) != 4 or qs[0] != ks[0] or qs[2] != ks[3]:
        raise ValueError(f"q must be [B][Hq][d] matching the cache [B][Hkv][T][d]: "
                         f"q {tuple(qs)}, cache {tuple(ks)}")
    if q.dtype != torch.float32 or not q.is_contiguous():
        _expect(q, "q", qs, torch.float32)


def make_shape(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor | None = None) -> N.SrShape:
    """sr_shape from q [B][Hq][d] and a cache view [B][Hkv][T][d]."""
    ks, st, dtype = k.shape, k.stride(), k.dtype
    if len(ks) != 4:
        raise ValueError("cache must be [B][Hkv][T][d]")
    if v is not None and (v.shape != ks or v.stride() != st or v.dtype != dtype):
        raise ValueError("K and V caches must share shape, strides and dtype")
    if st[3] != 1:
        raise ValueError("head_dim must be contiguous")
    if dtype == torch.bfloat16:
        dt = N.SR_KV_BF16
    elif dtype == torch.float32:
        dt = N.SR_KV_F32
    else:
        raise ValueError(f"unsupported cache dtype {dtype}")
    B, Hkv, T, d = ks
    Hq = q.shape[1] if q is not None else Hkv
    return N.SrShape(B, Hq, Hkv, d, T, st[0], st[1], st[2], dt, 0)


def make_launch(num_splits: int = 0, kernel: int = SR_KERNEL_AUTO, wgs_per_cu: int = 0,
                waves_per_wg: int = 0):
    return N.SrLaunch(num_splits, kernel, wgs_per_cu, waves_per_wg)


def splits_for(shape: N.SrShape, launch: N.SrLaunch | None, n_active: int) -> int:
    return N.lib.sr_splits_for(ctypes.byref(shape), _lp(launch), n_active)


def split_cap(shape: N.SrShape, launch: N.SrLaunch | None) -> int:
    return N.lib.sr_split_cap(ctypes.byref(shape), _lp(launch))


def grid_size(shape: N.SrShape, launch: N.SrLaunch | None) -> int:
    return N.lib.sr_grid_size(ctypes.byref(shape), _lp(launch))


def plan_parts(shape: N.SrShape, launch: N.SrLaunch | None, n_active: int, wg: int) -> list:
    """Workgroup wg's parts of the work division (host-side, no device work):
    a list of dicts with item, part, parts, lanes, first, end, chunk."""
    buf = (N.SrPart * 2)()
    r = N.lib.sr_plan_parts(ctypes.byref(shape), _lp(launch), int(n_active), int(wg), buf, 2)
    if r < 0:
        raise SinkRouteError(N.SR_ERR_INVALID_ARG, "sr_plan_parts")
    return [{f: getattr(buf[i], f) for f, _ in N.SrPart._fields_} for i in range(r)]


def _lp(launch):
    return None if launch is None else ctypes.byref(launch)


class Workspace:
    """Scratch for the decode calls (split partials + tickets), zeroed once."""

    def __init__(self, shape: N.SrShape, launch: N.SrLaunch | None, device):
        self.nbytes = int(N.lib.sr_workspace_bytes(ctypes.byref(shape), _lp(launch)))
        if self.nbytes == 0:
            raise SinkRouteError(N.SR_ERR_UNSUPPORTED, "sr_workspace_bytes")
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        N.check(N.lib.sr_workspace_init(self.buf.data_ptr(), self.nbytes, _stream()),
                "sr_workspace_init")

    def fits(self, shape, launch) -> bool:
        return int(N.lib.sr_workspace_bytes(ctypes.byref(shape), _lp(launch))) <= self.nbytes


def rope_append(q_new, k_new, v_new, k_cache, v_cache, pos: int, inv_freq,
                q_out: torch.Tensor | None = None):
    """Rotate the new token's query/key to `pos`, append key and value to the
    full-capacity caches [B][Hkv][T_max][d] at `pos`; returns the rotated q."""
    _expect_q(q_new, k_cache)
    B, Hkv, _, d = k_cache.shape
    _expect(k_new, "k_new", (B, Hkv, d), torch.float32)
    _expect(v_new, "v_new", (B, Hkv, d), torch.float32)
    _expect(inv_freq, "inv_freq", (d // 2,), torch.float32)
    if q_out is not None:
        _expect(q_out, "q_out", q_new.shape, torch.float32)
    _on_device(q_new, "q_new")
    _on_device(k_cache, "k_cache")
    _on_device(v_cache, "v_cache")
    shape = make_shape(q_new, k_cache, v_cache)
    if q_out is None:
        q_out = torch.empty_like(q_new)
    N.check(N.lib.sr_rope_append(ctypes.byref(shape), q_new.data_ptr(), k_new.data_ptr(),
                                 v_new.data_ptr(), inv_freq.data_ptr(), int(pos),
                                 q_out.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                 _stream()), "sr_rope_append")
    return q_out


def record_sink(k: torch.Tensor, v: torch.Tensor, q_heads: int | None = None):
    _on_device(k, "k")
    _on_device(v, "v")
    shape = make_shape(None, k, v)
    B, Hkv, _, d = k.shape
    k0 = torch.empty((B, Hkv, d), dtype=torch.float32, device=k.device)
    v0 = torch.empty_like(k0)
    N.check(N.lib.sr_record_sink(ctypes.byref(shape), k.data_ptr(), v.data_ptr(), k0.data_ptr(),
                                 v0.data_ptr(), _stream()), "sr_record_sink")
    return k0, v0


@dataclass
class Routing:
    scores: torch.Tensor     # [B][Hq] fp32
    mask: torch.Tensor       # [B][Hkv] uint8, 1 = sink
    work_list: torch.Tensor  # [B*Hkv] int32
    n_active: torch.Tensor   # [1] int32 (device)


def _expect_routing(r: Routing, B: int, Hq: int, Hkv: int):
    _expect(r.scores, "scores", (B, Hq), torch.float32)
    _expect(r.mask, "mask", (B, Hkv), torch.uint8)
    _expect(r.work_list, "work_list", (B * Hkv,), torch.int32)
    _expect(r.n_active, "n_active", (1,), torch.int32)


def route(q: torch.Tensor, k0: torch.Tensor, tau: float = 0.5, out: Routing | None = None):
    if k0.dim() != 3 or q.dim() != 3 or q.shape[0] != k0.shape[0] or q.shape[2] != k0.shape[2]:
        raise ValueError(f"q [B][Hq][d] and k0 [B][Hkv][d] disagree: {tuple(q.shape)}, "
                         f"{tuple(k0.shape)}")
    B, Hkv, d = k0.shape
    Hq = q.shape[1]
    if q.dtype != torch.float32 or k0.dtype != torch.float32:
        raise ValueError("q and k0 are fp32")
    if out is not None:
        _expect_routing(out, B, Hq, Hkv)
    _on_device(q, "q")
    _on_device(k0, "k0")
    q = q.contiguous()
    k0 = k0.contiguous()
    shape = N.SrShape(B, Hq, Hkv, d, 1, Hkv * d, d, d, N.SR_KV_F32, 0)
    if out is None:
        dev = q.device
        out = Routing(torch.empty((B, Hq), dtype=torch.float32, device=dev),
                      torch.empty((B, Hkv), dtype=torch.uint8, device=dev),
                      torch.empty((B * Hkv,), dtype=torch.int32, device=dev),
                      torch.empty((1,), dtype=torch.int32, device=dev))
    N.check(N.lib.sr_route(ctypes.byref(shape), q.data_ptr(), k0.data_ptr(), float(tau),
                           out.scores.data_ptr(), out.mask.data_ptr(), out.work_list.data_ptr(),
                           out.n_active.data_ptr(), _stream()), "sr_route")
    return out


# The workspaces calls use when the caller passes none: one per (device,
# stream), replaced by a larger one when a layer needs more, so that repeated
# calls neither allocate nor clear scratch.  Calls on one stream run in order
# and each leaves its tickets at zero, so the next call may reuse the
# workspace; calls on different streams get different ones.  A replaced
# workspace is kept, not freed: a graph captured on that stream may still use
# it.  Graphs captured on one stream share its workspace, so graphs that may
# replay at the same time on different streams need workspaces of their own
# (the ws argument).
_default_ws: dict = {}
_replaced_ws: list = []


def _workspace_for(shape, launch, device):
    key = (device.index, _stream())
    ws = _default_ws.get(key)
    if ws is None or not ws.fits(shape, launch):
        if ws is not None:
            _replaced_ws.append(ws)
        ws = Workspace(shape, launch, device)
        _default_ws[key] = ws
    return ws


def _prep(q, k, v, launch, ws, out, q_checked=False):
    """Checks common to the decode calls, the shape, a workspace and the
    output."""
    if not q_checked:
        _expect_q(q, k)
    if out is not None:
        _expect(out, "out", q.shape, torch.float32)
    _on_device(q, "q")
    _on_device(k, "k")
    _on_device(v, "v")
    shape = make_shape(q, k, v)
    if ws is None:
        ws = _workspace_for(shape, launch, q.device)
    elif not ws.fits(shape, launch):
        ws = Workspace(shape, launch, q.device)
    if out is None:
        out = torch.empty_like(q)
    return shape, ws, out


def decode_attn(q, k, v, v0, work_list, n_active, sm_scale: float = 0.0,
                launch: N.SrLaunch | None = None, ws: Workspace | None = None,
                out: torch.Tensor | None = None):
    _expect_q(q, k)
    B, Hkv, _, d = k.shape
    _expect(v0, "v0", (B, Hkv, d), torch.float32)
    _expect(work_list, "work_list", (B * Hkv,), torch.int32)
    _expect(n_active, "n_active", (1,), torch.int32)
    shape, ws, out = _prep(q, k, v, launch, ws, out, q_checked=True)
    N.check(N.lib.sr_decode_attn(ctypes.byref(shape), _lp(launch), q.data_ptr(), k.data_ptr(),
                                 v.data_ptr(), v0.data_ptr(), work_list.data_ptr(),
                                 n_active.data_ptr(), float(sm_scale), ws.buf.data_ptr(),
                                 ws.nbytes, out.data_ptr(), _stream()), "sr_decode_attn")
    return out


def route_decode(q, k, v, k0, v0, tau: float = 0.5, sm_scale: float = 0.0,
                 launch: N.SrLaunch | None = None, ws: Workspace | None = None,
                 out: torch.Tensor | None = None, routing: Routing | None = None):
    """Routing and decode in one call (one launch up to 64 query heads, the
    routing kernel and then the decode above); returns (out, routing outputs)."""
    _expect_q(q, k)
    B, Hkv, _, d = k.shape
    _expect(k0, "k0", (B, Hkv, d), torch.float32)
    _expect(v0, "v0", (B, Hkv, d), torch.float32)
    if routing is not None:
        _expect_routing(routing, B, q.shape[1], Hkv)
    shape, ws, out = _prep(q, k, v, launch, ws, out, q_checked=True)
    if routing is None:
        dev = q.device
        routing = Routing(torch.empty((B, q.shape[1]), dtype=torch.float32, device=dev),
                          torch.empty((B, Hkv), dtype=torch.uint8, device=dev),
                          torch.empty((B * Hkv,), dtype=torch.int32, device=dev),
                          torch.empty((1,), dtype=torch.int32, device=dev))
    N.check(N.lib.sr_route_decode(ctypes.byref(shape), _lp(launch), q.data_ptr(), k.data_ptr(),
                                  v.data_ptr(), k0.data_ptr(), v0.data_ptr(), float(tau),
                                  float(sm_scale), routing.scores.data_ptr(),
                                  routing.mask.data_ptr(), routing.work_list.data_ptr(),
                                  routing.n_active.data_ptr(), ws.buf.data_ptr(), ws.nbytes,
                                  out.data_ptr(), _stream()), "sr_route_decode")
    return out, routing


def rope_route_decode(q_new, k_new, v_new, k, v, k0, v0, inv_freq, tau: float = 0.5,
                      sm_scale: float = 0.0, launch: N.SrLaunch | None = None,
                      ws: Workspace | None = None, out: torch.Tensor | None = None,
                      routing: Routing | None = None, q_out: torch.Tensor | None = None):
    """One decode step in one call (one launch up to 64 query heads, two
    above; q_out carries the rotated queries between them): rotate the new
    token's query and key to position T - 1 and append its key and value
    there, then route and attend over positions 0 .. T - 1.  k, v are cache
    views [B][Hkv][T][d] whose last row is the new token's (their storage
    must hold it).  Returns (out, routing outputs, rotated q)."""
    _expect_q(q_new, k)
    B, Hkv, _, d = k.shape
    for t, name in ((k_new, "k_new"), (v_new, "v_new"), (k0, "k0"), (v0, "v0")):
        _expect(t, name, (B, Hkv, d), torch.float32)
    _expect(inv_freq, "inv_freq", (d // 2,), torch.float32)
    if q_out is not None:
        _expect(q_out, "q_out", q_new.shape, torch.float32)
    if routing is not None:
        _expect_routing(routing, B, q_new.shape[1], Hkv)
    shape, ws, out = _prep(q_new, k, v, launch, ws, out, q_checked=True)
    dev = q_new.device
    if q_out is None:
        q_out = torch.empty_like(q_new)
    if routing is None:
        routing = Routing(torch.empty((B, q_new.shape[1]), dtype=torch.float32, device=dev),
                          torch.empty((B, Hkv), dtype=torch.uint8, device=dev),
                          torch.empty((B * Hkv,), dtype=torch.int32, device=dev),
                          torch.empty((1,), dtype=torch.int32, device=dev))
    N.check(N.lib.sr_rope_route_decode(
        ctypes.byref(shape), _lp(launch), q_new.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
        inv_freq.data_ptr(), q_out.data_ptr(), k.data_ptr(), v.data_ptr(), k0.data_ptr(),
        v0.data_ptr(), float(tau), float(sm_scale), routing.scores.data_ptr(),
        routing.mask.data_ptr(), routing.work_list.data_ptr(), routing.n_active.data_ptr(),
        ws.buf.data_ptr(), ws.nbytes, out.data_ptr(), _stream()), "sr_rope_route_decode")
    return out, routing, q_out


def dense_decode_alpha0(q, k, v, sm_scale: float = 0.0, launch: N.SrLaunch | None = None,
                        ws: Workspace | None = None, out: torch.Tensor | None = None):
    """Dense decode plus the attention weight of position 0 per head."""
    shape, ws, out = _prep(q, k, v, launch, ws, out)
    alpha0 = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    N.check(N.lib.sr_dense_decode_alpha0(ctypes.byref(shape), _lp(launch), q.data_ptr(),
                                         k.data_ptr(), v.data_ptr(), float(sm_scale),
                                         ws.buf.data_ptr(), ws.nbytes, out.data_ptr(),
                                         alpha0.data_ptr(), _stream()),
            "sr_dense_decode_alpha0")
    return out, alpha0


def dense_decode(q, k, v, sm_scale: float = 0.0, launch: N.SrLaunch | None = None,
                 ws: Workspace | None = None, out: torch.Tensor | None = None):
    shape, ws, out = _prep(q, k, v, launch, ws, out)
    N.check(N.lib.sr_dense_decode(ctypes.byref(shape), _lp(launch), q.data_ptr(), k.data_ptr(),
                                  v.data_ptr(), float(sm_scale), ws.buf.data_ptr(), ws.nbytes,
                                  out.data_ptr(), _stream()), "sr_dense_decode")
    return out
