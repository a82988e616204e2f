"""Seeded synthetic decode-attention layers.

Shared by the parity tests, the smoke check and the benchmark.  This module
only draws and lays out random numbers; it holds none of the routed-decode
arithmetic (no scores, no routing decision, no attention), so nothing here can
make the HIP path and the CPU oracle agree by sharing a mistake.

Shapes follow the Llama-3.1-8B/70B decode layers the SinkRouter pages use for
their long-context measurements (the README's decode benchmark at 128K, 256K
and 512K; the abstract's 8B and 70B backbones):

* caches K, V: [B][Hkv][T][d], N(0, 1) entries, bf16 (fp32 for the tiny case),
  with the key at position 0 of every group rescaled to norm 30;
* queries q: [B][Hq][d] fp32.  A head planted as a sink is
  0.9 * k0 / |k0| + 0.05 * N(0, I); any other head is N(0, I).  In bf16
  layers q is rounded to bf16 values so every consumer sees the same numbers.

Rounding to bf16 is round-to-nearest-even (torch's float->bfloat16 cast).
Nothing here checks how far a head's score lies from the threshold: the
tests do that with the oracle for every seed they use.

Random streams: item b of a layer with base seed s has item seed s + b; every
(item, tensor, group) draws from its own torch CPU generator so slabs can be
filled by several threads and still give the same bits.  The position-0 key
has a stream of its own, so queries (which depend on it) can be drawn without
drawing the whole cache.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field, replace

import torch

K0_NORM = 30.0
SINK_ALIGN = 0.9
SINK_NOISE = 0.05


@dataclass(frozen=True)
class Workload:
    """One decode layer-step to generate.

    sink_plan: "tiny" (group 0 sink, the rest active), ("count", n) (n of Hkv
    groups per item, seeded subset), ("bernoulli", p) (each group a sink with
    probability p), or ("none",)."""
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seq_len: int
    kv_dtype: str                 # "bf16" or "f32"
    seed: int
    sink_plan: tuple = ("none",)
    tau: float = 0.5
    k0_norm: float = K0_NORM
    tags: dict = field(default_factory=dict, compare=False)

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.kv_dtype == "bf16" else torch.float32

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five layer shapes of the benchmark and parity suite.
TINY = Workload("tiny-4k-f32", 1, 4, 2, 64, 4096, "f32", seed=0, sink_plan=("tiny",))
L8B_128K = Workload("llama8b-128k", 1, 32, 8, 128, 131072, "bf16", seed=2000,
                    sink_plan=("count", 4))
L8B_256K_B4 = Workload("llama8b-256k-b4", 4, 32, 8, 128, 262144, "bf16", seed=3000,
                       sink_plan=("count", 4))
L8B_512K = Workload("llama8b-512k", 1, 32, 8, 128, 524288, "bf16", seed=4000,
                    sink_plan=("count", 4))
L70B_128K_B8 = Workload("llama70b-128k-b8", 8, 64, 8, 128, 131072, "bf16", seed=5000,
                        sink_plan=("bernoulli", 0.5))

CONFIGS = [TINY, L8B_128K, L8B_256K_B4, L8B_512K, L70B_128K_B8]
SINK_FRACTIONS = (0.0, 0.25, 0.5, 0.75, 1.0)


def sweep(base: Workload, fraction: float) -> Workload:
    """`base` with round(fraction * Hkv) planted sink groups in every item."""
    n = int(round(fraction * base.num_kv_heads))
    return base.with_(sink_plan=("count", n), name=f"{base.name}-sink{int(fraction * 100)}")


def _stream(item_seed: int, tag: int) -> torch.Generator:
    return torch.Generator().manual_seed(item_seed * 4096 + tag)


_TAG_K0 = 2000      # + group
_TAG_SINK = 4000
_TAG_Q = 4001


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_k0(wl: Workload) -> torch.Tensor:
    """[B][Hkv][d] fp32: the stored key at position 0 of every group.

    Drawn from its own stream per (item, group), rescaled to norm 30 and
    rounded to the layer's dtype, so queries can be built without the cache."""
    B, Hkv, d = wl.batch, wl.num_kv_heads, wl.head_dim
    k0 = torch.empty((B, Hkv, d), dtype=torch.float32)
    for b in range(B):
        for g in range(Hkv):
            row = torch.randn(d, generator=_stream(wl.seed + b, _TAG_K0 + g),
                              dtype=torch.float32)
            k0[b, g] = row * (wl.k0_norm / row.norm())
    return k0.to(wl.torch_dtype).to(torch.float32)


def make_caches(wl: Workload, *, threads: int | None = None):
    """K, V as contiguous CPU tensors [B][Hkv][T][d] of the layer's dtype."""
    B, Hkv, T, d = wl.batch, wl.num_kv_heads, wl.seq_len, wl.head_dim
    k = torch.empty((B, Hkv, T, d), dtype=wl.torch_dtype)
    v = torch.empty((B, Hkv, T, d), dtype=wl.torch_dtype)
    k0 = make_k0(wl)

    def fill(job):
        b, g, which = job
        slab = torch.randn((T, d), generator=_stream(wl.seed + b, 2 * g + which),
                           dtype=torch.float32)
        if which == 0:
            k[b, g].copy_(slab)
            k[b, g, 0].copy_(k0[b, g])
        else:
            v[b, g].copy_(slab)

    jobs = [(b, g, w) for b in range(B) for g in range(Hkv) for w in (0, 1)]
    with _cf.ThreadPoolExecutor(threads or _workers()) as ex:
        list(ex.map(fill, jobs))
    return k, v


def make_caches_device(wl: Workload, device, *, seed_offset: int = 0):
    """K, V [B][Hkv][T][d] drawn on `device`, for timing runs: the same recipe
    as make_caches (N(0, 1) entries rounded to the layer's dtype, the key at
    position 0 of every group replaced by make_k0(wl), so make_queries(wl)
    plants the same sinks) from torch's device generator, so the bits differ
    from make_caches'.  A multi-GiB layer takes well under a second; the
    parity tests draw on the host with make_caches."""
    B, Hkv, T, d = wl.batch, wl.num_kv_heads, wl.seq_len, wl.head_dim
    gen = torch.Generator(device=device).manual_seed(wl.seed * 4096 + 7000 + seed_offset)
    k = torch.empty((B, Hkv, T, d), dtype=wl.torch_dtype, device=device)
    v = torch.empty_like(k)
    for b in range(B):  # one item at a time bounds the fp32 staging
        for t in (k, v):
            t[b].copy_(torch.randn((Hkv, T, d), generator=gen, device=device,
                                   dtype=torch.float32))
    k[:, :, 0] = make_k0(wl).to(device=device, dtype=wl.torch_dtype)
    return k, v


def planted_sinks(wl: Workload) -> torch.Tensor:
    """[B][Hkv] bool: the groups whose queries are built aligned with k0."""
    B, Hkv = wl.batch, wl.num_kv_heads
    plan = wl.sink_plan
    out = torch.zeros((B, Hkv), dtype=torch.bool)
    for b in range(B):
        gen = _stream(wl.seed + b, _TAG_SINK)
        if plan[0] == "tiny":
            out[b, 0] = True
        elif plan[0] == "count":
            idx = torch.randperm(Hkv, generator=gen)[: int(plan[1])]
            out[b, idx] = True
        elif plan[0] == "bernoulli":
            out[b] = torch.rand(Hkv, generator=gen) < float(plan[1])
        elif plan[0] != "none":
            raise ValueError(f"unknown sink plan {plan!r}")
    return out


def make_queries(wl: Workload, sinks: torch.Tensor | None = None):
    """q [B][Hq][d] fp32 (bf16-valued for bf16 layers) and the planted mask."""
    if sinks is None:
        sinks = planted_sinks(wl)
    B, Hq, d, G = wl.batch, wl.num_q_heads, wl.head_dim, wl.group_size
    k0 = make_k0(wl)
    q = torch.empty((B, Hq, d), dtype=torch.float32)
    for b in range(B):
        noise = torch.randn((Hq, d), generator=_stream(wl.seed + b, _TAG_Q),
                            dtype=torch.float32)
        for h in range(Hq):
            g = h // G
            if sinks[b, g]:
                q[b, h] = SINK_ALIGN * k0[b, g] / k0[b, g].norm() + SINK_NOISE * noise[h]
            else:
                q[b, h] = noise[h]
    if wl.kv_dtype == "bf16":
        q = q.to(torch.bfloat16).to(torch.float32)
    return q, sinks


@dataclass
class Layer:
    wl: Workload
    q: torch.Tensor        # [B][Hq][d] fp32
    k: torch.Tensor        # [B][Hkv][T][d]
    v: torch.Tensor
    planted: torch.Tensor  # [B][Hkv] bool


def make_layer(wl: Workload, *, threads: int | None = None) -> Layer:
    k, v = make_caches(wl, threads=threads)
    q, planted = make_queries(wl)
    return Layer(wl, q, k, v, planted)


def make_layer_bulk(wl: Workload) -> Layer:
    """A layer with the same distributions as make_layer, drawn in bulk: one
    generator per tensor (seeded from wl.seed) instead of one per item and
    group, so layers with tens of thousands of items take well under a
    second.  The bits differ from make_layer's for the same workload.
    Supports the "bernoulli" and "none" sink plans."""
    B, Hq, Hkv, T, d, G = (wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.seq_len, wl.head_dim,
                           wl.group_size)
    gens = [torch.Generator().manual_seed(wl.seed * 4096 + 3000 + i) for i in range(4)]
    k = torch.randn((B, Hkv, T, d), generator=gens[0], dtype=torch.float32)
    v = torch.randn((B, Hkv, T, d), generator=gens[1], dtype=torch.float32)
    k0 = k[:, :, 0]
    k0.mul_(wl.k0_norm / k0.norm(dim=-1, keepdim=True))
    k = k.to(wl.torch_dtype)
    v = v.to(wl.torch_dtype)
    k0 = k[:, :, 0].to(torch.float32)
    plan = wl.sink_plan
    if plan[0] == "bernoulli":
        sinks = torch.rand((B, Hkv), generator=gens[2]) < float(plan[1])
    elif plan[0] == "none":
        sinks = torch.zeros((B, Hkv), dtype=torch.bool)
    else:
        raise ValueError(f"make_layer_bulk: unsupported sink plan {plan!r}")
    noise = torch.randn((B, Hq, d), generator=gens[3], dtype=torch.float32)
    unit = (k0 / k0.norm(dim=-1, keepdim=True)).repeat_interleave(G, dim=1)
    aligned = SINK_ALIGN * unit + SINK_NOISE * noise
    q = torch.where(sinks.repeat_interleave(G, dim=1)[..., None], aligned, noise)
    if wl.kv_dtype == "bf16":
        q = q.to(torch.bfloat16).to(torch.float32)
    return Layer(wl, q.contiguous(), k.contiguous(), v.contiguous(), sinks)


def rope_inv_freq(head_dim: int, base: float = 500000.0) -> torch.Tensor:
    """Rotary frequencies base^(-2i/d), fp32 [d/2] (Llama-3.1 uses base 5e5)."""
    i = torch.arange(0, head_dim, 2, dtype=torch.float64)
    return (base ** (-i / head_dim)).to(torch.float32)


def as_numpy(t: torch.Tensor):
    """Exact host copy for the oracle: bf16 widens to fp32 without rounding."""
    if t.dtype == torch.bfloat16:
        t = t.to(torch.float32)
    return t.contiguous().numpy()
