"""Host-side argument checks of the Python binding (CPU tensors, no device
work): every array the kernels index from the cache shape is checked for
shape, dtype and contiguity, and for living on the device, before anything
reaches the library."""
import pytest
import torch

import kv_cache_routing_amd as sr

B, Hq, Hkv, T, d = 2, 8, 4, 64, 128


def layer():
    k = torch.zeros((B, Hkv, T, d), dtype=torch.bfloat16)
    return (torch.zeros((B, Hq, d)), k, torch.zeros_like(k),
            torch.zeros((B, Hkv, d)), torch.zeros((B, Hkv, d)))


def routing(**bad):
    parts = dict(scores=torch.zeros((B, Hq)), mask=torch.zeros((B, Hkv), dtype=torch.uint8),
                 work_list=torch.zeros(B * Hkv, dtype=torch.int32),
                 n_active=torch.zeros(1, dtype=torch.int32))
    parts.update(bad)
    return sr.Routing(**parts)


@pytest.fixture
def shapes_only(monkeypatch):
    """Each array's shape check is reached with host tensors in the earlier
    arguments: the device check (which those would fail first) is switched
    off.  Every call in these tests fails a shape check, so nothing reaches
    the library."""
    monkeypatch.setattr(sr, "_on_device", lambda t, name: None)


def test_well_formed_cpu_arguments_reach_the_device_check():
    q, k, v, k0, v0 = layer()
    with pytest.raises(ValueError, match="device tensors"):
        sr.dense_decode(q, k, v)
    with pytest.raises(ValueError, match="device tensors"):
        sr.route_decode(q, k, v, k0, v0, routing=routing())
    with pytest.raises(ValueError, match="device tensors"):
        sr.route(q, k0, out=routing())
    kn = torch.zeros((B, Hkv, d))
    with pytest.raises(ValueError, match="device tensors"):
        sr.rope_append(q, kn, kn, k, v, 0, torch.zeros(d // 2))
    # the first host array named
    with pytest.raises(ValueError, match="k0 is a host tensor"):
        sr.route_decode(q, k, v, k0, v0)
    with pytest.raises(ValueError, match="v0 is a host tensor"):
        sr.decode_attn(q, k, v, v0, torch.zeros(B * Hkv, dtype=torch.int32),
                       torch.zeros(1, dtype=torch.int32))


@pytest.mark.parametrize("bad_q", [torch.zeros((B + 1, Hq, d)), torch.zeros((B, Hq, 64)),
                                   torch.zeros((B, Hq, d), dtype=torch.float64),
                                   torch.zeros((B, d, Hq)).transpose(1, 2)])
def test_query_must_match_the_cache(bad_q):
    _, k, v, k0, v0 = layer()
    with pytest.raises(ValueError, match="q "):
        sr.dense_decode(bad_q, k, v)
    with pytest.raises(ValueError, match="q "):
        sr.route_decode(bad_q, k, v, k0, v0)


def test_output_and_sink_rows_are_checked(shapes_only):
    q, k, v, k0, v0 = layer()
    wl = torch.zeros(B * Hkv, dtype=torch.int32)
    na = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError, match="out "):
        sr.dense_decode(q, k, v, out=torch.zeros((B, Hq, d - 1)))
    with pytest.raises(ValueError, match="v0 "):
        sr.decode_attn(q, k, v, torch.zeros((B, Hkv + 1, d)), wl, na)
    with pytest.raises(ValueError, match="work_list "):
        sr.decode_attn(q, k, v, v0, wl[:-1], na)
    with pytest.raises(ValueError, match="n_active "):
        sr.decode_attn(q, k, v, v0, wl, torch.zeros(1, dtype=torch.int64))
    with pytest.raises(ValueError, match="k0 "):
        sr.route_decode(q, k, v, k0[:, :, :64], v0)


@pytest.mark.parametrize("field,bad", [("scores", torch.zeros((B, Hq + 1))),
                                       ("mask", torch.zeros((B, Hkv), dtype=torch.int32)),
                                       ("work_list", torch.zeros(B * Hkv + 1, dtype=torch.int32)),
                                       ("n_active", torch.zeros((), dtype=torch.int32))])
def test_routing_outputs_are_checked(field, bad, shapes_only):
    q, k, v, k0, v0 = layer()
    with pytest.raises(ValueError, match=f"{field} "):
        sr.route(q, k0, out=routing(**{field: bad}))
    with pytest.raises(ValueError, match=f"{field} "):
        sr.route_decode(q, k, v, k0, v0, routing=routing(**{field: bad}))


def test_route_query_and_key_must_agree():
    q, _, _, k0, _ = layer()
    with pytest.raises(ValueError, match="disagree"):
        sr.route(q[:, :, :64], k0)
    with pytest.raises(ValueError, match="disagree"):
        sr.route(q[:1], k0)


def test_rope_append_arguments_are_checked(shapes_only):
    q, k, v, _, _ = layer()
    kn = torch.zeros((B, Hkv, d))
    f = torch.zeros(d // 2)
    with pytest.raises(ValueError, match="inv_freq "):
        sr.rope_append(q, kn, kn, k, v, 0, torch.zeros(d))
    with pytest.raises(ValueError, match="k_new "):
        sr.rope_append(q, torch.zeros((B, Hq, d)), kn, k, v, 0, f)
    with pytest.raises(ValueError, match="q_out "):
        sr.rope_append(q, kn, kn, k, v, 0, f, q_out=torch.zeros((B, Hq, d), dtype=torch.float16))
