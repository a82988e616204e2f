"""The read probe (sr_stream_read) reads every byte it is given, in each of
its forms: into registers or staged through LDS, grid-strided or blocked,
default or non-temporal loads.  Each thread of the probe XORs the 16-byte
elements it loads and writes sink[w] only when its XOR equals a fixed
sentinel, so the test plants one sentinel word per workgroup in an element
that exactly one of its threads reads once (the last element of its part,
or an element of a ragged tail) and zeros everywhere else; every sink entry
is then written, and a load that was skipped or landed in the wrong LDS
slot leaves its entry 0."""
import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from kv_cache_routing_amd import _native as N
else:  # collected on CPU only to be deselected by -m "not gpu"
    N = None

SENTINEL = 0x9E3779B9
GRID = 37
ROUNDS = 3


def _layout(case, unroll):
    """(n16, sentinel element per workgroup) for a probe layout."""
    chunk = 256 * unroll                       # elements one workgroup reads per round
    if case == "strided-ragged":               # round 3 exists only for workgroup 0, 17 long
        n16 = GRID * chunk * ROUNDS + 17
        pos = [(ROUNDS - 1) * GRID * chunk + w * chunk for w in range(GRID)]
        pos[0] = ROUNDS * GRID * chunk + 5
    elif case == "blocked-exact":              # every slice is whole rounds: its last element
        per = chunk * ROUNDS
        n16 = GRID * per
        pos = [w * per + per - 1 for w in range(GRID)]
    else:                                      # blocked, the last slice 5 short: its first element
        per = chunk * ROUNDS
        n16 = GRID * per - 5
        pos = [w * per + per - 1 for w in range(GRID - 1)] + [(GRID - 1) * per]
    return n16, pos


@pytest.mark.parametrize("case", ["strided-ragged", "blocked-exact", "blocked-ragged"])
@pytest.mark.parametrize("lds", [0, 1])
@pytest.mark.parametrize("nontemporal", [0, 1])
@pytest.mark.parametrize("unroll", [1, 4, 16])
def test_every_workgroup_reads_its_whole_part(case, lds, nontemporal, unroll):
    n16, pos = _layout(case, unroll)
    words = torch.zeros(n16 * 4, dtype=torch.int32)
    for p in pos:
        words[4 * p + 1] = SENTINEL - (1 << 32)   # the same 32 bits, as int32
    buf = words.cuda()
    sink = torch.zeros(GRID, dtype=torch.int32, device="cuda")
    flags = ((case != "strided-ragged") * N.SR_READ_BLOCKED
             + nontemporal * N.SR_READ_NONTEMPORAL + lds * N.SR_READ_LDS)
    st = N.lib.sr_stream_read(ctypes.c_void_p(buf.data_ptr()), n16 * 16, GRID, unroll, flags,
                              ctypes.c_void_p(sink.data_ptr()),
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    N.check(st, "sr_stream_read")
    torch.cuda.synchronize()
    got = sink.cpu().to(torch.int64) & 0xFFFFFFFF
    assert torch.all(got == SENTINEL), got.tolist()
