"""The allocation-free fork attention (gdn_fork_attention_noalloc, whose tile
table is the library's static per-GPU array) against the workspace entry
point gdn_fork_attention, through the C ABI: two calls in a row on one
stream, the second over a smaller stream with fewer segments, so the second
call reads a table the first one left behind. Outputs must be bit-identical
(the same kernels run) and within the oracle bar; the static table's size
limit is an error before any launch."""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_recurrent_gdn_amd as gdn
import oracle
from linear_attention_recurrent_gdn_amd import _lib

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 2e-3


def host64(x):
    return x.float().cpu().numpy().astype(np.float64)


def both(t):
    N, H, d = t["q"].shape
    o_ws = torch.zeros((N, H, d), device=DEV)
    o_na = torch.full((N, H, d), 7.0, device=DEV)
    gdn.gdn_fork_attention(t["q"], t["k"], t["v"], t["cu"], o_ws, t["bcu"], t["bpar"])
    gdn.gdn_fork_attention_noalloc(t["q"], t["k"], t["v"], t["cu"], o_na, t["bcu"], t["bpar"])
    torch.cuda.synchronize()
    return o_ws, o_na


def oracle_err(t, o):
    ref = oracle.fork_attention(host64(t["q"]), host64(t["k"]), host64(t["v"]),
                                t["cu"].cpu().numpy(), t["bcu"].cpu().numpy(),
                                t["bpar"].cpu().numpy())
    cu, bcu = t["cu"].cpu().numpy(), t["bcu"].cpu().numpy()
    segs = [(int(cu[r]), int(cu[r + 1])) for r in range(len(cu) - 1)]
    segs += [(int(bcu[b]), int(bcu[b + 1])) for b in range(len(bcu) - 1)]
    g = o.cpu().numpy()
    return max(oracle.rel_err(g[a:b], ref[a:b], axes=(0, 2)) for a, b in segs if b > a)


def test_noalloc_matches_workspace_entry_point_twice_shrinking():
    print("noalloc call 1: 3 trunks, 6 branches, H=4, Hkv=2, d=128", flush=True)
    big = gi.torch_attention_inputs([40, 130, 200], [0, 1, 63, 64, 65, 130], [2, 0, 1, 2, 2, 1],
                                    H=4, Hkv=2, d=128, device=DEV, seed=21)
    a_ws, a_na = both(big)
    assert torch.equal(a_ws, a_na)
    e1 = oracle_err(big, a_na)
    print(f"call 1 rel err {e1:.3e}", flush=True)
    assert e1 <= TOL
    print("noalloc call 2: 1 trunk, 2 branches (smaller)", flush=True)
    small = gi.torch_attention_inputs([70], [5, 64], [0, 0], H=4, Hkv=2, d=128, device=DEV,
                                      seed=22)
    b_ws, b_na = both(small)
    assert torch.equal(b_ws, b_na)
    e2 = oracle_err(small, b_na)
    print(f"call 2 rel err {e2:.3e}", flush=True)
    assert e2 <= TOL


def test_noalloc_rejects_more_segments_than_its_table():
    t = gi.torch_attention_inputs([8], [], [], H=2, Hkv=2, d=64, device=DEV, seed=23)
    n = _lib.FORK_ATTENTION_NOALLOC_MAX_SEGMENTS + 1
    cu = torch.zeros(n + 1, dtype=torch.int32, device=DEV)   # n empty trunks
    o = torch.zeros_like(t["q"], dtype=torch.float32)
    with pytest.raises(gdn.GDNError) as ei:
        gdn.gdn_fork_attention_noalloc(t["q"], t["k"], t["v"], cu, o)
    assert ei.value.status == _lib.GDN_ERR_WORKSPACE
