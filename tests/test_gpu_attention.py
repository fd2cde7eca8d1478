"""Fork attention on the GPU against the fp64 oracle.

Small ragged streams are checked whole (every trunk and branch, every
head); the full-size fork workload (8 requests x 8192-token trunks, 20
branches of 64 tokens each, H=16, d=128) runs whole on the GPU in the
launch configuration the bench times and is checked on sampled branches
and trunk tiles, the oracle computing just those queries.
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_recurrent_gdn_amd as gdn
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 2e-3


def host64(x):
    return x.float().cpu().numpy().astype(np.float64)


def segments(cu, bcu):
    segs = [(int(cu[r]), int(cu[r + 1])) for r in range(len(cu) - 1)]
    segs += [(int(bcu[b]), int(bcu[b + 1])) for b in range(len(bcu) - 1)]
    return [s for s in segs if s[1] > s[0]]


def worst_err(g, ref, segs):
    """max over (segment, head) of max|g - ref| / max|ref|."""
    return max((oracle.rel_err(g[a:b], ref[a:b], axes=(0, 2)) for a, b in segs), default=0.0)


def bf16_within_rounding(g, ref, slack):
    """g (bf16 values) is a rounding of a value within `slack` of ref:
    |g - ref| <= ulp_bf16(ref) / 2 + slack."""
    e = np.floor(np.log2(np.maximum(np.abs(ref), 1e-30)))
    ulp = np.exp2(e - 7)
    return bool(np.all(np.abs(g - ref) <= ulp / 2 + slack))


def run(t, o_dtype=torch.float32, trunk_queries=True, fill=None, scale=None):
    N, H, d = t["q"].shape
    o = (torch.full((N, H, d), fill, device=DEV, dtype=o_dtype) if fill is not None
         else torch.zeros((N, H, d), device=DEV, dtype=o_dtype))
    gdn.gdn_fork_attention(t["q"], t["k"], t["v"], t["cu"], o, t["bcu"], t["bpar"], scale=scale,
                           trunk_queries=trunk_queries)
    torch.cuda.synchronize()
    return o


def ref(t, trunk_queries=True, fill=None, scale=None):
    o0 = None if fill is None else np.full(t["q"].shape, fill)
    return oracle.fork_attention(host64(t["q"]), host64(t["k"]), host64(t["v"]),
                                 t["cu"].cpu().numpy(), t["bcu"].cpu().numpy(),
                                 t["bpar"].cpu().numpy(), scale=scale,
                                 trunk_queries=trunk_queries, o=o0)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hkv", [4, 2, 1])
def test_ragged_stream(d, Hkv):
    """Trunks of 1, 70 and 200 tokens, branches of 0..130 tokens (partial,
    exact and multi-tile), branches stored before the trunks."""
    t = gi.torch_attention_inputs([1, 70, 200], [0, 1, 63, 64, 65, 130], [2, 0, 1, 2, 2, 1],
                                  H=4, Hkv=Hkv, d=d, order="branches_first", seed=d + Hkv)
    g = host64(run(t))
    r = ref(t)
    segs = segments(t["cu"].cpu(), t["bcu"].cpu())
    e = worst_err(g, r, segs)
    print(f"d={d} Hkv={Hkv}: {e:.2e}", flush=True)
    assert e <= TOL


@pytest.mark.parametrize("d,Hkv", [(128, 2), (64, 4)])
def test_branch_pairs(d, Hkv):
    """Consecutive branches 2i, 2i+1 of one request, each at most 64 tokens,
    share a tile: pairs with a full / one-token / empty member, pairs over
    an empty trunk (with a 64-token first member, the second member's whole
    first key block is invisible to it),
    a pair split because a member is longer than 64, an unpaired last
    branch, and branches of different requests side by side."""
    trunks = [0, 70, 130]
    blen = [64, 1, 5, 64, 0, 33, 40, 0, 64, 65, 3, 9, 64, 10, 17]
    par = [1, 1, 0, 0, 2, 2, 2, 2, 1, 1, 0, 2, 0, 0, 0]
    t = gi.torch_attention_inputs(trunks, blen, par, H=4, Hkv=Hkv, d=d, seed=5 + d)
    g = host64(run(t))
    r = ref(t)
    segs = segments(t["cu"].cpu(), t["bcu"].cpu())
    e = worst_err(g, r, segs)
    print(f"pairs d={d} Hkv={Hkv}: {e:.2e}", flush=True)
    assert e <= TOL


def test_bf16_output_is_a_rounding_of_the_exact_result():
    t = gi.torch_attention_inputs([130, 7], [64, 3], [0, 1], H=4, Hkv=2, d=128, seed=11)
    g = host64(run(t, o_dtype=torch.bfloat16))
    r = ref(t)
    segs = segments(t["cu"].cpu(), t["bcu"].cpu())
    for a, b in segs:
        assert bf16_within_rounding(g[a:b], r[a:b], 1e-5 * np.abs(r[a:b]).max())


def test_branch_round_against_earlier_trunks_and_scale():
    """trunk_queries=0 leaves trunk rows untouched; branch rows match the
    oracle; a non-default scale."""
    t = gi.torch_attention_inputs([100, 33], [5, 64, 17], [1, 0, 0], H=2, Hkv=2, d=64, seed=3)
    g = host64(run(t, trunk_queries=False, fill=7.0, scale=0.05))
    r = ref(t, trunk_queries=False, fill=7.0, scale=0.05)
    cu = t["cu"].cpu().numpy()
    assert np.all(g[cu[0]:cu[-1]] == 7.0)
    segs = segments(np.zeros(1, dtype=np.int64), t["bcu"].cpu())
    assert worst_err(g, r, segs) <= TOL


def test_invalid_parent_and_empty_request():
    """A branch whose parent is out of range gets NaN rows; a branch of an
    empty request attends only to itself; nothing else is disturbed."""
    t = gi.torch_attention_inputs([50, 0], [10, 6, 4], [0, 1, 5], H=2, Hkv=1, d=128, seed=4)
    g = host64(run(t, fill=3.0))
    bcu = t["bcu"].cpu().numpy()
    assert np.all(np.isnan(g[bcu[2]:bcu[3]]))
    t_ok = dict(t, bpar=torch.tensor([0, 1, 0], dtype=torch.int32, device=DEV))
    r = ref(t_ok)
    segs = segments(t["cu"].cpu(), bcu[:3])
    assert worst_err(g, r, segs) <= TOL


def test_repeat_is_bitwise_and_order_of_segments_is_irrelevant():
    """Two runs give identical bits; the same requests and branches laid
    out in a different stream order give identical bits too."""
    a = gi.torch_attention_inputs([90, 40], [20, 64, 5], [1, 0, 1], H=4, Hkv=4, d=128,
                                  order="trunks_first", seed=8)
    b = gi.torch_attention_inputs([90, 40], [20, 64, 5], [1, 0, 1], H=4, Hkv=4, d=128,
                                  order="branches_first", seed=8)
    oa1, oa2, ob = run(a), run(a), run(b)
    assert torch.equal(oa1, oa2)
    for sa, sb in zip(segments(a["cu"].cpu(), a["bcu"].cpu()),
                      segments(b["cu"].cpu(), b["bcu"].cpu())):
        assert torch.equal(oa1[sa[0]:sa[1]], ob[sb[0]:sb[1]])


def test_full_size_fork_round_sampled():
    """8 x 8192-token trunks + 160 branches of 64 tokens, H=16, d=128, bf16,
    one call as the bench times it; sampled branches and trunk tiles
    (including the last tile of a trunk) against the oracle, all heads."""
    w = gi.WORKLOADS["fork_prefill"]
    R, H, d = w["R"], w["H"], w["d"]
    pl, bl, par = gi.fork_layout(R, w["prefix"], w["branches_per_req"], w["branch_len"])
    t = gi.torch_attention_inputs(pl, bl, par, H=H, Hkv=H, d=d, seed=0)
    g = run(t)
    cu, bcu = t["cu"].cpu().numpy(), t["bcu"].cpu().numpy()
    worst = 0.0
    # branches: the oracle over (parent trunk as keys only, the branch)
    for b in (0, 37, 159):
        r = par[b]
        rows = np.r_[cu[r]:cu[r + 1], bcu[b]:bcu[b + 1]]
        sub = {n: t[n][torch.from_numpy(rows).to(DEV)] for n in ("q", "k", "v")}
        P = cu[r + 1] - cu[r]
        ro = oracle.fork_attention(host64(sub["q"]), host64(sub["k"]), host64(sub["v"]),
                                   [0, P], [P, len(rows)], [0], trunk_queries=False)
        worst = max(worst, oracle.rel_err(host64(g[bcu[b]:bcu[b + 1]]), ro[P:], axes=(0, 2)))
    # trunk tiles: tokens [s, e) of request r see [0, p]; the oracle treats
    # [0, s) as keys only and [s, e) as a branch
    for r, (s, e) in ((0, (0, 64)), (3, (4000, 4064)), (7, (8128, 8192))):
        rows = np.arange(cu[r], cu[r] + e)
        sub = {n: t[n][torch.from_numpy(rows).to(DEV)] for n in ("q", "k", "v")}
        ro = oracle.fork_attention(host64(sub["q"]), host64(sub["k"]), host64(sub["v"]),
                                   [0, s], [s, e], [0], trunk_queries=False)
        worst = max(worst, oracle.rel_err(host64(g[cu[r] + s:cu[r] + e]), ro[s:e],
                                          axes=(0, 2)))
    print(f"full-size fork attention, sampled: {worst:.2e}", flush=True)
    assert worst <= TOL
