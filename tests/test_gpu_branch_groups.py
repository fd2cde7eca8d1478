"""GPU parity of the branch call when its scan runs branches in groups.

A branch call with many branches per head runs consecutive branches of one
parent in one scan workgroup, from one load of the parent's state (the
group size grows with the branch count; below about 2 x 256 / (H x d_v/32)
branches every group has one branch). These rounds have enough branches to
form groups of 3 and more, with the cases that stress that path: runs of
one parent of many lengths, parents that alternate (runs of one), a parent
that comes back after other runs, invalid parents inside the round (NaN
outputs, the neighbours unaffected), empty branches, and branches of
several chunks inside a group (whose state updates must not leak into the
next branch). Each runs with and without the branch states and windows;
outputs are held to the fp64 oracle (2e-3, windows bitwise).
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_recurrent_gdn_amd as gdn
import oracle
from test_gpu_prefill import dev_io, f32, i32, slice_err, window_ref, window_to_bits

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 2e-3


def layout():
    prefix = [70, 0, 130, 64, 5, 200]
    runs = [[0] * 9, [1] * 3, [2] * 17, [3], [4, 3, 4, 3], [-1] * 4, [5] * 20, [2] * 6, [7] * 2]
    parent = [p for r in runs for p in r]
    cycle = [1, 5, 0, 64, 65, 30, 2, 130, 7]
    branches = [cycle[i % len(cycle)] for i in range(len(parent))]
    return prefix, branches, parent


def run(inp, variant, states):
    H, dk, dv, Np, Nb = inp.H, inp.dk, inp.dv, inp.Np, inp.Nb
    R, NB = len(inp.cu_seqlens) - 1, len(inp.branch_cu) - 1
    cc = H * (2 * dk + dv)
    q, k, v = (dev_io(getattr(inp, n), getattr(inp, n + "_bits")) for n in "qkv")
    la = f32(inp.log_alpha)
    beta = None if variant == "rwkv6" else f32(inp.beta)
    conv_w = f32(inp.conv_w)
    st = torch.empty((R, H, dk, dv), device=DEV)
    win = torch.zeros((R, 3, cc), device=DEV, dtype=torch.bfloat16)
    gdn.gdn_prefill_shared(q[:Np], k[:Np], v[:Np], la[:Np], None if beta is None else beta[:Np],
                           i32(inp.cu_seqlens), st, conv_w=conv_w, qk_l2norm=True,
                           final_window=win, variant=variant)
    o_b = torch.full((Nb, H, dv), float("nan"), device=DEV)
    st_b = torch.full((NB, H, dk, dv), float("nan"), device=DEV) if states else None
    win_b = torch.zeros((NB, 3, cc), device=DEV, dtype=torch.bfloat16) if states else None
    gdn.gdn_fork_branches(q[Np:], k[Np:], v[Np:], la[Np:], None if beta is None else beta[Np:],
                          i32(inp.branch_cu), i32(inp.branch_parent), st, o_b,
                          parent_window=win, branch_state=st_b, branch_window=win_b,
                          conv_w=conv_w, qk_l2norm=True, variant=variant)
    torch.cuda.synchronize()
    return o_b.cpu().numpy(), None if st_b is None else st_b.cpu().numpy(), win_b


def reference(inp, variant):
    """Oracle outputs of the valid-parent branches, as a reduced round."""
    Np = inp.Np
    beta = inp.beta
    o_p, st, win = oracle.prefill(inp.q[:Np], inp.k[:Np], inp.v[:Np], inp.log_alpha[:Np],
                                  beta[:Np], inp.cu_seqlens, conv_w=inp.conv_w, qk_norm=True,
                                  variant=variant)
    R = len(inp.cu_seqlens) - 1
    bcu, par = inp.branch_cu, inp.branch_parent
    valid = [b for b in range(len(par)) if 0 <= par[b] < R]
    rows = np.concatenate([np.arange(Np + bcu[b], Np + bcu[b + 1]) for b in valid])
    lens = [bcu[b + 1] - bcu[b] for b in valid]
    vcu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o_b, st_b, win_b = oracle.fork(inp.q[rows], inp.k[rows], inp.v[rows], inp.log_alpha[rows],
                                   beta[rows], vcu, par[valid], st, win, conv_w=inp.conv_w,
                                   qk_norm=True, variant=variant)
    return valid, vcu, o_b, st_b, win_b


@pytest.mark.parametrize("variant", ["gdn", "kda"])
@pytest.mark.parametrize("states", [False, True])
def test_grouped_branches(variant, states):
    prefix, branches, parent = layout()
    H, d = 4, 128
    # groups form: more branches than about 2 x 256 / (H x d_v / 32) = 32
    assert len(branches) > 2 * 256 // (H * d // 32)
    inp = gi.seq_inputs(prefix, branches, parent, H, d, d, io="bf16", conv=True,
                        per_key=variant != "gdn", seed=5 + states)
    o_b, st_b, win_b = run(inp, variant, states)
    valid, vcu, o_r, st_r, win_r = reference(inp, variant)
    bcu = inp.branch_cu
    # every valid branch's o against the oracle, per (branch, head)
    g_rows = np.concatenate([np.arange(bcu[b], bcu[b + 1]) for b in valid])
    e_o = slice_err(o_b[g_rows], o_r, vcu, H)
    e_s = oracle.rel_err(st_b[valid], st_r, axes=(2, 3)) if states else 0.0
    print(f"{variant} states={states}: o {e_o:.2e} state {e_s:.2e}", flush=True)
    assert e_o <= TOL and e_s <= TOL
    if states:
        wb = window_to_bits(win_b)
        assert np.array_equal(wb[valid], window_ref(win_r, "bf16"))
    # invalid parents: NaN outputs (and states), and only there
    for b in range(len(parent)):
        rows = slice(bcu[b], bcu[b + 1])
        if b in valid:
            assert not np.isnan(o_b[rows]).any(), b
        else:
            assert np.isnan(o_b[rows]).all(), b
            if states:
                assert np.isnan(st_b[b]).all(), b


@pytest.mark.parametrize("variant", ["gdn", "kda"])
def test_outputs_do_not_depend_on_branch_states(variant):
    """Asking for the branch states only adds the last update and its
    write-out: the outputs o are bit for bit the same either way."""
    prefix, branches, parent = layout()
    inp = gi.seq_inputs(prefix, branches, parent, 4, 128, 128, io="bf16", conv=True,
                        per_key=variant != "gdn", seed=9)
    o_without, _, _ = run(inp, variant, False)
    o_with, _, _ = run(inp, variant, True)
    assert np.array_equal(o_without, o_with, equal_nan=True)


@pytest.mark.parametrize("variant,states", [("gdn", True), ("kda", False)])
def test_more_groups_than_resident_workgroups(variant, states):
    """Parents that alternate make every branch its own group: 80 groups x
    4 heads x 4 value tiles = 1,280 scan units against a grid of 512, so a
    workgroup runs units b, b + 512 and b + 1024 in turn. Most branches
    pass one chunk (the scan's), the rest take the one-chunk kernel."""
    H, d = 4, 128
    prefix = [70, 130]
    parent = [i % 2 for i in range(80)]
    cycle = [65, 100, 3, 130, 64, 0, 70]
    branches = [cycle[i % len(cycle)] for i in range(len(parent))]
    target = -(-2 * 256 // (H * d // 32))  # groups giving one resident round
    G = -(-len(parent) // target)
    assert G > 1 and len(parent) * H * (d // 32) > 2 * 256  # groups of one branch each
    inp = gi.seq_inputs(prefix, branches, parent, H, d, d, io="bf16", conv=True,
                        per_key=variant != "gdn", seed=11)
    o_b, st_b, win_b = run(inp, variant, states)
    valid, vcu, o_r, st_r, win_r = reference(inp, variant)
    assert valid == list(range(len(parent)))
    e_o = slice_err(o_b, o_r, vcu, H)
    e_s = oracle.rel_err(st_b, st_r, axes=(2, 3)) if states else 0.0
    print(f"{variant} states={states}: o {e_o:.2e} state {e_s:.2e}", flush=True)
    assert e_o <= TOL and e_s <= TOL
    if states:
        assert np.array_equal(window_to_bits(win_b), window_ref(win_r, "bf16"))
