"""HIP graph capture of the library's calls.

Every entry point takes its metadata (offsets, parents, slots, log lengths)
from device memory and never synchronises with the host, so a decode step
loop or a two-call fork can be captured once and replayed (the Flide page's
"연구방법을 단계별로", step 3: counts in device buffers so a captured graph
serves changing rounds). Each test replays its graph several times, with
eager work and synchronisations in between, and checks every replay bit for
bit against the same calls launched one by one.
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_recurrent_gdn_amd as gdn

pytestmark = pytest.mark.gpu

DEV = "cuda"
REPLAYS = 3


def _decode_setup(B=16, H=4, d=128, T=12, M=4, seed=0):
    t = gi.torch_decode_inputs(B, H, d, d, T, seed=seed)
    base0 = t["state0"].clone()
    logs0 = dict(log_u=torch.zeros((B, H, M, d), device=DEV),
                 log_k=torch.zeros((B, H, M, d), device=DEV, dtype=torch.bfloat16),
                 log_lam=torch.zeros((B, H, M), device=DEV),
                 log_len=torch.zeros((B, H), device=DEV, dtype=torch.int32))
    return t, base0, logs0


def _decode_steps(t, base, logs, o, M):
    for s in range(t["q"].shape[0]):
        gdn.deltalog_append_decode(t["q"][s], t["k"][s], t["v"][s], t["log_alpha"][s],
                                   t["beta"][s], base, logs["log_u"], logs["log_k"],
                                   logs["log_lam"], logs["log_len"], o[s], merge_at=M)
    gdn.deltalog_merge(base, logs["log_u"], logs["log_k"], logs["log_lam"], logs["log_len"],
                       min_len=1)


def test_deferred_decode_loop_replays_bitwise():
    """12 deferred steps (M=4: appends and fused merges) plus the final
    flush, captured as one graph."""
    M = 4
    t, base0, logs0 = _decode_setup(M=M)
    T = t["q"].shape[0]
    B, H, d = t["q"].shape[1], t["q"].shape[2], t["v"].shape[-1]
    # eager reference
    base, logs = base0.clone(), {k: v.clone() for k, v in logs0.items()}
    o_ref = torch.empty((T, B, H, d), device=DEV)
    _decode_steps(t, base, logs, o_ref, M)
    torch.cuda.synchronize()
    base_ref = base.clone()
    # capture on static buffers
    gb, gl = base0.clone(), {k: v.clone() for k, v in logs0.items()}
    go = torch.empty((T, B, H, d), device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        _decode_steps(t, gb, gl, go, M)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _decode_steps(t, gb, gl, go, M)
    for rep in range(REPLAYS):
        # eager work between replays: reset the state the graph reads
        gb.copy_(base0)
        for k in gl:
            gl[k].copy_(logs0[k])
        go.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(go, o_ref), f"replay {rep}: o differs"
        assert torch.equal(gb, base_ref), f"replay {rep}: base differs"
        assert (gl["log_len"] == 0).all()


def test_two_call_fork_replays_bitwise():
    """gdn_prefill_shared + gdn_fork_branches (conv, ragged lengths)
    captured together; the workspace is allocated outside the capture."""
    prefix = [130, 64, 7]
    branches = [64, 9, 33, 1]
    parent = [0, 0, 1, 2]
    H, d = 2, 128
    t = gi.torch_seq_inputs(prefix, branches, parent, H, d, d, conv=True, seed=4)
    Np, Nb, R, NB = t["Np"], t["Nb"], len(prefix), len(branches)
    cc = H * 3 * d
    ws = torch.empty(gdn.prefill_workspace_bytes(max(Np, Nb), max(R, NB), H, d, d),
                     dtype=torch.uint8, device=DEV)

    def bufs():
        return dict(st=torch.empty((R, H, d, d), device=DEV),
                    win=torch.empty((R, 3, cc), device=DEV, dtype=torch.bfloat16),
                    o_p=torch.empty((Np, H, d), device=DEV),
                    o_b=torch.empty((Nb, H, d), device=DEV),
                    st_b=torch.empty((NB, H, d, d), device=DEV))

    def run(b):
        gdn.gdn_prefill_shared(t["q"][:Np], t["k"][:Np], t["v"][:Np], t["log_alpha"][:Np],
                               t["beta"][:Np], t["cu_seqlens"], b["st"], o=b["o_p"],
                               conv_w=t["conv_w"], qk_l2norm=True, final_window=b["win"],
                               workspace=ws)
        gdn.gdn_fork_branches(t["q"][Np:], t["k"][Np:], t["v"][Np:], t["log_alpha"][Np:],
                              t["beta"][Np:], t["branch_cu"], t["branch_parent"], b["st"],
                              b["o_b"], parent_window=b["win"], branch_state=b["st_b"],
                              conv_w=t["conv_w"], qk_l2norm=True, workspace=ws)

    ref = bufs()
    run(ref)
    torch.cuda.synchronize()
    g = bufs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(g)
    for rep in range(REPLAYS):
        for x in g.values():
            x.fill_(float("nan")) if x.dtype.is_floating_point else x.zero_()
        ws.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name in ref:
            assert torch.equal(g[name], ref[name]), f"replay {rep}: {name} differs"


def test_fixed_capacity_graph_serves_changing_rounds():
    """One graph captured for a stream capacity (4 sequences, 400 tokens)
    replays rounds with other layouts written into the device offsets in
    place: shorter streams (the rest of the capacity is tail padding that
    no sequence covers) and empty sequences. Each replay equals an eager
    call with the same offsets."""
    H, d, R, N = 2, 64, 4, 400
    t = gi.torch_seq_inputs([N], [], [], H, d, d, conv=True, seed=9)  # one stream of N tokens
    cc = H * 3 * d
    cu = torch.zeros(R + 1, dtype=torch.int32, device=DEV)
    ws = torch.empty(gdn.prefill_workspace_bytes(N, R, H, d, d), dtype=torch.uint8, device=DEV)
    st = torch.empty((R, H, d, d), device=DEV)
    win = torch.empty((R, 3, cc), device=DEV, dtype=torch.bfloat16)
    o = torch.empty((N, H, d), device=DEV)

    def run(cu_t, st_t, win_t, o_t):
        gdn.gdn_prefill_shared(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], cu_t, st_t,
                               o=o_t, conv_w=t["conv_w"], qk_l2norm=True, final_window=win_t,
                               workspace=ws)

    rounds = [[0, 100, 228, 300, 400], [0, 0, 64, 64, 65], [0, 37, 37, 200, 333]]
    cu.copy_(torch.tensor(rounds[0], dtype=torch.int32))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(cu, st, win, o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(cu, st, win, o)
    for lay in rounds * 2:
        cu.copy_(torch.tensor(lay, dtype=torch.int32))
        o.fill_(float("nan"))
        st.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        cu_ref = torch.tensor(lay, dtype=torch.int32, device=DEV)
        st_r = torch.empty_like(st)
        win_r = torch.empty_like(win)
        o_r = torch.full_like(o, float("nan"))
        run(cu_ref, st_r, win_r, o_r)
        torch.cuda.synchronize()
        used = lay[-1]
        assert torch.equal(st, st_r), lay
        assert torch.equal(win, win_r), lay
        assert torch.equal(o[:used], o_r[:used]), lay


def test_fork_attention_graph_serves_changing_rounds():
    """Fork attention captured once for a stream capacity (2 trunks, 3
    branches, 600 tokens) replays rounds whose trunk and branch offsets and
    parents are rewritten in place (shorter streams, empty segments, moved
    parents); each replay equals an eager call with the same metadata."""
    H, Hkv, d, N = 4, 2, 128, 600
    t = gi.torch_attention_inputs([N], [], [], H=H, Hkv=Hkv, d=d, seed=21)
    cu = torch.zeros(3, dtype=torch.int32, device=DEV)
    bcu = torch.zeros(4, dtype=torch.int32, device=DEV)
    par = torch.zeros(3, dtype=torch.int32, device=DEV)
    ws = torch.empty(gdn.fork_attention_workspace_bytes(2, 3), dtype=torch.uint8, device=DEV)
    o = torch.empty((N, H, d), device=DEV)

    def run(cu_t, bcu_t, par_t, o_t):
        gdn.gdn_fork_attention(t["q"], t["k"], t["v"], cu_t, o_t, bcu_t, par_t, workspace=ws)

    rounds = [([0, 300, 450], [450, 500, 564, 600], [0, 1, 0]),
              ([0, 0, 200], [200, 200, 264, 265], [1, 0, 1]),
              ([0, 129, 130], [130, 194, 258, 400], [1, 1, 0])]

    def load(lay):
        cu.copy_(torch.tensor(lay[0], dtype=torch.int32))
        bcu.copy_(torch.tensor(lay[1], dtype=torch.int32))
        par.copy_(torch.tensor(lay[2], dtype=torch.int32))

    load(rounds[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(cu, bcu, par, o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(cu, bcu, par, o)
    for lay in rounds * 2:
        load(lay)
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_r = torch.full_like(o, float("nan"))
        run(torch.tensor(lay[0], dtype=torch.int32, device=DEV),
            torch.tensor(lay[1], dtype=torch.int32, device=DEV),
            torch.tensor(lay[2], dtype=torch.int32, device=DEV), o_r)
        torch.cuda.synchronize()
        used = lay[1][-1]
        assert torch.equal(o[:used], o_r[:used]), lay
        assert not torch.isnan(o[:used]).any(), lay
