"""HIP graph capture of the library's calls.

Every entry point takes its metadata (offsets, parents, slots, log lengths)
from device memory and never synchronises with the host, so a decode step
loop or a two-call fork can be captured once and replayed (the Flide page's
"연구방법을 단계별로", step 3: counts in device buffers so a captured graph
serves changing rounds). Each test replays its graph several times, with
eager work and synchronisations in between, and checks every replay bit for
bit against the same calls launched one by one and against the fp64 oracle
(max |gpu - oracle| / max |oracle| per (sequence, head) slice within 2e-3,
conv windows bitwise). The last tests drive ForkGraphRunner, the binding's
per-capacity graph runner, through rounds that fit one bucket, overflow
every bucket (split at request boundaries) and hold a request larger than
every bucket (run without a graph).
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_recurrent_gdn_amd as gdn
import oracle
from test_gpu_prefill import slice_err, window_ref, window_to_bits

pytestmark = pytest.mark.gpu

DEV = "cuda"
REPLAYS = 3
TOL = 2e-3


def host(x):
    return None if x is None else x.float().cpu().numpy()


def oracle_fork(t, cu, bcu=None, par=None, Np=None):
    """fp64 oracle of the two calls on host copies of device inputs t (a
    torch_seq_inputs dict): prefix tokens [0, Np), branch tokens after."""
    q, k, v, la, beta = (host(t[n]) for n in ("q", "k", "v", "log_alpha", "beta"))
    cw = host(t["conv_w"])
    Np = q.shape[0] if Np is None else Np
    o_p, st, win = oracle.prefill(q[:Np], k[:Np], v[:Np], la[:Np], beta[:Np], cu, conv_w=cw,
                                  qk_norm=cw is not None)
    r = dict(o_p=o_p, st=st, win=win)
    if bcu is not None:
        r["o_b"], r["st_b"], r["win_b"] = oracle.fork(
            q[Np:], k[Np:], v[Np:], la[Np:], beta[Np:], bcu, par, st, win, conv_w=cw,
            qk_norm=cw is not None)
    return r


def assert_oracle(tag, H, got, ref, cu, bcu=None):
    """got: device outputs o_p, st, win (and o_b, st_b, win_b) of the same
    names as oracle_fork's; cu / bcu: the token offsets of o_p / o_b."""
    e = dict(o_p=slice_err(host(got["o_p"]), ref["o_p"], cu, H),
             st=oracle.rel_err(host(got["st"]), ref["st"], axes=(2, 3)))
    if bcu is not None:
        e["o_b"] = slice_err(host(got["o_b"]), ref["o_b"], bcu, H)
        e["st_b"] = oracle.rel_err(host(got["st_b"]), ref["st_b"], axes=(2, 3))
    print(tag, {k: f"{v:.2e}" for k, v in e.items()}, flush=True)
    assert all(v <= TOL for v in e.values()), (tag, e)
    for w in ("win", "win_b"):
        if got.get(w) is not None and w in ref:
            assert np.array_equal(window_to_bits(got[w]), window_ref(ref[w], "bf16")), (tag, w)


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
    o_or, st_or, _ = oracle.decode(host(t["q"]), host(t["k"]), host(t["v"]), host(t["log_alpha"]),
                                   host(t["beta"]), host(base0), variant="gdn")
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
        eo = oracle.rel_err(host(go), o_or, axes=(0, 3))
        es = oracle.rel_err(host(gb), st_or, axes=(2, 3))
        print(f"replay {rep}: oracle o={eo:.2e} state={es:.2e}", flush=True)
        assert eo <= TOL and es <= TOL, (rep, eo, es)


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
    cu_h, bcu_h = t["cu_seqlens"].cpu().numpy(), t["branch_cu"].cpu().numpy()
    orc = oracle_fork(t, cu_h, bcu_h, t["branch_parent"].cpu().numpy(), Np)
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
        assert_oracle(f"replay {rep}", H, dict(o_p=g["o_p"], st=g["st"], win=g["win"],
                                               o_b=g["o_b"], st_b=g["st_b"]), orc, cu_h, bcu_h)


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
        orc = oracle_fork({n: (x[:used] if n in ("q", "k", "v", "log_alpha", "beta") else x)
                           for n, x in t.items()}, np.asarray(lay, dtype=np.int32))
        assert_oracle(str(lay), H, dict(o_p=o[:used], st=st, win=win), orc, lay)


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
        ref = oracle.fork_attention(host(t["q"]), host(t["k"]), host(t["v"]),
                                    np.asarray(lay[0], np.int32), np.asarray(lay[1], np.int32),
                                    np.asarray(lay[2], np.int32))
        segs = [(a, b) for cuv in (lay[0], lay[1]) for a, b in zip(cuv[:-1], cuv[1:]) if b > a]
        e = max(oracle.rel_err(host(o[a:b]), ref[a:b], axes=(0, 2)) for a, b in segs)
        print(lay, f"oracle {e:.2e}", flush=True)
        assert e <= TOL, (lay, e)


# ------------------------------------------------------------------ runner
RUNNER_BUCKETS = [gdn.Bucket(tokens=256, requests=2, branch_tokens=192, branches=6),
                  gdn.Bucket(tokens=512, requests=4, branch_tokens=384, branches=12)]


def _round(prefix, branch_counts, branch_lens, H, d, seed):
    """A round as flat device streams: the prefix tokens by request, then
    the branch tokens grouped by request."""
    parent = np.repeat(np.arange(len(prefix)), branch_counts).tolist()
    inp = gi.seq_inputs(prefix, branch_lens, parent, H, d, d, io="bf16", conv=True, seed=seed)
    Np = inp.Np

    def dev(name):
        bits = getattr(inp, name + "_bits")
        return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)

    q, k, v = dev("q"), dev("k"), dev("v")
    la = torch.from_numpy(inp.log_alpha).to(DEV)
    beta = torch.from_numpy(inp.beta.astype(np.float32)).to(DEV)
    pre = dict(q=q[:Np], k=k[:Np], v=v[:Np], log_alpha=la[:Np], beta=beta[:Np])
    br = dict(q=q[Np:], k=k[Np:], v=v[Np:], log_alpha=la[Np:], beta=beta[Np:])
    return inp, pre, br


def _outputs(inp, H, d):
    R, NB = len(inp.cu_seqlens) - 1, len(inp.branch_cu) - 1
    cc = H * 3 * d
    nan = float("nan")
    return dict(o=torch.full((inp.Np, H, d), nan, device=DEV),
                state=torch.full((R, H, d, d), nan, device=DEV),
                window=torch.zeros((R, 3, cc), device=DEV, dtype=torch.bfloat16),
                bo=torch.full((inp.Nb, H, d), nan, device=DEV),
                bstate=torch.full((NB, H, d, d), nan, device=DEV),
                bwindow=torch.zeros((NB, 3, cc), device=DEV, dtype=torch.bfloat16))


def _check_runner(tag, inp, out, orc, H):
    torch.cuda.synchronize()
    got = dict(o_p=out["o"], st=out["state"], win=out["window"], o_b=out["bo"],
               st_b=out["bstate"], win_b=out["bwindow"])
    assert_oracle(tag, H, got, orc, inp.cu_seqlens, inp.branch_cu)


@pytest.fixture(scope="module")
def runner():
    H, d = 2, 64
    cw = torch.from_numpy(gi.seq_inputs([1], [], [], H, d, d, conv=True, seed=77).conv_w).to(DEV)
    return gdn.ForkGraphRunner(H, d, d, RUNNER_BUCKETS, conv_w=cw, qk_l2norm=True), cw


def _with_conv(inp, cw):
    """The runner's conv weights replace the round's drawn ones (a layer's
    weights are fixed across rounds)."""
    inp.conv_w = cw.cpu().numpy()
    return inp


def _round_for_runner(cw, prefix, counts, lens, seed, H=2, d=64):
    inp, pre, br = _round(prefix, counts, lens, H, d, seed)
    inp = _with_conv(inp, cw)
    Np = inp.Np
    o_p, st, win = oracle.prefill(inp.q[:Np], inp.k[:Np], inp.v[:Np], inp.log_alpha[:Np],
                                  inp.beta[:Np], inp.cu_seqlens, conv_w=inp.conv_w, qk_norm=True)
    o_b, st_b, win_b = oracle.fork(inp.q[Np:], inp.k[Np:], inp.v[Np:], inp.log_alpha[Np:],
                                   inp.beta[Np:], inp.branch_cu, inp.branch_parent, st, win,
                                   conv_w=inp.conv_w, qk_norm=True)
    return inp, pre, br, dict(o_p=o_p, st=st, win=win, o_b=o_b, st_b=st_b, win_b=win_b)


def test_runner_rounds_in_one_bucket(runner):
    """Rounds that fit the small or the large bucket, several in a row on
    the same graphs (tail padding, empty prefixes and branches)."""
    run, cw = runner
    rounds = [([100, 130], [2, 1], [64, 9, 33]),
              ([0, 200, 7], [1, 0, 3], [1, 64, 65, 2]),
              ([64, 1, 190, 64], [3, 3, 3, 3], [20] * 12),
              ([100, 130], [2, 1], [5, 0, 70])]
    for i, (pl, bc, bl) in enumerate(rounds):
        inp, pre, br, orc = _round_for_runner(cw, pl, bc, bl, seed=100 + i)
        out = _outputs(inp, 2, 64)
        plan = run.run(pre, br, pl, bc, bl, out)
        assert len(plan) == 1 and plan[0].bucket is not None, plan
        _check_runner(f"round {i} plan {plan}", inp, out, orc, 2)


def test_runner_splits_over_capacity_round(runner):
    """A round of 6 requests (651 prefix tokens) beyond the largest bucket
    (512 tokens, 4 requests) runs as two replays split at a request
    boundary."""
    run, cw = runner
    pl = [100, 130, 64, 200, 7, 150]
    bc = [2] * 6
    bl = [40, 3, 64, 1, 9, 9, 33, 0, 5, 5, 64, 64]
    inp, pre, br, orc = _round_for_runner(cw, pl, bc, bl, seed=7)
    out = _outputs(inp, 2, 64)
    plan = run.run(pre, br, pl, bc, bl, out)
    assert plan == [gdn.Replay(0, 4, 1), gdn.Replay(4, 6, 0)], plan
    _check_runner(f"split {plan}", inp, out, orc, 2)


def test_runner_oversize_request_runs_graphless(runner):
    """A 700-token request (beyond every bucket) between two small ones:
    the small ones replay graphs, the large one runs the calls directly."""
    run, cw = runner
    pl = [30, 700, 65]
    bc = [1, 2, 1]
    bl = [64, 9, 130, 3]
    inp, pre, br, orc = _round_for_runner(cw, pl, bc, bl, seed=8)
    out = _outputs(inp, 2, 64)
    plan = run.run(pre, br, pl, bc, bl, out)
    assert plan == [gdn.Replay(0, 1, 0), gdn.Replay(1, 2, None), gdn.Replay(2, 3, 0)], plan
    _check_runner(f"oversize {plan}", inp, out, orc, 2)
