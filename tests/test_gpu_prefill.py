"""GPU parity of the two-call fork (shared-context prefill, then branches
from the saved states) against the fp64 oracle.

Metric as for decode: max |gpu - oracle| / max |oracle| per (sequence,
head) slice, over all its tokens x d_v for o and over d_k x d_v for the
final state; conv windows are exact copies and compare bitwise.
"""

import numpy as np
import pytest
import torch

import _parity
import gdn_inputs as gi
import linear_attention_recurrent_gdn_amd as gdn
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 2e-3
TOL_F32 = 1e-4
TOL_C1 = 1e-5  # the tiny fp32 fork workload


def dev_io(vals, bits):
    if bits is not None:
        return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(vals)).to(DEV)


def f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(DEV)


def slice_err(x, ref, cu, H):
    """max over (sequence, head) slices of the o metric (token ranges cu)."""
    worst = 0.0
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b > a:
            worst = max(worst, oracle.rel_err(x[a:b], ref[a:b], axes=(0, 2)))
    return worst


def window_to_bits(win_t):
    if win_t.dtype == torch.bfloat16:
        return win_t.cpu().view(torch.int16).numpy().view(np.uint16)
    return win_t.cpu().numpy()


def window_ref(win64, io):
    if io == "bf16":
        return gi.bf16_round(win64.astype(np.float32))[0]
    return win64.astype(np.float32)


def run_fork(inp, *, init_state=None, init_window=None, o_dtype=torch.float32, variant="gdn"):
    """Both calls on the GPU; returns host copies of every output."""
    H, dk, dv, Np = inp.H, inp.dk, inp.dv, inp.Np
    R, NB = len(inp.cu_seqlens) - 1, len(inp.branch_cu) - 1
    cc = H * (2 * dk + dv)
    io_dtype = torch.bfloat16 if inp.io == "bf16" else torch.float32
    q, k, v = (dev_io(getattr(inp, n), getattr(inp, n + "_bits")) for n in "qkv")
    la = f32(inp.log_alpha)
    beta = None if variant == "rwkv6" else f32(inp.beta)  # beta may be NULL for RWKV6
    pick = lambda x, sl: None if x is None else x[sl]  # noqa: E731
    conv_w = None if inp.conv_w is None else f32(inp.conv_w)
    o_p = torch.full((Np, H, dv), float("nan"), device=DEV, dtype=o_dtype)
    st = torch.full((R, H, dk, dv), float("nan"), device=DEV)
    win = torch.zeros((R, 3, cc), device=DEV, dtype=io_dtype)
    gdn.gdn_prefill_shared(q[:Np], k[:Np], v[:Np], la[:Np], pick(beta, slice(None, Np)),
                           i32(inp.cu_seqlens), st, o=o_p, conv_w=conv_w,
                           qk_l2norm=conv_w is not None,
                           init_state=None if init_state is None else f32(init_state),
                           init_window=init_window, final_window=win, variant=variant)
    Nb = inp.Nb
    o_b = torch.full((Nb, H, dv), float("nan"), device=DEV, dtype=o_dtype)
    st_b = torch.full((NB, H, dk, dv), float("nan"), device=DEV)
    win_b = torch.zeros((NB, 3, cc), device=DEV, dtype=io_dtype)
    if NB > 0:
        gdn.gdn_fork_branches(q[Np:], k[Np:], v[Np:], la[Np:], pick(beta, slice(Np, None)),
                              i32(inp.branch_cu), i32(inp.branch_parent), st, o_b,
                              parent_window=win, branch_state=st_b, branch_window=win_b,
                              conv_w=conv_w, qk_l2norm=conv_w is not None, variant=variant)
    torch.cuda.synchronize()
    return dict(o_p=o_p.float().cpu().numpy(), st=st.cpu().numpy(), win=win,
                o_b=o_b.float().cpu().numpy(), st_b=st_b.cpu().numpy(), win_b=win_b)


def run_oracle(inp, *, init_state=None, init_window=None, variant="gdn"):
    Np = inp.Np
    conv = inp.conv_w is not None
    o_p, st, win = oracle.prefill(inp.q[:Np], inp.k[:Np], inp.v[:Np], inp.log_alpha[:Np],
                                  inp.beta[:Np], inp.cu_seqlens, conv_w=inp.conv_w,
                                  qk_norm=conv, state_in=init_state, win_in=init_window,
                                  variant=variant)
    o_b, st_b, win_b = oracle.fork(inp.q[Np:], inp.k[Np:], inp.v[Np:], inp.log_alpha[Np:],
                                   inp.beta[Np:], inp.branch_cu, inp.branch_parent, st, win,
                                   conv_w=inp.conv_w, qk_norm=conv, variant=variant)
    return dict(o_p=o_p, st=st, win=win, o_b=o_b, st_b=st_b, win_b=win_b)


def compare(g, r, inp, tol, config=None):
    """Assert the fork's outputs within tol of the oracle's (windows
    bitwise); with `config`, record both parity metrics under that name."""
    H = inp.H
    e = dict(
        o_prefix=slice_err(g["o_p"], r["o_p"], inp.cu_seqlens, H),
        state=oracle.rel_err(g["st"], r["st"], axes=(2, 3)),
        o_branch=slice_err(g["o_b"], r["o_b"], inp.branch_cu, H),
        branch_state=oracle.rel_err(g["st_b"], r["st_b"], axes=(2, 3)),
    )
    print({k: f"{v:.3e}" for k, v in e.items()}, flush=True)
    if config is not None:
        for name, (x, ref, cu) in dict(o_prefix=(g["o_p"], r["o_p"], inp.cu_seqlens),
                                       o_branch=(g["o_b"], r["o_b"], inp.branch_cu)).items():
            _parity.record(config, name, *_parity.seq_metrics(x, ref, cu), tol)
        for name, (x, ref) in dict(state=(g["st"], r["st"]),
                                   branch_state=(g["st_b"], r["st_b"])).items():
            _parity.record(config, name, _parity.rel_err(x, ref, (2, 3)),
                           _parity.elementwise(x, ref, (2, 3)), tol)
    assert all(v <= tol for v in e.values()), e
    assert np.array_equal(window_to_bits(g["win"]), window_ref(r["win"], inp.io))
    assert np.array_equal(window_to_bits(g["win_b"]), window_ref(r["win_b"], inp.io))


def test_tiny_fork_workload():
    """1 request, H=1, d=32, 128-token shared context, 4 branches of 8
    tokens, fp32 throughout, log a ~ U(-0.2,-0.01), no conv; held to 1e-5."""
    w = gi.WORKLOADS["tiny_fork"]
    pl, bl, par = gi.fork_layout(w["R"], w["prefix"], w["branches_per_req"], w["branch_len"])
    inp = gi.seq_inputs(pl, bl, par, w["H"], w["d"], w["d"], io="f32", la_range=w["la_range"],
                        conv=False, seed=0)
    compare(run_fork(inp), run_oracle(inp), inp, TOL_C1, config="C1 tiny_fork")


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_ragged_fork_with_conv(d, io):
    """Ragged contexts (empty, shorter than the conv window, exact chunk
    multiples, ragged tails) and ragged branches, random initial states and
    windows, conv + q/k norm."""
    prefix = [0, 1, 2, 3, 64, 65, 130, 200]
    branches = [5, 0, 1, 2, 64, 70, 3, 9, 1, 128]
    parent = [0, 1, 2, 3, 4, 5, 6, 7, 7, 4]
    H = 2
    inp = gi.seq_inputs(prefix, branches, parent, H, d, d, io=io, conv=True, seed=d)
    rng = np.random.default_rng(d + 1)
    R = len(prefix)
    cc = H * 3 * d
    s0 = (rng.standard_normal((R, H, d, d)) * 0.1).astype(np.float32)
    w0 = rng.standard_normal((R, 3, cc)).astype(np.float32)
    if io == "bf16":
        wbits, w0 = gi.bf16_round(w0)
        w0_dev = torch.from_numpy(wbits.view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        w0_dev = f32(w0)
    g = run_fork(inp, init_state=s0, init_window=w0_dev)
    r = run_oracle(inp, init_state=s0, init_window=w0)
    compare(g, r, inp, TOL if io == "bf16" else TOL_F32)


@pytest.mark.parametrize("variant", ["kda", "rwkv6"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_ragged_fork_per_key(variant, d, io):
    """Per-key decay (KDA delta rule, RWKV6-style raw value update): the
    ragged layout of test_ragged_fork_with_conv, per-key log a ~ U(-0.1,
    -0.001), random initial states and windows, conv + q/k norm; RWKV6 runs
    with beta = NULL."""
    prefix = [0, 1, 2, 3, 64, 65, 130, 200]
    branches = [5, 0, 1, 2, 64, 70, 3, 9, 1, 128]
    parent = [0, 1, 2, 3, 4, 5, 6, 7, 7, 4]
    H = 2
    inp = gi.seq_inputs(prefix, branches, parent, H, d, d, io=io, conv=True, per_key=True,
                        seed=d + 7)
    rng = np.random.default_rng(d + 8)
    R = len(prefix)
    cc = H * 3 * d
    s0 = (rng.standard_normal((R, H, d, d)) * 0.1).astype(np.float32)
    w0 = rng.standard_normal((R, 3, cc)).astype(np.float32)
    if io == "bf16":
        wbits, w0 = gi.bf16_round(w0)
        w0_dev = torch.from_numpy(wbits.view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        w0_dev = f32(w0)
    g = run_fork(inp, init_state=s0, init_window=w0_dev, variant=variant)
    r = run_oracle(inp, init_state=s0, init_window=w0, variant=variant)
    compare(g, r, inp, TOL if io == "bf16" else TOL_F32)


def _decays(case, shape, rng):
    """Per-key log a for the any-decay tests: 'strong' U(-3, -0.5) (a chunk
    decays by up to e^-190, the join factors stay in range); 'sum_1000'
    U(-16, -15.2) (chunk sums near -1000: every row block takes the direct
    diagonal); 'resets' U(-0.1, -0.001) with 5% of entries at -1000; 'one_key'
    key 0 at U(-40, -30), the rest U(-0.1, -0.001)."""
    if case == "strong":
        return rng.uniform(-3.0, -0.5, shape)
    if case == "sum_1000":
        return rng.uniform(-16.0, -15.2, shape)
    mild = rng.uniform(-0.1, -0.001, shape)
    if case == "resets":
        return np.where(rng.random(shape) < 0.05, -1000.0, mild)
    mild[..., 0] = rng.uniform(-40.0, -30.0, shape[:-1])
    return mild


@pytest.mark.parametrize("variant", ["kda", "rwkv6"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("case", ["strong", "sum_1000", "resets", "one_key"])
def test_per_key_any_decay(variant, d, case):
    """Per-key prefill + branches stay within the bar for any decay: the
    ragged layout with random initial states, conv + q/k norm, bf16, and
    per-key log a from _decays (down to chunk sums of -1000 and single
    steps of -1000)."""
    prefix = [0, 1, 3, 64, 65, 130, 200]
    branches = [5, 1, 64, 70, 9, 128]
    parent = [0, 1, 2, 3, 4, 6]
    H = 2
    inp = gi.seq_inputs(prefix, branches, parent, H, d, d, io="bf16", conv=True, per_key=True,
                        seed=d + 31)
    rng = np.random.default_rng(d + 32)
    inp.log_alpha = _decays(case, inp.log_alpha.shape, rng).astype(np.float32)
    s0 = (rng.standard_normal((len(prefix), H, d, d)) * 0.1).astype(np.float32)
    g = run_fork(inp, init_state=s0, variant=variant)
    r = run_oracle(inp, init_state=s0, variant=variant)
    compare(g, r, inp, TOL)


@pytest.mark.parametrize("variant", ["kda", "rwkv6"])
def test_per_key_strong_decay_f32(variant):
    """fp32 I/O at per-key log a ~ U(-3, -0.5), d = 128, held to the fp32
    bar."""
    prefix = [64, 130, 200]
    branches = [64, 7, 70]
    parent = [0, 1, 2]
    inp = gi.seq_inputs(prefix, branches, parent, 2, 128, 128, io="f32", conv=True,
                        per_key=True, la_range=(-3.0, -0.5), seed=41)
    compare(run_fork(inp, variant=variant), run_oracle(inp, variant=variant), inp, TOL_F32)


@pytest.mark.parametrize("variant", ["kda", "rwkv6"])
def test_long_context_per_key(variant):
    """Per-key decay over long contexts (16+ chunks per sequence), H=4,
    d=128, bf16, conv: errors must not grow with the number of chunks."""
    prefix = [1100, 1024, 64]
    branches = [64, 64, 33, 64]
    parent = [0, 1, 2, 0]
    inp = gi.seq_inputs(prefix, branches, parent, 4, 128, 128, io="bf16", conv=True,
                        per_key=True, seed=11)
    compare(run_fork(inp, variant=variant), run_oracle(inp, variant=variant), inp, TOL)


@pytest.mark.parametrize("variant", ["gdn", "kda"])
def test_checkpoints_match_truncated_runs_and_resume(variant):
    """Checkpoints every 2 chunks (128 tokens): each equals the oracle's
    final state / window of the sequence cut at that position; positions
    past a sequence (or past the capacity) are left untouched; and resuming
    from a checkpoint reproduces the rest of the sequence."""
    d, H, every, cap = 64, 2, 2, 3
    prefix = [300, 128, 64, 520, 0]
    inp = gi.seq_inputs(prefix, [], [], H, d, d, io="bf16", conv=True,
                        per_key=variant != "gdn", seed=21)
    R, Np, cc = len(prefix), inp.Np, H * 3 * d
    q, k, v = (dev_io(getattr(inp, n), getattr(inp, n + "_bits")) for n in "qkv")
    la, beta, conv_w = f32(inp.log_alpha), f32(inp.beta), f32(inp.conv_w)
    st = torch.empty((R, H, d, d), device=DEV)
    ck = torch.full((R, cap, H, d, d), 7.0, device=DEV)
    ckw = torch.zeros((R, cap, 3, cc), device=DEV, dtype=torch.bfloat16)
    o = torch.empty((Np, H, d), device=DEV)
    gdn.gdn_prefill_checkpointed(q, k, v, la, beta, i32(inp.cu_seqlens), st, every, ck, o=o,
                                 ckpt_window=ckw, conv_w=conv_w, qk_l2norm=True, variant=variant)
    torch.cuda.synchronize()
    ck_h, ckw_bits = ck.cpu().numpy(), window_to_bits(ckw)
    step = every * 64
    for r, n in enumerate(prefix):
        a = int(inp.cu_seqlens[r])
        for j in range(cap):
            pos = (j + 1) * step
            if pos > n:
                assert (ck_h[r, j] == 7.0).all(), (r, j)  # untouched
                continue
            sl = slice(a, a + pos)
            _, st_ref, win_ref = oracle.prefill(inp.q[sl], inp.k[sl], inp.v[sl], inp.log_alpha[sl],
                                                inp.beta[sl], np.array([0, pos]),
                                                conv_w=inp.conv_w, qk_norm=True, variant=variant)
            e = oracle.rel_err(ck_h[r, j][None], st_ref, axes=(2, 3))
            assert e <= TOL, (r, j, e)
            assert np.array_equal(ckw_bits[r, j], window_ref(win_ref[0], "bf16")), (r, j)
    # resume sequence 3 from its second checkpoint (256 tokens in)
    r, j = 3, 1
    pos, a, n = (j + 1) * step, int(inp.cu_seqlens[3]), prefix[3]
    sl = slice(a + pos, a + n)
    st2 = torch.empty((1, H, d, d), device=DEV)
    o2 = torch.empty((n - pos, H, d), device=DEV)
    gdn.gdn_prefill_shared(q[sl], k[sl], v[sl], la[sl], beta[sl], i32([0, n - pos]), st2, o=o2,
                           conv_w=conv_w, qk_l2norm=True, init_state=ck[r, j][None].contiguous(),
                           init_window=ckw[r, j][None].contiguous(), variant=variant)
    torch.cuda.synchronize()
    e_o = oracle.rel_err(o2.cpu().numpy().astype(np.float64),
                         o.cpu().numpy()[a + pos:a + n].astype(np.float64), axes=(0, 2))
    e_s = oracle.rel_err(st2.cpu().numpy(), st.cpu().numpy()[r:r + 1], axes=(2, 3))
    assert e_o <= TOL and e_s <= TOL, (e_o, e_s)


def test_fork_is_bitwise_the_full_run_at_chunk_boundaries():
    """Flide page, method step 2: forking from the saved state computes the
    same function as the independent prompt. When the shared context is a
    whole number of chunks the GPU processes the same chunks either way, so
    the branch outputs are bit-identical to running context + question."""
    H, d = 2, 128
    prefix = [128, 64]
    branches = [37, 64, 5]
    parent = [0, 1, 0]
    inp = gi.seq_inputs(prefix, branches, parent, H, d, d, conv=True, seed=3)
    g = run_fork(inp)
    # the same tokens as independent full sequences: context + question
    Np = inp.Np
    rows = []
    lens = []
    for b, p in enumerate(parent):
        pre = np.arange(inp.cu_seqlens[p], inp.cu_seqlens[p + 1])
        br = Np + np.arange(inp.branch_cu[b], inp.branch_cu[b + 1])
        rows.append(np.concatenate([pre, br]))
        lens.append(len(rows[-1]))
    idx = np.concatenate(rows)
    full = gi.SeqInputs(**{**inp.__dict__})
    for n in ["q", "k", "v", "q_bits", "k_bits", "v_bits", "log_alpha", "beta"]:
        setattr(full, n, getattr(inp, n)[idx])
    full.Np = len(idx)
    full.Nb = 0
    full.cu_seqlens = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    full.branch_cu = np.zeros(1, dtype=np.int32)
    full.branch_parent = np.zeros(0, dtype=np.int32)
    gf = run_fork(full)
    for b, p in enumerate(parent):
        P = prefix[p]
        a = full.cu_seqlens[b]
        assert np.array_equal(g["o_b"][inp.branch_cu[b]:inp.branch_cu[b + 1]],
                              gf["o_p"][a + P:a + lens[b]])
        assert np.array_equal(g["st_b"][b], gf["st"][b])


def test_invalid_parent_gives_nan_outputs():
    H, d = 1, 64
    inp = gi.seq_inputs([70], [4, 6], [0, 3], H, d, d, conv=True, seed=4)
    g = run_fork(inp)
    assert np.isnan(g["o_b"][4:10]).all() and not np.isnan(g["o_b"][:4]).any()
    assert np.isnan(g["st_b"][1]).all()


@pytest.mark.parametrize("variant", ["gdn", "kda"])
def test_full_size_fork_prefill_sampled(variant):
    """8 requests x 8192-token contexts, 20 branches of 64 tokens each,
    H=16, d=128, chunk 64, conv width 4, bf16 I/O (and the same with
    per-key decay, as the bench also times it): the GPU runs the whole
    workload in the launch configuration the bench times; the oracle checks
    two requests and all of their branches (every head)."""
    w = gi.WORKLOADS["fork_prefill"]
    R, H, d = w["R"], w["H"], w["d"]
    pl, bl, par = gi.fork_layout(R, w["prefix"], w["branches_per_req"], w["branch_len"])
    t = gi.torch_seq_inputs(pl, bl, par, H, d, d, conv=True, per_key=variant != "gdn", seed=0)
    Np, Nb = t["Np"], t["Nb"]
    cc = H * 3 * d
    st = torch.empty((R, H, d, d), device=DEV)
    win = torch.empty((R, 3, cc), device=DEV, dtype=torch.bfloat16)
    o_p = torch.empty((Np, H, d), device=DEV)
    gdn.gdn_prefill_shared(t["q"][:Np], t["k"][:Np], t["v"][:Np], t["log_alpha"][:Np],
                           t["beta"][:Np], t["cu_seqlens"], st, o=o_p, conv_w=t["conv_w"],
                           qk_l2norm=True, final_window=win, variant=variant)
    NB = len(bl)
    o_b = torch.empty((Nb, H, d), device=DEV)
    st_b = torch.empty((NB, H, d, d), device=DEV)
    gdn.gdn_fork_branches(t["q"][Np:], t["k"][Np:], t["v"][Np:], t["log_alpha"][Np:],
                          t["beta"][Np:], t["branch_cu"], t["branch_parent"], st, o_b,
                          parent_window=win, branch_state=st_b, conv_w=t["conv_w"],
                          qk_l2norm=True, variant=variant)
    # the call as the bench times it (o only): the same o bit for bit (the
    # state update runs after the outputs and changes nothing they read)
    o_b2 = torch.full((Nb, H, d), float("nan"), device=DEV)
    gdn.gdn_fork_branches(t["q"][Np:], t["k"][Np:], t["v"][Np:], t["log_alpha"][Np:],
                          t["beta"][Np:], t["branch_cu"], t["branch_parent"], st, o_b2,
                          parent_window=win, conv_w=t["conv_w"], qk_l2norm=True, variant=variant)
    torch.cuda.synchronize()
    assert torch.equal(o_b2, o_b)
    P, bpr, L = w["prefix"], w["branches_per_req"], w["branch_len"]
    host = lambda x: x.float().cpu().numpy()  # noqa: E731
    cw = host(t["conv_w"])
    for r in [0, R - 1]:
        rows = slice(r * P, (r + 1) * P)
        o_r, st_r, win_r = oracle.prefill(host(t["q"][rows]), host(t["k"][rows]),
                                          host(t["v"][rows]), host(t["log_alpha"][rows]),
                                          host(t["beta"][rows]), [0, P], conv_w=cw, qk_norm=True,
                                          variant=variant)
        e_o = oracle.rel_err(host(o_p[rows]), o_r, axes=(0, 2))
        e_s = oracle.rel_err(host(st[r:r + 1]), st_r, axes=(2, 3))
        brow = slice(Np + r * bpr * L, Np + (r + 1) * bpr * L)
        bcu = np.arange(bpr + 1) * L
        o_br, st_br, _ = oracle.fork(host(t["q"][brow]), host(t["k"][brow]), host(t["v"][brow]),
                                     host(t["log_alpha"][brow]), host(t["beta"][brow]), bcu,
                                     np.zeros(bpr, dtype=np.int32), st_r, win_r, conv_w=cw,
                                     qk_norm=True, variant=variant)
        g_ob = host(o_b[r * bpr * L:(r + 1) * bpr * L])
        e_ob = max(oracle.rel_err(g_ob[i * L:(i + 1) * L], o_br[i * L:(i + 1) * L], axes=(0, 2))
                   for i in range(bpr))
        e_sb = oracle.rel_err(host(st_b[r * bpr:(r + 1) * bpr]), st_br, axes=(2, 3))
        print(f"{variant} request {r}: o={e_o:.3e} state={e_s:.3e} branch o={e_ob:.3e} "
              f"branch state={e_sb:.3e}", flush=True)
        cfg = ("C3 fork_prefill (requests 0 and 7, all heads and their branches)" if variant == "gdn"
               else "C3 fork_prefill with per-key decay, KDA (requests 0 and 7, all heads and "
                    "their branches)")
        _parity.record(cfg, "o_prefix", e_o, _parity.elementwise(host(o_p[rows]), o_r, (0, 2)),
                       TOL)
        _parity.record(cfg, "state", e_s, _parity.elementwise(host(st[r:r + 1]), st_r, (2, 3)),
                       TOL)
        _parity.record(cfg, "o_branch", *_parity.seq_metrics(g_ob, o_br, bcu), TOL)
        _parity.record(cfg, "branch_state", e_sb,
                       _parity.elementwise(host(st_b[r * bpr:(r + 1) * bpr]), st_br, (2, 3)),
                       TOL)
        assert max(e_o, e_s, e_ob, e_sb) <= TOL
        wb = win[r].cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(wb, gi.bf16_round(win_r[0].astype(np.float32))[0])


@pytest.mark.parametrize("variant", ["gdn", "kda"])
def test_batch_composition_invariance(variant):
    """A request's outputs do not depend on what else shares the call: the
    middle request of three, run alone (at another stream offset), gives the
    same bits for its o, final state and window, and so do its branches
    when the other requests' branches are dropped."""
    prefix, branches, parent = [300, 130, 77], [9, 64, 40, 3], [1, 0, 1, 2]
    full = gi.seq_inputs(prefix, branches, parent, 4, 128, 128, io="bf16", conv=True,
                         per_key=variant != "gdn", seed=13)
    g_full = run_fork(full, variant=variant)
    # request 1 alone, with its own branches (0 and 2 of the full call)
    Np = full.Np
    rows_p = np.r_[300:430]
    keep_b = [0, 2]
    rows_b = np.concatenate([np.arange(full.branch_cu[b], full.branch_cu[b + 1]) + Np
                             for b in keep_b])
    rows = np.concatenate([rows_p, rows_b])
    sub = gi.SeqInputs(**{**full.__dict__})
    for n in ("q", "k", "v", "log_alpha", "beta"):
        setattr(sub, n, getattr(full, n)[rows])
    for n in ("q_bits", "k_bits", "v_bits"):
        setattr(sub, n, getattr(full, n)[rows])
    sub.Np, sub.Nb, sub.N = 130, len(rows_b), len(rows)
    sub.cu_seqlens = np.array([0, 130], dtype=np.int32)
    sub.branch_cu = np.array([0, branches[0], branches[0] + branches[2]], dtype=np.int32)
    sub.branch_parent = np.array([0, 0], dtype=np.int32)
    g_sub = run_fork(sub, variant=variant)
    assert np.array_equal(g_sub["o_p"], g_full["o_p"][300:430])
    assert np.array_equal(g_sub["st"][0], g_full["st"][1])
    assert torch.equal(g_sub["win"][0], g_full["win"][1])
    b0 = slice(int(full.branch_cu[0]), int(full.branch_cu[1]))
    b2 = slice(int(full.branch_cu[2]), int(full.branch_cu[3]))
    assert np.array_equal(g_sub["o_b"][:branches[0]], g_full["o_b"][b0])
    assert np.array_equal(g_sub["o_b"][branches[0]:], g_full["o_b"][b2])
    assert np.array_equal(g_sub["st_b"][0], g_full["st_b"][0])
    assert np.array_equal(g_sub["st_b"][1], g_full["st_b"][2])
