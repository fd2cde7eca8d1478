"""GPU parity of the one-chunk kernel.

Sequences of at most one chunk (64 tokens) -- the fork's branches, and
short sequences of a shared-context call -- run in one kernel instead of
passing a chunk record from the prep kernel to a later scan: with a scalar
decay the chunk's operands stay on chip, per key the record goes through
the (sequence, head)'s workspace slot and back within the workgroup. Its
arithmetic is theirs in the same order, so every output must equal the
chunked path's bit for bit
(GDN_PREFILL_ONE_CHUNK=0 sends the same sequences through the chunked
kernels), and both must hold the fp64 oracle's bar. The rounds mix short
and long sequences (the long ones still take the chunked kernels in the
same call), empty branches, invalid parents (NaN outputs), rectangular
heads, a head count that maps heads to XCDs (16) and ones that do not, with
and without the branch states, and a shared-context call of short
sequences from given initial states and windows.
"""

import contextlib
import os

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_recurrent_gdn_amd as gdn
import oracle
from test_gpu_prefill import (DEV, TOL, TOL_F32, dev_io, f32, i32, slice_err, window_ref,
                              window_to_bits)

pytestmark = pytest.mark.gpu

ENV = "GDN_PREFILL_ONE_CHUNK"


@contextlib.contextmanager
def chunked_path():
    old = os.environ.get(ENV)
    os.environ[ENV] = "0"
    try:
        yield
    finally:
        if old is None:
            del os.environ[ENV]
        else:
            os.environ[ENV] = old


def io_window(inp, w0):
    if inp.io == "bf16":
        bits, vals = gi.bf16_round(w0)
        return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16), vals
    return f32(w0), w0


def run(inp, states, s0=None, w0_dev=None, variant="gdn"):
    """Both calls; returns host copies (windows as bits)."""
    H, dk, dv, Np, Nb = inp.H, inp.dk, inp.dv, inp.Np, inp.Nb
    R, NB = len(inp.cu_seqlens) - 1, len(inp.branch_cu) - 1
    cc = H * (2 * dk + dv)
    io_dtype = torch.bfloat16 if inp.io == "bf16" else torch.float32
    q, k, v = (dev_io(getattr(inp, n), getattr(inp, n + "_bits")) for n in "qkv")
    la, beta, conv_w = f32(inp.log_alpha), f32(inp.beta), f32(inp.conv_w)
    o_p = torch.full((Np, H, dv), float("nan"), device=DEV)
    st = torch.full((R, H, dk, dv), float("nan"), device=DEV)
    win = torch.zeros((R, 3, cc), device=DEV, dtype=io_dtype)
    gdn.gdn_prefill_shared(q[:Np], k[:Np], v[:Np], la[:Np], beta[:Np], i32(inp.cu_seqlens), st,
                           o=o_p, conv_w=conv_w, qk_l2norm=True,
                           init_state=None if s0 is None else f32(s0), init_window=w0_dev,
                           final_window=win, variant=variant)
    out = dict(o_p=o_p.cpu().numpy(), st=st.cpu().numpy(), win=window_to_bits(win))
    if NB > 0:
        o_b = torch.full((Nb, H, dv), float("nan"), device=DEV)
        st_b = torch.full((NB, H, dk, dv), float("nan"), device=DEV) if states else None
        win_b = torch.zeros((NB, 3, cc), device=DEV, dtype=io_dtype) if states else None
        gdn.gdn_fork_branches(q[Np:], k[Np:], v[Np:], la[Np:], beta[Np:], i32(inp.branch_cu),
                              i32(inp.branch_parent), st, o_b, parent_window=win,
                              branch_state=st_b, branch_window=win_b, conv_w=conv_w,
                              qk_l2norm=True, variant=variant)
        out["o_b"] = o_b.cpu().numpy()
        if states:
            out["st_b"] = st_b.cpu().numpy()
            out["win_b"] = window_to_bits(win_b)
    torch.cuda.synchronize()
    return out


def assert_bitwise(a, b):
    assert a.keys() == b.keys()
    for name in a:
        assert np.array_equal(a[name], b[name], equal_nan=True), name


def prefix_oracle(inp, s0=None, w0=None, variant="gdn"):
    Np = inp.Np
    return oracle.prefill(inp.q[:Np], inp.k[:Np], inp.v[:Np], inp.log_alpha[:Np], inp.beta[:Np],
                          inp.cu_seqlens, conv_w=inp.conv_w, qk_norm=True, state_in=s0,
                          win_in=w0, variant=variant)


def branch_oracle(inp, st, win, variant="gdn"):
    """Oracle outputs of the branches with a valid parent, as a reduced round."""
    Np, R = inp.Np, len(inp.cu_seqlens) - 1
    bcu, par = inp.branch_cu, inp.branch_parent
    valid = [b for b in range(len(par)) if 0 <= par[b] < R]
    rows = np.concatenate([np.arange(Np + bcu[b], Np + bcu[b + 1]) for b in valid])
    vcu = np.concatenate([[0], np.cumsum([bcu[b + 1] - bcu[b] for b in valid])]).astype(np.int32)
    o_b, st_b, win_b = oracle.fork(inp.q[rows], inp.k[rows], inp.v[rows], inp.log_alpha[rows],
                                   inp.beta[rows], vcu, par[valid], st, win, conv_w=inp.conv_w,
                                   qk_norm=True, variant=variant)
    return valid, vcu, o_b, st_b, win_b


PREFIX = [130, 64, 7, 0, 1, 300]          # 64, 7, 0, 1: one chunk or none
BRANCHES = [0, 1, 5, 63, 64, 65, 130, 17, 40, 64, 3, 33]
PARENT = [0, 0, 1, 2, 3, 5, 5, -1, 4, 6, 2, 1]  # -1 and 6 (= R): invalid


SHAPES = [(16, 128, 128), (3, 64, 128), (3, 128, 32), (2, 32, 64)]
CASES = ([("gdn", H, dk, dv, io) for H, dk, dv in SHAPES for io in ("bf16", "f32")]
         + [(var, H, dk, dv, "bf16") for var in ("kda", "rwkv6") for H, dk, dv in SHAPES]
         + [(var, 16, 128, 128, "f32") for var in ("kda", "rwkv6")])


@pytest.mark.parametrize("states", [False, True])
@pytest.mark.parametrize("variant,H,dk,dv,io", CASES)
def test_one_chunk_is_bitwise_the_chunked_path(variant, H, dk, dv, io, states):
    inp = gi.seq_inputs(PREFIX, BRANCHES, PARENT, H, dk, dv, io=io, conv=True,
                        per_key=variant != "gdn", seed=dk + dv + H + states)
    fused = run(inp, states, variant=variant)
    with chunked_path():
        chunked = run(inp, states, variant=variant)
    assert_bitwise(fused, chunked)

    tol = TOL if io == "bf16" else TOL_F32
    o_p, st, win = prefix_oracle(inp, variant=variant)
    e_p = slice_err(fused["o_p"], o_p, inp.cu_seqlens, H)
    e_s = oracle.rel_err(fused["st"], st, axes=(2, 3))
    assert np.array_equal(fused["win"], window_ref(win, io))
    valid, vcu, o_r, st_r, win_r = branch_oracle(inp, st, win, variant=variant)
    bcu = inp.branch_cu
    g_rows = np.concatenate([np.arange(bcu[b], bcu[b + 1]) for b in valid])
    e_b = slice_err(fused["o_b"][g_rows], o_r, vcu, H)
    e_bs = oracle.rel_err(fused["st_b"][valid], st_r, axes=(2, 3)) if states else 0.0
    print(f"{variant} H={H} dk={dk} dv={dv} {io} states={states}: o_p {e_p:.2e} st {e_s:.2e} "
          f"o_b {e_b:.2e} st_b {e_bs:.2e}", flush=True)
    assert max(e_p, e_s, e_b, e_bs) <= tol
    if states:
        assert np.array_equal(fused["win_b"][valid], window_ref(win_r, io))
    for b in range(len(PARENT)):
        rows = slice(bcu[b], bcu[b + 1])
        if b in valid:
            assert not np.isnan(fused["o_b"][rows]).any(), b
        else:
            assert np.isnan(fused["o_b"][rows]).all(), b
            if states:
                assert np.isnan(fused["st_b"][b]).all(), b


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_short_sequences_from_initial_states(io):
    """A shared-context call of short sequences only, each from a given
    state and conv window (the window supplies the conv rows before the
    sequence, an empty sequence passes both through)."""
    H, dk, dv = 4, 128, 64
    lens = [64, 1, 33, 0, 17, 2]
    inp = gi.seq_inputs(lens, [], [], H, dk, dv, io=io, conv=True, seed=31)
    R, cc = len(lens), H * (2 * dk + dv)
    rng = np.random.default_rng(32)
    s0 = (rng.standard_normal((R, H, dk, dv)) * 0.1).astype(np.float32)
    w0_dev, w0 = io_window(inp, rng.standard_normal((R, 3, cc)).astype(np.float32))
    fused = run(inp, False, s0, w0_dev)
    with chunked_path():
        chunked = run(inp, False, s0, w0_dev)
    assert_bitwise(fused, chunked)
    o_p, st, win = prefix_oracle(inp, s0, w0)
    e_p = slice_err(fused["o_p"], o_p, inp.cu_seqlens, H)
    e_s = oracle.rel_err(fused["st"], st, axes=(2, 3))
    print(f"{io}: o {e_p:.2e} state {e_s:.2e}", flush=True)
    assert max(e_p, e_s) <= (TOL if io == "bf16" else TOL_F32)
    assert np.array_equal(fused["win"], window_ref(win, io))
    # the empty sequence: its state and window pass through unchanged
    assert np.array_equal(fused["st"][3], s0[3])
