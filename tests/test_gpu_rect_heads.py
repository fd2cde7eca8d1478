"""GPU parity with d_k != d_v (a rectangular d_k x d_v state, as the DeltaLog
page's problem section stores it: [B, H, d_k, d_v]) for every operation:
the eager step, deferred steps with merges, the stand-alone merge, and the
two-call fork (prefill + branches, with conv and q/k norm, scalar and per-key
decay). Same metric and bars as the square-head tests: max |gpu - oracle| /
max |oracle| per (row or sequence, head) slice, 2e-3 for bf16 I/O, and
bitwise conv windows."""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from _decode_helpers import (TOL, TOL_F32, gpu_deferred, gpu_eager, oracle_decode,
                             prepopulated_logs, rel_err_slices)
from test_gpu_prefill import TOL_F32 as TOL_F32_PREFILL, compare, run_fork, run_oracle

pytestmark = pytest.mark.gpu

PAIRS = [(128, 64), (64, 128), (32, 128), (128, 32), (64, 32)]


def check(o_gpu, st_gpu, o_ref, st_ref, tol):
    eo = rel_err_slices(o_gpu.float().cpu().numpy(), o_ref, axes=(0, 3))
    es = rel_err_slices(st_gpu.cpu().numpy(), st_ref, axes=(2, 3))
    print(f"rel err o={eo:.3e} state={es:.3e}", flush=True)
    assert eo <= tol and es <= tol, (eo, es)


@pytest.mark.parametrize("dk,dv", PAIRS)
@pytest.mark.parametrize("variant", ["gdn", "kda", "rwkv6"])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_eager_rect(dk, dv, variant, io):
    inp = gi.decode_inputs(3, 2, dk, dv, 10, per_key=variant != "gdn", io=io, seed=dk + dv)
    o_ref, st_ref, _ = oracle_decode(inp, variant)
    o, st = gpu_eager(inp, variant)
    check(o, st, o_ref, st_ref, TOL if io == "bf16" else TOL_F32)


@pytest.mark.parametrize("dk,dv", PAIRS)
@pytest.mark.parametrize("variant", ["gdn", "kda", "rwkv6"])
def test_deferred_rect(dk, dv, variant):
    """Deferred steps at M=8 from logs of per-slot lengths in [0, 8), then a
    flush by the stand-alone merge."""
    M = 8
    inp = gi.decode_inputs(5, 3, dk, dv, 2 * M + 3, per_key=variant != "gdn", seed=dk * 3 + dv,
                           phases_M=M)
    ent, lengths, logical = prepopulated_logs(inp, M, inp.phase)
    o_ref, st_ref, _ = oracle_decode(inp, variant, state0=logical)
    o, base, _ = gpu_deferred(inp, variant, M, ent, lengths)
    check(o, base, o_ref, st_ref, TOL)


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128)])
def test_merge_every_step_is_bitwise_eager_rect(dk, dv):
    inp = gi.decode_inputs(3, 2, dk, dv, 5, seed=4)
    o_e, st_e = gpu_eager(inp, "gdn")
    o_d, base, _ = gpu_deferred(inp, "gdn", 1)
    assert torch.equal(o_e, o_d) and torch.equal(st_e, base)


@pytest.mark.parametrize("dk,dv", PAIRS)
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_fork_rect(dk, dv, io):
    """Ragged contexts and branches (empty, shorter than the conv window,
    chunk multiples, ragged tails), random initial states and windows, conv
    + q/k norm, scalar decay."""
    prefix = [0, 2, 64, 130, 200]
    branches = [5, 0, 64, 70, 1, 9]
    parent = [0, 1, 2, 3, 4, 4]
    H = 2
    inp = gi.seq_inputs(prefix, branches, parent, H, dk, dv, io=io, conv=True, seed=dk + 2 * dv)
    rng = np.random.default_rng(dk + dv)
    R = len(prefix)
    cc = H * (2 * dk + dv)
    s0 = (rng.standard_normal((R, H, dk, dv)) * 0.1).astype(np.float32)
    w0 = rng.standard_normal((R, 3, cc)).astype(np.float32)
    if io == "bf16":
        wbits, w0 = gi.bf16_round(w0)
        w0_dev = torch.from_numpy(wbits.view(np.int16)).to("cuda").view(torch.bfloat16)
    else:
        w0_dev = torch.from_numpy(w0).to("cuda")
    g = run_fork(inp, init_state=s0, init_window=w0_dev)
    r = run_oracle(inp, init_state=s0, init_window=w0)
    compare(g, r, inp, TOL if io == "bf16" else TOL_F32_PREFILL)


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128)])
@pytest.mark.parametrize("variant", ["kda", "rwkv6"])
def test_fork_rect_per_key(dk, dv, variant):
    prefix = [3, 64, 150]
    branches = [64, 7, 0, 40]
    parent = [0, 1, 2, 2]
    inp = gi.seq_inputs(prefix, branches, parent, 2, dk, dv, io="bf16", conv=True, per_key=True,
                        seed=dk + dv + 1)
    compare(run_fork(inp, variant=variant), run_oracle(inp, variant=variant), inp, TOL)
