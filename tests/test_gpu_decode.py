"""GPU parity of the decode operations against the fp64 oracle.

Metric: for every (row, head) slice, max |gpu - oracle| / max |oracle| over
the slice (all steps x d_v for o; d_k x d_v for the state); the max over
slices must stay within 2e-3 for bf16 I/O (fp32 state), and within 2e-5 for
fp32 I/O.
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_recurrent_gdn_amd as gdn
import oracle
from _decode_helpers import (DEV, TOL, TOL_F32, gpu_deferred, gpu_eager, oracle_decode,
                             prepopulated_logs, rel_err_slices, to_dev)

pytestmark = pytest.mark.gpu

VARIANTS = ["gdn", "kda", "rwkv6"]


def small(variant, io="bf16", d=128, B=3, H=2, steps=12, seed=0, phases_M=None):
    return gi.decode_inputs(B, H, d, d, steps, per_key=variant != "gdn", io=io, seed=seed,
                            phases_M=phases_M)


def check(o_gpu, st_gpu, o_ref, st_ref, tol):
    o_gpu = o_gpu.float().cpu().numpy()
    st_gpu = st_gpu.cpu().numpy()
    eo = rel_err_slices(o_gpu, o_ref, axes=(0, 3))
    es = rel_err_slices(st_gpu, st_ref, axes=(2, 3))
    print(f"rel err o={eo:.3e} state={es:.3e}", flush=True)
    assert eo <= tol and es <= tol, (eo, es)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_eager_matches_oracle(variant, io, d):
    inp = small(variant, io, d)
    o_ref, st_ref, _ = oracle_decode(inp, variant)
    o, st = gpu_eager(inp, variant)
    check(o, st, o_ref, st_ref, TOL if io == "bf16" else TOL_F32)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("M", [1, 4, 8, 16])
def test_deferred_with_phases_matches_oracle(variant, M):
    """Logs start with per-slot lengths in [0, M), so merges of different
    slots fall on different steps; a final flush materialises every slot."""
    inp = small(variant, B=5, H=3, steps=2 * M + 5, seed=M, phases_M=M)
    ent, lengths, logical = prepopulated_logs(inp, M, inp.phase)
    o_ref, st_ref, _ = oracle_decode(inp, variant, state0=logical)
    o, base, _ = gpu_deferred(inp, variant, M, ent, lengths)
    check(o, base, o_ref, st_ref, TOL)


@pytest.mark.parametrize("variant", VARIANTS)
def test_logged_factors_match_oracle(variant):
    """Without merges the log holds u_t (the oracle's rank-1 value factor),
    an exact copy of k_t, and the running log-decay since the base."""
    M = 8
    inp = small(variant, steps=M - 1, seed=3)
    o_ref, st_ref, u_ref = oracle_decode(inp, variant)
    o, base, (log_u, log_k, log_lam, log_len) = gpu_deferred(inp, variant, M, flush=False)
    assert torch.equal(base.cpu(), torch.from_numpy(inp.state0))  # base untouched
    assert (log_len.cpu().numpy() == M - 1).all()
    lu = log_u.cpu().numpy()[:, :, : M - 1].transpose(2, 0, 1, 3)
    assert rel_err_slices(lu, u_ref, axes=(0, 3)) <= TOL
    kb = log_k.cpu().view(torch.int16).numpy()[:, :, : M - 1].transpose(2, 0, 1, 3)
    assert np.array_equal(kb.view(np.uint16), inp.k_bits)
    lam = log_lam.cpu().numpy()[:, :, : M - 1]
    lam = np.moveaxis(lam, 2, 0)
    np.testing.assert_allclose(lam, np.cumsum(inp.log_alpha.astype(np.float64), axis=0),
                               rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("variant", VARIANTS)
def test_merge_every_step_is_bitwise_eager(variant):
    inp = small(variant, steps=6, seed=5)
    o_e, st_e = gpu_eager(inp, variant)
    o_d, base, _ = gpu_deferred(inp, variant, 1)
    assert torch.equal(o_e, o_d) and torch.equal(st_e, base)


@pytest.mark.parametrize("variant", ["gdn", "kda"])
def test_merge_only_matches_materialize_and_skips_short_logs(variant):
    inp = small(variant, B=4, H=2, steps=1, seed=6)
    M = 8
    lengths_slot = np.array([0, 3, 8, 5])
    ent, lengths, logical = prepopulated_logs(inp, M, lengths_slot)
    inp.steps = 0
    inp.q = inp.q[:0]
    inp.k = inp.k[:0]
    inp.v = inp.v[:0]
    inp.log_alpha = inp.log_alpha[:0]
    inp.beta = inp.beta[:0]
    inp.q_bits = inp.q_bits[:0]
    inp.k_bits = inp.k_bits[:0]
    inp.v_bits = inp.v_bits[:0]
    _, base, (log_u, log_k, log_lam, log_len) = gpu_deferred(inp, variant, M, ent, lengths,
                                                             flush=False)
    base0 = base.clone()
    gdn.deltalog_merge(base, log_u, log_k, log_lam, log_len, min_len=4, variant=variant)
    torch.cuda.synchronize()
    b = base.cpu().numpy()
    for s, m in enumerate(lengths_slot):
        if m >= 4:
            assert rel_err_slices(b[s], logical[s], axes=(1, 2)) <= 1e-5
            assert (log_len[s].cpu().numpy() == 0).all()
        else:  # untouched bit for bit
            assert torch.equal(base[s], base0[s])
            assert (log_len[s].cpu().numpy() == m).all()


def test_slot_indirection_and_permutation_invariance():
    """Rows map to slots through slot_idx: a permuted mapping into a larger
    pool gives bit-identical per-sequence results (the kernels never mix
    rows, so the result of a sequence does not depend on its slot or on the
    batch around it)."""
    inp = small("gdn", B=6, H=2, steps=5, seed=7)
    o_a, st_a = gpu_eager(inp, "gdn")
    perm = [9, 2, 7, 0, 4, 11]
    o_b, st_b = gpu_eager(inp, "gdn", slot_idx=perm, n_slots=12)
    assert torch.equal(o_a, o_b)
    assert torch.equal(st_a, st_b[torch.tensor(perm, device=DEV).long()])


def test_invalid_slot_yields_nan_row_and_touches_nothing():
    inp = small("gdn", B=3, H=2, steps=1, seed=8)
    q = torch.from_numpy(inp.q_bits[0].view(np.int16)).to(DEV).view(torch.bfloat16)
    k = torch.from_numpy(inp.k_bits[0].view(np.int16)).to(DEV).view(torch.bfloat16)
    v = torch.from_numpy(inp.v_bits[0].view(np.int16)).to(DEV).view(torch.bfloat16)
    state = to_dev(inp.state0)
    st0 = state.clone()
    o = torch.zeros((3, 2, 128), device=DEV)
    sl = torch.tensor([0, 5, 2], dtype=torch.int32, device=DEV)  # 5 is out of range
    gdn.gdn_decode_eager(q, k, v, to_dev(inp.log_alpha[0]), to_dev(inp.beta[0]), state, o,
                         slot_idx=sl)
    torch.cuda.synchronize()
    assert torch.isnan(o[1]).all() and not torch.isnan(o[0]).any()
    assert torch.equal(state[1], st0[1])


def test_bf16_output_rounds_the_fp32_result():
    inp = small("gdn", steps=3, seed=9)
    o32, _ = gpu_eager(inp, "gdn")
    o16, _ = gpu_eager(inp, "gdn", o_dtype=torch.bfloat16)
    assert torch.equal(o32.to(torch.bfloat16), o16)


def test_repeat_runs_are_bitwise_identical():
    inp = small("kda", steps=5, seed=10, phases_M=4)
    ent, lengths, _ = prepopulated_logs(inp, 4, inp.phase)
    a = gpu_deferred(inp, "kda", 4, ent, lengths)
    b = gpu_deferred(inp, "kda", 4, ent, lengths)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
