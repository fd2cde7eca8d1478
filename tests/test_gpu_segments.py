"""GPU parity of prefills that run in segments.

A long prefill runs as several segments, each taking a proportional share
of every sequence's chunks, so that one segment's chunk records (not the
whole call's) bound the workspace; the state passes from one segment to
the next through the workspace. These tests force segments on small
inputs through the documented bound GDN_PREFILL_SEGMENT_RECORD_BYTES and
check that every output is bit for bit the one-segment result (the same
chunk steps in the same order) and within the bar of the fp64 oracle: the
shared-context call, the branch call (branches of several chunks, so it
segments too), per-key decay, and checkpoints across segment boundaries.
"""

import contextlib
import os

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_recurrent_gdn_amd as gdn
from test_gpu_prefill import (DEV, TOL, compare, dev_io, f32, i32, run_fork, run_oracle,
                              window_to_bits)

pytestmark = pytest.mark.gpu

ENV = "GDN_PREFILL_SEGMENT_RECORD_BYTES"


@contextlib.contextmanager
def segment_bound(nbytes):
    old = os.environ.get(ENV)
    os.environ[ENV] = str(nbytes)
    try:
        yield
    finally:
        if old is None:
            del os.environ[ENV]
        else:
            os.environ[ENV] = old


def outputs_equal(a, b):
    for name in ("o_p", "st", "o_b", "st_b"):
        assert np.array_equal(a[name], b[name], equal_nan=True), name
    for name in ("win", "win_b"):
        assert np.array_equal(window_to_bits(a[name]), window_to_bits(b[name])), name


@pytest.mark.parametrize("variant", ["gdn", "kda"])
def test_segmented_fork_is_bitwise_one_segment(variant):
    prefix = [1100, 64, 300, 7, 0, 640]
    branches = [5, 130, 64, 200, 0, 129, 70]
    parent = [0, 0, 1, 2, 3, 5, 5]
    H, d = 2, 128
    inp = gi.seq_inputs(prefix, branches, parent, H, d, d, io="bf16", conv=True,
                        per_key=variant != "gdn", seed=17)
    one = run_fork(inp, variant=variant)
    # the bound below gives every call the most segments its sizes allow
    # (one per chunk of an average sequence)
    with segment_bound(1):
        npre = gdn.prefill_workspace_bytes(inp.Np, len(prefix), H, d, d, variant=variant)
        seg = run_fork(inp, variant=variant)
    assert npre < gdn.prefill_workspace_bytes(inp.Np, len(prefix), H, d, d, variant=variant)
    outputs_equal(seg, one)
    compare(seg, run_oracle(inp, variant=variant), inp, TOL)


def test_segmented_checkpoints_are_bitwise_one_segment():
    """Checkpoints every 2 chunks of sequences 8-9 chunks long, with the
    prefill in segments of about 2 chunks each: the checkpoints and the
    final states fall on and between segment boundaries and equal the
    one-segment run bit for bit."""
    d, H, every, cap = 64, 2, 2, 4
    prefix = [520, 576, 130]
    inp = gi.seq_inputs(prefix, [], [], H, d, d, io="bf16", conv=True, seed=23)
    R, Np, cc = len(prefix), inp.Np, H * 3 * d
    q, k, v = (dev_io(getattr(inp, n), getattr(inp, n + "_bits")) for n in "qkv")
    la, beta, conv_w = f32(inp.log_alpha), f32(inp.beta), f32(inp.conv_w)

    def run():
        st = torch.empty((R, H, d, d), device=DEV)
        ck = torch.full((R, cap, H, d, d), 7.0, device=DEV)
        ckw = torch.zeros((R, cap, 3, cc), device=DEV, dtype=torch.bfloat16)
        o = torch.empty((Np, H, d), device=DEV)
        gdn.gdn_prefill_checkpointed(q, k, v, la, beta, i32(inp.cu_seqlens), st, every, ck, o=o,
                                     ckpt_window=ckw, conv_w=conv_w, qk_l2norm=True)
        torch.cuda.synchronize()
        return st.cpu().numpy(), ck.cpu().numpy(), window_to_bits(ckw), o.cpu().numpy()

    one = run()
    with segment_bound(1):
        seg = run()
    for x, y in zip(seg, one):
        assert np.array_equal(x, y)
