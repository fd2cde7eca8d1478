"""Shared drivers for the GPU decode tests: run eager / deferred steps through
the C ABI binding and the matching fp64 oracle runs."""

import numpy as np
import torch

import gdn_inputs as gi
import linear_attention_recurrent_gdn_amd as gdn
import oracle

DEV = "cuda"
TOL = 2e-3           # max relative error per (row, head) slice
TOL_F32 = 2e-5       # the same metric for fp32 I/O


def to_dev(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype)


def io_tensor(inp, name):
    """q/k/v of a DecodeInputs as a device tensor of the io dtype (bf16 from
    the exact bit patterns)."""
    if inp.io == "bf16":
        bits = getattr(inp, name + "_bits")
        return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    return to_dev(getattr(inp, name))


def oracle_decode(inp, variant, state0=None):
    s0 = inp.state0 if state0 is None else state0
    beta = None if variant == "rwkv6" else inp.beta
    return oracle.decode(inp.q, inp.k, inp.v, inp.log_alpha, beta, s0, variant=variant,
                         want_u=True)


def gpu_eager(inp, variant, o_dtype=torch.float32, slot_idx=None, n_slots=None):
    q, k, v = io_tensor(inp, "q"), io_tensor(inp, "k"), io_tensor(inp, "v")
    la, beta = to_dev(inp.log_alpha), to_dev(inp.beta)
    B, H = inp.B, inp.H
    S = B if n_slots is None else n_slots
    state = torch.zeros((S, H, inp.dk, inp.dv), device=DEV)
    sl = None
    if slot_idx is not None:
        sl = torch.tensor(slot_idx, dtype=torch.int32, device=DEV)
        state[sl.long()] = to_dev(inp.state0)
    else:
        state[:B] = to_dev(inp.state0)
    outs = torch.empty((inp.steps, B, H, inp.dv), device=DEV, dtype=o_dtype)
    for t in range(inp.steps):
        gdn.gdn_decode_eager(q[t], k[t], v[t], la[t], None if variant == "rwkv6" else beta[t],
                             state, outs[t], slot_idx=sl, variant=variant)
    torch.cuda.synchronize()
    return outs, state


def empty_logs(S, H, Mcap, dk, dv, per_key, io_dtype):
    log_u = torch.zeros((S, H, Mcap, dv), device=DEV)
    log_k = torch.zeros((S, H, Mcap, dk), device=DEV, dtype=io_dtype)
    lam_shape = (S, H, Mcap, dk) if per_key else (S, H, Mcap)
    log_lam = torch.zeros(lam_shape, device=DEV)
    log_len = torch.zeros((S, H), device=DEV, dtype=torch.int32)
    return log_u, log_k, log_lam, log_len


def prepopulated_logs(inp, Mcap, phase, seed=1):
    """Random logs of phase[b] entries for every head of slot b (numpy) and
    the logical state they represent (oracle)."""
    rng = np.random.default_rng(seed)
    B, H = inp.B, inp.H
    n = B * H
    lengths = np.repeat(np.asarray(phase), H)
    ent = gi.log_entries(rng, n, Mcap, inp.dk, inp.dv, lengths, per_key=inp.per_key, io=inp.io)
    logical = oracle.materialize(inp.state0.reshape(n, inp.dk, inp.dv), ent["u"], ent["k"],
                                 ent["lam"], lengths)
    return ent, lengths, logical.reshape(B, H, inp.dk, inp.dv)


def gpu_deferred(inp, variant, M, ent=None, lengths=None, o_dtype=torch.float32, flush=True,
                 slot_idx=None):
    B, H, dk, dv = inp.B, inp.H, inp.dk, inp.dv
    io_dtype = torch.bfloat16 if inp.io == "bf16" else torch.float32
    q, k, v = io_tensor(inp, "q"), io_tensor(inp, "k"), io_tensor(inp, "v")
    la, beta = to_dev(inp.log_alpha), to_dev(inp.beta)
    base = to_dev(inp.state0).contiguous()
    log_u, log_k, log_lam, log_len = empty_logs(B, H, M, dk, dv, inp.per_key, io_dtype)
    if ent is not None:
        log_u.copy_(to_dev(ent["u"]).view(B, H, M, dv))
        if inp.io == "bf16":
            log_k.copy_(torch.from_numpy(ent["k_bits"].view(np.int16)).to(DEV)
                        .view(torch.bfloat16).view(B, H, M, dk))
        else:
            log_k.copy_(to_dev(ent["k"]).view(B, H, M, dk))
        log_lam.copy_(to_dev(ent["lam"]).view(log_lam.shape))
        log_len.copy_(torch.from_numpy(lengths.astype(np.int32)).to(DEV).view(B, H))
    sl = None if slot_idx is None else torch.tensor(slot_idx, dtype=torch.int32, device=DEV)
    outs = torch.empty((inp.steps, B, H, dv), device=DEV, dtype=o_dtype)
    for t in range(inp.steps):
        gdn.deltalog_append_decode(q[t], k[t], v[t], la[t],
                                   None if variant == "rwkv6" else beta[t], base, log_u, log_k,
                                   log_lam, log_len, outs[t], merge_at=M, slot_idx=sl,
                                   variant=variant)
    if flush:
        gdn.deltalog_merge(base, log_u, log_k, log_lam, log_len, min_len=1, variant=variant)
    torch.cuda.synchronize()
    return outs, base, (log_u, log_k, log_lam, log_len)


def rel_err_slices(x, ref, axes):
    return oracle.rel_err(x, ref, axes)
