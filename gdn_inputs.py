"""Seeded synthetic inputs for the GDN recurrence workloads.

This module is the one thing the oracle side and the HIP side share: it
draws random inputs and holds none of the method's arithmetic (no decay,
no state update, no convolution). Both sides receive the same arrays.

Workloads (the shapes, sizes and distributions of the five configurations
this library is measured on; the datasets the pages use are replaced by
these synthetic draws):

  tiny_fork      1 request, H=1, d=32, 128-token shared context, 4 branches
                 of 8 tokens; fp32 I/O; log a ~ U(-0.2,-0.01); no conv.
  decode_small   B=64, H=16, d=128, 256 steps; S0 ~ N(0, 0.1^2) fp32;
                 bf16 q/k/v; scalar log a ~ U(-0.1,-0.001).
  fork_prefill   8 requests x 8192-token shared context, 20 branches of 64
                 tokens per request, H=16, d=128, chunk 64, conv width 4
                 (w ~ U(-0.5,0.5)), bf16 I/O.
  decode_large   B=256, H=32, d=128, 512 steps, deferred schedule M=8 with
                 per-slot log phases (pre-populated logs of 0..M-1 entries).
  perkey         B=128, H=32, d=128, per-key log a in R^128 ~ U(-0.1,-0.001),
                 256 steps (KDA and RWKV6-style).
  fork attention the fork_prefill stream (8 x 8192-token trunks, 160
                 branches of 64 tokens) for the softmax-attention half of
                 the fork: q, k, v ~ N(0,1) per element rounded to bf16
                 (not normalised, so scores q.k/sqrt(d) spread like N(0,1)
                 and the softmax is neither flat nor one-hot), H = H_kv = 16,
                 d = 128.

Common distributions: q, k ~ N(0,1) per element, L2-normalised per
(token, head) in fp32 and then rounded to bf16 (round to nearest even);
v ~ N(0,1) rounded to bf16; beta = sigmoid(N(0,1)) fp32.
Draw order inside one workload: S0, q, k, v, log a, beta, conv w, phases,
log entries. Seed 0 unless stated.

Two back ends draw these distributions: NumPy's PCG64 for sizes the oracle
handles whole, and torch's generator on the GPU for full-size workloads,
whose oracle checks use slices copied back to the host. The two back ends
give different (equally distributed) values.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_round",
    "bf16_bits_to_f32",
    "unit_rows",
    "DecodeInputs",
    "SeqInputs",
    "decode_inputs",
    "seq_inputs",
    "log_entries",
    "torch_attention_inputs",
    "WORKLOADS",
]


# ---------------------------------------------------------------- rounding
def bf16_round(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Round to bfloat16, nearest-even. Returns (uint16 bits, float32 values)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    return r, bf16_bits_to_f32(r)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def unit_rows(x: np.ndarray) -> np.ndarray:
    """Scale each vector along the last axis to unit L2 length (fp32)."""
    x = x.astype(np.float32)
    n = np.sqrt((x * x).sum(axis=-1, keepdims=True, dtype=np.float32))
    return x / n


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


# ---------------------------------------------------------------- decode
class DecodeInputs:
    """Per-step decode inputs, every step pre-drawn.

    q, k : [steps, B, H, dk]   v : [steps, B, H, dv]   (io dtype values as
           float32; *_bits hold the bf16 bit patterns when io is bf16)
    log_alpha : [steps, B, H] or [steps, B, H, dk] float32
    beta : [steps, B, H] float32
    state0 : [B, H, dk, dv] float32
    phase : [B] int32 (initial log length per slot), or None
    """

    def __init__(self, **kw):
        self.__dict__.update(kw)


def decode_inputs(B, H, dk, dv, steps, *, per_key=False, io="bf16",
                  la_range=(-0.1, -0.001), state_std=0.1, seed=0,
                  phases_M=None) -> DecodeInputs:
    rng = np.random.default_rng(seed)
    state0 = (rng.standard_normal((B, H, dk, dv)) * state_std).astype(np.float32)
    q = unit_rows(rng.standard_normal((steps, B, H, dk), dtype=np.float32))
    k = unit_rows(rng.standard_normal((steps, B, H, dk), dtype=np.float32))
    v = rng.standard_normal((steps, B, H, dv), dtype=np.float32)
    la_shape = (steps, B, H, dk) if per_key else (steps, B, H)
    log_alpha = rng.uniform(la_range[0], la_range[1], la_shape).astype(np.float32)
    beta = _sigmoid(rng.standard_normal((steps, B, H)))
    phase = None
    if phases_M:
        phase = rng.integers(0, phases_M, size=B).astype(np.int32)
    out = dict(B=B, H=H, dk=dk, dv=dv, steps=steps, per_key=per_key, io=io,
               state0=state0, log_alpha=log_alpha, beta=beta, phase=phase,
               seed=seed)
    for name, arr in (("q", q), ("k", k), ("v", v)):
        if io == "bf16":
            bits, vals = bf16_round(arr)
            out[name], out[name + "_bits"] = vals, bits
        else:
            out[name], out[name + "_bits"] = arr, None
    return DecodeInputs(**out)


def log_entries(rng, n_units, Mcap, dk, dv, lengths, *, per_key=False,
                la_range=(-0.1, -0.001), u_std=0.5, io="bf16"):
    """Random contents for pre-populated deferred-update logs.

    Unit n holds lengths[n] entries: u ~ N(0, u_std^2) fp32, k a unit
    vector rounded to the io dtype, and a cumulative log-decay that is a
    running total of U(la_range) draws (a random decreasing sequence).
    Entries past the length are zero.
    """
    lam_shape = (n_units, Mcap, dk) if per_key else (n_units, Mcap)
    u = (rng.standard_normal((n_units, Mcap, dv)) * u_std).astype(np.float32)
    k = unit_rows(rng.standard_normal((n_units, Mcap, dk), dtype=np.float32))
    steps = rng.uniform(la_range[0], la_range[1], lam_shape)
    lam = np.cumsum(steps, axis=1).astype(np.float32)
    if io == "bf16":
        k_bits, k = bf16_round(k)
    else:
        k_bits = None
    mask = np.arange(Mcap)[None, :] < np.asarray(lengths)[:, None]
    u = np.where(mask[..., None], u, 0).astype(np.float32)
    k = np.where(mask[..., None], k, 0).astype(np.float32)
    if k_bits is not None:
        k_bits = np.where(mask[..., None], k_bits, 0).astype(np.uint16)
    lam = np.where(mask[..., None] if per_key else mask, lam, 0).astype(np.float32)
    return dict(u=u, k=k, k_bits=k_bits, lam=lam)


# ---------------------------------------------------------------- prefill / fork
class SeqInputs:
    """A flat token stream of shared contexts followed by branch tokens.

    q, k : [N, H, dk]   v : [N, H, dv]   log_alpha, beta : [N, H]
    cu_seqlens : [R+1] int32 offsets of the shared contexts in the prefix
                 stream; branch_cu : [NB+1] offsets in the branch stream;
    branch_parent : [NB] int32 request index of each branch.
    Prefix tokens are rows [0, Np), branch tokens rows [Np, Np+Nb).
    conv_w : [H*(2dk+dv), 4] float32 or None.
    """

    def __init__(self, **kw):
        self.__dict__.update(kw)

    def prefix(self, name):
        return getattr(self, name)[: self.Np]

    def branch(self, name):
        return getattr(self, name)[self.Np:]


def seq_inputs(prefix_lens, branch_lens, branch_parent, H, dk, dv, *,
               io="bf16", la_range=(-0.1, -0.001), conv=True, per_key=False, seed=0):
    rng = np.random.default_rng(seed)
    prefix_lens = np.asarray(prefix_lens, dtype=np.int64)
    branch_lens = np.asarray(branch_lens, dtype=np.int64)
    Np, Nb = int(prefix_lens.sum()), int(branch_lens.sum())
    N = Np + Nb
    q = unit_rows(rng.standard_normal((N, H, dk), dtype=np.float32))
    k = unit_rows(rng.standard_normal((N, H, dk), dtype=np.float32))
    v = rng.standard_normal((N, H, dv), dtype=np.float32)
    la_shape = (N, H, dk) if per_key else (N, H)
    log_alpha = rng.uniform(la_range[0], la_range[1], la_shape).astype(np.float32)
    beta = _sigmoid(rng.standard_normal((N, H)))
    conv_w = None
    if conv:
        conv_w = rng.uniform(-0.5, 0.5, (H * (2 * dk + dv), 4)).astype(np.float32)
    cu = np.zeros(len(prefix_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(prefix_lens)
    bcu = np.zeros(len(branch_lens) + 1, dtype=np.int32)
    bcu[1:] = np.cumsum(branch_lens)
    out = dict(H=H, dk=dk, dv=dv, io=io, Np=Np, Nb=Nb, N=N, log_alpha=log_alpha,
               beta=beta, conv_w=conv_w, cu_seqlens=cu, branch_cu=bcu,
               branch_parent=np.asarray(branch_parent, dtype=np.int32), seed=seed)
    for name, arr in (("q", q), ("k", k), ("v", v)):
        if io == "bf16":
            bits, vals = bf16_round(arr)
            out[name], out[name + "_bits"] = vals, bits
        else:
            out[name], out[name + "_bits"] = arr, None
    return SeqInputs(**out)


# ---------------------------------------------------------------- presets
WORKLOADS = {
    "tiny_fork": dict(R=1, H=1, d=32, prefix=128, branches_per_req=4,
                      branch_len=8, io="f32", la_range=(-0.2, -0.01),
                      conv=False, chunk=64),
    "decode_small": dict(B=64, H=16, d=128, steps=256, io="bf16",
                         la_range=(-0.1, -0.001), Ms=(1, 4, 8, 16)),
    "fork_prefill": dict(R=8, H=16, d=128, prefix=8192, branches_per_req=20,
                         branch_len=64, io="bf16", la_range=(-0.1, -0.001),
                         conv=True, chunk=64),
    "decode_large": dict(B=256, H=32, d=128, steps=512, io="bf16",
                         la_range=(-0.1, -0.001), M=8),
    "perkey": dict(B=128, H=32, d=128, steps=256, io="bf16",
                   la_range=(-0.1, -0.001), M=8),
}


def fork_layout(R, prefix, branches_per_req, branch_len):
    """Prefix lengths, branch lengths and parents of a uniform fork workload."""
    prefix_lens = [prefix] * R
    branch_lens = [branch_len] * (R * branches_per_req)
    parents = [r for r in range(R) for _ in range(branches_per_req)]
    return prefix_lens, branch_lens, parents


# ---------------------------------------------------------------- GPU back end
def torch_decode_inputs(B, H, dk, dv, steps, *, per_key=False, device="cuda",
                        la_range=(-0.1, -0.001), state_std=0.1, seed=0):
    """Full-size decode inputs drawn on the device with torch's generator.

    Same distributions and draw order as `decode_inputs`; q/k/v are bf16
    tensors, everything else float32.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    f32 = torch.float32
    state0 = torch.randn((B, H, dk, dv), generator=g, device=device, dtype=f32) * state_std

    def unit(shape):
        x = torch.randn(shape, generator=g, device=device, dtype=f32)
        return (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)

    q = unit((steps, B, H, dk))
    k = unit((steps, B, H, dk))
    v = torch.randn((steps, B, H, dv), generator=g, device=device, dtype=f32).to(torch.bfloat16)
    la_shape = (steps, B, H, dk) if per_key else (steps, B, H)
    lo, hi = la_range
    log_alpha = torch.rand(la_shape, generator=g, device=device, dtype=f32) * (hi - lo) + lo
    beta = torch.sigmoid(torch.randn((steps, B, H), generator=g, device=device, dtype=f32))
    return dict(state0=state0, q=q, k=k, v=v, log_alpha=log_alpha, beta=beta)


def torch_seq_inputs(prefix_lens, branch_lens, branch_parent, H, dk, dv, *, conv=True,
                     device="cuda", la_range=(-0.1, -0.001), per_key=False, seed=0):
    """Full-size flat-stream inputs drawn on the device (same distributions
    and draw order as `seq_inputs`; q/k/v bf16, the rest float32)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    f32 = torch.float32
    Np, Nb = int(sum(prefix_lens)), int(sum(branch_lens))
    N = Np + Nb

    def unit(shape):
        x = torch.randn(shape, generator=g, device=device, dtype=f32)
        return (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)

    q = unit((N, H, dk))
    k = unit((N, H, dk))
    v = torch.randn((N, H, dv), generator=g, device=device, dtype=f32).to(torch.bfloat16)
    lo, hi = la_range
    la_shape = (N, H, dk) if per_key else (N, H)
    log_alpha = torch.rand(la_shape, generator=g, device=device, dtype=f32) * (hi - lo) + lo
    beta = torch.sigmoid(torch.randn((N, H), generator=g, device=device, dtype=f32))
    conv_w = None
    if conv:
        conv_w = torch.rand((H * (2 * dk + dv), 4), generator=g, device=device, dtype=f32) - 0.5
    cu = torch.zeros(len(prefix_lens) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(prefix_lens, dtype=torch.int64), 0).to(torch.int32)
    bcu = torch.zeros(len(branch_lens) + 1, dtype=torch.int32)
    bcu[1:] = torch.cumsum(torch.tensor(branch_lens, dtype=torch.int64), 0).to(torch.int32)
    return dict(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, conv_w=conv_w,
                cu_seqlens=cu.to(device), branch_cu=bcu.to(device),
                branch_parent=torch.tensor(branch_parent, dtype=torch.int32, device=device),
                Np=Np, Nb=Nb, N=N)


def torch_attention_inputs(trunk_lens, branch_lens, branch_parent, *, H, Hkv, d,
                           order="trunks_first", device="cuda", seed=0):
    """A flat stream for fork attention, drawn on the device: q [N,H,d],
    k, v [N,Hkv,d] ~ N(0,1) rounded to bf16, and int32 device offsets
    (cu [R+1] of the trunks, bcu [NB+1] of the branches, both absolute).

    Segment contents are drawn in a fixed order (trunks, then branches) and
    then laid out: `order` "trunks_first" stores every trunk before every
    branch, "branches_first" the reverse. The same seed gives the same
    segments in either layout.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    tl = [int(x) for x in trunk_lens]
    bl = [int(x) for x in branch_lens]
    Nt, Nb = sum(tl), sum(bl)
    N = Nt + Nb

    def draw(heads):
        return torch.randn((N, heads, d), generator=g, device=device).to(torch.bfloat16)

    q, k, v = draw(H), draw(Hkv), draw(Hkv)
    if order == "trunks_first":
        t0, b0 = 0, Nt
    elif order == "branches_first":
        t0, b0 = Nb, 0
        perm = torch.cat([torch.arange(Nt, N), torch.arange(0, Nt)]).to(device)
        q, k, v = q[perm].contiguous(), k[perm].contiguous(), v[perm].contiguous()
    else:
        raise ValueError(order)
    cu = t0 + np.concatenate([[0], np.cumsum(tl)])
    bcu = b0 + np.concatenate([[0], np.cumsum(bl)])
    return dict(q=q, k=k, v=v,
                cu=torch.from_numpy(cu.astype(np.int32)).to(device),
                bcu=torch.from_numpy(bcu.astype(np.int32)).to(device),
                bpar=torch.tensor(list(branch_parent), dtype=torch.int32, device=device))
