"""Full-size decode workloads on the GPU, checked against the fp64 oracle.

The GPU runs every slot-head of the workload with the same calls and
launch configuration the bench times; the oracle checks the whole
workload where it finishes in seconds (decode_small) and a sample of
slots, all heads and all steps, elsewhere (decode_large, perkey).
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


def host64(x):
    return x.float().cpu().numpy().astype(np.float64)


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def test_decode_small_whole_workload():
    """B=64, H=16, d=128, 256 steps: eager and the deferred schedule with
    M in {1, 4, 8, 16} (empty logs at the start, final flush)."""
    w = gi.WORKLOADS["decode_small"]
    B, H, d, T = w["B"], w["H"], w["d"], w["steps"]
    inp = gi.decode_inputs(B, H, d, d, T, seed=0)
    o_ref, st_ref, _ = oracle.decode(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, inp.state0)
    q, k, v = bf16_dev(inp.q_bits), bf16_dev(inp.k_bits), bf16_dev(inp.v_bits)
    la = torch.from_numpy(inp.log_alpha).to(DEV)
    beta = torch.from_numpy(inp.beta).to(DEV)
    o = torch.empty((T, B, H, d), device=DEV)
    state = torch.from_numpy(inp.state0).to(DEV)
    for t in range(T):
        gdn.gdn_decode_eager(q[t], k[t], v[t], la[t], beta[t], state, o[t])
    torch.cuda.synchronize()
    cfg = "C2 decode_small (whole workload)"

    def rec(sched, o_g, st_g):
        og, sg = host64(o_g), host64(st_g)
        _parity.record(cfg, f"o {sched}", _parity.rel_err(og, o_ref, (0, 3)),
                       _parity.elementwise(og, o_ref, (0, 3)), TOL)
        _parity.record(cfg, f"state {sched}", _parity.rel_err(sg, st_ref, (2, 3)),
                       _parity.elementwise(sg, st_ref, (2, 3)), TOL)

    rec("eager", o, state)
    errs = {"eager": (oracle.rel_err(host64(o), o_ref, (0, 3)),
                      oracle.rel_err(host64(state), st_ref, (2, 3)))}
    for M in w["Ms"]:
        base = torch.from_numpy(inp.state0).to(DEV)
        log_u = torch.zeros((B, H, M, d), device=DEV)
        log_k = torch.zeros((B, H, M, d), device=DEV, dtype=torch.bfloat16)
        log_lam = torch.zeros((B, H, M), device=DEV)
        log_len = torch.zeros((B, H), device=DEV, dtype=torch.int32)
        for t in range(T):
            gdn.deltalog_append_decode(q[t], k[t], v[t], la[t], beta[t], base, log_u, log_k,
                                       log_lam, log_len, o[t], merge_at=M)
        gdn.deltalog_merge(base, log_u, log_k, log_lam, log_len, min_len=1)
        torch.cuda.synchronize()
        errs[f"M={M}"] = (oracle.rel_err(host64(o), o_ref, (0, 3)),
                          oracle.rel_err(host64(base), st_ref, (2, 3)))
        rec(f"M={M}", o, base)
    print({k_: f"o {a:.2e} state {b:.2e}" for k_, (a, b) in errs.items()}, flush=True)
    assert all(max(e) <= TOL for e in errs.values()), errs


def _sampled_deferred(B, H, d, T, M, *, per_key, variant, phases, sample, seed=0, config=None):
    t_in = gi.torch_decode_inputs(B, H, d, d, T, per_key=per_key, seed=seed)
    rng = np.random.default_rng(seed + 1)
    phase = rng.integers(0, M, size=B) if phases else np.zeros(B, dtype=np.int64)
    lengths = np.repeat(phase, H)
    ent = gi.log_entries(rng, B * H, M, d, d, lengths, per_key=per_key, io="bf16")
    base = t_in["state0"].clone()
    log_u = torch.from_numpy(ent["u"]).to(DEV).view(B, H, M, d)
    log_k = bf16_dev(ent["k_bits"]).view(B, H, M, d)
    lam_shape = (B, H, M, d) if per_key else (B, H, M)
    log_lam = torch.from_numpy(ent["lam"]).to(DEV).view(lam_shape)
    log_len = torch.from_numpy(lengths.astype(np.int32)).to(DEV).view(B, H)
    sel = torch.tensor(sample, device=DEV)
    o = torch.empty((B, H, d), device=DEV)
    o_s = torch.empty((T, len(sample), H, d), device=DEV)
    beta = None if variant == "rwkv6" else t_in["beta"]
    for t in range(T):
        gdn.deltalog_append_decode(t_in["q"][t], t_in["k"][t], t_in["v"][t],
                                   t_in["log_alpha"][t], None if beta is None else beta[t],
                                   base, log_u, log_k, log_lam, log_len, o, merge_at=M,
                                   variant=variant)
        o_s[t] = o.index_select(0, sel)
    gdn.deltalog_merge(base, log_u, log_k, log_lam, log_len, min_len=1, variant=variant)
    torch.cuda.synchronize()
    # oracle on the sampled slots: start from the logical state of base + log
    n = B * H
    idx = (np.asarray(sample)[:, None] * H + np.arange(H)[None, :]).ravel()
    lam_np = ent["lam"].reshape((n, M, d) if per_key else (n, M))
    s0 = oracle.materialize(host64(t_in["state0"].index_select(0, sel)).reshape(-1, d, d),
                            ent["u"].reshape(n, M, d)[idx], ent["k"].reshape(n, M, d)[idx],
                            lam_np[idx], lengths[idx]).reshape(len(sample), H, d, d)
    pick = lambda x: host64(x.index_select(1, sel))  # noqa: E731
    o_ref, st_ref, _ = oracle.decode(pick(t_in["q"]), pick(t_in["k"]), pick(t_in["v"]),
                                     pick(t_in["log_alpha"]),
                                     None if beta is None else pick(t_in["beta"]), s0,
                                     variant=variant)
    og, sg = host64(o_s), host64(base.index_select(0, sel))
    e_o = oracle.rel_err(og, o_ref, (0, 3))
    e_s = oracle.rel_err(sg, st_ref, (2, 3))
    if config is not None:
        _parity.record(config, "o", e_o, _parity.elementwise(og, o_ref, (0, 3)), TOL)
        _parity.record(config, "state", e_s, _parity.elementwise(sg, st_ref, (2, 3)), TOL)
    return e_o, e_s


def test_decode_large_sampled():
    """B=256, H=32, d=128, M=8 with per-slot log phases, 512 steps; the
    oracle checks 8 slots (256 slot-heads) over every step."""
    w = gi.WORKLOADS["decode_large"]
    sample = [0, 37, 101, 128, 170, 203, 241, 255]
    e_o, e_s = _sampled_deferred(w["B"], w["H"], w["d"], w["steps"], w["M"], per_key=False,
                                 variant="gdn", phases=True, sample=sample,
                                 config="C4 decode_large (8 of 256 slots, all heads and steps)")
    print(f"decode_large: o {e_o:.2e} state {e_s:.2e}", flush=True)
    assert e_o <= TOL and e_s <= TOL


@pytest.mark.parametrize("variant", ["kda", "rwkv6"])
def test_perkey_sampled(variant):
    """B=128, H=32, d=128, per-key log a, M=8, 256 steps; 8 slots checked."""
    w = gi.WORKLOADS["perkey"]
    sample = [0, 19, 50, 64, 77, 99, 111, 127]
    e_o, e_s = _sampled_deferred(w["B"], w["H"], w["d"], w["steps"], w["M"], per_key=True,
                                 variant=variant, phases=True, sample=sample,
                                 config=f"C5 perkey {variant} (8 of 128 slots, all heads and steps)")
    print(f"perkey {variant}: o {e_o:.2e} state {e_s:.2e}", flush=True)
    assert e_o <= TOL and e_s <= TOL
