"""Benchmark of the GDN decode / fork hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--fork-reps R] [--no-cpu]

Headline workload (one JSON line on stdout): large-batch decode under the
deferred base + log schedule -- B=256 sequences, H=32 heads, d_k=d_v=128,
merge every M=8 steps with per-slot log phases (each slot starts with a
pre-populated log of 0..M-1 entries, so every step merges a different
eighth of the slots), bf16 q/k/v, fp32 state, fp32 o. A step is one
deltalog_append_decode launch over the whole batch (8192 head-steps); all
512 steps of inputs are pre-staged in HBM and the timed region cycles
through them. `value` is head-steps per second.

Alongside: the eager step on the same workload (state-write ratio and
speedup), the two-call fork (8 requests x 8192-token contexts, 20 branches
of 64 tokens each, H=16, d=128, conv width 4) as branches per second, the
softmax-attention half of the fork on the same stream (one fork-attention
call over trunks and branches), the per-key decode workload (KDA and the
RWKV6-style update, B=128, H=32, M=8), the small decode workload launched
plainly and as one replayed HIP graph, the roofline of the deferred kernel
from HIP events on its stream, and the fp64 CPU oracle timed on a bounded
sample of the same decode workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD public figure

METRIC = "GDN decode head-steps/s + achieved HBM GB/s (DeltaLog M=8); fork branches/s"

# algorithmic bytes of one head-step (d_k = d_v = 128, bf16 q/k/v, fp32 o,
# fp32 state / log_u / log_lambda, bf16 log_k, scalar decay)
D = 128
STATE_B = 4 * D * D                # one fp32 [d_k][d_v] state tile
QKV_B = 2 * 3 * D                  # bf16 q, k, v
SCAL_B = 4 + 4                     # log_alpha, beta
O_B = 4 * D                        # fp32 o
LEN_B = 4 + 4                      # log length read + write
ENTRY_B = 4 * D + 2 * D + 4        # one log entry: u (fp32), k (bf16), Lambda (fp32)


def entry_bytes(per_key=False):
    """One log entry; a per-key entry keeps a d_k-vector of cumulative
    log-decay in place of the scalar."""
    return ENTRY_B + (4 * D - 4 if per_key else 0)


def deferred_bytes(m, merges, per_key=False, has_beta=True):
    """Bytes one head-step moves under the deferred schedule with m logged
    entries: base read, inputs, replay of m entries, o, and either a base
    write (merging step) or one appended entry. Per-key decay reads a
    d_k-vector of log a per step; the RWKV6-style update reads no beta."""
    e = entry_bytes(per_key)
    scal = (4 * D if per_key else 4) + (4 if has_beta else 0)
    return STATE_B + QKV_B + scal + O_B + LEN_B + e * m + (STATE_B if merges else e)


def eager_bytes():
    return 2 * STATE_B + QKV_B + SCAL_B + O_B


def state_write_bytes(merges, per_key=False):
    """Bytes of recurrent state written per head-step: base and log."""
    return STATE_B if merges else entry_bytes(per_key)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--fork-reps", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-fork", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target duration of the CPU oracle sample")
    ap.add_argument("--only-attention", action="store_true",
                    help="profiling aid: run only the fork-attention round (warmup + steps "
                         "calls), report its time on stderr, print no JSON line")
    ap.add_argument("--attention-requests", type=int, default=None,
                    help="with --only-attention: requests of the fork_prefill shape (default 8)")
    ap.add_argument("--only-fork", action="store_true",
                    help="profiling aid: run only the two-call fork (fork-reps timed rounds) "
                         "and the device-copy probe, report on stderr, print no JSON line")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Timer:
    """HIP events on the stream the kernels are launched on."""

    def __init__(self, torch, stream):
        self.torch = torch
        self.stream = stream
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.torch.cuda.synchronize()
        self.a.record(self.stream)
        return self

    def __exit__(self, *exc):
        self.b.record(self.stream)
        self.torch.cuda.synchronize()
        self.ms = self.a.elapsed_time(self.b)


# ---------------------------------------------------------------- decode
def setup_decode(torch, gdn, gi, B=256, H=32, steps=512, M=8, seed=0, per_key=False):
    dev = "cuda"
    t = gi.torch_decode_inputs(B, H, D, D, steps, per_key=per_key, seed=seed)
    rng = np.random.default_rng(seed + 1)
    phase = rng.integers(0, M, size=B)
    lengths = np.repeat(phase, H)
    ent = gi.log_entries(rng, B * H, M, D, D, lengths, per_key=per_key, io="bf16")
    logs = dict(
        log_u=torch.from_numpy(ent["u"]).to(dev).view(B, H, M, D),
        log_k=torch.from_numpy(ent["k_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
        .view(B, H, M, D),
        log_lam=torch.from_numpy(ent["lam"]).to(dev).view((B, H, M, D) if per_key else (B, H, M)),
        log_len=torch.from_numpy(lengths.astype(np.int32)).to(dev).view(B, H),
    )
    return t, logs, phase


def run_deferred(torch, gdn, t, logs, base, o, M, steps_range, variant="gdn"):
    S = t["q"].shape[0]
    for i in steps_range:
        s = i % S
        gdn.deltalog_append_decode(t["q"][s], t["k"][s], t["v"][s], t["log_alpha"][s],
                                   None if variant == "rwkv6" else t["beta"][s], base,
                                   logs["log_u"], logs["log_k"], logs["log_lam"],
                                   logs["log_len"], o, merge_at=M, variant=variant)


def run_eager(torch, gdn, t, state, o, steps_range):
    S = t["q"].shape[0]
    for i in steps_range:
        s = i % S
        gdn.gdn_decode_eager(t["q"][s], t["k"][s], t["v"][s], t["log_alpha"][s], t["beta"][s],
                             state, o)


def schedule_bytes(phase, H, M, first, K, per_key=False, has_beta=True):
    """Exact algorithmic bytes of K deferred steps starting at step `first`,
    from the deterministic per-slot log lengths; plus state-write bytes."""
    m = np.asarray(phase, dtype=np.int64).copy()
    for _ in range(first):
        m = np.where(m + 1 >= M, 0, m + 1)
    total = 0
    writes = 0
    for _ in range(K):
        merges = m + 1 >= M
        total += int(sum(deferred_bytes(int(mi), bool(mg), per_key, has_beta)
                         for mi, mg in zip(m, merges))) * H
        writes += int(sum(state_write_bytes(bool(mg), per_key) for mg in merges)) * H
        m = np.where(merges, 0, m + 1)
    return total, writes


# ---------------------------------------------------------------- fork
def bench_fork(torch, gdn, gi, reps, variant="gdn"):
    w = gi.WORKLOADS["fork_prefill"]
    R, H, d = w["R"], w["H"], w["d"]
    pl, bl, par = gi.fork_layout(R, w["prefix"], w["branches_per_req"], w["branch_len"])
    t = gi.torch_seq_inputs(pl, bl, par, H, d, d, conv=True, per_key=variant != "gdn", seed=0)
    Np, Nb, NB = t["Np"], t["Nb"], len(bl)
    cc = H * 3 * d
    dev = "cuda"
    st = torch.empty((R, H, d, d), device=dev)
    win = torch.empty((R, 3, cc), device=dev, dtype=torch.bfloat16)
    o_p = torch.empty((Np, H, d), device=dev)
    o_b = torch.empty((Nb, H, d), device=dev)
    ws = torch.empty(max(gdn.prefill_workspace_bytes(max(Np, Nb), max(R, NB), H, d, d,
                                                      variant=variant), 1),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def prefill():
        gdn.gdn_prefill_shared(t["q"][:Np], t["k"][:Np], t["v"][:Np], t["log_alpha"][:Np],
                               t["beta"][:Np], t["cu_seqlens"], st, o=o_p, conv_w=t["conv_w"],
                               qk_l2norm=True, final_window=win, workspace=ws, variant=variant)

    # call 2 as timed: o of every branch token. A caller that goes on
    # decoding from the branches also wants each branch's final state and
    # conv window; that variant is timed alongside.
    b_st = torch.empty((NB, H, d, d), device=dev)
    b_win = torch.empty((NB, 3, cc), device=dev, dtype=torch.bfloat16)

    def fork(states=False):
        gdn.gdn_fork_branches(t["q"][Np:], t["k"][Np:], t["v"][Np:], t["log_alpha"][Np:],
                              t["beta"][Np:], t["branch_cu"], t["branch_parent"], st, o_b,
                              parent_window=win, branch_state=b_st if states else None,
                              branch_window=b_win if states else None, conv_w=t["conv_w"],
                              qk_l2norm=True, workspace=ws, variant=variant)

    # three untimed rounds first (the timed calls each start from an idle
    # GPU, so the first rounds after the input staging run below the steady
    # clock); the median over the timed rounds is reported
    for _ in range(3):
        prefill()
        fork()
        fork(states=True)
    tp, tf, tfs = [], [], []
    for _ in range(reps):
        with Timer(torch, stream) as a:
            prefill()
        with Timer(torch, stream) as b:
            fork()
        with Timer(torch, stream) as c:
            fork(states=True)
        tp.append(a.ms)
        tf.append(b.ms)
        tfs.append(c.ms)
    tp_ms, tf_ms, tfs_ms = float(np.median(tp)), float(np.median(tf)), float(np.median(tfs))
    # dense-tile work of the chunked form per token-head (d_k = d_v = d,
    # chunk C): 5Cd + 3d^2 + C^2/6 multiply-adds; split-bf16 issues 3x
    C = w["chunk"]
    mac = 5 * C * d + 3 * d * d + C * C / 6
    pre_tflops = Np * H * 2 * mac / (tp_ms / 1e3) / 1e12
    # roofline of call 1 (plan + prep + scan): HBM-bound at the algorithmic
    # level (about 141 issued FLOP per byte against the bf16 ridge of
    # 2500 / 8 = 312): bytes the recurrence must move per token-head are q,
    # k, v (bf16), log a and beta (fp32), o (fp32)
    alg_bytes = Np * H * (3 * d * 2 + 8 + d * 4)
    achieved = alg_bytes / (tp_ms / 1e3) / 1e9
    traffic = prefill_traffic() if variant == "gdn" else None
    roofline = {"bound": "hbm", "kernels": "plan + prep + scan (the prefix prefill call)",
                "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS, "algorithmic_bytes": alg_bytes,
                "traffic": traffic,
                "traffic_over_algorithmic": None if traffic is None else traffic / alg_bytes}
    # roofline of call 2 (the one-chunk kernel for these one-chunk
    # branches): the same algorithmic bytes per branch token-head plus each
    # parent's state once per (parent, head)
    b_alg = Nb * H * (3 * d * 2 + 8 + d * 4) + R * H * d * d * 4
    b_ach = b_alg / (tf_ms / 1e3) / 1e9
    b_traffic = one_chunk_traffic() if variant == "gdn" else None
    b_roofline = {"bound": "hbm", "kernels": "the branch call (one-chunk kernel and the empty "
                  "chunked-path launches)", "achieved": b_ach, "peak": HBM_PEAK_GBPS,
                  "unit": "GB/s", "frac": b_ach / HBM_PEAK_GBPS, "algorithmic_bytes": b_alg,
                  "traffic": b_traffic,
                  "traffic_over_algorithmic": None if b_traffic is None else b_traffic / b_alg}
    return dict(branches=NB, prefill_ms=tp_ms, fork_ms=tf_ms, prefill_roofline=roofline,
                branch_roofline=b_roofline,
                fork_with_states_ms=tfs_ms,
                branches_per_s_with_states=NB / ((tp_ms + tfs_ms) / 1e3),
                prefill_dense_tile_tflops=pre_tflops,
                prefill_mfma_issued_tflops=3 * pre_tflops,
                prefill_mfma_frac_of_bf16_peak=3 * pre_tflops / BF16_MFMA_PEAK_TFLOPS,
                branches_per_s=NB / ((tp_ms + tf_ms) / 1e3),
                branch_phase_branches_per_s=NB / (tf_ms / 1e3),
                prefix_token_heads_per_s=Np * H / (tp_ms / 1e3))


# ---------------------------------------------------------------- fork attention
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, AMD public figure


def bench_fork_attention(torch, gdn, gi, reps, warmup=1, branches_only=True, requests=None):
    """The softmax-attention half of the fork on the fork_prefill stream (8
    requests x 8192-token trunks, 20 branches of 64 tokens each, H=16, d=128,
    bf16): one gdn_fork_attention call over the whole stream (trunks and
    branches), and the branch round alone (trunks as keys only). `requests`
    takes fewer requests of the same shape (a shorter launch, e.g. for
    counters that would saturate on the full round)."""
    w = gi.WORKLOADS["fork_prefill"]
    R, H, d, P, Lb = w["R"], w["H"], w["d"], w["prefix"], w["branch_len"]
    R = R if requests is None else requests
    pl, bl, par = gi.fork_layout(R, P, w["branches_per_req"], Lb)
    t = gi.torch_attention_inputs(pl, bl, par, H=H, Hkv=H, d=d, seed=0)
    N, NB = t["q"].shape[0], len(bl)
    o = torch.empty((N, H, d), device="cuda")
    ws = torch.empty(gdn.fork_attention_workspace_bytes(R, NB), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    # useful flops: per (query, visible key, head), q.k and p.v, 2 * 2 * d
    trunk_pairs = R * P * (P + 1) // 2
    branch_pairs = NB * (Lb * P + Lb * (Lb + 1) // 2)
    out = {}
    legs = [("round", True, trunk_pairs + branch_pairs)]
    if branches_only:
        legs.append(("branches_only", False, branch_pairs))
    for name, tq, pairs in legs:
        def call():
            gdn.gdn_fork_attention(t["q"], t["k"], t["v"], t["cu"], o, t["bcu"], t["bpar"],
                                   trunk_queries=tq, workspace=ws)
        for _ in range(warmup):
            call()
        ts = []
        for _ in range(reps):
            with Timer(torch, stream) as a:
                call()
            ts.append(a.ms)
        ms = float(np.median(ts))
        useful = pairs * H * 4 * d / (ms / 1e3) / 1e12
        out[name] = dict(ms=ms, branches_per_s=NB / (ms / 1e3), useful_tflops=useful,
                         mfma_issued_tflops=1.5 * useful,
                         frac_of_bf16_peak=1.5 * useful / BF16_MFMA_PEAK_TFLOPS)
    out["workload"] = (f"fork attention: {R} x 8192-token trunks + {NB} branches x 64 tokens, "
                       "H=16, d=128, bf16 q/k/v, fp32 o; split-bf16 probabilities (the "
                       "p.v products issue 2 MFMAs, so issued = 1.5 x useful)")
    return out


# ---------------------------------------------------------------- per-key decode
def bench_decode_perkey(torch, gdn, gi, variant, K=64, W=16):
    """The per-key decode workload (B=128, H=32, d=128, per-key log a, M=8
    with per-slot log phases): deferred steps of the KDA delta rule or of
    the RWKV6-style raw value update, head-steps/s and algorithmic GB/s."""
    w = gi.WORKLOADS["perkey"]
    B, H, T, M = w["B"], w["H"], w["steps"], w["M"]
    t, logs, phase = setup_decode(torch, gdn, gi, B, H, T, M, per_key=True)
    base = t["state0"].clone()
    o = torch.empty((B, H, D), device="cuda")
    stream = torch.cuda.current_stream()
    run_deferred(torch, gdn, t, logs, base, o, M, range(W), variant)
    with Timer(torch, stream) as tm:
        run_deferred(torch, gdn, t, logs, base, o, M, range(W, W + K), variant)
    alg, writes = schedule_bytes(phase, H, M, W, K, per_key=True, has_beta=variant != "rwkv6")
    # eager on the same inputs
    state = t["state0"].clone()
    beta = None if variant == "rwkv6" else t["beta"]

    def eager(rng):
        for i in rng:
            s = i % T
            gdn.gdn_decode_eager(t["q"][s], t["k"][s], t["v"][s], t["log_alpha"][s],
                                 None if beta is None else beta[s], state, o, variant=variant)
    eager(range(W))
    with Timer(torch, stream) as te:
        eager(range(W, W + K))
    hs = B * H * K
    eager_b = 2 * STATE_B + QKV_B + 4 * D + (4 if beta is not None else 0) + O_B
    return dict(workload=f"perkey {variant}: deferred M=8, B={B}, H={H}, d=128, per-key "
                         "log a, per-slot log phases",
                value=hs / (tm.ms / 1e3), unit="head-steps/s",
                us_per_step=tm.ms * 1e3 / K, hbm_gbps_effective=alg / (tm.ms / 1e3) / 1e9,
                eager_head_steps_per_s=hs / (te.ms / 1e3), eager_us_per_step=te.ms * 1e3 / K,
                eager_gbps_effective=eager_b * hs / (te.ms / 1e3) / 1e9,
                speedup_deferred_vs_eager=te.ms / tm.ms,
                state_write_ratio_eager_vs_deferred=STATE_B * hs / writes)


# ---------------------------------------------------------------- decode_small
def bench_decode_small(torch, gdn, gi, reps=5):
    """The small decode workload (B=64, H=16, d=128: a 64 MiB state that the
    256 MB last-level cache holds), 256 steps from empty logs: eager and the
    deferred schedule with M in {1, 4, 8, 16}, each launched one call at a
    time and as one captured HIP graph replayed (the steps are short enough
    that launch gaps matter); head-steps/s, algorithmic GB/s and state-write
    bytes per head-step."""
    w = gi.WORKLOADS["decode_small"]
    B, H, d, T = w["B"], w["H"], w["d"], w["steps"]
    t = gi.torch_decode_inputs(B, H, d, d, T, seed=0)
    o = torch.empty((B, H, d), device="cuda")
    stream = torch.cuda.current_stream()
    hs = B * H * T
    zero = np.zeros(B, dtype=np.int64)

    def timed(steps):
        steps()
        plain = []
        for _ in range(reps):
            with Timer(torch, stream) as a:
                steps()
            plain.append(a.ms)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            steps()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            steps()
        graph.replay()
        graphed = []
        for _ in range(reps):
            with Timer(torch, stream) as a:
                graph.replay()
            graphed.append(a.ms)
        return float(np.median(plain)), float(np.median(graphed))

    out = {"workload": "decode_small: B=64, H=16, d=128, 256 steps from empty logs "
                       "(64 MiB state, cache-resident)"}
    cases = [("eager", None)] + [(f"M={M}", M) for M in w["Ms"]]
    for name, M in cases:
        if M is None:
            state = t["state0"].clone()

            def steps():
                run_eager(torch, gdn, t, state, o, range(T))
            nbytes, writes = eager_bytes() * hs, STATE_B * hs
        else:
            base = t["state0"].clone()
            logs = dict(log_u=torch.zeros((B, H, M, d), device="cuda"),
                        log_k=torch.zeros((B, H, M, d), device="cuda", dtype=torch.bfloat16),
                        log_lam=torch.zeros((B, H, M), device="cuda"),
                        log_len=torch.zeros((B, H), device="cuda", dtype=torch.int32))

            def steps(base=base, logs=logs, M=M):
                run_deferred(torch, gdn, t, logs, base, o, M, range(T))
            nbytes, writes = schedule_bytes(zero, H, M, 0, T)
        p_ms, g_ms = timed(steps)
        out[name] = dict(plain_head_steps_per_s=hs / (p_ms / 1e3), plain_us_per_step=p_ms * 1e3 / T,
                         graph_head_steps_per_s=hs / (g_ms / 1e3), graph_us_per_step=g_ms * 1e3 / T,
                         graph_gbps_effective=nbytes / (g_ms / 1e3) / 1e9,
                         state_write_bytes_per_head_step=writes / hs)
    return out


# ---------------------------------------------------------------- HBM probe
def stream_probe(torch, gdn, stream, nbytes=4 << 30, reps=5):
    """Attainable HBM rate measured with the library's streaming probe
    (gdn_stream_probe: the decode step's access form, non-temporal 16-byte
    loads / stores over a 4 GiB buffer, far beyond the caches): read-only and
    copy (read + write bytes both counted), best of reps."""
    a = torch.rand(nbytes // 4, device="cuda")
    b = torch.empty_like(a)
    gdn.gdn_stream_probe(a, b, copy=False)
    gdn.gdn_stream_probe(a, b, copy=True)
    read, copy = [], []
    for _ in range(reps):
        with Timer(torch, stream) as t:
            gdn.gdn_stream_probe(a, b, copy=False)
        read.append(nbytes / (t.ms / 1e3) / 1e9)
        with Timer(torch, stream) as t:
            gdn.gdn_stream_probe(a, b, copy=True)
        copy.append(2 * nbytes / (t.ms / 1e3) / 1e9)
    del a, b
    return dict(read_gbps=max(read), copy_gbps=max(copy), bytes=nbytes)


def hbm_probe(torch, stream, nbytes=4 << 30, reps=5):
    """Reference rates of two library kernels on this GPU: torch's device
    copy (read + write nbytes each) and torch's sum over nbytes, best of
    reps. They are what those library kernels reach, not the attainable HBM
    bandwidth (the deferred decode kernel streams faster than both); the
    copy also calibrates the FETCH_SIZE / WRITE_SIZE counters."""
    n = nbytes // 4
    a = torch.rand(n, device="cuda")
    b = torch.empty_like(a)
    copy, read = [], []
    b.copy_(a)
    a.sum()
    for _ in range(reps):
        with Timer(torch, stream) as t:
            b.copy_(a)
        copy.append(2 * nbytes / (t.ms / 1e3) / 1e9)
        with Timer(torch, stream) as t:
            a.sum()
        read.append(nbytes / (t.ms / 1e3) / 1e9)
    del a, b
    return dict(torch_copy_gbps=max(copy), torch_sum_read_gbps=max(read), bytes=nbytes,
                note="library kernels (torch copy_ / sum), not an attainable-bandwidth bound")


# ---------------------------------------------------------------- CPU oracle
def cpu_baseline(torch, t, target_s):
    """The fp64 oracle (plain step-by-step recurrence) on a bounded sample
    of the decode workload: the first b sequences (all heads, all staged
    steps), b chosen from a calibration run to take about target_s."""
    import oracle

    steps, B, H = t["q"].shape[:3]

    def sample(b, nsteps):
        host = lambda x: x[:nsteps, :b].float().cpu().numpy().astype(np.float64)  # noqa: E731
        return (host(t["q"]), host(t["k"]), host(t["v"]), host(t["log_alpha"]), host(t["beta"]),
                t["state0"][:b].cpu().numpy().astype(np.float64))

    threads = oracle.max_threads()
    q, k, v, la, be, s0 = sample(2, 64)
    t0 = time.perf_counter()
    oracle.decode(q, k, v, la, be, s0, nthreads=threads)
    rate = 2 * H * 64 / (time.perf_counter() - t0)
    b = int(max(1, min(B, target_s * rate / (H * steps))))
    q, k, v, la, be, s0 = sample(b, steps)
    t0 = time.perf_counter()
    oracle.decode(q, k, v, la, be, s0, nthreads=threads)
    dt = time.perf_counter() - t0
    hs = b * H * steps
    # one thread, on a small sample
    q, k, v, la, be, s0 = sample(1, 64)
    t0 = time.perf_counter()
    oracle.decode(q, k, v, la, be, s0, nthreads=1)
    one = H * 64 / (time.perf_counter() - t0)
    return dict(value=hs / dt, unit="head-steps/s", cores=threads, kind="oracle",
                sample=f"{b} of {B} sequences x {H} heads x {steps} steps ({hs} head-steps, "
                       f"plain fp64 recurrence, {dt:.1f} s)",
                value_one_thread=one, sample_one_thread=f"1 sequence x {H} heads x 64 steps")


def cpu_fork_baseline(torch, gi):
    """The fp64 oracle on a bounded sample of the fork workload: one request
    of the fork_prefill stream cut to a 1024-token context, its 20 branches
    of 64 tokens, all 16 heads (prefill + branches, conv, q/k norm)."""
    import oracle

    w = gi.WORKLOADS["fork_prefill"]
    prefix = 1024
    pl, bl, par = gi.fork_layout(1, prefix, w["branches_per_req"], w["branch_len"])
    inp = gi.seq_inputs(pl, bl, par, w["H"], w["d"], w["d"], io="bf16", conv=True,
                        la_range=w["la_range"], seed=0)
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    _, st, win = oracle.prefill(inp.q[:prefix], inp.k[:prefix], inp.v[:prefix],
                                inp.log_alpha[:prefix], inp.beta[:prefix], inp.cu_seqlens,
                                conv_w=inp.conv_w, qk_norm=True, nthreads=threads)
    oracle.fork(inp.q[prefix:], inp.k[prefix:], inp.v[prefix:], inp.log_alpha[prefix:],
                inp.beta[prefix:], inp.branch_cu, inp.branch_parent, st, parent_window=win,
                conv_w=inp.conv_w, qk_norm=True, nthreads=threads)
    dt = time.perf_counter() - t0
    nb = len(bl)
    toks = (prefix + nb * w["branch_len"]) * w["H"]
    return dict(branches_per_s=nb / dt, token_heads_per_s=toks / dt, cores=threads,
                sample=f"1 request, {prefix}-token context + {nb} branches x "
                       f"{w['branch_len']} tokens, H={w['H']}, d={w['d']} ({dt:.1f} s)")


def prefill_traffic():
    """HBM bytes of one prefix prefill call on fork_prefill (prep + scan)
    from the committed counter summaries, or None when the prefill sources
    changed since the counters were taken."""
    from linear_attention_recurrent_gdn_amd import profiling

    here = os.path.dirname(os.path.abspath(__file__))
    total = 0.0
    for name in ("fork_prefill_prep_traffic.md", "fork_prefill_scan_traffic.md"):
        prof = profiling.read_profile_block(os.path.join(here, "profiles", name))
        if not prof or prof.get("source_hash") != profiling.source_hash(profiling.PREFILL_SOURCES):
            return None
        total += prof["traffic_bytes"] * prof.get("dispatches_per_call", 1)
    return total


def one_chunk_traffic():
    """HBM bytes of the branch call's one-chunk kernel on fork_prefill from
    the committed counter summary, or None when the prefill sources changed
    since the counters were taken."""
    from linear_attention_recurrent_gdn_amd import profiling

    here = os.path.dirname(os.path.abspath(__file__))
    prof = profiling.read_profile_block(
        os.path.join(here, "profiles", "fork_branches_one_chunk_traffic.md"))
    if not prof or prof.get("source_hash") != profiling.source_hash(profiling.PREFILL_SOURCES):
        return None
    return prof["traffic_bytes"]


def measured_traffic(ms_per_launch):
    """HBM bytes per launch of the deferred kernel from the committed
    counter summary (two rocprofv3 --pmc passes, copy-calibrated), or None
    when the decode sources changed since the counters were taken."""
    from linear_attention_recurrent_gdn_amd import profiling

    here = os.path.dirname(os.path.abspath(__file__))
    prof = profiling.read_profile_block(os.path.join(here, "profiles", "decode_large_traffic.md"))
    if not prof or prof.get("source_hash") != profiling.source_hash(profiling.DECODE_SOURCES):
        return None, None
    t = prof["traffic_bytes"]
    return t, t / (ms_per_launch / 1e3) / 1e9


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): this library "
              "has no multi-GPU path. Decode slot-heads and fork requests would shard across "
              "GPUs with no exchange, each GPU running the one-GPU kernels on its share.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import gdn_inputs as gi
    import linear_attention_recurrent_gdn_amd as gdn

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    gdn.load()
    torch.manual_seed(0)
    if args.only_fork:
        res = bench_fork(torch, gdn, gi, args.fork_reps)
        res["hbm_probe"] = hbm_probe(torch, torch.cuda.current_stream())
        log(json.dumps(res))
        return
    if args.only_attention:
        res = bench_fork_attention(torch, gdn, gi, max(args.steps, 1), warmup=args.warmup,
                                   branches_only=False, requests=args.attention_requests)
        log(json.dumps(res))
        return
    B, H, M, NSTEP = 256, 32, 8, 512
    K, W = args.steps, args.warmup
    stream = torch.cuda.current_stream()

    log("staging decode inputs ...")
    t, logs, phase = setup_decode(torch, gdn, gi, B, H, NSTEP, M)
    base = t["state0"].clone()
    o = torch.empty((B, H, D), device="cuda")

    log(f"deferred decode: {W} warmup + {K} timed steps")
    run_deferred(torch, gdn, t, logs, base, o, M, range(W))
    with Timer(torch, stream) as tm:
        run_deferred(torch, gdn, t, logs, base, o, M, range(W, W + K))
    ms_step = tm.ms / K
    head_steps = B * H * K
    value = head_steps / (tm.ms / 1e3)
    alg_bytes, state_writes = schedule_bytes(phase, H, M, W, K)
    achieved = alg_bytes / (tm.ms / 1e3) / 1e9
    traffic, traffic_gbps = measured_traffic(ms_step)

    log("eager decode on the same workload")
    state = t["state0"].clone()
    run_eager(torch, gdn, t, state, o, range(W))
    with Timer(torch, stream) as te:
        run_eager(torch, gdn, t, state, o, range(W, W + K))
    eager_value = head_steps / (te.ms / 1e3)
    eager_gbps = eager_bytes() * head_steps / (te.ms / 1e3) / 1e9
    eager_writes = STATE_B * head_steps

    fork = fork_kda = None
    if not args.no_fork:
        log("two-call fork ...")
        fork = bench_fork(torch, gdn, gi, args.fork_reps)
        log("two-call fork, per-key decay (KDA) ...")
        fork_kda = bench_fork(torch, gdn, gi, args.fork_reps, variant="kda")

    fork_attn = None
    if not args.no_fork:
        log("fork attention ...")
        fork_attn = bench_fork_attention(torch, gdn, gi, args.fork_reps)
        torch.cuda.empty_cache()

    log("per-key decode (KDA, RWKV6-style) ...")
    perkey = {v: bench_decode_perkey(torch, gdn, gi, v) for v in ("kda", "rwkv6")}
    torch.cuda.empty_cache()

    log("decode_small, plain launches and one captured graph ...")
    small = bench_decode_small(torch, gdn, gi)

    probe = hbm_probe(torch, stream)
    probe["stream"] = stream_probe(torch, gdn, stream)

    cpu = None
    if not args.no_cpu:
        log("CPU oracle baseline ...")
        cpu = cpu_baseline(torch, t, args.cpu_seconds)
        cpu["fork"] = cpu_fork_baseline(torch, gi)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "head-steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "decode_large: deferred base+log decode, B=256, H=32, d_k=d_v=128, "
                        "merge every M=8 steps with per-slot log phases, bf16 q/k/v, fp32 "
                        "state and o, 512 pre-staged steps",
            "B": B, "H": H, "d_k": D, "d_v": D, "M": M, "io": "bf16", "state": "f32",
        },
        "hbm_gbps_effective": achieved,
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_kernel<128,128,GDN,bf16,f32,append>",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE/WRITE_SIZE, copy-calibrated)",
            "traffic_gbps": traffic_gbps,
            "bytes_per_launch": alg_bytes / K,
            "launch_ms": ms_step,
            # attainable rates measured in this run with the library's
            # streaming probe (same access form, 4 GiB buffer)
            "measured_read_gbps": probe["stream"]["read_gbps"],
            "measured_copy_gbps": probe["stream"]["copy_gbps"],
            "frac_of_measured_read": achieved / probe["stream"]["read_gbps"],
        },
        "eager": {"value": eager_value, "unit": "head-steps/s", "ms_per_step": te.ms / K,
                  "hbm_gbps_effective": eager_gbps,
                  "speedup_deferred_vs_eager": value / eager_value},
        "state_write_bytes_per_head_step": {
            "deferred": state_writes / head_steps, "eager": eager_writes / head_steps,
            "ratio": eager_writes / state_writes},
        "fork": fork,
        "fork_kda": fork_kda,
        "fork_attention": fork_attn,
        "decode_perkey": perkey,
        "decode_small": small,
        "hbm_probe": probe,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
