"""The committed counter summaries back the traffic claims (CPU only).

The decode_large summaries hold HBM bytes per launch from two rocprofv3
--pmc passes (FETCH_SIZE, WRITE_SIZE, copy-calibrated). They must agree with
the algorithmic bytes of the same launches within a stated band, and the
deferred schedule must write at least 3x fewer bytes than the eager step.
A summary taken from other kernel sources (hash mismatch) is stale: the
test says so instead of judging it.
"""

import os

import numpy as np
import pytest

import bench
import gdn_inputs as gi
from linear_attention_recurrent_gdn_amd import profiling

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BAND = (0.98, 1.05)  # measured / algorithmic bytes per launch


def block(name):
    prof = profiling.read_profile_block(os.path.join(ROOT, "profiles", name))
    assert prof is not None, f"profiles/{name} missing"
    if prof["source_hash"] != profiling.source_hash(profiling.DECODE_SOURCES):
        pytest.skip(f"profiles/{name} was taken from other decode sources")
    return prof


def profiled_phases():
    # the profiled command stages decode_large exactly as the bench does
    B, H, M = 256, 32, 8
    rng = np.random.default_rng(1)
    return rng.integers(0, M, size=B), H, M


def test_deferred_traffic_matches_algorithmic_bytes():
    prof = block("decode_large_traffic.md")
    phase, H, M = profiled_phases()
    n = prof["dispatches"]  # warm-up and timed launches of the profiled run
    alg, _ = bench.schedule_bytes(phase, H, M, 0, n)
    ratio = prof["traffic_bytes"] / (alg / n)
    assert BAND[0] <= ratio <= BAND[1], ratio


def test_eager_traffic_matches_algorithmic_bytes():
    prof = block("decode_large_eager_traffic.md")
    ratio = prof["traffic_bytes"] / (bench.eager_bytes() * 256 * 32)
    assert BAND[0] <= ratio <= BAND[1], ratio


def test_deferred_writes_at_least_3x_less_than_eager():
    deferred = block("decode_large_traffic.md")["write_bytes"]
    eager = block("decode_large_eager_traffic.md")["write_bytes"]
    assert eager / deferred >= 3.0, eager / deferred


def test_workload_shapes_match_the_profiled_command():
    w = gi.WORKLOADS["decode_large"]
    assert (w["B"], w["H"], w["d"], w["M"]) == (256, 32, bench.D, 8)


def prefill_block(name):
    prof = profiling.read_profile_block(os.path.join(ROOT, "profiles", name))
    assert prof is not None, f"profiles/{name} missing"
    if prof["source_hash"] != profiling.source_hash(profiling.PREFILL_SOURCES):
        pytest.skip(f"profiles/{name} was taken from other prefill sources")
    return prof


def record_bytes(d, C):
    """Bytes of one (chunk, head) record of the scalar-decay prefill: T' and
    P as hi / lo planes of their 6 stored 16 x 32 blocks, the fp32 factor
    slot (4C floats), K and Q as hi / lo planes [C][d]."""
    return 4 * 6 * 16 * 32 * 2 + 4 * C * 4 + 4 * C * d * 2


def test_prefill_traffic_against_algorithmic_bytes():
    """The prefix prefill of fork_prefill (prep + scan, H=16, d=128, C=64,
    65,536 tokens) against the 1,288 bytes per token-head the recurrence has
    to move: q, k, v bf16 (768), log a and beta fp32 (8), o fp32 (512). The
    chunk record (written by prep, read back by the scan) is overhead; each
    kernel's reads and writes per call are held to their parts: prep reads
    q, k, log a, beta plus the conv halo (3 rows per 16-row block of q and
    k), and at most the q / k conv taps of every workgroup (4 KiB each, one
    workgroup per chunk-head; 64 KiB in all, so mostly L2 hits), and
    writes the record once; the scan reads V and the record
    once and writes o and the final states. The call runs in segments (one
    prep and one scan launch each); the state passes between consecutive
    segments through the workspace, written by one scan and read by the
    next."""
    w = gi.WORKLOADS["fork_prefill"]
    d, C, H, R, P = w["d"], w["chunk"], w["H"], w["R"], w["prefix"]
    token_heads = R * P * H
    chunk_heads = R * (P // C) * H
    prep = prefill_block("fork_prefill_prep_traffic.md")
    scan = prefill_block("fork_prefill_scan_traffic.md")
    nseg = prep.get("dispatches_per_call", 1)
    assert scan.get("dispatches_per_call", 1) == nseg

    def per_call(prof, key):
        return prof[key] * nseg

    rec = chunk_heads * record_bytes(d, C)
    qk = token_heads * 2 * d * 2
    states = R * H * d * d * 4
    carry = (nseg - 1) * states
    prep_reads = qk * (1 + 3 / 16) + token_heads * 8
    taps = chunk_heads * 2 * d * 4 * 4
    scan_reads = token_heads * d * 2 + rec + carry
    scan_writes = token_heads * d * 4 + states + carry
    r = per_call(prep, "read_bytes")
    assert 0.98 * prep_reads <= r <= 1.10 * (prep_reads + taps), r / prep_reads
    r = per_call(prep, "write_bytes") / rec
    assert abs(r - 1) < 0.02, r
    r = per_call(scan, "read_bytes") / scan_reads
    assert 0.95 <= r <= 1.10, r
    r = per_call(scan, "write_bytes") / scan_writes
    assert abs(r - 1) < 0.03, r
    alg = token_heads * 1288
    total = per_call(prep, "traffic_bytes") + per_call(scan, "traffic_bytes")
    print(f"prefix prefill in {nseg} segment(s): {total / 1e9:.2f} GB measured = "
          f"{total / alg:.2f} x the {alg / 1e9:.2f} GB algorithmic; record overhead "
          f"{2 * rec / 1e9:.2f} GB ({record_bytes(d, C) / (C * 1024):.2f} KiB per token-head, "
          f"written and read once); carried state {2 * carry / 1e6:.1f} MB")
    # the measured total is the algorithmic bytes plus the halo, the
    # record's round trip and the carried state, nothing more
    assert total <= 1.05 * (alg + 2 * rec + qk * 3 / 16 + 2 * carry), total / alg


def test_one_chunk_traffic_against_algorithmic_bytes():
    """The branch call of fork_prefill (160 branches x 64 tokens, H=16,
    d=128) in the one-chunk kernel: it reads q, k, v (bf16), log a and beta
    and each parent's state tile once per (parent, head) -- the branches of
    a parent run on one XCD and share its L2 -- and writes o; with branch
    states it also writes every branch's state and conv window. No chunk
    record: nothing else moves but the conv halo and window rows and the
    few registers the compiler spills (a few MB), held within 20 %."""
    w = gi.WORKLOADS["fork_prefill"]
    d, H, R = w["d"], w["H"], w["R"]
    NB = R * w["branches_per_req"]
    token_heads = NB * w["branch_len"] * H
    reads = token_heads * (3 * d * 2 + 8) + R * H * d * d * 4
    o = token_heads * d * 4
    plain = prefill_block("fork_branches_one_chunk_traffic.md")
    st = prefill_block("fork_branches_one_chunk_states_traffic.md")
    for prof in (plain, st):
        r = prof["read_bytes"] / reads
        assert 1.0 <= r <= 1.2, r
    r = plain["write_bytes"] / o
    assert 1.0 <= r <= 1.12, r
    states = NB * H * d * d * 4 + NB * 3 * H * 3 * d * 2
    r = st["write_bytes"] / (o + states)
    assert abs(r - 1) < 0.03, r


def test_committed_counters_are_not_saturated():
    """No committed counter value is a clipped reading (rocprofv3 reports a
    saturated counter as 0xFFF00000 or more): every figure derived from the
    summaries rests on real counts."""
    limit = 0xFFF00000
    checked = 0
    for name in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        if not name.endswith(".md"):
            continue
        prof = profiling.read_profile_block(os.path.join(ROOT, "profiles", name))
        if not isinstance(prof, dict):
            continue
        values = dict(prof.get("counters", {}))
        for key in ("fetch_kib_raw", "write_kib_raw"):
            if key in prof:
                values[key] = prof[key]
        for counter, v in values.items():
            assert v < limit, (name, counter, v)
            checked += 1
    assert checked > 0
