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
    k) and the q / k conv taps (4 KiB per workgroup, one workgroup per
    chunk-head) and writes the record once; the scan reads V and the record
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
    prep_reads = qk * (1 + 3 / 16) + token_heads * 8 + chunk_heads * 2 * d * 4 * 4
    scan_reads = token_heads * d * 2 + rec + carry
    scan_writes = token_heads * d * 4 + states + carry
    r = per_call(prep, "read_bytes") / prep_reads
    assert 0.98 <= r <= 1.10, r
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
