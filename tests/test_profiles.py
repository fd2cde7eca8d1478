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


def test_prep_traffic_matches_algorithmic_bytes():
    """The scalar prep kernel on the fork_prefill prefix: q and k rows (bf16),
    log a and beta read once; the chunk record written once (its all-zero
    T' / P blocks above the diagonal are not written). Reads run above the
    algorithmic count by the conv halo rows (3 extra rows per 16-row block),
    so the band is on the total."""
    prof = profiling.read_profile_block(os.path.join(ROOT, "profiles",
                                                     "fork_prefill_prep_traffic.md"))
    assert prof is not None, "profiles/fork_prefill_prep_traffic.md missing"
    if prof["source_hash"] != profiling.source_hash(profiling.PREFILL_SOURCES):
        pytest.skip("profiles/fork_prefill_prep_traffic.md was taken from other prefill sources")
    w = gi.WORKLOADS["fork_prefill"]
    d, C, H = w["d"], w["chunk"], w["H"]
    chunk_heads = w["R"] * (w["prefix"] // C) * H
    reads = C * d * 2 * 2 + C * 4 * 2                       # q, k rows; log a, beta
    record = (4 * C * C + 6 * C * d) * 2 + 4 * max(d, C)     # bf16 planes + fp32 slot
    zero_blocks = 2 * 2 * 2 * 16 * 32 * 2                    # T', P: hi / lo, 2 blocks each
    alg = chunk_heads * (reads + record - zero_blocks)
    ratio = prof["traffic_bytes"] / alg
    assert 0.98 <= ratio <= 1.10, ratio
    assert abs(prof["write_bytes"] / (chunk_heads * (record - zero_blocks)) - 1) < 0.02
