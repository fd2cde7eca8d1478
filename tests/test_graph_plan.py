"""Host-side planning of the fork graph runner (no GPU): which captured
capacity bucket serves which requests of a round. The Flide page
("연구방법을 단계별로", step 3) fixes the rules checked here: a round runs on
the smallest pre-captured capacity that holds it, padding only the tail; a
round larger than every capacity is split at request boundaries; a request
larger than every capacity runs without a graph."""

import numpy as np
import pytest

from linear_attention_recurrent_gdn_amd.graphs import Bucket, Replay, plan_round, sort_buckets

BUCKETS = sort_buckets([Bucket(512, 4, 384, 12), Bucket(256, 2, 192, 6)])


def _fits(b, pl, bc, btok, r0, r1):
    return (sum(pl[r0:r1]) <= b.tokens and r1 - r0 <= b.requests
            and sum(btok[r0:r1]) <= b.branch_tokens and sum(bc[r0:r1]) <= b.branches)


def check_plan(plan, buckets, pl, bc, bl):
    """Coverage in order, each replay fits its bucket (the smallest that
    does), each graph replay is maximal (the next request would not fit the
    largest bucket) and graphless replays hold exactly one request that no
    bucket holds."""
    bstart = np.concatenate([[0], np.cumsum(bc)]).astype(int)
    btok = [int(sum(bl[bstart[r]:bstart[r + 1]])) for r in range(len(pl))]
    r = 0
    for rp in plan:
        assert rp.r0 == r and rp.r1 > rp.r0
        if rp.bucket is None:
            assert rp.r1 == rp.r0 + 1
            assert not _fits(buckets[-1], pl, bc, btok, rp.r0, rp.r1)
        else:
            assert _fits(buckets[rp.bucket], pl, bc, btok, rp.r0, rp.r1)
            assert all(not _fits(b, pl, bc, btok, rp.r0, rp.r1) for b in buckets[:rp.bucket])
            if rp.r1 < len(pl):
                assert not _fits(buckets[-1], pl, bc, btok, rp.r0, rp.r1 + 1)
        r = rp.r1
    assert r == len(pl)


def test_round_in_smallest_bucket():
    plan = plan_round(BUCKETS, [100, 130], [1, 2], [64, 9, 33])
    assert plan == [Replay(0, 2, 0)]


def test_round_needs_larger_bucket():
    plan = plan_round(BUCKETS, [100, 130, 7], [1, 0, 1], [64, 1])
    assert plan == [Replay(0, 3, 1)]


def test_over_capacity_round_splits_at_request_boundaries():
    pl = [100, 130, 64, 200, 7, 150]
    bc = [2] * 6
    bl = [40, 3, 64, 1, 9, 9, 33, 0, 5, 5, 64, 64]
    plan = plan_round(BUCKETS, pl, bc, bl)
    assert plan == [Replay(0, 4, 1), Replay(4, 6, 0)]
    check_plan(plan, BUCKETS, pl, bc, bl)


def test_branch_capacity_also_splits():
    pl = [10] * 3
    bc = [6, 6, 1]  # 13 branches > 12
    bl = [1] * 13
    plan = plan_round(BUCKETS, pl, bc, bl)
    assert plan == [Replay(0, 2, 1), Replay(2, 3, 0)]


def test_oversize_request_runs_graphless():
    plan = plan_round(BUCKETS, [10, 700, 20], [1, 1, 1], [5, 5, 5])
    assert plan == [Replay(0, 1, 0), Replay(1, 2, None), Replay(2, 3, 0)]
    plan = plan_round(BUCKETS, [10], [13], [1] * 13)  # too many branches for any bucket
    assert plan == [Replay(0, 1, None)]


def test_empty_round_and_no_buckets():
    assert plan_round(BUCKETS, [], [], []) == []
    assert plan_round([], [5, 6], [0, 1], [3]) == [Replay(0, 1, None), Replay(1, 2, None)]


def test_random_rounds_keep_the_invariants():
    rng = np.random.default_rng(0)
    for _ in range(300):
        R = int(rng.integers(0, 12))
        pl = rng.integers(0, 400, R).tolist()
        bc = rng.integers(0, 5, R).tolist()
        bl = rng.integers(0, 120, int(sum(bc))).tolist()
        check_plan(plan_round(BUCKETS, pl, bc, bl), BUCKETS, pl, bc, bl)


def test_bad_arguments():
    with pytest.raises(ValueError):
        plan_round(BUCKETS, [1, 2], [1], [1])
    with pytest.raises(ValueError):
        plan_round(BUCKETS, [1], [2], [1])
    with pytest.raises(ValueError):
        sort_buckets([Bucket(100, 4, 10, 10), Bucket(200, 2, 10, 10)])
