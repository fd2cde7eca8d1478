"""A numpy model of how the per-key chunk prep evaluates its decayed
products, checked against their definition for any decay (no GPU).

With per-key decay the chunk form of the recurrence (the Gated DeltaNet
page's chunkwise section, with the decay taken per key as in the DeltaLog
page's problem statement) needs, inside a chunk of C = 64 rows with
running log-decay sums g_r[d] (inclusive, <= 0 and non-increasing),

  KK[r][s] = sum_d k_r[d] k_s[d] e^{g_r[d] - g_s[d]}   (s <= r)
  QK[r][s] = sum_d q_r[d] k_s[d] e^{g_r[d] - g_s[d]}   (s <= r)

and the record rows Q^ = q e^{g}, K^ = k e^{g}, K~ = k e^{g_L - g}. The
products run on matrix cores, so e^{g_r - g_s} must be split into a row
factor and a column factor. Taken against the chunk start (e^{g_r} times
e^{-g_s}) the column factor overflows fp32 once a chunk's decay passes
e^{-88}. The kernel takes each 16-row block against its own first row
(row factor e^{g_r - g_{16R}} <= 1) and each column against its block's
last row (e^{g_{16S+15} - g_s} <= 1), and joins the two by a per-key
factor e^{g_{16R} - g_{16S+15}}. That factor is <= 1 off the diagonal and
e^{(decay across the block)} on it. Where a block's decay exceeds e^{-80}
in some key, the diagonal 16 x 16 tile is evaluated from the definition
instead (exponents <= 0 only). The model below repeats those steps in
fp32, with the kernel's three-product bf16 split for the matrix products,
and is held to the fp64 definition evaluated on the same fp32 sums g.
"""

import numpy as np
import pytest

import gdn_inputs as gi

C, RB = 64, 16
LIMIT = 80.0  # largest exponent of the join factor taken as a product


def split(x):
    """x = hi + lo in bf16 (round to nearest even), as fp32 arrays."""
    _, hi = gi.bf16_round(np.asarray(x, dtype=np.float32))
    _, lo = gi.bf16_round((x - hi).astype(np.float32))
    return hi, lo


def mma3(a, b):
    """a @ b.T from the split operands: hi hi + hi lo + lo hi (fp32 sums)."""
    ah, al = split(a)
    bh, bl = split(b)
    f = np.float32
    return (ah @ bh.T).astype(f) + (ah @ bl.T).astype(f) + (al @ bh.T).astype(f)


def model(q, k, la):
    """The kernel's evaluation (fp32). Returns KK, QK (lower triangles
    valid), Q^, K^, K~, whether the chunk took the direct diagonal, and g."""
    f = np.float32
    q, k, la = q.astype(f), k.astype(f), la.astype(f)
    g = np.cumsum(la, axis=0, dtype=f)
    blk = np.arange(C) // RB
    g0, g15, gL = g[0::RB], g[RB - 1::RB], g[-1]
    e1 = np.exp(g - g0[blk]).astype(f)
    ahat, qhat = k * e1, q * e1
    bchk = k * np.exp(g15[blk] - g).astype(f)
    KK = np.zeros((C, C), f)
    QK = np.zeros((C, C), f)
    for R in range(C // RB):
        rr = slice(R * RB, (R + 1) * RB)
        for S in range(R + 1):
            ss = slice(S * RB, (S + 1) * RB)
            m = np.exp(np.minimum(g0[R] - g15[S], f(LIMIT))).astype(f)
            b = bchk[ss] * m
            KK[rr, ss] = mma3(ahat[rr], b)
            QK[rr, ss] = mma3(qhat[rr], b)
    slow = bool(np.any(g0 - g15 > LIMIT))
    if slow:
        for R in range(C // RB):
            rr = np.arange(R * RB, (R + 1) * RB)
            for r in rr:
                for s in rr[rr <= r]:
                    fac = np.exp(g[r] - g[s]).astype(f)
                    KK[r, s] = np.sum(k[r] * k[s] * fac, dtype=f)
                    QK[r, s] = np.sum(q[r] * k[s] * fac, dtype=f)
    qrec = qhat * np.exp(g0[blk]).astype(f)
    krec = ahat * np.exp(g0[blk]).astype(f)
    ktil = bchk * np.exp(gL - g15[blk]).astype(f)
    return KK, QK, qrec, krec, ktil, slow, g


def definition(q, k, g):
    """fp64 evaluation of the same quantities from the sums g."""
    q, k, g = (np.asarray(x, dtype=np.float64) for x in (q, k, g))
    diff = g[:, None, :] - g[None, :, :]  # [r, s, d]
    low = np.tril(np.ones((C, C), bool))
    fac = np.where(low[:, :, None], np.exp(np.minimum(diff, 0.0)), 0.0)
    KK = np.einsum("rd,sd,rsd->rs", k, k, fac)
    QK = np.einsum("rd,sd,rsd->rs", q, k, fac)
    return KK, QK, q * np.exp(g), k * np.exp(g), k * np.exp(g[-1] - g)


def inputs(la_fn, dk=128, L=C, seed=0):
    rng = np.random.default_rng(seed)
    q = gi.unit_rows(rng.standard_normal((C, dk), dtype=np.float32))
    k = gi.unit_rows(rng.standard_normal((C, dk), dtype=np.float32))
    la = la_fn(rng, (C, dk)).astype(np.float32)
    q[L:] = 0.0
    k[L:] = 0.0
    la[L:] = 0.0  # rows past the sequence end add nothing
    return q, k, la


CASES = {
    "mild": lambda rng, sh: rng.uniform(-0.1, -0.001, sh),
    "strong": lambda rng, sh: rng.uniform(-3.0, -0.5, sh),
    "sum_minus_1000": lambda rng, sh: rng.uniform(-16.0, -15.2, sh),
    "resets": lambda rng, sh: np.where(rng.random(sh) < 0.05, -1000.0,
                                       rng.uniform(-0.1, -0.001, sh)),
    "one_key_extreme": lambda rng, sh: np.concatenate(
        [rng.uniform(-40.0, -30.0, (sh[0], 1)), rng.uniform(-0.1, -0.001, (sh[0], sh[1] - 1))],
        axis=1),
    "no_decay": lambda rng, sh: np.zeros(sh),
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("dk,L", [(128, 64), (32, 64), (64, 37)])
def test_factoring_matches_definition(case, dk, L):
    q, k, la = inputs(CASES[case], dk, L, seed=dk + L)
    KK, QK, qrec, krec, ktil, slow, g = model(q, k, la)
    rKK, rQK, rq, rk, rkt = definition(q, k, g)
    low = np.tril(np.ones((C, C), bool))
    for name, x in (("KK", KK), ("QK", QK), ("Q^", qrec), ("K^", krec), ("K~", ktil)):
        assert np.all(np.isfinite(x)), (case, name)
    # the rows are unit vectors, so every entry is at most 1 in magnitude:
    # absolute error bars (bf16 split ~ 2^-16 relative per product)
    assert np.max(np.abs(KK - rKK)[low]) <= 2e-5, case
    assert np.max(np.abs(QK - rQK)[low]) <= 2e-5, case
    for x, r in ((qrec, rq), (krec, rk), (ktil, rkt)):
        assert np.max(np.abs(x - r)) <= 1e-6, case
    assert slow == (case in ("sum_minus_1000", "resets", "one_key_extreme")), case


def test_chunk_start_reference_overflows():
    """The reason for the block references: against the chunk start the
    column factor e^{-g_s} is not representable for a chunk decaying past
    e^{-88} in some key."""
    _, k, la = inputs(CASES["sum_minus_1000"])
    g = np.cumsum(la, axis=0, dtype=np.float32)
    with np.errstate(over="ignore"):
        col = k * np.exp(-g)
    assert not np.all(np.isfinite(col))


def test_join_factor_off_diagonal_at_most_one():
    """Off the diagonal every factor of the product is <= 1, so the
    factored form can only underflow where the definition itself is below
    fp32's range."""
    _, _, la = inputs(CASES["resets"], seed=3)
    g = np.cumsum(la, axis=0, dtype=np.float32)
    g0, g15 = g[0::RB], g[RB - 1::RB]
    for R in range(C // RB):
        for S in range(R):
            assert np.all(g0[R] - g15[S] <= 0.0)
