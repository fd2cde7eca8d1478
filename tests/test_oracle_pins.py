"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each test names what fixes the expected value: a hand-derived worked
example, brute-force products of explicit transition matrices, a closed
form, an invariant or an exact special case. Sizes are tiny; the whole file
runs in seconds on the CPU. Non-square d_k != d_v is used wherever it
catches a transposed operand.
"""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_decode(rng, T, B, H, dk, dv, per_key=False, la=(-0.3, -0.01)):
    q = unit(rng.standard_normal((T, B, H, dk)))
    k = unit(rng.standard_normal((T, B, H, dk)))
    v = rng.standard_normal((T, B, H, dv))
    lshape = (T, B, H, dk) if per_key else (T, B, H)
    log_a = rng.uniform(la[0], la[1], lshape)
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, B, H))))
    s0 = rng.standard_normal((B, H, dk, dv)) * 0.3
    return q, k, v, log_a, beta, s0


# --------------------------------------------------------------- worked examples
def _golden_cases():
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_derived_worked_examples(case):
    S0 = np.array(case["S0"], dtype=np.float64)  # math orientation, dv x dk
    steps = case["steps"]
    T = len(steps)
    dv, dk = S0.shape
    per_key = isinstance(steps[0]["alpha"], list)
    q = np.array([s["q"] for s in steps], dtype=np.float64).reshape(T, 1, 1, dk)
    k = np.array([s["k"] for s in steps], dtype=np.float64).reshape(T, 1, 1, dk)
    v = np.array([s["v"] for s in steps], dtype=np.float64).reshape(T, 1, 1, dv)
    a = np.array([s["alpha"] for s in steps], dtype=np.float64)
    la = np.log(a).reshape((T, 1, 1, dk) if per_key else (T, 1, 1))
    beta = np.array([s["beta"] for s in steps], dtype=np.float64).reshape(T, 1, 1)
    o, st, _ = oracle.decode(q, k, v, la, beta, S0.T.reshape(1, 1, dk, dv),
                             variant=case["variant"])
    np.testing.assert_allclose(o[:, 0, 0], np.array(case["o"]), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(st[0, 0].T, np.array(case["S_final"]), rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------- brute force
def _transition(variant, a, beta, k):
    dk = k.shape[0]
    if variant == "rwkv6":
        return np.diag(a)
    return np.diag(a) @ (np.eye(dk) - beta * np.outer(k, k))


def _brute_force(variant, S0, q, k, v, a, beta):
    """S_t = S_0 A_1...A_t + sum_s B_s A_{s+1}...A_t, o_t = S_t q_t, with
    A_t, B_t explicit matrices (math orientation, S is dv x dk)."""
    T = q.shape[0]
    dk = q.shape[1]
    A = [_transition(variant, a[t], beta[t], k[t]) for t in range(T)]
    Bm = [np.outer(v[t], k[t]) * (1.0 if variant == "rwkv6" else beta[t]) for t in range(T)]
    outs, S = [], None
    for t in range(T):
        prod = np.eye(dk)
        for r in range(t + 1):
            prod = prod @ A[r]
        S = S0 @ prod
        for s in range(t + 1):
            tail = np.eye(dk)
            for r in range(s + 1, t + 1):
                tail = tail @ A[r]
            S = S + Bm[s] @ tail
        outs.append(S @ q[t])
    return np.array(outs), S


@pytest.mark.parametrize("variant", ["gdn", "kda", "rwkv6"])
@pytest.mark.parametrize("dk,dv,T", [(5, 3, 16), (4, 7, 9), (8, 8, 12)])
def test_bruteforce_unrolled_products(variant, dk, dv, T):
    rng = RNG(11)
    per_key = variant != "gdn"
    q, k, v, la, beta, s0 = rand_decode(rng, T, 1, 1, dk, dv, per_key=per_key)
    o, st, _ = oracle.decode(q, k, v, la, None if variant == "rwkv6" else beta,
                             s0, variant=variant)
    a = np.exp(la[:, 0, 0]) if per_key else np.exp(la[:, 0, 0])[:, None] * np.ones(dk)
    ob, Sb = _brute_force(variant, s0[0, 0].T, q[:, 0, 0], k[:, 0, 0], v[:, 0, 0],
                          a, beta[:, 0, 0])
    np.testing.assert_allclose(o[:, 0, 0], ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(st[0, 0].T, Sb, rtol=0, atol=1e-12)


# --------------------------------------------------------------- closed forms
@pytest.mark.parametrize("variant", ["gdn", "kda"])
def test_beta_zero_is_pure_decay(variant):
    """b = 0: S_T = S_0 diag(prod a), o_t = S_0 diag(prod_{r<=t} a_r) q_t."""
    rng = RNG(3)
    T, dk, dv = 10, 6, 5
    q, k, v, la, beta, s0 = rand_decode(rng, T, 2, 2, dk, dv, per_key=variant == "kda")
    beta = np.zeros_like(beta)
    o, st, _ = oracle.decode(q, k, v, la, beta, s0, variant=variant)
    cum = np.cumsum(la, axis=0)
    if variant == "gdn":
        cum = cum[..., None] * np.ones(dk)
    for t in range(T):
        # storage Sig = S^T: o_j = sum_i Sig[i][j] e^{cum_i} q_i
        exp_o = np.einsum("bhij,bhi->bhj", s0, np.exp(cum[t]) * q[t])
        np.testing.assert_allclose(o[t], exp_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st, s0 * np.exp(cum[-1])[..., None], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("variant", ["gdn", "kda"])
def test_write_then_read(variant):
    """b = 1, |k| = 1, q = k: the step overwrites the state along k with v,
    so o_t = S_t k_t = v_t for any decay."""
    rng = RNG(5)
    T, dk, dv = 12, 7, 4
    q, k, v, la, beta, s0 = rand_decode(rng, T, 3, 2, dk, dv, per_key=variant == "kda")
    o, _, _ = oracle.decode(k, k, v, la, np.ones_like(beta), s0, variant=variant)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-13)


def test_lookup_table_exact():
    """a = 1, b = 1, one-hot keys e_i: each step replaces column i of S with
    v; a one-hot query e_j reads the last v written to j (or S_0's column).
    Small integers keep every operation exact."""
    rng = RNG(9)
    T, dk, dv = 20, 6, 3
    keys = rng.integers(0, dk, T)
    qs = rng.integers(0, dk, T)
    v = rng.integers(-4, 5, (T, dv)).astype(np.float64)
    S0 = rng.integers(-3, 4, (dv, dk)).astype(np.float64)
    k = np.eye(dk)[keys].reshape(T, 1, 1, dk)
    q = np.eye(dk)[qs].reshape(T, 1, 1, dk)
    o, st, _ = oracle.decode(q, k, v.reshape(T, 1, 1, dv), np.zeros((T, 1, 1)),
                             np.ones((T, 1, 1)), S0.T.reshape(1, 1, dk, dv))
    table = S0.copy()
    for t in range(T):
        table[:, keys[t]] = v[t]
        assert np.array_equal(o[t, 0, 0], table[:, qs[t]])
    assert np.array_equal(st[0, 0].T, table)


@pytest.mark.parametrize("variant", ["gdn", "kda", "rwkv6"])
def test_joint_linearity_in_state_and_values(variant):
    rng = RNG(21)
    T, dk, dv = 9, 5, 6
    q, k, v1, la, beta, s1 = rand_decode(rng, T, 1, 2, dk, dv, per_key=variant != "gdn")
    v2 = rng.standard_normal(v1.shape)
    s2 = rng.standard_normal(s1.shape)
    b = None if variant == "rwkv6" else beta
    c1, c2 = 0.7, -1.3
    o1, f1, _ = oracle.decode(q, k, v1, la, b, s1, variant=variant)
    o2, f2, _ = oracle.decode(q, k, v2, la, b, s2, variant=variant)
    o3, f3, _ = oracle.decode(q, k, c1 * v1 + c2 * v2, la, b, c1 * s1 + c2 * s2, variant=variant)
    np.testing.assert_allclose(o3, c1 * o1 + c2 * o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(f3, c1 * f1 + c2 * f2, rtol=0, atol=1e-12)


def test_state_norm_bound():
    """|k| = 1, b in (0,1): ||S_t||_2 <= a_t ||S_{t-1}||_2 + b_t ||v_t||
    because ||I - b k k^T||_2 = 1."""
    rng = RNG(4)
    T, dk, dv = 30, 6, 6
    q, k, v, la, beta, s0 = rand_decode(rng, T, 1, 1, dk, dv)
    prev = np.linalg.norm(s0[0, 0], 2)
    st = s0
    for t in range(T):
        _, st, _ = oracle.decode(q[t:t + 1], k[t:t + 1], v[t:t + 1], la[t:t + 1],
                                 beta[t:t + 1], st)
        cur = np.linalg.norm(st[0, 0], 2)
        bound = np.exp(la[t, 0, 0]) * prev + beta[t, 0, 0] * np.linalg.norm(v[t, 0, 0])
        assert cur <= bound * (1 + 1e-12)
        prev = cur


def test_rwkv6_parallel_closed_form():
    """S_t = S_0 diag(e^{L_t}) + sum_{s<=t} v_s (k_s . e^{L_t - L_s})^T with
    L_t the running sum of per-key log-decays: o_t needs no recurrence."""
    rng = RNG(8)
    T, dk, dv = 14, 5, 4
    q, k, v, la, _, s0 = rand_decode(rng, T, 1, 1, dk, dv, per_key=True)
    o, st, _ = oracle.decode(q, k, v, la, None, s0, variant="rwkv6")
    L = np.cumsum(la[:, 0, 0], axis=0)
    S0 = s0[0, 0].T
    for t in range(T):
        ref = S0 @ (np.exp(L[t]) * q[t, 0, 0])
        for s in range(t + 1):
            ref = ref + v[s, 0, 0] * np.dot(k[s, 0, 0] * np.exp(L[t] - L[s]), q[t, 0, 0])
        np.testing.assert_allclose(o[t, 0, 0], ref, rtol=0, atol=1e-12)


def test_kda_equal_entries_is_gdn():
    rng = RNG(13)
    T, dk, dv = 8, 6, 5
    q, k, v, la, beta, s0 = rand_decode(rng, T, 2, 2, dk, dv)
    la_key = np.repeat(la[..., None], dk, axis=-1)
    o1, f1, _ = oracle.decode(q, k, v, la, beta, s0, variant="gdn")
    o2, f2, _ = oracle.decode(q, k, v, la_key, beta, s0, variant="kda")
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(f2, f1, rtol=0, atol=1e-14)


# --------------------------------------------------------------- convolution
def _conv_inputs(rng, T, H, dk, dv):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    cc = H * (2 * dk + dv)
    w = rng.uniform(-0.5, 0.5, (cc, 4))
    win = rng.standard_normal((3, cc))
    return q, k, v, w, win


def test_conv_identity_taps_is_noop():
    rng = RNG(1)
    q, k, v, w, win = _conv_inputs(rng, 9, 2, 4, 3)
    w = np.zeros_like(w)
    w[:, 3] = 1.0
    yq, yk, yv, _ = oracle.conv(q, k, v, w, win)
    assert np.array_equal(yq, q) and np.array_equal(yk, k) and np.array_equal(yv, v)


def test_conv_impulse_reproduces_taps():
    """A unit impulse at token t0 of one channel (zero window) comes out as
    the reversed taps on tokens t0..t0+3 of that channel only."""
    rng = RNG(2)
    T, H, dk, dv = 10, 2, 3, 4
    _, _, _, w, _ = _conv_inputs(rng, T, H, dk, dv)
    cc = H * (2 * dk + dv)
    for c in [0, 4, H * dk + 1, 2 * H * dk + 5, cc - 1]:
        x = np.zeros((T, cc))
        t0 = 3
        x[t0, c] = 1.0
        q = x[:, : H * dk].reshape(T, H, dk)
        k = x[:, H * dk: 2 * H * dk].reshape(T, H, dk)
        v = x[:, 2 * H * dk:].reshape(T, H, dv)
        yq, yk, yv, _ = oracle.conv(q, k, v, w, None)
        y = np.concatenate([yq.reshape(T, -1), yk.reshape(T, -1), yv.reshape(T, -1)], 1)
        exp = np.zeros_like(y)
        for r in range(4):
            if t0 + r < T:
                exp[t0 + r, c] = w[c, 3 - r]
        assert np.array_equal(y, exp)


def test_conv_window_in_and_out():
    """Positions before the start read the incoming window (oldest row
    first); the outgoing window is the last three raw inputs, reaching into
    the incoming window for sequences shorter than three."""
    rng = RNG(3)
    H, dk, dv = 1, 2, 2
    for T in [0, 1, 2, 3, 6]:
        q, k, v, w, win = _conv_inputs(rng, T, H, dk, dv)
        flat = lambda a: a.reshape(T, a.shape[1] * a.shape[2])  # noqa: E731
        x = np.concatenate([flat(q), flat(k), flat(v)], 1)
        full = np.concatenate([win, x], 0)  # positions -3 .. T-1
        yq, yk, yv, wout = oracle.conv(q, k, v, w, win)
        y = np.concatenate([flat(yq), flat(yk), flat(yv)], 1)
        for t in range(T):
            exp = (w * full[t: t + 4].T).sum(1)
            np.testing.assert_allclose(y[t], exp, rtol=1e-15, atol=1e-15)
        assert np.array_equal(wout, full[-3:])


def test_conv_split_anywhere_matches_unsplit():
    rng = RNG(4)
    T, H, dk, dv = 13, 2, 3, 2
    q, k, v, w, win = _conv_inputs(rng, T, H, dk, dv)
    y_all = oracle.conv(q, k, v, w, win, qk_norm=True)
    for p in [0, 1, 2, 3, 7, 13]:
        a = oracle.conv(q[:p], k[:p], v[:p], w, win, qk_norm=True)
        b = oracle.conv(q[p:], k[p:], v[p:], w, a[3], qk_norm=True)
        for i in range(3):
            assert np.array_equal(np.concatenate([a[i], b[i]]), y_all[i])
        assert np.array_equal(b[3], y_all[3])


def test_qk_norm_unit_length_v_untouched():
    rng = RNG(6)
    q, k, v, w, win = _conv_inputs(rng, 7, 3, 5, 4)
    yq, yk, yv, _ = oracle.conv(q, k, v, w, win, qk_norm=True)
    _, _, yv0, _ = oracle.conv(q, k, v, w, win, qk_norm=False)
    yq0, yk0, _, _ = oracle.conv(q, k, v, w, win, qk_norm=False)
    for y, y0 in ((yq, yq0), (yk, yk0)):
        n0 = np.linalg.norm(y0, axis=-1, keepdims=True)
        np.testing.assert_allclose(y, y0 / np.sqrt(n0 ** 2 + oracle.NORM_EPS), rtol=1e-14)
    assert np.array_equal(yv, yv0)


# --------------------------------------------------------------- fork
def _stream(rng, lens, H, dk, dv):
    N = int(sum(lens))
    q = unit(rng.standard_normal((N, H, dk)))
    k = unit(rng.standard_normal((N, H, dk)))
    v = rng.standard_normal((N, H, dv))
    la = rng.uniform(-0.2, -0.01, (N, H))
    beta = 1 / (1 + np.exp(-rng.standard_normal((N, H))))
    return q, k, v, la, beta


@pytest.mark.parametrize("conv", [False, True])
def test_fork_equals_independent_full_runs(conv):
    """Flide page, method step 2: prefill stores state + conv window, each
    branch runs from its own request's saved state; in exact arithmetic this
    is the independent prompt. In the oracle it is bitwise."""
    rng = RNG(7)
    H, dk, dv = 2, 4, 3
    prefix = [9, 1, 0, 5]
    branches = [4, 0, 2, 7, 1, 3]
    parent = [0, 0, 1, 2, 3, 3]
    R = len(prefix)
    q, k, v, la, beta = _stream(rng, prefix + branches, H, dk, dv)
    cc = H * (2 * dk + dv)
    w = rng.uniform(-0.5, 0.5, (cc, 4)) if conv else None
    s_init = rng.standard_normal((R, H, dk, dv)) * 0.2
    w_init = rng.standard_normal((R, 3, cc))
    Np = sum(prefix)
    cu = np.concatenate([[0], np.cumsum(prefix)])
    bcu = np.concatenate([[0], np.cumsum(branches)])
    o_p, st, win = oracle.prefill(q[:Np], k[:Np], v[:Np], la[:Np], beta[:Np], cu,
                                  conv_w=w, qk_norm=conv, state_in=s_init, win_in=w_init)
    o_b, st_b, win_b = oracle.fork(q[Np:], k[Np:], v[Np:], la[Np:], beta[Np:], bcu,
                                   parent, st, win, conv_w=w, qk_norm=conv)
    for b, p in enumerate(parent):
        pre = slice(cu[p], cu[p + 1])
        br = slice(Np + bcu[b], Np + bcu[b + 1])
        cat = lambda x: np.concatenate([x[pre], x[br]])  # noqa: E731
        Tb = branches[b]
        o_f, st_f, win_f = oracle.prefill(cat(q), cat(k), cat(v), cat(la), cat(beta),
                                          [0, prefix[p] + Tb], conv_w=w, qk_norm=conv,
                                          state_in=s_init[p:p + 1], win_in=w_init[p:p + 1])
        assert np.array_equal(o_b[bcu[b]:bcu[b + 1]], o_f[prefix[p]:])
        assert np.array_equal(st_b[b], st_f[0])
        assert np.array_equal(win_b[b], win_f[0])
        assert np.array_equal(o_p[pre], o_f[:prefix[p]])


def test_empty_sequence_passes_state_and_window_through():
    rng = RNG(10)
    H, dk, dv = 2, 3, 3
    q, k, v, la, beta = _stream(rng, [0, 4], H, dk, dv)
    cc = H * (2 * dk + dv)
    s_init = rng.standard_normal((2, H, dk, dv))
    w_init = rng.standard_normal((2, 3, cc))
    w = rng.uniform(-0.5, 0.5, (cc, 4))
    _, st, win = oracle.prefill(q, k, v, la, beta, [0, 0, 4], conv_w=w, qk_norm=True,
                                state_in=s_init, win_in=w_init)
    assert np.array_equal(st[0], s_init[0]) and np.array_equal(win[0], w_init[0])


def test_decode_and_sequence_entry_points_agree():
    rng = RNG(12)
    T, H, dk, dv = 6, 3, 4, 5
    q, k, v, la, beta = _stream(rng, [T], H, dk, dv)
    s0 = rng.standard_normal((1, H, dk, dv))
    o1, st1, _ = oracle.prefill(q, k, v, la, beta, [0, T], state_in=s0)
    o2, st2, _ = oracle.decode(q[:, None], k[:, None], v[:, None], la[:, None],
                               beta[:, None], s0)
    assert np.array_equal(o1, o2[:, 0]) and np.array_equal(st1, st2)


# --------------------------------------------------------------- deferred base + log
@pytest.mark.parametrize("variant", ["gdn", "kda", "rwkv6"])
def test_replay_of_logged_factors_equals_recurrence(variant):
    """DeltaLog page, 'Base + Log': the logical state is the base plus the
    replayed log. Logging u_t, k_t and the running log-decay of m plain
    recurrence steps and replaying them onto the base gives the state the
    recurrence reached after those m steps."""
    rng = RNG(14)
    Mcap, dk, dv, B, H = 9, 5, 6, 2, 2
    per_key = variant != "gdn"
    q, k, v, la, beta, s0 = rand_decode(rng, Mcap, B, H, dk, dv, per_key=per_key)
    b = None if variant == "rwkv6" else beta
    for m in range(Mcap + 1):
        _, st, u = oracle.decode(q[:m], k[:m], v[:m], la[:m], None if b is None else b[:m],
                                 s0, variant=variant, want_u=True)
        n = B * H
        lu = np.zeros((n, Mcap, dv))
        lk = np.zeros((n, Mcap, dk))
        ll = np.zeros((n, Mcap, dk) if per_key else (n, Mcap))
        if m:
            lu[:, :m] = u.reshape(m, n, dv).transpose(1, 0, 2)
            lk[:, :m] = k[:m].reshape(m, n, dk).transpose(1, 0, 2)
            lam = np.cumsum(la[:m], axis=0)
            ll[:, :m] = lam.reshape((m, n, dk) if per_key else (m, n)).swapaxes(0, 1)
        S = oracle.materialize(s0.reshape(n, dk, dv), lu, lk, ll, np.full(n, m))
        np.testing.assert_allclose(S.reshape(B, H, dk, dv), st, rtol=0, atol=1e-12)


@pytest.mark.parametrize("M", [1, 4, 8, 16])
def test_deferred_schedule_with_phases_equals_recurrence(M):
    """A decode run kept as base + log, with per-slot phases (slot n merges
    when its log would reach M entries), reproduces the plain recurrence's
    outputs and final state. The per-step output is read from the logical
    state (replayed log) advanced by one recurrence step."""
    rng = RNG(15 + M)
    T, B, H, dk, dv = 20, 3, 2, 4, 5
    q, k, v, la, beta, s0 = rand_decode(rng, T, B, H, dk, dv)
    o_ref, st_ref, _ = oracle.decode(q, k, v, la, beta, s0)
    n = B * H
    base = s0.reshape(n, dk, dv).copy()
    lu, lk, ll = np.zeros((n, M, dv)), np.zeros((n, M, dk)), np.zeros((n, M))
    phase = rng.integers(0, M, B)
    length = np.zeros(n, dtype=np.int64)
    # per-slot phase: slot b starts as if it had already taken phase[b] steps
    # since its last merge (an empty log merges early on its first cycle)
    budget = np.repeat(M - phase, H)
    for t in range(T):
        S = oracle.materialize(base, lu, lk, ll, length)
        o, S1, u = oracle.decode(q[t:t + 1], k[t:t + 1], v[t:t + 1], la[t:t + 1],
                                 beta[t:t + 1], S.reshape(B, H, dk, dv), want_u=True)
        np.testing.assert_allclose(o[0], o_ref[t], rtol=0, atol=1e-12)
        lam_prev = np.where(length > 0, ll[np.arange(n), np.maximum(length - 1, 0)], 0.0)
        for i in range(n):
            m = length[i]
            if m + 1 >= budget[i]:
                base[i] = S1.reshape(n, dk, dv)[i]
                length[i] = 0
                budget[i] = M
            else:
                lu[i, m] = u[0].reshape(n, dv)[i]
                lk[i, m] = k[t].reshape(n, dk)[i]
                ll[i, m] = lam_prev[i] + la[t].reshape(n)[i]
                length[i] = m + 1
    S = oracle.materialize(base, lu, lk, ll, length)
    np.testing.assert_allclose(S.reshape(B, H, dk, dv), st_ref, rtol=0, atol=1e-12)
