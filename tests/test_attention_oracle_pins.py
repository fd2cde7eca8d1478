"""Pins of the fork-attention oracle (CPU only).

Each test ties the oracle to something other than itself: a library
causal attention (torch, fp64), the page's claim that a branch computes the
same function as an independent prompt (trunk ++ branch as one sequence),
closed forms (identical keys give the running mean of the visible values;
a dominant key returns its value), invisibility of other questions and
requests, and grouped heads equal repeated heads.
"""

import numpy as np
import pytest
import torch

import oracle


def stream(rng, trunk_lens, branch_lens, branch_parent, H, Hkv, d):
    """A flat stream: every trunk, then every branch; absolute offsets."""
    cu = np.concatenate([[0], np.cumsum(trunk_lens)]).astype(np.int32)
    bcu = (cu[-1] + np.concatenate([[0], np.cumsum(branch_lens)])).astype(np.int32)
    N = int(bcu[-1])
    q = rng.standard_normal((N, H, d))
    k = rng.standard_normal((N, Hkv, d))
    v = rng.standard_normal((N, Hkv, d))
    return q, k, v, cu, bcu, np.asarray(branch_parent, dtype=np.int32)


def torch_causal(q, k, v, scale):
    """Library causal attention of one sequence: q [T,H,d], k,v [T,H,d]."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2)))  # noqa: E731
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True,
                                                         scale=scale)
    return o.numpy().transpose(1, 0, 2)


def test_trunks_match_library_causal_attention():
    rng = np.random.default_rng(0)
    H, d = 3, 16
    q, k, v, cu, bcu, bpar = stream(rng, [1, 7, 20], [], [], H, H, d)
    scale = 0.3
    o = oracle.fork_attention(q, k, v, cu, bcu, bpar, scale=scale)
    for r in range(3):
        s, e = cu[r], cu[r + 1]
        ref = torch_causal(q[s:e], k[s:e], v[s:e], scale)
        np.testing.assert_allclose(o[s:e], ref, rtol=0, atol=1e-12)


def test_branches_equal_independent_prompts():
    """A branch token's output equals causal attention over trunk ++ branch
    run as one sequence (library routine and the oracle's own trunk rule)."""
    rng = np.random.default_rng(1)
    H, d = 2, 8
    trunk, blen, par = [9, 5], [3, 1, 4, 2], [1, 0, 1, 0]
    q, k, v, cu, bcu, bpar = stream(rng, trunk, blen, par, H, H, d)
    o = oracle.fork_attention(q, k, v, cu, bcu, bpar)
    for b in range(len(blen)):
        r = par[b]
        rows = np.r_[cu[r]:cu[r + 1], bcu[b]:bcu[b + 1]]
        ref = torch_causal(q[rows], k[rows], v[rows], 1 / np.sqrt(d))[-blen[b]:]
        np.testing.assert_allclose(o[bcu[b]:bcu[b + 1]], ref, rtol=0, atol=1e-12)
        alone = oracle.fork_attention(q[rows], k[rows], v[rows], [0, len(rows)])
        np.testing.assert_array_equal(o[bcu[b]:bcu[b + 1]], alone[-blen[b]:])


def test_identical_keys_give_running_mean():
    rng = np.random.default_rng(2)
    H, d = 2, 8
    trunk, blen, par = [6, 4], [3, 5], [1, 0]
    q, k, v, cu, bcu, bpar = stream(rng, trunk, blen, par, H, H, d)
    k[:] = rng.standard_normal((1, H, d))
    o = oracle.fork_attention(q, k, v, cu, bcu, bpar)
    for r in range(2):
        s, e = cu[r], cu[r + 1]
        mean = np.cumsum(v[s:e], axis=0) / np.arange(1, e - s + 1)[:, None, None]
        np.testing.assert_allclose(o[s:e], mean, rtol=0, atol=1e-12)
    for b in range(2):
        r = par[b]
        tv = v[cu[r]:cu[r + 1]]
        bv = v[bcu[b]:bcu[b + 1]]
        mean = (tv.sum(axis=0) + np.cumsum(bv, axis=0)) / (
            len(tv) + np.arange(1, len(bv) + 1))[:, None, None]
        np.testing.assert_allclose(o[bcu[b]:bcu[b + 1]], mean, rtol=0, atol=1e-12)


def test_dominant_key_returns_its_value():
    """One-hot keys in distinct directions; each query points at one visible
    key with a large score, so the output is that key's value."""
    rng = np.random.default_rng(3)
    d = 16
    trunk, blen, par = [5, 6], [4, 3], [0, 1]
    q, k, v, cu, bcu, bpar = stream(rng, trunk, blen, par, 1, 1, d)
    N = len(q)
    k[:] = 0
    dirs = np.zeros(N, dtype=int)
    for r in range(2):  # distinct directions within each visible set
        for j, i in enumerate(range(cu[r], cu[r + 1])):
            dirs[i] = j
    for b in range(2):
        for j, i in enumerate(range(bcu[b], bcu[b + 1])):
            dirs[i] = 8 + j
    k[np.arange(N), 0, dirs] = 1.0
    target = np.zeros(N, dtype=int)
    for r in range(2):
        for i in range(cu[r], cu[r + 1]):
            target[i] = rng.integers(cu[r], i + 1)
    for b in range(2):
        r = par[b]
        for i in range(bcu[b], bcu[b + 1]):
            vis = np.r_[cu[r]:cu[r + 1], bcu[b]:i + 1]
            target[i] = rng.choice(vis)
    q[:] = 0
    q[np.arange(N), 0, dirs[target]] = 60.0
    o = oracle.fork_attention(q, k, v, cu, bcu, bpar, scale=1.0)
    np.testing.assert_allclose(o[:, 0], v[target, 0], rtol=0, atol=1e-20 + 1e-12)


def test_invisible_tokens_have_no_effect():
    rng = np.random.default_rng(4)
    H, d = 2, 8
    trunk, blen, par = [7, 6], [3, 4, 2], [0, 1, 0]
    q, k, v, cu, bcu, bpar = stream(rng, trunk, blen, par, H, H, d)
    o = oracle.fork_attention(q, k, v, cu, bcu, bpar)
    # branch 0 (parent 0) must not see request 1 nor branches 1 and 2
    k2, v2 = k.copy(), v.copy()
    for s, e in ((cu[1], cu[2]), (bcu[1], bcu[3])):
        k2[s:e] = rng.standard_normal(k2[s:e].shape)
        v2[s:e] = rng.standard_normal(v2[s:e].shape)
    o2 = oracle.fork_attention(q, k2, v2, cu, bcu, bpar)
    np.testing.assert_array_equal(o2[bcu[0]:bcu[1]], o[bcu[0]:bcu[1]])
    np.testing.assert_array_equal(o2[cu[0]:cu[1]], o[cu[0]:cu[1]])
    # a token never sees later tokens of its own segment
    k3, v3 = k.copy(), v.copy()
    k3[bcu[0] + 2:bcu[0] + 3] += 1.0
    v3[bcu[0] + 2:bcu[0] + 3] += 1.0
    o3 = oracle.fork_attention(q, k3, v3, cu, bcu, bpar)
    np.testing.assert_array_equal(o3[bcu[0]:bcu[0] + 2], o[bcu[0]:bcu[0] + 2])
    assert not np.array_equal(o3[bcu[0] + 2], o[bcu[0] + 2])


def test_grouped_heads_equal_repeated_heads():
    rng = np.random.default_rng(5)
    H, Hkv, d = 6, 2, 8
    trunk, blen, par = [5, 3], [2, 3], [1, 0]
    q, k, v, cu, bcu, bpar = stream(rng, trunk, blen, par, H, Hkv, d)
    o = oracle.fork_attention(q, k, v, cu, bcu, bpar)
    rep = np.repeat(np.arange(Hkv), H // Hkv)
    o_rep = oracle.fork_attention(q, k[:, rep], v[:, rep], cu, bcu, bpar)
    np.testing.assert_array_equal(o, o_rep)


def test_trunk_queries_off_and_empty_segments():
    rng = np.random.default_rng(6)
    H, d = 2, 8
    trunk, blen, par = [4, 0], [3, 0, 2], [0, 0, 1]
    q, k, v, cu, bcu, bpar = stream(rng, trunk, blen, par, H, H, d)
    fill = rng.standard_normal(q.shape)
    o_all = oracle.fork_attention(q, k, v, cu, bcu, bpar)
    o_br = oracle.fork_attention(q, k, v, cu, bcu, bpar, trunk_queries=False, o=fill)
    np.testing.assert_array_equal(o_br[:cu[-1]], fill[:cu[-1]])
    np.testing.assert_array_equal(o_br[bcu[0]:], o_all[bcu[0]:])
    # the branch of the empty request sees only itself: plain causal attention
    s, e = bcu[2], bcu[3]
    ref = torch_causal(q[s:e], k[s:e], v[s:e], 1 / np.sqrt(d))
    np.testing.assert_allclose(o_all[s:e], ref, rtol=0, atol=1e-12)
