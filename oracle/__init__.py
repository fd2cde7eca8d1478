"""fp64 CPU oracle for the GDN recurrence hot path (Python side).

TEST INFRASTRUCTURE: only tests/, the smoke check and the bench's CPU
baseline leg import this package. It wraps `liboracle.so`, built by gcc
from `gdn_oracle.c` and `fork_attention_oracle.c` in this folder, which
compute every result in fp64 straight from the definitions (see the
headers of those files for the sources and readings). It shares no code
with the HIP library.

All array arguments are NumPy arrays of any float dtype; they are widened
to float64 (bf16 and fp32 values widen exactly).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "gdn_oracle.c"), os.path.join(HERE, "fork_attention_oracle.c")]
LIB = os.path.join(HERE, "liboracle.so")
_OVERRIDE = os.environ.get("ORACLE_LIB_OVERRIDE")

GDN, KDA, RWKV6 = 0, 1, 2
VARIANTS = {"gdn": GDN, "kda": KDA, "rwkv6": RWKV6}
NORM_EPS = 1e-6

_lib = None


def build(verbose=False):
    """Compile liboracle.so with gcc (OpenMP, -O2, strict IEEE: no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-o", LIB + ".tmp", *SRCS, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)


def lib():
    global _lib
    if _lib is None:
        if _OVERRIDE:
            _lib = ctypes.CDLL(_OVERRIDE)
        else:
            if not os.path.exists(LIB) or any(os.path.getmtime(LIB) < os.path.getmtime(s)
                                              for s in SRCS):
                build()
            _lib = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        _lib.oracle_decode.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, I]
        _lib.oracle_sequences.argtypes = [I, P, P, I, I, I, I, I, P, P, P, P, P,
                                          P, I, D, P, P, P, P, P, I]
        _lib.oracle_materialize.argtypes = [I, I, I, I, I, P, P, P, P, P, P, I]
        _lib.oracle_conv.argtypes = [I, I, I, I, P, P, P, P, P, I, D, P, P, P, P]
        _lib.oracle_fork_attention.argtypes = [I, I, I, I, P, P, P, I, P, I, P, P, D, I, P, I]
        _lib.oracle_max_threads.restype = I
    return _lib


def max_threads() -> int:
    return lib().oracle_max_threads()


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _variant(variant):
    return VARIANTS[variant] if isinstance(variant, str) else int(variant)


def decode(q, k, v, log_alpha, beta, state, variant="gdn", want_u=False,
           nthreads=0):
    """Plain recurrence over pre-drawn decode steps.

    q, k [steps,B,H,dk], v [steps,B,H,dv], log_alpha [steps,B,H] (scalar
    decay) or [steps,B,H,dk] (per-key), beta [steps,B,H] (None for RWKV6),
    state [B,H,dk,dv] (storage orientation, not modified).
    Returns (o [steps,B,H,dv], final state [B,H,dk,dv], u or None).
    """
    q, k, v, la, st = _f64(q), _f64(k), _f64(v), _f64(log_alpha), _f64(state).copy()
    beta = _f64(beta)
    steps, B, H, dk = q.shape
    dv = v.shape[-1]
    per_key = int(la.ndim == 4)
    o = np.zeros((steps, B, H, dv))
    u = np.zeros((steps, B, H, dv)) if want_u else None
    lib().oracle_decode(steps, B, H, dk, dv, _variant(variant), per_key,
                        _ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(beta),
                        _ptr(st), _ptr(o), _ptr(u), nthreads)
    return o, st, u


def sequences(q, k, v, log_alpha, beta, cu_seqlens, *, parent=None,
              conv_w=None, qk_norm=False, state_in=None, win_in=None,
              variant="gdn", eps=NORM_EPS, want_o=True, nthreads=0):
    """Run the sequences of a flat token stream (prefill, or branches when
    `parent` maps each sequence to the index of its starting state/window).

    q, k [N,H,dk], v [N,H,dv], log_alpha [N,H] or [N,H,dk], beta [N,H].
    Returns (o [N,H,dv] or None, final state [nseq,H,dk,dv],
    final window [nseq,3,H*(2dk+dv)]).
    """
    q, k, v, la, beta = _f64(q), _f64(k), _f64(v), _f64(log_alpha), _f64(beta)
    N, H, dk = q.shape
    dv = v.shape[-1]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    nseq = len(cu) - 1
    par = None if parent is None else np.ascontiguousarray(parent, dtype=np.int32)
    per_key = int(la.ndim == 3)
    cc = H * (2 * dk + dv)
    o = np.zeros((N, H, dv)) if want_o else None
    st = np.zeros((nseq, H, dk, dv))
    win = np.zeros((nseq, 3, cc))
    lib().oracle_sequences(nseq, _ptr(cu), _ptr(par), H, dk, dv,
                           _variant(variant), per_key, _ptr(q), _ptr(k),
                           _ptr(v), _ptr(la), _ptr(beta), _ptr(_f64(conv_w)),
                           int(bool(qk_norm)), float(eps),
                           _ptr(_f64(state_in)), _ptr(_f64(win_in)), _ptr(o),
                           _ptr(st), _ptr(win), nthreads)
    return o, st, win


def prefill(q, k, v, log_alpha, beta, cu_seqlens, **kw):
    """Call 1 of the two-call fork: every shared context from its own
    initial state (zeros when not given) -> o, final state, conv window."""
    return sequences(q, k, v, log_alpha, beta, cu_seqlens, **kw)


def fork(q, k, v, log_alpha, beta, branch_cu, branch_parent, parent_state,
         parent_window=None, **kw):
    """Call 2: every branch from its own request's saved state and window."""
    return sequences(q, k, v, log_alpha, beta, branch_cu, parent=branch_parent,
                     state_in=parent_state, win_in=parent_window, **kw)


def conv(q, k, v, conv_w=None, win_in=None, qk_norm=False, eps=NORM_EPS):
    """Short convolution (+ q/k normalisation) of one sequence.

    q, k [len,H,dk], v [len,H,dv]; conv_w [H*(2dk+dv),4] or None;
    win_in [3,H*(2dk+dv)] or None. Returns (yq, yk, yv, window_out).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, H, dk = q.shape
    dv = v.shape[-1]
    yq, yk, yv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    win = np.zeros((3, H * (2 * dk + dv)))
    lib().oracle_conv(T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                      _ptr(_f64(win_in)), _ptr(_f64(conv_w)),
                      int(bool(qk_norm)), float(eps), _ptr(yq), _ptr(yk),
                      _ptr(yv), _ptr(win))
    return yq, yk, yv, win


def materialize(base, log_u, log_k, log_lam, lengths, nthreads=0):
    """Logical state of deferred (base + log) slot-heads.

    base [n,dk,dv], log_u [n,Mcap,dv], log_k [n,Mcap,dk], log_lam [n,Mcap]
    or [n,Mcap,dk], lengths [n]. Returns [n,dk,dv].
    """
    base, lu, lk, ll = _f64(base), _f64(log_u), _f64(log_k), _f64(log_lam)
    n, dk, dv = base.shape
    Mcap = lu.shape[1]
    per_key = int(ll.ndim == 3)
    m = np.ascontiguousarray(lengths, dtype=np.int32)
    out = np.zeros_like(base)
    lib().oracle_materialize(n, dk, dv, per_key, Mcap, _ptr(m), _ptr(base),
                             _ptr(lu), _ptr(lk), _ptr(ll), _ptr(out), nthreads)
    return out


def fork_attention(q, k, v, cu_seqlens, branch_cu=None, branch_parent=None, *, scale=None,
                   trunk_queries=True, o=None, nthreads=0):
    """Softmax attention over a flat token stream under the fork visibility
    rule: a trunk token sees its request's trunk up to itself, a branch
    token its parent request's whole trunk and its own branch up to itself.

    q [N,H,d], k and v [N,H_kv,d]; cu_seqlens [R+1] and branch_cu [NB+1]
    are absolute offsets into the stream; branch_parent [NB]. `scale`
    defaults to 1/sqrt(d). Rows that no queried segment covers keep the
    values of `o` (zeros when not given). Returns o [N,H,d] in fp64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, H, d = q.shape
    Hkv = k.shape[1]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    if branch_cu is None:
        bcu, bpar = np.zeros(1, dtype=np.int32), np.zeros(0, dtype=np.int32)
    else:
        bcu = np.ascontiguousarray(branch_cu, dtype=np.int32)
        bpar = np.ascontiguousarray(branch_parent, dtype=np.int32)
    out = np.zeros((N, H, d)) if o is None else np.array(o, dtype=np.float64, copy=True)
    sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
    lib().oracle_fork_attention(N, H, Hkv, d, _ptr(q), _ptr(k), _ptr(v), len(cu) - 1, _ptr(cu),
                                len(bcu) - 1, _ptr(bcu), _ptr(bpar), sc, int(bool(trunk_queries)),
                                _ptr(out), nthreads)
    return out


def rel_err(x, ref, axes):
    """max |x - ref| / max |ref| over `axes` (per remaining slice); the max
    over slices is returned. A zero reference slice compares absolutely."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(x - ref).max(axis=axes)
    den = np.abs(ref).max(axis=axes)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max()) if num.size else 0.0
