"""ctypes binding of libgdn_mi355x.so: argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks
shapes/dtypes/contiguity against the layouts of include/gdn_mi355x.h,
passes raw device pointers and the current HIP stream to the C ABI, and
raises GDNError on a non-zero status. No computation happens here; when the
built library is missing the import fails loudly (there is no fallback).
"""

from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
# GDN_LIB_OVERRIDE: load another build of the same library instead (the
# sanitizer test loads one built with host-side ASan / UBSan)
LIB_PATH = os.environ.get("GDN_LIB_OVERRIDE") or os.path.join(PKG, "libgdn_mi355x.so")

GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE, GDN_ERR_HIP = 0, -1, -2, -3, -4
GDN_F32, GDN_BF16 = 0, 1
VARIANTS = {"gdn": 0, "scalar": 0, "kda": 1, "rwkv6": 2}

# every symbol the header declares, with its ctypes signature
_P, _I, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "gdn_status_string": (ctypes.c_char_p, [_I]),
    "gdn_last_hip_error": (_I, []),
    "gdn_max_log_capacity": (_I, []),
    "gdn_prefill_workspace_bytes": (_S, [_I, _I, _I, _I, _I, _I, _I]),
    "gdn_prefill_shared": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _I, _P, _P,
                                _P, _P, _P, _I, _I, _I, _P, _S, _P]),
    "gdn_prefill_checkpointed": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _I,
                                      _P, _P, _P, _P, _P, _I, _I, _P, _P, _I, _I, _I, _P, _S,
                                      _P]),
    "gdn_fork_branches": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _I,
                               _P, _P, _P, _P, _P, _I, _I, _I, _P, _S, _P]),
    "gdn_decode_eager": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                              _P]),
    "deltalog_append_decode": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I,
                                    _I, _I, _I, _I, _I, _I, _I, _P]),
    "deltalog_merge": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P]),
    "gdn_fork_attention_workspace_bytes": (_S, [_I, _I]),
    "gdn_fork_attention": (_I, [_P, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, ctypes.c_float,
                                _I, _P, _I, _I, _P, _S, _P]),
    "gdn_fork_attention_noalloc": (_I, [_P, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I,
                                        ctypes.c_float, _I, _P, _I, _I, _P]),
    "gdn_stream_probe": (_I, [_P, _P, _S, _I, _P]),
}

# segments the allocation-free fork attention's static tile table holds
FORK_ATTENTION_NOALLOC_MAX_SEGMENTS = 65536


class GDNError(RuntimeError):
    def __init__(self, fn, status, detail=""):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status}){detail}")


_lib = None


def load():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m "
                "linear_attention_recurrent_gdn_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().gdn_status_string(status).decode()


def _check(fn, status):
    if status != GDN_OK:
        detail = ""
        if status == GDN_ERR_HIP:
            detail = f", hipError {load().gdn_last_hip_error()}"
        raise GDNError(fn, status, detail)


# ------------------------------------------------------------------ helpers
def _dev(t, name, dtype=None, shape=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _io_code(t):
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise ValueError(f"unsupported io dtype {t.dtype}")


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _variant(variant):
    return VARIANTS[variant] if isinstance(variant, str) else int(variant)


_F32 = torch.float32
_I32 = torch.int32
_IO = (torch.float32, torch.bfloat16)


# ------------------------------------------------------------------ decode
def gdn_decode_eager(q, k, v, log_alpha, beta, state, o, slot_idx=None, variant="gdn",
                     stream=None):
    """One eager decode step (state rewritten in place). Shapes: q, k [B,H,dk],
    v [B,H,dv], log_alpha [B,H] or [B,H,dk], beta [B,H] (None for rwkv6),
    state [n_slots,H,dk,dv] fp32, o [B,H,dv], slot_idx [B] int32 or None."""
    B, H, dk = q.shape
    dv = v.shape[-1]
    n_slots = state.shape[0]
    io = _io_code(q)
    st = load().gdn_decode_eager(
        _dev(q, "q", q.dtype, (B, H, dk)), _dev(k, "k", q.dtype, (B, H, dk)),
        _dev(v, "v", q.dtype, (B, H, dv)), _dev(log_alpha, "log_alpha", _F32),
        _dev(beta, "beta", _F32, (B, H), optional=True), _dev(state, "state", _F32),
        _dev(slot_idx, "slot_idx", _I32, (B,), optional=True), _dev(o, "o", _IO, (B, H, dv)),
        B, H, dk, dv, n_slots, _variant(variant), io, _io_code(o), _stream(stream))
    _check("gdn_decode_eager", st)


def deltalog_append_decode(q, k, v, log_alpha, beta, base, log_u, log_k, log_lambda, log_len,
                           o, merge_at, slot_idx=None, variant="gdn", stream=None):
    """One deferred decode step. base [S,H,dk,dv], log_u [S,H,Mcap,dv] fp32,
    log_k [S,H,Mcap,dk] (q's dtype), log_lambda [S,H,Mcap] or [S,H,Mcap,dk],
    log_len [S,H] int32."""
    B, H, dk = q.shape
    dv = v.shape[-1]
    S = base.shape[0]
    Mcap = log_u.shape[2]
    io = _io_code(q)
    st = load().deltalog_append_decode(
        _dev(q, "q", q.dtype, (B, H, dk)), _dev(k, "k", q.dtype, (B, H, dk)),
        _dev(v, "v", q.dtype, (B, H, dv)), _dev(log_alpha, "log_alpha", _F32),
        _dev(beta, "beta", _F32, (B, H), optional=True),
        _dev(base, "base", _F32, (S, H, dk, dv)), _dev(log_u, "log_u", _F32, (S, H, Mcap, dv)),
        _dev(log_k, "log_k", q.dtype, (S, H, Mcap, dk)), _dev(log_lambda, "log_lambda", _F32),
        _dev(log_len, "log_len", _I32, (S, H)),
        _dev(slot_idx, "slot_idx", _I32, (B,), optional=True), _dev(o, "o", _IO, (B, H, dv)),
        B, H, dk, dv, S, Mcap, int(merge_at), _variant(variant), io, _io_code(o),
        _stream(stream))
    _check("deltalog_append_decode", st)


def deltalog_merge(base, log_u, log_k, log_lambda, log_len, min_len=1, slot_idx=None,
                   variant="gdn", stream=None):
    """Merge every listed slot-head whose log holds >= min_len entries."""
    S, H, dk, dv = base.shape
    Mcap = log_u.shape[2]
    B = S if slot_idx is None else slot_idx.shape[0]
    st = load().deltalog_merge(
        _dev(base, "base", _F32), _dev(log_u, "log_u", _F32, (S, H, Mcap, dv)),
        _dev(log_k, "log_k", _IO, (S, H, Mcap, dk)), _dev(log_lambda, "log_lambda", _F32),
        _dev(log_len, "log_len", _I32, (S, H)),
        _dev(slot_idx, "slot_idx", _I32, (B,), optional=True), B, H, dk, dv, S, Mcap,
        int(min_len), _variant(variant), _io_code(log_k), _stream(stream))
    _check("deltalog_merge", st)


# ------------------------------------------------------------------ prefill / fork
def prefill_workspace_bytes(n_tokens, n_seq, H, dk, dv, chunk=64, variant="gdn"):
    return int(load().gdn_prefill_workspace_bytes(n_tokens, n_seq, H, dk, dv, chunk,
                                                  _variant(variant)))


def _workspace(n_tokens, n_seq, H, dk, dv, chunk, device, workspace, variant):
    need = prefill_workspace_bytes(n_tokens, n_seq, H, dk, dv, chunk, variant)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return workspace, need


def _la_shape(variant, N, H, dk):
    return (N, H) if _variant(variant) == VARIANTS["gdn"] else (N, H, dk)


def gdn_prefill_shared(q, k, v, log_alpha, beta, cu_seqlens, final_state, o=None,
                       conv_w=None, qk_l2norm=False, init_state=None, init_window=None,
                       final_window=None, chunk=64, workspace=None, variant="gdn",
                       stream=None):
    """Call 1 of the two-call fork: the shared contexts of a flat stream.
    variant "gdn" (scalar log_alpha [N,H]), "kda" or "rwkv6" (per-key
    log_alpha [N,H,dk]; beta may be None for rwkv6)."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    R = cu_seqlens.shape[0] - 1
    cc = H * (2 * dk + dv)
    io = _io_code(q)
    ws, _ = _workspace(N, R, H, dk, dv, chunk, q.device, workspace, variant)
    st = load().gdn_prefill_shared(
        _dev(q, "q", q.dtype, (N, H, dk)), _dev(k, "k", q.dtype, (N, H, dk)),
        _dev(v, "v", q.dtype, (N, H, dv)),
        _dev(log_alpha, "log_alpha", _F32, _la_shape(variant, N, H, dk)),
        _dev(beta, "beta", _F32, (N, H), optional=True),
        _dev(cu_seqlens, "cu_seqlens", _I32, (R + 1,)),
        R, N, H, dk, dv, chunk, _dev(conv_w, "conv_w", _F32, (cc, 4), optional=True),
        int(bool(qk_l2norm)),
        _dev(init_state, "init_state", _F32, (R, H, dk, dv), optional=True),
        _dev(init_window, "init_window", q.dtype, (R, 3, cc), optional=True),
        _dev(o, "o", _IO, (N, H, dv), optional=True),
        _dev(final_state, "final_state", _F32, (R, H, dk, dv)),
        _dev(final_window, "final_window", q.dtype, (R, 3, cc), optional=True),
        _variant(variant), io, _io_code(o) if o is not None else GDN_F32, ws.data_ptr(),
        ws.numel(), _stream(stream))
    _check("gdn_prefill_shared", st)


def gdn_prefill_checkpointed(q, k, v, log_alpha, beta, cu_seqlens, final_state, ckpt_every,
                             ckpt_state, o=None, ckpt_window=None, conv_w=None, qk_l2norm=False,
                             init_state=None, init_window=None, final_window=None, chunk=64,
                             workspace=None, variant="gdn", stream=None):
    """Call 1 that also keeps checkpoints: ckpt_state[r, j] (and ckpt_window)
    = the state (window) after (j + 1) * ckpt_every * chunk tokens of
    sequence r, when that is inside the sequence or its end."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    R = cu_seqlens.shape[0] - 1
    cap = ckpt_state.shape[1]
    cc = H * (2 * dk + dv)
    io = _io_code(q)
    ws, _ = _workspace(N, R, H, dk, dv, chunk, q.device, workspace, variant)
    st = load().gdn_prefill_checkpointed(
        _dev(q, "q", q.dtype, (N, H, dk)), _dev(k, "k", q.dtype, (N, H, dk)),
        _dev(v, "v", q.dtype, (N, H, dv)),
        _dev(log_alpha, "log_alpha", _F32, _la_shape(variant, N, H, dk)),
        _dev(beta, "beta", _F32, (N, H), optional=True),
        _dev(cu_seqlens, "cu_seqlens", _I32, (R + 1,)),
        R, N, H, dk, dv, chunk, _dev(conv_w, "conv_w", _F32, (cc, 4), optional=True),
        int(bool(qk_l2norm)),
        _dev(init_state, "init_state", _F32, (R, H, dk, dv), optional=True),
        _dev(init_window, "init_window", q.dtype, (R, 3, cc), optional=True),
        _dev(o, "o", _IO, (N, H, dv), optional=True),
        _dev(final_state, "final_state", _F32, (R, H, dk, dv)),
        _dev(final_window, "final_window", q.dtype, (R, 3, cc), optional=True),
        int(ckpt_every), cap, _dev(ckpt_state, "ckpt_state", _F32, (R, cap, H, dk, dv)),
        _dev(ckpt_window, "ckpt_window", q.dtype, (R, cap, 3, cc), optional=True),
        _variant(variant), io, _io_code(o) if o is not None else GDN_F32, ws.data_ptr(),
        ws.numel(), _stream(stream))
    _check("gdn_prefill_checkpointed", st)


def gdn_fork_branches(q, k, v, log_alpha, beta, branch_cu, branch_parent, parent_state, o,
                      parent_window=None, branch_state=None, branch_window=None, conv_w=None,
                      qk_l2norm=False, chunk=64, workspace=None, variant="gdn", stream=None):
    """Call 2 of the two-call fork: every branch from its request's saved state
    (variants as gdn_prefill_shared)."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    NB = branch_cu.shape[0] - 1
    R = parent_state.shape[0]
    cc = H * (2 * dk + dv)
    io = _io_code(q)
    ws, _ = _workspace(N, NB, H, dk, dv, chunk, q.device, workspace, variant)
    st = load().gdn_fork_branches(
        _dev(q, "q", q.dtype, (N, H, dk)), _dev(k, "k", q.dtype, (N, H, dk)),
        _dev(v, "v", q.dtype, (N, H, dv)),
        _dev(log_alpha, "log_alpha", _F32, _la_shape(variant, N, H, dk)),
        _dev(beta, "beta", _F32, (N, H), optional=True),
        _dev(branch_cu, "branch_cu", _I32, (NB + 1,)),
        _dev(branch_parent, "branch_parent", _I32, (NB,)), NB, R, N, H, dk, dv, chunk,
        _dev(conv_w, "conv_w", _F32, (cc, 4), optional=True), int(bool(qk_l2norm)),
        _dev(parent_state, "parent_state", _F32, (R, H, dk, dv)),
        _dev(parent_window, "parent_window", q.dtype, (R, 3, cc), optional=True),
        _dev(o, "o", _IO, (N, H, dv)),
        _dev(branch_state, "branch_state", _F32, (NB, H, dk, dv), optional=True),
        _dev(branch_window, "branch_window", q.dtype, (NB, 3, cc), optional=True),
        _variant(variant), io, _io_code(o), ws.data_ptr(), ws.numel(), _stream(stream))
    _check("gdn_fork_branches", st)


# ------------------------------------------------------------------ fork attention
def fork_attention_workspace_bytes(n_req, n_branch):
    return int(load().gdn_fork_attention_workspace_bytes(n_req, n_branch))


def gdn_fork_attention(q, k, v, cu_seqlens, o, branch_cu=None, branch_parent=None, scale=None,
                       trunk_queries=True, workspace=None, stream=None):
    """Softmax attention over a flat stream under the fork visibility rule
    (a trunk token reads its request's trunk up to itself; a branch token
    its parent request's whole trunk and its own branch up to itself).
    q [N,H,d], k, v [N,H_kv,d] bf16; cu_seqlens [R+1], branch_cu [NB+1]
    (absolute offsets), branch_parent [NB] int32; o [N,H,d] fp32 or bf16.
    `scale` defaults to 1/sqrt(d)."""
    N, H, d = q.shape
    Hkv = k.shape[1]
    R = cu_seqlens.shape[0] - 1
    NB = 0 if branch_cu is None else branch_cu.shape[0] - 1
    need = fork_attention_workspace_bytes(R, NB)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    sc = float(d) ** -0.5 if scale is None else float(scale)
    st = load().gdn_fork_attention(
        _dev(q, "q", torch.bfloat16, (N, H, d)), _dev(k, "k", torch.bfloat16, (N, Hkv, d)),
        _dev(v, "v", torch.bfloat16, (N, Hkv, d)), _dev(cu_seqlens, "cu_seqlens", _I32, (R + 1,)),
        R, _dev(branch_cu, "branch_cu", _I32, (NB + 1,), optional=NB == 0),
        _dev(branch_parent, "branch_parent", _I32, (NB,), optional=NB == 0), NB, N, H, Hkv, d,
        sc, int(bool(trunk_queries)), _dev(o, "o", _IO, (N, H, d)), _io_code(q), _io_code(o),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))
    _check("gdn_fork_attention", st)


def gdn_fork_attention_noalloc(q, k, v, cu_seqlens, o, branch_cu=None, branch_parent=None,
                               scale=None, trunk_queries=True, stream=None):
    """gdn_fork_attention without a workspace: the tile table is the
    library's static per-GPU array (at most FORK_ATTENTION_NOALLOC_MAX_SEGMENTS
    trunks + branches; calls that overlap on one GPU race)."""
    N, H, d = q.shape
    Hkv = k.shape[1]
    R = cu_seqlens.shape[0] - 1
    NB = 0 if branch_cu is None else branch_cu.shape[0] - 1
    sc = float(d) ** -0.5 if scale is None else float(scale)
    st = load().gdn_fork_attention_noalloc(
        _dev(q, "q", torch.bfloat16, (N, H, d)), _dev(k, "k", torch.bfloat16, (N, Hkv, d)),
        _dev(v, "v", torch.bfloat16, (N, Hkv, d)), _dev(cu_seqlens, "cu_seqlens", _I32, (R + 1,)),
        R, _dev(branch_cu, "branch_cu", _I32, (NB + 1,), optional=NB == 0),
        _dev(branch_parent, "branch_parent", _I32, (NB,), optional=NB == 0), NB, N, H, Hkv, d,
        sc, int(bool(trunk_queries)), _dev(o, "o", _IO, (N, H, d)), _io_code(q), _io_code(o),
        _stream(stream))
    _check("gdn_fork_attention_noalloc", st)


def gdn_stream_probe(src, dst, copy=False, stream=None):
    """Measurement aid: stream src (a contiguous device tensor, size a
    multiple of 16 bytes) with non-temporal 16-byte loads; copy=True also
    writes it to dst (same size), else dst (>= 4 bytes) is normally left
    untouched."""
    nbytes = src.numel() * src.element_size()
    if copy and dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    st = load().gdn_stream_probe(_dev(src, "src"), _dev(dst, "dst"), nbytes, 1 if copy else 0,
                                 _stream(stream))
    _check("gdn_stream_probe", st)
