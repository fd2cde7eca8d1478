"""The C-ABI library loads, exports every symbol the header declares, and
rejects bad host-side arguments before any HIP call (no GPU needed)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn_mi355x.h")
LIB = os.path.join(ROOT, "linear_attention_recurrent_gdn_amd", "libgdn_mi355x.so")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import linear_attention_recurrent_gdn_amd.build as b
        b.build()
    from linear_attention_recurrent_gdn_amd import _lib
    return _lib.load()


def test_header_declares_the_five_operations():
    names = declared_functions()
    for op in ["gdn_prefill_shared", "gdn_fork_branches", "gdn_decode_eager",
               "deltalog_append_decode", "deltalog_merge"]:
        assert op in names


def test_every_declared_symbol_is_exported_and_bound(lib):
    from linear_attention_recurrent_gdn_amd import _lib
    names = declared_functions()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(lib, n), f"{n} declared but not exported"
        assert n in _lib.SIGNATURES, f"{n} has no binding"
    assert set(_lib.SIGNATURES) == set(names)


def test_status_strings(lib):
    assert lib.gdn_status_string(OK) == b"ok"
    assert b"invalid" in lib.gdn_status_string(INVALID)
    assert lib.gdn_max_log_capacity() >= 16


P = ctypes.c_void_p
FAKE = P(0x1000)  # never dereferenced: every call below fails validation first
NULL = None


def eager(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, la=FAKE, beta=FAKE, state=FAKE, slot=NULL, o=FAKE, B=2, H=2,
             dk=128, dv=128, S=2, var=0, io=1, od=0)
    a.update(kw)
    return lib.gdn_decode_eager(a["q"], a["k"], a["v"], a["la"], a["beta"], a["state"], a["slot"],
                                a["o"], a["B"], a["H"], a["dk"], a["dv"], a["S"], a["var"], a["io"],
                                a["od"], NULL)


def test_decode_validation(lib):
    assert eager(lib, q=NULL) == INVALID
    assert eager(lib, beta=NULL) == INVALID          # GDN needs beta
    assert eager(lib, H=0) == INVALID
    assert eager(lib, B=-1) == INVALID
    assert eager(lib, B=3, S=2) == INVALID            # identity slots need B <= n_slots
    assert eager(lib, var=7) == INVALID
    assert eager(lib, io=5) == INVALID
    assert eager(lib, dk=96, dv=96) == UNSUPPORTED
    assert eager(lib, dk=128, dv=48) == UNSUPPORTED
    assert eager(lib, dk=16, dv=64) == UNSUPPORTED


def test_append_validation(lib):
    def call(Mcap=8, merge_at=8, log_len=FAKE, var=0):
        return lib.deltalog_append_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                          log_len, NULL, FAKE, 2, 2, 128, 128, 2, Mcap, merge_at,
                                          var, 1, 0, NULL)
    assert call(log_len=NULL) == INVALID
    assert call(Mcap=0) == INVALID
    assert call(merge_at=9) == INVALID
    assert call(merge_at=-1) == INVALID
    assert call(Mcap=lib.gdn_max_log_capacity() + 1, merge_at=1) == UNSUPPORTED


def test_merge_validation(lib):
    assert lib.deltalog_merge(NULL, FAKE, FAKE, FAKE, FAKE, NULL, 2, 2, 128, 128, 2, 8, 1, 0, 1,
                              NULL) == INVALID
    assert lib.deltalog_merge(FAKE, FAKE, FAKE, FAKE, FAKE, NULL, 2, 2, 48, 48, 2, 8, 1, 0, 1,
                              NULL) == UNSUPPORTED


def test_prefill_validation_and_workspace(lib):
    need = lib.gdn_prefill_workspace_bytes(1000, 3, 4, 128, 128, 64, 0)
    assert lib.gdn_prefill_workspace_bytes(1000, 3, 4, 128, 128, 64, 1) > need  # per-key record
    assert need > 0

    def call(ws=FAKE, ws_bytes=need, chunk=64, final=FAKE, cu=FAKE, d=128, beta=FAKE,
             variant=0):
        return lib.gdn_prefill_shared(FAKE, FAKE, FAKE, FAKE, beta, cu, 3, 1000, 4, d, d, chunk,
                                      NULL, 0, NULL, NULL, FAKE, final, NULL, variant, 1, 0, ws,
                                      ws_bytes, NULL)
    assert call(final=NULL) == INVALID
    assert call(cu=NULL) == INVALID
    assert call(variant=3) == INVALID
    assert call(variant=-1) == INVALID
    # beta is required by the delta-rule variants (may be NULL only for RWKV6)
    assert call(beta=NULL, variant=0) == INVALID
    assert call(beta=NULL, variant=1) == INVALID
    # chunk: 16, 32 and 64 are the interface's sizes, only 64 is built;
    # anything else is not a chunk size
    assert call(chunk=48) == INVALID
    assert call(chunk=0) == INVALID
    assert call(chunk=-64) == INVALID
    assert call(chunk=16) == UNSUPPORTED
    assert call(chunk=32) == UNSUPPORTED
    assert call(d=80) == UNSUPPORTED
    assert call(ws=NULL) == WORKSPACE
    assert call(ws_bytes=need - 1) == WORKSPACE
    # checkpoints: spacing >= 1, capacity >= 0, a state buffer when capacity > 0
    def ck(every=1, cap=2, buf=FAKE):
        return lib.gdn_prefill_checkpointed(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3, 1000, 4, 128,
                                            128, 64, NULL, 0, NULL, NULL, FAKE, FAKE, NULL,
                                            every, cap, buf, NULL, 0, 1, 0, FAKE, need, NULL)
    assert ck(every=0) == INVALID
    assert ck(cap=-1) == INVALID
    assert ck(buf=NULL) == INVALID
    # fork: the parent state and o are required
    assert lib.gdn_fork_branches(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3, 1, 100, 4, 128, 128,
                                 64, NULL, 0, NULL, NULL, FAKE, NULL, NULL, 0, 1, 0, FAKE, need,
                                 NULL) == INVALID


def test_fork_attention_validation_and_workspace(lib):
    need = lib.gdn_fork_attention_workspace_bytes(2, 5)
    assert need == 4 * (2 + 5 + 1)

    def call(q=FAKE, cu=FAKE, bcu=FAKE, bpar=FAKE, nb=5, H=8, Hkv=2, d=128, scale=0.1,
             io=1, out=0, ws=FAKE, ws_bytes=need):
        return lib.gdn_fork_attention(q, FAKE, FAKE, cu, 2, bcu, bpar, nb, 100, H, Hkv, d, scale,
                                      1, FAKE, io, out, ws, ws_bytes, NULL)
    assert call(q=NULL) == INVALID
    assert call(cu=NULL) == INVALID
    assert call(bcu=NULL) == INVALID
    assert call(bpar=NULL) == INVALID
    assert call(Hkv=3) == INVALID                  # does not divide H
    assert call(Hkv=0) == INVALID
    assert call(scale=float("nan")) == INVALID
    assert call(scale=float("inf")) == INVALID
    assert call(scale=0.0) == INVALID
    assert call(scale=-0.1) == INVALID
    assert call(out=2) == INVALID
    assert call(nb=-1) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(d=32) == UNSUPPORTED
    assert call(io=0) == UNSUPPORTED               # fp32 q/k/v not built
    # 32-bit in-kernel row offsets: n_tokens * H * d < 2^31
    assert lib.gdn_fork_attention(FAKE, FAKE, FAKE, FAKE, 2, FAKE, FAKE, 5, 1 << 21, 8, 2, 128,
                                  0.1, 1, FAKE, 1, 0, FAKE, need, NULL) == UNSUPPORTED
    assert call(ws=NULL) == WORKSPACE
    assert call(ws_bytes=need - 1) == WORKSPACE


def test_fork_attention_noalloc_validation(lib):
    """Host-side checks run before any HIP call, including the bound on the
    static tile table (n_req + n_branch)."""
    from linear_attention_recurrent_gdn_amd import _lib
    cap = _lib.FORK_ATTENTION_NOALLOC_MAX_SEGMENTS
    text = open(HEADER).read()
    assert f"#define GDN_FORK_ATTENTION_NOALLOC_MAX_SEGMENTS {cap}" in text

    def call(q=FAKE, cu=FAKE, n_req=2, nb=5, H=8, Hkv=2, d=128, scale=0.1, io=1, out=0):
        return lib.gdn_fork_attention_noalloc(q, FAKE, FAKE, cu, n_req, FAKE, FAKE, nb, 100, H,
                                              Hkv, d, scale, 1, FAKE, io, out, NULL)
    assert call(q=NULL) == INVALID
    assert call(cu=NULL) == INVALID
    assert call(Hkv=3) == INVALID
    assert call(scale=0.0) == INVALID
    assert call(nb=-1) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(io=0) == UNSUPPORTED
    assert call(n_req=cap, nb=1) == WORKSPACE       # one segment past the table
    assert call(n_req=cap // 2, nb=cap - cap // 2 + 7) == WORKSPACE


def test_stream_probe_validation(lib):
    assert lib.gdn_stream_probe(NULL, FAKE, 1024, 0, NULL) == INVALID
    assert lib.gdn_stream_probe(FAKE, NULL, 1024, 1, NULL) == INVALID
    assert lib.gdn_stream_probe(FAKE, FAKE, 1000, 0, NULL) == INVALID   # not a multiple of 16
    assert lib.gdn_stream_probe(FAKE, FAKE, 1024, 2, NULL) == INVALID   # mode 0 or 1
    assert lib.gdn_stream_probe(NULL, NULL, 0, 1, NULL) == OK              # nothing to stream


def test_prefill_workspace_runs_in_segments(lib):
    """The fork_prefill prefix (65,536 tokens, 8 sequences, H=16, d=128)
    runs in segments whose records stay within 512 MiB: its workspace is at
    most 0.5 KiB per token-head (one segment would need 1.39 KiB), and a
    smaller bound gives a smaller workspace."""
    n, R, H, d = 65536, 8, 16, 128
    env = "GDN_PREFILL_SEGMENT_RECORD_BYTES"
    old = os.environ.pop(env, None)
    try:
        default = lib.gdn_prefill_workspace_bytes(n, R, H, d, d, 64, 0)
        assert default <= 512 * n * H, default / (n * H)
        os.environ[env] = str(1 << 40)  # one segment
        one = lib.gdn_prefill_workspace_bytes(n, R, H, d, d, 64, 0)
        assert one > 1.3 * 1024 * n * H
        os.environ[env] = str(64 << 20)
        assert lib.gdn_prefill_workspace_bytes(n, R, H, d, d, 64, 0) < default
    finally:
        os.environ.pop(env, None)
        if old is not None:
            os.environ[env] = old
