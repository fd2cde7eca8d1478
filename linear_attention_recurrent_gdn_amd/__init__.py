"""MI355X-native (gfx950) Gated DeltaNet recurrence library.

Thin Python binding over the C ABI of libgdn_mi355x.so (include/gdn_mi355x.h):
shared-context prefill and forked branches (the two-call GDN fork of the
Flide page), eager decode, and deferred base + log decode with its merge
(the DeltaLog page), and the softmax-attention half of the fork (attention
under the trunk + own-branch visibility rule), plus a runner that replays
pre-captured fork graphs per stream-capacity bucket. Tensors are torch device
tensors; every step of the computation runs in the HIP kernels.
"""

from ._lib import (  # noqa: F401
    GDN_BF16,
    GDN_F32,
    GDNError,
    deltalog_append_decode,
    deltalog_merge,
    fork_attention_workspace_bytes,
    gdn_decode_eager,
    gdn_fork_attention,
    gdn_fork_attention_noalloc,
    gdn_fork_branches,
    gdn_prefill_checkpointed,
    gdn_prefill_shared,
    gdn_stream_probe,
    load,
    prefill_workspace_bytes,
    status_string,
)
from .graphs import Bucket, ForkGraphRunner, Replay, plan_round  # noqa: F401

__all__ = [
    "gdn_prefill_shared",
    "gdn_fork_branches",
    "gdn_prefill_checkpointed",
    "gdn_decode_eager",
    "deltalog_append_decode",
    "deltalog_merge",
    "gdn_fork_attention",
    "gdn_fork_attention_noalloc",
    "fork_attention_workspace_bytes",
    "prefill_workspace_bytes",
    "gdn_stream_probe",
    "status_string",
    "load",
    "GDNError",
    "Bucket",
    "ForkGraphRunner",
    "Replay",
    "plan_round",
]
