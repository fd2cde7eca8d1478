"""Pre-captured HIP graphs for fork rounds: scheduling only.

The Flide page ("연구방법을 단계별로", step 3) runs each round of requests
through graphs captured ahead of time for a few stream capacities: counts and
offsets sit in device buffers, so one captured graph serves any round that
fits its capacity, with padding only at the tail of the stream; a round too
large for the largest graph is split at request boundaries, and a request
too large for any graph runs without one.

`ForkGraphRunner` does exactly that for the two-call GDN fork
(gdn_prefill_shared, then gdn_fork_branches). It owns, per capacity bucket,
static device buffers and one captured graph of the two calls on them. A
round is given as flat device streams (the prefix tokens of its requests in
request order, and the branch tokens grouped by request in the same order)
with host-side lengths; `run` plans the replays, copies each replay's token
ranges into the bucket's buffers, writes the offsets and parents into the
bucket's device metadata, replays the graph and copies the outputs out. It
computes nothing itself: every step of the recurrence runs in the library's
kernels. (An engine that builds its stream directly in `bucket.inputs`
skips the copies.)
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

from . import _lib


@dataclasses.dataclass
class Bucket:
    """One stream capacity: at most `tokens` prefix tokens in at most
    `requests` requests, with at most `branch_tokens` branch tokens in at
    most `branches` branches."""
    tokens: int
    requests: int
    branch_tokens: int
    branches: int


@dataclasses.dataclass
class Replay:
    """One unit of a round's plan: requests [r0, r1) of the round, on
    bucket `bucket` (an index into the runner's buckets), or without a graph
    (bucket None: one request larger than every bucket)."""
    r0: int
    r1: int
    bucket: int | None


def sort_buckets(buckets):
    """Buckets in increasing capacity; each must hold the previous one, so
    the smallest that fits a set of requests is the first that does."""
    out = sorted(buckets, key=lambda b: (b.tokens, b.requests, b.branch_tokens, b.branches))
    for a, b in zip(out, out[1:]):
        if not (a.requests <= b.requests and a.branch_tokens <= b.branch_tokens
                and a.branches <= b.branches):
            raise ValueError(f"bucket {b} does not hold {a}")
    return out


def plan_round(buckets, prefix_lens, branch_counts, branch_lens) -> list[Replay]:
    """Replays for a round: consecutive requests packed into the smallest
    bucket that holds them; a round beyond the largest bucket split at
    request boundaries; a request beyond every bucket alone and without a
    graph. `buckets` sorted by capacity; request r has prefix_lens[r] prefix
    tokens and branch_counts[r] branches, whose lengths are in branch_lens
    (grouped by request, in request order)."""
    pl = [int(x) for x in prefix_lens]
    bc = [int(x) for x in branch_counts]
    bl = [int(x) for x in branch_lens]
    if len(pl) != len(bc) or sum(bc) != len(bl) or min(pl + bc + bl + [0]) < 0:
        raise ValueError("branch_counts must give one non-negative count per request, "
                         "summing to len(branch_lens)")
    bstart = np.concatenate([[0], np.cumsum(bc)]).astype(int)
    btok = [sum(bl[bstart[r]:bstart[r + 1]]) for r in range(len(pl))]

    def fits(b, r0, r1):
        return (sum(pl[r0:r1]) <= b.tokens and r1 - r0 <= b.requests
                and sum(btok[r0:r1]) <= b.branch_tokens and sum(bc[r0:r1]) <= b.branches)

    big = buckets[-1] if buckets else None
    plan, r = [], 0
    while r < len(pl):
        if big is None or not fits(big, r, r + 1):
            plan.append(Replay(r, r + 1, None))
            r += 1
            continue
        r1 = r + 1  # extend while the largest bucket still holds the requests
        while r1 < len(pl) and fits(big, r, r1 + 1):
            r1 += 1
        b = next(i for i, bk in enumerate(buckets) if fits(bk, r, r1))
        plan.append(Replay(r, r1, b))
        r = r1
    return plan


class _Captured:
    def __init__(self, cap: Bucket, H, dk, dv, io_dtype, variant, conv, device):
        self.cap = cap
        N, R, Nb, NB = cap.tokens, cap.requests, cap.branch_tokens, cap.branches
        cc = H * (2 * dk + dv)
        la_shape = (lambda n: (n, H)) if variant == "gdn" else (lambda n: (n, H, dk))
        z = dict(device=device)
        self.inputs = dict(
            q=torch.zeros((N, H, dk), dtype=io_dtype, **z),
            k=torch.zeros((N, H, dk), dtype=io_dtype, **z),
            v=torch.zeros((N, H, dv), dtype=io_dtype, **z),
            log_alpha=torch.zeros(la_shape(N), **z),
            beta=torch.zeros((N, H), **z),
            cu=torch.zeros(R + 1, dtype=torch.int32, **z),
            bq=torch.zeros((Nb, H, dk), dtype=io_dtype, **z),
            bk=torch.zeros((Nb, H, dk), dtype=io_dtype, **z),
            bv=torch.zeros((Nb, H, dv), dtype=io_dtype, **z),
            blog_alpha=torch.zeros(la_shape(Nb), **z),
            bbeta=torch.zeros((Nb, H), **z),
            bcu=torch.zeros(NB + 1, dtype=torch.int32, **z),
            bpar=torch.zeros(NB, dtype=torch.int32, **z),
        )
        self.outputs = dict(
            o=torch.zeros((N, H, dv), **z),
            state=torch.zeros((R, H, dk, dv), **z),
            window=torch.zeros((R, 3, cc), dtype=io_dtype, **z) if conv else None,
            bo=torch.zeros((Nb, H, dv), **z),
            bstate=torch.zeros((NB, H, dk, dv), **z),
            bwindow=torch.zeros((NB, 3, cc), dtype=io_dtype, **z) if conv else None,
        )
        need = max(_lib.prefill_workspace_bytes(N, R, H, dk, dv, variant=variant),
                   _lib.prefill_workspace_bytes(Nb, NB, H, dk, dv, variant=variant), 1)
        self.ws = torch.empty(need, dtype=torch.uint8, device=device)
        self.graph = None


class ForkGraphRunner:
    """Captured two-call fork graphs, one per capacity bucket (see the
    module docstring). `buckets` are tried smallest first (by prefix token
    capacity); conv_w (or None) and qk_l2norm are fixed per runner, as in a
    model layer."""

    def __init__(self, H, dk, dv, buckets, *, conv_w=None, qk_l2norm=False,
                 io_dtype=torch.bfloat16, variant="gdn", device="cuda"):
        self.H, self.dk, self.dv = H, dk, dv
        self.conv_w, self.qk_l2norm = conv_w, qk_l2norm
        self.io_dtype, self.variant, self.device = io_dtype, variant, device
        self.buckets = sort_buckets(buckets)
        self._cap = [_Captured(b, H, dk, dv, io_dtype, variant, conv_w is not None, device)
                     for b in self.buckets]
        for c in self._cap:
            self._capture(c)
        self.last_plan: list[Replay] = []

    # ------------------------------------------------------------ capture
    def _calls(self, c: _Captured):
        i, o = c.inputs, c.outputs
        beta = None if self.variant == "rwkv6" else i["beta"]
        bbeta = None if self.variant == "rwkv6" else i["bbeta"]
        _lib.gdn_prefill_shared(i["q"], i["k"], i["v"], i["log_alpha"], beta, i["cu"],
                                o["state"], o=o["o"], conv_w=self.conv_w,
                                qk_l2norm=self.qk_l2norm, final_window=o["window"],
                                workspace=c.ws, variant=self.variant)
        _lib.gdn_fork_branches(i["bq"], i["bk"], i["bv"], i["blog_alpha"], bbeta, i["bcu"],
                               i["bpar"], o["state"], o["bo"], parent_window=o["window"],
                               branch_state=o["bstate"], branch_window=o["bwindow"],
                               conv_w=self.conv_w, qk_l2norm=self.qk_l2norm, workspace=c.ws,
                               variant=self.variant)

    def _capture(self, c: _Captured):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm-up outside the capture
            self._calls(c)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        c.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(c.graph):
            self._calls(c)

    # ------------------------------------------------------------ planning
    def plan(self, prefix_lens, branch_counts, branch_lens) -> list[Replay]:
        return plan_round(self.buckets, prefix_lens, branch_counts, branch_lens)

    # ------------------------------------------------------------ running
    def run(self, prefix, branch, prefix_lens, branch_counts, branch_lens, out):
        """Run one round. prefix / branch: dicts of flat device tensors q, k,
        v, log_alpha, beta (the round's prefix stream and branch stream);
        out: dict of result tensors o [N,H,dv], state [R,H,dk,dv], window
        [R,3,CC] (conv only), bo [Nb,H,dv], bstate [NB,H,dk,dv], bwindow
        [NB,3,CC] (conv only). Returns the plan it ran."""
        plan = self.plan(prefix_lens, branch_counts, branch_lens)
        pl = np.asarray(prefix_lens, dtype=np.int64)
        bcount = np.asarray(branch_counts, dtype=np.int64)
        bl = np.asarray(branch_lens, dtype=np.int64)
        pcu = np.concatenate([[0], np.cumsum(pl)])
        bstart = np.concatenate([[0], np.cumsum(bcount)])
        bcu = np.concatenate([[0], np.cumsum(bl)])
        for rp in plan:
            t0, t1 = int(pcu[rp.r0]), int(pcu[rp.r1])
            b0, b1 = int(bstart[rp.r0]), int(bstart[rp.r1])
            u0, u1 = int(bcu[b0]), int(bcu[b1])
            cu_loc = (pcu[rp.r0:rp.r1 + 1] - t0).astype(np.int32)
            bcu_loc = (bcu[b0:b1 + 1] - u0).astype(np.int32)
            par_loc = np.repeat(np.arange(rp.r1 - rp.r0), bcount[rp.r0:rp.r1]).astype(np.int32)
            if rp.bucket is None:
                self._run_direct(prefix, branch, t0, t1, u0, u1, cu_loc, bcu_loc, par_loc, out,
                                 rp, b0, b1)
            else:
                self._run_graph(self._cap[rp.bucket], prefix, branch, t0, t1, u0, u1, cu_loc,
                                bcu_loc, par_loc, out, rp, b0, b1)
        self.last_plan = plan
        return plan

    def _run_graph(self, c, prefix, branch, t0, t1, u0, u1, cu_loc, bcu_loc, par_loc, out, rp,
                   b0, b1):
        i, o = c.inputs, c.outputs
        n, nb = t1 - t0, u1 - u0
        nreq, nbr = rp.r1 - rp.r0, b1 - b0
        for name in ("q", "k", "v", "log_alpha", "beta"):
            if name == "beta" and self.variant == "rwkv6":
                continue
            i[name][:n].copy_(prefix[name][t0:t1])
            i["b" + name][:nb].copy_(branch[name][u0:u1])
        # offsets: the round's requests, then empty sequences at the tail
        cu = np.full(c.cap.requests + 1, n, dtype=np.int32)
        cu[:nreq + 1] = cu_loc
        bcu = np.full(c.cap.branches + 1, nb, dtype=np.int32)
        bcu[:nbr + 1] = bcu_loc
        par = np.zeros(c.cap.branches, dtype=np.int32)
        par[:nbr] = par_loc
        i["cu"].copy_(torch.from_numpy(cu))
        i["bcu"].copy_(torch.from_numpy(bcu))
        i["bpar"].copy_(torch.from_numpy(par))
        c.graph.replay()
        out["o"][t0:t1].copy_(o["o"][:n])
        out["state"][rp.r0:rp.r1].copy_(o["state"][:nreq])
        out["bo"][u0:u1].copy_(o["bo"][:nb])
        out["bstate"][b0:b1].copy_(o["bstate"][:nbr])
        if o["window"] is not None:
            out["window"][rp.r0:rp.r1].copy_(o["window"][:nreq])
            out["bwindow"][b0:b1].copy_(o["bwindow"][:nbr])

    def _run_direct(self, prefix, branch, t0, t1, u0, u1, cu_loc, bcu_loc, par_loc, out, rp,
                    b0, b1):
        dev = self.device
        beta = None if self.variant == "rwkv6" else prefix["beta"][t0:t1]
        bbeta = None if self.variant == "rwkv6" else branch["beta"][u0:u1]
        st = out["state"][rp.r0:rp.r1]
        win = None if out.get("window") is None else out["window"][rp.r0:rp.r1]
        _lib.gdn_prefill_shared(prefix["q"][t0:t1], prefix["k"][t0:t1], prefix["v"][t0:t1],
                                prefix["log_alpha"][t0:t1], beta,
                                torch.from_numpy(cu_loc).to(dev), st, o=out["o"][t0:t1],
                                conv_w=self.conv_w, qk_l2norm=self.qk_l2norm,
                                final_window=win, variant=self.variant)
        if b1 > b0:
            _lib.gdn_fork_branches(
                branch["q"][u0:u1], branch["k"][u0:u1], branch["v"][u0:u1],
                branch["log_alpha"][u0:u1], bbeta, torch.from_numpy(bcu_loc).to(dev),
                torch.from_numpy(par_loc).to(dev), st, out["bo"][u0:u1], parent_window=win,
                branch_state=out["bstate"][b0:b1],
                branch_window=None if out.get("bwindow") is None else out["bwindow"][b0:b1],
                conv_w=self.conv_w, qk_l2norm=self.qk_l2norm, variant=self.variant)
