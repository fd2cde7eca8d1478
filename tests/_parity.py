"""Parity figures per workload, gathered by the GPU parity tests.

Two metrics per quantity (o, final state) and workload, both taken per
(sequence or slot, head) slice and maxed over slices:
  - max_rel_err: max |x - r| / max |r| over the slice (the bar the tests
    assert);
  - elementwise: max over the slice's elements of
    |x - r| / max(|r|, 1e-3 max |r|), an elementwise relative error floored
    at a thousandth of the slice's largest reference value (without a floor
    it is ill-posed near zero).
`record` keeps them; conftest writes them as JSON at the end of the session
when GDN_PARITY_JSON names a file.
"""

import json
import os
import sys

import numpy as np

_RECORDS: dict = {}


def elementwise(x, ref, axes):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    m = np.max(np.abs(ref), axis=axes, keepdims=True)
    den = np.maximum(np.abs(ref), 1e-3 * m)
    diff = np.abs(x - ref)
    e = np.divide(diff, den, out=diff.copy(), where=den > 0)  # zero slice: absolute
    return float(np.max(e))


def rel_err(x, ref, axes):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    m = np.max(np.abs(ref), axis=axes)
    d = np.max(np.abs(x - ref), axis=axes)
    return float(np.max(np.where(m > 0, d / np.where(m > 0, m, 1.0), d)))


def seq_metrics(x, ref, cu):
    """(max_rel_err, elementwise) of [N, H, d] outputs over (sequence, head)
    slices given by token offsets cu."""
    rel = ele = 0.0
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b > a:
            rel = max(rel, rel_err(x[a:b], ref[a:b], (0, 2)))
            ele = max(ele, elementwise(x[a:b], ref[a:b], (0, 2)))
    return rel, ele


def record(config, quantity, rel, ele, bar):
    q = _RECORDS.setdefault(config, {})
    prev = q.get(quantity)
    if prev is not None:  # several cases of one workload: keep the worst
        rel, ele = max(rel, prev["max_rel_err"]), max(ele, prev["elementwise"])
    q[quantity] = {"max_rel_err": rel, "elementwise": ele, "bar": bar}


def write(path):
    if not _RECORDS:
        return
    out = {
        "command": " ".join(["python", "-m", "pytest"] + sys.argv[1:]),
        "metrics": {
            "max_rel_err": "per (sequence or slot, head) slice: max|x-r| / max|r|; max over slices",
            "elementwise": "max over elements of |x-r| / max(|r|, 1e-3 max|r| of the slice)",
        },
        "configs": _RECORDS,
    }
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
