"""The parity metrics the GPU tests record (no GPU): the slice-relative
error and the floored elementwise diagnostic on hand-made cases."""

import json

import numpy as np

import _parity


def test_rel_err_is_per_slice_max_over_slice_max():
    ref = np.array([[1.0, -4.0], [0.5, 0.25]])
    x = ref + np.array([[0.0, 0.4], [0.05, 0.0]])
    # row 0: 0.4 / 4 = 0.1; row 1: 0.05 / 0.5 = 0.1 -> axes=1 per row
    assert np.isclose(_parity.rel_err(x, ref, (1,)), 0.1)
    x[1, 1] += 0.1  # row 1: 0.1 / 0.5 = 0.2
    assert np.isclose(_parity.rel_err(x, ref, (1,)), 0.2)


def test_elementwise_floor_and_zero_slice():
    ref = np.array([[1000.0, 1e-9], [0.0, 0.0]])
    x = np.array([[1000.0, 0.5], [0.0, 3e-7]])
    # row 0: |0.5 - 1e-9| / max(1e-9, 1e-3 * 1000) = 0.5; row 1 (all zero): absolute 3e-7
    assert np.isclose(_parity.elementwise(x, ref, (1,)), 0.5)
    assert np.isclose(_parity.elementwise(x[1:], ref[1:], (1,)), 3e-7)


def test_seq_metrics_skips_empty_sequences():
    ref = np.ones((5, 1, 2))
    x = ref.copy()
    x[3, 0, 1] = 1.5
    rel, ele = _parity.seq_metrics(x, ref, [0, 0, 3, 5])
    assert np.isclose(rel, 0.5) and np.isclose(ele, 0.5)


def test_record_keeps_worst_and_writes(tmp_path):
    _parity._RECORDS.clear()
    _parity.record("cfg", "o", 1e-4, 2e-4, 2e-3)
    _parity.record("cfg", "o", 5e-5, 3e-4, 2e-3)
    path = tmp_path / "p.json"
    _parity.write(str(path))
    out = json.loads(path.read_text())
    assert out["configs"]["cfg"]["o"] == {"max_rel_err": 1e-4, "elementwise": 3e-4, "bar": 2e-3}
    _parity._RECORDS.clear()


def test_committed_parity_by_config():
    """profiles/parity_by_config.json (written by the GPU parity tests) holds
    all five workloads, each within its bar: C1 (fp32 throughout) 1e-5, the
    others 2e-3."""
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    with open(os.path.join(root, "profiles", "parity_by_config.json")) as f:
        data = json.load(f)
    configs = data["configs"]
    for tag in ("C1", "C2", "C3", "C4", "C5"):
        assert any(c.startswith(tag) for c in configs), tag
    for name, quantities in configs.items():
        bar = 1e-5 if name.startswith("C1") else 2e-3
        for q, v in quantities.items():
            assert v["bar"] == bar, (name, q)
            assert 0.0 <= v["max_rel_err"] <= bar, (name, q, v)
            assert v["elementwise"] >= v["max_rel_err"] * 0.999, (name, q, v)
