"""The oracle and the input recipe reproduce the stored tiny-workload answers.

tests/golden/tiny_oracle.json was written by tests/golden/make_golden.py,
which calls only the oracle and the input generator. This is a drift guard,
not an independent pin (the paper prints no worked example).
"""
import json
import os

import numpy as np

from tests.golden.make_golden import tiny_reference

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_oracle.json")


def test_tiny_workload_matches_golden():
    with open(GOLDEN) as fh:
        g = json.load(fh)
    W, out = tiny_reference()
    assert out["ids"].tolist() == g["ids"]
    np.testing.assert_allclose(out["w"], np.array(g["w"]), rtol=1e-12)
    np.testing.assert_allclose(out["y"][:4, :8], np.array(g["y_rows_0_3_first8"]), rtol=1e-10)
    np.testing.assert_allclose(np.abs(out["y"]).sum(), g["y_abs_sum"], rtol=1e-10)
    assert [float(v) for v in W["s_gate"][0, :8]] == g["s_gate_e0_first8"]
    assert [int(v) for v in W["q_gate"][0, 0, :16]] == g["q_gate_e0_row0_first16"]
    total = sum(int(np.abs(W["q_" + k].astype(np.int64)).sum()) for k in ("gate", "up", "down"))
    assert total == g["q_sum_abs"]
    # every token routed to two distinct experts, weights renormalised
    ids = np.array(g["ids"])
    assert np.all(ids[:, 0] != ids[:, 1])
    np.testing.assert_allclose(np.array(g["w"]).sum(axis=1), 1.0, rtol=1e-12)
