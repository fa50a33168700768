"""Write tests/golden/tiny_oracle.json from the oracle alone.

The paper prints no worked example for the MoE layer, so the only stored
values are the oracle's own answers on the tiny workload (T=64, d=256, f=512,
16 experts, top-2, fp32 activations and scales, seed 0). They guard the oracle
and the input recipe against silent drift; the independent pins are in
tests/test_oracle_*.py. Run from the repository root:

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402
from oracle import moe, quant  # noqa: E402


def tiny_reference():
    w = workloads.TINY
    x = workloads.draw_activations(w).double().numpy()
    wr, bias = workloads.draw_router(w)
    src = workloads.draw_expert_weights(w, "cpu")
    W = {}
    for k in ("gate", "up", "down"):
        W["q_" + k], W["s_" + k] = quant.quantize_rows(src["w_" + k].double().numpy(), w.scale)
    out = moe.moe_forward(x, wr.double().numpy(), None, W, w.K)
    return W, out


def main():
    W, out = tiny_reference()
    doc = {
        "source": "oracle on the tiny workload (T=64, d=256, f=512, E=16, K=2, seed 0); "
                  "written by tests/golden/make_golden.py",
        "ids": out["ids"].tolist(),
        "w": [[float(v) for v in r] for r in out["w"]],
        "y_rows_0_3_first8": [[float(v) for v in out["y"][t, :8]] for t in range(4)],
        "y_abs_sum": float(np.abs(out["y"]).sum()),
        "s_gate_e0_first8": [float(v) for v in W["s_gate"][0, :8]],
        "q_gate_e0_row0_first16": [int(v) for v in W["q_gate"][0, 0, :16]],
        "q_sum_abs": int(sum(int(np.abs(W["q_" + k].astype(np.int64)).sum()) for k in ("gate", "up", "down"))),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(path, "w") as fh:
        json.dump(doc, fh, indent=0)
    print("wrote", path)


if __name__ == "__main__":
    main()
