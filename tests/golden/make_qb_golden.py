"""Write qb_57344x896_k16.json: the oracle's QB routing of the routing-only
workload (T=57344 tokens, n=896 experts, k=16; logits N(0,1) plus a
per-expert offset N(0, 0.5^2), seed 0; fp32 sigmoid scores).

Calls only the oracle and the seeded input generator:

    python tests/golden/make_qb_golden.py
"""
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import workloads  # noqa: E402
from oracle import layer as olayer  # noqa: E402
from oracle import qb  # noqa: E402


def main():
    cfg = workloads.QB_SHAPE
    s = olayer.sigmoid(workloads.qb_logits(cfg["T"], cfg["n"], cfg["offset_std"], 0)).astype(np.float32)
    t0 = time.time()
    r = qb.route_qb(s, cfg["k"])
    out = {
        "workload": "QB routing T=57344 n=896 k=16, offset std 0.5, seed 0",
        "idx_sha256": hashlib.sha256(r["idx"].astype("<i4").tobytes()).hexdigest(),
        "bias_fixed": [int(v) for v in r["bfx"]],
        "info": [int(v) for v in r["info"]],
        "loads_min_max": [int(r["loads"].min()), int(r["loads"].max())],
        "oracle_seconds": round(time.time() - t0, 1),
    }
    with open(os.path.join(HERE, "qb_57344x896_k16.json"), "w") as f:
        json.dump(out, f)
    print(json.dumps({k: v for k, v in out.items() if k != "bias_fixed"}))


if __name__ == "__main__":
    main()
