"""Write tests/golden/thresholds.json: the oracle's threshold b for every named
workload, the fp64 sum of its p, the floor that rounding its p to fp32 puts
on |sum p - k|, and the input fingerprints they were computed from.

Calls only the CPU oracle (oracle/) and the seeded input generators; nothing
here touches the GPU path.  Run from the repository root:

    python tests/golden/make_golden.py [c1 c2 ...]
"""
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from differentiable_soft_top_amd.workloads import WORKLOADS, draw_grad, make_workload  # noqa: E402
from oracle import oracle as O  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "thresholds.json")


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def main(names):
    gold = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            gold = json.load(f)
    for name in names:
        t0 = time.time()
        s, k, alpha, w = make_workload(name)
        g = draw_grad(s.size, w.seed)
        p, b = O.forward(s, k, alpha)
        p32 = p.astype(np.float32)
        gold[name] = {
            "n": int(s.size), "k": k, "alpha": alpha, "seed": w.seed, "dist": w.dist,
            "b": b,
            "mass_p64": float(np.sum(p)),
            "mass_p32_rounding_floor": abs(float(np.sum(p32.astype(np.float64))) - k),
            "sha256_scores": sha(s), "sha256_grad": sha(g),
            "oracle_seconds": round(time.time() - t0, 2),
        }
        print(name, gold[name], flush=True)
        del s, g, p, p32
    with open(OUT, "w") as f:
        json.dump(gold, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:] or sorted(WORKLOADS))
