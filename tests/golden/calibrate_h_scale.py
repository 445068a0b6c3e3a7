"""Calibrate the drafter-hidden scale of the Qwen3-8B-shaped single-request
workload so that its mean per-position entropy is about 2 nats.

Runs the fp64 oracle only.  The entropy is the mean, over depths 1..D and over
the surviving beam rows evaluated at each depth, of the entropy of the T=1
corrected distribution softmax(z).  h = alpha * N(0,1); alpha is found by
bisection (entropy falls as alpha grows) to |mean - 2| <= 0.05 and written to
tests/golden/h_scale_qwen3_8b.json.

    python tests/golden/calibrate_h_scale.py
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from draft_tree_construction_02_amd import synth  # noqa: E402
from oracle import dartree_oracle as O  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "h_scale_qwen3_8b.json")


def mean_entropy(head, wl, alpha):
    req = synth.make_requests(wl.d, wl.D, wl.seeds, alpha, wl.root_tok)
    tree = O.build_supertree(head, req.h[0], req.s0[0], int(req.root_tok[0]), wl.D, wl.W, wl.k,
                             1.0, want_entropy=True)
    ents = [e for per_depth in tree.entropies for e in per_depth]
    return float(np.mean(ents))


def main():
    wl = synth.workloads()["qwen3_8b"]
    t0 = time.time()
    hw = synth.make_head(wl.V, wl.d, wl.wdtype, wl.weight_seed)
    head = O.OracleHead(hw.wdtype, hw.E, hw.W1t, hw.W2t, hw.Ut, cache_u=True)
    print(f"weights ready in {time.time() - t0:.1f}s", flush=True)
    lo, hi = 0.05, 1.0
    hist = []
    alpha = None
    for it in range(14):
        mid = 0.5 * (lo + hi)
        t1 = time.time()
        e = mean_entropy(head, wl, mid)
        hist.append((mid, e))
        print(f"alpha {mid:.5f}: mean entropy {e:.4f} nats ({time.time() - t1:.1f}s)", flush=True)
        if abs(e - 2.0) <= 0.05 and alpha is None:
            alpha = mid
        if e > 2.0:
            lo = mid
        else:
            hi = mid
        if hi - lo < 2e-4:
            break
    best = min(hist, key=lambda x: abs(x[1] - 2.0))
    a4 = float(f"{best[0]:.4g}")
    best = (a4, mean_entropy(head, wl, a4))
    print(f"rounded alpha {a4}: mean entropy {best[1]:.4f} nats", flush=True)
    res = {"workload": "Qwen3-8B-shaped single request (d=4096, V=151936, D=16, W=32, k=8, T=1)",
           "definition": "mean over depths and surviving beam rows of the entropy of softmax(z) at T=1, "
                         "oracle fp64 build, h = alpha * N(0,1)",
           "alpha": best[0], "mean_entropy_nats": best[1],
           "history": hist}
    with open(OUT, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res["alpha"]))


if __name__ == "__main__":
    main()
