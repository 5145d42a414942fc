"""Computes the two calibrated constants of lsa_inputs' workloads with the CPU
oracle only (test infrastructure; run by hand, prints the values to paste):

* THRESH_256K_TAU: sigmoid of the midpoint between the 1311th and 1312th
  largest step-0 scores pooled over the batch of the 256K threshold workload
  (0.5% of 4 x 65536 entries pass at step 0).
* SWAP_1M_DRIFT: the per-step redraw fraction of the 1M workload's indexer
  queries for which consecutive top-512 sets overlap by about 80%.
"""
import math
import os
import sys
import time

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import lsa_inputs as L
import oracle


def tau_256k() -> float:
    wl = L.WORKLOADS["thresh_256k"]
    allv = []
    for b in range(wl.batch):
        keys = L.indexer_keys(wl, b)
        q, w = L.indexer_query(wl, b, 0)
        allv.append(oracle.score(keys, wl.key_dtype, q, w, wl.ensemble))
    v = np.sort(np.concatenate(allv))[::-1].astype(np.float64)
    target = int(round(0.005 * v.size))
    hi = v[target - 1]
    lo_i = target
    while v[lo_i] == hi:
        lo_i += 1
    t = 0.5 * (hi + v[lo_i])
    tau = 1.0 / (1.0 + math.exp(-t))
    print(f"256K: t*={t!r} tau={tau!r} passing at step 0: {int((v > t).sum())} of {v.size}", flush=True)
    return tau


def overlap_1m(drift: float, steps: int) -> float:
    wl = L.WORKLOADS["swap_1m"].replace(drift=drift)
    keys = L.indexer_keys(wl, 0)
    q, w = L.indexer_query_steps(wl, 0, steps)
    prev, ovs = None, []
    for t in range(steps):
        s = oracle.select(oracle.score(keys, wl.key_dtype, q[t], w[t], wl.ensemble), "topk", wl.k)
        if prev is not None:
            ovs.append(np.intersect1d(prev, s).size / wl.k)
        prev = s
    return float(np.mean(ovs))


def drift_1m(steps: int = 12) -> float:
    lo, hi = 0.0, 0.2
    best = None
    for _ in range(7):
        mid = 0.5 * (lo + hi)
        t0 = time.time()
        ov = overlap_1m(mid, steps)
        print(f"1M: drift={mid:.5f} overlap={ov:.3f} ({time.time() - t0:.1f}s)", flush=True)
        if best is None or abs(ov - 0.80) < abs(best[1] - 0.80):
            best = (mid, ov)
        if ov > 0.80:
            lo = mid
        else:
            hi = mid
    return round(best[0], 5)


if __name__ == "__main__":
    which = sys.argv[1:] or ["tau", "drift"]
    if "tau" in which:
        print("THRESH_256K_TAU =", repr(tau_256k()))
    if "drift" in which:
        print("SWAP_1M_DRIFT =", drift_1m())
