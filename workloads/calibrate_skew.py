"""Find the skew strength beta that gives each target maxvio for the 384-expert layer
(T=8192, E=384, K=8) and write it to skew_bias.json beside this script.

The realised maxvio is measured with the CPU oracle's routing and counts only
(oracle.route_topk, oracle.count_offsets, oracle.maxvio); nothing from the HIP library
is used. beta = 0 when the unbiased logits already reach the target.

    python workloads/calibrate_skew.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle import moe_oracle as O  # noqa: E402
from workloads.gen import SKEW_TARGETS, skew_logits  # noqa: E402

T, E, K = 8192, 384, 8


def realised(beta: float, cid: int) -> float:
    idx, _ = O.route_topk(skew_logits(T, E, beta, seed=0, cid=cid), K)
    counts, _ = O.count_offsets(idx, E)
    return O.maxvio(counts, T, K, E)


def calibrate(target: float, cid: int):
    base = realised(0.0, cid)
    if base >= target:
        return 0.0, base
    lo, hi = 0.0, 0.5
    while realised(hi, cid) < target:
        lo, hi = hi, hi * 2
    best = (hi, realised(hi, cid))
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        v = realised(mid, cid)
        if abs(v - target) < abs(best[1] - target):
            best = (mid, v)
        if v < target:
            lo = mid
        else:
            hi = mid
        if abs(v - target) <= 0.005 * target:
            break
    return best


def main():
    table = {}
    # config ids of the skewed workloads (bf16 layer and its fp8 x MXFP4 variant)
    for cid, targets in ((3, SKEW_TARGETS), (4, (1.0,))):
        for tgt in targets:
            beta, got = calibrate(tgt, cid)
            key = f"T{T}_E{E}_K{K}_maxvio{tgt:g}" + ("" if cid == 3 else "_lowp")
            table[key] = dict(beta=beta, realised_maxvio=got, config_id=cid)
            print(key, table[key], flush=True)
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "skew_bias.json")
    with open(out, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    print("wrote", out)


if __name__ == "__main__":
    main()
