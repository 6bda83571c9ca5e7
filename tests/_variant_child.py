"""Child process of test_gpu_variants.py: one bf16 layer through the C ABI, checked against the
oracle. The kernel variant comes from the environment, which the library reads once per
process. Prints one line per case and exits non-zero on a mismatch."""
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

from oracle import moe_oracle as O  # noqa: E402
from workloads import gen, to_numpy_bits  # noqa: E402
from _gpu_run import run_layer, run_steps  # noqa: E402
from _oracle_run import oracle_layer, rel_err  # noqa: E402

CASES = [
    # several tiles per block (the cross-tile prefetch and its absence), K loops of 8 and 24
    dict(T=2048, H=256, Hp=256, E=1024, K=8, routing="skew", beta=0.6),
    dict(T=4096, H=768, Hp=768, E=16, K=6, routing="normal"),
    # ragged groups, empty experts
    dict(T=600, H=512, Hp=256, E=32, K=6, routing="skew", beta=3.0),
]


def main():
    bad = 0
    for spec in CASES:
        w = gen.make(**spec, act="bf16", wgt="bf16", out="bf16", cid=74, device="cuda:0")
        r = run_steps(w)
        out_layer, _, _ = run_layer(w)
        torch.cuda.synchronize()
        ref = oracle_layer(w)
        e_y = rel_err(O.decode_bf16(to_numpy_bits(r["y_rows"])), ref["y_rows"])
        e_out = rel_err(O.decode_bf16(to_numpy_bits(r["out"])), ref["out"])
        same = bool(torch.equal(out_layer.view(torch.int16), r["out"].view(torch.int16)))
        ok = e_y <= 2e-2 and e_out <= 2e-2 and same and np.array_equal(to_numpy_bits(r["row_src"]),
                                                                        ref["row_src"])
        print(f"variant {os.environ.get('MOE_FFN_PIPE', '-')}/{os.environ.get('MOE_FFN_PF', '-')}/"
              f"{os.environ.get('MOE_FFN_ORDER', '-')} {spec}: y {e_y:.3e} out {e_out:.3e} "
              f"layer==steps {same} -> {'ok' if ok else 'MISMATCH'}", flush=True)
        bad += not ok
    sys.exit(1 if bad else 0)


if __name__ == "__main__":
    main()
