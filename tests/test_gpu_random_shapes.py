"""moe_layer_forward and moe_layer_backward on seeded random shapes against the oracle:
token counts from 1 up, one to 48 experts, K up to 6, hidden and intermediate sizes over the
multiples each path takes, and the three routing kinds of the workloads (normal and skewed
logits, given ids). The shapes are drawn once from a fixed seed, so every run checks the same
cases. A bf16 case on a shape the single FFN launch takes is also run with the FFN as one
launch and as two, which must agree bit for bit; each forward case also runs the scatter-add
combine."""
import os
import sys

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from workloads import gen, to_numpy_bits

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from _backward_check import check_backward  # noqa: E402
from _gpu_run import run_layer  # noqa: E402
from _oracle_run import oracle_layer, rel_err  # noqa: E402

import mixture_experts_layer_counting_amd as moe  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}


def draw_cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        act = ("f32", "bf16", "fp8")[i % 3]
        T = int(rng.choice([1, 7, int(rng.integers(8, 700)), int(rng.integers(8, 700))]))
        E = int(rng.choice([1, int(rng.integers(2, 49)), int(rng.integers(2, 49)), int(rng.integers(2, 49))]))
        K = int(rng.integers(1, min(E, 6) + 1))
        if act == "f32":
            H, Hp = int(rng.integers(1, 9)) * 24, int(rng.integers(1, 9)) * 16
        else:
            H, Hp = int(rng.choice([256, 512, 768])), int(rng.choice([128, 256, 384, 512]))
        routing = str(rng.choice(["normal", "skew", "balanced"]))
        spec = dict(T=T, H=H, Hp=Hp, E=E, K=K, routing=routing)
        if routing == "skew":
            spec["beta"] = float(rng.uniform(0.2, 3.0))
        cases.append((act, spec))
    return cases


CASES = draw_cases()


def decode(w, out):
    bits = to_numpy_bits(out)
    return np.asarray(bits, np.float64) if w.out == "f32" else O.decode_bf16(bits)


@pytest.mark.parametrize("act,spec", CASES,
                         ids=[f"{a}_T{s['T']}_H{s['H']}_Hp{s['Hp']}_E{s['E']}_K{s['K']}_{s['routing']}"
                              for a, s in CASES])
def test_random_shape_against_the_oracle(act, spec):
    print(f"\n[case] random shape {act} {spec}", flush=True)
    wgt, out = {"f32": ("f32", "f32"), "bf16": ("bf16", "bf16"), "fp8": ("mxfp4", "bf16")}[act]
    w = gen.make(**spec, act=act, wgt=wgt, out=out, cid=401, device=DEV)
    got, _, _ = run_layer(w)
    sc, _, _ = run_layer(w, combine=moe.MOE_COMBINE_SCATTER_ATOMIC)
    torch.cuda.synchronize()
    ref = oracle_layer(w)["out"]
    e = rel_err(decode(w, got), ref)
    e_sc = rel_err(decode(w, sc), ref)
    print(f"  out rel err {e:.3e}, scatter-add combine {e_sc:.3e} (tol {TOL[act]})", flush=True)
    assert e <= TOL[act] and e_sc <= TOL[act]
    takes_single = (act == "bf16" and w.H % 256 == 0 and w.Hp % 128 == 0 and min(w.H, w.Hp) >= 256)
    if takes_single:
        res = {}
        for v in ("0", "1"):
            os.environ["MOE_LAYER_FUSED"] = v
            try:
                res[v], _, _ = run_layer(w)
            finally:
                del os.environ["MOE_LAYER_FUSED"]
        torch.cuda.synchronize()
        assert torch.equal(res["0"].view(torch.int16), res["1"].view(torch.int16))


def draw_backward_cases(n=8, seed=2025):
    """bf16 shapes the backward takes (H and H' multiples of 256)."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        T = int(rng.choice([1, 5, int(rng.integers(6, 500)), int(rng.integers(6, 500))]))
        E = int(rng.choice([1, int(rng.integers(2, 40)), int(rng.integers(2, 40))]))
        K = int(rng.integers(1, min(E, 6) + 1))
        spec = dict(T=T, H=int(rng.choice([256, 512, 768])), Hp=int(rng.choice([256, 512])), E=E, K=K,
                    routing=str(rng.choice(["normal", "skew", "balanced"])))
        if spec["routing"] == "skew":
            spec["beta"] = float(rng.uniform(0.2, 3.0))
        cases.append(spec)
    return cases


BWD_CASES = draw_backward_cases()


@pytest.mark.parametrize("spec", BWD_CASES,
                         ids=[f"T{s['T']}_H{s['H']}_Hp{s['Hp']}_E{s['E']}_K{s['K']}_{s['routing']}"
                              for s in BWD_CASES])
def test_random_shape_backward_against_the_oracle(spec):
    print(f"\n[case] random-shape backward {spec}", flush=True)
    w = gen.make(**spec, act="bf16", wgt="bf16", out="bf16", cid=402, device=DEV)
    g = torch.Generator(device="cpu").manual_seed(spec["T"] * 131 + spec["E"])
    dout = torch.randn((w.T, w.H), generator=g).to(torch.bfloat16).to(DEV)
    check_backward(w, dout)
