"""moe_layer_forward captured into a HIP graph and replayed. Each replay is compared with the
eager result on the same inputs. New inputs are copied in before each replay, and the program
makes its own eager call on the same workspace after it, so the graph has to recompute every
time and must not depend on what an earlier call left in the workspace. The gather combine is
deterministic, so those layers compare bit for bit. The scatter combine adds with fp32 atomics
in a varying order and is compared within one bf16 rounding of the output."""
import os
import sys

import pytest
import torch

from workloads import gen

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from _gpu_run import TORCH_DT, layer_desc  # noqa: E402

import mixture_experts_layer_counting_amd as moe  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

SKEW = dict(T=600, H=512, Hp=256, E=32, K=6, routing="skew", beta=0.8)
# (id, shape, act, wgt, combine, MOE_LAYER_FUSED or None for the default choice)
CASES = [
    ("bf16_one_ffn_launch", SKEW, "bf16", "bf16", "gather", "1"),
    ("bf16_two_ffn_launches", SKEW, "bf16", "bf16", "gather", "0"),
    ("fp8_mxfp4", dict(T=300, H=512, Hp=256, E=12, K=3, routing="skew", beta=0.5), "fp8", "mxfp4", "gather", None),
    ("bf16_scatter_combine_one_ffn_launch", SKEW, "bf16", "bf16", "scatter", "1"),
    ("bf16_scatter_combine_two_ffn_launches", SKEW, "bf16", "bf16", "scatter", "0"),
    ("f32", dict(T=333, H=200, Hp=72, E=9, K=3, routing="skew", beta=0.5), "f32", "f32", "gather", None),
]


def inputs_of(w):
    """The per-call inputs (activations, their fp8 scales, routing logits); weights stay."""
    return [t for t in (w.x, w.x_sf, w.logits) if t is not None]


@pytest.mark.parametrize("name,spec,act,wgt,combine,fused", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(name, spec, act, wgt, combine, fused):
    print(f"\n[case] graph replays {name} {spec}", flush=True)
    out_fmt = "f32" if act == "f32" else "bf16"
    draws = [gen.make(**spec, act=act, wgt=wgt, out=out_fmt, cid=301 + i, device=DEV) for i in range(3)]
    w = draws[0]
    sets = [[t.clone() for t in inputs_of(v)] for v in draws]
    cmode = moe.MOE_COMBINE_SCATTER_ATOMIC if combine == "scatter" else moe.MOE_COMBINE_GATHER
    d = layer_desc(w, cmode)
    nbytes = moe.moe_layer_workspace_bytes(d)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    out = torch.empty((w.T, w.H), dtype=TORCH_DT[out_fmt], device=DEV)
    out_e = torch.empty_like(out)

    def load(i):
        for dst, src in zip(inputs_of(w), sets[i]):
            dst.copy_(src)

    def call(o):
        moe.moe_layer_forward(d, w.x, w.x_sf, w.logits, w.topk_idx, w.topk_w, w.w_gate, w.w_up,
                              w.w_down, w.sf_gate, w.sf_up, w.sf_down, o, ws, nbytes)

    def check(got, ref):
        if combine == "gather":
            assert torch.equal(got.view(torch.int16) if out_fmt == "bf16" else got.view(torch.int32),
                               ref.view(torch.int16) if out_fmt == "bf16" else ref.view(torch.int32))
        else:
            scale = ref.float().abs().max().clamp_min(1e-30)
            assert float((got.float() - ref.float()).abs().max() / scale) <= 2.0 ** -7

    if fused is not None:
        os.environ["MOE_LAYER_FUSED"] = fused
    try:
        refs = []
        for i in range(3):
            load(i)
            call(out_e)
            torch.cuda.synchronize()
            refs.append(out_e.clone())
        # the three input sets give different outputs, so a replay that recomputed nothing fails
        assert not torch.equal(refs[0], refs[1]) and not torch.equal(refs[1], refs[2])

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            load(0)
            call(out)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call(out)
        torch.cuda.synchronize()

        for rnd, i in enumerate([0, 1, 2, 0, 2, 1]):
            load(i)
            out.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            print(f"  replay {rnd}: input set {i}", flush=True)
            check(out, refs[i])
            # the program's own eager call between replays, on the same workspace
            j = (i + 1) % 3
            load(j)
            call(out_e)
            torch.cuda.synchronize()
            check(out_e, refs[j])
    finally:
        if fused is not None:
            del os.environ["MOE_LAYER_FUSED"]
