"""The layer backward through the C ABI and its comparison with the oracle's backward (GPU
tests only)."""
import numpy as np
import torch

from oracle import moe_oracle as O
from workloads import to_numpy_bits as host

import mixture_experts_layer_counting_amd as moe
from _oracle_run import rel_err, weight_fn

DEV = "cuda:0"


def run_backward(w, dout):
    from _gpu_run import layer_desc
    d = layer_desc(w)
    n = moe.moe_layer_backward_workspace_bytes(d)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    r = dict(dx=torch.empty((w.T, w.H), dtype=torch.bfloat16, device=DEV),
             dWg=torch.full((w.E, w.H, w.Hp), float("nan"), **f32),
             dWu=torch.full((w.E, w.H, w.Hp), float("nan"), **f32),
             dWd=torch.full((w.E, w.Hp, w.H), float("nan"), **f32),
             dw=torch.empty((w.T, w.K), **f32),
             dl=torch.empty((w.T, w.E), **f32) if w.logits is not None else None)
    moe.moe_layer_backward(d, w.x, w.logits, w.topk_idx, w.topk_w, w.w_gate, w.w_up, w.w_down, dout,
                           r["dx"], r["dWg"], r["dWu"], r["dWd"], r["dw"], r["dl"], ws, n)
    return r


def check_backward(w, dout, tol=2e-2):
    r = run_backward(w, dout)
    torch.cuda.synchronize()
    b = {"logits": host(w.logits), "topk_idx": host(w.topk_idx), "topk_w": host(w.topk_w)}
    ref = O.layer_backward(O.decode_bf16(host(w.x)), w.E, w.K, weight_fn(w), O.decode_bf16(host(dout)),
                           logits=b["logits"], topk_idx=b["topk_idx"], topk_w=b["topk_w"])
    errs = {"dx": rel_err(O.decode_bf16(host(r["dx"])), ref["dx"]),
            "dWg": rel_err(host(r["dWg"]), ref["dWg"]), "dWu": rel_err(host(r["dWu"]), ref["dWu"]),
            "dWd": rel_err(host(r["dWd"]), ref["dWd"]), "dw": rel_err(host(r["dw"]), ref["dw"])}
    if r["dl"] is not None:
        errs["dlogits"] = rel_err(host(r["dl"]), ref["dlogits"])
    print("  " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= tol, (k, v)
    # experts without rows get exactly zero weight gradients
    counts = np.diff(ref["cu_seqlens"])
    for e in np.nonzero(counts == 0)[0]:
        assert not host(r["dWg"])[e].any() and not host(r["dWd"])[e].any()
    return r, ref
