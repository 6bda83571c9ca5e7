"""moe_permute_noalloc (the sort's scratch in the library's static device array) against
moe_permute with a caller workspace: bit for bit on every output, on two calls in a row,
the second with a smaller input, and the size limit rejected on the host."""
import os
import sys

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from workloads import gen, to_numpy_bits

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from _oracle_run import oracle_routing  # noqa: E402

import mixture_experts_layer_counting_amd as moe  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DT = {"bf16": moe.MOE_BF16, "fp8": moe.MOE_FP8_E4M3}


def _outputs(w, with_x_perm):
    T, H, E, K = w.T, w.H, w.E, w.K
    i32 = dict(dtype=torch.int32, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    o = dict(counts=torch.full((E,), -7, **i32), cu=torch.full((E + 1,), -7, **i32),
             pos=torch.full((T, K), -7, **i32), row_src=torch.full((T * K,), -7, **i32),
             row_w=torch.full((T * K,), -7.0, **f32))
    o["x_perm"] = torch.zeros((T * K, H), dtype=w.x.dtype, device=DEV) if with_x_perm else None
    o["x_perm_sf"] = torch.zeros((H // 128, T * K), **f32) if w.act == "fp8" else None
    return o


def _route(w):
    idx = torch.empty((w.T, w.K), dtype=torch.int32, device=DEV)
    wt = torch.empty((w.T, w.K), dtype=torch.float32, device=DEV)
    moe.moe_route_topk(w.logits, w.T, w.E, w.K, idx, wt)
    return idx, wt


def _compare(w, with_x_perm):
    idx, wt = _route(w)
    a, b = _outputs(w, with_x_perm), _outputs(w, with_x_perm)
    nws = moe.moe_permute_workspace_bytes(w.T, w.E, w.K)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    moe.moe_permute(w.x, w.x_sf, DT[w.act], idx, wt, w.T, w.H, w.E, w.K, a["counts"], a["cu"], a["pos"],
                    a["row_src"], a["row_w"], a["x_perm"], a["x_perm_sf"], ws, nws)
    moe.moe_permute_noalloc(w.x, w.x_sf, DT[w.act], idx, wt, w.T, w.H, w.E, w.K, b["counts"], b["cu"],
                            b["pos"], b["row_src"], b["row_w"], b["x_perm"], b["x_perm_sf"])
    torch.cuda.synchronize()
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), f"{w.name}: {k} differs"
    # and the integers are the oracle's
    ref = oracle_routing(w)
    assert np.array_equal(to_numpy_bits(b["counts"]), ref["counts"])
    assert np.array_equal(to_numpy_bits(b["cu"]), ref["cu_seqlens"])
    assert np.array_equal(to_numpy_bits(b["pos"]), ref["pos"])
    assert np.array_equal(to_numpy_bits(b["row_src"]), ref["row_src"])


@pytest.mark.parametrize("act", ["bf16", "fp8"])
def test_noalloc_permute_matches_workspace_permute_twice(act):
    print(f"\n[case] moe_permute_noalloc vs moe_permute, {act}: large then smaller call", flush=True)
    wgt = "mxfp4" if act == "fp8" else "bf16"
    big = gen.make(T=4000, H=1024, Hp=128, E=384, K=8, routing="skew", beta=0.5, act=act, wgt=wgt,
                   cid=70, device=DEV)
    small = gen.make(T=301, H=256, Hp=128, E=12, K=3, routing="normal", act=act, wgt=wgt, cid=71,
                     device=DEV)
    _compare(big, with_x_perm=True)
    _compare(small, with_x_perm=True)
    _compare(small, with_x_perm=False)     # metadata only (and, for fp8, the permuted scales)


def test_noalloc_permute_rejects_sizes_beyond_its_scratch():
    print("\n[case] moe_permute_noalloc size limit: T=16369, E=1024 rejected; T=16368 runs", flush=True)
    E, K, H = 1024, 1, 128
    for T, ok in ((16369, False), (16368, True)):
        idx = (torch.arange(T, dtype=torch.int32, device=DEV) % E).reshape(T, K)
        x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
        counts = torch.empty(E, dtype=torch.int32, device=DEV)
        cu = torch.empty(E + 1, dtype=torch.int32, device=DEV)
        pos = torch.empty((T, K), dtype=torch.int32, device=DEV)
        row_src = torch.empty(T * K, dtype=torch.int32, device=DEV)
        if ok:
            moe.moe_permute_noalloc(x, None, moe.MOE_BF16, idx, None, T, H, E, K, counts, cu, pos, row_src,
                                    None, None, None)
            torch.cuda.synchronize()
            assert torch.equal(counts.cpu(), torch.bincount(idx.cpu().long().ravel(), minlength=E).int())
        else:
            with pytest.raises(moe.MoeError) as ei:
                moe.moe_permute_noalloc(x, None, moe.MOE_BF16, idx, None, T, H, E, K, counts, cu, pos,
                                        row_src, None, None, None)
            assert ei.value.status == moe.MOE_EUNSUPPORTED
