"""The bf16 expert FFN as one persistent launch (moe_grouped_ffn_fused, and moe_layer_forward
with MOE_LAYER_FUSED=1) against the oracle and against the two-launch path, which it must
match bit for bit: it runs the same tiles with the same MFMA order, only scheduled from
device-side queues with down tiles waiting for the h rows they read."""
import os
import sys

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from workloads import gen, to_numpy_bits

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from _gpu_run import fused_tile_count, run_fused, run_layer, run_steps  # noqa: E402
from _oracle_run import oracle_layer, rel_err  # noqa: E402

import mixture_experts_layer_counting_amd as moe  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_BF16 = 2e-2


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def host(t):
    return to_numpy_bits(t)


def check_ctl(ctl, counts, H, Hp):
    c = host(ctl).astype(np.int64)
    want = fused_tile_count(counts, H, Hp)
    print(f"  tiles {c[9]} (want {want}), not prefetched {c[10]}, from other queues {c[11]}, "
          f"error {c[8]}", flush=True)
    assert c[8] == 0, "a readiness wait exceeded its bound"
    assert c[9] == want


def check_against_steps(w, r, y, h):
    rows = int(host(r["cu_seqlens"])[-1])
    assert torch.equal(y[:rows].view(torch.int16), r["y_rows"][:rows].view(torch.int16))
    assert torch.equal(h[:rows].view(torch.int16), r["h"][:rows].view(torch.int16))


EDGE_COUNTS = [0, 1, 31, 32, 33, 255, 256, 257, 300, 511, 512, 513, 769, 2]

CASES = [
    dict(T=600, H=512, Hp=256, E=32, K=6, routing="skew", beta=3.0),     # many empty experts
    dict(T=1000, H=256, Hp=384, E=40, K=4, routing="skew", beta=0.8),
    dict(T=1000, H=256, Hp=256, E=1, K=1, routing="normal"),             # one queue holds all
    dict(T=2048, H=256, Hp=256, E=1024, K=8, routing="skew", beta=0.6),  # 1024 experts
    dict(T=4096, H=768, Hp=768, E=16, K=6, routing="normal"),            # several m-tiles each
]


@pytest.fixture(params=["phases", "lag1"])
def queue_order(request):
    """Queue order of the single launch: the default (each queue's gate/up tiles, then its
    down tiles) and down tiles interleaved one expert behind their gate/up tiles, where many
    of them wait for their rows."""
    if request.param == "lag1":
        os.environ["MOE_FUSED_LAG"] = "1"
    yield request.param
    os.environ.pop("MOE_FUSED_LAG", None)


@pytest.mark.parametrize("spec", CASES, ids=lambda s: "T{T}_H{H}_Hp{Hp}_E{E}_K{K}_{routing}".format(**s))
def test_fused_matches_oracle_and_two_launches(spec, queue_order):
    say(f"single-launch FFN {spec}, queue order {queue_order}")
    w = gen.make(**spec, act="bf16", wgt="bf16", out="bf16", cid=90, device=DEV)
    r = run_steps(w)
    y, h, ctl, _ = run_fused(w, r["row_src"], r["cu_seqlens"])
    torch.cuda.synchronize()
    check_ctl(ctl, host(r["counts"]), w.H, w.Hp)
    check_against_steps(w, r, y, h)
    ref = oracle_layer(w)
    rows = int(ref["cu_seqlens"][-1])
    e_y = rel_err(O.decode_bf16(host(y)[:rows]), ref["y_rows"][:rows])
    print(f"  y_rows rel err {e_y:.3e}", flush=True)
    assert e_y <= TOL_BF16


def test_fused_expert_sizes_around_tile_boundaries():
    K = 2
    T, E = sum(EDGE_COUNTS) // K, len(EDGE_COUNTS)
    say(f"single-launch FFN, expert sizes {EDGE_COUNTS}")
    w = gen.make(T=T, H=512, Hp=256, E=E, K=K, act="bf16", wgt="bf16", out="bf16", routing="balanced",
                 cid=91, device=DEV)
    ids = np.repeat(np.arange(E), EDGE_COUNTS).reshape(K, T).T.copy().astype(np.int32)
    wts = np.random.default_rng(91).dirichlet(np.ones(K), size=T).astype(np.float32)
    w.topk_idx = torch.from_numpy(ids).to(DEV)
    w.topk_w = torch.from_numpy(wts).to(DEV)
    r = run_steps(w)
    y, h, ctl, _ = run_fused(w, r["row_src"], r["cu_seqlens"])
    torch.cuda.synchronize()
    assert np.array_equal(host(r["counts"]), np.asarray(EDGE_COUNTS))
    check_ctl(ctl, EDGE_COUNTS, w.H, w.Hp)
    check_against_steps(w, r, y, h)
    ref = oracle_layer(w)
    rows = int(ref["cu_seqlens"][-1])
    assert rel_err(O.decode_bf16(host(y)[:rows]), ref["y_rows"][:rows]) <= TOL_BF16


def test_fused_back_to_back_calls_share_a_workspace(queue_order):
    """Two routings of one shape through one workspace without a host synchronisation between
    them (the control words are reset by the launch itself), the second with the workspace
    poisoned first: an h row read before it was written would show up as NaN."""
    spec = dict(T=3000, H=512, Hp=512, E=24, K=4)
    say(f"single-launch FFN, two calls on one workspace {spec}")
    wa = gen.make(**spec, routing="skew", beta=1.5, act="bf16", wgt="bf16", out="bf16", cid=92, device=DEV)
    wb = gen.make(**spec, routing="normal", act="bf16", wgt="bf16", out="bf16", cid=92, device=DEV)
    wb.x, wb.w_gate, wb.w_up, wb.w_down = wa.x, wa.w_gate, wa.w_up, wa.w_down
    ra, rb = run_steps(wa), run_steps(wb)
    torch.cuda.synchronize()
    assert not np.array_equal(host(ra["counts"]), host(rb["counts"]))
    ya, ha, ctla, ws = run_fused(wa, ra["row_src"], ra["cu_seqlens"])
    ya, ha, ctla = ya.clone(), ha.clone(), ctla.clone()
    os.environ["MOE_DEBUG_POISON"] = "1"
    try:
        yb, hb, ctlb, _ = run_fused(wb, rb["row_src"], rb["cu_seqlens"], ws=ws)
    finally:
        del os.environ["MOE_DEBUG_POISON"]
    torch.cuda.synchronize()
    check_ctl(ctla, host(ra["counts"]), wa.H, wa.Hp)
    check_ctl(ctlb, host(rb["counts"]), wb.H, wb.Hp)
    check_against_steps(wa, ra, ya, ha)
    check_against_steps(wb, rb, yb, hb)


def test_wait_bound_ends_the_launch_and_sets_the_error_word():
    """The readiness waits are bounded. With the bound lowered to zero polls
    (MOE_FUSED_SPIN_MAX=0) and each expert's down tiles queued one expert behind its gate/up
    tiles (MOE_FUSED_LAG=1), down tiles taken before their rows are ready give up waiting at
    once. The launch still ends, runs every tile once and reports error 1 (its results are then
    invalid). The next call on the same workspace, with the default bound, is correct again:
    each launch resets its control words."""
    spec = CASES[0]
    say(f"single-launch FFN, readiness waits bounded at 0 polls {spec}")
    w = gen.make(**spec, act="bf16", wgt="bf16", out="bf16", cid=99, device=DEV)
    r = run_steps(w)
    os.environ["MOE_FUSED_LAG"] = "1"
    os.environ["MOE_FUSED_SPIN_MAX"] = "0"
    try:
        _, _, ctl, ws = run_fused(w, r["row_src"], r["cu_seqlens"])
        torch.cuda.synchronize()
        c = host(ctl).astype(np.int64)
    finally:
        del os.environ["MOE_FUSED_LAG"]
        del os.environ["MOE_FUSED_SPIN_MAX"]
    want = fused_tile_count(host(r["counts"]), w.H, w.Hp)
    print(f"  error {c[8]}, tiles {c[9]} (want {want}), not prefetched {c[10]}", flush=True)
    assert c[8] == 1
    assert c[9] == want
    y, h, ctl2, _ = run_fused(w, r["row_src"], r["cu_seqlens"], ws=ws)
    torch.cuda.synchronize()
    check_ctl(ctl2, host(r["counts"]), w.H, w.Hp)
    check_against_steps(w, r, y, h)


def run_layer_env(w, value, combine=moe.MOE_COMBINE_GATHER):
    os.environ["MOE_LAYER_FUSED"] = value
    try:
        return run_layer(w, combine)
    finally:
        del os.environ["MOE_LAYER_FUSED"]


def run_fused_scatter(w, r, ws=None):
    """moe_grouped_ffn_fused_scatter on the permutation of run_steps into a zeroed fp32
    accumulator: returns (acc [T, H], control words, workspace)."""
    M = w.T * w.K
    n = moe.moe_grouped_ffn_fused_workspace_bytes(M, w.E, w.Hp)
    if ws is None:
        ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    acc = torch.zeros((w.T, w.H), dtype=torch.float32, device=DEV)
    moe.moe_grouped_ffn_fused_scatter(w.x, moe.MOE_BF16, r["row_src"], w.T, w.K, r["cu_seqlens"], M, w.E,
                                      w.H, w.Hp, w.w_gate, w.w_up, w.w_down, moe.MOE_BF16, r["row_w"], acc,
                                      ws, n)
    o = (M * w.Hp * 2 + 255) // 256 * 256
    return acc, ws[o:o + 64].view(torch.int32), ws


def rel_to_max(got, ref):
    return float((got.float() - ref.float()).abs().max() / ref.float().abs().max().clamp_min(1e-30))


@pytest.mark.parametrize("spec", [CASES[0], CASES[1], CASES[4]],
                         ids=lambda s: "T{T}_H{H}_Hp{Hp}_E{E}_K{K}_{routing}".format(**s))
def test_fused_scatter_matches_oracle_and_two_launch_scatter(spec, queue_order):
    """The single launch with the weighted combine in its down epilogue: the same fp32
    products as moe_ffn_down_scatter after the two-launch gate/up, added with atomics in
    another order, and the oracle's layer output."""
    say(f"single-launch FFN with the scatter-add combine {spec}, queue order {queue_order}")
    w = gen.make(**spec, act="bf16", wgt="bf16", out="bf16", cid=97, device=DEV)
    r = run_steps(w)
    M = w.T * w.K
    acc_f, ctl, _ = run_fused_scatter(w, r)
    acc_2 = torch.zeros_like(acc_f)
    moe.moe_ffn_down_scatter(r["h"], None, moe.MOE_BF16, r["cu_seqlens"], M, w.E, w.H, w.Hp, w.w_down, None,
                             moe.MOE_BF16, r["row_src"], r["row_w"], w.T, w.K, acc_2)
    torch.cuda.synchronize()
    check_ctl(ctl, host(r["counts"]), w.H, w.Hp)
    d = rel_to_max(acc_f, acc_2)
    ref = oracle_layer(w)
    e = rel_err(host(acc_f), ref["out"])
    print(f"  against the two-launch scatter {d:.3e}, against the oracle {e:.3e}", flush=True)
    assert d <= 1e-5
    assert e <= TOL_BF16


@pytest.mark.parametrize("spec", [CASES[0], CASES[4]], ids=["E32_one_tile_per_expert", "E16_several_tiles"])
def test_layer_scatter_combine_in_the_single_launch(spec):
    """moe_layer_forward with MOE_COMBINE_SCATTER_ATOMIC as one launch (MOE_LAYER_FUSED=1) and as
    two (=0): within one bf16 rounding of each other, and the oracle's output."""
    say(f"moe_layer_forward, scatter-add combine, one launch vs two {spec}")
    w = gen.make(**spec, act="bf16", wgt="bf16", out="bf16", cid=98, device=DEV)
    out_1, ws_1, lay = run_layer_env(w, "1", moe.MOE_COMBINE_SCATTER_ATOMIC)
    out_2, _, _ = run_layer_env(w, "0", moe.MOE_COMBINE_SCATTER_ATOMIC)
    torch.cuda.synchronize()
    c = host(ws_1[lay["fused_ctl"]:lay["fused_ctl"] + 64].view(torch.int32))
    cu = host(ws_1[lay["cu_seqlens"]:lay["cu_seqlens"] + 4 * (w.E + 1)].view(torch.int32))
    assert c[8] == 0 and c[9] == fused_tile_count(np.diff(cu), w.H, w.Hp)
    d = rel_to_max(out_1, out_2)
    ref = oracle_layer(w)
    e = rel_err(O.decode_bf16(host(out_1)), ref["out"])
    print(f"  one launch vs two {d:.3e}, against the oracle {e:.3e}", flush=True)
    assert d <= 2.0 ** -7
    assert e <= TOL_BF16


@pytest.mark.parametrize("spec", [CASES[0], CASES[4]], ids=["E32_one_tile_per_expert", "E16_several_tiles"])
def test_layer_single_launch_is_bitwise_two_launches(spec):
    """moe_layer_forward with the FFN as one launch (MOE_LAYER_FUSED=1) and as two (=0), and
    the default, which picks one launch when T*K <= 256*E."""
    say(f"moe_layer_forward, one launch vs two {spec}")
    w = gen.make(**spec, act="bf16", wgt="bf16", out="bf16", cid=93, device=DEV)
    out_2, _, lay_2 = run_layer_env(w, "0")
    out_1, ws_1, lay_1 = run_layer_env(w, "1")
    out_d, ws_d, _ = run_layer(w)
    torch.cuda.synchronize()
    assert lay_1["fused_ctl"] is not None
    c = host(ws_1[lay_1["fused_ctl"]:lay_1["fused_ctl"] + 64].view(torch.int32))
    assert c[8] == 0 and c[9] > 0
    assert torch.equal(out_1.view(torch.int16), out_2.view(torch.int16))
    assert torch.equal(out_d.view(torch.int16), out_2.view(torch.int16))
    # the default took the single launch exactly when the groups average one tile
    cd = host(ws_d[lay_1["fused_ctl"]:lay_1["fused_ctl"] + 64].view(torch.int32))
    assert (cd[9] > 0) == (w.T * w.K <= 256 * w.E)


def test_fused_rejects_what_it_does_not_take():
    say("moe_grouped_ffn_fused argument checks")
    w = gen.make(T=64, H=512, Hp=256, E=4, K=2, routing="normal", act="bf16", wgt="bf16", out="bf16",
                 cid=94, device=DEV)
    r = run_steps(w)
    M = w.T * w.K
    n = moe.moe_grouped_ffn_fused_workspace_bytes(M, w.E, w.Hp)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    y = torch.empty((M, w.H), dtype=torch.bfloat16, device=DEV)
    args = lambda **kw: dict(dict(x=w.x, act=moe.MOE_BF16, row_src=r["row_src"], T=w.T, K=w.K,  # noqa: E731
                                  cu_seqlens=r["cu_seqlens"], M=M, E=w.E, H=w.H, Hp=w.Hp, w_gate=w.w_gate,
                                  w_up=w.w_up, w_down=w.w_down, wgt=moe.MOE_BF16, y_rows=y,
                                  out=moe.MOE_BF16, ws=ws, ws_bytes=n), **kw)
    for kw, status in ((dict(act=moe.MOE_F32), moe.MOE_EUNSUPPORTED), (dict(H=384), moe.MOE_EUNSUPPORTED),
                       (dict(Hp=128), moe.MOE_EUNSUPPORTED), (dict(ws_bytes=n - 1), moe.MOE_EWORKSPACE),
                       (dict(y_rows=None), moe.MOE_EINVAL)):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_grouped_ffn_fused(**args(**kw))
        assert ei.value.status == status
    acc = torch.zeros((w.T, w.H), dtype=torch.float32, device=DEV)
    sargs = lambda **kw: dict(dict(x=w.x, act=moe.MOE_BF16, row_src=r["row_src"], T=w.T, K=w.K,  # noqa: E731
                                   cu_seqlens=r["cu_seqlens"], M=M, E=w.E, H=w.H, Hp=w.Hp, w_gate=w.w_gate,
                                   w_up=w.w_up, w_down=w.w_down, wgt=moe.MOE_BF16, row_w=r["row_w"], acc=acc,
                                   ws=ws, ws_bytes=n), **kw)
    for kw, status in ((dict(act=moe.MOE_F32), moe.MOE_EUNSUPPORTED), (dict(H=384), moe.MOE_EUNSUPPORTED),
                       (dict(ws_bytes=n - 1), moe.MOE_EWORKSPACE), (dict(row_w=None), moe.MOE_EINVAL),
                       (dict(acc=None), moe.MOE_EINVAL)):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_grouped_ffn_fused_scatter(**sargs(**kw))
        assert ei.value.status == status


@pytest.mark.parametrize("spec", [dict(T=600, H=512, Hp=256, E=32, K=6, routing="skew", beta=3.0),
                                  dict(T=1100, H=768, Hp=384, E=16, K=3, routing="normal")],
                         ids=["T600_E32", "T1100_E16"])
def test_shared_expert_folded_into_the_single_launch(spec, queue_order):
    """moe_layer_forward_shared with the shared expert's tiles in the routed launch's queues
    (MOE_SHARED_FOLD=1; bf16, T*K <= 256*E, Hs = Hp): the oracle's result, and bitwise the
    result with the shared expert as its own two launches (the default), also given a side
    stream."""
    from _gpu_run import layer_desc, run_layer_shared
    from _oracle_run import oracle_layer_shared
    say(f"shared expert folded into the single launch {spec}, queue order {queue_order}")
    w = gen.make(**spec, act="bf16", wgt="bf16", out="bf16", cid=95, device=DEV, shared_hs=spec["Hp"])
    assert w.T * w.K <= 256 * w.E
    os.environ["MOE_SHARED_FOLD"] = "1"
    try:
        out_f, ws_f = run_layer_shared(w)
        out_fs, _ = run_layer_shared(w, side_stream=torch.cuda.Stream())
    finally:
        del os.environ["MOE_SHARED_FOLD"]
    out_s, _ = run_layer_shared(w)
    torch.cuda.synchronize()
    lay = moe.moe_layer_workspace_layout(layer_desc(w))
    c = host(ws_f[lay["fused_ctl"]:lay["fused_ctl"] + 64].view(torch.int32)).astype(np.int64)
    r = run_steps(w)
    torch.cuda.synchronize()
    routed = fused_tile_count(host(r["counts"]), w.H, w.Hp)
    shared = fused_tile_count([w.T], w.H, w.Hp)
    print(f"  tiles {c[9]} (routed {routed} + shared {shared}), not prefetched {c[10]}, error {c[8]}",
          flush=True)
    assert c[8] == 0 and c[9] == routed + shared
    assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16))
    assert torch.equal(out_fs.view(torch.int16), out_s.view(torch.int16))
    ref = oracle_layer_shared(w)
    e = rel_err(O.decode_bf16(host(out_f)), ref["out"])
    es = rel_err(O.decode_bf16(host(out_f)), ref["out"] - ref["y_shared"])
    print(f"  out rel err {e:.3e}; without the shared term {es:.3e}", flush=True)
    assert e <= TOL_BF16 and es > 10 * TOL_BF16


def test_layer_single_launch_empty_batch_and_dropped_copies():
    """The layer on a shape that takes the single launch: T = 0 gives an empty output; copies
    with invalid expert ids are dropped (cu_seqlens[E] < T*K), and the result is bitwise the
    two-launch layer's."""
    say("single launch: T=0, and invalid ids (dropped copies)")
    w0 = gen.make(T=0, H=512, Hp=256, E=16, K=2, routing="normal", act="bf16", wgt="bf16", out="bf16",
                  cid=96, device=DEV)
    out0, _, _ = run_layer(w0)
    torch.cuda.synchronize()
    assert out0.shape == (0, 512)
    w = gen.make(T=512, H=512, Hp=256, E=16, K=2, routing="balanced", act="bf16", wgt="bf16", out="bf16",
                 cid=96, device=DEV)
    bad = w.topk_idx.clone()
    bad[5, 1] = 17
    bad[9, 0] = -3
    bad[300, 1] = 99
    w.topk_idx = bad
    out_1, ws_1, lay = run_layer_env(w, "1")
    out_2, _, _ = run_layer_env(w, "0")
    torch.cuda.synchronize()
    c = host(ws_1[lay["fused_ctl"]:lay["fused_ctl"] + 64].view(torch.int32))
    cu = host(ws_1[lay["cu_seqlens"]:lay["cu_seqlens"] + 4 * (w.E + 1)].view(torch.int32))
    assert int(cu[-1]) == w.T * w.K - 3
    assert c[8] == 0 and c[9] == fused_tile_count(np.diff(cu), w.H, w.Hp)
    assert torch.equal(out_1.view(torch.int16), out_2.view(torch.int16))
