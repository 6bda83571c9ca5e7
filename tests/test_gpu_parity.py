"""Parity of the HIP path (called through the C ABI) with the CPU oracle on the same seeded
inputs. Integers (routing, counts, cu_seqlens, pos, row_src) and copied rows must be
bit-exact; floating point within the stated tolerance: max|err| / max|ref| <= 1e-5 for the
fp32 layer, <= 2e-2 for bf16; route weights within 1e-6 absolute."""
import os
import sys

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from workloads import gen, to_numpy_bits

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from _gpu_run import layer_desc, run_layer, run_steps  # noqa: E402
from _backward_check import check_backward, run_backward  # noqa: E402,F401
from _oracle_run import oracle_layer, oracle_routing, oracle_rows, rel_err  # noqa: E402

import mixture_experts_layer_counting_amd as moe  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}
DEV = "cuda:0"


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def host(t):
    return to_numpy_bits(t)


def check_integers(r, ref, K):
    assert np.array_equal(host(r["topk_idx"]), ref["topk_idx"])
    assert np.abs(host(r["topk_w"]).astype(np.float64) - ref["topk_w"]).max() <= 1e-6
    assert np.array_equal(host(r["counts"]), ref["counts"])
    assert np.array_equal(host(r["cu_seqlens"]), ref["cu_seqlens"])
    assert np.array_equal(host(r["pos"]), ref["pos"])
    assert np.array_equal(host(r["row_src"]), ref["row_src"])
    if r.get("row_w") is not None:
        tw = host(r["topk_w"]).ravel()
        assert np.array_equal(host(r["row_w"]), tw[ref["row_src"]])


def check_x_perm(w, r, ref):
    xb = host(w.x)
    assert np.array_equal(host(r["x_perm"]), xb[ref["row_src"] // w.K])
    if w.x_sf is not None:
        assert np.array_equal(host(r["x_perm_sf"]), host(w.x_sf)[ref["row_src"] // w.K].T)


def full_check(w, tol=None):
    tol = tol or TOL[w.act]
    r = run_steps(w)
    torch.cuda.synchronize()
    ref = oracle_layer(w)
    check_integers(r, ref, w.K)
    check_x_perm(w, r, ref)
    e_y = rel_err(host(r["y_rows"]).astype(np.float64) if w.act == "f32" else O.decode_bf16(host(r["y_rows"])),
                  ref["y_rows"])
    out = host(r["out"])
    out = out.astype(np.float64) if w.out == "f32" else O.decode_bf16(out)
    e_out = rel_err(out, ref["out"])
    print(f"  y_rows rel err {e_y:.3e}  out rel err {e_out:.3e}  maxvio {ref['maxvio']:.3f}", flush=True)
    assert e_y <= tol and e_out <= tol
    return r, ref


# ----------------------------------------------------------------------------- whole layer, small

def test_c1_fp32_full():
    say("c1 fp32 T=64 H=128 Hp=64 E=8 K=2")
    full_check(gen.config("c1", device=DEV))


SMALL = [
    dict(T=300, H=512, Hp=256, E=12, K=3, routing="normal"),
    dict(T=1000, H=256, Hp=384, E=40, K=4, routing="skew", beta=0.8),
    dict(T=700, H=768, Hp=128, E=10, K=4, routing="balanced"),
    dict(T=257, H=256, Hp=128, E=1, K=1, routing="normal"),
    dict(T=64, H=256, Hp=128, E=4, K=4, routing="normal"),
    dict(T=600, H=512, Hp=256, E=32, K=6, routing="skew", beta=3.0),   # many empty experts
]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: "T{T}_H{H}_Hp{Hp}_E{E}_K{K}_{routing}".format(**s))
def test_small_bf16_layer(spec):
    say(f"bf16 small {spec}")
    w = gen.make(**spec, act="bf16", wgt="bf16", out="bf16", cid=50, device=DEV)
    full_check(w)


def test_small_fp32_layer_ragged():
    spec = dict(T=333, H=200, Hp=72, E=9, K=3, routing="skew", beta=0.5)
    say(f"fp32 ragged {spec}")
    full_check(gen.make(**spec, act="f32", wgt="f32", out="f32", cid=51, device=DEV))


def test_c2_bf16_full():
    say("c2 bf16 T=4096 H=2048 Hp=1024 E=64 K=6 (full oracle)")
    full_check(gen.config("c2", device=DEV))


# ----------------------------------------------------------------------------- single steps, limits

@pytest.mark.parametrize("T,E,K", [(97, 4096, 32), (130, 1, 1), (1024, 384, 8), (65, 64, 64 // 2)])
def test_route_topk_limits_with_ties(T, E, K):
    say(f"route T={T} E={E} K={K}")
    rng = np.random.default_rng(E + K)
    lg = (np.round(rng.standard_normal((T, E)) * 3) / 3).astype(np.float32)   # many ties
    logits = torch.from_numpy(lg).to(DEV)
    idx = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    moe.moe_route_topk(logits, T, E, K, idx, w)
    ri, rw = O.route_topk(lg, K)
    assert np.array_equal(host(idx), ri)
    assert np.abs(host(w).astype(np.float64) - rw).max() <= 1e-6


@pytest.mark.parametrize("act", ["f32", "bf16", "fp8"])
def test_permute_max_experts(act):
    T, E, K, H = 3000, 1024, 8, 256
    say(f"permute E={E} K={K} T={T} act={act}")
    rng = np.random.default_rng(5)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    w = gen.make(T=T, H=H, Hp=128, E=8, K=1, act=act, wgt="bf16", routing="normal", cid=52, device=DEV)
    x, x_sf = w.x, w.x_sf
    M = T * K
    ti = torch.from_numpy(idx).to(DEV)
    tw = torch.rand((T, K), device=DEV)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    cu = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    pos = torch.empty((T, K), dtype=torch.int32, device=DEV)
    row_src = torch.empty(M, dtype=torch.int32, device=DEV)
    row_w = torch.empty(M, dtype=torch.float32, device=DEV)
    xp = torch.empty((M, H), dtype=x.dtype, device=DEV)
    xsf = torch.empty((H // 128, M), dtype=torch.float32, device=DEV) if act == "fp8" else None
    n = moe.moe_permute_workspace_bytes(T, E, K)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    dt = {"f32": moe.MOE_F32, "bf16": moe.MOE_BF16, "fp8": moe.MOE_FP8_E4M3}[act]
    moe.moe_permute(x, x_sf, dt, ti, tw, T, H, E, K, counts, cu, pos, row_src, row_w, xp, xsf, ws, n)
    c_ref, cu_ref = O.count_offsets(idx, E)
    p_ref, rs_ref = O.permute(idx, E)
    assert np.array_equal(host(counts), c_ref) and np.array_equal(host(cu), cu_ref)
    assert np.array_equal(host(pos), p_ref) and np.array_equal(host(row_src), rs_ref)
    assert np.array_equal(host(row_w), host(tw).ravel()[rs_ref])
    assert np.array_equal(host(xp), host(x)[rs_ref // K])
    if act == "fp8":
        assert np.array_equal(host(xsf), host(x_sf)[rs_ref // K].T)


ROUTE_PERMUTE = [
    # (T, H, E, K, act, pad, with x_perm)
    (300, 256, 12, 3, "fp8", 1, True),
    (1000, 256, 40, 4, "bf16", 1, False),
    (257, 128, 1024, 8, "bf16", 4, True),     # 16 logits per lane, two batches per wave
    (4096, 256, 64, 6, "bf16", 1, False),     # the c2 routing shape
    (130, 128, 384, 8, "f32", 16, True),
    (1, 128, 2, 2, "bf16", 1, True),
    (0, 128, 8, 2, "bf16", 1, True),
]


@pytest.mark.parametrize("T,H,E,K,act,pad,xp", ROUTE_PERMUTE,
                         ids=lambda v: str(v))
def test_route_permute_is_route_then_permute(T, H, E, K, act, pad, xp):
    """moe_route_permute gives bit for bit what moe_route_topk followed by moe_permute_padded
    gives (both are pinned to the oracle elsewhere)."""
    say(f"route_permute T={T} H={H} E={E} K={K} act={act} pad={pad} x_perm={xp}")
    w = gen.make(T=T, H=H, Hp=128, E=E, K=K, act=act, wgt="bf16", routing="skew", beta=1.0, cid=73,
                 device=DEV)
    i32 = dict(dtype=torch.int32, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    cap = moe.moe_padded_capacity(T, E, K, pad)
    dt = {"f32": moe.MOE_F32, "bf16": moe.MOE_BF16, "fp8": moe.MOE_FP8_E4M3}[act]
    nws = moe.moe_permute_workspace_bytes(T, E, K)
    res = []
    for fused in (False, True):
        o = dict(topk_idx=torch.full((T, K), -7, **i32), topk_w=torch.full((T, K), -7.0, **f32),
                 counts=torch.full((E,), -7, **i32), cu=torch.full((E + 1,), -7, **i32),
                 pos=torch.full((T, K), -7, **i32), row_src=torch.full((cap,), -7, **i32),
                 row_w=torch.full((cap,), -7.0, **f32),
                 x_perm=torch.full((cap, H), 7, dtype=w.x.dtype, device=DEV) if xp else None,
                 x_perm_sf=torch.full((H // 128, cap), -7.0, **f32) if xp and act == "fp8" else None)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=DEV)
        if fused:
            moe.moe_route_permute(w.logits, w.x, w.x_sf, dt, T, H, E, K, pad, o["topk_idx"], o["topk_w"],
                                  o["counts"], o["cu"], o["pos"], o["row_src"], o["row_w"], o["x_perm"],
                                  o["x_perm_sf"], ws, nws)
        else:
            moe.moe_route_topk(w.logits, T, E, K, o["topk_idx"], o["topk_w"])
            moe.moe_permute_padded(w.x, w.x_sf, dt, o["topk_idx"], o["topk_w"], T, H, E, K, pad, o["counts"],
                                   o["cu"], o["pos"], o["row_src"], o["row_w"], o["x_perm"], o["x_perm_sf"],
                                   ws, nws)
        torch.cuda.synchronize()
        res.append(o)
    a, b = res
    for k in a:
        if a[k] is None:
            continue
        assert torch.equal(a[k].view(torch.int32) if a[k].dtype == torch.float32 else a[k],
                           b[k].view(torch.int32) if b[k].dtype == torch.float32 else b[k]), k
    if T > 0:
        ref = oracle_routing(w)
        assert np.array_equal(host(b["topk_idx"]), ref["topk_idx"])
        assert np.array_equal(host(b["counts"]), ref["counts"])
        if pad == 1:
            assert np.array_equal(host(b["pos"]), ref["pos"])
            assert np.array_equal(host(b["row_src"]), ref["row_src"])


@pytest.mark.parametrize("T,H,E,K,pad", [(300, 512, 12, 3, 1), (1000, 8960, 16, 4, 1), (257, 256, 1024, 8, 16),
                                         (65, 128, 8, 2, 64), (1, 128, 2, 2, 1)])
def test_permute_writes_scales_without_x_perm(T, H, E, K, pad):
    """fp8 metadata-only permutation with x_perm_sf given: the block-major scales of every row
    holding a copy are x_sf of its token (scale 1 for padding rows), bit for bit what the
    permutation with x_perm writes, and rows past cu_seqlens[E] are left untouched."""
    say(f"scales without x_perm T={T} H={H} E={E} K={K} pad={pad}")
    w = gen.make(T=T, H=H, Hp=128, E=E, K=K, act="fp8", wgt="bf16", routing="skew", beta=1.0, cid=74,
                 device=DEV)
    i32 = dict(dtype=torch.int32, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    idx = torch.empty((T, K), **i32)
    tw = torch.empty((T, K), **f32)
    moe.moe_route_topk(w.logits, T, E, K, idx, tw)
    if T > 2:
        idx[T // 2, 0] = -1                    # a dropped copy: one row past cu_seqlens[E]
    cap = moe.moe_padded_capacity(T, E, K, pad)
    nws = moe.moe_permute_workspace_bytes(T, E, K)
    res = []
    for xp in (True, False):
        o = dict(counts=torch.full((E,), -7, **i32), cu=torch.full((E + 1,), -7, **i32),
                 pos=torch.full((T, K), -7, **i32), row_src=torch.full((cap,), -7, **i32),
                 x_perm=torch.full((cap, H), 7, dtype=w.x.dtype, device=DEV) if xp else None,
                 x_perm_sf=torch.full((H // 128, cap), -7.0, **f32))
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=DEV)
        moe.moe_permute_padded(w.x, w.x_sf, moe.MOE_FP8_E4M3, idx, tw, T, H, E, K, pad, o["counts"],
                               o["cu"], o["pos"], o["row_src"], None, o["x_perm"], o["x_perm_sf"], ws, nws)
        torch.cuda.synchronize()
        res.append(o)
    a, b = res
    for k in ("counts", "cu", "pos", "row_src", "x_perm_sf"):
        assert torch.equal(a[k].view(torch.int32), b[k].view(torch.int32)), k
    rows = int(host(b["cu"])[-1])
    rs = host(b["row_src"])[:rows]
    xsf = host(w.x_sf)
    want = np.where(rs[None, :] >= 0, xsf[np.maximum(rs, 0) // K].T, np.float32(1.0))
    got = host(b["x_perm_sf"])
    assert np.array_equal(got[:, :rows].view(np.int32), want.astype(np.float32).view(np.int32))
    assert np.all(got[:, rows:] == -7.0)
    if pad == 1:
        dropped = {(T // 2) * K} if T > 2 else set()
        assert sorted(rs.tolist()) == sorted(set(range(T * K)) - dropped)


def test_empty_batch():
    say("T=0")
    E, K, H = 16, 2, 256
    counts = torch.full((E,), 7, dtype=torch.int32, device=DEV)
    cu = torch.full((E + 1,), 7, dtype=torch.int32, device=DEV)
    n = moe.moe_permute_workspace_bytes(0, E, K)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
    moe.moe_permute(None, None, moe.MOE_BF16, None, None, 0, H, E, K, counts, cu, None, None, None,
                    None, None, ws, n)
    assert host(counts).tolist() == [0] * E and host(cu).tolist() == [0] * (E + 1)
    w = gen.make(T=0, H=H, Hp=128, E=E, K=K, routing="normal", cid=53, device=DEV)
    out, _, _ = run_layer(w)
    torch.cuda.synchronize()
    assert out.shape == (0, H)


def test_invalid_ids_are_dropped_and_validated():
    say("invalid expert ids")
    w = gen.make(T=128, H=256, Hp=128, E=8, K=2, routing="balanced", cid=54, device=DEV)
    bad = w.topk_idx.clone()
    bad[5, 1] = 11
    bad[9, 0] = -3
    w.topk_idx = bad
    r = run_steps(w)
    torch.cuda.synchronize()
    pos = host(r["pos"])
    assert pos[5, 1] == -1 and pos[9, 0] == -1
    assert int(host(r["cu_seqlens"])[-1]) == 128 * 2 - 2
    # the dropped copies contribute nothing: compare with weights zeroed in the oracle
    idx = host(bad).copy()
    tw = host(w.topk_w).astype(np.float64)
    tw[5, 1] = 0.0
    tw[9, 0] = 0.0
    idx[5, 1] = 0
    idx[9, 0] = 0
    x = O.decode_bf16(host(w.x))
    from _oracle_run import weight_fn
    ref = O.layer_token_loop(x, idx, tw, weight_fn(w))
    assert rel_err(O.decode_bf16(host(r["out"])), ref) <= 2e-2
    os.environ["MOE_VALIDATE"] = "1"
    try:
        with pytest.raises(moe.MoeError):
            run_steps(w)
        dup = w.topk_idx.clone()
        dup[:, :] = torch.from_numpy(((np.arange(128)[:, None] * 2 + np.arange(2)) % 8).astype(np.int32)).to(DEV)
        dup[3, 1] = dup[3, 0]
        w.topk_idx = dup
        with pytest.raises(moe.MoeError):
            run_steps(w)
    finally:
        del os.environ["MOE_VALIDATE"]


def test_layer_forward_matches_steps_and_is_deterministic():
    say("layer_forward == steps, bitwise, twice")
    w = gen.make(T=512, H=512, Hp=256, E=16, K=4, routing="skew", beta=0.5, cid=55, device=DEV)
    r = run_steps(w)
    out1, ws, lay = run_layer(w)
    out2, _, _ = run_layer(w)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), r["out"].view(torch.int16))
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    cu = ws[lay["cu_seqlens"]:lay["cu_seqlens"] + 4 * 17].view(torch.int32)
    assert torch.equal(cu, r["cu_seqlens"])


def test_debug_poison_leaves_no_nan():
    say("MOE_DEBUG_POISON")
    w = gen.make(T=200, H=256, Hp=128, E=8, K=2, routing="normal", cid=56, device=DEV)
    d = layer_desc(w)
    need = moe.moe_layer_workspace_bytes(d)
    extra = 4099   # never written by the layer; an odd length for the fill's tail
    ws = torch.zeros(need + extra, dtype=torch.uint8, device=DEV)
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=DEV)
    os.environ["MOE_DEBUG_POISON"] = "1"
    try:
        moe.moe_layer_forward(d, w.x, w.x_sf, w.logits, w.topk_idx, w.topk_w, w.w_gate, w.w_up,
                              w.w_down, w.sf_gate, w.sf_up, w.sf_down, out, ws, need + extra)
        torch.cuda.synchronize()
    finally:
        del os.environ["MOE_DEBUG_POISON"]
    # the poison covered the whole workspace the caller passed
    assert bool((ws[need:] == 0xFF).all())
    assert not torch.isnan(out.float()).any()
    ref = oracle_layer(w)
    assert rel_err(O.decode_bf16(host(out)), ref["out"]) <= 2e-2


# ----------------------------------------------------------------------------- fp8 x MXFP4

FP8_SMALL = [
    dict(T=300, H=512, Hp=256, E=12, K=3, routing="skew", beta=0.5),
    dict(T=600, H=256, Hp=384, E=24, K=4, routing="normal"),
    dict(T=130, H=768, Hp=128, E=5, K=2, routing="balanced"),
]


@pytest.mark.parametrize("spec", FP8_SMALL, ids=lambda s: "T{T}_H{H}_Hp{Hp}_E{E}_K{K}_{routing}".format(**s))
def test_small_fp8_mxfp4_layer(spec):
    say(f"fp8 x mxfp4 small {spec}")
    w = gen.make(**spec, act="fp8", wgt="mxfp4", out="bf16", cid=57, device=DEV)
    r, ref = full_check(w)
    # the requantised h: dequantised values within one e4m3 step, scales mostly identical
    from _oracle_run import weight_fn, x_f64
    x = x_f64(w)
    fn = weight_fn(w)
    cu = ref["cu_seqlens"]
    tok = ref["row_src"] // w.K
    h_gpu = O.decode_fp8_rows(host(r["h"]), host(r["h_sf"]).T)
    sf_gpu = host(r["h_sf"]).T.astype(np.float64)
    worst, same, n = 0.0, 0, 0
    for e in range(w.E):
        lo, hi = int(cu[e]), int(cu[e + 1])
        if hi == lo:
            continue
        wg, wu, _ = fn(e)
        xr = x[tok[lo:hi]]
        g, u = xr @ wg, xr @ wu
        h = g / (1 + np.exp(-g)) * u
        hq, s = O.requant_fp8_1x128(h)
        worst = max(worst, float(np.abs(h_gpu[lo:hi] - hq).max() / max(np.abs(h).max(), 1e-30)))
        same += int((sf_gpu[lo:hi] == s).sum())
        n += s.size
    print(f"  h rel err {worst:.3e}, identical block scales {same}/{n}", flush=True)
    assert worst <= 6e-2
    assert same >= 0.99 * n


# Expert sizes on both sides of the 32-row MFMA block and the 256-row tile: an expert's rows
# are spread evenly over its tiles in 32-row blocks (257 -> 160 + 97, 513 -> 192 + 192 + 129,
# 769 -> 4 tiles), blocks past a tile's rows are skipped, and the gathered-row loads of a
# tile read only rows of that tile.
EDGE_COUNTS = [0, 1, 31, 32, 33, 255, 256, 257, 300, 511, 512, 513, 769, 2]


def edge_routing(counts, K, seed):
    """topk_idx with exactly counts[e] copies of expert e, no token twice on one expert (the
    copies laid out expert by expert, column-major over [T, K]: an expert's copies in column 1
    start after its copies in column 0 end, since no count exceeds T), Dirichlet(1) weights."""
    T = sum(counts) // K
    assert sum(counts) == T * K and max(counts) <= T
    ids = np.repeat(np.arange(len(counts)), counts)
    idx = ids.reshape(K, T).T.copy()
    assert all(len(set(row)) == K for row in idx.tolist())
    wts = np.random.default_rng(seed).dirichlet(np.ones(K), size=T).astype(np.float32)
    return idx.astype(np.int32), wts


@pytest.mark.parametrize("act,wgt", [("bf16", "bf16"), ("fp8", "mxfp4")])
def test_expert_sizes_around_tile_boundaries(act, wgt):
    K = 2
    T, E = sum(EDGE_COUNTS) // K, len(EDGE_COUNTS)
    say(f"{act} x {wgt}: expert sizes {EDGE_COUNTS}")
    w = gen.make(T=T, H=512, Hp=256, E=E, K=K, act=act, wgt=wgt, out="bf16", routing="balanced", cid=61,
                 device=DEV)
    idx, wts = edge_routing(EDGE_COUNTS, K, 61)
    w.topk_idx = torch.from_numpy(idx).to(DEV)
    w.topk_w = torch.from_numpy(wts).to(DEV)
    r, ref = full_check(w)
    assert np.array_equal(ref["counts"], np.asarray(EDGE_COUNTS))
    # the layer (rows gathered from x, no x_perm) gives the same bits as the steps
    out, _, _ = run_layer(w)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), r["out"].view(torch.int16))


# Blocks that run several tiles each, so that the bf16 kernels decode the next tile, load its
# row sources and issue its first stages inside the current tile's K loop: 1024 experts, a
# third of them empty and the rest from 1 to over 1300 rows (one grid stride passes well over
# 64 experts), with K loops of 8 steps, and 16 large experts with K loops of 24 steps. The
# gathered layer must give the same bits as the steps on permuted rows.
SEVERAL_TILES = [
    dict(T=2048, H=256, Hp=256, E=1024, K=8, routing="skew", beta=0.6),
    dict(T=4096, H=768, Hp=768, E=16, K=6, routing="normal"),
]


@pytest.mark.parametrize("spec", SEVERAL_TILES, ids=lambda s: "T{T}_H{H}_Hp{Hp}_E{E}_K{K}".format(**s))
def test_bf16_several_tiles_per_block(spec):
    say(f"bf16 several tiles per block {spec}")
    w = gen.make(**spec, act="bf16", wgt="bf16", out="bf16", cid=72, device=DEV)
    r, ref = full_check(w)
    assert int((np.diff(ref["cu_seqlens"]) > 0).sum()) > 1
    out, _, _ = run_layer(w)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), r["out"].view(torch.int16))


# ----------------------------------------------------------------------------- row maps

GATHER_CASES = [
    ("f32", dict(T=333, H=200, Hp=72, E=9, K=3, routing="skew", beta=0.5)),
    ("bf16", dict(T=600, H=512, Hp=256, E=32, K=6, routing="skew", beta=3.0)),
    ("fp8", dict(T=300, H=512, Hp=256, E=12, K=3, routing="skew", beta=0.5)),
]
FMT = {"f32": ("f32", "f32"), "bf16": ("bf16", "bf16"), "fp8": ("mxfp4", "bf16")}


def make_case(act, spec, cid):
    wgt, out = FMT[act]
    return gen.make(**spec, act=act, wgt=wgt, out=out, cid=cid, device=DEV)


@pytest.mark.parametrize("act,spec", GATHER_CASES, ids=[c[0] for c in GATHER_CASES])
def test_gate_up_gather_is_bitwise_the_permuted_path(act, spec):
    say(f"gate/up gathered from x vs from x_perm, {act} {spec}")
    w = make_case(act, spec, 60)
    r = run_steps(w)
    M = w.T * w.K
    from _gpu_run import DT, TORCH_DT, h_fmt
    rows = int(host(r["cu_seqlens"])[-1])
    # fp8: the activation scales gathered from x_sf (token layout) and read from the permuted
    # block-major copy x_perm_sf give the same h
    for x_sf, x_perm_sf in ((w.x_sf, None),) + (((None, r["x_perm_sf"]),) if act == "fp8" else ()):
        h2 = torch.empty_like(r["h"])
        h2_sf = torch.empty_like(r["h_sf"]) if r["h_sf"] is not None else None
        moe.moe_ffn_gate_up_gather(w.x, x_sf, x_perm_sf, DT[w.act], r["row_src"], w.T, w.K, r["cu_seqlens"],
                                   M, w.E, w.H, w.Hp, w.w_gate, w.w_up, w.sf_gate, w.sf_up, DT[w.wgt], h2,
                                   h2_sf)
        torch.cuda.synchronize()
        assert np.array_equal(host(h2)[:rows], host(r["h"])[:rows])
        if h2_sf is not None:
            assert np.array_equal(host(h2_sf)[:, :rows], host(r["h_sf"])[:, :rows])


@pytest.mark.parametrize("act,spec", GATHER_CASES, ids=[c[0] for c in GATHER_CASES])
def test_layer_with_and_without_x_perm_bitwise(act, spec):
    say(f"layer: MOE_LAYER_XPERM=1 vs the gathered default, {act}")
    w = make_case(act, spec, 61)
    out_g, _, lay_g = run_layer(w)
    os.environ["MOE_LAYER_XPERM"] = "1"
    try:
        out_m, _, lay_m = run_layer(w)
    finally:
        del os.environ["MOE_LAYER_XPERM"]
    torch.cuda.synchronize()
    assert lay_g["x_perm"] is None and lay_m["x_perm"] is not None
    assert np.array_equal(host(out_g), host(out_m))


def decode_out(w, t):
    b = host(t)
    return b.astype(np.float64) if w.out == "f32" else O.decode_bf16(b)


@pytest.mark.parametrize("act,spec", GATHER_CASES, ids=[c[0] for c in GATHER_CASES])
def test_down_scatter_entry_point(act, spec):
    say(f"moe_ffn_down_scatter into a zeroed fp32 accumulator, {act}")
    w = make_case(act, spec, 62)
    r = run_steps(w)
    ref = oracle_layer(w)
    from _gpu_run import DT, h_fmt
    M = w.T * w.K
    acc = torch.zeros((w.T, w.H), dtype=torch.float32, device=DEV)
    moe.moe_ffn_down_scatter(r["h"], r["h_sf"], DT[h_fmt(w)], r["cu_seqlens"], M, w.E, w.H, w.Hp,
                             w.w_down, w.sf_down, DT[w.wgt], r["row_src"], r["row_w"], w.T, w.K, acc)
    torch.cuda.synchronize()
    e = rel_err(host(acc).astype(np.float64), ref["out"])
    # against the deterministic gather combine of the same y (before its bf16 rounding of y)
    e_g = rel_err(host(acc).astype(np.float64), decode_out(w, r["out"]))
    print(f"  acc rel err vs oracle {e:.3e}, vs gather combine {e_g:.3e}", flush=True)
    assert e <= TOL[w.act]


@pytest.mark.parametrize("act,spec", GATHER_CASES, ids=[c[0] for c in GATHER_CASES])
def test_layer_scatter_combine(act, spec):
    say(f"layer with MOE_COMBINE_SCATTER_ATOMIC, {act}")
    w = make_case(act, spec, 63)
    out, ws, lay = run_layer(w, combine=moe.MOE_COMBINE_SCATTER_ATOMIC)
    torch.cuda.synchronize()
    assert lay["y_rows"] is None and lay["row_w"] is not None
    assert (lay["acc_f32"] is None) == (w.out == "f32")
    ref = oracle_layer(w)
    e = rel_err(decode_out(w, out), ref["out"])
    print(f"  out rel err {e:.3e}", flush=True)
    assert e <= TOL[w.act]


def test_layer_scatter_combine_empty_experts_and_t0():
    say("scatter combine: many empty experts, then T=0")
    w = gen.make(T=97, H=256, Hp=128, E=40, K=2, routing="skew", beta=4.0, act="bf16", wgt="bf16",
                 out="bf16", cid=64, device=DEV)
    out, _, _ = run_layer(w, combine=moe.MOE_COMBINE_SCATTER_ATOMIC)
    torch.cuda.synchronize()
    assert rel_err(decode_out(w, out), oracle_layer(w)["out"]) <= TOL["bf16"]
    w0 = gen.make(T=0, H=256, Hp=128, E=8, K=2, routing="normal", cid=64, device=DEV)
    out0, _, _ = run_layer(w0, combine=moe.MOE_COMBINE_SCATTER_ATOMIC)
    torch.cuda.synchronize()
    assert out0.shape == (0, 256)


# ----------------------------------------------------------------------------- shared expert

SHARED_CASES = [
    ("f32", dict(T=333, H=200, Hp=72, E=9, K=3, routing="skew", beta=0.5), 96),
    ("bf16", dict(T=600, H=512, Hp=256, E=32, K=6, routing="skew", beta=3.0), 384),
    ("fp8", dict(T=300, H=512, Hp=256, E=12, K=3, routing="skew", beta=0.5), 256),
]


@pytest.mark.parametrize("act,spec,hs", SHARED_CASES, ids=[c[0] for c in SHARED_CASES])
def test_layer_shared_expert(act, spec, hs):
    say(f"layer + shared expert (Hs={hs}), {act}: one stream, side stream, scatter combine")
    from _gpu_run import run_layer_shared
    from _oracle_run import oracle_layer_shared
    wgt, outf = FMT[act]
    w = gen.make(**spec, act=act, wgt=wgt, out=outf, cid=65, device=DEV, shared_hs=hs)
    ref = oracle_layer_shared(w)
    out1, _ = run_layer_shared(w)
    side = torch.cuda.Stream()
    out2, _ = run_layer_shared(w, side_stream=side)
    out3, _ = run_layer_shared(w, combine=moe.MOE_COMBINE_SCATTER_ATOMIC, side_stream=side)
    torch.cuda.synchronize()
    e1 = rel_err(decode_out(w, out1), ref["out"])
    e3 = rel_err(decode_out(w, out3), ref["out"])
    es = rel_err(decode_out(w, out1), ref["out"] - ref["y_shared"])   # without the shared part
    print(f"  out rel err {e1:.3e} (scatter {e3:.3e}); without the shared term it would be {es:.3e}",
          flush=True)
    assert np.array_equal(host(out1), host(out2))          # the side stream changes nothing
    assert e1 <= TOL[w.act] and e3 <= TOL[w.act]
    assert es > 10 * TOL[w.act]                              # the shared term is really there


def test_combine_shared_entry_point():
    say("moe_combine_shared = moe_combine + the shared row, bitwise on exact inputs")
    T, H, K = 64, 256, 2
    g = torch.Generator(device="cpu").manual_seed(3)
    # values on a coarse grid so the fp32 sums are exact in any order
    y = (torch.randint(-64, 64, (T * K, H), generator=g).float() / 64).to(DEV)
    add = (torch.randint(-64, 64, (T, H), generator=g).float() / 64).to(DEV)
    pos = torch.randperm(T * K, generator=g).view(T, K).int().to(DEV)
    tw = torch.full((T, K), 0.5, device=DEV)
    out = torch.empty((T, H), device=DEV)
    base = torch.empty((T, H), device=DEV)
    moe.moe_combine_shared(y, moe.MOE_F32, pos, tw, T, H, K, add, out, moe.MOE_F32)
    moe.moe_combine(y, moe.MOE_F32, pos, tw, T, H, K, base, moe.MOE_F32)
    torch.cuda.synchronize()
    assert torch.equal(out, base + add)


# ----------------------------------------------------------------------------- quantisation, padding

@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_quantize_fp8_bit_exact(dt):
    say(f"moe_quantize_fp8 from {dt}: codes and scales bit-exact")
    g = torch.Generator(device="cpu").manual_seed(21)
    R, C = 333, 768
    x = torch.randn(R, C, generator=g) * torch.exp2(torch.randint(-12, 12, (R, 1), generator=g).float())
    x[5, :128] = 0.0                     # all-zero block
    x[6, 128:256] = 1e-30                # tiny block (subnormal scale range)
    x[7, 0] = 448.0 * 2 ** 10            # block amax exactly on a power-of-two boundary
    # blocks below the e8m0 floor (scale 2^-127): bf16 / fp32 subnormals, and one value of
    # 2^-149 whose amax / 448 would underflow to zero
    x[8, 256:384] = torch.randn(128, generator=g) * 2.0 ** -131
    x[9, 384:512] = torch.randn(128, generator=g) * 2.0 ** -140
    x[10, 128:256] = 0.0
    x[10, 130] = 2.0 ** -149
    x[11, 640:768] = torch.randn(128, generator=g) * 2.0 ** -120
    xt = x.to(torch.bfloat16 if dt == "bf16" else torch.float32)
    xd = xt.to(DEV)
    q = torch.empty((R, C), dtype=torch.uint8, device=DEV)
    sf = torch.empty((R, C // 128), dtype=torch.float32, device=DEV)
    moe.moe_quantize_fp8(xd, moe.MOE_BF16 if dt == "bf16" else moe.MOE_F32, R, C, q, sf)
    torch.cuda.synchronize()
    xv = O.decode_bf16(host(xt)) if dt == "bf16" else host(xt).astype(np.float64)
    codes, s = O.quantize_fp8_1x128(xv)
    assert np.array_equal(host(sf).astype(np.float64), s)
    assert np.array_equal(host(q), codes)


def padded_steps(w, pad, gather):
    """Padded permute -> grouped FFN over the padded groups (M = capacity) -> combine."""
    from _gpu_run import DT, TORCH_DT, h_fmt, y_fmt
    T, H, Hp, E, K = w.T, w.H, w.Hp, w.E, w.K
    cap = moe.moe_padded_capacity(T, E, K, pad)
    i32 = dict(dtype=torch.int32, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    r = dict(counts=torch.empty(E, **i32), cu_seqlens=torch.empty(E + 1, **i32),
             pos=torch.empty((T, K), **i32), row_src=torch.empty(cap, **i32), row_w=torch.empty(cap, **f32))
    r["x_perm"] = None if gather else torch.empty((cap, H), dtype=TORCH_DT[w.act], device=DEV)
    r["x_perm_sf"] = None if w.act != "fp8" else torch.empty((H // 128, cap), **f32)
    nws = moe.moe_permute_workspace_bytes(T, E, K)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    moe.moe_permute_padded(w.x, w.x_sf, DT[w.act], w.topk_idx, w.topk_w, T, H, E, K, pad, r["counts"],
                           r["cu_seqlens"], r["pos"], r["row_src"], r["row_w"], r["x_perm"], r["x_perm_sf"],
                           ws, nws)
    r["h"] = torch.empty((cap, Hp), dtype=TORCH_DT[h_fmt(w)], device=DEV)
    r["h_sf"] = torch.empty((Hp // 128, cap), **f32) if w.act == "fp8" else None
    if gather:
        # fp8: scales from the permuted copy; the token-layout gather must give the same h
        moe.moe_ffn_gate_up_gather(w.x, None if r["x_perm_sf"] is not None else w.x_sf, r["x_perm_sf"],
                                   DT[w.act], r["row_src"], T, K, r["cu_seqlens"], cap, E, H, Hp, w.w_gate,
                                   w.w_up, w.sf_gate, w.sf_up, DT[w.wgt], r["h"], r["h_sf"])
        if r["x_perm_sf"] is not None:
            h_t, h_t_sf = torch.empty_like(r["h"]), torch.empty_like(r["h_sf"])
            moe.moe_ffn_gate_up_gather(w.x, w.x_sf, None, DT[w.act], r["row_src"], T, K, r["cu_seqlens"], cap,
                                       E, H, Hp, w.w_gate, w.w_up, w.sf_gate, w.sf_up, DT[w.wgt], h_t, h_t_sf)
            torch.cuda.synchronize()
            rows = int(host(r["cu_seqlens"])[-1])
            assert np.array_equal(host(h_t)[:rows], host(r["h"])[:rows])
            assert np.array_equal(host(h_t_sf)[:, :rows], host(r["h_sf"])[:, :rows])
    else:
        moe.moe_ffn_gate_up(r["x_perm"], r["x_perm_sf"], DT[w.act], r["cu_seqlens"], cap, E, H, Hp,
                            w.w_gate, w.w_up, w.sf_gate, w.sf_up, DT[w.wgt], r["h"], r["h_sf"])
    r["y_rows"] = torch.empty((cap, H), dtype=TORCH_DT[y_fmt(w)], device=DEV)
    moe.moe_ffn_down(r["h"], r["h_sf"], DT[h_fmt(w)], r["cu_seqlens"], cap, E, H, Hp, w.w_down, w.sf_down,
                     DT[w.wgt], r["y_rows"], DT[y_fmt(w)])
    r["out"] = torch.empty((T, H), dtype=TORCH_DT[w.out], device=DEV)
    moe.moe_combine(r["y_rows"], DT[y_fmt(w)], r["pos"], w.topk_w, T, H, K, r["out"], DT[w.out])
    r["acc"] = torch.zeros((T, H), **f32)
    moe.moe_ffn_down_scatter(r["h"], r["h_sf"], DT[h_fmt(w)], r["cu_seqlens"], cap, E, H, Hp, w.w_down,
                             w.sf_down, DT[w.wgt], r["row_src"], r["row_w"], T, K, r["acc"])
    return r, cap


PAD_CASES = [("bf16", 128, False), ("bf16", 128, True), ("fp8", 128, False), ("fp8", 64, True),
             ("f32", 16, True)]


@pytest.mark.parametrize("act,pad,gather", PAD_CASES, ids=[f"{a}_pad{p}_{'gather' if g else 'xperm'}"
                                                          for a, p, g in PAD_CASES])
def test_padded_layout_and_results(act, pad, gather):
    say(f"padded permute (pad {pad}), {act}, {'gathered' if gather else 'materialised'} rows")
    spec = {"f32": dict(T=333, H=200, Hp=72, E=9, K=3), "bf16": dict(T=600, H=512, Hp=256, E=32, K=6),
            "fp8": dict(T=300, H=512, Hp=256, E=12, K=3)}[act]
    w = make_case(act, dict(spec, routing="balanced"), 66)
    idx = host(w.topk_idx)
    # skew the given routing so groups are ragged and some experts are empty
    rng = np.random.default_rng(5)
    idx = np.stack([rng.choice(w.E // 2 + 1, w.K, replace=False) for _ in range(w.T)]).astype(np.int32)
    w.topk_idx = torch.from_numpy(idx).to(DEV)
    r, cap = padded_steps(w, pad, gather)
    base = run_steps(w)
    torch.cuda.synchronize()
    ppos, prs, pcu = O.permute_padded(idx, w.E, pad)
    counts, _ = O.count_offsets(idx, w.E)
    assert cap == len(prs)
    assert np.array_equal(host(r["counts"]), counts)
    assert np.array_equal(host(r["cu_seqlens"]), pcu)
    assert np.array_equal(host(r["pos"]), ppos)
    assert np.array_equal(host(r["row_src"]), prs)
    tw = host(w.topk_w).ravel()
    assert np.array_equal(host(r["row_w"]), np.where(prs >= 0, tw[np.maximum(prs, 0)], 0).astype(np.float32))
    real = prs[:pcu[-1]] >= 0
    if not gather:
        xp = host(r["x_perm"])[:pcu[-1]]
        assert np.array_equal(xp[real], host(w.x)[prs[:pcu[-1]][real] // w.K])
        assert not xp[~real].any()
    if w.act == "fp8":   # written with and without x_perm
        sfp = host(r["x_perm_sf"])[:, :pcu[-1]].T
        assert np.array_equal(sfp[real], host(w.x_sf)[prs[:pcu[-1]][real] // w.K])
        assert np.all(sfp[~real] == 1.0)
    # per-row results do not depend on where a group starts: same output, bit for bit
    assert np.array_equal(host(r["out"]), host(base["out"]))
    ref = oracle_layer(w)
    assert rel_err(host(r["acc"]).astype(np.float64), ref["out"]) <= TOL[w.act]


@pytest.mark.parametrize("spec", FP8_SMALL[:2], ids=lambda s: "T{T}_H{H}_Hp{Hp}_E{E}_K{K}_{routing}".format(**s))
def test_layer_bf16_activations_mxfp4_experts(spec):
    say(f"(BF16, MXFP4) layer: quantised on entry, {spec}")
    w = gen.make(**spec, act="bf16", wgt="mxfp4", out="bf16", cid=67, device=DEV)
    out, ws, lay = run_layer(w)
    torch.cuda.synchronize()
    assert lay["x_q"] is not None and lay["x_q_sf"] is not None
    # the oracle quantises the same bf16 values with its own 1x128 rule, then runs the fp8 layer
    from _oracle_run import weight_fn
    b = host(w.x)
    codes, s = O.quantize_fp8_1x128(O.decode_bf16(b))
    xq = O.decode_fp8_rows(codes, s)
    bits = {"logits": host(w.logits), "topk_idx": host(w.topk_idx), "topk_w": host(w.topk_w)}
    ref = O.layer(xq, w.E, w.K, weight_fn(w), logits=bits["logits"], topk_idx=bits["topk_idx"],
                  topk_w=bits["topk_w"], fp8_requant=True)
    e = rel_err(decode_out(w, out), ref["out"])
    print(f"  out rel err {e:.3e}", flush=True)
    assert e <= TOL["fp8"]
    # and the quantised activations in the workspace are the oracle's bytes
    n = w.T * w.H
    assert np.array_equal(host(ws[lay["x_q"]:lay["x_q"] + n]).reshape(w.T, w.H), codes)


# ----------------------------------------------------------------------------- paired MXFP4 layout

def test_pack_mxfp4_pairs_layout():
    """moe_pack_mxfp4_pairs writes [E][N/2][K/128][2][64] from [E][N][K/2]: output byte
    (e, p, s, h, b) is input byte (e, 2p + h, 64 s + b), checked with numpy index arithmetic."""
    rng = np.random.default_rng(71)
    for E, N, K in ((3, 6, 256), (2, 258, 384), (1, 2, 128), (4, 128, 7168)):
        say(f"pack MXFP4 pairs E={E} N={N} K={K}")
        w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
        wt = torch.from_numpy(w).to(DEV)
        out = torch.full_like(wt, 0xA5)
        moe.moe_pack_mxfp4_pairs(wt, out, E, N, K)
        torch.cuda.synchronize()
        want = w.reshape(E, N // 2, 2, K // 128, 64).transpose(0, 1, 3, 2, 4).reshape(E, N, K // 2)
        assert np.array_equal(host(out), want)


@pytest.mark.parametrize("spec", FP8_SMALL, ids=lambda s: "T{T}_H{H}_Hp{Hp}_E{E}_K{K}_{routing}".format(**s))
def test_paired_mxfp4_weights_give_bitwise_the_same_results(spec):
    """The fp8 x MXFP4 steps and layer with the weights repacked to MOE_MXFP4_PAIRED: h, its
    scales, y_rows and out are bit for bit those of the stored layout (the kernels stage the
    same bytes); the same for the layer that quantises bf16 activations on entry. The
    scatter-add combine agrees within its atomic order."""
    from _gpu_run import paired
    say(f"MXFP4 paired layout against the stored one {spec}")
    w = gen.make(**spec, act="fp8", wgt="mxfp4", out="bf16", cid=72, device=DEV)
    wp = paired(w)
    r, rp = run_steps(w), run_steps(wp)
    out_l, _, _ = run_layer(w)
    out_p, _, _ = run_layer(wp)
    sc_l, _, _ = run_layer(w, combine=moe.MOE_COMBINE_SCATTER_ATOMIC)
    sc_p, _, _ = run_layer(wp, combine=moe.MOE_COMBINE_SCATTER_ATOMIC)
    torch.cuda.synchronize()
    for k in ("h", "h_sf", "y_rows", "out"):
        assert torch.equal(r[k], rp[k]), k
    assert torch.equal(out_p, out_l)
    d = float((sc_p.float() - sc_l.float()).abs().max() / sc_l.float().abs().max())
    assert d <= 2.0 ** -7
    wb = gen.make(**spec, act="bf16", wgt="mxfp4", out="bf16", cid=73, device=DEV)
    ob, _, _ = run_layer(wb)
    obp, _, _ = run_layer(paired(wb))
    torch.cuda.synchronize()
    assert torch.equal(obp, ob)


# ----------------------------------------------------------------------------- backward

BWD_CASES = [
    dict(T=300, H=512, Hp=256, E=12, K=3, routing="normal"),
    dict(T=600, H=256, Hp=512, E=32, K=4, routing="skew", beta=3.0),   # empty experts
    dict(T=130, H=768, Hp=256, E=5, K=2, routing="balanced"),          # given routing
]


@pytest.mark.parametrize("spec", BWD_CASES, ids=lambda s: "T{T}_H{H}_Hp{Hp}_E{E}_K{K}_{routing}".format(**s))
def test_layer_backward(spec):
    say(f"layer backward {spec}")
    w = gen.make(**spec, act="bf16", wgt="bf16", out="bf16", cid=70, device=DEV)
    g = torch.Generator(device="cpu").manual_seed(7)
    dout = torch.randn((w.T, w.H), generator=g).to(torch.bfloat16).to(DEV)
    check_backward(w, dout)


def test_layer_backward_c2_full():
    say("layer backward, c2 full size (oracle backward over every expert)")
    w = gen.config("c2", device=DEV)
    g = torch.Generator(device="cpu").manual_seed(8)
    dout = torch.randn((w.T, w.H), generator=g).to(torch.bfloat16).to(DEV)
    check_backward(w, dout)


def test_layer_backward_t0():
    say("layer backward, T=0: zero weight gradients")
    w = gen.make(T=0, H=256, Hp=256, E=4, K=2, routing="normal", cid=71, device=DEV)
    dout = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    r = run_backward(w, dout)
    torch.cuda.synchronize()
    assert not r["dWg"].any() and not r["dWu"].any() and not r["dWd"].any()


# ----------------------------------------------------------------------------- full size, every group
#
# The full-size workloads, with every step at its real shape (224-step K loops at H = 7168,
# several tiles per block, the cross-tile prefetch tail): routing, counts, cu_seqlens, the
# permutation and the permuted rows compared in full; y_rows compared with the oracle at the
# first and last row of every non-empty expert group and at all K rows of 16 tokens (whose
# out is then the oracle's combine of those rows); moe_layer_forward, the path bench.py
# times (rows gathered from x), bitwise equal to the step-by-step path; the layer with the
# scatter-add combine within tolerance at the same tokens. Every expert's weights are
# decoded once per test, for all its routings.

def probe_rows(ref, K, n_tokens=16, seed=0):
    """(rows, tokens): the first and last row of every non-empty group, and all K rows of
    the first and last token, of the tokens at both ends of the busiest and of the least busy
    group, and of seeded random tokens up to ``n_tokens``."""
    cu, counts, row_src = ref["cu_seqlens"], ref["counts"], ref["row_src"]
    T = ref["pos"].shape[0]
    rows = set()
    for e in np.nonzero(counts)[0]:
        rows.update((int(cu[e]), int(cu[e + 1]) - 1))
    hot = int(np.argmax(counts))
    cold = int(np.argmin(np.where(counts > 0, counts, np.iinfo(np.int64).max)))
    toks = {0, T - 1}
    for e in (hot, cold):
        toks.update(int(row_src[r]) // K for r in (int(cu[e]), int(cu[e + 1]) - 1))
    rng = np.random.default_rng(seed)
    while len(toks) < min(n_tokens, T):
        toks.add(int(rng.integers(T)))
    toks = sorted(toks)
    for t in toks:
        rows.update(int(p) for p in ref["pos"][t])
    return sorted(rows), toks


def full_size_check(variants):
    """``variants``: [(label, workload)], all with the same x and weights (c4's routings)."""
    cases = []
    for label, w in variants:
        say(f"  {label}: steps, moe_layer_forward (gather combine and scatter-add combine)")
        r = run_steps(w, with_row_w=False)
        torch.cuda.synchronize()
        ref = oracle_routing(w)
        check_integers(r, ref, w.K)
        check_x_perm(w, r, ref)
        del r["x_perm"]
        # bf16: the layer with the FFN as two persistent launches, then as one (gate/up and
        # down tiles from device-side queues): the same out, bit for bit, and for the single
        # launch the same y_rows, every tile run once and no wait past its bound
        for fused in (("0", "1") if w.act == "bf16" else (None,)):
            if fused is not None:
                os.environ["MOE_LAYER_FUSED"] = fused
            try:
                out_l, ws, lay = run_layer(w)
            finally:
                os.environ.pop("MOE_LAYER_FUSED", None)
            torch.cuda.synchronize()
            assert torch.equal(out_l, r["out"]), f"{label}: moe_layer_forward ({fused}) differs from the steps"
            if fused == "1":
                M = w.T * w.K
                y_f = ws[lay["y_rows"]:lay["y_rows"] + M * w.H * 2].view(torch.bfloat16).view(M, w.H)
                ctl = host(ws[lay["fused_ctl"]:lay["fused_ctl"] + 64].view(torch.int32))
                print(f"  single launch: tiles {ctl[9]}, not prefetched {ctl[10]}, from other queues "
                      f"{ctl[11]}", flush=True)
                assert ctl[8] == 0 and ctl[9] == sum((int(c) + 255) // 256 for c in ref["counts"]) * (
                    w.Hp // 128 + w.H // 256)
                assert torch.equal(y_f, r["y_rows"]), f"{label}: single-launch y_rows differ"
                del y_f
            del out_l, ws
        if w.wgt == "mxfp4":
            # the weights repacked to the paired layout: the same out, bit for bit
            from _gpu_run import paired
            wp = paired(w)
            out_p, ws, _ = run_layer(wp)
            torch.cuda.synchronize()
            assert torch.equal(out_p, r["out"]), f"{label}: paired MXFP4 weights give another out"
            del wp, out_p, ws
        out_sc, ws, _ = run_layer(w, combine=moe.MOE_COMBINE_SCATTER_ATOMIC)
        torch.cuda.synchronize()
        del ws
        rows, toks = probe_rows(ref, w.K)
        ri = torch.tensor(rows, dtype=torch.int64, device=DEV)
        ti = torch.tensor(toks, dtype=torch.int64, device=DEV)
        c = dict(label=label, ref=ref, rows=rows, toks=toks, y=host(r["y_rows"].index_select(0, ri)),
                 out=host(r["out"].index_select(0, ti)), out_sc=host(out_sc.index_select(0, ti)),
                 maxvio=O.maxvio(ref["counts"], w.T, w.K, w.E))
        if w.act == "fp8":
            c["h"] = host(r["h"].index_select(0, ri))
            c["h_sf"] = host(r["h_sf"].index_select(1, ri)).T
        cases.append(c)
        del r, out_sc
        torch.cuda.empty_cache()
    w0 = variants[0][1]
    tol = TOL[w0.act]
    say(f"  oracle: {sum(len(c['rows']) for c in cases)} rows over {w0.E} experts")
    want = oracle_rows(w0, [(c["ref"], c["rows"]) for c in cases])
    for c, wr in zip(cases, want):
        ref = c["ref"]
        y_ref = np.stack([wr[r][1] for r in c["rows"]])
        e_y = max(rel_err(g, f) for g, f in zip(O.decode_bf16(c["y"]), y_ref))
        # out at the sampled tokens: the oracle's combine of the oracle's rows
        at = {r: i for i, r in enumerate(c["rows"])}
        pos_sub = np.array([[at[int(p)] for p in ref["pos"][t]] for t in c["toks"]])
        out_ref = O.combine(y_ref, pos_sub, ref["topk_w"][c["toks"]])
        e_out = max(rel_err(g, f) for g, f in zip(O.decode_bf16(c["out"]), out_ref))
        e_sc = max(rel_err(g, f) for g, f in zip(O.decode_bf16(c["out_sc"]), out_ref))
        msg = (f"  {c['label']}: maxvio {c['maxvio']:.3f}, rows/group {ref['counts'].min()}-"
               f"{ref['counts'].max()}; {len(c['rows'])} rows: y rel err {e_y:.2e}; {len(c['toks'])} "
               f"tokens: out {e_out:.2e}, scatter-add out {e_sc:.2e}")
        if w0.act == "fp8":
            h_ref = np.stack([wr[r][0] for r in c["rows"]])
            s_ref = np.stack([wr[r][2] for r in c["rows"]])
            h_got = O.decode_fp8_rows(c["h"], c["h_sf"])
            e_h = max(rel_err(g, f) for g, f in zip(h_got, h_ref))
            same = float((c["h_sf"].astype(np.float64) == s_ref).mean())
            msg += f"; h rel err {e_h:.2e}, identical h scales {same:.4f}"
            assert e_h <= tol and same >= 0.99, msg
        print(msg, flush=True)
        assert e_y <= tol and e_out <= tol and e_sc <= tol, msg


@pytest.mark.slow
def test_c3_full_size_every_group():
    say("c3 bf16 rank share (52 slots, 65536 rows, H=7168, Hp=2048), full size")
    full_size_check([("c3", gen.config("c3", device=DEV))])


@pytest.mark.slow
def test_c4_full_size_every_group_all_maxvio():
    say("c4 bf16 T=8192 E=384 K=8, full size, maxvio 0.2 / 1 / 10 / 20 (same x and weights)")
    base = gen.config("c4", device=DEV, maxvio=1.0)
    full_size_check([(f"c4 maxvio {mv:g}", gen.with_maxvio(base, mv)) for mv in gen.SKEW_TARGETS])


@pytest.mark.slow
def test_c5_full_size_every_group():
    say("c5 fp8 x MXFP4 T=8192 E=384 K=8 maxvio 1, full size (h checked too)")
    full_size_check([("c5", gen.config("c5", device=DEV))])
