"""Properties of the seeded synthetic workloads (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from workloads import gen
from workloads.gen import _to_e4m3_blocked, _to_mxfp4, to_numpy_bits


def test_c1_shapes_and_reproducibility():
    a = gen.config("c1")
    b = gen.config("c1")
    assert a.x.shape == (64, 128) and a.x.dtype == torch.float32
    assert a.logits.shape == (64, 8) and a.w_gate.shape == (8, 128, 64) and a.w_down.shape == (8, 64, 128)
    assert torch.equal(a.x, b.x) and torch.equal(a.w_down, b.w_down) and torch.equal(a.logits, b.logits)
    # weights N(0, 1/fan_in)
    assert abs(a.w_gate.std().item() - 128 ** -0.5) < 0.01
    assert abs(a.w_down.std().item() - 64 ** -0.5) < 0.01


def test_balanced_slot_routing_counts():
    """Given routing of the 52-slot share: 1261 rows in slots 0-15, 1260 in 16-51, and a
    token's 8 copies land in 8 distinct slots."""
    T, E, K = 8192, 52, 8
    t = np.arange(T)[:, None]
    k = np.arange(K)[None, :]
    idx = (K * t + k) % E
    counts, cu = O.count_offsets(idx, E)
    assert counts.tolist() == [1261] * 16 + [1260] * 36
    assert all(len(set(r)) == K for r in idx)
    small = gen.make(T=64, H=128, Hp=128, E=52, K=8, routing="balanced", cid=2)
    assert np.array_equal(small.topk_idx.numpy(), idx[:64])
    np.testing.assert_allclose(small.topk_w.sum(dim=1).numpy(), 1.0, rtol=1e-6)


@pytest.mark.parametrize("target", gen.SKEW_TARGETS)
def test_skew_calibration_hits_target(target):
    beta = gen.skew_beta(8192, 384, 8, target)
    idx, _ = O.route_topk(gen.skew_logits(8192, 384, beta, cid=3), 8)
    counts, _ = O.count_offsets(idx, 384)
    mv = O.maxvio(counts, 8192, 8, 384)
    if beta == 0.0:
        assert mv >= target           # unbiased routing already reaches the target
    else:
        assert abs(mv - target) <= 0.01 * target
    assert (counts > 0).all()         # every expert stays active


def test_mxfp4_generator_exact_on_grid_and_nearest_off_grid():
    rng = np.random.default_rng(0)
    Kred, N = 64, 5
    codes = rng.integers(0, 16, size=(Kred, N))
    codes[0, :] = 7                   # amax of each block is 6 * 2^s
    codes[32, :] = 15
    s = rng.integers(-8, 3, size=(2, N))
    table = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    vals = np.where(codes & 8, -1, 1) * table[codes & 7] * np.exp2(np.repeat(s, 32, axis=0))
    packed, sb = _to_mxfp4(torch.from_numpy(vals.astype(np.float32)))
    assert np.array_equal(O.decode_mxfp4(packed.numpy(), sb.numpy()), vals)
    # random values: each decoded element is a nearest grid point of w / X
    w = torch.from_numpy(rng.standard_normal((Kred, N)).astype(np.float32))
    packed, sb = _to_mxfp4(w)
    dec = O.decode_mxfp4(packed.numpy(), sb.numpy())
    X = np.repeat(np.exp2(sb.numpy().astype(np.float64) - 127), 32, axis=0)
    v = w.numpy().astype(np.float64) / X
    grid = np.concatenate([-table[::-1], table])
    nearest = np.abs(np.clip(v, -6, 6)[..., None] - grid).min(axis=-1)
    assert np.allclose(np.abs(np.clip(v, -6, 6) - dec / X), nearest, atol=1e-12)


def test_fp8_activation_generator_error_bound():
    rng = np.random.default_rng(1)
    x = torch.from_numpy(rng.standard_normal((4, 256)).astype(np.float32))
    q, s = _to_e4m3_blocked(x)
    dec = O.decode_fp8_rows(q.numpy(), s.numpy())
    amax = np.abs(x.numpy()).reshape(4, 2, 128).max(axis=2)
    assert np.all(amax / s.numpy() <= 448) and np.all(amax / s.numpy() > 224)
    # e4m3 keeps 3 mantissa bits: relative error <= 2^-4 for normal values
    xx = x.numpy().astype(np.float64)
    big = np.abs(xx) > 2.0 ** -6 * np.repeat(s.numpy(), 128, axis=1)
    assert np.all(np.abs(dec - xx)[big] <= 2.0 ** -4 * np.abs(xx)[big])


def test_numpy_bits_roundtrip():
    t = torch.randn(8, dtype=torch.float32).to(torch.bfloat16)
    bits = to_numpy_bits(t)
    assert bits.dtype == np.uint16
    assert np.array_equal(O.decode_bf16(bits), t.to(torch.float64).numpy())


def test_oracle_rows_matches_whole_layer():
    """The row-sampling helper of the full-size GPU checks (one weight decode per expert,
    several routings, MXFP4 experts decoded in spawned worker processes) gives the oracle
    layer's own y_rows, h and h scales at the rows it is asked for."""
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from _oracle_run import oracle_layer, oracle_routing, oracle_rows, rel_err, x_f64, weight_fn
    for act, wgt in (("bf16", "bf16"), ("fp8", "mxfp4")):
        w = gen.make(T=200, H=256, Hp=128, E=10, K=3, routing="skew", beta=0.7, act=act, wgt=wgt, cid=5)
        ref = oracle_routing(w)
        full = oracle_layer(w)
        rows = [0, 5, 17, 599]
        res = oracle_rows(w, [(ref, rows), (ref, [3, 5])], workers=2)
        assert sorted(res[0]) == rows and sorted(res[1]) == [3, 5]
        for r in rows:
            assert rel_err(res[0][r][1], full["y_rows"][r]) <= 1e-12
        assert np.array_equal(res[1][5][1], res[0][5][1])
        if act == "fp8":
            # h and its scales: the oracle's requantisation of the row's SwiGLU output
            e = int(np.searchsorted(ref["cu_seqlens"], 17, side="right") - 1)
            wg, wu, _ = weight_fn(w)(e)
            xr = x_f64(w)[ref["row_src"][17] // w.K][None, :]
            g, u = xr @ wg, xr @ wu
            hq, s = O.requant_fp8_1x128(O.silu(g) * u)
            assert rel_err(res[0][17][0], hq[0]) <= 1e-12 and np.array_equal(res[0][17][2], s[0])
        else:
            assert res[0][17][2] is None


def test_with_maxvio_keeps_inputs_and_swaps_routing():
    """A layer of the full-size routing shape (T=8192, E=384, K=8; small H and H') rebuilt
    for another maxvio target keeps x and the weights and takes that target's logits."""
    w = gen.make(T=8192, H=128, Hp=128, E=384, K=8, routing="skew", beta=0.0, maxvio=0.2, cid=3)
    w2 = gen.with_maxvio(w, 10.0)
    assert w2.x is w.x and w2.w_gate is w.w_gate and w2.w_down is w.w_down
    assert w2.meta["maxvio_target"] == 10.0 and w2.meta["beta"] == gen.skew_beta(8192, 384, 8, 10.0)
    ref = gen.skew_logits(8192, 384, w2.meta["beta"], 0, 3)
    assert np.array_equal(w2.logits.numpy(), ref)
    idx, _ = O.route_topk(ref, 8)
    counts, _ = O.count_offsets(idx, 384)
    assert abs(O.maxvio(counts, 8192, 8, 384) - 10.0) <= 0.1
