"""Pins of the CPU oracle against facts that do not come from the oracle itself:
the pages' worked example, closed forms, brute force on tiny inputs, invariants the
pages state, and independent library routines for the number formats."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- worked example

def test_four_rank_example_routing_counts_permutation():
    g = _golden("four_rank_example.json")
    logits = np.array(g["logits"], dtype=np.float32)
    idx, w = O.route_topk(logits, g["K"])
    assert idx.tolist() == g["topk_idx"]
    e = math.e
    np.testing.assert_allclose(w, [[e / (1 + e), 1 / (1 + e)]] * 3, rtol=0, atol=1e-15)
    counts, cu = O.count_offsets(idx, g["E"])
    assert counts.tolist() == g["counts"]
    assert cu.tolist() == g["cu_seqlens"]
    per_rank = counts.reshape(g["ranks"], -1).sum(axis=1)
    assert per_rank.tolist() == g["copies_per_rank"]      # keeps 2, sends 1 / 2 / 1
    pos, row_src = O.permute(idx, g["E"])
    assert row_src.tolist() == g["row_src"]
    assert pos.tolist() == g["pos"]


def test_four_rank_example_combine_adds_scaled_outputs():
    """Combine of the worked example: token A ends up as w_A0 * E1(A) + w_A1 * E5(A), with
    w_A its two routing weights (accumulated, not overwritten)."""
    g = _golden("four_rank_example.json")
    rng = np.random.default_rng(1)
    H = 4
    x = rng.standard_normal((3, H))
    # expert e scales its input by (e + 1): Wg = I (gate), Wu = I, Wd = (e+1) I
    def weights(e):
        return np.eye(H), np.eye(H), (e + 1.0) * np.eye(H)
    res = O.layer(x, g["E"], g["K"], weights, logits=np.array(g["logits"], np.float32))
    e = math.e
    wA = [e / (1 + e), 1 / (1 + e)]
    base = x[0] / (1 + np.exp(-x[0])) * x[0]            # silu(x) * x
    expect_A = wA[0] * 2.0 * base + wA[1] * 6.0 * base   # experts 1 and 5
    np.testing.assert_allclose(res["out"][0], expect_A, rtol=1e-14, atol=1e-14)


# ----------------------------------------------------------------------------- routing

def _brute_topk(lg, K):
    T, E = lg.shape
    idx = np.zeros((T, K), np.int64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))
        idx[t] = order[:K]
    return idx


@pytest.mark.parametrize("T,E,K,seed", [(40, 8, 2, 0), (33, 16, 4, 1), (17, 64, 8, 2), (9, 5, 5, 3)])
def test_topk_matches_brute_force_with_ties(T, E, K, seed):
    rng = np.random.default_rng(seed)
    lg = np.round(rng.standard_normal((T, E)) * 2) / 2      # coarse grid -> many ties
    lg = lg.astype(np.float32)
    idx, _ = O.route_topk(lg, K)
    assert np.array_equal(idx, _brute_topk(lg, K))


def test_topk_weights_are_renormalised_full_softmax():
    rng = np.random.default_rng(7)
    lg = rng.standard_normal((50, 12)).astype(np.float32)
    idx, w = O.route_topk(lg, 3)
    full = np.exp(lg.astype(np.float64))
    full /= full.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(full, idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13)
    # descending weights, sum 1
    assert np.all(np.diff(w, axis=1) <= 0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-15)


def test_topk_special_cases():
    lg = np.zeros((3, 6), np.float32)
    idx, w = O.route_topk(lg, 4)                 # all equal -> ids 0..3, weights 1/K
    assert idx.tolist() == [[0, 1, 2, 3]] * 3
    np.testing.assert_allclose(w, 0.25)
    lg = np.array([[0.5, -1.0, 3.0]], np.float32)
    idx, w = O.route_topk(lg, 1)                 # K = 1 -> argmax, weight 1
    assert idx.tolist() == [[2]] and w.tolist() == [[1.0]]
    idx, w = O.route_topk(np.array([[1.25, 0.0]], np.float32), 2)
    sig = 1.0 / (1.0 + math.exp(-1.25))          # two experts: logistic of the gap
    np.testing.assert_allclose(w, [[sig, 1 - sig]], rtol=1e-15)
    with pytest.raises(ValueError):
        O.route_topk(np.zeros((1, 3), np.float32), 4)


# ----------------------------------------------------------------------------- counts / permutation

@pytest.mark.parametrize("T,E,K,seed", [(100, 8, 2, 0), (257, 64, 6, 1), (31, 52, 8, 2)])
def test_permutation_is_stable_counting_sort(T, E, K, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    counts, cu = O.count_offsets(idx, E)
    assert counts.sum() == T * K
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    pos, row_src = O.permute(idx, E)
    # the same permutation as a stable sort of the flat copies by expert id
    assert np.array_equal(row_src, np.argsort(idx.ravel(), kind="stable"))
    # exact inversion and bijection
    flat = np.arange(T * K).reshape(T, K)
    assert np.array_equal(row_src[pos], flat)
    assert np.array_equal(np.sort(pos.ravel()), np.arange(T * K))
    # each row of group e really belongs to expert e, ascending inside the group
    for e in range(E):
        grp = row_src[cu[e]:cu[e + 1]]
        assert np.all(idx.ravel()[grp] == e)
        assert np.all(np.diff(grp) > 0)


def test_empty_experts_and_empty_batch():
    idx = np.array([[3, 1]], np.int32)
    counts, cu = O.count_offsets(idx, 6)
    assert counts.tolist() == [0, 1, 0, 1, 0, 0]
    assert cu.tolist() == [0, 0, 1, 1, 2, 2, 2]
    pos, row_src = O.permute(np.zeros((0, 2), np.int32), 4)
    assert pos.shape == (0, 2) and row_src.shape == (0,)


def test_maxvio_closed_forms():
    T, E, K = 64, 8, 2
    assert O.maxvio(np.full(E, T * K // E), T, K, E) == 0.0
    skew = np.zeros(E, int)
    skew[:K] = T                                  # every token picks the same K experts
    assert O.maxvio(skew, T, K, E) == pytest.approx(E / K - 1)
    # the 52-slot balanced share: 16 slots hold 1261 rows, 36 hold 1260
    c = np.array([1261] * 16 + [1260] * 36)
    assert c.sum() == 8192 * 8
    assert O.maxvio(c, 8192, 8, 52) == pytest.approx(1261 * 52 / 65536 - 1, abs=1e-15)


# ----------------------------------------------------------------------------- FFN

def test_silu_closed_form_values():
    z = np.array([0.0, 1.0, -1.0, 20.0])
    np.testing.assert_allclose(O.silu(z), [0.0, 1 / (1 + math.exp(-1)), -1 / (1 + math.e),
                                           20.0 / (1 + math.exp(-20.0))], rtol=1e-15)


def test_expert_ffn_hand_computable_non_square():
    """H=3, Hp=2 with selection matrices: every operand order matters."""
    x = np.array([[0.5, -2.0, 1.5]])
    wg = np.array([[0, 2.0], [0, 0], [1.0, 0]])    # g = [x2, 2 x0]
    wu = np.array([[0, 0], [3.0, 0], [0, -1.0]])   # u = [3 x1, -x2]
    wd = np.array([[0, 1.0, 0], [4.0, 0, 0]])      # y = [4 h1, h0, 0]
    h, y = O.expert_ffn(x, wg, wu, wd)
    s = lambda z: z / (1 + math.exp(-z))
    h0 = s(1.5) * (3 * -2.0)
    h1 = s(1.0) * (-1.5)
    np.testing.assert_allclose(h, [[h0, h1]], rtol=1e-15)
    np.testing.assert_allclose(y, [[4 * h1, h0, 0.0]], rtol=1e-15)


def test_identical_experts_reduce_to_dense_ffn():
    """Sum of weights is 1, so identical experts give the dense FFN: top-k results are
    added, not overwritten."""
    rng = np.random.default_rng(3)
    T, H, Hp, E, K = 20, 16, 8, 6, 3
    x = rng.standard_normal((T, H))
    wg, wu, wd = rng.standard_normal((H, Hp)), rng.standard_normal((H, Hp)), rng.standard_normal((Hp, H))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    res = O.layer(x, E, K, lambda e: (wg, wu, wd), logits=lg)
    g, u = x @ wg, x @ wu
    dense = (g / (1 + np.exp(-g)) * u) @ wd
    np.testing.assert_allclose(res["out"], dense, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("T,H,Hp,E,K,seed", [(64, 128, 64, 8, 2, 0), (37, 32, 16, 10, 4, 5)])
def test_layer_equals_direct_expert_loop(T, H, Hp, E, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    W = [(rng.standard_normal((H, Hp)) / math.sqrt(H), rng.standard_normal((H, Hp)) / math.sqrt(H),
          rng.standard_normal((Hp, H)) / math.sqrt(Hp)) for _ in range(E)]
    lg = rng.standard_normal((T, E)).astype(np.float32)
    res = O.layer(x, E, K, lambda e: W[e], logits=lg)
    ref = O.layer_token_loop(x, res["topk_idx"], res["topk_w"], lambda e: W[e])
    scale = np.abs(ref).max()
    assert np.abs(res["out"] - ref).max() <= 1e-12 * scale


def test_shared_expert_hand_computable_and_added():
    """Shared expert with H = Hs and Ws_gate = a I, Ws_up = I, Ws_down = P (a permutation):
    SharedExpert(x) = P-permuted silu(a x) * x elementwise, and it is added to the routed
    sum (MoE(x) = SharedExpert(x) + sum_k w_k Expert_k(x), "Mixture of Kittens", Step 1)."""
    x = np.array([[1.0, -2.0, 0.0], [0.5, 3.0, -1.0]])
    a = 2.0
    P = np.array([[0, 1.0, 0], [0, 0, 1.0], [1.0, 0, 0]])     # column j of the output = input j-1
    ys = O.shared_expert(x, a * np.eye(3), np.eye(3), P)
    s = lambda z: z / (1 + math.exp(-z))
    elem = np.array([[s(a * v) * v for v in row] for row in x])
    np.testing.assert_allclose(ys, elem[:, [2, 0, 1]], rtol=1e-15)
    # routed part: one expert with zero down weights contributes nothing, so out == ys
    zero = (np.eye(3), np.eye(3), np.zeros((3, 3)))
    res = O.layer_with_shared(x, x, 1, 1, lambda e: zero, (a * np.eye(3), np.eye(3), P),
                              topk_idx=np.zeros((2, 1), np.int32), topk_w=np.ones((2, 1)))
    np.testing.assert_allclose(res["out"], elem[:, [2, 0, 1]], rtol=1e-15)


def test_shared_expert_equal_to_the_routed_one_doubles_the_output():
    """E=1, K=1 (weight 1) and shared weights equal to the expert's: out = 2 x dense FFN
    (the shared output is added, not overwritten or dropped)."""
    rng = np.random.default_rng(7)
    T, H, Hs = 9, 8, 4
    x = rng.standard_normal((T, H))
    wg, wu, wd = rng.standard_normal((H, Hs)), rng.standard_normal((H, Hs)), rng.standard_normal((Hs, H))
    res = O.layer_with_shared(x, x, 1, 1, lambda e: (wg, wu, wd), (wg, wu, wd),
                              topk_idx=np.zeros((T, 1), np.int32), topk_w=np.ones((T, 1)))
    g, u = x @ wg, x @ wu
    dense = (g / (1 + np.exp(-g)) * u) @ wd
    np.testing.assert_allclose(res["out"], 2 * dense, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- backward

def _fd_layer(T=5, H=6, Hp=4, E=3, K=2, seed=21):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    W = [[rng.standard_normal((H, Hp)) / 2, rng.standard_normal((H, Hp)) / 2, rng.standard_normal((Hp, H)) / 2]
         for _ in range(E)]
    lg = rng.standard_normal((T, E)).astype(np.float32)
    dout = rng.standard_normal((T, H))
    return x, W, lg, dout


def test_backward_matches_finite_differences():
    """Every gradient of layer_backward against central differences of the fp64 forward
    (loss = <dout, out>); routing is held by giving the forward the same top-k ids."""
    T, H, Hp, E, K = 5, 6, 4, 3, 2
    x, W, lg, dout = _fd_layer(T, H, Hp, E, K)
    idx, w = O.route_topk(lg, K)
    fn = lambda e: tuple(W[e])
    g = O.layer_backward(x, E, K, fn, dout, topk_idx=idx, topk_w=w)
    loss = lambda xx, WW, ww: float(np.sum(dout * O.layer(xx, E, K, lambda e: tuple(WW[e]),
                                                            topk_idx=idx, topk_w=ww)["out"]))
    eps = 1e-6
    def fd(f, arr, index):
        a = arr.copy(); a[index] += eps; up = f(a)
        a = arr.copy(); a[index] -= eps; dn = f(a)
        return (up - dn) / (2 * eps)
    rng = np.random.default_rng(0)
    for _ in range(6):
        i = (rng.integers(T), rng.integers(H))
        assert abs(fd(lambda a: loss(a, W, w), x, i) - g["dx"][i]) < 1e-6
        i = (rng.integers(T), rng.integers(K))
        assert abs(fd(lambda a: loss(x, W, a), w, i) - g["dw"][i]) < 1e-6
        for m, key in enumerate(("dWg", "dWu", "dWd")):
            e = int(rng.integers(E))
            shp = W[e][m].shape
            i = (int(rng.integers(shp[0])), int(rng.integers(shp[1])))
            def f(a, e=e, m=m):
                WW = [list(t) for t in W]
                WW[e][m] = a
                return loss(x, WW, w)
            assert abs(fd(f, W[e][m], i) - g[key][e][i]) < 1e-6


def test_backward_logit_gradient_through_topk_softmax():
    T, H, Hp, E, K = 5, 6, 4, 3, 2
    x, W, lg, dout = _fd_layer(T, H, Hp, E, K, seed=22)
    lg64 = lg.astype(np.float64)
    g = O.layer_backward(x, E, K, lambda e: tuple(W[e]), dout, logits=lg)
    idx = g["topk_idx"]
    def loss(l):
        # the same selection, weights from the perturbed logits (softmax over the selected K)
        sel = np.take_along_axis(l, idx.astype(np.int64), axis=1)
        z = np.exp(sel - sel.max(axis=1, keepdims=True))
        ww = z / z.sum(axis=1, keepdims=True)
        return float(np.sum(dout * O.layer(x, E, K, lambda e: tuple(W[e]), topk_idx=idx, topk_w=ww)["out"]))
    eps = 1e-6
    for t in range(T):
        for e in range(E):
            a = lg64.copy(); a[t, e] += eps; up = loss(a)
            a = lg64.copy(); a[t, e] -= eps; dn = loss(a)
            assert abs((up - dn) / (2 * eps) - g["dlogits"][t, e]) < 1e-6
    assert np.allclose(g["dlogits"].sum(axis=1), 0.0, atol=1e-12)   # softmax invariance


# ----------------------------------------------------------------------------- padding, quantisation

def test_padded_offsets_four_rank_example_and_closed_forms():
    ex = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "four_rank_example.json")))
    counts = np.array(ex["counts"])
    # pad 2: each group rounded up to even -> [2,2,0,2,0,2,2,0]
    assert O.padded_offsets(counts, 2).tolist() == [0, 2, 4, 4, 6, 6, 8, 10, 10]
    assert O.padded_offsets(counts, 1).tolist() == ex["cu_seqlens"]
    rng = np.random.default_rng(11)
    c = rng.integers(0, 300, size=37)
    cu = O.padded_offsets(c, 128)
    sizes = np.diff(cu)
    assert np.all(sizes % 128 == 0) and np.all(sizes >= c) and np.all(sizes - c < 128)
    assert np.all((sizes == 0) == (c == 0))


def test_permute_padded_matches_unpadded_within_groups():
    rng = np.random.default_rng(12)
    T, K, E, pad = 50, 3, 7, 8
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    pos, rs = O.permute(idx, E)
    ppos, prs, cu = O.permute_padded(idx, E, pad)
    counts, cu0 = O.count_offsets(idx, E)
    assert len(prs) == T * K + E * (pad - 1)
    for e in range(E):   # same copies, same order, shifted to the padded group start
        assert np.array_equal(prs[cu[e]:cu[e] + counts[e]], rs[cu0[e]:cu0[e + 1]])
        assert np.all(prs[cu[e] + counts[e]:cu[e + 1]] == -1)
    assert np.all(prs[cu[-1]:] == -1)
    flat = np.arange(T * K).reshape(T, K)
    assert np.array_equal(prs[ppos], flat)    # exact inversion


def test_encode_e4m3fn_inverts_decode_for_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(O.encode_e4m3fn(O.decode_e4m3fn(codes)), codes)
    assert O.encode_e4m3fn(np.array([-0.0]))[0] == 0x80
    with pytest.raises(ValueError):
        O.encode_e4m3fn(np.array([0.3]))          # not on the grid


def test_quantize_fp8_matches_requant_and_torch():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((6, 384)) * np.exp2(rng.integers(-8, 8, size=(6, 1)))
    x[2, :128] = 0.0                                   # an all-zero block: scale 1, codes 0
    codes, s = O.quantize_fp8_1x128(x)
    vals, s2 = O.requant_fp8_1x128(x)
    assert np.array_equal(s, s2)
    assert np.array_equal(O.decode_e4m3fn(codes) * np.repeat(s, 128, axis=1), vals)
    assert np.all(codes[2, :128] == 0) and s[2, 0] == 1.0
    # torch's float8_e4m3fn cast of the same exact fp32 quotients gives the same bytes
    q32 = torch.from_numpy((x.astype(np.float32).astype(np.float64) / np.repeat(s, 128, axis=1)).astype(np.float32))
    tb = q32.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(tb, codes)


# ----------------------------------------------------------------------------- formats

def test_e2m1_and_e8m0_tables():
    assert O.decode_e2m1(np.arange(8)).tolist() == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert O.decode_e2m1(np.arange(8, 16)).tolist() == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    assert O.decode_e8m0(np.array([127, 128, 0, 254])).tolist() == [1.0, 2.0, 2.0 ** -127, 2.0 ** 127]
    assert math.isnan(O.decode_e8m0(np.array([255]))[0])


def test_e4m3fn_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert np.isnan(ours).sum() == 2                 # 0x7F and 0xFF
    assert ours[0x7E] == 448.0 and ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9


def test_round_e4m3fn_matches_torch_cast():
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.standard_normal(20000) * 50, rng.standard_normal(5000) * 1e-2,
                        O.decode_e4m3fn(np.arange(0, 0x7F, dtype=np.uint8)),
                        np.array([448.0, -448.0, 0.0, 2.0 ** -10, 3 * 2.0 ** -11])])
    v = v[np.abs(v) <= 448.0].astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(O.round_e4m3fn(v), ref)


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(2)
    t = torch.from_numpy(rng.standard_normal(4096).astype(np.float32)).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.decode_bf16(bits), t.to(torch.float64).numpy())


def test_fp8_block_scale_and_requant_identity_on_grid():
    s = O.fp8_block_scale(np.array([448.0, 449.0, 224.0, 0.0, 1.0, 448.0 * 2 ** -20]))
    assert s.tolist() == [1.0, 2.0, 0.5, 1.0, 2.0 ** -8, 2.0 ** -20]
    # the e8m0 floor: no scale below 2^-127 (byte 0), however small the block
    s = O.fp8_block_scale(np.array([448.0 * 2 ** -127, 448.0 * 2 ** -127 * 1.5, 2.0 ** -130, 2.0 ** -149]))
    assert s.tolist() == [2.0 ** -127, 2.0 ** -126, 2.0 ** -127, 2.0 ** -127]


def test_quantize_fp8_tiny_block_codes():
    """A block far below the e8m0 range keeps the 2^-127 scale; its codes are then the
    values times 2^127, rounded on the e4m3 grid: 2^-130 -> 2^-3 (code 0x20), 2^-137 ->
    2^-10, which rounds to the smallest subnormal 2^-9 only from above half of it (so 0),
    3 * 2^-138 -> 1.5 * 2^-10 (rounds to 2^-9, code 0x01), and -2^-128 -> -0.5 (0xB0)."""
    x = np.zeros((1, 128))
    x[0, :5] = [2.0 ** -130, 2.0 ** -137, 3 * 2.0 ** -138, -2.0 ** -128, 0.0]
    codes, s = O.quantize_fp8_1x128(x)
    assert s.tolist() == [[2.0 ** -127]]
    assert codes[0, :5].tolist() == [0x20, 0x00, 0x01, 0xB0, 0x00]
    assert np.all(codes[0, 5:] == 0)
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 0x7F, size=(3, 256), dtype=np.uint8)
    codes[:, ::128] = 0x7E                          # make each block's amax exactly 448
    vals = O.decode_e4m3fn(codes) * np.where(rng.random((3, 1)) < 0.5, -1, 1) * 2.0 ** -5
    deq, sc = O.requant_fp8_1x128(vals)
    assert np.array_equal(deq, vals)
    assert np.all(sc == 2.0 ** -5)


def test_mxfp4_decode_layout():
    """Build a known 64 x 3 matrix element by element and pack it by hand."""
    Kred, N = 64, 3
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 16, size=(Kred, N))
    sbytes = np.array([[120, 127, 140], [130, 100, 127]], np.uint8)   # [Kred/32, N]
    packed = np.zeros((N, Kred // 2), np.uint8)
    for n in range(N):
        for k in range(Kred):
            packed[n, k // 2] |= np.uint8(codes[k, n] << (4 * (k % 2)))
    W = O.decode_mxfp4(packed, sbytes)
    table = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for k in range(Kred):
        for n in range(N):
            c = int(codes[k, n])
            v = (-1 if c & 8 else 1) * table[c & 7] * 2.0 ** (int(sbytes[k // 32, n]) - 127)
            assert W[k, n] == v
