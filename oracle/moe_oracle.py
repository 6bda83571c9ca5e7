"""Plain, slow CPU oracle of the MoE layer hot path (numpy, float64).

TEST INFRASTRUCTURE ONLY. Nothing in the library calls this module; only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may use it.
It shares no code, tables or constants with the HIP library.

What it computes, with the passage each step follows:

* Routing -- "Mixture of Kittens" article, Step 1 "The Math": each token picks its
  top-k experts and the routed outputs are summed with router weights; "Distributed
  expert parallelism", "The dispatch-compute-combine lifecycle" item 1 (each token
  selects k expert ids). Weights are the softmax restricted to the selected k (equal to
  the full softmax renormalised over the top k). Selection compares fp32 logits, larger
  first, ties to the lower expert id.
* Counts and offsets -- "Distributed expert parallelism", "Token permutation and
  metadata" (per-local-expert token counts); MoonEP README, "API walkthrough /
  dispatch fwd" (``tokens_per_expert``, ``cu_seqlens``). Here ``cu_seqlens`` has E+1
  entries with a leading 0.
* Permutation -- "Distributed expert parallelism", lifecycle items 2-3 and "Token
  permutation and metadata": copy each token k times and group the copies by expert.
  Within an expert the copies keep ascending flat index t*K + k (a stable order).
* Expert FFN -- "Mixture of Kittens", Step 1: Expert_i(x) = Down_i(SwiGLU(Up_i x,
  Gate_i x)), read as silu(x.Wg) * (x.Wu) then .Wd, silu(z) = z / (1 + exp(-z)).
* Combine -- "Distributed expert parallelism", lifecycle item 8 and "A four-rank
  example": restore token order, scale by route weights, add the k results.
* maxvio -- MoonEP README, "Performance": max_e(T_e / T_bar) - 1 with
  T_bar = T*K/E.
* Formats -- OCP 8-bit floating point (e4m3fn: bias 7, max 448, no infinities) and OCP
  Microscaling v1.0 (e2m1 elements, e8m0 scales); bf16 is the top half of an fp32.

Floating point is float64 throughout; inputs are decoded exactly from the stored bits.
The one low-precision decision the layer makes itself -- requantising the SwiGLU output
to fp8 with 1x128 power-of-two scales in the fp8 x MXFP4 variant -- is taken here on
the fp32-rounded value, the precision the kernel takes it in.
"""
from __future__ import annotations

from typing import Callable, Dict, Optional, Tuple

import numpy as np

# ----------------------------------------------------------------------------- decoders


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact: bf16 is the high half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3fn codes (uint8) -> float64. 1 sign, 4 exponent (bias 7), 3 mantissa
    bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
    return sign * mag


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """OCP e2m1 nibbles (0..15) -> float64. 1 sign, 2 exponent (bias 1), 1 mantissa bit;
    exponent 0 is subnormal (m * 0.5)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c >> 3, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return sign * mag


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    """OCP e8m0 scale bytes -> float64 2^(b-127); 0xFF is NaN."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    return np.where(b == 255, np.nan, np.exp2(b - 127.0))


def decode_mxfp4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """One expert's MXFP4 matrix stored reduction-contiguous -> logical float64 W[k, n].

    ``packed`` [N, Kred/2]: byte j of row n holds k=2j (low nibble), k=2j+1 (high).
    ``scales`` [Kred/32, N]: byte [b][n] scales k in [32b, 32b+32) of column n.
    """
    packed = np.asarray(packed, dtype=np.uint8)
    N, half = packed.shape
    # the two elements of every possible byte: (low nibble, high nibble)
    byte_vals = np.stack([decode_e2m1(np.arange(256) & 0xF), decode_e2m1(np.arange(256) >> 4)], axis=1)
    vals = byte_vals[packed].reshape(N, 2 * half)          # [n, k]: k = 2j low, 2j+1 high
    vals *= np.repeat(decode_e8m0(np.asarray(scales).T), 32, axis=1)
    return vals.T


def decode_fp8_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """e4m3fn rows [R, C] with fp32 1x128 block scales [R, C/128] -> float64 [R, C]."""
    return decode_e4m3fn(codes) * np.repeat(np.asarray(scales, np.float64), 128, axis=1)


# ----------------------------------------------------------------------------- fp8 requant


def round_e4m3fn(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest e4m3fn value, ties to even, saturating at
    +-448. On [2^p, 2^(p+1)) the spacing is 2^(p-3) for p >= -6; below 2^-6
    (subnormals) it is 2^-9."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        p = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # log2 can be off by one ulp near powers of two: correct p so 2^p <= a < 2^(p+1)
    p = np.where(np.exp2(p) > a, p - 1, p)
    p = np.where(np.exp2(p + 1) <= a, p + 1, p)
    quantum = np.exp2(np.maximum(p, -6.0) - 3.0)
    q = np.round(a / quantum) * quantum        # numpy rounds half to even
    q = np.minimum(q, 448.0)
    return np.where(a > 0, np.sign(v) * q, 0.0)


def fp8_block_scale(amax: np.ndarray) -> np.ndarray:
    """Smallest power of two s with 448*s >= amax, but never below 2^-127, the smallest
    value an e8m0 scale byte can hold (OCP Microscaling v1.0, scale format E8M0), so that
    every scale is one the block-scaled matrix instructions can take (s = 1 when amax = 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.ones_like(amax)
    nz = amax > 0
    e = np.ceil(np.log2(amax[nz] / 448.0))
    e = np.where(448.0 * np.exp2(e) < amax[nz], e + 1, e)
    e = np.where(448.0 * np.exp2(e - 1) >= amax[nz], e - 1, e)
    out[nz] = np.exp2(np.maximum(e, -127.0))
    return out


def requant_fp8_1x128(h: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Quantise rows of h to e4m3fn with a power-of-two scale per 1x128 block and return
    (dequantised float64 values, scales [R, C/128]). The decision is taken on h rounded
    to fp32."""
    h32 = np.asarray(h, dtype=np.float64).astype(np.float32).astype(np.float64)
    R, C = h32.shape
    blocks = h32.reshape(R, C // 128, 128)
    s = fp8_block_scale(np.abs(blocks).max(axis=2))
    q = round_e4m3fn(blocks / s[:, :, None])
    return (q * s[:, :, None]).reshape(R, C), s


def encode_e4m3fn(v: np.ndarray) -> np.ndarray:
    """e4m3fn values (already on the grid, |v| <= 448) -> codes uint8. The sign bit is the
    value's (so -0.0 -> 0x80); magnitudes >= 2^-6 are normal (exponent field floor(log2|v|)
    + 7, 3 mantissa bits), smaller ones subnormal (mantissa |v| / 2^-9)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    with np.errstate(divide="ignore"):
        p = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    p = np.where(np.exp2(p) > a, p - 1, p)
    p = np.where(np.exp2(p + 1) <= a, p + 1, p)
    normal = a >= 2.0 ** -6
    mant_n = np.round((a / np.exp2(p) - 1.0) * 8).astype(np.int64)
    code_n = ((p.astype(np.int64) + 7) << 3) | mant_n
    code_s = np.round(a / 2.0 ** -9).astype(np.int64)
    code = np.where(normal, code_n, code_s)
    if np.any(code > 0x7E) or np.any(round_e4m3fn(v) != v):
        raise ValueError("value not representable in e4m3fn")
    return (sign | code).astype(np.uint8)


def quantize_fp8_1x128(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Activation quantisation ("Mixture of Kittens", Step 8: activations are quantised
    to fp8 before the GEMMs, with the quantisation fused into dispatch): rows of x [R, C]
    -> (e4m3fn codes uint8 [R, C], power-of-two scales [R, C/128]) by the 1x128 rule of
    ``requant_fp8_1x128`` (decision on the fp32 value)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    R, C = x32.shape
    blocks = x32.reshape(R, C // 128, 128)
    s = fp8_block_scale(np.abs(blocks).max(axis=2))
    q = round_e4m3fn(blocks / s[:, :, None])
    # a block of zeros keeps the signs of its zeros; others round ties to even
    return encode_e4m3fn(q.reshape(R, C)), s


# ----------------------------------------------------------------------------- routing


def route_topk(logits: np.ndarray, K: int) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k routing on fp32 logits [T, E] -> (topk_idx int32 [T, K], topk_w float64).

    Experts are ordered by descending logit, equal logits by ascending id; the weights
    are exp(l_j - l_0) / sum_i exp(l_i - l_0) over the K selected logits.
    """
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    # stable sort on the negated logit keeps equal logits in ascending expert order
    order = np.argsort(-lg, axis=1, kind="stable")[:, :K]
    sel = np.take_along_axis(lg, order, axis=1).astype(np.float64)
    z = np.exp(sel - sel[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w


def count_offsets(topk_idx: np.ndarray, E: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per-expert copy counts [E] and cu_seqlens [E+1] (leading 0, exclusive prefix)."""
    counts = np.zeros(E, dtype=np.int64)
    for e in np.asarray(topk_idx).ravel():
        counts[int(e)] += 1
    cu = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        cu[e + 1] = cu[e] + counts[e]
    return counts, cu


def permute(topk_idx: np.ndarray, E: int) -> Tuple[np.ndarray, np.ndarray]:
    """Counting-sort placement of the T*K token copies into expert-contiguous rows.

    Returns pos [T, K] (row of copy (t, k)) and row_src [T*K] (flat index t*K + k of the
    copy in each row). Copies are visited in ascending flat index, so each expert's rows
    hold its copies in token order.
    """
    idx = np.asarray(topk_idx)
    T, K = idx.shape
    _, cu = count_offsets(idx, E)
    fill = cu[:-1].copy()
    pos = np.empty((T, K), dtype=np.int64)
    row_src = np.empty(T * K, dtype=np.int64)
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            r = fill[e]
            fill[e] += 1
            pos[t, k] = r
            row_src[r] = t * K + k
    return pos, row_src


def padded_offsets(counts: np.ndarray, pad: int) -> np.ndarray:
    """cu_seqlens [E+1] when every expert's group is padded up to a multiple of ``pad``
    rows (MoonEP "API walkthrough": token_padding and a padded cu_seqlens; "Distributed
    expert parallelism", "Static-capacity versus dropless dispatch": groups padded to
    hardware-friendly multiples). The counts themselves stay the real ones."""
    cu = np.zeros(len(counts) + 1, dtype=np.int64)
    for e, c in enumerate(counts):
        cu[e + 1] = cu[e] + (int(c) + pad - 1) // pad * pad
    return cu


def permute_padded(topk_idx: np.ndarray, E: int, pad: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """``permute`` into padded groups: expert e's copies fill rows cu[e] .. cu[e]+counts[e]-1
    (same stable order) and the rest of its group is padding (row_src = -1). Returns
    (pos [T, K], row_src [capacity], cu [E+1]) with capacity = T*K + E*(pad-1), the static
    buffer size that any routing fits."""
    idx = np.asarray(topk_idx)
    T, K = idx.shape
    counts, _ = count_offsets(idx, E)
    cu = padded_offsets(counts, pad)
    fill = cu[:-1].copy()
    pos = np.empty((T, K), dtype=np.int64)
    row_src = np.full(T * K + E * (pad - 1), -1, dtype=np.int64)
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            pos[t, k] = fill[e]
            row_src[fill[e]] = t * K + k
            fill[e] += 1
    return pos, row_src, cu


def maxvio(counts: np.ndarray, T: int, K: int, E: int) -> float:
    """max_e(T_e / T_bar) - 1 with T_bar = T*K/E (0 = perfectly balanced)."""
    tbar = T * K / E
    return float(max(int(c) for c in counts) / tbar - 1.0)


# ----------------------------------------------------------------------------- expert FFN


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def expert_ffn(xr: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
               fp8_requant: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """One expert on rows xr [n, H] (float64) -> (h [n, Hp], y [n, H]).

    h = silu(xr.Wg) * (xr.Wu); with ``fp8_requant`` h is replaced by its e4m3fn 1x128
    requantisation before y = h.Wd.
    """
    g = xr @ wg
    u = xr @ wu
    h = silu(g) * u
    hq = requant_fp8_1x128(h)[0] if fp8_requant else h
    return h, hq @ wd


def combine(y_rows: np.ndarray, pos: np.ndarray, w: np.ndarray) -> np.ndarray:
    """out[t] = sum_k w[t,k] * y_rows[pos[t,k]] (accumulated in k order)."""
    T, K = pos.shape
    out = np.zeros((T, y_rows.shape[1]), dtype=np.float64)
    for k in range(K):
        out += np.asarray(w[:, k], np.float64)[:, None] * y_rows[pos[:, k]]
    return out


# ----------------------------------------------------------------------------- whole layer

WeightFn = Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]


def layer(x: np.ndarray, E: int, K: int, weights: WeightFn, *, logits: Optional[np.ndarray] = None,
          topk_idx: Optional[np.ndarray] = None, topk_w: Optional[np.ndarray] = None,
          fp8_requant: bool = False, experts: Optional[range] = None) -> Dict[str, np.ndarray]:
    """The whole layer, one expert at a time.

    ``x`` [T, H] float64 (already decoded); either ``logits`` [T, E] fp32 or a given
    routing (``topk_idx``, ``topk_w``). ``weights(e)`` returns expert e's logical
    (Wg [H,Hp], Wu [H,Hp], Wd [Hp,H]) in float64. ``experts`` limits the FFN to a
    subset (rows of other experts stay zero), for bounded timing samples.
    """
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    if logits is not None:
        idx, w = route_topk(logits, K)
    else:
        idx, w = np.asarray(topk_idx, np.int32), np.asarray(topk_w, np.float64)
    counts, cu = count_offsets(idx, E)
    pos, row_src = permute(idx, E)
    tok = row_src // K
    y_rows = None
    for e in (experts if experts is not None else range(E)):
        lo, hi = int(cu[e]), int(cu[e + 1])
        if hi == lo:
            continue
        wg, wu, wd = weights(e)
        _, ye = expert_ffn(x[tok[lo:hi]], wg, wu, wd, fp8_requant)
        if y_rows is None:
            y_rows = np.zeros((T * K, ye.shape[1]), dtype=np.float64)
        y_rows[lo:hi] = ye
    if y_rows is None:
        y_rows = np.zeros((T * K, H), dtype=np.float64)
    out = combine(y_rows, pos, w)
    return dict(topk_idx=idx, topk_w=w, counts=counts, cu_seqlens=cu, pos=pos,
                row_src=row_src, row_w=np.asarray(w).ravel()[row_src], y_rows=y_rows,
                out=out, maxvio=maxvio(counts, T, K, E))


def shared_expert(xs: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """The shared expert on every token ("Mixture of Kittens", Step 1, "The Math": the layer
    output is SharedExpert(x) plus the weighted sum of the routed experts; the shared expert
    is an FFN of the same SwiGLU form, applied to all tokens). ``xs`` [T, H] float64 (the
    activations the shared expert reads: bf16 even in a low-precision layer, Step 8), weights
    Ws_gate, Ws_up [H, Hs], Ws_down [Hs, H] float64. No requantisation of its h (bf16 path)."""
    return expert_ffn(xs, wg, wu, wd, False)[1]


def layer_with_shared(x: np.ndarray, xs: np.ndarray, E: int, K: int, weights: WeightFn,
                      shared_weights: Tuple[np.ndarray, np.ndarray, np.ndarray],
                      **kw) -> Dict[str, np.ndarray]:
    """``layer`` plus the shared expert's output added to every token's combined row
    ("Mixture of Kittens", Step 1, "The Math")."""
    res = layer(x, E, K, weights, **kw)
    ys = shared_expert(np.asarray(xs, np.float64), *shared_weights)
    res["y_shared"] = ys
    res["out"] = res["out"] + ys
    return res


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d silu(z) / dz = sigma(z) * (1 + z * (1 - sigma(z)))."""
    sg = 1.0 / (1.0 + np.exp(-z))
    return sg * (1.0 + z * (1.0 - sg))


def layer_backward(x: np.ndarray, E: int, K: int, weights: WeightFn, dout: np.ndarray, *,
                   logits: Optional[np.ndarray] = None, topk_idx: Optional[np.ndarray] = None,
                   topk_w: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Gradients of the layer output ``out`` (see ``layer``) for an upstream gradient
    ``dout`` [T, H], in float64, following the forward steps backwards (MoonEP "API
    walkthrough": combine bwd, the expert GEMMs' dgrad and wgrad, dispatch bwd):

    * combine bwd: dy[r] = w[t,k] * dout[t] for the row r = pos[t,k]; the gradient of a
      routing weight is dw[t,k] = <dout[t], y[pos[t,k]]>;
    * down: dh = dy . Wd^T, dWd[e] = h_e^T . dy_e;
    * SwiGLU: dg = dh * u * silu'(g), du = dh * silu(g);
    * gate/up: dx_rows = dg . Wg^T + du . Wu^T, dWg[e] = x_e^T . dg_e, dWu[e] = x_e^T . du_e;
    * dispatch bwd: dx[t] = sum_k dx_rows[pos[t,k]];
    * routing (logits given): the weights are a softmax over the K selected logits, so
      dlogits[t, e_k] = w_k (dw_k - sum_j w_j dw_j) and 0 for the other experts.

    Returns dx [T, H], dWg/dWu [E, H, Hp], dWd [E, Hp, H], dw [T, K], dlogits [T, E] (when
    logits are given) and the per-row intermediates dy, dh, dg, du, dx_rows."""
    x = np.asarray(x, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    T, H = x.shape
    if logits is not None:
        idx, w = route_topk(logits, K)
    else:
        idx, w = np.asarray(topk_idx, np.int32), np.asarray(topk_w, np.float64)
    counts, cu = count_offsets(idx, E)
    pos, row_src = permute(idx, E)
    tok = row_src // K
    wr = np.asarray(w).ravel()[row_src]
    M = T * K
    dy = wr[:, None] * dout[tok]
    dx_rows = np.zeros((M, H))
    dw = np.zeros((T, K))
    Hp = None
    dWg = dWu = dWd = None
    dh_all = dg_all = du_all = None
    for e in range(E):
        lo, hi = int(cu[e]), int(cu[e + 1])
        wg, wu, wd = weights(e)
        if Hp is None:
            Hp = wg.shape[1]
            dWg, dWu = np.zeros((E, H, Hp)), np.zeros((E, H, Hp))
            dWd = np.zeros((E, Hp, H))
            dh_all, dg_all, du_all = np.zeros((M, Hp)), np.zeros((M, Hp)), np.zeros((M, Hp))
        if hi == lo:
            continue
        xe = x[tok[lo:hi]]
        g, u = xe @ wg, xe @ wu
        h = silu(g) * u
        ye = h @ wd
        # routing-weight gradient of the rows of this expert
        rs = row_src[lo:hi]
        dw[rs // K, rs % K] = np.sum(dout[tok[lo:hi]] * ye, axis=1)
        dye = dy[lo:hi]
        dh = dye @ wd.T
        dWd[e] = h.T @ dye
        dg = dh * u * silu_grad(g)
        du = dh * silu(g)
        dx_rows[lo:hi] = dg @ wg.T + du @ wu.T
        dWg[e] = xe.T @ dg
        dWu[e] = xe.T @ du
        dh_all[lo:hi], dg_all[lo:hi], du_all[lo:hi] = dh, dg, du
    dx = np.zeros((T, H))
    for k in range(K):
        dx += dx_rows[pos[:, k]]
    res = dict(dx=dx, dWg=dWg, dWu=dWu, dWd=dWd, dw=dw, dy=dy, dh=dh_all, dg=dg_all, du=du_all,
               dx_rows=dx_rows, topk_idx=idx, topk_w=w, pos=pos, row_src=row_src, cu_seqlens=cu)
    if logits is not None:
        Et = np.asarray(logits).shape[1]
        dl = np.zeros((T, Et))
        s = np.sum(w * dw, axis=1, keepdims=True)
        np.put_along_axis(dl, idx.astype(np.int64), w * (dw - s), axis=1)
        res["dlogits"] = dl
    return res


def layer_token_loop(x: np.ndarray, idx: np.ndarray, w: np.ndarray, weights: WeightFn,
                     fp8_requant: bool = False) -> np.ndarray:
    """Independent formulation with no permutation at all:
    out[t] = sum_k w[t,k] * Expert_{idx[t,k]}(x[t]) (the direct expert loop asked for by
    "Distributed expert parallelism", Exercises, item 3)."""
    x = np.asarray(x, dtype=np.float64)
    T, K = idx.shape
    out = np.zeros_like(x)
    cache: Dict[int, tuple] = {}
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            if e not in cache:
                cache[e] = weights(e)
            wg, wu, wd = cache[e]
            _, y = expert_ffn(x[t:t + 1], wg, wu, wd, fp8_requant)
            out[t] += float(w[t, k]) * y[0]
    return out


# ----------------------------------------------------------------------------- weight access


def dense_weight_fn(w_gate, w_up, w_down, fmt: str) -> WeightFn:
    """Weight accessor over host bit arrays: fmt 'f32' (float32 arrays) or 'bf16'
    (uint16 arrays) with gate/up [E,H,Hp] and down [E,Hp,H]."""
    def dec(a):
        return np.asarray(a, np.float64) if fmt == "f32" else decode_bf16(a)

    def fn(e):
        return dec(w_gate[e]), dec(w_up[e]), dec(w_down[e])
    return fn


def mxfp4_weight_fn(w_gate, w_up, w_down, sf_gate, sf_up, sf_down) -> WeightFn:
    """Weight accessor over MXFP4 host bytes (layouts as in ``decode_mxfp4``)."""
    def fn(e):
        return (decode_mxfp4(w_gate[e], sf_gate[e]), decode_mxfp4(w_up[e], sf_up[e]),
                decode_mxfp4(w_down[e], sf_down[e]))
    return fn


def decode_activations(x_bits: np.ndarray, act: str, x_sf: Optional[np.ndarray] = None) -> np.ndarray:
    if act == "f32":
        return np.asarray(x_bits, np.float64)
    if act == "bf16":
        return decode_bf16(x_bits)
    if act == "fp8":
        return decode_fp8_rows(x_bits, x_sf)
    raise ValueError(act)


def ffn_flops(M: int, H: int, Hp: int) -> float:
    """Algorithmic FFN work: 2*M*H*Hp for each of gate, up and down."""
    return 6.0 * M * H * Hp

