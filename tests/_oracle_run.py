"""Oracle-side helpers for the tests: decode a workload's stored bits and run the oracle."""
import numpy as np

from oracle import moe_oracle as O
from workloads import to_numpy_bits


def host_bits(w):
    b = dict(x=to_numpy_bits(w.x), x_sf=to_numpy_bits(w.x_sf), logits=to_numpy_bits(w.logits),
             topk_idx=to_numpy_bits(w.topk_idx), topk_w=to_numpy_bits(w.topk_w))
    return b


def weight_fn(w):
    """Per-expert fp64 weights, copying only expert e's bits from wherever they live."""
    if w.wgt == "mxfp4":
        def fn(e):
            return (O.decode_mxfp4(to_numpy_bits(w.w_gate[e]), to_numpy_bits(w.sf_gate[e])),
                    O.decode_mxfp4(to_numpy_bits(w.w_up[e]), to_numpy_bits(w.sf_up[e])),
                    O.decode_mxfp4(to_numpy_bits(w.w_down[e]), to_numpy_bits(w.sf_down[e])))
        return fn

    def dec(t):
        bits = to_numpy_bits(t)
        return np.asarray(bits, np.float64) if w.wgt == "f32" else O.decode_bf16(bits)

    def fn(e):
        return dec(w.w_gate[e]), dec(w.w_up[e]), dec(w.w_down[e])
    return fn


def x_f64(w, b=None):
    b = b or host_bits(w)
    return O.decode_activations(b["x"], w.act, b["x_sf"])


def oracle_layer(w, experts=None):
    b = host_bits(w)
    return O.layer(x_f64(w, b), w.E, w.K, weight_fn(w), logits=b["logits"], topk_idx=b["topk_idx"],
                   topk_w=b["topk_w"], fp8_requant=(w.act == "fp8"), experts=experts)


def shared_weights_f64(w):
    def dec(t):
        bits = to_numpy_bits(t)
        return np.asarray(bits, np.float64) if bits.dtype == np.float32 else O.decode_bf16(bits)
    return dec(w.ws_gate), dec(w.ws_up), dec(w.ws_down)


def shared_input_f64(w, b=None):
    """The activations the shared expert reads: x_shared (bf16) for an fp8 layer, else x."""
    if w.x_shared is not None:
        return O.decode_bf16(to_numpy_bits(w.x_shared))
    return x_f64(w, b)


def oracle_layer_shared(w):
    b = host_bits(w)
    return O.layer_with_shared(x_f64(w, b), shared_input_f64(w, b), w.E, w.K, weight_fn(w),
                               shared_weights_f64(w), logits=b["logits"], topk_idx=b["topk_idx"],
                               topk_w=b["topk_w"], fp8_requant=(w.act == "fp8"))


def oracle_routing(w):
    """Integer results only (routing, counts, offsets, permutation)."""
    b = host_bits(w)
    if b["logits"] is not None:
        idx, wts = O.route_topk(b["logits"], w.K)
    else:
        idx, wts = b["topk_idx"], np.asarray(b["topk_w"], np.float64)
    counts, cu = O.count_offsets(idx, w.E)
    pos, row_src = O.permute(idx, w.E)
    return dict(topk_idx=idx, topk_w=wts, counts=counts, cu_seqlens=cu, pos=pos, row_src=row_src)


def oracle_tokens(w, tokens, routing):
    """out[t] for selected tokens via the direct expert loop, one expert at a time."""
    b = host_bits(w)
    x = x_f64(w, b)
    idx, wts = routing["topk_idx"], routing["topk_w"]
    need = {}
    for t in tokens:
        for k in range(w.K):
            need.setdefault(int(idx[t, k]), []).append((t, k))
    fn = weight_fn(w)
    out = {t: np.zeros(w.H) for t in tokens}
    for e, uses in need.items():
        wg, wu, wd = fn(e)
        rows = np.stack([x[t] for t, _ in uses])
        _, y = O.expert_ffn(rows, wg, wu, wd, fp8_requant=(w.act == "fp8"))
        for (t, k), yr in zip(uses, y):
            out[t] += float(wts[t, k]) * yr
    return out


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (scale if scale > 0 else 1.0))
