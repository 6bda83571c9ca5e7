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


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (scale if scale > 0 else 1.0))


def expert_of_rows(cu, rows):
    """Expert (group) of each permuted row: the e with cu[e] <= r < cu[e+1]."""
    return np.searchsorted(np.asarray(cu), np.asarray(rows), side="right") - 1


def oracle_rows(w, jobs, workers=8):
    """The oracle's h and y at selected permuted rows, for several routings of one workload.

    ``jobs`` is a list of (routing, rows): ``routing`` as returned by ``oracle_routing`` (its
    cu_seqlens and row_src place the rows), ``rows`` the permuted row indices wanted. Every
    expert's weights are decoded once for all jobs. bf16 / fp32 weights are decoded in this
    process by an exact cast to float64; MXFP4 experts are decoded by the oracle's own decoder
    in a pool of spawned worker processes. Returns, per job, {row: (h, y, h_scales)}; in the
    fp8 layer h is the requantised value and h_scales its 1x128 block scales, else None."""
    x = x_f64(w)
    fp8 = w.act == "fp8"
    need = {}
    for j, (ref, rows) in enumerate(jobs):
        rows = np.asarray(rows, dtype=np.int64)
        ex = expert_of_rows(ref["cu_seqlens"], rows)
        tok = np.asarray(ref["row_src"])[rows] // w.K
        for r, e, t in zip(rows.tolist(), ex.tolist(), tok.tolist()):
            need.setdefault(e, []).append((j, r, t))
    res = [dict() for _ in jobs]

    def store(e, h, y, hs=None):
        for i, (j, r, _) in enumerate(need[e]):
            res[j][r] = (h[i], y[i], None if hs is None else hs[i])

    if w.wgt != "mxfp4":
        import torch

        def dec(t):   # bf16 -> float64 is exact; the cast equals O.decode_bf16 (pinned)
            return t.detach().cpu().to(torch.float64).numpy()
        for e in sorted(need):
            wg, wu, wd = dec(w.w_gate[e]), dec(w.w_up[e]), dec(w.w_down[e])
            h, y = O.expert_ffn(x[[t for _, _, t in need[e]]], wg, wu, wd, fp8_requant=fp8)
            store(e, h, y)
        return res

    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor

    from _oracle_pool import mxfp4_expert_rows
    experts = sorted(need)
    ctx = multiprocessing.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        for i0 in range(0, len(experts), 4 * workers):      # bounded number of pending jobs
            futs = []
            for e in experts[i0:i0 + 4 * workers]:
                packed = tuple(to_numpy_bits(t[e]) for t in (w.w_gate, w.w_up, w.w_down))
                scales = tuple(to_numpy_bits(t[e]) for t in (w.sf_gate, w.sf_up, w.sf_down))
                xr = x[[t for _, _, t in need[e]]]
                futs.append(ex.submit(mxfp4_expert_rows, (e, xr, packed, scales, fp8)))
            for f in futs:
                store(*f.result(timeout=900))   # a broken pool raises instead of waiting forever
    return res
