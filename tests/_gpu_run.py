"""Run the MoE layer through the C ABI, one entry point at a time (GPU tests only)."""
import torch

import mixture_experts_layer_counting_amd as moe

DT = {"f32": moe.MOE_F32, "bf16": moe.MOE_BF16, "fp8": moe.MOE_FP8_E4M3, "mxfp4": moe.MOE_MXFP4,
      "mxfp4_paired": moe.MOE_MXFP4_PAIRED}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}


def h_fmt(w):
    return "fp8" if w.act == "fp8" else w.act


def y_fmt(w):
    return "f32" if w.act == "f32" else "bf16"


def run_steps(w, with_row_w=True):
    """route -> permute -> gate/up -> down -> combine on the workload's device tensors."""
    dev = w.x.device
    T, H, Hp, E, K = w.T, w.H, w.Hp, w.E, w.K
    M = T * K
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    r = {}
    if w.logits is not None:
        r["topk_idx"] = torch.empty((T, K), **i32)
        r["topk_w"] = torch.empty((T, K), **f32)
        moe.moe_route_topk(w.logits, T, E, K, r["topk_idx"], r["topk_w"])
    else:
        r["topk_idx"], r["topk_w"] = w.topk_idx, w.topk_w
    r["counts"] = torch.empty(E, **i32)
    r["cu_seqlens"] = torch.empty(E + 1, **i32)
    r["pos"] = torch.empty((T, K), **i32)
    r["row_src"] = torch.empty(M, **i32)
    r["row_w"] = torch.empty(M, **f32) if with_row_w else None
    r["x_perm"] = torch.empty((M, H), dtype=TORCH_DT[w.act], device=dev)
    r["x_perm_sf"] = torch.empty((H // 128, M), **f32) if w.act == "fp8" else None
    nws = moe.moe_permute_workspace_bytes(T, E, K)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    moe.moe_permute(w.x, w.x_sf, DT[w.act], r["topk_idx"], r["topk_w"], T, H, E, K, r["counts"],
                    r["cu_seqlens"], r["pos"], r["row_src"], r["row_w"], r["x_perm"], r["x_perm_sf"],
                    ws, nws)
    r["h"] = torch.empty((M, Hp), dtype=TORCH_DT[h_fmt(w)], device=dev)
    r["h_sf"] = torch.empty((Hp // 128, M), **f32) if w.act == "fp8" else None
    moe.moe_ffn_gate_up(r["x_perm"], r["x_perm_sf"], DT[w.act], r["cu_seqlens"], M, E, H, Hp,
                        w.w_gate, w.w_up, w.sf_gate, w.sf_up, DT[w.wgt], r["h"], r["h_sf"])
    r["y_rows"] = torch.empty((M, H), dtype=TORCH_DT[y_fmt(w)], device=dev)
    moe.moe_ffn_down(r["h"], r["h_sf"], DT[h_fmt(w)], r["cu_seqlens"], M, E, H, Hp, w.w_down,
                     w.sf_down, DT[w.wgt], r["y_rows"], DT[y_fmt(w)])
    r["out"] = torch.empty((T, H), dtype=TORCH_DT[w.out], device=dev)
    moe.moe_combine(r["y_rows"], DT[y_fmt(w)], r["pos"], r["topk_w"], T, H, K, r["out"], DT[w.out])
    return r


def paired(w):
    """The workload with its MXFP4 weight codes repacked by moe_pack_mxfp4_pairs into the
    MOE_MXFP4_PAIRED layout (gate/up: N = Hp output columns over K = H; down: N = H over
    K = Hp). The scale tensors are shared: they keep their layout."""
    import dataclasses
    assert w.wgt == "mxfp4"

    def pack(t, N, K):
        out = torch.empty_like(t)
        moe.moe_pack_mxfp4_pairs(t, out, w.E, N, K)
        return out
    return dataclasses.replace(w, wgt="mxfp4_paired", w_gate=pack(w.w_gate, w.Hp, w.H),
                               w_up=pack(w.w_up, w.Hp, w.H), w_down=pack(w.w_down, w.H, w.Hp))


def layer_desc(w, combine=moe.MOE_COMBINE_GATHER):
    return moe.LayerDesc(w.T, w.H, w.Hp, w.E, w.K, DT[w.act], DT[w.wgt], DT[w.out], combine)


def run_layer(w, combine=moe.MOE_COMBINE_GATHER):
    """The fused entry point; returns (out, workspace tensor, layout dict)."""
    d = layer_desc(w, combine)
    nbytes = moe.moe_layer_workspace_bytes(d)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=w.x.device)
    out = torch.empty((w.T, w.H), dtype=TORCH_DT[w.out], device=w.x.device)
    moe.moe_layer_forward(d, w.x, w.x_sf, w.logits, w.topk_idx, w.topk_w, w.w_gate, w.w_up,
                          w.w_down, w.sf_gate, w.sf_up, w.sf_down, out, ws, nbytes)
    return out, ws, moe.moe_layer_workspace_layout(d)


def run_layer_shared(w, combine=moe.MOE_COMBINE_GATHER, side_stream=None):
    """moe_layer_forward_shared; returns (out, workspace tensor)."""
    d = layer_desc(w, combine)
    nbytes = moe.moe_layer_shared_workspace_bytes(d, w.Hs)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=w.x.device)
    out = torch.empty((w.T, w.H), dtype=TORCH_DT[w.out], device=w.x.device)
    moe.moe_layer_forward_shared(d, w.Hs, w.x, w.x_sf, w.x_shared, w.logits, w.topk_idx, w.topk_w,
                                 w.w_gate, w.w_up, w.w_down, w.sf_gate, w.sf_up, w.sf_down,
                                 w.ws_gate, w.ws_up, w.ws_down, out, ws, nbytes,
                                 side_stream=side_stream)
    return out, ws


def run_fused(w, row_src, cu_seqlens, ws=None):
    """moe_grouped_ffn_fused (bf16) on the permutation of run_steps: returns (y_rows, h,
    control words as a host int64 array, workspace). ``ws`` may be given to reuse one."""
    dev = w.x.device
    M = w.T * w.K
    nbytes = moe.moe_grouped_ffn_fused_workspace_bytes(M, w.E, w.Hp)
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    y = torch.empty((M, w.H), dtype=torch.bfloat16, device=dev)
    moe.moe_grouped_ffn_fused(w.x, DT[w.act], row_src, w.T, w.K, cu_seqlens, M, w.E, w.H, w.Hp, w.w_gate,
                              w.w_up, w.w_down, DT[w.wgt], y, DT["bf16"], ws, nbytes)
    h_bytes = M * w.Hp * 2
    ctl_off = (h_bytes + 255) // 256 * 256
    h = ws[:h_bytes].view(torch.bfloat16).view(M, w.Hp)
    ctl = ws[ctl_off:ctl_off + 16 * 4].view(torch.int32)
    return y, h, ctl, ws


def fused_tile_count(counts, H, Hp):
    """Tiles of the single-launch FFN: per expert ceil(rows / 256) m-tiles, each with Hp/128
    gate/up and H/256 down tiles."""
    mt = sum((int(c) + 255) // 256 for c in counts)
    return mt * (Hp // 128 + H // 256)
