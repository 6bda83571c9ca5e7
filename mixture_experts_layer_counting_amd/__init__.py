"""Python binding of the MI355X MoE-layer C ABI (``include/moe.h``).

Argument marshalling only: every function here forwards to the function of the same name
in ``libmoe_mi355x.so`` (built by ``python -m mixture_experts_layer_counting_amd.build``)
and raises :class:`MoeError` on a non-OK status. Buffers may be passed as torch tensors
(their ``data_ptr()`` is used), raw integer addresses, or ``None`` for NULL. ``stream``
defaults to torch's current stream. There is no fallback: without the built library
every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

# moe_status_t
MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = range(5)
# moe_dtype_t
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4, MOE_MXFP4_PAIRED = range(5)
# moe_combine_t
MOE_COMBINE_GATHER, MOE_COMBINE_SCATTER_ATOMIC = range(2)

# offsets reported by moe_layer_workspace_layout, in order
WS_FIELDS = ("topk_idx", "topk_w", "counts", "cu_seqlens", "pos", "row_src", "row_w", "x_perm",
             "x_perm_sf", "h", "h_sf", "y_rows", "permute_scratch", "acc_f32", "x_q", "x_q_sf",
             "fused_ctl")

EXPORTS = ("moe_route_topk", "moe_permute_workspace_bytes", "moe_permute", "moe_permute_noalloc",
           "moe_padded_capacity",
           "moe_permute_padded", "moe_route_permute", "moe_quantize_fp8", "moe_pack_mxfp4_pairs", "moe_ffn_gate_up",
           "moe_ffn_gate_up_gather", "moe_ffn_down", "moe_ffn_down_scatter",
           "moe_grouped_ffn_workspace_bytes", "moe_grouped_ffn",
           "moe_grouped_ffn_fused_workspace_bytes", "moe_grouped_ffn_fused",
           "moe_grouped_ffn_fused_scatter", "moe_combine",
           "moe_combine_shared", "moe_layer_workspace_bytes", "moe_layer_forward",
           "moe_layer_shared_workspace_bytes", "moe_layer_forward_shared", "moe_layer_workspace_layout",
           "moe_layer_backward_workspace_bytes", "moe_layer_backward",
           "moe_status_str")


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


class LayerDesc(ctypes.Structure):
    """moe_layer_desc_t."""
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("Hp", ctypes.c_int32),
                ("E", ctypes.c_int32), ("K", ctypes.c_int32), ("act", ctypes.c_int),
                ("wgt", ctypes.c_int), ("out", ctypes.c_int), ("combine", ctypes.c_int)]


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_I = ctypes.c_int32
_E = ctypes.c_int
_S = ctypes.c_size_t

_SIGS = {
    "moe_route_topk": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "moe_permute_workspace_bytes": (_S, [_I, _I, _I]),
    "moe_permute": (_I, [_P, _P, _E, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _S, _P]),
    "moe_permute_noalloc": (_I, [_P, _P, _E, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_ffn_gate_up": (_I, [_P, _P, _E, _P, _I, _I, _I, _I, _P, _P, _P, _P, _E, _P, _P, _P]),
    "moe_padded_capacity": (ctypes.c_int64, [_I, _I, _I, _I]),
    "moe_permute_padded": (_I, [_P, _P, _E, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P,
                                _P, _S, _P]),
    "moe_route_permute": (_I, [_P, _P, _P, _E, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                               _P, _P, _S, _P]),
    "moe_quantize_fp8": (_I, [_P, _E, _I, _I, _P, _P, _P]),
    "moe_pack_mxfp4_pairs": (_I, [_P, _P, _I, _I, _I, _P]),
    "moe_ffn_gate_up_gather": (_I, [_P, _P, _P, _E, _P, _I, _I, _P, _I, _I, _I, _I, _P, _P, _P, _P, _E,
                                    _P, _P, _P]),
    "moe_ffn_down_scatter": (_I, [_P, _P, _E, _P, _I, _I, _I, _I, _P, _P, _E, _P, _P, _I, _I, _P,
                                  _P]),
    "moe_ffn_down": (_I, [_P, _P, _E, _P, _I, _I, _I, _I, _P, _P, _E, _P, _E, _P]),
    "moe_grouped_ffn_workspace_bytes": (_S, [_I, _I, _E, _E]),
    "moe_grouped_ffn": (_I, [_P, _P, _E, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _E, _P, _E,
                             _P, _S, _P]),
    "moe_grouped_ffn_fused_workspace_bytes": (_S, [_I, _I, _I]),
    "moe_grouped_ffn_fused": (_I, [_P, _E, _P, _I, _I, _P, _I, _I, _I, _I, _P, _P, _P, _E, _P, _E, _P,
                                   _S, _P]),
    "moe_grouped_ffn_fused_scatter": (_I, [_P, _E, _P, _I, _I, _P, _I, _I, _I, _I, _P, _P, _P, _E, _P,
                                           _P, _P, _S, _P]),
    "moe_combine": (_I, [_P, _E, _P, _P, _I, _I, _I, _P, _E, _P]),
    "moe_layer_workspace_bytes": (_S, [ctypes.POINTER(LayerDesc)]),
    "moe_layer_forward": (_I, [ctypes.POINTER(LayerDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                               _P, _P, _P, _S, _P]),
    "moe_layer_workspace_layout": (_I, [ctypes.POINTER(LayerDesc), ctypes.POINTER(_S), _I]),
    "moe_combine_shared": (_I, [_P, _E, _P, _P, _I, _I, _I, _P, _P, _E, _P]),
    "moe_layer_backward_workspace_bytes": (_S, [ctypes.POINTER(LayerDesc)]),
    "moe_layer_backward": (_I, [ctypes.POINTER(LayerDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                _P, _P, _P, _S, _P]),
    "moe_layer_shared_workspace_bytes": (_S, [ctypes.POINTER(LayerDesc), _I]),
    "moe_layer_forward_shared": (_I, [ctypes.POINTER(LayerDesc), _I, _P, _P, _P, _P, _P, _P, _P, _P,
                                      _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _P, _P]),
    "moe_status_str": (ctypes.c_char_p, [_I]),
}


def lib() -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} missing "
                               "(run `python -m mixture_experts_layer_counting_amd.build`)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_str(status: int) -> str:
    try:
        return lib().moe_status_str(status).decode()
    except Exception:  # the library itself is unavailable
        return f"status {status}"


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)


def moe_route_topk(logits, T, E, K, topk_idx, topk_w, stream=None):
    _check(lib().moe_route_topk(_ptr(logits), T, E, K, _ptr(topk_idx), _ptr(topk_w),
                                _stream(stream)), "moe_route_topk")


def moe_permute_workspace_bytes(T, E, K) -> int:
    return int(lib().moe_permute_workspace_bytes(T, E, K))


def moe_permute(x, x_sf, act, topk_idx, topk_w, T, H, E, K, counts, cu_seqlens, pos, row_src,
                row_w, x_perm, x_perm_sf, ws, ws_bytes, stream=None):
    _check(lib().moe_permute(_ptr(x), _ptr(x_sf), act, _ptr(topk_idx), _ptr(topk_w), T, H, E, K,
                             _ptr(counts), _ptr(cu_seqlens), _ptr(pos), _ptr(row_src), _ptr(row_w),
                             _ptr(x_perm), _ptr(x_perm_sf), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_permute")


def moe_permute_noalloc(x, x_sf, act, topk_idx, topk_w, T, H, E, K, counts, cu_seqlens, pos, row_src,
                        row_w, x_perm, x_perm_sf, stream=None):
    _check(lib().moe_permute_noalloc(_ptr(x), _ptr(x_sf), act, _ptr(topk_idx), _ptr(topk_w), T, H, E, K,
                                     _ptr(counts), _ptr(cu_seqlens), _ptr(pos), _ptr(row_src), _ptr(row_w),
                                     _ptr(x_perm), _ptr(x_perm_sf), _stream(stream)),
           "moe_permute_noalloc")


def moe_padded_capacity(T, E, K, pad) -> int:
    return int(lib().moe_padded_capacity(T, E, K, pad))


def moe_permute_padded(x, x_sf, act, topk_idx, topk_w, T, H, E, K, pad, counts, cu_seqlens, pos,
                       row_src, row_w, x_perm, x_perm_sf, ws, ws_bytes, stream=None):
    _check(lib().moe_permute_padded(_ptr(x), _ptr(x_sf), act, _ptr(topk_idx), _ptr(topk_w), T, H, E,
                                    K, pad, _ptr(counts), _ptr(cu_seqlens), _ptr(pos), _ptr(row_src),
                                    _ptr(row_w), _ptr(x_perm), _ptr(x_perm_sf), _ptr(ws), ws_bytes,
                                    _stream(stream)), "moe_permute_padded")


def moe_route_permute(logits, x, x_sf, act, T, H, E, K, pad, topk_idx, topk_w, counts, cu_seqlens,
                      pos, row_src, row_w, x_perm, x_perm_sf, ws, ws_bytes, stream=None):
    _check(lib().moe_route_permute(_ptr(logits), _ptr(x), _ptr(x_sf), act, T, H, E, K, pad,
                                   _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(cu_seqlens),
                                   _ptr(pos), _ptr(row_src), _ptr(row_w), _ptr(x_perm),
                                   _ptr(x_perm_sf), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_route_permute")


def moe_quantize_fp8(x, x_dtype, R, C, q, sf, stream=None):
    _check(lib().moe_quantize_fp8(_ptr(x), x_dtype, R, C, _ptr(q), _ptr(sf), _stream(stream)),
           "moe_quantize_fp8")


def moe_pack_mxfp4_pairs(w, w_paired, E, N, K, stream=None):
    _check(lib().moe_pack_mxfp4_pairs(_ptr(w), _ptr(w_paired), E, N, K, _stream(stream)),
           "moe_pack_mxfp4_pairs")


def moe_ffn_gate_up(x_perm, x_perm_sf, act, cu_seqlens, M, E, H, Hp, w_gate, w_up, sf_gate, sf_up,
                    wgt, h, h_sf, stream=None):
    _check(lib().moe_ffn_gate_up(_ptr(x_perm), _ptr(x_perm_sf), act, _ptr(cu_seqlens), M, E, H, Hp,
                                 _ptr(w_gate), _ptr(w_up), _ptr(sf_gate), _ptr(sf_up), wgt, _ptr(h),
                                 _ptr(h_sf), _stream(stream)), "moe_ffn_gate_up")


def moe_ffn_gate_up_gather(x, x_sf, x_perm_sf, act, row_src, T, K, cu_seqlens, M, E, H, Hp, w_gate,
                           w_up, sf_gate, sf_up, wgt, h, h_sf, stream=None):
    _check(lib().moe_ffn_gate_up_gather(_ptr(x), _ptr(x_sf), _ptr(x_perm_sf), act, _ptr(row_src), T, K,
                                        _ptr(cu_seqlens), M, E, H, Hp, _ptr(w_gate), _ptr(w_up),
                                        _ptr(sf_gate), _ptr(sf_up), wgt, _ptr(h), _ptr(h_sf),
                                        _stream(stream)), "moe_ffn_gate_up_gather")


def moe_ffn_down_scatter(h, h_sf, h_dtype, cu_seqlens, M, E, H, Hp, w_down, sf_down, wgt, row_src,
                         row_w, T, K, acc, stream=None):
    _check(lib().moe_ffn_down_scatter(_ptr(h), _ptr(h_sf), h_dtype, _ptr(cu_seqlens), M, E, H, Hp,
                                      _ptr(w_down), _ptr(sf_down), wgt, _ptr(row_src), _ptr(row_w),
                                      T, K, _ptr(acc), _stream(stream)), "moe_ffn_down_scatter")


def moe_ffn_down(h, h_sf, h_dtype, cu_seqlens, M, E, H, Hp, w_down, sf_down, wgt, y_rows, out,
                 stream=None):
    _check(lib().moe_ffn_down(_ptr(h), _ptr(h_sf), h_dtype, _ptr(cu_seqlens), M, E, H, Hp,
                              _ptr(w_down), _ptr(sf_down), wgt, _ptr(y_rows), out, _stream(stream)),
           "moe_ffn_down")


def moe_grouped_ffn_workspace_bytes(M, Hp, act, wgt) -> int:
    return int(lib().moe_grouped_ffn_workspace_bytes(M, Hp, act, wgt))


def moe_grouped_ffn(x_perm, x_perm_sf, act, cu_seqlens, M, E, H, Hp, w_gate, w_up, w_down, sf_gate,
                    sf_up, sf_down, wgt, y_rows, out, ws, ws_bytes, stream=None):
    _check(lib().moe_grouped_ffn(_ptr(x_perm), _ptr(x_perm_sf), act, _ptr(cu_seqlens), M, E, H, Hp,
                                 _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(sf_gate), _ptr(sf_up),
                                 _ptr(sf_down), wgt, _ptr(y_rows), out, _ptr(ws), ws_bytes,
                                 _stream(stream)), "moe_grouped_ffn")


def moe_grouped_ffn_fused_workspace_bytes(M, E, Hp) -> int:
    return int(lib().moe_grouped_ffn_fused_workspace_bytes(M, E, Hp))


def moe_grouped_ffn_fused(x, act, row_src, T, K, cu_seqlens, M, E, H, Hp, w_gate, w_up, w_down, wgt,
                          y_rows, out, ws, ws_bytes, stream=None):
    _check(lib().moe_grouped_ffn_fused(_ptr(x), act, _ptr(row_src), T, K, _ptr(cu_seqlens), M, E, H, Hp,
                                       _ptr(w_gate), _ptr(w_up), _ptr(w_down), wgt, _ptr(y_rows), out,
                                       _ptr(ws), ws_bytes, _stream(stream)), "moe_grouped_ffn_fused")


def moe_grouped_ffn_fused_scatter(x, act, row_src, T, K, cu_seqlens, M, E, H, Hp, w_gate, w_up, w_down,
                                  wgt, row_w, acc, ws, ws_bytes, stream=None):
    _check(lib().moe_grouped_ffn_fused_scatter(_ptr(x), act, _ptr(row_src), T, K, _ptr(cu_seqlens), M, E,
                                               H, Hp, _ptr(w_gate), _ptr(w_up), _ptr(w_down), wgt,
                                               _ptr(row_w), _ptr(acc), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_grouped_ffn_fused_scatter")


def moe_combine(y_rows, y_dtype, pos, topk_w, T, H, K, out, out_dtype, stream=None):
    _check(lib().moe_combine(_ptr(y_rows), y_dtype, _ptr(pos), _ptr(topk_w), T, H, K, _ptr(out),
                             out_dtype, _stream(stream)), "moe_combine")


def moe_layer_workspace_bytes(desc: LayerDesc) -> int:
    return int(lib().moe_layer_workspace_bytes(ctypes.byref(desc)))


def moe_layer_workspace_layout(desc: LayerDesc) -> dict:
    arr = (ctypes.c_size_t * len(WS_FIELDS))()
    _check(lib().moe_layer_workspace_layout(ctypes.byref(desc), arr, len(WS_FIELDS)),
           "moe_layer_workspace_layout")
    none = (1 << (8 * ctypes.sizeof(ctypes.c_size_t))) - 1
    return {k: (None if v == none else int(v)) for k, v in zip(WS_FIELDS, arr)}


def moe_layer_forward(desc: LayerDesc, x, x_sf, logits, topk_idx_in, topk_w_in, w_gate, w_up,
                      w_down, sf_gate, sf_up, sf_down, out, ws, ws_bytes, stream=None):
    _check(lib().moe_layer_forward(ctypes.byref(desc), _ptr(x), _ptr(x_sf), _ptr(logits),
                                   _ptr(topk_idx_in), _ptr(topk_w_in), _ptr(w_gate), _ptr(w_up),
                                   _ptr(w_down), _ptr(sf_gate), _ptr(sf_up), _ptr(sf_down),
                                   _ptr(out), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_layer_forward")


def moe_combine_shared(y_rows, y_dtype, pos, topk_w, T, H, K, shared_y, out, out_dtype, stream=None):
    _check(lib().moe_combine_shared(_ptr(y_rows), y_dtype, _ptr(pos), _ptr(topk_w), T, H, K,
                                    _ptr(shared_y), _ptr(out), out_dtype, _stream(stream)),
           "moe_combine_shared")


def moe_layer_shared_workspace_bytes(desc: LayerDesc, Hs) -> int:
    return int(lib().moe_layer_shared_workspace_bytes(ctypes.byref(desc), Hs))


def moe_layer_forward_shared(desc: LayerDesc, Hs, x, x_sf, x_shared, logits, topk_idx_in, topk_w_in,
                             w_gate, w_up, w_down, sf_gate, sf_up, sf_down, ws_gate, ws_up, ws_down,
                             out, ws, ws_bytes, stream=None, side_stream=None):
    """``side_stream``: a torch stream (or raw handle) for the shared expert, or None to run
    it on ``stream``."""
    side = None if side_stream is None else (side_stream.cuda_stream if hasattr(side_stream, "cuda_stream")
                                             else side_stream)
    _check(lib().moe_layer_forward_shared(ctypes.byref(desc), Hs, _ptr(x), _ptr(x_sf), _ptr(x_shared),
                                          _ptr(logits), _ptr(topk_idx_in), _ptr(topk_w_in), _ptr(w_gate),
                                          _ptr(w_up), _ptr(w_down), _ptr(sf_gate), _ptr(sf_up),
                                          _ptr(sf_down), _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down),
                                          _ptr(out), _ptr(ws), ws_bytes, _stream(stream), side),
           "moe_layer_forward_shared")


def moe_layer_backward_workspace_bytes(desc: LayerDesc) -> int:
    return int(lib().moe_layer_backward_workspace_bytes(ctypes.byref(desc)))


def moe_layer_backward(desc: LayerDesc, x, logits, topk_idx_in, topk_w_in, w_gate, w_up, w_down, dout,
                       dx, dw_gate, dw_up, dw_down, d_topk_w, d_logits, ws, ws_bytes, stream=None):
    _check(lib().moe_layer_backward(ctypes.byref(desc), _ptr(x), _ptr(logits), _ptr(topk_idx_in),
                                    _ptr(topk_w_in), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(dout),
                                    _ptr(dx), _ptr(dw_gate), _ptr(dw_up), _ptr(dw_down), _ptr(d_topk_w),
                                    _ptr(d_logits), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_layer_backward")
