"""The C-ABI library loads, exports every symbol include/moe.h declares, and rejects bad
arguments on the host before touching the GPU (no compute calls here)."""
import ctypes
import os
import re
import subprocess

import pytest

import mixture_experts_layer_counting_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(moe.LIB_PATH),
                                reason="library not built (run __graft_entry__.build())")


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared()
    for n in ("moe_route_topk", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_layer_forward",
              "moe_layer_workspace_bytes", "moe_status_str"):
        assert n in names
    assert set(names) == set(moe.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    for n in declared():
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (moe_\w+)", out))
    assert exported == set(declared())          # nothing else leaks out of the library


def prototypes():
    """name -> list of parameter declarations, from the MOE_API prototypes of the header."""
    text = re.sub(r"/\*.*?\*/", " ", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(([^)]*)\)\s*;", text):
        params = [q.strip() for q in m.group(2).split(",") if q.strip()]
        out[m.group(1)] = [] if params == ["void"] else params
    return out


def test_binding_signatures_match_the_header():
    # ctypes does not check arity or types: a binding out of step with a prototype would pass
    # the wrong pointer for an argument without any error
    protos = prototypes()
    assert set(protos) == set(moe.EXPORTS)
    for name, params in protos.items():
        restype, argtypes = moe._SIGS[name]
        assert len(argtypes) == len(params), (name, len(argtypes), len(params))
        for decl, ct in zip(params, argtypes):
            if "*" in decl or decl.startswith("hipStream_t"):
                assert ct is ctypes.c_void_p or (isinstance(ct, type) and issubclass(ct, ctypes._Pointer)), (name, decl)
            elif decl.startswith("size_t"):
                assert ct is ctypes.c_size_t, (name, decl)
            else:
                assert ct in (ctypes.c_int32, ctypes.c_int), (name, decl)


def test_status_strings():
    assert moe.status_str(moe.MOE_OK) == "MOE_OK"
    assert "workspace" in moe.status_str(moe.MOE_EWORKSPACE)
    assert moe.status_str(99) == "MOE_UNKNOWN"


def _expect(status, fn, *args):
    with pytest.raises(moe.MoeError) as ei:
        fn(*args)
    assert ei.value.status == status


def test_route_argument_checks():
    f = moe.moe_route_topk
    _expect(moe.MOE_EINVAL, f, None, 4, 8, 9, None, None, 0)          # K > E
    _expect(moe.MOE_EINVAL, f, None, 4, 8, 0, None, None, 0)          # K < 1
    _expect(moe.MOE_EINVAL, f, None, 4, 8, 2, None, None, 0)          # NULL buffers
    _expect(moe.MOE_EUNSUPPORTED, f, 16, 4, 64, 33, 16, 16, 0)        # K > 32
    _expect(moe.MOE_EUNSUPPORTED, f, 16, 4, 5000, 2, 16, 16, 0)       # E > 4096


def test_permute_argument_checks():
    f = moe.moe_permute
    n = moe.moe_permute_workspace_bytes(100, 8, 2)
    assert n > 0
    args = [16, None, moe.MOE_BF16, 16, 16, 100, 64, 8, 2, 16, 16, 16, 16, None, 16, None, 16, n, 0]
    a = list(args); a[16] = 16; a[17] = n - 1
    _expect(moe.MOE_EWORKSPACE, f, *a)                                   # workspace too small
    a = list(args); a[7] = 2000
    _expect(moe.MOE_EUNSUPPORTED, f, *a)                                 # E > 1024
    a = list(args); a[2] = moe.MOE_MXFP4
    _expect(moe.MOE_EUNSUPPORTED, f, *a)                                 # no MXFP4 activations
    a = list(args); a[2] = moe.MOE_FP8_E4M3                              # fp8 needs H % 128
    _expect(moe.MOE_EUNSUPPORTED, f, *a)
    a = list(args); a[2] = moe.MOE_FP8_E4M3; a[6] = 128                  # fp8 needs scales
    _expect(moe.MOE_EINVAL, f, *a)
    a = list(args); a[2] = moe.MOE_FP8_E4M3; a[6] = 128; a[14] = None; a[15] = 16
    _expect(moe.MOE_EINVAL, f, *a)                                       # permuted scales need x_sf
    a = list(args); a[0] = None
    _expect(moe.MOE_EINVAL, f, *a)


def test_ffn_and_combine_argument_checks():
    g = moe.moe_ffn_gate_up
    _expect(moe.MOE_EUNSUPPORTED, g, 16, None, moe.MOE_BF16, 16, 64, 4, 128, 128, 16, 16, None, None,
            moe.MOE_F32, 16, None, 0)                                    # mixed formats
    _expect(moe.MOE_EUNSUPPORTED, g, 16, None, moe.MOE_BF16, 16, 64, 4, 96, 128, 16, 16, None, None,
            moe.MOE_BF16, 16, None, 0)                                   # H % 64
    _expect(moe.MOE_EINVAL, g, None, None, moe.MOE_BF16, 16, 64, 4, 128, 128, 16, 16, None, None,
            moe.MOE_BF16, 16, None, 0)                                   # NULL x_perm
    d = moe.moe_ffn_down
    _expect(moe.MOE_EUNSUPPORTED, d, 16, None, moe.MOE_BF16, 16, 64, 4, 128, 128, 16, None,
            moe.MOE_BF16, 16, moe.MOE_BF16, 0)                           # H % 256
    _expect(moe.MOE_EUNSUPPORTED, d, 16, None, moe.MOE_BF16, 16, 64, 4, 256, 128, 16, None,
            moe.MOE_BF16, 16, moe.MOE_F32, 0)                            # out must be bf16
    c = moe.moe_combine
    _expect(moe.MOE_EINVAL, c, None, moe.MOE_BF16, 16, 16, 4, 64, 2, 16, moe.MOE_BF16, 0)
    _expect(moe.MOE_EUNSUPPORTED, c, 16, moe.MOE_MXFP4, 16, 16, 4, 64, 2, 16, moe.MOE_BF16, 0)
    _expect(moe.MOE_EUNSUPPORTED, c, 16, moe.MOE_BF16, 16, 16, 4, 64, 64, 16, moe.MOE_BF16, 0)


def test_layer_workspace_sizes_and_layout():
    d = moe.LayerDesc(8192, 7168, 2048, 384, 8, moe.MOE_BF16, moe.MOE_BF16, moe.MOE_BF16, 0)
    n = moe.moe_layer_workspace_bytes(d)
    M = 8192 * 8
    big = M * 7168 * 2 + M * 2048 * 2              # y_rows + h (gate/up gathers from x)
    assert big < n < big + 8 * 2 ** 20
    lay = moe.moe_layer_workspace_layout(d)
    used = [v for v in lay.values() if v is not None]
    assert used == sorted(used) and all(v % 256 == 0 for v in used)
    assert lay["x_perm"] is None and lay["x_perm_sf"] is None and lay["row_w"] is None
    assert lay["h_sf"] is None and lay["acc_f32"] is None
    assert lay["y_rows"] + M * 7168 * 2 <= n
    os.environ["MOE_LAYER_XPERM"] = "1"       # the materialised permuted copy
    try:
        n_mat = moe.moe_layer_workspace_bytes(d)
        lay_mat = moe.moe_layer_workspace_layout(d)
    finally:
        del os.environ["MOE_LAYER_XPERM"]
    assert lay_mat["x_perm"] is not None and big + M * 7168 * 2 < n_mat < big + M * 7168 * 2 + 8 * 2 ** 20
    sc = moe.LayerDesc(8192, 7168, 2048, 384, 8, moe.MOE_BF16, moe.MOE_BF16, moe.MOE_BF16,
                       moe.MOE_COMBINE_SCATTER_ATOMIC)
    lay_sc = moe.moe_layer_workspace_layout(sc)
    assert lay_sc["y_rows"] is None and lay_sc["row_w"] is not None and lay_sc["acc_f32"] is not None
    assert moe.moe_layer_workspace_bytes(sc) < M * 2048 * 2 + 8192 * 7168 * 4 + 8 * 2 ** 20
    sc32 = moe.LayerDesc(64, 128, 64, 8, 2, moe.MOE_F32, moe.MOE_F32, moe.MOE_F32, 1)
    assert moe.moe_layer_workspace_layout(sc32)["acc_f32"] is None   # accumulates into out
    bad = moe.LayerDesc(8, 128, 64, 4, 5, moe.MOE_F32, moe.MOE_F32, moe.MOE_F32, 0)   # K > E
    assert moe.moe_layer_workspace_bytes(bad) == 0
    mixed = moe.LayerDesc(8, 128, 64, 4, 2, moe.MOE_BF16, moe.MOE_F32, moe.MOE_BF16, 0)
    assert moe.moe_layer_workspace_bytes(mixed) == 0
    fp8 = moe.LayerDesc(64, 256, 128, 4, 2, moe.MOE_FP8_E4M3, moe.MOE_MXFP4, moe.MOE_BF16, 0)
    lay8 = moe.moe_layer_workspace_layout(fp8)
    # the gathered fp8 gate/up reads the permuted block-major scales, not x_perm
    assert lay8["x_perm"] is None and lay8["x_perm_sf"] is not None and lay8["h_sf"] is not None


def test_gather_and_scatter_argument_checks():
    g = moe.moe_ffn_gate_up_gather
    # (x, x_sf, x_perm_sf, act, row_src, T, K, cu, M, E, H, Hp, wg, wu, sfg, sfu, wgt, h, h_sf)
    _expect(moe.MOE_EINVAL, g, 16, None, None, moe.MOE_BF16, 16, -4, 2, 16, 8, 4, 128, 128, 16, 16,
            None, None, moe.MOE_BF16, 16, None, 0)                        # T < 0
    _expect(moe.MOE_EINVAL, g, 16, None, None, moe.MOE_BF16, None, 4, 2, 16, 8, 4, 128, 128, 16, 16,
            None, None, moe.MOE_BF16, 16, None, 0)                        # NULL row_src
    _expect(moe.MOE_EUNSUPPORTED, g, 16, None, None, moe.MOE_BF16, 16, 2 ** 20, 2, 16, 8, 4, 1024, 128,
            16, 16, None, None, moe.MOE_BF16, 16, None, 0)                # x past 2 GiB
    _expect(moe.MOE_EINVAL, g, 16, None, None, moe.MOE_FP8_E4M3, 16, 4, 2, 16, 8, 4, 128, 128, 16,
            16, 16, 16, moe.MOE_MXFP4, 16, 16, 0)                         # fp8 without scales
    d = moe.moe_ffn_down_scatter
    # (h, h_sf, h_dtype, cu, M, E, H, Hp, wd, sfd, wgt, row_src, row_w, T, K, acc)
    _expect(moe.MOE_EINVAL, d, 16, None, moe.MOE_BF16, 16, 8, 4, 256, 128, 16, None, moe.MOE_BF16,
            16, 16, 4, 2, None, 0)                                        # NULL accumulator
    _expect(moe.MOE_EUNSUPPORTED, d, 16, None, moe.MOE_BF16, 16, 8, 4, 128, 128, 16, None,
            moe.MOE_BF16, 16, 16, 4, 2, 16, 0)                            # H % 256


def test_single_launch_argument_checks():
    """moe_grouped_ffn_fused and moe_grouped_ffn_fused_scatter reject on the host, before any
    launch: unsupported formats and shapes, a short workspace, missing buffers."""
    M, E, H, Hp = 64, 4, 512, 256
    n = moe.moe_grouped_ffn_fused_workspace_bytes(M, E, Hp)
    assert n >= M * Hp * 2 + 16 * 4
    assert moe.moe_grouped_ffn_fused_workspace_bytes(-1, E, Hp) == 0
    f = moe.moe_grouped_ffn_fused
    # (x, act, row_src, T, K, cu, M, E, H, Hp, wg, wu, wd, wgt, y_rows, out, ws, ws_bytes, stream)
    base = dict(x=16, act=moe.MOE_BF16, row_src=16, T=32, K=2, cu_seqlens=16, M=M, E=E, H=H, Hp=Hp,
                w_gate=16, w_up=16, w_down=16, wgt=moe.MOE_BF16, y_rows=16, out=moe.MOE_BF16, ws=16,
                ws_bytes=n, stream=0)
    for kw, status in ((dict(act=moe.MOE_F32), moe.MOE_EUNSUPPORTED),
                       (dict(out=moe.MOE_F32), moe.MOE_EUNSUPPORTED),
                       (dict(H=384), moe.MOE_EUNSUPPORTED),             # H % 256
                       (dict(Hp=128), moe.MOE_EUNSUPPORTED),            # K loop of down too short
                       (dict(E=1025), moe.MOE_EUNSUPPORTED),
                       (dict(K=0), moe.MOE_EINVAL),
                       (dict(ws_bytes=n - 1), moe.MOE_EWORKSPACE),
                       (dict(cu_seqlens=None), moe.MOE_EINVAL),
                       (dict(y_rows=None), moe.MOE_EINVAL)):
        _expect(status, lambda: f(**dict(base, **kw)))
    s = moe.moe_grouped_ffn_fused_scatter
    # (x, act, row_src, T, K, cu, M, E, H, Hp, wg, wu, wd, wgt, row_w, acc, ws, ws_bytes, stream)
    sbase = dict(base, row_w=16, acc=16)
    del sbase["y_rows"], sbase["out"]
    for kw, status in ((dict(act=moe.MOE_FP8_E4M3), moe.MOE_EUNSUPPORTED),
                       (dict(H=384), moe.MOE_EUNSUPPORTED),
                       (dict(ws_bytes=n - 1), moe.MOE_EWORKSPACE),
                       (dict(row_w=None), moe.MOE_EINVAL),
                       (dict(acc=None), moe.MOE_EINVAL)):
        _expect(status, lambda: s(**dict(sbase, **kw)))


def test_pack_mxfp4_pairs_argument_checks():
    f = moe.moe_pack_mxfp4_pairs
    _expect(moe.MOE_EUNSUPPORTED, f, 16, 32, 2, 3, 256, 0)      # N odd
    _expect(moe.MOE_EUNSUPPORTED, f, 16, 32, 2, 4, 192, 0)      # K % 128
    _expect(moe.MOE_EINVAL, f, 16, 16, 2, 4, 256, 0)            # in place
    _expect(moe.MOE_EINVAL, f, None, 32, 2, 4, 256, 0)
    _expect(moe.MOE_EINVAL, f, 16, 40, 2, 4, 256, 0)            # output not 16-byte aligned
    _expect(moe.MOE_EINVAL, f, 16, 32, -1, 4, 256, 0)


def test_layer_forward_rejects_small_workspace():
    d = moe.LayerDesc(64, 128, 64, 8, 2, moe.MOE_F32, moe.MOE_F32, moe.MOE_F32, 0)
    n = moe.moe_layer_workspace_bytes(d)
    _expect(moe.MOE_EWORKSPACE, moe.moe_layer_forward, d, 16, None, 16, None, None, 16, 16, 16,
            None, None, None, 16, 16, n - 1, 0)
    d.combine = 7
    _expect(moe.MOE_EINVAL, moe.moe_layer_forward, d, 16, None, 16, None, None, 16, 16, 16,
            None, None, None, 16, 16, n, 0)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        moe.lib()
