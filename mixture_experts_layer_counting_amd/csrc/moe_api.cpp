// Host side of the C ABI declared in include/moe.h: argument checks, workspace layout and
// the launch sequence of each entry point. No device code here; every launch goes through
// the kernel files.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <limits>

#include "moe_common.h"
#include "noalloc.h"

namespace moe {

moe_status_t launch_route_topk(const float*, int, int, int, int*, float*, hipStream_t);
size_t permute_ws_bytes(int T, int E, int K);
moe_status_t launch_permute(const void* x, const float* x_sf, int elem_bytes, const int* topk_idx,
                            const float* topk_w, int T, int H, int E, int K, int* counts,
                            int* cu_seqlens, int* pos, int* row_src, float* row_w, void* x_perm,
                            float* x_perm_sf, void* ws, bool validate, int pad, int cap,
                            int** err_out, hipStream_t s, bool hist_done);
moe_status_t launch_route_hist(const float* logits, int T, int E, int K, int* topk_idx,
                               float* topk_w, void* ws, hipStream_t s);
moe_status_t launch_quantize_fp8(const void* x, moe_dtype_t xt, int R, int C, void* q, float* sf,
                                 hipStream_t s);
moe_status_t launch_combine(const void*, moe_dtype_t, const int*, const float*, int, int, int,
                            const void*, void*, moe_dtype_t, hipStream_t);
moe_status_t launch_ffn_gate_up_bf16(const void*, const int*, int, int, int, int, const void*,
                                     const void*, void*, const RowMaps&, hipStream_t);
moe_status_t launch_ffn_down_bf16(const void*, const int*, int, int, int, int, const void*, void*,
                                  const RowMaps&, hipStream_t);
moe_status_t launch_ffn_gate_up_fp8(const void*, const float*, const int*, int, int, int, int,
                                    const void*, const uint8_t*, const void*, const uint8_t*, void*,
                                    float*, const RowMaps&, bool paired, hipStream_t);
moe_status_t launch_ffn_down_fp8(const void*, const float*, const int*, int, int, int, int,
                                 const void*, const uint8_t*, void*, const RowMaps&, bool paired, hipStream_t);
moe_status_t launch_pack_mxfp4_pairs(const void* w, void* out, int E, int N, int K, hipStream_t s);
moe_status_t launch_ffn_gate_up_f32(const void*, const int*, int, int, int, int, const void*,
                                    const void*, void*, const RowMaps&, hipStream_t);
moe_status_t launch_ffn_down_f32(const void*, const int*, int, int, int, int, const void*, void*,
                                 const RowMaps&, hipStream_t);
size_t fused_ctl_ints(int M, int E);
moe_status_t launch_ffn_fused_bf16(const void* x, const int* row_src, int T, int K, const int* cu, int M,
                                   int E, int H, int Hp, const void* wg, const void* wu, const void* wd,
                                   void* h, void* y, int* ctl, hipStream_t s, const SharedFold& sf,
                                   const float* row_w, float* s_acc);
moe_status_t launch_acc_zero(float* acc, size_t n, hipStream_t s);
moe_status_t launch_fill_bytes(void* p, size_t n, unsigned char v, hipStream_t s);
moe_status_t launch_acc_store(const float* acc, size_t n, const void* add, moe_dtype_t add_dtype,
                              void* out, moe_dtype_t out_dtype, hipStream_t s);
moe_status_t launch_dense_cu(int* cu, int T, hipStream_t s);
moe_status_t launch_bwd_down_swiglu(const void* dy, const int* cu, int M, int E, int H, int Hp,
                                    const void* wd, const void* g, const void* u, void* dg, void* du,
                                    hipStream_t s);
moe_status_t launch_bwd_gate_up(const void* dg, const void* du, const int* cu, int M, int E, int H,
                                int Hp, const void* wg, const void* wu, void* dx_rows, hipStream_t s);
moe_status_t launch_bwd_wgrad(const void* A, const void* B, const int* cu, int E, int Md, int Nd,
                              float* W, hipStream_t s);
moe_status_t launch_combine_bwd(const void* dout, const void* y, const int* pos, const float* w,
                                int T, int H, int K, void* dy, float* dw, hipStream_t s);
moe_status_t launch_route_bwd(const int* idx, const float* w, const float* dw, int T, int E, int K,
                              float* dl, hipStream_t s);

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

bool env_flag(const char* name) {
  const char* v = std::getenv(name);
  return v && v[0] && std::strcmp(v, "0") != 0;
}

static int act_bytes(moe_dtype_t d) {
  switch (d) {
    case MOE_F32: return 4;
    case MOE_BF16: return 2;
    case MOE_FP8_E4M3: return 1;
    default: return 0;
  }
}

enum Path { PATH_NONE, PATH_F32, PATH_BF16, PATH_FP8_MXFP4 };

static Path ffn_path(moe_dtype_t act, moe_dtype_t wgt) {
  if (act == MOE_F32 && wgt == MOE_F32) return PATH_F32;
  if (act == MOE_BF16 && wgt == MOE_BF16) return PATH_BF16;
  if (act == MOE_FP8_E4M3 && (wgt == MOE_MXFP4 || wgt == MOE_MXFP4_PAIRED)) return PATH_FP8_MXFP4;
  return PATH_NONE;
}

// h / y formats of a path
static moe_dtype_t h_dtype_of(Path p) {
  return p == PATH_F32 ? MOE_F32 : p == PATH_BF16 ? MOE_BF16 : MOE_FP8_E4M3;
}
static moe_dtype_t y_dtype_of(Path p) { return p == PATH_F32 ? MOE_F32 : MOE_BF16; }

static moe_status_t check_ffn_dims(Path p, int64_t M, int E, int H, int Hp, bool gate_up) {
  if (M < 0 || E < 1 || H < 1 || Hp < 1) return MOE_EINVAL;
  if (M > std::numeric_limits<int32_t>::max() / 2) return MOE_EUNSUPPORTED;
  switch (p) {
    case PATH_F32:
      if (E > 512) return MOE_EUNSUPPORTED;
      return MOE_OK;
    case PATH_BF16:
      if (E > 1024) return MOE_EUNSUPPORTED;
      // 32-bit buffer offsets: one expert matrix and 256 activation rows must stay < 2 GiB
      if ((int64_t)H * Hp * 2 >= (1ll << 31) || 256ll * (H > Hp ? H : Hp) * 2 >= (1ll << 31))
        return MOE_EUNSUPPORTED;
      if (gate_up) return (H % 64 == 0 && Hp % 128 == 0) ? MOE_OK : MOE_EUNSUPPORTED;
      return (H % 256 == 0 && Hp % 64 == 0) ? MOE_OK : MOE_EUNSUPPORTED;
    case PATH_FP8_MXFP4:
      if (E > 1024) return MOE_EUNSUPPORTED;
      if ((int64_t)H * Hp >= (1ll << 31) || 256ll * (H > Hp ? H : Hp) >= (1ll << 31)) return MOE_EUNSUPPORTED;
      if (gate_up) return (H % 128 == 0 && Hp % 128 == 0) ? MOE_OK : MOE_EUNSUPPORTED;
      return (H % 256 == 0 && Hp % 128 == 0) ? MOE_OK : MOE_EUNSUPPORTED;
    default:
      return MOE_EUNSUPPORTED;
  }
}

// Shapes the single-launch bf16 FFN (moe_grouped_ffn_fused) takes: those of both bf16 kernels
// with K loops of at least eight 32-deep steps, and rows gathered with 32-bit offsets into x.
static moe_status_t check_fused_dims(int64_t M, int T, int K, int E, int H, int Hp) {
  if (T < 0 || K < 1) return MOE_EINVAL;
  moe_status_t st = check_ffn_dims(PATH_BF16, M, E, H, Hp, true);
  if (st == MOE_OK) st = check_ffn_dims(PATH_BF16, M, E, H, Hp, false);
  if (st != MOE_OK) return st;
  if (H % 256 || Hp % 128 || H < 256 || Hp < 256) return MOE_EUNSUPPORTED;
  if ((int64_t)T * H * 2 >= (1ll << 31)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

static void poison(void* ws, size_t bytes, hipStream_t s) {
  if (ws && bytes && env_flag("MOE_DEBUG_POISON")) (void)launch_fill_bytes(ws, bytes, 0xFF, s);
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_str(moe_status_t st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: unsupported dtype combination or size";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace too small";
    case MOE_EHIP: return "MOE_EHIP: HIP launch or runtime error";
    default: return "MOE_UNKNOWN";
  }
}

moe_status_t moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t K,
                            int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  if (T < 0 || E < 1 || K < 1 || K > E) return MOE_EINVAL;
  if (K > 32 || E > 4096) return MOE_EUNSUPPORTED;
  if (T > 0 && (!logits || !topk_idx || !topk_w)) return MOE_EINVAL;
  return launch_route_topk(logits, T, E, K, topk_idx, topk_w, stream);
}

size_t moe_permute_workspace_bytes(int32_t T, int32_t E, int32_t K) {
  if (T < 0 || E < 1 || K < 1) return 0;
  return permute_ws_bytes(T, E, K);
}

// With logits, topk_idx and topk_w are outputs: the routing is computed together with the
// permutation's histogram (moe_route_permute).
static moe_status_t permute_impl(const float* logits, const void* x, const float* x_sf, moe_dtype_t act,
                                 const int32_t* topk_idx, const float* topk_w, int32_t T, int32_t H,
                                 int32_t E, int32_t K, int32_t pad, int32_t* counts,
                                 int32_t* cu_seqlens, int32_t* pos, int32_t* row_src, float* row_w,
                                 void* x_perm, float* x_perm_sf, void* ws, size_t ws_bytes,
                                 hipStream_t stream, bool noalloc = false) {
  if (T < 0 || H < 1 || E < 1 || K < 1 || pad < 1) return MOE_EINVAL;
  if (E > 1024 || K > 32) return MOE_EUNSUPPORTED;
  const int eb = act_bytes(act);
  if (eb == 0) return MOE_EUNSUPPORTED;
  if (!counts || !cu_seqlens) return MOE_EINVAL;
  if (T > 0 && (!topk_idx || !pos || !row_src)) return MOE_EINVAL;
  if (logits && (K > E || (T > 0 && !topk_w))) return MOE_EINVAL;
  if (T > 0 && x_perm && !x) return MOE_EINVAL;
  if (row_w && T > 0 && !topk_w) return MOE_EINVAL;
  if (act == MOE_FP8_E4M3) {
    if (H % 128) return MOE_EUNSUPPORTED;
    if (T > 0 && x_perm && !x_perm_sf) return MOE_EINVAL;
    if (T > 0 && x_perm_sf && !x_sf) return MOE_EINVAL;
  }
  const int64_t cap = (int64_t)T * K + (int64_t)E * (pad - 1);
  if (cap > std::numeric_limits<int32_t>::max() / 2) return MOE_EUNSUPPORTED;
  const size_t need = permute_ws_bytes(T, E, K);
  if (noalloc) {
    // the static scratch: sizes beyond it are rejected before anything touches the device
    if (need > kNoallocScratchBytes) return MOE_EUNSUPPORTED;
    ws = permute_noalloc_scratch();
    ws_bytes = kNoallocScratchBytes;
    if (!ws) return MOE_EHIP;
  }
  if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
  // the no-alloc variant enqueues kernels only: no poison fill, no validation (which needs
  // a memset, a copy to the host and a stream synchronisation)
  if (!noalloc) poison(ws, ws_bytes, stream);
  // routed here, the ids are valid and distinct: nothing to validate
  const bool validate = !logits && !noalloc && env_flag("MOE_VALIDATE");
  int* err = nullptr;
  // fp8: the block-major scales are written whenever x_perm_sf is given, also without x_perm
  const bool sf = act == MOE_FP8_E4M3 && x_perm_sf;
  if (logits && T > 0) {
    const moe_status_t st = launch_route_hist(logits, T, E, K, const_cast<int32_t*>(topk_idx),
                                              const_cast<float*>(topk_w), ws, stream);
    if (st != MOE_OK) return st;
  }
  moe_status_t st = launch_permute(x, sf ? x_sf : nullptr, eb, topk_idx, topk_w, T, H, E, K, counts,
                                   cu_seqlens, pos, row_src, row_w, x_perm, sf ? x_perm_sf : nullptr,
                                   ws, validate, pad, (int)cap, &err, stream, logits != nullptr);
  if (st != MOE_OK || !validate) return st;
  int h_err = 0;
  if (hipMemcpyAsync(&h_err, err, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return MOE_EHIP;
  return h_err ? MOE_EINVAL : MOE_OK;
}

moe_status_t moe_permute(const void* x, const float* x_sf, moe_dtype_t act,
                         const int32_t* topk_idx, const float* topk_w, int32_t T, int32_t H,
                         int32_t E, int32_t K, int32_t* counts, int32_t* cu_seqlens,
                         int32_t* pos, int32_t* row_src, float* row_w, void* x_perm,
                         float* x_perm_sf, void* ws, size_t ws_bytes, hipStream_t stream) {
  return permute_impl(nullptr, x, x_sf, act, topk_idx, topk_w, T, H, E, K, 1, counts, cu_seqlens, pos,
                      row_src, row_w, x_perm, x_perm_sf, ws, ws_bytes, stream);
}

moe_status_t moe_permute_noalloc(const void* x, const float* x_sf, moe_dtype_t act,
                                 const int32_t* topk_idx, const float* topk_w, int32_t T, int32_t H,
                                 int32_t E, int32_t K, int32_t* counts, int32_t* cu_seqlens,
                                 int32_t* pos, int32_t* row_src, float* row_w, void* x_perm,
                                 float* x_perm_sf, hipStream_t stream) {
  return permute_impl(nullptr, x, x_sf, act, topk_idx, topk_w, T, H, E, K, 1, counts, cu_seqlens, pos,
                      row_src, row_w, x_perm, x_perm_sf, nullptr, 0, stream, /*noalloc=*/true);
}

int64_t moe_padded_capacity(int32_t T, int32_t E, int32_t K, int32_t pad) {
  if (T < 0 || E < 1 || K < 1 || pad < 1) return -1;
  return (int64_t)T * K + (int64_t)E * (pad - 1);
}

moe_status_t moe_permute_padded(const void* x, const float* x_sf, moe_dtype_t act,
                                const int32_t* topk_idx, const float* topk_w, int32_t T, int32_t H,
                                int32_t E, int32_t K, int32_t pad, int32_t* counts,
                                int32_t* cu_seqlens, int32_t* pos, int32_t* row_src, float* row_w,
                                void* x_perm, float* x_perm_sf, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  return permute_impl(nullptr, x, x_sf, act, topk_idx, topk_w, T, H, E, K, pad, counts, cu_seqlens, pos,
                      row_src, row_w, x_perm, x_perm_sf, ws, ws_bytes, stream);
}

moe_status_t moe_route_permute(const float* logits, const void* x, const float* x_sf,
                               moe_dtype_t act, int32_t T, int32_t H, int32_t E, int32_t K,
                               int32_t pad, int32_t* topk_idx, float* topk_w, int32_t* counts,
                               int32_t* cu_seqlens, int32_t* pos, int32_t* row_src, float* row_w,
                               void* x_perm, float* x_perm_sf, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  if (T > 0 && !logits) return MOE_EINVAL;
  return permute_impl(T > 0 ? logits : nullptr, x, x_sf, act, topk_idx, topk_w, T, H, E, K, pad,
                      counts, cu_seqlens, pos, row_src, row_w, x_perm, x_perm_sf, ws, ws_bytes, stream);
}

moe_status_t moe_quantize_fp8(const void* x, moe_dtype_t x_dtype, int32_t R, int32_t C, uint8_t* q,
                              float* sf, hipStream_t stream) {
  if (R < 0 || C < 1) return MOE_EINVAL;
  if (C % 128 || (x_dtype != MOE_BF16 && x_dtype != MOE_F32)) return MOE_EUNSUPPORTED;
  if (R > 0 && (!x || !q || !sf)) return MOE_EINVAL;
  if ((uintptr_t)x % 16 || (uintptr_t)q % 8) return MOE_EINVAL;
  return launch_quantize_fp8(x, x_dtype, R, C, q, sf, stream);
}

moe_status_t moe_pack_mxfp4_pairs(const uint8_t* w, uint8_t* w_paired, int32_t E, int32_t N, int32_t K,
                                  hipStream_t stream) {
  if (E < 0 || N < 0 || K < 0) return MOE_EINVAL;
  if (N % 2 || K % 128) return MOE_EUNSUPPORTED;
  if ((size_t)E * N * K == 0) return MOE_OK;
  if (!w || !w_paired || w == w_paired) return MOE_EINVAL;
  if ((uintptr_t)w % 16 || (uintptr_t)w_paired % 16) return MOE_EINVAL;
  return launch_pack_mxfp4_pairs(w, w_paired, E, N, K, stream);
}

moe_status_t moe_ffn_gate_up(const void* x_perm, const float* x_perm_sf, moe_dtype_t act,
                             const int32_t* cu_seqlens, int32_t M, int32_t E, int32_t H,
                             int32_t Hp, const void* w_gate, const void* w_up,
                             const uint8_t* sf_gate, const uint8_t* sf_up, moe_dtype_t wgt,
                             void* h, float* h_sf, hipStream_t stream) {
  const Path p = ffn_path(act, wgt);
  if (p == PATH_NONE) return MOE_EUNSUPPORTED;
  moe_status_t st = check_ffn_dims(p, M, E, H, Hp, true);
  if (st != MOE_OK) return st;
  if (!cu_seqlens) return MOE_EINVAL;
  if (M > 0 && (!x_perm || !w_gate || !w_up || !h)) return MOE_EINVAL;
  if (p == PATH_FP8_MXFP4) {
    if (M > 0 && (!x_perm_sf || !sf_gate || !sf_up || !h_sf)) return MOE_EINVAL;
    return launch_ffn_gate_up_fp8(x_perm, x_perm_sf, cu_seqlens, M, E, H, Hp, w_gate, sf_gate, w_up,
                                  sf_up, h, h_sf, RowMaps{}, wgt == MOE_MXFP4_PAIRED, stream);
  }
  if (p == PATH_F32)
    return launch_ffn_gate_up_f32(x_perm, cu_seqlens, M, E, H, Hp, w_gate, w_up, h, RowMaps{}, stream);
  return launch_ffn_gate_up_bf16(x_perm, cu_seqlens, M, E, H, Hp, w_gate, w_up, h, RowMaps{}, stream);
}

// Gate/up with rows gathered from x through row_src. fp8: the activation scales come from
// x_perm_sf ([H/128, M] block-major, as the permutation writes them) when it is given, else
// they are gathered from x_sf row by row.
static moe_status_t gate_up_gather(const void* x, const float* x_sf, const float* x_perm_sf,
                                   moe_dtype_t act, const int32_t* row_src, int32_t T, int32_t K,
                                   const int32_t* cu_seqlens, int32_t M, int32_t E, int32_t H,
                                   int32_t Hp, const void* w_gate, const void* w_up,
                                   const uint8_t* sf_gate, const uint8_t* sf_up, moe_dtype_t wgt,
                                   void* h, float* h_sf, hipStream_t stream) {
  const Path p = ffn_path(act, wgt);
  if (p == PATH_NONE) return MOE_EUNSUPPORTED;
  if (T < 0 || K < 1) return MOE_EINVAL;
  moe_status_t st = check_ffn_dims(p, M, E, H, Hp, true);
  if (st != MOE_OK) return st;
  // the gathered rows are addressed with 32-bit byte offsets into x
  if ((int64_t)T * H * act_bytes(act) >= (1ll << 31)) return MOE_EUNSUPPORTED;
  if (!cu_seqlens) return MOE_EINVAL;
  if (M > 0 && (!x || !row_src || !w_gate || !w_up || !h)) return MOE_EINVAL;
  RowMaps maps;
  maps.a_src = row_src;
  maps.a_k = K;
  maps.a_rows = T;
  if (p == PATH_FP8_MXFP4) {
    if (M > 0 && ((!x_sf && !x_perm_sf) || !sf_gate || !sf_up || !h_sf)) return MOE_EINVAL;
    maps.a_sf_perm = x_perm_sf;
    return launch_ffn_gate_up_fp8(x, x_sf, cu_seqlens, M, E, H, Hp, w_gate, sf_gate, w_up, sf_up, h,
                                  h_sf, maps, wgt == MOE_MXFP4_PAIRED, stream);
  }
  if (p == PATH_F32) return launch_ffn_gate_up_f32(x, cu_seqlens, M, E, H, Hp, w_gate, w_up, h, maps, stream);
  return launch_ffn_gate_up_bf16(x, cu_seqlens, M, E, H, Hp, w_gate, w_up, h, maps, stream);
}

moe_status_t moe_ffn_gate_up_gather(const void* x, const float* x_sf, const float* x_perm_sf,
                                    moe_dtype_t act, const int32_t* row_src, int32_t T, int32_t K,
                                    const int32_t* cu_seqlens, int32_t M, int32_t E, int32_t H,
                                    int32_t Hp, const void* w_gate, const void* w_up,
                                    const uint8_t* sf_gate, const uint8_t* sf_up, moe_dtype_t wgt,
                                    void* h, float* h_sf, hipStream_t stream) {
  return gate_up_gather(x, x_sf, x_perm_sf, act, row_src, T, K, cu_seqlens, M, E, H, Hp, w_gate, w_up,
                        sf_gate, sf_up, wgt, h, h_sf, stream);
}

moe_status_t moe_ffn_down(const void* h, const float* h_sf, moe_dtype_t h_dtype,
                          const int32_t* cu_seqlens, int32_t M, int32_t E, int32_t H,
                          int32_t Hp, const void* w_down, const uint8_t* sf_down,
                          moe_dtype_t wgt, void* y_rows, moe_dtype_t out, hipStream_t stream) {
  const Path p = ffn_path(h_dtype, wgt);
  if (p == PATH_NONE || out != y_dtype_of(p)) return MOE_EUNSUPPORTED;
  moe_status_t st = check_ffn_dims(p, M, E, H, Hp, false);
  if (st != MOE_OK) return st;
  if (!cu_seqlens) return MOE_EINVAL;
  if (M > 0 && (!h || !w_down || !y_rows)) return MOE_EINVAL;
  if (p == PATH_FP8_MXFP4) {
    if (M > 0 && (!h_sf || !sf_down)) return MOE_EINVAL;
    return launch_ffn_down_fp8(h, h_sf, cu_seqlens, M, E, H, Hp, w_down, sf_down, y_rows, RowMaps{},
                               wgt == MOE_MXFP4_PAIRED, stream);
  }
  if (p == PATH_F32) return launch_ffn_down_f32(h, cu_seqlens, M, E, H, Hp, w_down, y_rows, RowMaps{}, stream);
  return launch_ffn_down_bf16(h, cu_seqlens, M, E, H, Hp, w_down, y_rows, RowMaps{}, stream);
}

moe_status_t moe_ffn_down_scatter(const void* h, const float* h_sf, moe_dtype_t h_dtype,
                                  const int32_t* cu_seqlens, int32_t M, int32_t E, int32_t H,
                                  int32_t Hp, const void* w_down, const uint8_t* sf_down,
                                  moe_dtype_t wgt, const int32_t* row_src, const float* row_w,
                                  int32_t T, int32_t K, float* acc, hipStream_t stream) {
  const Path p = ffn_path(h_dtype, wgt);
  if (p == PATH_NONE) return MOE_EUNSUPPORTED;
  if (T < 0 || K < 1) return MOE_EINVAL;
  moe_status_t st = check_ffn_dims(p, M, E, H, Hp, false);
  if (st != MOE_OK) return st;
  if (!cu_seqlens) return MOE_EINVAL;
  if (M > 0 && (!h || !w_down || !row_src || !row_w || !acc)) return MOE_EINVAL;
  RowMaps maps;
  maps.s_src = row_src;
  maps.s_w = row_w;
  maps.s_k = K;
  maps.s_acc = acc;
  if (p == PATH_FP8_MXFP4) {
    if (M > 0 && (!h_sf || !sf_down)) return MOE_EINVAL;
    return launch_ffn_down_fp8(h, h_sf, cu_seqlens, M, E, H, Hp, w_down, sf_down, nullptr, maps,
                               wgt == MOE_MXFP4_PAIRED, stream);
  }
  if (p == PATH_F32) return launch_ffn_down_f32(h, cu_seqlens, M, E, H, Hp, w_down, nullptr, maps, stream);
  return launch_ffn_down_bf16(h, cu_seqlens, M, E, H, Hp, w_down, nullptr, maps, stream);
}

size_t moe_grouped_ffn_workspace_bytes(int32_t M, int32_t Hp, moe_dtype_t act, moe_dtype_t wgt) {
  const Path p = ffn_path(act, wgt);
  if (p == PATH_NONE || M < 0 || Hp < 1) return 0;
  const size_t hb = (size_t)act_bytes(h_dtype_of(p));
  size_t n = align_up((size_t)M * Hp * hb, 256);
  if (p == PATH_FP8_MXFP4) n += align_up((size_t)M * (Hp / 128) * 4, 256);
  return n + 256;
}

moe_status_t moe_grouped_ffn(const void* x_perm, const float* x_perm_sf, moe_dtype_t act,
                             const int32_t* cu_seqlens, int32_t M, int32_t E, int32_t H,
                             int32_t Hp, const void* w_gate, const void* w_up,
                             const void* w_down, const uint8_t* sf_gate, const uint8_t* sf_up,
                             const uint8_t* sf_down, moe_dtype_t wgt, void* y_rows,
                             moe_dtype_t out, void* ws, size_t ws_bytes, hipStream_t stream) {
  const Path p = ffn_path(act, wgt);
  if (p == PATH_NONE) return MOE_EUNSUPPORTED;
  const size_t need = moe_grouped_ffn_workspace_bytes(M, Hp, act, wgt);
  if (need == 0) return MOE_EINVAL;
  if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
  moe_status_t st = check_ffn_dims(p, M, E, H, Hp, true);
  if (st == MOE_OK) st = check_ffn_dims(p, M, E, H, Hp, false);
  if (st != MOE_OK) return st;
  if (out != y_dtype_of(p)) return MOE_EUNSUPPORTED;
  poison(ws, ws_bytes, stream);
  void* h = ws;
  float* h_sf = p == PATH_FP8_MXFP4
                    ? reinterpret_cast<float*>(static_cast<char*>(ws) +
                                               align_up((size_t)M * Hp * act_bytes(h_dtype_of(p)), 256))
                    : nullptr;
  st = moe_ffn_gate_up(x_perm, x_perm_sf, act, cu_seqlens, M, E, H, Hp, w_gate, w_up, sf_gate,
                       sf_up, wgt, h, h_sf, stream);
  if (st != MOE_OK) return st;
  return moe_ffn_down(h, h_sf, h_dtype_of(p), cu_seqlens, M, E, H, Hp, w_down, sf_down, wgt,
                      y_rows, out, stream);
}

size_t moe_grouped_ffn_fused_workspace_bytes(int32_t M, int32_t E, int32_t Hp) {
  if (M < 0 || E < 1 || Hp < 1) return 0;
  return align_up((size_t)M * Hp * 2, 256) + align_up(fused_ctl_ints(M, E) * 4, 256) + 256;
}

moe_status_t moe_grouped_ffn_fused(const void* x, moe_dtype_t act, const int32_t* row_src, int32_t T,
                                   int32_t K, const int32_t* cu_seqlens, int32_t M, int32_t E,
                                   int32_t H, int32_t Hp, const void* w_gate, const void* w_up,
                                   const void* w_down, moe_dtype_t wgt, void* y_rows, moe_dtype_t out,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  if (act != MOE_BF16 || wgt != MOE_BF16 || out != MOE_BF16) return MOE_EUNSUPPORTED;
  moe_status_t st = check_fused_dims(M, T, K, E, H, Hp);
  if (st != MOE_OK) return st;
  const size_t need = moe_grouped_ffn_fused_workspace_bytes(M, E, Hp);
  if (need == 0) return MOE_EINVAL;
  if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
  if (!cu_seqlens) return MOE_EINVAL;
  if (M > 0 && (!x || !row_src || !w_gate || !w_up || !w_down || !y_rows)) return MOE_EINVAL;
  poison(ws, ws_bytes, stream);
  char* base = static_cast<char*>(ws);
  int* ctl = reinterpret_cast<int*>(base + align_up((size_t)M * Hp * 2, 256));
  return launch_ffn_fused_bf16(x, row_src, T, K, cu_seqlens, M, E, H, Hp, w_gate, w_up, w_down, base,
                               y_rows, ctl, stream, SharedFold{}, nullptr, nullptr);
}

moe_status_t moe_grouped_ffn_fused_scatter(const void* x, moe_dtype_t act, const int32_t* row_src,
                                           int32_t T, int32_t K, const int32_t* cu_seqlens, int32_t M,
                                           int32_t E, int32_t H, int32_t Hp, const void* w_gate,
                                           const void* w_up, const void* w_down, moe_dtype_t wgt,
                                           const float* row_w, float* acc, void* ws, size_t ws_bytes,
                                           hipStream_t stream) {
  if (act != MOE_BF16 || wgt != MOE_BF16) return MOE_EUNSUPPORTED;
  moe_status_t st = check_fused_dims(M, T, K, E, H, Hp);
  if (st != MOE_OK) return st;
  const size_t need = moe_grouped_ffn_fused_workspace_bytes(M, E, Hp);
  if (need == 0) return MOE_EINVAL;
  if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
  if (!cu_seqlens) return MOE_EINVAL;
  if (M > 0 && (!x || !row_src || !w_gate || !w_up || !w_down || !row_w || !acc)) return MOE_EINVAL;
  poison(ws, ws_bytes, stream);
  char* base = static_cast<char*>(ws);
  int* ctl = reinterpret_cast<int*>(base + align_up((size_t)M * Hp * 2, 256));
  return launch_ffn_fused_bf16(x, row_src, T, K, cu_seqlens, M, E, H, Hp, w_gate, w_up, w_down, base,
                               nullptr, ctl, stream, SharedFold{}, row_w, acc);
}

moe_status_t moe_combine(const void* y_rows, moe_dtype_t y_dtype, const int32_t* pos,
                         const float* topk_w, int32_t T, int32_t H, int32_t K, void* out,
                         moe_dtype_t out_dtype, hipStream_t stream) {
  if (T < 0 || H < 1 || K < 1) return MOE_EINVAL;
  if (K > 32) return MOE_EUNSUPPORTED;
  if ((y_dtype != MOE_F32 && y_dtype != MOE_BF16) || (out_dtype != MOE_F32 && out_dtype != MOE_BF16))
    return MOE_EUNSUPPORTED;
  if (T > 0 && (!y_rows || !pos || !out)) return MOE_EINVAL;   // topk_w NULL: unit weights
  return launch_combine(y_rows, y_dtype, pos, topk_w, T, H, K, nullptr, out, out_dtype, stream);
}

moe_status_t moe_combine_shared(const void* y_rows, moe_dtype_t y_dtype, const int32_t* pos,
                                const float* topk_w, int32_t T, int32_t H, int32_t K,
                                const void* shared_y, void* out, moe_dtype_t out_dtype,
                                hipStream_t stream) {
  if (T < 0 || H < 1 || K < 1) return MOE_EINVAL;
  if (K > 32) return MOE_EUNSUPPORTED;
  if ((y_dtype != MOE_F32 && y_dtype != MOE_BF16) || (out_dtype != MOE_F32 && out_dtype != MOE_BF16))
    return MOE_EUNSUPPORTED;
  if (T > 0 && (!y_rows || !pos || !topk_w || !out || !shared_y)) return MOE_EINVAL;
  return launch_combine(y_rows, y_dtype, pos, topk_w, T, H, K, shared_y, out, out_dtype, stream);
}

enum {
  WS_TOPK_IDX, WS_TOPK_W, WS_COUNTS, WS_CU, WS_POS, WS_ROW_SRC, WS_ROW_W, WS_X_PERM,
  WS_X_PERM_SF, WS_H, WS_H_SF, WS_Y, WS_PERM_SCRATCH, WS_ACC, WS_XQ, WS_XQ_SF, WS_FUSED_CTL, WS_N
};

// A BF16 layer with MXFP4 experts quantises its activations to fp8 (1x128 scales) once on
// entry and then runs the fp8 x MXFP4 path ("Mixture of Kittens", Step 8).
static bool layer_quantizes(const moe_layer_desc_t* d) {
  return d->act == MOE_BF16 && (d->wgt == MOE_MXFP4 || d->wgt == MOE_MXFP4_PAIRED);
}
static moe_dtype_t layer_act(const moe_layer_desc_t* d) {
  return layer_quantizes(d) ? MOE_FP8_E4M3 : d->act;
}

// Whether moe_layer_forward writes the permuted copy x_perm (and gate/up reads it) or gate/up
// gathers its rows from x through row_src. Gathering is the default; MOE_LAYER_XPERM=1 forces
// the copy, and so does an x too large for 32-bit row offsets.
static bool layer_materializes(const moe_layer_desc_t* d) {
  return env_flag("MOE_LAYER_XPERM") || (int64_t)d->T * d->H * act_bytes(layer_act(d)) >= (1ll << 31);
}

// Whether moe_layer_forward runs the expert FFN as the single persistent launch
// (moe_grouped_ffn_fused, or moe_grouped_ffn_fused_scatter with the scatter-add combine): by
// default, bf16 layers that gather their rows and combine deterministically, on the shapes
// that launch takes, when the average expert group fits one 256-row m-tile
// (T*K <= 256*E). With several m-tiles per expert the two-launch schedule is faster: its
// rounds start all m-tiles of a weight panel together, so they share the panel through L2,
// which a dynamic queue staggers (T=8192 K=8 E=384: single launch 7.75 vs 7.83 ms per layer,
// 8.59 vs 9.01 ms at maxvio 20; 65536 rows over 52 experts: 5.29 vs 5.07 ms). With the
// scatter-add combine the two launches stay the default: at T=8192 K=8 E=384 the layer took
// 9.58 ms with them against 9.79 ms as one launch. The environment variable MOE_LAYER_FUSED=1
// or 0 forces either path for both combines.
static bool layer_fused(const moe_layer_desc_t* d) {
  if (d->act != MOE_BF16 || d->wgt != MOE_BF16) return false;
  if (layer_materializes(d)) return false;
  if (check_fused_dims((int64_t)d->T * d->K, d->T, d->K, d->E, d->H, d->Hp) != MOE_OK) return false;
  const char* v = std::getenv("MOE_LAYER_FUSED");
  if (v && v[0]) return v[0] != '0';
  return d->combine == MOE_COMBINE_GATHER && (int64_t)d->T * d->K <= 256ll * d->E;
}

static moe_status_t layer_layout(const moe_layer_desc_t* d, size_t* off, size_t* total) {
  if (!d) return MOE_EINVAL;
  if (d->T < 0 || d->H < 1 || d->Hp < 1 || d->E < 1 || d->K < 1 || d->K > d->E) return MOE_EINVAL;
  const Path p = ffn_path(layer_act(d), d->wgt);
  if (p == PATH_NONE || d->out != y_dtype_of(p)) return MOE_EUNSUPPORTED;
  if (d->combine != MOE_COMBINE_GATHER && d->combine != MOE_COMBINE_SCATTER_ATOMIC) return MOE_EINVAL;
  const size_t T = d->T, H = d->H, Hp = d->Hp, E = d->E, K = d->K, M = T * K;
  const size_t ab = act_bytes(layer_act(d)), hb = act_bytes(h_dtype_of(p)), yb = act_bytes(y_dtype_of(p));
  const bool mat = layer_materializes(d), scatter = d->combine == MOE_COMBINE_SCATTER_ATOMIC;
  const bool fp8 = p == PATH_FP8_MXFP4;
  size_t sz[WS_N] = {0};
  bool used[WS_N] = {false};
  auto want = [&](int i, size_t bytes) { sz[i] = bytes; used[i] = true; };
  want(WS_TOPK_IDX, M * 4);
  want(WS_TOPK_W, M * 4);
  want(WS_COUNTS, E * 4);
  want(WS_CU, (E + 1) * 4);
  want(WS_POS, M * 4);
  want(WS_ROW_SRC, M * 4);
  if (scatter) want(WS_ROW_W, M * 4);
  if (mat) want(WS_X_PERM, M * H * ab);
  if (fp8) want(WS_X_PERM_SF, M * (H / 128) * 4);
  want(WS_H, M * Hp * hb);
  if (fp8) want(WS_H_SF, M * (Hp / 128) * 4);
  if (!scatter) want(WS_Y, M * H * yb);
  want(WS_PERM_SCRATCH, permute_ws_bytes(d->T, d->E, d->K));
  if (scatter && d->out != MOE_F32) want(WS_ACC, T * H * 4);  // fp32 out accumulates in place
  if (layer_quantizes(d)) {
    if (H % 128) return MOE_EUNSUPPORTED;
    want(WS_XQ, T * H);
    want(WS_XQ_SF, T * (H / 128) * 4);
  }
  // (sized to also hold the shared expert's rows and m-tiles when moe_layer_forward_shared
  // folds it into the launch)
  if (d->act == MOE_BF16 && d->wgt == MOE_BF16) want(WS_FUSED_CTL, fused_ctl_ints((int)(M + T), d->E + 1) * 4);
  size_t o = 0;
  for (int i = 0; i < WS_N; ++i) {
    if (!used[i]) {
      off[i] = SIZE_MAX;
      continue;
    }
    off[i] = o;
    o = align_up(o + sz[i], 256);
  }
  *total = o + 256;
  return MOE_OK;
}

// The shared expert runs in bf16 (fp32 in the fp32 layer) whatever the routed format
// ("Mixture of Kittens", Step 8: the shared expert stays in BF16).
static Path shared_path(const moe_layer_desc_t* d) {
  return ffn_path(layer_act(d), d->wgt) == PATH_F32 ? PATH_F32 : PATH_BF16;
}

// Workspace of moe_layer_forward_shared: the routed layout, then h_s [T, Hs], y_s [T, H] and
// the one-group cu_seqlens [2].
static moe_status_t shared_layout(const moe_layer_desc_t* d, int32_t Hs, size_t* off, size_t* total,
                                  size_t* h_s, size_t* y_s, size_t* cu_s) {
  if (Hs < 1) return MOE_EINVAL;
  const moe_status_t st = layer_layout(d, off, total);
  if (st != MOE_OK) return st;
  const Path sp = shared_path(d);
  const size_t eb = sp == PATH_F32 ? 4 : 2, T = d->T, H = d->H;
  size_t o = align_up(*total, 256);
  *h_s = o;
  o = align_up(o + T * (size_t)Hs * eb, 256);
  *y_s = o;
  o = align_up(o + T * H * eb, 256);
  *cu_s = o;
  *total = o + 256;
  return MOE_OK;
}

size_t moe_layer_workspace_bytes(const moe_layer_desc_t* d) {
  size_t off[WS_N], total = 0;
  return layer_layout(d, off, &total) == MOE_OK ? total : 0;
}

moe_status_t moe_layer_workspace_layout(const moe_layer_desc_t* d, size_t* offsets, int32_t n) {
  size_t off[WS_N], total = 0;
  const moe_status_t st = layer_layout(d, off, &total);
  if (st != MOE_OK) return st;
  if (!offsets || n < 0) return MOE_EINVAL;
  for (int i = 0; i < n && i < WS_N; ++i) offsets[i] = off[i];
  return MOE_OK;
}

}  // extern "C"

namespace moe {

// Per-device events that order the shared expert's side stream with the main stream
// (created once per device, kept for the process lifetime).
static moe_status_t side_events(hipEvent_t** ev) {
  static hipEvent_t cache[64][2];
  static bool made[64] = {false};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_EHIP;
  if (!made[dev]) {
    for (int i = 0; i < 2; ++i)
      if (hipEventCreateWithFlags(&cache[dev][i], hipEventDisableTiming) != hipSuccess) return MOE_EHIP;
    made[dev] = true;
  }
  *ev = cache[dev];
  return MOE_OK;
}

struct SharedArgs {
  int32_t Hs = 0;
  const void* x_shared = nullptr;
  const void *w_gate = nullptr, *w_up = nullptr, *w_down = nullptr;
  hipStream_t side = nullptr;
};

static moe_status_t layer_forward_impl(const moe_layer_desc_t* d, const void* x, const float* x_sf,
                                       const float* logits, const int32_t* topk_idx_in,
                                       const float* topk_w_in, const void* w_gate, const void* w_up,
                                       const void* w_down, const uint8_t* sf_gate,
                                       const uint8_t* sf_up, const uint8_t* sf_down,
                                       const SharedArgs* sh, void* out, void* ws, size_t ws_bytes,
                                       hipStream_t stream) {
  size_t off[WS_N], total = 0, h_s_off = 0, y_s_off = 0, cu_s_off = 0;
  moe_status_t st = sh ? shared_layout(d, sh->Hs, off, &total, &h_s_off, &y_s_off, &cu_s_off)
                       : layer_layout(d, off, &total);
  if (st != MOE_OK) return st;
  if (!ws || ws_bytes < total) return MOE_EWORKSPACE;
  const Path p = ffn_path(layer_act(d), d->wgt);
  const moe_dtype_t act = layer_act(d);
  st = check_ffn_dims(p, (int64_t)d->T * d->K, d->E, d->H, d->Hp, true);
  if (st == MOE_OK) st = check_ffn_dims(p, (int64_t)d->T * d->K, d->E, d->H, d->Hp, false);
  if (st != MOE_OK) return st;
  if (d->T > 0 && (!x || !out || !w_gate || !w_up || !w_down)) return MOE_EINVAL;
  if (d->T > 0 && !logits && (!topk_idx_in || !topk_w_in)) return MOE_EINVAL;
  const Path sp = sh ? shared_path(d) : PATH_NONE;
  const void* xs = nullptr;
  if (sh) {
    st = check_ffn_dims(sp, d->T, 1, d->H, sh->Hs, true);
    if (st == MOE_OK) st = check_ffn_dims(sp, d->T, 1, d->H, sh->Hs, false);
    if (st != MOE_OK) return st;
    xs = sh->x_shared ? sh->x_shared : (d->act == MOE_FP8_E4M3 ? nullptr : x);
    if (d->T > 0 && (!xs || !sh->w_gate || !sh->w_up || !sh->w_down)) return MOE_EINVAL;
  }
  poison(ws, ws_bytes, stream);
  char* base = static_cast<char*>(ws);
  auto at = [&](int i) -> void* { return off[i] == SIZE_MAX ? nullptr : base + off[i]; };
  const int T = d->T, E = d->E, K = d->K, H = d->H, Hp = d->Hp, M = T * K;
  if (layer_quantizes(d) && T > 0) {
    // activation quantisation on entry: the routed experts read the fp8 rows from here on
    st = moe_quantize_fp8(x, MOE_BF16, T, H, static_cast<uint8_t*>(at(WS_XQ)),
                          static_cast<float*>(at(WS_XQ_SF)), stream);
    if (st != MOE_OK) return st;
    x = at(WS_XQ);
    x_sf = static_cast<float*>(at(WS_XQ_SF));
  }

  // The shared expert (one group of all T rows): its own two launches, on the side stream when
  // one is given. With MOE_SHARED_FOLD=1, when the routed FFN runs as the single launch and the
  // shared expert has the routed intermediate size, its tiles join that launch's queues as one
  // more expert instead ("Mixture of Kittens", Step 9: the shared expert's work overlaps the
  // routed experts'). That is bitwise the same and no faster: T=8192 E=384 K=8 with Hs=2048
  // took 8.43 ms against 8.42 ms. In a dynamic queue the shared expert's 32 m-tiles per weight
  // panel start staggered and lose the L2 sharing of the panel that the two-launch schedule's
  // rounds give them.
  void* y_s = sh ? base + y_s_off : nullptr;
  const bool fold = sh && T > 0 && layer_fused(d) && d->combine == MOE_COMBINE_GATHER && sp == PATH_BF16 &&
                    sh->Hs == Hp && E < 1024 && env_flag("MOE_SHARED_FOLD");
  SharedFold sfold;
  if (fold) {
    sfold.x = static_cast<const uint16_t*>(xs);
    sfold.wg = static_cast<const uint16_t*>(sh->w_gate);
    sfold.wu = static_cast<const uint16_t*>(sh->w_up);
    sfold.wd = static_cast<const uint16_t*>(sh->w_down);
    sfold.h = reinterpret_cast<uint16_t*>(base + h_s_off);
    sfold.y = static_cast<uint16_t*>(y_s);
    sfold.T = T;
  }
  hipEvent_t* ev = nullptr;
  const bool side = sh && sh->side && sh->side != stream && T > 0 && !fold;
  if (sh && T > 0 && !fold) {
    hipStream_t ss = stream;
    if (side) {
      st = side_events(&ev);
      if (st != MOE_OK) return st;
      if (hipEventRecord(ev[0], stream) != hipSuccess || hipStreamWaitEvent(sh->side, ev[0], 0) != hipSuccess)
        return MOE_EHIP;
      ss = sh->side;
    }
    int32_t* cu_s = reinterpret_cast<int32_t*>(base + cu_s_off);
    const moe_dtype_t sdt = sp == PATH_F32 ? MOE_F32 : MOE_BF16;
    st = launch_dense_cu(cu_s, T, ss);
    if (st == MOE_OK)
      st = moe_ffn_gate_up(xs, nullptr, sdt, cu_s, T, 1, H, sh->Hs, sh->w_gate, sh->w_up, nullptr,
                           nullptr, sdt, base + h_s_off, nullptr, ss);
    if (st == MOE_OK)
      st = moe_ffn_down(base + h_s_off, nullptr, sdt, cu_s, T, 1, H, sh->Hs, sh->w_down, nullptr, sdt,
                        y_s, sdt, ss);
    if (st != MOE_OK) return st;
    if (side && hipEventRecord(ev[1], sh->side) != hipSuccess) return MOE_EHIP;
  }
  auto join_side = [&]() -> moe_status_t {
    if (side && hipStreamWaitEvent(stream, ev[1], 0) != hipSuccess) return MOE_EHIP;
    return MOE_OK;
  };

  int32_t* topk_idx = static_cast<int32_t*>(at(WS_TOPK_IDX));
  float* topk_w = static_cast<float*>(at(WS_TOPK_W));
  if (!logits) {
    topk_idx = const_cast<int32_t*>(topk_idx_in);
    topk_w = const_cast<float*>(topk_w_in);
  }
  int32_t* counts = static_cast<int32_t*>(at(WS_COUNTS));
  int32_t* cu = static_cast<int32_t*>(at(WS_CU));
  int32_t* pos = static_cast<int32_t*>(at(WS_POS));
  int32_t* row_src = static_cast<int32_t*>(at(WS_ROW_SRC));
  float* row_w = static_cast<float*>(at(WS_ROW_W));
  float* h_sf = static_cast<float*>(at(WS_H_SF));
  const bool mat = layer_materializes(d), scatter = d->combine == MOE_COMBINE_SCATTER_ATOMIC;
  const size_t perm_ws = permute_ws_bytes(T, E, K);
  // routing from logits: top-k and the permutation's histogram come out of one kernel
  st = logits ? moe_route_permute(logits, x, x_sf, act, T, H, E, K, 1, topk_idx, topk_w, counts, cu, pos,
                                  row_src, row_w, at(WS_X_PERM), static_cast<float*>(at(WS_X_PERM_SF)),
                                  at(WS_PERM_SCRATCH), perm_ws, stream)
              : moe_permute(x, x_sf, act, topk_idx, topk_w, T, H, E, K, counts, cu, pos, row_src, row_w,
                            at(WS_X_PERM), static_cast<float*>(at(WS_X_PERM_SF)), at(WS_PERM_SCRATCH),
                            perm_ws, stream);
  if (st != MOE_OK) return st;
  if (layer_fused(d) && !scatter) {
    // gate/up and down in one persistent launch, then the deterministic combine
    st = launch_ffn_fused_bf16(x, row_src, T, K, cu, M, E, H, Hp, w_gate, w_up, w_down, at(WS_H), at(WS_Y),
                               static_cast<int*>(at(WS_FUSED_CTL)), stream, sfold, nullptr, nullptr);
    if (st == MOE_OK) st = join_side();
    if (st != MOE_OK) return st;
    return launch_combine(at(WS_Y), y_dtype_of(p), pos, topk_w, T, H, K, y_s, out, d->out, stream);
  }
  if (layer_fused(d)) {
    // one persistent launch whose down tiles add the weighted rows into the fp32 accumulator
    float* acc = d->out == MOE_F32 ? static_cast<float*>(out) : static_cast<float*>(at(WS_ACC));
    const size_t n = (size_t)T * H;
    if (n == 0) return join_side();
    st = launch_acc_zero(acc, n, stream);
    if (st == MOE_OK)
      st = launch_ffn_fused_bf16(x, row_src, T, K, cu, M, E, H, Hp, w_gate, w_up, w_down, at(WS_H), nullptr,
                                 static_cast<int*>(at(WS_FUSED_CTL)), stream, SharedFold{}, row_w, acc);
    if (st == MOE_OK) st = join_side();
    if (st != MOE_OK) return st;
    return launch_acc_store(acc, n, y_s, y_dtype_of(p), out, d->out, stream);
  }
  if (mat)
    st = moe_ffn_gate_up(at(WS_X_PERM), static_cast<float*>(at(WS_X_PERM_SF)), act, cu, M, E, H, Hp,
                         w_gate, w_up, sf_gate, sf_up, d->wgt, at(WS_H), h_sf, stream);
  else
    st = gate_up_gather(x, x_sf, static_cast<float*>(at(WS_X_PERM_SF)), act, row_src, T, K, cu, M, E,
                        H, Hp, w_gate, w_up, sf_gate, sf_up, d->wgt, at(WS_H), h_sf, stream);
  if (st != MOE_OK) return st;
  if (!scatter) {
    st = moe_ffn_down(at(WS_H), h_sf, h_dtype_of(p), cu, M, E, H, Hp, w_down, sf_down, d->wgt, at(WS_Y),
                      y_dtype_of(p), stream);
    if (st == MOE_OK) st = join_side();
    if (st != MOE_OK) return st;
    return launch_combine(at(WS_Y), y_dtype_of(p), pos, topk_w, T, H, K, y_s, out, d->out, stream);
  }
  // weighted scatter-add fused into the down projection, into an fp32 accumulator
  float* acc = d->out == MOE_F32 ? static_cast<float*>(out) : static_cast<float*>(at(WS_ACC));
  const size_t n = (size_t)T * H;
  if (n == 0) return MOE_OK;
  st = launch_acc_zero(acc, n, stream);
  if (st != MOE_OK) return st;
  st = moe_ffn_down_scatter(at(WS_H), h_sf, h_dtype_of(p), cu, M, E, H, Hp, w_down, sf_down, d->wgt,
                            row_src, row_w, T, K, acc, stream);
  if (st == MOE_OK) st = join_side();
  if (st != MOE_OK) return st;
  if (d->out == MOE_F32 && !y_s) return MOE_OK;
  return launch_acc_store(acc, n, y_s, y_dtype_of(p), out, d->out, stream);
}

}  // namespace moe

extern "C" {

moe_status_t moe_layer_forward(const moe_layer_desc_t* d, const void* x, const float* x_sf,
                               const float* logits, const int32_t* topk_idx_in,
                               const float* topk_w_in, const void* w_gate, const void* w_up,
                               const void* w_down, const uint8_t* sf_gate, const uint8_t* sf_up,
                               const uint8_t* sf_down, void* out, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  return layer_forward_impl(d, x, x_sf, logits, topk_idx_in, topk_w_in, w_gate, w_up, w_down, sf_gate,
                            sf_up, sf_down, nullptr, out, ws, ws_bytes, stream);
}

size_t moe_layer_shared_workspace_bytes(const moe_layer_desc_t* d, int32_t Hs) {
  size_t off[WS_N], total = 0, a, b, c;
  return shared_layout(d, Hs, off, &total, &a, &b, &c) == MOE_OK ? total : 0;
}

moe_status_t moe_layer_forward_shared(const moe_layer_desc_t* d, int32_t Hs, const void* x,
                                      const float* x_sf, const void* x_shared, const float* logits,
                                      const int32_t* topk_idx_in, const float* topk_w_in,
                                      const void* w_gate, const void* w_up, const void* w_down,
                                      const uint8_t* sf_gate, const uint8_t* sf_up,
                                      const uint8_t* sf_down, const void* ws_gate,
                                      const void* ws_up, const void* ws_down, void* out, void* ws,
                                      size_t ws_bytes, hipStream_t stream, hipStream_t side_stream) {
  SharedArgs sh;
  sh.Hs = Hs;
  sh.x_shared = x_shared;
  sh.w_gate = ws_gate;
  sh.w_up = ws_up;
  sh.w_down = ws_down;
  sh.side = side_stream;
  return layer_forward_impl(d, x, x_sf, logits, topk_idx_in, topk_w_in, w_gate, w_up, w_down, sf_gate,
                            sf_up, sf_down, &sh, out, ws, ws_bytes, stream);
}

// ---- layer backward ---------------------------------------------------------------------

enum {
  BW_TOPK_IDX, BW_TOPK_W, BW_COUNTS, BW_CU, BW_POS, BW_ROW_SRC, BW_ROW_W, BW_X_PERM, BW_G, BW_U,
  BW_H, BW_Y, BW_DY, BW_DG, BW_DU, BW_DW, BW_PERM_SCRATCH, BW_N
};

static moe_status_t bwd_check(const moe_layer_desc_t* d) {
  if (!d) return MOE_EINVAL;
  if (d->T < 0 || d->H < 1 || d->Hp < 1 || d->E < 1 || d->K < 1 || d->K > d->E) return MOE_EINVAL;
  if (d->act != MOE_BF16 || d->wgt != MOE_BF16 || d->out != MOE_BF16) return MOE_EUNSUPPORTED;
  if (d->E > 1024 || d->K > 32) return MOE_EUNSUPPORTED;
  if (d->H % 256 || d->Hp % 256) return MOE_EUNSUPPORTED;
  if ((int64_t)d->T * d->K * (d->H > d->Hp ? d->H : d->Hp) * 2 >= (1ll << 31)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

static moe_status_t bwd_layout(const moe_layer_desc_t* d, size_t* off, size_t* total) {
  const moe_status_t st = bwd_check(d);
  if (st != MOE_OK) return st;
  const size_t T = d->T, H = d->H, Hp = d->Hp, E = d->E, K = d->K, M = T * K;
  size_t sz[BW_N] = {M * 4, M * 4, E * 4, (E + 1) * 4, M * 4, M * 4, M * 4, M * H * 2, M * Hp * 2,
                     M * Hp * 2, M * Hp * 2, M * H * 2, M * H * 2, M * Hp * 2, M * Hp * 2, M * 4,
                     permute_ws_bytes(d->T, d->E, d->K)};
  size_t o = 0;
  for (int i = 0; i < BW_N; ++i) {
    off[i] = o;
    o = align_up(o + sz[i], 256);
  }
  *total = o + 256;
  return MOE_OK;
}

size_t moe_layer_backward_workspace_bytes(const moe_layer_desc_t* d) {
  size_t off[BW_N], total = 0;
  return bwd_layout(d, off, &total) == MOE_OK ? total : 0;
}

moe_status_t moe_layer_backward(const moe_layer_desc_t* d, const void* x, const float* logits,
                                const int32_t* topk_idx_in, const float* topk_w_in,
                                const void* w_gate, const void* w_up, const void* w_down,
                                const void* dout, void* dx, float* dw_gate, float* dw_up,
                                float* dw_down, float* d_topk_w, float* d_logits, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  size_t off[BW_N], total = 0;
  moe_status_t st = bwd_layout(d, off, &total);
  if (st != MOE_OK) return st;
  if (!ws || ws_bytes < total) return MOE_EWORKSPACE;
  if (!dw_gate || !dw_up || !dw_down || !w_gate || !w_up || !w_down) return MOE_EINVAL;
  if (d->T > 0 && (!x || !dout || !dx)) return MOE_EINVAL;
  if (d->T > 0 && !logits && (!topk_idx_in || !topk_w_in)) return MOE_EINVAL;
  poison(ws, ws_bytes, stream);
  char* base = static_cast<char*>(ws);
  auto at = [&](int i) -> void* { return base + off[i]; };
  const int T = d->T, E = d->E, K = d->K, H = d->H, Hp = d->Hp, M = T * K;
  int32_t* topk_idx = static_cast<int32_t*>(at(BW_TOPK_IDX));
  float* topk_w = static_cast<float*>(at(BW_TOPK_W));
  if (!logits) {
    topk_idx = const_cast<int32_t*>(topk_idx_in);
    topk_w = const_cast<float*>(topk_w_in);
  }
  int32_t* cu = static_cast<int32_t*>(at(BW_CU));
  int32_t* pos = static_cast<int32_t*>(at(BW_POS));
  int32_t* row_src = static_cast<int32_t*>(at(BW_ROW_SRC));
  float* row_w = static_cast<float*>(at(BW_ROW_W));
  int32_t* counts = static_cast<int32_t*>(at(BW_COUNTS));
  st = logits ? moe_route_permute(logits, x, nullptr, MOE_BF16, T, H, E, K, 1, topk_idx, topk_w, counts, cu,
                                  pos, row_src, row_w, at(BW_X_PERM), nullptr, at(BW_PERM_SCRATCH),
                                  permute_ws_bytes(T, E, K), stream)
              : moe_permute(x, nullptr, MOE_BF16, topk_idx, topk_w, T, H, E, K, counts, cu, pos, row_src,
                            row_w, at(BW_X_PERM), nullptr, at(BW_PERM_SCRATCH), permute_ws_bytes(T, E, K),
                            stream);
  if (st != MOE_OK) return st;
  // forward recomputed, keeping g and u
  RowMaps save;
  save.save_g = static_cast<uint16_t*>(at(BW_G));
  save.save_u = static_cast<uint16_t*>(at(BW_U));
  if (M > 0) {
    st = launch_ffn_gate_up_bf16(at(BW_X_PERM), cu, M, E, H, Hp, w_gate, w_up, at(BW_H), save, stream);
    if (st == MOE_OK) st = launch_ffn_down_bf16(at(BW_H), cu, M, E, H, Hp, w_down, at(BW_Y), RowMaps{}, stream);
    if (st != MOE_OK) return st;
  }
  // combine backward: dy and the routing-weight gradient (then the top-k softmax backward)
  float* dw = d_topk_w ? d_topk_w : static_cast<float*>(at(BW_DW));
  st = launch_combine_bwd(dout, at(BW_Y), pos, topk_w, T, H, K, at(BW_DY), dw, stream);
  if (st == MOE_OK && logits && d_logits) st = launch_route_bwd(topk_idx, topk_w, dw, T, E, K, d_logits, stream);
  if (st != MOE_OK) return st;
  // down: dh with the SwiGLU backward fused (dg, du), and dWd = h^T dy
  if (M > 0) {
    st = launch_bwd_down_swiglu(at(BW_DY), cu, M, E, H, Hp, w_down, at(BW_G), at(BW_U), at(BW_DG), at(BW_DU),
                                stream);
    if (st != MOE_OK) return st;
  }
  st = launch_bwd_wgrad(at(BW_H), at(BW_DY), cu, E, Hp, H, dw_down, stream);
  if (st != MOE_OK) return st;
  // gate/up: dx_rows = dg Wg^T + du Wu^T (into the y buffer, no longer needed), the weights'
  // gradients, then the dispatch backward (unit-weight combine of dx_rows)
  if (M > 0) {
    st = launch_bwd_gate_up(at(BW_DG), at(BW_DU), cu, M, E, H, Hp, w_gate, w_up, at(BW_Y), stream);
    if (st != MOE_OK) return st;
  }
  st = launch_bwd_wgrad(at(BW_X_PERM), at(BW_DG), cu, E, H, Hp, dw_gate, stream);
  if (st == MOE_OK) st = launch_bwd_wgrad(at(BW_X_PERM), at(BW_DU), cu, E, H, Hp, dw_up, stream);
  if (st != MOE_OK) return st;
  return launch_combine(at(BW_Y), MOE_BF16, pos, nullptr, T, H, K, nullptr, dx, MOE_BF16, stream);
}

}  // extern "C"
