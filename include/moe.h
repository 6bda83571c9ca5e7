/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE-layer hot path: top-k routing, permute into
 * expert-contiguous rows, grouped SwiGLU expert FFN over stacked weights, and the
 * weighted combine back to token order, all on one GPU.
 *
 * The operations follow these pages:
 *  - "Mixture of Kittens" (MoE megakernel article), Step 1 "The Math": a router picks the
 *    top-k experts of each token, each expert is Down(SwiGLU(Up x, Gate x)), and the
 *    routed outputs are summed with their router weights.
 *  - "Distributed expert parallelism" (open-llm-engineering), "The dispatch-compute-combine
 *    lifecycle", "Token permutation and metadata" and "Grouped expert computation": copy each
 *    token k times, group the copies by expert, run one grouped GEMM over the groups, restore
 *    token order, scale by route weights and add.
 *  - MoonEP README, "Integration" / "Weight buffer" and "API walkthrough": stacked contiguous
 *    expert weights addressed purely by expert index, cu_seqlens selecting each expert's rows,
 *    dispatch/combine taking [S,H] activations, [S,K] fp32 weights and [S,K] int32 expert ids.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers, row-major and densely packed, unless stated otherwise.
 *    The caller owns every buffer and keeps it alive until the stream has passed the call.
 *    The library never allocates, frees or retains caller memory.
 *  - Calls only enqueue work on `stream` and return; there is no host synchronisation, except
 *    when the environment variable MOE_VALIDATE=1 asks for the data checks described below.
 *    All shapes are static (M = T*K rows), cu_seqlens stays on the device.
 *  - Errors are returned as moe_status_t; nothing is thrown. Argument checks happen on the
 *    host before anything is enqueued: MOE_EINVAL (bad sizes, NULL where a buffer is needed,
 *    K > E), MOE_EUNSUPPORTED (a dtype combination or a dimension multiple the library does not
 *    implement), MOE_EWORKSPACE (workspace too small). A failed launch gives MOE_EHIP.
 *  - T = 0 and experts that receive no rows are legal and produce valid (empty) groups.
 *  - Expert ids outside [0, E) in a caller-given top-k are memory-safe: that copy is dropped
 *    (pos = -1, no row, no contribution). With MOE_VALIDATE=1 the library also checks for
 *    such ids and for an expert repeated within one token, synchronises the stream and
 *    returns MOE_EINVAL if any is found.
 *  - MOE_DEBUG_POISON=1 fills the whole workspace with 0xFF bytes (NaN in every float
 *    format) before use, so a read of an unwritten workspace byte shows up as NaN.
 *
 * Notation: T tokens, H hidden size, Hp expert intermediate size (H'), E experts (or expert
 * slots), K experts per token, M = T*K routed rows.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#define MOE_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,
  MOE_EUNSUPPORTED = 2,
  MOE_EWORKSPACE = 3,
  MOE_EHIP = 4
} moe_status_t;

/* Storage formats.
 *  MOE_F32       IEEE binary32.
 *  MOE_BF16      bfloat16 (top half of binary32), results rounded to nearest even.
 *  MOE_FP8_E4M3  OCP e4m3fn bytes (bias 7, max 448, no infinities). Activations in this
 *                format come with fp32 scales, one per 1x128 block along the row, each an
 *                exact power of two: value = decode(code) * scale[row][col / 128].
 *  MOE_MXFP4     OCP MX e2m1 codes, two per byte, with one e8m0 scale byte per 32 elements
 *                along the reduction dimension: value = e2m1(code) * 2^(scale - 127).
 *                Stored reduction-contiguous: byte j of output column n holds reduction
 *                index 2j in its low nibble and 2j+1 in its high nibble. Scale bytes are
 *                stored block-major, [K/32][N] per expert, so the scales one K step needs
 *                for consecutive columns are contiguous.
 *  MOE_MXFP4_PAIRED  the same codes and scales with the code bytes of each expert matrix in
 *                the paired layout [N/2][K/128][2][64]: for columns 2p and 2p+1 and each step
 *                of 128 reduction elements, column 2p's 64 bytes then column 2p+1's, so one
 *                128-byte line holds both (written by moe_pack_mxfp4_pairs). Accepted wherever
 *                MOE_MXFP4 weights are, with bitwise the same results. */
typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_FP8_E4M3 = 2,
  MOE_MXFP4 = 3,
  MOE_MXFP4_PAIRED = 4
} moe_dtype_t;

/* How the K expert results of a token are summed.
 *  MOE_COMBINE_GATHER  deterministic gather-reduce in fixed k order (bitwise reproducible),
 *                      following "Mixture of Kittens", Step 8 "Full Determinism".
 *  MOE_COMBINE_SCATTER_ATOMIC  weighted scatter-add fused into the down-projection epilogue
 *                      (fp32 atomics; the sum order, hence the last bit, may vary). */
typedef enum { MOE_COMBINE_GATHER = 0, MOE_COMBINE_SCATTER_ATOMIC = 1 } moe_combine_t;

/* Whole-layer description. Supported (act, wgt, out) combinations:
 *  (F32, F32, F32), (BF16, BF16, BF16), (FP8_E4M3, MXFP4, BF16), and (BF16, MXFP4, BF16):
 *  BF16 activations quantised on entry to FP8_E4M3 with 1x128 scales (moe_quantize_fp8),
 *  then the FP8_E4M3 x MXFP4 path. MXFP4_PAIRED may stand for MXFP4 in both. */
typedef struct {
  int32_t T, H, Hp, E, K;
  moe_dtype_t act, wgt, out;
  moe_combine_t combine;
} moe_layer_desc_t;

/* Top-k routing ("Mixture of Kittens", Step 1; "Distributed expert parallelism", lifecycle
 * item 1).
 *  logits    [T, E] fp32.
 *  topk_idx  [T, K] int32 out: the K experts with the largest logits, largest first; equal
 *            logits are ordered by ascending expert id.
 *  topk_w    [T, K] fp32 out: softmax over the K selected logits (= the full softmax
 *            renormalised over the top K): w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).
 * Limits: 1 <= K <= min(E, 32), E <= 4096. */
MOE_API moe_status_t moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t K,
                            int32_t* topk_idx, float* topk_w, hipStream_t stream);

/* Scratch bytes moe_permute needs for (T, E, K). */
MOE_API size_t moe_permute_workspace_bytes(int32_t T, int32_t E, int32_t K);

/* Permute token copies into expert-contiguous rows ("Distributed expert parallelism",
 * "Token permutation and metadata"; MoonEP "dispatch fwd" without the remote writes).
 *  x          [T, H] activations of format `act` (F32, BF16 or FP8_E4M3).
 *  x_sf       [T, H/128] fp32 block scales when act = FP8_E4M3, else ignored (may be NULL).
 *  topk_idx   [T, K] int32 expert ids; topk_w [T, K] fp32 (may be NULL when row_w is NULL).
 *  counts     [E] int32 out: copies routed to each expert.
 *  cu_seqlens [E+1] int32 out: cu_seqlens[0] = 0, cu_seqlens[e+1] = cu_seqlens[e] + counts[e].
 *  pos        [T, K] int32 out: row of copy (t, k); -1 for a dropped (invalid-id) copy.
 *  row_src    [T*K] int32 out: flat index t*K + k of the copy stored in each row.
 *  row_w      [T*K] fp32 out (or NULL): topk_w of the copy stored in each row.
 *  x_perm     [T*K, H] out, format `act`: x_perm[pos[t,k]] = x[t], bit for bit. May be NULL:
 *             then x is not read, for consumers that gather rows through row_src, such as
 *             moe_ffn_gate_up_gather.
 *  x_perm_sf  [H/128, T*K] fp32 out or NULL, block-major: x_perm_sf[b][r] is the scale of
 *             block b of row r (the transpose of x_sf's layout). act = FP8_E4M3 only, where
 *             it is required with x_perm and may also be given without it (then x_sf is
 *             required and only the scales are permuted: T*K*H/32 bytes, against T*K*H for
 *             the rows). Rows past cu_seqlens[E] (dropped copies) are not written.
 * Row order is a stable counting sort: the rows of expert e hold its copies in ascending
 * t*K + k. The result is deterministic. Limits: E <= 1024, K <= 32. */
MOE_API moe_status_t moe_permute(const void* x, const float* x_sf, moe_dtype_t act,
                         const int32_t* topk_idx, const float* topk_w, int32_t T, int32_t H,
                         int32_t E, int32_t K, int32_t* counts, int32_t* cu_seqlens,
                         int32_t* pos, int32_t* row_src, float* row_w, void* x_perm,
                         float* x_perm_sf, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_permute for callers that cannot allocate device memory or pass a workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments,
 * outputs (bit for bit) and limits as moe_permute, without ws / ws_bytes: the sort's scratch
 * (the per-chunk histograms, ceil(T/16)*E*4 bytes + 256) lives in a static 4 MiB device array
 * of the library, one per device, held until the process ends. The call allocates nothing
 * and enqueues kernels only.
 *  - Returns MOE_EUNSUPPORTED, before touching the device, when ceil(T/16)*E*4 + 256 bytes
 *    exceed 4 MiB (e.g. T = 8192 allows E <= 2047 within the E <= 1024 limit; E = 1024 allows
 *    T <= 16368); MOE_EHIP if the scratch's device address cannot be obtained.
 *  - Every call on one device uses that device's one array, which keeps the last call's
 *    contents (every entry a call reads is written by that call first). Calls that can overlap
 *    on one device (different streams without ordering, or several host threads) race on it:
 *    order them on one stream.
 *  - MOE_VALIDATE and MOE_DEBUG_POISON do not apply (both need host-side work). */
MOE_API moe_status_t moe_permute_noalloc(const void* x, const float* x_sf, moe_dtype_t act,
                                 const int32_t* topk_idx, const float* topk_w, int32_t T,
                                 int32_t H, int32_t E, int32_t K, int32_t* counts,
                                 int32_t* cu_seqlens, int32_t* pos, int32_t* row_src,
                                 float* row_w, void* x_perm, float* x_perm_sf,
                                 hipStream_t stream);

/* The static-capacity (padded) variant of moe_permute (MoonEP "API walkthrough": buffer
 * token_padding and a padded cu_seqlens; "Distributed expert parallelism", "Static-capacity
 * versus dropless dispatch" and "Hidden padding in metrics"): every expert group is padded
 * up to a multiple of `pad` rows inside a static buffer of moe_padded_capacity(T, E, K, pad)
 * = T*K + E*(pad-1) rows, which holds any routing.
 *  counts      [E] out: the real copies per expert (log these beside the padded sizes).
 *  cu_seqlens  [E+1] out: padded group offsets, cu[e+1] - cu[e] = ceil(counts[e]/pad)*pad.
 *  row_src, row_w [capacity] out: real rows as in moe_permute; padding rows (inside the
 *              groups and past cu[E]) hold row_src = -1 and row_w = 0.
 *  x_perm      [capacity, H] out or NULL: real rows as in moe_permute, padding rows inside
 *              the groups zero; x_perm_sf [H/128, capacity] (FP8) with scale 1 for them.
 * The grouped FFN entry points accept the padded cu_seqlens with M = capacity; padding rows
 * compute zeros (and are skipped by the gather and scatter row maps, which read
 * row_src = -1 as a padding row). Other arguments and limits as moe_permute; pad >= 1
 * (pad = 1 is moe_permute). */
MOE_API int64_t moe_padded_capacity(int32_t T, int32_t E, int32_t K, int32_t pad);

MOE_API moe_status_t moe_permute_padded(const void* x, const float* x_sf, moe_dtype_t act,
                                const int32_t* topk_idx, const float* topk_w, int32_t T, int32_t H,
                                int32_t E, int32_t K, int32_t pad, int32_t* counts,
                                int32_t* cu_seqlens, int32_t* pos, int32_t* row_src, float* row_w,
                                void* x_perm, float* x_perm_sf, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* Routing and the permutation in one call: moe_route_topk on `logits` followed by
 * moe_permute_padded on its result, with the same outputs bit for bit ("Distributed expert
 * parallelism", lifecycle items 1-3). The first kernel ranks the tokens of each 16-token
 * chunk and counts the chunk's picks per expert, which saves the permutation's separate
 * histogram pass and one launch.
 *  logits [T, E] fp32 in; topk_idx [T, K] int32 and topk_w [T, K] fp32 out (both required);
 *  every other argument, the workspace (moe_permute_workspace_bytes) and the limits as
 *  moe_permute_padded, with K <= E. The ids are produced here, so MOE_VALIDATE has nothing
 *  to check. */
MOE_API moe_status_t moe_route_permute(const float* logits, const void* x, const float* x_sf,
                               moe_dtype_t act, int32_t T, int32_t H, int32_t E, int32_t K,
                               int32_t pad, int32_t* topk_idx, float* topk_w, int32_t* counts,
                               int32_t* cu_seqlens, int32_t* pos, int32_t* row_src, float* row_w,
                               void* x_perm, float* x_perm_sf, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* MXFP4 weight codes to the paired layout of MOE_MXFP4_PAIRED (the MoonEP news article,
 * "Design principles and technical details": the weights are laid out for the GEMM). The
 * fp8 x MXFP4 kernels stage 64 bytes of each column per K step; in the stored layout that is
 * half a 128-byte line, in the paired layout two columns share each line, which halves the
 * lines a weight load touches. A one-time preparation of a weight tensor, like loading it:
 *  w [E, N, K/2] code bytes (MOE_MXFP4 layout of one projection: N output columns, reduction
 *  K); w_paired [E, N/2, K/128, 2, 64] out, same size, not overlapping w. Both 16-byte
 *  aligned. Needs N % 2 == 0 and K % 128 == 0 (MOE_EUNSUPPORTED otherwise). The scale bytes
 *  are not touched: they keep their layout. One kernel launch, HBM-bound. */
MOE_API moe_status_t moe_pack_mxfp4_pairs(const uint8_t* w, uint8_t* w_paired, int32_t E, int32_t N,
                                          int32_t K, hipStream_t stream);

/* Activation quantisation to FP8_E4M3 with 1x128 power-of-two scales ("Mixture of
 * Kittens", Step 8: activations are quantised for the fp8 GEMMs, fused into dispatch):
 * for each row r and block b of 128 columns, s[r][b] = the smallest power of two with
 * 448*s >= max |x[r][128b..128b+127]| (1 for an all-zero block) and
 * q[r][c] = e4m3fn round-to-nearest-even(x[r][c] / s[r][b]) (an exact zero gives code 0).
 *  x [R, C] of x_dtype (BF16 or F32), 16-byte aligned, C % 128 == 0;
 *  q [R, C] codes out (8-byte aligned); sf [R, C/128] fp32 out (the x_sf layout). */
MOE_API moe_status_t moe_quantize_fp8(const void* x, moe_dtype_t x_dtype, int32_t R, int32_t C,
                              uint8_t* q, float* sf, hipStream_t stream);

/* First half of the grouped expert FFN ("Mixture of Kittens", Step 1; "Distributed expert
 * parallelism", "Grouped expert computation"): for every expert e and its rows
 * r in [cu_seqlens[e], cu_seqlens[e+1]):
 *     g = x_perm[r] . Wg[e],  u = x_perm[r] . Wu[e],  h[r] = silu(g) * u,
 * silu(z) = z / (1 + exp(-z)), accumulated in fp32.
 *  Formats: act F32 + wgt F32 -> h F32; act BF16 + wgt BF16 -> h BF16;
 *           act FP8_E4M3 + wgt MXFP4 -> h FP8_E4M3 with h_sf [Hp/128, M] (block-major) fp32
 *           power-of-two
 *           scales (s = smallest power of two with 448*s >= block amax; code = e4m3fn
 *           round-to-nearest-even of h/s).
 *  F32/BF16 weights: w_gate, w_up [E, H, Hp] (g = x . W). MXFP4 weights: bytes [E, Hp, H/2]
 *  with sf_gate, sf_up [E, H/32, Hp]; x_perm_sf [H/128, M].
 * One kernel launch; the tile schedule over the variable-size groups is derived on the device
 * from cu_seqlens. Needs H % 64 == 0 and Hp % 128 == 0 (BF16), H % 128 == 0 and
 * Hp % 128 == 0 (FP8/MXFP4); F32 has no multiple requirement. */
MOE_API moe_status_t moe_ffn_gate_up(const void* x_perm, const float* x_perm_sf, moe_dtype_t act,
                             const int32_t* cu_seqlens, int32_t M, int32_t E, int32_t H,
                             int32_t Hp, const void* w_gate, const void* w_up,
                             const uint8_t* sf_gate, const uint8_t* sf_up, moe_dtype_t wgt,
                             void* h, float* h_sf, hipStream_t stream);

/* moe_ffn_gate_up with its input rows gathered from the token matrix instead of a permuted
 * copy ("Mixture of Kittens", Step 6 reads each expert's tokens through their indices; the
 * DeepGEMM Mega-MoE how-to fuses dispatch into the expert GEMM): row r of expert e's group
 * is x[row_src[r] / K], so
 *     h[r] = silu(x[row_src[r]/K] . Wg[e]) * (x[row_src[r]/K] . Wu[e]),
 * bitwise the same h as moe_ffn_gate_up on the x_perm that moe_permute would write.
 *  x [T, H] of format `act`; row_src [M] from moe_permute or moe_permute_padded (a row with
 *  row_src = -1 is a padding row and reads zeros); other arguments as moe_ffn_gate_up.
 *  FP8_E4M3 only, one of the two scale layouts (ignored otherwise, may be NULL):
 *  x_perm_sf  [H/128, M] fp32, the permuted block-major scales that moe_permute writes when
 *             given x_perm_sf without x_perm. Preferred: each stage reads them as contiguous
 *             runs, once per row instead of once per row and output tile.
 *  x_sf       [T, H/128] fp32, the token layout of moe_permute's x_sf, read when x_perm_sf
 *             is NULL: each row's scales are gathered through row_src.
 * Needs T*H*bytes(act) < 2^31 (MOE_EUNSUPPORTED otherwise). */
MOE_API moe_status_t moe_ffn_gate_up_gather(const void* x, const float* x_sf,
                                    const float* x_perm_sf, moe_dtype_t act,
                                    const int32_t* row_src, int32_t T, int32_t K,
                                    const int32_t* cu_seqlens, int32_t M, int32_t E, int32_t H,
                                    int32_t Hp, const void* w_gate, const void* w_up,
                                    const uint8_t* sf_gate, const uint8_t* sf_up, moe_dtype_t wgt,
                                    void* h, float* h_sf, hipStream_t stream);

/* Second half of the grouped expert FFN: y_rows[r] = h[r] . Wd[e] for the rows of expert e.
 *  h_dtype F32 (wgt F32, out F32), BF16 (wgt BF16, out BF16) or FP8_E4M3 with h_sf
 *  (wgt MXFP4, out BF16). F32/BF16 w_down [E, Hp, H]; MXFP4 bytes [E, H, Hp/2] with
 *  sf_down [E, Hp/32, H]; h_sf [Hp/128, M]. Needs H % 256 == 0 and Hp % 64 == 0 (BF16), H % 128 == 0 and
 *  Hp % 128 == 0 (FP8/MXFP4). One kernel launch. */
MOE_API moe_status_t moe_ffn_down(const void* h, const float* h_sf, moe_dtype_t h_dtype,
                          const int32_t* cu_seqlens, int32_t M, int32_t E, int32_t H,
                          int32_t Hp, const void* w_down, const uint8_t* sf_down,
                          moe_dtype_t wgt, void* y_rows, moe_dtype_t out, hipStream_t stream);

/* moe_ffn_down with the weighted combine fused into its epilogue (DeepGEMM Mega-MoE how-to:
 * combine fused into the expert kernel; MoonEP "combine fwd" weights the rows): for every row
 * r of expert e's group,
 *     acc[row_src[r] / K] += row_w[r] * (h[r] . Wd[e]),
 * added with fp32 atomics, so the order of the K additions of a token (and its last bit) may
 * vary between runs. acc [T, H] fp32 is accumulated into: the caller zeroes it first.
 * row_src, row_w [M] from moe_permute or moe_permute_padded (rows with row_src = -1 are
 * skipped). Formats and limits as moe_ffn_down (y_rows is not written). */
MOE_API moe_status_t moe_ffn_down_scatter(const void* h, const float* h_sf, moe_dtype_t h_dtype,
                                  const int32_t* cu_seqlens, int32_t M, int32_t E, int32_t H,
                                  int32_t Hp, const void* w_down, const uint8_t* sf_down,
                                  moe_dtype_t wgt, const int32_t* row_src, const float* row_w,
                                  int32_t T, int32_t K, float* acc, hipStream_t stream);

/* Scratch bytes moe_grouped_ffn needs (the intermediate h and its scales). */
MOE_API size_t moe_grouped_ffn_workspace_bytes(int32_t M, int32_t Hp, moe_dtype_t act, moe_dtype_t wgt);

/* moe_ffn_gate_up followed by moe_ffn_down, with h kept in `ws`. y_rows [M, H] of format
 * `out`. MoonEP "Integration": the group GEMM consumes one stacked weight tensor per
 * projection and cu_seqlens selects the rows of each expert. */
MOE_API moe_status_t moe_grouped_ffn(const void* x_perm, const float* x_perm_sf, moe_dtype_t act,
                             const int32_t* cu_seqlens, int32_t M, int32_t E, int32_t H,
                             int32_t Hp, const void* w_gate, const void* w_up,
                             const void* w_down, const uint8_t* sf_gate, const uint8_t* sf_up,
                             const uint8_t* sf_down, moe_dtype_t wgt, void* y_rows,
                             moe_dtype_t out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Scratch bytes moe_grouped_ffn_fused needs for M rows, E experts and intermediate size Hp:
 * h [M, Hp] bf16 at offset 0, then the control words at offset align_up(M*Hp*2, 256). The
 * control words are int32: [0, 8) queue counters, 8 error flag (0 when the call succeeded;
 * 1: a readiness wait exceeded its bound of about a second, 2: a queue entry matched no tile;
 * the results are then invalid), 9 tiles run, 10 tiles started without
 * prefetch because their rows were not ready, 11 tiles taken from another XCD's queue, then
 * from 16 on one readiness counter per m-tile. 0 if the arguments are invalid. */
MOE_API size_t moe_grouped_ffn_fused_workspace_bytes(int32_t M, int32_t E, int32_t Hp);

/* The bf16 grouped expert FFN in one persistent launch ("Mixture of Kittens", Step 7, the
 * megakernel whose blocks coordinate through counters in global memory; the DeepGEMM
 * Mega-MoE how-to, dispatch and both expert GEMMs in one kernel): gate/up + SwiGLU with rows
 * gathered from x through row_src (as moe_ffn_gate_up_gather), then the down projection, as
 * tiles of device-side work queues. A down tile starts as soon as the 256-row block of h it
 * reads is complete, so the two projections overlap instead of running as two launches.
 *     h[r] = silu(x[row_src[r]/K] . Wg[e]) * (x[row_src[r]/K] . Wu[e]),  y_rows[r] = h[r] . Wd[e]
 * for the rows r of expert e, bitwise the same y_rows (and h) as moe_ffn_gate_up_gather
 * followed by moe_ffn_down.
 *  x [T, H] bf16; row_src [M] from moe_permute (-1: padding row, reads zeros); cu_seqlens
 *  [E+1]; w_gate, w_up [E, H, Hp], w_down [E, Hp, H] bf16; y_rows [M, H] bf16 out. act, wgt
 *  and out must be MOE_BF16 (MOE_EUNSUPPORTED otherwise). ws: moe_grouped_ffn_fused_workspace_bytes
 *  bytes, holding h and the control words (layout above); they are reset on every call, so
 *  calls sharing a workspace must be ordered (same stream).
 * Needs H % 256 == 0, Hp % 128 == 0, H >= 256, Hp >= 256, E <= 1024 and T*H*2 < 2^31
 * (MOE_EUNSUPPORTED otherwise). Two kernel launches: a reset of the control words and the
 * persistent kernel. Test hooks: MOE_FUSED_LAG=n queues each expert's down tiles n experts
 * behind its gate/up tiles (default: all gate/up tiles of a queue first), and
 * MOE_FUSED_SPIN_MAX=n lowers the bound of a readiness wait to n polls (error 1 when reached). */
MOE_API moe_status_t moe_grouped_ffn_fused(const void* x, moe_dtype_t act, const int32_t* row_src,
                                   int32_t T, int32_t K, const int32_t* cu_seqlens, int32_t M,
                                   int32_t E, int32_t H, int32_t Hp, const void* w_gate,
                                   const void* w_up, const void* w_down, moe_dtype_t wgt,
                                   void* y_rows, moe_dtype_t out, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* moe_grouped_ffn_fused with the weighted combine in the down tiles' epilogue instead of
 * y_rows (DeepGEMM Mega-MoE how-to: dispatch, both expert GEMMs, SwiGLU and the combine in
 * one kernel; MoonEP "combine fwd" weights the rows): for every row r of expert e's group,
 *     acc[row_src[r] / K] += row_w[r] * (h[r] . Wd[e]),
 * added with fp32 atomics, as moe_ffn_down_scatter does, so the order of a token's K
 * additions (and its last bit) may vary between runs. acc [T, H] fp32 is accumulated into:
 * the caller zeroes it first. row_w [M] from moe_permute; rows with row_src = -1 are skipped.
 * Other arguments, the workspace (h and the control words), limits and launches as
 * moe_grouped_ffn_fused; act and wgt must be MOE_BF16. */
MOE_API moe_status_t moe_grouped_ffn_fused_scatter(const void* x, moe_dtype_t act, const int32_t* row_src,
                                           int32_t T, int32_t K, const int32_t* cu_seqlens, int32_t M,
                                           int32_t E, int32_t H, int32_t Hp, const void* w_gate,
                                           const void* w_up, const void* w_down, moe_dtype_t wgt,
                                           const float* row_w, float* acc, void* ws, size_t ws_bytes,
                                           hipStream_t stream);

/* Combine ("Distributed expert parallelism", lifecycle item 8 and "A four-rank example";
 * MoonEP "combine fwd"): out[t] = sum_{k=0..K-1} topk_w[t,k] * y_rows[pos[t,k]], summed in
 * fp32 in increasing k and rounded once to `out_dtype`; rows with pos < 0 are skipped.
 *  y_rows [T*K, H] of y_dtype (F32 or BF16); out [T, H] of out_dtype (F32 or BF16).
 *  topk_w may be NULL: unit weights (the sum of a token's rows, as in the dispatch backward).
 * Deterministic: the same inputs give bitwise the same output. */
MOE_API moe_status_t moe_combine(const void* y_rows, moe_dtype_t y_dtype, const int32_t* pos,
                         const float* topk_w, int32_t T, int32_t H, int32_t K, void* out,
                         moe_dtype_t out_dtype, hipStream_t stream);

/* moe_combine with the shared expert's output added to each token ("Mixture of Kittens",
 * Step 1, "The Math": MoE(x) = SharedExpert(x) + sum_k w_k * RoutedExpert_k(x)):
 *   out[t] = (sum_{k=0..K-1} topk_w[t,k] * y_rows[pos[t,k]]) + shared_y[t],
 * summed in fp32 (k in increasing order, then the shared row) and rounded once.
 *  shared_y [T, H] of y_dtype. Deterministic. */
MOE_API moe_status_t moe_combine_shared(const void* y_rows, moe_dtype_t y_dtype, const int32_t* pos,
                                const float* topk_w, int32_t T, int32_t H, int32_t K,
                                const void* shared_y, void* out, moe_dtype_t out_dtype,
                                hipStream_t stream);

/* Workspace bytes of moe_layer_forward for `d` (0 if `d` is invalid). */
MOE_API size_t moe_layer_workspace_bytes(const moe_layer_desc_t* d);

/* The whole layer on one stream, no host synchronisation ("Distributed expert parallelism",
 * "The dispatch-compute-combine lifecycle", without the exchanges):
 *   route (skipped when logits == NULL: topk_idx_in / topk_w_in are used instead)
 *   -> permute metadata (counts, cu_seqlens, pos, row_src)
 *   -> gate/up + SwiGLU, its rows gathered from x (moe_ffn_gate_up_gather; with the
 *      environment variable MOE_LAYER_XPERM=1, or when T*H*bytes(act) >= 2^31, x_perm is
 *      written by moe_permute and read instead: same result, bit for bit). A bf16 layer
 *      with the gather combine, on the shapes moe_grouped_ffn_fused takes and with
 *      T*K <= 256*E (about one 256-row tile per expert), runs gate/up and down as that one
 *      persistent launch instead (same result, bit for bit); MOE_LAYER_FUSED=1 or 0 forces
 *      the choice.
 *   -> d->combine == MOE_COMBINE_GATHER: down -> y_rows -> moe_combine (deterministic);
 *      d->combine == MOE_COMBINE_SCATTER_ATOMIC: down with the weighted scatter-add fused
 *      into its epilogue (moe_ffn_down_scatter) into an fp32 accumulator (the output itself
 *      when d->out is F32, else a workspace buffer rounded once into out at the end). With
 *      this combine the FFN runs as two launches unless MOE_LAYER_FUSED=1 asks for the
 *      single launch, which then adds the rows in its down epilogue
 *      (moe_grouped_ffn_fused_scatter; bf16 layers on the shapes it takes).
 *  x [T, H] (format d->act, with x_sf for FP8_E4M3); logits [T, E] fp32 or NULL;
 *  topk_idx_in / topk_w_in [T, K] when logits == NULL; weights as for moe_grouped_ffn;
 *  out [T, H] of d->out, 16-byte aligned. `ws` must hold moe_layer_workspace_bytes(d) bytes;
 *  the intermediates live there, at offsets reported by moe_layer_workspace_layout. */
MOE_API moe_status_t moe_layer_forward(const moe_layer_desc_t* d, const void* x, const float* x_sf,
                               const float* logits, const int32_t* topk_idx_in,
                               const float* topk_w_in, const void* w_gate, const void* w_up,
                               const void* w_down, const uint8_t* sf_gate, const uint8_t* sf_up,
                               const uint8_t* sf_down, void* out, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* Workspace bytes of moe_layer_forward_shared for `d` and shared intermediate size Hs (0 if
 * invalid): the moe_layer_forward workspace followed by h_s [T, Hs], y_s [T, H] (bf16, fp32
 * for an F32 layer) and a two-entry cu_seqlens. */
MOE_API size_t moe_layer_shared_workspace_bytes(const moe_layer_desc_t* d, int32_t Hs);

/* moe_layer_forward plus a shared expert ("Mixture of Kittens", Step 1: every token also
 * goes through one shared expert whose output is added to the weighted routed sum):
 *   out[t] = SharedExpert(xs[t]) + sum_k topk_w[t,k] * Expert_{topk_idx[t,k]}(x[t]),
 *   SharedExpert(v) = (silu(v . Ws_gate) * (v . Ws_up)) . Ws_down.
 * The shared expert runs in BF16 (F32 for an F32 layer) even when the routed experts are
 * FP8 x MXFP4 ("Mixture of Kittens", Step 8: the shared expert stays in BF16); it is one
 * grouped-GEMM group of all T rows. Its input xs is x_shared [T, H] when given, else x
 * (x_shared is required for an FP8_E4M3 layer: the BF16 activations). Weights ws_gate,
 * ws_up [H, Hs], ws_down [Hs, H] in that format; needs the moe_ffn_gate_up / moe_ffn_down
 * limits with Hp = Hs. Its output is added in the combine (gather: moe_combine_shared;
 * scatter: to the fp32 accumulator before the rounding).
 * With the environment variable MOE_SHARED_FOLD=1, when the routed FFN runs as the single
 * persistent launch (see moe_layer_forward) and Hs = Hp, the shared expert's tiles join that
 * launch's queues as one more expert, alongside the routed tiles ("Mixture of Kittens",
 * Step 9); side_stream is then not used, and the result is bitwise the same.
 * side_stream: otherwise, when non-NULL and different from `stream`, the shared expert runs there,
 * overlapping the routed path ("Mixture of Kittens", Step 9: the shared expert FFN overlaps
 * the first dispatch); the call orders it after the work already on `stream` and makes
 * `stream` wait for it before the combine, so completion on `stream` covers everything.
 * Calls that overlap on one device must not share side_stream. */
MOE_API moe_status_t moe_layer_forward_shared(const moe_layer_desc_t* d, int32_t Hs, const void* x,
                                      const float* x_sf, const void* x_shared, const float* logits,
                                      const int32_t* topk_idx_in, const float* topk_w_in,
                                      const void* w_gate, const void* w_up, const void* w_down,
                                      const uint8_t* sf_gate, const uint8_t* sf_up,
                                      const uint8_t* sf_down, const void* ws_gate,
                                      const void* ws_up, const void* ws_down, void* out, void* ws,
                                      size_t ws_bytes, hipStream_t stream, hipStream_t side_stream);

/* Workspace bytes of moe_layer_backward for `d` (0 if invalid or unsupported). */
MOE_API size_t moe_layer_backward_workspace_bytes(const moe_layer_desc_t* d);

/* Gradients of the layer (moe_layer_forward with the gather combine) for an upstream gradient
 * dout, following MoonEP's "API walkthrough" order backwards: the forward is recomputed with
 * x_perm, g = x.Wg and u = x.Wu kept, then
 *   combine bwd  dy[r] = w[t,k] * dout[t] (r = pos[t,k]), d_topk_w[t,k] = <dout[t], y[r]>
 *   down         dh = dy . Wd[e]^T (with the SwiGLU backward fused:
 *                dg = dh * u * silu'(g), du = dh * silu(g)),  dWd[e] = h_e^T . dy_e
 *   gate/up      dx_rows = dg . Wg[e]^T + du . Wu[e]^T,  dWg[e] = x_e^T . dg_e, dWu[e] = x_e^T . du_e
 *   dispatch bwd dx[t] = sum_k dx_rows[pos[t,k]]
 *   routing      (logits given and d_logits non-NULL) the weights are a softmax over the K
 *                selected logits: d_logits[t, e_k] = w_k (d_topk_w_k - sum_j w_j d_topk_w_j),
 *                0 for the other experts.
 * BF16 layers only (d->act = wgt = out = BF16, gather combine); H % 256 == 0, Hp % 256 == 0.
 * Intermediates are bf16, accumulation fp32.
 *  x, dout, dx [T, H] bf16; logits or topk_idx_in / topk_w_in as in moe_layer_forward;
 *  dw_gate, dw_up [E, H, Hp] and dw_down [E, Hp, H] fp32 out (written, not accumulated; zero
 *  for experts without rows); d_topk_w [T, K] fp32 out (may be NULL); d_logits [T, E] fp32
 *  out or NULL. */
MOE_API moe_status_t moe_layer_backward(const moe_layer_desc_t* d, const void* x, const float* logits,
                                const int32_t* topk_idx_in, const float* topk_w_in,
                                const void* w_gate, const void* w_up, const void* w_down,
                                const void* dout, void* dx, float* dw_gate, float* dw_up,
                                float* dw_down, float* d_topk_w, float* d_logits, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/* Byte offsets of the intermediates inside the moe_layer_forward workspace, for inspection.
 * offsets[i] (i in order): 0 topk_idx, 1 topk_w, 2 counts, 3 cu_seqlens, 4 pos, 5 row_src,
 * 6 row_w (scatter combine), 7 x_perm (only when it is written), 8 x_perm_sf (FP8: the
 * gathered gate/up reads the permuted block-major scales),
 * 9 h, 10 h_sf, 11 y_rows (gather combine), 12 permute scratch, 13 fp32 accumulator (scatter
 * combine with a BF16 output), 14 x_q and 15 x_q_sf (the quantised activations of a
 * (BF16, MXFP4) layer), 16 the control words of the single-launch FFN (BF16 layers; layout
 * as in moe_grouped_ffn_fused_workspace_bytes). Unused entries are set to SIZE_MAX. Writes
 * n <= 17 entries; returns MOE_EINVAL for an invalid `d`. Host-only; the sizes depend on
 * MOE_LAYER_XPERM. */
MOE_API moe_status_t moe_layer_workspace_layout(const moe_layer_desc_t* d, size_t* offsets, int32_t n);

/* Static text for a status code. */
MOE_API const char* moe_status_str(moe_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
