// Backward of the grouped expert FFN and of the combine, in bf16 with fp32 accumulation.
//
// MoonEP "API walkthrough" runs the layer backwards as combine bwd -> the expert GEMMs'
// data and weight gradients -> dispatch bwd; "Mixture of Kittens", Step 1 fixes the expert
// as Down(SwiGLU(Up x, Gate x)). For the rows r of expert e (token t = row_src[r] / K):
//   combine bwd:  dy[r] = row_w[r] * dout[t],   dw[t,k] = <dout[t], y[pos[t,k]]>
//   down:         dh = dy . Wd[e]^T,            dWd[e] = h_e^T . dy_e
//   SwiGLU:       dg = dh * u * silu'(g),       du = dh * silu(g)
//   gate/up:      dx_rows = dg . Wg[e]^T + du . Wu[e]^T
//                 dWg[e] = x_e^T . dg_e,        dWu[e] = x_e^T . du_e
//   dispatch bwd: dx[t] = sum_k dx_rows[pos[t,k]]   (the combine with unit weights)
//
// Kernels:
//  * bwd_dgrad_kernel: grouped GEMM over the rows of each expert with the weights read
//    transposed, C[r, n] = sum_k A[r, k] W[e][n][k]. Both the activations and the weight
//    tile are staged K-contiguous ([256][64] bf16, 16-byte chunks XOR-swizzled by row), so
//    both MFMA fragments are plain ds_read_b128 reads. DUAL accumulates a second (A, W) pair
//    (dg . Wg^T + du . Wu^T). The SwiGLU-backward epilogue loads g and u and writes dg, du.
//    Persistent grid, the forward's tile schedule, 256x256 tiles, K step 64, two stages of
//    direct global->LDS loads.
//  * bwd_wgrad_kernel: per expert, dW[e] = A_e^T . B_e, a reduction over the expert's rows
//    (variable length, the ragged last step zero-filled). Both operands are row-major
//    [rows][cols] and staged as [64 rows][256 cols]; the MFMA fragments come from the
//    gfx950 transposing LDS read (ds_read_b64_tr_b16), as for the forward weights. Output in
//    fp32 (the gradient buffers mirror the weights in fp32, MoonEP "Gradient buffers").
//  * combine_bwd_kernel, route_bwd_kernel: one block / wave per token.
#include "lds_dma.h"
#include "moe_common.h"
#include "tile_sched.h"

namespace moe {

constexpr int BW_THREADS = 512;
constexpr int BW_MAX_E = 1024;
constexpr int BW_BK = 64;                       // K step (dgrad) / rows per step (wgrad)
constexpr int BW_TILE = 256;                    // rows and columns of a block tile
constexpr int BW_ROWB = BW_BK * 2;              // bytes of one staged 64-element row (dgrad)
constexpr int BW_OPB = BW_TILE * BW_ROWB;       // one staged operand: 32 KiB
constexpr int BW_STAGE = 2 * BW_OPB;            // A + B
constexpr int BW_SCHED = (BW_MAX_E + 1 + 16) * 4;
constexpr int BW_LDS = 2 * BW_STAGE + BW_SCHED;
constexpr int BW_LD = BW_OPB / (1024 * 8);      // 1 KiB loads per wave per operand and stage (4)
static_assert(BW_LDS <= 160 * 1024, "LDS budget");

enum { BW_EPI_STORE = 0, BW_EPI_SWIGLU = 1 };

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Epilogue of the data-gradient kernels. Row-lane accumulators (the weight fragment is the
// first MFMA operand): lane l holds row mt*128 + wm*32 + l%32 and, for j = 0..3, the
// columns nt*32 + 8j + 4(l/32) + 0..3 in acc[..][4j .. 4j+3]; outputs leave as 16-byte row
// runs (pack_row16: lane l < 32 writes columns 16p + 0..7, lane l + 32 columns 16p + 8..15).
// EPI_STORE writes C = acc in bf16; EPI_SWIGLU takes acc as dh and writes dg, du from g, u.
template <int EPI>
__device__ __forceinline__ void dgrad_epilogue(const f32x16_t (&acc)[2][4], int row0, int rows_valid, int n0,
                                               int N, int wm, int wn, int lane, uint16_t* __restrict__ C,
                                               const uint16_t* __restrict__ G, const uint16_t* __restrict__ U,
                                               uint16_t* __restrict__ DG, uint16_t* __restrict__ DU) {
  const int h4 = 4 * (lane >> 5);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int r = mt * 128 + wm * 32 + (lane & 31);
    const bool ok = r < rows_valid;
    const size_t ro = (size_t)(row0 + (ok ? r : 0)) * N + n0 + wn * 128;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const f32x16_t& a = acc[mt][nt];
        const size_t o = ro + nt * 32 + 16 * p;  // this 16-column run
        float v[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] = a[8 * p + c];
        if constexpr (EPI == BW_EPI_STORE) {
          const uint4 q = pack_row16(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]);
          if (ok) *reinterpret_cast<uint4*>(C + o + 8 * (lane >> 5)) = q;
        } else {
          // g, u of the lane's eight columns 16p + h4 + 0..3 and 16p + 8 + h4 + 0..3
          uint2 gq[2] = {make_uint2(0, 0), make_uint2(0, 0)}, uq[2] = {make_uint2(0, 0), make_uint2(0, 0)};
          if (ok) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              gq[hh] = *reinterpret_cast<const uint2*>(G + o + 8 * hh + h4);
              uq[hh] = *reinterpret_cast<const uint2*>(U + o + 8 * hh + h4);
            }
          }
          float dg[8], du[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const uint2 gw = gq[c >> 2], uw = uq[c >> 2];
            const uint32_t gb = ((c & 2) ? gw.y : gw.x) >> (16 * (c & 1));
            const uint32_t ub = ((c & 2) ? uw.y : uw.x) >> (16 * (c & 1));
            const float g = bf16f((uint16_t)gb), u = bf16f((uint16_t)ub);
            const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g));  // sigmoid(g)
            dg[c] = v[c] * u * sg * (1.0f + g * (1.0f - sg));
            du[c] = v[c] * g * sg;
          }
          const uint4 qg = pack_row16(dg[0], dg[1], dg[2], dg[3], dg[4], dg[5], dg[6], dg[7]);
          const uint4 qu = pack_row16(du[0], du[1], du[2], du[3], du[4], du[5], du[6], du[7]);
          if (ok) {
            *reinterpret_cast<uint4*>(DG + o + 8 * (lane >> 5)) = qg;
            *reinterpret_cast<uint4*>(DU + o + 8 * (lane >> 5)) = qu;
          }
        }
      }
  }
}

template <int EPI, bool DUAL>
__global__ __launch_bounds__(BW_THREADS, 1) void bwd_dgrad_kernel(
    const uint16_t* __restrict__ A0, const uint16_t* __restrict__ A1, const int* __restrict__ cu,
    int M, int E, int Kd, int N, const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
    uint16_t* __restrict__ C, const uint16_t* __restrict__ G, const uint16_t* __restrict__ U,
    uint16_t* __restrict__ DG, uint16_t* __restrict__ DU) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int* tstart = reinterpret_cast<int*>(smem + 2 * BW_STAGE);
  int* wsum = tstart + BW_MAX_E + 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1;  // rows: blocks wm*32 and 128 + wm*32
  const int wn = wave & 1;   // columns: wn*128 .. +127
  const int ntn = N / BW_TILE;
  const int total = build_tile_prefix<BW_TILE, BW_THREADS>(cu, E, ntn, tstart, wsum);
  const int nk = Kd / BW_BK;
  const int nks = DUAL ? 2 * nk : nk;  // stages: pair 0 over K, then pair 1
  const int G_ = gridDim.x;
  const int slot = xcd_slot(blockIdx.x, G_);
  const uint32_t smem_lds = lds_addr(smem);

  // staging of a [256][64] operand (rows of A, or weight rows n): wave load j = wave + 8 i
  // fills rows 8j .. 8j+7; lane -> row 8j + lane/8, LDS slot lane%8 holds chunk
  // slot ^ ((row/2) % 8). Identical for A and W.
  int voff[BW_LD];
#pragma unroll
  for (int i = 0; i < BW_LD; ++i) {
    const int r = (wave + 8 * i) * 8 + (lane >> 3);
    voff[i] = r * Kd * 2 + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
  }
  // fragments: row (or weight row) base + lane%32, 16-byte chunk 2kk + lane/32, swizzled by
  // ((lane%32)/2) % 8 -- the block offsets (32, 128 rows) keep the swizzle term
  const int sw = ((lane & 31) >> 1) & 7;
  int fk[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) fk[kk] = (lane & 31) * BW_ROWB + ((((kk << 1) | (lane >> 5)) ^ sw) << 4);

  for (int t = slot; t < total; t += G_) {
    const int e = find_expert(tstart, E, t);
    const int lt = t - tstart[e];
    const int gbeg = cu[e];
    const int rows_e = cu[e + 1] - gbeg;
    const int mte = (rows_e + BW_TILE - 1) / BW_TILE;
    const int ntile = lt / mte;
    const int mtile = lt - ntile * mte;
    const int chunk = even_chunk(rows_e, mte);
    const int row0 = gbeg + mtile * chunk;
    const int rows_valid = min(chunk, rows_e - mtile * chunk);
    const int n0 = ntile * BW_TILE;
    const uint32_t a_bytes = (uint32_t)rows_valid * (uint32_t)Kd * 2u;  // rows past: zeros
    const i32x4_t rA0 = make_rsrc(A0 + (size_t)row0 * Kd, a_bytes);
    const i32x4_t rA1 = DUAL ? make_rsrc(A1 + (size_t)row0 * Kd, a_bytes) : rA0;
    const size_t wb = ((size_t)e * N + n0) * Kd;
    const i32x4_t rW0 = make_rsrc(W0 + wb, (uint32_t)BW_TILE * (uint32_t)Kd * 2u);
    const i32x4_t rW1 = DUAL ? make_rsrc(W1 + wb, (uint32_t)BW_TILE * (uint32_t)Kd * 2u) : rW0;

    auto issue = [&](int s) __attribute__((always_inline)) {
      const uint32_t so = smem_lds + (uint32_t)((s & 1) * BW_STAGE);
      const bool second = DUAL && s >= nk;
      const int koff = (second ? s - nk : s) * BW_BK * 2;
#pragma unroll
      for (int i = 0; i < BW_LD; ++i) lds_dma16(second ? rA1 : rA0, so + (wave + 8 * i) * 1024, voff[i], koff);
#pragma unroll
      for (int i = 0; i < BW_LD; ++i)
        lds_dma16(second ? rW1 : rW0, so + BW_OPB + (wave + 8 * i) * 1024, voff[i], koff);
    };

    f32x16_t acc[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;

    __syncthreads();
    issue(0);
    for (int s = 0; s < nks; ++s) {
      wait_barrier<0>();                       // stage s landed; stage s-1 fully read
      if (s + 1 < nks) issue(s + 1);
      const unsigned char* sa = smem + (s & 1) * BW_STAGE;
      const unsigned char* sw_ = sa + BW_OPB;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8_t af[2], bfr[4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          af[mt] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const i32x4_t*>(
                                                    sa + (mt * 128 + wm * 32) * BW_ROWB + fk[kk]));
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          bfr[nt] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const i32x4_t*>(
                                                     sw_ + (wn * 128 + nt * 32) * BW_ROWB + fk[kk]));
        // weight fragment first: the accumulator comes out transposed (one output row per lane)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nt], af[mt], acc[mt][nt], 0, 0, 0);
      }
    }

    dgrad_epilogue<EPI>(acc, row0, rows_valid, n0, N, wm, wn, lane, C, G, U, DG, DU);
  }
}

// dW[e][m][n] = sum over the rows r of expert e of A[r][m] * B[r][n]  (fp32 out)
__global__ __launch_bounds__(BW_THREADS, 1) void bwd_wgrad_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, const int* __restrict__ cu,
    int E, int Md, int Nd, float* __restrict__ W) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int ROW = BW_TILE * 2;  // bytes of a staged row: 256 bf16
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1;  // m: wm*64 .. +63
  const int wn = wave & 1;   // n: wn*128 .. +127
  const int mtn = Md / BW_TILE, ntn = Nd / BW_TILE;
  const int per_e = mtn * ntn;
  const int total = E * per_e;
  const int G_ = gridDim.x;
  const int slot = xcd_slot(blockIdx.x, G_);
  const uint32_t smem_lds = lds_addr(smem);

  // staging of [64 rows][256 cols]: wave load j = wave + 8 i fills rows 2j, 2j+1 (512 B each);
  // lane -> row 2j + lane/32, LDS slot q = lane%32 of the row holds the 32-byte segment
  // (q/2) ^ 2*(row%4) (half q%2) -- the forward's weight layout, conflict-free for the
  // transposing reads
  int v_row[BW_LD], v_col[BW_LD];
#pragma unroll
  for (int i = 0; i < BW_LD; ++i) {
    const int r = 2 * (wave + 8 * i) + (lane >> 5);
    const int q = lane & 31;
    const int sgm = (q >> 1) ^ ((r & 3) << 1);
    v_row[i] = r;
    v_col[i] = ((sgm << 1) + (q & 1)) * 16;
  }
  // transposing fragment reads (see ffn_bf16.hip): 16-lane group g, lane jj in it
  const int g = lane >> 4, jj = lane & 15;
  auto frag_base = [&](int c16) {  // c16: first 16-column segment of the 32 columns
    return (8 * (g >> 1) + (jj >> 2)) * ROW + 8 * (jj & 3) + (((c16 + (g & 1)) ^ ((jj >> 2) << 1)) << 5);
  };
  const int a_fb = frag_base(wm * 4);   // m columns wm*64 + mt*32: mt flips bit 6
  const int b_fb = frag_base(wn * 8);   // n columns wn*128 + nt*32

  for (int t = slot; t < total; t += G_) {
    const int e = t / per_e;
    const int rem = t - e * per_e;
    const int mtile = rem / ntn, ntile = rem - mtile * ntn;
    const int m0 = mtile * BW_TILE, n0 = ntile * BW_TILE;
    const int gbeg = cu[e];
    const int rows_e = cu[e + 1] - gbeg;
    const int nk = (rows_e + BW_BK - 1) / BW_BK;
    // descriptors start at the group's first row and this tile's first column; the row of a
    // load stays in the per-lane offset so rows past the group fall past the range (zeros)
    const i32x4_t rA = make_rsrc(A + (size_t)gbeg * Md + m0, (uint32_t)rows_e * Md * 2u - (uint32_t)m0 * 2u);
    const i32x4_t rB = make_rsrc(B + (size_t)gbeg * Nd + n0, (uint32_t)rows_e * Nd * 2u - (uint32_t)n0 * 2u);

    auto issue = [&](int s) __attribute__((always_inline)) {
      const uint32_t so = smem_lds + (uint32_t)((s & 1) * BW_STAGE);
#pragma unroll
      for (int i = 0; i < BW_LD; ++i) {
        const int r = s * BW_BK + v_row[i];
        lds_dma16(rA, so + (wave + 8 * i) * 1024, r * Md * 2 + v_col[i], 0);
        lds_dma16(rB, so + BW_OPB + (wave + 8 * i) * 1024, r * Nd * 2 + v_col[i], 0);
      }
    };

    f32x16_t acc[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;

    __syncthreads();
    if (nk > 0) issue(0);
    for (int s = 0; s < nk; ++s) {
      wait_barrier<0>();
      if (s + 1 < nk) issue(s + 1);
      const unsigned char* sa = smem + (s & 1) * BW_STAGE;
      const unsigned char* sb = sa + BW_OPB;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8_t af[2], bfr[4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const unsigned char* p = sa + (a_fb ^ (mt << 6)) + kk * 16 * ROW;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4_t*)(p));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4_t*)(p + 4 * ROW));
          af[mt] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const unsigned char* p = sb + (b_fb ^ (nt << 6)) + kk * 16 * ROW;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4_t*)(p));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4_t*)(p + 4 * ROW));
          bfr[nt] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        // B fragment first: the accumulator comes out transposed, lane l holding row m of dW
        // (l % 32 of the block) and runs of four consecutive n
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nt], af[mt], acc[mt][nt], 0, 0, 0);
      }
    }

    // dW[e][m][n]: lane holds row m = wm*64 + mt*32 + lane%32 and, for j = 0..3, the columns
    // n = nt*32 + 8j + 4(lane/32) + 0..3 in acc[..][4j .. 4j+3]: 16-byte row stores
    float* We = W + (size_t)e * Md * Nd;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float* row = We + (size_t)(m0 + wm * 64 + mt * 32 + (lane & 31)) * Nd + n0 + wn * 128 + 4 * (lane >> 5);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x16_t& a = acc[mt][nt];
          *reinterpret_cast<float4*>(row + nt * 32 + 8 * j) = make_float4(a[4 * j], a[4 * j + 1], a[4 * j + 2], a[4 * j + 3]);
        }
    }
  }
}

// Combine backward, one 128-thread block per token: dy[pos[t,k]] = w[t,k] * dout[t] (bf16,
// rounded once) and dw[t,k] = <dout[t], y[pos[t,k]]> (fp32); dropped copies (pos < 0) get
// dw = 0.
template <int KMAX>
__global__ __launch_bounds__(128) void combine_bwd_kernel(const uint16_t* __restrict__ dout,
                                                          const uint16_t* __restrict__ y,
                                                          const int* __restrict__ pos,
                                                          const float* __restrict__ w, int H, int K,
                                                          uint16_t* __restrict__ dy,
                                                          float* __restrict__ dw) {
  const int t = blockIdx.x;
  __shared__ float red[4][KMAX];
  int p[KMAX];
  float wk[KMAX], dot[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    p[k] = k < K ? pos[(size_t)t * K + k] : -1;
    wk[k] = k < K ? w[(size_t)t * K + k] : 0.f;
    dot[k] = 0.f;
  }
  for (int c = threadIdx.x; c < H / 8; c += blockDim.x) {
    const int4 dv = *reinterpret_cast<const int4*>(dout + (size_t)t * H + c * 8);
    const uint32_t du[4] = {(uint32_t)dv.x, (uint32_t)dv.y, (uint32_t)dv.z, (uint32_t)dv.w};
    float d[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      d[2 * i] = __uint_as_float(du[i] << 16);
      d[2 * i + 1] = __uint_as_float(du[i] & 0xffff0000u);
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      if (p[k] < 0) continue;
      const int4 yv = *reinterpret_cast<const int4*>(y + (size_t)p[k] * H + c * 8);
      const uint32_t yu[4] = {(uint32_t)yv.x, (uint32_t)yv.y, (uint32_t)yv.z, (uint32_t)yv.w};
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s = fmaf(d[2 * i], __uint_as_float(yu[i] << 16), s);
        s = fmaf(d[2 * i + 1], __uint_as_float(yu[i] & 0xffff0000u), s);
      }
      dot[k] += s;
      int4 o;
      o.x = (int)pack_bf16x2(wk[k] * d[0], wk[k] * d[1]);
      o.y = (int)pack_bf16x2(wk[k] * d[2], wk[k] * d[3]);
      o.z = (int)pack_bf16x2(wk[k] * d[4], wk[k] * d[5]);
      o.w = (int)pack_bf16x2(wk[k] * d[6], wk[k] * d[7]);
      *reinterpret_cast<int4*>(dy + (size_t)p[k] * H + c * 8) = o;
    }
  }
  // block reduction of the K dot products (2 waves of 64)
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    float v = dot[k];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) red[wv][k] = v;
  }
  __syncthreads();
  if (threadIdx.x < K) dw[(size_t)t * K + threadIdx.x] = red[0][threadIdx.x] + red[1][threadIdx.x];
}

// Top-k softmax backward, one wave per token: the weights are a softmax over the K selected
// logits, so dlogits[t, e_k] = w_k (dw_k - sum_j w_j dw_j); the other experts get 0.
__global__ __launch_bounds__(256) void route_bwd_kernel(const int* __restrict__ idx,
                                                        const float* __restrict__ w,
                                                        const float* __restrict__ dw, int T, int E,
                                                        int K, float* __restrict__ dl) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  float s = 0.f;
  for (int k = lane; k < K; k += 64) s += w[(size_t)t * K + k] * dw[(size_t)t * K + k];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  for (int e = lane; e < E; e += 64) dl[(size_t)t * E + e] = 0.f;
  // the zero stores above and the stores below come from the same wave, in program order
  for (int k = lane; k < K; k += 64) {
    const int e = idx[(size_t)t * K + k];
    if ((unsigned)e < (unsigned)E)
      dl[(size_t)t * E + e] = w[(size_t)t * K + k] * (dw[(size_t)t * K + k] - s);
  }
}

// ---- launchers -------------------------------------------------------------------------

template <int EPI, bool DUAL>
static moe_status_t launch_dgrad(const uint16_t* A0, const uint16_t* A1, const int* cu, int M, int E,
                                 int Kd, int N, const uint16_t* W0, const uint16_t* W1, uint16_t* C,
                                 const uint16_t* G, const uint16_t* U, uint16_t* DG, uint16_t* DU,
                                 hipStream_t s) {
  static std::atomic<unsigned char> lds_set[MOE_MAX_DEVICES];
  if (ensure_lds_limit(reinterpret_cast<const void*>(&bwd_dgrad_kernel<EPI, DUAL>), BW_LDS, lds_set) != MOE_OK)
    return MOE_EHIP;
  bwd_dgrad_kernel<EPI, DUAL><<<device_cu_count(), BW_THREADS, BW_LDS, s>>>(A0, A1, cu, M, E, Kd, N, W0,
                                                                           W1, C, G, U, DG, DU);
  return launch_status();
}

// dh = dy . Wd^T with the SwiGLU backward fused: dg, du [M, Hp]
moe_status_t launch_bwd_down_swiglu(const void* dy, const int* cu, int M, int E, int H, int Hp,
                                    const void* wd, const void* g, const void* u, void* dg, void* du,
                                    hipStream_t s) {
  if (M == 0) return MOE_OK;
  return launch_dgrad<BW_EPI_SWIGLU, false>(static_cast<const uint16_t*>(dy), nullptr, cu, M, E, H, Hp,
                                            static_cast<const uint16_t*>(wd), nullptr, nullptr,
                                            static_cast<const uint16_t*>(g), static_cast<const uint16_t*>(u),
                                            static_cast<uint16_t*>(dg), static_cast<uint16_t*>(du), s);
}

// dx_rows = dg . Wg^T + du . Wu^T  [M, H]
moe_status_t launch_bwd_gate_up(const void* dg, const void* du, const int* cu, int M, int E, int H,
                                int Hp, const void* wg, const void* wu, void* dx_rows, hipStream_t s) {
  if (M == 0) return MOE_OK;
  return launch_dgrad<BW_EPI_STORE, true>(static_cast<const uint16_t*>(dg), static_cast<const uint16_t*>(du),
                                          cu, M, E, Hp, H, static_cast<const uint16_t*>(wg),
                                          static_cast<const uint16_t*>(wu), static_cast<uint16_t*>(dx_rows),
                                          nullptr, nullptr, nullptr, nullptr, s);
}

// dW[e] = A_e^T . B_e for every expert (zero for empty experts)  [E, Md, Nd] fp32
moe_status_t launch_bwd_wgrad(const void* A, const void* B, const int* cu, int E, int Md, int Nd,
                              float* W, hipStream_t s) {
  static std::atomic<unsigned char> lds_set[MOE_MAX_DEVICES];
  if (ensure_lds_limit(reinterpret_cast<const void*>(&bwd_wgrad_kernel), 2 * BW_STAGE, lds_set) != MOE_OK)
    return MOE_EHIP;
  bwd_wgrad_kernel<<<device_cu_count(), BW_THREADS, 2 * BW_STAGE, s>>>(
      static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), cu, E, Md, Nd, W);
  return launch_status();
}

moe_status_t launch_combine_bwd(const void* dout, const void* y, const int* pos, const float* w,
                                int T, int H, int K, void* dy, float* dw, hipStream_t s) {
  if (T == 0) return MOE_OK;
  const uint16_t* d = static_cast<const uint16_t*>(dout);
  const uint16_t* yy = static_cast<const uint16_t*>(y);
  uint16_t* o = static_cast<uint16_t*>(dy);
  if (K <= 2) combine_bwd_kernel<2><<<T, 128, 0, s>>>(d, yy, pos, w, H, K, o, dw);
  else if (K <= 4) combine_bwd_kernel<4><<<T, 128, 0, s>>>(d, yy, pos, w, H, K, o, dw);
  else if (K <= 8) combine_bwd_kernel<8><<<T, 128, 0, s>>>(d, yy, pos, w, H, K, o, dw);
  else if (K <= 16) combine_bwd_kernel<16><<<T, 128, 0, s>>>(d, yy, pos, w, H, K, o, dw);
  else combine_bwd_kernel<32><<<T, 128, 0, s>>>(d, yy, pos, w, H, K, o, dw);
  return launch_status();
}

moe_status_t launch_route_bwd(const int* idx, const float* w, const float* dw, int T, int E, int K,
                              float* dl, hipStream_t s) {
  if (T == 0) return MOE_OK;
  route_bwd_kernel<<<(T + 3) / 4, 256, 0, s>>>(idx, w, dw, T, E, K, dl);
  return launch_status();
}

}  // namespace moe
