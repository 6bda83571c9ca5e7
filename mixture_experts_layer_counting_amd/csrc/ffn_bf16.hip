// Grouped expert FFN in bf16 on gfx950 matrix cores.
//
// "Distributed expert parallelism", "Grouped expert computation": one launch runs the
// matrix products of every expert over its variable-size group of rows. "Mixture of
// Kittens", Step 1: each expert is Down(SwiGLU(Up x, Gate x)); the gate/up kernel fuses
// SwiGLU into its epilogue (h = silu(x.Wg) * (x.Wu)), the down kernel computes h.Wd.
// MoonEP "Integration": the stacked [E, ., .] weight tensors are addressed purely by expert
// index and cu_seqlens selects each expert's rows.
//
// Design (one kernel body, GATED selects gate/up + SwiGLU or the plain down projection):
//  * Persistent grid of one 512-thread block per CU. Each block derives the tile list from
//    cu_seqlens in LDS (tiles per expert = ceil(rows / BM) * N / BN, exclusive prefix) and
//    walks it with stride gridDim. Tile t of round r maps to XCD-contiguous slots, so the
//    32 CUs of one XCD work on neighbouring tiles: the same expert's weight panel (tiles
//    of one n-panel are consecutive over its m-tiles) and the same rows stay in that XCD's
//    L2.
//  * Block tile BM=256 rows x BN columns (per weight matrix), K step 64, two LDS stages.
//    8 waves as 4 (rows) x 2 (columns), each wave 64 x BN/2 with MFMA 32x32x16 bf16 and
//    fp32 accumulators (128 per lane).
//  * A (activations, reduction-contiguous) is staged as [256][64] with the 16-byte chunk
//    index XOR-swizzled by (row/2) mod 8 so ds_read_b128 of 16 consecutive rows is free of
//    bank conflicts. B (weights [K][N], N contiguous) is staged in its global layout and
//    turned into the MFMA B operand by ds_read_b64_tr_b16 (two per fragment); its 32-byte
//    segments are XOR-swizzled by 2*(row mod 4) so the four rows a transpose read touches
//    land on distinct banks.
//  * Global loads for step k+1 are issued before the MFMAs of step k; one barrier per step.
//  * Rows past the expert's group are computed on whatever rows follow (clamped to M-1) and
//    never stored.
#include "moe_common.h"
#include "tile_sched.h"

namespace moe {

constexpr int FB_BM = 256;
constexpr int FB_BK = 64;
constexpr int FB_THREADS = 512;
constexpr int FB_MAX_E = 1024;

template <bool GATED, int BN>
struct FbCfg {
  static constexpr int NB = GATED ? 2 : 1;
  static constexpr int WN = BN / 2;
  static constexpr int NT = WN / 32;
  static constexpr int MT = 2;
  static constexpr int A_BYTES = FB_BM * FB_BK * 2;
  static constexpr int B_BYTES = FB_BK * BN * 2;
  static constexpr int STAGE = A_BYTES + NB * B_BYTES;
  static constexpr int A_LD = FB_BM * (FB_BK / 8) / FB_THREADS;  // 16-byte chunks per thread
  static constexpr int B_LD = FB_BK * (BN / 8) / FB_THREADS;      // per matrix
  static constexpr int SCHED_BYTES = (FB_MAX_E + 1 + 16) * 4;
  static constexpr int LDS_BYTES = 2 * STAGE + SCHED_BYTES;
};

template <bool GATED, int BN>
__global__ __launch_bounds__(FB_THREADS, 1) void ffn_bf16_kernel(
    const uint16_t* __restrict__ A, const int* __restrict__ cu, int M, int E, int Kd, int N,
    const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, uint16_t* __restrict__ C) {
  using CF = FbCfg<GATED, BN>;
  constexpr int BCH = BN / 8;                    // 16-byte chunks per B row
  constexpr int B_ROWS_PER_LD = FB_THREADS / BCH;  // B rows covered by one load round
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int* tstart = reinterpret_cast<int*>(smem + 2 * CF::STAGE);
  int* wsum = tstart + FB_MAX_E + 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;  // 0..3: 64-row strip
  const int wn = wave & 1;   // 0..1: BN/2-column half
  const int ntn = N / BN;
  const int total = build_tile_prefix<FB_BM, FB_THREADS>(cu, E, ntn, tstart, wsum);
  const int nk = Kd / FB_BK;
  const int G = gridDim.x;
  const int slot = xcd_slot(blockIdx.x, G);

  // global -> LDS: thread owns A chunks (row tid/8 + 64 i, chunk tid%8) and B chunks
  // (row tid/BCH + B_ROWS_PER_LD i, chunk tid%BCH); the swizzle only depends on tid.
  const int a_voff = (tid >> 3) * Kd * 2 + (tid & 7) * 16;
  const int a_lds0 = (tid >> 3) * 128 + (((tid & 7) ^ ((tid >> 4) & 7)) << 4);
  const int b_row = tid / BCH, b_ch = tid % BCH;
  const int b_voff = b_row * N * 2 + b_ch * 16;
  const int b_lds0 = b_row * (BN * 2) + ((((b_ch >> 1) ^ ((b_row & 3) << 1))) << 5) + ((b_ch & 1) << 4);

  // LDS -> MFMA fragments. A: row wm*64 + mt*32 + lane%32, 16-byte chunk 2*kk + lane/32,
  // stored at chunk ^ ((row/2) % 8). B (transpose read): lane group g = lane/16 reads rows
  // kk*16 + 8*(g/2) + (lane%16)/4 (+4 for the second half) at columns
  // wn*WN + nt*32 + 16*(g%2) + 4*(lane%4); its 32-byte segment is stored at
  // segment ^ 2*(row % 4). Both reduce to a per-lane base XOR a compile-time constant.
  const int a_fbase = (wm * 64 + (lane & 31)) * 128;
  const int a_t0 = (((lane >> 5) ^ ((lane >> 1) & 7))) << 4;
  int a_fk[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) a_fk[kk] = a_fbase + ((kk << 5) ^ a_t0);
  const int g = lane >> 4, jj = lane & 15;
  const int bP = (wn * CF::WN) / 16 + (g & 1);
  const int b_fbase = (8 * (g >> 1) + (jj >> 2)) * (BN * 2) + 8 * (jj & 3) +
                      ((bP ^ ((jj >> 2) << 1)) << 5);
  int b_fn[CF::NT];
#pragma unroll
  for (int nt = 0; nt < CF::NT; ++nt) b_fn[nt] = b_fbase ^ (nt << 6);

  for (int t = slot; t < total; t += G) {
    const int e = find_expert(tstart, E, t);
    const int lt = t - tstart[e];
    const int gbeg = cu[e];
    const int rows_e = cu[e + 1] - gbeg;
    const int mte = (rows_e + FB_BM - 1) / FB_BM;
    const int ntile = lt / mte;
    const int mtile = lt - ntile * mte;
    const int row0 = gbeg + mtile * FB_BM;
    const int rows_valid = min(FB_BM, rows_e - mtile * FB_BM);
    const int n0 = ntile * BN;

    // buffer descriptors: rows past M read as zero (hardware range check)
    const size_t a_rem = (size_t)(M - row0) * Kd * 2;
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(A + (size_t)row0 * Kd), 0, (int)(a_rem > 0x7fffffffu ? 0x7fffffffu : a_rem), 0x00020000);
    const size_t woff = (size_t)e * Kd * N + n0;
    const int b_rem = (int)(((size_t)Kd * N - n0) * 2);
    const __amdgpu_buffer_rsrc_t rB0 = __builtin_amdgcn_make_buffer_rsrc((void*)(B0 + woff), 0, b_rem, 0x00020000);
    __amdgpu_buffer_rsrc_t rB1 = rB0;
    if constexpr (GATED) rB1 = __builtin_amdgcn_make_buffer_rsrc((void*)(B1 + woff), 0, b_rem, 0x00020000);

    i32x4_t ra[CF::A_LD];
    i32x4_t rb[CF::NB][CF::B_LD];
    auto gload = [&](int kt) {
#pragma unroll
      for (int i = 0; i < CF::A_LD; ++i)
        ra[i] = __builtin_bit_cast(i32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                rA, a_voff, i * 64 * Kd * 2 + kt * FB_BK * 2, 0));
#pragma unroll
      for (int i = 0; i < CF::B_LD; ++i) {
        const int so = (kt * FB_BK + i * B_ROWS_PER_LD) * N * 2;
        rb[0][i] = __builtin_bit_cast(i32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rB0, b_voff, so, 0));
        if constexpr (GATED)
          rb[1][i] = __builtin_bit_cast(i32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rB1, b_voff, so, 0));
      }
    };
    auto sstore = [&](int st) {
      unsigned char* base = smem + st * CF::STAGE;
#pragma unroll
      for (int i = 0; i < CF::A_LD; ++i) *reinterpret_cast<i32x4_t*>(base + a_lds0 + i * 64 * 128) = ra[i];
#pragma unroll
      for (int nb = 0; nb < CF::NB; ++nb)
#pragma unroll
        for (int i = 0; i < CF::B_LD; ++i)
          *reinterpret_cast<i32x4_t*>(base + CF::A_BYTES + nb * CF::B_BYTES + b_lds0 +
                                      i * B_ROWS_PER_LD * BN * 2) = rb[nb][i];
    };

    f32x16_t acc[CF::NB][CF::MT][CF::NT];
#pragma unroll
    for (int nb = 0; nb < CF::NB; ++nb)
#pragma unroll
      for (int mt = 0; mt < CF::MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < CF::NT; ++nt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[nb][mt][nt][i] = 0.f;

    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) gload(kt + 1);
      const unsigned char* sa = smem + cur * CF::STAGE;
      const unsigned char* sb = sa + CF::A_BYTES;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8_t af[CF::MT];
#pragma unroll
        for (int mt = 0; mt < CF::MT; ++mt)
          af[mt] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const i32x4_t*>(sa + a_fk[kk] + mt * 32 * 128));
#pragma unroll
        for (int nb = 0; nb < CF::NB; ++nb) {
#pragma unroll
          for (int nt = 0; nt < CF::NT; ++nt) {
            const unsigned char* p = sb + nb * CF::B_BYTES + b_fn[nt] + kk * 16 * BN * 2;
            const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4_t*)(p));
            const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4_t*)(p + 4 * BN * 2));
            const bf16x8_t bfr = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int mt = 0; mt < CF::MT; ++mt)
              acc[nb][mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mt], bfr, acc[nb][mt][nt], 0, 0, 0);
          }
        }
      }
      if (kt + 1 < nk) sstore(cur ^ 1);
      __syncthreads();
    }

    // epilogue: lane holds column lane%32 of rows 8*(i/4) + 4*(lane/32) + i%4
#pragma unroll
    for (int mt = 0; mt < CF::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < CF::NT; ++nt) {
        const int col = n0 + wn * CF::WN + nt * 32 + (lane & 31);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = wm * 64 + mt * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          if (r < rows_valid) {
            float v;
            if constexpr (GATED)
              v = silu_f32(acc[0][mt][nt][i]) * acc[1][mt][nt][i];
            else
              v = acc[0][mt][nt][i];
            C[(size_t)(row0 + r) * N + col] = f32_to_bf16_bits(v);
          }
        }
      }
  }
}

template <bool GATED, int BN>
static moe_status_t launch_fb(const uint16_t* A, const int* cu, int M, int E, int Kd, int N,
                              const uint16_t* B0, const uint16_t* B1, uint16_t* C, hipStream_t s) {
  using CF = FbCfg<GATED, BN>;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_bf16_kernel<GATED, BN>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, CF::LDS_BYTES) != hipSuccess)
      return MOE_EHIP;
    attr_set = true;
  }
  const int grid = device_cu_count();
  ffn_bf16_kernel<GATED, BN><<<grid, FB_THREADS, CF::LDS_BYTES, s>>>(A, cu, M, E, Kd, N, B0, B1, C);
  return launch_status();
}

moe_status_t launch_ffn_gate_up_bf16(const void* x_perm, const int* cu, int M, int E, int H, int Hp,
                                     const void* wg, const void* wu, void* h, hipStream_t s) {
  if (M == 0) return MOE_OK;
  return launch_fb<true, 128>(static_cast<const uint16_t*>(x_perm), cu, M, E, H, Hp,
                              static_cast<const uint16_t*>(wg), static_cast<const uint16_t*>(wu),
                              static_cast<uint16_t*>(h), s);
}

moe_status_t launch_ffn_down_bf16(const void* h, const int* cu, int M, int E, int H, int Hp,
                                  const void* wd, void* y, hipStream_t s) {
  if (M == 0) return MOE_OK;
  return launch_fb<false, 256>(static_cast<const uint16_t*>(h), cu, M, E, Hp, H,
                               static_cast<const uint16_t*>(wd), nullptr, static_cast<uint16_t*>(y), s);
}

}  // namespace moe
