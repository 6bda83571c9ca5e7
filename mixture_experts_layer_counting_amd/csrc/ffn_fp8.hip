// Grouped expert FFN with fp8 (e4m3fn, 1x128 power-of-two block scales) activations and
// MXFP4 (e2m1 + e8m0 per 32 along the reduction) weights, on gfx950 scaled matrix cores.
//
// "Mixture of Kittens", Step 1 (expert = Down(SwiGLU(Up x, Gate x))) and Step 8 (low
// precision with activation quantisation fused into the GEMMs and SwiGLU); DeepGEMM's
// Mega-MoE how-to names the same dual FP8 x FP4 GEMMs with per-block scale factors for the
// inputs and for the activations between the two GEMMs. Here:
//   gate/up:  h = silu(x.Wg) * (x.Wu) in fp32, requantised in the epilogue to e4m3fn with one
//             power-of-two scale per 1x128 block of each row (s = smallest 2^e with
//             448 s >= block amax; code = round-to-nearest-even(h / s)),
//   down:     y = h.Wd, bf16 output.
//
// MFMA v_mfma_scale_f32_32x32x64_f8f6f4 (A fp8, B fp4). Operand layouts (verified on the
// device): an fp8 operand lane in group G = lane/32 holds two 16-byte runs of consecutive k,
// at k = 16G and k = 32 + 16G; an fp4 operand lane holds the 32 consecutive k = 32G.. in 16
// bytes, low nibble first; the scale register of lane (row or column, G) applies to k-block
// [32G, 32G+32). Activation scales are per 128 k, so one exponent covers a whole K step.
//
// Same persistent, XCD-contiguous tile schedule and direct global->LDS staging as the bf16
// kernels. Block tile 256 rows x BN columns per weight matrix, K step 128, three LDS stages
// (two in flight while one is consumed: with fp4 weights a stage is short, and one stage in
// flight leaves the HBM latency exposed). Activations are staged [256][128 B] (16-byte chunk
// ^ (row/2 mod 8)); weights, stored reduction-contiguous [N][K/2], are staged [BN][64 B]
// (chunk ^ (col/4 mod 4)). Both fragment reads are ds_read_b128 without transposes. Scales are
// stored block-major (activations [K/128][M], weights [E][K/32][N]), so a stage's scales are
// contiguous runs; they are staged in LDS with the tile data by the same direct loads, and all
// of a stage's loads complete under one explicit wait. As in the bf16 kernels, a wave's two
// 32-row blocks are rows wm*32 + [0,32) and 128 + wm*32 + [0,32), blocks wholly past the
// group's rows skip their MFMAs, and rows past the group's last row load as zeros from past
// the A descriptor's range. The optional row maps (gathering A rows and their scales from
// the token matrix x [T, H] with x_sf [T, H/128]; scattering row_w * y into an fp32
// accumulator) work as in the bf16 kernels.
#include "lds_dma.h"
#include "moe_common.h"
#include "tile_sched.h"

#include <type_traits>

namespace moe {

constexpr int F8_BM = 256;
constexpr int F8_BK = 128;  // reduction elements per stage
constexpr int F8_NS = 3;
constexpr int F8_THREADS = 512;
constexpr int F8_MAX_E = 1024;

template <bool GATED, int BN>
struct F8Cfg {
  static constexpr int NB = GATED ? 2 : 1;
  static constexpr int WN = BN / 2;
  static constexpr int NT = WN / 32;
  static constexpr int MT = 2;
  static constexpr int NF = NB * NT;
  static constexpr int KK = F8_BK / 64;                   // MFMA k-steps per stage
  static constexpr int A_BYTES = F8_BM * F8_BK;            // 32 KiB, 128 B per row
  static constexpr int A_LD = A_BYTES / (1024 * 8);        // wave loads per stage (8 rows each)
  static constexpr int B_ROW = F8_BK / 2;                  // 64 B per weight column
  static constexpr int B_BYTES = BN * B_ROW;               // per matrix
  static constexpr int B_LD = NB * B_BYTES / (1024 * 8);   // wave loads per stage (16 cols each)
  // per-stage scales: activations [256] fp32, weights [NB][4 k-blocks][BN] e8m0 bytes
  static constexpr int SF_A = A_BYTES + NB * B_BYTES;
  static constexpr int SF_B = SF_A + F8_BM * 4;
  static constexpr int STAGE = SF_B + NB * 4 * BN;
  static constexpr int VM_PER_STAGE = A_LD + B_LD + 1;  // + one scale load per wave
  // tile prefix per expert, per-wave scan sums, and the gate/up epilogue's per-row amax of
  // the two column waves ([2][256] fp32)
  static constexpr int SCHED_BYTES = (F8_MAX_E + 1 + 16 + 2 * F8_BM) * 4;
  static constexpr int LDS_BYTES = F8_NS * STAGE + SCHED_BYTES;
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small");
  // the scale loads: waves 0-3 take 64 activation rows each (4 B per lane), waves 4-7 take
  // 256 bytes each of the weight scale block
  static_assert(NB * 4 * BN == 4 * 256, "weight scale block must be four 256-byte loads");
  static_assert(STAGE % 16 == 0, "stage alignment");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <bool GATED, int BN, bool MAPPED>
__global__ __launch_bounds__(F8_THREADS, 1) void ffn_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ A_sf, const int* __restrict__ cu,
    int M, int E, int Kd, int N, const uint8_t* __restrict__ B0, const uint8_t* __restrict__ B0_sf,
    const uint8_t* __restrict__ B1, const uint8_t* __restrict__ B1_sf, uint8_t* __restrict__ C8,
    float* __restrict__ C8_sf, uint16_t* __restrict__ C16, RowMaps maps, int paired) {
  using CF = F8Cfg<GATED, BN>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int* tstart = reinterpret_cast<int*>(smem + F8_NS * CF::STAGE);
  int* wsum = tstart + F8_MAX_E + 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int ntn = N / BN;
  const int total = build_tile_prefix<F8_BM, F8_THREADS>(cu, E, ntn, tstart, wsum);
  const int nk = Kd / F8_BK;
  const int kbytes = Kd / 2;     // bytes per weight column
  const int ksf_b = Kd / 32;     // weight scale bytes per column
  const int G = gridDim.x;
  const int slot = xcd_slot(blockIdx.x, G);
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(const MOE_LDS void*)smem;

  // global -> LDS coordinates. A wave load j (= wave + 8 i) covers rows 8j..8j+7 (128 B each):
  // lane -> row 8j + lane/8, slot lane%8 holds chunk slot ^ ((row/2) % 8).
  // (when gathering, the row part of a_voff is replaced per tile by the source row's offset)
  int a_voff[CF::A_LD], a_row[CF::A_LD];
#pragma unroll
  for (int i = 0; i < CF::A_LD; ++i) {
    const int r = (wave + 8 * i) * 8 + (lane >> 3);
    a_row[i] = r;
    a_voff[i] = r * Kd + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
  }
  const int nsf = Kd / 128;  // activation scale blocks per row
  // B wave load j covers columns 16j'..16j'+15 (64 B each) of matrix j / (B_BYTES/1024):
  // lane -> column lane/4, slot lane%4 holds chunk slot ^ ((col/4) % 4). The stored [N][K/2]
  // layout gives each column's 64 bytes of a K step half a 128-byte line; the paired layout
  // ([N/2][K/128][2][64 B]) puts the 64-byte runs of columns 2p and 2p+1 side by side in one
  // line, so a load touches 8 lines instead of 16. The bytes staged in LDS are the same.
  int b_voff[CF::B_LD];
#pragma unroll
  for (int i = 0; i < CF::B_LD; ++i) {
    const int j = wave + 8 * i;
    const int c = (j % (CF::B_BYTES / 1024)) * 16 + (lane >> 2);
    const int chunk = ((lane & 3) ^ ((c >> 2) & 3)) << 4;
    b_voff[i] = paired ? (c >> 1) * Kd + (c & 1) * (F8_BK / 2) + chunk : c * kbytes + chunk;
  }
  const int b_kstep = paired ? F8_BK : F8_BK / 2;   // bytes between K steps of one column

  // fragment offsets. A (fp8, 32x64 per MFMA): row mt*128 + wm*32 + lane%32, chunks 4kk + G
  // and 4kk + 2 + G. B (fp4): column wn*WN + nt*32 + lane%32, chunk 2kk + G.
  const int g2 = lane >> 5;
  const int ar = wm * 32 + (lane & 31);
  const int a_sw = (ar >> 1) & 7;  // (mt*128)/2 is a multiple of 8: same swizzle for both mt
  int a_off[CF::KK][2];
#pragma unroll
  for (int kk = 0; kk < CF::KK; ++kk)
#pragma unroll
    for (int h = 0; h < 2; ++h) a_off[kk][h] = ar * F8_BK + (((4 * kk + 2 * h + g2) ^ a_sw) << 4);
  int b_off[CF::NT][CF::KK];
#pragma unroll
  for (int nt = 0; nt < CF::NT; ++nt) {
    const int c = wn * CF::WN + nt * 32 + (lane & 31);
#pragma unroll
    for (int kk = 0; kk < CF::KK; ++kk) b_off[nt][kk] = c * CF::B_ROW + (((2 * kk + g2) ^ ((c >> 2) & 3)) << 4);
  }

  // Operand order of the MFMA: with the weight fragment first the accumulator comes out
  // transposed, lane l holding one output row (l % 32 of its 32-row block) and runs of four
  // consecutive columns, which the epilogues write as 8- and 16-byte row runs. The scatter
  // epilogue keeps the other order (32 lanes of a row add into 32 consecutive floats).
  constexpr bool ROW_LANES = !(!GATED && MAPPED);
  float* xpart = reinterpret_cast<float*>(wsum + 16);  // [2][F8_BM] row amax of the column waves

  // one output tile: rows, columns, the stage buffer its stage 0 uses, load descriptors
  struct Tile {
    int e, row0, rows_valid, n0, nmt, base, sc_voff;
    i32x4_t rA, rB0, rB1;
    int a_ld_off[CF::A_LD];
  };
  const int sc_row = (wave & 3) * 64 + lane;  // activation-scale row of waves 0-3
  const bool sf_perm = GATED && MAPPED && maps.a_sf_perm != nullptr;
  auto decode = [&](int t, int base) __attribute__((always_inline)) {
    Tile d;
    d.e = find_expert(tstart, E, t);
    const int lt = t - tstart[d.e];
    const int gbeg = cu[d.e];
    const int rows_e = cu[d.e + 1] - gbeg;
    const int mte = (rows_e + F8_BM - 1) / F8_BM;
    const int ntile = lt / mte;
    const int mtile = lt - ntile * mte;
    const int chunk = even_chunk(rows_e, mte);
    d.row0 = gbeg + mtile * chunk;
    d.rows_valid = min(chunk, rows_e - mtile * chunk);
    d.n0 = ntile * BN;
    d.base = base;
    // A rows of this tile (see the bf16 kernels): rows past rows_valid load past the range.
    if constexpr (GATED && MAPPED) {
      d.rA = make_rsrc(A, (uint32_t)maps.a_rows * (uint32_t)Kd);
      // Branch-free so that the loads go out together: each reads a row of this tile (also
      // for rows past it), and the offset is chosen after the arithmetic. -1: padding row.
      int src[CF::A_LD];
#pragma unroll
      for (int i = 0; i < CF::A_LD; ++i) src[i] = maps.a_src[d.row0 + min(a_row[i], d.rows_valid - 1)];
      const int ssrc0 = maps.a_src[d.row0 + min(sc_row, d.rows_valid - 1)];
#pragma unroll
      for (int i = 0; i < CF::A_LD; ++i) {
        const int off = (src[i] / maps.a_k - a_row[i]) * Kd + a_voff[i];
        d.a_ld_off[i] = (a_row[i] < d.rows_valid && src[i] >= 0) ? off : (int)0x80000000u;
      }
      const int ssrc = sc_row < d.rows_valid ? ssrc0 : -1;
      d.sc_voff = sf_perm ? (d.row0 + sc_row) * 4 : ssrc >= 0 ? (ssrc / maps.a_k) * nsf * 4 : (int)0x80000000u;
    } else {
      d.rA = make_rsrc(A + (size_t)d.row0 * Kd, (uint32_t)d.rows_valid * (uint32_t)Kd);
#pragma unroll
      for (int i = 0; i < CF::A_LD; ++i) d.a_ld_off[i] = a_voff[i];
      d.sc_voff = (d.row0 + sc_row) * 4;
    }
    d.nmt = __builtin_amdgcn_readfirstlane((wm * 32 < d.rows_valid) + (128 + wm * 32 < d.rows_valid));
    const size_t wbase = ((size_t)d.e * N + d.n0) * kbytes;
    const uint32_t b_rem = (uint32_t)((size_t)(N - d.n0) * kbytes);
    d.rB0 = make_rsrc(B0 + wbase, b_rem);
    d.rB1 = GATED ? make_rsrc(B1 + wbase, b_rem) : d.rB0;
    return d;
  };
  // this wave's share of stage kt of tile d, into buffer (d.base + kt) mod F8_NS
  auto issue = [&](const Tile& d, int kt) __attribute__((always_inline)) {
    const uint32_t so = smem_lds + (uint32_t)(((unsigned)(d.base + kt) % F8_NS) * CF::STAGE);
#pragma unroll
    for (int i = 0; i < CF::A_LD; ++i) lds_dma16(d.rA, so + (wave + 8 * i) * 1024, d.a_ld_off[i], kt * F8_BK);
#pragma unroll
    for (int i = 0; i < CF::B_LD; ++i) {
      const int j = wave + 8 * i;
      const bool second = GATED && (j / (CF::B_BYTES / 1024)) != 0;
      lds_dma16(second ? d.rB1 : d.rB0, so + CF::A_BYTES + j * 1024, b_voff[i], kt * b_kstep);
    }
    if (wave < 4) {
      // activation scales of block kt for tile rows 64 wave + lane. Plain (or gathered rows
      // with permuted scales): block-major [Kd/128][M], rows >= M read as zero, one 256-byte
      // run per wave. Gathered: x_sf [a_rows][Kd/128] of the row's token, a line per lane.
      if (GATED && MAPPED && !sf_perm)
        lds_dma4(make_rsrc(A_sf, (uint32_t)maps.a_rows * (uint32_t)nsf * 4u), so + CF::SF_A + wave * 256,
                d.sc_voff, kt * 4);
      else if (GATED && MAPPED)
        lds_dma4(make_rsrc(maps.a_sf_perm + (size_t)kt * M, (uint32_t)M * 4u), so + CF::SF_A + wave * 256,
                d.sc_voff, 0);
      else
        lds_dma4(make_rsrc(A_sf + (size_t)kt * M, (uint32_t)M * 4u), so + CF::SF_A + wave * 256, d.sc_voff, 0);
    } else {
      // weight scales of k-blocks 4kt..4kt+3, LDS [nb][kb][BN]: load j covers bytes
      // 256 j .. 256 j + 255 of that block, i.e. matrix nb = j*256 / (4 BN), k-block rows of BN
      const int j = wave - 4;
      const int byte = j * 256 + lane * 4;
      const int nb = byte / (4 * BN);
      const int kb = (byte % (4 * BN)) / BN;
      const int col = byte % BN;
      const uint8_t* sfb = (GATED && nb) ? B1_sf : B0_sf;
      lds_dma4(make_rsrc(sfb + ((size_t)d.e * ksf_b + 4 * (size_t)kt) * N, (uint32_t)N * 4u),
              so + CF::SF_B + j * 256, kb * N + d.n0 + col, 0);
    }
  };

  // The first two stages of a tile go out as soon as their buffers are free: for the first
  // tile here, for the others right after the previous tile's K loop (its last barrier
  // follows every read of the buffers they use), so that they land during that tile's
  // epilogue. Each tile's stages continue the buffer rotation of the previous one.
  Tile cur;
  if (slot < total) {
    cur = decode(slot, 0);
    issue(cur, 0);
    if (nk > 1) issue(cur, 1);
  }
  for (int t = slot; t < total; t += G) {
    const int row0 = cur.row0, rows_valid = cur.rows_valid, n0 = cur.n0, nmt = cur.nmt, base = cur.base;
    f32x16_t acc[CF::NB][CF::MT][CF::NT];
#pragma unroll
    for (int nb = 0; nb < CF::NB; ++nb)
#pragma unroll
      for (int mt = 0; mt < CF::MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < CF::NT; ++nt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[nb][mt][nt][i] = 0.f;

    // the K loop over the first MTV row blocks of this wave (MTV fixed at compile time; a
    // wave with none still issues its loads and meets every barrier)
    auto k_loop = [&](auto mtv) {
      constexpr int MTV = decltype(mtv)::value;
      for (int kt = 0; kt < nk; ++kt) {
        // stage kt complete for every wave; stage kt+1 (if any) may still be in flight (and
        // the previous tile's output stores, issued after both, only add to the count). The
        // barrier also means every wave is done with stage kt-1, whose buffer stage kt+2 reuses.
        if (kt + 1 < nk) wait_barrier<CF::VM_PER_STAGE>();
        else wait_barrier<0>();
        if (kt + 2 < nk) issue(cur, kt + 2);
        if constexpr (MTV > 0) {
          const unsigned char* sa_l = smem + ((unsigned)(base + kt) % F8_NS) * CF::STAGE;
          const unsigned char* sb_l = sa_l + CF::A_BYTES;
          // this stage's scales as e8m0 bytes: one per row block (the row's 1x128 block), and
          // per fragment and MFMA step the byte of k-block 2kk + G of the lane's column
          const float* sfa = reinterpret_cast<const float*>(sa_l + CF::SF_A);
          const uint8_t* sfb = sa_l + CF::SF_B;
          int sa[MTV];
#pragma unroll
          for (int mt = 0; mt < MTV; ++mt) sa[mt] = pow2_to_e8m0(sfa[ar + mt * 128]);
#pragma unroll
          for (int kk = 0; kk < CF::KK; ++kk) {
            i32x8_t af[MTV];
#pragma unroll
            for (int mt = 0; mt < MTV; ++mt) {
              const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(sa_l + a_off[kk][0] + mt * 128 * F8_BK);
              const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(sa_l + a_off[kk][1] + mt * 128 * F8_BK);
              af[mt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
#pragma unroll
            for (int nb = 0; nb < CF::NB; ++nb) {
#pragma unroll
              for (int nt = 0; nt < CF::NT; ++nt) {
                const i32x4_t bq = *reinterpret_cast<const i32x4_t*>(sb_l + nb * CF::B_BYTES + b_off[nt][kk]);
                const i32x4_t z = {0, 0, 0, 0};
                const i32x8_t bfr = __builtin_shufflevector(bq, z, 0, 1, 2, 3, 4, 5, 6, 7);
                const int sbw = sfb[(nb * 4 + 2 * kk + g2) * BN + wn * CF::WN + nt * 32 + (lane & 31)];
#pragma unroll
                for (int mt = 0; mt < MTV; ++mt) {
                  if constexpr (ROW_LANES)  // weights (fp4, format 4) as the first operand
                    acc[nb][mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        bfr, af[mt], acc[nb][mt][nt], 4, 0, 0, sbw, 0, sa[mt]);
                  else
                    acc[nb][mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        af[mt], bfr, acc[nb][mt][nt], 0, 4, 0, sa[mt], 0, sbw);
                }
              }
            }
          }
        }
      }
    };
    if (nmt == 2) k_loop(std::integral_constant<int, 2>{});
    else if (nmt == 1) k_loop(std::integral_constant<int, 1>{});
    else k_loop(std::integral_constant<int, 0>{});

    if (t + G < total) {
      cur = decode(t + G, (unsigned)(base + nk) % F8_NS);
      issue(cur, 0);
      if (nk > 1) issue(cur, 1);
    }

    if constexpr (GATED) {
      // Row-lane layout: lane l holds row mt*128 + wm*32 + l%32, and block nt's acc[..][4j+c]
      // is column nt*32 + 8j + 4(l/32) + c of this wave's WN columns. h = silu(g) * u replaces
      // g in place; the row's amax over the wave's columns combines the lane's values with
      // lane l^32's, then over the tile's 128-column scale block with the other column wave's
      // through LDS.
      float rmax[CF::MT];
#pragma unroll
      for (int mt = 0; mt < CF::MT; ++mt) {
        float mx = 0.f;
#pragma unroll
        for (int nt = 0; nt < CF::NT; ++nt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float v = silu_f32(acc[0][mt][nt][i]) * acc[1][mt][nt][i];
            acc[0][mt][nt][i] = v;
            mx = fmaxf(mx, __builtin_fabsf(v));
          }
        rmax[mt] = fmaxf(mx, __shfl_xor(mx, 32, 64));
      }
      if (lane < 32) {
#pragma unroll
        for (int mt = 0; mt < CF::MT; ++mt) xpart[wn * F8_BM + mt * 128 + wm * 32 + lane] = rmax[mt];
      }
      __syncthreads();  // xpart is written again only after the next tile's K loop barriers
#pragma unroll
      for (int mt = 0; mt < CF::MT; ++mt) {
        const int r = mt * 128 + wm * 32 + (lane & 31);
        const bool ok = r < rows_valid;
        const float s = fp8_pow2_scale(fmaxf(xpart[r], xpart[F8_BM + r]));
        const float inv = 1.0f / s;  // exact: s is a power of two
        uint8_t* rowp = C8 + (size_t)(row0 + (ok ? r : 0)) * N + n0 + wn * CF::WN + 8 * (lane >> 5);
#pragma unroll
        for (int nt = 0; nt < CF::NT; ++nt)
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const f32x16_t& h = acc[0][mt][nt];
            const int i0 = 8 * p;
            const uint2 q = pack_row8_e4m3(h[i0] * inv, h[i0 + 1] * inv, h[i0 + 2] * inv, h[i0 + 3] * inv,
                                           h[i0 + 4] * inv, h[i0 + 5] * inv, h[i0 + 6] * inv, h[i0 + 7] * inv);
            if (ok) *reinterpret_cast<uint2*>(rowp + nt * 32 + 16 * p) = q;
          }
        if (ok && wn == 0 && lane < 32) C8_sf[(size_t)(n0 / 128) * M + row0 + r] = s;  // [N/128][M]
      }
    } else if constexpr (MAPPED) {
#pragma unroll
      for (int mt = 0; mt < CF::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = mt * 128 + wm * 32 + 8 * (i >> 2) + 4 * g2 + (i & 3);
          const int src = r < rows_valid ? maps.s_src[row0 + r] : -1;  // -1: padding row
          if (src >= 0) {
            const int gr = row0 + r;
            float* dst = maps.s_acc + (size_t)(src / maps.s_k) * N + n0 + wn * CF::WN + (lane & 31);
            const float w = maps.s_w[gr];
#pragma unroll
            for (int nt = 0; nt < CF::NT; ++nt) unsafeAtomicAdd(dst + nt * 32, w * acc[0][mt][nt][i]);
          }
        }
    } else {
      // row-lane layout as above; 16-byte bf16 row runs
      const int col_l = n0 + wn * CF::WN + 8 * (lane >> 5);
#pragma unroll
      for (int mt = 0; mt < CF::MT; ++mt) {
        const int r = mt * 128 + wm * 32 + (lane & 31);
        const bool ok = r < rows_valid;
        const size_t ro = (size_t)(row0 + (ok ? r : 0)) * N + col_l;
#pragma unroll
        for (int nt = 0; nt < CF::NT; ++nt)
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const uint4 v = pack_row16(acc[0][mt][nt], 8 * p);
            if (ok) *reinterpret_cast<uint4*>(C16 + ro + nt * 32 + 16 * p) = v;
          }
      }
    }
  }
}

template <bool GATED, int BN, bool MAPPED>
static moe_status_t launch_f8_k(const uint8_t* A, const float* A_sf, const int* cu, int M, int E,
                              int Kd, int N, const uint8_t* B0, const uint8_t* B0_sf,
                              const uint8_t* B1, const uint8_t* B1_sf, uint8_t* C8, float* C8_sf,
                              uint16_t* C16, const RowMaps& maps, bool paired, hipStream_t s) {
  using CF = F8Cfg<GATED, BN>;
  static std::atomic<unsigned char> lds_set[MOE_MAX_DEVICES];
  if (ensure_lds_limit(reinterpret_cast<const void*>(&ffn_fp8_kernel<GATED, BN, MAPPED>), CF::LDS_BYTES,
                       lds_set) != MOE_OK)
    return MOE_EHIP;
  ffn_fp8_kernel<GATED, BN, MAPPED><<<device_cu_count(), F8_THREADS, CF::LDS_BYTES, s>>>(
      A, A_sf, cu, M, E, Kd, N, B0, B0_sf, B1, B1_sf, C8, C8_sf, C16, maps, paired ? 1 : 0);
  return launch_status();
}

template <bool GATED, int BN>
static moe_status_t launch_f8(const uint8_t* A, const float* A_sf, const int* cu, int M, int E,
                              int Kd, int N, const uint8_t* B0, const uint8_t* B0_sf,
                              const uint8_t* B1, const uint8_t* B1_sf, uint8_t* C8, float* C8_sf,
                              uint16_t* C16, const RowMaps& maps, bool paired, hipStream_t s) {
  const bool mapped = GATED ? maps.a_src != nullptr : maps.s_acc != nullptr;
  if (mapped)
    return launch_f8_k<GATED, BN, true>(A, A_sf, cu, M, E, Kd, N, B0, B0_sf, B1, B1_sf, C8, C8_sf, C16, maps,
                                        paired, s);
  return launch_f8_k<GATED, BN, false>(A, A_sf, cu, M, E, Kd, N, B0, B0_sf, B1, B1_sf, C8, C8_sf, C16, maps,
                                       paired, s);
}

moe_status_t launch_ffn_gate_up_fp8(const void* x_perm, const float* x_sf, const int* cu, int M,
                                    int E, int H, int Hp, const void* wg, const uint8_t* sg,
                                    const void* wu, const uint8_t* su, void* h, float* h_sf,
                                    const RowMaps& maps, bool paired, hipStream_t s) {
  if (M == 0) return MOE_OK;
  return launch_f8<true, 128>(static_cast<const uint8_t*>(x_perm), x_sf, cu, M, E, H, Hp,
                              static_cast<const uint8_t*>(wg), sg, static_cast<const uint8_t*>(wu),
                              su, static_cast<uint8_t*>(h), h_sf, nullptr, maps, paired, s);
}

moe_status_t launch_ffn_down_fp8(const void* h, const float* h_sf, const int* cu, int M, int E,
                                 int H, int Hp, const void* wd, const uint8_t* sd, void* y,
                                 const RowMaps& maps, bool paired, hipStream_t s) {
  if (M == 0) return MOE_OK;
  return launch_f8<false, 256>(static_cast<const uint8_t*>(h), h_sf, cu, M, E, Hp, H,
                               static_cast<const uint8_t*>(wd), sd, nullptr, nullptr, nullptr,
                               nullptr, static_cast<uint16_t*>(y), maps, paired, s);
}

}  // namespace moe
