// Grouped expert FFN in bf16 on gfx950 matrix cores.
//
// "Distributed expert parallelism", "Grouped expert computation": one launch runs the
// matrix products of every expert over its variable-size group of rows. "Mixture of
// Kittens", Step 1: each expert is Down(SwiGLU(Up x, Gate x)); the gate/up kernel fuses
// SwiGLU into its epilogue (h = silu(x.Wg) * (x.Wu)), the down kernel computes h.Wd.
// MoonEP "Integration": the stacked [E, ., .] weight tensors are addressed purely by expert
// index and cu_seqlens selects each expert's rows.
//
// Two schedules share the tiling, the LDS layouts and the row maps described here: the plain
// kernel ffn_bf16_kernel (this header) and the ping-pong kernel ffn_bf16_pp_kernel further
// down, the default, which differs in its schedule, wave layout and cross-tile prefetch.
// Design (one kernel body, GATED selects gate/up + SwiGLU or the plain down projection):
//  * Persistent grid of one 512-thread block per CU. Each block derives the tile list from
//    cu_seqlens in LDS (tiles per expert = ceil(rows / BM) * N / BN, exclusive prefix) and
//    walks it with stride gridDim. Tile t of round r maps to XCD-contiguous slots, so the
//    32 CUs of one XCD work on neighbouring tiles: the same expert's weight panel (tiles
//    of one n-panel are consecutive over its m-tiles) and the same rows stay in that XCD's
//    L2.
//  * Block tile BM=256 rows x BN columns (per weight matrix), K step 64, two LDS stages
//    (the plain kernel's default; K step 32 with four stages is its other variant).
//    8 waves as 4 (rows) x 2 (columns), each wave 64 x BN/2 with MFMA 32x32x16 bf16 and
//    fp32 accumulators (128 per lane). A wave's two 32-row blocks are rows wm*32 + [0,32)
//    and 128 + wm*32 + [0,32): with this interleave the padded rows of an expert's last tile
//    fall evenly on the four SIMDs (waves w and w+4 share one), and a wave skips the MFMAs
//    and fragment reads of any 32-row block that lies wholly past the group's rows.
//  * A (activations, reduction-contiguous) is staged as [256][64] with the 16-byte chunk
//    index XOR-swizzled by (row/2) mod 8 so ds_read_b128 of 16 consecutive rows is free of
//    bank conflicts. B (weights [K][N], N contiguous) is staged in its global layout and
//    turned into the MFMA B operand by ds_read_b64_tr_b16 (two per fragment); its 32-byte
//    segments are XOR-swizzled by 2*(row mod 4) so the four rows a transpose read touches
//    land on distinct banks.
//  * Global loads for step k+1 are issued before the MFMAs of step k; one barrier per step.
//  * Rows past the group's last row of the tile are loaded out of the A descriptor's range,
//    so they read as zeros without memory traffic; they are never stored.
//  * Optional row maps ("Mixture of Kittens", Step 6 gathers its inputs by token index and
//    scatters its outputs): with `a_src`, A row r of the group is
//    row a_src[r] / a_k of A (the token matrix x, no permuted copy); with `s_acc`, the down
//    epilogue adds s_w[r] * y[r] into s_acc[s_src[r] / s_k] with fp32 atomics instead of
//    storing y (the weighted combine fused into the down projection). A negative source
//    index marks a padding row of a padded layout: it gathers zeros and scatters nothing.
#include "lds_dma.h"
#include "moe_common.h"
#include "tile_sched.h"

#include <cstdlib>
#include <cstring>
#include <type_traits>

namespace moe {

constexpr int FB_BM = 256;
constexpr int FB_THREADS = 512;
constexpr int FB_MAX_E = 1024;

template <bool GATED, int BN, int BK, int NS>
struct FbCfg {
  static constexpr int NB = GATED ? 2 : 1;
  static constexpr int WN = BN / 2;
  static constexpr int NT = WN / 32;
  static constexpr int MT = 2;
  static constexpr int KK = BK / 16;                   // MFMA k-steps per stage
  static constexpr int CPR = BK / 8;                   // 16-byte chunks per staged A row
  static constexpr int A_ROW = BK * 2;
  static constexpr int A_BYTES = FB_BM * A_ROW;
  static constexpr int A_RPL = 1024 / A_ROW;           // A rows one wave load fills
  static constexpr int A_LD = A_BYTES / (1024 * 8);    // A loads per wave per stage
  static constexpr int A_SWZ_DIV = 16 / CPR;           // rows sharing one swizzle value
  static constexpr int B_ROW = BN * 2;                 // bytes per staged weight row
  static constexpr int B_BYTES = BK * B_ROW;           // per matrix
  static constexpr int B_RPL = 1024 / B_ROW;           // weight rows one wave load fills
  static constexpr int B_LD = NB * B_BYTES / (1024 * 8);
  static constexpr int STAGE = A_BYTES + NB * B_BYTES;
  static constexpr int VM_PER_STAGE = A_LD + B_LD;     // vector-memory ops per lane per stage
  static constexpr int SCHED_BYTES = (FB_MAX_E + 1 + 16) * 4;
  static constexpr int LDS_BYTES = NS * STAGE + SCHED_BYTES;
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for one load per wave");
  static_assert(VM_PER_STAGE * (NS - 2) < 16, "vmcnt wait count out of range");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <bool GATED, int BN, int BK, int NS, bool MAPPED>
__global__ __launch_bounds__(FB_THREADS, 1) void ffn_bf16_kernel(
    const uint16_t* __restrict__ A, const int* __restrict__ cu, int M, int E, int Kd, int N,
    const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, uint16_t* __restrict__ C,
    int n_fastest, RowMaps maps) {
  using CF = FbCfg<GATED, BN, BK, NS>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int* tstart = reinterpret_cast<int*>(smem + NS * CF::STAGE);
  int* wsum = tstart + FB_MAX_E + 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;  // 0..3: 64-row strip
  const int wn = wave & 1;   // 0..1: BN/2-column half
  const int ntn = N / BN;
  const int total = build_tile_prefix<FB_BM, FB_THREADS>(cu, E, ntn, tstart, wsum);
  const int nk = Kd / BK;
  const int G = gridDim.x;
  const int slot = xcd_slot(blockIdx.x, G);

  // ---- global -> LDS (direct). A stage: [256 rows][BK] bf16; 16-byte slot p of row r holds
  // chunk p ^ ((r / A_SWZ_DIV) % CPR), so 16 consecutive rows of one chunk hit 16 distinct
  // bank groups. Wave load j (j = wave + 8 i) fills rows [j*A_RPL, (j+1)*A_RPL), lane l ->
  // row j*A_RPL + l / CPR, slot l % CPR.
  // (when gathering, a_voff is reset per tile from the tile's source rows)
  int a_voff[CF::A_LD], a_ldo[CF::A_LD], a_row[CF::A_LD];
#pragma unroll
  for (int i = 0; i < CF::A_LD; ++i) {
    const int j = wave + 8 * i;
    const int r = j * CF::A_RPL + lane / CF::CPR;
    const int p = lane % CF::CPR;
    a_row[i] = r;
    a_voff[i] = r * Kd * 2 + ((p ^ ((r / CF::A_SWZ_DIV) % CF::CPR)) << 4);
    a_ldo[i] = j * 1024;
  }
  // B stage per matrix: [BK rows][BN] bf16; 32-byte segment s of row k stored at
  // s ^ 2*(k % 4). Wave load j covers B_RPL rows of matrix j / (B_BYTES / 1024).
  int b_voff[CF::B_LD], b_ldo[CF::B_LD], b_mat[CF::B_LD];
#pragma unroll
  for (int i = 0; i < CF::B_LD; ++i) {
    const int j = wave + 8 * i;
    const int per_mat = CF::B_BYTES / 1024;
    const int nb = j / per_mat;
    const int r = (j % per_mat) * CF::B_RPL + lane / (64 / CF::B_RPL);
    const int q = lane % (64 / CF::B_RPL);  // 16-byte slot within the row
    const int sgm = (q >> 1) ^ ((r & 3) << 1);
    b_voff[i] = r * N * 2 + ((sgm << 1) + (q & 1)) * 16;
    b_ldo[i] = CF::A_BYTES + j * 1024;
    b_mat[i] = nb;
  }

  // ---- LDS -> MFMA fragments (block mt of this wave: rows mt*128 + wm*32 + lane%32; the
  // swizzle term depends on lane%32 only, since 32 and 128 are multiples of A_SWZ_DIV*CPR)
  static_assert((32 / CF::A_SWZ_DIV) % CF::CPR == 0, "row interleave must keep the A swizzle");
  const int a_fbase = (wm * 32 + (lane & 31)) * CF::A_ROW;
  const int a_sw = ((lane & 31) / CF::A_SWZ_DIV) % CF::CPR;
  int a_fk[CF::KK];
#pragma unroll
  for (int kk = 0; kk < CF::KK; ++kk) a_fk[kk] = a_fbase + ((((kk << 1) | (lane >> 5)) ^ a_sw) << 4);
  const int g = lane >> 4, jj = lane & 15;
  const int bP = (wn * CF::WN) / 16 + (g & 1);
  const int b_fbase = (8 * (g >> 1) + (jj >> 2)) * CF::B_ROW + 8 * (jj & 3) + ((bP ^ ((jj >> 2) << 1)) << 5);
  int b_fn[CF::NT];
#pragma unroll
  for (int nt = 0; nt < CF::NT; ++nt) b_fn[nt] = b_fbase ^ (nt << 6);
  const uint32_t smem_lds = lds_addr(smem);

  for (int t = slot; t < total; t += G) {
    const int e = find_expert(tstart, E, t);
    const int lt = t - tstart[e];
    const int gbeg = cu[e];
    const int rows_e = cu[e + 1] - gbeg;
    const int mte = (rows_e + FB_BM - 1) / FB_BM;
    // tile order inside an expert: m fastest (a weight panel's m-tiles are neighbours) or
    // n fastest (neighbours cover whole weight rows, one m-tile at a time)
    const int ntile = n_fastest ? lt % ntn : lt / mte;
    const int mtile = n_fastest ? lt / ntn : lt - ntile * mte;
    const int chunk = even_chunk(rows_e, mte);
    const int row0 = gbeg + mtile * chunk;
    const int rows_valid = min(chunk, rows_e - mtile * chunk);
    const int n0 = ntile * BN;

    // A rows of this tile: rows past rows_valid get an offset past the descriptor's range.
    // Plain: the descriptor starts at row row0 and spans rows_valid rows (< 2^31 bytes by the
    // host checks). Gathered: it spans all a_rows rows of A (< 2^31 bytes, host checks).
    i32x4_t rA;
    int a_off[CF::A_LD];
    if constexpr (GATED && MAPPED) {
      // the chunk part of a_voff is (a_voff - row * Kd * 2); the row part is replaced by the
      // source row's offset
      rA = make_rsrc(A, (uint32_t)maps.a_rows * (uint32_t)Kd * 2u);
#pragma unroll
      for (int i = 0; i < CF::A_LD; ++i) {
        const int src = a_row[i] < rows_valid ? maps.a_src[row0 + a_row[i]] : -1;  // -1: padding row
        a_off[i] = src >= 0 ? (src / maps.a_k - a_row[i]) * Kd * 2 + a_voff[i] : (int)0x80000000u;
      }
    } else {
      rA = make_rsrc(A + (size_t)row0 * Kd, (uint32_t)rows_valid * (uint32_t)Kd * 2u);
#pragma unroll
      for (int i = 0; i < CF::A_LD; ++i) a_off[i] = a_voff[i];
    }
    // 32-row blocks of this wave that hold rows of the group (block 1 implies block 0)
    const int nmt = __builtin_amdgcn_readfirstlane((wm * 32 < rows_valid) + (128 + wm * 32 < rows_valid));
    const size_t woff = (size_t)e * Kd * N + n0;
    const uint32_t b_rem = (uint32_t)(((size_t)Kd * N - n0) * 2);
    const i32x4_t rB0 = make_rsrc(B0 + woff, b_rem);
    const i32x4_t rB1 = GATED ? make_rsrc(B1 + woff, b_rem) : rB0;

    auto issue = [&](int kt) {  // A_LD + B_LD direct loads per lane for stage kt
      const uint32_t so = smem_lds + (uint32_t)((kt % NS) * CF::STAGE);
#pragma unroll
      for (int i = 0; i < CF::A_LD; ++i) lds_dma16(rA, so + a_ldo[i], a_off[i], kt * BK * 2);
#pragma unroll
      for (int i = 0; i < CF::B_LD; ++i)
        lds_dma16(b_mat[i] ? rB1 : rB0, so + b_ldo[i], b_voff[i], kt * BK * N * 2);
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

    __syncthreads();  // previous tile's readers are done with every stage
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
      if (s < nk) issue(s);
    // the K loop over the first MTV row blocks of this wave (MTV fixed at compile time; a
    // wave with none still issues its loads and meets every barrier)
    auto k_loop = [&](auto mtv) {
      constexpr int MTV = decltype(mtv)::value;
      for (int kt = 0; kt < nk; ++kt) {
        // stage kt has landed once at most (stages issued after it) * VM_PER_STAGE remain
        wait_barrier_dyn<CF::VM_PER_STAGE*(NS - 2)>(min(NS - 2, nk - 1 - kt) * CF::VM_PER_STAGE);
        if (kt + NS - 1 < nk) issue(kt + NS - 1);
        if constexpr (MTV > 0) {
          const unsigned char* sa = smem + (kt % NS) * CF::STAGE;
          const unsigned char* sb = sa + CF::A_BYTES;
#pragma unroll
          for (int kk = 0; kk < CF::KK; ++kk) {
            bf16x8_t af[MTV];
#pragma unroll
            for (int mt = 0; mt < MTV; ++mt)
              af[mt] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const i32x4_t*>(sa + a_fk[kk] + mt * 128 * CF::A_ROW));
#pragma unroll
            for (int nb = 0; nb < CF::NB; ++nb) {
#pragma unroll
              for (int nt = 0; nt < CF::NT; ++nt) {
                const unsigned char* p = sb + nb * CF::B_BYTES + b_fn[nt] + kk * 16 * CF::B_ROW;
                const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4_t*)(p));
                const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4_t*)(p + 4 * CF::B_ROW));
                const bf16x8_t bfr = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int mt = 0; mt < MTV; ++mt)
                  acc[nb][mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mt], bfr, acc[nb][mt][nt], 0, 0, 0);
              }
            }
          }
        }
      }
    };
    if (nmt == 2) k_loop(std::integral_constant<int, 2>{});
    else if (nmt == 1) k_loop(std::integral_constant<int, 1>{});
    else k_loop(std::integral_constant<int, 0>{});

    // epilogue: lane holds column lane%32 of rows 8*(i/4) + 4*(lane/32) + i%4
    if constexpr (!GATED && MAPPED) {
#pragma unroll
      for (int mt = 0; mt < CF::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = mt * 128 + wm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
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
#pragma unroll
      for (int mt = 0; mt < CF::MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < CF::NT; ++nt) {
          const int col = n0 + wn * CF::WN + nt * 32 + (lane & 31);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = mt * 128 + wm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            if (r < rows_valid) {
              float v;
              if constexpr (GATED) {
                v = silu_f32(acc[0][mt][nt][i]) * acc[1][mt][nt][i];
                if (maps.save_g) {
                  maps.save_g[(size_t)(row0 + r) * N + col] = f32_to_bf16_bits(acc[0][mt][nt][i]);
                  maps.save_u[(size_t)(row0 + r) * N + col] = f32_to_bf16_bits(acc[1][mt][nt][i]);
                }
              } else {
                v = acc[0][mt][nt][i];
              }
              C[(size_t)(row0 + r) * N + col] = f32_to_bf16_bits(v);
            }
          }
        }
    }
  }
}

// ---- ping-pong schedule ---------------------------------------------------------------
// The default kernel. Same tiles (256 rows x BN columns), A/B LDS layouts and swizzles as
// ffn_bf16_kernel; by default K step BK = 32 with four stages (BK = 64 with two stages is
// the older variant). The eight waves form two groups of four, waves 0-3 and 4-7, so each
// SIMD holds one wave of each. Time is cut into slots, one per MFMA half-stage (two 16-deep
// k-steps) and group, separated by workgroup barriers. In every slot one wave of a SIMD runs
// its MFMAs from fragments already in its registers while its partner reads the fragments of
// its next slot from LDS (and, in group 0, issues the direct global->LDS loads of a later
// stage). With the plain schedule both waves of a SIMD waited for the same stage and then
// computed together, so load time and compute time added up.
//
//   group 0: read kt   | compute kt | read kt+1 | compute kt+1 | ...
//   group 1:  (wait)   | read kt    | compute kt | read kt+1   | ...
// Both groups execute the same instruction sequence; group 1 passes one extra barrier at the
// start (and group 0 one at the end), which is all that offsets them. Group 0 issues the
// direct loads of stage kt+NS-1 while reading stage kt (into the buffer of stage kt-1, which
// group 1 finished reading one slot earlier) and, before the last barrier of stage kt, waits
// until stage kt+1 has landed, so a stage has NS-1 steps to land. Every barrier is preceded
// by lgkmcnt(0), so no LDS read of a buffer is in flight when a later slot refills it. The
// wave layout (column strips, even/odd row blocks) and the cross-tile prefetch are described
// at the kernel.
__device__ __forceinline__ void pp_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// With PF (cross-tile prefetch) the next tile of the block is decoded inside the K loop of
// the current one, from LDS copies of the tile prefix and cu_seqlens; when gathering, group 0
// loads its 256 row sources straight into LDS NS steps before they are needed, counting that
// load in its stage waits. The next tile's stages 0..NS-2 then go out in the last NS-1 K steps
// (the slots that load nothing for the current tile) into the buffers they use in the next
// tile (stage s -> buffer s % NS needs nk % NS == 0), and only stage NS-1 is issued after
// the last barrier. Needs nk >= 2 NS: the decode happens at K step kd = nk - 2 NS + 1 >= 1.
// NTB (gate/up only): load the weight panels non-temporally; chosen by the host when the
// average group fits one m-tile (see launch_fb_any).
template <bool GATED, int BN, int BK, int NS, bool MAPPED, bool PF, bool NTB = false>
__global__ __launch_bounds__(FB_THREADS, 1) void ffn_bf16_pp_kernel(
    const uint16_t* __restrict__ A, const int* __restrict__ cu, int M, int E, int Kd, int N,
    const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, uint16_t* __restrict__ C,
    int n_fastest, RowMaps maps) {
  using CF = FbCfg<GATED, BN, BK, NS>;
  constexpr int KH = 2;                                   // MFMA k-steps per slot
  constexpr int UPS = CF::KK / KH;                        // slots (units) per stage: 2 or 1
  constexpr int A_LDP = CF::A_BYTES / (1024 * 4);         // A loads per group-0 wave per stage
  constexpr int B_LDP = CF::NB * CF::B_BYTES / (1024 * 4);
  constexpr int VMG = A_LDP + B_LDP;
  constexpr int PER_MAT = CF::B_BYTES / 1024;             // 1 KiB weight loads per matrix
  // Wave layout: the block's columns form four strips of WS = BN/4 (PNT 32-column MFMA
  // blocks, per weight matrix); waves w and w+4 share a SIMD and strip w % 4, and split its
  // 32-row blocks between them, wave w the even ones (0, 2, 4, 6) and wave w+4 the odd ones.
  // A tile of b row blocks gives the two waves of a SIMD ceil(b/2) and floor(b/2) blocks, so
  // their slots stay even on the 192-row tiles an expert of 384 rows splits into.
  constexpr int PMT = 4;                                  // row blocks per wave (at most)
  constexpr int WS = BN / 4;
  constexpr int PNT = WS / 32;
  constexpr int NF = CF::NB * PNT;                        // B fragments per k-step
  // Operand order of the MFMA. With the weight fragment first the accumulator comes out
  // transposed: lane l holds one output row (l % 32 of the 32-row block) and four runs of four
  // consecutive columns, which the epilogue writes as 8-byte stores. The scatter epilogue keeps
  // the other order, where the 32 lanes of a row add into 32 consecutive floats of one token.
  constexpr bool ROW_LANES = !(!GATED && MAPPED);
  static_assert(CF::KK % KH == 0 && PER_MAT % 4 == 0 && A_LDP >= 1, "ping-pong tiling");
  static_assert(VMG * (NS - 1) < 64, "vmcnt range");
  static_assert(!PF || NS >= 3, "prefetch needs at least three stages");
  // a row-source load rides in group 0's stage waits when prefetching a gathered tile
  constexpr bool XA = PF && GATED && MAPPED;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int* tstart = reinterpret_cast<int*>(smem + NS * CF::STAGE);
  int* wsum = tstart + FB_MAX_E + 1;
  int* cu_l = wsum + 16;              // PF: copy of cu_seqlens[0..E]
  int* src_l = cu_l + FB_MAX_E + 1;   // PF, gathering: the next tile's FB_BM row sources

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sc = wave & 3;            // column strip
  const int hf = wave >> 2;           // 0: even row blocks, 1: odd ones
  const bool g0 = wave < 4;
  const int gw = wave & 3;
  const int ntn = N / BN;
  if constexpr (PF)
    for (int i = tid; i <= E; i += FB_THREADS) cu_l[i] = cu[i];  // ordered by the prefix's barriers
  const int total = build_tile_prefix<FB_BM, FB_THREADS>(cu, E, ntn, tstart, wsum);
  const int nk = Kd / BK;
  const int kd = nk - 2 * NS + 1;     // PF: K step at which the next tile is decoded
  const int G = gridDim.x;
  const int slot = xcd_slot(blockIdx.x, G);

  // loads of group-0 wave gw: A load j = gw + 4i fills rows [8j, 8j+8); weight load
  // j = gw + 4i fills B_RPL rows of matrix j / PER_MAT. The weight offsets differ only by
  // whole rows, uniform over the wave, so they ride in the scalar offset.
  int a_row[A_LDP], a_voff[A_LDP];
#pragma unroll
  for (int i = 0; i < A_LDP; ++i) {
    const int j = gw + 4 * i;
    const int r = j * CF::A_RPL + lane / CF::CPR;
    const int p = lane % CF::CPR;
    a_row[i] = r;
    a_voff[i] = r * Kd * 2 + ((p ^ ((r / CF::A_SWZ_DIV) % CF::CPR)) << 4);
  }
  int b_voff0;
  {
    const int r = gw * CF::B_RPL + lane / (64 / CF::B_RPL);
    const int q = lane % (64 / CF::B_RPL);
    const int sgm = (q >> 1) ^ ((r & 3) << 1);
    b_voff0 = r * N * 2 + ((sgm << 1) + (q & 1)) * 16;
  }

  // LDS -> fragment offsets (as in ffn_bf16_kernel)
  // (row block 2 mt + hf starts 64 mt rows after block hf; the A swizzle repeats every 16 rows)
  const int a_fbase = (hf * 32 + (lane & 31)) * CF::A_ROW;
  const int a_sw = ((lane & 31) / CF::A_SWZ_DIV) % CF::CPR;
  int a_fk[CF::KK];
#pragma unroll
  for (int kk = 0; kk < CF::KK; ++kk) a_fk[kk] = a_fbase + ((((kk << 1) | (lane >> 5)) ^ a_sw) << 4);
  const int g = lane >> 4, jj = lane & 15;
  const int bP = (sc * WS) / 16 + (g & 1);
  const int b_fbase = (8 * (g >> 1) + (jj >> 2)) * CF::B_ROW + 8 * (jj & 3) + ((bP ^ ((jj >> 2) << 1)) << 5);
  const uint32_t smem_lds = lds_addr(smem);
  constexpr int SRC_OFF = NS * CF::STAGE + CF::SCHED_BYTES + (FB_MAX_E + 1) * 4;  // src_l in smem

  // one output tile: its expert, rows, columns and load descriptors
  struct Tile {
    int e, row0, rows_valid, n0, nmt;
    bool stream_b;   // NTB: the expert has one m-tile, so this tile is its panel's only reader
    i32x4_t rA, rB0, rB1;
    int a_off[A_LDP];
  };
  // A offsets of a gathered tile from the sources of this wave's A rows. The rows past the
  // tile read a clamped source and are then pointed out of range. -1: padding row.
  auto gather_offsets = [&](Tile& d, const int (&src)[A_LDP]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_LDP; ++i) {
      const int off = (src[i] / maps.a_k - a_row[i]) * Kd * 2 + a_voff[i];
      d.a_off[i] = (a_row[i] < d.rows_valid && src[i] >= 0) ? off : (int)0x80000000u;
    }
  };
  // tile t of expert e, whose rows start at gbeg: everything but a gathered tile's A offsets
  auto decode_tile = [&](int t, int e, int gbeg, int rows_e) __attribute__((always_inline)) {
    Tile d;
    d.e = e;
    const int lt = t - tstart[e];
    const int mte = (rows_e + FB_BM - 1) / FB_BM;
    const int ntile = n_fastest ? lt % ntn : lt / mte;
    const int mtile = n_fastest ? lt / ntn : lt - ntile * mte;
    const int chunk = even_chunk(rows_e, mte);
    d.row0 = gbeg + mtile * chunk;
    d.rows_valid = min(chunk, rows_e - mtile * chunk);
    d.n0 = ntile * BN;
    d.stream_b = NTB && __builtin_amdgcn_readfirstlane(mte) == 1;
    if constexpr (GATED && MAPPED) {
      d.rA = make_rsrc(A, (uint32_t)maps.a_rows * (uint32_t)Kd * 2u);
    } else {
      d.rA = make_rsrc(A + (size_t)d.row0 * Kd, (uint32_t)d.rows_valid * (uint32_t)Kd * 2u);
#pragma unroll
      for (int i = 0; i < A_LDP; ++i) d.a_off[i] = a_voff[i];
    }
    const size_t woff = (size_t)e * Kd * N + d.n0;
    const uint32_t b_rem = (uint32_t)(((size_t)Kd * N - d.n0) * 2);
    d.rB0 = make_rsrc(B0 + woff, b_rem);
    d.rB1 = GATED ? make_rsrc(B1 + woff, b_rem) : d.rB0;
    // row blocks hf, hf + 2, ... below the tile's ceil(rows_valid / 32) blocks
    d.nmt = __builtin_amdgcn_readfirstlane(min(PMT, ((d.rows_valid + 31) / 32 - hf + 1) / 2));
    return d;
  };
  auto decode = [&](int t) __attribute__((always_inline)) {
    const int e = find_expert(tstart, E, t);
    const int gbeg = cu[e];
    Tile d = decode_tile(t, e, gbeg, cu[e + 1] - gbeg);
    if constexpr (GATED && MAPPED) {
      // Branch-free so that the loads go out together: each reads a row of this tile (also
      // for rows past it), and the offset is chosen after the arithmetic.
      int src[A_LDP];
#pragma unroll
      for (int i = 0; i < A_LDP; ++i) src[i] = maps.a_src[d.row0 + min(a_row[i], d.rows_valid - 1)];
      gather_offsets(d, src);
    }
    return d;
  };
  // PF: tile t, a later tile than one of expert e_prev, from LDS only. The tile prefix is
  // nondecreasing and tstart[E] = total > t, so the owner is e_prev plus the number of
  // experts after it that start at or before t, counted 64 at a time with a ballot.
  auto decode_next = [&](int t, int e_prev) __attribute__((always_inline)) {
    int e = e_prev;
    for (;;) {
      const int i = e + 1 + lane;
      const int c = __popcll(__ballot(i < E && tstart[min(i, E)] <= t));
      e += c;
      if (c < 64) break;
    }
    const int gbeg = __builtin_amdgcn_readfirstlane(cu_l[e]);
    return decode_tile(t, e, gbeg, __builtin_amdgcn_readfirstlane(cu_l[e + 1]) - gbeg);
  };
  // group 0 only: this wave's share of stage kt of tile d
  auto issue = [&](const Tile& d, int kt) __attribute__((always_inline)) {
    const uint32_t so = smem_lds + (uint32_t)((kt % NS) * CF::STAGE);
#pragma unroll
    for (int i = 0; i < A_LDP; ++i) lds_dma16(d.rA, so + (gw + 4 * i) * 1024, d.a_off[i], kt * BK * 2);
#pragma unroll
    for (int i = 0; i < B_LDP; ++i) {
      const int j = gw + 4 * i;  // j / PER_MAT == (4 i) / PER_MAT since gw < 4
      const int rows = ((4 * i) % PER_MAT) * CF::B_RPL;
      // NTB: a tile whose expert has a single m-tile is its weight panel's only reader; the
      // panel streams past the caches (non-temporal), which keeps them for the activation rows
      // that the expert's other n-tiles read again (T=8192 E=384 K=8, about 170 rows per
      // expert: gate/up 5.11 -> 4.97 ms). Panels shared by several m-tiles (hot experts) keep
      // the default policy, so the m-tiles after the first find them in L2.
      if (GATED && NTB && d.stream_b)
        lds_dma16_nt(((4 * i) / PER_MAT) ? d.rB1 : d.rB0, so + CF::A_BYTES + j * 1024, b_voff0,
                     kt * BK * N * 2 + rows * N * 2);
      else
        lds_dma16(((4 * i) / PER_MAT) ? d.rB1 : d.rB0, so + CF::A_BYTES + j * 1024, b_voff0,
                  kt * BK * N * 2 + rows * N * 2);
    }
  };

  // The first NS stages of a tile go out as soon as the buffers are free: for the first tile
  // here, for the others right after the previous tile's last MFMA read, so that they land
  // while that tile's outputs are being written.
  Tile cur;
  if (slot < total) {
    cur = decode(slot);
    if (g0)
      for (int st = 0; st < NS && st < nk; ++st) issue(cur, st);
  }
  for (int t = slot; t < total; t += G) {
    const int row0 = cur.row0, rows_valid = cur.rows_valid, n0 = cur.n0, nmt = cur.nmt;
    const bool has_next = t + G < total;
    Tile nxt;

    f32x16_t acc[CF::NB][PMT][PNT];
#pragma unroll
    for (int nb = 0; nb < CF::NB; ++nb)
#pragma unroll
      for (int mt = 0; mt < PMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < PNT; ++nt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[nb][mt][nt][i] = 0.f;

    auto run = [&](auto mtv) __attribute__((always_inline)) {
      constexpr int MTV = decltype(mtv)::value;
      bf16x8_t fa[MTV > 0 ? MTV : 1][KH];
      bf16x8_t fb[NF][KH];
      // read the fragments of half HF of stage kt
      auto mread = [&](int kt, auto hfc) __attribute__((always_inline)) {
        constexpr int HF = decltype(hfc)::value;
        if constexpr (MTV > 0) {
          const unsigned char* sa = smem + (kt % NS) * CF::STAGE;
          const unsigned char* sb = sa + CF::A_BYTES;
#pragma unroll
          for (int q = 0; q < KH; ++q) {
            const int kk = HF * KH + q;
#pragma unroll
            for (int mt = 0; mt < MTV; ++mt)
              fa[mt][q] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const i32x4_t*>(sa + a_fk[kk] + mt * 64 * CF::A_ROW));
#pragma unroll
            for (int nb = 0; nb < CF::NB; ++nb)
#pragma unroll
              for (int nt = 0; nt < PNT; ++nt) {
                const unsigned char* p = sb + nb * CF::B_BYTES + (b_fbase ^ (nt << 6)) + kk * 16 * CF::B_ROW;
                const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4_t*)(p));
                const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4_t*)(p + 4 * CF::B_ROW));
                fb[nb * PNT + nt][q] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
              }
          }
        }
      };
      auto compute = [&]() __attribute__((always_inline)) {
        if constexpr (MTV > 0) {
#pragma unroll
          for (int q = 0; q < KH; ++q)
#pragma unroll
            for (int nb = 0; nb < CF::NB; ++nb)
#pragma unroll
              for (int nt = 0; nt < PNT; ++nt)
#pragma unroll
                for (int mt = 0; mt < MTV; ++mt) {
                  if constexpr (ROW_LANES)
                    acc[nb][mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[nb * PNT + nt][q], fa[mt][q],
                                                                              acc[nb][mt][nt], 0, 0, 0);
                  else
                    acc[nb][mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mt][q], fb[nb * PNT + nt][q],
                                                                              acc[nb][mt][nt], 0, 0, 0);
                }
        }
      };
      constexpr std::integral_constant<int, 0> H0{};
      constexpr std::integral_constant<int, 1> H1{};
      // Both groups run the same sequence (read, barrier, compute, barrier per slot);
      // group 1 starts one barrier later, which puts it one slot behind group 0.
      // stages 0 .. NS-1 are in flight; stage 0 has landed once at most the younger ones are
      // outstanding (the previous tile's output stores, issued after them, can only add to
      // the count, so they never end the wait early)
      if (g0) wait_vm_dyn<VMG * (NS - 1)>(min(NS - 1, nk - 1) * VMG);
      pp_barrier();                 // stage 0 has landed for everyone
      if (!g0) pp_barrier();        // group 1: one slot behind
      // One K step. The steps before kd (all of them without prefetch, or without a next
      // tile) run the plain body; the last 2 NS - 1 steps of a tile with a successor also
      // decode it, load its row sources and issue its first stages.
      auto step = [&](int kt, auto tailc) __attribute__((always_inline)) {
        constexpr bool TAIL = decltype(tailc)::value;
        mread(kt, H0);
        // buffer (kt+NS-1) % NS held stage kt-1, whose last reader (group 1) is done
        if constexpr (TAIL) {
          if constexpr (XA) {
            // the row sources landed before the last barrier of step kd + NS - 1; step kd + NS
            // is also the first to issue a stage of the next tile
            if (g0 && kt == kd + NS) {
              int src[A_LDP];
#pragma unroll
              for (int i = 0; i < A_LDP; ++i) src[i] = src_l[min(a_row[i], nxt.rows_valid - 1)];
              gather_offsets(nxt, src);
            }
          }
          if (g0) {
            if (kt + NS - 1 < nk) issue(cur, kt + NS - 1);
            else issue(nxt, kt + NS - 1 - nk);
          }
          if (kt == kd) {
            nxt = decode_next(t + G, cur.e);
            // group-0 wave gw loads row sources [64 gw, 64 gw + 64) of the next tile, after
            // stage kd + NS - 1; the entries past its rows read as zeros and are never used
            if (XA && g0)
              lds_dma4(make_rsrc(maps.a_src + nxt.row0, (uint32_t)nxt.rows_valid * 4u),
                       smem_lds + (uint32_t)(SRC_OFF + 256 * gw), (64 * gw + lane) * 4, 0);
          }
        } else {
          if (g0 && kt >= 1 && kt + NS - 1 < nk) issue(cur, kt + NS - 1);
        }
        pp_barrier();
        compute();
        if constexpr (UPS == 2) {
          pp_barrier();
          mread(kt, H1);
          pp_barrier();
          compute();
        }
        // stage kt+1 landed before it is read (younger stages may stay in flight)
        if constexpr (TAIL) {
          // NS-2 younger stages are always in flight (some of them the next tile's), and the
          // row-source load issued at step kd after stage kd+NS-1 is younger than stage kt+1
          // for kt <= kd+NS-2
          if (g0 && kt + 1 < nk) wait_vm_dyn<VMG * (NS - 2) + XA>((NS - 2) * VMG + (XA && kt <= kd + NS - 2));
        } else {
          if (g0 && kt + 1 < nk) wait_vm_dyn<VMG * (NS - 2)>(min(NS - 2, nk - 2 - kt) * VMG);
        }
        pp_barrier();
      };
      const int kmain = (PF && has_next) ? kd : nk;
      for (int kt = 0; kt < kmain; ++kt) step(kt, std::false_type{});
      if constexpr (PF)
        for (int kt = kmain; kt < nk; ++kt) step(kt, std::true_type{});
      if (g0) pp_barrier();         // same number of barriers in both groups
    };
    if (nmt == 4) run(std::integral_constant<int, 4>{});
    else if (nmt == 3) run(std::integral_constant<int, 3>{});
    else if (nmt == 2) run(std::integral_constant<int, 2>{});
    else if (nmt == 1) run(std::integral_constant<int, 1>{});
    else run(std::integral_constant<int, 0>{});
    // The last barrier of run() follows every LDS read of this tile in both groups, so every
    // buffer is free: the next tile's first stages go out before this tile's stores.
    if constexpr (PF) {
      if (has_next) {
        cur = nxt;
        if (g0) issue(cur, NS - 1);   // into the buffer of this tile's last stage
      }
    } else {
      if (t + G < total) {
        cur = decode(t + G);
        if (g0)
          for (int st = 0; st < NS && st < nk; ++st) issue(cur, st);
      }
    }

    // epilogue
    if constexpr (!GATED && MAPPED) {
#pragma unroll
      for (int mt = 0; mt < PMT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = (2 * mt + hf) * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          const int src = r < rows_valid ? maps.s_src[row0 + r] : -1;
          if (src >= 0) {
            float* dst = maps.s_acc + (size_t)(src / maps.s_k) * N + n0 + sc * WS + (lane & 31);
            const float w = maps.s_w[row0 + r];
#pragma unroll
            for (int nt = 0; nt < PNT; ++nt) unsafeAtomicAdd(dst + nt * 32, w * acc[0][mt][nt][i]);
          }
        }
    } else {
      // row-lane layout: block (mt, nt) holds row (2 mt + hf)*32 + lane%32 in this lane, and
      // columns nt*32 + 8j + 4(lane/32) + c in acc[..][4j + c], j, c = 0..3
      const int col_l = n0 + sc * WS + 8 * (lane >> 5);
#pragma unroll
      for (int mt = 0; mt < PMT; ++mt) {
        const int r = (2 * mt + hf) * 32 + (lane & 31);
        const bool ok = r < rows_valid;
        const size_t ro = (size_t)(row0 + (ok ? r : 0)) * N + col_l;
#pragma unroll
        for (int nt = 0; nt < PNT; ++nt)
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const size_t o = ro + nt * 32 + 16 * p;
            const f32x16_t& a0 = acc[0][mt][nt];
            const int i0 = 8 * p;
            uint4 v;  // this lane's 16 bytes of C
            if constexpr (GATED) {
              const f32x16_t& a1 = acc[1][mt][nt];
              float h[8];
#pragma unroll
              for (int c = 0; c < 8; ++c) h[c] = silu_f32(a0[i0 + c]) * a1[i0 + c];
              v = pack_row16(h[0], h[1], h[2], h[3], h[4], h[5], h[6], h[7]);
              if (maps.save_g) {
                const uint4 g = pack_row16(a0, i0), u = pack_row16(a1, i0);
                if (ok) {
                  *reinterpret_cast<uint4*>(maps.save_g + o) = g;
                  *reinterpret_cast<uint4*>(maps.save_u + o) = u;
                }
              }
            } else {
              v = pack_row16(a0, i0);
            }
            if (ok) *reinterpret_cast<uint4*>(C + o) = v;
          }
      }
    }
  }
}

// Tile order inside an expert group. MOE_FFN_ORDER = "m" | "n" overrides the default.
static int tile_order_n_fastest(int M, int E) {
  const char* p = std::getenv("MOE_FFN_ORDER");
  if (p && p[0] == 'n') return 1;
  if (p && p[0] == 'm') return 0;
  (void)M;
  (void)E;
  return 0;
}

template <bool GATED, int BN, int BK, int NS, bool MAPPED>
static moe_status_t launch_fb_k(const uint16_t* A, const int* cu, int M, int E, int Kd, int N,
                                const uint16_t* B0, const uint16_t* B1, uint16_t* C,
                                const RowMaps& maps, hipStream_t s) {
  using CF = FbCfg<GATED, BN, BK, NS>;
  static std::atomic<unsigned char> lds_set[MOE_MAX_DEVICES];
  if (ensure_lds_limit(reinterpret_cast<const void*>(&ffn_bf16_kernel<GATED, BN, BK, NS, MAPPED>),
                       CF::LDS_BYTES, lds_set) != MOE_OK)
    return MOE_EHIP;
  const int grid = device_cu_count();
  ffn_bf16_kernel<GATED, BN, BK, NS, MAPPED><<<grid, FB_THREADS, CF::LDS_BYTES, s>>>(
      A, cu, M, E, Kd, N, B0, B1, C, tile_order_n_fastest(M, E), maps);
  return launch_status();
}

template <bool GATED, int BN, int BK, int NS>
static moe_status_t launch_fb(const uint16_t* A, const int* cu, int M, int E, int Kd, int N,
                              const uint16_t* B0, const uint16_t* B1, uint16_t* C,
                              const RowMaps& maps, hipStream_t s) {
  const bool mapped = GATED ? maps.a_src != nullptr : maps.s_acc != nullptr;
  if (mapped) return launch_fb_k<GATED, BN, BK, NS, true>(A, cu, M, E, Kd, N, B0, B1, C, maps, s);
  return launch_fb_k<GATED, BN, BK, NS, false>(A, cu, M, E, Kd, N, B0, B1, C, maps, s);
}

// K-step / LDS-stage pipeline variant. Default: the ping-pong schedule with K step 32 and
// four stages (fastest on every measured shape). MOE_FFN_PIPE = "64x2" or "32x4" selects the
// plain schedule with that K step and stage count, "pp" the ping-pong one with K step 64 and
// two stages.
static int pipe_variant() {
  static int v = -1;
  if (v < 0) {
    const char* p = std::getenv("MOE_FFN_PIPE");
    v = !p ? 3 : !std::strcmp(p, "64x2") ? 0 : !std::strcmp(p, "32x4") ? 1 : !std::strcmp(p, "pp") ? 2 : 3;
  }
  return v;
}

// Cross-tile prefetch in the ping-pong kernel: on wherever the K loop is long enough and a
// whole number of stage rounds (MOE_FFN_PF = "0" turns it off).
static bool prefetch_enabled() {
  static int v = -1;
  if (v < 0) {
    const char* p = std::getenv("MOE_FFN_PF");
    v = !(p && p[0] == '0');
  }
  return v != 0;
}

template <bool GATED, int BN, int BK, int NS, bool MAPPED, bool PF, bool NTB = false>
static moe_status_t launch_pp_k(const uint16_t* A, const int* cu, int M, int E, int Kd, int N,
                                const uint16_t* B0, const uint16_t* B1, uint16_t* C,
                                const RowMaps& maps, hipStream_t s) {
  using CF = FbCfg<GATED, BN, BK, NS>;
  // PF adds the cu_seqlens copy and the row sources of the next tile
  constexpr int LDS = CF::LDS_BYTES + (PF ? (FB_MAX_E + 1 + FB_BM) * 4 : 0);
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static std::atomic<unsigned char> lds_set[MOE_MAX_DEVICES];
  if (ensure_lds_limit(reinterpret_cast<const void*>(&ffn_bf16_pp_kernel<GATED, BN, BK, NS, MAPPED, PF, NTB>),
                       LDS, lds_set) != MOE_OK)
    return MOE_EHIP;
  ffn_bf16_pp_kernel<GATED, BN, BK, NS, MAPPED, PF, NTB><<<device_cu_count(), FB_THREADS, LDS, s>>>(
      A, cu, M, E, Kd, N, B0, B1, C, tile_order_n_fastest(M, E), maps);
  return launch_status();
}

template <bool GATED, int BN>
static moe_status_t launch_fb_any(const uint16_t* A, const int* cu, int M, int E, int Kd, int N,
                                  const uint16_t* B0, const uint16_t* B1, uint16_t* C,
                                  const RowMaps& maps, hipStream_t s) {
  if (pipe_variant() == 1) return launch_fb<GATED, BN, 32, 4>(A, cu, M, E, Kd, N, B0, B1, C, maps, s);
  if (pipe_variant() >= 2) {
    const bool mapped = GATED ? maps.a_src != nullptr : maps.s_acc != nullptr;
    if (pipe_variant() == 3) {
      // (not with the scatter epilogue, whose registers leave no room for the next tile)
      const int nk = Kd / 32;
      if (prefetch_enabled() && nk % 4 == 0 && nk >= 8) {
        if constexpr (GATED) {
          // Gate/up weight panels are read non-temporally when the average group fits one
          // m-tile (M <= 256 E): then most panels have a single reader. With several m-tiles
          // per expert they share the panel through L2, and non-temporal loads were slower
          // (T=4096 E=64: 0.213 -> 0.226 ms; 65536 rows over 52 experts: 3.11 -> 3.16 ms).
          const bool ntb = (int64_t)M <= (int64_t)FB_BM * E;
          if (mapped && ntb) return launch_pp_k<GATED, BN, 32, 4, true, true, true>(A, cu, M, E, Kd, N, B0, B1, C, maps, s);
          if (mapped) return launch_pp_k<GATED, BN, 32, 4, true, true>(A, cu, M, E, Kd, N, B0, B1, C, maps, s);
          if (ntb) return launch_pp_k<GATED, BN, 32, 4, false, true, true>(A, cu, M, E, Kd, N, B0, B1, C, maps, s);
        }
        if (!mapped) return launch_pp_k<GATED, BN, 32, 4, false, true>(A, cu, M, E, Kd, N, B0, B1, C, maps, s);
      }
      if (mapped) return launch_pp_k<GATED, BN, 32, 4, true, false>(A, cu, M, E, Kd, N, B0, B1, C, maps, s);
      return launch_pp_k<GATED, BN, 32, 4, false, false>(A, cu, M, E, Kd, N, B0, B1, C, maps, s);
    }
    if (mapped) return launch_pp_k<GATED, BN, 64, 2, true, false>(A, cu, M, E, Kd, N, B0, B1, C, maps, s);
    return launch_pp_k<GATED, BN, 64, 2, false, false>(A, cu, M, E, Kd, N, B0, B1, C, maps, s);
  }
  return launch_fb<GATED, BN, 64, 2>(A, cu, M, E, Kd, N, B0, B1, C, maps, s);
}

moe_status_t launch_ffn_gate_up_bf16(const void* a, const int* cu, int M, int E, int H, int Hp,
                                     const void* wg, const void* wu, void* h, const RowMaps& maps,
                                     hipStream_t s) {
  if (M == 0) return MOE_OK;
  return launch_fb_any<true, 128>(static_cast<const uint16_t*>(a), cu, M, E, H, Hp,
                                  static_cast<const uint16_t*>(wg), static_cast<const uint16_t*>(wu),
                                  static_cast<uint16_t*>(h), maps, s);
}

moe_status_t launch_ffn_down_bf16(const void* h, const int* cu, int M, int E, int H, int Hp,
                                  const void* wd, void* y, const RowMaps& maps, hipStream_t s) {
  if (M == 0) return MOE_OK;
  return launch_fb_any<false, 256>(static_cast<const uint16_t*>(h), cu, M, E, Hp, H,
                                   static_cast<const uint16_t*>(wd), nullptr,
                                   static_cast<uint16_t*>(y), maps, s);
}

}  // namespace moe
