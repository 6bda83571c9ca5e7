// Grouped expert FFN in one persistent launch (bf16): the gate/up + SwiGLU tiles and the down
// tiles of every expert come from device-side work queues, and a down tile starts as soon as
// the h rows it reads have been written, without a second launch and its tail.
//
// "Mixture of Kittens", Step 7 (the megakernel: one persistent launch whose blocks coordinate
// through counters in global memory) and Step 3 (work of the next chunk overlaps the current
// one); the DeepGEMM Mega-MoE how-to (dispatch, both expert GEMMs and SwiGLU in one kernel).
// Gate/up rows are gathered from the token matrix through row_src ("no permute in"); the
// down tiles write y_rows for the deterministic combine, or, in the scattering instantiation,
// add their weighted rows into the token accumulator with atomics (the combine in the down
// epilogue).
//
// Work list. Expert e with rows_e rows has mte = ceil(rows_e / 256) m-tiles (the row split of
// even_chunk, as in the two-launch kernels), giving mte * Hp/128 gate/up tiles (G) and
// mte * H/256 down tiles (D). The experts are cut into 8 contiguous ranges of about equal
// m-tile count, one queue per XCD; block b takes tiles from queue b % 8 first (blocks are
// dispatched round-robin over the XCDs, so the tiles of one expert share that XCD's L2) and
// then from the other queues. Queue order within a range a..b-1 with lag L (experts):
//   G(a) .. G(a+L-1), then G(j), D(j-L) for j = a+L .. b-1, then the remaining D blocks,
// m-tile fastest inside a block. Every down tile thus follows all gate/up tiles it reads
// in its own queue, L experts later. The launch uses L = E: each queue runs all its gate/up
// tiles, then all its down tiles. Interleaving them (L of about 3 experts at T=8192 E=384
// K=8 H=7168 H'=2048) was 6 % slower: the down tiles' weight panels then stream through the
// L2 that the gate/up tiles of the same XCD share their activation rows in. The XCDs still
// move from gate/up to down independently, and a block that finds its queue empty takes
// tiles from the others, so there is no global tail between the two projections.
//
// Readiness. Down tile (e, mt) reads the h rows of m-tile mt, written by the Hp/128 gate/up
// tiles of (e, mt). Those store h with agent-scope (sc1) stores, which write through to
// memory, wait for them, and each of their 8 waves adds 1 to ready[e, mt]. A block takes a
// down tile only once its counter reads 8 * Hp/128. No block reads an h row before that point,
// so its L2 holds no stale copy of it and plain loads fetch the written values.
//
// Progress. A block never waits inside a tile. Its next tile is dequeued while the current
// one runs. If that next tile is a down tile whose rows are not ready at the point where its
// first stages would be prefetched, the block finishes and signals the current tile first, then
// waits, then starts the next tile without prefetch. Every down tile depends only on gate/up
// tiles dequeued before it from the same queue. So the unfinished tile that was dequeued
// earliest can always run, and the launch completes. Each wait is bounded: past the bound the
// block sets the error word and goes on.
//
// The K loop, LDS layouts and wave layout are those of the ping-pong kernel (ffn_bf16.hip):
// K step 32, four 32 KiB stages, MFMA 32x32x16 bf16, 8 waves in two groups offset by one slot,
// group 0 issuing the direct global->LDS loads, cross-tile prefetch of the next tile's first
// stages. Both tile kinds stage A as [256][32] bf16 and 16 KiB of weights per stage: gate/up as
// Wg and Wu panels of 128 columns, down as one 256-column panel of Wd.
#include "lds_dma.h"
#include "moe_common.h"
#include "tile_sched.h"

#include <algorithm>
#include <cstdlib>
#include <type_traits>

namespace moe {

namespace {

constexpr int F_BM = 256, F_BK = 32, F_NS = 4, F_THREADS = 512, F_MAX_E = 1024, F_NQ = 8;
constexpr int F_A_ROW = F_BK * 2;              // bytes of one staged A row
constexpr int F_A_BYTES = F_BM * F_A_ROW;      // 16 KiB
constexpr int F_CPR = F_BK / 8;                // 16-byte chunks per staged A row
constexpr int F_A_RPL = 1024 / F_A_ROW;        // A rows per 1 KiB load
constexpr int F_A_SWZ_DIV = 16 / F_CPR;
constexpr int F_STAGE = 2 * F_A_BYTES;         // A + 16 KiB of weights
constexpr int F_LDP = 4;                       // A (and weight) loads per group-0 wave per stage
constexpr int F_VMG = 2 * F_LDP;
constexpr int F_KK = F_BK / 16;                // MFMA k-steps per stage
constexpr int F_PMT = 4;                       // row blocks per wave (at most)
constexpr int F_SPIN_MAX = 1 << 20;            // default bound of one readiness wait (polls, about 1 s)

// control words (int32) at the start of the caller's control area; ready[] follows
enum { C_QCTR = 0, C_ERR = F_NQ, C_TILES, C_COLD, C_STEAL, C_HDR = 16 };

// LDS after the stages: schedule arrays, the row sources of the next gathered tile, misc
// (schedule experts: up to F_MAX_E routed ones, or F_MAX_E - 1 and the folded shared expert)
constexpr int L_CU = 0;                                  // cu_seqlens [E+1]
constexpr int L_MPRE = L_CU + F_MAX_E + 1;               // m-tile prefix [EE+1]
constexpr int L_SG = L_MPRE + F_MAX_E + 1;               // start of G(e) in the queues [EE]
constexpr int L_SD = L_SG + F_MAX_E;                     // start of D(e) [EE]
constexpr int L_SRC = L_SD + F_MAX_E;                    // next tile's row sources [256]
constexpr int L_RS = L_SRC + F_BM;                       // range starts [9]
constexpr int L_QB = L_RS + 12;                          // queue bases [9]
constexpr int L_TQ = L_QB + 12;                          // published next tile [4]
constexpr int L_WSUM = L_TQ + 4;                         // scan scratch [8]
constexpr int L_SF = L_WSUM + 8;                         // shared-expert pointers [6 x 2]
constexpr int L_INTS = L_SF + 12;
constexpr int F_LDS = F_NS * F_STAGE + L_INTS * 4;
static_assert(F_LDS <= 160 * 1024, "LDS budget");

__device__ __forceinline__ void f_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Largest e in [0, n) with arr[e] <= x, or -1 (arr nondecreasing). Whole wave, uniform
// result; two LDS reads per lane for n <= 4096.
__device__ __forceinline__ int wave_find_le(const int* arr, int n, int x) {
  const int lane = threadIdx.x & 63;
  int lo = 0;
  while (n > 64) {
    const int step = (n + 63) / 64;
    const bool ok = lane * step < n && arr[lo + lane * step] <= x;
    const int c = __popcll(__ballot(ok));
    if (c == 0) return -1;
    lo += (c - 1) * step;
    n = min(step, n - (c - 1) * step);
  }
  const bool ok = lane < n && arr[lo + lane] <= x;
  const int c = __popcll(__ballot(ok));
  return c == 0 ? -1 : lo + c - 1;
}

}  // namespace

__global__ void fused_ctl_reset_kernel(int* ctl, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) ctl[i] = 0;
}

// x [T, H] bf16 (gathered through row_src / K); w_gate, w_up [E, H, Hp]; w_down [E, Hp, H];
// h [M, Hp] and y [M, H] bf16; ctl: control words + ready counters (zeroed before the launch).
// SHARED: the shared expert is folded in as expert E (sf); otherwise sf is unused.
// SCATTER: the down tiles add row_w[r] * y[r] into s_acc [T, H] (fp32) at token row_src[r] / K
// with atomics instead of storing y (the weighted combine in the down epilogue); y is unused.
template <bool SHARED, bool SCATTER>
__global__ __launch_bounds__(F_THREADS, 1) void ffn_bf16_fused_kernel(
    const uint16_t* __restrict__ x, const int* __restrict__ row_src, int T, int K,
    const int* __restrict__ cu, int E, int H, int Hp, const uint16_t* __restrict__ wg,
    const uint16_t* __restrict__ wu, const uint16_t* __restrict__ wd, uint16_t* __restrict__ h,
    uint16_t* __restrict__ y, int* __restrict__ ctl, int lag, int spin_max, SharedFold sf,
    const float* __restrict__ row_w, float* __restrict__ s_acc) {
  static_assert(!(SHARED && SCATTER), "the shared expert is folded in with the gather combine only");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int* li = reinterpret_cast<int*>(smem + F_NS * F_STAGE);
  int* cu_l = li + L_CU;
  int* mpre = li + L_MPRE;
  int* sG = li + L_SG;
  int* sD = li + L_SD;
  int* rs = li + L_RS;
  int* qb = li + L_QB;
  int* tq = li + L_TQ;
  int* wsum = li + L_WSUM;
  int* sfp = li + L_SF;
  int* ready = ctl + C_HDR;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sc = wave & 3;            // column strip
  const int hf = wave >> 2;           // 0: even row blocks, 1: odd ones
  const bool g0 = wave < 4;
  const int gw = wave & 3;
  const int ntg = Hp / 128, ntd = H / 256;           // n-tiles of a gate/up / down m-tile
  const int tgt = 8 * ntg;                           // ready count of a finished m-tile
  // schedule experts: the E routed ones, then the shared expert (index E) when folded in
  const int EE = E + (SHARED ? 1 : 0);
  auto rows_of = [&](int e) { return e < E ? cu[e + 1] - cu[e] : sf.T; };

  // ---- schedule in LDS: m-tile prefix, ranges, queue bases, block starts ----
  for (int i = tid; i <= E; i += F_THREADS) cu_l[i] = cu[i];
  // The shared expert's pointers wait in LDS and are read where a tile is decoded or stored,
  // so that they do not hold scalar registers through the K loops.
  if (SHARED && tid < 6) {
    const void* pv[6] = {sf.x, sf.wg, sf.wu, sf.wd, sf.h, sf.y};
    const uint64_t a = reinterpret_cast<uint64_t>(pv[tid]);
    sfp[2 * tid] = (int)(uint32_t)a;
    sfp[2 * tid + 1] = (int)(uint32_t)(a >> 32);
  }
  {
    const int e0 = 2 * tid, e1 = 2 * tid + 1;
    int c0 = 0, c1 = 0;
    if (e0 < EE) c0 = (rows_of(e0) + F_BM - 1) / F_BM;
    if (e1 < EE) c1 = (rows_of(e1) + F_BM - 1) / F_BM;
    const int s = c0 + c1;
    const int incl = sched_wave_incl_scan(s);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int base = 0, tot = 0;
    for (int w = 0; w < F_THREADS / 64; ++w) {
      if (w < wave) base += wsum[w];
      tot += wsum[w];
    }
    const int ex = base + incl - s;
    if (e0 < EE) mpre[e0] = ex;
    if (e1 < EE) mpre[e1] = ex + c0;
    if (tid == 0) mpre[EE] = tot;
  }
  __syncthreads();
  const int mtot = mpre[EE];
  if (mtot == 0) return;
  // expert e belongs to range v(e) = floor(8 * midpoint of its m-tiles / mtot), nondecreasing
  auto range_of = [&](int e) { return min(F_NQ - 1, (4 * (mpre[e] + mpre[e + 1])) / mtot); };
  for (int e = tid; e < EE; e += F_THREADS) {
    const int ve = range_of(e), vp = e > 0 ? range_of(e - 1) : -1;
    for (int v = vp + 1; v <= ve; ++v) rs[v] = e;
    if (e == EE - 1)
      for (int v = ve + 1; v <= F_NQ; ++v) rs[v] = EE;
  }
  __syncthreads();
  for (int v = tid; v <= F_NQ; v += F_THREADS) qb[v] = mpre[rs[v]] * (ntg + ntd);
  for (int e = tid; e < EE; e += F_THREADS) {
    const int v = range_of(e), a = rs[v], n = rs[v + 1] - a;
    sG[e] = mpre[e] * ntg + mpre[a + max(0, e - a - lag)] * ntd;
    sD[e] = mpre[a + min(n, e - a + lag + 1)] * ntg + mpre[e] * ntd;
  }
  __syncthreads();

  // ---- per-wave offsets (recomputed where used: cheap ALU, fewer live registers) ----
  // A load i of group-0 wave gw fills staged rows [16 j, 16 j + 16), j = gw + 4 i; lane l
  // brings 16-byte chunk l % 4 of row 16 j + l / 4, XOR-swizzled by (row / 4) % 4
  auto a_row = [&](int i) __attribute__((always_inline)) { return (gw + 4 * i) * F_A_RPL + lane / F_CPR; };
  auto a_voff = [&](int i, int rowlen) __attribute__((always_inline)) {
    const int r = a_row(i);
    return r * rowlen * 2 + (((lane % F_CPR) ^ ((r / F_A_SWZ_DIV) % F_CPR)) << 4);
  };
  const int a_fbase = (hf * 32 + (lane & 31)) * F_A_ROW;
  const int a_sw = ((lane & 31) / F_A_SWZ_DIV) % F_CPR;
  int a_fk[F_KK];
#pragma unroll
  for (int kk = 0; kk < F_KK; ++kk) a_fk[kk] = a_fbase + ((((kk << 1) | (lane >> 5)) ^ a_sw) << 4);
  const uint32_t smem_lds = lds_addr(smem);
  constexpr int SRC_OFF = F_NS * F_STAGE + L_SRC * 4;

  struct Tile {
    int kind;        // 0 gate/up, 1 down
    int e, mt, row0, rows_valid, n0, nmt, nk;
    bool stream_b;   // gate/up of a single-m-tile expert: its panels' only reader
    bool gathered;   // gate/up rows gathered from x through row_src (routed experts)
    i32x4_t rA, rB0, rB1;
    int a_off[F_LDP];
  };
  // shared-expert pointer i (0 x, 1 wg, 2 wu, 3 wd, 4 h, 5 y) from LDS
  auto sfptr = [&](int i) __attribute__((always_inline)) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane(sfp[2 * i]);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane(sfp[2 * i + 1]);
    return reinterpret_cast<uint16_t*>(((uint64_t)hi << 32) | lo);
  };
  // tile `id` of kind `kind` of expert e (everything but a gathered tile's A offsets)
  auto decode = [&](int id, int kind, int e) __attribute__((always_inline)) {
    Tile d;
    d.kind = kind;
    d.e = e;
    const bool shared = SHARED && e >= E;   // the shared expert: rows 0..T-1 of its own h and y
    const int gbeg = shared ? 0 : cu_l[e], rows_e = shared ? sf.T : cu_l[e + 1] - gbeg;
    const int mte = mpre[e + 1] - mpre[e];
    const int lt = id - (kind == 0 ? sG[e] : sD[e]);
    const int ntile = lt / mte, mtile = lt - ntile * mte;
    const int chunk = even_chunk(rows_e, mte);
    d.mt = mtile;
    d.row0 = gbeg + mtile * chunk;
    d.rows_valid = min(chunk, rows_e - mtile * chunk);
    d.stream_b = kind == 0 && mte == 1;
    d.gathered = kind == 0 && !shared;
    if (kind == 0) {
      d.n0 = ntile * 128;
      d.nk = H / F_BK;
      const size_t woff = (shared ? 0 : (size_t)e * H * Hp) + d.n0;
      const uint32_t rem = (uint32_t)(((size_t)H * Hp - d.n0) * 2);
      d.rB0 = make_rsrc((shared ? sfptr(1) : wg) + woff, rem);
      d.rB1 = make_rsrc((shared ? sfptr(2) : wu) + woff, rem);
      if (shared) {
        // the shared expert reads the token rows in order: x row t is its row t
        d.rA = make_rsrc(sfptr(0) + (size_t)d.row0 * H, (uint32_t)d.rows_valid * (uint32_t)H * 2u);
#pragma unroll
        for (int i = 0; i < F_LDP; ++i) d.a_off[i] = a_voff(i, H);
      } else {
        d.rA = make_rsrc(x, (uint32_t)T * (uint32_t)H * 2u);
      }
    } else {
      d.n0 = ntile * 256;
      d.nk = Hp / F_BK;
      d.rA = make_rsrc((shared ? sfptr(4) : h) + (size_t)d.row0 * Hp, (uint32_t)d.rows_valid * (uint32_t)Hp * 2u);
#pragma unroll
      for (int i = 0; i < F_LDP; ++i) d.a_off[i] = a_voff(i, Hp);
      const size_t woff = (shared ? 0 : (size_t)e * Hp * H) + d.n0;
      d.rB0 = make_rsrc((shared ? sfptr(3) : wd) + woff, (uint32_t)(((size_t)Hp * H - d.n0) * 2));
      d.rB1 = d.rB0;
    }
    d.nmt = __builtin_amdgcn_readfirstlane(min(F_PMT, ((d.rows_valid + 31) / 32 - hf + 1) / 2));
    return d;
  };
  // A offsets of a gathered (gate/up) tile from the sources of this wave's A rows; rows past
  // the tile read a clamped source and are then pointed out of range; -1 marks padding
  auto gather_offsets = [&](Tile& d, const int (&src)[F_LDP]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < F_LDP; ++i) {
      const int off = (src[i] / K - a_row(i)) * H * 2 + a_voff(i, H);
      d.a_off[i] = (a_row(i) < d.rows_valid && src[i] >= 0) ? off : (int)0x80000000u;
    }
  };
  auto gather_from_global = [&](Tile& d) __attribute__((always_inline)) {
    int src[F_LDP];
#pragma unroll
    for (int i = 0; i < F_LDP; ++i) src[i] = row_src[d.row0 + min(a_row(i), d.rows_valid - 1)];
    gather_offsets(d, src);
  };
  // group 0: this wave's share of stage kt of tile d, of kind KIND. Weight rows are staged as
  // in the global layout with their 32-byte segments XOR-swizzled by 2 (row % 4): a gate/up
  // load fills 4 rows of 128 columns (16 lanes per row), a down load 2 rows of 256 columns
  // (32 lanes per row).
  const int bv_g = [&] {
    const int r = gw * 4 + lane / 16, q = lane % 16;
    return r * Hp * 2 + ((((q >> 1) ^ ((r & 3) << 1)) << 1) + (q & 1)) * 16;
  }();
  const int bv_d = [&] {
    const int r = gw * 2 + lane / 32, q = lane % 32;
    return r * H * 2 + ((((q >> 1) ^ ((r & 3) << 1)) << 1) + (q & 1)) * 16;
  }();
  auto issue_k = [&](auto kindc, const Tile& d, int kt) __attribute__((always_inline)) {
    constexpr int KIND = decltype(kindc)::value;
    const uint32_t so = smem_lds + (uint32_t)((kt % F_NS) * F_STAGE);
#pragma unroll
    for (int i = 0; i < F_LDP; ++i) lds_dma16(d.rA, so + (gw + 4 * i) * 1024, d.a_off[i], kt * F_BK * 2);
    if constexpr (KIND == 0) {
      // loads i = 0, 1: Wg rows [0,16) and [16,32) of the stage; i = 2, 3: the same of Wu
      const int kso = kt * F_BK * Hp * 2;
#pragma unroll
      for (int i = 0; i < F_LDP; ++i) {
        const int soff = kso + (i & 1) * 16 * Hp * 2;
        const uint32_t dst = so + F_A_BYTES + (gw + 4 * i) * 1024;
        if (d.stream_b) lds_dma16_nt(i < 2 ? d.rB0 : d.rB1, dst, bv_g, soff);
        else lds_dma16(i < 2 ? d.rB0 : d.rB1, dst, bv_g, soff);
      }
    } else {
      const int kso = kt * F_BK * H * 2;
#pragma unroll
      for (int i = 0; i < F_LDP; ++i)
        lds_dma16(d.rB0, so + F_A_BYTES + (gw + 4 * i) * 1024, bv_d, kso + 8 * i * H * 2);
    }
  };
  auto issue = [&](const Tile& d, int kt) __attribute__((always_inline)) {
    if (d.kind == 0) issue_k(std::integral_constant<int, 0>{}, d, kt);
    else issue_k(std::integral_constant<int, 1>{}, d, kt);
  };

  // ---- queue access (wave 4 only; values uniform over the wave) ----
  int qv = blockIdx.x % F_NQ;
  unsigned qmask = 0;
  auto qlen = [&](int q) { return qb[q + 1] - qb[q]; };
  auto deq_sync = [&]() -> int {
    for (int k = 0; k < F_NQ; ++k) {
      const int q = (qv + k) % F_NQ;
      if (qmask & (1u << q)) continue;
      int r = 0;
      if (lane == 0) r = __hip_atomic_fetch_add(ctl + C_QCTR + q, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      r = __builtin_amdgcn_readfirstlane(r);
      if (r < qlen(q)) {
        if (k != 0 && lane == 0) __hip_atomic_fetch_add(ctl + C_STEAL, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        qv = q;
        return qb[q] + r;
      }
      qmask |= 1u << q;
    }
    return -1;
  };
  // kind (0 G, 1 D, -1 none), expert and ready-counter index of tile id
  auto classify = [&](int id, int& kind, int& e, int& rix) {
    kind = -1;
    e = 0;
    rix = 0;
    if (id < 0) return;
    const int eg = wave_find_le(sG, EE, id);
    if (eg >= 0 && id < sG[eg] + (mpre[eg + 1] - mpre[eg]) * ntg) {
      kind = 0;
      e = eg;
      return;
    }
    const int ed = wave_find_le(sD, EE, id);
    const int mte = ed >= 0 ? mpre[ed + 1] - mpre[ed] : 0;
    if (mte == 0 || id >= sD[ed] + mte * ntd) {   // not a tile of the schedule (never expected)
      if (lane == 0) __hip_atomic_store(ctl + C_ERR, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    kind = 1;
    e = ed;
    rix = mpre[ed] + (id - sD[ed]) % mte;
  };
  auto ready_now = [&](int rix) -> bool {
    const int v = __hip_atomic_load(ready + rix, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __builtin_amdgcn_readfirstlane(v) >= tgt;
  };
  // Bounded: past spin_max polls, or as soon as any block has set the error word, give up
  // (the results are then invalid and the error word says so).
  auto wait_ready = [&](int rix) {
    for (int n = 0;; ++n) {
      if (ready_now(rix)) return;
      if ((n & 255) == 255 &&
          __builtin_amdgcn_readfirstlane(__hip_atomic_load(ctl + C_ERR, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)))
        return;
      if (n >= spin_max) {
        if (lane == 0) __hip_atomic_store(ctl + C_ERR, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  };
  auto publish = [&](int id, int kind, int e, int pf) {
    if (lane == 0) {
      tq[0] = id;
      tq[1] = kind;
      tq[2] = e;
      tq[3] = pf;
    }
  };

  // wave 4: the lookahead tile (the one after the next), the early dequeue and readiness poll
  // issued inside the K loop, and whether a dequeue result waits to be resolved
  int la_id = -1, la_kind = -1, la_e = 0, la_rix = 0, pend = 0, poll = 0;
  bool pend_out = false;
  // between tiles (no accumulators live): turn the early dequeue into the next lookahead
  auto resolve_pend = [&]() {
    if (!pend_out) return;
    pend_out = false;
    const int p = __builtin_amdgcn_readfirstlane(pend);
    int id2;
    if (p < qlen(qv)) {
      id2 = qb[qv] + p;
    } else {
      qmask |= 1u << qv;
      id2 = deq_sync();
    }
    classify(id2, la_kind, la_e, la_rix);
    la_id = id2;
  };

  // ---- first tile ----
  if (wave == 4) {
    int id0 = deq_sync(), k0, e0, r0;
    classify(id0, k0, e0, r0);
    if (k0 == 1) wait_ready(r0);
    la_id = k0 >= 0 ? deq_sync() : -1;
    classify(la_id, la_kind, la_e, la_rix);
    publish(id0, k0, e0, 1);
  }
  __syncthreads();
  Tile cur;
  {
    const int id0 = __builtin_amdgcn_readfirstlane(tq[0]);
    const int k0 = __builtin_amdgcn_readfirstlane(tq[1]);
    const int e0 = __builtin_amdgcn_readfirstlane(tq[2]);
    if (k0 < 0) return;
    cur = decode(id0, k0, e0);
    if (cur.gathered) gather_from_global(cur);
    if (g0)
      for (int st = 0; st < F_NS; ++st) issue(cur, st);
  }

  for (;;) {
    const int nk = cur.nk;
    const int kd = nk - 2 * F_NS + 1;            // K step at which the next tile is taken
    const int kq = max(0, kd - 4);               // wave 4: early dequeue and readiness poll
    bool has_next = false, pf = false, xa = false;
    int nx_id = -1, nx_kind = -1, nx_e = 0;
    Tile nxt;

    f32x16_t acc[2][F_PMT];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int mt = 0; mt < F_PMT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[f][mt][i] = 0.f;

    // wave 4, before the first barrier of K step kt: take the tile after the next one from the
    // queue and poll the readiness of the next one early, publish the next one at kd - 1
    auto queue_work = [&](int kt) __attribute__((always_inline)) {
      if (wave != 4 || la_kind < 0) {
        if (wave == 4 && kt == kd - 1) publish(-1, -1, 0, 0);
        return;
      }
      if (kt == kq) {
        if (lane == 0) pend = __hip_atomic_fetch_add(ctl + C_QCTR + qv, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (la_kind == 1) poll = __hip_atomic_load(ready + la_rix, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (kt == kd - 1) {
        const bool rdy = la_kind == 0 || __builtin_amdgcn_readfirstlane(poll) >= tgt;
        publish(la_id, la_kind, la_e, rdy ? 1 : 0);
        pend_out = true;
        la_kind = -1;
      }
    };

    auto run = [&](auto kindc, auto mtv) __attribute__((always_inline)) {
      constexpr int KIND = decltype(kindc)::value;
      constexpr int MTV = decltype(mtv)::value;
      constexpr int BROW = KIND == 0 ? 256 : 512;     // bytes of one staged weight row
      // weight fragment of this lane: column strip sc (32 or 64 columns per matrix), 16-byte
      // transpose reads of rows 8 (g / 2) + jj / 4, segment swizzle as staged
      const int g = lane >> 4, jj = lane & 15;
      const int bP = (KIND == 0 ? 2 : 4) * sc + (g & 1);
      const int b_fbase = (8 * (g >> 1) + (jj >> 2)) * BROW + 8 * (jj & 3) + ((bP ^ ((jj >> 2) << 1)) << 5);
      bf16x8_t fa[MTV > 0 ? MTV : 1][2];
      bf16x8_t fb[2][2];
      auto mread = [&](int kt, auto hfc) __attribute__((always_inline)) {
        constexpr int HF = decltype(hfc)::value;
        if constexpr (MTV > 0) {
          const unsigned char* sa = smem + (kt % F_NS) * F_STAGE;
          const unsigned char* sb = sa + F_A_BYTES;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int kk = HF * 2 + q;
#pragma unroll
            for (int mt = 0; mt < MTV; ++mt)
              fa[mt][q] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const i32x4_t*>(sa + a_fk[kk] + mt * 64 * F_A_ROW));
#pragma unroll
            for (int f = 0; f < 2; ++f) {
              const unsigned char* p = KIND == 0 ? sb + f * 8192 + b_fbase + kk * 16 * BROW
                                                 : sb + (b_fbase ^ (f << 6)) + kk * 16 * BROW;
              const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4_t*)(p));
              const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4_t*)(p + 4 * BROW));
              fb[f][q] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
          }
        }
      };
      // weights as the first operand: each lane holds one output row (row-lane layout); the
      // scattering down tiles take the other order, each lane then holding one column
      auto compute = [&]() __attribute__((always_inline)) {
        if constexpr (MTV > 0) {
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
              for (int mt = 0; mt < MTV; ++mt) {
                if constexpr (SCATTER && KIND == 1)
                  acc[f][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mt][q], fb[f][q], acc[f][mt], 0, 0, 0);
                else
                  acc[f][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[f][q], fa[mt][q], acc[f][mt], 0, 0, 0);
              }
        }
      };
      constexpr std::integral_constant<int, 0> H0{};
      // stage 0 has landed once at most the younger stages are outstanding
      if (g0) wait_vm_dyn<F_VMG * (F_NS - 1)>(min(F_NS - 1, nk - 1) * F_VMG);
      f_barrier();
      if (!g0) f_barrier();        // group 1: one slot behind
      auto step = [&](int kt, auto tailc) __attribute__((always_inline)) {
        constexpr bool TAIL = decltype(tailc)::value;
        mread(kt, H0);
        if constexpr (TAIL) {
          if (g0 && xa && kt == kd + F_NS) {
            // the next tile's row sources landed before the last barrier of step kd + NS - 1
            int src[F_LDP];
            const int* sl = reinterpret_cast<const int*>(smem + SRC_OFF);
#pragma unroll
            for (int i = 0; i < F_LDP; ++i) src[i] = sl[min(a_row(i), nxt.rows_valid - 1)];
            gather_offsets(nxt, src);
          }
          if (g0) {
            if (kt + F_NS - 1 < nk) issue_k(kindc, cur, kt + F_NS - 1);
            else if (pf) issue(nxt, kt + F_NS - 1 - nk);
          }
          if (kt == kd) {
            nx_id = __builtin_amdgcn_readfirstlane(tq[0]);
            nx_kind = __builtin_amdgcn_readfirstlane(tq[1]);
            nx_e = __builtin_amdgcn_readfirstlane(tq[2]);
            has_next = nx_kind >= 0;
            pf = has_next && __builtin_amdgcn_readfirstlane(tq[3]) != 0;
            if (pf) {
              nxt = decode(nx_id, nx_kind, nx_e);
              xa = nxt.gathered;
              // group-0 wave gw loads row sources [64 gw, 64 gw + 64) of the next gathered
              // tile after stage kd + NS - 1; entries past its rows read as zeros
              if (xa && g0)
                lds_dma4(make_rsrc(row_src + nxt.row0, (uint32_t)nxt.rows_valid * 4u),
                         smem_lds + (uint32_t)(SRC_OFF + 256 * gw), (64 * gw + lane) * 4, 0);
            }
          }
        } else {
          if (g0 && kt >= 1) issue_k(kindc, cur, kt + F_NS - 1);
          if (kt == kq || kt == kd - 1) queue_work(kt);
        }
        f_barrier();
        compute();
        if constexpr (TAIL) {
          if (g0 && kt + 1 < nk) {
            if (pf) wait_vm_dyn<F_VMG * (F_NS - 2) + 1>((F_NS - 2) * F_VMG + (xa && kt <= kd + F_NS - 2));
            else wait_vm_dyn<F_VMG * (F_NS - 2)>(min(F_NS - 2, nk - 2 - kt) * F_VMG);
          }
        } else {
          if (g0 && kt + 1 < nk) wait_vm_dyn<F_VMG * (F_NS - 2)>(F_VMG * (F_NS - 2));
        }
        f_barrier();
      };
      for (int kt = 0; kt < kd; ++kt) step(kt, std::false_type{});
      for (int kt = kd; kt < nk; ++kt) step(kt, std::true_type{});
      if (g0) f_barrier();         // same number of barriers in both groups
    };
    auto run_kind = [&](auto kindc) __attribute__((always_inline)) {
      const int nmt = cur.nmt;
      if (nmt == 4) run(kindc, std::integral_constant<int, 4>{});
      else if (nmt == 3) run(kindc, std::integral_constant<int, 3>{});
      else if (nmt == 2) run(kindc, std::integral_constant<int, 2>{});
      else if (nmt == 1) run(kindc, std::integral_constant<int, 1>{});
      else run(kindc, std::integral_constant<int, 0>{});
    };
    if (cur.kind == 0) run_kind(std::integral_constant<int, 0>{});
    else run_kind(std::integral_constant<int, 1>{});
    // Every LDS read of this tile is done, so the next tile's last prefetched stage may go out.
    // After a gate/up tile it goes out after the h stores have been waited for, so that the
    // wait does not also cover this load.
    if (pf && g0 && cur.kind == 1) issue(nxt, F_NS - 1);

    // ---- epilogue: row-lane layout, block (mt, f) holds row (2 mt + hf) * 32 + lane % 32 ----
    if (cur.kind == 0) {
      // h = silu(g) * u, stored write-through (agent scope) for the down tiles of other XCDs
      const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(
          (SHARED && cur.e >= E ? sfptr(4) : h) + (size_t)cur.row0 * Hp, (short)0, cur.rows_valid * Hp * 2,
          0x00020000);
      const int col = cur.n0 + sc * 32 + 8 * (lane >> 5);
#pragma unroll
      for (int mt = 0; mt < F_PMT; ++mt) {
        const int r = (2 * mt + hf) * 32 + (lane & 31);
        const bool ok = r < cur.rows_valid;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          float hv[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) hv[c] = silu_f32(acc[0][mt][8 * p + c]) * acc[1][mt][8 * p + c];
          const uint4 v = pack_row16(hv[0], hv[1], hv[2], hv[3], hv[4], hv[5], hv[6], hv[7]);
          typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
          const u32x4 vv = {v.x, v.y, v.z, v.w};
          if (ok) __builtin_amdgcn_raw_buffer_store_b128(vv, hr, (r * Hp + col + 16 * p) * 2, 0, 16);
        }
      }
      // this wave's h stores are complete (and visible device-wide): count them
      asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
      if (lane == 0)
        __hip_atomic_fetch_add(ready + mpre[cur.e] + cur.mt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (pf && g0) issue(nxt, F_NS - 1);
    } else if constexpr (SCATTER) {
      // column-lane layout: element i of block (mt, f) is row (2 mt + hf) * 32 + 8 (i / 4) +
      // 4 (lane / 32) + i % 4 and column f * 32 + lane % 32 of this wave's 64-column strip, so
      // the 32 lanes of a row add into 32 consecutive floats of its token's accumulator row
      const int col = cur.n0 + sc * 64 + (lane & 31);
#pragma unroll
      for (int mt = 0; mt < F_PMT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = (2 * mt + hf) * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          const int src = r < cur.rows_valid ? row_src[cur.row0 + r] : -1;   // -1: padding row
          if (src >= 0) {
            float* dst = s_acc + (size_t)(src / K) * H + col;
            const float wr = row_w[cur.row0 + r];
#pragma unroll
            for (int f = 0; f < 2; ++f) unsafeAtomicAdd(dst + f * 32, wr * acc[f][mt][i]);
          }
        }
    } else {
      const int col = cur.n0 + sc * 64 + 8 * (lane >> 5);
#pragma unroll
      for (int mt = 0; mt < F_PMT; ++mt) {
        const int r = (2 * mt + hf) * 32 + (lane & 31);
        const bool ok = r < cur.rows_valid;
        const size_t ro = (size_t)(cur.row0 + (ok ? r : 0)) * H + col;
        uint16_t* yo = SHARED && cur.e >= E ? sfptr(5) : y;
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const uint4 v = pack_row16(acc[f][mt], 8 * p);
            if (ok) *reinterpret_cast<uint4*>(yo + ro + f * 32 + 16 * p) = v;
          }
      }
    }
    if (tid == 0) __hip_atomic_fetch_add(ctl + C_TILES, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (wave == 4) resolve_pend();

    if (!has_next) break;
    if (!pf) {
      // the next tile was not ready at the prefetch point: this tile is finished and counted,
      // so the block now waits holding no unfinished tile, then starts the next one cold
      nxt = decode(nx_id, nx_kind, nx_e);
      if (wave == 4) {
        if (lane == 0) __hip_atomic_fetch_add(ctl + C_COLD, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (nxt.kind == 1) wait_ready(mpre[nxt.e] + nxt.mt);
      }
      if (nxt.gathered && g0) gather_from_global(nxt);
      f_barrier();
      cur = nxt;
      if (g0)
        for (int st = 0; st < F_NS; ++st) issue(cur, st);
      continue;
    }
    cur = nxt;
  }
}

// Control words the fused launch needs for M rows over E schedule experts (the shared
// expert, when folded in, counts as one more expert with T more rows): header + one ready
// counter per m-tile (sum over experts of ceil(rows / 256) <= M / 256 + E).
size_t fused_ctl_ints(int M, int E) { return (size_t)C_HDR + (size_t)M / F_BM + (size_t)E + 1; }

moe_status_t launch_ffn_fused_bf16(const void* x, const int* row_src, int T, int K, const int* cu, int M,
                                   int E, int H, int Hp, const void* wg, const void* wu, const void* wd,
                                   void* h, void* y, int* ctl, hipStream_t s, const SharedFold& sf,
                                   const float* row_w, float* s_acc) {
  if (M == 0 && sf.T == 0) return MOE_OK;
  if (E + (sf.T > 0 ? 1 : 0) > F_MAX_E || H % 256 || Hp % 128 || H < 256 || Hp < 256) return MOE_EUNSUPPORTED;
  if (s_acc && (sf.T > 0 || !row_w)) return MOE_EINVAL;
  static std::atomic<unsigned char> lds_set[3][MOE_MAX_DEVICES];
  if (ensure_lds_limit(reinterpret_cast<const void*>(&ffn_bf16_fused_kernel<false, false>), F_LDS, lds_set[0]) !=
          MOE_OK ||
      ensure_lds_limit(reinterpret_cast<const void*>(&ffn_bf16_fused_kernel<true, false>), F_LDS, lds_set[1]) !=
          MOE_OK ||
      ensure_lds_limit(reinterpret_cast<const void*>(&ffn_bf16_fused_kernel<false, true>), F_LDS, lds_set[2]) != MOE_OK)
    return MOE_EHIP;
  const int n = (int)fused_ctl_ints(M + sf.T, E + (sf.T > 0 ? 1 : 0));
  fused_ctl_reset_kernel<<<(n + 255) / 256, 256, 0, s>>>(ctl, n);
  // lag E + 1: every queue holds all its gate/up tiles before all its down tiles.
  // MOE_FUSED_LAG=n (n >= 1) interleaves them instead, n experts apart; then many down tiles
  // wait for their rows (the readiness path the tests exercise).
  int lag = E + 1;
  if (const char* v = std::getenv("MOE_FUSED_LAG")) {
    const int l = std::atoi(v);
    if (l >= 1) lag = std::min(l, E + 1);
  }
  // MOE_FUSED_SPIN_MAX=n (n >= 0) lowers the bound of a readiness wait, so that a test can
  // make waits give up and check that the launch still ends and reports it in the error word.
  int spin_max = F_SPIN_MAX;
  if (const char* v = std::getenv("MOE_FUSED_SPIN_MAX")) {
    if (v[0]) spin_max = std::max(0, std::min(std::atoi(v), F_SPIN_MAX));
  }
  auto kern = s_acc ? &ffn_bf16_fused_kernel<false, true>
                    : sf.T > 0 ? &ffn_bf16_fused_kernel<true, false> : &ffn_bf16_fused_kernel<false, false>;
  kern<<<device_cu_count(), F_THREADS, F_LDS, s>>>(
      static_cast<const uint16_t*>(x), row_src, T, K, cu, E, H, Hp, static_cast<const uint16_t*>(wg),
      static_cast<const uint16_t*>(wu), static_cast<const uint16_t*>(wd), static_cast<uint16_t*>(h),
      static_cast<uint16_t*>(y), ctl, lag, spin_max, sf, row_w, s_acc);
  return launch_status();
}

}  // namespace moe
