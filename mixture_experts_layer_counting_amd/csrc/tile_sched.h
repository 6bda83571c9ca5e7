// Device-side tile schedule over variable-size expert groups (shared by the grouped FFN
// kernels). cu_seqlens [E+1] gives each expert's rows; expert e contributes
// ceil(rows_e / BM) * ntn tiles. The exclusive prefix lives in LDS and a tile index is
// mapped back to its expert by binary search, so no host synchronisation is needed.
#pragma once
#include "moe_common.h"

namespace moe {

__device__ __forceinline__ int sched_wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

// Writes tstart[0..E] (exclusive prefix, tstart[E] = total) and returns the total.
// Needs E <= 2 * THREADS and wsum[THREADS / 64] of LDS scratch.
template <int BM, int THREADS>
__device__ int build_tile_prefix(const int* __restrict__ cu, int E, int ntn, int* tstart,
                                 int* wsum) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int e0 = 2 * tid, e1 = 2 * tid + 1;
  int c0 = 0, c1 = 0;
  if (e0 < E) c0 = ((cu[e0 + 1] - cu[e0] + BM - 1) / BM) * ntn;
  if (e1 < E) c1 = ((cu[e1 + 1] - cu[e1] + BM - 1) / BM) * ntn;
  const int s = c0 + c1;
  const int incl = sched_wave_incl_scan(s);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < THREADS / 64; ++w) {
    if (w < wave) base += wsum[w];
    total += wsum[w];
  }
  const int ex = base + incl - s;
  if (e0 < E) tstart[e0] = ex;
  if (e1 < E) tstart[e1] = ex + c0;
  if (tid == 0) tstart[E] = total;
  __syncthreads();
  return total;
}

// Largest e in [0, E) with tstart[e] <= t: the (non-empty) expert owning tile t.
__device__ __forceinline__ int find_expert(const int* tstart, int E, int t) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tstart[mid] <= t)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// Rows per m-tile when an expert's rows_e rows are spread evenly over its mte = ceil(rows_e / bm)
// tiles: ceil(rows_e / mte) rounded up to whole 32-row blocks. That is at most bm, and since
// (mte - 1) * bm < rows_e the last tile keeps at least one row. The tiles of one expert then
// run the same number of 32-row MFMA blocks and stream the shared weight panel in step, so
// the panel is fetched from HBM once and reused from L2 instead of being re-read by a
// straggler tile that has fallen behind.
__device__ __forceinline__ int even_chunk(int rows_e, int mte) {
  return ((rows_e + mte - 1) / mte + 31) & ~31;
}

// Block slot for the persistent loop: blocks are dispatched round-robin over the 8 XCDs,
// so block b runs on XCD b % 8; giving XCD x the contiguous slots [x*G/8, (x+1)*G/8)
// keeps neighbouring tiles (same expert, same weight panel) in one L2.
__device__ __forceinline__ int xcd_slot(int b, int G) {
  return (G % 8 == 0) ? (b % 8) * (G / 8) + (b / 8) : b;
}

}  // namespace moe
