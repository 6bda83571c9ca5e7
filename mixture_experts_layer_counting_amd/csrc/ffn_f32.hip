// Grouped expert FFN in fp32 (plain FMA, for fp32 layers).
//
// Same operation and schedule as the bf16 kernels ("Mixture of Kittens", Step 1: expert =
// Down(SwiGLU(Up x, Gate x)); "Distributed expert parallelism", "Grouped expert
// computation"): a persistent loop over 64x64 output tiles of every expert's row group,
// 16-deep K steps staged in LDS, 4x4 outputs per thread, any H / Hp (edges masked). The
// optional row maps gather A rows by token index and scatter row_w * y into an fp32
// accumulator, as in the bf16 kernels.
#include "moe_common.h"
#include "tile_sched.h"

namespace moe {

constexpr int FF_BM = 64;
constexpr int FF_BN = 64;
constexpr int FF_BK = 16;
constexpr int FF_THREADS = 256;
constexpr int FF_MAX_E = 512;  // 2 * threads

template <bool GATED>
__global__ __launch_bounds__(FF_THREADS) void ffn_f32_kernel(
    const float* __restrict__ A, const int* __restrict__ cu, int M, int E, int Kd, int N,
    const float* __restrict__ B0, const float* __restrict__ B1, float* __restrict__ C,
    RowMaps maps) {
  constexpr int NB = GATED ? 2 : 1;
  __shared__ int tstart[FF_MAX_E + 1];
  __shared__ int wsum[FF_THREADS / 64];
  __shared__ float sA[FF_BK][FF_BM + 1];
  __shared__ float sB[NB][FF_BK][FF_BN];
  __shared__ int sRow[FF_BM];  // source row of A for each tile row
  const int tid = threadIdx.x;
  const int ntn = (N + FF_BN - 1) / FF_BN;
  const int total = build_tile_prefix<FF_BM, FF_THREADS>(cu, E, ntn, tstart, wsum);
  const int ty = tid >> 4, tx = tid & 15;
  for (int t = xcd_slot(blockIdx.x, gridDim.x); t < total; t += gridDim.x) {
    const int e = find_expert(tstart, E, t);
    const int lt = t - tstart[e];
    const int rows_e = cu[e + 1] - cu[e];
    const int mte = (rows_e + FF_BM - 1) / FF_BM;
    const int ntile = lt / mte, mtile = lt - ntile * mte;
    const int row0 = cu[e] + mtile * FF_BM;
    const int rows_valid = min(FF_BM, rows_e - mtile * FF_BM);
    const int n0 = ntile * FF_BN;
    const float* W0 = B0 + (size_t)e * Kd * N;
    const float* W1 = GATED ? B1 + (size_t)e * Kd * N : nullptr;
    __syncthreads();  // previous tile's readers of sRow are done
    for (int r = tid; r < FF_BM; r += FF_THREADS)
      sRow[r] = r < rows_valid ? (maps.a_src ? maps.a_src[row0 + r] : (row0 + r) * maps.a_k) : -1;
    __syncthreads();
    float acc[NB][4][4];
    for (int b = 0; b < NB; ++b)
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[b][i][j] = 0.f;
    for (int k0 = 0; k0 < Kd; k0 += FF_BK) {
      for (int q = tid; q < FF_BM * FF_BK; q += FF_THREADS) {
        const int r = q / FF_BK, k = q % FF_BK;
        sA[k][r] = (sRow[r] >= 0 && k0 + k < Kd) ? A[(size_t)(sRow[r] / maps.a_k) * Kd + k0 + k] : 0.f;
      }
      for (int q = tid; q < FF_BK * FF_BN; q += FF_THREADS) {
        const int k = q / FF_BN, n = q % FF_BN;
        const bool ok = (k0 + k < Kd) && (n0 + n < N);
        sB[0][k][n] = ok ? W0[(size_t)(k0 + k) * N + n0 + n] : 0.f;
        if constexpr (GATED) sB[1][k][n] = ok ? W1[(size_t)(k0 + k) * N + n0 + n] : 0.f;
      }
      __syncthreads();
      for (int k = 0; k < FF_BK; ++k) {
        float a[4], bv[NB][4];
        for (int i = 0; i < 4; ++i) a[i] = sA[k][ty * 4 + i];
        for (int b = 0; b < NB; ++b)
          for (int j = 0; j < 4; ++j) bv[b][j] = sB[b][k][tx * 4 + j];
        for (int b = 0; b < NB; ++b)
          for (int i = 0; i < 4; ++i)
            for (int j = 0; j < 4; ++j) acc[b][i][j] = fmaf(a[i], bv[b][j], acc[b][i][j]);
      }
      __syncthreads();
    }
    for (int i = 0; i < 4; ++i) {
      const int r = ty * 4 + i;
      if (r >= rows_valid) continue;
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + tx * 4 + j;
        if (n >= N) continue;
        float v;
        if constexpr (GATED)
          v = silu_f32(acc[0][i][j]) * acc[1][i][j];
        else
          v = acc[0][i][j];
        if (!GATED && maps.s_acc) {
          const int src = maps.s_src[row0 + r];  // -1: padding row
          if (src >= 0) unsafeAtomicAdd(maps.s_acc + (size_t)(src / maps.s_k) * N + n, maps.s_w[row0 + r] * v);
        } else
          C[(size_t)(row0 + r) * N + n] = v;
      }
    }
  }
}

moe_status_t launch_ffn_gate_up_f32(const void* a, const int* cu, int M, int E, int H, int Hp,
                                    const void* wg, const void* wu, void* h, const RowMaps& maps,
                                    hipStream_t s) {
  if (M == 0) return MOE_OK;
  ffn_f32_kernel<true><<<device_cu_count(), FF_THREADS, 0, s>>>(
      static_cast<const float*>(a), cu, M, E, H, Hp, static_cast<const float*>(wg),
      static_cast<const float*>(wu), static_cast<float*>(h), maps);
  return launch_status();
}

moe_status_t launch_ffn_down_f32(const void* h, const int* cu, int M, int E, int H, int Hp,
                                 const void* wd, void* y, const RowMaps& maps, hipStream_t s) {
  if (M == 0) return MOE_OK;
  ffn_f32_kernel<false><<<device_cu_count(), FF_THREADS, 0, s>>>(
      static_cast<const float*>(h), cu, M, E, Hp, H, static_cast<const float*>(wd), nullptr,
      static_cast<float*>(y), maps);
  return launch_status();
}

}  // namespace moe
