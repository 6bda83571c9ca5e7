// Permute token copies into expert-contiguous rows: a deterministic counting sort.
//
// "Distributed expert parallelism", lifecycle items 2-3 and "Token permutation and
// metadata": each token is copied k times and the copies are grouped by expert; the
// metadata kept (row of each copy, source of each row, per-expert counts) is what the
// combine needs to restore token order. MoonEP "dispatch fwd" returns the same things for
// one rank (tokens_per_expert, cu_seqlens, expert-grouped hidden rows and their weights).
//
// Row order inside an expert is ascending flat index t*K + k, i.e. a stable sort. No
// atomics on global memory:
//  1. hist:    one block per chunk of PERM_CHUNK tokens counts its copies per expert in
//              LDS and writes them expert-major: hist[e][chunk].
//  2. scan:    one wave per expert turns hist[e][*] into exclusive chunk offsets and the
//              expert total (counts[e]).
//  3. scatter: one block per PERM_TB tokens. It rebuilds cu_seqlens from counts in LDS,
//              counts the copies of earlier tokens of its chunk, ranks its own copies
//              with wave ballots (match by key bits + mbcnt) in flat order, and writes pos /
//              row_src / row_w.
//  4. copy:    (only when x_perm is wanted) one block per token copies its row once from x
//              to its K rows of x_perm with 16-byte loads and stores (the HBM-bound part).
//  (fp8 only) sf: transposes the 1x128 block scales of the rows into the block-major
//              x_perm_sf through LDS, with or without the row copy.
// With routing in the same call (moe_route_permute), step 1 is route_hist_kernel: top-k of
// each token of a chunk and the chunk's histogram in one kernel.
// Padded variant (MoonEP "API walkthrough": token_padding and padded cu_seqlens;
// "Distributed expert parallelism", "Static-capacity versus dropless dispatch"): every
// group is rounded up to a multiple of `pad` rows inside a static buffer of
// T*K + E*(pad-1) rows. counts stay the real ones; cu_seqlens is padded; padding rows have
// row_src = -1, row_w = 0, zero activations and scale 1.
#include <mutex>

#include "moe_common.h"
#include "noalloc.h"
#include "route_common.h"

#include <algorithm>

namespace moe {

moe_status_t launch_fill_bytes(void* p, size_t n, unsigned char v, hipStream_t s);

constexpr int PERM_CHUNK = 16;   // tokens per histogram chunk
constexpr int PERM_TB = 16;      // tokens per scatter block (divides PERM_CHUNK)
constexpr int PERM_THREADS = 256;
constexpr int PERM_WAVES = PERM_THREADS / MOE_WAVE;
constexpr int PERM_MAX_E = 1024;

__global__ __launch_bounds__(PERM_THREADS) void permute_hist_kernel(
    const int* __restrict__ topk_idx, int T, int E, int K, int nch, int* __restrict__ hist,
    int* __restrict__ err) {
  __shared__ int h[PERM_MAX_E];
  for (int e = threadIdx.x; e < E; e += PERM_THREADS) h[e] = 0;
  __syncthreads();
  const int c = blockIdx.x;
  const int t0 = c * PERM_CHUNK;
  const int t1 = min(T, t0 + PERM_CHUNK);
  const int n = (t1 - t0) * K;
  const int* idx = topk_idx + (size_t)t0 * K;
  int bad = 0;
  for (int i = threadIdx.x; i < n; i += PERM_THREADS) {
    const int e = idx[i];
    if ((unsigned)e < (unsigned)E)
      atomicAdd(&h[e], 1);
    else
      bad = 1;
  }
  if (bad) atomicOr(err, 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += PERM_THREADS) hist[(size_t)e * nch + c] = h[e];
}

// Routing and step 1 in one kernel, for moe_route_permute: the block of chunk c routes the
// chunk's PERM_CHUNK tokens, one per wave, exactly as route_topk_kernel does, writes topk_idx / topk_w, and
// counts the picks in LDS into hist[e][c]. The ids it produces are valid and distinct, so
// there is nothing to check.
constexpr int RH_THREADS = 1024;

template <int ITEMS>
__global__ __launch_bounds__(RH_THREADS) void route_hist_kernel(
    const float* __restrict__ logits, int T, int E, int K, int nch, int* __restrict__ topk_idx,
    float* __restrict__ topk_w, int* __restrict__ hist) {
  constexpr int TPW = PERM_CHUNK / (RH_THREADS / MOE_WAVE);  // tokens per wave
  constexpr int BATCH = (ITEMS <= 8 || TPW < 4) ? TPW : TPW / 4;  // logits held at once
  __shared__ int h[PERM_MAX_E];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int e = tid; e < E; e += RH_THREADS) h[e] = 0;
  __syncthreads();
  const int c = blockIdx.x;
  const int tw = c * PERM_CHUNK + wave * TPW;
  for (int b = 0; b < TPW; b += BATCH) {
    float v[BATCH][ITEMS];
#pragma unroll
    for (int j = 0; j < BATCH; ++j)  // tokens past T load row T-1 and are not ranked
      route_load<ITEMS>(logits + (size_t)min(tw + b + j, T - 1) * E, E, lane, v[j]);
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int t = tw + b + j;
      if (t >= T) break;
      int my_e;
      float my_w;
      route_pick<ITEMS>(v[j], E, K, lane, my_e, my_w);
      if (lane < K) {
        topk_idx[(size_t)t * K + lane] = my_e;
        topk_w[(size_t)t * K + lane] = my_w;
        atomicAdd(&h[my_e], 1);
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += RH_THREADS) hist[(size_t)e * nch + c] = h[e];
}

// Wave-inclusive scan of v across the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

__global__ __launch_bounds__(256) void permute_scan_kernel(int* __restrict__ hist, int nch, int E,
                                                           int* __restrict__ counts) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (e >= E) return;
  int running = 0;
  int* row = hist + (size_t)e * nch;
  // SCAN_BATCH groups of 64 chunk counts are loaded before any is scanned, so a wave waits
  // for one load round trip per 64 * SCAN_BATCH chunks rather than one per 64
  constexpr int SCAN_BATCH = 8;
  for (int base = 0; base < nch; base += 64 * SCAN_BATCH) {
    int v[SCAN_BATCH];
#pragma unroll
    for (int u = 0; u < SCAN_BATCH; ++u) {
      const int i = base + 64 * u + lane;
      v[u] = i < nch ? row[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < SCAN_BATCH; ++u) {
      const int i = base + 64 * u + lane;
      const int incl = wave_incl_scan(v[u]);
      if (i < nch) row[i] = running + incl - v[u];
      running += __shfl(incl, 63, 64);
    }
  }
  if (lane == 0) counts[e] = running;
}

// Duplicate expert ids within one token (validation mode only).
__global__ void permute_dup_check_kernel(const int* __restrict__ topk_idx, int T, int K,
                                         int* __restrict__ err) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int* r = topk_idx + (size_t)t * K;
  for (int a = 0; a < K; ++a)
    for (int b = a + 1; b < K; ++b)
      if (r[a] == r[b]) atomicOr(err, 2);
}

template <int VB>  // bytes per vector access: 16, 4 or 1
struct VecT;
template <>
struct VecT<16> {
  typedef int4 type;
};
template <>
struct VecT<4> {
  typedef int type;
};
template <>
struct VecT<1> {
  typedef unsigned char type;
};

__global__ __launch_bounds__(PERM_THREADS) void permute_scatter_kernel(
    const int* __restrict__ topk_idx, const float* __restrict__ topk_w, int T, int E, int K,
    int nch, const int* __restrict__ counts, const int* __restrict__ choff,
    int* __restrict__ cu_seqlens, int* __restrict__ pos, int* __restrict__ row_src,
    float* __restrict__ row_w, int key_bits, int pad, int* __restrict__ err) {
  __shared__ int cu[PERM_MAX_E + 1];
  __shared__ int pre[PERM_MAX_E];
  __shared__ int wh[PERM_WAVES][PERM_MAX_E];
  __shared__ int wsum[PERM_WAVES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const int tb0 = blockIdx.x * PERM_TB;
  const int tb1 = min(T, tb0 + PERM_TB);
  const int chunk = tb0 / PERM_CHUNK;
  const int tc0 = chunk * PERM_CHUNK;
  const int nb = (tb1 - tb0) * K;
  const int* idx = topk_idx + (size_t)tb0 * K;
  // the first group's expert ids, their chunk offsets and weights are loaded before the scan
  // of counts below, so that their round trips overlap it instead of following it
  const int e_first = tid < nb ? idx[tid] : -1;
  const bool v_first = tid < nb && (unsigned)e_first < (unsigned)E;
  const int co_first = v_first ? choff[(size_t)e_first * nch + chunk] : 0;
  const float w_first = (v_first && row_w) ? topk_w[(size_t)tb0 * K + tid] : 0.f;

  // 1. cu_seqlens from counts (block-wide exclusive scan, E <= 1024: 4 per thread)
  {
    int loc[4];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid * 4 + j;
      loc[j] = e < E ? (counts[e] + pad - 1) / pad * pad : 0;  // group rows (padded)
      sum += loc[j];
    }
    const int incl = wave_incl_scan(sum);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    int run = base + incl - sum;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid * 4 + j;
      if (e < E) cu[e] = run;
      run += loc[j];
    }
    if (tid == 0) {
      int total = 0;
      for (int w = 0; w < PERM_WAVES; ++w) total += wsum[w];
      cu[E] = total;
    }
  }
  for (int e = tid; e < E; e += PERM_THREADS) {
    pre[e] = 0;
#pragma unroll
    for (int w = 0; w < PERM_WAVES; ++w) wh[w][e] = 0;
  }
  __syncthreads();
  if (blockIdx.x == 0)
    for (int e = tid; e <= E; e += PERM_THREADS) cu_seqlens[e] = cu[e];
  if (T == 0) return;

  // 2. copies of earlier tokens in the same chunk
  {
    const int n = (tb0 - tc0) * K;
    const int* idx = topk_idx + (size_t)tc0 * K;
    for (int i = tid; i < n; i += PERM_THREADS) {
      const int e = idx[i];
      if ((unsigned)e < (unsigned)E) atomicAdd(&pre[e], 1);
    }
  }
  __syncthreads();

  // 3. stable ranks of this block's copies, 256 at a time in flat order
  for (int g = 0; g < nb; g += PERM_THREADS) {
    const int i = g + tid;
    const bool in = i < nb;
    const int e = g == 0 ? e_first : in ? idx[i] : -1;
    const bool valid = in && (unsigned)e < (unsigned)E;
    const int key = valid ? e : (1 << key_bits) - 1;
    const uint64_t m = match_any(key, key_bits);
    const int r = popc_below(m);
    if (valid && r == 0) wh[wave][e] = __popcll(m);
    __syncthreads();
    if (in) {
      int p = -1;
      if (valid) {
        p = cu[e] + (g == 0 ? co_first : choff[(size_t)e * nch + chunk]) + pre[e] + r;
        for (int w = 0; w < wave; ++w) p += wh[w][e];
        if (p < cu[e] || p >= cu[e + 1]) {  // cannot happen; keeps every store in bounds
          atomicOr(err, 4);
          p = -1;
        } else {
          const int flat = tb0 * K + i;
          row_src[p] = flat;
          if (row_w) row_w[p] = g == 0 ? w_first : topk_w[flat];
        }
      }
      pos[(size_t)tb0 * K + i] = p;
    }
    __syncthreads();
    // fold this group's counts into pre[] and clear wh for the next group
    if (g + PERM_THREADS < nb) {
      for (int j = tid; j < E; j += PERM_THREADS) {
        int tot = 0;
        for (int w = 0; w < PERM_WAVES; ++w) {
          tot += wh[w][j];
          wh[w][j] = 0;
        }
        pre[j] += tot;
      }
      __syncthreads();
    }
  }

}

// Copy each token row once from x to its K rows of x_perm (16-byte, 4-byte or 1-byte
// accesses). One block per token keeps every CU busy on this HBM-bound copy; the block has a
// thread per vector of the row (up to 1024), so a row is one pass (T=8192 K=8, 14 KiB rows:
// 194 -> 178 us, 5.95 TB/s, against 256 threads; non-temporal stores were slower).
template <int VB>
__global__ __launch_bounds__(1024) void permute_copy_kernel(const unsigned char* __restrict__ x,
                                                           const int* __restrict__ pos, int K,
                                                           unsigned char* __restrict__ x_perm,
                                                           int row_bytes) {
  typedef typename VecT<VB>::type V;
  __shared__ int p[32];
  const int t = blockIdx.x;
  if (threadIdx.x < K) p[threadIdx.x] = pos[(size_t)t * K + threadIdx.x];
  __syncthreads();
  const int nv = row_bytes / VB;
  const V* src = reinterpret_cast<const V*>(x + (size_t)t * row_bytes);
  for (int c = threadIdx.x; c < nv; c += blockDim.x) {
    const V v = src[c];
    for (int k = 0; k < K; ++k)
      if (p[k] >= 0) reinterpret_cast<V*>(x_perm + (size_t)p[k] * row_bytes)[c] = v;
  }
}

// Block scales of the permuted rows, block-major [H/128][M], transposed through LDS: a block
// takes 64 rows and up to 64 scale columns; it reads each row's source scales as one
// contiguous run of x_sf [T][H/128] and writes each column's 64 rows as one 256-byte run.
// Rows past cu_seqlens[E] (dropped copies) are left as they are; padding rows get scale 1.
constexpr int PSF_ROWS = 64;
constexpr int PSF_PER_THREAD = PSF_ROWS * PSF_ROWS / 256;
__global__ __launch_bounds__(256) void permute_sf_kernel(const float* __restrict__ x_sf,
                                                         const int* __restrict__ row_src,
                                                         const int* __restrict__ cu_seqlens, int E,
                                                         int K, int M, int nsf,
                                                         float* __restrict__ x_perm_sf) {
  __shared__ float tile[PSF_ROWS][PSF_ROWS + 1];
  const int p0 = blockIdx.x * PSF_ROWS;
  const int c0 = blockIdx.y * PSF_ROWS;
  const int rows = cu_seqlens[E];  // rows actually holding a copy
  const int nr = min(PSF_ROWS, rows - p0);
  if (nr <= 0) return;
  const int nc = min(PSF_ROWS, nsf - c0);
  // thread -> column lane % 64 of rows wave + 4 i: each wave reads whole row runs; all loads
  // of a thread are issued before the first LDS store
  const int lane = threadIdx.x % PSF_ROWS, rq = threadIdx.x / PSF_ROWS;
  float v[PSF_PER_THREAD];
#pragma unroll
  for (int i = 0; i < PSF_PER_THREAD; ++i) {
    const int r = rq + 4 * i;
    const int sr = r < nr ? row_src[p0 + r] : -1;
    v[i] = (sr >= 0 && lane < nc) ? x_sf[(size_t)(sr / K) * nsf + c0 + lane] : 1.0f;  // padding: 1
  }
#pragma unroll
  for (int i = 0; i < PSF_PER_THREAD; ++i) tile[rq + 4 * i][lane] = v[i];
  __syncthreads();
  // thread -> row lane % 64 of columns wave + 4 i: 256-byte runs of one column
#pragma unroll
  for (int i = 0; i < PSF_PER_THREAD; ++i) {
    const int c = rq + 4 * i;
    if (lane < nr && c < nc) x_perm_sf[(size_t)(c0 + c) * M + p0 + lane] = tile[lane][c];
  }
}

// Padded layout: mark every row of the static buffer as padding before the scatter fills
// the real ones.
__global__ __launch_bounds__(256) void permute_pad_fill_kernel(int* __restrict__ row_src,
                                                               float* __restrict__ row_w, int cap) {
  for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < cap; r += gridDim.x * blockDim.x) {
    row_src[r] = -1;
    if (row_w) row_w[r] = 0.f;
  }
}

// Padded layout: zero the activation rows of padding rows inside the groups.
__global__ __launch_bounds__(256) void permute_zero_pad_kernel(const int* __restrict__ row_src,
                                                               const int* __restrict__ cu_seqlens,
                                                               int E, unsigned char* __restrict__ x_perm,
                                                               int row_bytes) {
  const int r = blockIdx.x;
  if (r >= cu_seqlens[E] || row_src[r] >= 0) return;
  unsigned char* dst = x_perm + (size_t)r * row_bytes;
  if (row_bytes % 16 == 0 && (uintptr_t)dst % 16 == 0) {
    for (int c = threadIdx.x; c < row_bytes / 16; c += blockDim.x)
      reinterpret_cast<int4*>(dst)[c] = make_int4(0, 0, 0, 0);
  } else {
    for (int c = threadIdx.x; c < row_bytes; c += blockDim.x) dst[c] = 0;
  }
}

// Scratch for callers that cannot allocate (moe_permute_noalloc): the chunk histograms and
// the error word live in this file-scope array instead of a caller workspace. Every device
// the library runs on holds its own copy until the process ends. In host code the array's
// name is a host-side stand-in, not a device address: its address on a device comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that
// address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

void* permute_noalloc_scratch() {
  static std::mutex mu;
  static void* ptr[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}

size_t permute_ws_bytes(int T, int E, int K) {
  (void)K;
  const size_t nch = (size_t)(T + PERM_CHUNK - 1) / PERM_CHUNK;
  return align_up(sizeof(int) * (nch * (size_t)E), 256) + 256;  // hist/offsets + error word
}

moe_status_t launch_permute(const void* x, const float* x_sf, int elem_bytes,
                            const int* topk_idx, const float* topk_w, int T, int H, int E, int K,
                            int* counts, int* cu_seqlens, int* pos, int* row_src, float* row_w,
                            void* x_perm, float* x_perm_sf, void* ws, bool validate, int pad,
                            int cap, int** err_out, hipStream_t s, bool hist_done) {
  const int nch = (T + PERM_CHUNK - 1) / PERM_CHUNK;
  int* hist = static_cast<int*>(ws);
  int* err = reinterpret_cast<int*>(static_cast<char*>(ws) +
                                    align_up(sizeof(int) * ((size_t)nch * E), 256));
  *err_out = err;
  if (validate) {
    const moe_status_t st = launch_fill_bytes(err, sizeof(int), 0, s);
    if (st != MOE_OK) return st;
  }
  if (nch > 0 && !hist_done) {
    permute_hist_kernel<<<nch, PERM_THREADS, 0, s>>>(topk_idx, T, E, K, nch, hist, err);
    if (validate && K > 1)
      permute_dup_check_kernel<<<(T + 255) / 256, 256, 0, s>>>(topk_idx, T, K, err);
  }
  permute_scan_kernel<<<(E + 3) / 4, 256, 0, s>>>(hist, nch, E, counts);
  int key_bits = 1;
  while ((1 << key_bits) <= E) ++key_bits;  // E itself (invalid) must be representable
  const int row_bytes = H * elem_bytes;
  const int sf_per_row = x_sf ? H / 128 : 0;
  const int nblk = T > 0 ? (T + PERM_TB - 1) / PERM_TB : 1;
  const unsigned char* xb = static_cast<const unsigned char*>(x);
  unsigned char* xp = static_cast<unsigned char*>(x_perm);
  if (pad > 1 && cap > 0)
    permute_pad_fill_kernel<<<std::min((cap + 255) / 256, 1024), 256, 0, s>>>(row_src, row_w, cap);
  permute_scatter_kernel<<<nblk, PERM_THREADS, 0, s>>>(topk_idx, topk_w, T, E, K, nch, counts, hist,
                                                       cu_seqlens, pos, row_src, row_w, key_bits, pad,
                                                       err);
  if (T > 0 && x_perm) {
    const bool a16 = (row_bytes % 16 == 0) && ((uintptr_t)x % 16 == 0) && ((uintptr_t)x_perm % 16 == 0);
    const bool a4 = (row_bytes % 4 == 0) && ((uintptr_t)x % 4 == 0) && ((uintptr_t)x_perm % 4 == 0);
    const int vb = a16 ? 16 : a4 ? 4 : 1;
    // a thread per vector, whole waves, at least K (the block stages pos[t, 0..K-1])
    const int nt = std::min(1024, std::max(64, (row_bytes / vb + 63) / 64 * 64));
    if (a16)
      permute_copy_kernel<16><<<T, nt, 0, s>>>(xb, pos, K, xp, row_bytes);
    else if (a4)
      permute_copy_kernel<4><<<T, nt, 0, s>>>(xb, pos, K, xp, row_bytes);
    else
      permute_copy_kernel<1><<<T, nt, 0, s>>>(xb, pos, K, xp, row_bytes);
  }
  if (T > 0 && x_perm && pad > 1)
    permute_zero_pad_kernel<<<cap, 256, 0, s>>>(row_src, cu_seqlens, E, xp, row_bytes);
  if (x_sf && x_perm_sf && T > 0) {
    const dim3 grid((cap + PSF_ROWS - 1) / PSF_ROWS, (sf_per_row + PSF_ROWS - 1) / PSF_ROWS);
    permute_sf_kernel<<<grid, 256, 0, s>>>(x_sf, row_src, cu_seqlens, E, K, cap, sf_per_row, x_perm_sf);
  }
  return launch_status();
}

moe_status_t launch_route_hist(const float* logits, int T, int E, int K, int* topk_idx,
                               float* topk_w, void* ws, hipStream_t s) {
  const int nch = (T + PERM_CHUNK - 1) / PERM_CHUNK;
  if (nch == 0) return MOE_OK;
  int* hist = static_cast<int*>(ws);
  if (E <= 64)
    route_hist_kernel<1><<<nch, RH_THREADS, 0, s>>>(logits, T, E, K, nch, topk_idx, topk_w, hist);
  else if (E <= 128)
    route_hist_kernel<2><<<nch, RH_THREADS, 0, s>>>(logits, T, E, K, nch, topk_idx, topk_w, hist);
  else if (E <= 256)
    route_hist_kernel<4><<<nch, RH_THREADS, 0, s>>>(logits, T, E, K, nch, topk_idx, topk_w, hist);
  else if (E <= 512)
    route_hist_kernel<8><<<nch, RH_THREADS, 0, s>>>(logits, T, E, K, nch, topk_idx, topk_w, hist);
  else
    route_hist_kernel<16><<<nch, RH_THREADS, 0, s>>>(logits, T, E, K, nch, topk_idx, topk_w, hist);
  return launch_status();
}

}  // namespace moe
