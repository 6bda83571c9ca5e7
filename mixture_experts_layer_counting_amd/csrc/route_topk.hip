// Top-k routing: one wave per token.
//
// "Mixture of Kittens", Step 1 "The Math" (router picks the top-k experts and weights
// them); "Distributed expert parallelism", lifecycle item 1. Selection compares the fp32
// logits exactly (larger first, equal logits -> lower expert id); the weights are the
// softmax over the K selected logits, computed in fp32.
//
// Each lane keeps ITEMS logits of the token in registers (expert lane + 64*i). K rounds
// of a wave-wide (value, id) arg-max pick the experts; the owner lane masks its pick.
// Reading the [T, E] logits once is the whole memory traffic.
#include "moe_common.h"

namespace moe {

struct Cand {
  float v;
  int e;
};

__device__ __forceinline__ bool better(float av, int ae, float bv, int be) {
  return av > bv || (av == bv && ae < be);
}

template <int ITEMS>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int K, int* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  float v[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int e = lane + 64 * i;
    float x = e < E ? row[e] : -__builtin_inff();
    v[i] = (x != x) ? -__builtin_inff() : x;  // NaN never wins
  }
  uint64_t taken = 0;
  for (int i = 0; i < ITEMS; ++i)
    if (lane + 64 * i >= E) taken |= (1ull << i);

  float my_v = 0.f, top_v = 0.f;
  int my_e = 0;
  for (int k = 0; k < K; ++k) {
    float bv = -__builtin_inff();
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int e = lane + 64 * i;
      if (!((taken >> i) & 1) && better(v[i], e, bv, be)) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      if (better(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= (1ull << (be >> 6));
    if (k == 0) top_v = bv;
    if (lane == k) {
      my_v = bv;
      my_e = be;
    }
  }
  const float z = lane < K ? expf(my_v - top_v) : 0.f;
  float s = z;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane < K) {
    topk_idx[(size_t)t * K + lane] = my_e;
    topk_w[(size_t)t * K + lane] = z / s;
  }
}

moe_status_t launch_route_topk(const float* logits, int T, int E, int K, int* topk_idx,
                               float* topk_w, hipStream_t s) {
  if (T == 0) return MOE_OK;
  const dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    route_topk_kernel<1><<<grid, block, 0, s>>>(logits, T, E, K, topk_idx, topk_w);
  else if (E <= 128)
    route_topk_kernel<2><<<grid, block, 0, s>>>(logits, T, E, K, topk_idx, topk_w);
  else if (E <= 256)
    route_topk_kernel<4><<<grid, block, 0, s>>>(logits, T, E, K, topk_idx, topk_w);
  else if (E <= 512)
    route_topk_kernel<8><<<grid, block, 0, s>>>(logits, T, E, K, topk_idx, topk_w);
  else if (E <= 1024)
    route_topk_kernel<16><<<grid, block, 0, s>>>(logits, T, E, K, topk_idx, topk_w);
  else
    route_topk_kernel<64><<<grid, block, 0, s>>>(logits, T, E, K, topk_idx, topk_w);
  return launch_status();
}

}  // namespace moe
