// Top-k routing: one wave per token (the selection itself is in route_common.h).
// Reading the [T, E] logits once is the whole memory traffic.
#include "route_common.h"

namespace moe {

template <int ITEMS>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int K, int* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[ITEMS];
  route_load<ITEMS>(logits + (size_t)t * E, E, lane, v);
  int my_e;
  float my_w;
  route_pick<ITEMS>(v, E, K, lane, my_e, my_w);
  if (lane < K) {
    topk_idx[(size_t)t * K + lane] = my_e;
    topk_w[(size_t)t * K + lane] = my_w;
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
