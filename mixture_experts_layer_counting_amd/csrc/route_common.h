// Top-k routing of one token by one wave, shared by the routing kernels.
//
// "Mixture of Kittens", Step 1 "The Math" (router picks the top-k experts and weights
// them); "Distributed expert parallelism", lifecycle item 1. Selection compares the fp32
// logits exactly (larger first, equal logits -> lower expert id); the weights are the
// softmax over the K selected logits, computed in fp32.
//
// Each lane keeps ITEMS logits of the token in registers (expert lane + 64*i). K rounds
// of a wave-wide (value, id) arg-max pick the experts; the owner lane masks its pick.
#pragma once

#include "moe_common.h"

namespace moe {

__device__ __forceinline__ bool route_better(float av, int ae, float bv, int be) {
  return av > bv || (av == bv && ae < be);
}

// This lane's ITEMS logits of the token at `row` (-inf past E; NaN never wins).
template <int ITEMS>
__device__ __forceinline__ void route_load(const float* __restrict__ row, int E, int lane, float (&v)[ITEMS]) {
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int e = lane + 64 * i;
    const float x = e < E ? row[e] : -__builtin_inff();
    v[i] = (x != x) ? -__builtin_inff() : x;
  }
}

// The K picks of the token whose logits are in v: lane k < K gets the k-th expert and its
// weight.
template <int ITEMS>
__device__ __forceinline__ void route_pick(const float (&v)[ITEMS], int E, int K, int lane, int& my_e,
                                           float& my_w) {
  uint64_t taken = 0;
  for (int i = 0; i < ITEMS; ++i)
    if (lane + 64 * i >= E) taken |= (1ull << i);
  float my_v = 0.f, top_v = 0.f;
  my_e = 0;
  for (int k = 0; k < K; ++k) {
    float bv = -__builtin_inff();
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int e = lane + 64 * i;
      if (!((taken >> i) & 1) && route_better(v[i], e, bv, be)) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      if (route_better(ov, oe, bv, be)) {
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
  my_w = z / s;
}

}  // namespace moe
