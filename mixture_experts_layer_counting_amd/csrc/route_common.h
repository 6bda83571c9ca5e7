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

#include <type_traits>

namespace moe {

__device__ __forceinline__ bool route_better(float av, int ae, float bv, int be) {
  return av > bv || (av == bv && ae < be);
}

// Wave-wide reductions without the LDS crossbar: within each 16-lane row, DPP moves pair lane
// l with l^1, l^2 (quad permutes), then with the mirror lane of its 8 and of its 16; across
// rows, v_permlane16_swap and v_permlane32_swap applied to a value and itself hand every lane
// the values of both rows of its row pair, then of both halves. After each stage every lane
// of a group holds the group's result, so the next stage only has to pair groups.
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int x) {
  return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7 - i within each 8
constexpr int DPP_MIRROR = 0x140;      // lane i <-> 15 - i within each 16

// The better of (bv, be) over the 64 lanes, in every lane ("better": larger value, then lower
// id; the order is total, so the result does not depend on the pairing).
__device__ __forceinline__ void wave_best(float& bv, int& be) {
  auto take = [&](float ov, int oe) {
    if (route_better(ov, oe, bv, be)) {
      bv = ov;
      be = oe;
    }
  };
  auto dpp = [&](auto ctrl) {
    constexpr int C = decltype(ctrl)::value;
    take(__int_as_float(dpp_mov<C>(__float_as_int(bv))), dpp_mov<C>(be));
  };
  dpp(std::integral_constant<int, DPP_XOR1>{});
  dpp(std::integral_constant<int, DPP_XOR2>{});
  dpp(std::integral_constant<int, DPP_HALF_MIRROR>{});
  dpp(std::integral_constant<int, DPP_MIRROR>{});
  const auto v16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
  const auto e16 = __builtin_amdgcn_permlane16_swap((uint32_t)be, (uint32_t)be, false, false);
  bv = __uint_as_float(v16[0]);
  be = (int)e16[0];
  take(__uint_as_float(v16[1]), (int)e16[1]);
  const auto v32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
  const auto e32 = __builtin_amdgcn_permlane32_swap((uint32_t)be, (uint32_t)be, false, false);
  bv = __uint_as_float(v32[0]);
  be = (int)e32[0];
  take(__uint_as_float(v32[1]), (int)e32[1]);
}

// The sum of s over the 64 lanes, in every lane (in the pairing order above).
__device__ __forceinline__ float wave_sum(float s) {
  s += __int_as_float(dpp_mov<DPP_XOR1>(__float_as_int(s)));
  s += __int_as_float(dpp_mov<DPP_XOR2>(__float_as_int(s)));
  s += __int_as_float(dpp_mov<DPP_HALF_MIRROR>(__float_as_int(s)));
  s += __int_as_float(dpp_mov<DPP_MIRROR>(__float_as_int(s)));
  const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  s = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
  const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
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
    wave_best(bv, be);
    if ((be & 63) == lane) taken |= (1ull << (be >> 6));
    if (k == 0) top_v = bv;
    if (lane == k) {
      my_v = bv;
      my_e = be;
    }
  }
  const float z = lane < K ? expf(my_v - top_v) : 0.f;
  my_w = z / wave_sum(z);
}

}  // namespace moe
