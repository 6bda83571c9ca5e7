// Internal helpers shared by the MoE kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <atomic>

#include "../../include/moe.h"

#define MOE_WAVE 64

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

#define MOE_LDS __attribute__((address_space(3)))

namespace moe {

// ---- host-side launch helpers -------------------------------------------------------

// Number of compute units of the current device (cached per device id).
int device_cu_count();

inline moe_status_t launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr int MOE_MAX_DEVICES = 64;

// Raise a kernel's dynamic LDS limit to `bytes` on the current device, once per device:
// `done` is the caller's per-kernel table of device flags (a zero-initialised static). Two
// threads arriving together may both set it, which is harmless.
inline moe_status_t ensure_lds_limit(const void* kernel, int bytes, std::atomic<unsigned char>* done) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MOE_MAX_DEVICES) return MOE_EHIP;
  if (done[dev].load(std::memory_order_acquire)) return MOE_OK;
  if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
    return MOE_EHIP;
  done[dev].store(1, std::memory_order_release);
  return MOE_OK;
}

bool env_flag(const char* name);

// Optional row maps of a grouped-FFN launch; null pointers select the plain layout.
//  gather  (gate/up): A row of group row r is row a_src[r] / a_k of A, which has a_rows rows.
//                     fp8 only: with a_sf_perm set, the activation scales are read from the
//                     permuted block-major copy a_sf_perm [Kd/128][M] (row r's scales at
//                     column r) instead of being gathered from A's scales row by row.
//  scatter (down):    instead of storing y[r], add s_w[r] * y[r] to row s_src[r] / s_k of the
//                     fp32 accumulator s_acc (fp32 atomics).
struct RowMaps {
  const int* a_src = nullptr;
  int a_k = 1;
  int a_rows = 0;
  const float* a_sf_perm = nullptr;
  const int* s_src = nullptr;
  const float* s_w = nullptr;
  int s_k = 1;
  float* s_acc = nullptr;
  // gate/up only: also store g = x.Wg and u = x.Wu (bf16, [rows, N]) for the backward
  uint16_t* save_g = nullptr;
  uint16_t* save_u = nullptr;
};

// The shared expert folded into the single-launch bf16 FFN as one more expert (T = 0: none):
// a dense SwiGLU FFN of intermediate size Hp (the routed experts' own) over the T token rows
// of x in order, with its own weights wg, wu [H, Hp] and wd [Hp, H] and its own h [T, Hp] and
// y [T, H] ("Mixture of Kittens", Step 1: MoE(x) = SharedExpert(x) + the routed sum).
struct SharedFold {
  const uint16_t* x = nullptr;
  const uint16_t *wg = nullptr, *wu = nullptr, *wd = nullptr;
  uint16_t *h = nullptr, *y = nullptr;
  int T = 0;
};

// ---- device helpers -----------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
// fp32 -> bf16, round to nearest even (NaN stays NaN): gfx950's v_cvt_pk_bf16_f32, which
// converts two values per instruction.
typedef __bf16 bf16x2_cvt_t __attribute__((ext_vector_type(2)));
typedef float f32x2_cvt_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_cvt_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_cvt_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// silu(z) = z * sigmoid(z). The reciprocal is the hardware one (about 1 ulp of fp32), far
// below the bf16 rounding the results get; the IEEE division it replaces costs ten
// instructions per element in the epilogues.
__device__ __forceinline__ float silu_f32(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Sixteen columns of one row of a row-lane 32x32 block, as bf16 (rounded to nearest even).
// Lane l holds row l % 32: v0..v3 are columns 4(l / 32) + 0..3 and v4..v7 columns
// 8 + 4(l / 32) + 0..3. v_permlane32_swap trades the second group of the lower half for the
// first group of the upper half, after which lane l < 32 holds columns 0..7 and lane l + 32
// columns 8..15: the 16 bytes this lane writes at its column 8(l / 32). All 64 lanes must be
// active.
__device__ __forceinline__ uint4 pack_row16(float v0, float v1, float v2, float v3, float v4, float v5,
                                            float v6, float v7) {
  const uint32_t a0 = pack_bf16x2(v0, v1), a1 = pack_bf16x2(v2, v3);
  const uint32_t b0 = pack_bf16x2(v4, v5), b1 = pack_bf16x2(v6, v7);
  // swap(x, y) returns (x of lanes 0..31 | y of lanes 0..31, x of lanes 32..63 | y of lanes
  // 32..63): the lower half keeps x and receives the upper half's x as the second result; the
  // upper half receives the lower half's y as the first result and keeps y
  const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
  return make_uint4(s0[0], s1[0], s0[1], s1[1]);
}

__device__ __forceinline__ uint4 pack_row16(const f32x16_t& a, int i0) {
  return pack_row16(a[i0], a[i0 + 1], a[i0 + 2], a[i0 + 3], a[i0 + 4], a[i0 + 5], a[i0 + 6], a[i0 + 7]);
}

// fp32 -> OCP e4m3fn codes of four values (gfx950's v_cvt_pk_fp8_f32: round to nearest even;
// identical to f32_to_e4m3 below on every |v| <= 448, which was checked on the device for all
// such fp32 values), packed low byte first. Adding +0 turns -0 into +0, so an exact zero
// encodes as 0x00 as f32_to_e4m3 does; callers keep |v| <= 448.
__device__ __forceinline__ uint32_t pack_e4m3x4(float v0, float v1, float v2, float v3) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v0 + 0.0f, v1 + 0.0f, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v2 + 0.0f, v3 + 0.0f, lo, true);
}

// Sixteen columns of one row of a row-lane 32x32 block as e4m3 codes, laid out as in
// pack_row16: lane l < 32 gets columns 0..7 and lane l + 32 columns 8..15 (8 bytes).
__device__ __forceinline__ uint2 pack_row8_e4m3(float v0, float v1, float v2, float v3, float v4, float v5,
                                               float v6, float v7) {
  const uint32_t a = pack_e4m3x4(v0, v1, v2, v3), b = pack_e4m3x4(v4, v5, v6, v7);
  const auto sw = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  return make_uint2(sw[0], sw[1]);
}

// ---- OCP 8-bit formats -----------------------------------------------------------------

// e8m0 byte of an fp32 power of two
__device__ __forceinline__ int pow2_to_e8m0(float s) { return (__float_as_uint(s) >> 23) & 0xff; }

// fp32 -> OCP e4m3fn code, round to nearest even; |v| <= 448 by construction of the scale.
// An exact zero (either sign) gives code 0.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sgn = (u >> 24) & 0x80u;
  const float a = __builtin_fabsf(v);
  if (a == 0.0f) return 0u;
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: subnormal grid of step 2^-9 (code 8 is 2^-6 itself)
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    const uint32_t m = u & 0x7fffffffu;
    const uint32_t r = (m + 0x7ffffu + ((m >> 20) & 1u)) >> 20;  // keep 3 mantissa bits, RNE
    code = r - ((127u - 7u) << 3);
    if (code > 0x7eu) code = 0x7eu;                               // saturate at 448
  }
  return sgn | code;
}

// Scale of a 1x128 block: the smallest power of two s with 448 s >= amax, at least 2^-127
// (the smallest e8m0 value, so pow2_to_e8m0 gives byte 0 for it and 1 / s = 2^127 stays
// finite); amax = 0 -> 1. With amax = m 2^ea, m in [0.5, 1) (frexp is exact, subnormals
// included) and 448 = 0.875 2^9: s = 2^(ea - 9) when m <= 0.875, else 2^(ea - 8). No division,
// so nothing underflows for tiny blocks; the exponent is clamped before ldexp, so s is exact.
__device__ __forceinline__ float fp8_pow2_scale(float amax) {
  if (!(amax > 0.f)) return 1.0f;
  int ea;
  const float m = __builtin_frexpf(amax, &ea);
  const int e = ea - 9 + (m > 0.875f ? 1 : 0);
  return __builtin_ldexpf(1.0f, e < -127 ? -127 : e);
}

// Wave-uniform broadcast from lane `src`.
__device__ __forceinline__ int wave_bcast(int v, int src) { return __shfl(v, src, MOE_WAVE); }

// Set of lanes in the wave whose `key` equals this lane's key (keys < 2^bits).
__device__ __forceinline__ uint64_t match_any(int key, int bits) {
  uint64_t m = __ballot(1);
  for (int b = 0; b < bits; ++b) {
    uint64_t ones = __ballot((key >> b) & 1);
    m &= ((key >> b) & 1) ? ones : ~ones;
  }
  return m;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Number of set bits of `m` below this lane.
__device__ __forceinline__ int popc_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

}  // namespace moe
