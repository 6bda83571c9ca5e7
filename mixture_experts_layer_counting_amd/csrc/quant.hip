// Activation quantisation to OCP e4m3fn with one power-of-two scale per 1x128 block of a
// row ("Mixture of Kittens", Step 8: activations are quantised before the fp8 GEMMs, the
// quantisation fused into dispatch). Scale s = smallest power of two with 448 s >= block
// amax (amax = 0 -> 1); code = round-to-nearest-even(v / s). Because s is a power of two,
// v / s is exact in fp32 and the codes do not depend on evaluation order.
//
// Layout: x [R, C] (bf16 or fp32, C % 128 == 0) -> q [R, C] codes, sf [R, C/128] fp32.
// 16 lanes per block, 8 elements per lane (one 16-byte bf16 load or two fp32 loads); a wave
// covers four blocks. HBM-bound: R*C*(2 or 4) bytes read, R*C + R*C/32 bytes written.
#include "moe_common.h"

namespace moe {

template <typename XT>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const XT* __restrict__ x, size_t nblk,
                                                           int bpr, uint8_t* __restrict__ q,
                                                           float* __restrict__ sf) {
  const size_t g = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;  // block index
  const int l = threadIdx.x & 15;
  const bool live = g < nblk;
  const size_t b = live ? g : 0;
  const size_t row = b / bpr, cb = b % bpr;
  const size_t off = (row * bpr + cb) * 128 + l * 8;
  float v[8];
  if constexpr (sizeof(XT) == 2) {
    const int4 w = *reinterpret_cast<const int4*>(x + off);
    const uint32_t u[4] = {(uint32_t)w.x, (uint32_t)w.y, (uint32_t)w.z, (uint32_t)w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  } else {
    const float4 a = reinterpret_cast<const float4*>(x + off)[0];
    const float4 c = reinterpret_cast<const float4*>(x + off)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, __builtin_fabsf(v[i]));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  const float s = fp8_pow2_scale(m);
  const float inv = 1.0f / s;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= f32_to_e4m3(v[i] * inv) << (8 * i);
    hi |= f32_to_e4m3(v[4 + i] * inv) << (8 * i);
  }
  if (live) {
    *reinterpret_cast<uint2*>(q + off) = make_uint2(lo, hi);
    if (l == 0) sf[b] = s;
  }
}

moe_status_t launch_quantize_fp8(const void* x, moe_dtype_t xt, int R, int C, void* q, float* sf,
                                 hipStream_t s) {
  if (R == 0) return MOE_OK;
  const size_t nblk = (size_t)R * (C / 128);
  const size_t threads = nblk * 16;
  const int grid = (int)((threads + 255) / 256);
  if (xt == MOE_BF16)
    quantize_fp8_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(x), nblk, C / 128,
                                                       static_cast<uint8_t*>(q), sf);
  else if (xt == MOE_F32)
    quantize_fp8_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(x), nblk, C / 128,
                                                    static_cast<uint8_t*>(q), sf);
  else
    return MOE_EUNSUPPORTED;
  return launch_status();
}

// MXFP4 weight codes from the stored layout [E][N][K/2] (each column's K/2 bytes contiguous)
// to the paired layout [E][N/2][K/128][2][64]: for every pair of columns (2p, 2p+1) and every
// step of 128 reduction elements, the two columns' 64-byte runs side by side, so that one
// 128-byte line holds what the fp8 x MXFP4 kernels stage for both columns in one K step (the
// MoonEP news article, "Design principles and technical details": the weights are laid out
// for the GEMM). The scale bytes keep their layout. A thread per 16 output bytes; a plain
// HBM-bound copy, run once per weight tensor.
__global__ __launch_bounds__(256) void pack_mxfp4_pairs_kernel(const uint8_t* __restrict__ w,
                                                               uint8_t* __restrict__ out, size_t n16,
                                                               size_t per_e, int K) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < n16; q += stride) {
    const size_t o = q * 16;
    const size_t e = o / per_e, r = o % per_e;
    const size_t p = r / K, r2 = r % K;          // column pair, then [K/128][2][64] within it
    const size_t st = r2 / 128, r3 = r2 % 128;   // K step, then [2][64]
    const size_t hcol = r3 / 64, b = r3 % 64;     // which column of the pair, byte in its run
    const size_t src = e * per_e + (2 * p + hcol) * (size_t)(K / 2) + st * 64 + b;
    *reinterpret_cast<uint4*>(out + o) = *reinterpret_cast<const uint4*>(w + src);
  }
}

moe_status_t launch_pack_mxfp4_pairs(const void* w, void* out, int E, int N, int K, hipStream_t s) {
  const size_t per_e = (size_t)N * (K / 2);
  const size_t n16 = (size_t)E * per_e / 16;
  if (n16 == 0) return MOE_OK;
  const size_t want = (n16 + 255) / 256;
  const int grid = (int)(want < 8192 ? want : 8192);
  pack_mxfp4_pairs_kernel<<<grid, 256, 0, s>>>(static_cast<const uint8_t*>(w), static_cast<uint8_t*>(out),
                                               n16, per_e, K);
  return launch_status();
}

}  // namespace moe
