// Combine: deterministic weighted gather-reduce back to token order.
//
// "Distributed expert parallelism", lifecycle item 8 and "A four-rank example": restore
// the original token index, multiply by the route weights and add the k results (the
// results are added, not overwritten -- "Duplicate route accumulation"). "Mixture of
// Kittens", Step 8 "Full Determinism": the sum runs in a fixed order (k = 0..K-1, fp32
// FMA) and is rounded once, so the output is bitwise reproducible.
//
// One block per token; each thread owns 16-byte column chunks and keeps the K row loads
// of two chunks in flight together; the routed rows are read with non-temporal loads. HBM-bound: M*H*b read + T*H*b written. An optional addend
// row per token (the shared expert's output: "Mixture of Kittens", Step 1, MoE(x) =
// SharedExpert(x) + the weighted routed sum) is added after the k sum, before the rounding.
#include <algorithm>

#include "moe_common.h"

namespace moe {

__device__ __forceinline__ void load8(const uint16_t* p, float* f) {
  const int4 v = *reinterpret_cast<const int4*>(p);
  const uint32_t w[4] = {(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* f) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
// The routed rows are read once: non-temporal loads, so they stream past the caches instead of
// displacing lines that are still in use (combine 212 -> 187-192 us at T=8192, K=8, H=7168).
// Raw 16-byte words (eight bf16 or four fp32) are held until their FMAs: the loads of several
// rows then go out together without unpacked copies in registers.
template <typename YT>
struct Raw8 {
  i32x4_t q[sizeof(YT) / 2];
};
template <typename YT>
__device__ __forceinline__ Raw8<YT> load8_nt(const YT* p) {
  Raw8<YT> r;
#pragma unroll
  for (int j = 0; j < (int)(sizeof(YT) / 2); ++j)
    r.q[j] = __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(p) + j);
  return r;
}
__device__ __forceinline__ void unpack8(const Raw8<uint16_t>& r, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float((uint32_t)r.q[0][i] << 16);
    f[2 * i + 1] = __uint_as_float((uint32_t)r.q[0][i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack8(const Raw8<float>& r, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = __int_as_float(r.q[0][i]);
    f[4 + i] = __int_as_float(r.q[1][i]);
  }
}
__device__ __forceinline__ void store8(uint16_t* p, const float* f) {
  int4 v;
  v.x = (int)pack_bf16x2(f[0], f[1]);
  v.y = (int)pack_bf16x2(f[2], f[3]);
  v.z = (int)pack_bf16x2(f[4], f[5]);
  v.w = (int)pack_bf16x2(f[6], f[7]);
  *reinterpret_cast<int4*>(p) = v;
}
__device__ __forceinline__ void store8(float* p, const float* f) {
  reinterpret_cast<float4*>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
}

// NU: chunks per thread and pass. Two measured best at H = 7168 (three and four were no
// faster). The block has about H / 16 threads (a multiple of 64, at most 512), so one pass
// covers a whole row at H = 7168 (448 threads).
template <typename YT, typename OT, int KMAX, int NU = 2>
__global__ __launch_bounds__(512) void combine_kernel(const YT* __restrict__ y_rows,
                                                      const int* __restrict__ pos,
                                                      const float* __restrict__ topk_w, int T,
                                                      int H, int K, const YT* __restrict__ add,
                                                      OT* __restrict__ out) {
  constexpr int KG = KMAX < 8 ? KMAX : 8;   // rows whose loads go out together
  const int t = blockIdx.x;
  int p[KMAX];
  float w[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    p[k] = k < K ? pos[(size_t)t * K + k] : -1;
    w[k] = k < K ? (topk_w ? topk_w[(size_t)t * K + k] : 1.0f) : 0.f;  // NULL: unit weights
  }
  const int nchunk = H / 8;
  const int B = blockDim.x;
  // NU chunks per thread and pass; the loads of KG rows x NU chunks are issued before their
  // FMAs, which then run in k order
  int c = threadIdx.x;
  for (; c + (NU - 1) * B < nchunk; c += NU * B) {
    float acc[NU][8];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
#pragma unroll
    for (int k0 = 0; k0 < KMAX; k0 += KG) {
      Raw8<YT> v[KG][NU];
#pragma unroll
      for (int k = 0; k < KG; ++k)
        if (p[k0 + k] >= 0)
#pragma unroll
          for (int u = 0; u < NU; ++u) v[k][u] = load8_nt(y_rows + (size_t)p[k0 + k] * H + (c + u * B) * 8);
#pragma unroll
      for (int k = 0; k < KG; ++k)
        if (p[k0 + k] >= 0)
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            float f[8];
            unpack8(v[k][u], f);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[u][i] = fmaf(w[k0 + k], f[i], acc[u][i]);
          }
    }
    if (add) {
      float v[NU][8];
#pragma unroll
      for (int u = 0; u < NU; ++u) load8(add + (size_t)t * H + (c + u * B) * 8, v[u]);
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] += v[u][i];
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) store8(out + (size_t)t * H + (c + u * B) * 8, acc[u]);
  }
  for (; c < nchunk; c += B) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < KMAX; k0 += KG) {
      Raw8<YT> v[KG];
#pragma unroll
      for (int k = 0; k < KG; ++k)
        if (p[k0 + k] >= 0) v[k] = load8_nt(y_rows + (size_t)p[k0 + k] * H + c * 8);
#pragma unroll
      for (int k = 0; k < KG; ++k)
        if (p[k0 + k] >= 0) {
          float f[8];
          unpack8(v[k], f);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(w[k0 + k], f[i], acc[i]);
        }
    }
    if (add) {
      float v[8];
      load8(add + (size_t)t * H + c * 8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    store8(out + (size_t)t * H + c * 8, acc);
  }
}

// Scalar fallback for H not a multiple of 8.
template <typename YT, typename OT>
__global__ __launch_bounds__(128) void combine_scalar_kernel(const YT* __restrict__ y_rows,
                                                             const int* __restrict__ pos,
                                                             const float* __restrict__ topk_w,
                                                             int T, int H, int K,
                                                             const YT* __restrict__ add,
                                                             OT* __restrict__ out) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x; c < H; c += blockDim.x) {
    float acc = 0.f;
    for (int k = 0; k < K; ++k) {
      const int p = pos[(size_t)t * K + k];
      if (p < 0) continue;
      float v;
      if constexpr (sizeof(YT) == 2)
        v = bf16_bits_to_f32(y_rows[(size_t)p * H + c]);
      else
        v = y_rows[(size_t)p * H + c];
      acc = fmaf(topk_w ? topk_w[(size_t)t * K + k] : 1.0f, v, acc);
    }
    if (add) {
      if constexpr (sizeof(YT) == 2)
        acc += bf16_bits_to_f32(add[(size_t)t * H + c]);
      else
        acc += add[(size_t)t * H + c];
    }
    if constexpr (sizeof(OT) == 2)
      out[(size_t)t * H + c] = f32_to_bf16_bits(acc);
    else
      out[(size_t)t * H + c] = acc;
  }
}

template <typename YT, typename OT>
static moe_status_t dispatch_combine(const void* y, const int* pos, const float* w, int T, int H,
                                     int K, const void* add, void* out, hipStream_t s) {
  const YT* yr = static_cast<const YT*>(y);
  const YT* ad = static_cast<const YT*>(add);
  OT* o = static_cast<OT*>(out);
  const bool vec = (H % 8 == 0) && ((uintptr_t)y % 16 == 0) && ((uintptr_t)out % 16 == 0) &&
                   ((uintptr_t)add % 16 == 0);
  // threads: two 16-byte chunks each per pass, whole waves, 64 .. 512
  const int nchunk = H / 8;
  const int nb = std::min(512, std::max(64, ((nchunk + 1) / 2 + 63) / 64 * 64));
  if (!vec) {
    combine_scalar_kernel<YT, OT><<<T, 128, 0, s>>>(yr, pos, w, T, H, K, ad, o);
  } else if (K <= 2) {
    combine_kernel<YT, OT, 2><<<T, nb, 0, s>>>(yr, pos, w, T, H, K, ad, o);
  } else if (K <= 4) {
    combine_kernel<YT, OT, 4><<<T, nb, 0, s>>>(yr, pos, w, T, H, K, ad, o);
  } else if (K <= 8) {
    combine_kernel<YT, OT, 8><<<T, nb, 0, s>>>(yr, pos, w, T, H, K, ad, o);
  } else if (K <= 16) {
    combine_kernel<YT, OT, 16><<<T, nb, 0, s>>>(yr, pos, w, T, H, K, ad, o);
  } else {
    combine_kernel<YT, OT, 32><<<T, nb, 0, s>>>(yr, pos, w, T, H, K, ad, o);
  }
  return launch_status();
}

moe_status_t launch_combine(const void* y, moe_dtype_t yt, const int* pos, const float* w, int T,
                            int H, int K, const void* add, void* out, moe_dtype_t ot, hipStream_t s) {
  if (T == 0 || H == 0) return MOE_OK;
  if (yt == MOE_BF16 && ot == MOE_BF16) return dispatch_combine<uint16_t, uint16_t>(y, pos, w, T, H, K, add, out, s);
  if (yt == MOE_BF16 && ot == MOE_F32) return dispatch_combine<uint16_t, float>(y, pos, w, T, H, K, add, out, s);
  if (yt == MOE_F32 && ot == MOE_F32) return dispatch_combine<float, float>(y, pos, w, T, H, K, add, out, s);
  if (yt == MOE_F32 && ot == MOE_BF16) return dispatch_combine<float, uint16_t>(y, pos, w, T, H, K, add, out, s);
  return MOE_EUNSUPPORTED;
}

// ---- fp32 accumulator of the fused scatter-add combine --------------------------------
// (the down projection adds row_w * y of every row into acc[token] with fp32 atomics; the
// accumulator starts at zero and is rounded once into the output format at the end)

__global__ __launch_bounds__(256) void acc_zero_kernel(float* __restrict__ acc, size_t n) {
  const size_t n4 = n / 4;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    reinterpret_cast<float4*>(acc)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (size_t i = n4 * 4 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) acc[i] = 0.f;
}

// out = round(acc + add): add (nullable) has the format of y (bf16 or fp32); out may alias
// acc when both are fp32.
template <typename AT, typename OT>
__global__ __launch_bounds__(256) void acc_store_kernel(const float* acc, const AT* __restrict__ add,
                                                        OT* out, size_t n) {
  const size_t n8 = n / 8;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    float f[8];
    load8(acc + 8 * i, f);
    if (add) {
      float a[8];
      load8(add + 8 * i, a);
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] += a[j];
    }
    store8(out + 8 * i, f);
  }
  for (size_t i = n8 * 8 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    float v = acc[i];
    if (add) {
      if constexpr (sizeof(AT) == 2)
        v += bf16_bits_to_f32(add[i]);
      else
        v += add[i];
    }
    if constexpr (sizeof(OT) == 2)
      out[i] = f32_to_bf16_bits(v);
    else
      out[i] = v;
  }
}

static int stream_grid(size_t items) {
  const size_t cap = (size_t)device_cu_count() * 8;
  const size_t need = (items + 255) / 256;
  return (int)(need < cap ? (need > 0 ? need : 1) : cap);
}

moe_status_t launch_acc_zero(float* acc, size_t n, hipStream_t s) {
  if (n == 0) return MOE_OK;
  if ((uintptr_t)acc % 16) return MOE_EINVAL;
  acc_zero_kernel<<<stream_grid(n / 4), 256, 0, s>>>(acc, n);
  return launch_status();
}

// Byte fill: the debug poison of a workspace and the clearing of an error word. A kernel
// rather than hipMemsetAsync, so that a stream captured into a HIP graph records no memset
// node.
__global__ __launch_bounds__(256) void fill_bytes_kernel(unsigned char* __restrict__ p, size_t n,
                                                         unsigned char v) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t head = (16 - (uintptr_t)p % 16) % 16 < n ? (16 - (uintptr_t)p % 16) % 16 : n;
  const size_t n16 = (n - head) / 16;
  const uint32_t w = 0x01010101u * v;
  uint4* q = reinterpret_cast<uint4*>(p + head);
  for (size_t i = i0; i < n16; i += stride) q[i] = make_uint4(w, w, w, w);
  for (size_t i = i0; i < head; i += stride) p[i] = v;
  for (size_t i = head + n16 * 16 + i0; i < n; i += stride) p[i] = v;
}

moe_status_t launch_fill_bytes(void* p, size_t n, unsigned char v, hipStream_t s) {
  if (n == 0) return MOE_OK;
  fill_bytes_kernel<<<stream_grid(n / 16 + 1), 256, 0, s>>>(static_cast<unsigned char*>(p), n, v);
  return launch_status();
}

moe_status_t launch_acc_store(const float* acc, size_t n, const void* add, moe_dtype_t add_dtype,
                              void* out, moe_dtype_t ot, hipStream_t s) {
  if (n == 0) return MOE_OK;
  if ((uintptr_t)acc % 16 || (uintptr_t)out % 16 || (uintptr_t)add % 16) return MOE_EINVAL;
  const int g = stream_grid(n / 8);
  if (ot == MOE_BF16 && add_dtype == MOE_BF16)
    acc_store_kernel<uint16_t, uint16_t><<<g, 256, 0, s>>>(acc, static_cast<const uint16_t*>(add),
                                                           static_cast<uint16_t*>(out), n);
  else if (ot == MOE_F32 && add_dtype == MOE_F32)
    acc_store_kernel<float, float><<<g, 256, 0, s>>>(acc, static_cast<const float*>(add),
                                                     static_cast<float*>(out), n);
  else
    return MOE_EUNSUPPORTED;
  return launch_status();
}

// cu_seqlens of one group holding all T rows (the shared expert run as a one-group launch)
__global__ void dense_cu_kernel(int* cu, int T) {
  if (threadIdx.x == 0) {
    cu[0] = 0;
    cu[1] = T;
  }
}

moe_status_t launch_dense_cu(int* cu, int T, hipStream_t s) {
  dense_cu_kernel<<<1, 64, 0, s>>>(cu, T);
  return launch_status();
}

}  // namespace moe
