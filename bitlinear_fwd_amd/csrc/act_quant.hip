// Per-token absmax int8 activation quantiser.
//
// aratech.ae BitNet b1.58 article, "BitLinear: the building block": activations are
// quantised to int8 per token with an absmax scale that sends the largest magnitude of
// the row to 127.  Here a = max_k |x|, s = fl32(127/a), xq = clamp(rint(fl32(x*s)),
// -127, 127) with ties to even; an all-zero row gives zeros and a = 0.
//
// One workgroup per row (256 threads, or 1024 for rows longer than 8192 elements).  The
// row is read once from HBM into registers (up to kMaxVecPerThread groups of 8 elements
// per thread), reduced to its maximum, then quantised from registers and written as
// int8; rows longer than the registers hold re-read the rest, 16 bytes at a time.
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxVecPerThread = 4;  // groups of 8 elements held in registers per thread

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

template <int kTh>
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < kTh / 64; ++w) m = fmaxf(m, red[w]);
  return m;
}

// Group gi (8 consecutive elements) of row m, widened exactly to fp32.
template <bool kBf16>
__device__ __forceinline__ void load_group(const void* X, int64_t m, int64_t K, int64_t gi, float (&v)[8]) {
  if (kBf16) {
    const uint4 u = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(X) + m * K)[gi];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_to_f32(w[e] & 0xFFFFu);
      v[2 * e + 1] = bf16_to_f32(w[e] >> 16);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(X) + m * K) + 2 * gi;
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

__device__ __forceinline__ uint2 quant_group(const float (&v)[8], float s) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo |= (uint32_t)(uint8_t)quant_code(v[e], s) << (8 * e);
    hi |= (uint32_t)(uint8_t)quant_code(v[4 + e], s) << (8 * e);
  }
  return make_uint2(lo, hi);
}

// Vector path: 8 elements per 16-byte load (bf16) or 4 per 16-byte load (fp32, two
// loads per group of 8).  Requires K % 8 == 0 and a 16-byte aligned X; each group of 8
// elements produces one 8-byte store of codes.
template <bool kBf16, int kTh>
__global__ __launch_bounds__(kTh) void k_act_quant_vec(const void* __restrict__ X, int64_t K, int64_t K_pad,
                                                       int8_t* __restrict__ Xq, float* __restrict__ absmax) {
  __shared__ float red[kTh / 64];
  const int64_t m = blockIdx.x;
  const int64_t groups = K / 8;
  float v[kMaxVecPerThread][8];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxVecPerThread; ++j) {
    const int64_t gi = threadIdx.x + (int64_t)j * kTh;
    if (gi < groups) {
      load_group<kBf16>(X, m, K, gi, v[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[j][e]));
    }
  }
  for (int64_t gi = threadIdx.x + (int64_t)kMaxVecPerThread * kTh; gi < groups; gi += kTh) {
    float t[8];
    load_group<kBf16>(X, m, K, gi, t);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(t[e]));
  }
  const float a = block_max<kTh>(amax, red);
  const float s = a > 0.0f ? 127.0f / a : 0.0f;
  if (threadIdx.x == 0) absmax[m] = a;
  uint2* out = reinterpret_cast<uint2*>(Xq + m * K_pad);
#pragma unroll
  for (int j = 0; j < kMaxVecPerThread; ++j) {
    const int64_t gi = threadIdx.x + (int64_t)j * kTh;
    if (gi < groups) out[gi] = quant_group(v[j], s);
  }
  for (int64_t gi = threadIdx.x + (int64_t)kMaxVecPerThread * kTh; gi < groups; gi += kTh) {
    float t[8];
    load_group<kBf16>(X, m, K, gi, t);
    out[gi] = quant_group(t, s);
  }
  // zero padding columns K .. K_pad-1 (K is a multiple of 8 here, K_pad of 256)
  for (int64_t gi = groups + threadIdx.x; gi < K_pad / 8; gi += kTh) out[gi] = make_uint2(0u, 0u);
}

// Scalar path for any K and alignment.
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void k_act_quant_scalar(const void* __restrict__ X, int64_t K, int64_t K_pad,
                                                               int8_t* __restrict__ Xq, float* __restrict__ absmax) {
  __shared__ float red[kThreads / 64];
  const int64_t m = blockIdx.x;
  auto load = [&](int64_t k) -> float {
    return kBf16 ? bf16_to_f32(static_cast<const uint16_t*>(X)[m * K + k]) : static_cast<const float*>(X)[m * K + k];
  };
  float amax = 0.0f;
  for (int64_t k = threadIdx.x; k < K; k += kThreads) amax = fmaxf(amax, fabsf(load(k)));
  const float a = block_max<kThreads>(amax, red);
  const float s = a > 0.0f ? 127.0f / a : 0.0f;
  if (threadIdx.x == 0) absmax[m] = a;
  int8_t* out = Xq + m * K_pad;
  for (int64_t k = threadIdx.x; k < K_pad; k += kThreads) out[k] = k < K ? quant_code(load(k), s) : (int8_t)0;
}

}  // namespace

hipError_t launch_act_quant(const void* X, int bf16, int64_t M, int64_t K, int8_t* Xq, float* absmax,
                            hipStream_t s) {
  const int64_t K_pad = k_pad(K);
  const bool vec = (K % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15u) == 0);
  const dim3 grid((unsigned)M), block(kThreads);
  if (vec) {
    // rows beyond the registers of 256 threads take 1024
    const bool wide = K / 8 > (int64_t)kMaxVecPerThread * kThreads;
    const dim3 wblock(wide ? 1024 : kThreads);
    if (wide) {
      if (bf16) hipLaunchKernelGGL((k_act_quant_vec<true, 1024>), grid, wblock, 0, s, X, K, K_pad, Xq, absmax);
      else hipLaunchKernelGGL((k_act_quant_vec<false, 1024>), grid, wblock, 0, s, X, K, K_pad, Xq, absmax);
    } else {
      if (bf16) hipLaunchKernelGGL((k_act_quant_vec<true, kThreads>), grid, block, 0, s, X, K, K_pad, Xq, absmax);
      else hipLaunchKernelGGL((k_act_quant_vec<false, kThreads>), grid, block, 0, s, X, K, K_pad, Xq, absmax);
    }
  } else {
    if (bf16) hipLaunchKernelGGL(k_act_quant_scalar<true>, grid, block, 0, s, X, K, K_pad, Xq, absmax);
    else hipLaunchKernelGGL(k_act_quant_scalar<false>, grid, block, 0, s, X, K, K_pad, Xq, absmax);
  }
  return hipGetLastError();
}

}  // namespace bl
