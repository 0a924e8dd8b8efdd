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
//
// kNorm adds the sub-layer normalisation that the same article places right before the
// quantiser (a simplified LayerNorm, taken as RMS normalisation with a per-feature gain
// g and an eps): n = x g / sqrt(mean(x^2) + eps).  The factor 1/sqrt(...) is positive
// and the same for the whole row, and absmax quantisation gives a row and any positive
// multiple of it the same codes, so the codes are decided on h = fl32(x g) exactly as
// above, and the factor only enters the scale written out: a = max|h| / sqrt(mean(x^2)
// + eps) = max|n|.  The sum of squares is accumulated in fp64 (each square is exact),
// so its summation order moves a by far less than one fp32 ulp.
//
// Optionally the row sum of the codes, sum_k xq[m][k], is written as an exact int32
// (|sum| <= 127 K): v_dot4 of each group's codes with ones, then an integer reduction.
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxVecPerThread = 4;  // groups of 8 elements held in registers per thread

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Row maximum of v over the workgroup; with kNorm also the row sum of ss (fp64, summed
// in wave order after the shuffles).
template <int kTh, bool kNorm>
__device__ __forceinline__ float block_max(float v, double& ss, float* red, double* red_ss) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  if constexpr (kNorm) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6] = v;
    if constexpr (kNorm) red_ss[threadIdx.x >> 6] = ss;
  }
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < kTh / 64; ++w) m = fmaxf(m, red[w]);
  if constexpr (kNorm) {
    ss = red_ss[0];
#pragma unroll
    for (int w = 1; w < kTh / 64; ++w) ss += red_ss[w];
  }
  return m;
}

// Scale written out by the normalising form: max|h| / sqrt(ss / K + eps), 0 for h = 0.
__device__ __forceinline__ float norm_scale(float amax_h, double ss, int64_t K, float eps) {
  return amax_h > 0.0f ? (float)((double)amax_h / sqrt(ss / (double)K + (double)eps)) : 0.0f;
}

// kNorm: accumulate the squares of x, then replace x by h = fl32(x * g) (g null: h = x).
template <bool kNorm>
__device__ __forceinline__ void norm_group(const float* __restrict__ gain, int64_t k0, float (&v)[8], double& ss) {
  if constexpr (kNorm) {
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fma((double)v[e], (double)v[e], ss);
    if (gain) {
      const float4 a = reinterpret_cast<const float4*>(gain + k0)[0];
      const float4 b = reinterpret_cast<const float4*>(gain + k0)[1];
      const float g[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = v[e] * g[e];
    }
  }
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
  return make_uint2(quant_code4(v[0], v[1], v[2], v[3], s), quant_code4(v[4], v[5], v[6], v[7], s));
}

// Sum of the eight int8 codes of a group (exact).
__device__ __forceinline__ int group_sum(uint2 q) {
  return __builtin_amdgcn_sdot4((int)q.y, 0x01010101, __builtin_amdgcn_sdot4((int)q.x, 0x01010101, 0, false), false);
}

// Row sum of the codes over the workgroup: shuffles, then the waves' partials in order.
template <int kTh>
__device__ __forceinline__ void block_rowsum(int v, int* red_i, int32_t* out) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  if ((threadIdx.x & 63) == 0) red_i[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
#pragma unroll
    for (int w = 0; w < kTh / 64; ++w) t += red_i[w];
    *out = t;
  }
}

// Vector path: 8 elements per 16-byte load (bf16) or 4 per 16-byte load (fp32, two
// loads per group of 8).  Requires K % 8 == 0, a 16-byte aligned X (and gain); each
// group of 8 elements produces one 8-byte store of codes.
template <bool kBf16, int kTh, bool kNorm>
__global__ __launch_bounds__(kTh) void k_act_quant_vec(const void* __restrict__ X, int64_t K, int64_t K_pad,
                                                       const float* __restrict__ gain, float eps,
                                                       int8_t* __restrict__ Xq, float* __restrict__ absmax,
                                                       int32_t* __restrict__ rowsum) {
  __shared__ float red[kTh / 64];
  __shared__ double red_ss[kNorm ? kTh / 64 : 1];
  __shared__ int red_i[kTh / 64];
  const int64_t m = blockIdx.x;
  const int64_t groups = K / 8;
  float v[kMaxVecPerThread][8];
  float amax = 0.0f;
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < kMaxVecPerThread; ++j) {
    const int64_t gi = threadIdx.x + (int64_t)j * kTh;
    if (gi < groups) {
      load_group<kBf16>(X, m, K, gi, v[j]);
      norm_group<kNorm>(gain, 8 * gi, v[j], ss);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[j][e]));
    }
  }
  for (int64_t gi = threadIdx.x + (int64_t)kMaxVecPerThread * kTh; gi < groups; gi += kTh) {
    float t[8];
    load_group<kBf16>(X, m, K, gi, t);
    norm_group<kNorm>(gain, 8 * gi, t, ss);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(t[e]));
  }
  const float a = block_max<kTh, kNorm>(amax, ss, red, red_ss);
  const float s = a > 0.0f ? 127.0f / a : 0.0f;
  if (threadIdx.x == 0) absmax[m] = kNorm ? norm_scale(a, ss, K, eps) : a;
  uint2* out = reinterpret_cast<uint2*>(Xq + m * K_pad);
  int rs = 0;
#pragma unroll
  for (int j = 0; j < kMaxVecPerThread; ++j) {
    const int64_t gi = threadIdx.x + (int64_t)j * kTh;
    if (gi < groups) {
      const uint2 q = quant_group(v[j], s);
      out[gi] = q;
      rs += group_sum(q);
    }
  }
  for (int64_t gi = threadIdx.x + (int64_t)kMaxVecPerThread * kTh; gi < groups; gi += kTh) {
    float t[8];
    double unused = 0.0;
    load_group<kBf16>(X, m, K, gi, t);
    norm_group<kNorm>(gain, 8 * gi, t, unused);
    const uint2 q = quant_group(t, s);
    out[gi] = q;
    rs += group_sum(q);
  }
  // zero padding columns K .. K_pad-1 (K is a multiple of 8 here, K_pad of 256)
  for (int64_t gi = groups + threadIdx.x; gi < K_pad / 8; gi += kTh) out[gi] = make_uint2(0u, 0u);
  if (rowsum) block_rowsum<kTh>(rs, red_i, rowsum + m);
}

// Scalar path for any K and alignment.
template <bool kBf16, bool kNorm>
__global__ __launch_bounds__(kThreads) void k_act_quant_scalar(const void* __restrict__ X, int64_t K, int64_t K_pad,
                                                               const float* __restrict__ gain, float eps,
                                                               int8_t* __restrict__ Xq, float* __restrict__ absmax,
                                                               int32_t* __restrict__ rowsum) {
  __shared__ float red[kThreads / 64];
  __shared__ double red_ss[kNorm ? kThreads / 64 : 1];
  __shared__ int red_i[kThreads / 64];
  const int64_t m = blockIdx.x;
  auto load = [&](int64_t k) -> float {
    return kBf16 ? bf16_to_f32(static_cast<const uint16_t*>(X)[m * K + k]) : static_cast<const float*>(X)[m * K + k];
  };
  auto h_of = [&](float x, int64_t k) -> float { return kNorm && gain ? x * gain[k] : x; };
  float amax = 0.0f;
  double ss = 0.0;
  for (int64_t k = threadIdx.x; k < K; k += kThreads) {
    const float x = load(k);
    if constexpr (kNorm) ss = fma((double)x, (double)x, ss);
    amax = fmaxf(amax, fabsf(h_of(x, k)));
  }
  const float a = block_max<kThreads, kNorm>(amax, ss, red, red_ss);
  const float s = a > 0.0f ? 127.0f / a : 0.0f;
  if (threadIdx.x == 0) absmax[m] = kNorm ? norm_scale(a, ss, K, eps) : a;
  int8_t* out = Xq + m * K_pad;
  int rs = 0;
  for (int64_t k = threadIdx.x; k < K_pad; k += kThreads) {
    const int8_t q = k < K ? quant_code(h_of(load(k), k), s) : (int8_t)0;
    out[k] = q;
    rs += q;
  }
  if (rowsum) block_rowsum<kThreads>(rs, red_i, rowsum + m);
}

template <bool kNorm>
void launch_rows(const void* X, int bf16, int64_t M, int64_t K, const float* gain, float eps, int8_t* Xq,
                 float* absmax, int32_t* rowsum, hipStream_t s) {
  const int64_t K_pad = k_pad(K);
  const bool vec = (K % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15u) == 0) &&
                   ((reinterpret_cast<uintptr_t>(gain) & 15u) == 0);
  const dim3 grid((unsigned)M), block(kThreads);
  if (vec) {
    // rows beyond the registers of 256 threads take 1024
    const bool wide = K / 8 > (int64_t)kMaxVecPerThread * kThreads;
    const dim3 wblock(wide ? 1024 : kThreads);
    if (wide) {
      if (bf16) hipLaunchKernelGGL((k_act_quant_vec<true, 1024, kNorm>), grid, wblock, 0, s, X, K, K_pad, gain, eps, Xq, absmax, rowsum);
      else hipLaunchKernelGGL((k_act_quant_vec<false, 1024, kNorm>), grid, wblock, 0, s, X, K, K_pad, gain, eps, Xq, absmax, rowsum);
    } else {
      if (bf16) hipLaunchKernelGGL((k_act_quant_vec<true, kThreads, kNorm>), grid, block, 0, s, X, K, K_pad, gain, eps, Xq, absmax, rowsum);
      else hipLaunchKernelGGL((k_act_quant_vec<false, kThreads, kNorm>), grid, block, 0, s, X, K, K_pad, gain, eps, Xq, absmax, rowsum);
    }
  } else {
    if (bf16) hipLaunchKernelGGL((k_act_quant_scalar<true, kNorm>), grid, block, 0, s, X, K, K_pad, gain, eps, Xq, absmax, rowsum);
    else hipLaunchKernelGGL((k_act_quant_scalar<false, kNorm>), grid, block, 0, s, X, K, K_pad, gain, eps, Xq, absmax, rowsum);
  }
}

}  // namespace

hipError_t launch_act_quant(const void* X, int bf16, int64_t M, int64_t K, int8_t* Xq, float* absmax,
                            hipStream_t s, int32_t* rowsum) {
  launch_rows<false>(X, bf16, M, K, nullptr, 0.0f, Xq, absmax, rowsum, s);
  return hipGetLastError();
}

hipError_t launch_subln_quant(const void* X, int bf16, int64_t M, int64_t K, const float* gain, float eps,
                              int8_t* Xq, float* scale, hipStream_t s) {
  launch_rows<true>(X, bf16, M, K, gain, eps, Xq, scale, nullptr, s);
  return hipGetLastError();
}

}  // namespace bl
