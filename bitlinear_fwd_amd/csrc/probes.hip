// Measurement probes: the ceilings the benchmark sets the BitLinear kernels against.
//
//   k_probe_stream  reads a buffer with the decode kernels' access pattern (1 KiB tiles,
//                   16 bytes per lane, non-temporal, every load of a wave's 8-tile run
//                   issued at once) and does nothing else with it: the HBM read ceiling
//                   for that pattern at a given size.  Each workgroup (4 waves, 32 KiB)
//                   stores the XOR of the 32-bit words it read, so the result is checkable.
//   k_probe_read    a plain grid-stride read of a buffer, 16 bytes per lane, 8 loads in
//                   flight per lane, as many workgroups as the caller asks for: the HBM
//                   read ceiling of a launch of that size with no access pattern of the
//                   BitLinear kernels.  Each workgroup stores the XOR of the words it read.
//   k_probe_mfma    independent v_mfma_i32_16x16x64_i8 back to back, no memory traffic:
//                   the int8 matrix-core ceiling.
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kStreamRun = 8;         // tiles per wave
constexpr int kStreamWaves = 4;       // waves per workgroup
constexpr int kMfmaChains = 16;       // independent accumulators per wave
constexpr int kReadUnroll = 8;        // loads in flight per lane in the plain read

__device__ __forceinline__ uint32_t xor4(const uint4& v) { return v.x ^ v.y ^ v.z ^ v.w; }

template <bool kNonTemporal>
__device__ __forceinline__ uint4 read16(const uint4* p) {
  if constexpr (kNonTemporal)
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p)));
  else
    return *p;
}

// Lane i of the grid reads 16-byte words i, i + S, i + 2S, ... (S = 256 x workgroups), eight
// at a time; the loop bound keeps every access below n16.
template <bool kNonTemporal>
__global__ __launch_bounds__(256) void k_probe_read(const uint4* __restrict__ buf, int64_t n16,
                                                    uint32_t* __restrict__ out) {
  __shared__ uint32_t red[4];
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = read16<kNonTemporal>(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) x ^= xor4(v[u]);
  }
  for (; i < n16; i += stride) x ^= xor4(read16<kNonTemporal>(buf + i));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(kStreamWaves * 64) void k_probe_stream(const uint4* __restrict__ buf, int64_t tiles,
                                                                    uint32_t* __restrict__ out) {
  __shared__ uint32_t red[kStreamWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t t0 = ((int64_t)blockIdx.x * kStreamWaves + wave) * kStreamRun;
  uint4 v[kStreamRun];
#pragma unroll
  for (int t = 0; t < kStreamRun; ++t) {
    const int64_t tile = min(t0 + t, tiles - 1);  // past the end: re-read the last tile, not counted
    v[t] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4i*>(buf + tile * 64 + lane)));
  }
  uint32_t x = 0;
#pragma unroll
  for (int t = 0; t < kStreamRun; ++t)
    if (t0 + t < tiles) x ^= v[t].x ^ v[t].y ^ v[t].z ^ v[t].w;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off, 64);
  if (lane == 0) red[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(256) void k_probe_mfma(int64_t iters, uint32_t* __restrict__ out) {
  // operands like the prefill kernel's: int8 activations against ternary {-1, 0, +1} bytes
  const uint32_t h = (threadIdx.x + 1) * 0x9E3779B1u ^ blockIdx.x * 0x85EBCA6Bu;
  const v4i a = {(int)h, (int)(h * 0x27D4EB2Fu), (int)(h ^ 0x5A3C96E1u), (int)(h * 0x165667B1u)};
  const v4i b = {0x01FF0001, 0x00FF01FF, 0x01000100, (int)0xFF0001FF};
  v4i c[kMfmaChains];
#pragma unroll
  for (int i = 0; i < kMfmaChains; ++i) c[i] = (v4i){i, 0, 0, 0};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kMfmaChains; ++i) c[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c[i], 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int i = 0; i < kMfmaChains; ++i) s ^= c[i].x ^ c[i].y ^ c[i].z ^ c[i].w;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s ^= __shfl_xor(s, off, 64);
  if (threadIdx.x == 0) out[blockIdx.x] = (uint32_t)s;
}

}  // namespace

int64_t probe_stream_groups(int64_t bytes) {
  const int64_t tiles = bytes / kTileBytes;
  const int64_t per_group = (int64_t)kStreamWaves * kStreamRun;
  return (tiles + per_group - 1) / per_group;
}

hipError_t launch_probe_stream(const void* buf, int64_t bytes, uint32_t* out, hipStream_t s) {
  const int64_t tiles = bytes / kTileBytes;
  hipLaunchKernelGGL(k_probe_stream, dim3((unsigned)probe_stream_groups(bytes)), dim3(kStreamWaves * 64), 0, s,
                     static_cast<const uint4*>(buf), tiles, out);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* buf, int64_t bytes, int64_t groups, bool nontemporal, uint32_t* out,
                             hipStream_t s) {
  const auto* p = static_cast<const uint4*>(buf);
  if (nontemporal)
    hipLaunchKernelGGL(k_probe_read<true>, dim3((unsigned)groups), dim3(256), 0, s, p, bytes / 16, out);
  else
    hipLaunchKernelGGL(k_probe_read<false>, dim3((unsigned)groups), dim3(256), 0, s, p, bytes / 16, out);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int64_t iters, int64_t groups, uint32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_probe_mfma, dim3((unsigned)groups), dim3(256), 0, s, iters, out);
  return hipGetLastError();
}

}  // namespace bl
