// Table-lookup decode (one to four tokens): the CPU technique of the bitnet.cpp-style
// kernels (T-MAC lookup tables), rebuilt for gfx950 LDS as a point of comparison with the
// matrix-core decode kernel.
//
// The 2-bit packed layout puts codes of columns c and c + 4 in one nibble (byte b of word
// i holds columns 16 i + 4 f + b at bits 2 f .. 2 f + 1; a nibble is f = 2 h, 2 h + 1).  For
// each such pair of activations (x0, x1) a 16-entry table holds w(lo) x0 + w(hi) x1 for
// every nibble value (lo = nib & 3, hi = nib >> 2, w = {0, +1, -1, 0} per the code table
// 00 -> 0, 01 -> +1, 10 -> -1, 11 -> padding), as int16.  A weight byte then costs two
// lookups and two integer adds instead of a decode and a multiply; the sums are exact.
//
// Structure: a workgroup owns one 16-row block; wave w owns a run of T K tiles and builds
// the tables of exactly those columns in its own slice of LDS (4352 B per tile per token),
// so no cross-wave barrier stands before the lookups.  Every weight load of the run is
// issued before the tables are built.  Lane (r, g) of a tile looks up row r's 64 codes of
// column group g; the partial sums are reduced over g by shuffles and over the waves in
// LDS, then rescaled as in the other decode kernels.
#include "gemv_lut.h"
#include "decode_common.h"

#include <atomic>

namespace bl {
namespace {

constexpr int kPairBytes = 32;  // 16 int16 entries
// A 16-column block holds 8 pair tables (256 B) plus 16 B of padding: the lanes of column
// group g read block 4 g + i, so the four groups' tables sit 1088 B apart, which puts them
// in four different 16-bank ranges instead of on the same banks.
constexpr int kBlockBytes = 8 * kPairBytes + 16;
constexpr int kTileTableBytes = 16 * kBlockBytes;  // 16 blocks per 256-column tile

__device__ __forceinline__ int sbyte(uint32_t word, int b) { return (int)(int8_t)(word >> (8 * b)); }

// The 16 entries of the pair (x0, x1) as 8 words of two int16: entry n = w(n & 3) x0 +
// w(n >> 2) x1.
__device__ __forceinline__ void pair_table(int x0, int x1, uint32_t (&e)[8]) {
  const int a[4] = {0, x0, -x0, 0};
  const int bv[4] = {0, x1, -x1, 0};
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const int hi = d >> 1, lo = 2 * (d & 1);
    const int v0 = a[lo] + bv[hi], v1 = a[lo + 1] + bv[hi];
    e[d] = ((uint32_t)v0 & 0xFFFFu) | ((uint32_t)v1 << 16);
  }
}

template <int T, int MM>
__global__ __launch_bounds__(1024) void k_gemv_lut(const uint8_t* __restrict__ packed,
                                                   const float* __restrict__ gamma, const int8_t* __restrict__ Xq,
                                                   const float* __restrict__ absmax, int M, int N, int K_pad,
                                                   int chunks, float* __restrict__ Y, int32_t* __restrict__ acc_out) {
  extern __shared__ uint4 lut_lds[];
  __shared__ int32_t red[16][4][16];  // [wave][token][row]
  const int W = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int c0 = wave * T;
  const int rb0 = blockIdx.x;
  uint8_t* tab = reinterpret_cast<uint8_t*>(lut_lds) + (size_t)wave * T * MM * kTileTableBytes;

  // activation blocks of 16 columns, (token m, tile t, block q = 4 g + i): 16 T MM per wave
  constexpr int kBlocks = 16 * T * MM;
  constexpr int kPer = (kBlocks + 63) / 64;
  uint4 xa[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int blk = lane + 64 * j;
    xa[j] = make_uint4(0u, 0u, 0u, 0u);
    if (blk < kBlocks) {
      const int m = blk / (16 * T), t = (blk / 16) % T, q = blk % 16;
      const int tile = min(c0 + t, chunks - 1);  // a clamped tile is never read: its codes are zeroed below
      xa[j] = *reinterpret_cast<const uint4*>(Xq + (size_t)min(m, M - 1) * K_pad + tile * kTileCols + 16 * q);
    }
  }
  const uint4* wsrc = reinterpret_cast<const uint4*>(packed) + (size_t)rb0 * chunks * 64 + lane;
  uint4 w[T];
  static_for<T>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    w[t] = load_nt(wsrc + (size_t)min(c0 + t, chunks - 1) * 64);
  });

  // tables: block (m, t, q) = (m T + t) 16 + q holds the pairs (h, b), h = 0, 1 and b = 0..3,
  // at block * kBlockBytes + (4 h + b) * kPairBytes
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int blk = lane + 64 * j;
    if (blk < kBlocks) {
      const uint32_t xw[4] = {xa[j].x, xa[j].y, xa[j].z, xa[j].w};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          // columns 8 h + b and 8 h + b + 4 of the block
          const int e0 = 8 * h + b, e1 = e0 + 4;
          uint32_t e[8];
          pair_table(sbyte(xw[e0 >> 2], e0 & 3), sbyte(xw[e1 >> 2], e1 & 3), e);
          uint4* dst = reinterpret_cast<uint4*>(tab + (size_t)blk * kBlockBytes + (4 * h + b) * kPairBytes);
          dst[0] = make_uint4(e[0], e[1], e[2], e[3]);
          dst[1] = make_uint4(e[4], e[5], e[6], e[7]);
        }
      }
    }
  }
  // the tables are this wave's own: LDS operations of one wave complete in order, so only
  // the compiler has to keep the lookups after the stores
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  int acc[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) acc[m] = 0;
  static_for<T>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    const bool live = c0 + t < chunks;  // tiles past the matrix contribute nothing
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t word = live ? word_of(w[t], i) : 0u;  // nibble 0 looks up entry 0 = 0
      const uint8_t* base = tab + (size_t)(t * 16 + 4 * g + i) * kBlockBytes;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t nib = (word >> (8 * b + 4 * h)) & 0xFu;
          const uint8_t* p = base + (4 * h + b) * kPairBytes + 2 * nib;
#pragma unroll
          for (int m = 0; m < MM; ++m)
            acc[m] += *reinterpret_cast<const int16_t*>(p + (size_t)m * T * kTileTableBytes);
        }
      }
    }
  });
#pragma unroll
  for (int m = 0; m < MM; ++m) {
    acc[m] += __shfl_xor(acc[m], 16, 64);
    acc[m] += __shfl_xor(acc[m], 32, 64);
    if (g == 0) red[wave][m][r] = acc[m];
  }
  __syncthreads();
  if (wave == 0 && lane < 16 * MM) {
    const int m = lane >> 4, rr = lane & 15;
    int32_t sum = 0;
    for (int w2 = 0; w2 < W; ++w2) sum += red[w2][m][rr];
    const int n = rb0 * kTileRows + rr;
    if (n < N && m < M) {
      if (acc_out) acc_out[(size_t)m * N + n] = sum;
      if (Y) Y[(size_t)m * N + n] = (float)sum * gamma[0] * absmax[m] * (1.0f / 127.0f);
    }
  }
}

constexpr int kLutRuns[] = {1, 2, 3, 4, 5, 6, 7, 8};

template <int T, int MM>
hipError_t launch_lut(const LutPlan& p, const uint8_t* packed, const float* gamma, const int8_t* Xq,
                      const float* absmax, int M, int N, int K_pad, int chunks, float* Y, int32_t* acc,
                      hipStream_t s) {
  auto kern = k_gemv_lut<T, MM>;
  // per instantiation and device: allow dynamic LDS beyond 64 KiB (set once; a repeated
  // set from a concurrent first call is harmless)
  static std::atomic<uint64_t> raised{0};
  if (p.lds_bytes > 64 * 1024) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = uint64_t(1) << (dev & 63);
    if (!(raised.load(std::memory_order_relaxed) & bit)) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kMaxLutBytes);
      if (e != hipSuccess) return e;
      raised.fetch_or(bit, std::memory_order_relaxed);
    }
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)p.groups), dim3(p.waves * 64), (unsigned)p.lds_bytes, s, packed, gamma, Xq,
                     absmax, M, N, K_pad, chunks, Y, acc);
  return hipGetLastError();
}

template <int T>
hipError_t launch_lut_m(const LutPlan& p, int M, const uint8_t* packed, const float* gamma, const int8_t* Xq,
                        const float* absmax, int N, int K_pad, int chunks, float* Y, int32_t* acc, hipStream_t s) {
  switch (M) {
    case 1: return launch_lut<T, 1>(p, packed, gamma, Xq, absmax, M, N, K_pad, chunks, Y, acc, s);
    case 2: return launch_lut<T, 2>(p, packed, gamma, Xq, absmax, M, N, K_pad, chunks, Y, acc, s);
    case 3: return launch_lut<T, 3>(p, packed, gamma, Xq, absmax, M, N, K_pad, chunks, Y, acc, s);
    default: return launch_lut<T, 4>(p, packed, gamma, Xq, absmax, M, N, K_pad, chunks, Y, acc, s);
  }
}

}  // namespace

LutPlan plan_gemv_lut(int64_t M, int64_t N, int64_t K) {
  LutPlan p;
  const int64_t chunks = k_pad(K) / kTileCols;
  if (M < 1 || M > 4) return p;
  // at most 16 waves, each with a run of at most 8 tiles; about two tiles per wave
  int64_t w = std::min<int64_t>(16, std::max<int64_t>(1, (chunks + 1) / 2));
  int64_t t = (chunks + w - 1) / w;
  if (t > 8) return p;
  for (int r : kLutRuns)
    if (r >= t) {
      t = r;
      break;
    }
  w = (chunks + t - 1) / t;
  p.run = (int)t;
  p.waves = (int)w;
  p.groups = n_pad(N) / kTileRows;
  p.lds_bytes = w * t * M * kTileTableBytes;
  p.ok = p.lds_bytes <= kMaxLutBytes && p.groups <= (int64_t(1) << 30);
  return p;
}

hipError_t launch_gemv_lut(const uint8_t* packed, const float* gamma, const int8_t* Xq, const float* absmax,
                           int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, hipStream_t s) {
  const LutPlan p = plan_gemv_lut(M, N, K);
  if (!p.ok) return hipErrorInvalidConfiguration;
  const int K_pad = (int)k_pad(K), chunks = K_pad / kTileCols;
  switch (p.run) {
    case 1: return launch_lut_m<1>(p, (int)M, packed, gamma, Xq, absmax, (int)N, K_pad, chunks, Y, acc, s);
    case 2: return launch_lut_m<2>(p, (int)M, packed, gamma, Xq, absmax, (int)N, K_pad, chunks, Y, acc, s);
    case 3: return launch_lut_m<3>(p, (int)M, packed, gamma, Xq, absmax, (int)N, K_pad, chunks, Y, acc, s);
    case 4: return launch_lut_m<4>(p, (int)M, packed, gamma, Xq, absmax, (int)N, K_pad, chunks, Y, acc, s);
    case 5: return launch_lut_m<5>(p, (int)M, packed, gamma, Xq, absmax, (int)N, K_pad, chunks, Y, acc, s);
    case 6: return launch_lut_m<6>(p, (int)M, packed, gamma, Xq, absmax, (int)N, K_pad, chunks, Y, acc, s);
    case 7: return launch_lut_m<7>(p, (int)M, packed, gamma, Xq, absmax, (int)N, K_pad, chunks, Y, acc, s);
    default: return launch_lut_m<8>(p, (int)M, packed, gamma, Xq, absmax, (int)N, K_pad, chunks, Y, acc, s);
  }
}

}  // namespace bl
