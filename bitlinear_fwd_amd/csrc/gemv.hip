// Decode kernel (M = 1..16 tokens): packed-ternary x int8 with exact int32 accumulation
// and the fp32 rescale in the epilogue.
//
// bhfrc.com news 56965, section 1.1: a ternary weight times an activation adds it,
// subtracts it or skips it; section 4.1: the weights travel as 2-bit codes so that one
// load carries many of them.  aratech.ae BitNet b1.58 article, "BitLinear": y is the
// int8 x ternary product rescaled by both scales.
//
// The decode regime is HBM-bound (0.25 byte of weights per multiply-add at M = 1), so
// the kernel is built around streaming the packed matrix once:
//   * a workgroup owns one 16-row block of outputs; its waves split the 1 KiB tiles of
//     that block along K, so every wave-wide 16-byte-per-lane load is one contiguous
//     tile;
//   * each lane's 16 bytes are 64 consecutive codes of one row, decoded in registers
//     (decode16) straight into the B operand of v_mfma_i32_16x16x64_i8; the A operand
//     is the matching 16 int8 activations of token lane%16 (zero for lanes >= M), so
//     the matrix core does the dot products and the VALU only decodes;
//   * partial 16x16 int32 tiles of the waves are summed through LDS (exact), and the
//     first wave rescales and stores.
#include "bl_internal.h"

namespace bl {
namespace {

template <int kWaves, int kUnroll>
__global__ __launch_bounds__(kWaves * 64) void k_gemv_mfma(const uint8_t* __restrict__ packed,
                                                            const float* __restrict__ gamma,
                                                            const int8_t* __restrict__ Xq,
                                                            const float* __restrict__ absmax, int M, int N,
                                                            int K_pad, int chunks, float* __restrict__ Y,
                                                            int32_t* __restrict__ acc_out) {
  __shared__ v4i red[kWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int nb = blockIdx.x;
  const uint4* wp = reinterpret_cast<const uint4*>(packed + (size_t)nb * chunks * kTileBytes) + lane;
  const bool has_row = r < M;
  const int8_t* xrow = Xq + (size_t)(has_row ? r : 0) * K_pad + 64 * g;
  v4i c = {0, 0, 0, 0};
  int ch = wave;
  for (; ch + (kUnroll - 1) * kWaves < chunks; ch += kUnroll * kWaves) {
    uint4 wv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) wv[u] = wp[(size_t)(ch + u * kWaves) * 64];
    uint4 av[kUnroll][4];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (has_row) {
        const uint4* ap = reinterpret_cast<const uint4*>(xrow + (size_t)(ch + u * kWaves) * kTileCols);
#pragma unroll
        for (int i = 0; i < 4; ++i) av[u][i] = ap[i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) av[u][i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      c = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(av[u][0]), decode16(wv[u].x), c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(av[u][1]), decode16(wv[u].y), c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(av[u][2]), decode16(wv[u].z), c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(av[u][3]), decode16(wv[u].w), c, 0, 0, 0);
    }
  }
  for (; ch < chunks; ch += kWaves) {
    const uint4 wv = wp[(size_t)ch * 64];
    uint4 av[4];
    if (has_row) {
      const uint4* ap = reinterpret_cast<const uint4*>(xrow + (size_t)ch * kTileCols);
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = ap[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(av[0]), decode16(wv.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(av[1]), decode16(wv.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(av[2]), decode16(wv.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(av[3]), decode16(wv.w), c, 0, 0, 0);
  }
  if (kWaves > 1) {
    red[wave][lane] = c;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 1; w < kWaves; ++w) c += red[w][lane];
  }
  // lane holds D[4*g + v][r] for v = 0..3: token m = 4g + v, output n = 16*nb + r
  const int n = nb * kTileRows + r;
  if (n >= N) return;
  const float gm = gamma[0];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * g + v;
    if (m < M) {
      const int32_t a = c[v];
      if (acc_out) acc_out[(size_t)m * N + n] = a;
      if (Y) Y[(size_t)m * N + n] = (float)a * gm * absmax[m] * (1.0f / 127.0f);
    }
  }
}

}  // namespace

hipError_t launch_gemv(const uint8_t* packed, const float* gamma, const int8_t* Xq, const float* absmax,
                       int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, hipStream_t s) {
  const int64_t K_pad = k_pad(K);
  const int chunks = (int)(K_pad / kTileCols);
  const unsigned blocks = (unsigned)(n_pad(N) / kTileRows);
  hipLaunchKernelGGL((k_gemv_mfma<4, 2>), dim3(blocks), dim3(256), 0, s, packed, gamma, Xq, absmax, (int)M,
                     (int)N, (int)K_pad, chunks, Y, acc);
  return hipGetLastError();
}

}  // namespace bl
