// Prefill kernel (M > 16 tokens): a dense int8 x ternary contraction on the matrix
// cores.  The packed ternary tiles are decoded once per workgroup into LDS as int8 and
// fed, together with the int8 activations, to v_mfma_i32_16x16x64_i8; accumulation is
// exact int32 and the fp32 rescale (y = acc * gamma * a[m] / 127) is the epilogue.
//
// bhfrc.com news 56965, section 1.1 (ternary x activation = add / subtract / skip) and
// section 4.1 (2-bit codes); aratech.ae BitNet b1.58 article, "BitLinear".
//
// Workgroup tile 128 (tokens) x 128 (outputs), K step 128 (half a packed tile column):
// 256 threads = 4 waves in a 2 x 2 grid, each wave a 64 x 64 block of 4 x 4 MFMA tiles.
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int LDS_STRIDE = BK + 16;  // bytes per LDS row; the pad staggers 16-byte reads

__global__ __launch_bounds__(256) void k_gemm_mfma(const uint8_t* __restrict__ packed, const float* __restrict__ gamma,
                                                   const int8_t* __restrict__ Xq, const float* __restrict__ absmax,
                                                   int M, int N, int n_blocks, int K_pad, int chunks,
                                                   float* __restrict__ Y, int32_t* __restrict__ acc_out) {
  __shared__ __attribute__((aligned(16))) uint8_t As[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[BN * LDS_STRIDE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  v4i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4i){0, 0, 0, 0};

  for (int step = 0; step < 2 * chunks; ++step) {
    const int ch = step >> 1, half = step & 1;
    const int kbase = ch * kTileCols + half * BK;
    // A: 128 rows x 128 bytes = 1024 16-byte pieces, 4 per thread
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = tid + 256 * j;
      const int row = idx >> 3, piece = idx & 7;
      const int m = m0 + row;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (m < M) v = *reinterpret_cast<const uint4*>(Xq + (size_t)m * K_pad + kbase + 16 * piece);
      *reinterpret_cast<uint4*>(&As[row * LDS_STRIDE + 16 * piece]) = v;
    }
    // B: 8 row blocks x 32 slots (the half tile) = 256 slots, one per thread
    {
      const int nbl = tid >> 5, slot = 32 * half + (tid & 31);
      const int nb = n0 / kTileRows + nbl;
      uint4 wv = make_uint4(0u, 0u, 0u, 0u);  // code 00 decodes to 0
      if (nb < n_blocks) wv = reinterpret_cast<const uint4*>(packed + ((size_t)nb * chunks + ch) * kTileBytes)[slot];
      const int row = nbl * kTileRows + (slot & 15);
      const int col = 64 * ((slot >> 4) & 1);  // 64 columns per slot inside the half tile
      uint8_t* dst = &Bs[row * LDS_STRIDE + col];
      *reinterpret_cast<v4i*>(dst + 0) = decode16(wv.x);
      *reinterpret_cast<v4i*>(dst + 16) = decode16(wv.y);
      *reinterpret_cast<v4i*>(dst + 32) = decode16(wv.z);
      *reinterpret_cast<v4i*>(dst + 48) = decode16(wv.w);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK / 64; ++ks) {
      v4i a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const v4i*>(&As[(64 * wm + 16 * i + r) * LDS_STRIDE + 64 * ks + 16 * g]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const v4i*>(&Bs[(64 * wn + 16 * j + r) * LDS_STRIDE + 64 * ks + 16 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  const float gm = gamma[0];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + 64 * wm + 16 * i + 4 * g + v;
      if (m >= M) continue;
      const float sc = gm * absmax[m] * (1.0f / 127.0f);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + 64 * wn + 16 * j + r;
        if (n < N) {
          const int32_t a = acc[i][j][v];
          if (acc_out) acc_out[(size_t)m * N + n] = a;
          if (Y) Y[(size_t)m * N + n] = (float)a * sc;
        }
      }
    }
  }
}

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
  (void)K;
  GemmPlan p;
  p.bm = BM;
  p.bn = BN;
  p.threads = 256;
  p.groups = ((N + BN - 1) / BN) * ((M + BM - 1) / BM);
  return p;
}

hipError_t launch_gemm(const uint8_t* packed, const float* gamma, const int8_t* Xq, const float* absmax,
                       int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, hipStream_t s) {
  const int64_t K_pad = k_pad(K);
  const int chunks = (int)(K_pad / kTileCols);
  const int n_blocks = (int)(n_pad(N) / kTileRows);
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  hipLaunchKernelGGL(k_gemm_mfma, grid, dim3(256), 0, s, packed, gamma, Xq, absmax, (int)M, (int)N, n_blocks,
                     (int)K_pad, chunks, Y, acc);
  return hipGetLastError();
}

}  // namespace bl
