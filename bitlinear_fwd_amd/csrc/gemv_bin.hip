// 1-bit sign-binary decode (one to four tokens, int8 activations): the contrast point to
// the ternary path.  lpnh.cn news 2861808, section 2.1 binarises the weights with sign()
// and a magnitude-compensating scale; here q = +1 for W >= 0, -1 for W < 0, scale beta =
// mean |W|, and the same per-token int8 activations, exact int32 contraction and fp32
// rescale y = acc * beta * a / 127.  One bit per weight halves the packed bytes.
//
// Layout (binary.h): 1024-byte tiles of 16 rows x 512 columns; lane (r, g) of a tile load
// holds row r, and word j covers column group g of the 256-column half s = j / 2, steps
// i = 2 (j % 2) and 2 (j % 2) + 1, column e of step i at bit 8 (e % 4) + 4 (i % 2) + e / 4.
// So the four bytes of MFMA operand dword d of step i are bit f = 4 (i % 2) + d of the
// word's four bytes: (word >> f) & 0x03030303 selects, through v_perm_b32, 0xFF (bit 0,
// -1) or 0x01 (bit 1, +1) from the bytes {FF, 01, FF, 01} (the neighbouring bit f + 1 only
// picks between equal bytes).  Three VALU per four weights, straight into the B operand of
// v_mfma_i32_16x16x64_i8.
//
// Structure as the register-run decode kernel: a workgroup owns one 16-row block, wave w
// a run of T binary tiles (2 T halves of 256 columns) with all of its weight loads issued
// at once; activation pieces stay in registers and reach the A operand through DPP.
#include "binary.h"
#include "decode_common.h"

#include <algorithm>

namespace bl {
namespace {

// MFMA B operand of step i (0..3 within a 256-column half) from the half's word pair.
__device__ __forceinline__ v4i decode_bin16(uint32_t word, int f0) {
  v4i b;
  b.x = (int)__builtin_amdgcn_perm(0u, 0x01FF01FFu, (word >> f0) & 0x03030303u);
  b.y = (int)__builtin_amdgcn_perm(0u, 0x01FF01FFu, (word >> (f0 + 1)) & 0x03030303u);
  b.z = (int)__builtin_amdgcn_perm(0u, 0x01FF01FFu, (word >> (f0 + 2)) & 0x03030303u);
  b.w = (int)__builtin_amdgcn_perm(0u, 0x01FF01FFu, (word >> (f0 + 3)) & 0x03030303u);
  return b;
}

template <int T, int MM>
__global__ __launch_bounds__(1024) void k_gemv_bin(const uint8_t* __restrict__ packed, const float* __restrict__ beta,
                                                   const int8_t* __restrict__ Xq, const float* __restrict__ absmax,
                                                   int M, int N, int K_pad, int chunks_b, float* __restrict__ Y,
                                                   int32_t* __restrict__ acc_out) {
  static_assert(MM >= 1 && MM <= 4, "one to four tokens");
  constexpr int UA = 16 / (4 * MM);  // 256-column halves per activation piece
  constexpr int TS = 2 * T;          // halves per wave run
  constexpr int NA = (TS + UA - 1) / UA;
  __shared__ v4i red[16 * 64];
  const int W = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int c0 = wave * T;
  const int rb0 = blockIdx.x;
  const int pm = r % MM, pq = r / MM;
  const int pu = min(pq / 4, UA - 1), pi = pq % 4;

  // activation pieces: lane (r, g) holds token r % MM, step (r / MM) % 4 of half
  // 2 c0 + j UA + r / (4 MM); halves past the activation row (K_pad) are zero
  uint4 act[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int col = (2 * c0 + j * UA + pu) * 256 + 64 * g + 16 * pi;
    act[j] = col < K_pad ? *reinterpret_cast<const uint4*>(Xq + (size_t)pm * K_pad + col) : make_uint4(0u, 0u, 0u, 0u);
  }
  const uint4* wsrc = reinterpret_cast<const uint4*>(packed) + (size_t)rb0 * chunks_b * 64 + lane;
  uint4 w[T];
  static_for<T>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    w[t] = load_nt(wsrc + (size_t)min(c0 + t, chunks_b - 1) * 64);
  });
  __builtin_amdgcn_sched_barrier(0);

  v4i c = {0, 0, 0, 0};
  static_for<NA>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    static_for<UA>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      constexpr int hl = j * UA + u;  // half within the run
      if constexpr (hl < TS) {
        constexpr int t = hl / 2, s = hl % 2;
        const bool live = c0 + t < chunks_b;  // tiles past the matrix contribute nothing
        static_for<4>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          constexpr int sft = MM * (4 * u + i);
          v4i av;
          if constexpr (MM == 1) {
            const uint64_t lo = row_bcast64<sft>((uint64_t)act[j].x | ((uint64_t)act[j].y << 32));
            const uint64_t hi = row_bcast64<sft>((uint64_t)act[j].z | ((uint64_t)act[j].w << 32));
            av.x = (int)(uint32_t)lo;
            av.y = (int)(uint32_t)(lo >> 32);
            av.z = (int)(uint32_t)hi;
            av.w = (int)(uint32_t)(hi >> 32);
          } else {
            av.x = row_shl<sft>((int)act[j].x);
            av.y = row_shl<sft>((int)act[j].y);
            av.z = row_shl<sft>((int)act[j].z);
            av.w = row_shl<sft>((int)act[j].w);
          }
          v4i bv = decode_bin16(word_of(w[t], 2 * s + i / 2), 4 * (i % 2));
          if (!live) bv = (v4i){0, 0, 0, 0};
          c = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, c, 0, 0, 0);
        });
      }
    });
  });

  red[wave * 64 + lane] = c;
  __syncthreads();
  if (wave == 0) {
    v4i sum = red[lane];
    for (int w2 = 1; w2 < W; ++w2) sum += red[w2 * 64 + lane];
    const int n = rb0 * kTileRows + r;
    if (n < N) {
      const float bt = beta[0];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * g + v;
        if (m < M) {
          if (acc_out) acc_out[(size_t)m * N + n] = sum[v];
          if (Y) Y[(size_t)m * N + n] = (float)sum[v] * bt * absmax[m] * (1.0f / 127.0f);
        }
      }
    }
  }
}

template <int T>
hipError_t launch_bin_m(const BinPlan& p, int M, const uint8_t* packed, const float* beta, const int8_t* Xq,
                        const float* absmax, int N, int K_pad, int chunks_b, float* Y, int32_t* acc, hipStream_t s) {
  const dim3 grid((unsigned)p.groups), block(p.waves * 64);
  switch (M) {
    case 1: hipLaunchKernelGGL((k_gemv_bin<T, 1>), grid, block, 0, s, packed, beta, Xq, absmax, M, N, K_pad, chunks_b, Y, acc); break;
    case 2: hipLaunchKernelGGL((k_gemv_bin<T, 2>), grid, block, 0, s, packed, beta, Xq, absmax, M, N, K_pad, chunks_b, Y, acc); break;
    case 3: hipLaunchKernelGGL((k_gemv_bin<T, 3>), grid, block, 0, s, packed, beta, Xq, absmax, M, N, K_pad, chunks_b, Y, acc); break;
    default: hipLaunchKernelGGL((k_gemv_bin<T, 4>), grid, block, 0, s, packed, beta, Xq, absmax, M, N, K_pad, chunks_b, Y, acc); break;
  }
  return hipGetLastError();
}

}  // namespace

BinPlan plan_gemv_bin(int64_t M, int64_t N, int64_t K) {
  BinPlan p;
  if (M < 1 || M > 4) return p;
  const int64_t chunks_b = kb_pad(K) / kBinTileCols;
  const int64_t rblocks = n_pad(N) / kTileRows;
  // as the ternary register-run kernel: about 32 waves per compute unit, at least two
  // tiles per wave, then the shortest run (at most 8 tiles) that covers the row with at
  // most 16 waves
  int64_t w = std::min<int64_t>(16, std::max<int64_t>(1, 8192 / rblocks));
  w = std::min<int64_t>(w, std::max<int64_t>(1, (chunks_b + 1) / 2));
  const int64_t t = (chunks_b + w - 1) / w;
  if (t > 8) return p;
  p.run = (int)t;
  p.waves = (int)((chunks_b + t - 1) / t);
  p.groups = rblocks;
  p.ok = p.waves <= 16 && p.groups <= (int64_t(1) << 30);
  return p;
}

hipError_t launch_gemv_bin(const uint8_t* packed, const float* beta, const int8_t* Xq, const float* absmax, int64_t M,
                           int64_t N, int64_t K, float* Y, int32_t* acc, hipStream_t s) {
  const BinPlan p = plan_gemv_bin(M, N, K);
  if (!p.ok) return hipErrorInvalidConfiguration;
  const int K_pad = (int)k_pad(K), chunks_b = (int)(kb_pad(K) / kBinTileCols);
  switch (p.run) {
    case 1: return launch_bin_m<1>(p, (int)M, packed, beta, Xq, absmax, (int)N, K_pad, chunks_b, Y, acc, s);
    case 2: return launch_bin_m<2>(p, (int)M, packed, beta, Xq, absmax, (int)N, K_pad, chunks_b, Y, acc, s);
    case 3: return launch_bin_m<3>(p, (int)M, packed, beta, Xq, absmax, (int)N, K_pad, chunks_b, Y, acc, s);
    case 4: return launch_bin_m<4>(p, (int)M, packed, beta, Xq, absmax, (int)N, K_pad, chunks_b, Y, acc, s);
    case 5: return launch_bin_m<5>(p, (int)M, packed, beta, Xq, absmax, (int)N, K_pad, chunks_b, Y, acc, s);
    case 6: return launch_bin_m<6>(p, (int)M, packed, beta, Xq, absmax, (int)N, K_pad, chunks_b, Y, acc, s);
    case 7: return launch_bin_m<7>(p, (int)M, packed, beta, Xq, absmax, (int)N, K_pad, chunks_b, Y, acc, s);
    default: return launch_bin_m<8>(p, (int)M, packed, beta, Xq, absmax, (int)N, K_pad, chunks_b, Y, acc, s);
  }
}

}  // namespace bl
