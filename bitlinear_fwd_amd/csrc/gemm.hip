// Prefill kernel (M > 16 tokens): a dense int8 x ternary contraction on the matrix cores,
// exact int32 accumulation and the fp32 rescale (y = acc * gamma * a[m] / 127) in the
// epilogue.
//
// bhfrc.com news 56965, section 1.1 (ternary x activation = add / subtract / skip) and
// section 4.1 (2-bit codes); aratech.ae BitNet b1.58 article, "BitLinear".
//
// Structure (workgroup = 4 waves in a GM x GN grid, each wave a WM x WN block of 16 x 16
// v_mfma_i32_16x16x64_i8 tiles; K advances half a 256-column packed chunk per stage):
//   * activations (A): each half-stage's BM x 128-byte slab (the pieces two MFMA steps
//     use) goes straight from global memory into LDS (direct global -> LDS loads, no
//     registers) through a ring of D slabs, so D - 1 half-stages are in flight while
//     one computes; the wait at the end of a half-stage counts only the loads still
//     allowed to be outstanding, and one barrier per half-stage hands the slab over;
//   * weights (B): every wave loads its own 16-byte slots of the packed tiles (a 1 KiB
//     tile is one coalesced wave load) into a register ring of the same depth and
//     decodes them straight into the B operand - the packed layout is the MFMA lane
//     layout, and 2-bit codes are 4x fewer bytes through the cache than int8;
//   * one 16-byte word of a slot feeds one MFMA step and serves WM / 16 MFMAs, which
//     keeps the decode VALU below the matrix-core time;
//   * shapes: 64 x 256 or 64 x 192 output tiles (waves 1 x 4 of 64 x 64 or 64 x 48,
//     three-slot ring), whichever leaves the lighter last round of tiles, and two K groups
//     of four waves per tile where there are few tiles (plan_gemm);
//   * the loop body is unrolled over lcm(D, 2 CB) half-stages so that every ring index is
//     static; half-stages past the end of K are skipped whole (measured: 2048 x 6912 x 2560
//     48.9 -> 46.9 us, 4096 x 6912 x 2560 87.6 -> 82.3 us, 48 x 30000 x 512 9.4 -> 7.6 us),
//     and the loop ends by waiting for every load still in flight;
//   * tile order is XCD-aware: consecutive workgroup ids go to different XCDs, so each
//     XCD gets a contiguous run of output tiles (sharing activation rows in its L2).
#include "bl_internal.h"

#include <numeric>

namespace bl {
namespace {

// Activation staging.  MFMA step i of a 256-column chunk uses, in lane group g, the
// 16-byte piece 4g + i of each activation row (columns 64g + 16i .. +15), so steps
// {2h, 2h+1} need only the 8 pieces 4g + 2h + i' (g = 0..3, i' = 0..1): a half-stage.
// A half-stage slab is BM rows x 128 bytes in LDS; row r keeps its local piece
// lp = 2g + i' in slot lp ^ ((r >> 1) & 7), which puts the 16 lanes of a fragment read
// (16 consecutive rows, one piece) on 16 distinct 16-byte bank groups.  One direct-load
// wave instruction fills 1 KiB of LDS contiguously (lane i at +16 i), i.e. 8 rows; the
// swizzle is applied by choosing which global piece each lane fetches.
__device__ __forceinline__ int a_slot(int row, int lp) { return lp ^ ((row >> 1) & 7); }

// s_waitcnt that waits only for vmcnt <= n (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// Work-group barrier for the LDS ring.  Unlike __syncthreads() it carries no release
// fence, so it does not drain the direct global->LDS loads still in flight for later ring
// slots; the caller has already waited (wait_vmcnt) for the slot the next half-stage reads.
// The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Vector-memory instructions a wave issues in half-stage hs: the activation slab, plus
// the weight slots of a chunk at its first half-stage.
template <int kDma, int NB>
constexpr int loads_at(int hs) { return kDma + ((hs & 1) == 0 ? NB : 0); }

// Number of loads issued in half-stages (a, b] (a < b), for the ring wait counts.
template <int kDma, int NB>
constexpr int loads_between(int a, int b) {
  int n = 0;
  for (int h = a + 1; h <= b; ++h) n += loads_at<kDma, NB>(h);
  return n;
}

template <int GM, int GN, int WM, int WN, int D, int KS = 1>
__global__ __launch_bounds__(256 * KS) void k_gemm_mfma(const uint8_t* __restrict__ packed, const float* __restrict__ gamma,
                                                   const int8_t* __restrict__ Xq, const float* __restrict__ absmax,
                                                   int M, int N, int n_blocks, int K_pad, int chunks, int tiles_m,
                                                   int tiles_n, float* __restrict__ Y, int32_t* __restrict__ acc_out) {
  static_assert(GM * GN == 4, "four waves");
  static_assert(D >= 2, "at least two ring slots");
  static_assert(KS == 1 || KS == 2, "one or two K groups");
  constexpr int BM = GM * WM, BN = GN * WN;
  constexpr int MB = WM / 16, NB = WN / 16;
  constexpr int kHalf = kTileCols / 2;        // bytes per activation row in a half-stage
  constexpr int kDma = BM / 32;               // direct loads per wave per half-stage (8 rows each, 4 waves)
  constexpr int P = D - 1;                    // prefetch distance in half-stages
  constexpr int CB = (P + 1) / 2 + 1;         // weight register ring (chunks live at once)
  constexpr int kBody = std::lcm(D, 2 * CB);  // half-stages per trip: both ring indices static
  constexpr int kSlab = BM * kHalf;           // one K group's slab of a ring slot
  static_assert(KS == 1 || (MB % 2 == 0 && 4 * NB * 64 * 16 <= KS * kSlab), "K-group exchange fits a ring slot");
  // one LDS object per ring slot: distinct objects let the compiler see that the direct
  // loads into one slot do not alias reads of another (otherwise it waits for all of them)
  __shared__ __attribute__((aligned(1024))) uint8_t As0[KS * kSlab];
  __shared__ __attribute__((aligned(1024))) uint8_t As1[KS * kSlab];
  __shared__ __attribute__((aligned(1024))) uint8_t As2[D > 2 ? KS * kSlab : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t As3[D > 3 ? KS * kSlab : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t As4[D > 4 ? KS * kSlab : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t As5[D > 5 ? KS * kSlab : 16];
  static_assert(D <= 6, "ring of at most 6 slots");
  auto slab = [&](auto sc) -> uint8_t* {
    constexpr int sl = decltype(sc)::value;
    if constexpr (sl == 0) return As0;
    else if constexpr (sl == 1) return As1;
    else if constexpr (sl == 2) return As2;
    else if constexpr (sl == 3) return As3;
    else if constexpr (sl == 4) return As4;
    else return As5;
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave = KS == 1 ? wave_all : wave_all & 3;  // wave within its K group
  const int kg = KS == 1 ? 0 : wave_all >> 2;            // K group
  const int kgoff = kg * kSlab;                          // the group's half of each ring slot
  const int r = lane & 15, g = lane >> 4;
  const int wm = wave / GN, wn = wave % GN;

  // XCD-aware tile order: workgroup b runs on XCD b % 8; give XCD x the x-th contiguous
  // run of tiles in row-major (m, n) order
  const int tiles = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int per_xcd = (tiles + 7) / 8;
  const int full = tiles - 8 * (per_xcd - 1);  // XCDs holding per_xcd tiles (the rest hold one fewer)
  const int t = xcd < full ? xcd * per_xcd + slot : full * per_xcd + (xcd - full) * (per_xcd - 1) + slot;
  if (slot >= (xcd < full ? per_xcd : per_xcd - 1)) return;
  const int m0 = (t / tiles_n) * BM, n0 = (t % tiles_n) * BN;
  // K group kg takes chunks [c_lo, c_hi).  Both groups run the same number of half-stages
  // (they share the barriers); where the chunks do not split evenly the second group skips
  // the compute of its last ones and its loads repeat a valid chunk.
  const int cg = (chunks + KS - 1) / KS;
  const int c_lo = kg * cg, c_hi = min(chunks, c_lo + cg);
  const int hstages = 2 * cg;                                       // loop length, both groups
  const int hs_mine = KS == 1 ? hstages : 2 * max(c_hi - c_lo, 0);  // half-stages this group computes
  auto chunk_of = [&](int h) {
    if constexpr (KS == 1) return min(h, hstages - 1) >> 1;
    else return min(c_lo + (min(h, hstages - 1) >> 1), chunks - 1);
  };

  // this lane's source for each direct load: row 8 (4 j + wave) + lane / 8, LDS slot
  // lane % 8 holding local piece lp = slot ^ swizzle, global piece 4 (lp >> 1) + 2h + (lp & 1)
  // (rows past M repeat row M-1: their outputs are never stored)
  const int8_t* asrc[kDma];
#pragma unroll
  for (int j = 0; j < kDma; ++j) {
    const int row = 8 * (4 * j + wave) + (lane >> 3);
    const int lp = a_slot(row, lane & 7);
    asrc[j] = Xq + (size_t)min(m0 + row, M - 1) * K_pad + 16 * (4 * (lp >> 1) + (lp & 1));
  }
  // weight slots of this wave's NB row blocks (blocks past the matrix re-read the last
  // block: their outputs are never stored)
  const uint4* bsrc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int nb = min(n0 / kTileRows + wn * NB + j, n_blocks - 1);
    bsrc[j] = reinterpret_cast<const uint4*>(packed) + (size_t)nb * chunks * 64 + lane;
  }
  uint4 bw[CB][NB];

  v4i acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = (v4i){0, 0, 0, 0};

  // compute half-stage in ring slot s (steps 2h, 2h+1 of its chunk) with weights cb
  auto compute = [&](auto sc, int half, const uint4 (&wcur)[NB]) {
    const uint8_t* slabp = slab(sc) + kgoff;
#pragma unroll
    for (int ip = 0; ip < 2; ++ip) {
      const int i = 2 * half + ip;
      v4i bf[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const uint32_t word = i == 0 ? wcur[j].x : (i == 1 ? wcur[j].y : (i == 2 ? wcur[j].z : wcur[j].w));
        bf[j] = decode16(word);
      }
#pragma unroll
      for (int mi = 0; mi < MB; ++mi) {
        const int row = wm * WM + 16 * mi + r;
        const v4i af = *reinterpret_cast<const v4i*>(&slabp[row * kHalf + 16 * a_slot(row, 2 * g + ip)]);
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[mi][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf[j], acc[mi][j], 0, 0, 0);
      }
    }
  };

  // Ring: half-stage hs computes LDS slot hs % D and refills slot (hs + P) % D (last read
  // at hs - 1); the weights of chunk c live in register slot c % CB from half-stage 2c - P
  // (issue) to 2c + 1 (last use).  The loop body covers D half-stages, so every slot
  // index below is a compile-time constant.
  // Prologue: half-stages 0 .. P-1.
  static_for<P>([&](auto hc) {
    constexpr int hs = decltype(hc)::value;
    const int c = chunk_of(hs);
    uint8_t* dst = slab(std::integral_constant<int, hs>{}) + kgoff;
#pragma unroll
    for (int j = 0; j < kDma; ++j)
      load_g2lds16(asrc[j] + (size_t)c * kTileCols + 32 * (min(hs, hstages - 1) & 1), &dst[8 * (4 * j + wave) * kHalf]);
    if constexpr ((hs & 1) == 0) {
#pragma unroll
      for (int j = 0; j < NB; ++j) bw[(hs / 2) % CB][j] = bsrc[j][(size_t)c * 64];
    }
    __builtin_amdgcn_sched_barrier(0);
  });
  wait_vmcnt<loads_between<kDma, NB>(0, P - 1)>();  // half-stage 0 has landed
  ring_barrier();
  // a do-while (there is always at least one chunk): a loop the compiler may skip lets it
  // sink the prologue's weight loads below the barrier, which breaks the wait counts
  int base = 0;
  do {
    static_for<kBody>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      const int hs = base + k;
      const int nh = hs + P;  // half-stage to issue
      // past the last half-stage: nothing left to compute or wait for (the body covers
      // lcm(D, 2 CB) half-stages, up to 12, whatever the K length).  Uniform across the
      // workgroup; the waits of the half-stages that run count the same loads as before.
      if (hs >= hstages) return;
      {
        const int hc = min(nh, hstages - 1);
        const int c = chunk_of(nh);
        uint8_t* dst = slab(std::integral_constant<int, (k + P) % D>{}) + kgoff;
#pragma unroll
        for (int j = 0; j < kDma; ++j)
          load_g2lds16(asrc[j] + (size_t)c * kTileCols + 32 * (hc & 1), &dst[8 * (4 * j + wave) * kHalf]);
        if constexpr (((k + P) & 1) == 0) {
#pragma unroll
          for (int j = 0; j < NB; ++j) bw[((k + P) / 2) % CB][j] = bsrc[j][(size_t)c * 64];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (hs < hs_mine) compute(std::integral_constant<int, k % D>{}, k & 1, bw[(k / 2) % CB]);
      // half-stage hs + 1 has landed: loads issued after it are those of hs + 2 .. hs + P
      wait_vmcnt<loads_between<kDma, NB>(k + 1, k + P)>();
      ring_barrier();
    });
    base += kBody;
  } while (base < hstages);
  // the refills of the last P half-stages (clamped re-reads of the last chunk, never
  // computed) land before the epilogue reuses registers and the workgroup ends
  wait_vmcnt<0>();

  const float gm = gamma[0];
  // store row block mi of the wave's tile, adding `other` (the other K group's partial of
  // the same row block, lane-major per column block)
  auto store_block = [&](auto mc, const v4i* other) {
    constexpr int mi = decltype(mc)::value;
    v4i part[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) part[j] = other[j * 64];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + wm * WM + 16 * mi + 4 * g + v;
      if (m >= M) continue;
      const float sc = gm * absmax[m] * (1.0f / 127.0f);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = n0 + wn * WN + 16 * j + r;
        if (n < N) {
          const int32_t a = acc[mi][j][v] + part[j][v];
          if (acc_out) acc_out[(size_t)m * N + n] = a;
          if (Y) Y[(size_t)m * N + n] = (float)a * sc;
        }
      }
    }
  };
  if constexpr (KS == 1) {
#pragma unroll
    for (int mi = 0; mi < MB; ++mi) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wm * WM + 16 * mi + 4 * g + v;
        if (m >= M) continue;
        const float sc = gm * absmax[m] * (1.0f / 127.0f);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int n = n0 + wn * WN + 16 * j + r;
          if (n < N) {
            const int32_t a = acc[mi][j][v];
            if (acc_out) acc_out[(size_t)m * N + n] = a;
            if (Y) Y[(size_t)m * N + n] = (float)a * sc;
          }
        }
      }
    }
  } else {
    // Group 0 stores row blocks mi < MB/2 and group 1 the rest, each adding the other
    // group's partial (int32, exact), which comes through LDS one row block per pass.
    // The accumulators are only read (no VALU writes to them), which keeps the register
    // count at the one-group kernel's.
    ring_barrier();  // every load has landed (the wait after the loop)
    v4i* out = reinterpret_cast<v4i*>(kg == 0 ? As0 : As1) + wave * NB * 64 + lane;
    const v4i* in = reinterpret_cast<const v4i*>(kg == 0 ? As1 : As0) + wave * NB * 64 + lane;
    static_for<MB / 2>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      if (kg == 0) {
#pragma unroll
        for (int j = 0; j < NB; ++j) out[j * 64] = acc[MB / 2 + p][j];
      } else {
#pragma unroll
        for (int j = 0; j < NB; ++j) out[j * 64] = acc[p][j];
      }
      ring_barrier();
      if (kg == 0) store_block(std::integral_constant<int, p>{}, in);
      else store_block(std::integral_constant<int, MB / 2 + p>{}, in);
      ring_barrier();
    });
  }
}

template <int GM, int GN, int WM, int WN, int D, int KS = 1>
hipError_t launch(const uint8_t* packed, const float* gamma, const int8_t* Xq, const float* absmax, int64_t M,
                  int64_t N, int64_t K, float* Y, int32_t* acc, hipStream_t s) {
  const int64_t K_pad = k_pad(K);
  const int chunks = (int)(K_pad / kTileCols);
  const int n_blocks = (int)(n_pad(N) / kTileRows);
  constexpr int BM = GM * WM, BN = GN * WN;
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  const int tiles = tiles_m * tiles_n;
  const int grid = 8 * ((tiles + 7) / 8);
  hipLaunchKernelGGL((k_gemm_mfma<GM, GN, WM, WN, D, KS>), dim3(grid), dim3(256 * KS), 0, s, packed, gamma, Xq, absmax, (int)M,
                     (int)N, n_blocks, (int)K_pad, chunks, tiles_m, tiles_n, Y, acc);
  return hipGetLastError();
}

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
  (void)K;
  GemmPlan p;
  // Tile shapes of 64 rows; each K group is four waves:
  //   64 x 256: waves of 64 x 64 side by side (three-slot ring, 24 KiB of LDS, 152
  //             registers, three workgroups per CU): the most work per operand byte;
  //   64 x 192: waves of 64 x 48 (118 registers, four per CU): the same structure, for
  //             column counts that 256 would leave a ragged last round on.
  // Where the tiles do not fill the chip, two K groups of four waves share each tile (eight
  // waves, each group half the chunks, partials summed through LDS): twice the waves per
  // tile at the same operand bytes per tile.  64 x 256 tiles when that gives 193..256 of
  // them (one eight-wave workgroup per CU), else 64 x 192 tiles when there are at most 512
  // (two per CU fit).  Measured against the one-group tiles: 1024 x 2560 x 6912 35.7 -> 27.4
  // us, 1024 x 2560 x 2560 18.1 -> 14.1 us, 512 x 8192 x 8192 43.2 -> 37.4 us, 512 x 6912 x
  // 2560 19.2 -> 17.2 us, 1536 x 2560 x 2560 18.4 -> 17.2 us, and with 448 tiles (2048 x 2560)
  // 47.8 -> 42.3 us at K = 6912, 52.0 -> 46.6 us at K = 8192, 30.4 -> 27.6 us at K = 4096,
  // 22.5 -> 20.4 us at K = 2560; the one shape measured slower, 512 x 2560 x 6912, by 3 %
  // (25.2 -> 25.9 us).  With more tiles the split costs more than it gives (2048 x 6912 x
  // 2560: 45.2 -> 47.8 us; 4096 x 2560 x 6912: 72.5 -> 78.2 us).
  // Otherwise, between 64 x 256 and 64 x 192, the cost of the last round decides: rounds of
  // 256 tiles times the tile width, the 48-column waves counted at 0.976 of the 64-column
  // rate (measured 8192^3: 486 vs 474 us).  Measured at M = 2048 x 6912 columns: 46.8 us
  // (64 x 256) -> 45.9 us (64 x 192); 8192^3, 4096 x 2560 x 6912 and 2048 x 28672 x 8192
  // stay on 64 x 256.
  const int64_t tm = (M + 63) / 64;
  const int64_t t256 = tm * ((N + 255) / 256), t192 = tm * ((N + 191) / 192);
  p.bm = 64;
  p.ks = 1;
  if (t256 > 192 && t256 <= 256) {
    p.bn = 256;
    p.ks = 2;
  } else if (t192 <= 512) {
    p.bn = 192;
    p.ks = 2;
  } else {
    const double c256 = (double)((t256 + 255) / 256) * 256.0;
    const double c192 = (double)((t192 + 255) / 256) * 192.0 / 0.976;
    p.bn = c192 < c256 ? 192 : 256;
  }
  p.threads = 256 * p.ks;
  const int64_t tiles = ((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn);
  p.groups = 8 * ((tiles + 7) / 8);
  return p;
}

hipError_t launch_gemm(const uint8_t* packed, const float* gamma, const int8_t* Xq, const float* absmax,
                       int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, hipStream_t s) {
  const GemmPlan p = plan_gemm(M, N, K);
  if (p.ks == 2) {
    if (p.bn == 256) return launch<1, 4, 64, 64, 3, 2>(packed, gamma, Xq, absmax, M, N, K, Y, acc, s);
    return launch<1, 4, 64, 48, 3, 2>(packed, gamma, Xq, absmax, M, N, K, Y, acc, s);
  }
  if (p.bn == 256) return launch<1, 4, 64, 64, 3>(packed, gamma, Xq, absmax, M, N, K, Y, acc, s);
  return launch<1, 4, 64, 48, 3>(packed, gamma, Xq, absmax, M, N, K, Y, acc, s);
}

}  // namespace bl
