// Prefill kernel (M > 16 tokens): a dense int8 x ternary contraction on the matrix cores,
// exact int32 accumulation and the fp32 rescale (y = acc * gamma * a[m] / 127) in the
// epilogue.
//
// bhfrc.com news 56965, section 1.1 (ternary x activation = add / subtract / skip) and
// section 4.1 (2-bit codes); aratech.ae BitNet b1.58 article, "BitLinear".
//
// Structure (workgroup = 4 or 8 waves in a GM x GN grid, each wave a WM x WN block of 16 x 16
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
//     three-slot ring), or 64 x 384 (eight waves 1 x 8 of 64 x 48, which share each
//     activation slab over twice the columns: half the activation re-reads), whichever
//     leaves the lighter last round of tiles, and two K groups of four waves per tile where
//     there are few tiles (plan_gemm);
//   * the loop body is unrolled over lcm(D, 2 CB) half-stages so that every ring index is
//     static; half-stages past the end of K are skipped whole (measured: 2048 x 6912 x 2560
//     48.9 -> 46.9 us, 4096 x 6912 x 2560 87.6 -> 82.3 us, 48 x 30000 x 512 9.4 -> 7.6 us),
//     and the loop ends by waiting for every load still in flight;
//   * tile order is XCD-aware: consecutive workgroup ids go to different XCDs, so each
//     XCD gets a contiguous run of output tiles (sharing activation rows in its L2);
//   * the compiler's own waits: it cannot count the direct loads against the weight loads
//     into registers, so it waits for every load in flight before the first read of a
//     weight register, and before any LDS read it waits for every direct load (it cannot
//     tell which ring slot one writes).  So the A fragments are read in inline assembly
//     (invisible to it; the ring's waits order them), and each half-stage reads its
//     weight registers before it issues its own loads, which leaves the compiler's wait
//     there with only the loads of the next half-stage in flight, issued a half-stage
//     before.  Before, every half-stage waited for the refills it had just issued
//     (measured: 2048 x 6912 x 2560 47.7 -> 45.1 us, 2048 x 2560 x 6912 44.0 -> 41.5 us,
//     8192^3 504 -> 478 us);
//   * epilogue: the wave's 16 row scales are loaded together before the first store (one
//     wait, not one memory round trip per row), and each row takes one address with the
//     column blocks at constant offsets from it (measured: 2048 x 6912 x 2560 45.3 -> 42.2
//     us, 4096 x 6912 x 2560 79.5 -> 73.4 us, 2048 x 2560 x 6912 42.6 -> 42.1 us);
//   * split-tail form (bitlinear_forward_ws): the whole rounds of tiles as above, then the
//     tiles left over split along K over the freed slots, their exact int32 partial tiles
//     summed by a second launch (k_gemm_fixup).
#include "bl_internal.h"

#include <algorithm>
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

// The wave's four A fragments of one MFMA step: rows r, r + 16, r + 32, r + 48 of its
// 64-row block (2048 bytes apart in a slab; the swizzle slot repeats every 16 rows), read
// from LDS in one block that ends by waiting for them, so the values are in place when it
// returns.  Written as inline assembly so that the compiler's wait insertion does not see
// LDS reads here: it cannot tell which ring slot a direct global->LDS load writes, and
// before any LDS read it would wait for every such load in flight, including the refills
// of later slots issued just before (which would empty the ring every half-stage).  The
// ring's own waits (wait_vmcnt + ring_barrier) order each slot's loads before its reads.
__device__ __forceinline__ void lds_read_frag4(v4i (&af)[4], const uint8_t* p) {
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:2048\n\t"
      "ds_read_b128 %2, %4 offset:4096\n\t"
      "ds_read_b128 %3, %4 offset:6144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3])
      : "v"(a));
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

// Arguments of the split-tail form (see the end of k_gemm_mfma).
struct SkArgs {
  int tail = 0;                // tiles left after the whole-tile rounds, split along K
  int parts = 1;               // K ranges per tail tile
  int cpp = 0;                 // chunks per K range (the last range may hold fewer)
  v4i* partials = nullptr;     // [tail][parts][4 waves][MB][NB][64 lanes] int32 partial tiles
};

template <int GM, int GN, int WM, int WN, int D, int KS = 1, bool kSK = false>
__global__ __launch_bounds__(64 * GM * GN * KS) __attribute__((amdgpu_waves_per_eu(kSK ? (WN == 64 ? 3 : 4) : 1))) void k_gemm_mfma(const uint8_t* __restrict__ packed, const float* __restrict__ gamma,
                                                   const int8_t* __restrict__ Xq, const float* __restrict__ absmax,
                                                   int M, int N, int n_blocks, int K_pad, int chunks, int tiles_m,
                                                   int tiles_n, float* __restrict__ Y, int32_t* __restrict__ acc_out,
                                                   SkArgs sk) {
  constexpr int NW = GM * GN;  // waves per K group
  static_assert(NW == 4 || (NW == 8 && KS == 1 && !kSK), "four waves, or eight in one K group");
  static_assert(D >= 2, "at least two ring slots");
  static_assert(KS == 1 || KS == 2, "one or two K groups");
  static_assert(!kSK || KS == 1, "the split-tail form runs one K group per tile");
  constexpr int BM = GM * WM, BN = GN * WN;
  constexpr int MB = WM / 16, NB = WN / 16;
  constexpr int kHalf = kTileCols / 2;        // bytes per activation row in a half-stage
  constexpr int kDma = BM / (8 * NW);        // direct loads per wave per half-stage (8 rows each)
  static_assert(kDma >= 1 && BM % (8 * NW) == 0, "the waves share the activation slab's rows evenly");
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

  // asrc / bsrc / acc / bw are per tile; run() below sets them up for one tile and one
  // range of its K chunks
  const int8_t* asrc[kDma];
  const uint4* bsrc[NB];
  uint4 bw[CB][NB];
  v4i acc[MB][NB];

  // compute half-stage in ring slot s (steps 2h, 2h+1 of its chunk) with weights cb
  // B operand of MFMA step i (0..3) of a chunk: the i-th 32-bit word of each 16-byte slot
  auto decode_step = [&](int i, const uint4 (&wcur)[NB], v4i (&bf)[NB]) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const uint32_t word = i == 0 ? wcur[j].x : (i == 1 ? wcur[j].y : (i == 2 ? wcur[j].z : wcur[j].w));
      bf[j] = decode16(word);
    }
  };
  // MFMA step 2 half + ip of the slab in a ring slot, with its decoded B operand
  auto mfma_step = [&](const uint8_t* slabp, int ip, const v4i (&bf)[NB]) {
    static_assert(MB == 4, "four 16-row fragments per wave");
    const int row = wm * WM + r;
    v4i af[4];
    lds_read_frag4(af, &slabp[row * kHalf + 16 * a_slot(row, 2 * g + ip)]);
#pragma unroll
    for (int mi = 0; mi < MB; ++mi) {
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[mi][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mi], bf[j], acc[mi][j], 0, 0, 0);
    }
  };

  // run(m0, n0, cb, ce): acc = the contraction of the tile at (m0, n0) over the packed
  // chunks [cb, ce) (the K group kg takes its share of them).  Ends with every load of
  // this wave landed (wait_vmcnt<0>); the caller adds a barrier before the ring is refilled.
  auto run = [&](int m0, int n0, int cb, int ce) {
    // K group kg takes chunks [c_lo, c_hi).  Both groups run the same number of half-stages
    // (they share the barriers); where the chunks do not split evenly the second group skips
    // the compute of its last ones and its loads repeat a valid chunk.
    const int cg = (ce - cb + KS - 1) / KS;
    const int c_lo = cb + kg * cg, c_hi = min(ce, c_lo + cg);
    const int hstages = 2 * cg;                                       // loop length, both groups
    const int hs_mine = KS == 1 ? hstages : 2 * max(c_hi - c_lo, 0);  // half-stages this group computes
    auto chunk_of = [&](int h) {
      if constexpr (KS == 1) return cb + (min(h, hstages - 1) >> 1);
      else return min(c_lo + (min(h, hstages - 1) >> 1), ce - 1);
    };

    // this lane's source for each direct load: row 8 (NW j + wave) + lane / 8, LDS slot
    // lane % 8 holding local piece lp = slot ^ swizzle, global piece 4 (lp >> 1) + 2h + (lp & 1)
    // (rows past M repeat row M-1: their outputs are never stored)
#pragma unroll
    for (int j = 0; j < kDma; ++j) {
      const int row = 8 * (NW * j + wave) + (lane >> 3);
      const int lp = a_slot(row, lane & 7);
      asrc[j] = Xq + (size_t)min(m0 + row, M - 1) * K_pad + 16 * (4 * (lp >> 1) + (lp & 1));
    }
    // weight slots of this wave's NB row blocks (blocks past the matrix re-read the last
    // block: their outputs are never stored)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int nb = min(n0 / kTileRows + wn * NB + j, n_blocks - 1);
      bsrc[j] = reinterpret_cast<const uint4*>(packed) + (size_t)nb * chunks * 64 + lane;
    }
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = (v4i){0, 0, 0, 0};

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
        load_g2lds16(asrc[j] + (size_t)c * kTileCols + 32 * (min(hs, hstages - 1) & 1), &dst[8 * (NW * j + wave) * kHalf]);
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
        // the first step's B operand is decoded before this half-stage's loads are issued:
        // the compiler waits for the weight registers at their first read with every load in
        // flight (it cannot count the direct loads against the others), and here that is
        // only the loads of half-stage hs + 1, issued one half-stage ago
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const uint4 w = bw[(k / 2) % CB][j];
          asm volatile("" ::"v"(w.x), "v"(w.y), "v"(w.z), "v"(w.w) : "memory");
        }
        v4i bf[NB];
        decode_step(2 * (k & 1), bw[(k / 2) % CB], bf);
        {
          const int hc = min(nh, hstages - 1);
          const int c = chunk_of(nh);
          uint8_t* dst = slab(std::integral_constant<int, (k + P) % D>{}) + kgoff;
#pragma unroll
          for (int j = 0; j < kDma; ++j)
            load_g2lds16(asrc[j] + (size_t)c * kTileCols + 32 * (hc & 1), &dst[8 * (NW * j + wave) * kHalf]);
          if constexpr (((k + P) & 1) == 0) {
#pragma unroll
            for (int j = 0; j < NB; ++j) bw[((k + P) / 2) % CB][j] = bsrc[j][(size_t)c * 64];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (hs < hs_mine) {
          const uint8_t* slabp = slab(std::integral_constant<int, k % D>{}) + kgoff;
          mfma_step(slabp, 0, bf);
          decode_step(2 * (k & 1) + 1, bw[(k / 2) % CB], bf);
          mfma_step(slabp, 1, bf);
        }
        // half-stage hs + 1 has landed: loads issued after it are those of hs + 2 .. hs + P
        wait_vmcnt<loads_between<kDma, NB>(k + 1, k + P)>();
        ring_barrier();
      });
      base += kBody;
    } while (base < hstages);
    // the refills of the last P half-stages (clamped re-reads of the last chunk, never
    // computed) land before the epilogue reuses registers and the workgroup moves on
    wait_vmcnt<0>();
  };

  const float gm = gamma[0];
  // Row scales gamma * a[m] / 127 of the wave's rows 16 mi + 4 g + v, loaded together
  // before any store (rows past M read row M-1; their outputs are never stored).
  float sc[MB][4];
  auto load_scales = [&](int m0) {
    float am[MB][4];
#pragma unroll
    for (int mi = 0; mi < MB; ++mi)
#pragma unroll
      for (int v = 0; v < 4; ++v) am[mi][v] = absmax[min(m0 + wm * WM + 16 * mi + 4 * g + v, M - 1)];
#pragma unroll
    for (int mi = 0; mi < MB; ++mi)
#pragma unroll
      for (int v = 0; v < 4; ++v) sc[mi][v] = gm * am[mi][v] * (1.0f / 127.0f);
  };
  // store row block mi of the wave's tile at (m0, n0) from its int32 values `part`: one
  // row address per row, the column blocks at constant offsets from it, and the column
  // bound checked only in a tile that crosses N
  auto store_rows = [&](auto mc, int m0, int n0, const v4i (&part)[NB]) {
    constexpr int mi = decltype(mc)::value;
    const int nl = n0 + wn * WN + r;  // column of block j: nl + 16 j
    const bool full_n = n0 + BN <= N;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + wm * WM + 16 * mi + 4 * g + v;
      if (m >= M) continue;
      const size_t off = (size_t)m * N + nl;
      if (acc_out) {
#pragma unroll
        for (int j = 0; j < NB; ++j)
          if (full_n || nl + 16 * j < N) acc_out[off + 16 * j] = part[j][v];
      }
      if (Y) {
#pragma unroll
        for (int j = 0; j < NB; ++j)
          if (full_n || nl + 16 * j < N) Y[off + 16 * j] = (float)part[j][v] * sc[mi][v];
      }
    }
  };
  // store row block mi: (acc + the sum of `np` partials at `other`, stride `pstride` v4i,
  // lane-major per column block) * scale
  auto store_block = [&](auto mc, int m0, int n0, const v4i* other, int np, size_t pstride) {
    constexpr int mi = decltype(mc)::value;
    v4i part[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) part[j] = acc[mi][j];
    for (int q = 0; q < np; ++q) {
#pragma unroll
      for (int j = 0; j < NB; ++j) part[j] += other[(size_t)q * pstride + j * 64];
    }
    store_rows(mc, m0, n0, part);
  };
  // the whole tile, from the accumulators alone
  auto store_tile = [&](int m0, int n0) {
    load_scales(m0);
    static_for<MB>([&](auto mc) { store_rows(mc, m0, n0, acc[decltype(mc)::value]); });
  };

  const int tiles = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int xcd = b & 7;
  if constexpr (!kSK) {
    // XCD-aware tile order: workgroup b runs on XCD b % 8; give XCD x the x-th contiguous
    // run of tiles in row-major (m, n) order
    const int slot = b >> 3;
    const int per_xcd = (tiles + 7) / 8;
    const int full = tiles - 8 * (per_xcd - 1);  // XCDs holding per_xcd tiles (the rest hold one fewer)
    const int t = xcd < full ? xcd * per_xcd + slot : full * per_xcd + (xcd - full) * (per_xcd - 1) + slot;
    if (slot >= (xcd < full ? per_xcd : per_xcd - 1)) return;
    const int m0 = (t / tiles_n) * BM, n0 = (t % tiles_n) * BN;
    run(m0, n0, 0, chunks);
    if constexpr (KS == 1) {
      store_tile(m0, n0);
    } else {
      // Group 0 stores row blocks mi < MB/2 and group 1 the rest, each adding the other
      // group's partial (int32, exact), which comes through LDS one row block per pass.
      load_scales(m0);
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
        if (kg == 0) store_block(std::integral_constant<int, p>{}, m0, n0, in, 1, 0);
        else store_block(std::integral_constant<int, MB / 2 + p>{}, m0, n0, in, 1, 0);
        ring_barrier();
      });
    }
  } else {
    // Split-tail form.  Workgroups b < tdp = rounds x slots take one whole tile each,
    // mapped as above (XCD x owns a contiguous run); the hardware starts the later
    // workgroups as slots free up, so the workgroups past tdp run once the last round of
    // whole tiles ends, and the y stores of those tiles drain while they compute.  They
    // take the sk.tail tiles left (the last ones in row-major order), split along K into
    // sk.parts ranges of sk.cpp chunks, one range each: tail tile i goes to XCD i % 8, and
    // part j of it to the workgroup of that XCD with slot parts * (i / 8) + j past tdp.
    // Each part writes its exact int32 partial tile to the workspace; k_gemm_fixup, the
    // next launch on the stream, adds them and stores the tail tiles.  (Adding them in
    // this launch, by the part that draws the last ticket of a per-tile counter, needs a
    // device-scope release and acquire per part, which write back and invalidate the XCD's
    // L2: measured 2048 x 6912 x 2560 46.6 -> 132.6 us.)  No workgroup waits for another.
    const int tdp = tiles - sk.tail;
    int t, cb = 0, ce = chunks, j = 0, i = 0;
    if (b < tdp) {
      t = xcd * (tdp >> 3) + (b >> 3);
    } else {
      const int s = (b - tdp) >> 3;
      j = s % sk.parts;
      i = 8 * (s / sk.parts) + xcd;
      if (i >= sk.tail) return;
      t = tdp + i;
      cb = j * sk.cpp;
      ce = min(chunks, cb + sk.cpp);
    }
    const int m0 = (t / tiles_n) * BM, n0 = (t % tiles_n) * BN;
    run(m0, n0, cb, ce);
    if (b < tdp) {
      store_tile(m0, n0);
      return;
    }
    // partial tiles: [tail][parts][4 waves][MB][NB][64 lanes] v4i, summed by k_gemm_fixup
    constexpr int kWaveTile = MB * NB * 64;
    v4i* mine = sk.partials + ((size_t)(i * sk.parts + j) * 4 + wave) * kWaveTile + lane;
#pragma unroll
    for (int mi = 0; mi < MB; ++mi)
#pragma unroll
      for (int jj = 0; jj < NB; ++jj) mine[(mi * NB + jj) * 64] = acc[mi][jj];
  }
}

// The split tail's second kernel: tile i of the tail is the int32 sum of its `parts`
// partial tiles (exact in any order; added in part order), rescaled and stored like a
// whole tile.  One thread per 4-output vector of the partial layout (wave w, row block
// mi, column block jj, lane): consecutive threads read consecutive 16-byte vectors.
template <int GM, int GN, int WM, int WN>
__global__ __launch_bounds__(256) void k_gemm_fixup(const v4i* __restrict__ partials, const float* __restrict__ gamma,
                                                    const float* __restrict__ absmax, int M, int N, int tiles_n,
                                                    int tdp, int parts, float* __restrict__ Y,
                                                    int32_t* __restrict__ acc_out) {
  constexpr int BN = GN * WN, BM = GM * WM;
  constexpr int MB = WM / 16, NB = WN / 16;
  constexpr int kTileVecs = 4 * MB * NB * 64;
  constexpr int kBlocks = kTileVecs / 256;  // workgroups per tail tile
  const int i = blockIdx.x / kBlocks;
  const int e = (blockIdx.x % kBlocks) * 256 + threadIdx.x;
  const v4i* src = partials + (size_t)i * parts * kTileVecs + e;
  v4i sum = src[0];
  for (int q = 1; q < parts; ++q) sum += src[(size_t)q * kTileVecs];
  const int lane = e & 63, blk = e >> 6;
  const int jj = blk % NB, mi = (blk / NB) % MB, w = blk / (NB * MB);
  const int r = lane & 15, g = lane >> 4;
  const int t = tdp + i;
  const int m0 = (t / tiles_n) * BM + (w / GN) * WM + 16 * mi + 4 * g;
  const int n = (t % tiles_n) * BN + (w % GN) * WN + 16 * jj + r;
  if (n >= N) return;
  const float gm = gamma[0];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = m0 + v;
    if (m < M) {
      if (acc_out) acc_out[(size_t)m * N + n] = sum[v];
      if (Y) Y[(size_t)m * N + n] = (float)sum[v] * (gm * absmax[m] * (1.0f / 127.0f));
    }
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
  hipLaunchKernelGGL((k_gemm_mfma<GM, GN, WM, WN, D, KS>), dim3(grid), dim3(64 * GM * GN * KS), 0, s, packed, gamma, Xq, absmax, (int)M,
                     (int)N, n_blocks, (int)K_pad, chunks, tiles_m, tiles_n, Y, acc, SkArgs{});
  return hipGetLastError();
}

// The split-tail form (one K group) with the plan's rounds and tail; the workspace holds
// the tail tiles' partial tiles, written by the first launch and summed by the second.
template <int GM, int GN, int WM, int WN, int D>
hipError_t launch_sk(const uint8_t* packed, const float* gamma, const int8_t* Xq, const float* absmax, int64_t M,
                     int64_t N, int64_t K, float* Y, int32_t* acc, const GemmPlan& p, void* workspace, hipStream_t s) {
  const int64_t K_pad = k_pad(K);
  const int chunks = (int)(K_pad / kTileCols);
  const int n_blocks = (int)(n_pad(N) / kTileRows);
  constexpr int BM = GM * WM, BN = GN * WN;
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  SkArgs sk;
  sk.tail = p.sk_tail;
  sk.parts = p.sk_parts;
  sk.cpp = p.sk_cpp;
  sk.partials = static_cast<v4i*>(workspace);
  hipLaunchKernelGGL((k_gemm_mfma<GM, GN, WM, WN, D, 1, true>), dim3(p.groups), dim3(256), 0, s, packed, gamma, Xq,
                     absmax, (int)M, (int)N, n_blocks, (int)K_pad, chunks, tiles_m, tiles_n, Y, acc, sk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int kBlocks = 4 * (WM / 16) * (WN / 16) * 64 / 256;
  const int tdp = tiles_m * tiles_n - p.sk_tail;
  hipLaunchKernelGGL((k_gemm_fixup<GM, GN, WM, WN>), dim3(p.sk_tail * kBlocks), dim3(256), 0, s,
                     static_cast<const v4i*>(workspace), gamma, absmax, (int)M, (int)N, tiles_n, tdp, p.sk_parts, Y,
                     acc);
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
  //             column counts that 256 would leave a ragged last round on;
  //   64 x 384: eight waves of 64 x 48 in one K group (two workgroups per CU): the
  //             64 x 192 waves with each activation slab shared by twice the columns.
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
  // Otherwise, between 64 x 256, 64 x 192 and 64 x 384, the cost of the last round decides:
  // rounds of 256 tiles times the tile width, the 48-column waves counted at 0.976 of the
  // 64-column rate (measured 8192^3: 486 vs 474 us) and the eight-wave 384-column tiles at
  // 1.14 of it (half the activation re-reads; fitted to interleaved A/B runs, 64 x 384 against
  // the four-wave tile the rule chose before, outputs identical, M x K x N: 1536 x 2560 x
  // 6912 33.9 -> 31.5 us, 1792 x 2560 x 6912 35.9 -> 33.0, 2560 x 2560 x 6912 49.5 -> 47.3,
  // 3584 x 2560 x 6912 64.8 -> 61.0, 4096 x 6912 x 2560 76.2 -> 72.0, 3000 x 700 x 9000 37.2
  // -> 36.4, 8192^3 457 -> 446, 4096 x 2560 x 6912 75.7 -> 76.2, 2048 x 8192 x 28672 402 ->
  // 402, 4000 x 1000 x 8190 47.9 -> 48.3; where the 384-column tiles leave a light last
  // round the rule keeps the narrower tile: 2048 x 2560 x 6912 41.6 -> 42.5 us, 3072 x 2560
  // x 6912 57.8 -> 56.8).  Measured at M = 2048 x 6912 columns: 46.8 us (64 x 256) -> 45.9 us
  // (64 x 192).
  const int64_t tm = (M + 63) / 64;
  const int64_t t256 = tm * ((N + 255) / 256), t192 = tm * ((N + 191) / 192), t384 = tm * ((N + 383) / 384);
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
    const double c384 = N >= 384 ? (double)((t384 + 255) / 256) * 384.0 / 1.14 : 1e300;
    p.bn = c192 < c256 ? 192 : 256;
    if (c384 < std::min(c192, c256)) p.bn = 384;
  }
  p.threads = (p.bn == 384 ? 512 : 256) * p.ks;
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
  if (p.bn == 384) return launch<1, 8, 64, 48, 3>(packed, gamma, Xq, absmax, M, N, K, Y, acc, s);
  if (p.bn == 256) return launch<1, 4, 64, 64, 3>(packed, gamma, Xq, absmax, M, N, K, Y, acc, s);
  return launch<1, 4, 64, 48, 3>(packed, gamma, Xq, absmax, M, N, K, Y, acc, s);
}

// Resident workgroups per compute unit of the one-group kernels (registers decide: 152
// per lane for the 64 x 64 wave tile, three waves per SIMD; 118 for 64 x 48, four),
// checked against the runtime's occupancy query by the GPU tests.
int gemm_slots_per_cu(int bn) { return bn == 256 ? 3 : 4; }

GemmPlan plan_gemm_ws(int64_t M, int64_t N, int64_t K) {
  GemmPlan p = plan_gemm(M, N, K);
  if (p.ks != 1 || p.bn == 384) return p;  // the split-tail form runs four-wave tiles
  // With plan_gemm's tile, where the tiles need more than one round of the resident slots
  // and the last round is partial: every slot takes `rounds` whole tiles, and the tiles
  // left over are split along K so that every slot carries the same work to within one K
  // range.  Each of the 8 XCDs holds slots / 8 workgroups and ceil(tail / 8) tail tiles,
  // so up to floor(slots / 8 / ceil(tail / 8)) ranges per tail tile fit, each of at least
  // one 256-column chunk.
  const int64_t chunks = k_pad(K) / kTileCols;
  const int bn = p.bn;
  const int64_t tiles = ((M + 63) / 64) * ((N + bn - 1) / bn);
  const int64_t slots = (int64_t)kGemmCUs * gemm_slots_per_cu(bn);
  if (tiles <= slots) return p;
  const int64_t rounds = tiles / slots, tail = tiles - rounds * slots;
  if (tail == 0) return p;
  const int64_t pmax = std::max<int64_t>(1, (slots / 8) / ((tail + 7) / 8));
  const int64_t cpp = (chunks + pmax - 1) / pmax;
  const int64_t parts = (chunks + cpp - 1) / cpp;
  if (parts < 2) return p;  // whole tiles: nothing to split
  // The partial tiles cost their bytes twice (written here, read by the second launch) on
  // top of the fp32 output, and the second launch costs a few microseconds of its own.
  // Measured against whole tiles (one launch): 1600 x 8000 x 1000, 5.1 MB of partials:
  // 28.5 -> 27.2 us; 2048 x 6912 x 2560, 31 MB: 45.1 -> 48.8 us; 4096 x 6912 x 2560, 50 MB:
  // 76.5 -> 90.5 us; 1291 x 12000 x 3000, 43 MB: 57.5 -> 65.2 us; 8192^3, 50 MB: 478 ->
  // 479 us.  So the split runs only where the partials stay within 8 MiB.
  const int64_t ws = tail * parts * 64 * bn * 4;
  if (ws > (int64_t(8) << 20)) return p;
  GemmPlan q = p;
  q.sk = true;
  q.sk_rounds = (int)rounds;
  q.sk_tail = (int)tail;
  q.sk_parts = (int)parts;
  q.sk_cpp = (int)cpp;
  q.groups = rounds * slots + 8 * parts * ((tail + 7) / 8);
  q.ws_bytes = ws;
  return q;
}

hipError_t gemm_occupancy(int out[4]) {
  const void* fns[4] = {reinterpret_cast<const void*>(&k_gemm_mfma<1, 4, 64, 64, 3, 1, false>),
                        reinterpret_cast<const void*>(&k_gemm_mfma<1, 4, 64, 48, 3, 1, false>),
                        reinterpret_cast<const void*>(&k_gemm_mfma<1, 4, 64, 64, 3, 1, true>),
                        reinterpret_cast<const void*>(&k_gemm_mfma<1, 4, 64, 48, 3, 1, true>)};
  for (int i = 0; i < 4; ++i) {
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&out[i], fns[i], 256, 0);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm_ws(const uint8_t* packed, const float* gamma, const int8_t* Xq, const float* absmax,
                          int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, void* workspace, hipStream_t s) {
  const GemmPlan p = plan_gemm_ws(M, N, K);
  if (!p.sk) return launch_gemm(packed, gamma, Xq, absmax, M, N, K, Y, acc, s);
  if (p.bn == 256) return launch_sk<1, 4, 64, 64, 3>(packed, gamma, Xq, absmax, M, N, K, Y, acc, p, workspace, s);
  return launch_sk<1, 4, 64, 48, 3>(packed, gamma, Xq, absmax, M, N, K, Y, acc, p, workspace, s);
}

}  // namespace bl
