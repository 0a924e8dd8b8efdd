// Decode kernels (M = 1..16 tokens): packed-ternary x int8 with exact int32 accumulation
// and the fp32 rescale in the epilogue.
//
// bhfrc.com news 56965, section 1.1: a ternary weight times an activation adds it,
// subtracts it or skips it; section 4.1: the weights travel as 2-bit codes so that one
// load carries many of them.  aratech.ae BitNet b1.58 article, "BitLinear": activations
// are int8 with a per-token absmax scale; y is the product rescaled by both scales.
//
// Decode is HBM-bound (0.25 byte of weights per multiply-add at M = 1), so every kernel
// here is a streaming read of the packed matrix in which the arithmetic hides:
//   * each lane loads 16 bytes of a 1 KiB tile (non-temporal): 64 consecutive codes of
//     one row, decoded in registers (decode16) straight into the B operand of
//     v_mfma_i32_16x16x64_i8; one wave-wide load is one whole tile;
//   * the waves of a workgroup split the K tiles of its 16-row block(s) into contiguous
//     runs; all loads are unconditional (indices past a run are clamped to a valid tile
//     and its codes zeroed), so the compiler emits exact vmcnt waits;
//   * rows of the A operand beyond M repeat a real token or carry other pieces; they only
//     feed output rows that are never stored;
//   * the waves' partial 16x16 int32 tiles are summed in LDS in wave order (exact) and
//     rescaled by y = acc * gamma * a[m] / 127.
//
// The kernels differ in where the activations (the A operand) come from:
//   k_gemv_dpp   1..4 tokens: every load of a wave's run is issued at once and the
//                activations stay in registers, put into place by DPP lane shifts; the
//                fused form (bf16/fp32 x) quantises in the kernel; k_gemv_dpp_group runs
//                several matrices of one input in one launch;
//   k_gemv_dppm  5..16 tokens on rows of at most 4096: the same register runs for a
//                token group of 8 or 16, activation registers shared by 1 or 2 row blocks;
//   k_gemv_fq16  the fused form for 5..16 tokens (bf16 x): every workgroup quantises the
//                token rows into LDS, one wave per row, while its weights stream in;
//   k_gemv_reg   other 5..16-token shapes: activation fragments loaded per tile with
//                the weights of a ring of batches, shared by 1, 2 or 4 row blocks;
//   k_gemv_lds   the fused form where its register pieces would not fit (many row
//                blocks, short rows): every workgroup quantises the rows into LDS with an
//                exact, compile-time number of 16-byte pieces per thread issued before
//                the weight loads (vector-memory loads retire in order, so their wait
//                does not wait for the weights).
#include "bl_internal.h"
#include "decode_common.h"

#include <algorithm>
#include <atomic>

namespace bl {
namespace {

constexpr int kMaxLdsActBytes = 48 * 1024;
constexpr int64_t kMaxFusedElems = 8192;  // M*K limit of the one-kernel quantise + decode
constexpr int kMaxFq16Lds = 120 * 1024;   // dynamic LDS of the fused 5..16-token kernel
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Sum the W waves' partial tiles (red[w][t][j][lane]) and write y / acc for token group t
// (tokens 16 t .. 16 t + 15) of row block j.
template <int W, int RB, int TG = 1>
__device__ __forceinline__ void gemv_epilogue(const v4i* red, int wave, int lane, int rb0, int rblocks, int M, int N,
                                              float gm, const float* absmax, float* Y, int32_t* acc_out) {
  const int r = lane & 15, g = lane >> 4;
  for (int jj = wave; jj < RB * TG; jj += W) {
    const int t = TG == 1 ? 0 : jj / RB, j = TG == 1 ? jj : jj % RB;
    if (rb0 + j >= rblocks) continue;
    v4i s = red[jj * 64 + lane];
    for (int w = 1; w < W; ++w) s += red[(w * RB * TG + jj) * 64 + lane];
    // lane holds D[4g + v][r]: token m = 16t + 4g + v, output n = 16*(rb0 + j) + r
    const int n = (rb0 + j) * kTileRows + r;
    if (n >= N) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 16 * t + 4 * g + v;
      if (m < M) {
        if (acc_out) acc_out[(size_t)m * N + n] = s[v];
        if (Y) Y[(size_t)m * N + n] = (float)s[v] * gm * absmax[m] * (1.0f / 127.0f);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// k_gemv_lds: the fused form with the activations quantised into LDS by every workgroup.
// kSrc: 1 = bf16 x, 2 = fp32 x (K columns).  S = 16-byte pieces per thread (exact: the
// launcher picks S = ceil(pieces / threads)).
template <int W, int U, int NB, int S, int kSrc>
__global__ __launch_bounds__(W * 64) void k_gemv_lds(const uint8_t* __restrict__ packed,
                                                     const float* __restrict__ gamma, const void* __restrict__ X,
                                                     int M, int N, int K,
                                                     int K_pad, int chunks, int rblocks, float* __restrict__ Y,
                                                     int32_t* __restrict__ acc_out, int8_t* __restrict__ xq_out,
                                                     float* __restrict__ absmax_out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t act_lds[];  // [M][K_pad + 16] int8
  __shared__ v4i red[W * 64];
  __shared__ float amax_red[W][4];
  __shared__ float row_amax[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int rb0 = blockIdx.x;
  const int tpw = (chunks + W - 1) / W;
  const int c0 = wave * tpw;
  const int c1 = min(chunks, c0 + tpw);
  const int row = min(r, M - 1);
  const int lds_stride = K_pad + 16;
  const uint4* wsrc = reinterpret_cast<const uint4*>(packed) + (size_t)rb0 * chunks * 64 + lane;

  // activation pieces: bf16 -> 8 elements, fp32 -> 4 elements per 16 bytes
  static_assert(kSrc == 1 || kSrc == 2, "the LDS-staged kernel is the fused form only");
  constexpr int kElems = kSrc == 1 ? 8 : 4;
  constexpr int kElemBytes = kSrc == 1 ? 2 : 4;
  const int row_elems = K;
  const int per_row = row_elems / kElems;
  const int pieces = M * per_row;
  uint4 st[S];
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const int idx = min((int)threadIdx.x + j * W * 64, pieces - 1);
    const int m = idx / per_row, p = idx - m * per_row;
    const uint8_t* base = static_cast<const uint8_t*>(X) + (size_t)m * row_elems * kElemBytes;
    st[j] = reinterpret_cast<const uint4*>(base)[p];
  }
  __builtin_amdgcn_sched_barrier(0);  // activation loads are issued before the weights

  uint4 w[NB][U];
  auto load = [&](int b, int cb) {
#pragma unroll
    for (int u = 0; u < U; ++u) w[b][u] = load_nt(wsrc + (size_t)min(cb + u, c1 - 1) * 64);
    __builtin_amdgcn_sched_barrier(0);
  };
  // Unconditional: a wave without tiles re-reads a valid tile (c1 - 1 >= 0) and never
  // computes, so the waits below count exactly the loads issued after each one.
#pragma unroll
  for (int b = 0; b < NB; ++b) load(b, c0 + b * U);

  {
    // fused activation quantiser: per-row absmax, s = 127/a, xq = clamp(rint(x*s))
    float v[S][kElems];
    float pm[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const int idx = (int)threadIdx.x + j * W * 64;
      if (kSrc == 1) {
        const uint32_t q4[4] = {st[j].x, st[j].y, st[j].z, st[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[j][2 * e] = __uint_as_float(q4[e] << 16);
          v[j][2 * e + 1] = __uint_as_float(q4[e] & 0xFFFF0000u);
        }
      } else {
        v[j][0] = __uint_as_float(st[j].x);
        v[j][1] = __uint_as_float(st[j].y);
        v[j][2] = __uint_as_float(st[j].z);
        v[j][3] = __uint_as_float(st[j].w);
      }
      if (idx < pieces) {
        const int m = idx / per_row;
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < kElems; ++e) a = fmaxf(a, fabsf(v[j][e]));
#pragma unroll
        for (int mm = 0; mm < 4; ++mm)
          if (m == mm) pm[mm] = fmaxf(pm[mm], a);
      }
    }
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      if (mm < M) {
        float a = pm[mm];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
        if (lane == 0) amax_red[wave][mm] = a;
      }
    }
    __syncthreads();
    // every thread forms the row maxima and scales itself (no second barrier); the
    // epilogue reads row_amax after the reduction barrier further down
    float scale[4];
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      float a = 0.0f;
      if (mm < M)
        for (int ww = 0; ww < W; ++ww) a = fmaxf(a, amax_red[ww][mm]);
      scale[mm] = a > 0.0f ? 127.0f / a : 0.0f;
      if ((int)threadIdx.x == mm) {
        row_amax[mm] = a;
        if (blockIdx.x == 0 && mm < M) absmax_out[mm] = a;
      }
    }
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const int idx = (int)threadIdx.x + j * W * 64;
      if (idx < pieces) {
        const int m = idx / per_row, p = idx - m * per_row;
        const float s = m == 0 ? scale[0] : (m == 1 ? scale[1] : (m == 2 ? scale[2] : scale[3]));
        uint32_t packed_q[kElems / 4];
#pragma unroll
        for (int e4 = 0; e4 < kElems / 4; ++e4)
          packed_q[e4] = quant_code4(v[j][4 * e4], v[j][4 * e4 + 1], v[j][4 * e4 + 2], v[j][4 * e4 + 3], s);
        uint8_t* dst = act_lds + m * lds_stride + kElems * p;
        if (kSrc == 1) *reinterpret_cast<uint2*>(dst) = make_uint2(packed_q[0], packed_q[1]);
        else *reinterpret_cast<uint32_t*>(dst) = packed_q[0];
        if (blockIdx.x == 0) {
          int8_t* gdst = xq_out + (size_t)m * K_pad + kElems * p;
          if (kSrc == 1) *reinterpret_cast<uint2*>(gdst) = make_uint2(packed_q[0], packed_q[1]);
          else *reinterpret_cast<uint32_t*>(gdst) = packed_q[0];
        }
      }
    }
    // padding columns K .. K_pad-1 are zero (K is a multiple of 4 here)
    const int per_pad = (K_pad - K) / 4;
    for (int idx = threadIdx.x; idx < M * per_pad; idx += W * 64) {
      const int m = idx / per_pad, p = idx - m * per_pad;
      *reinterpret_cast<uint32_t*>(act_lds + m * lds_stride + K + 4 * p) = 0u;
      if (blockIdx.x == 0) *reinterpret_cast<uint32_t*>(xq_out + (size_t)m * K_pad + K + 4 * p) = 0u;
    }
  }
  __syncthreads();

  v4i c = {0, 0, 0, 0};
  auto compute = [&](int b, int cb, bool tail) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(cb + u, c1 - 1);
      const bool live = !tail || cb + u < c1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t word = word_of(w[b][u], i);
        if (tail) word = live ? word : 0u;  // code 00 decodes to 0
        const v4i av = *reinterpret_cast<const v4i*>(act_lds + row * lds_stride + t * kTileCols + 64 * g + 16 * i);
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, decode16(word), c, 0, 0, 0);
      }
    }
  };
  if (c0 < c1) {
    const int nbat = (c1 - c0 + U - 1) / U;
    int j = 0;
    for (; j + 2 * NB <= nbat; j += NB) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        compute(b, c0 + (j + b) * U, false);
        load(b, c0 + (j + b + NB) * U);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (j + b < nbat) compute(b, c0 + (j + b) * U, true);
      if (j + b + NB < nbat) load(b, c0 + (j + b + NB) * U);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (j + NB + b < nbat) compute(b, c0 + (j + NB + b) * U, true);
  }

  red[wave * 64 + lane] = c;
  __syncthreads();
  gemv_epilogue<W, 1>(red, wave, lane, rb0, rblocks, M, N, gamma[0], row_amax, Y, acc_out);
}

// ---------------------------------------------------------------------------------------
// k_gemv_reg: activation fragments in registers, loaded per tile index with the weights
// of that batch and shared by the RB row blocks of the workgroup.  TG token groups of 16
// (up to 64 tokens): each decoded weight fragment feeds TG matrix-core steps.
template <int W, int RB, int U, int NB, int TG = 1>
__global__ __launch_bounds__(W * 64) void k_gemv_reg(const uint8_t* __restrict__ packed,
                                                     const float* __restrict__ gamma, const int8_t* __restrict__ Xq,
                                                     const float* __restrict__ absmax, int M, int N, int K_pad,
                                                     int chunks, int rblocks, float* __restrict__ Y,
                                                     int32_t* __restrict__ acc_out) {
  __shared__ v4i red[W * RB * TG * 64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int rb0 = blockIdx.x * RB;
  const int tpw = (chunks + W - 1) / W;
  const int c0 = wave * tpw;
  const int c1 = min(chunks, c0 + tpw);
  const uint4* wsrc[RB];
#pragma unroll
  for (int j = 0; j < RB; ++j)
    wsrc[j] = reinterpret_cast<const uint4*>(packed) + (size_t)min(rb0 + j, rblocks - 1) * chunks * 64 + lane;
  // token group tg reads token rows 16 tg + r (rows past M repeat row M-1: never stored)
  const int8_t* xrow[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) xrow[tg] = Xq + (size_t)min(16 * tg + r, M - 1) * K_pad + 64 * g;
  uint4 w[NB][U][RB];
  uint4 a[NB][U][TG][4];
  auto load = [&](int b, int cb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(cb + u, c1 - 1);
#pragma unroll
      for (int j = 0; j < RB; ++j) w[b][u][j] = load_nt(wsrc[j] + (size_t)t * 64);
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        const uint4* p = reinterpret_cast<const uint4*>(xrow[tg] + (size_t)t * kTileCols);
#pragma unroll
        for (int i = 0; i < 4; ++i) a[b][u][tg][i] = p[i];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  v4i c[TG][RB];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int j = 0; j < RB; ++j) c[tg][j] = (v4i){0, 0, 0, 0};
  auto compute = [&](int b, int cb, bool tail) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = !tail || cb + u < c1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (TG == 1) {
          const v4i av = as_v4i(a[b][u][0][i]);
#pragma unroll
          for (int j = 0; j < RB; ++j) {
            uint32_t word = word_of(w[b][u][j], i);
            if (tail) word = live ? word : 0u;
            c[0][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, decode16(word), c[0][j], 0, 0, 0);
          }
        } else {
          v4i wd[RB];
#pragma unroll
          for (int j = 0; j < RB; ++j) {
            uint32_t word = word_of(w[b][u][j], i);
            if (tail) word = live ? word : 0u;
            wd[j] = decode16(word);
          }
#pragma unroll
          for (int tg = 0; tg < TG; ++tg)
#pragma unroll
            for (int j = 0; j < RB; ++j)
              c[tg][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(a[b][u][tg][i]), wd[j], c[tg][j], 0, 0, 0);
        }
      }
    }
  };
#pragma unroll
  for (int b = 0; b < NB; ++b) load(b, c0 + b * U);
  if (c0 < c1) {
    const int nbat = (c1 - c0 + U - 1) / U;
    int j = 0;
    for (; j + 2 * NB <= nbat; j += NB) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        compute(b, c0 + (j + b) * U, false);
        load(b, c0 + (j + b + NB) * U);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (j + b < nbat) compute(b, c0 + (j + b) * U, true);
      if (j + b + NB < nbat) load(b, c0 + (j + b + NB) * U);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (j + NB + b < nbat) compute(b, c0 + (j + NB + b) * U, true);
  }
  // a missing row block (past rblocks) re-read a valid block's codes: never stored
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int j = 0; j < RB; ++j) red[((wave * TG + tg) * RB + j) * 64 + lane] = c[tg][j];
  __syncthreads();
  gemv_epilogue<W, RB, TG>(red, wave, lane, rb0, rblocks, M, N, gamma[0], absmax, Y, acc_out);
}

// ---------------------------------------------------------------------------------------
// k_gemv_dpp (M = MM <= 4 tokens): no LDS staging of activations and no barrier in front
// of the weight stream.  A workgroup owns one 16-row block; wave w owns tiles
// [w T, w T + T) of it (T a compile-time run length; tiles past the matrix re-read the
// last tile and decode as zeros) and issues every one of its loads at once, so the whole
// matrix is in flight from the start.  Activations travel in registers: with
// UA = 16 / (4 MM) tiles per activation piece, lane (r, g) holds the 16 activations of
// token r % MM, step (r / MM) % 4, tile r / (4 MM) of its group, at columns 64 g + 16 step;
// the A operand of step i of tile u is that register shifted down MM (4 u + i) lanes inside
// each 16-lane row (DPP), which puts the piece of token m in lane m.  Lanes r >= MM
// receive other pieces: they feed output rows of tokens that do not exist and are never
// stored.
//
// kSrc = 0 reads int8 xq.  kSrc = 1 (bf16) / 2 (fp32) is the fused form: the pieces are
// read from x itself, and since the pieces of a workgroup's waves cover every column of
// every token, the per-token absmax is the maximum over them (wave reductions, then one
// barrier across the waves); each lane then quantises its own pieces with the
// arithmetic of the standalone quantiser, and workgroup 0 stores xq and absmax.  Where the
// weight loads go relative to that phase (after the barrier, before it, or as soon as the
// wave's own pieces land) is a planner choice: kSrcEarly / kSrcMid below.
// kSrc = 3 (bf16) / 4 (fp32) adds the sub-layer RMS normalisation in front of the
// quantiser, as the standalone normalising quantiser does: the pieces become
// h = fl32(x g) before the absmax, each lane also sums the squares of x over the pieces
// it alone covers (fp64), and the scale stored and used in the rescale is
// max|h| / sqrt(mean(x^2) + eps).
// Matrices that share one activation input (bitlinear_forward_grouped); a single forward
// is a group of one.  rb_end[j] = row blocks of matrices 0..j.
struct MatGroup {
  int count;
  int rb_end[kMaxGroup];
  int N[kMaxGroup];
  const uint8_t* packed[kMaxGroup];
  const float* gamma[kMaxGroup];
  float* Y[kMaxGroup];
  int32_t* acc[kMaxGroup];
};

// Squared-ReLU gating of one output pair, in fp32: relu(g)^2 * u.
__device__ __forceinline__ float gated_relu2(float g, float u) {
  const float r = g > 0.0f ? g : 0.0f;
  return r * r * u;
}

// Work-group barrier that only orders LDS: unlike __syncthreads() it carries no release
// fence, so it does not wait for the weight loads still in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Activation sources of the decode kernels: 0 = int8 xq, 1 / 2 = bf16 / fp32 x, 3 / 4 =
// bf16 / fp32 x through the sub-layer normalisation.  kSrcEarly added to 1 / 2 selects the
// fused form that issues its weight loads before the activation barrier; kSrcMid added to
// 1..4 the form that issues them as soon as its own activation pieces have landed.
// kSrcPrio added to 1 / 2 raises the waves' issue priority while they issue their
// activation loads (weights after the barrier, as in the plain fused form); kSrcLead does
// the same and also issues the first two weight tiles of each run ahead of the barrier.
constexpr int kSrcEarly = 8;
constexpr int kSrcMid = 32;
constexpr int kSrcPrio = 64;
constexpr int kSrcLead = 128;
constexpr int kLeadTiles = 2;
constexpr bool src_bf16(int src) { return (src & 7) == 1 || (src & 7) == 3; }
constexpr bool src_norm(int src) { return (src & 7) >= 3; }
constexpr bool src_early(int src) { return (src & kSrcEarly) != 0; }
constexpr bool src_mid(int src) { return (src & kSrcMid) != 0; }
constexpr bool src_prio(int src) { return (src & (kSrcPrio | kSrcLead)) != 0; }
constexpr bool src_lead(int src) { return (src & kSrcLead) != 0; }

template <int MM, int kSrc>
struct DppShape {
  static constexpr int UA = 16 / (4 * MM);                                // tiles per activation piece
  static constexpr int kParts = kSrc == 0 ? 1 : (src_bf16(kSrc) ? 2 : 4);  // 16-byte loads per piece
};

// kPair: a gate / up pair of matrices with the same shape (packed, gamma = gate; packed2,
// gamma2 = up).  The workgroup streams row block rb0 of both with one set of activation
// registers and writes the squared-ReLU gating relu(y_gate)^2 * y_up to Y.
template <int T, int MM, int kSrc, bool kPair = false>
__device__ __forceinline__ void gemv_dpp_body(const uint8_t* __restrict__ packed, const float* __restrict__ gamma,
                                              int N, float* __restrict__ Y, int32_t* __restrict__ acc_out, int rb0,
                                              const void* __restrict__ X, const float* __restrict__ absmax_in, int M,
                                              int K, int K_pad, int chunks, int8_t* __restrict__ xq_out,
                                              float* __restrict__ absmax_out, const float* __restrict__ gain,
                                              float eps, const uint8_t* __restrict__ packed2 = nullptr,
                                              const float* __restrict__ gamma2 = nullptr) {
  static_assert(MM >= 1 && MM <= 4, "one to four tokens");
  static_assert(!kPair || kSrc != 0, "the gated pair is formed by the fused (x input) calls only");
  constexpr bool kNorm = src_norm(kSrc);
  constexpr int UA = DppShape<MM, kSrc>::UA;
  constexpr int NA = (T + UA - 1) / UA;    // activation pieces per lane
  constexpr int kParts = DppShape<MM, kSrc>::kParts;
  constexpr int kPartElems = 16 / kParts;  // elements per 16-byte load
  __shared__ v4i red[(kPair ? 2 : 1) * 16 * 64];
  __shared__ float amax_w[16][4];
  __shared__ double ss_w[kNorm ? 16 : 1][4];
  const int W = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int c0 = wave * T;
  const uint4* wsrc = reinterpret_cast<const uint4*>(packed) + (size_t)rb0 * chunks * 64 + lane;
  const uint4* wsrc2 = kPair ? reinterpret_cast<const uint4*>(packed2) + (size_t)rb0 * chunks * 64 + lane : nullptr;
  const int pm = r % MM, pq = r / MM;
  const int pu = min(pq / 4, UA - 1), pi = pq % 4;
  // Piece j of this lane is one the wave uses: not a repeat (lanes past 4 UA pieces per
  // token), inside the wave's run, and not a clamped tile past the matrix.  Every
  // (token, column) is the piece of exactly one such lane in the workgroup.  The fused
  // forms load x (and the gain) for these pieces only; the others hold zeros, which
  // change neither the absmax nor the sum of squares and never reach a computed tile.
  auto own = [&](int j) { return pq < 4 * UA && j * UA + pu < T && c0 + j * UA + pu < chunks; };

  // every activation load first (their wait then does not wait for the weights), then
  // every weight load of the run.  A compute unit issues the memory instructions of its
  // waves oldest first, so with several workgroups per unit the activation loads of the
  // younger ones wait behind the weight loads of the older ones, and their barrier with
  // them.  kSrcPrio lifts the wave's priority over the activation loads alone, so they
  // go out ahead of weight loads that older waves have not yet issued.  kSrcLead (long
  // runs, at most two workgroups per unit) also issues the first weight tiles of the run
  // right behind the activation loads, so the unit's weight stream starts before the
  // barrier.
  if constexpr (src_prio(kSrc)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(3);
    __builtin_amdgcn_sched_barrier(0);
  }
  uint4 raw[NA][kParts];
  static_for<NA>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    const int col = min(c0 + j * UA + pu, chunks - 1) * kTileCols + 64 * g + 16 * pi;
    if constexpr (kSrc == 0) {
      raw[j][0] = *reinterpret_cast<const uint4*>(static_cast<const int8_t*>(X) + (size_t)pm * K_pad + col);
    } else {
      constexpr int kEB = src_bf16(kSrc) ? 2 : 4;
      const bool ld = own(j);
      static_for<kParts>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        const int e = col + kPartElems * h;
        // K is a multiple of the 16-byte load: a load is wholly inside the row or past
        // it, and pieces past it stay zero
        raw[j][h] = make_uint4(0u, 0u, 0u, 0u);
        if (ld && e + kPartElems <= K)
          raw[j][h] = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(X) + ((size_t)pm * K + e) * kEB);
      });
    }
  });
  // normalising form: the gain of the piece's 16 columns (4 loads; null gain: all ones)
  uint4 graw[kNorm ? NA : 1][4];
  if constexpr (kNorm) {
    if (gain) {
      static_for<NA>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        const int col = min(c0 + j * UA + pu, chunks - 1) * kTileCols + 64 * g + 16 * pi;
        const bool ld = own(j);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int e = col + 4 * h;
          graw[j][h] = make_uint4(0u, 0u, 0u, 0u);
          if (ld) graw[j][h] = *reinterpret_cast<const uint4*>(gain + (e + 4 <= K ? e : K - 4));
        }
      });
    }
  }
  // The fused form issues its weight loads only after the absmax barrier: loads issued
  // earlier by any wave of the compute unit delay the activation loads queued behind
  // them, and with them the barrier (measured: up to 5 us on 58.7 MB matrices).  With one
  // workgroup per compute unit (kSrcEarly, chosen by the planner) nothing else queues on
  // the unit: after a barrier that only orders the issue (every wave's activation loads
  // go first) the weights are issued before the activation barrier and stream during it.
  // With up to two workgroups per unit and short runs (kSrcMid) each wave waits for its
  // own activation pieces and then issues its weights, which stream during the
  // conversion, the absmax barrier and the quantisation.
  if constexpr (src_prio(kSrc)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  }
  constexpr int kEarly = (kSrc == 0 || src_early(kSrc) || src_mid(kSrc)) ? T : (src_lead(kSrc) ? (T < kLeadTiles ? T : kLeadTiles) : 0);
  if constexpr (src_early(kSrc)) asm volatile("s_barrier" ::: "memory");
  if constexpr (src_mid(kSrc)) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), other counters at their maxima
  uint4 w[T];
  uint4 w2[kPair ? T : 1];
  static_for<kEarly>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    w[t] = load_nt(wsrc + (size_t)min(c0 + t, chunks - 1) * 64);
    if constexpr (kPair && src_mid(kSrc)) w2[t] = load_nt(wsrc2 + (size_t)min(c0 + t, chunks - 1) * 64);
  });
  __builtin_amdgcn_sched_barrier(0);

  uint4 act[NA];
  float am[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // fused form: absmax of tokens 0..MM-1
  double lss = 0.0;                         // kNorm: sum of x^2 over this lane's pieces
  if constexpr (kSrc == 0) {
    static_for<NA>([&](auto jc) { act[decltype(jc)::value] = raw[decltype(jc)::value][0]; });
  } else {
    float v[NA][16];
    float lmax = 0.0f;
    static_for<NA>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      static_for<kParts>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        const uint32_t d[4] = {raw[j][h].x, raw[j][h].y, raw[j][h].z, raw[j][h].w};
#pragma unroll
        for (int e = 0; e < kPartElems; ++e) {
          constexpr int kBf = src_bf16(kSrc);
          float f;
          if constexpr (kBf) f = __uint_as_float(e & 1 ? (d[e >> 1] & 0xFFFF0000u) : (d[e >> 1] << 16));
          else f = __uint_as_float(d[e]);
          if constexpr (kNorm) {
            lss = fma((double)f, (double)f, lss);  // zero for the pieces the lane does not own
            if (gain) {
              const int q = kPartElems * h + e;  // column offset inside the piece
              const uint4 gq = graw[j][q >> 2];
              const uint32_t gb = (q & 3) == 0 ? gq.x : ((q & 3) == 1 ? gq.y : ((q & 3) == 2 ? gq.z : gq.w));
              f = f * __uint_as_float(gb);
            }
          }
          v[j][kPartElems * h + e] = f;
          lmax = fmaxf(lmax, fabsf(f));
        }
      });
    });
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      float x = pm == m ? lmax : 0.0f;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
      if (lane == 0) amax_w[wave][m] = x;
    }
    lds_barrier();
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      float a = 0.0f;
      for (int w2 = 0; w2 < W; ++w2) a = fmaxf(a, amax_w[w2][m]);
      am[m] = a;
    }
    const float apm = pm == 0 ? am[0] : (pm == 1 ? am[1] : (pm == 2 ? am[2] : am[3]));
    const float sc = apm > 0.0f ? 127.0f / apm : 0.0f;
    static_for<NA>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      uint32_t q[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) q[d] = quant_code4(v[j][4 * d], v[j][4 * d + 1], v[j][4 * d + 2], v[j][4 * d + 3], sc);
      act[j] = make_uint4(q[0], q[1], q[2], q[3]);
      if (blockIdx.x == 0 && own(j)) {
        const int col = min(c0 + j * UA + pu, chunks - 1) * kTileCols + 64 * g + 16 * pi;
        *reinterpret_cast<uint4*>(xq_out + (size_t)pm * K_pad + col) = act[j];
      }
    });
  }
  static_for<T>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    if constexpr (t >= kEarly) w[t] = load_nt(wsrc + (size_t)min(c0 + t, chunks - 1) * 64);
    if constexpr (kPair && !src_mid(kSrc)) w2[t] = load_nt(wsrc2 + (size_t)min(c0 + t, chunks - 1) * 64);
  });
  __builtin_amdgcn_sched_barrier(0);
  // kNorm: the per-token sums of squares are only needed by the rescale: they are reduced
  // here, while the weight loads are in flight, and cross the waves with the partial tiles
  if constexpr (kNorm) {
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      double y = pm == m ? lss : 0.0;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) y += __shfl_xor(y, off, 64);
      if (lane == 0) ss_w[wave][m] = y;
    }
  }

  v4i c = {0, 0, 0, 0};
  v4i c2 = {0, 0, 0, 0};
  static_for<NA>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    static_for<UA>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      constexpr int t = j * UA + u;
      if constexpr (t < T) {
        const bool live = c0 + t < chunks;  // tiles past the matrix decode as 0
        static_for<4>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          constexpr int sft = MM * (4 * u + i);
          const uint32_t word = live ? word_of(w[t], i) : 0u;
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
          c = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, decode16(word), c, 0, 0, 0);
          if constexpr (kPair) {
            const uint32_t word2 = live ? word_of(w2[t], i) : 0u;
            c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, decode16(word2), c2, 0, 0, 0);
          }
        });
      }
    });
  });

  red[wave * 64 + lane] = c;
  if constexpr (kPair) red[(16 + wave) * 64 + lane] = c2;
  __syncthreads();
  // sum the W partial tiles in wave order (exact) and store row block rb0
  if (wave == 0) {
    float asc[4] = {am[0], am[1], am[2], am[3]};  // fused forms: the scale of each token
    if constexpr (kNorm) {
#pragma unroll
      for (int m = 0; m < MM; ++m) {
        double ss = 0.0;
        for (int w2 = 0; w2 < W; ++w2) ss += ss_w[w2][m];
        asc[m] = am[m] > 0.0f ? (float)((double)am[m] / sqrt(ss / (double)K + (double)eps)) : 0.0f;
      }
    }
    if (kSrc != 0 && blockIdx.x == 0 && lane < MM)
      absmax_out[lane] = lane == 0 ? asc[0] : (lane == 1 ? asc[1] : (lane == 2 ? asc[2] : asc[3]));
    v4i sum = red[lane];
    for (int w2 = 1; w2 < W; ++w2) sum += red[w2 * 64 + lane];
    v4i sum2 = {0, 0, 0, 0};
    if constexpr (kPair) {
      sum2 = red[16 * 64 + lane];
      for (int w2 = 1; w2 < W; ++w2) sum2 += red[(16 + w2) * 64 + lane];
    }
    const int n = rb0 * kTileRows + r;
    if (n < N) {
      const float gm = gamma[0];
      const float gm2 = kPair ? gamma2[0] : 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * g + v;
        if (m < M) {
          const float a = kSrc == 0 ? absmax_in[m] : (m == 0 ? asc[0] : (m == 1 ? asc[1] : (m == 2 ? asc[2] : asc[3])));
          const float y = (float)sum[v] * gm * a * (1.0f / 127.0f);
          if constexpr (kPair) {
            Y[(size_t)m * N + n] = gated_relu2(y, (float)sum2[v] * gm2 * a * (1.0f / 127.0f));
          } else {
            if (acc_out) acc_out[(size_t)m * N + n] = sum[v];
            if (Y) Y[(size_t)m * N + n] = y;
          }
        }
      }
    }
  }
}

template <int T, int MM, int kSrc>
__global__ __launch_bounds__(1024) void k_gemv_dpp(const uint8_t* __restrict__ packed,
                                                  const float* __restrict__ gamma, const void* __restrict__ X,
                                                  const float* __restrict__ absmax_in, int M, int N, int K,
                                                  int K_pad, int chunks, float* __restrict__ Y,
                                                  int32_t* __restrict__ acc_out, int8_t* __restrict__ xq_out,
                                                  float* __restrict__ absmax_out) {
  gemv_dpp_body<T, MM, kSrc>(packed, gamma, N, Y, acc_out, (int)blockIdx.x, X, absmax_in, M, K, K_pad, chunks,
                             xq_out, absmax_out, nullptr, 0.0f);
}

// The normalising form (kSrc 3 / 4) of the same kernel, with the gain and eps.
template <int T, int MM, int kSrc>
__global__ __launch_bounds__(1024) void k_gemv_dpp_norm(const uint8_t* __restrict__ packed,
                                                       const float* __restrict__ gamma, const void* __restrict__ X,
                                                       const float* __restrict__ gain, float eps, int M, int N, int K,
                                                       int K_pad, int chunks, float* __restrict__ Y,
                                                       int32_t* __restrict__ acc_out, int8_t* __restrict__ xq_out,
                                                       float* __restrict__ absmax_out) {
  gemv_dpp_body<T, MM, kSrc>(packed, gamma, N, Y, acc_out, (int)blockIdx.x, X, nullptr, M, K, K_pad, chunks, xq_out,
                             absmax_out, gain, eps);
}

// The gate / up pair with the squared-ReLU gating (kSrc 1..4; gain null unless 3 / 4).
template <int T, int MM, int kSrc>
__global__ __launch_bounds__(1024) void k_gemv_dpp_pair(const uint8_t* __restrict__ packed,
                                                       const float* __restrict__ gamma,
                                                       const uint8_t* __restrict__ packed2,
                                                       const float* __restrict__ gamma2, const void* __restrict__ X,
                                                       const float* __restrict__ gain, float eps, int M, int N, int K,
                                                       int K_pad, int chunks, float* __restrict__ H,
                                                       int8_t* __restrict__ xq_out, float* __restrict__ absmax_out) {
  gemv_dpp_body<T, MM, kSrc, true>(packed, gamma, N, H, nullptr, (int)blockIdx.x, X, nullptr, M, K, K_pad, chunks,
                                   xq_out, absmax_out, gain, eps, packed2, gamma2);
}

// Squared-ReLU gating of separately computed outputs (the path for shapes the pair kernel
// does not take): h = relu(y_gate)^2 * y_up; h may be y_gate itself.
__global__ __launch_bounds__(256) void k_gated_relu2(const float* yg, const float* __restrict__ yu, int64_t count,
                                                     float* h) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256)
    h[i] = gated_relu2(yg[i], yu[i]);
}

// Grouped form: workgroups take the row blocks of the group's matrices one after another.
template <int T, int MM, int kSrc>
__global__ __launch_bounds__(1024) void k_gemv_dpp_group(const MatGroup grp, const void* __restrict__ X, int M,
                                                        int K, int K_pad, int chunks, int8_t* __restrict__ xq_out,
                                                        float* __restrict__ absmax_out, const float* __restrict__ gain,
                                                        float eps) {
  int mat = 0;  // uniform
#pragma unroll
  for (int k = 0; k + 1 < kMaxGroup; ++k)
    if (k + 1 < grp.count && (int)blockIdx.x >= grp.rb_end[k]) mat = k + 1;
  const uint8_t* packed = grp.packed[0];
  const float* gamma = grp.gamma[0];
  float* Y = grp.Y[0];
  int32_t* acc_out = grp.acc[0];
  int N = grp.N[0], rb_base = 0;
#pragma unroll
  for (int k = 1; k < kMaxGroup; ++k)
    if (mat == k) {
      packed = grp.packed[k];
      gamma = grp.gamma[k];
      Y = grp.Y[k];
      acc_out = grp.acc[k];
      N = grp.N[k];
      rb_base = grp.rb_end[k - 1];
    }
  gemv_dpp_body<T, MM, kSrc>(packed, gamma, N, Y, acc_out, (int)blockIdx.x - rb_base, X, nullptr, M, K, K_pad,
                             chunks, xq_out, absmax_out, gain, eps);
}

// ---------------------------------------------------------------------------------------
// k_gemv_dppm (5..16 tokens, int8 activations): the register-run structure of k_gemv_dpp
// for a token group of MM = 8 or 16 (tokens M..MM-1 repeat token M-1; their rows are
// never stored).  A tile needs 4 MM activation pieces per 16-lane row, i.e. RA = MM / 4
// registers: register q of lane (r, g) holds piece p = 16 q + r = token p % MM of step
// p / MM; step i reads register MM i / 16 shifted down (MM i) % 16 lanes.  Each wave
// covers RB row blocks over its run of T tiles, so one set of activation registers
// feeds RB weight tiles.
template <int T, int MM, int RB>
__device__ __forceinline__ void gemv_dppm_body(const uint8_t* __restrict__ packed, const float* __restrict__ gamma,
                                               const int8_t* __restrict__ Xq, const float* __restrict__ absmax, int M,
                                               int N, int K_pad, int chunks, int rblocks, float* __restrict__ Y,
                                               int32_t* __restrict__ acc_out, int blk) {
  static_assert(MM == 8 || MM == 16, "token group of 8 or 16");
  constexpr int RA = MM / 4;
  __shared__ v4i red[16 * 64];  // W * RB <= 16 partial tiles
  const int W = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int rb0 = blk * RB;
  const int c0 = wave * T;
  const uint4* wsrc[RB];
#pragma unroll
  for (int j = 0; j < RB; ++j)
    wsrc[j] = reinterpret_cast<const uint4*>(packed) + (size_t)min(rb0 + j, rblocks - 1) * chunks * 64 + lane;

  uint4 a[T][RA];
  uint4 w[T][RB];
  static_for<T>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    const int tile = min(c0 + t, chunks - 1);
#pragma unroll
    for (int q = 0; q < RA; ++q) {
      const int p = 16 * q + r;
      const int m = min(p % MM, M - 1), i = p / MM;
      a[t][q] = *reinterpret_cast<const uint4*>(Xq + (size_t)m * K_pad + tile * kTileCols + 64 * g + 16 * i);
    }
#pragma unroll
    for (int j = 0; j < RB; ++j) w[t][j] = load_nt(wsrc[j] + (size_t)tile * 64);
  });
  __builtin_amdgcn_sched_barrier(0);

  v4i c[RB];
#pragma unroll
  for (int j = 0; j < RB; ++j) c[j] = (v4i){0, 0, 0, 0};
  static_for<T>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    const bool live = c0 + t < chunks;  // tiles past the matrix decode as 0
    static_for<4>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int q = MM * i / 16, sft = (MM * i) % 16;
      v4i av;
      av.x = row_shl<sft>((int)a[t][q].x);
      av.y = row_shl<sft>((int)a[t][q].y);
      av.z = row_shl<sft>((int)a[t][q].z);
      av.w = row_shl<sft>((int)a[t][q].w);
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const uint32_t word = live ? word_of(w[t][j], i) : 0u;
        c[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, decode16(word), c[j], 0, 0, 0);
      }
    });
  });
#pragma unroll
  for (int j = 0; j < RB; ++j) red[(wave * RB + j) * 64 + lane] = c[j];
  __syncthreads();
  const float gm = gamma[0];
  for (int j = wave; j < RB; j += W) {
    if (rb0 + j >= rblocks) continue;
    v4i sum = red[j * 64 + lane];
    for (int w2 = 1; w2 < W; ++w2) sum += red[(w2 * RB + j) * 64 + lane];
    const int n = (rb0 + j) * kTileRows + r;
    if (n >= N) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g + v;
      if (m < M) {
        if (acc_out) acc_out[(size_t)m * N + n] = sum[v];
        if (Y) Y[(size_t)m * N + n] = (float)sum[v] * gm * absmax[m] * (1.0f / 127.0f);
      }
    }
  }
}

template <int T, int MM, int RB>
__global__ __launch_bounds__(1024) void k_gemv_dppm(const uint8_t* __restrict__ packed,
                                                   const float* __restrict__ gamma, const int8_t* __restrict__ Xq,
                                                   const float* __restrict__ absmax, int M, int N, int K_pad,
                                                   int chunks, int rblocks, float* __restrict__ Y,
                                                   int32_t* __restrict__ acc_out) {
  gemv_dppm_body<T, MM, RB>(packed, gamma, Xq, absmax, M, N, K_pad, chunks, rblocks, Y, acc_out, (int)blockIdx.x);
}

// Matrices that share one quantised input (the 5..16-token grouped call): workgroups
// [wg_end[j-1], wg_end[j]) take the row blocks of matrix j, RB at a time.
struct DppmGroup {
  int count;
  int wg_end[kMaxGroup];
  int N[kMaxGroup];
  int rblocks[kMaxGroup];
  const uint8_t* packed[kMaxGroup];
  const float* gamma[kMaxGroup];
  float* Y[kMaxGroup];
  int32_t* acc[kMaxGroup];
};

template <int T, int MM, int RB>
__global__ __launch_bounds__(1024) void k_gemv_dppm_group(const DppmGroup grp, const int8_t* __restrict__ Xq,
                                                         const float* __restrict__ absmax, int M, int K_pad,
                                                         int chunks) {
  int mat = 0;  // uniform
#pragma unroll
  for (int k = 0; k + 1 < kMaxGroup; ++k)
    if (k + 1 < grp.count && (int)blockIdx.x >= grp.wg_end[k]) mat = k + 1;
  const uint8_t* packed = grp.packed[0];
  const float* gamma = grp.gamma[0];
  float* Y = grp.Y[0];
  int32_t* acc_out = grp.acc[0];
  int N = grp.N[0], rblocks = grp.rblocks[0], wg_base = 0;
#pragma unroll
  for (int k = 1; k < kMaxGroup; ++k)
    if (mat == k) {
      packed = grp.packed[k];
      gamma = grp.gamma[k];
      Y = grp.Y[k];
      acc_out = grp.acc[k];
      N = grp.N[k];
      rblocks = grp.rblocks[k];
      wg_base = grp.wg_end[k - 1];
    }
  gemv_dppm_body<T, MM, RB>(packed, gamma, Xq, absmax, M, N, K_pad, chunks, rblocks, Y, acc_out,
                            (int)blockIdx.x - wg_base);
}

// ---------------------------------------------------------------------------------------
// k_gemv_fq16: the fused form for 5..16 tokens (bf16 x): quantiser and decode in one
// launch.  Every workgroup quantises the whole M x K input into LDS: token m belongs to
// wave m % W, which loads its row with coalesced 16-byte pieces (lane l takes pieces
// l, l + 64, ...), takes the absmax over them with a wave reduction (no barrier: the wave
// holds the whole row) and writes the codes to LDS row m, with the standalone quantiser's
// arithmetic.  The weights of the workgroup (RB row blocks, a run of T tiles per wave) are
// issued right behind the row loads and stream in meanwhile.  One barrier, then the A operand of
// step i of tile t comes from LDS (lane (r, g): token r, columns 256 t + 64 g + 16 i) and
// the B operand from the weight registers, as in k_gemv_dppm.  Rows of tokens >= M are
// never written or stored.  Workgroup 0 also stores xq (zero-padded to K_pad) and absmax.
// KL = loads per lane per token row (16-byte pieces l + 64 k < K / 8).
template <int W, int T, int RB, int KL>
__global__ __launch_bounds__(W * 64) void k_gemv_fq16(const DppmGroup grp, const uint16_t* __restrict__ X, int M, int K,
                                                     int K_pad, int chunks, int8_t* __restrict__ xq_out,
                                                     float* __restrict__ absmax_out) {
  constexpr int TPW = (16 + W - 1) / W;  // token rows per wave
  extern __shared__ __attribute__((aligned(16))) uint8_t act[];  // [16][K_pad + 16] int8 codes
  __shared__ v4i red[W * RB * 64];
  __shared__ float amax_s[16];
  int mat = 0;  // uniform
#pragma unroll
  for (int k = 0; k + 1 < kMaxGroup; ++k)
    if (k + 1 < grp.count && (int)blockIdx.x >= grp.wg_end[k]) mat = k + 1;
  const uint8_t* packed = grp.packed[0];
  const float* gamma = grp.gamma[0];
  float* Y = grp.Y[0];
  int32_t* acc_out = grp.acc[0];
  int N = grp.N[0], rblocks = grp.rblocks[0], wg_base = 0;
#pragma unroll
  for (int k = 1; k < kMaxGroup; ++k)
    if (mat == k) {
      packed = grp.packed[k];
      gamma = grp.gamma[k];
      Y = grp.Y[k];
      acc_out = grp.acc[k];
      N = grp.N[k];
      rblocks = grp.rblocks[k];
      wg_base = grp.wg_end[k - 1];
    }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int rb0 = ((int)blockIdx.x - wg_base) * RB;
  const int c0 = wave * T;
  const int stride = K_pad + 16;

  // the wave's token rows first (L2 hits that return while the weights stream from HBM):
  // pieces past the row are not loaded and stay zero
  const int pieces = K / 8;
  uint4 x[TPW][KL];
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int m = min(wave + W * q, M - 1);
#pragma unroll
    for (int k = 0; k < KL; ++k) {
      const int p = lane + 64 * k;
      x[q][k] = p < pieces ? reinterpret_cast<const uint4*>(X + (size_t)m * K)[p] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // then every weight load of the wave's run, for its RB row blocks
  uint4 w[T][RB];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int j = 0; j < RB; ++j)
      w[t][j] = load_nt(reinterpret_cast<const uint4*>(packed) +
                        ((size_t)min(rb0 + j, rblocks - 1) * chunks + min(c0 + t, chunks - 1)) * 64 + lane);
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int m = wave + W * q;
    if (m >= M) continue;  // uniform across the wave
    // absmax: the largest |x| bit pattern, two bf16 values per 32-bit word (for values that
    // are not NaN the order of the patterns with the sign cleared is the order of |x|)
    u16x2 mx = {0, 0};
#pragma unroll
    for (int k = 0; k < KL; ++k) {
      const uint32_t d[4] = {x[q][k].x, x[q][k].y, x[q][k].z, x[q][k].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, d[e] & 0x7FFF7FFFu));
    }
    uint32_t mb = max((uint32_t)mx.x, (uint32_t)mx.y);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, off, 64));
    float a = __uint_as_float(mb << 16);
    if (mb > 0x7F80u) {
      // a NaN in the row: the float maximum, which passes over NaN as the standalone
      // quantiser's does
      a = 0.0f;
#pragma unroll
      for (int k = 0; k < KL; ++k) {
        const uint32_t d[4] = {x[q][k].x, x[q][k].y, x[q][k].z, x[q][k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a = fmaxf(a, fmaxf(fabsf(__uint_as_float(d[e] << 16)), fabsf(__uint_as_float(d[e] & 0xFFFF0000u))));
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    }
    const float sc = a > 0.0f ? 127.0f / a : 0.0f;
    if (lane == 0) {
      amax_s[m] = a;
      if (blockIdx.x == 0) absmax_out[m] = a;
    }
#pragma unroll
    for (int k = 0; k < KL; ++k) {
      const int p = lane + 64 * k;
      if (p >= pieces) continue;
      const uint32_t d[4] = {x[q][k].x, x[q][k].y, x[q][k].z, x[q][k].w};
      const uint32_t lo = quant_code4(__uint_as_float(d[0] << 16), __uint_as_float(d[0] & 0xFFFF0000u),
                                      __uint_as_float(d[1] << 16), __uint_as_float(d[1] & 0xFFFF0000u), sc);
      const uint32_t hi = quant_code4(__uint_as_float(d[2] << 16), __uint_as_float(d[2] & 0xFFFF0000u),
                                      __uint_as_float(d[3] << 16), __uint_as_float(d[3] & 0xFFFF0000u), sc);
      *reinterpret_cast<uint2*>(act + m * stride + 8 * p) = make_uint2(lo, hi);
      if (blockIdx.x == 0) *reinterpret_cast<uint2*>(xq_out + (size_t)m * K_pad + 8 * p) = make_uint2(lo, hi);
    }
    // padding columns K .. K_pad - 1 of xq are zero (the LDS copy needs none: the packed
    // padding codes decode to 0)
    if (blockIdx.x == 0)
      for (int p = pieces + lane; p < K_pad / 8; p += 64)
        *reinterpret_cast<uint2*>(xq_out + (size_t)m * K_pad + 8 * p) = make_uint2(0u, 0u);
  }
  lds_barrier();

  v4i c[RB];
#pragma unroll
  for (int j = 0; j < RB; ++j) c[j] = (v4i){0, 0, 0, 0};
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int tile = min(c0 + t, chunks - 1);
    const bool live = c0 + t < chunks;  // tiles past the matrix decode as 0
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v4i av = *reinterpret_cast<const v4i*>(act + r * stride + tile * kTileCols + 64 * g + 16 * i);
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const uint32_t word = live ? word_of(w[t][j], i) : 0u;
        c[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, decode16(word), c[j], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < RB; ++j) red[(wave * RB + j) * 64 + lane] = c[j];
  lds_barrier();
  const float gm = gamma[0];
  for (int j = wave; j < RB; j += W) {
    if (rb0 + j >= rblocks) continue;
    v4i sum = red[j * 64 + lane];
    for (int w2 = 1; w2 < W; ++w2) sum += red[(w2 * RB + j) * 64 + lane];
    const int n = (rb0 + j) * kTileRows + r;
    if (n >= N) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g + v;
      if (m < M) {
        if (acc_out) acc_out[(size_t)m * N + n] = sum[v];
        if (Y) Y[(size_t)m * N + n] = (float)sum[v] * gm * amax_s[m] * (1.0f / 127.0f);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
struct Args {
  const uint8_t* packed;
  const float* gamma;
  const void* X;
  const float* absmax;
  int M, N, K, K_pad, chunks, rblocks;
  float* Y;
  int32_t* acc;
  int8_t* xq_out;
  float* absmax_out;
  const float* gain = nullptr;  // normalising sources only
  float eps = 0.0f;
};

template <int W, int U, int NB, int S, int kSrc>
hipError_t launch_lds(const Args& a, hipStream_t s) {
  const size_t lds = (size_t)a.M * (a.K_pad + 16);
  hipLaunchKernelGGL((k_gemv_lds<W, U, NB, S, kSrc>), dim3(a.rblocks), dim3(W * 64), lds, s, a.packed, a.gamma, a.X,
                     a.M, a.N, a.K, a.K_pad, a.chunks, a.rblocks, a.Y, a.acc, a.xq_out, a.absmax_out);
  return hipGetLastError();
}

template <int W, int U, int NB, int kSrc>
hipError_t launch_lds_s(int S, const Args& a, hipStream_t s) {
  switch (S) {
    case 1: return launch_lds<W, U, NB, 1, kSrc>(a, s);
    case 2: return launch_lds<W, U, NB, 2, kSrc>(a, s);
    case 3: return launch_lds<W, U, NB, 3, kSrc>(a, s);
    default: return launch_lds<W, U, NB, 4, kSrc>(a, s);
  }
}

template <int kSrc>
hipError_t launch_lds_w(int W, int S, const Args& a, hipStream_t s) {
  switch (W) {
    case 16: return launch_lds_s<16, 1, 3, kSrc>(S, a, s);
    case 8: return launch_lds_s<8, 2, 2, kSrc>(S, a, s);
    case 4: return launch_lds_s<4, 2, 3, kSrc>(S, a, s);
    case 2: return launch_lds_s<2, 2, 3, kSrc>(S, a, s);
    default: return launch_lds_s<1, 2, 3, kSrc>(S, a, s);
  }
}

template <int W, int RB, int U, int NB, int TG = 1>
hipError_t launch_reg(const Args& a, hipStream_t s) {
  const unsigned groups = (unsigned)((a.rblocks + RB - 1) / RB);
  hipLaunchKernelGGL((k_gemv_reg<W, RB, U, NB, TG>), dim3(groups), dim3(W * 64), 0, s, a.packed, a.gamma,
                     static_cast<const int8_t*>(a.X), a.absmax, a.M, a.N, a.K_pad, a.chunks, a.rblocks, a.Y, a.acc);
  return hipGetLastError();
}

template <int RB, int U, int NB>
hipError_t launch_reg_w(int W, const Args& a, hipStream_t s) {
  switch (W) {
    case 16: return launch_reg<16, RB, U, NB>(a, s);
    case 8: return launch_reg<8, RB, U, NB>(a, s);
    case 4: return launch_reg<4, RB, U, NB>(a, s);
    case 2: return launch_reg<2, RB, U, NB>(a, s);
    default: return launch_reg<1, RB, U, NB>(a, s);
  }
}

// 17..64 tokens: token groups of 16 and RB row blocks per workgroup; the planner keeps
// W * RB * TG <= 32 (the partial-tile buffer is W * RB * TG KiB of LDS)
template <int TG, int RB>
hipError_t launch_reg_tg_rb(int W, const Args& a, hipStream_t s) {
  if constexpr (8 * RB * TG <= 32)
    if (W == 8) return launch_reg<8, RB, 1, 2, TG>(a, s);
  if constexpr (4 * RB * TG <= 32)
    if (W == 4) return launch_reg<4, RB, 1, 2, TG>(a, s);
  if (W == 2) return launch_reg<2, RB, 1, 2, TG>(a, s);
  if (W == 1) return launch_reg<1, RB, 1, 2, TG>(a, s);
  return hipErrorInvalidConfiguration;  // not planned
}
template <int TG>
hipError_t launch_reg_tg_w(int W, int RB, const Args& a, hipStream_t s) {
  if (RB == 4) return launch_reg_tg_rb<TG, 4>(W, a, s);
  if (RB == 2) return launch_reg_tg_rb<TG, 2>(W, a, s);
  return launch_reg_tg_rb<TG, 1>(W, a, s);
}

// Fused forms hold the raw activation pieces in registers until the barrier: limit them
// to 8 sixteen-byte loads per lane, or 12 with the 4 gain loads of each piece.
constexpr bool dpp_fits_n(int T, int M, int src) {
  if (src == 0) return true;
  const int ua = 16 / (4 * M), parts = src_bf16(src) ? 2 : 4, na = (T + ua - 1) / ua;
  return src_norm(src) ? na * (parts + 4) <= 12 : na * parts <= 8;
}
template <int T, int MM, int kSrc>
constexpr bool dpp_fits() {
  return dpp_fits_n(T, MM, kSrc);
}


template <int T, int MM, int kSrc>
hipError_t launch_dpp(int W, const Args& a, hipStream_t s, const MatGroup* grp = nullptr) {
  if constexpr (dpp_fits<T, MM, kSrc>()) {
    if (grp) {
      if constexpr (kSrc != 0) {
        hipLaunchKernelGGL((k_gemv_dpp_group<T, MM, kSrc>), dim3(grp->rb_end[grp->count - 1]), dim3(W * 64), 0, s,
                           *grp, a.X, a.M, a.K, a.K_pad, a.chunks, a.xq_out, a.absmax_out, a.gain, a.eps);
        return hipGetLastError();
      }
      return hipErrorInvalidConfiguration;  // groups are formed by the fused (x input) call only
    }
    if constexpr (src_norm(kSrc)) {
      hipLaunchKernelGGL((k_gemv_dpp_norm<T, MM, kSrc>), dim3(a.rblocks), dim3(W * 64), 0, s, a.packed, a.gamma, a.X,
                         a.gain, a.eps, a.M, a.N, a.K, a.K_pad, a.chunks, a.Y, a.acc, a.xq_out, a.absmax_out);
    } else {
      hipLaunchKernelGGL((k_gemv_dpp<T, MM, kSrc>), dim3(a.rblocks), dim3(W * 64), 0, s, a.packed, a.gamma, a.X,
                         a.absmax, a.M, a.N, a.K, a.K_pad, a.chunks, a.Y, a.acc, a.xq_out, a.absmax_out);
    }
    return hipGetLastError();
  } else {
    return hipErrorInvalidConfiguration;  // not planned (dpp_fused_ok)
  }
}

// Supported dpp run lengths (K tiles per wave); returns the smallest one >= t, or 0.
constexpr int kDppRuns[] = {1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 14, 16};
int64_t dpp_run(int64_t t) {
  for (int r : kDppRuns)
    if (r >= t) return r;
  return 0;
}

template <int T, int kSrc>
hipError_t launch_dpp_m(int M, int W, const Args& a, hipStream_t s, const MatGroup* grp) {
  switch (M) {
    case 1: return launch_dpp<T, 1, kSrc>(W, a, s, grp);
    case 2: return launch_dpp<T, 2, kSrc>(W, a, s, grp);
    case 3: return launch_dpp<T, 3, kSrc>(W, a, s, grp);
    default: return launch_dpp<T, 4, kSrc>(W, a, s, grp);
  }
}

template <int kSrc>
hipError_t launch_dpp_run(int T, int M, int W, const Args& a, hipStream_t s, const MatGroup* grp = nullptr) {
  switch (T) {
    case 1: return launch_dpp_m<1, kSrc>(M, W, a, s, grp);
    case 2: return launch_dpp_m<2, kSrc>(M, W, a, s, grp);
    case 3: return launch_dpp_m<3, kSrc>(M, W, a, s, grp);
    case 4: return launch_dpp_m<4, kSrc>(M, W, a, s, grp);
    case 5: return launch_dpp_m<5, kSrc>(M, W, a, s, grp);
    case 6: return launch_dpp_m<6, kSrc>(M, W, a, s, grp);
    case 7: return launch_dpp_m<7, kSrc>(M, W, a, s, grp);
    case 8: return launch_dpp_m<8, kSrc>(M, W, a, s, grp);
    case 10: return launch_dpp_m<10, kSrc>(M, W, a, s, grp);
    case 12: return launch_dpp_m<12, kSrc>(M, W, a, s, grp);
    case 14: return launch_dpp_m<14, kSrc>(M, W, a, s, grp);
    default: return launch_dpp_m<16, kSrc>(M, W, a, s, grp);
  }
}

// One token only (the priority form is planned for M = 1).
template <int kSrc>
hipError_t launch_dpp_prio(int T, int W, const Args& a, hipStream_t s) {
  switch (T) {
    case 1: return launch_dpp<1, 1, kSrc>(W, a, s);
    case 2: return launch_dpp<2, 1, kSrc>(W, a, s);
    case 3: return launch_dpp<3, 1, kSrc>(W, a, s);
    case 4: return launch_dpp<4, 1, kSrc>(W, a, s);
    case 5: return launch_dpp<5, 1, kSrc>(W, a, s);
    case 6: return launch_dpp<6, 1, kSrc>(W, a, s);
    case 7: return launch_dpp<7, 1, kSrc>(W, a, s);
    case 8: return launch_dpp<8, 1, kSrc>(W, a, s);
    case 10: return launch_dpp<10, 1, kSrc>(W, a, s);
    case 12: return launch_dpp<12, 1, kSrc>(W, a, s);
    case 14: return launch_dpp<14, 1, kSrc>(W, a, s);
    default: return launch_dpp<16, 1, kSrc>(W, a, s);
  }
}

// One token, runs of 14 or 16 tiles (the lead form's plan).
template <int kSrc>
hipError_t launch_dpp_lead(int T, int W, const Args& a, hipStream_t s) {
  switch (T) {
    case 14: return launch_dpp<14, 1, kSrc>(W, a, s);
    case 16: return launch_dpp<16, 1, kSrc>(W, a, s);
    default: return hipErrorInvalidConfiguration;
  }
}

// Runs of at most four tiles (the forms the planner only picks for short runs).
template <int kSrc>
hipError_t launch_dpp_run4(int T, int M, int W, const Args& a, hipStream_t s, const MatGroup* grp = nullptr) {
  switch (T) {
    case 1: return launch_dpp_m<1, kSrc>(M, W, a, s, grp);
    case 2: return launch_dpp_m<2, kSrc>(M, W, a, s, grp);
    case 3: return launch_dpp_m<3, kSrc>(M, W, a, s, grp);
    case 4: return launch_dpp_m<4, kSrc>(M, W, a, s, grp);
    default: return hipErrorInvalidConfiguration;
  }
}

// The gated pair keeps two weight runs in registers: runs of at most 8 tiles.
constexpr int kPairMaxRun = 8;

template <int T, int MM, int kSrc>
hipError_t launch_pair(int W, const Args& a, const uint8_t* packed2, const float* gamma2, hipStream_t s) {
  if constexpr (dpp_fits<T, MM, kSrc>() && T <= kPairMaxRun) {
    hipLaunchKernelGGL((k_gemv_dpp_pair<T, MM, kSrc>), dim3(a.rblocks), dim3(W * 64), 0, s, a.packed, a.gamma, packed2,
                       gamma2, a.X, a.gain, a.eps, a.M, a.N, a.K, a.K_pad, a.chunks, a.Y, a.xq_out, a.absmax_out);
    return hipGetLastError();
  } else {
    return hipErrorInvalidConfiguration;  // not planned
  }
}

template <int T, int kSrc>
hipError_t launch_pair_m(int M, int W, const Args& a, const uint8_t* p2, const float* g2, hipStream_t s) {
  switch (M) {
    case 1: return launch_pair<T, 1, kSrc>(W, a, p2, g2, s);
    case 2: return launch_pair<T, 2, kSrc>(W, a, p2, g2, s);
    case 3: return launch_pair<T, 3, kSrc>(W, a, p2, g2, s);
    default: return launch_pair<T, 4, kSrc>(W, a, p2, g2, s);
  }
}

template <int kSrc>
hipError_t launch_pair_run(int T, int M, int W, const Args& a, const uint8_t* p2, const float* g2, hipStream_t s) {
  switch (T) {
    case 1: return launch_pair_m<1, kSrc>(M, W, a, p2, g2, s);
    case 2: return launch_pair_m<2, kSrc>(M, W, a, p2, g2, s);
    case 3: return launch_pair_m<3, kSrc>(M, W, a, p2, g2, s);
    case 4: return launch_pair_m<4, kSrc>(M, W, a, p2, g2, s);
    case 5: return launch_pair_m<5, kSrc>(M, W, a, p2, g2, s);
    case 6: return launch_pair_m<6, kSrc>(M, W, a, p2, g2, s);
    case 7: return launch_pair_m<7, kSrc>(M, W, a, p2, g2, s);
    case 8: return launch_pair_m<8, kSrc>(M, W, a, p2, g2, s);
    default: return hipErrorInvalidConfiguration;
  }
}

template <int kSrc>
hipError_t launch_pair_run4(int T, int M, int W, const Args& a, const uint8_t* p2, const float* g2, hipStream_t s) {
  switch (T) {
    case 1: return launch_pair_m<1, kSrc>(M, W, a, p2, g2, s);
    case 2: return launch_pair_m<2, kSrc>(M, W, a, p2, g2, s);
    case 3: return launch_pair_m<3, kSrc>(M, W, a, p2, g2, s);
    case 4: return launch_pair_m<4, kSrc>(M, W, a, p2, g2, s);
    default: return hipErrorInvalidConfiguration;
  }
}

template <int T, int MM, int RB>
hipError_t launch_dppm(int W, const Args& a, hipStream_t s) {
  if (W * RB > 16 || (int64_t)W * T < a.chunks) return hipErrorInvalidConfiguration;  // LDS partials, coverage
  const unsigned groups = (unsigned)((a.rblocks + RB - 1) / RB);
  hipLaunchKernelGGL((k_gemv_dppm<T, MM, RB>), dim3(groups), dim3(W * 64), 0, s, a.packed, a.gamma,
                     static_cast<const int8_t*>(a.X), a.absmax, a.M, a.N, a.K_pad, a.chunks, a.rblocks, a.Y, a.acc);
  return hipGetLastError();
}

template <int T, int MM, int RB>
hipError_t launch_dppm_group(int W, const DppmGroup& g, const int8_t* Xq, const float* absmax, int M, int K_pad,
                             int chunks, hipStream_t s) {
  if (W * RB > 16 || (int64_t)W * T < chunks) return hipErrorInvalidConfiguration;  // LDS partials, coverage
  hipLaunchKernelGGL((k_gemv_dppm_group<T, MM, RB>), dim3(g.wg_end[g.count - 1]), dim3(W * 64), 0, s, g, Xq, absmax, M,
                     K_pad, chunks);
  return hipGetLastError();
}

template <int W, int T, int RB, int KL>
hipError_t launch_fq16_k(const DppmGroup& g, const void* X, int M, int K, int K_pad, int chunks, int8_t* xq_out,
                         float* absmax_out, int64_t lds_bytes, hipStream_t s) {
  if ((int64_t)W * T < chunks || (int64_t)KL * 512 < K) return hipErrorInvalidConfiguration;  // coverage
  auto kern = k_gemv_fq16<W, T, RB, KL>;
  // the LDS limit above 64 KiB is raised once per device for this kernel (a repeated set
  // from a concurrent first call is harmless)
  static std::atomic<uint64_t> raised{0};
  if (lds_bytes > 64 * 1024) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = uint64_t(1) << (dev & 63);
    if (!(raised.load(std::memory_order_relaxed) & bit)) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kMaxFq16Lds);
      if (e != hipSuccess) return e;
      raised.fetch_or(bit, std::memory_order_relaxed);
    }
  }
  hipLaunchKernelGGL(kern, dim3(g.wg_end[g.count - 1]), dim3(W * 64), (unsigned)lds_bytes, s, g,
                     static_cast<const uint16_t*>(X), M, K, K_pad, chunks, xq_out, absmax_out);
  return hipGetLastError();
}

// dpp_fits for the planner.
bool dpp_fused_ok(int64_t T, int64_t M, int src) { return dpp_fits_n((int)T, (int)M, src); }

// waves per workgroup: enough waves in flight without splitting K finer than ~2 tiles
// per wave, and at most ~32 waves per compute unit overall
int pick_waves(int64_t chunks, int64_t groups) {
  int w = 16;
  while (w > 1 && (2 * w > chunks || groups * w > 256 * 32)) w /= 2;
  return w;
}

}  // namespace

// row blocks per workgroup of the token-group decode
static int token_group_rb(int64_t rblocks) { return rblocks >= 1024 ? 4 : (rblocks >= 384 ? 2 : 1); }

bool token_groups_win(int64_t M, int64_t N, int64_t K) {
  // 17..64 tokens.  The token-group decode kernel re-reads every token row once per
  // workgroup from L2 (about 8 TB/s measured); the prefill kernel has one 64-row tile per
  // 192 columns and is bound by the latency of its K loop (about 1.35 us per pair of
  // 256-column chunks with two K groups).  Fitted to 17..64 tokens on 2560 -> 2560 / 6912,
  // 6912 -> 2560, 8192 -> 28672 and 28672 -> 8192; the rule picks the faster path at all
  // 20 measured points (decode 4.3-15 us where the prefill kernel took 11-24 us on the
  // 2B-class shapes; 8192 -> 28672: 18-24 us against 27 us up to 32 tokens, then the
  // prefill kernel; 28672 -> 8192: 22-73 us against 39-79 us).
  if (M <= 16 || M > 64) return false;
  const int64_t K_pad = k_pad(K), chunks = K_pad / kTileCols, rblocks = n_pad(N) / kTileRows;
  const int64_t groups = (rblocks + token_group_rb(rblocks) - 1) / token_group_rb(rblocks);
  const double reread_s = (double)groups * (double)M * (double)K_pad / 8e12;
  const double kloop_s = 1.35e-6 * (double)((chunks + 1) / 2);
  return reread_s < kloop_s;
}

GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, int src) {
  GemvPlan p;
  const int64_t K_pad = k_pad(K);
  const int64_t chunks = K_pad / kTileCols;
  const int64_t rblocks = n_pad(N) / kTileRows;
  // the fused forms read x in whole 16-byte pieces
  const bool k_ok = src == 0 || (src_bf16(src) ? K % 8 == 0 : K % 4 == 0);
  if (M <= 4 && k_ok) {
    // about 32 waves per compute unit over the launch, at least two tiles per wave, then
    // the shortest supported run that covers the row block with at most 16 waves
    int64_t w = std::min<int64_t>(16, std::max<int64_t>(1, 8192 / rblocks));
    w = std::min<int64_t>(w, std::max<int64_t>(1, (chunks + 1) / 2));
    // the fused form waits at a barrier for the activations of every wave of the group:
    // prefer at most 9 waves (measured: 2560 x 6912 at 9 waves 4.8 us, at 14 waves 5.3 us)
    // unless the longer runs that needs would not fit in registers
    const int64_t tries[2] = {src != 0 ? std::min<int64_t>(w, 9) : w, w};
    int64_t runs[3] = {dpp_run((chunks + tries[0] - 1) / tries[0]), dpp_run((chunks + tries[1] - 1) / tries[1]), 0};
    // the normalising sources have no LDS form: else the longest run that fits in registers
    if (src_norm(src))
      for (int r : kDppRuns)
        if (dpp_fused_ok(r, M, src) && (chunks + r - 1) / r <= 16) runs[2] = r;
    for (const int64_t t : runs) {
      if (t > 0 && (chunks + t - 1) / t <= 16 && dpp_fused_ok(t, M, src)) {
        p.dpp = true;
        p.run = (int)t;
        p.waves = (int)((chunks + t - 1) / t);
        p.groups = rblocks;
        p.ok = true;
        // measured on 2B-class shapes: 160 workgroups 4.82 -> 4.38 us; 432 workgroups
        // 4.60 -> 4.91 us (two per unit queue behind each other's weights)
        // (normalising sources: 6912 x 2560 5.46 -> 5.29 us, 2560 x 2560 4.61 -> 4.51 us)
        p.early = src != 0 && rblocks <= 256;
        // measured (bf16 x, M = 1): 2560 x 6912 (432 workgroups, 2-tile runs) 4.63 -> 4.20
        // us, 4096 x 8192 5.30 -> 4.90 us, 8192 x 8192 (4-tile runs) 6.55 -> 6.22 us; with
        // more workgroups per unit or longer runs the activation loads of later
        // workgroups queue behind the weights (8192 x 16384 9.25 -> 9.38 us, 16384 x 8192
        // 9.16 -> 9.92 us, 28672 x 8192 14.1 -> 22.3 us)
        p.mid = src != 0 && !p.early && rblocks <= 512 && t <= 4;
        // one token, more than two workgroups per unit (weights after the barrier):
        // measured (bf16 x) 8192 x 28672 12.95 -> 12.19 us and 13.00 -> 12.35 us in two
        // interleaved runs; no gain at two tokens (16.07 -> 16.12 us), and on 28672 x 8192
        // (512 workgroups) 13.62 -> 14.10 and 13.71 -> 13.69 us, so not taken there
        p.prio = (src == 1 || src == 2) && M == 1 && !p.early && !p.mid && rblocks > 512;
        // one token, at most two workgroups per unit and runs of 14 or 16 tiles: the raised
        // priority plus two weight tiles issued before the barrier (measured, bf16 x,
        // interleaved: 8192 x 28672 13.80 -> 13.25 and 13.60 -> 13.22 us, 6144 x 28672
        // 12.46 -> 12.23 us, 8192 x 32000 19.38 -> 18.95 us; with 8- and 12-tile runs it
        // lost: 8192 x 16384 9.15 -> 9.53 us, 8192 x 24576 11.61 -> 11.83 us)
        p.lead = (src == 1 || src == 2) && M == 1 && !p.early && !p.mid && !p.prio && t >= 14;
        return p;
      }
    }
  }
  // fused form for short rows when the register form does not fit: every workgroup
  // quantises all M*K activations into LDS
  const bool small = M <= 4 && M * (K_pad + 16) <= kMaxLdsActBytes;
  if ((src == 1 || src == 2) && small && k_ok && M * K <= kMaxFusedElems) {
    p.lds_act = true;
    p.rb = 1;
    p.groups = rblocks;
    p.waves = pick_waves(chunks, rblocks);
    const int64_t elems = src_bf16(src) ? 8 : 4;
    const int64_t pieces = M * K / elems;
    // every piece must be covered by at most 4 loads per thread
    while (p.waves < 16 && pieces > 4 * 64 * p.waves) p.waves *= 2;
    p.stage = (int)((pieces + 64 * p.waves - 1) / (64 * p.waves));
    p.ok = p.stage <= 4;
    return p;
  }
  p.lds_act = false;
  p.rb = 1;
  p.ok = src == 0;  // the register paths read int8 activations only
  if (M > 16) {
    // 17..64 tokens: token groups of 16 through k_gemv_reg (N / (16 RB) workgroups where
    // the prefill kernel would have N / 192 tiles).  RB row blocks share each workgroup's
    // activation registers, which divides the L2 re-reads of the token rows by RB, as long
    // as about one workgroup per CU remains (measured, 17..64 tokens: 432 and 512 row
    // blocks fastest with 2, 1792 with 4, 160 with 1).  At most 32 / (RB TG) waves, and the
    // same wave rule as below.
    p.tg = (int)((M + 15) / 16);
    p.rb = token_group_rb(rblocks);
    p.groups = (rblocks + p.rb - 1) / p.rb;
    int cap = 8;
    while (cap * p.rb * p.tg > 32) cap /= 2;
    p.waves = std::min(pick_waves(chunks, p.groups), cap);
    while (p.waves > 1 && chunks < 8 * p.waves && p.groups * (p.waves / 2) >= 1024) p.waves /= 2;
    return p;
  }
  if (M > 4 && chunks <= 16) {
    // 5..16 tokens on short rows: two-tile register runs (a token group of 8 or 16),
    // activation registers shared by two row blocks once there are enough blocks to fill
    // the chip (measured at M = 8, 2560 -> 6912: 5.49 us per-tile loads, 4.40 us here)
    p.dpp = true;
    p.run = 2;
    p.rb = rblocks >= 384 ? 2 : 1;
    p.waves = (int)((chunks + 1) / 2);
    p.groups = (rblocks + p.rb - 1) / p.rb;
    return p;
  }
  if (M > 4 && rblocks >= 4 * 256) p.rb = 4;
  else if (M > 4 && rblocks >= 2 * 256) p.rb = 2;
  p.groups = (rblocks + p.rb - 1) / p.rb;
  p.waves = pick_waves(chunks, p.groups);
  // 5..16 tokens on long rows: runs of at least 8 tiles per wave while the launch keeps
  // 1024 or more waves (measured at M = 8: 8192 x 28672 14.8 -> 13.1 us with 4 waves,
  // 28672 x 8192 15.4 -> 14.9 us with 8; 6912 x 2560 keeps 8, 8192 x 8192 6.6 us either way)
  if (M > 4)
    while (p.waves > 1 && chunks < 8 * p.waves && p.groups * (p.waves / 2) >= 1024) p.waves /= 2;
  return p;
}

hipError_t launch_gemv(const uint8_t* packed, const float* gamma, const int8_t* Xq, const float* absmax,
                       int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, hipStream_t s) {
  const GemvPlan p = plan_gemv(M, N, K, 0);
  Args a{packed, gamma, Xq, absmax, (int)M, (int)N, (int)K, (int)k_pad(K), (int)(k_pad(K) / kTileCols),
         (int)(n_pad(N) / kTileRows), Y, acc, nullptr, nullptr};
  switch (p.tg) {
    case 2: return launch_reg_tg_w<2>(p.waves, p.rb, a, s);
    case 3: return launch_reg_tg_w<3>(p.waves, p.rb, a, s);
    case 4: return launch_reg_tg_w<4>(p.waves, p.rb, a, s);
    default: break;
  }
  if (p.dpp && M > 8) return p.rb == 2 ? launch_dppm<2, 16, 2>(p.waves, a, s) : launch_dppm<2, 16, 1>(p.waves, a, s);
  if (p.dpp && M > 4) return p.rb == 2 ? launch_dppm<2, 8, 2>(p.waves, a, s) : launch_dppm<2, 8, 1>(p.waves, a, s);
  if (p.dpp) return launch_dpp_run<0>(p.run, (int)M, p.waves, a, s);
  if (p.rb == 4) return launch_reg_w<4, 1, 2>(p.waves, a, s);
  if (p.rb == 2) return launch_reg_w<2, 1, 2>(p.waves, a, s);
  return launch_reg_w<1, 2, 2>(p.waves, a, s);
}

hipError_t launch_gemv_fused(const uint8_t* packed, const float* gamma, const void* X, int bf16, int64_t M, int64_t N,
                             int64_t K, float* Y, int32_t* acc, int8_t* Xq_out, float* absmax_out, hipStream_t s,
                             const NormArgs* norm) {
  const int src = (bf16 ? 1 : 2) + (norm ? 2 : 0);
  const GemvPlan p = plan_gemv(M, N, K, src);
  Args a{packed, gamma, X, nullptr, (int)M, (int)N, (int)K, (int)k_pad(K), (int)(k_pad(K) / kTileCols),
         (int)(n_pad(N) / kTileRows), Y, acc, Xq_out, absmax_out, norm ? norm->gain : nullptr,
         norm ? norm->eps : 0.0f};
  if (norm) {
    if (!p.dpp || !p.ok) return hipErrorInvalidConfiguration;  // not planned: the caller checks the plan
    if (p.early)
      return bf16 ? launch_dpp_run<3 + kSrcEarly>(p.run, (int)M, p.waves, a, s)
                  : launch_dpp_run<4 + kSrcEarly>(p.run, (int)M, p.waves, a, s);
    if (p.mid)
      return bf16 ? launch_dpp_run4<3 + kSrcMid>(p.run, (int)M, p.waves, a, s)
                  : launch_dpp_run4<4 + kSrcMid>(p.run, (int)M, p.waves, a, s);
    return bf16 ? launch_dpp_run<3>(p.run, (int)M, p.waves, a, s) : launch_dpp_run<4>(p.run, (int)M, p.waves, a, s);
  }
  if (p.dpp && p.mid)
    return bf16 ? launch_dpp_run4<1 + kSrcMid>(p.run, (int)M, p.waves, a, s)
                : launch_dpp_run4<2 + kSrcMid>(p.run, (int)M, p.waves, a, s);
  if (p.dpp && p.early)
    return bf16 ? launch_dpp_run<1 + kSrcEarly>(p.run, (int)M, p.waves, a, s)
                : launch_dpp_run<2 + kSrcEarly>(p.run, (int)M, p.waves, a, s);
  if (p.dpp && p.prio)
    return bf16 ? launch_dpp_prio<1 + kSrcPrio>(p.run, p.waves, a, s) : launch_dpp_prio<2 + kSrcPrio>(p.run, p.waves, a, s);
  if (p.dpp && p.lead)
    return bf16 ? launch_dpp_lead<1 + kSrcLead>(p.run, p.waves, a, s) : launch_dpp_lead<2 + kSrcLead>(p.run, p.waves, a, s);
  if (p.dpp) return bf16 ? launch_dpp_run<1>(p.run, (int)M, p.waves, a, s) : launch_dpp_run<2>(p.run, (int)M, p.waves, a, s);
  if (bf16) return launch_lds_w<1>(p.waves, p.stage, a, s);
  return launch_lds_w<2>(p.waves, p.stage, a, s);
}

hipError_t launch_gemv_grouped(const GroupMat* mats, int count, const void* X, int bf16, int64_t M, int64_t K,
                               int8_t* Xq_out, float* absmax_out, hipStream_t s, bool* launched,
                               const NormArgs* norm) {
  *launched = false;
  if (count < 1 || count > kMaxGroup || M > 4) return hipSuccess;
  int64_t rb_total = 0;
  for (int j = 0; j < count; ++j) rb_total += n_pad(mats[j].N) / kTileRows;
  const int src = (bf16 ? 1 : 2) + (norm ? 2 : 0);
  const GemvPlan p = plan_gemv(M, rb_total * kTileRows, K, src);
  if (!(p.dpp && p.ok)) return hipSuccess;
  *launched = true;
  MatGroup g{};
  g.count = count;
  int end = 0;
  for (int j = 0; j < count; ++j) {
    end += (int)(n_pad(mats[j].N) / kTileRows);
    g.rb_end[j] = end;
    g.N[j] = (int)mats[j].N;
    g.packed[j] = mats[j].packed;
    g.gamma[j] = mats[j].gamma;
    g.Y[j] = mats[j].Y;
    g.acc[j] = mats[j].acc;
  }
  Args a{nullptr, nullptr, X, nullptr, (int)M, 0, (int)K, (int)k_pad(K), (int)(k_pad(K) / kTileCols), 0,
         nullptr, nullptr, Xq_out, absmax_out, norm ? norm->gain : nullptr, norm ? norm->eps : 0.0f};
  // the weight-issue order the planner picks for the group's total row blocks
  if (p.early) {
    switch (src) {
      case 1: return launch_dpp_run<1 + kSrcEarly>(p.run, (int)M, p.waves, a, s, &g);
      case 2: return launch_dpp_run<2 + kSrcEarly>(p.run, (int)M, p.waves, a, s, &g);
      case 3: return launch_dpp_run<3 + kSrcEarly>(p.run, (int)M, p.waves, a, s, &g);
      default: return launch_dpp_run<4 + kSrcEarly>(p.run, (int)M, p.waves, a, s, &g);
    }
  }
  if (p.mid) {
    switch (src) {
      case 1: return launch_dpp_run4<1 + kSrcMid>(p.run, (int)M, p.waves, a, s, &g);
      case 2: return launch_dpp_run4<2 + kSrcMid>(p.run, (int)M, p.waves, a, s, &g);
      case 3: return launch_dpp_run4<3 + kSrcMid>(p.run, (int)M, p.waves, a, s, &g);
      default: return launch_dpp_run4<4 + kSrcMid>(p.run, (int)M, p.waves, a, s, &g);
    }
  }
  switch (src) {
    case 1: return launch_dpp_run<1>(p.run, (int)M, p.waves, a, s, &g);
    case 2: return launch_dpp_run<2>(p.run, (int)M, p.waves, a, s, &g);
    case 3: return launch_dpp_run<3>(p.run, (int)M, p.waves, a, s, &g);
    default: return launch_dpp_run<4>(p.run, (int)M, p.waves, a, s, &g);
  }
}

hipError_t launch_gemv_grouped_int8(const GroupMat* mats, int count, const int8_t* Xq, const float* absmax, int64_t M,
                                    int64_t K, hipStream_t s, bool* launched) {
  *launched = false;
  const int64_t K_pad = k_pad(K), chunks = K_pad / kTileCols;
  // 5..16 tokens on rows of at most 16 tiles: the register form of k_gemv_dppm for every
  // matrix of the group, in one launch (the single-matrix planner takes the same form)
  if (count < 2 || count > kMaxGroup || M < 5 || M > 16 || chunks > 16) return hipSuccess;
  int64_t rb_total = 0;
  for (int j = 0; j < count; ++j) rb_total += n_pad(mats[j].N) / kTileRows;
  // two row blocks per workgroup once the group fills the chip (the single-matrix rule)
  const int RB = rb_total >= 384 ? 2 : 1;
  DppmGroup g{};
  g.count = count;
  int end = 0;
  for (int j = 0; j < count; ++j) {
    const int rb = (int)(n_pad(mats[j].N) / kTileRows);
    end += (rb + RB - 1) / RB;
    g.wg_end[j] = end;
    g.N[j] = (int)mats[j].N;
    g.rblocks[j] = rb;
    g.packed[j] = mats[j].packed;
    g.gamma[j] = mats[j].gamma;
    g.Y[j] = mats[j].Y;
    g.acc[j] = mats[j].acc;
  }
  const int W = (int)((chunks + 1) / 2);
  *launched = true;
  if (M > 8) return RB == 2 ? launch_dppm_group<2, 16, 2>(W, g, Xq, absmax, (int)M, (int)K_pad, (int)chunks, s)
                            : launch_dppm_group<2, 16, 1>(W, g, Xq, absmax, (int)M, (int)K_pad, (int)chunks, s);
  return RB == 2 ? launch_dppm_group<2, 8, 2>(W, g, Xq, absmax, (int)M, (int)K_pad, (int)chunks, s)
                 : launch_dppm_group<2, 8, 1>(W, g, Xq, absmax, (int)M, (int)K_pad, (int)chunks, s);
}

Fq16Plan plan_fq16(int64_t M, int64_t rb_total, int64_t K, int src) {
  Fq16Plan p;
  // bf16 x in whole 16-byte pieces, 5..16 tokens, rows of at most 7168 columns and at most
  // 64 Ki values quantised by every workgroup.  Eight waves with two token rows each; row
  // blocks shared per workgroup once there are more than about 1.25 workgroups per compute
  // unit (rows up to 4096 columns).  Measured against the quantiser plus the decode
  // (2B-class grouped calls): M = 16, K = 2560: 7.9 -> 6.7 us (Q/K/V), 8.1 -> 6.4 us (O),
  // 9.6 -> 8.7 us (gate/up); M = 8, K = 6912: 8.9 -> 8.2 us; but M = 16, K = 6912 (110 K
  // values per workgroup) 10.4 -> 10.7 us, so the bound on M K.
  if (src != 1 || M < 5 || M > 16 || K % 8 != 0 || K > 7168 || M * K > 65536) return p;
  const int64_t K_pad = k_pad(K), chunks = K_pad / kTileCols;
  p.W = 8;
  p.T = (int)((chunks + 7) / 8);
  if (K <= 4096) {
    p.KL = K <= 2048 ? 4 : 8;
    p.RB = rb_total > 640 ? 4 : (rb_total > 320 ? 2 : 1);
  } else {
    p.KL = 14;
    p.RB = 1;
  }
  p.lds_bytes = 16 * (K_pad + 16);
  p.ok = p.lds_bytes <= kMaxFq16Lds && (int64_t)p.W * p.T >= chunks && (int64_t)p.KL * 512 >= K;
  return p;
}

int64_t fq16_groups(const Fq16Plan& p, const GroupMat* mats, int count) {
  int64_t groups = 0;
  for (int j = 0; j < count; ++j) groups += (n_pad(mats[j].N) / kTileRows + p.RB - 1) / p.RB;
  return groups;
}

hipError_t launch_gemv_fq16(const GroupMat* mats, int count, const void* X, int bf16, int64_t M, int64_t K,
                            int8_t* Xq_out, float* absmax_out, hipStream_t s, bool* launched) {
  *launched = false;
  if (count < 1 || count > kMaxGroup) return hipSuccess;
  int64_t rb_total = 0;
  for (int j = 0; j < count; ++j) rb_total += n_pad(mats[j].N) / kTileRows;
  const Fq16Plan p = plan_fq16(M, rb_total, K, bf16 ? 1 : 2);
  if (!p.ok) return hipSuccess;
  DppmGroup g{};
  g.count = count;
  int end = 0;
  for (int j = 0; j < count; ++j) {
    const int rb = (int)(n_pad(mats[j].N) / kTileRows);
    end += (rb + p.RB - 1) / p.RB;
    g.wg_end[j] = end;
    g.N[j] = (int)mats[j].N;
    g.rblocks[j] = rb;
    g.packed[j] = mats[j].packed;
    g.gamma[j] = mats[j].gamma;
    g.Y[j] = mats[j].Y;
    g.acc[j] = mats[j].acc;
  }
  const int K_pad = (int)k_pad(K), chunks = K_pad / kTileCols;
  *launched = true;
  auto go = [&](auto wc, auto tc, auto rc, auto kc) {
    return launch_fq16_k<decltype(wc)::value, decltype(tc)::value, decltype(rc)::value, decltype(kc)::value>(
        g, X, (int)M, (int)K, K_pad, chunks, Xq_out, absmax_out, p.lds_bytes, s);
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  using I8 = std::integral_constant<int, 8>;
  auto by_rb = [&](auto tc, auto kc) {
    return p.RB == 4 ? go(I8{}, tc, I4{}, kc) : (p.RB == 2 ? go(I8{}, tc, I2{}, kc) : go(I8{}, tc, I1{}, kc));
  };
  if (p.KL == 14) {
    using I14 = std::integral_constant<int, 14>;
    return p.T == 3 ? go(I8{}, std::integral_constant<int, 3>{}, I1{}, I14{}) : go(I8{}, I4{}, I1{}, I14{});
  }
  if (p.T == 1) return p.KL == 4 ? by_rb(I1{}, I4{}) : by_rb(I1{}, I8{});
  return p.KL == 4 ? by_rb(I2{}, I4{}) : by_rb(I2{}, I8{});
}

bool gated_fused_ok(int64_t M, int64_t N, int64_t K, int src) {
  if (M > 4 || src == 0) return false;
  const GemvPlan p = plan_gemv(M, N, K, src);
  return p.dpp && p.ok && p.run <= kPairMaxRun;
}

hipError_t launch_gemv_gated(const uint8_t* packed_gate, const float* gamma_gate, const uint8_t* packed_up,
                             const float* gamma_up, const void* X, int bf16, int64_t M, int64_t N, int64_t K, float* H,
                             int8_t* Xq_out, float* absmax_out, hipStream_t s, const NormArgs* norm) {
  const int src = (bf16 ? 1 : 2) + (norm ? 2 : 0);
  if (!gated_fused_ok(M, N, K, src)) return hipErrorInvalidConfiguration;
  const GemvPlan p = plan_gemv(M, N, K, src);
  Args a{packed_gate, gamma_gate, X, nullptr, (int)M, (int)N, (int)K, (int)k_pad(K), (int)(k_pad(K) / kTileCols),
         (int)(n_pad(N) / kTileRows), H, nullptr, Xq_out, absmax_out, norm ? norm->gain : nullptr,
         norm ? norm->eps : 0.0f};
  // the pair streams two runs per wave: with the mid ordering measured 5.66 -> 5.04 us
  // (2560 x 6912, M = 1), 6.15 -> 5.30 us (M = 2), 6.28 -> 5.93 us (normalised)
  if (p.mid && p.run <= 4) {
    switch (src) {
      case 1: return launch_pair_run4<1 + kSrcMid>(p.run, (int)M, p.waves, a, packed_up, gamma_up, s);
      case 2: return launch_pair_run4<2 + kSrcMid>(p.run, (int)M, p.waves, a, packed_up, gamma_up, s);
      case 3: return launch_pair_run4<3 + kSrcMid>(p.run, (int)M, p.waves, a, packed_up, gamma_up, s);
      default: return launch_pair_run4<4 + kSrcMid>(p.run, (int)M, p.waves, a, packed_up, gamma_up, s);
    }
  }
  switch (src) {
    case 1: return launch_pair_run<1>(p.run, (int)M, p.waves, a, packed_up, gamma_up, s);
    case 2: return launch_pair_run<2>(p.run, (int)M, p.waves, a, packed_up, gamma_up, s);
    case 3: return launch_pair_run<3>(p.run, (int)M, p.waves, a, packed_up, gamma_up, s);
    default: return launch_pair_run<4>(p.run, (int)M, p.waves, a, packed_up, gamma_up, s);
  }
}

hipError_t launch_gated_relu2(const float* y_gate, const float* y_up, int64_t count, float* h, hipStream_t s) {
  const int64_t groups = std::min<int64_t>((count + 255) / 256, 8192);
  hipLaunchKernelGGL(k_gated_relu2, dim3((unsigned)groups), dim3(256), 0, s, y_gate, y_up, count, h);
  return hipGetLastError();
}

}  // namespace bl
