// Weight quantiser: gamma = mean |W| (exact, order-independent) and the ternarise + 2-bit
// pack into the tiled layout of bitlinear.h.
//
// aratech.ae BitNet b1.58 article, "Ternary weights {-1, 0, +1}": the scale is the
// reciprocal of the mean magnitude over the whole tensor, weights are multiplied by it,
// rounded and clamped to [-1, 1].  bhfrc.com news 56965, section 4.1: 2-bit code table.
//
// gamma must be bit-reproducible: one ulp of gamma moves codes near +-gamma/2.  A float
// tree reduction is order-dependent, so the sum of |W| is taken exactly instead: every
// fp32 is sig * 2^(e-150) with a 24-bit significand, so per exponent field e the
// significands add exactly in a uint64 (up to 2^39 entries).  Integer atomics commute,
// so the bins are identical for any schedule.  One thread then forms the exact 320-bit
// sum and divides it by N*K with round-to-nearest-even into fp32.
#include "bl_internal.h"
#include "binary.h"

#include <mutex>

namespace bl {

// Scratch of the no-allocation weight quantiser (bitlinear_quantize_weights_noalloc): the
// exponent bins and 1/gamma, one copy per GPU, held until the process ends.  Host code
// never uses this name as an address: it is resolved per device with hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[kWqWorkspaceBytes];

namespace {

constexpr int kBinThreads = 256;

__global__ __launch_bounds__(64) void k_wq_clear(unsigned long long* bins) {
  for (int i = threadIdx.x; i < kWqBins; i += 64) bins[i] = 0ull;
}

constexpr int kBinCopies = 16;  // LDS copies of the bins: lane l adds into copy l % 16

// hc = this lane's copy: bin b of copy c sits at hc[b * kBinCopies]
__device__ __forceinline__ void bin_add(unsigned long long* hc, float v) {
  const uint32_t bits = __float_as_uint(v) & 0x7FFFFFFFu;
  const uint32_t e = bits >> 23;
  const uint32_t sig = (bits & 0x7FFFFFu) | (e ? 0x800000u : 0u);
  atomicAdd(&hc[(e ? e : 1u) * kBinCopies], (unsigned long long)sig);  // subnormals share the scale of e = 1
}

// LDS histograms (one uint64 bin per exponent field) in 16 interleaved copies, so that
// the lanes of a wave, whose weights mostly share a few exponents, contend four at a
// time rather than all 64 (the 16 copies of a bin span all 32 banks); merged into the
// global bins with one atomic per non-empty bin per workgroup.
__global__ __launch_bounds__(kBinThreads) void k_wq_bins(const float* __restrict__ W, int64_t count,
                                                         int vec4, unsigned long long* __restrict__ bins) {
  __shared__ unsigned long long h[kWqBins * kBinCopies];
  for (int i = threadIdx.x; i < kWqBins * kBinCopies; i += kBinThreads) h[i] = 0ull;
  __syncthreads();
  unsigned long long* hw = h + (threadIdx.x % kBinCopies);
  const int64_t stride = (int64_t)gridDim.x * kBinThreads;
  int64_t start = (int64_t)blockIdx.x * kBinThreads + threadIdx.x;
  int64_t tail_from = 0;
  if (vec4) {
    const int64_t n4 = count >> 2;
    const float4* W4 = reinterpret_cast<const float4*>(W);
    for (int64_t i = start; i < n4; i += stride) {
      const float4 v = W4[i];
      bin_add(hw, v.x);
      bin_add(hw, v.y);
      bin_add(hw, v.z);
      bin_add(hw, v.w);
    }
    tail_from = n4 << 2;
  }
  for (int64_t i = tail_from + start; i < count; i += stride) bin_add(hw, W[i]);
  __syncthreads();
  for (int b = threadIdx.x; b < kWqBins; b += kBinThreads) {
    unsigned long long t = 0;
    for (int c = 0; c < kBinCopies; ++c) t += h[b * kBinCopies + c];
    if (t) atomicAdd(&bins[b], t);
  }
}

// ---- exact finalisation (one thread) -------------------------------------------------
constexpr int kLimbs = 11;  // 352 bits: bins (< 2^63) shifted by up to 253 bits

// Limb w of x, for a w known only at run time: a select chain, so x stays in registers.
__device__ __forceinline__ uint32_t limbs_get(const uint32_t (&x)[kLimbs], int w) {
  uint32_t v = 0;
#pragma unroll
  for (int i = 0; i < kLimbs; ++i) v = i == w ? x[i] : v;
  return v;
}

__global__ __launch_bounds__(64) void k_wq_finalize(const unsigned long long* __restrict__ bins, uint64_t count,
                                                    float* __restrict__ gamma_out, float* __restrict__ inv_out) {
  if (threadIdx.x != 0) return;
  // S = sum_e bins[e] * 2^(e-1), the exact sum of |W| in units of 2^-149.  Every bin is
  // split into 32-bit pieces added to 64-bit per-limb accumulators (254 bins: no
  // overflow), and the carries are propagated once at the end; the loop is unrolled so
  // that every limb index is a constant and the limbs stay in registers.
  uint64_t acc[kLimbs];
#pragma unroll
  for (int i = 0; i < kLimbs; ++i) acc[i] = 0ull;
#pragma unroll
  for (int e = 1; e < 255; ++e) {
    const uint64_t v = bins[e];
    const int sh = e - 1, word = sh >> 5, bit = sh & 31;
    const uint64_t lo = v << bit;
    const uint64_t hi = bit ? v >> (64 - bit) : 0ull;
    acc[word] += lo & 0xFFFFFFFFull;
    if (word + 1 < kLimbs) acc[word + 1] += lo >> 32;
    if (word + 2 < kLimbs) acc[word + 2] += hi;
  }
  uint32_t s[kLimbs];
  uint64_t carry = 0;
#pragma unroll
  for (int i = 0; i < kLimbs; ++i) {
    const uint64_t t = acc[i] + carry;
    s[i] = (uint32_t)t;
    carry = t >> 32;
  }
  float g;
  if (bins[255] != 0ull) {
    g = __builtin_nanf("");  // a non-finite weight: no meaningful scale
  } else {
    // Q = floor(S / count), R = S mod count
    uint32_t q[kLimbs];
    uint64_t r = 0;
    if (count < (1ull << 32)) {
      // one limb at a time: r < count < 2^32, so (r << 32) | limb fits 64 bits
#pragma unroll
      for (int i = kLimbs - 1; i >= 0; --i) {
        const uint64_t cur = (r << 32) | s[i];
        q[i] = (uint32_t)(cur / count);
        r = cur - (uint64_t)q[i] * count;
      }
    } else {
      // restoring binary long division (r < count < 2^63)
#pragma unroll
      for (int i = 0; i < kLimbs; ++i) q[i] = 0u;
      for (int i = kLimbs * 32 - 1; i >= 0; --i) {
        r = (r << 1) | ((limbs_get(s, i >> 5) >> (i & 31)) & 1u);
        if (r >= count) {
          r -= count;
#pragma unroll
          for (int w = 0; w < kLimbs; ++w) q[w] |= w == (i >> 5) ? 1u << (i & 31) : 0u;
        }
      }
    }
    // bit length of Q
    int len = 0;
#pragma unroll
    for (int i = 0; i < kLimbs; ++i) len = q[i] ? 32 * i + 32 - __builtin_clz(q[i]) : len;
    // the mean is (Q + R/count) * 2^-149; keep 24 significant bits, round half to even
    const int shift = len > 24 ? len - 24 : 0;
    // m = bits [shift, shift + 24) of Q: a 64-bit window of limbs shift/32 and shift/32 + 1
    const int w0 = shift >> 5, b0 = shift & 31;
    const uint64_t win = (uint64_t)limbs_get(q, w0) | ((uint64_t)limbs_get(q, w0 + 1) << 32);
    uint32_t m = (uint32_t)(win >> b0) & 0xFFFFFFu;
    bool up;
    if (shift == 0) {
      const uint64_t twice = r << 1;  // r < count < 2^63
      up = twice > count || (twice == count && (m & 1u));
    } else {
      const int hb = shift - 1;  // the first bit below the kept ones
      const uint32_t half = (limbs_get(q, hb >> 5) >> (hb & 31)) & 1u;
      // sticky: any bit of Q below bit hb, or a nonzero remainder
      bool sticky = r != 0;
#pragma unroll
      for (int i = 0; i < kLimbs; ++i) {
        const int lo_bit = 32 * i;
        const uint32_t mask = hb <= lo_bit ? 0u : (hb >= lo_bit + 32 ? 0xFFFFFFFFu : (1u << (hb - lo_bit)) - 1u);
        sticky = sticky || (q[i] & mask) != 0u;
      }
      up = half && (sticky || (m & 1u));
    }
    m += up ? 1u : 0u;
    // value = m * 2^(shift - 149): for shift >= 1 the exponent field is shift + 1 (a carry
    // to m = 2^24 moves into the exponent); for shift == 0 the bits are m itself
    // (subnormal, or the lowest normal binade).
    g = __uint_as_float(((uint32_t)shift << 23) + m);
  }
  gamma_out[0] = g;
  // s_w = fl32(1/gamma); gamma == 0 (every |W| rounds the mean to 0) gives all-zero codes
  inv_out[0] = g == 0.0f ? 0.0f : 1.0f / g;
}

// ---- ternarise + pack ----------------------------------------------------------------
__device__ __forceinline__ uint32_t tern_code(float w, float s_w) {
  const float t = w * s_w;
  // clamp(rint(t), -1, 1) with ties to even: +1 iff t > 1/2, -1 iff t < -1/2
  return t > 0.5f ? 1u : (t < -0.5f ? 2u : 0u);
}

// One thread per 16-byte slot: row n = 16*nb + (slot % 16), columns 256*c + 64*(slot/16)
// + 0..63; a 64-lane wave writes one whole 1 KiB tile.
__global__ __launch_bounds__(256) void k_ternarise_pack(const float* __restrict__ W, int64_t N, int64_t K,
                                                        int64_t n_tiles, int64_t chunks, int vec4,
                                                        const float* __restrict__ inv_gamma,
                                                        uint8_t* __restrict__ packed) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t tile = t >> 6;
  if (tile >= n_tiles) return;
  const int slot = (int)(t & 63);
  const int64_t nb = tile / chunks, c = tile - nb * chunks;
  const int64_t n = nb * kTileRows + (slot & 15);
  const int64_t k0 = c * kTileCols + 64 * (slot >> 4);
  const float s_w = inv_gamma[0];
  uint32_t word[4];
  if (vec4 && n < N && k0 + 64 <= K) {
    const float4* src = reinterpret_cast<const float4*>(W + n * K + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t x = 0;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const float4 v = src[4 * i + f];  // columns 16i + 4f + b, b = 0..3
        x |= tern_code(v.x, s_w) << (2 * f);
        x |= tern_code(v.y, s_w) << (8 + 2 * f);
        x |= tern_code(v.z, s_w) << (16 + 2 * f);
        x |= tern_code(v.w, s_w) << (24 + 2 * f);
      }
      word[i] = x;
    }
  } else {
    for (int i = 0; i < 4; ++i) {
      uint32_t x = 0;
      for (int j = 0; j < 16; ++j) {
        const int64_t k = k0 + 16 * i + j;
        const uint32_t code = (n < N && k < K) ? tern_code(W[n * K + k], s_w) : 3u;
        x |= code << (8 * (j & 3) + 2 * (j >> 2));
      }
      word[i] = x;
    }
  }
  reinterpret_cast<uint4*>(packed + tile * kTileBytes)[slot] = make_uint4(word[0], word[1], word[2], word[3]);
}

// 1-bit binary variant: one thread per 16-byte slot (g, r) of a 1024-byte binary tile
// (layout in binary.h): word j covers column group g of the 256-column half s = j / 2,
// steps i = 2 (j % 2) and 2 (j % 2) + 1; column e of step i sits at bit
// 8 (e % 4) + 4 (i % 2) + e / 4.
__global__ __launch_bounds__(256) void k_binarise_pack(const float* __restrict__ W, int64_t N, int64_t K,
                                                       int64_t n_tiles, int64_t chunks_b,
                                                       uint8_t* __restrict__ packed) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t tile = t >> 6;
  if (tile >= n_tiles) return;
  const int slot = (int)(t & 63);
  const int64_t nb = tile / chunks_b, c = tile - nb * chunks_b;
  const int64_t n = nb * kTileRows + (slot & 15);
  const int g = slot >> 4;
  uint32_t word[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int s = j >> 1;
    uint32_t x = 0;
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * (j & 1) + ii;
      const int64_t k0 = c * kBinTileCols + 256 * s + 64 * g + 16 * i;
      for (int e = 0; e < 16; ++e) {
        const int64_t k = k0 + e;
        const bool plus = n < N && k < K && !(W[n * K + k] < 0.0f);
        x |= (uint32_t)plus << (8 * (e & 3) + 4 * ii + (e >> 2));
      }
    }
    word[j] = x;
  }
  reinterpret_cast<uint4*>(packed + tile * kTileBytes)[slot] = make_uint4(word[0], word[1], word[2], word[3]);
}

}  // namespace

hipError_t launch_weight_quant_binary(const float* W, int64_t N, int64_t K, uint8_t* packed, float* beta,
                                      void* workspace, hipStream_t s) {
  unsigned long long* bins = static_cast<unsigned long long*>(workspace);
  float* inv = reinterpret_cast<float*>(static_cast<char*>(workspace) + kWqBins * 8);
  const int64_t count = N * K;
  const int vec4_all = ((reinterpret_cast<uintptr_t>(W) & 15u) == 0) ? 1 : 0;
  hipLaunchKernelGGL(k_wq_clear, dim3(1), dim3(64), 0, s, bins);
  int64_t blocks = (count / 4 + kBinThreads - 1) / kBinThreads;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_wq_bins, dim3((unsigned)blocks), dim3(kBinThreads), 0, s, W, count, vec4_all, bins);
  hipLaunchKernelGGL(k_wq_finalize, dim3(1), dim3(64), 0, s, bins, (uint64_t)count, beta, inv);
  const int64_t chunks_b = kb_pad(K) / kBinTileCols;
  const int64_t n_tiles = n_pad(N) / kTileRows * chunks_b;
  const int64_t threads = n_tiles * 64;
  hipLaunchKernelGGL(k_binarise_pack, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, W, N, K, n_tiles,
                     chunks_b, packed);
  return hipGetLastError();
}

hipError_t launch_weight_quant(const float* W, int64_t N, int64_t K, uint8_t* packed, float* gamma,
                               void* workspace, hipStream_t s) {
  unsigned long long* bins = static_cast<unsigned long long*>(workspace);
  float* inv = reinterpret_cast<float*>(static_cast<char*>(workspace) + kWqBins * 8);
  const int64_t count = N * K;
  const int vec4_all = ((reinterpret_cast<uintptr_t>(W) & 15u) == 0) ? 1 : 0;
  hipLaunchKernelGGL(k_wq_clear, dim3(1), dim3(64), 0, s, bins);
  int64_t blocks = (count / 4 + kBinThreads - 1) / kBinThreads;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_wq_bins, dim3((unsigned)blocks), dim3(kBinThreads), 0, s, W, count, vec4_all, bins);
  hipLaunchKernelGGL(k_wq_finalize, dim3(1), dim3(64), 0, s, bins, (uint64_t)count, gamma, inv);
  const int64_t chunks = k_pad(K) / kTileCols;
  const int64_t n_tiles = n_pad(N) / kTileRows * chunks;
  const int vec4_rows = (vec4_all && (K % 4) == 0) ? 1 : 0;
  const int64_t threads = n_tiles * 64;
  hipLaunchKernelGGL(k_ternarise_pack, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, W, N, K,
                     n_tiles, chunks, vec4_rows, inv, packed);
  return hipGetLastError();
}

// Device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept; null if the lookup fails.
static void* scratch_address() {
  constexpr int kMaxDevices = 64;
  static std::mutex lock;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> guard(lock);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

hipError_t launch_weight_quant_noalloc(const float* W, int64_t N, int64_t K, uint8_t* packed, float* gamma,
                                       hipStream_t s) {
  void* ws = scratch_address();
  if (!ws) return hipErrorInvalidSymbol;
  // the bins are cleared by k_wq_clear at the start of every call (a kernel, not a memset)
  return launch_weight_quant(W, N, K, packed, gamma, ws, s);
}

}  // namespace bl
