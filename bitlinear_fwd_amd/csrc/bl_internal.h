// Internal declarations shared by the HIP sources of libbitlinear.so (not installed).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kTileRows = 16;      // rows (output features) per packed tile
constexpr int kTileCols = 256;     // columns (input features) per packed tile
constexpr int kTileBytes = 1024;   // 16 x 256 codes at 2 bits
constexpr int kWqBins = 256;       // one exact bin per fp32 exponent field
constexpr int kMaxGroup = 8;       // matrices sharing one activation input in a grouped call
// quantiser workspace: 256 uint64 bins, then fp32 1/gamma
constexpr int64_t kWqWorkspaceBytes = kWqBins * 8 + 256;

// Decode one packed 32-bit word (16 consecutive codes, layout of bitlinear.h) into 16
// int8 values in column order, four per dword.  Code table: 00 -> 0, 01 -> +1,
// 10 -> -1, 11 -> 0 (padding).  Fields 0 and 2 use the low two bits of each byte as a
// v_perm_b32 selector into the bytes {00, 01, FF, 00}; fields 1 and 3 keep the selector
// in bits 2-3 (values 0, 4, 8, 12), which v_perm_b32 maps to byte 0 of the low source
// (0x00), byte 0 of the high source (0x01), the sign of byte 1 of the low source (0x80
// -> 0xFF) and the constant 0x00.  One shift, four ANDs and four permutes per 16 weights.
__device__ __forceinline__ v4i decode16(uint32_t w) {
  const uint32_t hi = w >> 4;
  v4i r;
  r.x = (int)__builtin_amdgcn_perm(0u, 0x00FF0100u, w & 0x03030303u);
  r.y = (int)__builtin_amdgcn_perm(0x00000001u, 0x00008000u, w & 0x0C0C0C0Cu);
  r.z = (int)__builtin_amdgcn_perm(0u, 0x00FF0100u, hi & 0x03030303u);
  r.w = (int)__builtin_amdgcn_perm(0x00000001u, 0x00008000u, hi & 0x0C0C0C0Cu);
  return r;
}

// Direct global -> LDS load of 16 bytes per lane (gfx950 global_load_lds_dwordx4): lane
// i of the wave writes lds_base + 16 i, so one wave instruction fills 1 KiB of LDS.
// lds_base must be the same for the whole wave.  Completion is counted by vmcnt; the
// compiler does not order later LDS reads after it, so callers wait explicitly.  (Kept
// in a plain function: inside a kernel template in an anonymous namespace the builtin
// stops clang from emitting the kernel's host launch stub.)
__device__ __forceinline__ void load_g2lds16(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// static_for<N>(f): calls f(std::integral_constant<int, k>{}) for k = 0 .. N-1, so the
// body can use k where a constant expression is required (template arguments).
template <typename F, int... ks>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, ks...>) {
  (f(std::integral_constant<int, ks>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ v4i as_v4i(uint4 u) {
  v4i r;
  r.x = (int)u.x;
  r.y = (int)u.y;
  r.z = (int)u.z;
  r.w = (int)u.w;
  return r;
}

// Activation code of one element: clamp(rint(x * s), -127, 127) with s = fl32(127 / a)
// (0 for an all-zero row); round-half-to-even.  Shared by the standalone activation
// quantiser and the fused decode kernel so both produce identical codes.
__device__ __forceinline__ int8_t quant_code(float x, float s) {
  float r = rintf(x * s);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int8_t)(int)r;
}

// quant_code of four values, packed little-endian into one word.  For |r| < 2^22, adding
// 1.5 * 2^23 to r = fl32(x * s) rounds r to an integer (half to even, as rintf) held in the
// low mantissa bits, so the low byte of the sum is the two's-complement code; |r| <= 127
// whenever s = fl32(127 / a) is finite and |x| <= a, so no clamp is needed.  Two permutes
// and an OR gather the four low bytes.  Multiply and add stay separate roundings.
__device__ __forceinline__ uint32_t quant_code4(float a, float b, float c, float d, float s) {
  const float k = 12582912.0f;
  const uint32_t ta = __float_as_uint(__fadd_rn(__fmul_rn(a, s), k));
  const uint32_t tb = __float_as_uint(__fadd_rn(__fmul_rn(b, s), k));
  const uint32_t tc = __float_as_uint(__fadd_rn(__fmul_rn(c, s), k));
  const uint32_t td = __float_as_uint(__fadd_rn(__fmul_rn(d, s), k));
  return __builtin_amdgcn_perm(tb, ta, 0x0c0c0400u) | __builtin_amdgcn_perm(td, tc, 0x04000c0cu);
}

// Launch plan of the decode kernel for one shape (exposed for tests and the benchmark).
struct GemvPlan {
  int waves = 1;        // waves per workgroup; they split the K tiles into contiguous runs
  int rb = 1;           // 16-row output blocks per workgroup
  bool lds_act = false; // activations staged in LDS (fused quantise + decode)
  bool dpp = false;     // activations held in registers, shifted into place by DPP (M <= 4,
                        // or 5..16 tokens on rows of at most 4096 elements)
  int run = 0;          // dpp: K tiles per wave (all loads of a wave issued at once)
  bool early = false;   // fused dpp with at most one workgroup per compute unit: weight
                        // loads issued before the activation barrier
  bool mid = false;     // fused dpp, up to two workgroups per unit and short runs: weight
                        // loads issued once the activation pieces have landed
  bool prio = false;    // fused dpp, one token, more than two workgroups per unit: raised
                        // wave priority while the activation loads are issued
  bool lead = false;    // fused dpp, one token, at most two workgroups per unit, runs of 14
                        // or 16 tiles: raised priority and two weight tiles before the barrier
  int stage = 0;        // LDS staging: 16-byte activation pieces per thread
  int tg = 1;           // token groups of 16 (17..64 tokens: 2..4)
  bool ok = true;       // the requested activation source is supported by this plan
  int64_t groups = 0;   // workgroups
};
// src: 0 = int8 activations (bitlinear_forward), 1 = bf16 x, 2 = fp32 x (fused form),
// 3 / 4 = bf16 / fp32 x through the sub-layer normalisation (register form only)
GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, int src);
// 17..64 tokens: true where the decode kernel with token groups of 16 is the faster path
// (else the prefill kernel takes them)
bool token_groups_win(int64_t M, int64_t N, int64_t K);

// Launch plan of the prefill kernel.
struct GemmPlan {
  int bm = 128, bn = 128;  // output tile
  int ks = 1;              // K groups of four waves per tile (1 or 2)
  int threads = 256;
  int64_t groups = 0;
  // split-tail form (plan_gemm_ws only): sk_rounds rounds of whole tiles over the resident
  // slots, then the sk_tail tiles left split into sk_parts K ranges of sk_cpp chunks
  bool sk = false;
  int sk_rounds = 0, sk_tail = 0, sk_parts = 1, sk_cpp = 0;
  int64_t ws_bytes = 0;    // workspace: the tail's int32 partial tiles
};
constexpr int kGemmCUs = 256;  // compute units of one MI355X
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K);
// The plan of the workspace form (bitlinear_forward_ws): the split tail where it evens
// out a partial last round with at most 8 MiB of partial tiles, else plan_gemm's.
GemmPlan plan_gemm_ws(int64_t M, int64_t N, int64_t K);
int gemm_slots_per_cu(int bn);
// Resident workgroups per compute unit the runtime reports for the one-group prefill
// kernels: 64 x 256 and 64 x 192 whole-tile, then 64 x 256 and 64 x 192 split-tail.
hipError_t gemm_occupancy(int out[4]);


// Launchers (return hipSuccess or the launch error).  All sizes are validated by the
// C ABI before these are called.
hipError_t launch_weight_quant(const float* W, int64_t N, int64_t K, uint8_t* packed, float* gamma,
                               void* workspace, hipStream_t s);
// The same with the workspace in the library's per-device static scratch (allocates nothing).
hipError_t launch_weight_quant_noalloc(const float* W, int64_t N, int64_t K, uint8_t* packed, float* gamma,
                                       hipStream_t s);
// rowsum (nullable): int32 [M], the exact sum of each row's codes.
hipError_t launch_act_quant(const void* X, int bf16, int64_t M, int64_t K, int8_t* Xq, float* absmax,
                            hipStream_t s, int32_t* rowsum = nullptr);
// The quantiser behind the sub-layer RMS normalisation: codes of fl32(x * gain), scale
// max|x * gain| / sqrt(mean(x^2) + eps) (gain null: all ones).
hipError_t launch_subln_quant(const void* X, int bf16, int64_t M, int64_t K, const float* gain, float eps,
                              int8_t* Xq, float* scale, hipStream_t s);
// Sub-layer normalisation arguments of the fused decode forms.
struct NormArgs {
  const float* gain;  // fp32 [K], 16-byte aligned, or null
  float eps;
};
hipError_t launch_gemv(const uint8_t* packed, const float* gamma, const int8_t* Xq, const float* absmax,
                       int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, hipStream_t s);
// norm non-null: the normalising form, only where plan_gemv(M, N, K, 3 or 4) gives the
// register form (hipErrorInvalidConfiguration otherwise, nothing enqueued).
hipError_t launch_gemv_fused(const uint8_t* packed, const float* gamma, const void* X, int bf16, int64_t M, int64_t N,
                             int64_t K, float* Y, int32_t* acc, int8_t* Xq_out, float* absmax_out, hipStream_t s,
                             const NormArgs* norm = nullptr);
// One matrix of a grouped call (matrices sharing one activation input).
struct GroupMat {
  const uint8_t* packed;
  const float* gamma;
  int64_t N;
  float* Y;
  int32_t* acc;
};
// One fused launch for the whole group when the register form of the decode kernel
// covers it (M <= 4): *launched tells whether it did (nothing is enqueued otherwise).
hipError_t launch_gemv_grouped(const GroupMat* mats, int count, const void* X, int bf16, int64_t M, int64_t K,
                               int8_t* Xq_out, float* absmax_out, hipStream_t s, bool* launched,
                               const NormArgs* norm = nullptr);
// Matrices of one int8-quantised input, 5..16 tokens on rows of at most 16 K tiles, in one
// launch of the 5..16-token register decode: *launched tells whether it did (nothing is
// enqueued otherwise).
hipError_t launch_gemv_grouped_int8(const GroupMat* mats, int count, const int8_t* Xq, const float* absmax, int64_t M,
                                    int64_t K, hipStream_t s, bool* launched);
// The fused 5..16-token form (bf16 x, K a multiple of 8 up to 7168, M K <= 65536,
// k_gemv_fq16): every
// workgroup quantises the whole input into LDS and decodes RB row blocks with W waves,
// runs of T tiles, KL 16-byte row pieces per lane.  ok false where it does not apply.
struct Fq16Plan {
  bool ok = false;
  int W = 0, T = 0, RB = 1, KL = 0;
  int64_t lds_bytes = 0;  // dynamic LDS: the codes of 16 token rows
};
// rb_total: row blocks of all the matrices of the call; src as plan_gemv's
Fq16Plan plan_fq16(int64_t M, int64_t rb_total, int64_t K, int src);
// Workgroups of the fused 5..16-token launch over these matrices' row blocks.
int64_t fq16_groups(const Fq16Plan& p, const GroupMat* mats, int count);
// The fused 5..16-token launch for a group of matrices (a single forward is a group of
// one): *launched tells whether it did (nothing is enqueued otherwise).
hipError_t launch_gemv_fq16(const GroupMat* mats, int count, const void* X, int bf16, int64_t M, int64_t K,
                            int8_t* Xq_out, float* absmax_out, hipStream_t s, bool* launched);
// Gate / up pair with the squared-ReLU gating: one launch where gated_fused_ok (M <= 4,
// register form of the fused decode kernel, runs of at most 8 tiles); otherwise
// hipErrorInvalidConfiguration and nothing enqueued.
bool gated_fused_ok(int64_t M, int64_t N, int64_t K, int src);
hipError_t launch_gemv_gated(const uint8_t* packed_gate, const float* gamma_gate, const uint8_t* packed_up,
                             const float* gamma_up, const void* X, int bf16, int64_t M, int64_t N, int64_t K, float* H,
                             int8_t* Xq_out, float* absmax_out, hipStream_t s, const NormArgs* norm);
// h = relu(y_gate)^2 * y_up elementwise (h may alias y_gate).
hipError_t launch_gated_relu2(const float* y_gate, const float* y_up, int64_t count, float* h, hipStream_t s);
hipError_t launch_gemm(const uint8_t* packed, const float* gamma, const int8_t* Xq, const float* absmax,
                       int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, hipStream_t s);
hipError_t launch_gemm_ws(const uint8_t* packed, const float* gamma, const int8_t* Xq, const float* absmax,
                          int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, void* workspace, hipStream_t s);

// Measurement probes (probes.hip).
int64_t probe_stream_groups(int64_t bytes);
hipError_t launch_probe_stream(const void* buf, int64_t bytes, uint32_t* out, hipStream_t s);
hipError_t launch_probe_mfma(int64_t iters, int64_t groups, uint32_t* out, hipStream_t s);
hipError_t launch_probe_read(const void* buf, int64_t bytes, int64_t groups, bool nontemporal, uint32_t* out,
                             hipStream_t s);

inline int64_t n_pad(int64_t n) { return (n + kTileRows - 1) / kTileRows * kTileRows; }
inline int64_t k_pad(int64_t k) { return (k + kTileCols - 1) / kTileCols * kTileCols; }

}  // namespace bl
