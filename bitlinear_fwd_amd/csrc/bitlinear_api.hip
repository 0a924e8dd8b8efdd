// C ABI of libbitlinear.so: argument validation, kernel selection, launch on the caller's
// stream.  Declarations and the contract of each call are in include/bitlinear.h.
#include "../../include/bitlinear.h"

#include "bl_internal.h"
#include "gemv_lut.h"
#include "binary.h"

namespace {

constexpr int kVersion = 10000;  // 1.0.0
constexpr int64_t kMaxCount = int64_t(1) << 40;  // exactness bound of the gamma bins
constexpr int64_t kMaxK = int64_t(1) << 24;      // |acc| <= 127 K < 2^31, and exact in fp32 for K < 2^17
constexpr int64_t kMaxDim = int64_t(1) << 31;
constexpr int kDecodeMaxM = 16;                  // tokens always handled by the decode kernels

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
// decode kernels for up to 16 tokens, and for 17..64 where token groups beat the prefill kernel
bool use_decode(int64_t M, int64_t N, int64_t K) { return M <= kDecodeMaxM || bl::token_groups_win(M, N, K); }

int hip_status(hipError_t e) { return e == hipSuccess ? BL_OK : BL_ERR_HIP; }

// eps of the sub-layer normalisation: finite and >= 0 (NaN fails both comparisons)
bool eps_ok(float eps) { return eps >= 0.0f && eps <= 3.4028234663852886e38f; }

int grouped_impl(const bl_matrix* mats, int count, const void* X, int dt, int64_t M, int64_t K, const float* gain,
                 float eps, int8_t* Xq, float* absmax, void* stream, bool norm);

}  // namespace

extern "C" {

int bitlinear_version(void) { return kVersion; }

const char* bitlinear_status_string(int status) {
  switch (status) {
    case BL_OK: return "ok";
    case BL_ERR_INVALID_ARG: return "invalid argument (null pointer, size, alignment or workspace)";
    case BL_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case BL_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int64_t bitlinear_n_pad(int64_t N) { return N < 1 ? -1 : bl::n_pad(N); }
int64_t bitlinear_k_pad(int64_t K) { return K < 1 ? -1 : bl::k_pad(K); }
int64_t bitlinear_packed_bytes(int64_t N, int64_t K) {
  return (N < 1 || K < 1) ? -1 : bl::n_pad(N) * bl::k_pad(K) / 4;
}
int64_t bitlinear_wq_workspace_bytes(int64_t N, int64_t K) {
  return (N < 1 || K < 1) ? -1 : bl::kWqWorkspaceBytes;
}

int bitlinear_quantize_weights(const float* W, int64_t N, int64_t K, uint8_t* packed, float* gamma,
                               void* workspace, int64_t ws_bytes, void* stream) {
  if (!W || !packed || !gamma || !workspace) return BL_ERR_INVALID_ARG;
  if (N < 1 || K < 1 || N >= kMaxDim || K >= kMaxDim) return BL_ERR_INVALID_ARG;
  if (N > kMaxCount / K) return BL_ERR_UNSUPPORTED;
  if (ws_bytes < bl::kWqWorkspaceBytes) return BL_ERR_INVALID_ARG;
  if (!aligned(W, 4) || !aligned(packed, 16) || !aligned(gamma, 4) || !aligned(workspace, 8))
    return BL_ERR_INVALID_ARG;
  return hip_status(bl::launch_weight_quant(W, N, K, packed, gamma, workspace, static_cast<hipStream_t>(stream)));
}

int bitlinear_quantize_weights_noalloc(const float* W, int64_t N, int64_t K, uint8_t* packed, float* gamma,
                                       void* stream) {
  if (!W || !packed || !gamma) return BL_ERR_INVALID_ARG;
  if (N < 1 || K < 1 || N >= kMaxDim || K >= kMaxDim) return BL_ERR_INVALID_ARG;
  if (N > kMaxCount / K) return BL_ERR_UNSUPPORTED;
  if (!aligned(W, 4) || !aligned(packed, 16) || !aligned(gamma, 4)) return BL_ERR_INVALID_ARG;
  return hip_status(bl::launch_weight_quant_noalloc(W, N, K, packed, gamma, static_cast<hipStream_t>(stream)));
}

int bitlinear_quantize_acts(const void* X, int dt, int64_t M, int64_t K, int8_t* Xq, float* absmax,
                            int32_t* rowsum, void* stream) {
  if (!X || !Xq || !absmax) return BL_ERR_INVALID_ARG;
  if (M < 1 || K < 1 || M >= kMaxDim || K > kMaxK) return BL_ERR_INVALID_ARG;
  if (dt != BL_F32 && dt != BL_BF16) return BL_ERR_UNSUPPORTED;
  if (!aligned(X, dt == BL_F32 ? 4 : 2) || !aligned(Xq, 16) || !aligned(absmax, 4) || !aligned(rowsum, 4))
    return BL_ERR_INVALID_ARG;
  return hip_status(
      bl::launch_act_quant(X, dt == BL_BF16 ? 1 : 0, M, K, Xq, absmax, static_cast<hipStream_t>(stream), rowsum));
}

int bitlinear_subln_quantize_acts(const void* X, int dt, int64_t M, int64_t K, const float* gain, float eps,
                                  int8_t* Xq, float* scale, void* stream) {
  if (!X || !Xq || !scale) return BL_ERR_INVALID_ARG;
  if (M < 1 || K < 1 || M >= kMaxDim || K > kMaxK || !eps_ok(eps)) return BL_ERR_INVALID_ARG;
  if (dt != BL_F32 && dt != BL_BF16) return BL_ERR_UNSUPPORTED;
  if (!aligned(X, dt == BL_F32 ? 4 : 2) || !aligned(Xq, 16) || !aligned(scale, 4) || !aligned(gain, 4))
    return BL_ERR_INVALID_ARG;
  return hip_status(bl::launch_subln_quant(X, dt == BL_BF16 ? 1 : 0, M, K, gain, eps, Xq, scale,
                                           static_cast<hipStream_t>(stream)));
}

int bitlinear_forward(const uint8_t* packed, const float* gamma, const int8_t* Xq, const float* absmax,
                      int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, void* stream) {
  if (!packed || !gamma || !Xq || !absmax || (!Y && !acc)) return BL_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < 1 || M >= kMaxDim || N >= kMaxDim || K > kMaxK) return BL_ERR_INVALID_ARG;
  if (!aligned(packed, 16) || !aligned(Xq, 16) || !aligned(gamma, 4) || !aligned(absmax, 4) ||
      (Y && !aligned(Y, 4)) || (acc && !aligned(acc, 4)))
    return BL_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (use_decode(M, N, K)) return hip_status(bl::launch_gemv(packed, gamma, Xq, absmax, M, N, K, Y, acc, s));
  if (bl::plan_gemm(M, N, K).groups > (int64_t(1) << 30)) return BL_ERR_UNSUPPORTED;  // grid size
  return hip_status(bl::launch_gemm(packed, gamma, Xq, absmax, M, N, K, Y, acc, s));
}

int64_t bitlinear_forward_ws_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1 || M >= kMaxDim || N >= kMaxDim || K > kMaxK) return -1;
  if (use_decode(M, N, K)) return 0;
  return bl::plan_gemm_ws(M, N, K).ws_bytes;
}

int bitlinear_forward_ws(const uint8_t* packed, const float* gamma, const int8_t* Xq, const float* absmax,
                         int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, void* workspace, int64_t ws_bytes,
                         void* stream) {
  const int64_t need = bitlinear_forward_ws_bytes(M, N, K);
  if (need <= 0) return bitlinear_forward(packed, gamma, Xq, absmax, M, N, K, Y, acc, stream);
  if (!packed || !gamma || !Xq || !absmax || (!Y && !acc)) return BL_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, 256) || ws_bytes < need) return BL_ERR_INVALID_ARG;
  if (!aligned(packed, 16) || !aligned(Xq, 16) || !aligned(gamma, 4) || !aligned(absmax, 4) ||
      (Y && !aligned(Y, 4)) || (acc && !aligned(acc, 4)))
    return BL_ERR_INVALID_ARG;
  return hip_status(bl::launch_gemm_ws(packed, gamma, Xq, absmax, M, N, K, Y, acc, workspace,
                                       static_cast<hipStream_t>(stream)));
}

int bitlinear_probe_prefill_occupancy(int32_t out[4]) {
  if (!out) return BL_ERR_INVALID_ARG;
  int v[4];
  if (bl::gemm_occupancy(v) != hipSuccess) return BL_ERR_HIP;
  for (int i = 0; i < 4; ++i) out[i] = v[i];
  return BL_OK;
}

int bitlinear_forward_ws_plan(int64_t M, int64_t N, int64_t K, int32_t out[10]) {
  if (!out) return BL_ERR_INVALID_ARG;
  for (int i = 6; i < 10; ++i) out[i] = 0;
  const int st = bitlinear_forward_plan(M, N, K, out);
  if (st != BL_OK || use_decode(M, N, K)) return st;
  const bl::GemmPlan p = bl::plan_gemm_ws(M, N, K);
  if (!p.sk) return BL_OK;
  out[0] = 6;
  out[1] = (int32_t)p.groups;
  out[2] = p.threads;
  out[3] = p.bm;
  out[4] = p.bn;
  out[5] = 1;
  out[6] = p.sk_rounds;
  out[7] = p.sk_tail;
  out[8] = p.sk_parts;
  out[9] = p.sk_cpp;
  return BL_OK;
}

int bitlinear_forward_fused(const uint8_t* packed, const float* gamma, const void* X, int dt, int64_t M, int64_t N,
                            int64_t K, float* Y, int32_t* acc, int8_t* Xq, float* absmax, void* stream) {
  if (!packed || !gamma || !X || !Xq || !absmax || (!Y && !acc)) return BL_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < 1 || M >= kMaxDim || N >= kMaxDim || K > kMaxK) return BL_ERR_INVALID_ARG;
  if (dt != BL_F32 && dt != BL_BF16) return BL_ERR_UNSUPPORTED;
  if (!aligned(packed, 16) || !aligned(Xq, 16) || !aligned(gamma, 4) || !aligned(absmax, 4) ||
      !aligned(X, dt == BL_F32 ? 4 : 2) || (Y && !aligned(Y, 4)) || (acc && !aligned(acc, 4)))
    return BL_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int src = dt == BL_BF16 ? 1 : 2;
  if (M <= kDecodeMaxM && aligned(X, 16)) {
    const bl::GemvPlan p = bl::plan_gemv(M, N, K, src);
    if ((p.lds_act || p.dpp) && p.ok)
      return hip_status(bl::launch_gemv_fused(packed, gamma, X, dt == BL_BF16, M, N, K, Y, acc, Xq, absmax, s));
  }
  if (M >= 5 && M <= 16 && aligned(X, 16)) {
    // 5..16 tokens: the fused form that quantises into LDS in every workgroup
    const bl::GroupMat gm{packed, gamma, N, Y, acc};
    bool launched = false;
    const hipError_t e = bl::launch_gemv_fq16(&gm, 1, X, dt == BL_BF16, M, K, Xq, absmax, s, &launched);
    if (launched || e != hipSuccess) return hip_status(e);
  }
  // general case: the activation quantiser, then the forward, both on the stream
  hipError_t e = bl::launch_act_quant(X, dt == BL_BF16 ? 1 : 0, M, K, Xq, absmax, s);
  if (e != hipSuccess) return BL_ERR_HIP;
  return bitlinear_forward(packed, gamma, Xq, absmax, M, N, K, Y, acc, stream);
}

int bitlinear_forward_subln(const uint8_t* packed, const float* gamma, const void* X, int dt, int64_t M, int64_t N,
                            int64_t K, const float* gain, float eps, float* Y, int32_t* acc, int8_t* Xq,
                            float* scale, void* stream) {
  if (!packed || !gamma || !X || !Xq || !scale || (!Y && !acc)) return BL_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < 1 || M >= kMaxDim || N >= kMaxDim || K > kMaxK || !eps_ok(eps)) return BL_ERR_INVALID_ARG;
  if (dt != BL_F32 && dt != BL_BF16) return BL_ERR_UNSUPPORTED;
  if (!aligned(packed, 16) || !aligned(Xq, 16) || !aligned(gamma, 4) || !aligned(scale, 4) || !aligned(gain, 4) ||
      !aligned(X, dt == BL_F32 ? 4 : 2) || (Y && !aligned(Y, 4)) || (acc && !aligned(acc, 4)))
    return BL_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int bf16 = dt == BL_BF16 ? 1 : 0;
  if (M <= kDecodeMaxM && aligned(X, 16) && aligned(gain, 16)) {
    const bl::GemvPlan p = bl::plan_gemv(M, N, K, bf16 ? 3 : 4);
    if (p.dpp && p.ok) {
      const bl::NormArgs norm{gain, eps};
      return hip_status(bl::launch_gemv_fused(packed, gamma, X, bf16, M, N, K, Y, acc, Xq, scale, s, &norm));
    }
  }
  // general case: the normalising quantiser, then the forward, both on the stream
  if (bl::launch_subln_quant(X, bf16, M, K, gain, eps, Xq, scale, s) != hipSuccess) return BL_ERR_HIP;
  return bitlinear_forward(packed, gamma, Xq, scale, M, N, K, Y, acc, stream);
}

int64_t bitlinear_kb_pad(int64_t K) { return K < 1 ? -1 : bl::kb_pad(K); }
int64_t bitlinear_packed_bytes_binary(int64_t N, int64_t K) {
  return (N < 1 || K < 1) ? -1 : bl::packed_bytes_binary(N, K);
}

int bitlinear_quantize_weights_binary(const float* W, int64_t N, int64_t K, uint8_t* packed, float* beta,
                                      void* workspace, int64_t ws_bytes, void* stream) {
  if (!W || !packed || !beta || !workspace) return BL_ERR_INVALID_ARG;
  if (N < 1 || K < 1 || N >= kMaxDim || K >= kMaxDim) return BL_ERR_INVALID_ARG;
  if (N > kMaxCount / K) return BL_ERR_UNSUPPORTED;
  if (ws_bytes < bl::kWqWorkspaceBytes) return BL_ERR_INVALID_ARG;
  if (!aligned(W, 4) || !aligned(packed, 16) || !aligned(beta, 4) || !aligned(workspace, 8)) return BL_ERR_INVALID_ARG;
  return hip_status(
      bl::launch_weight_quant_binary(W, N, K, packed, beta, workspace, static_cast<hipStream_t>(stream)));
}

int bitlinear_forward_binary(const uint8_t* packed, const float* beta, const int8_t* Xq, const float* absmax,
                             int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, void* stream) {
  if (!packed || !beta || !Xq || !absmax || (!Y && !acc)) return BL_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < 1 || M >= kMaxDim || N >= kMaxDim || K > kMaxK) return BL_ERR_INVALID_ARG;
  if (!aligned(packed, 16) || !aligned(Xq, 16) || !aligned(beta, 4) || !aligned(absmax, 4) ||
      (Y && !aligned(Y, 4)) || (acc && !aligned(acc, 4)))
    return BL_ERR_INVALID_ARG;
  if (!bl::plan_gemv_bin(M, N, K).ok) return BL_ERR_UNSUPPORTED;
  return hip_status(bl::launch_gemv_bin(packed, beta, Xq, absmax, M, N, K, Y, acc, static_cast<hipStream_t>(stream)));
}

int bitlinear_forward_binary_plan(int64_t M, int64_t N, int64_t K, int32_t out[6]) {
  if (!out || M < 1 || N < 1 || K < 1 || M >= kMaxDim || N >= kMaxDim || K > kMaxK) return BL_ERR_INVALID_ARG;
  const bl::BinPlan p = bl::plan_gemv_bin(M, N, K);
  if (!p.ok) return BL_ERR_UNSUPPORTED;
  out[0] = 5;
  out[1] = (int32_t)p.groups;
  out[2] = p.waves * 64;
  out[3] = 1;
  out[4] = p.run;
  out[5] = 0;
  return BL_OK;
}

int bitlinear_forward_lut(const uint8_t* packed, const float* gamma, const int8_t* Xq, const float* absmax,
                          int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, void* stream) {
  if (!packed || !gamma || !Xq || !absmax || (!Y && !acc)) return BL_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < 1 || M >= kMaxDim || N >= kMaxDim || K > kMaxK) return BL_ERR_INVALID_ARG;
  if (!aligned(packed, 16) || !aligned(Xq, 16) || !aligned(gamma, 4) || !aligned(absmax, 4) ||
      (Y && !aligned(Y, 4)) || (acc && !aligned(acc, 4)))
    return BL_ERR_INVALID_ARG;
  if (!bl::plan_gemv_lut(M, N, K).ok) return BL_ERR_UNSUPPORTED;
  return hip_status(bl::launch_gemv_lut(packed, gamma, Xq, absmax, M, N, K, Y, acc, static_cast<hipStream_t>(stream)));
}

int bitlinear_forward_lut_plan(int64_t M, int64_t N, int64_t K, int32_t out[6]) {
  if (!out || M < 1 || N < 1 || K < 1 || M >= kMaxDim || N >= kMaxDim || K > kMaxK) return BL_ERR_INVALID_ARG;
  const bl::LutPlan p = bl::plan_gemv_lut(M, N, K);
  if (!p.ok) return BL_ERR_UNSUPPORTED;
  out[0] = 4;
  out[1] = (int32_t)p.groups;
  out[2] = p.waves * 64;
  out[3] = 1;
  out[4] = p.run;
  out[5] = (int32_t)p.lds_bytes;
  return BL_OK;
}

int64_t bitlinear_gated_relu2_workspace_bytes(int64_t M, int64_t N) {
  if (M < 1 || N < 1 || M >= kMaxDim || N >= kMaxDim) return -1;
  return M * N * (int64_t)sizeof(float);
}

int bitlinear_forward_gated_relu2(const uint8_t* gate_packed, const float* gate_gamma, const uint8_t* up_packed,
                                  const float* up_gamma, const void* X, int dt, int64_t M, int64_t N, int64_t K,
                                  int subln, const float* gain, float eps, float* H, int8_t* Xq, float* scale,
                                  void* workspace, int64_t ws_bytes, void* stream) {
  if (!gate_packed || !gate_gamma || !up_packed || !up_gamma || !X || !H || !Xq || !scale) return BL_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < 1 || M >= kMaxDim || N >= kMaxDim || K > kMaxK) return BL_ERR_INVALID_ARG;
  if (subln != 0 && subln != 1) return BL_ERR_INVALID_ARG;
  if (subln && (!eps_ok(eps) || !aligned(gain, 4))) return BL_ERR_INVALID_ARG;
  if (dt != BL_F32 && dt != BL_BF16) return BL_ERR_UNSUPPORTED;
  if (!aligned(gate_packed, 16) || !aligned(up_packed, 16) || !aligned(gate_gamma, 4) || !aligned(up_gamma, 4) ||
      !aligned(Xq, 16) || !aligned(scale, 4) || !aligned(H, 4) || !aligned(X, dt == BL_F32 ? 4 : 2))
    return BL_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int bf16 = dt == BL_BF16 ? 1 : 0;
  const bl::NormArgs nargs{subln ? gain : nullptr, eps};
  const int src = (bf16 ? 1 : 2) + (subln ? 2 : 0);
  if (aligned(X, 16) && aligned(nargs.gain, 16) && bl::gated_fused_ok(M, N, K, src))
    return hip_status(bl::launch_gemv_gated(gate_packed, gate_gamma, up_packed, up_gamma, X, bf16, M, N, K, H, Xq,
                                            scale, s, subln ? &nargs : nullptr));
  // general case: one quantisation, the two forwards (gate into H, up into the workspace),
  // then the gating in place
  if (!workspace || ws_bytes < M * N * (int64_t)sizeof(float) || !aligned(workspace, 4)) return BL_ERR_INVALID_ARG;
  const hipError_t eq = subln ? bl::launch_subln_quant(X, bf16, M, K, gain, eps, Xq, scale, s)
                              : bl::launch_act_quant(X, bf16, M, K, Xq, scale, s);
  if (eq != hipSuccess) return BL_ERR_HIP;
  float* yu = static_cast<float*>(workspace);
  int st = bitlinear_forward(gate_packed, gate_gamma, Xq, scale, M, N, K, H, nullptr, stream);
  if (st != BL_OK) return st;
  st = bitlinear_forward(up_packed, up_gamma, Xq, scale, M, N, K, yu, nullptr, stream);
  if (st != BL_OK) return st;
  return hip_status(bl::launch_gated_relu2(H, yu, M * N, H, s));
}

int bitlinear_forward_gated_relu2_plan(int64_t M, int64_t N, int64_t K, int dt, int subln, int32_t out[6]) {
  if (!out || M < 1 || N < 1 || K < 1 || M >= kMaxDim || N >= kMaxDim || K > kMaxK) return BL_ERR_INVALID_ARG;
  if (subln != 0 && subln != 1) return BL_ERR_INVALID_ARG;
  if (dt != BL_F32 && dt != BL_BF16) return BL_ERR_UNSUPPORTED;
  const int src = (dt == BL_BF16 ? 1 : 2) + (subln ? 2 : 0);
  if (bl::gated_fused_ok(M, N, K, src)) {
    const bl::GemvPlan p = bl::plan_gemv(M, N, K, src);
    out[0] = 3;
    out[1] = (int32_t)p.groups;
    out[2] = p.waves * 64;
    out[3] = p.rb;
    out[4] = 2;
    out[5] = p.run;
    return BL_OK;
  }
  return bitlinear_forward_plan(M, N, K, out);
}

int bitlinear_forward_grouped(const bl_matrix* mats, int count, const void* X, int dt, int64_t M, int64_t K,
                              int8_t* Xq, float* absmax, void* stream) {
  return grouped_impl(mats, count, X, dt, M, K, nullptr, 0.0f, Xq, absmax, stream, false);
}

int bitlinear_forward_grouped_subln(const bl_matrix* mats, int count, const void* X, int dt, int64_t M, int64_t K,
                                    const float* gain, float eps, int8_t* Xq, float* scale, void* stream) {
  if (!eps_ok(eps) || !aligned(gain, 4)) return BL_ERR_INVALID_ARG;
  return grouped_impl(mats, count, X, dt, M, K, gain, eps, Xq, scale, stream, true);
}

int64_t bitlinear_probe_stream_words(int64_t bytes) {
  return (bytes < bl::kTileBytes || bytes % bl::kTileBytes) ? -1 : bl::probe_stream_groups(bytes);
}

int bitlinear_probe_stream(const void* buf, int64_t bytes, uint32_t* out, int64_t out_words, void* stream) {
  if (!buf || !out || bytes < bl::kTileBytes || bytes % bl::kTileBytes || bytes >= (int64_t(1) << 40))
    return BL_ERR_INVALID_ARG;
  if (!aligned(buf, 16) || !aligned(out, 4) || out_words < bl::probe_stream_groups(bytes)) return BL_ERR_INVALID_ARG;
  return hip_status(bl::launch_probe_stream(buf, bytes, out, static_cast<hipStream_t>(stream)));
}

int bitlinear_probe_read(const void* buf, int64_t bytes, int64_t workgroups, int nontemporal, uint32_t* out,
                         void* stream) {
  if (!buf || !out || bytes < 16 || bytes % 16 || bytes >= (int64_t(1) << 40) || workgroups < 1 ||
      workgroups > (int64_t(1) << 20) || (nontemporal != 0 && nontemporal != 1))
    return BL_ERR_INVALID_ARG;
  if (!aligned(buf, 16) || !aligned(out, 4)) return BL_ERR_INVALID_ARG;
  return hip_status(bl::launch_probe_read(buf, bytes, workgroups, nontemporal != 0, out, static_cast<hipStream_t>(stream)));
}

int bitlinear_probe_mfma(int64_t iters, int64_t workgroups, uint32_t* out, void* stream) {
  if (!out || iters < 1 || iters > (int64_t(1) << 32) || workgroups < 1 || workgroups > (int64_t(1) << 20) ||
      !aligned(out, 4))
    return BL_ERR_INVALID_ARG;
  return hip_status(bl::launch_probe_mfma(iters, workgroups, out, static_cast<hipStream_t>(stream)));
}

int bitlinear_forward_fused_plan(int64_t M, int64_t N, int64_t K, int dt, int32_t out[6]) {
  if (!out || M < 1 || N < 1 || K < 1 || M >= kMaxDim || N >= kMaxDim || K > kMaxK) return BL_ERR_INVALID_ARG;
  if (dt != BL_F32 && dt != BL_BF16) return BL_ERR_UNSUPPORTED;
  if (M <= kDecodeMaxM) {
    const bl::GemvPlan p = bl::plan_gemv(M, N, K, dt == BL_BF16 ? 1 : 2);
    if ((p.lds_act || p.dpp) && p.ok) {
      out[0] = 3;
      out[1] = (int32_t)p.groups;
      out[2] = p.waves * 64;
      out[3] = p.rb;
      out[4] = p.dpp ? 2 : 1;
      out[5] = p.dpp ? p.run : (int32_t)(M * (bl::k_pad(K) + 16));
      return BL_OK;
    }
  }
  {
    const bl::Fq16Plan q = bl::plan_fq16(M, bl::n_pad(N) / bl::kTileRows, K, dt == BL_BF16 ? 1 : 2);
    if (q.ok) {
      const bl::GroupMat gm{nullptr, nullptr, N, nullptr, nullptr};
      out[0] = 3;
      out[1] = (int32_t)bl::fq16_groups(q, &gm, 1);
      out[2] = q.W * 64;
      out[3] = q.RB;
      out[4] = 4;
      out[5] = q.T;
      return BL_OK;
    }
  }
  return bitlinear_forward_plan(M, N, K, out);
}

int bitlinear_forward_subln_plan(int64_t M, int64_t N, int64_t K, int dt, int32_t out[6]) {
  if (!out || M < 1 || N < 1 || K < 1 || M >= kMaxDim || N >= kMaxDim || K > kMaxK) return BL_ERR_INVALID_ARG;
  if (dt != BL_F32 && dt != BL_BF16) return BL_ERR_UNSUPPORTED;
  if (M <= kDecodeMaxM) {
    const bl::GemvPlan p = bl::plan_gemv(M, N, K, dt == BL_BF16 ? 3 : 4);
    if (p.dpp && p.ok) {
      out[0] = 3;
      out[1] = (int32_t)p.groups;
      out[2] = p.waves * 64;
      out[3] = p.rb;
      out[4] = 2;
      out[5] = p.run;
      return BL_OK;
    }
  }
  return bitlinear_forward_plan(M, N, K, out);
}

int bitlinear_forward_plan(int64_t M, int64_t N, int64_t K, int32_t out[6]) {
  if (!out || M < 1 || N < 1 || K < 1 || M >= kMaxDim || N >= kMaxDim || K > kMaxK) return BL_ERR_INVALID_ARG;
  if (use_decode(M, N, K)) {
    const bl::GemvPlan p = bl::plan_gemv(M, N, K, 0);
    out[0] = 1;
    out[1] = (int32_t)p.groups;
    out[2] = p.waves * 64;
    out[3] = p.rb;
    out[4] = p.dpp ? 2 : (p.lds_act ? 1 : 0);
    out[5] = p.dpp ? p.run : (p.lds_act ? (int32_t)(M * (bl::k_pad(K) + 16)) : 0);
  } else {
    const bl::GemmPlan p = bl::plan_gemm(M, N, K);
    out[0] = 2;
    out[1] = (int32_t)p.groups;
    out[2] = p.threads;
    out[3] = p.bm;
    out[4] = p.bn;
    out[5] = p.ks;
  }
  return BL_OK;
}

}  // extern "C"

namespace {

int grouped_impl(const bl_matrix* mats, int count, const void* X, int dt, int64_t M, int64_t K, const float* gain,
                 float eps, int8_t* Xq, float* absmax, void* stream, bool norm) {
  if (!mats || !X || !Xq || !absmax) return BL_ERR_INVALID_ARG;
  if (count < 1 || count > bl::kMaxGroup) return BL_ERR_INVALID_ARG;
  if (M < 1 || K < 1 || M >= kMaxDim || K > kMaxK) return BL_ERR_INVALID_ARG;
  if (dt != BL_F32 && dt != BL_BF16) return BL_ERR_UNSUPPORTED;
  if (!aligned(Xq, 16) || !aligned(absmax, 4) || !aligned(X, dt == BL_F32 ? 4 : 2)) return BL_ERR_INVALID_ARG;
  bl::GroupMat gm[bl::kMaxGroup];
  for (int j = 0; j < count; ++j) {
    const bl_matrix& m = mats[j];
    if (!m.packed || !m.gamma || (!m.Y && !m.acc)) return BL_ERR_INVALID_ARG;
    if (m.N < 1 || m.N >= kMaxDim) return BL_ERR_INVALID_ARG;
    if (!aligned(m.packed, 16) || !aligned(m.gamma, 4) || (m.Y && !aligned(m.Y, 4)) || (m.acc && !aligned(m.acc, 4)))
      return BL_ERR_INVALID_ARG;
    gm[j] = bl::GroupMat{m.packed, m.gamma, m.N, m.Y, m.acc};
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bl::NormArgs nargs{gain, eps};
  if (aligned(X, 16) && aligned(gain, 16)) {
    bool launched = false;
    const hipError_t e =
        bl::launch_gemv_grouped(gm, count, X, dt == BL_BF16, M, K, Xq, absmax, s, &launched, norm ? &nargs : nullptr);
    if (launched || e != hipSuccess) return hip_status(e);
  }
  if (!norm && aligned(X, 16)) {
    bool launched = false;
    const hipError_t e = bl::launch_gemv_fq16(gm, count, X, dt == BL_BF16, M, K, Xq, absmax, s, &launched);
    if (launched || e != hipSuccess) return hip_status(e);
  }
  // general case: one activation quantisation, then one forward per matrix
  const hipError_t eq = norm ? bl::launch_subln_quant(X, dt == BL_BF16 ? 1 : 0, M, K, gain, eps, Xq, absmax, s)
                             : bl::launch_act_quant(X, dt == BL_BF16 ? 1 : 0, M, K, Xq, absmax, s);
  if (eq != hipSuccess) return BL_ERR_HIP;
  {
    bool launched = false;
    const hipError_t e = bl::launch_gemv_grouped_int8(gm, count, Xq, absmax, M, K, s, &launched);
    if (launched || e != hipSuccess) return hip_status(e);
  }
  for (int j = 0; j < count; ++j) {
    const int st = bitlinear_forward(mats[j].packed, mats[j].gamma, Xq, absmax, M, mats[j].N, K, mats[j].Y,
                                     mats[j].acc, stream);
    if (st != BL_OK) return st;
  }
  return BL_OK;
}

}  // namespace

