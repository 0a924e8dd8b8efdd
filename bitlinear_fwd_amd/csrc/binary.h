// 1-bit sign-binary weight variant: declarations shared by its kernels and the C ABI.
#pragma once
#include "bl_internal.h"

namespace bl {

constexpr int kBinTileCols = 512;  // columns per 1024-byte binary tile (16 rows x 512 bits)

inline int64_t kb_pad(int64_t k) { return (k + kBinTileCols - 1) / kBinTileCols * kBinTileCols; }
inline int64_t packed_bytes_binary(int64_t n, int64_t k) { return n_pad(n) * kb_pad(k) / 8; }

// beta = exact mean |W| (the weight quantiser's bins) and the 1-bit pack: bit 1 for
// W >= 0 (+1), bit 0 for W < 0 (-1); bits outside N x K are 0.
hipError_t launch_weight_quant_binary(const float* W, int64_t N, int64_t K, uint8_t* packed, float* beta,
                                      void* workspace, hipStream_t s);

// Decode plan of the binary kernel (1..4 tokens, int8 activations).
struct BinPlan {
  bool ok = false;
  int waves = 1;
  int run = 1;  // binary tiles (512 columns) per wave
  int64_t groups = 0;
};
BinPlan plan_gemv_bin(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemv_bin(const uint8_t* packed, const float* beta, const int8_t* Xq, const float* absmax, int64_t M,
                           int64_t N, int64_t K, float* Y, int32_t* acc, hipStream_t s);

}  // namespace bl
