// Table-lookup (LUT) decode kernel: declarations shared by gemv_lut.hip and the C ABI.
#pragma once
#include "bl_internal.h"

namespace bl {

// Launch plan of the table-lookup decode kernel: one 16-row block per workgroup, `waves`
// waves of `run` K tiles each, `lds_bytes` of lookup tables (4352 B per tile per token).
struct LutPlan {
  bool ok = false;  // the shape fits (M <= 4, tables within kMaxLutBytes)
  int waves = 1;
  int run = 1;
  int64_t groups = 0;
  int64_t lds_bytes = 0;
};
constexpr int64_t kMaxLutBytes = 148 * 1024;  // tables; with the 4 KiB reduction, within 160 KiB of LDS
LutPlan plan_gemv_lut(int64_t M, int64_t N, int64_t K);

// acc / y of bitlinear_forward computed by table lookups; hipErrorInvalidConfiguration
// (nothing enqueued) where plan_gemv_lut(M, N, K).ok is false.
hipError_t launch_gemv_lut(const uint8_t* packed, const float* gamma, const int8_t* Xq, const float* absmax,
                           int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, hipStream_t s);

}  // namespace bl
