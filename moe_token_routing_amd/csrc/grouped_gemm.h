// grouped_gemm.h -- the align-output consumer launch (mr_grouped_gemm_bf16).
// Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mr {

struct GemmParams {
  const uint16_t *x;   // [M, H] bf16
  int M, H;
  const uint16_t *w;   // [Ep, N, H] bf16
  int Ep, N, S, A;
  const int32_t *sorted;      // sorted_token_ids [sorted_cap]
  int64_t sorted_cap;
  const int32_t *expert_ids;  // [>= npp / A]
  const int32_t *npp;         // device scalar
  float *y;                   // [M * S, N] fp32
};

hipError_t launch_grouped_gemm(const GemmParams &p, hipStream_t stream);

}  // namespace mr
