// argmax.h -- the row-wise argmax launch (mr_argmax_rows_f32).  Internal to
// the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mr {

constexpr int kArgmaxU = 4;  // 16-byte loads per thread: a chunk is 256 * 4 * 4 = 4096 values
constexpr int kArgmaxTicketStride = 64;  // words between row tickets (256 bytes)

struct ArgmaxParams {
  const float *x;  // [R, ld] fp32, 16-byte aligned, ld % 4 == 0
  int64_t R, N, ld;
  int64_t C;                 // chunks per row (argmax_chunks(N))
  int64_t *out;              // [R] indices
  uint32_t *ticket;          // [R] at stride kArgmaxTicketStride words, zero between launches
  unsigned long long *part;  // [R, C] block keys
};

int64_t argmax_chunks(int64_t N);
hipError_t launch_argmax(const ArgmaxParams &p, hipStream_t stream);

}  // namespace mr
