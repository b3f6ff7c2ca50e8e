// argmax.hip -- row-wise argmax of an fp32 matrix in one launch, with the
// semantics "Open-Source ROCm Kernels for AMD MI350X" (Netra Kernel blog),
// section "Sampling: make small batches large enough", requires of it
// (PyTorch's argmax): a NaN beats every number and the first NaN beats later
// ones; among equal numbers the lowest index wins; -0 and +0 are equal.
//
// Launch shape: row r is cut into C chunks of 4096 values and block
// r * C + c scans chunk c, so a few long rows still fill the chip (the page's
// point: [16, 248320] is 16 rows but 976 blocks here).  Every thread issues
// its kArgmaxU 16-byte non-temporal loads at once, then keeps, in index order, the
// first value that beats its current winner (plain float compares give -0 ==
// +0 for free; a NaN is taken only when the winner is not one already).  The
// candidates then meet as 64-bit keys -- the value's order code in the high
// half (every NaN above +inf, -0 folded onto +0) and the complement of the
// index in the low half -- so one unsigned maximum picks the value winner and,
// among equals, the lowest index.  Lanes meet by a xor butterfly, waves in
// LDS.
//
// Hand-off: with C > 1 each block writes its key with a write-through store,
// waits for it, and takes a ticket on its row (each row's ticket in its own
// 256-byte slot: tickets sharing a line serialise every block's atomic, which
// cost 5 us at [16, 248320]); in the block taking the row's last ticket, the
// first wave reads the C keys with coherent loads (one per lane), writes the
// index, and re-zeroes the ticket, so the workspace is clean again for the
// next launch.
#include "argmax.h"
#include "device_common.h"

namespace mr {

namespace {

constexpr int kThreads = 256;

// Order code of a float: unsigned order equals numeric order, -0 maps to +0,
// and every NaN maps above +inf.  Never 0 (the code of -inf is 0x007FFFFF).
__device__ __forceinline__ uint32_t order_code(float f) {
  if (f != f) return 0xFFFFFFFFu;
  const uint32_t b = f == 0.0f ? 0u : __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ void key_max(uint32_t &hi, uint32_t &lo, uint32_t ph, uint32_t pl) {
  const bool take = ph > hi || (ph == hi && pl > lo);
  hi = take ? ph : hi;
  lo = take ? pl : lo;
}

// Maximum 64-bit key over the wave, left in every lane.
__device__ __forceinline__ void wave_key_max(uint32_t &hi, uint32_t &lo, int lane) {
  key_max(hi, lo, xor_lane_u32<1>(hi, lane), xor_lane_u32<1>(lo, lane));
  key_max(hi, lo, xor_lane_u32<2>(hi, lane), xor_lane_u32<2>(lo, lane));
  key_max(hi, lo, xor_lane_u32<4>(hi, lane), xor_lane_u32<4>(lo, lane));
  key_max(hi, lo, xor_lane_u32<8>(hi, lane), xor_lane_u32<8>(lo, lane));
  key_max(hi, lo, xor_lane_u32<16>(hi, lane), xor_lane_u32<16>(lo, lane));
  key_max(hi, lo, xor_lane_u32<32>(hi, lane), xor_lane_u32<32>(lo, lane));
}

__global__ __launch_bounds__(kThreads) void argmax_kernel(ArgmaxParams p) {
  __shared__ uint32_t wk[2][kThreads / kWave];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x / p.C, chunk = blockIdx.x % p.C;
  const float *xr = p.x + row * p.ld;
  const int64_t nq = p.N >> 2;                            // whole 16-byte groups in the row
  const int64_t q0 = chunk * (int64_t)(kThreads * kArgmaxU);  // first group of the chunk

  // ---- this thread's values, in index order ------------------------------
  u32x4_t v[kArgmaxU];
  bool ok[kArgmaxU];
#pragma unroll
  for (int u = 0; u < kArgmaxU; ++u) {
    const int64_t q = q0 + u * kThreads + tid;
    ok[u] = q < nq;
    v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(xr) + (ok[u] ? q : 0));
  }
  float best = __uint_as_float(v[0].x);
  int bi = ok[0] ? 0 : -1;  // u * 4 + component of the winner
#pragma unroll
  for (int u = 0; u < kArgmaxU; ++u)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (u == 0 && c == 0) continue;
      const float f = __uint_as_float(v[u][c]);
      const bool take = ok[u] && (f > best || (f != f && best == best));
      best = take ? f : best;
      bi = take ? u * 4 + c : bi;
    }
  uint32_t hi = 0u, lo = 0u;  // key 0: no candidate
  if (bi >= 0) {
    const int64_t idx = 4 * (q0 + (bi >> 2) * kThreads + tid) + (bi & 3);
    hi = order_code(best);
    lo = 0xFFFFFFFFu - (uint32_t)idx;
  }
  // the last 1..3 values of a row whose length is not a multiple of 4
  if (chunk == p.C - 1 && tid < (int)(p.N & 3)) {
    const int64_t idx = 4 * nq + tid;
    key_max(hi, lo, order_code(xr[idx]), 0xFFFFFFFFu - (uint32_t)idx);
  }

  // ---- block winner ------------------------------------------------------
  wave_key_max(hi, lo, lane);
  if (lane == 0) {
    wk[0][wave] = hi;
    wk[1][wave] = lo;
  }
  __syncthreads();
  if (wave != 0) return;
  hi = wk[0][0];
  lo = wk[1][0];
#pragma unroll
  for (int w = 1; w < kThreads / kWave; ++w) key_max(hi, lo, wk[0][w], wk[1][w]);
  if (p.C == 1) {
    if (lane == 0) p.out[row] = (int64_t)(0xFFFFFFFFu - lo);
    return;
  }
  // ---- row winner: the last of the row's C blocks (wave 0) ----------------
  uint32_t t = 0u;
  if (lane == 0) {
    st_agent(p.part + row * p.C + chunk, ((unsigned long long)hi << 32) | lo);
    wait_own_stores();
    t = __hip_atomic_fetch_add(p.ticket + row * kArgmaxTicketStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  t = __builtin_amdgcn_readfirstlane(t);
  if (t != (uint32_t)p.C - 1u) return;
  hi = 0u;
  lo = 0u;
  for (int64_t c = lane; c < p.C; c += kWave) {
    const unsigned long long k = ld_agent(p.part + row * p.C + c);
    key_max(hi, lo, (uint32_t)(k >> 32), (uint32_t)k);
  }
  wave_key_max(hi, lo, lane);
  if (lane == 0) {
    p.out[row] = (int64_t)(0xFFFFFFFFu - lo);
    st_agent(p.ticket + row * kArgmaxTicketStride, 0u);
  }
}

}  // namespace

int64_t argmax_chunks(int64_t N) {
  const int64_t chunk = (int64_t)kThreads * kArgmaxU * 4;
  return (N + chunk - 1) / chunk;
}

hipError_t launch_argmax(const ArgmaxParams &p, hipStream_t stream) {
  if (p.R == 0) return hipSuccess;
  const int64_t blocks = (int64_t)p.R * p.C;
  argmax_kernel<<<(unsigned)blocks, kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace mr
