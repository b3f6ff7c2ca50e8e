// grouped_gemm.hip -- a minimal bf16 grouped-expert GEMM that consumes the
// align output, for measuring what the alignment costs downstream.
//
// It follows the consumer "W4A16 MoE prefill: M-aware moe_align block size"
// (ROCm vLLM), Purpose, describes: block b of A slots runs only while
// b * A < num_tokens_post_padded (its one early exit), multiplies the x rows
// of its slots by the weights of expert expert_ids[b], and stores the rows
// of real pairs; a padding slot inside npp still takes part in the full
// K contraction and only its store is skipped.  The work is therefore
// proportional to npp, not to the routed rows.  Each output element is one
// row's full-K contraction against one expert in a fixed order, whatever
// block the row lands in, so the output does not depend on A.
//
//   y[p][n] = sum_h x[p / S][h] * W[e][n][h]   (bf16 in, fp32 accumulation)
//
// Launch shape: grid (sorted_cap / A, N / 64), 256 threads.  Wave w takes
// the 32 output features 32 (w & 1) of the block's 64 and the token groups
// (w >> 1) + 2 g, g < A / 64, of 32 slots each, as v_mfma_f32_32x32x16_bf16
// tiles (weights as the 32-row operand, gathered x rows as the 32-column
// operand).  Nothing is shared between waves, so the operands go straight
// from global memory into the MFMA registers (16 bytes per lane per 16-k
// step, four steps per round, the next round's loads issued before this
// round's MFMAs); no LDS, no barriers.
#include "device_common.h"
#include "grouped_gemm.h"

namespace mr {

namespace {

constexpr int kThreads = 256;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_g;
typedef __attribute__((ext_vector_type(16))) float f32x16_g;

__device__ __forceinline__ bf16x8_g as_bf16x8_g(uint4 u) { return __builtin_bit_cast(bf16x8_g, u); }

template <int NTG>  // token groups of 32 slots per wave: A / 64
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmParams p) {
  const int64_t b = blockIdx.x;
  if (b * p.A >= (int64_t)*p.npp) return;  // the consumer's only early exit
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int fw = wave & 1, tw = wave >> 1;
  const int e = p.expert_ids[b];
  if (e < 0 || e >= p.Ep) return;
  const int n0 = blockIdx.y * 64 + fw * 32;
  const int64_t npairs = (int64_t)p.M * p.S;
  const int kh = lane >> 5;  // which 8 of a 16-k step this lane holds
  const uint4 *wrow = reinterpret_cast<const uint4 *>(p.w + ((size_t)e * p.N + n0 + (lane & 31)) * p.H) + kh;
  const uint4 *xrow[NTG];
  int32_t pair[NTG];
  bool valid[NTG];
#pragma unroll
  for (int g = 0; g < NTG; ++g) {
    const int32_t q = p.sorted[b * p.A + 32 * (tw + 2 * g) + (lane & 31)];
    valid[g] = q >= 0 && (int64_t)q < npairs;
    pair[g] = q;
    xrow[g] = reinterpret_cast<const uint4 *>(p.x + (size_t)(valid[g] ? q / p.S : 0) * p.H) + kh;
  }
  f32x16_g acc[NTG];
#pragma unroll
  for (int g = 0; g < NTG; ++g)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[g][i] = 0.f;

  // one round = 4 steps of 16 k = 64 k; a step's 16 bytes sit at uint4 index
  // 2 s.  Two register buffers alternate; the loop is unrolled by two so
  // that each buffer is named at compile time (a buffer picked by a runtime
  // index would live in scratch memory).
  uint4 a0[4], x0[4][NTG], a1[4], x1[4][NTG];
  auto load = [&](uint4 (&a)[4], uint4 (&x)[4][NTG], int k0) {
    const int c0 = k0 >> 3;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      a[s] = wrow[c0 + 2 * s];
#pragma unroll
      for (int g = 0; g < NTG; ++g) x[s][g] = xrow[g][c0 + 2 * s];
    }
  };
  auto round = [&](const uint4 (&a)[4], const uint4 (&x)[4][NTG]) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int g = 0; g < NTG; ++g) {
        const uint4 xv = valid[g] ? x[s][g] : make_uint4(0u, 0u, 0u, 0u);
        acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8_g(a[s]), as_bf16x8_g(xv), acc[g], 0, 0, 0);
      }
  };
  const int rounds = p.H >> 6;
  load(a0, x0, 0);
  for (int r = 0; r < rounds; r += 2) {
    if (r + 1 < rounds) load(a1, x1, (r + 1) << 6);
    round(a0, x0);
    if (r + 1 == rounds) break;
    if (r + 2 < rounds) load(a0, x0, (r + 2) << 6);
    round(a1, x1);
  }
  // lane holds slot column lane % 32 of each group and the features
  // n0 + 8 q + 4 (lane / 32) + {0..3} in elements 4q .. 4q + 3
#pragma unroll
  for (int g = 0; g < NTG; ++g) {
    if (!valid[g]) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float4 v;
      v.x = acc[g][4 * q + 0];
      v.y = acc[g][4 * q + 1];
      v.z = acc[g][4 * q + 2];
      v.w = acc[g][4 * q + 3];
      *reinterpret_cast<float4 *>(p.y + (size_t)pair[g] * p.N + n0 + 8 * q + 4 * kh) = v;
    }
  }
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmParams &p, hipStream_t stream) {
  const int64_t blocks = p.sorted_cap / p.A;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks, (unsigned)(p.N / 64));
  if (p.A == 64) grouped_gemm_kernel<1><<<grid, kThreads, 0, stream>>>(p);
  else grouped_gemm_kernel<2><<<grid, kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace mr
