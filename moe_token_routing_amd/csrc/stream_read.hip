// stream_read.hip -- a plain streaming read, as a yardstick for the route
// kernels: what one launch of the simplest bandwidth kernel achieves on a
// buffer of a given size (a 4 MiB read is dominated by launch and first-byte
// latency, a 512 MiB read approaches the HBM rate).
//
// Every thread reads 16-byte chunks in a grid-stride loop, kUnroll chunks in
// flight per iteration, with non-temporal loads, and folds them with XOR.
// Block b stores the XOR of everything it read in out[b] (a plain store: one
// shared word taking an atomic per wave would serialise at the memory).
#include "device_common.h"
#include "stream_read.h"

namespace mr {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4_t *src, size_t nchunks, uint32_t *out) {
  __shared__ uint32_t wave_acc[kThreads / kWave];
  const size_t stride = (size_t)gridDim.x * kThreads;
  uint32_t acc = 0u;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < nchunks; i += kUnroll * stride) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t j = i + u * stride;
      v[u] = j < nchunks ? __builtin_nontemporal_load(src + j) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) wave_acc[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = 0u;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) b ^= wave_acc[w];
    out[blockIdx.x] = b;
  }
}

}  // namespace

hipError_t launch_stream_read(const void *src, size_t nbytes, uint32_t *out, hipStream_t stream) {
  const size_t nchunks = nbytes / 16;
  if (nchunks == 0) return hipSuccess;
  // one chunk per thread up to kStreamReadMaxBlocks blocks (16 per CU), then
  // grid-stride
  size_t grid = (nchunks + kThreads - 1) / kThreads;
  if (grid > (size_t)kStreamReadMaxBlocks) grid = kStreamReadMaxBlocks;
  stream_read_kernel<<<(unsigned)grid, kThreads, 0, stream>>>(static_cast<const u32x4_t *>(src), nchunks, out);
  return hipGetLastError();
}

}  // namespace mr
