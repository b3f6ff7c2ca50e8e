// align.hip -- moe_align_block_size for arbitrary ids, one launch.
//
// Computes what "W4A16 MoE prefill: M-aware moe_align block size" (ROCm
// vLLM), Purpose, describes: the n = M*S (token, slot) pairs grouped by
// expert, each touched expert padded to a multiple of A, so that
// num_tokens_post_padded = sum over touched experts of ceil(c_e / A) * A.
// Inside an expert, pairs keep ascending flat index; padding holds M*S.
// With an expert map (one expert-parallel rank), each pair's expert is its
// local id and pairs of other ranks' experts are skipped.
//
// Launch shape: one block of 256 threads per chunk of 64*W pairs.
//   Phase one (every block): per-expert bitmaps of the chunk's pairs in LDS
//   (W 64-bit words per expert, set with LDS atomic OR -- order free), then a
//   per-expert prefix of the word popcounts gives the chunk's count of each
//   expert and every pair's stable rank inside the chunk.  Counts and ranks
//   go to the workspace; the block pre-fills a slice of sorted_token_ids with
//   the sentinel and takes a ticket.
//   The last block: per-expert totals over chunks, padded sizes, a block scan
//   for the expert offsets, expert_ids and npp, and for every chunk the base
//   offset of each expert; then it publishes.
//   Scatter: the winner and every block that can safely wait (all blocks have
//   begun) take chunks from a queue and write sorted[base + rank] = i.
//   The last block to exit re-zeroes the counters.
#include "device_common.h"
#include "kernels.h"

namespace mr {

namespace {

constexpr int kThreads = 256;

// Expert of pair i as the align sees it: its id, or with an expert map its
// local id (-1 for an expert another rank owns or an id outside the map).
__device__ __forceinline__ int32_t pair_expert(const AlignParams &p, int64_t i) {
  const int32_t e = p.ids[i];
  if (!p.map) return e;
  return (uint32_t)e < (uint32_t)p.Eg ? p.map[e] : -1;
}

__global__ __launch_bounds__(kThreads) void align_kernel(AlignParams p) {
  extern __shared__ uint64_t smem[];
  __shared__ uint32_t flag, slot;
  __shared__ uint32_t scan_tmp[kThreads / kWave + 1];
  const int tid = threadIdx.x;
  const int W = p.W, Ep = p.Ep, A = p.A;
  const int64_t CH = 64 * (int64_t)W;
  uint32_t *ctr = p.ctr;
  if (tid == 0) __hip_atomic_fetch_add(&ctr[kCtrStarted], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- phase one: this block's chunk ------------------------------------
  {
    uint64_t *bm = smem;                                         // [Ep * W]
    uint16_t *pre = reinterpret_cast<uint16_t *>(smem + (size_t)Ep * W);  // [Ep * W]
    const int c = blockIdx.x;
    const int64_t lo = c * CH;
    const int64_t hi = min(p.n, lo + CH);
    for (int j = tid; j < Ep * W; j += kThreads) bm[j] = 0ull;
    __syncthreads();
    for (int64_t i = lo + tid; i < hi; i += kThreads) {
      const int32_t e = pair_expert(p, i);
      if (e >= 0 && e < Ep) {
        const int li = (int)(i - lo);
        atomicOr(reinterpret_cast<unsigned long long *>(&bm[(size_t)e * W + (li >> 6)]), 1ull << (li & 63));
      }
    }
    __syncthreads();
    for (int e = tid; e < Ep; e += kThreads) {
      uint32_t run = 0;
      for (int w = 0; w < W; ++w) {
        pre[(size_t)e * W + w] = (uint16_t)run;
        run += __popcll(bm[(size_t)e * W + w]);
      }
      st_agent(p.counts + (size_t)c * p.cstride + e, (int32_t)run);
    }
    __syncthreads();
    for (int64_t i = lo + tid; i < hi; i += kThreads) {
      const int32_t e = pair_expert(p, i);
      if (e >= 0 && e < Ep) {
        const int li = (int)(i - lo);
        const size_t j = (size_t)e * W + (li >> 6);
        st_agent(p.ranks + i, (int32_t)(pre[j] + __popcll(bm[j] & ((1ull << (li & 63)) - 1ull))));
      }
    }
    const int32_t sentinel = (int32_t)p.n;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + tid; i < p.fill_count; i += (int64_t)gridDim.x * kThreads)
      st_agent(p.sorted + i, sentinel);
  }

  // ---- the last chunk block computes offsets and bases -----------------
  const bool winner = last_block_ticket(&ctr[kCtrDone], gridDim.x, &flag);
  bool help = winner;
  if (winner) {
    // Thread t owns the 4-expert column group g = t (+ 256, ...) of the
    // [nchunks, cstride] count table and reads it with 16-byte coherent
    // loads, 16 chunk rows per batch: the padded totals, one block scan for
    // the expert offsets (carried across column rounds), expert_ids, then a
    // second batched pass that turns each chunk's counts into its bases.
    const int nch = p.nchunks, cs = p.cstride, ncol = cs / 4;
    uint32_t carry = 0;
    for (int g0 = 0; g0 < ncol; g0 += kThreads) {  // block-uniform
      const int g = g0 + tid;
      const bool has = g < ncol;
      const u32x4_coh *col = reinterpret_cast<const u32x4_coh *>(p.counts) + (has ? g : 0);
      uint32_t tot[4] = {0u, 0u, 0u, 0u};
      for (int c0 = 0; c0 < nch; c0 += 16) {
        const u32x4_coh *a[16];
        u32x4_coh v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) a[j] = col + (size_t)min(c0 + j, nch - 1) * ncol;
        ld_coherent16(v, a);
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (c0 + j < nch)
#pragma unroll
            for (int i = 0; i < 4; ++i) tot[i] += v[j][i];
      }
      uint32_t P[4], run = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        P[i] = (has && 4 * g + i < Ep) ? (tot[i] + A - 1) / A * A : 0u;
        run += P[i];
      }
      uint32_t total;
      uint32_t base = carry + block_excl_scan_u32<kThreads>(run, scan_tmp, &total);
      carry += total;
      uint32_t b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b[i] = base;
        if (P[i] > 0u)
          for (uint32_t blk = base / A; blk < (base + P[i]) / A; ++blk)
            if (blk < (uint64_t)p.expert_cap) p.expert_ids[blk] = 4 * g + i;
        base += P[i];
      }
      if (has)
        for (int c0 = 0; c0 < nch; c0 += 16) {
          const u32x4_coh *a[16];
          u32x4_coh v[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) a[j] = col + (size_t)min(c0 + j, nch - 1) * ncol;
          ld_coherent16(v, a);
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (c0 + j < nch)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (4 * g + i < Ep) {
                  st_agent(p.counts + (size_t)(c0 + j) * cs + 4 * g + i, (int32_t)b[i]);
                  b[i] += v[j][i];
                }
        }
    }
    if (tid == 0) *p.npp = (int32_t)carry;
    publish(&ctr[kCtrPublished]);
  } else {
    help = join_after_publish(&ctr[kCtrStarted], gridDim.x, &ctr[kCtrPublished], &flag);
  }

  // ---- scatter: chunks from the queue -----------------------------------
  if (help) {
    for (;;) {
      const uint32_t c = next_work_item(&ctr[kCtrWork], &slot);
      if (c >= (uint32_t)p.nchunks) break;
      const int64_t lo = c * CH;
      const int64_t hi = min(p.n, lo + CH);
      // four pairs per thread per round: their base and rank loads (eight
      // coherent loads) are in flight together
      for (int64_t i0 = lo + tid; i0 < hi; i0 += 4 * kThreads) {
        int32_t ev[4];
        const uint32_t *a[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t i = i0 + (int64_t)u * kThreads;
          const int32_t e = i < hi ? pair_expert(p, i) : -1;
          const bool ok = e >= 0 && e < Ep;
          ev[u] = ok ? e : -1;
          a[2 * u] = reinterpret_cast<const uint32_t *>(p.counts) + (ok ? (size_t)c * p.cstride + e : 0);
          a[2 * u + 1] = reinterpret_cast<const uint32_t *>(p.ranks) + (ok ? i : 0);
        }
        uint32_t v[8];
        ld_coherent8(v, a);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (ev[u] < 0) continue;
          const int64_t pos = (int64_t)v[2 * u] + v[2 * u + 1];
          if (pos < p.sorted_cap) p.sorted[pos] = (int32_t)(i0 + (int64_t)u * kThreads);
        }
      }
    }
  }

  if (last_to_exit(&ctr[kCtrExited], gridDim.x, &flag) && tid == 0) {
    reset_counter(&ctr[kCtrStarted]);
    reset_counter(&ctr[kCtrDone]);
    reset_counter(&ctr[kCtrPublished]);
    reset_counter(&ctr[kCtrWork]);
    reset_counter(&ctr[kCtrExited]);
  }
}

__global__ void zero_words_kernel(uint32_t *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

__global__ void store_zero_kernel(int32_t *p) { *p = 0; }

// Reads the status word past every cache (the route kernels OR bits into it
// with agent-scope atomics) into the caller's buffer.
__global__ void read_status_kernel(const uint32_t *ctr, int32_t *out) {
  *out = (int32_t)ld_agent(ctr + kCtrError);
}

}  // namespace

int align_words_per_expert(int Ep) {
  // Largest power of two <= 16 with the bitmaps within 48 KiB of LDS.
  int W = 16;
  while (W > 1 && (size_t)Ep * W * 8 > 48 * 1024) W >>= 1;
  return W;
}

hipError_t launch_align(const AlignParams &p, hipStream_t stream) {
  const size_t lds = (size_t)p.Ep * p.W * (8 + 2);
  align_kernel<<<p.nchunks, kThreads, lds, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_zero_words(uint32_t *p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int grid = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
  zero_words_kernel<<<grid, 256, 0, stream>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_store_zero(int32_t *p, hipStream_t stream) {
  store_zero_kernel<<<1, 1, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_read_status(const uint32_t *ctr, int32_t *out, hipStream_t stream) {
  read_status_kernel<<<1, 1, 0, stream>>>(ctr, out);
  return hipGetLastError();
}

}  // namespace mr
