// route_small.hip -- one-launch router + align for small token counts
// (M <= 16): the gate pass is a weight-streaming GEMV.
//
// What it computes follows "[AMD] One-launch small-M MoE router ... on
// gfx950" (sglang), Modifications, and "W4A16 MoE prefill: M-aware
// moe_align block size" (ROCm vLLM), Purpose:
//   z[m][e] = sum_h x[m][h] * W[e][h]         (fp32 accumulation)
//   s[m]    = sum_h x[m][h] * ws[h]
//   r = bf16(z) (nearest even); top-k of r with the lower id winning ties;
//   w_j = exp(r_j - r_0) / sum_{i<k} exp(r_i - r_0)  (softmax renormalised
//   over the chosen k); slot k = (E, scale * sigmoid(s));
//   then moe_align_block_size over the M*S (token, slot) pairs.
//
// Launch shape (one kernel):
//   grid = ceil(E' / RPB) blocks of 256 threads; block b owns gate rows
//   [b*RPB, b*RPB + RPB) of the E' = E + shared rows (the shared row is
//   row E).  Each row is split over 4/RPB waves; a thread streams 16-byte
//   chunks of its row (coalesced 128-bit loads) and of the M token rows,
//   accumulating with v_dot2_f32_bf16.  Partial sums are reduced with DPP
//   butterflies and across waves through LDS; the block writes fp32 logits
//   to the workspace, every block pre-fills its slice of sorted_token_ids
//   with the sentinel, releases its writes and takes a ticket.
//   The block that takes the last ticket (acquire) runs the tail: one wave
//   per token row does the top-k as k rounds of a wave-wide max over packed
//   32-bit keys (value code << 16 | 0xFFFF - id) with DPP, then the softmax,
//   shared slot and stores; then the align: per-expert 32-bit row bitmaps in
//   LDS give counts and stable ranks, a block scan gives padded offsets, and
//   each pair is scattered to offset + rank.  The tail resets the ticket.
#include "device_common.h"
#include "kernels.h"

namespace mr {

namespace {

constexpr int kThreads = 256;

// Tail of the launch: top-k, softmax, shared slot for rows m = wave, wave+4, ...
// NK = keys per lane (E <= 64 * NK).
template <int NK>
__device__ void route_tail_rows(const SmallParams &p, int32_t *lds_ids) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.E, k = p.k, S = p.S, Ep = p.Ep;
  for (int m = wave; m < p.M; m += kThreads / kWave) {
    const float *zr = p.logits + (size_t)m * Ep;
    uint32_t keys[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int e = lane + kWave * i;
      keys[i] = (e < E) ? make_key(zr[e], (uint32_t)e) : 0u;
    }
    uint32_t mine = 0u;  // lane j < k keeps the j-th chosen key
    for (int j = 0; j < k; ++j) {
      uint32_t lm = keys[0];
#pragma unroll
      for (int i = 1; i < NK; ++i) lm = max(lm, keys[i]);
      const uint32_t top = wave_max_u32(lm);
      mine = (lane == j) ? top : mine;
#pragma unroll
      for (int i = 0; i < NK; ++i) keys[i] = (keys[i] == top) ? 0u : keys[i];
    }
    const float r = key_value(mine);
    const float r0 = readlane_f32(r, 0);
    const float ex = (lane < k) ? expf(r - r0) : 0.0f;
    const float den = wave_sum_f32(ex);
    int32_t id = (int32_t)key_id(mine);
    float w = ex / den;
    if (p.has_shared && lane == k) {
      const float s = zr[E];
      id = E;
      w = p.scale / (1.0f + expf(-s));
    }
    if (lane < S) {
      p.ids[(size_t)m * S + lane] = id;
      p.wts[(size_t)m * S + lane] = w;
      lds_ids[m * S + lane] = id;
    }
  }
}

// Align over the n = M*S pairs whose ids are in lds_ids.  Every id in a row
// is distinct (top-k ids plus the shared id E), so a 32-bit bitmap of rows
// per expert gives both the count and the stable rank of each pair.
__device__ void align_tail_small(const SmallParams &p, const int32_t *lds_ids, uint32_t *bm,
                                 uint32_t *off, uint32_t *scan_tmp) {
  const int tid = threadIdx.x;
  const int S = p.S, Ep = p.Ep, A = p.A;
  const int n = p.M * S;
  for (int e = tid; e < Ep; e += kThreads) bm[e] = 0u;
  __syncthreads();
  for (int i = tid; i < n; i += kThreads) {
    const int e = lds_ids[i];
    if (e >= 0 && e < Ep) atomicOr(&bm[e], 1u << (i / S));
  }
  __syncthreads();
  // padded sizes, exclusive scan over experts: thread t owns a contiguous
  // run of experts [t*per, t*per + per)
  const int per = (Ep + kThreads - 1) / kThreads;
  const int e0 = tid * per;
  uint32_t local = 0;
  for (int e = e0; e < e0 + per && e < Ep; ++e) {
    const uint32_t c = __builtin_popcount(bm[e]);
    local += (c + A - 1) / A * A;
  }
  uint32_t total;
  uint32_t base = block_excl_scan_u32<kThreads>(local, scan_tmp, &total);
  for (int e = e0; e < e0 + per && e < Ep; ++e) {
    const uint32_t c = __builtin_popcount(bm[e]);
    const uint32_t P = (c + A - 1) / A * A;
    off[e] = base;
    for (uint32_t b = base / A; b < (base + P) / A; ++b)
      if (b < (uint64_t)p.expert_cap) p.expert_ids[b] = e;
    base += P;
  }
  __syncthreads();
  for (int i = tid; i < n; i += kThreads) {
    const int e = lds_ids[i];
    if (e < 0 || e >= Ep) continue;
    const int m = i / S;
    const uint32_t rank = __builtin_popcount(bm[e] & ((1u << m) - 1u));
    const uint32_t pos = off[e] + rank;
    if (pos < (uint64_t)p.sorted_cap) p.sorted[pos] = i;
  }
  if (tid == 0) *p.npp = (int32_t)total;
}

template <int RPB, int MAXM, int NK>
__global__ __launch_bounds__(kThreads) void route_small_kernel(SmallParams p) {
  constexpr int WPR = (kThreads / kWave) / RPB;  // waves per gate row
  __shared__ float red[kThreads / kWave][MAXM];
  __shared__ uint32_t flag;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rloc = wave / WPR, sub = wave % WPR;
  const int row = blockIdx.x * RPB + rloc;
  const int H = p.H, M = p.M;
  const int nch = H >> 3;  // 16-byte chunks per row

  // ---- gate: stream this wave's share of one gate row -----------------
  float acc[MAXM];
#pragma unroll
  for (int m = 0; m < MAXM; ++m) acc[m] = 0.0f;
  if (row < p.Ep) {
    const uint4 *wrow = reinterpret_cast<const uint4 *>(row < p.E ? p.w + (size_t)row * H : p.ws_row);
    const uint4 *xb = reinterpret_cast<const uint4 *>(p.x);
    constexpr int kU = 4;  // chunks in flight per thread
    for (int c0 = sub * kWave + lane; c0 < nch; c0 += kU * WPR * kWave) {
      uint4 wv[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int c = c0 + u * WPR * kWave;
        wv[u] = (c < nch) ? ld_stream_16(wrow + c) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        if (m < M) {
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const int c = c0 + u * WPR * kWave;
            if (c < nch) acc[m] = dot8_bf16(wv[u], xb[(size_t)m * nch + c], acc[m]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MAXM; ++m) {
    if (m < M) {
      const float v = wave_sum_f32(acc[m]);
      if (lane == 0) red[wave][m] = v;
    }
  }

  // ---- sentinel pre-fill of this block's slice of sorted_token_ids ------
  if (p.do_align) {
    const int32_t sentinel = M * p.S;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + tid; i < p.fill_count; i += (int64_t)gridDim.x * kThreads)
      p.sorted[i] = sentinel;
  }
  __syncthreads();
  if (tid < RPB * M) {
    const int rl = tid / M, m = tid % M;
    const int e = blockIdx.x * RPB + rl;
    float z = 0.0f;
#pragma unroll
    for (int s = 0; s < WPR; ++s) z += red[rl * WPR + s][m];
    if (e < p.Ep) p.logits[(size_t)m * p.Ep + e] = z;
  }
  if (p.logits_only) return;

  // ---- hand-off: the last block runs the tail ---------------------------
  if (!last_block_ticket(p.ticket, gridDim.x, &flag)) return;

  __shared__ int32_t lds_ids[MAXM * (kMaxTopK + 1)];
  route_tail_rows<NK>(p, lds_ids);
  if (p.do_align) {
    __shared__ uint32_t bm[kMaxRouteExperts + 1];
    __shared__ uint32_t off[kMaxRouteExperts + 1];
    __shared__ uint32_t scan_tmp[kThreads / kWave + 1];
    __syncthreads();
    align_tail_small(p, lds_ids, bm, off, scan_tmp);
  }
  if (tid == 0) reset_counter(p.ticket);
}

template <int RPB, int MAXM>
hipError_t launch_nk(const SmallParams &p, hipStream_t stream) {
  const int grid = (p.Ep + RPB - 1) / RPB;
  const int nk = (p.E + kWave - 1) / kWave;
  if (nk <= 2) route_small_kernel<RPB, MAXM, 2><<<grid, kThreads, 0, stream>>>(p);
  else if (nk <= 4) route_small_kernel<RPB, MAXM, 4><<<grid, kThreads, 0, stream>>>(p);
  else if (nk <= 8) route_small_kernel<RPB, MAXM, 8><<<grid, kThreads, 0, stream>>>(p);
  else route_small_kernel<RPB, MAXM, 16><<<grid, kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

template <int RPB>
hipError_t launch_m(const SmallParams &p, hipStream_t stream) {
  if (p.M <= 4) return launch_nk<RPB, 4>(p, stream);
  if (p.M <= 8) return launch_nk<RPB, 8>(p, stream);
  return launch_nk<RPB, 16>(p, stream);
}

}  // namespace

int small_rows_per_block(int Ep) {
  // Enough blocks to spread the weight stream over the CUs: one or two gate
  // rows per block up to 512 rows, four beyond.
  return Ep <= 256 ? 1 : (Ep <= 1024 ? 2 : 4);
}

hipError_t launch_route_small(const SmallParams &p, hipStream_t stream) {
  switch (small_rows_per_block(p.Ep)) {
    case 1: return launch_m<1>(p, stream);
    case 2: return launch_m<2>(p, stream);
    default: return launch_m<4>(p, stream);
  }
}

}  // namespace mr
