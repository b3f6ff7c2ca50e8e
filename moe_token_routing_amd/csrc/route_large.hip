// route_large.hip -- one-launch router + align for large token counts
// (M > 16): the gate pass is an MFMA bf16 tile contraction.
//
// Computes what "[AMD] One-launch small-M MoE router ... on gfx950"
// (sglang), Modifications, and "W4A16 MoE prefill: M-aware moe_align block
// size" (ROCm vLLM), Purpose, describe (see route_small.hip for the
// formulas), with fp32 accumulation and the same tie and rounding rules.
//
// Launch shape: one block of 256 threads (4 waves) per tile of BT tokens x
// 128 routed experts, plus idle padding blocks; block b works on row tile
// r = (b / 8 / NE) * 8 + b % 8 and expert tile et = (b / 8) % NE, so all
// expert tiles of a row tile run on the same XCD (blocks are dealt to the 8
// XCDs round-robin) and share that row tile's activations in its L2.
//
// 1. Gate: wave w computes experts [32w, 32w + 32) of the tile against all BT
//    tokens with v_mfma_f32_16x16x32_bf16 -- the gate rows are the A operand
//    and the tokens the B operand, so each lane accumulates 4 experts of one
//    token per 16x16 tile.  Both operands come straight from global memory in
//    16-byte loads, PD steps of 32 k-values ahead.  In the expert tile 0
//    blocks, wave 0 also dots the same token fragments with the shared gate
//    row (v_dot2_f32_bf16), so the shared logit costs one extra load a step.
// 2. Tile top-k: keys (see make_key) go to a padded LDS tile; each group of 16
//    lanes (a DPP row) takes one token and selects its k best keys among the
//    tile's 128 experts in k rounds of a row-wide maximum.
// 3. Row tail: with one expert tile the tile block finishes its tokens
//    itself; otherwise every tile block publishes its k candidates per token
//    (write-through agent-scope stores) and takes a ticket on its row tile;
//    the last one merges the row tile's NE candidate lists per token the same
//    way, then the softmax, the shared slot, and the outputs.  For the align
//    it then counts its row tile's pairs per expert and ranks them (64-bit
//    row bitmaps in LDS).
// 4. Global: the last row tail (second ticket) turns the per-tile counts into
//    padded expert offsets (block scan) and per-tile bases, writes
//    expert_ids and npp, and publishes.  It and every block that may safely
//    wait (the whole grid is resident) scatter row tiles from a work queue:
//    sorted_token_ids[base + rank] = flat index.  The last block to exit
//    re-zeroes the counters.
#include "device_common.h"
#include "kernels.h"

namespace mr {

namespace {

constexpr int kThreads = 256;
constexpr int kPad = kLargeBE + 1;  // LDS row stride of the key tile (no bank conflicts)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

// Maximum / sum over the 16 lanes of this lane's DPP row, in all 16 lanes.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kQuadXor1>(v));
  v = max(v, dpp_u32<kQuadXor2>(v));
  v = max(v, dpp_u32<kRowHalfMirror>(v));
  v = max(v, dpp_u32<kRowMirror>(v));
  return v;
}
__device__ __forceinline__ float row_sum_f32(float v) {
  v += dpp_f32<kQuadXor1>(v);
  v += dpp_f32<kQuadXor2>(v);
  v += dpp_f32<kRowHalfMirror>(v);
  v += dpp_f32<kRowMirror>(v);
  return v;
}

// Max of N keys held in registers (a balanced tree).
template <int N>
__device__ __forceinline__ uint32_t max_of_keys(const uint32_t (&a)[N]) {
  uint32_t t[N];
#pragma unroll
  for (int i = 0; i < N; ++i) t[i] = a[i];
#pragma unroll
  for (int w = N / 2; w > 0; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = max(t[i], t[i + w]);
  return t[0];
}

// k rounds of a row-wide maximum over the row's 16 x N keys (unique, 0 =
// empty): lane q of the row ends with the q-th best key in res[0] and the
// (q+16)-th in res[1].
template <int N>
__device__ __forceinline__ void row_select(uint32_t (&keys)[N], int k, int q, uint32_t (&res)[2]) {
  res[0] = res[1] = 0u;
  for (int j = 0; j < k; ++j) {
    const uint32_t top = row_max_u32(max_of_keys(keys));
    if (q == (j & 15)) res[j >> 4] = top;
#pragma unroll
    for (int i = 0; i < N; ++i) keys[i] = (keys[i] == top) ? 0u : keys[i];
  }
}

template <int BT, int NKR, int PD>
__global__ __launch_bounds__(kThreads) void route_large_kernel(LargeParams p) {
  constexpr int NB = BT / 16;  // token fragments per wave
  __shared__ uint32_t tilek[BT * kPad];
  __shared__ float sh_s[BT];
  __shared__ int32_t res_ids[BT * (kMaxTopK + 1)];
  __shared__ unsigned long long bm[kMaxRouteExperts + 1];
  __shared__ uint32_t flag, slot;
  __shared__ uint32_t scan_tmp[kThreads / kWave + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = p.M, H = p.H, E = p.E, Ep = p.Ep, k = p.k, S = p.S;
  uint32_t *ctr = p.ctr;

  if (p.may_help && tid == 0)
    __hip_atomic_fetch_add(&ctr[kCtrStarted], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (p.do_align) {
    const int32_t sentinel = M * S;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + tid; i < p.fill_count; i += (int64_t)gridDim.x * kThreads)
      st_agent(p.sorted + i, sentinel);
  }

  const int b = blockIdx.x;
  const int slot8 = b >> 3;
  const int r = (slot8 / p.NE) * 8 + (b & 7);  // row tile
  const int et = slot8 % p.NE;                 // expert tile
  bool global_winner = false;

  if (r < p.MT) {
    const int t0 = r * BT;
    const int rows = min(BT, M - t0);
    // ---- 1. gate: MFMA over the full hidden size ----------------------------
    f32x4_t acc[2][NB];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int c = 0; c < NB; ++c) acc[a][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float sacc[NB];
#pragma unroll
    for (int c = 0; c < NB; ++c) sacc[c] = 0.f;
    const bool do_sh = p.has_shared && et == 0 && wave == 0;
    const int kg = (lane >> 4) * 8;  // this lane's k offset inside a 32-step
    const uint16_t *wp[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int e = min(et * kLargeBE + wave * 32 + a * 16 + (lane & 15), E - 1);
      wp[a] = p.w + (size_t)e * H + kg;
    }
    const uint16_t *xp[NB];
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      const int t = min(t0 + c * 16 + (lane & 15), M - 1);
      xp[c] = p.x + (size_t)t * H + kg;
    }
    // the shared row (or, without one, gate row 0 as a harmless stand-in) is
    // dotted in every wave so the main loop has no branches; only wave 0 of
    // expert tile 0 keeps the result
    const uint16_t *sp = (p.has_shared ? p.ws_row : p.w) + kg;
    const int nfull = H >> 5;                // full 32-wide k steps
    const int nmain = nfull - nfull % PD;    // steps in whole groups of PD

    uint4 abuf[PD][2], bbuf[PD][NB], sbuf[PD];
    auto load_step = [&](int u, int s) {
#pragma unroll
      for (int a = 0; a < 2; ++a) abuf[u][a] = ld16(wp[a] + 32 * s);
#pragma unroll
      for (int c = 0; c < NB; ++c) bbuf[u][c] = ld16(xp[c] + 32 * s);
      sbuf[u] = ld16(sp + 32 * s);
    };
    auto compute_step = [&](int u) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < NB; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(abuf[u][a]), as_bf16x8(bbuf[u][c]),
                                                             acc[a][c], 0, 0, 0);
#pragma unroll
      for (int c = 0; c < NB; ++c) sacc[c] = dot8_bf16(bbuf[u][c], sbuf[u], sacc[c]);
    };
    if (nmain > 0) {
#pragma unroll
      for (int u = 0; u < PD; ++u) load_step(u, u);
      // steady state: PD steps always in flight, no branches inside a group
      for (int s0 = 0; s0 + PD < nmain; s0 += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u) {
          compute_step(u);
          load_step(u, s0 + PD + u);
        }
      }
#pragma unroll
      for (int u = 0; u < PD; ++u) compute_step(u);
    }
    for (int s = nmain; s < nfull; ++s) {  // leftover full steps
      load_step(0, s);
      compute_step(0);
    }
    if ((H & 31) != 0) {  // ragged last step: lanes past H contribute zeros
      const int kk = nfull * 32;
      const bool ok = kk + kg < H;
      uint4 av[2], bv[NB], sv = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int a = 0; a < 2; ++a) av[a] = ok ? ld16(wp[a] + kk) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int c = 0; c < NB; ++c) bv[c] = ok ? ld16(xp[c] + kk) : make_uint4(0, 0, 0, 0);
      if (ok) sv = ld16(sp + kk);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < NB; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[a]), as_bf16x8(bv[c]), acc[a][c], 0, 0, 0);
#pragma unroll
      for (int c = 0; c < NB; ++c) sacc[c] = dot8_bf16(bv[c], sv, sacc[c]);
    }
    // shared logits: sum the four lane groups holding the same token
    if (do_sh) {
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        float v = sacc[c];
        const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(x16[0]) + __uint_as_float(x16[1]);
        const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(x32[0]) + __uint_as_float(x32[1]);
        if (lane < 16) {
          const int tl = c * 16 + lane;
          sh_s[tl] = v;
          if (t0 + tl < M) {
            if (p.logits_only) p.logits_out[(size_t)(t0 + tl) * Ep + E] = v;
            else if (p.NE > 1) st_agent(p.shared_logit + t0 + tl, v);
          }
        }
      }
    }
    // ---- 2. tile keys to LDS (or the raw logits for the debug hook) -------
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int c = 0; c < NB; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int el = wave * 32 + a * 16 + (lane >> 4) * 4 + i;  // expert inside the tile
          const int tl = c * 16 + (lane & 15);                      // token inside the tile
          const int e = et * kLargeBE + el;
          const float z = acc[a][c][i];
          if (p.logits_only) {
            if (e < E && t0 + tl < M) p.logits_out[(size_t)(t0 + tl) * Ep + e] = z;
          } else {
            tilek[tl * kPad + el] = (e < E) ? make_key(z, (uint32_t)e) : 0u;
          }
        }
    if (p.logits_only) return;
    __syncthreads();

    const int q = tid & 15, rho = tid >> 4;  // lane in the DPP row, row id (16 rows)
    // per-token results of this tile: row rho handles tokens rho, rho+16, ...
    uint32_t fin[NB][2];
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      const int tl = c * 16 + rho;
      uint32_t keys[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) keys[i] = tilek[tl * kPad + q + 16 * i];
      row_select(keys, k, q, fin[c]);
    }

    bool tail = true;
    if (p.NE > 1) {
      // publish this tile's candidates; the last tile of the row tile merges
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        const int t = t0 + c * 16 + rho;
        if (t < M) {
          uint32_t *cp = p.cand + ((size_t)t * p.NE + et) * k;
          if (q < k) st_agent(cp + q, fin[c][0]);
          if (q + 16 < k) st_agent(cp + q + 16, fin[c][1]);
        }
      }
      tail = last_block_ticket(p.tile_ticket + r, (uint32_t)p.NE, &flag);
      if (tail) {
        if (tid == 0) reset_counter(p.tile_ticket + r);
        const int nc = p.NE * k;
        uint32_t keys[NB][NKR];  // every load first, then the selections
#pragma unroll
        for (int c = 0; c < NB; ++c) {
          const int t = min(t0 + c * 16 + rho, M - 1);
          const uint32_t *cp = p.cand + (size_t)t * p.NE * k;
#pragma unroll
          for (int i = 0; i < NKR; ++i) keys[c][i] = ld_agent(cp + min(q + 16 * i, nc - 1));
        }
#pragma unroll
        for (int c = 0; c < NB; ++c) {
#pragma unroll
          for (int i = 0; i < NKR; ++i) keys[c][i] = (q + 16 * i < nc) ? keys[c][i] : 0u;
          row_select(keys[c], k, q, fin[c]);
        }
        if (p.has_shared && tid < BT) sh_s[tid] = (t0 + tid < M) ? ld_agent(p.shared_logit + t0 + tid) : 0.f;
        __syncthreads();
      }
    }

    if (tail) {
      // ---- 3. softmax, shared slot, outputs for the row tile ---------------
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        const int tl = c * 16 + rho;
        const int t = t0 + tl;
        const uint32_t topkey = row_max_u32(fin[c][0]);  // the best key of the token
        const float r0 = key_value(topkey);
        float ex[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) ex[h] = (q + 16 * h < k) ? expf(key_value(fin[c][h]) - r0) : 0.f;
        const float den = row_sum_f32(ex[0] + ex[1]);
        if (t < M) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int j = q + 16 * h;
            if (j < k) {
              const int32_t id = (int32_t)key_id(fin[c][h]);
              st_agent(p.ids + (size_t)t * S + j, id);
              p.wts[(size_t)t * S + j] = ex[h] / den;
              res_ids[tl * S + j] = id;
            }
          }
          if (p.has_shared && q == 0) {
            st_agent(p.ids + (size_t)t * S + k, E);
            p.wts[(size_t)t * S + k] = p.scale / (1.0f + expf(-sh_s[tl]));
            res_ids[tl * S + k] = E;
          }
        }
      }
      if (p.do_align) {
        // ---- row tile align statistics ----------------------------------------
        for (int e = tid; e < E; e += kThreads) bm[e] = 0ull;
        __syncthreads();
        for (int i = tid; i < rows * S; i += kThreads) {
          const int e = res_ids[i];
          if (e < E) atomicOr(&bm[e], 1ull << __umulhi((uint32_t)i, p.S_magic));
        }
        __syncthreads();
        for (int e = tid; e < Ep; e += kThreads) {
          const int32_t c = (e < E) ? (int32_t)__popcll(bm[e]) : rows;
          st_agent(p.tile_counts + (size_t)r * Ep + e, c);
        }
        for (int i = tid; i < rows * S; i += kThreads) {
          const int e = res_ids[i];
          const uint32_t tl = __umulhi((uint32_t)i, p.S_magic);
          const int32_t rank = (e < E) ? (int32_t)__popcll(bm[e] & ((1ull << tl) - 1ull)) : (int32_t)tl;
          st_agent(p.ranks + (size_t)t0 * S + i, rank);
        }
        global_winner = last_block_ticket2<kTicketLanes>(ctr + 64, kTicketLaneStride, ctr + kCtrTicket,
                                                          (uint32_t)p.MT, &flag, (uint32_t)r);
      }
    }
  }

  if (!p.do_align) return;

  // ---- 4. global offsets (winner), then the scatter -------------------------
  bool help = global_winner;
  if (global_winner) {
    if (tid < kTicketLanes) reset_counter(ctr + 64 + tid * kTicketLaneStride);
    if (tid == 0) reset_counter(ctr + kCtrTicket);
    const int MT = p.MT, A = p.A, sh = p.log2A;
    const uint32_t amask = (uint32_t)A - 1u;
    // Thread t owns expert columns t, t + 256, ...: the column's per-tile
    // counts become per-tile exclusive prefixes (loads issued 32 rows at a
    // time), and its padded total feeds a block scan per 256 experts.
    uint32_t carry = 0;
    for (int e0 = 0; e0 < Ep; e0 += kThreads) {
      const int e = e0 + tid;
      uint32_t run = 0;
      if (e < Ep) {
        for (int r0 = 0; r0 < MT; r0 += 32) {
          uint32_t v[32];
#pragma unroll
          for (int u = 0; u < 32; ++u)
            v[u] = (uint32_t)ld_agent(p.tile_counts + (size_t)min(r0 + u, MT - 1) * Ep + e);
#pragma unroll
          for (int u = 0; u < 32; ++u) {
            if (r0 + u < MT) {
              st_agent(p.tile_counts + (size_t)(r0 + u) * Ep + e, (int32_t)run);
              run += v[u];
            }
          }
        }
      }
      const uint32_t P = (run + amask) & ~amask;
      uint32_t tot;
      const uint32_t off = carry + block_excl_scan_u32<kThreads>(P, scan_tmp, &tot);
      carry += tot;
      if (e < Ep) {
        st_agent(p.expert_off + e, (int32_t)off);
        for (uint32_t blk = off >> sh; blk < (off + P) >> sh; ++blk)
          if (blk < (uint64_t)p.expert_cap) p.expert_ids[blk] = e;
      }
    }
    const uint32_t total = carry;
    if (tid == 0) *p.npp = (int32_t)total;
    publish(&ctr[kCtrPublished]);
  } else if (p.may_help) {
    help = join_after_publish(&ctr[kCtrStarted], gridDim.x, &ctr[kCtrPublished], &flag);
  }
  if (help) {
    // a row tile's pairs: at most BT * S <= 64 * 33, so <= 9 per thread
    constexpr int kPer = (BT * (kMaxTopK + 1) + kThreads - 1) / kThreads;
    int32_t *base_lds = reinterpret_cast<int32_t *>(tilek);  // Ep <= BT * kPad words
    for (;;) {
      const uint32_t rr = next_work_item(&ctr[kCtrWork], &slot);
      if (rr >= (uint32_t)p.MT) break;
      const int tb = rr * BT;
      const int n_lo = tb * S, n_hi = min(M, tb + BT) * S;
      int32_t ev[kPer], rk[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int i = min(n_lo + tid + u * kThreads, n_hi - 1);
        ev[u] = ld_agent(p.ids + i);
        rk[u] = ld_agent(p.ranks + i);
      }
      for (int e = tid; e < Ep; e += kThreads)
        base_lds[e] = ld_agent(p.expert_off + e) + ld_agent(p.tile_counts + (size_t)rr * Ep + e);
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int i = n_lo + tid + u * kThreads;
        const int32_t e = ev[u];
        if (i < n_hi && e >= 0 && e < Ep) {
          const int64_t pos = (int64_t)base_lds[e] + rk[u];
          if (pos < p.sorted_cap) p.sorted[pos] = i;
        }
      }
    }
  }
  if (last_to_exit(&ctr[kCtrExited], gridDim.x, &flag) && tid == 0) {
    reset_counter(&ctr[kCtrStarted]);
    reset_counter(&ctr[kCtrPublished]);
    reset_counter(&ctr[kCtrWork]);
    reset_counter(&ctr[kCtrExited]);
  }
}

template <int BT>
hipError_t launch_bt(const LargeParams &p, hipStream_t stream) {
  const int grid = large_grid(p);
  const int nc = p.NE * p.k;
  constexpr int PD = BT == 64 ? 4 : 8;
  if (nc <= 32) route_large_kernel<BT, 2, PD><<<grid, kThreads, 0, stream>>>(p);
  else if (nc <= 64) route_large_kernel<BT, 4, PD><<<grid, kThreads, 0, stream>>>(p);
  else if (nc <= 128) route_large_kernel<BT, 8, PD><<<grid, kThreads, 0, stream>>>(p);
  else route_large_kernel<BT, 16, PD><<<grid, kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

template <int BT>
int resident_blocks() {
  int per_cu = 0, dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, route_large_kernel<BT, 16, BT == 64 ? 4 : 8>,
                                                   kThreads, 0) != hipSuccess)
    return 0;
  return per_cu * cus;
}

}  // namespace

int large_tile_tokens(int M, int E) {
  // Enough tiles to spread over the CUs: 64-token tiles when there are at
  // least 256 of them, else 32, else 16.
  const int NE = (E + kLargeBE - 1) / kLargeBE;
  if ((int64_t)((M + 63) / 64) * NE >= 256) return 64;
  if ((int64_t)((M + 31) / 32) * NE >= 128) return 32;
  return 16;
}

int large_grid(const LargeParams &p) { return ((p.MT + 7) / 8) * 8 * p.NE; }

int large_max_resident_blocks(int BT) {
  // worst case over the instantiations: the NKR = 16 one holds the most registers
  static int cache[3] = {-1, -1, -1};
  const int idx = BT == 64 ? 2 : (BT == 32 ? 1 : 0);
  if (cache[idx] < 0) cache[idx] = BT == 64 ? resident_blocks<64>() : (BT == 32 ? resident_blocks<32>() : resident_blocks<16>());
  return cache[idx];
}

hipError_t launch_route_large(const LargeParams &p, int BT, hipStream_t stream) {
  if (BT == 64) return launch_bt<64>(p, stream);
  if (BT == 32) return launch_bt<32>(p, stream);
  return launch_bt<16>(p, stream);
}

}  // namespace mr
