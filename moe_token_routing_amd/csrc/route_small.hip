// route_small.hip -- one-launch router + align for small token counts
// (M <= 32, and up to 128 while the gate's multiply-adds stay small; the
// host decides): the gate pass is a weight-streaming GEMV.
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
// Launch shape (one kernel), blocks of 256 threads over the E' = E + shared
//   gate rows (the shared row is row E):
//   - M <= 4: ceil(E' / RPB) blocks, block b owns rows [b*RPB, b*RPB + RPB)
//     (RPB = 2 at E' > 256, else 1), each row split over the block's waves:
//     a thread streams 16-byte chunks of its row (coalesced 128-bit
//     non-temporal loads) and the same chunks of every token row.
//   - 5 <= M <= 8: the same grid with RPB = 2; thread t streams the chunks
//     t, t + 256, ... of both gate rows and of the M token rows (each token
//     chunk loaded once per block), and its 16 sums are reduced by a halving
//     DPP butterfly.
//   - M >= 9: token tiles: a block takes 4 gate rows against 4 (M <= 20), 8
//     (M <= 64) or 16 token rows in the same way, so it streams 8, 12 or 20
//     rows whatever M.
//     With T token tiles, block b takes row group 8 * ((b / 8) / T) + b mod 8
//     and token tile (b / 8) mod T: the T blocks of a row group run on one
//     XCD (b mod 8) and share its L2.
//   Either way all loads of a batch are issued before any arithmetic
//   (v_dot2_f32_bf16), and partial sums meet across waves in LDS.
//
// Hand-off (no ticket): every block writes, with write-through agent-scope
//   stores, the 32-bit selection key of each routed logit -- the bf16 order
//   code in the high half and 0xFFFF - e in the low half, never 0 -- and the
//   shared logit as (1 << 32 | fp32 bits).  Each tail wave polls its token
//   row of the key buffer with coherent loads until it is complete (a zero
//   marks a slot not yet written); the poll IS the load of the tail's input.
//   It then re-zeroes the row for the next launch.  Only tail blocks wait,
//   on gate work that never waits, and every wait is bounded.  The sentinel
//   pre-fill of sorted_token_ids is issued first, only by blocks that block
//   0 waits for (blocks with a live gate row and tail blocks), and completed
//   before such a block publishes its keys or hands over its ids, so the
//   align never races it.
//
// Tail: the first ceil(M/4) blocks each take four token rows, one per wave
//   (at M <= 4 that is block 0 alone); blocks 1.. hand their ids to block 0
//   (id + 1, written through, polled), which aligns.  A wave selects the
//   top-k as k rounds of a wave-wide maximum over the packed keys (DPP within
//   rows of 16, then gfx950's permlane16/32 swaps), then the softmax, shared
//   slot and stores, marking each pair in LDS bitmaps (token rows per expert,
//   one to four words; touched experts); then the align: up to 32 rows with
//   M <= A every touched expert takes exactly one block, so the bitmap of
//   touched experts (block index = rank among them, one wave scan) and the
//   one of token rows per expert (slot in the block) place every pair, one
//   pair per thread; otherwise the experts' row counts, padded to whole
//   blocks of A, go through one block scan first (align_small_wide).
#include "device_common.h"
#include "kernels.h"

namespace mr {

namespace {

constexpr int kThreads = 256;
// What a tail block hands block 0 in place of its ids when its own key wait
// gave up (a real hand-off value is id + 1 <= 65536).
constexpr uint32_t kFailedHandOff = 0xFFFFFFFFu;
static_assert(kSmallMaxTokens <= 128, "up to 4 words of token-row bits per expert in rowbm");

// Max of N keys held in registers (a balanced tree, depth log2 N).
template <int N>
__device__ __forceinline__ uint32_t max_of(const uint32_t (&a)[N]) {
  uint32_t t[N];
#pragma unroll
  for (int i = 0; i < N; ++i) t[i] = a[i];
#pragma unroll
  for (int w = N / 2; w > 0; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = max(t[i], t[i + w]);
  return t[0];
}

// Align bitmaps (block 0's LDS, zeroed at the block's start): bit m of
// rowbm[e] marks that token row m chose expert e, bit e & 31 of
// touched[e >> 5] that some row did.  The tail marks each pair as it stores
// it; ids outside [0, E') are skipped.
template <int BW>
__device__ __forceinline__ void mark_pair(const SmallParams &p, int32_t id, int m, uint32_t *rowbm,
                                          uint32_t *touched) {
  if ((uint32_t)id < (uint32_t)p.Ep) {
    atomicOr(&rowbm[id * BW + (m >> 5)], 1u << (m & 31));
    // the touched bitmap serves the one-word align only (at most E' / 32
    // words, so every pair's atomic lands on a few addresses)
    if constexpr (BW == 1) atomicOr(&touched[id >> 5], 1u << (id & 31));
  }
}

// Phase stamp i of this block (thread 0), when the caller asked for stamps:
// 0 start, 1 gate keys published; block 0 (its first token row): 2 keys
// arrived, 3 keys sorted, 4 top-k selected, 5 slots stored, 6 align done.
__device__ __forceinline__ void stamp(const SmallParams &p, int i) {
  if (p.stamps && threadIdx.x == 0 && (int)blockIdx.x < p.stamp_blocks)
    p.stamps[(size_t)blockIdx.x * kStamps + i] = __builtin_amdgcn_s_memrealtime();
}

// A bounded wait that gave up: its bit goes into the status word (agent-scope
// atomic OR) and the block's LDS flag is raised.
__device__ __forceinline__ void wait_failed(const SmallParams &p, uint32_t bit, uint32_t *failed, int lane) {
  if (lane == 0) {
    __hip_atomic_fetch_or(p.ctr + kCtrError, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *failed = 1u;
  }
}

// Tail, part 1: token rows m0 + wave (< m1), one per wave.  Each lane
// holds NK keys (experts lane, lane + 64, ...); a selection round is a
// wave-wide maximum of the lanes' sorted heads, and the lane that held it
// drops its head (keys are unique).  The ids go to the outputs and either
// into lds_ids and the align bitmaps (block 0) or, with hand_off, to block 0
// through the hids row (id + 1, written through; kFailedHandOff if this
// wave's key wait gave up).
template <int NK, int BW>
__device__ void route_tail_rows1(const SmallParams &p, int32_t *lds_ids, uint32_t *rowbm, uint32_t *touched,
                                 int m0, int m1, bool hand_off, uint32_t *failed) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.E, k = p.k, S = p.S;
  for (int m = m0 + wave; m < m1; m += kThreads / kWave) {
    uint32_t *kr = p.keys + (size_t)m * E;
    uint32_t keys[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) keys[i] = 0u;
    unsigned long long sv = 0;
    // Poll until every key of this row (and its shared logit) has arrived,
    // at most wait_limit times.  Every poll is the same 1 + NK loads (the
    // shared-logit slot exists in every workspace, used or not).
    bool arrived = false;
    for (int it = 0; it < p.wait_limit; ++it) {
#pragma unroll
      for (int i = 0; i < NK; ++i) keys[i] = ld_agent(kr + min(lane + kWave * i, E - 1));
      sv = ld_agent(p.shared_logit + m);
      bool missing = p.has_shared && (sv >> 32) == 0;
#pragma unroll
      for (int i = 0; i < NK; ++i) missing |= (lane + kWave * i < E) && keys[i] == 0u;
      if (__builtin_amdgcn_ballot_w64(missing) == 0) {
        arrived = true;
        break;
      }
    }
    if (!arrived) wait_failed(p, kWaitKeys, failed, lane);
    stamp(p, 2);
#pragma unroll
    for (int i = 0; i < NK; ++i) keys[i] = (lane + kWave * i < E) ? keys[i] : 0u;  // lanes past E
    sort_desc_u32(keys);
    stamp(p, 3);
    const uint32_t mine = topk_sorted_u32(keys, k, lane);  // lane j < k: the j-th chosen key
    stamp(p, 4);
    const float r = key_value(mine);
    const float r0 = readlane_f32(r, 0);
    const float ex = (lane < k) ? expf(r - r0) : 0.0f;
    const float den = wave_sum_f32(ex);
    int32_t id = (int32_t)key_id(mine);
    float w = ex / den;
    if (p.has_shared && lane == k) {
      const float s = __uint_as_float((uint32_t)sv);
      id = E;
      w = p.scale / (1.0f + expf(-s));
    }
    if (lane < S) {
      // every output of this launch is written through, like the keys: the
      // end-of-launch L2 write-back then finds fewer dirty lines (measured
      // -0.04 to -0.07 us per launch at M = 1..8)
      st_agent(p.ids + (size_t)m * S + lane, id);
      st_agent(p.wts + (size_t)m * S + lane, w);
      if (hand_off) {
        // for block 0's align
        st_agent(p.hids + (size_t)m * S + lane, arrived ? (uint32_t)id + 1u : kFailedHandOff);
      } else {
        lds_ids[m * S + lane] = id;
        if (p.do_align) mark_pair<BW>(p, id, m, rowbm, touched);
      }
    }
    // Re-zero the row's slots for the next launch.  Branch-free: lanes past
    // E re-zero slot E - 1 too (one branch per slot, and a conditional
    // shared-logit load in the poll, cost 0.25 us per launch at M = 1..4).
#pragma unroll
    for (int i = 0; i < NK; ++i) st_agent(kr + min(lane + kWave * i, E - 1), 0u);
    if (p.has_shared && lane == 0) st_agent(p.shared_logit + m, 0ull);
    stamp(p, 5);
  }
}

// Block 0's side of the hand-off at M >= 5: wave w gathers the ids of rows
// 4 + w, 8 + w, ... (< M) that tail blocks 1.. wrote as id + 1 with
// write-through stores, polling until every slot is non-zero (bounded, as
// the key poll), then puts them in lds_ids, marks the align bitmaps and
// re-zeroes the slots for the next launch.  A slot holding kFailedHandOff
// (that block's key wait gave up) raises the block's failed flag.
template <int MAXM, int BW>
__device__ void gather_tail_rows(const SmallParams &p, int32_t *lds_ids, uint32_t *rowbm, uint32_t *touched,
                                uint32_t *failed) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int S = p.S;
  constexpr int kRows = MAXM / (kThreads / kWave) - 1;  // rows 4 + w + 4 r
  uint32_t v[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) v[r] = 0u;
  bool arrived = false;
  for (int it = 0; it < p.wait_limit; ++it) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int m = min(4 + wave + 4 * r, p.M - 1);  // branch-free: rows past M reload row M - 1
      v[r] = ld_agent(p.hids + (size_t)m * S + min(lane, S - 1));
    }
    bool missing = false;
#pragma unroll
    for (int r = 0; r < kRows; ++r) missing |= (4 + wave + 4 * r < p.M) && lane < S && v[r] == 0u;
    if (__builtin_amdgcn_ballot_w64(missing) == 0) {
      arrived = true;
      break;
    }
  }
  if (!arrived) wait_failed(p, kWaitIds, failed, lane);
  bool marker = false;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int m = 4 + wave + 4 * r;
    if (m < p.M && lane < S) {
      marker |= v[r] == kFailedHandOff;
      const int32_t id = (int32_t)v[r] - 1;  // kFailedHandOff and 0 give ids < 0: skipped
      lds_ids[m * S + lane] = id;
      mark_pair<BW>(p, id, m, rowbm, touched);
      st_agent(p.hids + (size_t)m * S + lane, 0u);
    }
  }
  if (__builtin_amdgcn_ballot_w64(marker) != 0 && lane == 0) *failed = 1u;
}

// The same for up to 128 rows: blocks 1.. wrote the ids of
// rows 4.. as id + 1 with write-through stores into hids, which is dense
// [M, S] like topk_ids, so block 0 polls it as a flat array: thread t takes
// the 16-byte chunks t, t + 256, ... from the one holding row 4's first slot,
// one round of loads per poll (bounded, as the key poll), then puts the ids
// in lds_ids, marks the align bitmaps and re-zeroes its chunks for the next
// launch.  A slot holding kFailedHandOff (that block's key wait gave up)
// raises the block's failed flag.
// kPer: 16-byte chunks per thread, as many as this launch's hand-off needs.
template <int kPer, int BW>
__device__ void gather_flat_kp(const SmallParams &p, int32_t *lds_ids, uint32_t *rowbm, uint32_t *touched,
                               uint32_t *failed) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int S = p.S, n = p.M * S, i0 = 4 * S;  // entries [i0, n): rows 4 ..
  const int c0 = i0 >> 2, c1 = (n + 3) >> 2;
  const u32x4_coh *hv = reinterpret_cast<const u32x4_coh *>(p.hids);
  const u32x4_coh *a[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) a[u] = hv + min(c0 + tid + kThreads * u, c1 - 1);
  u32x4_coh v[kPer];
  auto want = [&](int u, int q) {  // entry q of this thread's chunk u is one of rows 4 ..
    const int i = 4 * (c0 + tid + kThreads * u) + q;
    return c0 + tid + kThreads * u < c1 && i >= i0 && i < n;
  };
  bool arrived = false;
  for (int it = 0; it < p.wait_limit; ++it) {
    ld_coherent_x4<kPer>(v, a);
    bool missing = false;
#pragma unroll
    for (int u = 0; u < kPer; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) missing |= want(u, q) && v[u][q] == 0u;
    if (__builtin_amdgcn_ballot_w64(missing) == 0) {
      arrived = true;
      break;
    }
  }
  if (!arrived) wait_failed(p, kWaitIds, failed, lane);
  // the loaded entries go to lds_ids as they are (id + 1) and their slots are
  // re-zeroed; then one compact pass over the entries of rows 4 .. turns
  // them into ids and marks the bitmaps (the unrolled form of that pass,
  // 4 * kPer entries per thread, ran for about a microsecond)
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = c0 + tid + kThreads * u;
    if (c < c1) {
#pragma unroll
      for (int q = 0; q < 4; ++q)  // entries below i0 are block 0's own rows
        if (4 * c + q >= i0 && 4 * c + q < n) lds_ids[4 * c + q] = (int32_t)v[u][q];
      unsigned long long *z = reinterpret_cast<unsigned long long *>(p.hids) + 2 * c;
      st_agent(z, 0ull);
      st_agent(z + 1, 0ull);
    }
  }
  __syncthreads();
  bool marker = false;
  for (int i = i0 + tid; i < n; i += kThreads) {
    const uint32_t h = (uint32_t)lds_ids[i];
    marker |= h == kFailedHandOff;
    const int32_t id = (int32_t)h - 1;  // kFailedHandOff and 0 give ids < 0: skipped
    lds_ids[i] = id;
    const int m = S == 1 ? i : (int)__umulhi((uint32_t)i, p.S_magic);  // token row i / S
    mark_pair<BW>(p, id, m, rowbm, touched);
  }
  if (__builtin_amdgcn_ballot_w64(marker) != 0 && lane == 0) *failed = 1u;
}

template <int MAXM, int BW>
__device__ void gather_tail_flat(const SmallParams &p, int32_t *lds_ids, uint32_t *rowbm, uint32_t *touched,
                                 uint32_t *failed) {
  constexpr int kChunks = (MAXM * (kMaxTopK + 1) + 3) / 4;  // 16-byte chunks of the largest hids
  // the poll loads only the chunks this launch's hand-off covers (a round of
  // loads takes longer the more loads it holds)
  const int nch = ((p.M * p.S + 3) >> 2) - p.S;
  if (nch <= kThreads) gather_flat_kp<1, BW>(p, lds_ids, rowbm, touched, failed);
  else if (nch <= 2 * kThreads) gather_flat_kp<2, BW>(p, lds_ids, rowbm, touched, failed);
  else if (kChunks <= 4 * kThreads || nch <= 4 * kThreads) gather_flat_kp<4, BW>(p, lds_ids, rowbm, touched, failed);
  else gather_flat_kp<8, BW>(p, lds_ids, rowbm, touched, failed);
}

// Tail, part 2: align of the n = M*S pairs in lds_ids.  Here M <= A,
// and a token row holds an expert at most once, so an expert's pairs always
// fit one block of A slots: every touched expert pads to exactly A.  Its
// block index is its rank among the touched experts -- the touched-bitmap
// words' popcounts, scanned by each wave that holds pairs (at most 33 words,
// one wave scan; the base of word e >> 5 fetched with ds_bpermute) -- and a
// pair's slot in the block is the number of earlier token rows that chose
// the same expert, which keeps ascending flat index inside the expert.  The
// shared expert (id E, every row) is handled like the others and comes last.
// The sentinel pre-fill already holds every slot the pairs do not.  Every
// thread of the block calls this after the block barrier that follows the
// tail's marks.
__device__ void align_small(const SmallParams &p, const int32_t *lds_ids, const uint32_t *rowbm,
                            const uint32_t *touched, const uint32_t *failed) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = p.M * p.S, Ep = p.Ep, sh = p.log2A;
  const int words = (Ep + 31) >> 5;  // <= 33 for E' <= 1025: one wave scan covers them
  if (wave * kWave >= n) return;  // wave-uniform: this wave holds no pairs (wave 0 always does)
  const uint32_t pc = lane < words ? __builtin_popcount(touched[lane]) : 0u;
  const uint32_t incl = wave_incl_scan_u32(pc, lane);
  const uint32_t excl = incl - pc;  // touched experts in the words before lane's
  // npp = -1 marks a launch one of whose waits gave up
  if (tid == 0) st_agent(p.npp, *failed ? -1 : (int32_t)(__builtin_amdgcn_readlane(incl, 63) << sh));
  for (int i0 = wave * kWave; i0 < n; i0 += kThreads) {  // wave-uniform trip count: every lane active
    const int i = i0 + lane;
    const int e = lds_ids[min(i, n - 1)];
    const bool valid = i < n && e >= 0 && e < Ep;
    const int ew = valid ? e >> 5 : 0;
    const uint32_t base = (uint32_t)__builtin_amdgcn_ds_bpermute(ew << 2, (int)excl);
    if (!valid) continue;
    const uint32_t m = p.S == 1 ? (uint32_t)i : __umulhi((uint32_t)i, p.S_magic);  // token row i / S
    const uint32_t blk = base + __builtin_popcount(touched[ew] & ((1u << (e & 31)) - 1u));
    const uint32_t rank = __builtin_popcount(rowbm[e] & ((1u << m) - 1u));
    const uint64_t pos = ((uint64_t)blk << sh) + rank;
    if (pos < (uint64_t)p.sorted_cap) p.sorted[pos] = (int32_t)i;
    if (rank == 0 && blk < (uint64_t)p.expert_cap) p.expert_ids[blk] = (int32_t)e;
  }
}

// Tail, part 2 for up to 128 token rows and any A (BW words of token-row
// bits per expert): an expert's pairs may fill several blocks of A slots.
// Thread t counts the pairs of ceil(E' / 256) consecutive experts
// (popcounts of their bits), pads each to blocks of A, and one block scan gives every expert
// its first block (boff, LDS); the thread writes those experts' expert_ids.
// A pair's slot is its expert's first slot plus the number of earlier token
// rows that chose the same expert (ascending flat index inside the expert).
// Every thread of the block calls this after the barrier that follows the
// tail's marks.
// The BW row-bit words of one expert (16- or 8-byte aligned in rowbm).
template <int BW>
__device__ __forceinline__ void load_row_words(const uint32_t *bits, uint32_t (&w)[BW]) {
  static_assert(BW == 2 || BW == 4, "2 or 4 words");
  if constexpr (BW == 4) {
    const uint4 v = *reinterpret_cast<const uint4 *>(bits);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else {
    const uint2 v = *reinterpret_cast<const uint2 *>(bits);
    w[0] = v.x; w[1] = v.y;
  }
}

template <int BW>
__device__ void align_small_wide(const SmallParams &p, const int32_t *lds_ids, const uint32_t *rowbm,
                                 uint32_t *boff, uint32_t *scan_tmp, const uint32_t *failed) {
  constexpr int EPT = (kMaxRouteExperts + 1 + kThreads - 1) / kThreads;  // most experts per thread
  const int tid = threadIdx.x;
  const int n = p.M * p.S, Ep = p.Ep, sh = p.log2A;
  const uint32_t amask = (uint32_t)p.A - 1u;
  // thread t takes the ept consecutive experts from t * ept, as few as E'
  // allows, so each thread's expert_ids stores stay few
  const int ept = (Ep + kThreads - 1) / kThreads;
  const int e0 = tid * ept;
  uint32_t nb[EPT], run = 0;
  uint32_t wd[EPT][BW];
#pragma unroll
  for (int j = 0; j < EPT; ++j) load_row_words<BW>(rowbm + min(e0 + j, Ep - 1) * BW, wd[j]);
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    uint32_t c = 0;
#pragma unroll
    for (int w = 0; w < BW; ++w) c += __builtin_popcount(wd[j][w]);
    nb[j] = (j < ept && e0 + j < Ep) ? (c + amask) >> sh : 0u;
    run += nb[j];
  }
  uint32_t total;
  uint32_t o = block_excl_scan_u32<kThreads>(run, scan_tmp, &total);
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    if (j < ept && e0 + j < Ep) {
      boff[e0 + j] = o;
      for (uint32_t b = 0; b < nb[j]; ++b)
        if (o + b < (uint64_t)p.expert_cap) p.expert_ids[o + b] = (int32_t)(e0 + j);
      o += nb[j];
    }
  }
  // npp = -1 marks a launch one of whose waits gave up
  if (tid == 0) st_agent(p.npp, *failed ? -1 : (int32_t)(total << sh));
  __syncthreads();  // boff complete
  // A pair's slot: its expert's first slot plus the expert's row bits below
  // its token row.  Four pairs per thread at a time, branch-free until the
  // store, so their LDS reads overlap.
  constexpr int kUnroll = 4;
  for (int i0 = tid; i0 < n; i0 += kUnroll * kThreads) {
    int eu[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = i0 + u * kThreads;
      const int e = i < n ? lds_ids[i] : -1;
      ok[u] = e >= 0 && e < Ep;
      eu[u] = ok[u] ? e : 0;
    }
    uint32_t rw[kUnroll][BW], bo[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      load_row_words<BW>(rowbm + eu[u] * BW, rw[u]);
      bo[u] = boff[eu[u]];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = i0 + u * kThreads;
      const uint32_t m = p.S == 1 ? (uint32_t)i : __umulhi((uint32_t)i, p.S_magic);  // token row i / S
      const uint32_t mw = m >> 5, below = (1u << (m & 31)) - 1u;
      uint32_t rank = 0;
#pragma unroll
      for (int w = 0; w < BW; ++w)
        rank += __builtin_popcount(rw[u][w] & ((uint32_t)w < mw ? ~0u : (uint32_t)w == mw ? below : 0u));
      const uint64_t pos = ((uint64_t)bo[u] << sh) + rank;
      // plain stores: a write-through store per scattered slot costs a memory
      // transaction each; the sentinel pre-fill of these slots (other blocks,
      // written through) completed before those blocks published their keys
      if (ok[u] && pos < (uint64_t)p.sorted_cap) p.sorted[pos] = (int32_t)i;
    }
  }
}

// Value held by lane (lane ^ J) of a float (see xor_lane_u32).
template <int J>
__device__ __forceinline__ float xor_lane_f32(float v, int lane) {
  return __uint_as_float(xor_lane_u32<J>(__float_as_uint(v), lane));
}

// One halving step of the butterfly below: lanes at distance J pair up, the
// lane with bit J clear keeps the lower half of its N values and the other
// the upper half, and each adds the partner's matching half to its own.
template <int N, int J, int V>
__device__ __forceinline__ void halve(float (&v)[V], int lane) {
  const bool upper = (lane & J) != 0;
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float lo = v[i], hi = v[i + N / 2];
    const float keep = upper ? hi : lo, send = upper ? lo : hi;
    v[i] = keep + xor_lane_f32<J>(send, lane);
  }
}

// Gate layouts.  SHARED: thread t takes the 16-byte chunks t, t + 256, ...
// of all RPB gate rows of the block, so each token chunk is loaded once per
// block (RPB * MAXM = 16 sums per thread, reduced by a halving butterfly).
// Otherwise each gate row is split over 4 / RPB waves and a thread streams
// its share of one row against every token row (one sum per token, reduced
// by wave sums).  Both leave thread tid < RPB * MAXM with the logit of gate
// row row0 + tid / MAXM and token tid % MAXM (valid for tokens < M).
// Wave totals of V = 16 or 32 sums per lane: log2(V) halving steps leave
// lane l with one sum over V lanes (value index bitrev(l mod V)), full steps
// add the rest of the wave.  A fixed tree: the result does not depend on
// timing.  Returns the total and sets idx to its value index.
template <int V>
__device__ __forceinline__ float wave_totals(float (&v)[V], int lane, int &idx) {
  static_assert(V == 16 || V == 32 || V == 64, "16, 32 or 64 sums per lane");
  halve<V, 1>(v, lane);
  halve<V / 2, 2>(v, lane);
  halve<V / 4, 4>(v, lane);
  halve<V / 8, 8>(v, lane);
  if constexpr (V >= 32) halve<V / 16, 16>(v, lane);
  if constexpr (V == 64) halve<2, 32>(v, lane);
  float t = v[0];
  if constexpr (V == 16) t += xor_lane_f32<16>(t, lane);
  if constexpr (V <= 32) t += xor_lane_f32<32>(t, lane);
  idx = 0;
#pragma unroll
  for (int b = 0; (1 << b) < V; ++b) idx |= ((lane >> b) & 1) << (__builtin_ctz(V) - 1 - b);
  return t;
}

// ML: token rows the shared-chunk gate loads and dots (the others keep zero
// sums): fewer than MAXM when a launch is known to have M <= ML.
// GT > 0: token-tiled gate (shared-chunk layout): a block takes RPB gate
// rows against GT token rows only, so it streams RPB + GT rows instead of
// RPB + M.
template <int RPB, int MAXM, bool SHARED, int NK, int ML = MAXM, int GT = 0>
__global__ __launch_bounds__(kThreads) void route_small_kernel(SmallParams p) {
  static_assert(GT == 0 || SHARED, "token tiles use the shared-chunk layout");
  constexpr int GM = GT ? GT : MAXM;  // token rows in a block's gate sums
  constexpr int GL = GT ? GT : ML;    // of which the gate loads
  constexpr int V = RPB * GM;
  constexpr int WPR = (kThreads / kWave) / RPB;  // waves per gate row (split layout)
  static_assert(!SHARED || V == 16 || V == 32 || V == 64, "the butterfly reduces 16, 32 or 64 sums per thread");
  __shared__ float red[kThreads / kWave][SHARED ? V : MAXM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // token tiles: the blocks of one gate-row group sit on one XCD (block b
  // runs on XCD b mod 8), so each gate row is fetched into one L2 only
  const int ntg = GT ? (p.M + GT - 1) / GT : 1;
  const int q8 = (int)blockIdx.x >> 3;
  const int row0 = (GT ? (q8 / ntg) * 8 + ((int)blockIdx.x & 7) : (int)blockIdx.x) * RPB;
  const int m0 = GT ? (q8 % ntg) * GT : 0;  // first token row of the gate sums
  const int H = p.H, M = p.M;
  const int nch = H >> 3;  // 16-byte chunks per row

  // align bitmaps of block 0's tail: zeroed now, off the tail's path (the
  // gate's block barrier orders these stores before the tail's marks)
  constexpr int BW = (MAXM + 31) / 32;  // words of token-row bits per expert
  __shared__ __attribute__((aligned(16))) uint32_t rowbm[(kWave * NK + 1) * BW];  // E' <= 64 NK + 1
  __shared__ uint32_t touched[kMaxRouteExperts / 32 + 1];
  __shared__ uint32_t failed;  // a wait of this block gave up
  if (blockIdx.x == 0 && p.do_align && !p.logits_only) {
    for (int e = tid; e < p.Ep * BW; e += kThreads) rowbm[e] = 0u;
    for (int w = tid; w < ((p.Ep + 31) >> 5); w += kThreads) touched[w] = 0u;
  }
  if (tid == 0) failed = 0u;
  stamp(p, 0);

  // ---- sentinel pre-fill of sorted_token_ids ---------------------------
  // Only blocks that block 0 waits for take a slice: a block with a live
  // gate row publishes keys (or the shared logit) after its slice is
  // complete, and a tail wave polls every key of its row before it hands its
  // ids to block 0; a tail block hands its ids over itself.  Untiled, every
  // block is one or the other.  With token tiles the grid rounds the row
  // groups up to whole XCDs, and a block of a padding row group that is no
  // tail block publishes nothing and is waited for by no one: a slice of its
  // could still be in flight when block 0 writes the same slots.  There the
  // first p.fill_blocks blocks, chosen by the launch, take the slices.
  if (p.do_align && (GT == 0 || (int)blockIdx.x < p.fill_blocks)) {
    const int32_t sentinel = M * p.S;
    const int64_t nf = GT ? (int64_t)p.fill_blocks : (int64_t)gridDim.x;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + tid; i < p.fill_count; i += nf * kThreads)
      st_agent(p.sorted + i, sentinel);
  }

  if constexpr (SHARED) {
    // ---- gate: the block's RPB gate rows against the M token rows ---------
    // Thread t takes the 16-byte chunks t, t + 256, ... of every row, so each
    // token chunk is loaded once per block and serves all RPB gate rows.  A
    // batch issues all its loads (gate chunks non-temporal: read once) before
    // any arithmetic.  Tokens past M reload token M-1 and rows past E' row
    // E'-1 (those sums are dropped), but a block with no row below E' (the
    // row groups that round the grid up to whole XCDs) skips the loop: their
    // clamped loads of row E'-1, non-temporal and from many blocks at once,
    // delayed that row's own blocks by up to 4 us (M = 16).
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.0f;
    const uint4 *wr[RPB];
#pragma unroll
    for (int r = 0; r < RPB; ++r) {
      const int e = min(row0 + r, p.Ep - 1);
      wr[r] = reinterpret_cast<const uint4 *>(e < p.E ? p.w + (size_t)e * H : p.ws_row);
    }
    const uint4 *xb = reinterpret_cast<const uint4 *>(p.x);
    constexpr int UB = (RPB + GL <= 18) ? 2 : 1;  // chunk positions per batch
    const int c_end = row0 < p.Ep ? nch : 0;  // block-uniform
    for (int c0 = tid; c0 < c_end; c0 += UB * kThreads) {
      uint4 wv[UB][RPB], xv[UB][GL];
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int c = min(c0 + u * kThreads, nch - 1);
#pragma unroll
        for (int r = 0; r < RPB; ++r) {
          // rows past E' load nothing (block-uniform), in the untiled layout:
          // with token tiles the per-row branch measured slower than the
          // clamped loads of the one partly used row group (C3 +0.7 us)
          if (GT > 0 || row0 + r < p.Ep) wv[u][r] = ld_stream_16(wr[r] + c);
          else wv[u][r] = make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int m = 0; m < GL; ++m) xv[u][m] = xb[(size_t)min(m0 + m, M - 1) * nch + c];
      }
      // branch-free (a selected sum for a chunk past the row), and fenced from
      // the loads, so that all the batch's loads are issued together
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const bool in = c0 + u * kThreads < nch;
#pragma unroll
        for (int r = 0; r < RPB; ++r)
#pragma unroll
          for (int m = 0; m < GL; ++m) {
            const float t = dot8_bf16(wv[u][r], xv[u][m], acc[r * GM + m]);
            acc[r * GM + m] = in ? t : acc[r * GM + m];
          }
      }
    }
    int idx;
    const float tot = wave_totals<V>(acc, lane, idx);
    if (lane < V) red[wave][idx] = tot;
    wait_own_stores();  // the pre-fill is complete before any key is published
    __syncthreads();
  } else {
    const int rloc = wave / WPR, sub = wave % WPR;
    const int row = row0 + rloc;
    // ---- gate: stream this wave's share of one gate row -----------------
    // Each iteration first issues every load it needs -- the gate-row chunks
    // (non-temporal: read once) and the same chunks of every token row -- and
    // only then accumulates, so a thread has all its loads in flight at once.
    float acc[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) acc[m] = 0.0f;
    if (row < p.Ep) {
      const uint4 *wrow = reinterpret_cast<const uint4 *>(row < p.E ? p.w + (size_t)row * H : p.ws_row);
      const uint4 *xb = reinterpret_cast<const uint4 *>(p.x);
      constexpr int kChunks = 2 * RPB;             // chunks per thread per iteration (H = 4096: one iteration)
      constexpr int kStride = WPR * kWave;         // threads sharing the row
      // token rows whose chunks are loaded together: 16 loads per group, but
      // never more rows than acc holds (with one gate row per block, 16 loads
      // would be 8 rows of 4 sums)
      constexpr int kRowsPerGroup = 16 / kChunks < MAXM ? 16 / kChunks : MAXM;
      static_assert(MAXM % kRowsPerGroup == 0, "whole groups of token rows");
      int c0 = sub * kWave + lane;
      for (; c0 + (kChunks - 1) * kStride < nch; c0 += kChunks * kStride) {
        uint4 wv[kChunks];
#pragma unroll
        for (int u = 0; u < kChunks; ++u) wv[u] = ld_stream_16(wrow + c0 + u * kStride);
#pragma unroll
        for (int g = 0; g < MAXM; g += kRowsPerGroup) {
          if (g < M) {
            uint4 xv[kRowsPerGroup][kChunks];
#pragma unroll
            for (int r = 0; r < kRowsPerGroup; ++r) {
              const int m = min(g + r, M - 1);  // rows past M reload row M-1; their sums are dropped
#pragma unroll
              for (int u = 0; u < kChunks; ++u) xv[r][u] = xb[(size_t)m * nch + c0 + u * kStride];
            }
#pragma unroll
            for (int r = 0; r < kRowsPerGroup; ++r)
#pragma unroll
              for (int u = 0; u < kChunks; ++u) acc[g + r] = dot8_bf16(wv[u], xv[r][u], acc[g + r]);
          }
        }
      }
      for (; c0 < nch; c0 += kStride) {  // ragged tail: one chunk at a time
        const uint4 wv = ld_stream_16(wrow + c0);
#pragma unroll
        for (int m = 0; m < MAXM; ++m)
          if (m < M) acc[m] = dot8_bf16(wv, xb[(size_t)m * nch + c0], acc[m]);
      }
    }
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
      if (m < M) {
        const float v = wave_sum_f32(acc[m]);
        if (lane == 0) red[wave][m] = v;
      }
    }
    wait_own_stores();  // the pre-fill is complete before any key is published
    __syncthreads();
  }
  if (tid < V) {
    const int r = tid / GM, m = m0 + tid % GM;
    const int e = row0 + r;
    float z;
    if constexpr (SHARED) {
      z = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
    } else {
      z = 0.0f;
#pragma unroll
      for (int s = 0; s < WPR; ++s) z += red[r * WPR + s][m];
    }
    if (m < M) {
      if (p.logits_only) {
        if (e < p.Ep) p.logits_out[(size_t)m * p.Ep + e] = z;
      } else if (e < p.E) {
        st_agent(p.keys + (size_t)m * p.E + e, make_key(z, (uint32_t)e));
      } else if (e == p.E && p.has_shared) {
        st_agent(p.shared_logit + m, (1ull << 32) | __float_as_uint(z));
      }
    }
  }
  stamp(p, 1);
  if (p.logits_only) return;
  if constexpr (MAXM > kThreads / kWave) {
    // M >= 5: the first ceil(M / 4) blocks take four token rows each, one
    // per wave; blocks 1.. hand their ids to block 0, which aligns (against
    // block 0 alone taking two rows per wave: -0.7 to -0.9 us at M = 5..8,
    // -2.7 to -3.8 us at M = 9..16).
    if ((int)blockIdx.x >= (M + 3) / 4) return;
    __shared__ int32_t lds_ids[MAXM * (kMaxTopK + 1)];
    const int m0 = 4 * blockIdx.x;
    route_tail_rows1<NK, BW>(p, lds_ids, rowbm, touched, m0, min(M, m0 + 4), blockIdx.x != 0 && p.do_align, &failed);
    if (blockIdx.x != 0 || !p.do_align) return;
    // up to 32 rows: one row per wave and poll; more: the flat poll (measured
    // at E' = 513: M = 40 13.2 -> 12.8 us, 64 16.6 -> 15.7; M = 5..17 were
    // 0.1 to 0.4 us faster with the rows)
    if constexpr (MAXM <= 32) gather_tail_rows<MAXM, BW>(p, lds_ids, rowbm, touched, &failed);
    else gather_tail_flat<MAXM, BW>(p, lds_ids, rowbm, touched, &failed);
    __syncthreads();  // every pair is marked and in lds_ids
    if constexpr (BW == 1) {
      align_small(p, lds_ids, rowbm, touched, &failed);
    } else {
      __shared__ uint32_t boff[kMaxRouteExperts + 1];
      __shared__ uint32_t scan_tmp[kThreads / kWave + 1];
      align_small_wide<BW>(p, lds_ids, rowbm, boff, scan_tmp, &failed);
    }
    stamp(p, 6);
    return;
  }
  if (blockIdx.x != 0) return;

  // ---- block 0: the tail ---------------------------------------------------
  __shared__ int32_t lds_ids[MAXM * (kMaxTopK + 1)];
  route_tail_rows1<NK, BW>(p, lds_ids, rowbm, touched, 0, p.M, false, &failed);
  if (p.do_align) {
    __syncthreads();  // every pair is marked and in lds_ids
    align_small(p, lds_ids, rowbm, touched, &failed);
  }
  stamp(p, 6);
}

template <int RPB, int MAXM, bool SHARED, int ML = MAXM, int GT = 0>
hipError_t launch_nk(const SmallParams &p, hipStream_t stream) {
  const int nrg = (p.Ep + RPB - 1) / RPB;  // gate-row groups
  // token tiles: row groups rounded up to a multiple of 8 (one XCD per group)
  int grid = GT ? (nrg + 7) / 8 * 8 * ((p.M + GT - 1) / GT) : nrg;
  // at M >= 5 the first ceil(M / 4) blocks also run the tail: there must be
  // that many (extra blocks own no gate rows: their sums are dropped)
  if (MAXM > kThreads / kWave && grid < (p.M + 3) / 4) grid = (p.M + 3) / 4;
  // Token tiles: the pre-fill slices go to blocks that block 0 waits for.
  // Block b holds row group 8 * (b / 8 / T) + b % 8 of T token tiles, so
  // the first 8 * T * floor(nrg / 8) blocks own live rows, and the first
  // ceil(M / 4) are tail blocks.
  SmallParams q = p;
  q.fill_blocks = grid;
  if (GT) {
    const int live = nrg / 8 * 8 * ((p.M + GT - 1) / GT), tail = (p.M + 3) / 4;
    q.fill_blocks = live > tail ? live : tail;
  }
  const int nk = (p.E + kWave - 1) / kWave;
  if (nk <= 2) route_small_kernel<RPB, MAXM, SHARED, 2, ML, GT><<<grid, kThreads, 0, stream>>>(q);
  else if (nk <= 4) route_small_kernel<RPB, MAXM, SHARED, 4, ML, GT><<<grid, kThreads, 0, stream>>>(q);
  else if (nk <= 8) route_small_kernel<RPB, MAXM, SHARED, 8, ML, GT><<<grid, kThreads, 0, stream>>>(q);
  else route_small_kernel<RPB, MAXM, SHARED, 16, ML, GT><<<grid, kThreads, 0, stream>>>(q);
  return hipGetLastError();
}

}  // namespace

int small_rows_per_block(int Ep, int M) {
  // Measured per token count at E' = 513, H = 4096: the shared-chunk layout
  // (2 rows per block, 16 or 32 sums per thread) is faster for M >= 5; the
  // row-split layout (2 rows per block at E' > 256, else 1) for M <= 4.
  if (M >= 5) return 2;
  return Ep > 256 ? 2 : 1;
}

hipError_t launch_route_small(const SmallParams &p, hipStream_t stream) {
  if (p.M <= 4) return small_rows_per_block(p.Ep, p.M) == 2 ? launch_nk<2, 4, false>(p, stream)
                                                            : launch_nk<1, 4, false>(p, stream);
  if (p.M <= 8) return launch_nk<2, 8, true>(p, stream);
  // M >= 9: token tiles.  A block dots 4 gate rows with 4 (M <= 20) or 8
  // token rows, the blocks of one row group on one XCD.  Measured at E' =
  // 513, H = 4096 against every block taking 2 gate rows and all M token
  // rows: M = 9 -0.5 us, 16 -0.5, 17 -2.1, 24 -2.3, 32 -2.9 (4 x 8 tiles are
  // the faster of the two from M = 24; at M = 5..8 and M <= 4 tiles were
  // slower by 0.35 to 0.5 us)
  // More than 32 rows, or an align whose blocks of A slots can hold more
  // than one block's worth of an expert's pairs: 4 words of row bits per
  // expert and the general align.
  // The token tile depends on M alone, so mr_route, mr_route_align and the
  // logits hook sum every logit in the same order.  Above 64 rows 16-row
  // tiles (C3: 12.0 -> 11.2 us; at M = 40 they were 1.4 us slower than 8).
  if (p.M > 64) return launch_nk<4, 128, true, 128, 16>(p, stream);
  const bool wide = p.M > 32 || (p.do_align && p.A < p.M);
  if (p.M <= 20) return wide ? launch_nk<4, 64, true, 64, 4>(p, stream) : launch_nk<4, 32, true, 32, 4>(p, stream);
  return wide ? launch_nk<4, 64, true, 64, 8>(p, stream) : launch_nk<4, 32, true, 32, 8>(p, stream);
}

}  // namespace mr
