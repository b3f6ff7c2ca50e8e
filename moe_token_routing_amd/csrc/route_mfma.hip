// route_mfma.hip -- one-launch router + align for prefill token counts
// (M > 128, or M > 32 with more gate work than the small-M launch takes):
// the gate pass is a split-K MFMA tile contraction.
//
// Computes what "[AMD] One-launch small-M MoE router ... on gfx950"
// (sglang), Modifications, and "W4A16 MoE prefill: M-aware moe_align block
// size" (ROCm vLLM), Purpose, describe: routed logits z = x W^T and the
// shared logit s = x ws in fp32, r = bf16(z) (nearest even), the k largest r
// with the lower id winning ties, softmax renormalised over the chosen k,
// slot k = (E, scale * sigmoid(s)), then moe_align_block_size over the M*S
// (token, slot) pairs.
//
// One persistent launch of `grid` blocks (every block resident: the host
// sizes the grid from the occupancy API), 256 threads each, in three phases
// separated by grid barriers:
//
// G. Gate.  Work items are (expert tile of 128, token tile of 128, K split).
//    Operands stream into a 4-stage LDS ring with gfx950's 16-byte global ->
//    LDS loads (64 k-values per stage: 16 KB of gate rows + 16 KB of
//    tokens); 16-byte chunks are XOR-swizzled inside each 128-byte row so
//    the MFMA fragment reads are free of bank conflicts.  The 4 waves form a
//    2 x 2 grid of 64 x 64 wave tiles, each 2 x 2 v_mfma_f32_32x32x16_bf16
//    tiles; the LDS reads of one 16-k step are issued before the MFMAs of
//    the previous one.  Each item writes its fp32 partial tile, transposed
//    through LDS into whole token rows, with write-through stores.  Items
//    are numbered token tile first, then K split, then expert tile, and the
//    blocks of one XCD (block b runs on XCD b mod 8 when the grid is a
//    multiple of 8) take consecutive items: every split of a token tile is
//    computed on one XCD, and the top-k phase reads those partial rows on
//    the same XCD, from its L2.  Correctness does not depend on this
//    placement: the partial rows are written through to memory.
// T. Top-k.  Each block owns token groups of tpb tokens (numbered like its
//    gate items, so they sit on the XCD that wrote them); a wave takes two
//    tokens at a time, sums their K-split partial rows straight from the
//    16-byte loads in a fixed split order (so the logits do not depend on
//    which block finished first), takes the shared-expert logits (those of
//    the block's first group are computed between its arrival at the first
//    barrier and the barrier's release, from x and the shared gate row
//    alone; a further group dots its two x rows with the shared gate row
//    while its partial-row loads are in flight), builds the packed keys,
//    takes k rounds of a wave-wide maximum, then the softmax, the shared
//    slot and the stores.  With more than one token tile, each routed pair
//    also bumps a per-(128-token tile, expert) counter.
// A. Align.  Every block turns the tile counters into padded expert offsets
//    (block scan) and the prefix of earlier tiles, adds the counts of the
//    earlier tokens of its own tile (read back from topk_ids, in the same
//    round of loads as the counters) and of its own earlier tokens (a bit
//    mask per expert), and scatters its pairs in parallel: inside an expert,
//    pairs keep ascending flat index.  With one token tile (M <= 128) there
//    are no counters: every block reads all M * S ids and counts them in
//    LDS (the counters' atomics, all on a few cache lines, cost more: C3
//    17.3 -> 15.8 us).  Blocks also pad the experts dealt to them and write
//    expert_ids; block 0 writes npp.
//
// Workspace: the counter words as the library leaves them (the grid
// barriers use one of two counter sets by the parity of a launch count; each
// launch clears the other set and block 0 advances the count at the end);
// the tile counters (one word per expert and 128-token tile, used with more
// than one tile) are cleared during phase G.
#include <atomic>

#include "device_common.h"
#include "kernels.h"

namespace mr {

namespace {

constexpr int kThreads = 256;
constexpr int kTE = 128, kTT = 128;      // experts x tokens per work item
constexpr int kKS = 64;                  // k-values per pipeline stage
constexpr int kNS = 4;                   // pipeline stages
constexpr int kRowBytes = kKS * 2;       // one operand row of a stage
constexpr int kStageBytes = (kTE + kTT) * kRowBytes;  // 32 KB
constexpr int kRingBytes = kNS * kStageBytes;          // 128 KB
constexpr int kTilePitch = kTT + 4;      // fp32 pitch of the transpose tile
constexpr int kOwnBytes = 17408;         // phases T and A: a group's ids (tpb * S <= 128 * 33) at the start of LDS

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// Slot of 16-byte chunk c of LDS row r (rows of 128 bytes).  Rows r and r+1
// differ in bank half, and the 8 even (odd) rows of any 16 consecutive rows
// take 8 different slots, so 16 lanes reading one chunk of 16 rows hit 16
// different bank groups.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// s_waitcnt on the vector memory counter only (GFX9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt and lgkmcnt at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 16-byte global -> LDS load: this lane's 16 bytes at `src` land at
// lds_base + 16 * lane.  Issued through inline assembly so the compiler does
// not treat every later LDS read as dependent on it (it would wait for all
// outstanding loads); the pipeline waits for these loads itself with
// wait_vmcnt before the barrier that publishes a stage.
// The LDS base goes in through an M0 operand (the compiler writes M0); the
// s_nop gives the M0 write its wait state before the load reads it.
__device__ __forceinline__ void load_lds16(const void *src, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "{m0}"(lds_base)
               : "memory");
}

__device__ __forceinline__ uint4 lds16(const uint8_t *p) { return *reinterpret_cast<const uint4 *>(p); }

__device__ __forceinline__ void st_agent2(float *p, float a, float b) {
  const unsigned long long v = (unsigned long long)__float_as_uint(a) | ((unsigned long long)__float_as_uint(b) << 32);
  st_agent(reinterpret_cast<unsigned long long *>(p), v);
}

// 16-byte write-through store (sc1, like st_agent): the partial tiles are
// read by other blocks after a grid barrier.  A store of more than 8 bytes
// reads its data registers after it issues, and a VALU write to them must
// wait; the compiler cannot see that this asm is such a store and may write
// those registers in the very next instruction, so the wait states are
// part of the asm (the store otherwise writes lanes' later values: seen as
// a few wrong partial sums).
__device__ __forceinline__ void st_agent16(float *p, u32x4_coh v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" : : "v"(p), "v"(v) : "memory");
}

// Launches with at most this many gate items store their partial tiles with
// 16-byte stores (measured: -0.7 us at 8-64 items; within noise or slightly
// slower at 128-256 items).
constexpr int kWideStoreItems = 64;

// Waits until this wave has at most n younger stages of DMA loads in flight
// (per = loads per stage for this wave).
template <int PER>
__device__ __forceinline__ void wait_stages(int n) {
  if (n >= 2) wait_vmcnt<2 * PER>();
  else if (n == 1) wait_vmcnt<PER>();
  else wait_vmcnt<0>();
}

// Grid barrier over all `grid` blocks, generation `gen` (1, 2, ...) of this
// launch, on counter set `set` (zero at launch start): each block takes a
// ticket on one of up to kTicketLanes first-level counters (256 bytes apart,
// so arrivals do not serialise on one address); the arrival that completes a
// lane takes a ticket on the set's top counter, and the one that completes
// the top counter writes `gen` into every lane's release word.  A block
// waits on its own lane's release word, so no address has more than
// grid / kTicketLanes pollers.  Data written with st_agent (or agent-scope
// atomics) before the barrier is visible to coherent loads (ld_agent,
// ld_coherent8) after it.  The wait is bounded (limit polls): if it gives
// up, its bit goes into the status word, the block's failed flag is raised
// and the block goes on.  Only thread 0's arguments matter.
__device__ __forceinline__ uint32_t *barrier_lane(uint32_t *ctr, uint32_t set, uint32_t r) {
  return ctr + 64 + (size_t)r * kTicketLaneStride + 32 * set;
}
__device__ __forceinline__ uint32_t *barrier_release(uint32_t *ctr, uint32_t set, uint32_t r) {
  return barrier_lane(ctr, set, r) + kReleaseWord;
}
__device__ __forceinline__ uint32_t *barrier_top(uint32_t *ctr, uint32_t set) {
  return ctr + (set ? kCtrBarTop1 : kCtrBarTop0);
}
// The barrier is split: grid_arrive publishes this block's arrival, and
// grid_wait returns once every block has arrived; work that needs no other
// block's data can run between the two.
__device__ __forceinline__ void grid_arrive(uint32_t *ctr, uint32_t set, uint32_t gen, uint32_t grid) {
  wait_own_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t nl = grid < (uint32_t)kTicketLanes ? grid : (uint32_t)kTicketLanes;
    const uint32_t r = blockIdx.x % nl;
    const uint32_t in_lane = (grid - 1 - r) / nl + 1;
    const uint32_t t = __hip_atomic_fetch_add(barrier_lane(ctr, set, r), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t == gen * in_lane - 1) {
      const uint32_t u = __hip_atomic_fetch_add(barrier_top(ctr, set), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (u == gen * nl - 1)
        for (uint32_t l = 0; l < nl; ++l)
          __hip_atomic_store(barrier_release(ctr, set, l), gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}
// Thread 0 polls *word until it reaches `target`, at most `limit` times
// (none at limit 0); on giving up it ORs `bit` into the status word and
// raises *failed.
__device__ __forceinline__ void bounded_wait(const uint32_t *word, uint32_t target, int limit, uint32_t *ctr,
                                             uint32_t bit, uint32_t *failed) {
  bool done = false;
  for (int it = 0; it < limit; ++it) {
    if (__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) {
      done = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (!done) {
    __hip_atomic_fetch_or(ctr + kCtrError, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *failed = 1u;
  }
}
__device__ __forceinline__ void grid_wait(uint32_t *ctr, uint32_t set, uint32_t gen, uint32_t grid, int limit,
                                          uint32_t *failed) {
  if (threadIdx.x == 0) {
    const uint32_t nl = grid < (uint32_t)kTicketLanes ? grid : (uint32_t)kTicketLanes;
    bounded_wait(barrier_release(ctr, set, blockIdx.x % nl), gen, limit, ctr, kWaitGrid, failed);
  }
  __syncthreads();
}
__device__ __forceinline__ void grid_barrier(uint32_t *ctr, uint32_t set, uint32_t gen, uint32_t grid, int limit,
                                             uint32_t *failed) {
  grid_arrive(ctr, set, gen, grid);
  grid_wait(ctr, set, gen, grid, limit, failed);
}

// Tile-ready counter of token tile t in counter set `set` (zero at launch
// start): every gate item of the tile takes one after its partial tile and
// its share of the tile's counter-row clear have completed.
__device__ __forceinline__ uint32_t *tile_ready(uint32_t *ctr, uint32_t set, int t) {
  return ctr + kReadyBase + (size_t)(2 * t + (int)set) * kReadyStride;
}
__device__ __forceinline__ void tile_arrive(uint32_t *ctr, uint32_t set, int t) {
  wait_own_stores();
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(tile_ready(ctr, set, t), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until all `count` items of token tile t have arrived (bounded, like
// grid_wait).  Every thread of the block must call it.
__device__ __forceinline__ void tile_wait(uint32_t *ctr, uint32_t set, int t, uint32_t count, int limit,
                                          uint32_t *failed) {
  if (threadIdx.x == 0) bounded_wait(tile_ready(ctr, set, t), count, limit, ctr, kWaitTile, failed);
  __syncthreads();
}

// Phase stamp i of this block (thread 0), when the caller asked for stamps.
__device__ __forceinline__ void stamp(const MfmaParams &p, int i) {
  if (p.stamps && threadIdx.x == 0) p.stamps[(size_t)blockIdx.x * kStamps + i] = __builtin_amdgcn_s_memrealtime();
}

// ------------------------------------------------------------- phase G ---

__device__ void gate_item(const MfmaParams &p, uint8_t *smem, int et, int tt, int sp, bool first) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = p.M, H = p.H, E = p.E;
  const int st0 = sp * p.spp;
  const int nst = min(p.spp, p.nstages - st0);
  const uint32_t sbase = (uint32_t)(uintptr_t)smem;

  // DMA sources: this wave fills rows [32w, 32w+32) of both operand tiles, 8
  // rows per instruction; lane = row (lane / 8), destination slot lane % 8.
  const int lr = lane >> 3, slot = lane & 7;
  const uint16_t *arow[4], *brow[4];
  int acol[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 32 + i * 8 + lr;
    arow[i] = p.w + (size_t)min(et * kTE + r, E - 1) * H;
    brow[i] = p.x + (size_t)min(tt * kTT + r, M - 1) * H;
    acol[i] = swz(r, slot) * 8;  // element offset of the chunk this lane fetches
  }
  auto issue = [&](int st) {  // stage st of this item into ring slot st % kNS
    const int k0 = (st0 + st) * kKS;
    const uint32_t dst = sbase + (st % kNS) * kStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = k0 + acol[i];
      const void *src = kk < H ? (const void *)(arow[i] + kk) : (const void *)p.zero16;
      load_lds16(src, __builtin_amdgcn_readfirstlane(dst + (wave * 32 + i * 8) * kRowBytes));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = k0 + acol[i];
      const void *src = kk < H ? (const void *)(brow[i] + kk) : (const void *)p.zero16;
      load_lds16(src, __builtin_amdgcn_readfirstlane(dst + kTE * kRowBytes + (wave * 32 + i * 8) * kRowBytes));
    }
  };
  constexpr int kPerStage = 8;  // loads per stage per wave

  const int wr = wave >> 1, wc = wave & 1;
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  int ra[2], rb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    ra[i] = wr * 64 + i * 32 + (lane & 31);
    rb[i] = wc * 64 + i * 32 + (lane & 31);
  }

  // Fragments of one 16-k step: a[2] (gate rows), b[2] (tokens).  Step g
  // reads stage g / 4, chunk pair g % 4.
  auto load_frags = [&](int g, uint4 (&a)[2], uint4 (&b)[2]) {
    const int st = g >> 2, q = g & 3;
    const uint8_t *As = smem + (st % kNS) * kStageBytes;
    const uint8_t *Bs = As + kTE * kRowBytes;
    const int c = q * 2 + (lane >> 5);  // this lane's 8-value chunk of the step
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = lds16(As + ra[i] * kRowBytes + swz(ra[i], c) * 16);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = lds16(Bs + rb[j] * kRowBytes + swz(rb[j], c) * 16);
  };
  auto mma = [&](const uint4 (&a)[2], const uint4 (&b)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i]), as_bf16x8(b[j]), acc[i][j], 0, 0, 0);
  };
  // Stage st is usable once this wave has waited for its own loads of it
  // and every wave has passed the barrier; the barrier also frees the ring
  // slot of stage st - 1, which takes stage st + kNS - 1.  While st + kNS - 1
  // < nst the lookahead is full (kNS - 2 younger stages may stay in flight).
  auto enter_full = [&](int st) {
    wait_vmcnt<kPerStage * (kNS - 2)>();
    __syncthreads();
    issue(st + kNS - 1);
  };
  auto enter_tail = [&](int st) {
    wait_stages<kPerStage>(nst - st - 1);  // every remaining stage is already issued
    __syncthreads();
  };

  const int npre = min(nst, kNS - 1);
  for (int st = 0; st < npre; ++st) issue(st);
  // Software pipeline over 16-k steps (4 per stage): the LDS reads of step
  // g + 1 are issued before the MFMAs of step g, so the two overlap.  Stage
  // boundaries sit between the MFMAs of a stage's third step and its last.
  uint4 a0[2], b0[2], a1[2], b1[2];
  if (kNS - 1 < nst) enter_full(0);
  else enter_tail(0);
  load_frags(0, a0, b0);
  auto stage_head = [&](int st) {  // steps 4st .. 4st+2 and the reads of 4st+3
    const int g = st * 4;
    load_frags(g + 1, a1, b1);
    mma(a0, b0);
    load_frags(g + 2, a0, b0);
    mma(a1, b1);
    load_frags(g + 3, a1, b1);
    mma(a0, b0);
  };
  int st = 0;
  for (; st + kNS < nst; ++st) {  // the next stage enters with full lookahead
    stage_head(st);
    enter_full(st + 1);
    load_frags(st * 4 + 4, a0, b0);
    mma(a1, b1);
  }
  for (; st + 1 < nst; ++st) {  // the next stage enters from the tail
    stage_head(st);
    enter_tail(st + 1);
    load_frags(st * 4 + 4, a0, b0);
    mma(a1, b1);
  }
  stage_head(st);  // last stage
  mma(a1, b1);

  // partial tile -> LDS [token][expert] -> whole token rows in global memory
  __syncthreads();  // every wave is done with the ring
  if (first) stamp(p, 1);
  float *tile = reinterpret_cast<float *>(smem);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // 32x32 output layout: lane holds column (token) lane % 32 and rows
        // (experts) 8g + 4 (lane / 32) + {0..3} in elements 4g..4g+3
        const int t = rb[j];
        const int e0 = wr * 64 + i * 32 + 8 * g + 4 * (lane >> 5);
        float4 v;
        v.x = acc[i][j][4 * g + 0];
        v.y = acc[i][j][4 * g + 1];
        v.z = acc[i][j][4 * g + 2];
        v.w = acc[i][j][4 * g + 3];
        *reinterpret_cast<float4 *>(tile + t * kTilePitch + e0) = v;
      }
  __syncthreads();
  if (p.items <= kWideStoreItems) {
    // Few items: each block's store issue rate sets the time, so every lane
    // stores 16 bytes (a wave instruction covers two token rows, wave + 4i
    // and wave + 4i + 4); 8 instructions' LDS reads are issued first.
    const int half = lane >> 5, l32 = lane & 31;
    const int ecol = et * kTE + 4 * l32;
    for (int r0 = wave; r0 < kTT; r0 += 16 * (kThreads / kWave)) {
      u32x4_coh v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = *reinterpret_cast<const u32x4_coh *>(tile + (r0 + 4 * (2 * u + half)) * kTilePitch + 4 * l32);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int t = tt * kTT + r0 + 4 * (2 * u + half);
        if (t < M && ecol < E) st_agent16(p.part + ((size_t)sp * M + t) * p.Epad + ecol, v[u]);
      }
    }
  } else {
    // Many items: the XCDs' write paths set the time; 8-byte stores, each
    // wave writing rows wave, wave + 4, ... (8 rows' LDS reads issued first).
    const int ecol = et * kTE + 2 * lane;
    for (int r0 = wave; r0 < kTT; r0 += 8 * (kThreads / kWave)) {
      float2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float2 *>(tile + (r0 + 4 * u) * kTilePitch + 2 * lane);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int t = tt * kTT + r0 + 4 * u;
        if (t < M && ecol < E)
          st_agent(reinterpret_cast<unsigned long long *>(p.part + ((size_t)sp * M + t) * p.Epad + ecol),
                   (unsigned long long)__float_as_uint(v[u].x) | ((unsigned long long)__float_as_uint(v[u].y) << 32));
      }
    }
  }
  __syncthreads();  // the tile region is the next item's ring
}

// ------------------------------------------------------------- phase T ---

// Shared-expert logits of tokens ma and mb: their x rows dotted with the
// shared gate row in fp32, in a fixed summation order.  A lane takes the
// 16-byte chunks lane + 64 u of the rows, 8 chunks per batch, and the gate
// chunks of a batch serve both tokens; all loads of a batch are issued before
// its arithmetic.  x and the gate rows are never written by the launch, so
// plain loads are fine.  Returns wave-uniform values.
__device__ float2 shared_pair(const MfmaParams &p, int ma, int mb) {
  const int lane = threadIdx.x & 63;
  const int H = p.H, nch = H >> 3;  // 16-byte chunks per row
  const uint4 *wrow = reinterpret_cast<const uint4 *>(p.ws_row);
  const uint4 *xa = reinterpret_cast<const uint4 *>(p.x + (size_t)ma * H);
  const uint4 *xb = reinterpret_cast<const uint4 *>(p.x + (size_t)mb * H);
  float acc_a[8], acc_b[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc_a[u] = acc_b[u] = 0.f;
  for (int c0 = 0; c0 < nch; c0 += 64 * 8) {
    uint4 wv[8], av[8], bv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = min(c0 + 64 * u + lane, nch - 1);
      wv[u] = wrow[c];
      av[u] = xa[c];
      bv[u] = xb[c];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c0 + 64 * u + lane < nch) {
        acc_a[u] = dot8_bf16(av[u], wv[u], acc_a[u]);
        acc_b[u] = dot8_bf16(bv[u], wv[u], acc_b[u]);
      }
  }
  float2 r;
  r.x = wave_sum_f32(((acc_a[0] + acc_a[1]) + (acc_a[2] + acc_a[3])) + ((acc_a[4] + acc_a[5]) + (acc_a[6] + acc_a[7])));
  r.y = wave_sum_f32(((acc_b[0] + acc_b[1]) + (acc_b[2] + acc_b[3])) + ((acc_b[4] + acc_b[5]) + (acc_b[6] + acc_b[7])));
  return r;
}


// Shared logits of the tokens [t0, t1) (t1 - t0 <= 128) into sh[m - t0]:
// wave w takes the token pairs (t0 + w + 8 i, t0 + w + 8 i + 4), the pairs
// phase T gives it.
__device__ void shared_logits(const MfmaParams &p, int t0, int t1, float *sh) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int ma = t0 + wave; ma < t1; ma += 8) {
    const int mb = ma + 4 < t1 ? ma + 4 : ma;
    const float2 v = shared_pair(p, ma, mb);
    if (lane == 0) {
      sh[ma - t0] = v.x;
      sh[mb - t0] = v.y;
    }
  }
}

// Phase T for E <= 128 and S <= 32: a token's logits fill half a wave (32
// lanes of 4 experts), so a wave takes its two tokens side by side, lanes
// 0..31 the first (ma) and 32..63 the second (mb): the partial-row loads
// (every lane's 16 bytes are a real chunk), the key sort and every
// selection round run once for both, with maxima and sums over 32 lanes.
// The split order of the sums, the keys and the selection rule are those of
// the full-wave path, and the softmax sum adds the same values in the same
// order, so the outputs are the same.  Tokens as there: t0 + wave + 4 i,
// two at a time.
__device__ void topk_halves(const MfmaParams &p, int32_t *own, int t0, int t1, const float *sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, hl = lane & 31;
  const int M = p.M, E = p.E, k = p.k, S = p.S, SK = p.SK, Epad = p.Epad;
  const int ch = min(hl, (Epad >> 2) - 1);  // this lane's 16-byte chunk of a partial row
  const int ntw = (t1 - t0 > wave) ? (t1 - t0 - wave + 3) / 4 : 0;
  constexpr int SB = 16;  // splits per batch of loads
  for (int ti = 0; ti < ntw; ti += 2) {
    const bool two = ti + 1 < ntw;
    const int ma = t0 + wave + 4 * ti, mb = two ? ma + 4 : ma;
    const int m = half ? mb : ma;
    const bool mine_store = half == 0 || two;  // with one token the upper half only shadows it
    float z[4] = {0.f, 0.f, 0.f, 0.f};
    float2 shl = make_float2(0.f, 0.f);
    for (int s0 = 0; s0 < SK; s0 += SB) {
      u32x4_coh v[SB];
#pragma unroll
      for (int s = 0; s < SB; ++s) {
        const int sp = min(s0 + s, SK - 1);
        v[s] = reinterpret_cast<const u32x4_coh *>(p.part + ((size_t)sp * M + m) * Epad)[ch];
      }
      if (s0 == 0 && p.has_shared) shl = sh ? make_float2(sh[ma - t0], sh[mb - t0]) : shared_pair(p, ma, mb);
#pragma unroll
      for (int s = 0; s < SB; ++s)
        if (s0 + s < SK) {
#pragma unroll
          for (int i = 0; i < 4; ++i) z[i] += __uint_as_float(v[s][i]);
        }
    }
    const float sl = half ? shl.y : shl.x;
    if (p.logits_only) {
      if (mine_store) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * hl + i < E) p.logits_out[(size_t)m * p.Ep + 4 * hl + i] = z[i];
        if (p.has_shared && hl == 0) p.logits_out[(size_t)m * p.Ep + E] = sl;
      }
      continue;
    }
    uint32_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) key[i] = 4 * hl + i < E ? make_key(z[i], (uint32_t)(4 * hl + i)) : 0u;
    sort_desc_u32(key);
    // k rounds of the half-wave maximum of the lanes' heads; the lane that
    // held it drops its head (keys are unique)
    uint32_t mine = 0u;
    for (int j = 0; j < k; ++j) {
      const uint32_t top = half_max_all_u32(key[0]);
      mine = hl == j ? top : mine;
      const uint32_t keep = key[0] != top ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int i = 0; i < 3; ++i) key[i] = min(key[i], key[i + 1] | keep);
      key[3] &= keep;
    }
    // softmax over the chosen k (each half's own first logit and sum), the
    // shared slot, the stores
    const float r = key_value(mine);
    const float r0a = readlane_f32(r, 0), r0b = readlane_f32(r, 32);
    const float ex = hl < k ? expf(r - (half ? r0b : r0a)) : 0.0f;
    float t = ex;
    t += dpp_f32<kQuadXor1>(t);
    t += dpp_f32<kQuadXor2>(t);
    t += dpp_f32<kRowHalfMirror>(t);
    t += dpp_f32<kRowMirror>(t);
    const float da = readlane_f32(t, 0) + readlane_f32(t, 16), db = readlane_f32(t, 32) + readlane_f32(t, 48);
    int32_t id = (int32_t)key_id(mine);
    float w = ex / (half ? db : da);
    if (p.has_shared && hl == k) {
      id = E;
      w = p.scale / (1.0f + expf(-sl));
    }
    if (hl < S && mine_store) {
      st_agent(p.ids + (size_t)m * S + hl, id);
      p.wts[(size_t)m * S + hl] = w;
      own[(m - t0) * S + hl] = id;
      if (p.do_align && p.NT > 1 && hl < k)  // (one token tile: the align counts the ids itself)
        __hip_atomic_fetch_add(p.tcnt + (size_t)(m >> 7) * p.tcnt_row + id, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// sh: the shared logits of group g's tokens when the caller computed them
// already (else null).
template <int NKP>  // E <= 128 * NKP
__device__ void topk_group(const MfmaParams &p, int32_t *own, int g, const float *sh) {
  constexpr int NCH = NKP >= 2 ? NKP / 2 : 1;  // 16-byte chunks of a partial row per lane
  constexpr int NK = 4 * NCH;                  // keys per lane
  constexpr int SB = 8 / NCH > 0 ? 8 / NCH : 1; // splits per batch of loads (<= 16 loads for two tokens)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int M = p.M, E = p.E, k = p.k, S = p.S, SK = p.SK, Epad = p.Epad;
  const int t0 = g * p.tpb, t1 = min(M, t0 + p.tpb);
  if constexpr (NKP == 1) {
    if (S <= 32) {
      topk_halves(p, own, t0, t1, sh);
      return;
    }
  }
  // compiled in only where E > 128 (E <= 128 takes all its splits in one
  // batch at H <= 2048, and the extra code slowed that instantiation)
  constexpr bool kCoop = NCH >= 2;
  const int rowc = Epad >> 2;  // 16-byte chunks per partial row
  // Lane l holds experts 4c .. 4c + 3 of the chunks c = l + 64 j, j < NCH:
  // the partial rows are summed straight from their 16-byte loads, in split
  // order (the logits do not depend on which block finished first).  Lanes
  // past the row read a clamped in-bounds chunk and are masked in the keys.
  int chunk[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) chunk[j] = min(lane + 64 * j, rowc - 1);
  // This wave's tokens are t0 + wave + 4i, taken two at a time.
  const int ntw = (t1 - t0 > wave) ? (t1 - t0 - wave + 3) / 4 : 0;
  auto sum_rows = [&](int ma, int mb, float (&za)[NK], float (&zb)[NK], float2 &shl) {
#pragma unroll
    for (int i = 0; i < NK; ++i) za[i] = zb[i] = 0.f;
    for (int s0 = 0; s0 < SK; s0 += SB) {
      u32x4_coh va[SB][NCH], vb[SB][NCH];
#pragma unroll
      for (int s = 0; s < SB; ++s) {
        const int sp = min(s0 + s, SK - 1);
        const u32x4_coh *ra = reinterpret_cast<const u32x4_coh *>(p.part + ((size_t)sp * M + ma) * Epad);
        const u32x4_coh *rb = reinterpret_cast<const u32x4_coh *>(p.part + ((size_t)sp * M + mb) * Epad);
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          va[s][j] = ra[chunk[j]];
          vb[s][j] = rb[chunk[j]];
        }
      }
      // the shared logits' loads follow the first batch, so their latency
      // overlaps it
      if (s0 == 0 && p.has_shared) shl = sh ? make_float2(sh[ma - t0], sh[mb - t0]) : shared_pair(p, ma, mb);
#pragma unroll
      for (int s = 0; s < SB; ++s)
        if (s0 + s < SK) {
#pragma unroll
          for (int j = 0; j < NCH; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              za[4 * j + i] += __uint_as_float(va[s][j][i]);
              zb[4 * j + i] += __uint_as_float(vb[s][j][i]);
            }
        }
    }
  };
  auto token_keys = [&](const float (&z)[NK], uint32_t (&keys)[NK]) {
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * (lane + 64 * j) + i;
        keys[4 * j + i] = e < E ? make_key(z[4 * j + i], (uint32_t)e) : 0u;
      }
    sort_desc_u32(keys);
  };
  // softmax over the chosen k, the shared slot, the stores
  auto finish = [&](int m, uint32_t mine, float sl) {
    const float r = key_value(mine);
    const float r0 = readlane_f32(r, 0);
    const float ex = (lane < k) ? expf(r - r0) : 0.0f;
    const float den = wave_sum_f32(ex);
    int32_t id = (int32_t)key_id(mine);
    float w = ex / den;
    if (p.has_shared && lane == k) {
      id = E;
      w = p.scale / (1.0f + expf(-sl));
    }
    if (lane < S) {
      st_agent(p.ids + (size_t)m * S + lane, id);
      p.wts[(size_t)m * S + lane] = w;
      own[(m - t0) * S + lane] = id;
      if (p.do_align && p.NT > 1 && lane < k)  // (one token tile: the align counts the ids itself)
        __hip_atomic_fetch_add(p.tcnt + (size_t)(m >> 7) * p.tcnt_row + id, 1u,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  if (kCoop && t1 - t0 == 1 && SK > SB) {
    const int ma = t0, mb = t0;
    float za[NK], zb[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) za[i] = zb[i] = 0.f;
    for (int s0 = wave; s0 < SK; s0 += 4 * SB) {
      u32x4_coh va[SB][NCH], vb[SB][NCH];
#pragma unroll
      for (int s = 0; s < SB; ++s) {
        const int sp = min(s0 + 4 * s, SK - 1);
        const u32x4_coh *ra = reinterpret_cast<const u32x4_coh *>(p.part + ((size_t)sp * M + ma) * Epad);
        const u32x4_coh *rb = reinterpret_cast<const u32x4_coh *>(p.part + ((size_t)sp * M + mb) * Epad);
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          va[s][j] = ra[chunk[j]];
          vb[s][j] = rb[chunk[j]];
        }
      }
#pragma unroll
      for (int s = 0; s < SB; ++s)
        if (s0 + 4 * s < SK) {
#pragma unroll
          for (int j = 0; j < NCH; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              za[4 * j + i] += __uint_as_float(va[s][j][i]);
              zb[4 * j + i] += __uint_as_float(vb[s][j][i]);
            }
        }
    }
    float *red = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(own) + kOwnBytes);  // [wave][token][NK][lane]
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      red[((2 * wave + 0) * NK + i) * 64 + lane] = za[i];
      red[((2 * wave + 1) * NK + i) * 64 + lane] = zb[i];
    }
    __syncthreads();
  }
  // A one-token group (M <= grid) whose splits take more than one batch of
  // loads: the four waves split the K splits (wave w sums splits w, w + 4,
  // ... in order), meet in LDS in a fixed order, and wave 0 goes on; the
  // logits still do not depend on timing.  (Measured: -0.4 us at M = 40;
  // with one batch (C3) or two-token groups (M = 512) it was slower, so
  // those keep the one-wave-per-token path.)
  const bool coop = kCoop && t1 - t0 == 1 && SK > SB;
  const int nsel = coop ? (wave == 0 ? 2 : 0) : ntw;
  for (int ti = 0; ti < nsel; ti += 2) {
    const bool two = coop ? t1 - t0 == 2 : ti + 1 < ntw;
    const int ma = coop ? t0 : t0 + wave + 4 * ti, mb = two ? (coop ? t0 + 1 : ma + 4) : ma;
    float za[NK], zb[NK];
    float2 shl = make_float2(0.f, 0.f);
    if (coop) {
      // every wave's share is in LDS (written before this loop)
      const float *red = reinterpret_cast<const float *>(reinterpret_cast<const uint8_t *>(own) + kOwnBytes);
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        za[i] = ((red[(0 * NK + i) * 64 + lane] + red[(2 * NK + i) * 64 + lane]) + red[(4 * NK + i) * 64 + lane]) +
                red[(6 * NK + i) * 64 + lane];
        zb[i] = ((red[(1 * NK + i) * 64 + lane] + red[(3 * NK + i) * 64 + lane]) + red[(5 * NK + i) * 64 + lane]) +
                red[(7 * NK + i) * 64 + lane];
      }
      if (p.has_shared) shl = sh ? make_float2(sh[ma - t0], sh[mb - t0]) : shared_pair(p, ma, mb);
    } else {
      sum_rows(ma, mb, za, zb, shl);
    }
    if (p.logits_only) {
      for (int h = 0; h < (two ? 2 : 1); ++h) {
        const int m = h ? mb : ma;
        const float(&z)[NK] = h ? zb : za;
#pragma unroll
        for (int j = 0; j < NCH; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 4 * (lane + 64 * j) + i;
            if (e < E) p.logits_out[(size_t)m * p.Ep + e] = z[4 * j + i];
          }
        if (p.has_shared && lane == 0) p.logits_out[(size_t)m * p.Ep + E] = h ? shl.y : shl.x;
      }
      continue;
    }
    uint32_t ka[NK], kb[NK];
    token_keys(za, ka);
    if (two) {
      token_keys(zb, kb);
      uint32_t mine_a, mine_b;  // the two selections interleave
      topk_sorted2_u32(ka, kb, k, lane, mine_a, mine_b);
      finish(ma, mine_a, shl.x);
      finish(mb, mine_b, shl.y);
    } else {
      finish(ma, topk_sorted_u32(ka, k, lane), shl.x);
    }
  }
  if (coop) __syncthreads();  // wave 0 is done with the LDS sums before they are reused
}

// ------------------------------------------------------------- phase A ---

// LDS layout of phase A (byte offsets into the dynamic LDS).  The group's ids
// (`own`, written in phase T) stay at the start; the phase-T staging slices
// above them are free again.
constexpr int kMaskOff = kOwnBytes;                     // per expert: 4 words of token bits
constexpr int kMaskWords = (kMaxRouteExperts + 1) * 4;
constexpr int kArrOff = kMaskOff + kMaskWords * 4;      // tot, pre, off, hist: per expert
constexpr int kArrWords = kMaxRouteExperts + 4;
constexpr int kRowBatch = 16;                          // tile rows of the counter table per round of loads
static_assert(kArrOff + 4 * kArrWords * 4 <= kRingBytes, "phase A layout");
static_assert(kMaxRouteExperts <= 4 * kThreads, "one 4-expert column chunk per thread");

// Places the pairs of token group g (own[] holds its ids) into
// sorted_token_ids and leaves, for every expert e, tot[e] (pairs over all
// tokens) and off[e] (padded start of its segment) in LDS; returns npp.
//
// A pair (m, j) of routed expert e goes to
//   off[e] + (pairs of e in the 128-token tiles before m's)
//          + (pairs of e among the earlier tokens of m's tile),
// so each expert's pairs keep ascending flat index m * S + j.  The first
// term comes from the per-(tile, expert) counters (one tile: none, and the
// totals come from counting all the ids), the second from the ids
// of the tile's tokens before the group (read back from topk_ids) plus a bit
// mask per expert of the group's own tokens.  The shared slot of token m
// sits at off[E] + m.  The counter table and the earlier ids are fetched in
// one round of loads.
__device__ uint32_t align_group(const MfmaParams &p, int g, const int32_t *own, uint8_t *smem,
                                uint32_t *scan_tmp) {
  const int tid = threadIdx.x;
  const int M = p.M, E = p.E, Ep = p.Ep, S = p.S, W = p.tcnt_row, NT = p.NT;
  uint32_t *mask = reinterpret_cast<uint32_t *>(smem + kMaskOff);
  uint32_t *tot = reinterpret_cast<uint32_t *>(smem + kArrOff);
  uint32_t *pre = tot + kArrWords, *off = pre + kArrWords, *hist = off + kArrWords;
  const bool has = g < p.ngroups;
  const int t0 = has ? g * p.tpb : 0, t1 = has ? min(M, t0 + p.tpb) : 0;
  const int tile = t0 >> 7, tstart = tile << 7;
  const int nmw = (p.tpb + 31) >> 5;  // mask words per expert
  // Loads first: the routed ids of the tile's tokens before the group
  // (contiguous in topk_ids; 8 per thread now, any rest later), then the
  // first rows of the counter table (one word per expert, tcnt_row words
  // per tile).  The histogram of the earlier ids and the masks of the own
  // tokens are built while the table is in flight.
  // A launch of one token tile keeps no counter table: every block reads all
  // M * S ids instead (at most 128 * 33) and counts the totals itself.
  const bool one_tile = NT == 1;
  const int nprev = (t0 - tstart) * S;
  const int nread = one_tile ? M * S : nprev;
  const uint32_t *prev = reinterpret_cast<const uint32_t *>(p.ids + (size_t)tstart * S);
  uint32_t pv[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) pv[u] = prev[min(u * kThreads + tid, max(nread - 1, 0))];
  // The counter table: thread t sums the column chunk of experts 4t .. 4t+3
  // over every tile row (tot) and over the rows before the group's tile
  // (pre), straight from 16-byte loads, kRowBatch rows per round.
  const int ce = 4 * tid;
  const bool has_c = ce < E;
  u32x4_coh v[kRowBatch];
  auto load_rows = [&](int r0) {
    const u32x4_coh *src = reinterpret_cast<const u32x4_coh *>(p.tcnt + (size_t)r0 * W + (has_c ? ce : 0));
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) v[u] = src[(size_t)min(u, NT - 1 - r0) * (W / 4)];
  };
  if (one_tile) {
    for (int e = tid; e < Ep; e += kThreads) {
      hist[e] = 0u;
      tot[e] = 0u;
      for (int w = 0; w < nmw; ++w) mask[e * nmw + w] = 0u;
    }
    __syncthreads();
    auto count = [&](int i, uint32_t e) {  // id e at flat index i of the tile
      if (i < nread && e < (uint32_t)E) {
        if (i < nprev) atomicAdd(hist + e, 1u);
        atomicAdd(tot + e, 1u);
      }
    };
#pragma unroll
    for (int u = 0; u < 8; ++u) count(u * kThreads + tid, pv[u]);
    for (int i0 = 8 * kThreads; i0 < nread; i0 += 8 * kThreads) {
      uint32_t w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = prev[min(i0 + u * kThreads + tid, nread - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) count(i0 + u * kThreads + tid, w[u]);
    }
  } else {
    load_rows(0);
    for (int e = tid; e < Ep; e += kThreads) {
      hist[e] = 0u;
      for (int w = 0; w < nmw; ++w) mask[e * nmw + w] = 0u;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u * kThreads + tid < nprev && pv[u] < (uint32_t)E) atomicAdd(hist + pv[u], 1u);
    for (int i0 = 8 * kThreads; i0 < nprev; i0 += 8 * kThreads) {
      uint32_t w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = prev[min(i0 + u * kThreads + tid, nprev - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u * kThreads + tid < nprev && w[u] < (uint32_t)E) atomicAdd(hist + w[u], 1u);
    }
  }
  const int npairs = (t1 - t0) * S;
  for (int i = tid; i < npairs; i += kThreads) {
    const int32_t e = own[i];
    if ((uint32_t)e < (uint32_t)E) {
      const int tok = i / S;
      atomicOr(mask + e * nmw + (tok >> 5), 1u << (tok & 31));
    }
  }
  uint32_t tot4[4] = {0u, 0u, 0u, 0u}, pre4[4] = {0u, 0u, 0u, 0u};
  if (one_tile) {
    __syncthreads();  // every id is counted
#pragma unroll
    for (int j = 0; j < 4; ++j) tot4[j] = (has_c && ce + j < E) ? tot[ce + j] : 0u;
  } else for (int r0 = 0; r0 < NT; r0 += kRowBatch) {
    if (r0) load_rows(r0);
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u)
      if (r0 + u < NT) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          tot4[j] += v[u][j];
          pre4[j] += (r0 + u < tile) ? v[u][j] : 0u;
        }
      }
  }
  // padded offsets: thread t's run is its own 4 experts; the shared expert
  // (id E, every token) comes after all routed experts
  const uint32_t amask = (uint32_t)p.A - 1u;
  uint32_t P[4], run = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    P[j] = (has_c && ce + j < E) ? (tot4[j] + amask) & ~amask : 0u;
    run += P[j];
  }
  uint32_t routed;
  uint32_t o = block_excl_scan_u32<kThreads>(run, scan_tmp, &routed);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (has_c && ce + j < E) {
      tot[ce + j] = tot4[j];
      pre[ce + j] = pre4[j];
      off[ce + j] = o;
      o += P[j];
    }
  uint32_t npp = routed;
  if (Ep > E) {
    npp += ((uint32_t)M + amask) & ~amask;
    if (tid == 0) {
      tot[E] = (uint32_t)M;
      off[E] = routed;
    }
  }
  __syncthreads();
  for (int i = tid; i < npairs; i += kThreads) {
    const int32_t e = own[i];
    const int tok = i / S;
    uint32_t dst;
    if ((uint32_t)e < (uint32_t)E) {
      const uint32_t *mk = mask + e * nmw;
      uint32_t rank = __popc(mk[tok >> 5] & ((1u << (tok & 31)) - 1u));
      for (int w = 0; w < (tok >> 5); ++w) rank += __popc(mk[w]);
      dst = off[e] + pre[e] + hist[e] + rank;
    } else if (e == E && p.has_shared) {
      dst = off[E] + (uint32_t)(t0 + tok);
    } else {
      continue;
    }
    // in range unless a wait gave up (the counts are then not to be trusted)
    if (dst < (uint64_t)p.sorted_cap) p.sorted[dst] = (t0 + tok) * S + (i - tok * S);
  }
  return npp;
}

template <int NKP>
__global__ __launch_bounds__(kThreads) void route_mfma_kernel(MfmaParams p) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  __shared__ uint32_t scan_tmp[kThreads / kWave + 1];
  __shared__ float sh_first[128];  // shared logits of the block's first token group
  __shared__ uint32_t failed;      // a wait of this block gave up (set by thread 0 only)
  const int b = blockIdx.x;
  const uint32_t grid = gridDim.x;
  if (threadIdx.x == 0) failed = 0u;
  stamp(p, 0);

  // Barrier counter set of this launch: the parity of the launch count.  The
  // other set was used by the previous launch (which has finished); block 0
  // clears it for the next launch.  Every block reads the count before its
  // first barrier arrival, and block 0 advances it only after the last
  // barrier, so all blocks agree on the set.
  uint32_t set = 0;
  if (threadIdx.x == 0 || b == 0) set = ld_agent(p.ctr + kCtrEpoch) & 1u;
  if (b == 0) {
    if (threadIdx.x < kTicketLanes) {
      __hip_atomic_store(barrier_lane(p.ctr, set ^ 1u, threadIdx.x), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(barrier_release(p.ctr, set ^ 1u, threadIdx.x), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (threadIdx.x == kTicketLanes) {
      __hip_atomic_store(barrier_top(p.ctr, set ^ 1u), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int t = threadIdx.x; t < kMaxReadyTiles; t += kThreads)
      __hip_atomic_store(tile_ready(p.ctr, set ^ 1u, t), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- G: gate partials -------------------------------------------------
  // The tile counters start from zero in every launch (the workspace layout
  // moves with M, so nothing else may be assumed about this region).  With
  // tile waits, the items of a token tile clear that tile's counter row
  // (each its share) before they arrive; otherwise every block clears a
  // slice and the grid barrier orders the clear before the top-k phase.
  const bool clear_tcnt = p.do_align && !p.logits_only && p.NT > 1;
  if (clear_tcnt && !p.tile_wait)
    for (int i = b * kThreads + threadIdx.x; i < p.NT * p.tcnt_row; i += (int)grid * kThreads)
      __hip_atomic_fetch_and(p.tcnt + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int per_xcd = p.xcd_map ? (int)grid / 8 : 0;
  const int lmap = p.xcd_map ? (b % 8) * per_xcd + b / 8 : b;
  const int tile_items = p.NE * p.SK;
  for (int it = 0;; ++it) {
    const int L = it * (int)grid + lmap;
    if (L >= p.items) break;
    const int et = L % p.NE, sp = (L / p.NE) % p.SK, tt = L / (p.NE * p.SK);
    gate_item(p, smem, et, tt, sp, it == 0);
    if (p.tile_wait) {
      if (clear_tcnt) {
        const int share = (p.tcnt_row + tile_items - 1) / tile_items, q = sp * p.NE + et;
        const int i1 = min(p.tcnt_row, (q + 1) * share);
        for (int i = q * share + threadIdx.x; i < i1; i += kThreads)
          __hip_atomic_fetch_and(p.tcnt + (size_t)tt * p.tcnt_row + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      tile_arrive(p.ctr, set, tt);
    }
  }
  stamp(p, 2);
  // phases T and A: block b takes token group lmap (+ grid, ...), so a
  // group's partial rows were written by blocks of its own XCD
  const int gb = lmap;
  // Touch the pages phases T and A read (this block's partial rows of every
  // split, the tile counters, its tile's ids) so that their address
  // translations are cached when those phases start; the latency overlaps
  // the wait at the barrier.  The values only keep the loads alive.  These
  // lines must not be cached in L2 before their writers are done (phases T
  // and A read them with plain loads after the barriers), hence ld_agent.
  uint32_t touch = 0;
  if (gb < p.ngroups) {
    const int lane = threadIdx.x & 63, m0 = gb * p.tpb;
    const int tstart = (m0 >> 7) << 7;
    if (threadIdx.x < 64) {
      const uint32_t *a = reinterpret_cast<const uint32_t *>(p.tcnt);
      if (lane < p.SK) a = reinterpret_cast<const uint32_t *>(p.part + ((size_t)lane * p.M + m0) * p.Epad);
      else if (lane == p.SK + 1 && p.ids) a = reinterpret_cast<const uint32_t *>(p.ids + (size_t)tstart * p.S);
      else if (lane == p.SK + 2 && p.ids) a = reinterpret_cast<const uint32_t *>(p.ids + (size_t)m0 * p.S);
      // a coherent load: it warms the translation without leaving a copy of
      // the line in this XCD's L2 (the data is written only after this)
      touch = ld_agent(a);
    }
  }
  // The shared logits of the block's first token group need only x and the
  // shared gate row: they are computed while the other blocks' items finish.
  if (!p.tile_wait) grid_arrive(p.ctr, set, 1, grid);
  if (p.has_shared && gb < p.ngroups) shared_logits(p, gb * p.tpb, min(p.M, gb * p.tpb + p.tpb), sh_first);
  if (!p.tile_wait) grid_wait(p.ctr, set, 1, grid, p.wait_limit, &failed);
  asm volatile("" : : "v"(touch));  // keeps the warm-up loads: their value is otherwise unused

  // ---- T: logits, top-k, weights ----------------------------------------
  // LDS from here on: this block's ids at the start (kept until phase A);
  // phase A's arrays follow them
  int32_t *own = reinterpret_cast<int32_t *>(smem);
  const bool align = p.do_align && !p.logits_only;
  // A block owns more than one group only for M > 128 * grid; then `own`
  // holds one group at a time and is reloaded in phase A.
  const bool multi = (int)grid < p.ngroups;
  for (int g = gb; g < p.ngroups; g += grid) {
    // with tile waits, a group starts once its own token tile's items are in
    if (p.tile_wait) tile_wait(p.ctr, set, (g * p.tpb) >> 7, (uint32_t)tile_items, p.wait_limit, &failed);
    if (g == gb) stamp(p, 3);
    topk_group<NKP>(p, own, g, (p.has_shared && g == gb) ? sh_first : nullptr);
  }
  stamp(p, 4);
  if (align) {
    grid_barrier(p.ctr, set, p.tile_wait ? 1 : 2, grid, p.wait_limit, &failed);
    stamp(p, 5);
    // A wait of any block that gave up before this barrier has set the
    // status word before arriving here; block 0 reads it now and uses it
    // last, so the load's latency hides under the align.
    uint32_t status = 0;
    if (b == 0 && threadIdx.x == 0) status = ld_agent(p.ctr + kCtrError);
    uint32_t npp = 0;
    if (!multi) {
      npp = align_group(p, gb, own, smem, scan_tmp);
    } else {
      for (int g = gb; g < p.ngroups; g += grid) {
        const int t0 = g * p.tpb, t1 = min(p.M, t0 + p.tpb);
        __syncthreads();  // the previous group is placed
        for (int i = threadIdx.x; i < (t1 - t0) * p.S; i += kThreads) own[i] = ld_agent(p.ids + (size_t)t0 * p.S + i);
        __syncthreads();
        npp = align_group(p, g, own, smem, scan_tmp);
      }
    }
    // npp = -1 marks a launch one of whose waits gave up
    if (b == 0 && threadIdx.x == 0) *p.npp = (failed || status) ? -1 : (int32_t)npp;
    // padding and expert_ids of the experts dealt to this block (the bounds
    // matter only after a wait gave up: the counts are then not to be trusted)
    const uint32_t *tot = reinterpret_cast<const uint32_t *>(smem + kArrOff);
    const uint32_t *off = tot + 2 * kArrWords;
    for (int e = b; e < p.Ep; e += grid) {
      const uint64_t c = tot[e], o = off[e];
      const uint64_t P = (c + (uint64_t)p.A - 1u) & ~((uint64_t)p.A - 1u);
      for (uint64_t i = c + threadIdx.x; i < P && o + i < (uint64_t)p.sorted_cap; i += kThreads)
        p.sorted[o + i] = p.M * p.S;
      for (uint64_t blk = (o >> p.log2A) + threadIdx.x; blk < ((o + P) >> p.log2A) && blk < (uint64_t)p.expert_cap;
           blk += kThreads)
        p.expert_ids[blk] = e;
    }
  }

  // ---- exit: block 0 advances the launch count ---------------------------
  // (every block has passed this launch's last barrier, so each has read the
  // count already)
  if (b == 0 && threadIdx.x == 0)
    __hip_atomic_fetch_add(p.ctr + kCtrEpoch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  stamp(p, 6);
}

template <int NKP>
const void *kernel_ptr() {
  return reinterpret_cast<const void *>(&route_mfma_kernel<NKP>);
}

}  // namespace

size_t mfma_lds_bytes() { return (size_t)kRingBytes; }

int mfma_nkp(int E) {
  const int need = (E + 127) / 128;
  return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
}

namespace {
std::atomic<int> g_capacity[4][kMaxDevices];  // [nkp index][device]: resident blocks, 0 = not yet known
}  // namespace

// Sets the dynamic-LDS limit of the instantiation for nkp index ki on the
// current device and caches how many of its blocks fit on the device at
// once.  Returns that number, or 0 if a runtime query failed.
static int mfma_setup(int ki, int dev) {
  const void *fn = ki == 0 ? kernel_ptr<1>() : ki == 1 ? kernel_ptr<2>() : ki == 2 ? kernel_ptr<4>() : kernel_ptr<8>();
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)mfma_lds_bytes()) != hipSuccess)
    return 0;
  int ncu = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, mfma_lds_bytes()) != hipSuccess) return 0;
  const int cap = ncu * per_cu;
  g_capacity[ki][dev].store(cap, std::memory_order_relaxed);
  return cap;
}

int mfma_capacity(int E) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  const int nkp = mfma_nkp(E);
  const int ki = nkp == 1 ? 0 : nkp == 2 ? 1 : nkp == 4 ? 2 : 3;
  const int cap = g_capacity[ki][dev].load(std::memory_order_relaxed);
  return cap > 0 ? cap : mfma_setup(ki, dev);
}

bool mfma_prepare(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return false;
  for (int ki = 0; ki < 4; ++ki)
    if (mfma_setup(ki, dev) < 1) return false;
  return true;
}

hipError_t launch_route_mfma(const MfmaParams &p, hipStream_t stream) {
  const size_t lds = mfma_lds_bytes();
  switch (mfma_nkp(p.E)) {
    case 1: route_mfma_kernel<1><<<p.grid, kThreads, lds, stream>>>(p); break;
    case 2: route_mfma_kernel<2><<<p.grid, kThreads, lds, stream>>>(p); break;
    case 4: route_mfma_kernel<4><<<p.grid, kThreads, lds, stream>>>(p); break;
    default: route_mfma_kernel<8><<<p.grid, kThreads, lds, stream>>>(p); break;
  }
  return hipGetLastError();
}

}  // namespace mr
