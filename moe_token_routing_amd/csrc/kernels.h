// kernels.h -- launch parameters shared by the host entry points (api.cpp)
// and the kernels.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mr {

constexpr int kMaxTopK = 32;            // routed k
constexpr int kMaxRouteExperts = 1024;  // routed E for the route kernels
constexpr int kMaxAlignExperts = 4096;  // E' for align
constexpr int kSmallMaxTokens = 128;    // the most token rows route_small takes

// Counter words at the start of the workspace.  The first 256 bytes hold
// single counters; then kTicketLanes first-level barrier counters follow,
// each in its own 256-byte slot so that blocks arriving at a grid barrier
// spread their atomics over several addresses.  Every counter is zero
// between launches except the prefill kernel's launch count (kCtrEpoch): its
// parity picks which of two barrier counter sets a launch uses, and each
// launch clears the other set for the next one.
enum CounterIndex : int {
  kCtrBarTop0 = 0,    // prefill grid barrier, set 0: completed lanes
  kCtrStarted = 1,    // blocks that have begun
  kCtrDone = 2,       // phase-one completions
  kCtrPublished = 3,  // winner's publication flag
  kCtrWork = 4,       // work-queue head
  kCtrExited = 5,     // block exits
  kCtrError = 6,      // status: kWait* bits of the bounded waits that gave up (sticky until a reset)
  kCtrEpoch = 16,     // prefill launches so far (any value is a valid start)
  kCtrBarTop1 = 32,   // prefill grid barrier, set 1: completed lanes
  kCtrZero16 = 60,    // words 60..63: always zero (a 16-byte zero source)
};
// Bits of the status word (kCtrError), one per kind of bounded wait.  A
// wait that gives up ORs its bit in and the launch goes on with whatever data
// it has; its outputs are then undefined and an align launch writes npp = -1.
constexpr uint32_t kWaitKeys = 1;     // small M: a tail wave's poll of the gate keys (MR_STATUS_KEY_WAIT)
constexpr uint32_t kWaitIds = 2;      // small M: block 0's poll of the other tail blocks' ids (MR_STATUS_ID_WAIT)
constexpr uint32_t kWaitGrid = 4;     // prefill: a grid barrier (MR_STATUS_GRID_WAIT)
constexpr uint32_t kWaitTile = 8;     // prefill: a token tile's gate items (MR_STATUS_TILE_WAIT)
// Bounds on the waits (polls), unless the caller sets one for tests.
constexpr int kPollSpin = 1 << 21;     // small M: each poll is one memory round trip
constexpr int kBarrierSpin = 1 << 22;  // prefill: each poll is a load and a short sleep
constexpr int kTicketLanes = 16;
constexpr int kTicketLaneStride = 64;  // words (256 bytes); set s of lane r at word 64 + 64 r + 32 s
constexpr int kReleaseWord = 8;        // words after a lane counter: its barrier release word
// Then the prefill route's tile-ready counters: set s of token tile t at word
// kReadyBase + (2 t + s) * kReadyStride, each in its own 128-byte slot (items
// of different tiles arriving on one line would serialise).  Launches with
// more than kMaxReadyTiles token tiles use a grid barrier instead.
constexpr int kMaxReadyTiles = 256;
constexpr int kReadyStride = 32;  // words
constexpr int kReadyBase = 64 + kTicketLanes * kTicketLaneStride;
constexpr size_t kCounterBytes = (size_t)(kReadyBase + 2 * kMaxReadyTiles * kReadyStride) * 4;

// Small-M fused route (+ align).
struct SmallParams {
  const uint16_t *x;       // [M, H] bf16
  const uint16_t *w;       // [E, H] bf16
  const uint16_t *ws_row;  // [H] bf16 or null
  int M, H, E, k, S, Ep, has_shared;
  float scale;
  int32_t *ids;   // [M, S]
  float *wts;     // [M, S]
  // Workspace, all zero between launches: selection keys [M, E] (0 = not yet
  // written), the shared logits [M] as (1 << 32 | fp32 bits), and hids.
  uint32_t *keys;
  unsigned long long *shared_logit;
  uint32_t *hids;  // [M, S] at M >= 5: tail blocks 1.. hand block 0 their ids as id + 1 (0 = not yet)
  float *logits_out;  // logits_only: the caller's [M, Ep] fp32 buffer
  uint32_t *ctr;      // counter words (kCounterBytes)
  int logits_only;
  int wait_limit;     // polls a wait makes before it gives up (0: gives up at once)
  uint64_t *stamps;   // null, or [stamp_blocks, kStamps]: per-block phase times (100 MHz clock)
  int stamp_blocks;   // blocks b < stamp_blocks record
  // align
  int do_align, A, log2A;
  uint32_t S_magic;  // ceil(2^32 / S) for S >= 2: i / S == umulhi(i, S_magic) for i < 2^32 / S
                     // (2^32 does not fit: S = 1 is not divided at all)
  int32_t *sorted;
  int64_t sorted_cap;
  int32_t *expert_ids;
  int64_t expert_cap;
  int32_t *npp;
  int64_t fill_count;  // sentinel pre-fill length
  int fill_blocks;     // blocks 0 .. fill_blocks - 1 take the pre-fill slices (set by the launch)
};

// Standalone align.
struct AlignParams {
  const int32_t *ids;  // [n]
  const int32_t *map;  // null, or [Eg]: each global expert's local id (-1: another rank's)
  int Eg;              // global experts (with map)
  int64_t n;
  int S, Ep, A;
  int32_t *sorted;
  int64_t sorted_cap;
  int32_t *expert_ids;
  int64_t expert_cap;
  int32_t *npp;
  int64_t fill_count;
  int W;        // bitmap words per expert; a chunk is 64 * W pairs
  int nchunks;
  uint32_t *ctr;    // counter words
  int32_t *counts;  // [nchunks, cstride]: per-chunk counts, then per-chunk bases
  int cstride;      // Ep rounded up to 4 (16-byte rows)
  int32_t *ranks;   // [n] rank of each pair inside its chunk
};

// Prefill route (+ align) in one persistent launch: split-K MFMA gate,
// top-k per token, align; grid barriers between the phases.
constexpr int kMfmaMaxGrid = 256;  // blocks of one launch (one per CU on MI355X)
struct MfmaParams {
  const uint16_t *x;       // [M, H] bf16
  const uint16_t *w;       // [E, H] bf16
  const uint16_t *ws_row;  // [H] bf16 or null
  int M, H, E, k, S, Ep, has_shared;
  float scale;
  int32_t *ids;  // [M, S]
  float *wts;    // [M, S]
  int NE, NT;    // expert tiles (ceil(E / 128)) and token tiles (ceil(M / 128))
  int SK;        // K splits
  int spp;       // 64-wide k stages per split
  int nstages;   // ceil(H / 64)
  int items;     // NE * NT * SK
  int grid;      // blocks (all resident)
  int xcd_map;   // deal items to XCDs (grid % 8 == 0)
  int Epad;      // row stride of the partials (E rounded up to 32: one 128-byte line per row start)
  float *part;   // [SK, M, Epad] fp32 gate partials
  uint32_t *tcnt;       // [NT, tcnt_row]: pairs per (128-token tile, expert)
  int tcnt_row;         // words per tcnt row: Ep rounded up to 4
  const uint4 *zero16;  // 16 zero bytes (stands in for k past H): kCtrZero16 of the counters
  uint32_t *ctr;        // counter words
  int tile_wait;        // top-k groups wait for their own tile's items only (2 <= NT <= kMaxReadyTiles, with align)
  int tpb, ngroups;     // tokens per top-k group (power of two <= 128) and groups
  int do_align, A, log2A;
  int32_t *sorted;
  int64_t sorted_cap;
  int32_t *expert_ids;
  int64_t expert_cap;
  int32_t *npp;
  float *logits_out;  // logits_only: the caller's [M, Ep] fp32 buffer
  int logits_only;
  int wait_limit;     // polls a wait makes before it gives up (0: gives up at once)
  uint64_t *stamps;   // null, or [grid, kStamps]: per-block phase times (100 MHz clock)
};
// Phase stamps of the prefill launch (per block, thread 0): kernel start,
// first gate item's MFMA loop done, every gate item done (partial tiles
// stored), first top-k group ready to start, top-k done, align barrier
// passed, block end.
constexpr int kStamps = 8;
constexpr int kMaxDevices = 64;  // per-device set-up is kept for device ordinals below this
size_t mfma_lds_bytes();
// Blocks of the prefill launch for E routed experts that fit on the current
// device at once (0 if a runtime query failed); the first call on a device
// also sets the kernel's dynamic-LDS limit there.
int mfma_capacity(int E);
// Does that set-up for every instantiation on device dev (current).
bool mfma_prepare(int dev);
hipError_t launch_route_mfma(const MfmaParams &p, hipStream_t stream);


int small_rows_per_block(int Ep, int M);
hipError_t launch_route_small(const SmallParams &p, hipStream_t stream);

int align_words_per_expert(int Ep);
hipError_t launch_align(const AlignParams &p, hipStream_t stream);

// Fill n words with zero / write *npp = 0 (small kernels, graph-safe).
hipError_t launch_zero_words(uint32_t *p, size_t n, hipStream_t stream);
hipError_t launch_store_zero(int32_t *p, hipStream_t stream);
// *out = the status word (a coherent read), on the stream.
hipError_t launch_read_status(const uint32_t *ctr, int32_t *out, hipStream_t stream);

// The workspace of the entry point that allocates nothing: a static device
// array of kScratchBytes per GPU (static_scratch.hip).  scratch_setup looks
// up its device address on device dev (which must be current) once;
// scratch_ptr returns it (null before the set-up).
constexpr size_t kScratchBytes = (size_t)32 << 20;
hipError_t scratch_setup(int dev);
void *scratch_ptr(int dev);

}  // namespace mr
