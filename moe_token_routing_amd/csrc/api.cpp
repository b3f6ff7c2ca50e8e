// api.cpp -- the C ABI declared in include/moeroute.h: argument checks,
// workspace layout, path choice and launches on the caller's stream.
//
// Nothing here allocates device memory, synchronises, or reads device
// memory; every refusal is decided from the arguments alone and lists every
// failed check (the default-deny discipline of "Netra Kernel: Open-Source
// ROCm Kernels for AMD MI350X", Compile exact contracts).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "kernels.h"
#include "moeroute.h"
#include "stream_read.h"
#include "argmax.h"
#include "grouped_gemm.h"

static_assert(MR_MAX_ROUTED_EXPERTS == mr::kMaxRouteExperts, "route expert limit");
static_assert(MR_MAX_ALIGN_EXPERTS == mr::kMaxAlignExperts, "align expert limit");
static_assert(MR_MAX_TOPK == mr::kMaxTopK, "top-k limit");
static_assert(MR_STATUS_KEY_WAIT == mr::kWaitKeys && MR_STATUS_ID_WAIT == mr::kWaitIds &&
                  MR_STATUS_GRID_WAIT == mr::kWaitGrid && MR_STATUS_TILE_WAIT == mr::kWaitTile,
              "status bits");

namespace {

thread_local std::string g_last_error;

// Polls a bounded wait may make before giving up: < 0 keeps each kernel's
// own bound (mr_debug_set_wait_limit).
std::atomic<int> g_wait_limit{-1};

// Phase-stamp buffer for prefill launches (mr_debug_set_phase_stamps).
std::atomic<uint64_t *> g_stamps{nullptr};
std::atomic<size_t> g_stamp_words{0};
int wait_limit(int fallback) {
  const int v = g_wait_limit.load(std::memory_order_relaxed);
  return v < 0 ? fallback : v;
}

struct Checks {
  std::string msg;
  bool inval = false, unsupported = false, capacity = false;
  void fail(int c, const char *fmt, ...) {
    char buf[256];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (!msg.empty()) msg += "; ";
    msg += buf;
    inval |= c == MR_EINVAL;
    unsupported |= c == MR_EUNSUPPORTED;
    capacity |= c == MR_ECAPACITY;
  }
  // MR_EINVAL before MR_EUNSUPPORTED before MR_ECAPACITY
  int code() const {
    return inval ? MR_EINVAL : unsupported ? MR_EUNSUPPORTED : capacity ? MR_ECAPACITY : MR_OK;
  }
  int finish(const char *fn) {
    const int c = code();
    if (c != MR_OK) g_last_error = std::string(fn) + ": " + msg;
    else g_last_error.clear();
    return c;
  }
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Row stride (floats) of the prefill launch's split-K partial rows: E rounded
// up to 32, so that every partial row starts on its own 128-byte line (the
// workspace is 256-byte aligned and the region offsets are multiples of 256).
// Rows written by different gate items then never share a line, and a
// reader can never pull a line into its L2 before every writer of that line
// is done.
inline int64_t partial_stride(int64_t E) { return (E + 31) / 32 * 32; }
inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

int64_t tight_capacity(int64_t n, int64_t Ep, int64_t A) {
  const int64_t touched = Ep < n ? Ep : n;
  return n + touched * (A - 1);
}

// Workspace regions for one call.  Every region grows with M, so a workspace
// sized for M_max serves every M <= M_max.
struct Layout {
  size_t counters = 0, keys = 0, shared = 0, hids = 0;  // small-M route
  size_t counts = 0, ranks = 0;               // standalone align
  size_t part = 0, tcnt = 0;                   // prefill route (split-K partials, tile counters)
  size_t total = 0;
};

Layout layout_for(int64_t M, int64_t E, int64_t k, int64_t sh) {
  Layout L;
  const int64_t S = k + sh, Ep = E + sh, n = M * S;
  const int64_t NE = (E + 127) / 128;  // expert tiles of the prefill route
  auto take = [](size_t &o, size_t bytes) {
    const size_t at = o;
    o = align_up(o + (bytes ? bytes : 4), 256);
    return at;
  };
  size_t o = mr::kCounterBytes;
  L.keys = take(o, (size_t)mr::kSmallMaxTokens * (size_t)E * 4);
  L.shared = take(o, (size_t)mr::kSmallMaxTokens * 8);
  L.hids = take(o, (size_t)mr::kSmallMaxTokens * (mr::kMaxTopK + 1) * 4);
  const int W = mr::align_words_per_expert((int)(Ep > 0 ? Ep : 1));
  const int64_t nch = (n + 64 * W - 1) / (64 * W);
  L.counts = take(o, (size_t)(nch * ((Ep + 3) / 4 * 4)) * 4);
  L.ranks = take(o, (size_t)n * 4);
  // split-K partials: for any M' <= M, splits * M' <= max(M, (grid / NE) * min(M, 128))
  const int64_t Epad = partial_stride(E);
  const int64_t NT = (M + 127) / 128;
  int64_t rows = (mr::kMfmaMaxGrid / (NE > 0 ? NE : 1)) * (M < 128 ? M : 128);
  if (rows < M) rows = M;
  L.part = take(o, (size_t)(rows * Epad) * 4);
  L.tcnt = take(o, (size_t)(NT * ((Ep + 3) / 4 * 4)) * 4);
  L.total = o;
  return L;
}

int launch_result(hipError_t e, const char *fn) {
  if (e == hipSuccess) {
    g_last_error.clear();
    return MR_OK;
  }
  g_last_error = std::string(fn) + ": launch failed: " + hipGetErrorString(e);
  return MR_ELAUNCH;
}

void check_route_args(Checks &ck, const void *x, const void *gate_w, const void *shared_w, int32_t M,
                      int32_t H, int32_t E, int32_t k) {
  if (!x && M > 0) ck.fail(MR_EINVAL, "x is NULL");
  if (!gate_w) ck.fail(MR_EINVAL, "gate_w is NULL");
  if (M < 0) ck.fail(MR_EINVAL, "M=%d < 0", M);
  if (M > MR_MAX_TOKENS) ck.fail(MR_EUNSUPPORTED, "M=%d > %d", M, MR_MAX_TOKENS);
  if (H < 8) ck.fail(MR_EINVAL, "H=%d < 8", H);
  else if (H % 8) ck.fail(MR_EUNSUPPORTED, "H=%d is not a multiple of 8", H);
  if (E < 1) ck.fail(MR_EINVAL, "E=%d < 1", E);
  if (E > mr::kMaxRouteExperts) ck.fail(MR_EUNSUPPORTED, "E=%d > %d", E, mr::kMaxRouteExperts);
  if (k < 1) ck.fail(MR_EINVAL, "k=%d < 1", k);
  if (k > E && E >= 1) ck.fail(MR_EINVAL, "k=%d > E=%d", k, E);
  if (k > mr::kMaxTopK) ck.fail(MR_EUNSUPPORTED, "k=%d > %d", k, mr::kMaxTopK);
  if (x && !aligned16(x)) ck.fail(MR_EUNSUPPORTED, "x is not 16-byte aligned");
  if (gate_w && !aligned16(gate_w)) ck.fail(MR_EUNSUPPORTED, "gate_w is not 16-byte aligned");
  if (shared_w && !aligned16(shared_w)) ck.fail(MR_EUNSUPPORTED, "shared_w is not 16-byte aligned");
}

void check_align_outputs(Checks &ck, int64_t n, int64_t Ep, int32_t A, const int32_t *sorted,
                         int64_t sorted_cap, const int32_t *expert_ids, int64_t expert_cap, const int32_t *npp) {
  if (!sorted) ck.fail(MR_EINVAL, "sorted_token_ids is NULL");
  if (!expert_ids) ck.fail(MR_EINVAL, "expert_ids is NULL");
  if (!npp) ck.fail(MR_EINVAL, "npp is NULL");
  if (!pow2(A) || A < 16 || A > 256)
    ck.fail(MR_EUNSUPPORTED, "A=%d is not a power of two in [16, 256]", A);
  else {
    const int64_t need = tight_capacity(n, Ep, A);
    if (sorted_cap < need)
      ck.fail(MR_ECAPACITY, "sorted_cap=%lld < %lld", (long long)sorted_cap, (long long)need);
    if (expert_cap < need / A)
      ck.fail(MR_ECAPACITY, "expert_cap=%lld < %lld", (long long)expert_cap, (long long)(need / A));
  }
}

void check_workspace(Checks &ck, const void *ws, size_t ws_bytes, size_t need) {
  if (!ws) ck.fail(MR_EINVAL, "ws is NULL");
  else if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) ck.fail(MR_EUNSUPPORTED, "ws is not 256-byte aligned");
  if (ws_bytes < need) ck.fail(MR_ECAPACITY, "ws_bytes=%zu < %zu", ws_bytes, need);
}

// Shared implementation of mr_route / mr_route_align / mr_debug_gate_logits.
int route_impl(const char *fn, const void *x, const void *gate_w, const void *shared_w, int32_t M,
               int32_t H, int32_t E, int32_t k, float scale, int32_t A, int32_t *ids, float *wts,
               int32_t *sorted, int64_t sorted_cap, int32_t *expert_ids, int64_t expert_cap, int32_t *npp,
               float *logits_out, void *ws, size_t ws_bytes, void *stream, bool do_align) {
  Checks ck;
  const bool logits_only = logits_out != nullptr;
  check_route_args(ck, x, gate_w, shared_w, M, H, E, logits_only ? 1 : k);
  const int32_t sh = shared_w ? 1 : 0;
  const int64_t S = (int64_t)k + sh, Ep = (int64_t)E + sh, n = (int64_t)M * S;
  if (!logits_only) {
    if (!ids && M > 0) ck.fail(MR_EINVAL, "topk_ids is NULL");
    if (!wts && M > 0) ck.fail(MR_EINVAL, "topk_weights is NULL");
  }
  if (do_align) check_align_outputs(ck, n, Ep, A, sorted, sorted_cap, expert_ids, expert_cap, npp);
  const Layout L = layout_for(M, E > 0 ? E : 1, k > 0 ? k : 1, sh);
  check_workspace(ck, ws, ws_bytes, L.total);
  if (ck.code() != MR_OK) return ck.finish(fn);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (M == 0) {
    if (do_align) return launch_result(mr::launch_store_zero(npp, s), fn);
    g_last_error.clear();
    return MR_OK;
  }
  char *wsb = static_cast<char *>(ws);
  uint32_t *ctr = reinterpret_cast<uint32_t *>(wsb + L.counters);
  int log2A = 0;
  while ((1 << log2A) < A) ++log2A;
  // ceil(2^32 / S); at S = 1 it would need 33 bits (the kernel does not divide then)
  const uint32_t S_magic = S == 1 ? 0u : (uint32_t)((((uint64_t)1 << 32) + (uint64_t)S - 1) / (uint64_t)S);
  int64_t fill = 0;
  if (do_align) {
    fill = tight_capacity(n, Ep, A);
    if (fill > sorted_cap) fill = sorted_cap;
  }

  // The small-M launch (a gate that streams gate rows against tiles of
  // token rows on the VALU, then one wave per token row) up to 32 rows, and
  // up to kSmallMaxTokens rows while its gate's multiply-adds stay under
  // 160 M: measured against the prefill launch, M = 40 and 64 at E' = 513,
  // H = 4096 (84 M and 134 M) 12.8 and 15.7 us against 18.6 and 18.7; M = 128
  // at E = 128, H = 2048 (34 M) 12.0 against 15.2; M = 128 at E' = 513 (269 M)
  // 24.0 against 21.0.
  const bool small = M <= 32 || (M <= mr::kSmallMaxTokens && (int64_t)M * Ep * H <= (int64_t)160 << 20);
  if (!small) {
    const int cap = mr::mfma_capacity(E);
    if (cap < 1) {
      g_last_error = std::string(fn) + ": could not size the prefill launch (no device or occupancy query failed)";
      return MR_ELAUNCH;
    }
    mr::MfmaParams q{};
    q.x = static_cast<const uint16_t *>(x);
    q.w = static_cast<const uint16_t *>(gate_w);
    q.ws_row = static_cast<const uint16_t *>(shared_w);
    q.M = M;
    q.H = H;
    q.E = E;
    q.k = logits_only ? 1 : k;
    q.S = (int)S;
    q.Ep = (int)Ep;
    q.has_shared = sh;
    q.scale = scale;
    q.ids = ids;
    q.wts = wts;
    q.NE = (E + 127) / 128;
    q.NT = (M + 127) / 128;
    q.nstages = (H + 63) / 64;
    const int grid = cap < mr::kMfmaMaxGrid ? cap : mr::kMfmaMaxGrid;
    int sk = grid / (q.NE * q.NT);
    if (sk < 1) sk = 1;
    if (sk > q.nstages) sk = q.nstages;
    // at least 4 stages of 64 k per item: a split of one or two stages pays
    // the item's fixed costs (first loads, partial-tile stores, one more
    // partial row per token in the top-k phase) for too little work
    // (measured at M = 17 .. 128, E = 512; no change at M >= 512; 8 stages,
    // which halve the partial rows, cost 0.5 .. 1.5 us at M = 40 .. 512).  With a
    // single expert tile (E <= 128) a partial row is at most 512 bytes, so
    // the extra rows are cheap and 2 stages per item pay: twice as many CUs
    // run the gate (M = 128, E = 128: -0.4 us; M = 2048, E = 128: -0.5 us;
    // one stage per item: +1.4 us at M = 128)
    {
      const int min_stages = (q.NE == 1) ? 2 : 4;
      if (sk > q.nstages / min_stages) sk = q.nstages / min_stages > 0 ? q.nstages / min_stages : 1;
    }
    q.spp = (q.nstages + sk - 1) / sk;
    q.SK = (q.nstages + q.spp - 1) / q.spp;
    q.items = q.NE * q.NT * q.SK;
    q.grid = grid;
    q.xcd_map = (grid % 8 == 0) ? 1 : 0;
    q.Epad = (int)partial_stride(E);
    q.part = reinterpret_cast<float *>(wsb + L.part);
    q.tcnt = reinterpret_cast<uint32_t *>(wsb + L.tcnt);
    q.tcnt_row = (int)((Ep + 3) / 4 * 4);
    q.zero16 = reinterpret_cast<const uint4 *>(ctr + mr::kCtrZero16);
    q.ctr = ctr;
    // Tile waits replace the first grid barrier in multi-tile launches (a
    // single tile is the whole grid, and its up to 128 top-k groups polling
    // one counter measured slower than the two-level barrier: C3 +0.2 us;
    // C4 -0.45..-1.3 us), and only when the align's grid barrier follows:
    // some barrier must hold block 0's launch-count advance until every
    // block has read the count.
    q.tile_wait = (q.NT >= 2 && q.NT <= mr::kMaxReadyTiles && do_align && !logits_only) ? 1 : 0;
    int tpb = 1;
    while (tpb < 128 && (int64_t)tpb * grid < M) tpb *= 2;
    q.tpb = tpb;
    q.ngroups = (M + tpb - 1) / tpb;
    q.do_align = do_align ? 1 : 0;
    q.A = do_align ? A : 64;
    q.log2A = do_align ? log2A : 6;
    q.sorted = sorted;
    q.sorted_cap = sorted_cap;
    q.expert_ids = expert_ids;
    q.expert_cap = expert_cap;
    q.npp = npp;
    q.logits_out = logits_out;
    q.logits_only = logits_only ? 1 : 0;
    q.wait_limit = wait_limit(mr::kBarrierSpin);
    uint64_t *st = g_stamps.load(std::memory_order_relaxed);
    q.stamps = (st && g_stamp_words.load(std::memory_order_relaxed) >= (size_t)grid * mr::kStamps) ? st : nullptr;
    return launch_result(mr::launch_route_mfma(q, s), fn);
  }

  mr::SmallParams p{};
  p.x = static_cast<const uint16_t *>(x);
  p.w = static_cast<const uint16_t *>(gate_w);
  p.ws_row = static_cast<const uint16_t *>(shared_w);
  p.M = M;
  p.H = H;
  p.E = E;
  p.k = logits_only ? 1 : k;
  p.S = (int)S;
  p.Ep = (int)Ep;
  p.has_shared = sh;
  p.scale = scale;
  p.ids = ids;
  p.wts = wts;
  p.keys = reinterpret_cast<uint32_t *>(wsb + L.keys);
  p.shared_logit = reinterpret_cast<unsigned long long *>(wsb + L.shared);
  p.hids = reinterpret_cast<uint32_t *>(wsb + L.hids);
  p.logits_out = logits_out;
  p.ctr = ctr;
  p.logits_only = logits_only ? 1 : 0;
  p.wait_limit = wait_limit(mr::kPollSpin);
  uint64_t *st = g_stamps.load(std::memory_order_relaxed);
  const size_t words = g_stamp_words.load(std::memory_order_relaxed);
  p.stamps = (st && words >= (size_t)256 * mr::kStamps) ? st : nullptr;
  p.stamp_blocks = (int)std::min<size_t>(words / mr::kStamps, (size_t)1 << 20);
  p.do_align = do_align ? 1 : 0;
  p.A = do_align ? A : 64;
  p.log2A = do_align ? log2A : 6;
  p.S_magic = S_magic;
  p.sorted = sorted;
  p.sorted_cap = sorted_cap;
  p.expert_ids = expert_ids;
  p.expert_cap = expert_cap;
  p.npp = npp;
  p.fill_count = fill;
  return launch_result(mr::launch_route_small(p, s), fn);
}

}  // namespace

// Argmax workspace: one 256-byte slot per row ticket (tickets of different rows
// in one line would serialise every block's atomic), then the [R, C] block keys.
static size_t argmax_ticket_bytes(int64_t R) { return (size_t)R * mr::kArgmaxTicketStride * 4; }

extern "C" {

int mr_abi_version(void) { return MR_ABI_VERSION; }

int mr_init(void) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_error = std::string("mr_init: no current device: ") + hipGetErrorString(e);
    return MR_ELAUNCH;
  }
  if (dev < 0 || dev >= mr::kMaxDevices) {
    g_last_error = "mr_init: device ordinal " + std::to_string(dev) + " >= " + std::to_string(mr::kMaxDevices);
    return MR_EUNSUPPORTED;
  }
  if (!mr::mfma_prepare(dev)) {
    g_last_error = "mr_init: setting up the prefill kernel on device " + std::to_string(dev) + " failed";
    return MR_ELAUNCH;
  }
  const hipError_t se = mr::scratch_setup(dev);
  if (se != hipSuccess) {
    g_last_error = std::string("mr_init: looking up the static scratch array failed: ") + hipGetErrorString(se);
    return MR_ELAUNCH;
  }
  g_last_error.clear();
  return MR_OK;
}

const char *mr_last_error(void) { return g_last_error.c_str(); }

int32_t mr_select_alignment(int32_t M, int32_t k, int32_t E) {
  if (M < 0 || k < 1 || E < 1) return MR_EINVAL;
  return ((int64_t)M * k >= (int64_t)128 * E) ? 128 : 64;
}

int64_t mr_align_capacity(int32_t M, int32_t S, int32_t num_experts, int32_t A) {
  if (M < 0 || S < 1 || num_experts < 1 || A < 1) return MR_EINVAL;
  return tight_capacity((int64_t)M * S, num_experts, A);
}

int64_t mr_expert_ids_capacity(int32_t M, int32_t S, int32_t num_experts, int32_t A) {
  const int64_t c = mr_align_capacity(M, S, num_experts, A);
  return c < 0 ? c : c / A;
}

size_t mr_workspace_bytes(int32_t M_max, int32_t E, int32_t k, int32_t has_shared) {
  if (M_max < 0 || E < 1 || k < 1) return 0;
  return layout_for(M_max, E, k, has_shared ? 1 : 0).total;
}

int mr_workspace_reset(void *ws, size_t ws_bytes, void *stream) {
  Checks ck;
  if (!ws) ck.fail(MR_EINVAL, "ws is NULL");
  else if (!aligned16(ws)) ck.fail(MR_EUNSUPPORTED, "ws is not 16-byte aligned");
  if (ws_bytes < mr::kCounterBytes) ck.fail(MR_ECAPACITY, "ws_bytes=%zu < %zu", ws_bytes, mr::kCounterBytes);
  if (ck.code() != MR_OK) return ck.finish("mr_workspace_reset");
  return launch_result(mr::launch_zero_words(static_cast<uint32_t *>(ws), ws_bytes / 4,
                                             reinterpret_cast<hipStream_t>(stream)),
                       "mr_workspace_reset");
}

int mr_workspace_status(const void *ws, size_t ws_bytes, int32_t *status, void *stream) {
  Checks ck;
  if (!ws) ck.fail(MR_EINVAL, "ws is NULL");
  else if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) ck.fail(MR_EUNSUPPORTED, "ws is not 256-byte aligned");
  if (ws_bytes < mr::kCounterBytes) ck.fail(MR_ECAPACITY, "ws_bytes=%zu < %zu", ws_bytes, mr::kCounterBytes);
  if (!status) ck.fail(MR_EINVAL, "status is NULL");
  else if ((reinterpret_cast<uintptr_t>(status) & 3u) != 0) ck.fail(MR_EUNSUPPORTED, "status is not 4-byte aligned");
  if (ck.code() != MR_OK) return ck.finish("mr_workspace_status");
  return launch_result(mr::launch_read_status(static_cast<const uint32_t *>(ws), status,
                                              reinterpret_cast<hipStream_t>(stream)),
                       "mr_workspace_status");
}

int mr_debug_set_phase_stamps(uint64_t *stamps, size_t n_words) {
  g_stamps.store(n_words ? stamps : nullptr, std::memory_order_relaxed);
  g_stamp_words.store(stamps ? n_words : 0, std::memory_order_relaxed);
  g_last_error.clear();
  return MR_OK;
}

int mr_debug_set_wait_limit(int32_t polls) {
  g_wait_limit.store(polls < 0 ? -1 : polls, std::memory_order_relaxed);
  g_last_error.clear();
  return MR_OK;
}

int mr_route(const void *x, const void *gate_w, const void *shared_w, int32_t M, int32_t H, int32_t E,
             int32_t k, float scale, int32_t *topk_ids, float *topk_weights, void *ws, size_t ws_bytes,
             void *stream) {
  return route_impl("mr_route", x, gate_w, shared_w, M, H, E, k, scale, 64, topk_ids, topk_weights, nullptr, 0,
                    nullptr, 0, nullptr, nullptr, ws, ws_bytes, stream, false);
}

int mr_route_align(const void *x, const void *gate_w, const void *shared_w, int32_t M, int32_t H, int32_t E,
                   int32_t k, float scale, int32_t A, int32_t *topk_ids, float *topk_weights,
                   int32_t *sorted_token_ids, int64_t sorted_cap, int32_t *expert_ids, int64_t expert_cap,
                   int32_t *npp, void *ws, size_t ws_bytes, void *stream) {
  return route_impl("mr_route_align", x, gate_w, shared_w, M, H, E, k, scale, A, topk_ids, topk_weights,
                    sorted_token_ids, sorted_cap, expert_ids, expert_cap, npp, nullptr, ws, ws_bytes, stream, true);
}

int mr_route_align_noalloc(const void *x, const void *gate_w, const void *shared_w, int32_t M, int32_t H,
                           int32_t E, int32_t k, float scale, int32_t A, int32_t *topk_ids, float *topk_weights,
                           int32_t *sorted_token_ids, int64_t sorted_cap, int32_t *expert_ids, int64_t expert_cap,
                           int32_t *npp, void *stream) {
  static const char *fn = "mr_route_align_noalloc";
  // Sizes first, from the arguments alone (no device call): the call's
  // workspace must fit the static array.
  if (M >= 0 && E >= 1 && k >= 1 && M <= MR_MAX_TOKENS && E <= mr::kMaxRouteExperts && k <= mr::kMaxTopK) {
    const size_t need = layout_for(M, E, k, shared_w ? 1 : 0).total;
    if (need > mr::kScratchBytes) {
      g_last_error = std::string(fn) + ": M=" + std::to_string(M) + ", E=" + std::to_string(E) + ", k=" +
                     std::to_string(k) + " needs " + std::to_string(need) + " bytes of workspace, more than the " +
                     std::to_string(mr::kScratchBytes) + "-byte static scratch array (use mr_route_align)";
      return MR_ECAPACITY;
    }
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= mr::kMaxDevices)) e = hipErrorInvalidDevice;
  if (e == hipSuccess) e = mr::scratch_setup(dev);  // once per device, unless mr_init did it
  if (e != hipSuccess) {
    g_last_error = std::string(fn) + ": static scratch set-up failed: " + hipGetErrorString(e);
    return MR_ELAUNCH;
  }
  char *ws = static_cast<char *>(mr::scratch_ptr(dev));
  // The array keeps the last call's contents.  The route launches leave
  // their zero-between-launches regions (counters, keys, hand-off rows) at
  // zero, but a launch whose waits gave up does not: clear them.
  if (M > 0 && E >= 1 && k >= 1) {
    const Layout L = layout_for(M, E, k, shared_w ? 1 : 0);
    const hipError_t ze = mr::launch_zero_words(reinterpret_cast<uint32_t *>(ws), L.counts / 4,
                                                reinterpret_cast<hipStream_t>(stream));
    if (ze != hipSuccess) return launch_result(ze, fn);
  }
  return route_impl(fn, x, gate_w, shared_w, M, H, E, k, scale, A, topk_ids, topk_weights, sorted_token_ids,
                    sorted_cap, expert_ids, expert_cap, npp, nullptr, ws, mr::kScratchBytes, stream, true);
}

int mr_debug_gate_logits(const void *x, const void *gate_w, const void *shared_w, int32_t M, int32_t H,
                         int32_t E, float *logits, void *ws, size_t ws_bytes, void *stream) {
  if (!logits) {
    g_last_error = "mr_debug_gate_logits: logits is NULL";
    return MR_EINVAL;
  }
  return route_impl("mr_debug_gate_logits", x, gate_w, shared_w, M, H, E, 1, 1.0f, 64, nullptr, nullptr,
                    nullptr, 0, nullptr, 0, nullptr, logits, ws, ws_bytes, stream, false);
}

size_t mr_argmax_workspace_bytes(int32_t R, int64_t N) {
  if (R < 0 || N < 1) return 0;
  const int64_t C = mr::argmax_chunks(N);
  return argmax_ticket_bytes(R) + (size_t)R * (size_t)C * 8;
}

int mr_argmax_rows_f32(const float *x, int32_t R, int64_t N, int64_t ld, int64_t *out, void *ws, size_t ws_bytes,
                       void *stream) {
  Checks ck;
  if (R < 0) ck.fail(MR_EINVAL, "R=%d < 0", R);
  if (N < 1) ck.fail(MR_EINVAL, "N=%lld < 1", (long long)N);
  if (N >= ((int64_t)1 << 31)) ck.fail(MR_EUNSUPPORTED, "N=%lld >= 2^31", (long long)N);
  if (ld < N) ck.fail(MR_EINVAL, "ld=%lld < N=%lld", (long long)ld, (long long)N);
  if (ld % 4 != 0) ck.fail(MR_EUNSUPPORTED, "ld=%lld is not a multiple of 4", (long long)ld);
  if (R > 0) {
    if (!x) ck.fail(MR_EINVAL, "x is NULL");
    else if (!aligned16(x)) ck.fail(MR_EUNSUPPORTED, "x is not 16-byte aligned");
    if (!out) ck.fail(MR_EINVAL, "out is NULL");
    if (!ws) ck.fail(MR_EINVAL, "ws is NULL");
    else if (!aligned16(ws)) ck.fail(MR_EUNSUPPORTED, "ws is not 16-byte aligned");
    if (N >= 1 && N < ((int64_t)1 << 31) && (int64_t)R * mr::argmax_chunks(N) > (int64_t)0x7FFFFFFF)
      ck.fail(MR_EUNSUPPORTED, "R * chunks = %lld blocks > 2^31 - 1", (long long)((int64_t)R * mr::argmax_chunks(N)));
    if (R >= 0 && N >= 1) {
      const size_t need = mr_argmax_workspace_bytes(R, N);
      if (ws_bytes < need) ck.fail(MR_ECAPACITY, "ws_bytes=%zu < %zu", ws_bytes, need);
    }
  }
  if (ck.code() != MR_OK) return ck.finish("mr_argmax_rows_f32");
  if (R == 0) {
    g_last_error.clear();
    return MR_OK;
  }
  mr::ArgmaxParams p;
  p.x = x;
  p.R = R;
  p.N = N;
  p.ld = ld;
  p.C = mr::argmax_chunks(N);
  p.out = out;
  p.ticket = static_cast<uint32_t *>(ws);
  p.part = reinterpret_cast<unsigned long long *>(static_cast<char *>(ws) + argmax_ticket_bytes(R));
  return launch_result(mr::launch_argmax(p, reinterpret_cast<hipStream_t>(stream)), "mr_argmax_rows_f32");
}

int mr_grouped_gemm_bf16(const void *x, int32_t M, int32_t H, const void *w_experts, int32_t num_experts, int32_t N,
                         int32_t S, const int32_t *sorted_token_ids, int64_t sorted_cap, const int32_t *expert_ids,
                         const int32_t *npp, int32_t A, float *y, void *stream) {
  Checks ck;
  if (M < 0) ck.fail(MR_EINVAL, "M=%d < 0", M);
  if (S < 1) ck.fail(MR_EINVAL, "S=%d < 1", S);
  if (num_experts < 1) ck.fail(MR_EINVAL, "num_experts=%d < 1", num_experts);
  if (H < 64 || H % 64 != 0) ck.fail(MR_EUNSUPPORTED, "H=%d is not a positive multiple of 64", H);
  if (N < 64 || N % 64 != 0) ck.fail(MR_EUNSUPPORTED, "N=%d is not a positive multiple of 64", N);
  if (A != 64 && A != 128) ck.fail(MR_EUNSUPPORTED, "A=%d is not 64 or 128", A);
  if (sorted_cap < 0) ck.fail(MR_EINVAL, "sorted_cap=%lld < 0", (long long)sorted_cap);
  if (N >= 64 && (int64_t)num_experts * N > ((int64_t)1 << 31) / (H > 0 ? H : 1))
    ck.fail(MR_EUNSUPPORTED, "num_experts * N * H >= 2^31 elements");
  if (M > 0) {
    if (!x) ck.fail(MR_EINVAL, "x is NULL");
    else if (!aligned16(x)) ck.fail(MR_EUNSUPPORTED, "x is not 16-byte aligned");
    if (!w_experts) ck.fail(MR_EINVAL, "w_experts is NULL");
    else if (!aligned16(w_experts)) ck.fail(MR_EUNSUPPORTED, "w_experts is not 16-byte aligned");
    if (!sorted_token_ids) ck.fail(MR_EINVAL, "sorted_token_ids is NULL");
    if (!expert_ids) ck.fail(MR_EINVAL, "expert_ids is NULL");
    if (!npp) ck.fail(MR_EINVAL, "npp is NULL");
    if (!y) ck.fail(MR_EINVAL, "y is NULL");
    else if (!aligned16(y)) ck.fail(MR_EUNSUPPORTED, "y is not 16-byte aligned");
  }
  if (ck.code() != MR_OK) return ck.finish("mr_grouped_gemm_bf16");
  if (M == 0 || sorted_cap < A) {
    g_last_error.clear();
    return MR_OK;
  }
  mr::GemmParams p;
  p.x = static_cast<const uint16_t *>(x);
  p.M = M;
  p.H = H;
  p.w = static_cast<const uint16_t *>(w_experts);
  p.Ep = num_experts;
  p.N = N;
  p.S = S;
  p.A = A;
  p.sorted = sorted_token_ids;
  p.sorted_cap = sorted_cap;
  p.expert_ids = expert_ids;
  p.npp = npp;
  p.y = y;
  return launch_result(mr::launch_grouped_gemm(p, reinterpret_cast<hipStream_t>(stream)), "mr_grouped_gemm_bf16");
}

static_assert(MR_STREAM_READ_OUT_WORDS == mr::kStreamReadMaxBlocks, "stream-read output size");

int mr_debug_stream_read(const void *src, size_t nbytes, uint32_t *out, void *stream) {
  Checks ck;
  if (!src) ck.fail(MR_EINVAL, "src is NULL");
  else if (!aligned16(src)) ck.fail(MR_EUNSUPPORTED, "src is not 16-byte aligned");
  if (!out) ck.fail(MR_EINVAL, "out is NULL");
  else if (reinterpret_cast<uintptr_t>(out) % 4 != 0) ck.fail(MR_EUNSUPPORTED, "out is not 4-byte aligned");
  if (nbytes % 16 != 0) ck.fail(MR_EUNSUPPORTED, "nbytes=%zu is not a multiple of 16", nbytes);
  if (ck.code() != MR_OK) return ck.finish("mr_debug_stream_read");
  return launch_result(mr::launch_stream_read(src, nbytes, out, reinterpret_cast<hipStream_t>(stream)),
                       "mr_debug_stream_read");
}

// Shared implementation of mr_align and mr_align_local: num_experts is the
// number of experts the align groups by (local experts with a map).
static int align_impl(const char *fn, const int32_t *topk_ids, int32_t M, int32_t S, const int32_t *expert_map,
                      int32_t num_global, int32_t num_experts, int32_t A, int32_t *sorted_token_ids,
                      int64_t sorted_cap, int32_t *expert_ids, int64_t expert_cap, int32_t *npp, void *ws,
                      size_t ws_bytes, void *stream, Checks &ck) {
  if (!topk_ids && M > 0) ck.fail(MR_EINVAL, "topk_ids is NULL");
  if (M < 0) ck.fail(MR_EINVAL, "M=%d < 0", M);
  if (M > MR_MAX_TOKENS) ck.fail(MR_EUNSUPPORTED, "M=%d > %d", M, MR_MAX_TOKENS);
  if (S < 1) ck.fail(MR_EINVAL, "S=%d < 1", S);
  if (S > mr::kMaxTopK + 1) ck.fail(MR_EUNSUPPORTED, "S=%d > %d", S, mr::kMaxTopK + 1);
  if (num_experts < 1) ck.fail(MR_EINVAL, "num_experts=%d < 1", num_experts);
  if (num_experts > mr::kMaxAlignExperts)
    ck.fail(MR_EUNSUPPORTED, "num_experts=%d > %d", num_experts, mr::kMaxAlignExperts);
  const int64_t n = (int64_t)(M > 0 ? M : 0) * (S > 0 ? S : 0);
  const int Ep = num_experts > 0 ? num_experts : 1;
  check_align_outputs(ck, n, Ep, A, sorted_token_ids, sorted_cap, expert_ids, expert_cap, npp);
  // the align regions of a route workspace with E = Ep and k = S
  const Layout L = layout_for(M > 0 ? M : 0, Ep, S > 0 ? S : 1, 0);
  check_workspace(ck, ws, ws_bytes, L.total);
  if (ck.code() != MR_OK) return ck.finish(fn);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (n == 0) return launch_result(mr::launch_store_zero(npp, s), fn);
  char *wsb = static_cast<char *>(ws);
  mr::AlignParams p{};
  p.ids = topk_ids;
  p.map = expert_map;
  p.Eg = num_global;
  p.n = n;
  p.S = S;
  p.Ep = Ep;
  p.A = A;
  p.sorted = sorted_token_ids;
  p.sorted_cap = sorted_cap;
  p.expert_ids = expert_ids;
  p.expert_cap = expert_cap;
  p.npp = npp;
  const int64_t fill = tight_capacity(n, Ep, A);
  p.fill_count = fill < sorted_cap ? fill : sorted_cap;
  p.W = mr::align_words_per_expert(Ep);
  p.nchunks = (int)((n + 64 * p.W - 1) / (64 * p.W));
  p.ctr = reinterpret_cast<uint32_t *>(wsb + L.counters);
  p.counts = reinterpret_cast<int32_t *>(wsb + L.counts);
  p.cstride = (Ep + 3) / 4 * 4;
  p.ranks = reinterpret_cast<int32_t *>(wsb + L.ranks);
  return launch_result(mr::launch_align(p, s), fn);
}

int mr_align(const int32_t *topk_ids, int32_t M, int32_t S, int32_t num_experts, int32_t A,
             int32_t *sorted_token_ids, int64_t sorted_cap, int32_t *expert_ids, int64_t expert_cap, int32_t *npp,
             void *ws, size_t ws_bytes, void *stream) {
  Checks ck;
  return align_impl("mr_align", topk_ids, M, S, nullptr, 0, num_experts, A, sorted_token_ids, sorted_cap, expert_ids,
                    expert_cap, npp, ws, ws_bytes, stream, ck);
}

int mr_align_local(const int32_t *topk_ids, int32_t M, int32_t S, int32_t num_experts_global,
                   const int32_t *expert_map, int32_t num_local_experts, int32_t A, int32_t *sorted_token_ids,
                   int64_t sorted_cap, int32_t *expert_ids, int64_t expert_cap, int32_t *npp, void *ws,
                   size_t ws_bytes, void *stream) {
  Checks ck;
  if (!expert_map) ck.fail(MR_EINVAL, "expert_map is NULL");
  if (num_experts_global < 1) ck.fail(MR_EINVAL, "num_experts_global=%d < 1", num_experts_global);
  return align_impl("mr_align_local", topk_ids, M, S, expert_map, num_experts_global, num_local_experts, A,
                    sorted_token_ids, sorted_cap, expert_ids, expert_cap, npp, ws, ws_bytes, stream, ck);
}

}  // extern "C"
