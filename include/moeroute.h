/*
 * moeroute.h -- C ABI of the MI355X (gfx950) MoE token-routing library.
 *
 * The library turns router inputs into expert-grouped token slots:
 *
 *   route:  x [M, H] bf16, gate_w [E, H] bf16 (+ shared_w [H] bf16)
 *           -> topk_ids [M, S] int32, topk_weights [M, S] fp32, S = k + shared
 *   align:  topk_ids [M, S] -> sorted_token_ids, expert_ids, npp
 *
 * and mr_route_align does both in ONE kernel launch.
 *
 * Passages the operations follow (web pages, cited by title and section):
 *   [R] "[AMD] One-launch small-M MoE router ... on gfx950" (sglang PR),
 *       Modifications: the gate rows (routed and shared) are dot products
 *       over the hidden size with fp32 accumulation, read in place from the
 *       [out, in] gate weights; the routed logits are rounded to bf16; top-k
 *       with the lower id winning ties; softmax and renormalisation; slot k
 *       holds (E, sigmoid(shared logit) * scale); the launch is graph-safe
 *       through a self-resetting ticket counter; the outputs are ids [M, k+1]
 *       int32 and weights [M, k+1] fp32.
 *   [A] "W4A16 MoE prefill: M-aware moe_align block size" (ROCm vLLM),
 *       Purpose: moe_align_block_size groups the routed rows by expert and
 *       pads each touched expert to the alignment A, so that
 *       num_tokens_post_padded = sum over touched experts of ceil(c_e/A)*A;
 *       the alignment is 64 below one full block of routed rows per expert
 *       (tokens * top-k / E < 128) and 128 at or above it.
 *   [N] "Netra Kernel: Open-Source ROCm Kernels for AMD MI350X", Compile
 *       exact contracts: before capture the caller allocates persistent
 *       workspace; a launch then does no allocation, symbol lookup or host
 *       synchronisation.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Pointers named x, gate_w, shared_w, topk_*, sorted_token_ids,
 *   expert_ids, npp, ws are DEVICE pointers owned by the caller.  The
 *   library never allocates, frees, synchronises, or reads device memory
 *   on the host.  `stream` is a hipStream_t (NULL = the default stream);
 *   every kernel is enqueued on it, so calls are capturable into HIP graphs.
 * - Layouts are row-major and dense: x [M, H] (stride H), gate_w [E, H]
 *   (stride H, one row per routed expert), shared_w [H], topk_ids and
 *   topk_weights [M, S].  bf16 tensors are passed as raw 16-bit patterns.
 *   x, gate_w and shared_w must be 16-byte aligned and H a multiple of 8.
 * - S = k + (shared_w != NULL).  The shared expert, when present, has id E,
 *   so the align step sees num_experts = E' = E + 1 ids.
 * - Return value: MR_OK (0) or a negative MR_E* code.  On refusal nothing is
 *   launched and mr_last_error() lists every failed check (thread-local
 *   string, valid until the next call on the same thread).
 * - Device-side preconditions that are documented, not checked: inputs are
 *   finite; align's ids are in [0, num_experts) -- ids outside that range
 *   are skipped (never written out of bounds).
 * - Workspace `ws` (ws_bytes >= mr_workspace_bytes(...)), 256-byte aligned
 *   (as device allocators return it), must be zeroed ONCE by the caller
 *   before first use (e.g. torch.zeros).  Every launch leaves
 *   it ready for the next one (its counters at zero again, apart from a
 *   launch count kept by the prefill kernel, whose parity selects one of two
 *   grid-barrier counter sets), so the same workspace can be reused and
 *   replayed from a graph.  Launches that may overlap in time (different
 *   streams) need different workspaces.  If a launch was aborted,
 *   mr_workspace_reset() re-zeroes the counters.
 * - sorted_token_ids: entries [0, npp) are defined: for each touched expert
 *   e in ascending order, its pairs' flat indices i = m*S + slot in
 *   ascending order, then the sentinel M*S up to the next multiple of A.
 *   expert_ids[b] for b < npp/A is the expert of block b.  Entries at or
 *   past npp (and past npp/A) are unspecified.
 */
#ifndef MOEROUTE_H
#define MOEROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MR_ABI_VERSION 1

#define MR_OK 0
#define MR_EINVAL (-1)        /* null pointer, negative size, k < 1, k > E  */
#define MR_EUNSUPPORTED (-2)  /* outside the supported contract (H % 8,
                                 alignment, E or num_experts too large,
                                 k > MR_MAX_TOPK, A)                        */
#define MR_ECAPACITY (-3)     /* an output or the workspace is too small   */
#define MR_ELAUNCH (-4)       /* the HIP runtime reported a launch error   */

/* Largest supported sizes. */
#define MR_MAX_ROUTED_EXPERTS 1024  /* E for the route entry points          */
#define MR_MAX_ALIGN_EXPERTS 4096   /* num_experts for mr_align              */
#define MR_MAX_TOPK 32              /* routed k                              */
#define MR_MAX_TOKENS (1 << 20)

/* ABI version of the loaded library (MR_ABI_VERSION). */
int mr_abi_version(void);

/* Optional per-device set-up, for the CURRENT device: sets the prefill
 * kernel's dynamic-LDS limit and caches how many of its blocks fit on the
 * device at once.  The route entry points do the same on their first call on
 * a device; call this once per device before capturing launches into a HIP
 * graph, so that no runtime query runs during capture.  It also looks up
 * the device address of mr_route_align_noalloc's static scratch array on
 * this device.  Idempotent.  Returns
 * MR_OK; MR_ELAUNCH if there is no current device or a runtime query fails;
 * MR_EUNSUPPORTED for a device ordinal >= 64. */
int mr_init(void);

/* Every failed check of the last refused call on this thread, or "". */
const char *mr_last_error(void);

/* Alignment tier [A], Purpose: 128 when M*k >= 128*E, else 64 (routed k and
 * E, computed in 64-bit).  Returns MR_EINVAL for M < 0, k < 1 or E < 1. */
int32_t mr_select_alignment(int32_t M, int32_t k, int32_t E);

/* Entries sorted_token_ids needs so that any routing of M*S pairs over
 * num_experts ids fits: M*S + min(num_experts, M*S) * (A - 1).  [A], Scope
 * and safety, sizes this buffer (its num_slots figures) as the routed pairs
 * plus A - 1 padding slots per expert; since no more than M*S experts can be
 * touched, the min() bound is also enough.  (Passing that section's looser
 * M*S + num_experts*(A-1) is fine.)  Negative on bad input. */
int64_t mr_align_capacity(int32_t M, int32_t S, int32_t num_experts, int32_t A);

/* Entries expert_ids needs: mr_align_capacity(...) / A. */
int64_t mr_expert_ids_capacity(int32_t M, int32_t S, int32_t num_experts, int32_t A);

/* Workspace bytes for any call with M <= M_max tokens, E routed experts,
 * routed top-k, a shared expert or not.  Covers mr_route, mr_route_align,
 * mr_align (with S = k + has_shared, num_experts = E + has_shared) and
 * mr_debug_gate_logits. */
size_t mr_workspace_bytes(int32_t M_max, int32_t E, int32_t k, int32_t has_shared);

/* Re-zero the whole workspace (ws_bytes bytes) on `stream` with a small fill
 * kernel (safe to capture).  Needed only after an aborted launch, or after
 * one whose status (below) is not MR_STATUS_OK. */
int mr_workspace_reset(void *ws, size_t ws_bytes, void *stream);

/* Status of the launches on a workspace.  Blocks of one route launch wait
 * for each other (the small-M tail for the gate keys, the prefill launch at
 * its grid barriers and token-tile waits), which assumes that every block of
 * the launch runs: the prefill launch sizes its grid so that all its blocks
 * fit on the GPU at once, but other work holding compute units can still
 * delay some.  Every such wait is bounded; one that gives up ORs its bit
 * into a status word in the workspace and the launch runs to its end with
 * whatever data it has.  The outputs of such a launch are undefined, an
 * align launch writes *npp = -1, and the workspace must be reset
 * (mr_workspace_reset) before its next use, since blocks that arrived late
 * may have left its counters out of step.  This is the failure signal of
 * "monokernel decode for ..." (vLLM PR), Limitations/follow-ups, Failure:
 * a sticky failed word that the caller reads after each step, so that the
 * engine stops instead of hanging or going on with bad routing.
 * The word is sticky: it keeps its bits until mr_workspace_reset.
 *
 * mr_workspace_status enqueues on `stream` one small kernel that copies the
 * word into *status (device int32, caller-owned, 4-byte aligned), so it
 * orders after the launches before it on that stream and can be captured
 * into a graph.  Returns MR_OK; MR_EINVAL for a NULL ws or status;
 * MR_EUNSUPPORTED for a ws that is not 256-byte aligned or a misaligned
 * status; MR_ECAPACITY if ws_bytes is smaller than the counter region;
 * MR_ELAUNCH if the launch fails. */
#define MR_STATUS_OK 0
#define MR_STATUS_KEY_WAIT 1   /* small M: the tail's wait for the gate keys */
#define MR_STATUS_ID_WAIT 2    /* small M: block 0's wait for the other tail blocks' ids */
#define MR_STATUS_GRID_WAIT 4  /* prefill: a grid barrier */
#define MR_STATUS_TILE_WAIT 8  /* prefill: the wait for a token tile's gate items */
int mr_workspace_status(const void *ws, size_t ws_bytes, int32_t *status, void *stream);

/* Test hook, not part of the routing API: the number of polls every bounded
 * wait of later route launches (any workspace, this process) makes before it
 * gives up.  0 makes each wait give up at once, without polling, which lets
 * a test drive the failure path while every kernel still runs to its end;
 * a negative value restores the kernels' own bounds (millions of polls, far
 * beyond any launch that runs normally).  Always returns MR_OK. */
int mr_debug_set_wait_limit(int32_t polls);

/* Measurement hook, not part of the routing API: later route launches of
 * this process record, per block b, thread 0's 100 MHz clock (s_memrealtime)
 * at up to 8 points into stamps[b * 8 + i].  The prefill launch (above the
 * small-M range: M > 128, or M > 32 with M * E' * H over 160 * 2^20):
 * 0 kernel start, 1 the first gate item's MFMA loop done, 2 every gate item
 * done (partial tiles stored), 3 the first top-k group ready to start, 4
 * top-k done, 5 the align's grid barrier passed, 6 block end.  The small-M
 * launch (the blocks b < n_words / 8): 0 start, 1 gate keys published;
 * block 0, for its first token row: 2 keys arrived, 3 keys sorted, 4 top-k
 * selected, 5 slots stored, 6 align done.  stamps: device, n_words >= 8 *
 * 256 uint64 words, caller-owned; with fewer words the small-M launch
 * records nothing and the prefill launch records only if its blocks fit.
 * NULL or n_words = 0 turns it off.  Always returns MR_OK. */
int mr_debug_set_phase_stamps(uint64_t *stamps, size_t n_words);

/* Route [R], Modifications: gate contraction in fp32, bf16 rounding of the
 * routed logits, top-k (lower id wins ties), softmax + renormalise, shared
 * slot k = (E, sigmoid(s) * scale).  Writes topk_ids / topk_weights [M, S].
 * shared_w may be NULL (then S = k and there is no shared slot).
 * 0 <= M <= MR_MAX_TOKENS; 1 <= k <= min(E, MR_MAX_TOPK); H % 8 == 0. */
int mr_route(const void *x, const void *gate_w, const void *shared_w,
             int32_t M, int32_t H, int32_t E, int32_t k, float scale,
             int32_t *topk_ids, float *topk_weights,
             void *ws, size_t ws_bytes, void *stream);

/* moe_align_block_size [A], Purpose, on caller-given ids [M, S] over
 * num_experts ids with alignment A (a power of two in [16, 256]).
 * sorted_cap and expert_cap are the lengths of sorted_token_ids and
 * expert_ids; they must be at least mr_align_capacity() and
 * mr_expert_ids_capacity().  *npp (device int32) receives
 * num_tokens_post_padded.  Works for any ids, repeated or not. */
int mr_align(const int32_t *topk_ids, int32_t M, int32_t S, int32_t num_experts,
             int32_t A, int32_t *sorted_token_ids, int64_t sorted_cap,
             int32_t *expert_ids, int64_t expert_cap, int32_t *npp,
             void *ws, size_t ws_bytes, void *stream);

/* The align of one expert-parallel rank: as mr_align, but each pair's global
 * expert id e (0 <= e < num_experts_global) is first replaced by
 * expert_map[e], the rank's local id of that expert, or -1 when another rank
 * owns it; pairs with -1 (or any map entry outside [0, num_local_experts),
 * or a global id outside [0, num_experts_global)) are skipped, and the pairs
 * of local experts are grouped and padded by local id exactly as mr_align
 * does (expert_ids hold local ids, padding holds M*S).  This is the
 * single-GPU part of expert-parallel routing: each rank aligns only the
 * pairs its experts serve.  expert_map: device, [num_experts_global] int32,
 * caller-owned.  Capacities and the workspace are those of mr_align with
 * num_experts = num_local_experts.  Errors as mr_align, plus MR_EINVAL for a
 * NULL expert_map or num_experts_global < 1. */
int mr_align_local(const int32_t *topk_ids, int32_t M, int32_t S, int32_t num_experts_global,
                   const int32_t *expert_map, int32_t num_local_experts, int32_t A,
                   int32_t *sorted_token_ids, int64_t sorted_cap, int32_t *expert_ids,
                   int64_t expert_cap, int32_t *npp, void *ws, size_t ws_bytes, void *stream);

/* Route followed by align, in ONE launch: the arguments of mr_route plus
 * the alignment A (pass mr_select_alignment(M, k, E) for the M-aware tier)
 * and the align outputs.  num_experts is E + (shared_w != NULL). */
int mr_route_align(const void *x, const void *gate_w, const void *shared_w,
                   int32_t M, int32_t H, int32_t E, int32_t k, float scale,
                   int32_t A, int32_t *topk_ids, float *topk_weights,
                   int32_t *sorted_token_ids, int64_t sorted_cap,
                   int32_t *expert_ids, int64_t expert_cap, int32_t *npp,
                   void *ws, size_t ws_bytes, void *stream);

/* mr_route_align for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments minus the workspace, the same kernels and results.
 * Its workspace is a static device array of 32 MiB per GPU, part of the
 * library's code object (held on each GPU the library runs on until the
 * process ends); its address is looked up once per device, by mr_init or by
 * this call's first use on a device.  No call allocates or frees anything.
 * Each call first clears the array's counter and hand-off regions with a
 * small fill kernel on `stream`, so a call never depends on an earlier one,
 * even one whose waits gave up (such a call still writes *npp = -1; its
 * status word is cleared by the next call and cannot be read).  Every call
 * on one GPU shares that GPU's array: calls that may overlap in time on one
 * GPU (different streams, or graphs replayed concurrently) race and give
 * undefined results -- use mr_route_align with one workspace per stream
 * there.  Returns what mr_route_align returns, and MR_ECAPACITY (before
 * touching the device) when mr_workspace_bytes(M, E, k, shared) exceeds the
 * 32 MiB (about M <= 15000 at E = 512, k = 10); MR_ELAUNCH if the address
 * look-up fails. */
int mr_route_align_noalloc(const void *x, const void *gate_w, const void *shared_w,
                           int32_t M, int32_t H, int32_t E, int32_t k, float scale,
                           int32_t A, int32_t *topk_ids, float *topk_weights,
                           int32_t *sorted_token_ids, int64_t sorted_cap,
                           int32_t *expert_ids, int64_t expert_cap, int32_t *npp,
                           void *stream);

/* Test hook, not part of the routing API: writes the fp32 gate logits the
 * route kernels compute for these inputs -- logits [M, E + has_shared]
 * (the shared logit in the last column) -- using the same kernel code and
 * summation order as mr_route and mr_route_align for the same M. */
int mr_debug_gate_logits(const void *x, const void *gate_w, const void *shared_w,
                         int32_t M, int32_t H, int32_t E, float *logits,
                         void *ws, size_t ws_bytes, void *stream);

/* Row-wise argmax of an fp32 matrix, one launch: out[r] = the index of the
 * winner of row r of x, with the semantics "Open-Source ROCm Kernels for AMD
 * MI350X" (Netra Kernel blog), section "Sampling: make small batches large
 * enough", requires (PyTorch's argmax): a NaN beats every number and the
 * first NaN beats later NaNs; among equal numbers the lowest index wins; -0
 * and +0 compare equal.
 *   x    device, [R, ld] fp32 row-major (row r at x + r * ld), 16-byte
 *        aligned, ld % 4 == 0, ld >= N; only the first N values of a row
 *        are read.
 *   out  device, [R] int64, caller-owned.
 *   ws   device workspace of at least mr_argmax_workspace_bytes(R, N) bytes,
 *        16-byte aligned, zeroed once by the caller; every launch leaves it
 *        zeroed again (row tickets), so calls are graph-capturable.  One
 *        workspace per concurrently running stream.
 * Returns MR_OK; MR_EINVAL for NULL pointers, R < 0, N < 1 or ld < N;
 * MR_EUNSUPPORTED for a misaligned x or ws, ld % 4 != 0 or N >= 2^31;
 * MR_ECAPACITY for a short workspace; MR_ELAUNCH if the launch fails.
 * R == 0 launches nothing. */
size_t mr_argmax_workspace_bytes(int32_t R, int64_t N);
int mr_argmax_rows_f32(const float *x, int32_t R, int64_t N, int64_t ld, int64_t *out,
                       void *ws, size_t ws_bytes, void *stream);

/* A minimal bf16 grouped-expert GEMM that consumes the align output, the
 * consumer "W4A16 MoE prefill: M-aware moe_align block size" (ROCm vLLM),
 * Purpose, describes, for measuring what the alignment costs downstream:
 * block b of A slots runs only while b * A < *npp (its one early exit) and
 * multiplies the x rows of its slots by expert expert_ids[b]'s weights; for
 * every slot holding a pair index p < M*S it writes
 *   y[p][n] = sum_h x[p / S][h] * w_experts[e][n][h]   (fp32 accumulation),
 * while a padding slot inside npp still takes part in the contraction and
 * only skips its store (so the work follows npp).  The output does not
 * depend on A.
 *   x          device, [M, H] bf16 row-major, 16-byte aligned.
 *   w_experts  device, [num_experts, N, H] bf16 row-major, 16-byte aligned.
 *   sorted_token_ids [sorted_cap], expert_ids, npp: device, as mr_align
 *              writes them (npp and expert_ids are read on the device).
 *   y          device, [M*S, N] fp32, 16-byte aligned; rows of pairs not
 *              placed below npp are left untouched.
 * A must be 64 or 128, H and N multiples of 64.  Returns MR_OK; MR_EINVAL
 * for NULL pointers or M < 0, S < 1, num_experts < 1; MR_EUNSUPPORTED for
 * the shape and alignment limits above; MR_ELAUNCH if the launch fails.
 * M == 0 or sorted_cap < A launches nothing. */
int mr_grouped_gemm_bf16(const void *x, int32_t M, int32_t H, const void *w_experts,
                         int32_t num_experts, int32_t N, int32_t S,
                         const int32_t *sorted_token_ids, int64_t sorted_cap,
                         const int32_t *expert_ids, const int32_t *npp, int32_t A, float *y,
                         void *stream);

/* Measurement hook, not part of the routing API: one launch of a plain
 * streaming-read kernel over nbytes bytes at src (device memory, 16-byte
 * aligned, nbytes a multiple of 16), as a yardstick for what a single launch
 * of the simplest bandwidth kernel achieves at a given size.  out is a
 * caller-owned device array of MR_STREAM_READ_OUT_WORDS 32-bit words: block
 * b of the launch stores the XOR of the words it read in out[b] and leaves
 * the other entries alone, so with out zeroed first, the XOR of all entries
 * is the XOR of every word read (checkable, independent of the read order).
 * Returns MR_EINVAL for a NULL pointer, MR_EUNSUPPORTED for a misaligned src
 * or out or nbytes % 16 != 0, MR_ELAUNCH if the launch fails; nbytes == 0
 * launches nothing. */
#define MR_STREAM_READ_OUT_WORDS 4096
int mr_debug_stream_read(const void *src, size_t nbytes, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEROUTE_H */
